// probe.hip — rate probes behind bqa_debug_probe: what the device sustains
// for the operations the attention kernels are bound by, next to the
// published peaks that the roofline figures divide by.
//
//  * matrix probes: every wavefront issues `iters` rounds of eight dense
//    matrix instructions of one type on register operands, in four
//    independent accumulator chains (enough to cover the instruction's
//    latency at four wavefronts per SIMD);
//  * exp probe: every lane runs `iters` rounds of eight independent
//    v_exp_f32 chains, x <- 2^-x (the negation is a source modifier, so the
//    loop is exponentials only; the values stay in (1/4, 1));
//  * copy probe: a grid-stride 16-byte copy of `bytes` from src to dst;
//  * read probe: a grid-stride 16-byte read of `bytes` from src, folded into
//    one word per workgroup; the non-temporal read probe does the same with
//    the non-temporal cache policy (the policy of the decode kernel's
//    copies);
//  * issue probes: per round, every wavefront issues 8 dense i8 32x32x32
//    matrix instructions (four accumulator chains), 64 independent fp32
//    fused multiply-adds, 32 independent v_exp_f32, or the matrix
//    instructions interleaved with either (one matrix instruction, then 8
//    multiply-adds or 4 exponentials), or the multiply-adds interleaved with
//    the exponentials: the mixed time against the sum of the separate ones
//    says how much of one kind of work runs under the other;
//  * LDS read probes: 8 back-to-back 16-byte reads per round, with each
//    group of 16 lanes on its own 256-byte span or the four groups on
//    different chunks of the same 64-byte rows;
//  * instruction probes: 64 instances per round of one vector instruction
//    (fp32 multiply, multiply-add, int->float conversion, v_max3, fp8 pack,
//    scaled fp4 pack, permlane32 swap) over 16 independent chains.
// Each workgroup writes one checksum word to dst (matrix and exp probes) so
// that nothing is optimised away.
#include "common.hpp"
#include "internal.hpp"

namespace bqa {

namespace {

template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int64_t iters, uint32_t* __restrict__ out) {
    const int l = threadIdx.x & 63;
    // operands: small values, different per lane (the rate does not depend on them)
    const int seed = (int)(threadIdx.x * 2654435761u + blockIdx.x);
    const v4i a4 = {seed & 0x07070707, (seed >> 1) & 0x07070707, 0x01020304, l};
    const v8i a8 = {a4[0], a4[1], a4[2], a4[3], 0x01010101, 0x02020202, 0x03030303, 0x04040404};
    uint32_t sum = 0;
    if constexpr (KIND == PROBE_MFMA_I8) {
        v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c3, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += (uint32_t)(c0[i] ^ c1[i] ^ c2[i] ^ c3[i]);
    } else if constexpr (KIND == PROBE_MFMA_BF16) {
        const v8bf b = __builtin_bit_cast(v8bf, a4);
        v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += __builtin_bit_cast(uint32_t, c0[i] + c1[i] + c2[i] + c3[i]);
    } else {
        // f8f6f4 instructions: format 0 (e4m3) for the fp8 probe, 4 (e2m1, scaled) for fp4
        constexpr int FMT = KIND == PROBE_MFMA_F8 ? 0 : 4;
        v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, c0, FMT, FMT, 0, 127, 0, 127);
                c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, c1, FMT, FMT, 0, 127, 0, 127);
                c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, c2, FMT, FMT, 0, 127, 0, 127);
                c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, c3, FMT, FMT, 0, 127, 0, 127);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += __builtin_bit_cast(uint32_t, c0[i] + c1[i] + c2[i] + c3[i]);
    }
    sum = (uint32_t)wave_max((float)(sum & 0xFFFF));
    if (threadIdx.x == 0) out[blockIdx.x] = sum;
}

__global__ __launch_bounds__(256) void exp_probe_kernel(int64_t iters, uint32_t* __restrict__ out) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)((threadIdx.x + 37 * k) & 63) * (1.0f / 64.0f) + 0.25f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += x[k];
    s = wave_max(s);
    if (threadIdx.x == 0) out[blockIdx.x] = __builtin_bit_cast(uint32_t, s);
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                                         int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4i a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

template <bool NT>
__device__ __forceinline__ v4i probe_load(const v4i* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const v4i* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ out) {
    // each workgroup reads 32 KB contiguous per round (8 loads per thread)
    const int64_t stride = (int64_t)gridDim.x * 256 * 8;
    int64_t i = (int64_t)blockIdx.x * 256 * 8 + threadIdx.x;
    v4i acc = {0, 0, 0, 0};
    for (; i + 256 * 7 < n16; i += stride) {
        v4i a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = probe_load<NT>(src + i + 256 * u);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= a[u];
    }
    for (int u = 0; u < 8; ++u)
        if (i + 256 * u < n16) acc ^= probe_load<NT>(src + i + 256 * u);
    const float f = (float)((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) & 0xFFFF);
    const float m = wave_max(f);
    if (threadIdx.x == 0) out[blockIdx.x] = (uint32_t)m;
}

// Issue probes: MODE 0 matrix only, 1 multiply-adds only, 2 both, 3
// exponentials only, 4 matrix and exponentials, 5 multiply-adds and
// exponentials (the multiply-adds on chains of their own).
template <int MODE>
__global__ __launch_bounds__(256) void issue_probe_kernel(int64_t iters, uint32_t* __restrict__ out) {
    const int l = threadIdx.x & 63;
    const int seed = (int)(threadIdx.x * 2654435761u + blockIdx.x);
    const v4i a4 = {seed & 0x07070707, (seed >> 1) & 0x07070707, 0x01020304, l};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    float x[16], y[16];
    const float fa = 0.5f + (float)(l & 7) * (1.0f / 1024.0f);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        x[k] = (float)((threadIdx.x + 37 * k) & 63) * (1.0f / 64.0f) + 0.25f;
        y[k] = x[k] * 0.5f;
    }
    constexpr bool MF = MODE == 0 || MODE == 2 || MODE == 4, FM = MODE == 1 || MODE == 2 || MODE == 5,
                   EX = MODE == 3 || MODE == 4 || MODE == 5;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if constexpr (MF) {
                if (g % 4 == 0) c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c0, 0, 0, 0);
                if (g % 4 == 1) c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c1, 0, 0, 0);
                if (g % 4 == 2) c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c2, 0, 0, 0);
                if (g % 4 == 3) c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c3, 0, 0, 0);
            }
            if constexpr (FM) {
#pragma unroll
                for (int k = 0; k < 8; ++k) y[(8 * g + k) & 15] = __builtin_fmaf(y[(8 * g + k) & 15], fa, 0.25f);
            }
            if constexpr (EX) {
#pragma unroll
                for (int k = 0; k < 4; ++k) x[(4 * g + k) & 15] = __builtin_amdgcn_exp2f(-x[(4 * g + k) & 15]);
            }
            if constexpr (MF && (FM || EX)) {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x0002, FM ? 8 : 4, 0);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += x[k] + y[k];
    uint32_t sum = __builtin_bit_cast(uint32_t, s);
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += (uint32_t)(c0[i] ^ c1[i] ^ c2[i] ^ c3[i]);
    sum = (uint32_t)wave_max((float)(sum & 0xFFFF));
    if (threadIdx.x == 0) out[blockIdx.x] = sum;
}

// LDS read probes: every wavefront runs iters rounds of 8 independent 16-byte
// reads issued back to back (8 KB apart), then one wait.  Lane l = 16 g + q.
// SPANS: group g reads entry q of its own contiguous 256-byte span
// (2048 g + 16 q); SHARED_ROWS: group g reads chunk g ^ (q / 4) of the
// 64-byte row q, so that the four groups read different chunks of the same
// 16 rows.  In both, every group of 16 lanes covers all 64 banks once.
template <bool SPANS>
__global__ __launch_bounds__(256) void lds_probe_kernel(int64_t iters, uint32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) v4i buf[4096];   // 64 KB
    for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = v4i{i, i + 1, i + 2, i + 3};
    __syncthreads();
    const int l = threadIdx.x & 63, g = l >> 4, q = l & 15;
    const int off = SPANS ? 2048 * g + 16 * q : 64 * q + 16 * (g ^ ((q >> 2) & 3));   // below 8 KB
    const uint32_t a = lds_addr(buf) + (uint32_t)off;
    v4i acc = {0, 0, 0, 0};
    for (int64_t it = 0; it < iters; ++it) {
        v4i r0, r1, r2, r3, r4, r5, r6, r7;
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:8192\n\t"
            "ds_read_b128 %2, %8 offset:16384\n\t"
            "ds_read_b128 %3, %8 offset:24576\n\t"
            "ds_read_b128 %4, %8 offset:32768\n\t"
            "ds_read_b128 %5, %8 offset:40960\n\t"
            "ds_read_b128 %6, %8 offset:49152\n\t"
            "ds_read_b128 %7, %8 offset:57344\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
            : "v"(a)
            : "memory");
        acc ^= r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
    }
    const uint32_t sum = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
    const uint32_t m = (uint32_t)wave_max((float)(sum & 0xFFFF));
    if (threadIdx.x == 0) out[blockIdx.x] = m;
}

// Single-instruction issue probes: every round, each lane runs 64 instances
// of one vector instruction over 16 independent chains.
template <int OP>
__global__ __launch_bounds__(256) void op_probe_kernel(int64_t iters, uint32_t* __restrict__ out) {
    const int l = threadIdx.x & 63;
    float x[16];
    uint32_t u[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        x[q] = (float)((threadIdx.x + 37 * q) & 63) * (1.0f / 64.0f) + 0.25f;
        u[q] = threadIdx.x * 77u + (uint32_t)q;
    }
    const float fa = 0.5f + (float)(l & 7) * (1.0f / 1024.0f);
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            const int i = q & 15, j = (q + 5) & 15, k = (q + 9) & 15;
            if constexpr (OP == 0) x[i] = x[i] * x[j];                                           // v_mul_f32
            else if constexpr (OP == 1) x[i] = __builtin_fmaf(x[i], fa, x[j]);                   // v_fma_f32
            else if constexpr (OP == 2) x[i] = (float)__builtin_bit_cast(int, x[i]);             // v_cvt_f32_i32
            else if constexpr (OP == 3) x[i] = __builtin_fmaxf(__builtin_fmaxf(x[i], x[j]), x[k]);   // v_max3_f32
            else if constexpr (OP == 4) u[i] = __builtin_amdgcn_cvt_pk_fp8_f32(x[i], x[j], u[i], false);
            else if constexpr (OP == 5) u[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u[i], x[i], x[j], fa, 0);
            else {                                                                              // v_permlane32_swap
                const v2i r = __builtin_amdgcn_permlane32_swap((int)u[i], (int)u[j], false, false);
                u[i] = (uint32_t)r[0];
                u[j] = (uint32_t)r[1];
            }
        }
    }
    uint32_t s = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += __builtin_bit_cast(uint32_t, x[q]) + u[q];
    s = (uint32_t)wave_max((float)(s & 0xFFFF));
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_probe(int kind, int grid, int64_t iters, const void* src, void* dst, size_t bytes,
                        hipStream_t st) {
    uint32_t* out = (uint32_t*)dst;
    switch (kind) {
        case PROBE_MFMA_I8: mfma_probe_kernel<PROBE_MFMA_I8><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_MFMA_F8: mfma_probe_kernel<PROBE_MFMA_F8><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_MFMA_F4: mfma_probe_kernel<PROBE_MFMA_F4><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_MFMA_BF16: mfma_probe_kernel<PROBE_MFMA_BF16><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_EXP: exp_probe_kernel<<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_COPY:
            copy_probe_kernel<<<grid, 256, 0, st>>>((const v4i*)src, (v4i*)dst, (int64_t)(bytes / 16));
            break;
        case PROBE_READ:
            read_probe_kernel<false><<<grid, 256, 0, st>>>((const v4i*)src, (int64_t)(bytes / 16), out);
            break;
        case PROBE_READ_NT:
            read_probe_kernel<true><<<grid, 256, 0, st>>>((const v4i*)src, (int64_t)(bytes / 16), out);
            break;
        case PROBE_ISSUE_MFMA: issue_probe_kernel<0><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_ISSUE_FMA: issue_probe_kernel<1><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_ISSUE_MFMA_FMA: issue_probe_kernel<2><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_ISSUE_EXP: issue_probe_kernel<3><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_ISSUE_MFMA_EXP: issue_probe_kernel<4><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_OP_MUL: op_probe_kernel<0><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_OP_FMA: op_probe_kernel<1><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_OP_CVT_F32_I32: op_probe_kernel<2><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_OP_MAX3: op_probe_kernel<3><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_OP_CVT_PK_FP8: op_probe_kernel<4><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_OP_CVT_PK_FP4: op_probe_kernel<5><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_OP_PERMLANE32: op_probe_kernel<6><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_ISSUE_EXP_FMA: issue_probe_kernel<5><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_LDS_SHARED_ROWS: lds_probe_kernel<false><<<grid, 256, 0, st>>>(iters, out); break;
        case PROBE_LDS_SPANS: lds_probe_kernel<true><<<grid, 256, 0, st>>>(iters, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bqa
