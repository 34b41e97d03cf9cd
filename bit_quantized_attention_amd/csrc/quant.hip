// quant.hip — operand quantisation kernels (HBM-bound).
//
//  * K-smoothing ("SageBwd: A Trainable Low-bit Attention", Methodology 4 and
//    Results): per-channel token sums of K in fp64, then
//    mu = fp32(sum / N - eps).  The sums of bf16/fp16 inputs are exact in fp64
//    for the workloads here, so the result does not depend on the order of
//    the partial sums.
//  * INT8 per token block ("SageBwd", Methodology 1): absmax scale per block.
//  * Per-channel V in int8 or e4m3, written channel-major.
//  * MXFP4 along d (Q, K) with optional block means ("ThriftAttention",
//    Method step 1) and along tokens (V) ("Attn-QAT", §1; "ThriftAttention",
//    Method step 2).
//
// All kernels are coalesced on the [.., N, d] input rows; each thread moves
// 16 bytes per load.
#include "common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace bqa {

// ------------------------------------------------------------ K token sums
// grid (BH, chunks); 256 threads = 16 rows x 16 column groups of 8 channels;
// fp64 partial sums of each chunk of tokens.
template <bool IS_F16>
__global__ __launch_bounds__(256) void ksum_partial_kernel(Dense x, int H, int N, int d, int rows_per_chunk,
                                                            double* __restrict__ part) {
    const int bh = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
    const int b = bh / H, h = bh % H;
    const int cg = threadIdx.x % 16, r = threadIdx.x / 16;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH + cg * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int t0 = chunk * rows_per_chunk, t1 = min(N, t0 + rows_per_chunk);
    if (cg * 8 < d) {
        int t = t0 + r;
        for (; t + 48 < t1; t += 64) {                       // four rows in flight per thread
            v4i raw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) raw[u] = *(const v4i*)(base + (int64_t)(t + 16 * u) * x.sN);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint16_t* e = (const uint16_t*)&raw[u];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] += (double)load_half<IS_F16>(e + k);
            }
        }
        for (; t < t1; t += 16) {
            v4i raw = *(const v4i*)(base + (int64_t)t * x.sN);
            const uint16_t* e = (const uint16_t*)&raw;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += (double)load_half<IS_F16>(e + k);
        }
    }
    __shared__ double red[16][128];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (cg * 8 + k < d) red[r][cg * 8 + k] = acc[k];
    __syncthreads();
    if (threadIdx.x < d) {
        double sum = 0.0;
        for (int rr = 0; rr < 16; ++rr) sum += red[rr][threadIdx.x];
        part[((int64_t)bh * nchunks + chunk) * d + threadIdx.x] = sum;
    }
}

// ------------------------------------------------------------ INT8 token blocks
// grid BH * (N / blk); 256 threads; the block (blk x d) is held in registers:
// each thread owns NG groups of 8 consecutive elements (NG = blk*d/2048),
// always at the same 8 channels.  With `part` the K-smoothing mean is
// finalised here from the fp64 partial token sums, mu = fp32(S/N - eps), and
// the first block of each head writes it to `mu_out`.
template <bool IS_F16, int NG>
__global__ __launch_bounds__(256) void quant_i8_tokblock_kernel(Dense x, int H, int N, int d, int blk,
                                                                 const double* __restrict__ part, int nchunks,
                                                                 double eps, float* __restrict__ mu_out,
                                                                 int8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
    const int nb = N / blk;
    const int bh = blockIdx.x / nb, ib = blockIdx.x % nb;
    const int b = bh / H, h = bh % H;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH;
    const int gpr = d / 8;                               // groups per token row
    const int c0 = (threadIdx.x % gpr) * 8;              // this thread's channels (256 % gpr == 0)
    __shared__ float mu_s[128];
    __shared__ float wmax[4];
    v4i raw[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int g = threadIdx.x + k * 256;
        raw[k] = *(const v4i*)(base + (int64_t)(ib * blk + g / gpr) * x.sN + c0);
    }
    float mu[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (part) {
        if ((int)threadIdx.x < d) {
            double sum = 0.0;
            for (int k = 0; k < nchunks; ++k) sum += part[((int64_t)bh * nchunks + k) * d + threadIdx.x];
            const float m = (float)(sum / (double)N - eps);
            mu_s[threadIdx.x] = m;
            if (ib == 0 && mu_out) mu_out[(int64_t)bh * d + threadIdx.x] = m;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) mu[j] = mu_s[c0 + j];
    }
    float v[NG][8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const uint16_t* e = (const uint16_t*)&raw[k];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float f = load_half<IS_F16>(e + j);
            if (part) f = f - mu[j];
            v[k][j] = f;
            amax = __builtin_fmaxf(amax, __builtin_fabsf(f));
        }
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    float scale = amax / 127.0f;
    if (!(amax > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
    if (threadIdx.x == 0) scales[(int64_t)bh * nb + ib] = scale;
    int8_t* out = codes + ((int64_t)bh * N + (int64_t)ib * blk) * d;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int g = threadIdx.x + k * 256;
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w0 |= ((uint32_t)(enc_i8(v[k][j], inv) & 0xFF)) << (8 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) w1 |= ((uint32_t)(enc_i8(v[k][4 + j], inv) & 0xFF)) << (8 * j);
        *(uint2*)(out + (int64_t)g * 8) = make_uint2(w0, w1);
    }
}

// ------------------------------------------------------------ per-channel V
// pass 1: grid (BH, chunks): per-channel absmax of a token chunk.
template <bool IS_F16>
__global__ __launch_bounds__(256) void chan_amax_partial_kernel(Dense x, int H, int N, int d, int rows_per_chunk,
                                                                 float* __restrict__ part) {
    const int bh = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
    const int b = bh / H, h = bh % H;
    const int cg = threadIdx.x % 16, r = threadIdx.x / 16;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH + cg * 8;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int t0 = chunk * rows_per_chunk, t1 = min(N, t0 + rows_per_chunk);
    if (cg * 8 < d) {
        int t = t0 + r;
        for (; t + 48 < t1; t += 64) {
            v4i raw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) raw[u] = *(const v4i*)(base + (int64_t)(t + 16 * u) * x.sN);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint16_t* e = (const uint16_t*)&raw[u];
#pragma unroll
                for (int k = 0; k < 8; ++k) m[k] = __builtin_fmaxf(m[k], __builtin_fabsf(load_half<IS_F16>(e + k)));
            }
        }
        for (; t < t1; t += 16) {
            v4i raw = *(const v4i*)(base + (int64_t)t * x.sN);
            const uint16_t* e = (const uint16_t*)&raw;
#pragma unroll
            for (int k = 0; k < 8; ++k) m[k] = __builtin_fmaxf(m[k], __builtin_fabsf(load_half<IS_F16>(e + k)));
        }
    }
    __shared__ float red[16][128];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (cg * 8 + k < d) red[r][cg * 8 + k] = m[k];
    __syncthreads();
    if (threadIdx.x < d) {
        float mm = 0.0f;
        for (int rr = 0; rr < 16; ++rr) mm = __builtin_fmaxf(mm, red[rr][threadIdx.x]);
        part[((int64_t)bh * nchunks + chunk) * d + threadIdx.x] = mm;
    }
}

// pass 2: grid (BH, N / 64): encode 64 tokens of every channel, channel-major
// output; block (bh, 0) also writes the scales.  FMT 0: int8, 1: e4m3
// (hardware nearest-even conversion after clamping to +-448, i.e. saturating).
// Thread t owns 4 tokens x 8 channels; codes are transposed through LDS as
// 32-bit words (4 tokens of one channel) and written as 16-byte row chunks.
template <bool IS_F16, int FMT>
__global__ __launch_bounds__(256) void chan_encode_kernel(Dense x, int H, int N, int d,
                                                          const float* __restrict__ part, int nchunks,
                                                          uint8_t* __restrict__ codes_t,
                                                          float* __restrict__ scales) {
    const int bh = blockIdx.x, tb = blockIdx.y;
    const int b = bh / H, h = bh % H;
    __shared__ float inv_s[128];
    __shared__ uint32_t tile[128][16 + 1];
    if ((int)threadIdx.x < d) {
        float amax = 0.0f;
        for (int k = 0; k < nchunks; ++k)
            amax = __builtin_fmaxf(amax, part[((int64_t)bh * nchunks + k) * d + threadIdx.x]);
        const float top = FMT == 0 ? 127.0f : 448.0f;
        float inv = amax > 0.0f ? top / amax : 0.0f;
        float scale = amax / top;
        if (!(amax > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
        inv_s[threadIdx.x] = inv;
        if (tb == 0) scales[(int64_t)bh * d + threadIdx.x] = scale;
    }
    __syncthreads();
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH;
    const int gpr = d / 8;                                 // channel groups
    const int tpg = 256 / gpr;                             // threads per channel group
    const int c0 = (threadIdx.x % gpr) * 8;
    const int q = threadIdx.x / gpr;                       // token quad index (64/4 = 16 quads)
    for (int tq = q; tq < 16; tq += tpg) {
        v4i raw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[u] = *(const v4i*)(base + (int64_t)(tb * 64 + 4 * tq + u) * x.sN + c0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t word = 0;
            const float iv = inv_s[c0 + j];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = load_half<IS_F16>((const uint16_t*)&raw[u] + j) * iv;
                uint32_t code;
                if constexpr (FMT == 0) code = (uint32_t)(enc_i8(f, 1.0f) & 0xFF);
                else code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(f, -448.0f, 448.0f), 0.0f, 0, false) & 0xFFu;
                word |= code << (8 * u);
            }
            tile[c0 + j][tq] = word;
        }
    }
    __syncthreads();
    for (int qq = threadIdx.x; qq < d * 4; qq += 256) {
        const int c = qq / 4, p16 = qq % 4;
        *(uint4*)(codes_t + ((int64_t)bh * d + c) * N + tb * 64 + p16 * 16) =
            make_uint4(tile[c][4 * p16], tile[c][4 * p16 + 1], tile[c][4 * p16 + 2], tile[c][4 * p16 + 3]);
    }
}

// ------------------------------------------------------------ MXFP4
// Encode 32 values (already loaded) as one MX block; returns the E8M0 byte.
__device__ __forceinline__ uint32_t mx_encode32(const float* v, uint32_t* packed /* 4 words */) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[k]));
    const int e = mx_exponent(amax);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) word |= enc_e2m1(__builtin_ldexpf(v[w * 8 + k], -e)) << (4 * k);
        packed[w] = word;
    }
    return (uint32_t)(e + 127);
}

// Rows (Q, K): grid BH * ceil(N / 128); thread handles (token, 32-channel
// block) items; optional fp32 means over each 128-token block (over the
// tokens present when the last block is short, e.g. a single decode query).
template <bool IS_F16>
__global__ __launch_bounds__(256) void mx_rows_kernel(Dense x, int H, int N, int d, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, float* __restrict__ means) {
    const int nt = (N + 127) / 128;
    const int bh = blockIdx.x / nt, tb = blockIdx.x % nt;
    const int b = bh / H, h = bh % H;
    const int rows = min(128, N - tb * 128);
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH;
    const int nblk = d / 32;
    for (int it = threadIdx.x; it < rows * nblk; it += 256) {
        const int t = tb * 128 + it / nblk, g = it % nblk;
        float v[32];
        const uint16_t* row = base + (int64_t)t * x.sN + g * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint4 raw = *(const uint4*)(row + q * 8);
            const uint16_t* e = (const uint16_t*)&raw;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[q * 8 + j] = load_half<IS_F16>(e + j);
        }
        uint32_t packed[4];
        uint32_t s = mx_encode32(v, packed);
        *(uint4*)(codes + ((int64_t)bh * N + t) * (d / 2) + g * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        scales[((int64_t)bh * N + t) * nblk + g] = (uint8_t)s;
    }
    if (means) {
        // one thread per channel sums the block's tokens in fp64 (exact for bf16 inputs)
        for (int c = threadIdx.x; c < d; c += 256) {
            double s = 0.0;
            for (int t = 0; t < rows; ++t) s += (double)load_half<IS_F16>(base + (int64_t)(tb * 128 + t) * x.sN + c);
            means[((int64_t)bh * nt + tb) * d + c] = (float)(s / (double)rows);
        }
    }
}

// Columns (V): grid BH * (N / 128); the 128 x d tile is staged in LDS, then a
// thread encodes (channel, 32-token group) items into channel-major codes.
template <bool IS_F16>
__global__ __launch_bounds__(256) void mx_cols_kernel(Dense x, int H, int N, int d, uint8_t* __restrict__ codes_t,
                                                       uint8_t* __restrict__ scales_t) {
    const int nt = N / 128;
    const int bh = blockIdx.x / nt, tb = blockIdx.x % nt;
    const int b = bh / H, h = bh % H;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH;
    __shared__ float tile[128][129];
    const int gpr = d / 8;
    for (int g = threadIdx.x; g < 128 * gpr; g += 256) {
        const int t = g / gpr, c = (g % gpr) * 8;
        uint4 raw = *(const uint4*)(base + (int64_t)(tb * 128 + t) * x.sN + c);
        const uint16_t* e = (const uint16_t*)&raw;
#pragma unroll
        for (int j = 0; j < 8; ++j) tile[t][c + j] = load_half<IS_F16>(e + j);
    }
    __syncthreads();
    for (int it = threadIdx.x; it < d * 4; it += 256) {
        const int c = it / 4, grp = it % 4;
        float v[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) v[k] = tile[grp * 32 + k][c];
        uint32_t packed[4];
        uint32_t s = mx_encode32(v, packed);
        const int64_t tok = (int64_t)tb * 128 + grp * 32;
        *(uint4*)(codes_t + ((int64_t)bh * d + c) * (N / 2) + tok / 2) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        scales_t[((int64_t)bh * d + c) * (N / 32) + tok / 32] = (uint8_t)s;
    }
}

// ------------------------------------------------------------ launchers
static int chunks_for(int BH, int N) {
    // enough blocks to fill the chip (~2 per CU), at least 256 rows per chunk
    int want = (512 + BH - 1) / BH;
    int maxc = (N + 255) / 256;
    int c = want < maxc ? want : maxc;
    return c < 1 ? 1 : c;
}

size_t ws_kmean_bytes(int BH, int N, int d) { return (size_t)BH * chunks_for(BH, N) * d * sizeof(double); }
size_t ws_chan_bytes(int BH, int N, int d) { return (size_t)BH * chunks_for(BH, N) * d * sizeof(float); }

template <bool F16>
static hipError_t launch_tokblock_t(const Dense& x, int B, int H, int N, int d, int blk, const double* part,
                                    int nch, double eps, float* mu, int8_t* codes, float* scales, hipStream_t st) {
    const int grid = B * H * (N / blk);
    const int ng = blk * d / 2048;
    switch (ng) {
        case 2: quant_i8_tokblock_kernel<F16, 2><<<grid, 256, 0, st>>>(x, H, N, d, blk, part, nch, eps, mu, codes, scales); break;
        case 4: quant_i8_tokblock_kernel<F16, 4><<<grid, 256, 0, st>>>(x, H, N, d, blk, part, nch, eps, mu, codes, scales); break;
        default: quant_i8_tokblock_kernel<F16, 8><<<grid, 256, 0, st>>>(x, H, N, d, blk, part, nch, eps, mu, codes, scales); break;
    }
    return hipGetLastError();
}

// INT8 token blocks; with smoothing (mu != null) the K token sums go to the
// workspace first and the quantiser finalises the mean.
hipError_t launch_quant_i8_tokblock(const Dense& x, bool f16, int B, int H, int N, int d, int blk, bool smooth,
                                    double eps, float* mu, void* ws, int8_t* codes, float* scales,
                                    hipStream_t st) {
    const int BH = B * H, nch = chunks_for(BH, N), rpc = (N + nch - 1) / nch;
    double* part = nullptr;
    if (smooth) {
        part = (double*)ws;
        if (f16) ksum_partial_kernel<true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
        else ksum_partial_kernel<false><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    }
    return f16 ? launch_tokblock_t<true>(x, B, H, N, d, blk, part, nch, eps, mu, codes, scales, st)
               : launch_tokblock_t<false>(x, B, H, N, d, blk, part, nch, eps, mu, codes, scales, st);
}

hipError_t launch_quant_chan(const Dense& x, bool f16, int B, int H, int N, int d, int fmt, uint8_t* codes_t,
                             float* scales, void* ws, hipStream_t st) {
    const int BH = B * H, nch = chunks_for(BH, N), rpc = (N + nch - 1) / nch;
    float* part = (float*)ws;
    if (f16) chan_amax_partial_kernel<true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    else chan_amax_partial_kernel<false><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    dim3 g(BH, N / 64);
    if (fmt == 0) {
        if (f16) chan_encode_kernel<true, 0><<<g, 256, 0, st>>>(x, H, N, d, part, nch, codes_t, scales);
        else chan_encode_kernel<false, 0><<<g, 256, 0, st>>>(x, H, N, d, part, nch, codes_t, scales);
    } else {
        if (f16) chan_encode_kernel<true, 1><<<g, 256, 0, st>>>(x, H, N, d, part, nch, codes_t, scales);
        else chan_encode_kernel<false, 1><<<g, 256, 0, st>>>(x, H, N, d, part, nch, codes_t, scales);
    }
    return hipGetLastError();
}

hipError_t launch_quant_mx(const Dense& x, bool f16, int B, int H, int N, int d, int axis, uint8_t* codes,
                           uint8_t* scales, float* means, hipStream_t st) {
    const int grid = B * H * ((N + 127) / 128);
    if (axis == 0) {
        if (f16) mx_rows_kernel<true><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means);
        else mx_rows_kernel<false><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means);
    } else {
        if (f16) mx_cols_kernel<true><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales);
        else mx_cols_kernel<false><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales);
    }
    return hipGetLastError();
}

}  // namespace bqa
