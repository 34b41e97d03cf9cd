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
#include <atomic>
#include <chrono>
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace bqa {

// QK-norm ("SageBwd", Methodology 4) of one 128-channel row whose 16 groups
// of 8 channels sit in 16 consecutive lanes: S = sum of squares in fp64
// (exact for bf16 rows, so the lane order does not matter), r =
// fp32(1/sqrt(S)) (0 for a zero row), and the 8 values of this lane become
// bf16(fp32(x r)).  Returns r.
__device__ __forceinline__ float qk_norm8(float* v) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += (double)v[j] * (double)v[j];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off, 16);
    const float r = s > 0.0 ? (float)(1.0 / __builtin_sqrt(s)) : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = bf16_bits_to_f32(f32_to_bf16_bits(v[j] * r));
    return r;
}

// ------------------------------------------------------------ column partials
// grid (BH, chunks); 256 threads = 16 rows x 16 column groups of 8 channels.
// Each chunk of tokens is reduced per channel into part[bh][chunk][c]: SUM
// gives fp64 token sums (K smoothing), otherwise fp32 absolute maxima
// (per-channel V scales).  NORM (with SUM, d = 128): the sums are of the
// QK-normalised rows.
template <bool IS_F16, bool SUM, bool NORM = false>
__device__ __forceinline__ void col_partial_body(const Dense& x, int H, int N, int d, int rows_per_chunk,
                                                 void* __restrict__ part_out, int bh, int chunk, int nchunks) {
    using Acc = typename std::conditional<SUM, double, float>::type;
    const int b = bh / H, h = bh % H;
    const int cg = threadIdx.x % 16, r = threadIdx.x / 16;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH + cg * 8;
    Acc acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto take = [&](const v4i& raw) {
        const uint16_t* e = (const uint16_t*)&raw;
        float f[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = load_half<IS_F16>(e + k);
        if constexpr (NORM) qk_norm8(f);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (SUM) acc[k] += (double)f[k];
            else acc[k] = __builtin_fmaxf(acc[k], __builtin_fabsf(f[k]));
        }
    };
    const int t0 = chunk * rows_per_chunk, t1 = min(N, t0 + rows_per_chunk);
    if (cg * 8 < d) {
        // four rows in flight per thread (measured: two are too few for
        // 512-row chunks, eight or more slow the maxima down)
        int t = t0 + r;
        for (; t + 48 < t1; t += 64) {
            v4i raw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) raw[u] = *(const v4i*)(base + (int64_t)(t + 16 * u) * x.sN);
#pragma unroll
            for (int u = 0; u < 4; ++u) take(raw[u]);
        }
        for (; t < t1; t += 16) take(*(const v4i*)(base + (int64_t)t * x.sN));
    }
    __shared__ Acc red[16][128];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (cg * 8 + k < d) red[r][cg * 8 + k] = acc[k];
    __syncthreads();
    if ((int)threadIdx.x < d) {
        Acc v = red[0][threadIdx.x];
        for (int rr = 1; rr < 16; ++rr) {
            if constexpr (SUM) v += red[rr][threadIdx.x];
            else v = __builtin_fmaxf(v, red[rr][threadIdx.x]);
        }
        ((Acc*)part_out)[((int64_t)bh * nchunks + chunk) * d + threadIdx.x] = v;
    }
}

template <bool IS_F16, bool SUM, bool NORM = false>
__global__ __launch_bounds__(256) void col_partial_kernel(Dense x, int H, int N, int d, int rows_per_chunk,
                                                          void* __restrict__ part_out) {
    col_partial_body<IS_F16, SUM, NORM>(x, H, N, d, rows_per_chunk, part_out, blockIdx.x, blockIdx.y, gridDim.y);
}

// Per-chunk partials of one channel (stride d between chunks), combined in
// two steps so that the first eight loads can be issued ahead of the bulk
// loads of the consumer and overlap them.  Sums are exact here (fp64 sums of
// bf16/fp16 values) and maxima are order-free, so the grouping is free.
template <class Acc>
struct PartLoad {
    Acc t[8];
    __device__ __forceinline__ void issue(const Acc* p, int n, int d) {
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = u < n ? p[(int64_t)u * d] : Acc(0);
    }
    template <bool SUM>
    __device__ __forceinline__ Acc combine(Acc v) const {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if constexpr (SUM) v += t[u];
            else v = __builtin_fmaxf(v, t[u]);
        }
        return v;
    }
    template <bool SUM>
    __device__ __forceinline__ Acc finish(const Acc* p, int n, int d) const {
        Acc v = combine<SUM>(Acc(0));
        for (int k = 8; k < n; k += 8) {                 // further chunks, eight loads at a time
            PartLoad more;
            more.issue(p + (int64_t)k * d, n - k, d);
            v = more.combine<SUM>(v);
        }
        return v;
    }
};

// ------------------------------------------------------------ INT8 token blocks
// grid BH * (N / blk); 256 threads; the blk x d block is held in registers:
// each thread owns NG groups of 8 consecutive elements (NG = blk d / 2048),
// always at the same 8 channels.  With `part` the K-smoothing mean is
// finalised here from the fp64 partial token sums, mu = fp32(S/N - eps), and
// block 0 of each head writes it to `mu_out`.  NORM (d = 128): every row is
// QK-normalised first (qk_norm8) and its inverse norm written to inv_norm.
template <bool IS_F16, int NG, bool NORM = false>
__device__ __forceinline__ void tokblock_body(const Dense& x, int H, int N, int d, int blk,
                                              const double* __restrict__ part, int nchunks, double eps,
                                              float* __restrict__ mu_out, int8_t* __restrict__ codes,
                                              float* __restrict__ scales, int block_id,
                                              float* __restrict__ inv_norm = nullptr) {
    const int nb = N / blk;
    const int bh = block_id / nb, ib = block_id % nb;
    const int b = bh / H, h = bh % H;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH + (int64_t)ib * blk * x.sN;
    const int gpr = d / 8;                               // groups per token row
    const int c0 = (threadIdx.x % gpr) * 8;              // this thread's channels (256 % gpr == 0)
    __shared__ float mu_s[128];
    __shared__ float wmax[4];
    const bool has_mu = part != nullptr;
    const bool fin = has_mu && (int)threadIdx.x < d;
    const double* pch = part + (int64_t)bh * nchunks * d + threadIdx.x;
    PartLoad<double> pl;
    if (fin) pl.issue(pch, nchunks, d);
    v4i raw[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int g = threadIdx.x + k * 256;
        raw[k] = *(const v4i*)(base + (int64_t)(g / gpr) * x.sN + c0);
    }
    float mu[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (has_mu) {
        if (fin) {
            const float m = (float)(pl.finish<true>(pch, nchunks, d) / (double)N - eps);
            mu_s[threadIdx.x] = m;
            if (ib == 0 && mu_out) mu_out[(int64_t)bh * d + threadIdx.x] = m;
        }
        // LDS writes done; the bulk loads above stay in flight across the barrier
        __builtin_amdgcn_s_waitcnt(0xC07F);
        barrier_only();
#pragma unroll
        for (int j = 0; j < 8; ++j) mu[j] = mu_s[c0 + j];
    }
    float v[NG][8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const uint16_t* e = (const uint16_t*)&raw[k];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[k][j] = load_half<IS_F16>(e + j);
        if constexpr (NORM) {
            const float r = qk_norm8(v[k]);
            if (threadIdx.x % gpr == 0)
                inv_norm[(int64_t)bh * N + (int64_t)ib * blk + (threadIdx.x + k * 256) / gpr] = r;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (has_mu) v[k][j] = v[k][j] - mu[j];
            amax = __builtin_fmaxf(amax, __builtin_fabsf(v[k][j]));
        }
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    const float am = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    float inv = am > 0.0f ? 127.0f / am : 0.0f;
    float scale = am / 127.0f;
    if (!(am > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
    if (threadIdx.x == 0) scales[(int64_t)bh * nb + ib] = scale;
    int8_t* out = codes + ((int64_t)bh * N + (int64_t)ib * blk) * d;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int g = threadIdx.x + k * 256;
        // |v| <= am, so |v * inv| <= 127
        const uint32_t w0 = (uint32_t)q8x4(v[k][0], v[k][1], v[k][2], v[k][3], inv);
        const uint32_t w1 = (uint32_t)q8x4(v[k][4], v[k][5], v[k][6], v[k][7], inv);
        *(uint2*)(out + (int64_t)g * 8) = make_uint2(w0, w1);
    }
}

template <bool IS_F16, int NG, bool NORM = false>
__global__ __launch_bounds__(256) void quant_i8_tokblock_kernel(Dense x, int H, int N, int d, int blk,
                                                                 const double* __restrict__ part, int nchunks,
                                                                 double eps, float* __restrict__ mu_out,
                                                                 int8_t* __restrict__ codes,
                                                                 float* __restrict__ scales,
                                                                 float* __restrict__ inv_norm = nullptr) {
    tokblock_body<IS_F16, NG, NORM>(x, H, N, d, blk, part, nchunks, eps, mu_out, codes, scales, blockIdx.x,
                                    inv_norm);
}

// ------------------------------------------------------------ per-channel V
// pass 2: grid (BH, N / TT): encode TT tokens of every channel into
// channel-major codes; block (bh, 0) also writes the scales.  FMT 0: int8,
// 1: e4m3 (hardware nearest-even conversion after clamping to +-448, i.e.
// saturating).  Thread t owns quads of 4 tokens x 8 channels; codes are
// transposed through LDS as 32-bit words (4 tokens of one channel) and written
// as 16-byte chunks, TT bytes contiguous per channel.
template <bool IS_F16, int FMT, int TT>
__device__ __forceinline__ void chan_encode_body(const Dense& x, int H, int N, int d, const float* __restrict__ part,
                                                 int nchunks, uint8_t* __restrict__ codes_t,
                                                 float* __restrict__ scales, int bh, int tb) {
    constexpr int NQ = TT / 4;                             // token quads per tile
    const int b = bh / H, h = bh % H;
    __shared__ float inv_s[128];
    __shared__ uint32_t tile[128][NQ + 1];
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH;
    const int gpr = d / 8;                                 // channel groups
    const int tpg = 256 / gpr;                             // threads per channel group
    const int c0 = (threadIdx.x % gpr) * 8;
    const int q = threadIdx.x / gpr;
    constexpr int MAXQ = NQ * 16 / 256;                    // quads per thread at d = 128, the most (d <= 128)
    const bool fin = (int)threadIdx.x < d;
    const float* pch = part + (int64_t)bh * nchunks * d + threadIdx.x;
    PartLoad<float> pl;
    if (fin) pl.issue(pch, nchunks, d);
    v4i raw[MAXQ][4];
#pragma unroll
    for (int i = 0; i < MAXQ; ++i) {
        const int tq = q + i * tpg;
        if (tq < NQ) {
#pragma unroll
            for (int u = 0; u < 4; ++u) raw[i][u] = *(const v4i*)(base + (int64_t)(tb * TT + 4 * tq + u) * x.sN + c0);
        }
    }
    if (fin) {
        const float amax = pl.finish<false>(pch, nchunks, d);
        const float top = FMT == 0 ? 127.0f : 448.0f;
        float inv = amax > 0.0f ? top / amax : 0.0f;
        float scale = amax / top;
        if (!(amax > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
        inv_s[threadIdx.x] = inv;
        if (tb == 0) scales[(int64_t)bh * d + threadIdx.x] = scale;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // LDS writes done; bulk loads stay in flight
    barrier_only();
#pragma unroll
    for (int i = 0; i < MAXQ; ++i) {
        const int tq = q + i * tpg;
        if (tq < NQ) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float iv = inv_s[c0 + j];
                float f[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) f[u] = load_half<IS_F16>((const uint16_t*)&raw[i][u] + j) * iv;
                uint32_t word;
                if constexpr (FMT == 0) {
                    // |x| <= the channel's absmax, so |f| <= 127
                    word = (uint32_t)q8x4(f[0], f[1], f[2], f[3], 1.0f);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) f[u] = __builtin_amdgcn_fmed3f(f[u], -448.0f, 448.0f);
                    word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
                    word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], (int)word, true);
                }
                tile[c0 + j][tq] = word;
            }
        }
    }
    __syncthreads();
    for (int qq = threadIdx.x; qq < d * (TT / 16); qq += 256) {
        const int c = qq / (TT / 16), p16 = qq % (TT / 16);
        *(uint4*)(codes_t + ((int64_t)bh * d + c) * N + tb * TT + p16 * 16) =
            make_uint4(tile[c][4 * p16], tile[c][4 * p16 + 1], tile[c][4 * p16 + 2], tile[c][4 * p16 + 3]);
    }
}

template <bool IS_F16, int FMT, int TT>
__global__ __launch_bounds__(256) void chan_encode_kernel(Dense x, int H, int N, int d,
                                                          const float* __restrict__ part, int nchunks,
                                                          uint8_t* __restrict__ codes_t,
                                                          float* __restrict__ scales) {
    chan_encode_body<IS_F16, FMT, TT>(x, H, N, d, part, nchunks, codes_t, scales, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------ K and V together
// The same work as the K and V kernels above in two launches instead of four:
// the first takes the K token sums (with smoothing) and the V channel maxima,
// the second the K token blocks and the V codes; each workgroup picks its job
// from its index (K jobs first).
struct KvJob {
    Dense k, v;
    int H, N, d, nch, rpc;
    bool smooth;
    double eps;
    double* kpart; float* vpart;
    float* mu; int8_t* kc; float* ks; uint8_t* vc; float* vs;
};

template <bool IS_F16>
__global__ __launch_bounds__(256) void kv_partial_kernel(KvJob j, int nk) {
    const int id = blockIdx.x;
    if (id < nk) col_partial_body<IS_F16, true>(j.k, j.H, j.N, j.d, j.rpc, j.kpart, id / j.nch, id % j.nch, j.nch);
    else col_partial_body<IS_F16, false>(j.v, j.H, j.N, j.d, j.rpc, j.vpart, (id - nk) / j.nch, (id - nk) % j.nch, j.nch);
}

template <bool IS_F16, int FMT, int TT, int NG>
__global__ __launch_bounds__(256) void kv_encode_kernel(KvJob j, int nk) {
    const int id = blockIdx.x;
    if (id < nk) {
        tokblock_body<IS_F16, NG>(j.k, j.H, j.N, j.d, 64, j.smooth ? j.kpart : nullptr, j.nch, j.eps, j.mu, j.kc, j.ks, id);
    } else {
        const int nt = j.N / TT;
        chan_encode_body<IS_F16, FMT, TT>(j.v, j.H, j.N, j.d, j.vpart, j.nch, j.vc, j.vs, (id - nk) / nt, (id - nk) % nt);
    }
}

// ------------------------------------------------------------ K and V resident
// One launch for the same work when every workgroup of the grid can be
// resident at once (d = 128, N a multiple of 256): a workgroup loads 256
// tokens of one head, K and V (64 KB each), into registers, publishes its
// partials (K token sums in fp64, V channel maxima), waits until the other
// workgroups of its head have published theirs, and encodes from registers,
// so K and V cross HBM once instead of twice.  The outputs are bit for bit
// those of the two launches above: the fp64 sums are exact and maxima are
// order-free, so neither depends on how the tokens are grouped.
//
// Workgroups of a head meet through flags in the workspace: each publishes
// its partials, then writes the call's tag (a 64-bit value the host draws
// fresh for every call) into its own flag, and waits until every flag of its
// head holds the tag.  Whatever an earlier call or another operation left in
// the workspace differs from a fresh tag, so nothing needs clearing.  The
// host launches this kernel only when the whole grid fits on the device at
// once and the stream is not being captured (a captured tag would repeat on
// every replay); should a wait still run past its limit (other work holding
// compute units), the workgroup takes the statistics of its head from HBM
// itself, which gives the same values.
constexpr int RES_T = 256;

template <bool IS_F16, int FMT>
__global__ __launch_bounds__(256, 2) void kv_resident_kernel(KvJob j, uint64_t* __restrict__ flags,
                                                             int flag_stride, uint64_t tag, uint32_t spin_limit) {
    constexpr int D = 128;
    const int nch = j.N / RES_T;
    const int bh = blockIdx.x / nch, ch = blockIdx.x % nch;
    const int b = bh / j.H, h = bh % j.H;
    const int tid = threadIdx.x, r = tid >> 4, c0 = (tid & 15) * 8;
    const int t0 = ch * RES_T;
    const uint16_t* kbase = (const uint16_t*)j.k.p + b * j.k.sB + h * j.k.sH + c0;
    const uint16_t* vbase = (const uint16_t*)j.v.p + b * j.v.sB + h * j.v.sH + c0;
    // K: token block kb (64 tokens, the scale blocks), group g: token 64 kb + 16 g + r
    // V: 128-token tile vt, quad i, token 4 (r + 16 i) + u of the tile
    v4i kr[4][4], vr[2][2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) kr[kb][g] = *(const v4i*)(kbase + (int64_t)(t0 + 64 * kb + 16 * g + r) * j.k.sN);
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                vr[vt][i][u] = *(const v4i*)(vbase + (int64_t)(t0 + 128 * vt + 4 * (r + 16 * i) + u) * j.v.sN);

    __shared__ double red_k[16][D];
    __shared__ float red_v[16][D];
    __shared__ float mu_s[D], inv_s[D], wmax[4][4];
    __shared__ uint32_t tile[2][D][33];
    __shared__ int late;

    // ---- partials of this workgroup's 256 tokens
    {
        double sk[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        float mv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (j.smooth) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 8; ++e) sk[e] += (double)load_half<IS_F16>((const uint16_t*)&kr[kb][g] + e);
        }
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        mv[e] = __builtin_fmaxf(mv[e], __builtin_fabsf(load_half<IS_F16>((const uint16_t*)&vr[vt][i][u] + e)));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red_k[r][c0 + e] = sk[e];
            red_v[r][c0 + e] = mv[e];
        }
    }
    // the conversions are made again when encoding: holding the 256 converted
    // values across the wait would spill, the 128 packed ones fit
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) asm volatile("" : "+v"(kr[kb][g]));
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(vr[vt][i][u]));
    __syncthreads();
    if (tid < D) {
        double s = red_k[0][tid];
        float m = red_v[0][tid];
        for (int rr = 1; rr < 16; ++rr) {
            s += red_k[rr][tid];
            m = __builtin_fmaxf(m, red_v[rr][tid]);
        }
        // device-scope stores go through to where every XCD reads them; the
        // wait completes them before the flag is written.  (Partials and
        // flags use device-scope accesses only, so no cache-wide write-back
        // or invalidation is needed.)
        if (j.smooth)
            __hip_atomic_store((uint64_t*)j.kpart + ((int64_t)bh * nch + ch) * D + tid, __builtin_bit_cast(uint64_t, s),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store((uint32_t*)j.vpart + ((int64_t)bh * nch + ch) * D + tid, __builtin_bit_cast(uint32_t, m),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    uint64_t* hflags = flags + (int64_t)bh * flag_stride;   // this head's flags, one per workgroup
    if (tid == 0) __hip_atomic_store(hflags + ch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 64) {
        // wavefront 0 watches the head's flags (device-scope loads, so never
        // a stale cached copy)
        uint32_t n = 0;
        int timed_out = 0;
        for (;;) {
            bool mine = true;
            for (int c = tid; c < nch; c += 64)
                mine = mine && __hip_atomic_load(hflags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
            if (__all(mine)) break;
            if (++n >= spin_limit) {
                timed_out = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(32);
        }
        if (tid == 0) late = timed_out;
    }
    __syncthreads();
    const bool own = late != 0;

    // ---- the head's statistics: K mean and V channel scales
    if (own) {
        // the head's tokens read again from HBM by this workgroup alone
        double sk[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        float mv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int t = r; t < j.N; t += 16) {
            const v4i kx = *(const v4i*)(kbase + (int64_t)t * j.k.sN);
            const v4i vx = *(const v4i*)(vbase + (int64_t)t * j.v.sN);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (j.smooth) sk[e] += (double)load_half<IS_F16>((const uint16_t*)&kx + e);
                mv[e] = __builtin_fmaxf(mv[e], __builtin_fabsf(load_half<IS_F16>((const uint16_t*)&vx + e)));
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red_k[r][c0 + e] = sk[e];
            red_v[r][c0 + e] = mv[e];
        }
        __syncthreads();
    }
    if (tid < D) {
        double s = 0.0;
        float amax = 0.0f;
        if (own) {
            s = red_k[0][tid];
            amax = red_v[0][tid];
            for (int rr = 1; rr < 16; ++rr) {
                s += red_k[rr][tid];
                amax = __builtin_fmaxf(amax, red_v[rr][tid]);
            }
        } else {
            // device-scope loads: never a stale line of an earlier call
            const uint64_t* pk = (const uint64_t*)j.kpart + (int64_t)bh * nch * D + tid;
            const uint32_t* pv = (const uint32_t*)j.vpart + (int64_t)bh * nch * D + tid;
            for (int c = 0; c < nch; c += 8) {
                uint64_t tk[8];
                uint32_t tv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const bool in = c + u < nch;
                    tk[u] = j.smooth && in ? __hip_atomic_load((uint64_t*)pk + (int64_t)(c + u) * D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
                    tv[u] = in ? __hip_atomic_load((uint32_t*)pv + (int64_t)(c + u) * D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    s += __builtin_bit_cast(double, tk[u]);
                    amax = __builtin_fmaxf(amax, __builtin_bit_cast(float, tv[u]));
                }
            }
        }
        if (j.smooth) {
            const float m = (float)(s / (double)j.N - j.eps);
            mu_s[tid] = m;
            if (ch == 0 && j.mu) j.mu[(int64_t)bh * D + tid] = m;
        }
        const float top = FMT == 0 ? 127.0f : 448.0f;
        float inv = amax > 0.0f ? top / amax : 0.0f;
        float scale = amax / top;
        if (!(amax > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
        inv_s[tid] = inv;
        if (ch == 0) j.vs[(int64_t)bh * D + tid] = scale;
    }
    __syncthreads();

    // ---- K: INT8 per 64-token block, as tokblock_body
    float mu[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = j.smooth ? mu_s[c0 + e] : 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        float am = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float f = load_half<IS_F16>((const uint16_t*)&kr[kb][g] + e);
                if (j.smooth) f = f - mu[e];
                am = __builtin_fmaxf(am, __builtin_fabsf(f));
            }
        am = wave_max(am);
        if ((tid & 63) == 0) wmax[kb][tid >> 6] = am;
    }
    __syncthreads();
    const int nb = j.N / 64;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const float am = __builtin_fmaxf(__builtin_fmaxf(wmax[kb][0], wmax[kb][1]), __builtin_fmaxf(wmax[kb][2], wmax[kb][3]));
        float inv = am > 0.0f ? 127.0f / am : 0.0f;
        float scale = am / 127.0f;
        if (!(am > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
        const int ib = t0 / 64 + kb;
        if (tid == 0) j.ks[(int64_t)bh * nb + ib] = scale;
        int8_t* out = j.kc + ((int64_t)bh * j.N + (int64_t)ib * 64) * D;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                f[e] = load_half<IS_F16>((const uint16_t*)&kr[kb][g] + e);
                if (j.smooth) f[e] = f[e] - mu[e];
            }
            // |f| <= am, so |f * inv| <= 127
            const uint32_t w0 = (uint32_t)q8x4(f[0], f[1], f[2], f[3], inv);
            const uint32_t w1 = (uint32_t)q8x4(f[4], f[5], f[6], f[7], inv);
            *(uint2*)(out + (int64_t)(16 * g + r) * D + c0) = make_uint2(w0, w1);
        }
    }

    // ---- V: per-channel codes, channel-major, as chan_encode_body (128-token tiles)
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tq = r + 16 * i;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float iv = inv_s[c0 + e];
                float f[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) f[u] = load_half<IS_F16>((const uint16_t*)&vr[vt][i][u] + e) * iv;
                uint32_t word;
                if constexpr (FMT == 0) {
                    word = (uint32_t)q8x4(f[0], f[1], f[2], f[3], 1.0f);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) f[u] = __builtin_amdgcn_fmed3f(f[u], -448.0f, 448.0f);
                    word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
                    word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], (int)word, true);
                }
                tile[vt][c0 + e][tq] = word;
            }
        }
    __syncthreads();
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
        for (int qq = tid; qq < D * 8; qq += 256) {
            const int c = qq >> 3, p16 = qq & 7;
            *(uint4*)(j.vc + ((int64_t)bh * D + c) * j.N + t0 + 128 * vt + p16 * 16) =
                make_uint4(tile[vt][c][4 * p16], tile[vt][c][4 * p16 + 1], tile[vt][c][4 * p16 + 2], tile[vt][c][4 * p16 + 3]);
        }
}

// ------------------------------------------------------------ MXFP4
// Encode 32 values (already loaded) as one MX block; returns the E8M0 byte.
// The conversion is the hardware's scaled e2m1 conversion (the scale's
// exponent only, nearest-even, saturating at 6): the same bits as scaling by
// 2^-e and rounding to the OCP e2m1 grid (tested bit for bit against the
// oracle, ties, saturation and subnormal blocks included).
__device__ __forceinline__ uint32_t mx_encode32(const float* v, uint32_t* packed /* 4 words */) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[k]));
    const int e = mx_exponent(amax);
    const float sc = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t x = 0;
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[w * 8 + 0], v[w * 8 + 1], sc, 0);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[w * 8 + 2], v[w * 8 + 3], sc, 1);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[w * 8 + 4], v[w * 8 + 5], sc, 2);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[w * 8 + 6], v[w * 8 + 7], sc, 3);
        packed[w] = x;
    }
    return (uint32_t)(e + 127);
}

// Rows (Q, K): grid BH * ceil(N / 128); thread handles (token, 32-channel
// block) items.  SUB selects what is subtracted before encoding:
//  MX_PLAIN  nothing; with `means` the fp32 means over each 128-token block
//            are written too (over the tokens present when the last block is
//            short, e.g. a single decode query);
//  MX_QBLOCK query smoothing: the block's mean, fp32 as above, then rounded
//            to bf16, is subtracted from its rows and written to `means`;
//  MX_KMEAN  key smoothing: mu = fp32(S / N - eps) per channel from the fp64
//            partial token sums `part` (nch chunks per head), subtracted from
//            every row; block 0 of a head writes it to `means` if not null.
// Every difference is one fp32 subtraction.
enum { MX_PLAIN = 0, MX_QBLOCK = 1, MX_KMEAN = 2 };
template <bool IS_F16, int SUB>
__global__ __launch_bounds__(256) void mx_rows_kernel(Dense x, int H, int N, int d, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, float* __restrict__ means,
                                                       const double* __restrict__ part, int nch, double eps) {
    const int nt = (N + 127) / 128;
    const int bh = blockIdx.x / nt, tb = blockIdx.x % nt;
    const int b = bh / H, h = bh % H;
    const int rows = min(128, N - tb * 128);
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH;
    const int nblk = d / 32;
    __shared__ float shift[128];
    // one thread per channel sums the block's tokens in fp64, in token order;
    // sixteen tokens are loaded ahead of their additions
    auto block_mean = [&](int c) {
        const uint16_t* col = base + (int64_t)tb * 128 * x.sN + c;
        double s = 0.0;
        int t = 0;
        for (; t + 16 <= rows; t += 16) {
            uint16_t e[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) e[u] = col[(int64_t)(t + u) * x.sN];
#pragma unroll
            for (int u = 0; u < 16; ++u) s += (double)load_half<IS_F16>(&e[u]);
        }
        for (; t < rows; ++t) s += (double)load_half<IS_F16>(col + (int64_t)t * x.sN);
        return (float)(s / (double)rows);
    };
    if constexpr (SUB == MX_QBLOCK) {
        for (int c = threadIdx.x; c < d; c += 256) {
            const float m = bf16_bits_to_f32(f32_to_bf16_bits(block_mean(c)));
            shift[c] = m;
            means[((int64_t)bh * nt + tb) * d + c] = m;
        }
        __syncthreads();
    } else if constexpr (SUB == MX_KMEAN) {
        for (int c = threadIdx.x; c < d; c += 256) {
            double S = 0.0;
            for (int u = 0; u < nch; ++u) S += part[((int64_t)bh * nch + u) * d + c];
            const float mu = (float)(S / (double)N - eps);
            shift[c] = mu;
            if (means && tb == 0) means[(int64_t)bh * d + c] = mu;
        }
        __syncthreads();
    }
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
        if constexpr (SUB != MX_PLAIN) {
#pragma unroll
            for (int k = 0; k < 32; ++k) v[k] = v[k] - shift[g * 32 + k];
        }
        uint32_t packed[4];
        uint32_t s = mx_encode32(v, packed);
        *(uint4*)(codes + ((int64_t)bh * N + t) * (d / 2) + g * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        scales[((int64_t)bh * N + t) * nblk + g] = (uint8_t)s;
    }
    if constexpr (SUB == MX_PLAIN) {
        if (means)
            for (int c = threadIdx.x; c < d; c += 256) means[((int64_t)bh * nt + tb) * d + c] = block_mean(c);
    }
}

// Columns (V): grid BH * (N / 128); the 128 x d tile is staged in LDS, then a
// thread encodes (channel, 32-token group) items into channel-major codes.
// With `tiled` the layout is blocked by 128 tokens (axis 2): codes
// [BH][N/128][d][64 B], scales [BH][N/128][d][4], so one key block's V is
// one contiguous 8.5 KB stretch.
template <bool IS_F16>
__global__ __launch_bounds__(256) void mx_cols_kernel(Dense x, int H, int N, int d, uint8_t* __restrict__ codes_t,
                                                       uint8_t* __restrict__ scales_t, int tiled) {
    const int nt = N / 128;
    const int bh = blockIdx.x / nt, tb = blockIdx.x % nt;
    const int b = bh / H, h = bh % H;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH;
    // the raw 16-bit values (34 KB of LDS, so four workgroups fit a CU),
    // widened when read; row stride 130 halves keeps column reads spread
    // over the banks
    __shared__ uint16_t tile[128][130];
    const int gpr = d / 8;
    for (int g = threadIdx.x; g < 128 * gpr; g += 256) {
        const int t = g / gpr, c = (g % gpr) * 8;
        const v4i raw = *(const v4i*)(base + (int64_t)(tb * 128 + t) * x.sN + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) *(uint32_t*)&tile[t][c + 2 * j] = (uint32_t)raw[j];
    }
    __syncthreads();
    for (int it = threadIdx.x; it < d * 4; it += 256) {
        const int c = it / 4, grp = it % 4;
        float v[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) v[k] = load_half<IS_F16>(&tile[grp * 32 + k][c]);
        uint32_t packed[4];
        uint32_t s = mx_encode32(v, packed);
        const int64_t tok = (int64_t)tb * 128 + grp * 32;
        const int64_t ci = tiled ? (((int64_t)bh * nt + tb) * d + c) * 64 + grp * 16 : ((int64_t)bh * d + c) * (N / 2) + tok / 2;
        const int64_t si = tiled ? (((int64_t)bh * nt + tb) * d + c) * 4 + grp : ((int64_t)bh * d + c) * (N / 32) + tok / 32;
        *(uint4*)(codes_t + ci) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        scales_t[si] = (uint8_t)s;
    }
}

// ------------------------------------------------------------ NVFP4 emulation
// ("ThriftAttention", Method step 2: the FP4 path in NVFP4 micro-scaling.)
// The slice's tensor scale g (nv_tensor_scale of its absmax, reduced here
// from the per-channel chunk maxima `part`), then blocks of 16 values with
// the scale s_b = e4m3(fp32(amax_b / fp32(6 g))) and values
// e2m1(fp32(x / (s_b g))) s_b g, written back as bf16 (exact).  A block
// whose scale underflows is zero.
__device__ __forceinline__ float nv_slice_scale(const float* part, int nch, int d, int bh) {
    __shared__ float red[256];
    float m = 0.0f;
    for (int i = threadIdx.x; i < nch * d; i += 256) m = __builtin_fmaxf(m, part[(int64_t)bh * nch * d + i]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] = __builtin_fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    return nv_tensor_scale(red[0]);
}
__device__ __forceinline__ void nv_block16(float* v, float g) {
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) am = __builtin_fmaxf(am, __builtin_fabsf(v[k]));
    const float S = e4m3_round(am / (6.0f * g)) * g;
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
        if (S != 0.0f) {
            const v2f q = e2m1_round2(v[k] / S, v[k + 1] / S);
            v[k] = q[0] * S;
            v[k + 1] = q[1] * S;
        } else {
            v[k] = v[k + 1] = 0.0f;
        }
    }
}
// axis 0 (Q, K): grid BH * ceil(N / 16); thread = (token, 16-channel block)
template <bool IS_F16>
__global__ __launch_bounds__(256) void nv_rows_kernel(Dense x, int H, int N, int d, const float* __restrict__ part,
                                                      int nch, Dense out) {
    const int nt = (N + 15) / 16;
    const int bh = blockIdx.x / nt, tb = blockIdx.x % nt;
    const int b = bh / H, h = bh % H;
    const float g = nv_slice_scale(part, nch, d, bh);
    const int nblk = d / 16, t = tb * 16 + (int)threadIdx.x / nblk, blk = (int)threadIdx.x % nblk;
    if ((int)threadIdx.x >= 16 * nblk || t >= N) return;
    const uint16_t* row = (const uint16_t*)x.p + b * x.sB + h * x.sH + (int64_t)t * x.sN + 16 * blk;
    float v[16];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint4 raw = *(const uint4*)(row + 8 * q);
        const uint16_t* e = (const uint16_t*)&raw;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * q + j] = load_half<IS_F16>(e + j);
    }
    nv_block16(v, g);
    uint16_t* orow = (uint16_t*)out.p + b * out.sB + h * out.sH + (int64_t)t * out.sN + 16 * blk;
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = (uint32_t)f32_to_bf16_bits(v[2 * k]) | ((uint32_t)f32_to_bf16_bits(v[2 * k + 1]) << 16);
    *(uint4*)orow = make_uint4(w[0], w[1], w[2], w[3]);
    *(uint4*)(orow + 8) = make_uint4(w[4], w[5], w[6], w[7]);
}
// axis 1 (V): grid BH * (N / 32); thread = (channel, 16-token block), lanes
// on consecutive channels (each token row is read coalesced)
template <bool IS_F16>
__global__ __launch_bounds__(256) void nv_cols_kernel(Dense x, int H, int N, int d, const float* __restrict__ part,
                                                      int nch, Dense out) {
    const int nt = N / 32;
    const int bh = blockIdx.x / nt, tb = blockIdx.x % nt;
    const int b = bh / H, h = bh % H;
    const float g = nv_slice_scale(part, nch, d, bh);
    const int c = (int)threadIdx.x % d, grp = (int)threadIdx.x / d;
    if (grp >= 256 / d || 32 * tb + 16 * grp >= N) return;
    for (int t0 = 32 * tb + 16 * grp; t0 < 32 * tb + 32; t0 += 16 * (256 / d)) {
        const uint16_t* col = (const uint16_t*)x.p + b * x.sB + h * x.sH + (int64_t)t0 * x.sN + c;
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = load_half<IS_F16>(col + (int64_t)k * x.sN);
        nv_block16(v, g);
        uint16_t* ocol = (uint16_t*)out.p + b * out.sB + h * out.sH + (int64_t)t0 * out.sN + c;
#pragma unroll
        for (int k = 0; k < 16; ++k) ocol[(int64_t)k * out.sN] = f32_to_bf16_bits(v[k]);
    }
}

// ------------------------------------------------------------ launchers
static int chunks_for(int BH, int N) {
    // about one block per CU, at least 512 rows per chunk (measured: fewer,
    // longer streams beat two blocks per CU, and the consumers combine fewer
    // partials)
    int want = (256 + BH - 1) / BH;
    int maxc = (N + 511) / 512;
    int c = want < maxc ? want : maxc;
    return c < 1 ? 1 : c;
}

size_t ws_kmean_bytes(int BH, int N, int d) { return (size_t)BH * chunks_for(BH, N) * d * sizeof(double); }
size_t ws_chan_bytes(int BH, int N, int d) { return (size_t)BH * chunks_for(BH, N) * d * sizeof(float); }

template <bool F16>
static hipError_t launch_tokblock_t(const Dense& x, int B, int H, int N, int d, int blk, const double* part,
                                    int nch, double eps, float* mu, int8_t* codes, float* scales, hipStream_t st) {
    const int grid = B * H * (N / blk);
    switch (blk * d / 2048) {
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
        if (f16) col_partial_kernel<true, true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
        else col_partial_kernel<false, true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    }
    return f16 ? launch_tokblock_t<true>(x, B, H, N, d, blk, part, nch, eps, mu, codes, scales, st)
               : launch_tokblock_t<false>(x, B, H, N, d, blk, part, nch, eps, mu, codes, scales, st);
}

// QK-norm fused into the INT8 token-block quantiser (d = 128): rows are
// normalised, rounded to bf16 and quantised in one pass; with smoothing the
// token sums of the normalised rows go to the workspace first.
hipError_t launch_quant_i8_qknorm(const Dense& x, bool f16, int B, int H, int N, int d, int blk, bool smooth,
                                  double eps, float* mu, float* inv_norm, void* ws, int8_t* codes, float* scales,
                                  hipStream_t st) {
    const int BH = B * H, nch = chunks_for(BH, N), rpc = (N + nch - 1) / nch;
    double* part = nullptr;
    if (smooth) {
        part = (double*)ws;
        if (f16) col_partial_kernel<true, true, true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
        else col_partial_kernel<false, true, true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    }
    const int grid = BH * (N / blk);
#define BQA_QKN(F16, NG) \
    quant_i8_tokblock_kernel<F16, NG, true><<<grid, 256, 0, st>>>(x, H, N, d, blk, part, nch, eps, mu, codes, scales, \
                                                                   inv_norm)
    if (blk == 64) {
        if (f16) BQA_QKN(true, 4);
        else BQA_QKN(false, 4);
    } else {
        if (f16) BQA_QKN(true, 8);
        else BQA_QKN(false, 8);
    }
#undef BQA_QKN
    return hipGetLastError();
}

hipError_t launch_quant_chan(const Dense& x, bool f16, int B, int H, int N, int d, int fmt, uint8_t* codes_t,
                             float* scales, void* ws, hipStream_t st) {
    const int BH = B * H, nch = chunks_for(BH, N), rpc = (N + nch - 1) / nch;
    float* part = (float*)ws;
    if (f16) col_partial_kernel<true, false><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    else col_partial_kernel<false, false><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    // 128-token tiles (128-byte code rows) where N allows, else 64
    const bool wide = N % 128 == 0;
    dim3 g(BH, N / (wide ? 128 : 64));
#define BQA_CHAN(F16, FMT)                                                                                  \
    (wide ? chan_encode_kernel<F16, FMT, 128><<<g, 256, 0, st>>>(x, H, N, d, part, nch, codes_t, scales)   \
          : chan_encode_kernel<F16, FMT, 64><<<g, 256, 0, st>>>(x, H, N, d, part, nch, codes_t, scales))
    if (fmt == 0) {
        if (f16) BQA_CHAN(true, 0);
        else BQA_CHAN(false, 0);
    } else {
        if (f16) BQA_CHAN(true, 1);
        else BQA_CHAN(false, 1);
    }
#undef BQA_CHAN
    return hipGetLastError();
}

// Workspace of the joint call: K token sums (fp64) then V channel maxima, per
// (head, chunk); the resident kernel puts its per-head counters in front.
static size_t ws_kv_two_pass(int BH, int N, int d) {
    return (ws_kmean_bytes(BH, N, d) + 255) / 256 * 256 + ws_chan_bytes(BH, N, d);
}
// flags: one 64-bit word per workgroup, each head's on 256-byte lines of its own
static int kv_flag_stride(int N) { return (N / RES_T * 8 + 255) / 256 * 32; }
static size_t ws_kv_counters(int BH, int N) { return (size_t)BH * kv_flag_stride(N) * sizeof(uint64_t); }
static size_t ws_kv_resident(int BH, int N, int d) {
    const size_t nch = (size_t)(N / RES_T);
    return ws_kv_counters(BH, N) + ((size_t)BH * nch * d * sizeof(double) + 255) / 256 * 256 + (size_t)BH * nch * d * sizeof(float);
}
static bool resident_shape(int N, int d) { return d == 128 && N % RES_T == 0; }

size_t ws_kv_bytes(int BH, int N, int d) {
    const size_t a = ws_kv_two_pass(BH, N, d);
    if (!resident_shape(N, d)) return a;
    const size_t b = ws_kv_resident(BH, N, d);
    return a > b ? a : b;
}

// Tags of the resident kernel's flags: a process-wide 64-bit sequence from a
// start drawn from the clock and an address (distinct across processes and
// runs); zero is skipped.
static uint64_t next_kv_tag() {
    static std::atomic<uint64_t> seq{[] {
        uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        x ^= (uint64_t)(uintptr_t)&seq << 17;
        x ^= x >> 31; x *= 0x9E3779B97F4A7C15ull; x ^= x >> 29;   // mix
        return x;
    }()};
    uint64_t t;
    do t = seq.fetch_add(1, std::memory_order_relaxed); while (t == 0);
    return t;
}

// Polls of a workgroup waiting for the others of its head before it takes the
// head's statistics itself: a few tenths of a second by default.  Tests
// set BQA_KV_WAIT_LIMIT (read at each call) to a tiny value to run that path.
static uint32_t resident_spin_limit() {
    const char* e = std::getenv("BQA_KV_WAIT_LIMIT");
    const long n = e ? std::strtol(e, nullptr, 10) : 0;
    return n > 0 && n < (1L << 30) ? (uint32_t)n : (uint32_t)(1u << 17);
}

// Workgroups of kv_resident_kernel<F16, FMT> the current device holds at
// once (occupancy x compute units), cached per device and instance.
template <bool F16, int FMT>
static int resident_capacity() {
    static std::atomic<int> cache[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_acquire);
    if (v == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kv_resident_kernel<F16, FMT>, 256, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            per_cu = cus = 0;
        v = per_cu * cus > 0 ? per_cu * cus : -1;
        cache[dev].store(v, std::memory_order_release);
    }
    return v;
}

hipError_t launch_quant_kv(const Dense& k, const Dense& v, bool f16, int B, int H, int N, int d, bool smooth,
                           double eps, float* mu, int8_t* kc, float* ks, int vfmt, uint8_t* vc, float* vs, void* ws,
                           hipStream_t st) {
    KvJob j;
    j.k = k; j.v = v; j.H = H; j.N = N; j.d = d;
    const int BH = B * H;
    j.smooth = smooth; j.eps = eps;
    j.mu = mu; j.kc = kc; j.ks = ks; j.vc = vc; j.vs = vs;
    hipStreamCaptureStatus cap_st = hipStreamCaptureStatusNone;
    const bool capturing = hipStreamIsCapturing(st, &cap_st) == hipSuccess && cap_st != hipStreamCaptureStatusNone;
    if (resident_shape(N, d) && !capturing) {
        const int grid = BH * (N / RES_T);
        const int cap = f16 ? (vfmt == 0 ? resident_capacity<true, 0>() : resident_capacity<true, 1>())
                            : (vfmt == 0 ? resident_capacity<false, 0>() : resident_capacity<false, 1>());
        if (grid <= cap) {
            j.nch = N / RES_T;
            j.rpc = RES_T;
            j.kpart = (double*)((char*)ws + ws_kv_counters(BH, N));
            j.vpart = (float*)((char*)j.kpart + ((size_t)BH * j.nch * d * sizeof(double) + 255) / 256 * 256);
            uint64_t* flags = (uint64_t*)ws;
            const int fs = kv_flag_stride(N);
            const uint64_t tag = next_kv_tag();
            const uint32_t lim = resident_spin_limit();
            if (f16) {
                if (vfmt == 0) kv_resident_kernel<true, 0><<<grid, 256, 0, st>>>(j, flags, fs, tag, lim);
                else kv_resident_kernel<true, 1><<<grid, 256, 0, st>>>(j, flags, fs, tag, lim);
            } else {
                if (vfmt == 0) kv_resident_kernel<false, 0><<<grid, 256, 0, st>>>(j, flags, fs, tag, lim);
                else kv_resident_kernel<false, 1><<<grid, 256, 0, st>>>(j, flags, fs, tag, lim);
            }
            return hipGetLastError();
        }
    }
    j.nch = chunks_for(BH, N);
    j.rpc = (N + j.nch - 1) / j.nch;
    j.kpart = (double*)ws;
    j.vpart = (float*)((char*)ws + (ws_kmean_bytes(BH, N, d) + 255) / 256 * 256);
    const int nkp = smooth ? BH * j.nch : 0;
    if (f16) kv_partial_kernel<true><<<nkp + BH * j.nch, 256, 0, st>>>(j, nkp);
    else kv_partial_kernel<false><<<nkp + BH * j.nch, 256, 0, st>>>(j, nkp);
    // K token blocks of 64: 64 d / 2048 groups of 8 per thread (4 at d = 128, 2 at d = 64)
    const int nke = BH * (N / 64);
    const bool wide = N % 128 == 0;
    const int nve = BH * (N / (wide ? 128 : 64));
#define BQA_KV_T(F16, FMT, NG)                                                               \
    (wide ? kv_encode_kernel<F16, FMT, 128, NG><<<nke + nve, 256, 0, st>>>(j, nke)           \
          : kv_encode_kernel<F16, FMT, 64, NG><<<nke + nve, 256, 0, st>>>(j, nke))
#define BQA_KV(F16, FMT) (d == 128 ? BQA_KV_T(F16, FMT, 4) : BQA_KV_T(F16, FMT, 2))
    if (vfmt == 0) {
        if (f16) BQA_KV(true, 0);
        else BQA_KV(false, 0);
    } else {
        if (f16) BQA_KV(true, 1);
        else BQA_KV(false, 1);
    }
#undef BQA_KV
#undef BQA_KV_T
    return hipGetLastError();
}

hipError_t launch_quant_mx(const Dense& x, bool f16, int B, int H, int N, int d, int axis, uint8_t* codes,
                           uint8_t* scales, float* means, hipStream_t st) {
    const int grid = B * H * ((N + 127) / 128);
    if (axis == 0) {
        if (f16) mx_rows_kernel<true, MX_PLAIN><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means, nullptr, 0, 0.0);
        else mx_rows_kernel<false, MX_PLAIN><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means, nullptr, 0, 0.0);
    } else {
        if (f16) mx_cols_kernel<true><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, axis == 2);
        else mx_cols_kernel<false><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, axis == 2);
    }
    return hipGetLastError();
}

size_t ws_nvfp4_bytes(int BH, int N, int d) { return ws_chan_bytes(BH, N, d); }

// NVFP4 emulation: per-channel chunk maxima of the slice into the workspace,
// then the blocks of 16 along d (axis 0) or along the tokens (axis 1).
hipError_t launch_nvfp4(const Dense& x, bool f16, int B, int H, int N, int d, int axis, const Dense& out, void* ws,
                        hipStream_t st) {
    const int BH = B * H, nch = chunks_for(BH, N), rpc = (N + nch - 1) / nch;
    float* part = (float*)ws;
    if (f16) col_partial_kernel<true, false><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    else col_partial_kernel<false, false><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
    if (axis == 0) {
        const int grid = BH * ((N + 15) / 16);
        if (f16) nv_rows_kernel<true><<<grid, 256, 0, st>>>(x, H, N, d, part, nch, out);
        else nv_rows_kernel<false><<<grid, 256, 0, st>>>(x, H, N, d, part, nch, out);
    } else {
        const int grid = BH * (N / 32);
        if (f16) nv_cols_kernel<true><<<grid, 256, 0, st>>>(x, H, N, d, part, nch, out);
        else nv_cols_kernel<false><<<grid, 256, 0, st>>>(x, H, N, d, part, nch, out);
    }
    return hipGetLastError();
}

// Smoothed MXFP4 rows of the post-training FP4 baseline: Q less its bf16
// block means (written to `means`), or K less its token mean (the fp64 token
// sums go to the workspace first; mu to `means` when not null).
hipError_t launch_quant_mx_smooth(const Dense& x, bool f16, int B, int H, int N, int d, bool key, double eps,
                                  uint8_t* codes, uint8_t* scales, float* means, void* ws, hipStream_t st) {
    const int BH = B * H, grid = BH * ((N + 127) / 128);
    if (!key) {
        if (f16) mx_rows_kernel<true, MX_QBLOCK><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means, nullptr, 0, 0.0);
        else mx_rows_kernel<false, MX_QBLOCK><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means, nullptr, 0, 0.0);
        return hipGetLastError();
    }
    const int nch = chunks_for(BH, N), rpc = (N + nch - 1) / nch;
    double* part = (double*)ws;
    if (f16) {
        col_partial_kernel<true, true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
        mx_rows_kernel<true, MX_KMEAN><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means, part, nch, eps);
    } else {
        col_partial_kernel<false, true><<<dim3(BH, nch), 256, 0, st>>>(x, H, N, d, rpc, part);
        mx_rows_kernel<false, MX_KMEAN><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means, part, nch, eps);
    }
    return hipGetLastError();
}

}  // namespace bqa
