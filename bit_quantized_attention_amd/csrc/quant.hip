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
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace bqa {

// ------------------------------------------------------------ column partials
// grid (BH, chunks); 256 threads = 16 rows x 16 column groups of 8 channels.
// Each chunk of tokens is reduced per channel into part[bh][chunk][c]: SUM
// gives fp64 token sums (K smoothing), otherwise fp32 absolute maxima
// (per-channel V scales).
template <bool IS_F16, bool SUM>
__device__ __forceinline__ void col_partial_body(const Dense& x, int H, int N, int d, int rows_per_chunk,
                                                 void* __restrict__ part_out, int bh, int chunk, int nchunks) {
    using Acc = typename std::conditional<SUM, double, float>::type;
    const int b = bh / H, h = bh % H;
    const int cg = threadIdx.x % 16, r = threadIdx.x / 16;
    const uint16_t* base = (const uint16_t*)x.p + b * x.sB + h * x.sH + cg * 8;
    Acc acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto take = [&](const v4i& raw) {
        const uint16_t* e = (const uint16_t*)&raw;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float f = load_half<IS_F16>(e + k);
            if constexpr (SUM) acc[k] += (double)f;
            else acc[k] = __builtin_fmaxf(acc[k], __builtin_fabsf(f));
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

template <bool IS_F16, bool SUM>
__global__ __launch_bounds__(256) void col_partial_kernel(Dense x, int H, int N, int d, int rows_per_chunk,
                                                          void* __restrict__ part_out) {
    col_partial_body<IS_F16, SUM>(x, H, N, d, rows_per_chunk, part_out, blockIdx.x, blockIdx.y, gridDim.y);
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
// block 0 of each head writes it to `mu_out`.
template <bool IS_F16, int NG>
__device__ __forceinline__ void tokblock_body(const Dense& x, int H, int N, int d, int blk,
                                              const double* __restrict__ part, int nchunks, double eps,
                                              float* __restrict__ mu_out, int8_t* __restrict__ codes,
                                              float* __restrict__ scales, int block_id) {
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
        for (int j = 0; j < 8; ++j) {
            float f = load_half<IS_F16>(e + j);
            if (has_mu) f = f - mu[j];
            v[k][j] = f;
            amax = __builtin_fmaxf(amax, __builtin_fabsf(f));
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

template <bool IS_F16, int NG>
__global__ __launch_bounds__(256) void quant_i8_tokblock_kernel(Dense x, int H, int N, int d, int blk,
                                                                 const double* __restrict__ part, int nchunks,
                                                                 double eps, float* __restrict__ mu_out,
                                                                 int8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
    tokblock_body<IS_F16, NG>(x, H, N, d, blk, part, nchunks, eps, mu_out, codes, scales, blockIdx.x);
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
        // one thread per channel sums the block's tokens in fp64, in token
        // order; sixteen tokens are loaded ahead of their additions
        for (int c = threadIdx.x; c < d; c += 256) {
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

size_t ws_kv_bytes(int BH, int N, int d) {
    return (ws_kmean_bytes(BH, N, d) + 255) / 256 * 256 + ws_chan_bytes(BH, N, d);
}

hipError_t launch_quant_kv(const Dense& k, const Dense& v, bool f16, int B, int H, int N, int d, bool smooth,
                           double eps, float* mu, int8_t* kc, float* ks, int vfmt, uint8_t* vc, float* vs, void* ws,
                           hipStream_t st) {
    KvJob j;
    j.k = k; j.v = v; j.H = H; j.N = N; j.d = d;
    const int BH = B * H;
    j.nch = chunks_for(BH, N);
    j.rpc = (N + j.nch - 1) / j.nch;
    j.smooth = smooth; j.eps = eps;
    j.kpart = (double*)ws;
    j.vpart = (float*)((char*)ws + (ws_kmean_bytes(BH, N, d) + 255) / 256 * 256);
    j.mu = mu; j.kc = kc; j.ks = ks; j.vc = vc; j.vs = vs;
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
        if (f16) mx_rows_kernel<true><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means);
        else mx_rows_kernel<false><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales, means);
    } else {
        if (f16) mx_cols_kernel<true><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales);
        else mx_cols_kernel<false><<<grid, 256, 0, st>>>(x, H, N, d, codes, scales);
    }
    return hipGetLastError();
}

}  // namespace bqa
