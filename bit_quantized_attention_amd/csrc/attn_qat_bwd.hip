// attn_qat_bwd.hip — Attn-QAT backward for gfx950.
//
// "Attn-QAT: 4-Bit Attention With Quantization-Aware Training", technical
// summary §2 Principles 1 and 2: the backward recomputes P at the forward's
// precision (the same MXFP4 scores, P = exp(s - L); for dV = P^T dO the
// forward's rounding: MXFP4 codes of exp2((s - M) c) per 32 keys, M the row's
// largest raw score as the forward reports it, scaled by exp(tau M - L)),
// keeps the straight-through softmax Jacobian dS = P o (dP - delta') with the
// unquantised P, and takes delta' = rowsum(dO o O') from the forward's
// high-precision auxiliary output.  dP = dO V^T, dQ = tau dS K and
// dK = tau dS^T Q run as bf16 products against the FP4 operands (e2m1 times a
// power of two is exact in bf16); dS is rounded to bf16 for them.
// dV = P^T dO runs in fp16: the rounded P times its row's exp(M - L) is not a
// bf16 value, and fp16 keeps it to 2^-11.  dO enters that product scaled by
// a power of two per (batch, head), chosen so that the head's largest |dO|
// lands in [2^14, 2^15): small gradients keep fp16's full precision instead
// of going subnormal, large ones do not overflow; dV is scaled back at the
// end.
//
// Kernels:
//   qat_delta_kernel   delta' per query row, the largest |dO| per head
//   deq_t_fp4_kernel   bf16 copies in the layouts the products read:
//   deq_t_bf16_kernel  deq(V) token-major, deq(Q)^T, deq(K)^T (from the
//                      MXFP4 codes) and dO^T (fp16) channel-major
//   qbwd_dkdv_kernel   one workgroup per 64-key block over the 128-query
//                      tiles: the tile is computed with queries in lanes
//                      (P's MX blocks lie along a lane's registers), P^ and
//                      dS go to LDS transposed for dV = P^T dO, dK = dS^T Q
//   qbwd_dq_kernel     one workgroup per 128-query tile over the key tiles:
//                      dS is the A operand of dQ = dS K from registers
#include "common.hpp"
#include "internal.hpp"

namespace bqa {

namespace {

constexpr int D = 128;
constexpr int TQ = 128;
constexpr int TK = 64;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
__device__ __forceinline__ int fs64(int r) { return ((r >> 2) & 3) ^ (((r >> 4) & 1) << 1); }
__device__ __forceinline__ int fs256(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }
__device__ __forceinline__ int fc128(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int fc256(int r) { return r & 15; }

// ------------------------------------------------------------------ preprocess
// delta'_i = sum_c dO[i, c] O'[i, c] for the 128 rows of one workgroup (16
// rows at a time, 16 lanes per row, 8 channels each), and the largest |dO|
// of those rows folded into its head's word with one atomic (N is a multiple
// of 128, so a workgroup never spans two heads).
constexpr int DELTA_ROWS = 128;
__global__ __launch_bounds__(256) void qat_delta_kernel(Dense dO, Dense Oa, int H, int N, int64_t rows,
                                                        float* __restrict__ delta, uint32_t* __restrict__ do_amax) {
    __shared__ float wmax[4];
    const int part = threadIdx.x & 15;
    const int64_t row0 = (int64_t)blockIdx.x * DELTA_ROWS;
    float am = 0.0f;
    for (int it = 0; it < DELTA_ROWS / 16; ++it) {
        const int64_t row = row0 + 16 * it + (threadIdx.x >> 4);
        float acc = 0.0f;
        if (row < rows) {
            const int64_t bh = row / N, i = row % N, b = bh / H, h = bh % H;
            const v4i gv = *(const v4i*)((const uint16_t*)dO.p + b * dO.sB + h * dO.sH + i * dO.sN + 8 * part);
            const v4i ov = *(const v4i*)((const uint16_t*)Oa.p + b * Oa.sB + h * Oa.sH + i * Oa.sN + 8 * part);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float g0 = bf16_bits_to_f32((uint16_t)gv[k]), g1 = bf16_bits_to_f32((uint16_t)((uint32_t)gv[k] >> 16));
                acc = __builtin_fmaf(g0, bf16_bits_to_f32((uint16_t)ov[k]), acc);
                acc = __builtin_fmaf(g1, bf16_bits_to_f32((uint16_t)((uint32_t)ov[k] >> 16)), acc);
                am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(g0), __builtin_fabsf(g1)));
            }
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 16);
        if (row < rows && part == 0) delta[row] = acc;
    }
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0 && row0 < rows) {
        const float m = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
        atomicMax(do_amax + row0 / N, __builtin_bit_cast(uint32_t, m));   // non-negative floats order as integers
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Power of two k for a head's dO whose largest magnitude is amax (fp32
// bits): amax 2^k lies in [2^14, 2^15); 0 for an all-zero head.
__device__ __forceinline__ int do_shift(uint32_t amax_bits) {
    const int e = (int)((amax_bits >> 23) & 0xFF);
    if (amax_bits == 0u) return 0;
    const int k = 14 - ((e == 0 ? 1 : e) - 127);
    return k < -126 ? -126 : (k > 127 ? 127 : k);
}

// MXFP4 codes along C of a [BH][R][C] grid (rows of C/2 bytes, E8M0 per 32
// of C) to bf16, transposed: out[bh][c][r].  64 x 64 tiles; a thread reads 8
// code bytes (16 values of one row) and converts them with the hardware's
// scaled e2m1 -> bf16 conversion (exact: an e2m1 value times 2^e), the tile
// crosses LDS and leaves in 16-byte stores along r.
__global__ __launch_bounds__(256) void deq_t_fp4_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sc,
                                                        int R, int C, uint16_t* __restrict__ out) {
    __shared__ uint32_t t[64][33];     // [r][pair of c], stride 33 words
    const int tilesR = R / 64, tilesC = C / 64;
    int blk = blockIdx.x;
    const int tc = blk % tilesC; blk /= tilesC;
    const int tr = blk % tilesR;
    const int64_t bh = blk / tilesR;
    const int tid = threadIdx.x, r = tid >> 2, q = tid & 3;         // row r, columns 16 q .. 16 q + 15
    const int64_t row = bh * R + (int64_t)tr * 64 + r;
    const v2i x = *(const v2i*)(codes + row * (C / 2) + tc * 32 + 8 * q);
    const float s = __builtin_bit_cast(float, (uint32_t)sc[row * (C / 32) + 2 * tc + (q >> 1)] << 23);
    const uint32_t x0 = (uint32_t)x[0], x1 = (uint32_t)x[1];
    t[r][8 * q + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x0, s, 0));
    t[r][8 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x0, s, 1));
    t[r][8 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x0, s, 2));
    t[r][8 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x0, s, 3));
    t[r][8 * q + 4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x1, s, 0));
    t[r][8 * q + 5] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x1, s, 1));
    t[r][8 * q + 6] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x1, s, 2));
    t[r][8 * q + 7] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x1, s, 3));
    __syncthreads();
    // output row c (64 of the tile), r = 16 g .. 16 g + 15
    const int c = tid >> 2, g = tid & 3;
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t a = t[16 * g + 2 * k][c >> 1], b = t[16 * g + 2 * k + 1][c >> 1];
        w[k] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
    uint16_t* dst = out + (bh * C + (int64_t)tc * 64 + c) * R + (int64_t)tr * 64 + 16 * g;
    *(v4i*)dst = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    *(v4i*)(dst + 8) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
}

// Dense bf16 [B][H][R][C] view times 2^k of its head (do_shift) to fp16,
// transposed: out[bh][c][r]; the tiling of deq_t_fp4_kernel, a thread
// reading 16 values (32 bytes) of one row.  The scaled values lie below 2^15,
// and every bf16 value at or above 2^-14 after scaling is exact in fp16.
__global__ __launch_bounds__(256) void deq_t_bf16_kernel(Dense x, int H, int R, int C, const uint32_t* __restrict__ amax,
                                                         uint16_t* __restrict__ out) {
    __shared__ uint32_t t[64][33];
    const int tilesR = R / 64, tilesC = C / 64;
    int blk = blockIdx.x;
    const int tc = blk % tilesC; blk /= tilesC;
    const int tr = blk % tilesR;
    const int64_t bh = blk / tilesR, b = bh / H, h = bh % H;
    const int tid = threadIdx.x, r = tid >> 2, q = tid & 3;
    const float sc = __builtin_ldexpf(1.0f, do_shift(amax[bh]));
    const uint16_t* src = (const uint16_t*)x.p + b * x.sB + h * x.sH + ((int64_t)tr * 64 + r) * x.sN + tc * 64 + 16 * q;
    const v4i a0 = *(const v4i*)src, a1 = *(const v4i*)(src + 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t pr = (uint32_t)(j < 4 ? a0[j] : a1[j - 4]);
        t[r][8 * q + j] = (uint32_t)f32_to_f16_bits(bf16_bits_to_f32((uint16_t)pr) * sc) |
                          ((uint32_t)f32_to_f16_bits(bf16_bits_to_f32((uint16_t)(pr >> 16)) * sc) << 16);
    }
    __syncthreads();
    const int c = tid >> 2, g = tid & 3;
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t lo = t[16 * g + 2 * k][c >> 1], hi = t[16 * g + 2 * k + 1][c >> 1];
        w[k] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    uint16_t* dst = out + (bh * C + (int64_t)tc * 64 + c) * R + (int64_t)tr * 64 + 16 * g;
    *(v4i*)dst = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    *(v4i*)(dst + 8) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
}

// ------------------------------------------------------------------ the tile (queries in lanes)
// For one wavefront: 32 queries (lanes) x 64 keys of block J.  Inputs: K codes
// and scales of the block and deq(V) rows of the block in LDS (sigma reads);
// the lane's query codes, dO row (bf16), L (log2 units) and delta'.
// Outputs per lane: p[g][i], ds[g][i] for key 32 g + 16 h + i.
struct KeyTile {
    uint8_t kc[TK * D / 2];     // 64 keys x 64 B
    uint8_t ks[TK * D / 32];    // 64 keys x 4
    uint8_t vr[TK * D * 2];     // deq(V) rows, 64 keys x 256 B
};

__device__ __forceinline__ void key_tile_issue(const QatBwdArgs& a, int bh, int J, KeyTile& T, int w, int l) {
    const int k0 = J * TK;
    {   // K codes: 4 x 1 KB (16 rows of 64 B)
        const int r = 16 * w + (l >> 2);
        lds_copy16((uint32_t)(r * (D / 2) + 16 * ((l & 3) ^ fs64(r))), a.kc + ((int64_t)bh * a.N + k0) * (D / 2),
                   lds_addr(T.kc + 1024 * w));
    }
    // K scales: 256 B, one copy (repeated by every wavefront so that all count the same copies)
    lds_copy4((uint32_t)(4 * l), a.ks + ((int64_t)bh * a.N + k0) * (D / 32), lds_addr(T.ks));
#pragma unroll
    for (int u = 0; u < 4; ++u) {   // deq(V) rows: 16 x 1 KB (4 rows of 256 B)
        const int sgm = 4 * w + u, r = 4 * sgm + (l >> 4);
        lds_copy16((uint32_t)(2 * (r * D + 8 * ((l & 15) ^ fs256(r)))), a.vdeq + ((int64_t)bh * a.N + k0) * D,
                   lds_addr(T.vr + 1024 * sgm));
    }
}

struct RowIn {
    v4i qb[2];
    int qsb[2];
    v8bf gb[8];
    float lse2, dlt, mraw;  // L (log2 units), delta', the row's largest raw score M
};

__device__ __forceinline__ void row_load(const QatBwdArgs& a, int bh, int b, int hq, int qrow, int h, RowIn& r) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        r.qb[kk] = *(const v4i*)(a.qc + ((int64_t)bh * a.N + qrow) * (D / 2) + 32 * kk + 16 * h);
        r.qsb[kk] = a.qs[((int64_t)bh * a.N + qrow) * (D / 32) + 2 * kk + h];
    }
    const uint16_t* g = (const uint16_t*)a.d_o.p + b * a.d_o.sB + hq * a.d_o.sH + (int64_t)qrow * a.d_o.sN;
#pragma unroll
    for (int st = 0; st < 8; ++st) r.gb[st] = *(const v8bf*)(g + 16 * st + 8 * h);
    r.lse2 = a.lse[(int64_t)bh * a.N + qrow] * 1.4426950408889634f;
    r.dlt = a.delta[(int64_t)bh * a.N + qrow];
    r.mraw = a.row_max[(int64_t)bh * a.N + qrow];
}

// P (unrounded), its MXFP4 fake quantisation (as float) and dS (bf16-rounded)
// for keys 32 g .. 32 g + 31 of the tile (one MX block of P per query row)
__device__ __forceinline__ void tile_pds_g(const KeyTile& T, const RowIn& r, float c, int krow, int h, int g,
                                           float (&p)[16], float (&pq)[16], float (&ds)[16]) {
    const int rk = 32 * g + krow;
    v16f s = v16f{};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const v4i av = *(const v4i*)(T.kc + rk * 64 + 16 * ((2 * kk + h) ^ fs64(rk)));
        s = mfma_f4_32x32x64(av, (int)T.ks[4 * rk + 2 * kk + h], r.qb[kk], r.qsb[kk], s);
    }
    v16f dp = v16f{};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const v8bf av = *(const v8bf*)(T.vr + rk * 256 + 16 * ((2 * st + h) ^ fs256(rk)));
        dp = mfma_bf16_32x32x16(av, r.gb[st], dp);
    }
    // P relative to the row's maximum, formed as the forward forms it;
    // exp2(M c - L) brings it to P = exp(s - L)
    const float back = __builtin_amdgcn_exp2f(__builtin_fmaf(r.mraw, c, -r.lse2));
    float pr[16];
    float smax = s[0];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        pr[i] = __builtin_amdgcn_exp2f((s[i] - r.mraw) * c);
        p[i] = pr[i] * back;
        smax = __builtin_fmaxf(smax, s[i]);
        ds[i] = (float)(__bf16)(p[i] * (dp[i] - r.dlt));
    }
    // MX block g of the row: 16 keys here, 16 in the partner lane
    smax = __builtin_fmaxf(smax, partner32f(smax));
    const int e = mx_exponent(__builtin_amdgcn_exp2f((smax - r.mraw) * c));
    const float sc = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        const uint32_t code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, pr[i], pr[i + 1], sc, 0);
        const v2f dq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, sc, 0);
        pq[i] = dq[0] * back;
        pq[i + 1] = dq[1] * back;
    }
}
// both key halves of the tile
__device__ __forceinline__ void tile_pds(const KeyTile& T, const RowIn& r, float c, int krow, int h, float (&p)[2][16],
                                         float (&pq)[2][16], float (&ds)[2][16]) {
#pragma unroll
    for (int g = 0; g < 2; ++g) tile_pds_g(T, r, c, krow, h, g, p[g], pq[g], ds[g]);
}

// ------------------------------------------------------------------ dK, dV
// The query tile's per-row inputs (one slot): what the dQ kernel loads into
// each lane's registers once, this kernel reads from LDS for every tile.
struct RowTile {
    uint8_t qc[TQ * D / 2];     // Q codes, 128 rows x 64 B (chunk XOR (row >> 1) & 3)
    uint8_t qs[TQ * D / 32];    // Q scales, 128 rows x 4 B
    uint8_t dob[TQ * D * 2];    // dO bf16, 128 rows x 256 B (chunk XOR row & 15)
    float lse[TQ];
    float dlt[TQ];
    float rmax[TQ];
};
struct LdsKVq {
    KeyTile kt;                  // fixed: the workgroup's key block
    RowTile rt;                  // per-row inputs of the query tile
    uint8_t pt[TQ * TK * 2];     // P^: 128 queries x 64 keys fp16, 128-byte rows (chunks XOR query % 8)
    uint8_t st[TQ * TK * 2];     // dS, bf16, same layout
    uint8_t gT[D * TQ * 2];      // dO^T: 128 channels x 128 queries fp16
    uint8_t qT[D * TQ * 2];      // deq(Q)^T
};

// One wavefront's share (of 8) of the copies of a query tile, as per-lane
// offsets from tile bases.  "Rows" (RowTile) and "columns" (dO^T, deq(Q)^T).
struct KvqPlan {
    static constexpr int NR = 1 + 4 + 1, NC = 4 + 4;   // copies per wavefront
    static_assert(NR + NC < 64, "vmcnt range");
    uint32_t qc, g[4], t[4];
    __device__ __forceinline__ KvqPlan(int w, int l, int N, int64_t g_sN) {
        {                                  // Q codes: 8 x 1 KB (16 rows of 64 B)
            const int r = 16 * w + (l >> 2);
            qc = (uint32_t)(r * (D / 2) + 16 * ((l & 3) ^ ((r >> 1) & 3)));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {      // dO bf16: 32 x 1 KB (4 rows of 256 B)
            const int r = 4 * (4 * w + u) + (l >> 4);
            g[u] = (uint32_t)(2 * (r * g_sN + 8 * ((l & 15) ^ (r & 15))));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {      // channel-major bf16: 32 x 1 KB each (4 rows of 256 B)
            const int r = 4 * (4 * w + u) + (l >> 4);
            t[u] = (uint32_t)(2 * (r * N + 8 * ((l & 15) ^ fc256(r))));
        }
    }
};
__device__ __forceinline__ void rows_issue(const QatBwdArgs& a, const KvqPlan& cp, int bh, int b, int hq, int I,
                                           RowTile& R, int w, int l) {
    const int q0 = I * TQ;
    lds_copy16(cp.qc, a.qc + ((int64_t)bh * a.N + q0) * (D / 2), lds_addr(R.qc + 1024 * w));
    const uint16_t* gb = (const uint16_t*)a.d_o.p + b * a.d_o.sB + hq * a.d_o.sH + (int64_t)q0 * a.d_o.sN;
#pragma unroll
    for (int u = 0; u < 4; ++u) lds_copy16(cp.g[u], gb, lds_addr(R.dob + 1024 * (4 * w + u)));
    // scales, log-sum-exp, delta, maxima: eight 256-byte copies, one per wavefront
    const uint32_t o = (uint32_t)(4 * l);
    const int job = w, half = job & 1;
    if (job < 2) lds_copy4(o, a.qs + ((int64_t)bh * a.N + q0) * (D / 32) + 256 * half, lds_addr(R.qs + 256 * half));
    else if (job < 4) lds_copy4(o, a.lse + (int64_t)bh * a.N + q0 + 64 * half, lds_addr(R.lse + 64 * half));
    else if (job < 6) lds_copy4(o, a.delta + (int64_t)bh * a.N + q0 + 64 * half, lds_addr(R.dlt + 64 * half));
    else lds_copy4(o, a.row_max + (int64_t)bh * a.N + q0 + 64 * half, lds_addr(R.rmax + 64 * half));
}
__device__ __forceinline__ void cols_issue(const QatBwdArgs& a, const KvqPlan& cp, int bh, int I, LdsKVq& L, int w) {
    const uint16_t* gT = a.doT + (int64_t)bh * D * a.N + I * TQ;
    const uint16_t* qT = a.qT + (int64_t)bh * D * a.N + I * TQ;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        lds_copy16(cp.t[u], gT, lds_addr(L.gT + 1024 * (4 * w + u)));
        lds_copy16(cp.t[u], qT, lds_addr(L.qT + 1024 * (4 * w + u)));
    }
}
__device__ __forceinline__ void row_from_lds(const RowTile& R, int row, int h, RowIn& r) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        r.qb[kk] = *(const v4i*)(R.qc + row * 64 + 16 * ((2 * kk + h) ^ ((row >> 1) & 3)));
        r.qsb[kk] = R.qs[row * 4 + 2 * kk + h];
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) r.gb[st] = *(const v8bf*)(R.dob + row * 256 + 16 * ((2 * st + h) ^ (row & 15)));
    r.lse2 = R.lse[row] * 1.4426950408889634f;
    r.dlt = R.dlt[row];
    r.mraw = R.rmax[row];
}

// One workgroup of 8 wavefronts per 64-key block over the 128-query tiles.
// Step I: wavefront (qg, kh) computes P, its fake quantisation and dS for
// queries 32 qg .. (in lanes) and keys 32 kh .. from the rows of tile I and
// writes P^ and dS transposed to LDS; then wavefront (ko, co) accumulates dV
// and dK for 32 keys x 32 channels from them and the channel-major dO^T,
// deq(Q)^T of tile I.  The rows of tile I+1 are copied during the products,
// the columns of tile I+1 during the next step's P and dS.
__global__ __launch_bounds__(512, 1) void qbwd_dkdv_kernel(QatBwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsKVq L;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int nkt = a.N / TK, nqt = a.N / TQ;
    const int J = blockIdx.x % nkt;
    const int bh = blockIdx.x / nkt, b = bh / a.H, hq = bh % a.H;
    const int krow = sigma(lq);
    const float c = a.c_log2;
    const int qg = w & 3, kh = w >> 2;               // P, dS: queries 32 qg + lane, keys 32 kh ..
    const int ko = 32 * (w & 1), co = 32 * (w >> 1); // dV, dK: keys ko .., channels co ..
    const KvqPlan cp(w, l, a.N, a.d_o.sN);

    v16f dv = v16f{}, dk = v16f{};

    if (w < 4) key_tile_issue(a, bh, J, L.kt, w, l);
    rows_issue(a, cp, bh, b, hq, 0, L.rt, w, l);
    cols_issue(a, cp, bh, 0, L, w);
    BQA_WAIT_VM(0);
    barrier_only();
    for (int I = 0; I < nqt; ++I) {
        const bool more = I + 1 < nqt;
        const int qc = 32 * qg + lq;
        RowIn rin;
        row_from_lds(L.rt, qc, h, rin);
        float p[16], pq[16], ds[16];
        tile_pds_g(L.kt, rin, c, krow, h, kh, p, pq, ds);
        // P^ (fp16) and dS (bf16) to LDS, query-major: this lane's 16 keys are
        // two 16-byte chunks of its query's row
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
            v8h ph;
            v8bf sb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[e] = (_Float16)pq[8 * hc + e];
                sb[e] = (__bf16)ds[8 * hc + e];
            }
            const int off = qc * 128 + 16 * ((4 * kh + 2 * h + hc) ^ (qc & 7));
            *(v8h*)(L.pt + off) = ph;
            *(v8bf*)(L.st + off) = sb;
        }
        // the columns of tile I landed, P^ and dS are written, the rows are read
        BQA_WAIT_VM(0);
        barrier_only();
        if (more) rows_issue(a, cp, bh, b, hq, I + 1, L.rt, w, l);
        // dV += P^T dO, dK += dS^T deq(Q): K-steps of 16 queries.  The A
        // operands (key = lane % 32, 8 queries) come from the query-major P^
        // and dS by transposing reads: in each 16-lane group, lane j names 4
        // keys (4 (j % 4) ..) of query j / 4, and lane i receives key i of
        // the 4 queries.
        {
            const int ch = co + lq;
            const int grp = l >> 4, li = l & 15;
            const int kcol = ko + 16 * (grp & 1) + 4 * (li & 3);
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                v4s tp[2], ts[2];
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                    const int row = 16 * st + 8 * (grp >> 1) + 4 * part + (li >> 2);
                    const int off = row * 128 + 16 * ((kcol >> 3) ^ (row & 7)) + 2 * (kcol & 7);
                    tp[part] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(L.pt + off));
                    ts[part] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(L.st + off));
                }
                const v8h ap = __builtin_bit_cast(v8h, v8s{tp[0][0], tp[0][1], tp[0][2], tp[0][3], tp[1][0], tp[1][1], tp[1][2], tp[1][3]});
                const v8bf as = __builtin_bit_cast(v8bf, v8s{ts[0][0], ts[0][1], ts[0][2], ts[0][3], ts[1][0], ts[1][1], ts[1][2], ts[1][3]});
                const int cq = 2 * st + h;                // 16-byte chunk of 8 queries
                const v8h bg = *(const v8h*)(L.gT + ch * 256 + 16 * (cq ^ fc256(ch)));
                const v8bf bq = *(const v8bf*)(L.qT + ch * 256 + 16 * (cq ^ fc256(ch)));
                dv = mfma_f16_32x32x16(ap, bg, dv);
                dk = mfma_bf16_32x32x16(as, bq, dk);
            }
        }
        // every wavefront is done with P^, dS and the columns, and the next
        // rows have landed: copy the next columns (they land during the next
        // step's P and dS, which do not read them)
        BQA_WAIT_VM(0);
        barrier_only();
        if (more) cols_issue(a, cp, bh, I + 1, L, w);
    }
    // dv reg i: key ko + 8 (i / 4) + 4 h + i % 4, channel co + lq; dO entered scaled by 2^k
    uint16_t* dvp = (uint16_t*)a.dv.p + b * a.dv.sB + hq * a.dv.sH;
    uint16_t* dkp = (uint16_t*)a.dk.p + b * a.dk.sB + hq * a.dk.sH;
    const int kdo = do_shift(a.do_amax[bh]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t kpos = (int64_t)J * TK + ko + 8 * (i >> 2) + 4 * h + (i & 3);
        dvp[kpos * a.dv.sN + co + lq] = f32_to_bf16_bits(__builtin_ldexpf(dv[i], -kdo));
        dkp[kpos * a.dk.sN + co + lq] = f32_to_bf16_bits(dk[i] * a.tau);
    }
}

// ------------------------------------------------------------------ dQ
struct LdsQq {
    KeyTile kt;
    uint8_t kT[D * TK * 2];      // deq(K)^T: 128 channels x 64 keys bf16
};

__device__ __forceinline__ void dq_issue(const QatBwdArgs& a, int bh, int J, LdsQq& T, int w, int l) {
    key_tile_issue(a, bh, J, T.kt, w, l);
#pragma unroll
    for (int u = 0; u < 4; ++u) {   // deq(K)^T: 16 x 1 KB (8 rows of 128 B)
        const int sgm = 4 * w + u, r = 8 * sgm + (l >> 3);
        lds_copy16((uint32_t)(2 * (r * a.N + 8 * ((l & 7) ^ fc128(r)))), a.kT + (int64_t)bh * D * a.N + J * TK,
                   lds_addr(T.kT + 1024 * sgm));
    }
}

__global__ __launch_bounds__(256, 2) void qbwd_dq_kernel(QatBwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsQq L[2];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int nkt = a.N / TK, nqt = a.N / TQ;
    const int I = blockIdx.x % nqt;
    const int bh = blockIdx.x / nqt, b = bh / a.H, hq = bh % a.H;
    const int qrow = I * TQ + 32 * w + lq;
    const int krow = sigma(lq);
    const float c = a.c_log2;
    RowIn rin;
    row_load(a, bh, b, hq, qrow, h, rin);
    v16f dq[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) dq[cb] = v16f{};
    dq_issue(a, bh, 0, L[0], w, l);
    BQA_WAIT_VM(0);
    barrier_only();
    for (int J = 0; J < nkt; ++J) {
        const int cur = J & 1;
        if (J + 1 < nkt) dq_issue(a, bh, J + 1, L[cur ^ 1], w, l);
        const LdsQq& T = L[cur];
        float p[2][16], pq[2][16], ds[2][16];
        tile_pds(T.kt, rin, c, krow, h, p, pq, ds);
        // dQ += dS deq(K): step st takes keys 32 (st / 2) + 16 h + 8 (st % 2) + e
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            v8bf ab;
#pragma unroll
            for (int e = 0; e < 8; ++e) ab[e] = (__bf16)ds[st >> 1][8 * (st & 1) + e];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int rr = 32 * cb + lq;
                const int ck = 4 * (st >> 1) + 2 * h + (st & 1);
                const v8bf bk = *(const v8bf*)(T.kT + rr * 128 + 16 * (ck ^ fc128(rr)));
                dq[cb] = mfma_bf16_32x32x16(ab, bk, dq[cb]);
            }
        }
        // the next key tile landed, and every wavefront is done with this one
        BQA_WAIT_VM(0);
        barrier_only();
    }
    // dq[cb] reg i: query 32 w + 8 (i / 4) + 4 h + i % 4, channel 32 cb + lq
    uint16_t* dqp = (uint16_t*)a.dq.p + b * a.dq.sB + hq * a.dq.sH;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t qr = (int64_t)I * TQ + 32 * w + 8 * (i >> 2) + 4 * h + (i & 3);
            dqp[qr * a.dq.sN + 32 * cb + lq] = f32_to_bf16_bits(dq[cb][i] * a.tau);
        }
}

}  // namespace

size_t ws_qat_bwd_bytes(int B, int H, int N, int d) {
    const size_t bhn = (size_t)B * H * N;
    // delta', deq(V), deq(Q)^T, deq(K)^T, dO^T, |dO| maxima per head
    return bhn * 4 + 4 * bhn * d * 2 + (((size_t)B * H * 4 + 255) & ~(size_t)255) + 256;
}

hipError_t launch_qat_bwd(QatBwdArgs a, Dense o_aux, void* ws, hipStream_t st) {
    const int64_t bhn = (int64_t)a.B * a.H * a.N;
    uint8_t* p = (uint8_t*)ws;
    float* delta = (float*)p;          p += bhn * 4;
    uint16_t* vdeq = (uint16_t*)p;     p += bhn * D * 2;
    uint16_t* qT = (uint16_t*)p;       p += bhn * D * 2;
    uint16_t* kT = (uint16_t*)p;       p += bhn * D * 2;
    uint16_t* doT = (uint16_t*)p;      p += bhn * D * 2;
    uint32_t* do_amax = (uint32_t*)p;
    a.delta = delta; a.vdeq = vdeq; a.qT = qT; a.kT = kT; a.doT = doT; a.do_amax = do_amax;

    const int nbh = a.B * a.H;
    fill_zero_kernel<<<(nbh + 255) / 256, 256, 0, st>>>(do_amax, nbh);
    qat_delta_kernel<<<(unsigned)((bhn + DELTA_ROWS - 1) / DELTA_ROWS), 256, 0, st>>>(a.d_o, o_aux, a.H, a.N, bhn, delta,
                                                                                    do_amax);
    const unsigned tg = (unsigned)((int64_t)a.B * a.H * (a.N / 64) * (D / 64));
    // V codes are channel-major [d][N/2]: transposing the (channel, token) grid gives token-major rows
    deq_t_fp4_kernel<<<tg, 256, 0, st>>>(a.vc, a.vs, D, a.N, vdeq);
    deq_t_fp4_kernel<<<tg, 256, 0, st>>>(a.qc, a.qs, a.N, D, qT);
    deq_t_fp4_kernel<<<tg, 256, 0, st>>>(a.kc, a.ks, a.N, D, kT);
    deq_t_bf16_kernel<<<tg, 256, 0, st>>>(a.d_o, a.H, a.N, D, do_amax, doT);
    qbwd_dkdv_kernel<<<a.B * a.H * (a.N / TK), 512, 0, st>>>(a);
    qbwd_dq_kernel<<<a.B * a.H * (a.N / TQ), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace bqa
