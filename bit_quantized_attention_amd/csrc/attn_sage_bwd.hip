// attn_sage_bwd.hip — SageBwd INT8 attention backward for gfx950.
//
// "SageBwd: A Trainable Low-bit Attention", Methodology 2 and Limitations
// (and the Chinese duplicate page): the backward recomputes S from the
// forward's INT8 codes and P = exp(s - L) from the saved log-sum-exp; of the
// five backward products four are INT8 with per-block scales (P^T dO, the
// recompute Q K^T, dS K and dS^T Q) and the softmax-gradient product
// dP = dO V^T stays in 16-bit (bf16 operands, fp32 accumulation).
// dS = P o (dP - delta), delta = rowsum(dO o O) with the forward's O.  P and
// dS are rounded to INT8 with one scale per 128 x 64 backward tile; dO is
// INT8 per 128-token block.  The fully INT8 variant (I8DP, the open problem
// of the page's Limitations) also runs dP on INT8 codes: the dO codes
// against V's codes per 64 tokens, times both scales.
//
// Kernels:
//   do_prep_kernel        delta per query row (fp32) and the channel-major
//                         INT8 codes of dO with their scales, one pass over
//                         dO and O
//   transpose2_i8_kernel  channel-major copies of the Q and K codes (the
//                         second operand of the INT8 products reads tokens
//                         contiguously per channel)
//   sbwd_dkdv_kernel      one workgroup per 64-key block, over the query
//                         tiles; the tile is computed with keys in lanes, so
//                         P^T and dS^T are already the A operands of
//                         dV = P^T dO and dK = dS^T Q in registers
//   sbwd_dq_kernel        one workgroup per 128-query tile, over the key
//                         tiles; queries in lanes, so dS is the A operand of
//                         dQ = dS K in registers
#include "common.hpp"
#include "internal.hpp"

namespace bqa {

namespace {

constexpr int D = 128;
constexpr int TQ = 128;   // backward tile: queries
constexpr int TK = 64;    // backward tile: keys

__device__ __forceinline__ int sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
// XOR patterns of the 16-byte chunks per row: rows read through sigma
// (..s) or by consecutive rows (..c), for 64 / 128 / 256-byte rows.
__device__ __forceinline__ int fs128(int r) { return ((r >> 1) & 7) ^ (((r >> 4) & 1) << 2); }
__device__ __forceinline__ int fs256(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }
__device__ __forceinline__ int fc64(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int fc128(int r) { return (r >> 1) & 7; }

// 16 values (one lane half's keys or queries of a 32-group) -> v4i of INT8
// codes with the tile's inverse scale (q8x4).
__device__ __forceinline__ v4i pack16(const float* x, float inv) {
    return v4i{q8x4(x[0], x[1], x[2], x[3], inv), q8x4(x[4], x[5], x[6], x[7], inv),
               q8x4(x[8], x[9], x[10], x[11], inv), q8x4(x[12], x[13], x[14], x[15], inv)};
}

// ------------------------------------------------------------------ preprocess
// dO in one pass per 128-row block: delta_i = sum_c dO[i, c] O[i, c] (one row
// per 16 lanes, 8 channels each, fma in channel order, then a butterfly over
// the 16 lanes), and the block's INT8 codes with one absmax scale per 128
// tokens (the token-block quantiser's arithmetic), written channel-major only
// ([BH][d][N], the layout the products read) through an LDS transpose.
__global__ __launch_bounds__(256) void do_prep_kernel(Dense dO, Dense O, int H, int N, float* __restrict__ delta,
                                                      float* __restrict__ dos, int8_t* __restrict__ doT,
                                                      int8_t* __restrict__ doc) {
    const int nb = N / 128;
    const int bh = blockIdx.x / nb, ib = blockIdx.x % nb;
    const int b = bh / H, h = bh % H;
    // thread: rows 4 q + u + 64 i (u < 4, i < 2), channels 8 part .. 8 part + 7
    const int tid = threadIdx.x, part = tid & 15, q = tid >> 4;
    const uint16_t* gb = (const uint16_t*)dO.p + b * dO.sB + h * dO.sH + (int64_t)ib * 128 * dO.sN + 8 * part;
    const uint16_t* ob = (const uint16_t*)O.p + b * O.sB + h * O.sH + (int64_t)ib * 128 * O.sN + 8 * part;
    v4i gv[2][4], ov[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            gv[i][u] = *(const v4i*)(gb + (int64_t)(4 * q + u + 64 * i) * dO.sN);
            ov[i][u] = *(const v4i*)(ob + (int64_t)(4 * q + u + 64 * i) * O.sN);
        }
    __shared__ uint32_t tT[D][33];     // codes, channel-major: words of 4 rows (stride 33: two lanes per bank at most)
    __shared__ float wmax[4];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t g2 = (uint32_t)gv[i][u][w], o2 = (uint32_t)ov[i][u][w];
                const float g0 = bf16_bits_to_f32((uint16_t)g2), g1 = bf16_bits_to_f32((uint16_t)(g2 >> 16));
                acc = __builtin_fmaf(g0, bf16_bits_to_f32((uint16_t)o2), acc);
                acc = __builtin_fmaf(g1, bf16_bits_to_f32((uint16_t)(o2 >> 16)), acc);
                am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(g0), __builtin_fabsf(g1)));
            }
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 16);
            if (part == 0) delta[(int64_t)bh * N + ib * 128 + 4 * q + u + 64 * i] = acc;
        }
    am = wave_max(am);
    if ((tid & 63) == 0) wmax[tid >> 6] = am;
    __syncthreads();
    const float bm = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    float inv = bm > 0.0f ? 127.0f / bm : 0.0f;
    float scale = bm / 127.0f;
    if (!(bm > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
    if (tid == 0) dos[(int64_t)bh * nb + ib] = scale;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float f[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t w2 = (uint32_t)gv[i][u][e >> 1];
                f[u] = bf16_bits_to_f32((uint16_t)((e & 1) ? (w2 >> 16) : w2));
            }
            // one channel, four consecutive rows; |f| <= bm, so |f * inv| <= 127
            tT[8 * part + e][q + 16 * i] = (uint32_t)q8x4(f[0], f[1], f[2], f[3], inv);
        }
    if (doc) {
        // the same codes row-major (the INT8 dP reads dO by rows): 8 channels of one row per thread and row
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w2 = (uint32_t)gv[i][u][e >> 1];
                    f[e] = bf16_bits_to_f32((uint16_t)((e & 1) ? (w2 >> 16) : w2));
                }
                const int64_t row = (int64_t)bh * N + ib * 128 + 4 * q + u + 64 * i;
                *(uint2*)(doc + row * D + 8 * part) = make_uint2((uint32_t)q8x4(f[0], f[1], f[2], f[3], inv),
                                                                 (uint32_t)q8x4(f[4], f[5], f[6], f[7], inv));
            }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int it = tid + 256 * k, c = it >> 3, sg = it & 7;
        const v4i y = {(int)tT[c][4 * sg], (int)tT[c][4 * sg + 1], (int)tT[c][4 * sg + 2], (int)tT[c][4 * sg + 3]};
        *(v4i*)(doT + ((int64_t)bh * D + c) * N + ib * 128 + 16 * sg) = y;
    }
}

// Channel-major copies of two [BH][N][d] int8 tensors (the Q and K codes) in
// one launch, 64 tokens x d per workgroup: a thread reads 8 channels of 4
// consecutive tokens, packs each channel's 4 bytes into one word (byte
// permutes), and the words cross LDS (row stride 17 words: no more than two
// lanes per bank) to 16-byte stores along the tokens.
__global__ __launch_bounds__(256) void transpose2_i8_kernel(const int8_t* __restrict__ a, const int8_t* __restrict__ b,
                                                            int8_t* __restrict__ aT, int8_t* __restrict__ bT, int N,
                                                            int tiles) {
    __shared__ uint32_t t[D][17];
    int blk = blockIdx.x;
    const bool second = blk >= tiles;
    if (second) blk -= tiles;
    const int8_t* in = second ? b : a;
    int8_t* out = second ? bT : aT;
    const int tilesN = N / 64;
    const int tn = blk % tilesN;
    const int64_t bh = blk / tilesN;
    const int tid = threadIdx.x, part = tid & 15, q = tid >> 4;       // tokens 4 q + u, channels 8 part ..
    const int8_t* src = in + (bh * N + (int64_t)tn * 64 + 4 * q) * D + 8 * part;
    v2i x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *(const v2i*)(src + (int64_t)u * D);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int w = e >> 2;
        const uint32_t sel = 0x0c0c0400u | (uint32_t)(e & 3) * 0x0101u;     // byte e&3 of the low source, then of the high
        const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)x[1][w], (uint32_t)x[0][w], sel);
        const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)x[3][w], (uint32_t)x[2][w], sel);
        t[8 * part + e][q] = p01 | (p23 << 16);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int it = tid + 256 * k, c = it >> 2, sg = it & 3;
        const v4i y = {(int)t[c][4 * sg], (int)t[c][4 * sg + 1], (int)t[c][4 * sg + 2], (int)t[c][4 * sg + 3]};
        *(v4i*)(out + (bh * D + c) * N + (int64_t)tn * 64 + 16 * sg) = y;
    }
}

// ------------------------------------------------------------------ dK, dV
// One workgroup of 8 wavefronts per 64-key block, over the query tiles.
// Scores of tile I: wavefront (kh, qg) computes S and dP for its 32 keys x
// 32 queries with keys in lanes, then P and dS; after the tile's maxima it
// writes their INT8 codes, key-major, to LDS.  Products of a tile: wavefront
// (kh, cq) accumulates dV and dK for its 32 keys x 32 channels over the
// tile's 128 queries (P^T and dS^T codes from LDS, channel-major dO and Q
// codes).  Each wavefront thus holds 32 accumulator registers, which lets
// two of them share a SIMD.  Step I runs the scores of tile I, then, between
// its two barriers, the products of tile I+1 under the encoding of tile I's
// codes, which are written after the second barrier.
//
// Query-side tiles: "A" (Q codes, dO bf16, log-sum-exp, delta) in two slots,
// "B" (channel-major dO and Q codes, read by the products only) in one.  The
// query tiles go in descending order; the copy of the next tile's A is
// issued at the start of a step, the copy of a tile's B after its codes are
// written: every copy has most of a step to land.
struct LdsKV {
    uint8_t q[2][TQ * D];       // Q codes of the query tile, 128 x 128 B (sigma reads)
    uint8_t dob[2][TQ * D * 2]; // dO bf16, 128 x 256 B (sigma reads)
    float lse[2][TQ];
    float dlt[2][TQ];
    uint8_t doT[D * TQ];        // dO codes channel-major, 128 ch x 128 B
    uint8_t qT[D * TQ];         // Q codes channel-major, 128 ch x 128 B
    uint8_t pc[TK * TQ];        // P^T codes, 64 keys x 128 B
    uint8_t dc[TK * TQ];        // dS^T codes
    float red[16];
};

// One wavefront's share of the copies of a query tile, as per-lane offsets
// from a tile base (the swizzles come from the source each lane names).
struct KvPlan {
    // copies per wavefront of an A tile (Q codes, dO, log-sum-exp / delta; a
    // B tile: 2 + 2): dO as bf16 takes 4, as INT8 codes 2
    template <bool I8DP>
    static constexpr int na() { return I8DP ? 2 + 2 + 1 : 2 + 4 + 1; }
    uint32_t q[2], g[4], t[2];
    __device__ __forceinline__ KvPlan(int w, int l, int N, int64_t g_sN) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {      // Q codes: 16 x 1 KB (8 rows of 128 B)
            const int r = 8 * (2 * w + u) + (l >> 3);
            q[u] = (uint32_t)(r * D + 16 * ((l & 7) ^ fs128(r)));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {      // dO bf16: 32 x 1 KB (4 rows of 256 B)
            const int r = 4 * (4 * w + u) + (l >> 4);
            g[u] = (uint32_t)(2 * (r * g_sN + 8 * ((l & 15) ^ fs256(r))));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {      // channel-major codes: 16 x 1 KB each (8 rows of 128 B)
            const int r = 8 * (2 * w + u) + (l >> 3);
            t[u] = (uint32_t)r * (uint32_t)N + (uint32_t)(16 * ((l & 7) ^ fc128(r)));
        }
    }
};

template <bool I8DP>
__device__ __forceinline__ void kv_copy_a(const SageBwdArgs& a, const KvPlan& cp, int bh, int b, int hq, int I, LdsKV& L,
                                          int slot, int w, int l) {
    const int q0 = I * TQ;
    const int8_t* qbase = a.qc + ((int64_t)bh * a.N + q0) * D;
#pragma unroll
    for (int u = 0; u < 2; ++u) lds_copy16(cp.q[u], qbase, lds_addr(L.q[slot] + 1024 * (2 * w + u)));
    if constexpr (I8DP) {
        // dO codes in the layout of the Q codes (128 x 128 B, sigma reads)
        const int8_t* cbase = a.doc + ((int64_t)bh * a.N + q0) * D;
#pragma unroll
        for (int u = 0; u < 2; ++u) lds_copy16(cp.q[u], cbase, lds_addr(L.dob[slot] + 1024 * (2 * w + u)));
    } else {
        const uint16_t* gbase = (const uint16_t*)a.d_o.p + b * a.d_o.sB + hq * a.d_o.sH + (int64_t)q0 * a.d_o.sN;
#pragma unroll
        for (int u = 0; u < 4; ++u) lds_copy16(cp.g[u], gbase, lds_addr(L.dob[slot] + 1024 * (4 * w + u)));
    }
    // log-sum-exp and delta of the tile: 256-byte copies by wavefronts 0-3,
    // repeated by 4-7 (same bytes) so every wavefront counts the same copies
    const int v = w & 3;
    if (v < 2) lds_copy4(4 * l, a.lse + (int64_t)bh * a.N + q0 + 64 * v, lds_addr(L.lse[slot] + 64 * v));
    else lds_copy4(4 * l, a.delta + (int64_t)bh * a.N + q0 + 64 * (v - 2), lds_addr(L.dlt[slot] + 64 * (v - 2)));
}
__device__ __forceinline__ void kv_copy_b(const SageBwdArgs& a, const KvPlan& cp, int bh, int I, LdsKV& L, int w) {
    const int q0 = I * TQ;
    const int8_t* gT = a.doT + (int64_t)bh * D * a.N + q0;
    const int8_t* qT = a.qT + (int64_t)bh * D * a.N + q0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        lds_copy16(cp.t[u], gT, lds_addr(L.doT + 1024 * (2 * w + u)));
        lds_copy16(cp.t[u], qT, lds_addr(L.qT + 1024 * (2 * w + u)));
    }
}

template <bool I8DP>
__global__ __launch_bounds__(512, 1) void sbwd_dkdv_kernel(SageBwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsKV L;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int nkt = a.N / TK, nqt = a.N / TQ;
    // consecutive workgroups take different heads (a head stays on one XCD);
    // ascending J: the longest query ranges first
    const int BH = a.B * a.H;
    const int J = blockIdx.x / BH;
    const int bh = blockIdx.x % BH, b = bh / a.H, hq = bh % a.H;
    const int kh = w & 1, qg = w >> 1;               // scores: 32 keys x 32 queries; products: 32 keys x 32 channels
    const int key = J * TK + 32 * kh + lq;
    const int qrow_s = sigma(lq);
    const float c = a.c_log2;
    const auto qs_u = uniform_ptr(a.qs + (int64_t)bh * nqt);
    const auto dos_u = uniform_ptr(a.dos + (int64_t)bh * nqt);
    const float ks = uniform_ptr(a.ks)[(int64_t)bh * nkt + J];
    const KvPlan cp(w, l, a.N, a.d_o.sN);

    // this lane's key: K codes (B operand of S = Q K^T) and V in bf16 (B operand of dP = dO V^T)
    v4i kb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kb[kk] = *(const v4i*)(a.kc + ((int64_t)bh * a.N + key) * D + 32 * kk + 16 * h);
    v8bf vb[I8DP ? 1 : 8];
    v4i vcb[I8DP ? 4 : 1];
    float vsc = 0.0f;
    if constexpr (I8DP) {
        // INT8 dP: this lane's key as V codes (B operand), the block's V scale
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vcb[kk] = *(const v4i*)(a.vc8 + ((int64_t)bh * a.N + key) * D + 32 * kk + 16 * h);
        vsc = uniform_ptr(a.vs8)[(int64_t)bh * nkt + J];
    } else {
        const uint16_t* vrow = (const uint16_t*)a.v.p + b * a.v.sB + hq * a.v.sH + (int64_t)key * a.v.sN;
#pragma unroll
        for (int st = 0; st < 8; ++st) vb[st] = *(const v8bf*)(vrow + 16 * st + 8 * h);
    }
    __builtin_amdgcn_s_waitcnt(0);

    v16f dv = v16f{}, dk = v16f{};                   // keys 32 kh + 8 (i/4) + 4 h + i%4, channel 32 qg + lq
    const int prow = 32 * kh + lq;                   // key row of the P^T / dS^T codes this lane writes and reads
    const int crow = 32 * qg + lq;                   // channel row of doT / qT this lane reads

    const int I0 = a.causal ? (J * TK) / TQ : 0;
    // query tiles in descending order: the key blocks of a head that run at
    // the same time read the same query tile, which then comes from L2
    kv_copy_a<I8DP>(a, cp, bh, b, hq, nqt - 1, L, 0, w, l);
    BQA_WAIT_VM(0);
    barrier_only();
    // The products of tile I+1 run in step I, between its two barriers, under
    // the vector work of tile I's codes: their MFMA results are folded into
    // dV, dK at the end of the step with the scales of tile I+1.
    auto products = [&](v16i& tv, v16i& tk) __attribute__((always_inline)) {
        tv = v16i{};
        tk = v16i{};
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const int ch = 2 * kq + h;
            const v4i ap = *(const v4i*)(L.pc + prow * 128 + 16 * (ch ^ fc128(prow)));
            const v4i ad = *(const v4i*)(L.dc + prow * 128 + 16 * (ch ^ fc128(prow)));
            const v4i bo = *(const v4i*)(L.doT + crow * 128 + 16 * (ch ^ fc128(crow)));
            const v4i bq = *(const v4i*)(L.qT + crow * 128 + 16 * (ch ^ fc128(crow)));
            tv = mfma_i8_32x32x32(ap, bo, tv);
            tk = mfma_i8_32x32x32(ad, bq, tk);
        }
    };
    auto fold = [&](const v16i& tv, const v16i& tk, float sv, float sk) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            dv[i] = __builtin_fmaf((float)tv[i], sv, dv[i]);
            dk[i] = __builtin_fmaf((float)tk[i], sk, dk[i]);
        }
    };
    float sv_prev = 0.0f, sk_prev = 0.0f;
    for (int I = nqt - 1; I >= I0; --I) {
        const int s = (nqt - 1 - I) & 1;
        const bool more = I > I0, prev = I < nqt - 1;
        if (more) kv_copy_a<I8DP>(a, cp, bh, b, hq, I - 1, L, s ^ 1, w, l);   // that slot's reads ended a step ago
        const float qsc = qs_u[I];
        const float sc = qsc * ks * c;
        // ---- scores: S (int32), dP (fp32) of 32 queries x 32 keys; reg i of half h = query 16h + i
        const int rq = 32 * qg + qrow_s;             // A row fed by this lane
        v16i sacc = v16i{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const v4i av = *(const v4i*)(L.q[s] + rq * 128 + 16 * ((2 * kk + h) ^ fs128(rq)));
            sacc = mfma_i8_32x32x32(av, kb[kk], sacc);
        }
        v16f dp = v16f{};
        if constexpr (I8DP) {
            v16i dpi = v16i{};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const v4i av = *(const v4i*)(L.dob[s] + rq * 128 + 16 * ((2 * kk + h) ^ fs128(rq)));
                dpi = mfma_i8_32x32x32(av, vcb[kk], dpi);
            }
            const float dsc = dos_u[I] * vsc;
#pragma unroll
            for (int i = 0; i < 16; ++i) dp[i] = (float)dpi[i] * dsc;
        } else {
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const v8bf av = *(const v8bf*)(L.dob[s] + rq * 256 + 16 * ((2 * st + h) ^ fs256(rq)));
                dp = mfma_bf16_32x32x16(av, vb[st], dp);
            }
        }
        const int qb0 = 32 * qg + 16 * h;            // tile-local query of register 0
        float P[16], dS[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const v4f lse4 = *(const v4f*)(L.lse[s] + qb0 + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                P[4 * u + e] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sacc[4 * u + e], sc, -lse4[e] * 1.4426950408889634f));
        }
        // causal: only the first query tile of the key block crosses the diagonal
        if (a.causal && I == I0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) P[i] = key > I * TQ + qb0 + i ? 0.0f : P[i];
        }
        float pmax = 0.0f, dmax = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const v4f dl4 = *(const v4f*)(L.dlt[s] + qb0 + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * u + e;
                dS[i] = P[i] * (dp[i] - dl4[e]);
                pmax = __builtin_fmaxf(pmax, P[i]);
                dmax = __builtin_fmaxf(dmax, __builtin_fabsf(dS[i]));
            }
        }
        // ---- one INT8 scale per tile for P and for dS (one exchange for both)
        pmax = wave_max(pmax);
        dmax = wave_max(dmax);
        if (l == 0) {
            L.red[w] = pmax;
            L.red[8 + w] = dmax;
        }
        // maxima written; B(I+1) landed (the copies of A(I-1) may stay in flight)
        if (more) BQA_WAIT_VM(KvPlan::na<I8DP>());
        else BQA_WAIT_VM(0);
        barrier_only();
        // ---- products of tile I+1 (codes and B written / landed before the barrier)
        v16i tv, tk;
        if (prev) products(tv, tk);
        {
            const v4f p0 = *(const v4f*)L.red, p1 = *(const v4f*)(L.red + 4);
            const v4f d0 = *(const v4f*)(L.red + 8), d1 = *(const v4f*)(L.red + 12);
            pmax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(p0[0], p0[1]), __builtin_fmaxf(p0[2], p0[3])),
                                   __builtin_fmaxf(__builtin_fmaxf(p1[0], p1[1]), __builtin_fmaxf(p1[2], p1[3])));
            dmax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(d0[0], d0[1]), __builtin_fmaxf(d0[2], d0[3])),
                                   __builtin_fmaxf(__builtin_fmaxf(d1[0], d1[1]), __builtin_fmaxf(d1[2], d1[3])));
        }
        const float inv_p = pmax > 0.0f ? 127.0f / pmax : 0.0f;
        const float inv_d = dmax > 0.0f ? 127.0f / dmax : 0.0f;
        const bool p_ok = inv_p != 0.0f && inv_p < __builtin_inff();
        const bool d_ok = inv_d != 0.0f && inv_d < __builtin_inff();
        const v4i pcode = p_ok ? pack16(P, inv_p) : v4i{};
        const v4i dcode = d_ok ? pack16(dS, inv_d) : v4i{};
        const float sv = p_ok ? pmax * (1.0f / 127.0f) * dos_u[I] : 0.0f;
        const float sk = d_ok ? dmax * (1.0f / 127.0f) * qsc * a.tau : 0.0f;
        // ---- every wavefront is done with the codes and B of tile I+1 and with
        // the maxima; A(I-1) landed
        BQA_WAIT_VM(0);
        barrier_only();
        const int wch = (2 * qg + h) ^ fc128(prow);  // this lane's 16 queries: chunk 2 qg + h of its key row
        *(v4i*)(L.pc + prow * 128 + 16 * wch) = pcode;
        *(v4i*)(L.dc + prow * 128 + 16 * wch) = dcode;
        kv_copy_b(a, cp, bh, I, L, w);               // lands during the next step's scores
        if (prev) fold(tv, tk, sv_prev, sk_prev);
        sv_prev = sv;
        sk_prev = sk;
    }
    // products of the last tile
    BQA_WAIT_VM(0);
    barrier_only();
    {
        v16i tv, tk;
        products(tv, tk);
        fold(tv, tk, sv_prev, sk_prev);
    }
    if (a.k_rn) {
        // QK-norm backward ("SageBwd", Methodology 4): dk = r (g - y (y . g))
        // per key row, y = k_raw r; a row's channels span 32 lanes of 4 waves
        __shared__ float red[4][TK];
        const uint16_t* kr = (const uint16_t*)a.k_raw.p + b * a.k_raw.sB + hq * a.k_raw.sH;
        float rr[16], y[16], t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t kpos = (int64_t)J * TK + 32 * kh + 8 * (i >> 2) + 4 * h + (i & 3);
            rr[i] = a.k_rn[(int64_t)bh * a.N + kpos];
            y[i] = bf16_bits_to_f32(kr[kpos * a.k_raw.sN + crow]) * rr[i];
            t[i] = y[i] * dk[i];
        }
#pragma unroll
        for (int off = 1; off < 32; off <<= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] += __shfl_xor(t[i], off);
        if (lq == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) red[qg][32 * kh + 8 * (i >> 2) + 4 * h + (i & 3)] = t[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kl = 32 * kh + 8 * (i >> 2) + 4 * h + (i & 3);
            const float T = (red[0][kl] + red[1][kl]) + (red[2][kl] + red[3][kl]);
            dk[i] = rr[i] * (dk[i] - y[i] * T);
        }
    }
    uint16_t* dvp = (uint16_t*)a.dv.p + b * a.dv.sB + hq * a.dv.sH;
    uint16_t* dkp = (uint16_t*)a.dk.p + b * a.dk.sB + hq * a.dk.sH;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t kpos = (int64_t)J * TK + 32 * kh + 8 * (i >> 2) + 4 * h + (i & 3);
        dvp[kpos * a.dv.sN + crow] = f32_to_bf16_bits(dv[i]);
        dkp[kpos * a.dk.sN + crow] = f32_to_bf16_bits(dk[i]);
    }
}

// ------------------------------------------------------------------ dQ
struct LdsQ {
    uint8_t k[TK * D];          // K codes of the key tile, 64 x 128 B (sigma reads)
    uint8_t vb[TK * D * 2];     // V bf16, 64 x 256 B (sigma reads)
    uint8_t kT[D * TK];         // K codes channel-major, 128 ch x 64 B
};

// Largest value over the 4 wavefronts: wavefront maxima through LDS (a
// barrier that leaves the copies in flight).
__device__ __forceinline__ float block_max_nc(float v, float* red, int w, int l) {
    v = wave_max(v);
    if (l == 0) red[w] = v;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's LDS write is done
    barrier_only();
    return __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

struct QPlan {
    uint32_t k[2], v[4], t[2];
    __device__ __forceinline__ QPlan(int w, int l, int Ntok, int64_t v_sN) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {      // K codes: 8 x 1 KB (8 rows of 128 B)
            const int r = 8 * (2 * w + u) + (l >> 3);
            k[u] = (uint32_t)(r * D + 16 * ((l & 7) ^ fs128(r)));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {      // V bf16: 16 x 1 KB (4 rows of 256 B)
            const int r = 4 * (4 * w + u) + (l >> 4);
            v[u] = (uint32_t)(2 * (r * v_sN + 8 * ((l & 15) ^ fs256(r))));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {      // channel-major K codes: 8 x 1 KB (16 rows of 64 B)
            const int r = 16 * (2 * w + u) + (l >> 2);
            t[u] = (uint32_t)r * (uint32_t)Ntok + (uint32_t)(16 * ((l & 3) ^ fc64(r)));
        }
    }
};

template <bool I8DP>
__device__ __forceinline__ void q_copy(const SageBwdArgs& a, const QPlan& cp, int bh, int b, int hq, int J, LdsQ& L,
                                       int w) {
    const int k0 = J * TK;
    const int8_t* kbase = a.kc + ((int64_t)bh * a.N + k0) * D;
#pragma unroll
    for (int u = 0; u < 2; ++u) lds_copy16(cp.k[u], kbase, lds_addr(L.k + 1024 * (2 * w + u)));
    if constexpr (I8DP) {
        // V codes in the layout of the K codes (64 x 128 B, sigma reads)
        const int8_t* vbase = a.vc8 + ((int64_t)bh * a.N + k0) * D;
#pragma unroll
        for (int u = 0; u < 2; ++u) lds_copy16(cp.k[u], vbase, lds_addr(L.vb + 1024 * (2 * w + u)));
    } else {
        const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.sB + hq * a.v.sH + (int64_t)k0 * a.v.sN;
#pragma unroll
        for (int u = 0; u < 4; ++u) lds_copy16(cp.v[u], vbase, lds_addr(L.vb + 1024 * (4 * w + u)));
    }
    const int8_t* tbase = a.kT + (int64_t)bh * D * a.N + k0;
#pragma unroll
    for (int u = 0; u < 2; ++u) lds_copy16(cp.t[u], tbase, lds_addr(L.kT + 1024 * (2 * w + u)));
}

template <bool I8DP>
__global__ __launch_bounds__(256, 2) void sbwd_dq_kernel(SageBwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsQ L[2];
    __shared__ float red[8];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int nkt = a.N / TK, nqt = a.N / TQ;
    // heaviest tiles first; consecutive workgroups take different heads (a
    // head stays on one XCD, where its query tiles sweep the key tiles together)
    const int BH = a.B * a.H;
    const int I = nqt - 1 - (int)(blockIdx.x / BH);
    const int bh = blockIdx.x % BH, b = bh / a.H, hq = bh % a.H;
    const int qrow = I * TQ + 32 * w + lq;
    const int krow = sigma(lq);
    const float c = a.c_log2;
    const float qsc = uniform_ptr(a.qs)[(int64_t)bh * nqt + I];
    const auto ks_u = uniform_ptr(a.ks + (int64_t)bh * nkt);
    const QPlan cp(w, l, a.N, a.v.sN);

    // this lane's query: codes (B operand of S^T = K Q^T), dO bf16 (B operand of dP^T = V dO^T)
    v4i qb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = *(const v4i*)(a.qc + ((int64_t)bh * a.N + qrow) * D + 32 * kk + 16 * h);
    v8bf gb[I8DP ? 1 : 8];
    v4i gcb[I8DP ? 4 : 1];
    float dsq = 0.0f;
    if constexpr (I8DP) {
        // INT8 dP: this lane's query as dO codes (B operand of dP^T = V dO^T)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) gcb[kk] = *(const v4i*)(a.doc + ((int64_t)bh * a.N + qrow) * D + 32 * kk + 16 * h);
        dsq = uniform_ptr(a.dos)[(int64_t)bh * nqt + I];
    } else {
        const uint16_t* grow = (const uint16_t*)a.d_o.p + b * a.d_o.sB + hq * a.d_o.sH + (int64_t)qrow * a.d_o.sN;
#pragma unroll
        for (int st = 0; st < 8; ++st) gb[st] = *(const v8bf*)(grow + 16 * st + 8 * h);
    }
    const float lse2 = a.lse[(int64_t)bh * a.N + qrow] * 1.4426950408889634f;
    const float dlt = a.delta[(int64_t)bh * a.N + qrow];
    __builtin_amdgcn_s_waitcnt(0);

    v16f dq[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) dq[cb] = v16f{};

    const int nJ = a.causal ? (I * TQ + TQ - 1) / TK + 1 : nkt;
    q_copy<I8DP>(a, cp, bh, b, hq, 0, L[0], w);
    BQA_WAIT_VM(0);
    barrier_only();
    for (int J = 0; J < nJ; ++J) {
        const int cur = J & 1;
        const bool more = J + 1 < nJ;
        if (more) q_copy<I8DP>(a, cp, bh, b, hq, J + 1, L[cur ^ 1], w);   // that buffer's reads ended a step ago
        const LdsQ& T = L[cur];
        const float ks = ks_u[J];
        const float sc = qsc * ks * c;
        // causal: key tiles past the first query of the tile cross the diagonal
        const bool diag = a.causal && J * TK + TK - 1 > I * TQ;
        float dS[2][16];
        float dmax = 0.0f;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int rk = 32 * g + krow;
            v16i sacc = v16i{};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const v4i av = *(const v4i*)(T.k + rk * 128 + 16 * ((2 * kk + h) ^ fs128(rk)));
                sacc = mfma_i8_32x32x32(av, qb[kk], sacc);
            }
            v16f dp = v16f{};
            if constexpr (I8DP) {
                v16i dpi = v16i{};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const v4i av = *(const v4i*)(T.vb + rk * 128 + 16 * ((2 * kk + h) ^ fs128(rk)));
                    dpi = mfma_i8_32x32x32(av, gcb[kk], dpi);
                }
                const float dsc = dsq * uniform_ptr(a.vs8)[(int64_t)bh * nkt + J];
#pragma unroll
                for (int i = 0; i < 16; ++i) dp[i] = (float)dpi[i] * dsc;
            } else {
#pragma unroll
                for (int st = 0; st < 8; ++st) {
                    const v8bf av = *(const v8bf*)(T.vb + rk * 256 + 16 * ((2 * st + h) ^ fs256(rk)));
                    dp = mfma_bf16_32x32x16(av, gb[st], dp);
                }
            }
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sacc[i], sc, -lse2));
            if (diag) {
#pragma unroll
                for (int i = 0; i < 16; ++i) p[i] = J * TK + 32 * g + 16 * h + i > qrow ? 0.0f : p[i];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                dS[g][i] = p[i] * (dp[i] - dlt);
                dmax = __builtin_fmaxf(dmax, __builtin_fabsf(dS[g][i]));
            }
        }
        dmax = block_max_nc(dmax, red + 4 * (J & 1), w, l);
        const float inv_d = dmax > 0.0f ? 127.0f / dmax : 0.0f;
        const bool d_ok = inv_d != 0.0f && inv_d < __builtin_inff();
        v4i da[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) da[g] = d_ok ? pack16(dS[g], inv_d) : v4i{};
        const float sq = d_ok ? dmax * (1.0f / 127.0f) * ks * a.tau : 0.0f;
        // dQ += tau dS K: A = dS (queries x keys) from registers, B = K codes channel-major
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int rr = 32 * cb + lq;
            v16i t = v16i{};
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const v4i bk = *(const v4i*)(T.kT + rr * 64 + 16 * ((2 * g + h) ^ fc64(rr)));
                t = mfma_i8_32x32x32(da[g], bk, t);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) dq[cb][i] = __builtin_fmaf((float)t[i], sq, dq[cb][i]);
        }
        // the next key tile landed, and every wavefront is done with this one
        BQA_WAIT_VM(0);
        barrier_only();
    }
    // dq[cb] reg i: query 32 w + 8 (i / 4) + 4 h + i % 4, channel 32 cb + lq
    if (a.q_rn) {
        // QK-norm backward: dq = r (g - y (y . g)), y = q_raw r; a row's
        // channels span the 32 lanes of one half-wavefront (4 per lane)
        const uint16_t* qr = (const uint16_t*)a.q_raw.p + b * a.q_raw.sB + hq * a.q_raw.sH;
        float rr[16], t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t row = (int64_t)I * TQ + 32 * w + 8 * (i >> 2) + 4 * h + (i & 3);
            rr[i] = a.q_rn[(int64_t)bh * a.N + row];
            float acc = 0.0f;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                acc = __builtin_fmaf(bf16_bits_to_f32(qr[row * a.q_raw.sN + 32 * cb + lq]) * rr[i], dq[cb][i], acc);
            t[i] = acc;
        }
#pragma unroll
        for (int off = 1; off < 32; off <<= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] += __shfl_xor(t[i], off);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t row = (int64_t)I * TQ + 32 * w + 8 * (i >> 2) + 4 * h + (i & 3);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const float y = bf16_bits_to_f32(qr[row * a.q_raw.sN + 32 * cb + lq]) * rr[i];
                dq[cb][i] = rr[i] * (dq[cb][i] - y * t[i]);
            }
        }
    }
    uint16_t* dqp = (uint16_t*)a.dq.p + b * a.dq.sB + hq * a.dq.sH;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t qr = (int64_t)I * TQ + 32 * w + 8 * (i >> 2) + 4 * h + (i & 3);
            dqp[qr * a.dq.sN + 32 * cb + lq] = f32_to_bf16_bits(dq[cb][i]);
        }
}

}  // namespace

size_t ws_sage_bwd_bytes(int B, int H, int N, int d) {
    const size_t bhn = (size_t)B * H * N;
    return bhn * 4                 // delta
           + (bhn / 128) * 4       // dO scales
           + 4 * bhn * d           // channel-major dO, Q, K codes; row-major dO codes (INT8 dP)
           + 256;
}

hipError_t launch_sage_bwd(SageBwdArgs a, Dense o, void* ws, hipStream_t st) {
    const int64_t bhn = (int64_t)a.B * a.H * a.N;
    uint8_t* p = (uint8_t*)ws;
    float* delta = (float*)p;                 p += bhn * 4;
    float* dos = (float*)p;                   p += (bhn / 128) * 4;
    p = (uint8_t*)(((uintptr_t)p + 15) & ~(uintptr_t)15);
    int8_t* doT = (int8_t*)p;                 p += bhn * D;
    int8_t* qT = (int8_t*)p;                  p += bhn * D;
    int8_t* kT = (int8_t*)p;                  p += bhn * D;
    const bool i8dp = a.vc8 != nullptr;
    a.delta = delta; a.dos = dos; a.doT = doT; a.qT = qT; a.kT = kT;
    a.doc = i8dp ? (int8_t*)p : nullptr;

    do_prep_kernel<<<(unsigned)(bhn / 128), 256, 0, st>>>(a.d_o, o, a.H, a.N, delta, dos, doT, a.doc);
    const int tiles = (int)((int64_t)a.B * a.H * (a.N / 64));
    transpose2_i8_kernel<<<2 * tiles, 256, 0, st>>>(a.qc, a.kc, qT, kT, a.N, tiles);
    if (i8dp) {
        sbwd_dkdv_kernel<true><<<a.B * a.H * (a.N / TK), 512, 0, st>>>(a);
        sbwd_dq_kernel<true><<<a.B * a.H * (a.N / TQ), 256, 0, st>>>(a);
    } else {
        sbwd_dkdv_kernel<false><<<a.B * a.H * (a.N / TK), 512, 0, st>>>(a);
        sbwd_dq_kernel<false><<<a.B * a.H * (a.N / TQ), 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace bqa
