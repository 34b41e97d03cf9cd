// attn_qat.hip — Attn-QAT FP4 attention forward for gfx950.
//
// "Attn-QAT: 4-Bit Attention With Quantization-Aware Training", technical
// summary §2: the forward runs Q K^T and P.V as FP4 products (MXFP4 here:
// e2m1 values with an E8M0 scale per 32 elements, on the scaled f8f6f4
// matrix instructions), P quantised per 32 keys of a row with no smoothing or
// two-level step (§2 Implementation), and — for training — emits the
// high-precision auxiliary output O' = sum bf16(P) Vhat / l next to O
// (Principle 2).  The row sum l accumulates the unrounded P.
//
// Layout (inference, no O'): one workgroup of 8 wavefronts per 128 query
// rows, 16 rows per wavefront on the 16 x 16 matrix instructions, S^T =
// Khat Qhat^T so that each lane owns one query row; key tiles of 128 keys.
// The training forward (with O') keeps 32-row wavefronts and tiles of 64 keys
// (described with its kernel below).
// The rows of S MFMA b are the keys 32 (r / 4) + 4 b + r % 4, so lane l holds
// the 32 consecutive keys 32 (l / 16) .. + 31 of the tile: one whole MX block
// of P, whose codes are the lane's B operand of P.V as they stand.
//
// Online softmax: FlashAttention-2's running row maximum M of the raw scores,
// P = exp2((s - M) c) with c = tau log2(e), and O, O' and l scaled by
// exp2((M_old - M_new) c) whenever a tile raises M in any lane of the
// wavefront.  The difference s - M is exact near the maximum (both are fp32
// values within a factor of two), so the P of the score that set M is exactly
// 1 and the P near it are as accurate as fp32 allows: their MXFP4 codes,
// whose top steps are 33-50 %, then match the exact arithmetic's.  M of each
// row is also reported (row_max), for the backward to round P the same way.
//
// O' uses deq(Vhat) in bf16, prepared once per call by vdeq_kernel into a
// channel-major workspace tensor.
//
// LDS tiles are chunk-major, so that each group of 16 lanes reads one
// contiguous 256-byte span: K codes, chunk g (channels 32 g .. + 31) of the
// key at position p at kc + 2048 g + 16 p, position p = 16 b + 4 a + c holding
// key 32 a + 4 b + c (the order the S instructions read); K scales, the key at
// position p at word p; V^T codes, chunk g (keys 32 g .. + 31) of channel ch at
// vc + 2048 g + 16 ch; V scales channel-major.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace bqa {

namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int KB = 128;   // keys per tile
constexpr int D = 128;    // head dimension

struct LdsQ {
    uint8_t kc[KB * D / 2];              // K codes, chunk-major
    uint8_t ks[KB * D / 32];             // K E8M0 scales, by position
    uint8_t vc[D * KB / 2];              // Vhat^T codes, chunk-major
    uint8_t vs[D * KB / 32];             // Vhat^T scales, 4 per channel
};
__device__ __forceinline__ int key_at(int p) { return 32 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3); }

// Issue the copies of the key tile at t0 into L, all direct copies.
__device__ __forceinline__ void tile_issue(const QatFwdArgs& a, int bhk, int t0, LdsQ& L, int w, int l) {
    const uint8_t* kbase = a.kc + ((int64_t)bhk * a.Nk + t0) * (D / 2);
    const uint8_t* vbase = a.vc + (int64_t)bhk * D * (a.Nk / 2) + t0 / 2;
    const int j = w >> 1, p = 64 * (w & 1) + l;       // wavefront w: chunk w / 2, positions / channels 64 (w % 2) ..
    lds_copy16((uint32_t)(key_at(p) * (D / 2) + 16 * j), kbase, lds_addr(L.kc + 1024 * w));
    lds_copy16((uint32_t)p * (uint32_t)(a.Nk / 2) + (uint32_t)(16 * j), vbase, lds_addr(L.vc + 1024 * w));
    if (w < 2) {          // K scales: positions 64 w .. + 63
        lds_copy4((uint32_t)(4 * key_at(64 * w + l)), a.ks + ((int64_t)bhk * a.Nk + t0) * (D / 32),
                  lds_addr(L.ks + 256 * w));
    } else if (w < 4) {   // V scales: channel 64 (w - 2) + l, its four bytes for this tile
        lds_copy4((uint32_t)l * (uint32_t)(a.Nk / 32), a.vs + ((int64_t)bhk * D + 64 * (w - 2)) * (a.Nk / 32) + t0 / 32,
                  lds_addr(L.vs + 256 * (w - 2)));
    }
}

// The 8 S^T instructions of a key tile: s[b][i] is the raw fp32 score (before
// tau) of key 32 g + 4 b + i against this lane's query.
__device__ __forceinline__ void qk_block16(const uint8_t* kc, const uint8_t* ks, v4i qb, int qsb, int g, int q,
                                           v4f (&s)[8]) {
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
        s[bb] = mfma_f4_16x16x128(*(const v4i*)(kc + 2048 * g + 16 * q + 256 * bb), (int)ks[4 * q + g + 64 * bb], qb,
                                  qsb, v4f{});
}

__global__ __launch_bounds__(512, 4) void qat_fwd_kernel(QatFwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsQ lds[2];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, q = l & 15;
    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
    // contiguous range of (head, query block) so that the workgroups sharing
    // an XCD's L2 also share a head's K and V.
    const int nqt = (a.Nq + BM - 1) / BM;
    const int grid = gridDim.x;
    const int bid = (grid & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3);
    const int qt = bid % nqt;
    const int bh = bid / nqt, b = bh / a.Hq, hq = bh % a.Hq;
    const int bhk = b * a.Hkv + hq / (a.Hq / a.Hkv);
    const int qrow = qt * BM + 16 * w + q;
    const bool row_ok = qrow < a.Nq;

    // this lane's query codes: B operand of S^T, channels 32 g .. + 31, and their scale
    const v4i qb = row_ok ? *(const v4i*)(a.qc + ((int64_t)bh * a.Nq + qrow) * (D / 2) + 16 * g) : v4i{};
    const int qsb = row_ok ? (int)a.qs[((int64_t)bh * a.Nq + qrow) * (D / 32) + g] : 0;

    v4f oacc[D / 16];   // O^T tile cb: channels 16 cb + 4 g + i of row q
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) oacc[cb] = v4f{};
    float m_run = -__builtin_inff();          // running maximum of the raw scores
    float l_run = 0.0f;                        // this lane's share of the row sum
    const float c = a.c_log2;
    const int n_tiles = a.Nk / KB;

    tile_issue(a, bhk, 0, lds[0], w, l);
    BQA_WAIT_VM(0);
    barrier_only();

    auto step = [&](auto slot, int j) __attribute__((always_inline)) {
        constexpr int SB = decltype(slot)::value;
        if (j + 1 < n_tiles) tile_issue(a, bhk, (j + 1) * KB, lds[SB ^ 1], w, l);
        const LdsQ& L = lds[SB];
        v4f s[8];
        qk_block16(L.kc, L.ks, qb, qsb, g, q, s);
        // ---- the lane's MX block maximum, the row's over its four lanes; the
        // accumulators follow the running maximum
        float gm = max3f(s[0][0], s[0][1], s[0][2]);
#pragma unroll
        for (int k = 3; k < 31; k += 2) gm = max3f(gm, s[k >> 2][k & 3], s[(k + 1) >> 2][(k + 1) & 3]);
        gm = max2f(gm, s[7][3]);
        const float m_new = max2f(m_run, quad_max16(gm));
        if (__any(m_new > m_run)) {
            const float f = m_new > m_run ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
            l_run *= f;
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[cb][i] *= f;
        }
        m_run = m_new;
        float ps[4];
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[bb][i] = __builtin_amdgcn_exp2f((s[bb][i] - m_run) * c);
                ps[i] = bb == 0 ? s[bb][i] : ps[i] + s[bb][i];
            }
        l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        // ---- MXFP4 P of the lane's block: P is monotone in the score, so the
        // block's largest P is the P of its largest score
        const int e = mx_exponent(__builtin_amdgcn_exp2f((gm - m_run) * c));
        const float sc = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
        v4i pb;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            // the four conversions fill the word: its old value is moot
            uint32_t x = __builtin_bit_cast(uint32_t, s[2 * wd][0]);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[2 * wd][0], s[2 * wd][1], sc, 0);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[2 * wd][2], s[2 * wd][3], sc, 1);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[2 * wd + 1][0], s[2 * wd + 1][1], sc, 2);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[2 * wd + 1][2], s[2 * wd + 1][3], sc, 3);
            pb[wd] = (int)x;
        }
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
            oacc[cb] = mfma_f4_16x16x128(*(const v4i*)(L.vc + 2048 * g + 16 * q + 256 * cb), (int)L.vs[4 * q + g + 64 * cb],
                                         pb, e + 127, oacc[cb]);
        BQA_WAIT_VM(0);   // the tile copies have landed
        barrier_only();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    for (int j = 0; j < n_tiles; j += 2) {
        step(I0{}, j);
        if (j + 1 >= n_tiles) break;
        step(I1{}, j + 1);
    }

    const float l_tot = quad_sum16(l_run);
    if (!row_ok) return;
    const float inv_l = 1.0f / l_tot;
    uint16_t* orow = (uint16_t*)a.o.p + b * a.o.sB + hq * a.o.sH + (int64_t)qrow * a.o.sN;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
        uint16_t o4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = f32_to_bf16_bits(oacc[cb][i] * inv_l);
        *(uint2*)(orow + 16 * cb + 4 * g) =
            make_uint2((uint32_t)o4[0] | ((uint32_t)o4[1] << 16), (uint32_t)o4[2] | ((uint32_t)o4[3] << 16));
    }
    if (a.lse && g == 0) a.lse[(int64_t)bh * a.Nq + qrow] = __builtin_fmaf(m_run, c, __log2f(l_tot)) * 0.6931471805599453f;
    if (a.row_max && g == 0) a.row_max[(int64_t)bh * a.Nq + qrow] = m_run;
}

// ---------------------------------------------------------------------------
// The forward with O' (training): 4 wavefronts of 32 query rows on the 32 x 32
// matrix instructions, key tiles of 64.  S^T = Khat Qhat^T, each lane owning
// one query row and, through the sigma row permutation, 16 consecutive keys
// per 32-key half of a tile; the 32 keys of an MX block of P sit in two lane
// halves, and one permlane32 swap per code word gives each half one whole
// block (in key order) as the B operand of P.V.  With O' a 16-row layout
// needs about 200 registers and 100 KB of LDS per 128 rows, one workgroup per
// CU; this layout keeps two per CU.
constexpr int BN = 64;    // keys per tile of the O' kernel
constexpr int NBUF = 2;

__device__ __forceinline__ int sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// 64-byte rows (K codes): rows read through sigma hit distinct bank groups
__device__ __forceinline__ int swz64(int r, int c) { return r * 64 + 16 * (c ^ (((r >> 2) & 3) ^ (((r >> 4) & 1) << 1))); }
// 32-byte rows (Vhat^T codes, consecutive rows)
__device__ __forceinline__ int swz32(int r, int c) { return r * 32 + 16 * (c ^ ((r >> 3) & 1)); }
// 128-byte rows (deq(Vhat)^T bf16, consecutive rows)
__device__ __forceinline__ int swz128(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

struct LdsAux {
    uint8_t kc[BN * D / 2];        // K codes, 64 rows x 64 B
    uint8_t ks[BN * D / 32];       // K E8M0 scales, 64 rows x 4
    uint8_t vc[D * BN / 2];        // Vhat^T codes, 128 rows x 32 B
    uint8_t vs[D * BN / 32];       // Vhat^T scales, 128 rows x 2
    uint8_t vb[D * BN * 2];        // deq(Vhat)^T bf16, 128 rows x 128 B
};

// Direct global -> LDS copies (global_load_lds): every lane names its global
// source, the data lands at LDS base + 16 x lane (4 x lane for dwords), so
// the swizzled layouts are produced by choosing which source each lane reads.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// Issue the copies of key tile t0 into L (K codes and scales, Vhat^T codes,
// and for O' the bf16 deq(Vhat)^T); Vhat's scales come back in a register
// (128 strided 2-byte values) and are stored by vs_store.
__device__ __forceinline__ uint32_t tile_issue_aux(const QatFwdArgs& a, int bhk, int t0, LdsAux& L, int w, int l, int tid) {
    {   // K codes: wave w fills rows 16w .. 16w + 15
        const int r = 16 * w + (l >> 2);
        const int c = (l & 3) ^ (((r >> 2) & 3) ^ (((r >> 4) & 1) << 1));
        dma16(a.kc + ((int64_t)bhk * a.Nk + t0 + r) * (D / 2) + 16 * c, L.kc + 1024 * w);
    }
    {   // Vhat^T codes: wave w fills rows 32w .. 32w + 31
        const int r = 32 * w + (l >> 1);
        const int c = (l & 1) ^ ((r >> 3) & 1);
        dma16(a.vc + ((int64_t)bhk * D + r) * (a.Nk / 2) + t0 / 2 + 16 * c, L.vc + 1024 * w);
    }
    if (w == 0) dma4(a.ks + ((int64_t)bhk * a.Nk + t0 + l) * (D / 32), L.ks);
    {
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // 1 KB segments 4w + u: rows 8 (4w + u) .. + 7
            const int sgm = 4 * w + u, r = 8 * sgm + (l >> 3);
            const int c = (l & 7) ^ ((r >> 1) & 7);
            dma16(a.vdeq + ((int64_t)bhk * D + r) * a.Nk + t0 + 8 * c, L.vb + 1024 * sgm);
        }
    }
    return tid < 128 ? (uint32_t)*(const uint16_t*)(a.vs + ((int64_t)bhk * D + tid) * (a.Nk / 32) + t0 / 32) : 0u;
}

__device__ __forceinline__ void vs_store_aux(uint32_t vs, LdsAux& L, int tid) {
    if (tid < 128) *(uint16_t*)(L.vs + 2 * tid) = (uint16_t)vs;
}

// S^T tile (64 keys x 32 queries) from MXFP4 codes: acc0 keys 16h + i,
// acc1 keys 32 + 16h + i; raw fp32 products (before tau).
__device__ __forceinline__ void qk_tile_mx(const LdsAux& L, const v4i* qb, const int* qsb, int krow, int h, v16f& acc0,
                                           v16f& acc1) {
    acc0 = v16f{};
    acc1 = v16f{};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const v4i a0 = *(const v4i*)(L.kc + swz64(krow, 2 * kk + h));
        const v4i a1 = *(const v4i*)(L.kc + swz64(32 + krow, 2 * kk + h));
        const int s0 = L.ks[4 * krow + 2 * kk + h], s1 = L.ks[4 * (32 + krow) + 2 * kk + h];
        acc0 = mfma_f4_32x32x64(a0, s0, qb[kk], qsb[kk], acc0);
        acc1 = mfma_f4_32x32x64(a1, s1, qb[kk], qsb[kk], acc1);
    }
}

__global__ __launch_bounds__(256, 2) void qat_aux_kernel(QatFwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsAux lds[NBUF];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
    // contiguous range of (head, query block) so that the workgroups sharing
    // an XCD's L2 also share a head's K and V.
    const int nqt = (a.Nq + BM - 1) / BM;
    const int grid = gridDim.x;
    const int bid = (grid & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3);
    const int qt = bid % nqt;
    const int bh = bid / nqt, b = bh / a.Hq, hq = bh % a.Hq;
    const int bhk = b * a.Hkv + hq / (a.Hq / a.Hkv);
    const int qrow = qt * BM + 32 * w + lq;
    const bool row_ok = qrow < a.Nq;
    const int krow = sigma(lq);

    // this lane's query codes: B operand of S^T, Q[qrow][64kk + 32h .. +32) and its scale
    v4i qb[2];
    int qsb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        qb[kk] = row_ok ? *(const v4i*)(a.qc + ((int64_t)bh * a.Nq + qrow) * (D / 2) + 32 * kk + 16 * h) : v4i{};
        qsb[kk] = row_ok ? (int)a.qs[((int64_t)bh * a.Nq + qrow) * (D / 32) + 2 * kk + h] : 0;
    }
    __builtin_amdgcn_s_waitcnt(0);

    v16f oacc[D / 32], xacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = v16f{};
#pragma unroll
    for (int cb = 0; cb < (D / 32); ++cb) xacc[cb] = v16f{};
    float m_run = -__builtin_inff();          // running maximum of the raw scores
    float l_run = 0.0f;                        // this lane half's share of the row sum
    const float c = a.c_log2;
    const int n_tiles = a.Nk / BN;

    vs_store_aux(tile_issue_aux(a, bhk, 0, lds[0], w, l, tid), lds[0], tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // one copy of the tile code (the LDS buffer index is a run-time value): two
    // copies, one per buffer, cost the allocator 60 registers and spilled
    auto body = [&](int j, int B0) __attribute__((always_inline)) {
        uint32_t vs_next = 0;
        if (j + 1 < n_tiles) vs_next = tile_issue_aux(a, bhk, (j + 1) * BN, lds[B0 ^ 1], w, l, tid);
        const LdsAux& L = lds[B0];
        v16f s0, s1;
        qk_tile_mx(L, qb, qsb, krow, h, s0, s1);
        // ---- block maxima of the raw scores: keys 0..31 (s0 of both halves), 32..63 (s1)
        float b0 = __builtin_fmaxf(s0[0], s0[1]), b1 = __builtin_fmaxf(s1[0], s1[1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) {
            b0 = __builtin_fmaxf(__builtin_fmaxf(b0, s0[i]), s0[i + 1]);
            b1 = __builtin_fmaxf(__builtin_fmaxf(b1, s1[i]), s1[i + 1]);
        }
        b0 = __builtin_fmaxf(b0, partner32f(b0));
        b1 = __builtin_fmaxf(b1, partner32f(b1));
        // ---- running maximum; the accumulators follow it
        const float m_new = __builtin_fmaxf(m_run, __builtin_fmaxf(b0, b1));
        if (__any(m_new > m_run)) {
            const float f = m_new > m_run ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
            l_run *= f;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[cb][i] *= f;
            {
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) xacc[cb][i] *= f;
            }
        }
        m_run = m_new;
        float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = __builtin_amdgcn_exp2f((s0[i] - m_run) * c);
            s1[i] = __builtin_amdgcn_exp2f((s1[i] - m_run) * c);
            ps[i & 1] += s0[i];
            ps[2 + (i & 1)] += s1[i];
        }
        l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        // ---- MXFP4 P per 32-key block: P is monotone in the score, so the
        // block's largest P is the P of its largest score
        const int e0 = mx_exponent(__builtin_amdgcn_exp2f((b0 - m_run) * c));
        const int e1 = mx_exponent(__builtin_amdgcn_exp2f((b1 - m_run) * c));
        const float sc0 = __builtin_bit_cast(float, (uint32_t)(e0 + 127) << 23);
        const float sc1 = __builtin_bit_cast(float, (uint32_t)(e1 + 127) << 23);
        uint32_t p0w[2], p1w[2];
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
            uint32_t x0 = 0, x1 = 0;
            x0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x0, s0[8 * wd + 0], s0[8 * wd + 1], sc0, 0);
            x0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x0, s0[8 * wd + 2], s0[8 * wd + 3], sc0, 1);
            x0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x0, s0[8 * wd + 4], s0[8 * wd + 5], sc0, 2);
            x0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x0, s0[8 * wd + 6], s0[8 * wd + 7], sc0, 3);
            x1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x1, s1[8 * wd + 0], s1[8 * wd + 1], sc1, 0);
            x1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x1, s1[8 * wd + 2], s1[8 * wd + 3], sc1, 1);
            x1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x1, s1[8 * wd + 4], s1[8 * wd + 5], sc1, 2);
            x1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x1, s1[8 * wd + 6], s1[8 * wd + 7], sc1, 3);
            p0w[wd] = x0;
            p1w[wd] = x1;
        }
        // half 0 takes block 0 (own keys 0..15, partner's 16..31), half 1 block 1
        const v2i r0 = __builtin_amdgcn_permlane32_swap((int)p0w[0], (int)p1w[0], false, false);
        const v2i r1 = __builtin_amdgcn_permlane32_swap((int)p0w[1], (int)p1w[1], false, false);
        const v4i pb = {r0[0], r1[0], r0[1], r1[1]};
        const int psc = (h ? e1 : e0) + 127;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
            const int r = 32 * cb + lq;
            const v4i av = *(const v4i*)(L.vc + swz32(r, h));
            oacc[cb] = mfma_f4_32x32x64(av, (int)L.vs[2 * r + h], pb, psc, oacc[cb]);
        }
        {
            // O' = bf16(P) . deq(Vhat): four 16-key steps, keys 32(s/2) + 16h + 8(s%2) + e
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                v8bf pbf;
#pragma unroll
                for (int e = 0; e < 8; ++e) pbf[e] = (__bf16)(s < 2 ? s0[8 * (s % 2) + e] : s1[8 * (s % 2) + e]);
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb) {
                    const v8bf av = *(const v8bf*)(L.vb + swz128(32 * cb + lq, 4 * (s / 2) + 2 * h + (s % 2)));
                    xacc[cb] = mfma_bf16_32x32x16(av, pbf, xacc[cb]);
                }
            }
        }
        if (j + 1 < n_tiles) vs_store_aux(vs_next, lds[B0 ^ 1], tid);
        __builtin_amdgcn_s_waitcnt(0);   // the tile copies have landed
        __syncthreads();
    };
#pragma unroll 1
    for (int j = 0; j < n_tiles; ++j) body(j, j & 1);

    const float l_tot = l_run + partner32f(l_run);
    if (!row_ok) return;
    const float inv_l = 1.0f / l_tot;
    uint16_t* orow = (uint16_t*)a.o.p + b * a.o.sB + hq * a.o.sH + (int64_t)qrow * a.o.sN;
    uint16_t* xrow = (uint16_t*)a.oa.p + b * a.oa.sB + hq * a.oa.sH + (int64_t)qrow * a.oa.sN;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int ch0 = 32 * cb + 8 * g + 4 * h;
            uint16_t o4[4], x4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o4[e] = f32_to_bf16_bits(oacc[cb][4 * g + e] * inv_l);
                x4[e] = f32_to_bf16_bits(xacc[cb][4 * g + e] * inv_l);
            }
            *(uint2*)(orow + ch0) = make_uint2((uint32_t)o4[0] | ((uint32_t)o4[1] << 16), (uint32_t)o4[2] | ((uint32_t)o4[3] << 16));
            *(uint2*)(xrow + ch0) = make_uint2((uint32_t)x4[0] | ((uint32_t)x4[1] << 16), (uint32_t)x4[2] | ((uint32_t)x4[3] << 16));
        }
    }
    if (a.lse && h == 0) a.lse[(int64_t)bh * a.Nq + qrow] = __builtin_fmaf(m_run, c, __log2f(l_tot)) * 0.6931471805599453f;
    if (a.row_max && h == 0) a.row_max[(int64_t)bh * a.Nq + qrow] = m_run;
}

// deq(Vhat) in bf16, channel-major [B, H, d, N]: every e2m1 value times its
// power-of-two scale is exact in bf16.  One thread per 32-token block.
__global__ __launch_bounds__(256) void vdeq_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                   int64_t nblocks, uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nblocks) return;
    const v4i raw = *(const v4i*)(codes + 16 * i);
    // the hardware's scaled e2m1 -> bf16 conversion, two values per byte (low
    // nibble first); an e2m1 value times 2^e is exact in bf16
    const float sc = __builtin_bit_cast(float, (uint32_t)scales[i] << 23);
    uint32_t w[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t x = (uint32_t)raw[q];
        w[4 * q + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 0));
        w[4 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 1));
        w[4 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 2));
        w[4 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 3));
    }
    v4i* o = (v4i*)(out + 32 * i);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = v4i{(int)w[4 * q], (int)w[4 * q + 1], (int)w[4 * q + 2], (int)w[4 * q + 3]};
}

// Raw fp32 S tile (32 queries x 32 keys) of MXFP4 codes through the same tile
// code: two wavefronts of 16 queries, the 32 keys in positions of keys 0 .. 31
// of a 128-key tile whose other keys are zero.
__global__ __launch_bounds__(128) void debug_scores_mx_kernel(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                                                             const uint8_t* ks, float* out) {
    __shared__ __attribute__((aligned(16))) uint8_t kc_l[KB * D / 2];
    __shared__ __attribute__((aligned(16))) uint8_t ks_l[KB * D / 32];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, q = l & 15;
    for (int i = tid; i < 4 * KB; i += 128) {
        const int j = i / KB, p = i % KB, key = key_at(p);
        *(v4i*)(kc_l + 2048 * j + 16 * p) = key < 32 ? *(const v4i*)(kc + (int64_t)key * (D / 2) + 16 * j) : v4i{};
    }
    for (int p = tid; p < KB; p += 128) {
        const int key = key_at(p);
        *(uint32_t*)(ks_l + 4 * p) = key < 32 ? *(const uint32_t*)(ks + 4 * key) : 0u;
    }
    __syncthreads();
    const int qrow = 16 * w + q;
    const v4i qb = *(const v4i*)(qc + (int64_t)qrow * (D / 2) + 16 * g);
    const int qsb = qs[qrow * (D / 32) + g];
    v4f s[8];
    qk_block16(kc_l, ks_l, qb, qsb, g, q, s);
    if (g == 0) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i) out[qrow * 32 + 4 * bb + i] = s[bb][i];
    }
}

}  // namespace

hipError_t launch_qat_fwd(const QatFwdArgs& a, hipStream_t st) {
    if (a.vdeq) {
        const int64_t nblocks = (int64_t)a.B * a.Hkv * D * (a.Nk / 32);
        vdeq_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, st>>>(a.vc, a.vs, nblocks, a.vdeq);
    }
    // the copies' per-lane offsets are 32-bit
    if ((int64_t)D * a.Nk * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int grid = a.B * a.Hq * ((a.Nq + BM - 1) / BM);
    if (a.vdeq) qat_aux_kernel<<<grid, 256, 0, st>>>(a);
    else qat_fwd_kernel<<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
}

size_t ws_qat_fwd_bytes(int B, int Hkv, int Nk, int d) { return (size_t)B * Hkv * Nk * d * 2; }

hipError_t launch_mx_dequant(const uint8_t* codes, const uint8_t* scales, int64_t nblocks, uint16_t* out,
                             hipStream_t st) {
    if (nblocks > 0) vdeq_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, st>>>(codes, scales, nblocks, out);
    return hipGetLastError();
}

hipError_t launch_debug_scores_mx(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                  float* out, hipStream_t st) {
    debug_scores_mx_kernel<<<1, 128, 0, st>>>(qc, qs, kc, ks, out);
    return hipGetLastError();
}

}  // namespace bqa
