// attn_sage_fwd.hip — SageAttention INT8 forward for gfx950.
//
// "SageBwd: A Trainable Low-bit Attention", Methodology 1 (INT8 attention with
// per-block scales) and 4 (K-smoothing, which happens in the K quantiser):
//   S_int = Qhat Khat^T exactly in int32 (i8 matrix instructions), scores
//   s = S_int * s_q * s_k * tau; online softmax over key tiles of 64 with
//   FlashAttention-2's running row maximum m (P = exp(s - m), the sums so far
//   scaled by exp(m_old - m_new) when m moves); P rounded for the P.V product
//   as fp16 (V fp16), e4m3(448 P) (V per-channel e4m3) or int8 per
//   (row, tile) (V per-channel int8); the row sum accumulates the unrounded P.
//
// Work decomposition: one workgroup of 4 wavefronts per 128 query rows of one
// (batch, head); each wavefront owns 32 rows.  The score tile is computed
// transposed, S^T = Khat Qhat^T (A = key rows from LDS, B = the wavefront's
// query rows held in registers), so the 32x32 accumulator puts one query row
// in each lane.  The K rows are fed through a fixed permutation (sigma) so
// that each lane half holds 16 consecutive keys: row max and row sum are
// in-lane reductions plus one permlane32 swap, and the probabilities are
// already the B operand of O^T = V^T P^T against contiguous V^T chunks, with
// no LDS round trip.  K tiles and channel-major V tiles sit in LDS as
// XOR-swizzled 16-byte chunks (conflict-free for 16 consecutive lanes).
//
// Two kernels share these pieces.  The fp8 P.V path (the common one) is a
// three-stage software pipeline with direct global->LDS copies in rings of
// four tiles and, for causal masks, one workgroup per pair of query tiles
// (heaviest with lightest); see the section that defines it.  The fp16 and
// int8 P.V paths take one tile at a time, three tiles deep in LDS (fp16 V is
// transposed on the way in through registers), with causal workgroups issued
// heaviest-first.  Consecutive workgroup ids take different heads, which
// keeps each head on one XCD.
#include <type_traits>
#include "common.hpp"
#include "internal.hpp"

namespace bqa {

namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile (= INT8 K block)
constexpr int NBUF = 3;   // LDS tiles: the one being used, the next (landed), the one after (in flight)

// XOR swizzle of the 16-byte chunks of a tile row (rows of ROW_BYTES).  For
// the K tile (read through the row permutation below) and for the V^T tile
// (read by consecutive rows) 16 consecutive lanes reading one logical chunk
// hit 16 distinct 16-byte bank groups.
template <int ROW_BYTES>
__device__ __forceinline__ int swz_k(int r, int c) {
    if constexpr (ROW_BYTES == 128) return r * 128 + 16 * (c ^ (((r >> 1) & 7) ^ (((r >> 4) & 1) << 2)));
    else return r * 64 + 16 * (c ^ (((r >> 2) & 3) ^ (((r >> 4) & 1) << 1)));
}
template <int ROW_BYTES>
__device__ __forceinline__ int swz_v(int r, int c) {
    if constexpr (ROW_BYTES == 128) return r * 128 + 16 * (c ^ ((r >> 1) & 7));
    else return r * 64 + 16 * (c ^ ((r >> 2) & 3));
}

// Row of the K tile that lane l feeds into matrix row l%32 of the S^T product.
// With this permutation the accumulator register i of lane (q, half h) holds
// key 16h + i (plus 32 for the second 32-key half): every lane half owns 16
// consecutive keys, so the probabilities line up with contiguous V^T chunks.
__device__ __forceinline__ int sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// S^T tile of 64 keys x 32 queries for one wavefront.  acc0: keys 16h + i,
// acc1: keys 32 + 16h + i (i = register index).
template <int D>
__device__ __forceinline__ void qk_tile(const uint8_t* k_lds, const v4i* qb, int krow, int h, v16i& acc0, v16i& acc1) {
    acc0 = v16i{};
    acc1 = v16i{};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        v4i a0 = *(const v4i*)(k_lds + swz_k<D>(krow, 2 * kk + h));
        v4i a1 = *(const v4i*)(k_lds + swz_k<D>(32 + krow, 2 * kk + h));
        acc0 = mfma_i8_32x32x32(a0, qb[kk], acc0);
        acc1 = mfma_i8_32x32x32(a1, qb[kk], acc1);
    }
}

template <int PV, int D>
struct Staging {
    static constexpr int V_ROW = PV == PV_F16 ? BN * 2 : BN;   // bytes per V^T row in LDS
    static constexpr int KPT = BN * D / 16 / 256;              // 16-byte K chunks per thread
    static constexpr int VPT = D * V_ROW / 16 / 256;           // 16-byte V chunks per thread
    v4i k[KPT];
    v4i v[VPT];
    float ks;   // the tile's K scale
};

template <int PV, int D>
__device__ __forceinline__ void stage_load(Staging<PV, D>& st, const SageFwdArgs& a, const int8_t* kbase,
                                           int b, int hk, int bhk, int t0, int tid) {
    using S = Staging<PV, D>;
    st.ks = a.ks[(int64_t)bhk * (a.Nk / BN) + t0 / BN];
#pragma unroll
    for (int u = 0; u < S::KPT; ++u) {
        const int g = tid + 256 * u, r = g / (D / 16), c = g % (D / 16);
        st.k[u] = *(const v4i*)(kbase + (int64_t)(t0 + r) * D + 16 * c);
    }
    if constexpr (PV == PV_F16) {
        const uint16_t* vb = (const uint16_t*)a.v16.p + b * a.v16.sB + hk * a.v16.sH;
#pragma unroll
        for (int u = 0; u < S::VPT; ++u) {
            const int g = tid + 256 * u, key = g / (D / 8), c8 = (g % (D / 8)) * 8;
            st.v[u] = *(const v4i*)(vb + (int64_t)(t0 + key) * a.v16.sN + c8);
        }
    } else {
        const uint8_t* vb = a.vc + (int64_t)bhk * D * a.Nk + t0;
#pragma unroll
        for (int u = 0; u < S::VPT; ++u) {
            const int g = tid + 256 * u, r = g / 4, q = g % 4;
            st.v[u] = *(const v4i*)(vb + (int64_t)r * a.Nk + 16 * q);
        }
    }
}

template <int PV, int D>
__device__ __forceinline__ void stage_store(const Staging<PV, D>& st, uint8_t* k_lds, uint8_t* v_lds, float* ks_lds,
                                            int tid) {
    using S = Staging<PV, D>;
    if (tid == 0) *ks_lds = st.ks;
#pragma unroll
    for (int u = 0; u < S::KPT; ++u) {
        const int g = tid + 256 * u, r = g / (D / 16), c = g % (D / 16);
        *(v4i*)(k_lds + swz_k<D>(r, c)) = st.k[u];
    }
    if constexpr (PV == PV_F16) {
        // transpose fp16 V into V^T [channel][key] (128-byte rows)
#pragma unroll
        for (int u = 0; u < S::VPT; ++u) {
            const int g = tid + 256 * u, key = g / (D / 8), c8 = (g % (D / 8)) * 8;
            const uint16_t* e = (const uint16_t*)&st.v[u];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                *(uint16_t*)(v_lds + swz_v<128>(c8 + k, key / 8) + 2 * (key % 8)) = e[k];
        }
    } else {
#pragma unroll
        for (int u = 0; u < S::VPT; ++u) {
            const int g = tid + 256 * u, r = g / 4, q = g % 4;
            *(v4i*)(v_lds + swz_v<BN>(r, q)) = st.v[u];
        }
    }
}

// Per-wavefront running state of the online softmax: m is the running row
// maximum of the scaled scores (log2 units), and O and l are kept relative to
// it (FlashAttention-2): when a tile raises m in any lane of the wavefront,
// the wavefront scales its accumulators by exp2(m_old - m_new) (1 in the
// lanes whose maximum did not move).
template <int D>
struct RowState {
    v16f oacc[D / 32];      // O^T accumulator: lane (query lq, half h), channel 32cb + 8(i/4) + 4h + i%4
    float m;                // running maximum (log2 units)
    float l;                // this lane half's share of the row sum
};

// Scale the accumulators and the row sum to a new running maximum.
template <int D>
__device__ __forceinline__ void rescale(RowState<D>& st, float m_new) {
    // exp2(-inf) = 0 for a row's first visible tile; 1 where m did not move
    const float f = m_new > st.m ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.0f;
    st.l *= f;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.oacc[cb][i] *= f;
}

// Softmax of one 64-key tile: scores (int32, converted in place) -> P in
// registers (f0: keys 16h + i, f1: keys 32 + 16h + i), running maximum and
// rescale, row sum.  Returns the row's largest P (int8 P.V needs it).
// `diag_lim` >= 64 means no key of the tile is masked for this lane;
// otherwise register i (+32) is visible iff i (+32) <= diag_lim.
template <int PV, int D>
__device__ __forceinline__ float tile_softmax(RowState<D>& st, const v16i& s0, const v16i& s1, float c, bool diag,
                                              int diag_lim, float (&f0)[16], float (&f1)[16]) {
    constexpr float pbias = PV == PV_F8 ? 8.807354922057604f : 0.0f;    // log2(448): P scaled by 448
#pragma unroll
    for (int i = 0; i < 16; ++i) { f0[i] = (float)s0[i]; f1[i] = (float)s1[i]; }
    if (diag) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            f0[i] = i > diag_lim ? -__builtin_inff() : f0[i];
            f1[i] = i + 32 > diag_lim ? -__builtin_inff() : f1[i];
        }
    }
    float mx = __builtin_fmaxf(f0[0], f1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = __builtin_fmaxf(__builtin_fmaxf(mx, f0[i]), f1[i]);
    mx = __builtin_fmaxf(mx, partner32f(mx));
    const float m_new = __builtin_fmaxf(st.m, mx * c);
    if (__any(m_new > st.m)) rescale<D>(st, m_new);
    st.m = m_new;
    const float bias = m_new == -__builtin_inff() ? 0.0f : pbias - m_new;
    float ps[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        f0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(f0[i], c, bias));
        f1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(f1[i], c, bias));
        if (i < 2) {
            ps[i] = f0[i];
            ps[2 + i] = f1[i];
        } else {
            ps[i & 1] += f0[i];
            ps[2 + (i & 1)] += f1[i];
        }
    }
    st.l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    return mx == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(__builtin_fmaf(mx, c, bias));
}

// P.V of one tile into the accumulators (V^T tile in LDS).
template <int PV, int D>
__device__ __forceinline__ void tile_pv(RowState<D>& st, const float (&f0)[16], const float (&f1)[16], float pmax,
                                        const uint8_t* vt, int lq, int h) {
    if constexpr (PV == PV_F8) {
        v8i pb;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // the first conversion of a pair writes the low half-word; the
            // other half comes from the second one, so the old value is moot
            int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f0[4 * k], f0[4 * k + 1], __builtin_bit_cast(int, f0[4 * k]), false);
            pb[k] = __builtin_amdgcn_cvt_pk_fp8_f32(f0[4 * k + 2], f0[4 * k + 3], w0, true);
            int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f1[4 * k], f1[4 * k + 1], __builtin_bit_cast(int, f1[4 * k]), false);
            pb[4 + k] = __builtin_amdgcn_cvt_pk_fp8_f32(f1[4 * k + 2], f1[4 * k + 3], w1, true);
        }
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
            const int r = 32 * cb + lq;
            v4i lo = *(const v4i*)(vt + swz_v<BN>(r, h));
            v4i hi = *(const v4i*)(vt + swz_v<BN>(r, 2 + h));
            v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            st.oacc[cb] = mfma_f8_32x32x64(av, pb, st.oacc[cb]);
        }
    } else if constexpr (PV == PV_I8) {
        // int8 P per (row, tile): r = the row's largest P in the tile
        const float r = pmax;
        float inv = r > 0.0f ? 127.0f / r : 0.0f;
        if (__builtin_isinf(inv)) inv = 0.0f;
        const float rs = r * (1.0f / 127.0f);
        // every P of the row is at most r, so |P * inv| <= 127 (no clamp)
        v4i pb0, pb1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pb0[k] = q8x4(f0[4 * k], f0[4 * k + 1], f0[4 * k + 2], f0[4 * k + 3], inv);
            pb1[k] = q8x4(f1[4 * k], f1[4 * k + 1], f1[4 * k + 2], f1[4 * k + 3], inv);
        }
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
            const int rr = 32 * cb + lq;
            v4i v0 = *(const v4i*)(vt + swz_v<BN>(rr, h));
            v4i v1 = *(const v4i*)(vt + swz_v<BN>(rr, 2 + h));
            v16i pv = mfma_i8_32x32x32(v0, pb0, v16i{});
            pv = mfma_i8_32x32x32(v1, pb1, pv);
#pragma unroll
            for (int i = 0; i < 16; ++i) st.oacc[cb][i] = __builtin_fmaf((float)pv[i], rs, st.oacc[cb][i]);
        }
    } else {
        // fp16 P; four 16-key steps: keys 32(s/2) + 16h + 8(s%2) + e
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v8h pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = (_Float16)(s < 2 ? f0[8 * (s % 2) + e] : f1[8 * (s % 2) + e]);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int ch = 32 * cb + lq;
                v8h av = *(const v8h*)(vt + swz_v<128>(ch, 4 * (s / 2) + 2 * h + (s % 2)));
                st.oacc[cb] = mfma_f16_32x32x16(av, pb, st.oacc[cb]);
            }
        }
    }
}

// Direct global -> LDS copies (fp8 / int8 V): every lane names its global
// source and the data lands at LDS base + 16 x lane, so the swizzled layouts
// come from the choice of source per lane.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
// One K tile (64 rows of D bytes) and one V^T tile (D rows of 64 bytes): each
// wavefront issues a quarter of the 1 KB segments.
template <int D>
__device__ __forceinline__ void tile_dma(const int8_t* kbase, const uint8_t* vbase, int64_t Nk, int t0, uint8_t* kl,
                                         uint8_t* vl, int w, int l) {
    constexpr int KSEG = BN * D / 1024, RPS = 1024 / D, LPR = D / 16;   // segments, rows per segment, lanes per row
#pragma unroll
    for (int u = 0; u < KSEG / 4; ++u) {
        const int sgm = (KSEG / 4) * w + u, r = RPS * sgm + l / LPR, pc = l % LPR;
        int c;
        if constexpr (D == 128) c = pc ^ (((r >> 1) & 7) ^ (((r >> 4) & 1) << 2));
        else c = pc ^ (((r >> 2) & 3) ^ (((r >> 4) & 1) << 1));
        dma16(kbase + (int64_t)(t0 + r) * D + 16 * c, kl + 1024 * sgm);
    }
    constexpr int VSEG = D * BN / 1024;
#pragma unroll
    for (int u = 0; u < VSEG / 4; ++u) {
        const int sgm = (VSEG / 4) * w + u, r = 16 * sgm + (l >> 2);
        const int c = (l & 3) ^ ((r >> 2) & 3);
        dma16(vbase + (int64_t)r * Nk + t0 + 16 * c, vl + 1024 * sgm);
    }
}

template <int PV, int D, bool CAUSAL>
__global__ __launch_bounds__(256, (PV == PV_F16 || !CAUSAL) ? 2 : 3) void sage_fwd_kernel(SageFwdArgs a) {
    using S = Staging<PV, D>;
    __shared__ __attribute__((aligned(16))) uint8_t k_l0[BN * D], k_l1[BN * D], k_l2[BN * D];
    __shared__ __attribute__((aligned(16))) uint8_t v_l0[D * S::V_ROW], v_l1[D * S::V_ROW], v_l2[D * S::V_ROW];
    __shared__ float ks_lds[NBUF];
    uint8_t* const k_lds[NBUF] = {k_l0, k_l1, k_l2};
    uint8_t* const v_lds[NBUF] = {v_l0, v_l1, v_l2};

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int BHq = a.B * a.Hq;
    const int n_qt = (a.Nq + BM - 1) / BM;
    const int bid = blockIdx.x;
    const int qt = CAUSAL ? (n_qt - 1 - bid / BHq) : (bid / BHq);
    const int bh = bid % BHq, b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / (a.Hq / a.Hkv), bhk = b * a.Hkv + hk;
    const int q0 = qt * BM;
    const int qrow = q0 + 32 * w + lq;
    const bool row_ok = qrow < a.Nq;
    const int off = a.Nk - a.Nq;
    const int krow = sigma(lq);

    // this lane's query codes: B operand, Q[qrow][16h + 32kk .. +16)
    v4i qb[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        qb[kk] = row_ok ? *(const v4i*)(a.qc + ((int64_t)bh * a.Nq + qrow) * D + 16 * h + 32 * kk) : v4i{};
    const float cq = row_ok ? a.qs[(int64_t)bh * (a.Nq / a.q_blk) + qrow / a.q_blk] * a.c_log2 : 0.0f;
    __builtin_amdgcn_s_waitcnt(0);   // Q fragments and scales are in registers before the tile loop
    // K scales per tile through the scalar cache (uniform addresses)
    const __attribute__((address_space(4))) float* kscale =
        (const __attribute__((address_space(4))) float*)(a.ks + (int64_t)bhk * (a.Nk / BN));

    const int last_row = min(q0 + BM, a.Nq) - 1;
    const int n_tiles = CAUSAL ? min(a.Nk / BN, (last_row + off) / BN + 1) : a.Nk / BN;
    const int wave_row0 = q0 + 32 * w;
    // tiles this wavefront sees at all (causal: up to its last row's diagonal)
    const int wave_tiles = CAUSAL ? min(n_tiles, (wave_row0 + 31 + off) / BN + 1) : n_tiles;
    const int8_t* kbase = a.kc + (int64_t)bhk * a.Nk * D;

    RowState<D> rs;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) rs.oacc[cb] = v16f{};
    rs.m = -__builtin_inff();
    rs.l = 0.0f;

    // Tiles go to LDS three deep.  fp8 / int8 V: direct copies; while tile j
    // is in use, tile j+1 has landed or is landing and tile j+2 is in flight;
    // the barrier waits only for the older copies.  fp16 V (transposed on the
    // way in): global -> registers -> LDS, one tile ahead.
    const uint8_t* vbase = a.vc + (int64_t)bhk * D * a.Nk;
    S st;
    if constexpr (PV == PV_F16) {
        if (n_tiles > 0) { stage_load<PV, D>(st, a, kbase, b, hk, bhk, 0, tid); stage_store<PV, D>(st, k_lds[0], v_lds[0], &ks_lds[0], tid); }
        if (n_tiles > 1) { stage_load<PV, D>(st, a, kbase, b, hk, bhk, BN, tid); stage_store<PV, D>(st, k_lds[1], v_lds[1], &ks_lds[1], tid); }
        __syncthreads();
        if (n_tiles > 2) stage_load<PV, D>(st, a, kbase, b, hk, bhk, 2 * BN, tid);
    } else {
        (void)st;
        if (n_tiles > 0) tile_dma<D>(kbase, vbase, a.Nk, 0, k_lds[0], v_lds[0], w, l);
        if (n_tiles > 1) tile_dma<D>(kbase, vbase, a.Nk, BN, k_lds[1], v_lds[1], w, l);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (n_tiles > 2) tile_dma<D>(kbase, vbase, a.Nk, 2 * BN, k_lds[2], v_lds[2], w, l);
    }

    auto body = [&](int j, auto bufc) __attribute__((always_inline)) {
        constexpr int B0 = decltype(bufc)::value;
        if (j < wave_tiles) {
            v16i x0, x1;
            qk_tile<D>(k_lds[B0], qb, krow, h, x0, x1);
            const int t0 = j * BN;
            const bool diag = CAUSAL && (t0 + BN - 1 > wave_row0 + off);
            const float kscj = PV == PV_F16 ? ks_lds[B0] : kscale[j];
            const float c = __builtin_fmaxf(cq * kscj, 1.17549435e-38f);
            float f0[16], f1[16];
            const float pmax = tile_softmax<PV, D>(rs, x0, x1, c, diag, qrow + off - t0 - 16 * h, f0, f1);
            tile_pv<PV, D>(rs, f0, f1, pmax, v_lds[B0], lq, h);
        }
        if constexpr (PV == PV_F16) {
            if (j + 2 < n_tiles) stage_store<PV, D>(st, k_lds[(B0 + 2) % NBUF], v_lds[(B0 + 2) % NBUF], &ks_lds[(B0 + 2) % NBUF], tid);
            __syncthreads();
            if (j + 3 < n_tiles) stage_load<PV, D>(st, a, kbase, b, hk, bhk, (j + 3) * BN, tid);
        } else {
            // tile j+1 must have landed (this wavefront's copies, then the
            // barrier for everyone's); tile j+2's copies may stay in flight
            constexpr int per_tile = (BN * D / 1024) / 4 + (D * BN / 1024) / 4;   // copies per wavefront
            if (j + 2 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0070 | per_tile);   // vmcnt(per_tile), lgkmcnt(0)
            else __builtin_amdgcn_s_waitcnt(0);
            // a plain s_barrier: the workgroup fence of __syncthreads would also
            // wait for the copies still in flight
            asm volatile("s_barrier" ::: "memory");
            if (j + 3 < n_tiles) tile_dma<D>(kbase, vbase, a.Nk, (j + 3) * BN, k_lds[B0], v_lds[B0], w, l);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int j = 0; j < n_tiles; j += 3) {
        body(j, I0{});
        if (j + 1 >= n_tiles) break;
        body(j + 1, I1{});
        if (j + 2 >= n_tiles) break;
        body(j + 2, I2{});
    }

    // ---- epilogue: O = O^T acc / l (times the V channel scale), LSE in natural log
    const float l_tot = rs.l + partner32f(rs.l);
    if (!row_ok) return;
    const float inv_l = 1.0f / l_tot;
    uint16_t* orow = (uint16_t*)a.o.p + b * a.o.sB + hq * a.o.sH + (int64_t)qrow * a.o.sN;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int ch0 = 32 * cb + 8 * g + 4 * h;
            uint16_t out[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = rs.oacc[cb][4 * g + e] * inv_l;
                if constexpr (PV != PV_F16) v *= a.vs[(int64_t)bhk * D + ch0 + e];
                out[e] = PV == PV_F16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
            }
            *(uint2*)(orow + ch0) = make_uint2((uint32_t)out[0] | ((uint32_t)out[1] << 16),
                                               (uint32_t)out[2] | ((uint32_t)out[3] << 16));
        }
    }
    if (a.lse && h == 0) {
        // natural-log LSE; with P scaled by 448 the sum carries that factor
        float lse = rs.m * 0.6931471805599453f + __logf(l_tot);
        if (PV == PV_F8) lse -= 6.104793232414985f;   // ln(448)
        a.lse[(int64_t)bh * a.Nq + qrow] = lse;
    }
}

// ---- fp8 P.V: three-stage software pipeline -----------------------------------
// A wavefront overlaps its own matrix and vector work across three tiles: in
// step j it issues P.V of tile j-1 while it converts the scores of tile j, and
// the scores of tile j+1 while it computes the exponentials of tile j.  The
// matrix instructions are spread between the vector ones so that neither this
// wavefront nor the other one on its SIMD waits behind a burst of them.  Two
// score tiles in registers cost VGPRs, so two workgroups share a CU.  K tiles
// sit in a ring of four LDS slots (tile t is read in step t-1 and copied at
// the end of step t-4), V^T tiles in another ring of four (read in step t+1,
// copied at the end of step t-3).  The copies are issued from inline assembly
// with a scalar base: the compiler then leaves their completion to the
// kernel's own counted waits instead of waiting for every copy in flight
// before any LDS read.
constexpr int PRING = 4;
// Per-lane source offsets of one wavefront's share of a K tile and a V^T tile
// (1 KB segments; the LDS swizzle comes from the source each lane names).
template <int D>
struct CopyPlan {
    static constexpr int KU = BN * D / 1024 / 4, VU = D * BN / 1024 / 4;   // segments per wavefront
    uint32_t koff[KU], voff[VU];
    __device__ __forceinline__ CopyPlan(int w, int l, int Nk) {
        constexpr int RPS = 1024 / D, LPR = D / 16;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int sgm = KU * w + u, r = RPS * sgm + l / LPR, pc = l % LPR;
            int c;
            if constexpr (D == 128) c = pc ^ (((r >> 1) & 7) ^ (((r >> 4) & 1) << 2));
            else c = pc ^ (((r >> 2) & 3) ^ (((r >> 4) & 1) << 1));
            koff[u] = (uint32_t)(r * D + 16 * c);
        }
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            const int sgm = VU * w + u, r = 16 * sgm + (l >> 2);
            const int c = (l & 3) ^ ((r >> 2) & 3);
            voff[u] = (uint32_t)r * (uint32_t)Nk + (uint32_t)(16 * c);
        }
    }
    __device__ __forceinline__ void k_tile(const int8_t* kbase, int t0, const uint8_t* kl, int w) const {
#pragma unroll
        for (int u = 0; u < KU; ++u) lds_copy16(koff[u], kbase + (int64_t)t0 * D, lds_addr(kl) + 1024 * (KU * w + u));
    }
    __device__ __forceinline__ void v_tile(const uint8_t* vbase, int t0, const uint8_t* vl, int w) const {
#pragma unroll
        for (int u = 0; u < VU; ++u) lds_copy16(voff[u], vbase + t0, lds_addr(vl) + 1024 * (VU * w + u));
    }
};

// P of a finished tile, packed as the B operand of its P.V product.
struct PendF8 {
    v8i pb;   // e4m3 codes of 448 P: lane (query, half h), keys 16h + 4k .. (and +32)
};

template <int D>
__device__ __forceinline__ void pv_f8(v16f (&oacc)[D / 32], const PendF8& pp, const uint8_t* vt, int lq, int h, int cb) {
    const int r = 32 * cb + lq;
    v4i lo = *(const v4i*)(vt + swz_v<BN>(r, h));
    v4i hi = *(const v4i*)(vt + swz_v<BN>(r, 2 + h));
    v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    oacc[cb] = mfma_f8_32x32x64(av, pp.pb, oacc[cb]);
}

// One step of the pipeline (see above).  s0/s1: int32 scores of this tile on
// entry, of the next tile on exit; pend: P of the previous tile on entry, of
// this tile on exit.  The arithmetic is the one of tile_softmax + tile_pv
// (fp8 P.V), with the rescale of the accumulators done after P.V of the
// previous tile was issued (that product belongs to the old maximum) and after
// the exponentials (so that it does not delay them).
template <int D, bool DIAG>
__device__ __forceinline__ void f8_step(RowState<D>& st, PendF8& pend, v16i& s0, v16i& s1, const uint8_t* k_next,
                                        const uint8_t* v_prev, const v4i* qb, int krow, int lq, int h, float c,
                                        int diag_lim) {
    constexpr float pbias = 8.807354922057604f;   // log2(448): P scaled by 448
    float f0[16], f1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { f0[i] = (float)s0[i]; f1[i] = (float)s1[i]; }
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) pv_f8<D>(st.oacc, pend, v_prev, lq, h, cb);
    if constexpr (DIAG) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            f0[i] = i > diag_lim ? -__builtin_inff() : f0[i];
            f1[i] = i + 32 > diag_lim ? -__builtin_inff() : f1[i];
        }
    }
    float mx = __builtin_fmaxf(f0[0], f1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = __builtin_fmaxf(__builtin_fmaxf(mx, f0[i]), f1[i]);
    mx = __builtin_fmaxf(mx, partner32f(mx));
    const float m_new = __builtin_fmaxf(st.m, mx * c);
    const bool need = m_new > st.m;
    const float bias = m_new == -__builtin_inff() ? 0.0f : pbias - m_new;
    // scores of the next tile, one 32-channel slice every four exponentials;
    // each slice's K operands are read while the slice before is issued
    constexpr int NS = D / 32;
    v4i ka = *(const v4i*)(k_next + swz_k<D>(krow, h));
    v4i kb = *(const v4i*)(k_next + swz_k<D>(32 + krow, h));
    v16i n0 = v16i{}, n1 = v16i{};
    float ps[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i % 4 == 0 && i / 4 < NS) {
            const int kk = i / 4;
            n0 = mfma_i8_32x32x32(ka, qb[kk], n0);
            n1 = mfma_i8_32x32x32(kb, qb[kk], n1);
            if (kk + 1 < NS) {
                ka = *(const v4i*)(k_next + swz_k<D>(krow, 2 * (kk + 1) + h));
                kb = *(const v4i*)(k_next + swz_k<D>(32 + krow, 2 * (kk + 1) + h));
            }
        }
        f0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(f0[i], c, bias));
        f1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(f1[i], c, bias));
        if (i < 2) {
            ps[i] = f0[i];
            ps[2 + i] = f1[i];
        } else {
            ps[i & 1] += f0[i];
            ps[2 + (i & 1)] += f1[i];
        }
    }
    const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // the first conversion of a pair writes the low half-word, the second
        // one the high half-word: the old value is moot
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f0[4 * k], f0[4 * k + 1], __builtin_bit_cast(int, f0[4 * k]), false);
        pend.pb[k] = __builtin_amdgcn_cvt_pk_fp8_f32(f0[4 * k + 2], f0[4 * k + 3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f1[4 * k], f1[4 * k + 1], __builtin_bit_cast(int, f1[4 * k]), false);
        pend.pb[4 + k] = __builtin_amdgcn_cvt_pk_fp8_f32(f1[4 * k + 2], f1[4 * k + 3], w1, true);
    }
    s0 = n0;
    s1 = n1;
    // instruction order: the LDS reads of P.V and of the first score slice
    // first, the conversions over their latency, P.V of the previous tile
    // under the rest of the conversions and the maximum, then one score
    // instruction of the next tile every dozen vector instructions, each
    // slice's reads issued a slice ahead (the rare diagonal tiles keep the
    // compiler's own order)
    if constexpr (!DIAG) {
        __builtin_amdgcn_sched_group_barrier(0x0100, 2 * NS + 2, 0);      // V reads, K reads of slice 0
        __builtin_amdgcn_sched_group_barrier(0x0002, 20, 0);              // conversions
#pragma unroll
        for (int cb = 0; cb < NS; ++cb) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);           // P.V
            __builtin_amdgcn_sched_group_barrier(0x0002, 6, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x0002, 30, 0);              // conversions, maximum
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);           // scores
            if (k + 1 < NS) __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // next slice's reads
            __builtin_amdgcn_sched_group_barrier(0x0002, 96 / NS / 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            if (k + 1 < NS) __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x0002, 96 / NS / 2, 0);
        }
    }
    // keep this tile's vector work ahead of the branch below (the compiler
    // would otherwise sink it into the next step, away from the matrix
    // instructions it is meant to hide)
    asm volatile("" ::"v"(pend.pb[0]), "v"(pend.pb[1]), "v"(pend.pb[2]), "v"(pend.pb[3]), "v"(pend.pb[4]),
                 "v"(pend.pb[5]), "v"(pend.pb[6]), "v"(pend.pb[7]), "v"(psum));
    if (__any(need)) rescale<D>(st, m_new);
    st.l += psum;
    st.m = m_new;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void sage_fwd_f8_kernel(SageFwdArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[PRING][BN * D];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[PRING][D * BN];
    using CP = CopyPlan<D>;

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int BHq = a.B * a.Hq;
    const int n_qt = (a.Nq + BM - 1) / BM;
    const int bid = blockIdx.x;
    // causal: this workgroup takes query tile n_qt-1-p and then tile p, which
    // gives every workgroup the same number of key tiles (no tail of short
    // workgroups); the middle tile of an odd count goes alone
    const int p = bid / BHq;
    const int bh = bid % BHq, b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / (a.Hq / a.Hkv), bhk = b * a.Hkv + hk;
    const int off = a.Nk - a.Nq;
    const int krow = sigma(lq);
    const CP cp(w, l, a.Nk);
    const int8_t* kbase = a.kc + (int64_t)bhk * a.Nk * D;
    const uint8_t* vbase = a.vc + (int64_t)bhk * D * a.Nk;
    const __attribute__((address_space(4))) float* kscale =
        (const __attribute__((address_space(4))) float*)(a.ks + (int64_t)bhk * (a.Nk / BN));

    __shared__ float qmax_s[4];
    const bool q_in = a.q16.p != nullptr;

    auto qtile = [&](const int qt) __attribute__((always_inline)) {
        const int q0 = qt * BM;
        const int qrow = q0 + 32 * w + lq;
        const bool row_ok = qrow < a.Nq;
        v4i qb[D / 32];
        v4i qraw[D / 16];                // Q quantised here: this lane's D/2 bf16 values, 8 per vector
        float cq = 0.0f;
        if (q_in) {
            // the lane's channels are those of its INT8 operand: 32 kk + 16 h + 0..15
            const uint16_t* qsrc = (const uint16_t*)a.q16.p + b * a.q16.sB + hq * a.q16.sH + (int64_t)qrow * a.q16.sN + 16 * h;
#pragma unroll
            for (int u = 0; u < D / 16; ++u) qraw[u] = row_ok ? *(const v4i*)(qsrc + 32 * (u >> 1) + 8 * (u & 1)) : v4i{};
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                qb[kk] = row_ok ? *(const v4i*)(a.qc + ((int64_t)bh * a.Nq + qrow) * D + 16 * h + 32 * kk) : v4i{};
            cq = row_ok ? a.qs[(int64_t)bh * (a.Nq / a.q_blk) + qrow / a.q_blk] * a.c_log2 : 0.0f;
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (q_in) {
            // largest magnitude of the wavefront's 32 rows; the block's (q_blk rows,
            // whole wavefronts) is taken after the prologue barrier
            float am = 0.0f;
#pragma unroll
            for (int u = 0; u < D / 16; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t wd = (uint32_t)qraw[u][e];
                    am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(__builtin_bit_cast(float, wd << 16)),
                                                             __builtin_fabsf(__builtin_bit_cast(float, wd & 0xFFFF0000u))));
                }
            am = wave_max(am);
            if (l == 0) qmax_s[w] = am;
        }

        const int last_row = min(q0 + BM, a.Nq) - 1;
        const int n_tiles = CAUSAL ? min(a.Nk / BN, (last_row + off) / BN + 1) : a.Nk / BN;
        const int wave_row0 = q0 + 32 * w;
        const int wave_tiles = CAUSAL ? min(n_tiles, (wave_row0 + 31 + off) / BN + 1) : n_tiles;

        RowState<D> rs;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) rs.oacc[cb] = v16f{};
        rs.m = -__builtin_inff();
        rs.l = 0.0f;
        PendF8 pend;
        pend.pb = v8i{};

        // V slot 3 starts as zeros: the first step's P.V (of no tile, P = 0) reads it
#pragma unroll
        for (int u = 0; u < D * BN / 16 / 256; ++u) *(v4i*)(&v_lds[3][16 * (tid + 256 * u)]) = v4i{};
        // copies in the order of the steady state: K0 K1 V0 K2 V1 K3 V2 (a
        // short row repeats its last tile, which keeps the wait counts exact)
        if (n_tiles > 0) {
            const int tl = n_tiles - 1;
            cp.k_tile(kbase, 0, k_lds[0], w);
            cp.k_tile(kbase, min(1, tl) * BN, k_lds[1], w);
            cp.v_tile(vbase, 0, v_lds[0], w);
            cp.k_tile(kbase, min(2, tl) * BN, k_lds[2], w);
            cp.v_tile(vbase, min(1, tl) * BN, v_lds[1], w);
            cp.k_tile(kbase, min(3, tl) * BN, k_lds[3], w);
            cp.v_tile(vbase, min(2, tl) * BN, v_lds[2], w);
        }
        static_assert(CP::KU == CP::VU && 5 * CP::KU < 16, "wait counts");
        __builtin_amdgcn_s_waitcnt(0x0070 | (5 * CP::KU));   // K0 and K1 landed, zero fill and maxima written
        asm volatile("s_barrier" ::: "memory");
        if (q_in) {
            // per-block INT8 as the token-block quantiser: scale = amax / 127,
            // code = rint(fp32(x * (127 / amax))); no clamp since |x| <= amax
            const int nwb = a.q_blk / 32, w0 = w - w % nwb;
            float am = qmax_s[w0];
            for (int u = 1; u < nwb; ++u) am = __builtin_fmaxf(am, qmax_s[w0 + u]);
            float inv = am > 0.0f ? 127.0f / am : 0.0f;
            float scale = am / 127.0f;
            if (!(am > 0.0f) || __builtin_isinf(inv)) { inv = 0.0f; scale = 0.0f; }
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                float x[16];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t wd = (uint32_t)qraw[2 * kk + (e >> 2)][e & 3];
                    x[2 * e] = __builtin_bit_cast(float, wd << 16);
                    x[2 * e + 1] = __builtin_bit_cast(float, wd & 0xFFFF0000u);
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) qb[kk][g] = q8x4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3], inv);
            }
            if (row_ok) {
                cq = scale * a.c_log2;
                if (a.qc_out) {
#pragma unroll
                    for (int kk = 0; kk < D / 32; ++kk)
                        *(v4i*)(a.qc_out + ((int64_t)bh * a.Nq + qrow) * D + 16 * h + 32 * kk) = qb[kk];
                }
                if (a.qs_out && l == 0 && w == w0) a.qs_out[(int64_t)bh * (a.Nq / a.q_blk) + qrow / a.q_blk] = scale;
            }
            // stores count in vmcnt too: finish them so that the loop's copy
            // counts hold
            if (a.qc_out || a.qs_out) __builtin_amdgcn_s_waitcnt(0x0070);
        }

        v16i s0 = v16i{}, s1 = v16i{};   // scores of the tile about to be processed
        if (wave_tiles > 0) qk_tile<D>(k_lds[0], qb, krow, h, s0, s1);

        // end of step j: K(j+2) and V(j) must have landed; the copies issued
        // after K(j+2) (V(j+1), K(j+3), V(j+2)) may stay in flight
        auto sync = [&](int j, const uint8_t* k_free, const uint8_t* v_free) __attribute__((always_inline)) {
            if (j + 3 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0070 | (3 * CP::KU));
            else __builtin_amdgcn_s_waitcnt(0);
            asm volatile("s_barrier" ::: "memory");
            if (j + 4 < n_tiles) cp.k_tile(kbase, (j + 4) * BN, k_free, w);
            if (j + 3 < n_tiles) cp.v_tile(vbase, (j + 3) * BN, v_free, w);
        };
        // Steps before the first tile that reaches the diagonal of any row of
        // the workgroup: no masking, every wavefront active, ring slots as
        // immediates (unrolled by the ring size).
        const int J1 = CAUSAL ? min(n_tiles, max(0, q0 + off + 1) / BN) : n_tiles;
        auto body = [&](int j, auto slot) __attribute__((always_inline)) {
            constexpr int KB = decltype(slot)::value, KN = (KB + 1) % PRING, VP = (KB + PRING - 1) % PRING;
            const float c = __builtin_fmaxf(cq * kscale[j], 1.17549435e-38f);
            f8_step<D, false>(rs, pend, s0, s1, k_lds[KN], v_lds[VP], qb, krow, lq, h, c, 0);
            sync(j, k_lds[KB], v_lds[VP]);
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        for (int j = 0; j < J1; j += PRING) {
            body(j, I0{});
            if (j + 1 >= J1) break;
            body(j + 1, I1{});
            if (j + 2 >= J1) break;
            body(j + 2, I2{});
            if (j + 3 >= J1) break;
            body(j + 3, I3{});
        }
        // The few remaining steps (causal): masked tiles, and at j ==
        // wave_tiles a fully masked step that only adds the wave's last P.V.
        for (int j = J1; j < n_tiles; ++j) {
            const int kb = j & (PRING - 1), kn = (j + 1) & (PRING - 1), vp = (j + PRING - 1) & (PRING - 1);
            if (j <= wave_tiles) {
                const float c = __builtin_fmaxf(cq * kscale[j], 1.17549435e-38f);
                const int lim = j == wave_tiles ? -1 : qrow + off - j * BN - 16 * h;
                f8_step<D, true>(rs, pend, s0, s1, k_lds[kn], v_lds[vp], qb, krow, lq, h, c, lim);
            }
            sync(j, k_lds[kb], v_lds[vp]);
        }
        if (wave_tiles == n_tiles && n_tiles > 0) {
            const uint8_t* vt = v_lds[(n_tiles - 1) & (PRING - 1)];
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) pv_f8<D>(rs.oacc, pend, vt, lq, h, cb);
        }
        // every LDS read of this query tile is done before the slots are reused
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("s_barrier" ::: "memory");

        const float l_tot = rs.l + partner32f(rs.l);
        if (!row_ok) return;
        const float inv_l = 1.0f / l_tot;
        uint16_t* orow = (uint16_t*)a.o.p + b * a.o.sB + hq * a.o.sH + (int64_t)qrow * a.o.sN;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ch0 = 32 * cb + 8 * g + 4 * h;
                uint16_t out[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = f32_to_bf16_bits(rs.oacc[cb][4 * g + e] * inv_l * a.vs[(int64_t)bhk * D + ch0 + e]);
                *(uint2*)(orow + ch0) = make_uint2((uint32_t)out[0] | ((uint32_t)out[1] << 16),
                                                   (uint32_t)out[2] | ((uint32_t)out[3] << 16));
            }
        }
        if (a.lse && h == 0) {
            // natural-log LSE; with P scaled by 448 the sum carries that factor
            a.lse[(int64_t)bh * a.Nq + qrow] = rs.m * 0.6931471805599453f + __logf(l_tot) - 6.104793232414985f;
        }
    };
    const int n_pass = CAUSAL && p != n_qt - 1 - p ? 2 : 1;
    for (int pass = 0; pass < n_pass; ++pass) qtile(CAUSAL && pass == 0 ? n_qt - 1 - p : p);
}

// Raw int32 S tile (32 queries x 32 keys) through the same tile code.
template <int D>
__global__ __launch_bounds__(64) void debug_scores_i8_kernel(const int8_t* qc, const int8_t* kc, int32_t* out) {
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[BN * D];
    const int l = threadIdx.x, h = l >> 5, lq = l & 31;
    for (int g = l; g < 32 * D / 16; g += 64) {
        const int r = g / (D / 16), c = g % (D / 16);
        *(uint4*)(&k_lds[swz_k<D>(r, c)]) = *(const uint4*)(kc + (int64_t)r * D + 16 * c);
    }
    for (int g = l; g < 32 * D / 16; g += 64) {            // rows 32..63: zero
        const int r = 32 + g / (D / 16), c = g % (D / 16);
        *(uint4*)(&k_lds[swz_k<D>(r, c)]) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    v4i qb[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qb[kk] = *(const v4i*)(qc + (int64_t)lq * D + 16 * h + 32 * kk);
    v16i s0, s1;
    qk_tile<D>(k_lds, qb, sigma(lq), h, s0, s1);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[lq * 32 + 16 * h + i] = s0[i];
}

template <int PV, int D>
hipError_t launch_t(const SageFwdArgs& a, hipStream_t st) {
    const int grid = a.B * a.Hq * ((a.Nq + BM - 1) / BM);
    if constexpr (PV == PV_F16) {
        if (a.causal) sage_fwd_kernel<PV, D, true><<<grid, 256, 0, st>>>(a);
        else sage_fwd_kernel<PV, D, false><<<grid, 256, 0, st>>>(a);
    } else if constexpr (PV == PV_I8) {
        if (a.causal) sage_fwd_kernel<PV, D, true><<<grid, 256, 0, st>>>(a);
        else sage_fwd_kernel<PV, D, false><<<grid, 256, 0, st>>>(a);
    } else {
        // lane offsets of the copies are 32-bit
        if ((int64_t)D * a.Nk >= (int64_t)1 << 31) return hipErrorInvalidValue;
        // causal: one workgroup per pair of query tiles
        const int n_qt = (a.Nq + BM - 1) / BM;
        if (a.causal) sage_fwd_f8_kernel<D, true><<<a.B * a.Hq * ((n_qt + 1) / 2), 256, 0, st>>>(a);
        else sage_fwd_f8_kernel<D, false><<<grid, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sage_fwd(const SageFwdArgs& a, int pv, int d, hipStream_t st) {
    if (d == 128) {
        if (pv == PV_F8) return launch_t<PV_F8, 128>(a, st);
        if (pv == PV_I8) return launch_t<PV_I8, 128>(a, st);
        return launch_t<PV_F16, 128>(a, st);
    }
    if (pv == PV_F8) return launch_t<PV_F8, 64>(a, st);
    if (pv == PV_I8) return launch_t<PV_I8, 64>(a, st);
    return launch_t<PV_F16, 64>(a, st);
}

hipError_t launch_debug_scores_i8(const int8_t* qc, const int8_t* kc, int d, int64_t q_row0, int64_t k_row0,
                                  int32_t* out, hipStream_t st) {
    if (d == 128) debug_scores_i8_kernel<128><<<1, 64, 0, st>>>(qc + q_row0 * 128, kc + k_row0 * 128, out);
    else debug_scores_i8_kernel<64><<<1, 64, 0, st>>>(qc + q_row0 * 64, kc + k_row0 * 64, out);
    return hipGetLastError();
}

}  // namespace bqa
