// attn_thrift.hip — ThriftAttention mixed-precision prefill for gfx950.
//
// "ThriftAttention" technical summary, Methodology step 2: per query block,
// the key blocks that block selection did not pick run through the FP4 path
// (micro-scaled FP4 Q, K, V; MXFP4 here, on the scaled f8f6f4 matrix
// instructions) with P quantised in two levels (the row's largest P in the
// block is scaled to 6, then MXFP4 per 32 keys; the first-level factor is
// undone in fp32), then the selected blocks through the 16-bit path (bf16
// Q, K, V), all merged by one online softmax.  The diagonal block is masked
// in whichever path takes it.
//
// Layout: one workgroup per 128 query rows, S^T = K Q^T so that each lane
// owns one query row; FP4 key blocks of 128 keys.  The prefill kernel runs
// 8 wavefronts of 16 rows and takes the selected blocks in quarters of 32
// keys, each quarter one tile of the online softmax; the NVFP4 emulation
// kernel runs 4 wavefronts of 32 rows with tiles of 64 keys.  The softmax
// is FlashAttention-2's: P = exp(s - m)
// against the running row maximum m, the sums so far scaled by
// exp(m_old - m_new) when m moves.  The FP4 path's accumulator is kept in
// units of the current block's r/6 and rescaled when the next block brings a
// new r; that rescale also carries the running maximum's factor.  A block
// whose largest P is below 2^-64 adds nothing (as one whose P all underflow):
// its share of O is below 2^-64 of the row's, and the unit change would leave
// fp32's range.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace bqa {

namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int D = 128;    // head dimension
constexpr int KB = 128;   // FP4 key block
constexpr int HB = 64;    // bf16 half block

__device__ __forceinline__ int sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
// 64-byte rows read through sigma (K codes)
__device__ __forceinline__ int fk64(int r) { return ((r >> 2) & 3) ^ (((r >> 4) & 1) << 1); }
// 64-byte rows read consecutively (V^T codes)
__device__ __forceinline__ int fv64(int r) { return (r >> 2) & 3; }
// 256-byte rows read through sigma (bf16 K)
__device__ __forceinline__ int fk256(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }
// 128-byte rows read consecutively (bf16 V^T)
__device__ __forceinline__ int fv128(int r) { return (r >> 1) & 7; }

struct LdsF4 {
    uint8_t kc[KB * D / 2];    // 128 keys x 64 B
    uint8_t ks[KB * D / 32];   // 128 keys x 4 E8M0
    uint8_t vc[D * KB / 2];    // 128 channels x 64 B (128 keys)
    uint8_t vs[D * KB / 32];   // 128 channels x 4 E8M0
};
struct LdsBf {
    uint8_t k[HB * D * 2];     // 64 keys x 256 B
    uint8_t vt[D * HB * 2];    // 128 channels x 128 B (64 keys)
};
struct LdsF4Bias {              // the post-training baseline: an FP4 block and its keys' score shifts
    LdsF4 f;
    float bias[KB];
};
union LdsBuf {
    LdsF4 f;
    LdsBf b;
    LdsF4Bias p;
};

// bf16 half block (keys k0 .. k0 + 63): K rows by direct copies; V comes back
// in registers (4 keys x 8 channels per thread) for a transposed store.
struct VStage {
    v4i v[4];
};
__device__ __forceinline__ void issue_bf(const Dense& kx, const Dense& vx, int b, int hk, int k0, LdsBf& L, int w,
                                         int l, int tid, VStage& vs) {
    const uint16_t* kb = (const uint16_t*)kx.p + b * kx.sB + hk * kx.sH + (int64_t)k0 * kx.sN;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int sgm = 4 * w + u, r = 4 * sgm + (l >> 4);
        lds_copy16((uint32_t)(2 * (r * kx.sN + 8 * ((l & 15) ^ fk256(r)))), kb, lds_addr(L.k + 1024 * sgm));
    }
    const uint16_t* vb = (const uint16_t*)vx.p + b * vx.sB + hk * vx.sH;
    const int cg = tid & 15, kq = tid >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) vs.v[u] = *(const v4i*)(vb + (int64_t)(k0 + 4 * kq + u) * vx.sN + 8 * cg);
}
__device__ __forceinline__ void store_bf(const VStage& vs, LdsBf& L, int tid) {
    const int cg = tid & 15, kq = tid >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // channel 8 cg + e, keys 4 kq .. 4 kq + 3
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm((uint32_t)vs.v[1][e >> 1], (uint32_t)vs.v[0][e >> 1], sel);
        const uint32_t hi = __builtin_amdgcn_perm((uint32_t)vs.v[3][e >> 1], (uint32_t)vs.v[2][e >> 1], sel);
        const int r = 8 * cg + e;
        *(v2i*)(L.vt + r * 128 + 16 * ((kq >> 1) ^ fv128(r)) + 8 * (kq & 1)) = v2i{(int)lo, (int)hi};
    }
}

// Running maximum of a bf16 tile: when it moves in any lane, scale the
// accumulators and the row sum by exp2(m_old - m_new) (0 at a row's first
// visible tile, 1 where the maximum did not move).
__device__ __forceinline__ void follow_max(v16f* oacc, float& l_run, float& m_run, float m_new) {
    if (__any(m_new > m_run)) {
        const float f = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        l_run *= f;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[cb][i] *= f;
    }
    m_run = m_new;
}
constexpr float R_FLOOR = 0x1p-64f;   // two-level factors below this add nothing

// ---------------------------------------------------------------------------
// Prefill kernel.  Eight wavefronts per 128-row query block, 16 query rows
// each, on the 16 x 16 matrix instructions: a wavefront's accumulators and
// block scores fit in about 120 registers, so four wavefronts share a SIMD.
// Scores are S^T = K Q^T, lane l owning query row l % 16.  FP4 blocks: the
// rows of S MFMA b are the keys kappa(b, r) = 32 (r / 4) + 4 b + r % 4, so
// lane l holds keys 32 (l / 16) .. + 31 in order, one whole MX block of P:
// its codes are the lane's B operand of P.V as they stand and its scale
// needs no other lane.  bf16 quarters (32 keys): S MFMA b (16 keys) takes
// the keys 8 (r / 4) + 4 b + r % 4, so lane l holds keys 8 (l / 16) .. + 7,
// its B operand of P.V.
//
// PTQ: the post-training FP4 baseline (query and key smoothing, two-level
// P): no selected blocks, and key j's shift qbar . k^_j of the workgroup's
// query block (a.sbias) is added to its raw scores.

// LDS layout of the FP4 block: chunk-major.  A matrix instruction's operand
// read gives each group of 16 lanes (l / 16 = g) the 16-byte chunk g of 16
// rows; the rows' chunks g sit next to one another, so each group reads one
// contiguous 256-byte span.  Measured on gfx950, such reads have no bank
// conflicts, while four groups that read different chunks of the same
// 64-byte rows take twice the cycles under each row swizzle tried, although
// every group alone spreads over all banks.  K codes: chunk g (channels
// 32 g .. + 31) of the key
// at position p at kc + 2048 g + 16 p, with the keys in the order the S
// instructions read them: position p = 16 b + 4 a + c holds key
// 32 a + 4 b + c; K scales: the key at position p has its four bytes at word
// p.  V^T codes: chunk g (keys 32 g .. + 31) of channel ch at
// vc + 2048 g + 16 ch; V scales channel-major.
__device__ __forceinline__ int key_at(int p) { return 32 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3); }

// FP4 key block J into L, one K copy and one V copy per wavefront of eight.
__device__ __forceinline__ void issue_f4_16(const ThriftFwdArgs& a, int bhk, int J, LdsF4& L, int w, int l) {
    const int t0 = J * KB;
    const uint8_t* kbase = a.kc + ((int64_t)bhk * a.Nk + t0) * (D / 2);
    const uint8_t* vbase = a.vc + (int64_t)bhk * D * (a.Nk / 2) + t0 / 2;
    // wavefront w: chunk w / 2 of positions (K) and channels (V) 64 (w % 2) .. + 63
    const int j = w >> 1, p = 64 * (w & 1) + l;
    lds_copy16((uint32_t)(key_at(p) * (D / 2) + 16 * j), kbase, lds_addr(L.kc + 1024 * w));
    lds_copy16((uint32_t)p * (uint32_t)(a.Nk / 2) + (uint32_t)(16 * j), vbase, lds_addr(L.vc + 1024 * w));
    if (w < 2) lds_copy4((uint32_t)(4 * key_at(64 * w + l)), a.ks + ((int64_t)bhk * a.Nk + t0) * (D / 32), lds_addr(L.ks + 256 * w));
    else if (w < 4)
        lds_copy4((uint32_t)l * (uint32_t)(a.Nk / 32), a.vs + ((int64_t)bhk * D + 64 * (w - 2)) * (a.Nk / 32) + t0 / 32,
                  lds_addr(L.vs + 256 * (w - 2)));
}

// bf16 quarter block (keys k0 .. k0 + 31), chunk-major as the FP4 block: K
// chunk j (channels 8 j .. + 7) of the key at position p at k + 512 j + 16 p,
// position p = 16 b + 4 a + c holding key 8 a + 4 b + c, by direct copies (one
// per wavefront); V through registers (two keys x 4 channels per thread) for
// a transposed store: chunk j (keys 8 j .. + 7) of channel ch at
// vt + 2048 j + 16 ch.
struct LdsBq {
    uint8_t k[32 * D * 2];      // 32 keys x 256 B
    uint8_t vt[D * 32 * 2];     // 128 channels x 64 B (32 keys)
};
struct VStageQ {
    v2i v[2];
};
__device__ __forceinline__ void issue_bq(const ThriftFwdArgs& a, int b, int hk, int k0, LdsBq& L, int w, int l, int tid,
                                         VStageQ& vs) {
    const uint16_t* kb = (const uint16_t*)a.k_hi.p + b * a.k_hi.sB + hk * a.k_hi.sH + (int64_t)k0 * a.k_hi.sN;
    const int j = 2 * w + (l >> 5), p = l & 31;
    const int kk = 8 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3);
    lds_copy16((uint32_t)(2 * (kk * a.k_hi.sN + 8 * j)), kb, lds_addr(L.k + 1024 * w));
    const uint16_t* vb = (const uint16_t*)a.v_hi.p + b * a.v_hi.sB + hk * a.v_hi.sH;
    const int kp = tid & 15, cq = tid >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u) vs.v[u] = *(const v2i*)(vb + (int64_t)(k0 + 2 * kp + u) * a.v_hi.sN + 4 * cq);
}
__device__ __forceinline__ void store_bq(const VStageQ& vs, LdsBq& L, int tid) {
    const int kp = tid & 15, cq = tid >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // channel 4 cq + e, keys 2 kp and 2 kp + 1
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t x = __builtin_amdgcn_perm((uint32_t)vs.v[1][e >> 1], (uint32_t)vs.v[0][e >> 1], sel);
        const int r = 4 * cq + e;
        *(uint32_t*)(L.vt + 2048 * (kp >> 2) + 16 * r + 4 * (kp & 3)) = x;
    }
}
union LdsBuf16 {
    LdsF4 f;
    LdsBq b;
    LdsF4Bias p;
};

template <bool PTQ>
__global__ __launch_bounds__(512, 4) void thrift_fwd_kernel(ThriftFwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsBuf16 lds[2];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, q = l & 15;
    const int nqt = (a.Nq + BM - 1) / BM;
    const int grid = gridDim.x;
    // XCD-aware order: each XCD takes a contiguous range, heavy (late) query blocks first
    const int bid = (grid & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3);
    const int qt = nqt - 1 - bid % nqt;
    const int bh = bid / nqt, b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / (a.Hq / a.Hkv), bhk = b * a.Hkv + hk;
    const int qrow = qt * BM + 16 * w + q;
    const bool row_ok = qrow < a.Nq;
    const int off = a.Nk - a.Nq;                       // bottom-right alignment of the causal mask
    const int qpos = off + qrow;
    const int qpos_lo = off + qt * BM;                 // smallest position in the workgroup
    const int qpos_hi = off + (qt * BM + BM - 1 < a.Nq - 1 ? qt * BM + BM - 1 : a.Nq - 1);
    const int nkb = a.Nk / KB;
    const int nJ = a.causal ? (qpos_hi / KB + 1 < nkb ? qpos_hi / KB + 1 : nkb) : nkb;
    // the selection list through the scalar cache: its reads then wait on the
    // scalar counter, not on the vector one that also counts the block copies
    const __attribute__((address_space(4))) int32_t* sel =
        PTQ ? nullptr : uniform_ptr(a.sel_idx + ((int64_t)bh * nqt + qt) * a.max_sel);
    const int ns = PTQ ? 0 : a.sel_cnt[(int64_t)bh * nqt + qt];
    const float* brow = PTQ ? a.sbias + ((int64_t)bh * nqt + qt) * a.Nk : nullptr;
    // waves 4 and 5 copy the 128 shifts of key block J next to its codes
    auto issue_bias = [&](int J, LdsBuf16& L) {
        if (PTQ && (w == 4 || w == 5))
            lds_copy4((uint32_t)(4 * l), brow + J * KB + 64 * (w - 4), lds_addr(L.p.bias + 64 * (w - 4)));
    };
    const float c = a.c_log2;

    // FP4 query codes: B operand of S^T (channels 32 g .. 32 g + 31)
    const v4i qb = row_ok ? *(const v4i*)(a.qc + ((int64_t)bh * a.Nq + qrow) * (D / 2) + 16 * g) : v4i{};
    const int qsb = row_ok ? (int)a.qs[((int64_t)bh * a.Nq + qrow) * (D / 32) + g] : 0;

    v4f oacc[D / 16];                  // O^T tile cb: channels 16 cb + 4 g + i of row q
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) oacc[cb] = v4f{};
    float m_run = -__builtin_inff();   // running maximum (log2 units); -inf before the first finite score
    float l_run = 0.0f;                // this lane's share of the row sum
    float gsc = 1.0f;                  // FP4 path: oacc holds O / gsc, gsc = r / 6 of the last block

    // LDS byte offsets of this lane's operands (block-independent parts)
    // (S MFMA b reads key 32 (q / 4) + 4 b + q % 4, at position 16 b + q)
    const int koff = 2048 * g + 16 * q;      // + 256 b
    const int ksoff = 4 * q + g;             // + 64 b
    const int voff = 2048 * g + 16 * q;      // channel 16 cb + q: + 256 cb
    const int vsoff = 4 * q + g;             // + 64 cb

    // ------------------------------------------------------------ FP4 path
    int sp = 0;
    auto next_unsel = [&](int J) {
        while (sp < ns && sel[sp] < J) ++sp;
        while (J < nJ && sp < ns && sel[sp] == J) { ++J; ++sp; }
        return J;
    };
    auto f4_step = [&](auto slot, int J, int Jn) __attribute__((always_inline)) {
        constexpr int SB = decltype(slot)::value;
        if (Jn < nJ) {
            issue_f4_16(a, bhk, Jn, lds[SB ^ 1].f, w, l);
            issue_bias(Jn, lds[SB ^ 1]);
        }
        const LdsF4& L = lds[SB].f;
        // scores: s[b][i] is key 32 g + 4 b + i of the block
        v4f s[8];
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const v4i av = *(const v4i*)(L.kc + koff + 256 * bb);
            s[bb] = mfma_f4_16x16x128(av, (int)L.ks[ksoff + 64 * bb], qb, qsb, v4f{});
        }
        if constexpr (PTQ) {
#pragma unroll
            for (int bb = 0; bb < 8; ++bb) {
                const v4f sh = *(const v4f*)(lds[SB].p.bias + 32 * g + 4 * bb);
#pragma unroll
                for (int i = 0; i < 4; ++i) s[bb][i] += sh[i];
            }
        }
        if (a.causal && J * KB + KB - 1 > qpos_lo) {
#pragma unroll
            for (int bb = 0; bb < 8; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (J * KB + 32 * g + 4 * bb + i > qpos) s[bb][i] = -__builtin_inff();
        }
        // the lane's MX block maximum, then the row's over its four lanes
        float gm = max3f(s[0][0], s[0][1], s[0][2]);
#pragma unroll
        for (int k = 3; k < 31; k += 2) gm = max3f(gm, s[k >> 2][k & 3], s[(k + 1) >> 2][(k + 1) & 3]);
        gm = max2f(gm, s[7][3]);
        const float smax = quad_max16(gm);
        const float m_new = max2f(m_run, smax * c);
        const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        const float mu = m_new == -__builtin_inff() ? 0.0f : m_new;
        // two-level P: r = the row's largest P in the block, P' = P 6 / r =
        // 6 exp2((s - smax) c), formed directly by the exponential; the row
        // sum of P is r/6 times that of P'.  A block whose P all underflow
        // (r = 0) adds nothing.
        float r = __builtin_amdgcn_exp2f(__builtin_fmaf(smax, c, -mu));
        r = r >= R_FLOOR ? r : 0.0f;
        const float bias2 = r > 0.0f ? 2.584962500721156f - smax * c : -__builtin_inff();   // log2(6) - smax c
        float ps[4];
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[bb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][i], c, bias2));
                ps[i] = bb == 0 ? s[bb][i] : ps[i] + s[bb][i];
            }
        l_run *= alpha;
        if (r > 0.0f) l_run += ((ps[0] + ps[1]) + (ps[2] + ps[3])) * (r * (1.0f / 6.0f));
        m_run = m_new;
        const float six_r = r > 0.0f ? 6.0f * __builtin_amdgcn_rcpf(r) : 0.0f;
        const int e = mx_exponent(__builtin_amdgcn_exp2f(__builtin_fmaf(gm, c, bias2)));
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
        // accumulator units: from the previous block's r/6 (at the old maximum)
        // to this block's (when r = 0 the maximum did not move, alpha = 1)
        if (r > 0.0f) {
            const float ratio = gsc * six_r * alpha;
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[cb][i] *= ratio;
            gsc = r * (1.0f / 6.0f);
        }
        // P.V: the lane's P codes are its 32 keys; the scale is its MX block's
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
            const v4i av = *(const v4i*)(L.vc + voff + 256 * cb);
            oacc[cb] = mfma_f4_16x16x128(av, (int)L.vs[vsoff + 64 * cb], pb, e + 127, oacc[cb]);
        }
        BQA_WAIT_VM(0);
        barrier_only();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int J = next_unsel(0);
    if (J < nJ) {
        issue_f4_16(a, bhk, J, lds[0].f, w, l);
        issue_bias(J, lds[0]);
        BQA_WAIT_VM(0);
        barrier_only();
    }
    while (J < nJ) {
        int Jn = next_unsel(J + 1);
        f4_step(I0{}, J, Jn);
        J = Jn;
        if (J >= nJ) break;
        Jn = next_unsel(J + 1);
        f4_step(I1{}, J, Jn);
        J = Jn;
    }
    // back to plain units
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[cb][i] *= gsc;

    // ------------------------------------------------------------ bf16 path
    // selected blocks in quarters of 32 keys, each one tile of the online softmax
    const int n_items = 4 * ns;
    if (n_items > 0) {
        VStageQ vst;
        issue_bq(a, b, hk, sel[0] * KB, lds[0].b, w, l, tid, vst);
        store_bq(vst, lds[0].b, tid);
        BQA_WAIT_VM(0);
        barrier_only();
    }
    // Q in bf16, only for the selected blocks: channels 32 k + 8 g .. + 7
    v8bf qv[4];
    if (n_items > 0) {
        const uint16_t* qh = (const uint16_t*)a.q_hi.p + b * a.q_hi.sB + hq * a.q_hi.sH + (int64_t)(row_ok ? qrow : 0) * a.q_hi.sN;
#pragma unroll
        for (int k = 0; k < 4; ++k) qv[k] = *(const v8bf*)(qh + 32 * k + 8 * g);
    }
    // S MFMA bb of step k reads chunk 4 k + g of key 8 (q / 4) + 4 bb + q % 4
    // (position 16 bb + q); P.V reads chunk g of channel 16 cb + q
    const int kq = 512 * g + 16 * q;         // + 2048 k + 256 bb
    const int vq = 2048 * g + 16 * q;        // + 256 cb
    auto bf_step = [&](auto slot, int it) __attribute__((always_inline)) {
        constexpr int SB = decltype(slot)::value;
        const int k0 = sel[it >> 2] * KB + 32 * (it & 3);
        VStageQ vst;
        if (it + 1 < n_items)
            issue_bq(a, b, hk, sel[(it + 1) >> 2] * KB + 32 * ((it + 1) & 3), lds[SB ^ 1].b, w, l, tid, vst);
        const LdsBq& L = lds[SB].b;
        v4f s[2] = {v4f{}, v4f{}};
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const v8bf av = *(const v8bf*)(L.k + kq + 2048 * k + 256 * bb);
                s[bb] = mfma_bf16_16x16x32(av, qv[k], s[bb]);
            }
        // s[bb][i] is key k0 + 8 g + 4 bb + i
        if (a.causal && k0 + 31 > qpos_lo) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (k0 + 8 * g + 4 * bb + i > qpos) s[bb][i] = -__builtin_inff();
        }
        float m = max3f(max3f(s[0][0], s[0][1], s[0][2]), s[0][3], s[1][0]);
        m = max3f(m, s[1][1], max3f(s[1][2], s[1][3], m));
        const float m_new = max2f(m_run, quad_max16(m) * c);
        if (__any(m_new > m_run)) {
            const float f = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= f;
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[cb][i] *= f;
        }
        m_run = m_new;
        const float mu = m_run == -__builtin_inff() ? 0.0f : m_run;
        float ps[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[0][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][i], c, -mu));
            s[1][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1][i], c, -mu));
            ps[i] = s[0][i] + s[1][i];
        }
        l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        // P.V in bf16: the lane's keys 8 g + j of the quarter
        v8bf pbf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pbf[j] = (__bf16)s[j >> 2][j & 3];
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
            const v8bf av = *(const v8bf*)(L.vt + vq + 256 * cb);
            oacc[cb] = mfma_bf16_16x16x32(av, pbf, oacc[cb]);
        }
        if (it + 1 < n_items) store_bq(vst, lds[SB ^ 1].b, tid);
        BQA_WAIT_VM(0);
        barrier_only();
    };
    for (int it = 0; it < n_items; it += 2) {
        bf_step(I0{}, it);
        bf_step(I1{}, it + 1);
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
    if (a.lse && g == 0) a.lse[(int64_t)bh * a.Nq + qrow] = m_run * 0.6931471805599453f + __logf(l_tot);
}

// Score shifts of the post-training baseline: bias[b, hq, I, j] =
// qbar_I . k^_j, the bf16 block mean of query block I against the
// dequantised MXFP4 key j (exact in bf16), as one bf16 matrix product per
// head with fp32 sums: A = qbar rows (32 query blocks), B = k^ (32 keys per
// wavefront, 128 per workgroup).  grid B * Hq * (Nk / 128).
__global__ __launch_bounds__(256) void ptq_bias_kernel(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks,
                                                       const float* __restrict__ qbar, int Hq, int Hkv, int nqb,
                                                       int Nk, float* __restrict__ bias) {
    const int nkb = Nk / KB;
    const int bhq = blockIdx.x / nkb, kb = blockIdx.x % nkb;
    const int b = bhq / Hq, hq = bhq % Hq, bhk = b * Hkv + hq / (Hq / Hkv);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lq = l & 31, h = l >> 5;
    const int key = kb * KB + 32 * w + lq;
    // B operand: key `key`, channels 16 s + 8 h .. + 7 of step s
    const uint8_t* krow = kc + ((int64_t)bhk * Nk + key) * (D / 2);
    v4i raw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = *(const v4i*)(krow + 16 * q);
    const uint32_t sc4 = *(const uint32_t*)(ks + ((int64_t)bhk * Nk + key) * (D / 32));
    v8bf kb8[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const uint32_t word = (uint32_t)raw[st >> 1][2 * (st & 1) + h];
        const float sc = __builtin_bit_cast(float, ((sc4 >> (8 * (st >> 1))) & 0xFFu) << 23);
        const v4i pk = {__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0)),
                        __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1)),
                        __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2)),
                        __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3))};
        kb8[st] = __builtin_bit_cast(v8bf, pk);
    }
    const float* qb0 = qbar + (int64_t)bhq * nqb * D;
    float* out = bias + (int64_t)bhq * nqb * Nk + key;
    for (int q0 = 0; q0 < nqb; q0 += 32) {
        const int qb = q0 + lq;
        v16f acc = v16f{};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            v8bf av;
            if (qb < nqb) {
                const v4f x0 = *(const v4f*)(qb0 + (int64_t)qb * D + 16 * st + 8 * h);
                const v4f x1 = *(const v4f*)(qb0 + (int64_t)qb * D + 16 * st + 8 * h + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    av[e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(x0[e]));
                    av[4 + e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(x1[e]));
                }
            } else {
                av = v8bf{};
            }
            acc = mfma_bf16_32x32x16(av, kb8[st], acc);
        }
        // register r of half h is query block q0 + 8 (r / 4) + 4 h + r % 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (row < nqb) out[(int64_t)row * Nk] = acc[r];
        }
    }
}

// Two-level NVFP4 quantisation of 16 probabilities (one e2m1 block) of a
// row whose tile maximum r maps to 448 * 6 (f_in = 2688 / r): block scale
// e4m3(fp32(amax / 6)), values e2m1(fp32(P' / s_b)) s_b, then back by
// f_out = r / 2688 (the caller rounds the result to bf16 for P.V).
__device__ __forceinline__ void nv_p16(v16f& p, float f_in, float f_out) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        p[i] = p[i] * f_in;
        am = __builtin_fmaxf(am, p[i]);
    }
    const float sb = e4m3_round(am / 6.0f);
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        if (sb != 0.0f) {
            const v2f q = e2m1_round2(p[i] / sb, p[i + 1] / sb);
            p[i] = (q[0] * sb) * f_out;
            p[i + 1] = (q[1] * sb) * f_out;
        } else {
            p[i] = p[i + 1] = 0.0f;
        }
    }
}

// ThriftAttention prefill with the FP4 path in NVFP4 emulation ("Thrift-
// Attention", Method step 2 names NVFP4): the scaled matrix instructions take
// only power-of-two block scales, so the unselected blocks run the 16-bit
// instructions on the dequantised NVFP4 Q, K, V (exact in bf16) with P
// quantised in two levels to NVFP4 in registers (each lane's 16 keys of a
// half-tile form one e2m1 block); the selected blocks follow through the
// ordinary bf16 path.  Tiles of 64 keys, FlashAttention-2's online softmax.
__global__ __launch_bounds__(256, 2) void thrift_nv_kernel(ThriftFwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsBf lds[2];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int nqt = (a.Nq + BM - 1) / BM;
    const int grid = gridDim.x;
    const int bid = (grid & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3);
    const int qt = nqt - 1 - bid % nqt;
    const int bh = bid / nqt, b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int qrow = qt * BM + 32 * w + lq;
    const bool row_ok = qrow < a.Nq;
    const int krow = sigma(lq);
    const int off = a.Nk - a.Nq;
    const int qpos = off + qrow;
    const int qpos_lo = off + qt * BM;
    const int qpos_hi = off + (qt * BM + BM - 1 < a.Nq - 1 ? qt * BM + BM - 1 : a.Nq - 1);
    const int nkb = a.Nk / KB;
    const int nJ = a.causal ? (qpos_hi / KB + 1 < nkb ? qpos_hi / KB + 1 : nkb) : nkb;
    const int32_t* sel = a.sel_idx + ((int64_t)bh * nqt + qt) * a.max_sel;
    const int ns = a.sel_cnt[(int64_t)bh * nqt + qt];
    const float c = a.c_log2;

    v16f oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = v16f{};
    float m_run = -__builtin_inff(), l_run = 0.0f;

    // items: halves of 64 keys, first those of the unselected valid blocks
    // (phase 0, NVFP4), then those of the selected blocks (phase 1, bf16)
    int sp = 0;
    auto next_unsel = [&](int J) {
        while (sp < ns && sel[sp] < J) ++sp;
        while (J < nJ && sp < ns && sel[sp] == J) { ++J; ++sp; }
        return J;
    };
    struct Item { int J, half, phase, si; };
    auto after_phase0 = [&]() { return ns > 0 ? Item{sel[0], 0, 1, 0} : Item{-1, 0, 0, 0}; };
    auto advance = [&](Item x) {
        if (x.half == 0) return Item{x.J, 1, x.phase, x.si};
        if (x.phase == 0) {
            const int J = next_unsel(x.J + 1);
            return J < nJ ? Item{J, 0, 0, 0} : after_phase0();
        }
        return x.si + 1 < ns ? Item{sel[x.si + 1], 0, 1, x.si + 1} : Item{-1, 0, 0, 0};
    };
    auto issue = [&](const Item& x, LdsBf& L, VStage& vs) {
        const int k0 = x.J * KB + HB * x.half;
        if (x.phase == 0) issue_bf(a.k_nv, a.v_nv, b, hk, k0, L, w, l, tid, vs);
        else issue_bf(a.k_hi, a.v_hi, b, hk, k0, L, w, l, tid, vs);
    };
    Item cur;
    {
        const int J0 = next_unsel(0);
        cur = J0 < nJ ? Item{J0, 0, 0, 0} : after_phase0();
    }
    if (cur.J >= 0) {
        VStage vst;
        issue(cur, lds[0], vst);
        store_bf(vst, lds[0], tid);
        BQA_WAIT_VM(0);
        barrier_only();
    }
    int buf = 0;
    const int qr = row_ok ? qrow : 0;
    while (cur.J >= 0) {
        const Item nx = advance(cur);
        VStage vst;
        if (nx.J >= 0) issue(nx, lds[buf ^ 1], vst);
        const LdsBf& L = lds[buf];
        const int k0 = cur.J * KB + HB * cur.half;
        const Dense& qx = cur.phase == 0 ? a.q_nv : a.q_hi;
        const uint16_t* qh = (const uint16_t*)qx.p + b * qx.sB + hq * qx.sH + (int64_t)qr * qx.sN;
        v8bf qv[8];
#pragma unroll
        for (int st = 0; st < 8; ++st) qv[st] = *(const v8bf*)(qh + 16 * st + 8 * h);
        v16f s0 = v16f{}, s1 = v16f{};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const v8bf a0 = *(const v8bf*)(L.k + krow * 256 + 16 * ((2 * st + h) ^ fk256(krow)));
            const v8bf a1 = *(const v8bf*)(L.k + (32 + krow) * 256 + 16 * ((2 * st + h) ^ fk256(32 + krow)));
            s0 = mfma_bf16_32x32x16(a0, qv[st], s0);
            s1 = mfma_bf16_32x32x16(a1, qv[st], s1);
        }
        if (a.causal && k0 + HB - 1 > qpos_lo) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (k0 + 16 * h + i > qpos) s0[i] = -__builtin_inff();
                if (k0 + 32 + 16 * h + i > qpos) s1[i] = -__builtin_inff();
            }
        }
        float m = __builtin_fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) m = __builtin_fmaxf(__builtin_fmaxf(m, s0[i]), s1[i]);
        follow_max(oacc, l_run, m_run, __builtin_fmaxf(m_run, __builtin_fmaxf(m, partner32f(m)) * c));
        const float mu = m_run == -__builtin_inff() ? 0.0f : m_run;
        float ps[2] = {0.0f, 0.0f};
        float r = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -mu));
            s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -mu));
            ps[0] += s0[i];
            ps[1] += s1[i];
            r = __builtin_fmaxf(r, __builtin_fmaxf(s0[i], s1[i]));
        }
        l_run += ps[0] + ps[1];
        if (cur.phase == 0) {
            r = __builtin_fmaxf(r, partner32f(r));
            if (r > 0.0f) {
                const float f_in = 2688.0f / r, f_out = r / 2688.0f;
                nv_p16(s0, f_in, f_out);
                nv_p16(s1, f_in, f_out);
            }
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            v8bf pbf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pbf[e] = (__bf16)(st < 2 ? s0[8 * (st % 2) + e] : s1[8 * (st % 2) + e]);
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int rr = 32 * cb + lq;
                const v8bf av = *(const v8bf*)(L.vt + rr * 128 + 16 * ((4 * (st / 2) + 2 * h + (st % 2)) ^ fv128(rr)));
                oacc[cb] = mfma_bf16_32x32x16(av, pbf, oacc[cb]);
            }
        }
        if (nx.J >= 0) store_bf(vst, lds[buf ^ 1], tid);
        BQA_WAIT_VM(0);
        barrier_only();
        buf ^= 1;
        cur = nx;
    }

    const float l_tot = l_run + partner32f(l_run);
    if (!row_ok) return;
    const float inv_l = 1.0f / l_tot;
    uint16_t* orow = (uint16_t*)a.o.p + b * a.o.sB + hq * a.o.sH + (int64_t)qrow * a.o.sN;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int ch0 = 32 * cb + 8 * g + 4 * h;
            uint16_t o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = f32_to_bf16_bits(oacc[cb][4 * g + e] * inv_l);
            *(uint2*)(orow + ch0) =
                make_uint2((uint32_t)o4[0] | ((uint32_t)o4[1] << 16), (uint32_t)o4[2] | ((uint32_t)o4[3] << 16));
        }
    }
    if (a.lse && h == 0) a.lse[(int64_t)bh * a.Nq + qrow] = m_run * 0.6931471805599453f + __logf(l_tot);
}

}  // namespace

hipError_t launch_thrift_nv(const ThriftFwdArgs& a, hipStream_t st) {
    thrift_nv_kernel<<<a.B * a.Hq * ((a.Nq + BM - 1) / BM), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_thrift_fwd(const ThriftFwdArgs& a, hipStream_t st) {
    const int grid = a.B * a.Hq * ((a.Nq + BM - 1) / BM);
    thrift_fwd_kernel<false><<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
}

size_t ws_ptq_fwd_bytes(int B, int Hq, int Nq, int Nk) {
    return (size_t)B * Hq * ((Nq + BM - 1) / BM) * Nk * sizeof(float);
}

hipError_t launch_ptq_fwd(ThriftFwdArgs a, const float* qbar, void* ws, hipStream_t st) {
    const int nqb = (a.Nq + BM - 1) / BM;
    float* bias = (float*)ws;
    ptq_bias_kernel<<<a.B * a.Hq * (a.Nk / KB), 256, 0, st>>>(a.kc, a.ks, qbar, a.Hq, a.Hkv, nqb, a.Nk, bias);
    a.sbias = bias;
    thrift_fwd_kernel<true><<<a.B * a.Hq * nqb, 512, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace bqa

// ============================================================================
// ThriftAttention decode ("ThriftAttention" technical summary, Methodology
// step 2 and the decode results): one query token per (batch, query head)
// against the whole cache.  One wavefront per (batch, KV head, key-range
// split): the G = Hq / Hkv query heads of the KV head are the columns of the
// matrix tiles, so each K/V block is read once for all of them.  Inside a
// split the key blocks that not every head selected run through the FP4
// path (heads that selected the block are masked there), then the blocks
// any head selected run through the bf16 path in quarters of 32 keys (heads
// that did not select it are masked; each quarter is one tile of the online
// softmax).  Each split leaves a partial (running maximum m, l, O) per head;
// decode_combine merges them.
namespace bqa {
namespace {

constexpr int DQ = 32;     // bf16 keys per decode step
constexpr int PART = D + 4; // partial record: running maximum m, row sum l, 2 pad, O[d]

struct LdsDec {
    union {
        LdsF4 f;
        struct {
            uint8_t k[DQ * D * 2];    // 32 keys x 256 B
            uint8_t vt[D * DQ * 2];   // 128 channels x 64 B (32 keys)
        } b;
    };
};

// FP4 key block J: K codes and scales (token-major, contiguous) and V codes
// and scales (a decode step reads each byte of the cache once: the copies
// are non-temporal), either channel-major over the whole cache (a channel's 64
// bytes of the block are half of a 128-byte line, its 4 scale bytes a
// sliver of another) or blocked by 128 keys (the block's 8 KB of codes and
// 512 bytes of scales contiguous, each line read whole once).
__device__ __forceinline__ void dec_issue_f4(const ThriftDecArgs& a, int bhk, int J, LdsF4& L, int l) {
    const int t0 = J * KB;
    const uint8_t* kbase = a.kc + ((int64_t)bhk * a.Nk + t0) * (D / 2);
    const int nb = a.Nk / KB;
    const uint8_t* vbase = a.v_tiled ? a.vc + ((int64_t)bhk * nb + J) * D * (KB / 2)
                                     : a.vc + (int64_t)bhk * D * (a.Nk / 2) + t0 / 2;
    const uint32_t vrow = a.v_tiled ? (uint32_t)(KB / 2) : (uint32_t)(a.Nk / 2);
#pragma unroll
    for (int sgm = 0; sgm < 8; ++sgm) {
        const int r = 16 * sgm + (l >> 2);
        lds_copy16_nt((uint32_t)(r * (D / 2) + 16 * ((l & 3) ^ fk64(r))), kbase, lds_addr(L.kc + 1024 * sgm));
        lds_copy16_nt((uint32_t)r * vrow + (uint32_t)(16 * ((l & 3) ^ fv64(r))), vbase, lds_addr(L.vc + 1024 * sgm));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        lds_copy4_nt((uint32_t)(4 * l), a.ks + ((int64_t)bhk * a.Nk + t0 + 64 * u) * (D / 32), lds_addr(L.ks + 256 * u));
        if (a.v_tiled)
            lds_copy4_nt((uint32_t)(4 * l), a.vs + (((int64_t)bhk * nb + J) * D + 64 * u) * (KB / 32),
                      lds_addr(L.vs + 256 * u));
        else
            lds_copy4_nt((uint32_t)l * (uint32_t)(a.Nk / 32), a.vs + ((int64_t)bhk * D + 64 * u) * (a.Nk / 32) + t0 / 32,
                      lds_addr(L.vs + 256 * u));
    }
}

struct VQuarter {
    v4i v[8];
};
// 32 keys from k0: K rows by direct copies; V (keys 4 kq + u and 16 + 4 kq + u,
// channels 8 cg ..) into registers for the transposed store.
__device__ __forceinline__ void dec_issue_bf(const ThriftDecArgs& a, int b, int hk, int k0, LdsDec& L, int l,
                                             VQuarter& vq) {
    const uint16_t* kb = (const uint16_t*)a.k_hi.p + b * a.k_hi.sB + hk * a.k_hi.sH + (int64_t)k0 * a.k_hi.sN;
#pragma unroll
    for (int sgm = 0; sgm < 8; ++sgm) {
        const int r = 4 * sgm + (l >> 4);
        lds_copy16_nt((uint32_t)(2 * (r * a.k_hi.sN + 8 * ((l & 15) ^ fk256(r)))), kb, lds_addr(L.b.k + 1024 * sgm));
    }
    const uint16_t* vb = (const uint16_t*)a.v_hi.p + b * a.v_hi.sB + hk * a.v_hi.sH;
    const int cg = l & 15, kq = l >> 4;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int key = 16 * (u >> 2) + 4 * kq + (u & 3);
        vq.v[u] = __builtin_nontemporal_load((const v4i*)(vb + (int64_t)(k0 + key) * a.v_hi.sN + 8 * cg));
    }
}
__device__ __forceinline__ void dec_store_bf(const VQuarter& vq, LdsDec& L, int l) {
    const int cg = l & 15, kq = l >> 4;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int kw = 4 * hf + kq;    // 4-key group: keys 4 kw .. 4 kw + 3
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t lo = __builtin_amdgcn_perm((uint32_t)vq.v[4 * hf + 1][e >> 1], (uint32_t)vq.v[4 * hf][e >> 1], sel);
            const uint32_t hi = __builtin_amdgcn_perm((uint32_t)vq.v[4 * hf + 3][e >> 1], (uint32_t)vq.v[4 * hf + 2][e >> 1], sel);
            const int r = 8 * cg + e;
            *(v2i*)(L.b.vt + r * 64 + 16 * ((kw >> 1) ^ fv64(r)) + 8 * (kw & 1)) = v2i{(int)lo, (int)hi};
        }
    }
}

__global__ __launch_bounds__(64) void thrift_decode_kernel(ThriftDecArgs a) {
    __shared__ __attribute__((aligned(16))) LdsDec lds[2];
    extern __shared__ uint32_t hmask[];                 // per key block of the split: heads that selected it
    const int l = threadIdx.x, h = l >> 5, lq = l & 31;
    const int S = a.splits;
    const int sp = blockIdx.x % S;
    const int bhk = blockIdx.x / S, b = bhk / a.Hkv, hk = bhk % a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int nb = a.Nk / KB;
    const int b0 = (int)((int64_t)sp * nb / S), b1 = (int)((int64_t)(sp + 1) * nb / S);
    const bool col_ok = lq < G;
    const int hq = hk * G + (col_ok ? lq : 0);
    const int bhq = b * a.Hq + hq;
    const int krow = sigma(lq);
    const float c = a.c_log2;
    const uint32_t all = G >= 32 ? 0xFFFFFFFFu : ((1u << G) - 1u);

    for (int j = l; j < b1 - b0; j += 64) hmask[j] = 0u;
    __syncthreads();
    for (int g = 0; g < G; ++g) {
        const int32_t* sel = a.sel_idx + (int64_t)(b * a.Hq + hk * G + g) * a.max_sel;
        const int cnt = a.sel_cnt[b * a.Hq + hk * G + g];
        for (int u = l; u < cnt; u += 64) {
            const int J = sel[u];
            if (J >= b0 && J < b1) atomicOr(&hmask[J - b0], 1u << g);
        }
    }
    __syncthreads();

    v4i qb[2];
    int qsb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        qb[kk] = col_ok ? *(const v4i*)(a.qc + (int64_t)bhq * (D / 2) + 32 * kk + 16 * h) : v4i{};
        qsb[kk] = col_ok ? (int)a.qs[(int64_t)bhq * (D / 32) + 2 * kk + h] : 0;
    }
    __builtin_amdgcn_s_waitcnt(0);

    v16f oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = v16f{};
    float m_run = -__builtin_inff(), l_run = 0.0f, gsc = 1.0f;
    const uint32_t mybit = col_ok ? (1u << lq) : 0u;

    // ------------------------------------------------------------ FP4 blocks
    auto next_f4 = [&](int J) {
        while (J < b1 && hmask[J - b0] == all) ++J;
        return J;
    };
    int J = next_f4(b0), buf = 0;
    if (J < b1) {
        dec_issue_f4(a, bhk, J, lds[0].f, l);
        BQA_WAIT_VM(0);
        barrier_only();
    }
    while (J < b1) {
        const int Jn = next_f4(J + 1);
        if (Jn < b1) dec_issue_f4(a, bhk, Jn, lds[buf ^ 1].f, l);
        const LdsF4& L = lds[buf].f;
        const bool skip = !col_ok || (hmask[J - b0] & mybit);
        v16f s[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            s[t] = v16f{};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int r = 32 * t + krow;
                const v4i av = *(const v4i*)(L.kc + r * 64 + 16 * ((2 * kk + h) ^ fk64(r)));
                s[t] = mfma_f4_32x32x64(av, (int)L.ks[4 * r + 2 * kk + h], qb[kk], qsb[kk], s[t]);
            }
            if (skip) s[t] = v16f{} - __builtin_inff();
        }
        float bt[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float m = __builtin_fmaxf(s[t][0], s[t][1]);
#pragma unroll
            for (int i = 2; i < 16; i += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, s[t][i]), s[t][i + 1]);
            bt[t] = __builtin_fmaxf(m, partner32f(m));
        }
        const float smax = __builtin_fmaxf(__builtin_fmaxf(bt[0], bt[1]), __builtin_fmaxf(bt[2], bt[3]));
        const float m_new = __builtin_fmaxf(m_run, smax * c);
        const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        const float mu = m_new == -__builtin_inff() ? 0.0f : m_new;
        // two-level P formed directly as P' = 6 exp2((s - smax) c) (see the prefill)
        float r = __builtin_amdgcn_exp2f(__builtin_fmaf(smax, c, -mu));
        r = r >= R_FLOOR ? r : 0.0f;
        const float bias2 = r > 0.0f ? 2.584962500721156f - smax * c : -__builtin_inff();   // log2(6) - smax c
        float ps[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float q0 = 0.0f, q1 = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                s[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], c, bias2));
                s[t][i + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i + 1], c, bias2));
                q0 += s[t][i];
                q1 += s[t][i + 1];
            }
            ps[t] = q0 + q1;
        }
        l_run *= alpha;
        if (r > 0.0f) l_run += ((ps[0] + ps[1]) + (ps[2] + ps[3])) * (r * (1.0f / 6.0f));
        m_run = m_new;
        const float six_r = r > 0.0f ? 6.0f / r : 0.0f;
        int e[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) e[t] = mx_exponent(__builtin_amdgcn_exp2f(__builtin_fmaf(bt[t], c, bias2)));
        uint32_t pw[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float sc = __builtin_bit_cast(float, (uint32_t)(e[t] + 127) << 23);
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
                uint32_t x = 0;
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 0], s[t][8 * wd + 1], sc, 0);
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 2], s[t][8 * wd + 3], sc, 1);
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 4], s[t][8 * wd + 5], sc, 2);
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 6], s[t][8 * wd + 7], sc, 3);
                pw[t][wd] = x;
            }
        }
        // (when r = 0 the maximum did not move, alpha = 1)
        if (r > 0.0f) {
            const float ratio = gsc * six_r * alpha;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[cb][i] *= ratio;
            gsc = r * (1.0f / 6.0f);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const v2i r0 = __builtin_amdgcn_permlane32_swap((int)pw[2 * g][0], (int)pw[2 * g + 1][0], false, false);
            const v2i r1 = __builtin_amdgcn_permlane32_swap((int)pw[2 * g][1], (int)pw[2 * g + 1][1], false, false);
            const v4i pb = {r0[0], r1[0], r0[1], r1[1]};
            const int psc = (h ? e[2 * g + 1] : e[2 * g]) + 127;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int rr = 32 * cb + lq;
                const v4i av = *(const v4i*)(L.vc + rr * 64 + 16 * ((2 * g + h) ^ fv64(rr)));
                oacc[cb] = mfma_f4_32x32x64(av, (int)L.vs[4 * rr + 2 * g + h], pb, psc, oacc[cb]);
            }
        }
        BQA_WAIT_VM(0);
        barrier_only();
        J = Jn;
        buf ^= 1;
    }
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[cb][i] *= gsc;

    // ------------------------------------------------------------ bf16 blocks, 32 keys at a time
    auto next_bf = [&](int it) {        // item = 4 J + quarter
        while ((it >> 2) < b1 - b0 && hmask[it >> 2] == 0u) it = (it | 3) + 1;
        return it;
    };
    const int n_it = 4 * (b1 - b0);
    int it = next_bf(0);
    buf = 0;
    if (it < n_it) {
        VQuarter vq;
        dec_issue_bf(a, b, hk, (b0 + (it >> 2)) * KB + DQ * (it & 3), lds[0], l, vq);
        dec_store_bf(vq, lds[0], l);
        BQA_WAIT_VM(0);
        barrier_only();
    }
    const uint16_t* qh = (const uint16_t*)a.q_hi.p + b * a.q_hi.sB + hq * a.q_hi.sH;
    v8bf qv[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) qv[st] = *(const v8bf*)(qh + 16 * st + 8 * h);
    while (it < n_it) {
        const int itn = next_bf(it + 1);
        VQuarter vq;
        if (itn < n_it) dec_issue_bf(a, b, hk, (b0 + (itn >> 2)) * KB + DQ * (itn & 3), lds[buf ^ 1], l, vq);
        const LdsDec& L = lds[buf];
        const bool skip = !col_ok || !(hmask[it >> 2] & mybit);
        v16f s0 = v16f{};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const v8bf av = *(const v8bf*)(L.b.k + krow * 256 + 16 * ((2 * st + h) ^ fk256(krow)));
            s0 = mfma_bf16_32x32x16(av, qv[st], s0);
        }
        if (skip) s0 = v16f{} - __builtin_inff();
        float m = s0[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = __builtin_fmaxf(m, s0[i]);
        follow_max(oacc, l_run, m_run, __builtin_fmaxf(m_run, __builtin_fmaxf(m, partner32f(m)) * c));
        const float mu = m_run == -__builtin_inff() ? 0.0f : m_run;
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -mu));
            ps += s0[i];
        }
        l_run += ps;
        // keys 16 h + 8 st + e of the quarter
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            v8bf pbf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pbf[e] = (__bf16)s0[8 * st + e];
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int rr = 32 * cb + lq;
                const v8bf av = *(const v8bf*)(L.b.vt + rr * 64 + 16 * ((2 * h + st) ^ fv64(rr)));
                oacc[cb] = mfma_bf16_32x32x16(av, pbf, oacc[cb]);
            }
        }
        if (itn < n_it) dec_store_bf(vq, lds[buf ^ 1], l);
        BQA_WAIT_VM(0);
        barrier_only();
        it = itn;
        buf ^= 1;
    }

    // partial of this split: running maximum m (log2 units), row sum, unnormalised O
    const float l_tot = l_run + partner32f(l_run);
    if (!col_ok) return;
    float* part = a.part + ((int64_t)bhq * S + sp) * PART;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int ch0 = 32 * cb + 8 * g + 4 * h;
            *(v4f*)(part + 4 + ch0) = v4f{oacc[cb][4 * g], oacc[cb][4 * g + 1], oacc[cb][4 * g + 2], oacc[cb][4 * g + 3]};
        }
    if (h == 0) {
        part[0] = m_run;
        part[1] = l_tot;
    }
}

// Merge the splits of one (batch, query head): m = max m_s,
// l = sum 2^(m_s - m) l_s, O = sum 2^(m_s - m) O_s / l.
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ part, int S, Dense o,
                                                             float* lse, int Hq) {
    const int bhq = blockIdx.x, ch = threadIdx.x;
    const float* p = part + (int64_t)bhq * S * PART;
    float m = -__builtin_inff();
    for (int s = 0; s < S; ++s) m = __builtin_fmaxf(m, p[(int64_t)s * PART]);
    float lsum = 0.0f, acc = 0.0f;
    for (int s = 0; s < S; ++s) {
        const float ms = p[(int64_t)s * PART];
        if (ms == -__builtin_inff()) continue;
        const float wgt = __builtin_amdgcn_exp2f(ms - m);
        lsum += wgt * p[(int64_t)s * PART + 1];
        acc += wgt * p[(int64_t)s * PART + 4 + ch];
    }
    const int b = bhq / Hq, hq = bhq % Hq;
    uint16_t* orow = (uint16_t*)o.p + b * o.sB + hq * o.sH;
    orow[ch] = f32_to_bf16_bits(acc / lsum);
    if (lse && ch == 0) lse[bhq] = m * 0.6931471805599453f + __logf(lsum);
}

// Decode workgroups the current device holds at once (compute units x the
// kernel's residency per CU, which its LDS sets to 4 on gfx950), cached per
// device; 256 x 4 when there is no device to ask.
int decode_capacity() {
    static std::atomic<int> cache[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
    int v = cache[dev].load(std::memory_order_acquire);
    if (v == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, thrift_decode_kernel, 64, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu * cus < 1)
            per_cu = 4, cus = 256;
        v = per_cu * cus;
        cache[dev].store(v, std::memory_order_release);
    }
    return v;
}

}  // namespace

// Automatic split count: as many splits as give one full round of resident
// workgroups (B * Hkv * S <= capacity).  Measured at c5d (B * Hkv = 128, 1024
// resident): 8 splits 0.605 ms for decode and merge, against 0.656 (6), 0.638
// (16), 0.687 (12) and 0.921 (4): a partial last round costs as much as a
// full one.
int decode_splits(int B, int Hkv, int Nk, int requested) {
    const int nb = Nk / KB;
    int S = requested > 0 ? requested : decode_capacity() / (B * Hkv);
    if (S > nb) S = nb;
    if (S < 1) S = 1;
    return S;
}

size_t ws_decode_bytes(int B, int Hq, int Hkv, int Nk, int requested) {
    return (size_t)B * Hq * decode_splits(B, Hkv, Nk, requested) * PART * sizeof(float);
}

// ---- allocation-free decode: the split partials in a static device array
// Callers that cannot allocate (code under graph capture, serving loops)
// get the partials from this array instead of a workspace.  Each device
// holds its own copy for the life of the process; every call on a device
// shares it, so calls that overlap on one device race.  Every split writes
// its whole record before the merge reads it, so nothing needs clearing.
namespace {
constexpr size_t kScratchFloats = (size_t)4 << 20;    // 16 MiB
__device__ __attribute__((aligned(256))) float scratch[kScratchFloats];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

size_t decode_scratch_bytes() { return kScratchFloats * sizeof(float); }

// Device address of this device's copy of `scratch` (looked up once per device).
hipError_t decode_scratch(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = (float*)ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_thrift_decode(const ThriftDecArgs& a, Dense o, float* lse, hipStream_t st) {
    const int nb = a.Nk / KB;
    const int max_blocks = (nb + a.splits - 1) / a.splits;
    thrift_decode_kernel<<<a.B * a.Hkv * a.splits, 64, max_blocks * sizeof(uint32_t), st>>>(a);
    decode_combine_kernel<<<a.B * a.Hq, D, 0, st>>>(a.part, a.splits, o, lse, a.Hq);
    return hipGetLastError();
}

}  // namespace bqa
