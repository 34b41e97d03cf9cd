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
// Layout: one workgroup of 4 wavefronts per 128 query rows (32 rows per
// wavefront, S^T = K Q^T so each lane owns one query row); FP4 key blocks of
// 128 keys, bf16 key blocks in two halves of 64.  The softmax keeps P in a
// fixed per-row power-of-two frame (MXFP4 codes, the two-level factor and
// bf16 roundings are all invariant under it), moved exactly only when a
// row's scores climb 64 binades above it.  The FP4 path's accumulator is
// kept in units of the current block's r/6, rescaled when the next block
// brings a new r.
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
union LdsBuf {
    LdsF4 f;
    LdsBf b;
};

__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// FP4 key block J: codes and scales of K and V^T, all by direct copies.
__device__ __forceinline__ void issue_f4(const ThriftFwdArgs& a, int bhk, int J, LdsF4& L, int w, int l) {
    const int t0 = J * KB;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int sgm = 2 * w + u, r = 16 * sgm + (l >> 2);
        dma16(a.kc + ((int64_t)bhk * a.Nk + t0 + r) * (D / 2) + 16 * ((l & 3) ^ fk64(r)), L.kc + 1024 * sgm);
        dma16(a.vc + ((int64_t)bhk * D + r) * (a.Nk / 2) + t0 / 2 + 16 * ((l & 3) ^ fv64(r)), L.vc + 1024 * sgm);
    }
    if (w < 2) dma4(a.ks + ((int64_t)bhk * a.Nk + t0 + 64 * w + l) * (D / 32), L.ks + 256 * w);
    else dma4(a.vs + ((int64_t)bhk * D + 64 * (w - 2) + l) * (a.Nk / 32) + t0 / 32, L.vs + 256 * (w - 2));
}

// bf16 half block (keys k0 .. k0 + 63): K rows by direct copies; V comes back
// in registers (4 keys x 8 channels per thread) for a transposed store.
struct VStage {
    v4i v[4];
};
__device__ __forceinline__ void issue_bf(const ThriftFwdArgs& a, int b, int hk, int k0, LdsBf& L, int w, int l,
                                         int tid, VStage& vs) {
    const uint16_t* kb = (const uint16_t*)a.k_hi.p + b * a.k_hi.sB + hk * a.k_hi.sH;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int sgm = 4 * w + u, r = 4 * sgm + (l >> 4);
        dma16(kb + (int64_t)(k0 + r) * a.k_hi.sN + 8 * ((l & 15) ^ fk256(r)), L.k + 1024 * sgm);
    }
    const uint16_t* vb = (const uint16_t*)a.v_hi.p + b * a.v_hi.sB + hk * a.v_hi.sH;
    const int cg = tid & 15, kq = tid >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) vs.v[u] = *(const v4i*)(vb + (int64_t)(k0 + 4 * kq + u) * a.v_hi.sN + 8 * cg);
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

// Exact rescale of every accumulator and of the row sum by 2^(m_old - m_new).
__device__ __forceinline__ void move_frame(v16f* oacc, float& l_run, float& m_ref, float m_new) {
    if (m_ref != -__builtin_inff()) {
        const float f = __builtin_ldexpf(1.0f, (int)(m_ref - m_new));
        l_run *= f;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[cb][i] *= f;
    }
    m_ref = m_new;
}

__global__ __launch_bounds__(256, 2) void thrift_fwd_kernel(ThriftFwdArgs a) {
    __shared__ __attribute__((aligned(16))) LdsBuf lds[2];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, lq = l & 31;
    const int nqt = (a.Nq + BM - 1) / BM;
    const int grid = gridDim.x;
    // XCD-aware order: each XCD takes a contiguous range, heavy (late) query blocks first
    const int bid = (grid & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3);
    const int qt = nqt - 1 - bid % nqt;
    const int bh = bid / nqt, b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / (a.Hq / a.Hkv), bhk = b * a.Hkv + hk;
    const int qrow = qt * BM + 32 * w + lq;
    const bool row_ok = qrow < a.Nq;
    const int krow = sigma(lq);
    const int off = a.Nk - a.Nq;                       // bottom-right alignment of the causal mask
    const int qpos = off + qrow;
    const int qpos_lo = off + qt * BM;                 // smallest position in the workgroup
    const int qpos_hi = off + (qt * BM + BM - 1 < a.Nq - 1 ? qt * BM + BM - 1 : a.Nq - 1);
    const int nkb = a.Nk / KB;
    const int nJ = a.causal ? (qpos_hi / KB + 1 < nkb ? qpos_hi / KB + 1 : nkb) : nkb;
    const int32_t* sel = a.sel_idx + ((int64_t)bh * nqt + qt) * a.max_sel;
    const int ns = a.sel_cnt[(int64_t)bh * nqt + qt];
    const float c = a.c_log2;

    // FP4 query codes: B operand of S^T (channels 64 kk + 32 h .. + 31)
    v4i qb[2];
    int qsb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        qb[kk] = row_ok ? *(const v4i*)(a.qc + ((int64_t)bh * a.Nq + qrow) * (D / 2) + 32 * kk + 16 * h) : v4i{};
        qsb[kk] = row_ok ? (int)a.qs[((int64_t)bh * a.Nq + qrow) * (D / 32) + 2 * kk + h] : 0;
    }
    __builtin_amdgcn_s_waitcnt(0);

    v16f oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = v16f{};
    float m_ref = -__builtin_inff();   // frame (log2 units, an integer); -inf before the first finite score
    float l_run = 0.0f;                // this lane half's share of the row sum, in the frame
    float gsc = 1.0f;                  // FP4 path: oacc holds O / gsc, gsc = r / 6 of the last block

    // ------------------------------------------------------------ FP4 path
    int sp = 0;
    auto next_unsel = [&](int J) {
        while (sp < ns && sel[sp] < J) ++sp;
        while (J < nJ && sp < ns && sel[sp] == J) { ++J; ++sp; }
        return J;
    };
    int J = next_unsel(0);
    if (J < nJ) {
        issue_f4(a, bhk, J, lds[0].f, w, l);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    int buf = 0;
    while (J < nJ) {
        const int Jn = next_unsel(J + 1);
        if (Jn < nJ) issue_f4(a, bhk, Jn, lds[buf ^ 1].f, w, l);
        const LdsF4& L = lds[buf].f;
        // scores: s[t] reg i of half h is key 32 t + 16 h + i of the block
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
        }
        if (a.causal && J * KB + KB - 1 > qpos_lo) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (J * KB + 32 * t + 16 * h + i > qpos) s[t][i] = -__builtin_inff();
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
        const float mx = smax * c;
        if (__any(mx > m_ref + 64.0f)) {
            if (mx > m_ref) move_frame(oacc, l_run, m_ref, __builtin_ceilf(mx));
        }
        const float mu = m_ref == -__builtin_inff() ? 0.0f : m_ref;
        float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], c, -mu));
                ps[t] += s[t][i];
            }
        l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        // two-level P: r = the row's largest P in the block -> 6
        const float r = __builtin_amdgcn_exp2f(__builtin_fmaf(smax, c, -mu));
        const float six_r = r > 0.0f ? 6.0f / r : 0.0f;
        int e[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) e[t] = mx_exponent(__builtin_amdgcn_exp2f(__builtin_fmaf(bt[t], c, -mu)) * six_r);
        uint32_t pw[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float sc = __builtin_bit_cast(float, (uint32_t)(e[t] + 127) << 23);
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
                uint32_t x = 0;
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 0] * six_r, s[t][8 * wd + 1] * six_r, sc, 0);
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 2] * six_r, s[t][8 * wd + 3] * six_r, sc, 1);
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 4] * six_r, s[t][8 * wd + 5] * six_r, sc, 2);
                x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[t][8 * wd + 6] * six_r, s[t][8 * wd + 7] * six_r, sc, 3);
                pw[t][wd] = x;
            }
        }
        // accumulator units: from the previous block's r/6 to this block's
        if (r > 0.0f) {
            const float ratio = gsc * six_r;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[cb][i] *= ratio;
            gsc = r * (1.0f / 6.0f);
        }
        // P.V: K-step g covers keys 64 g .. 64 g + 63; half 0 takes MX block 2 g, half 1 block 2 g + 1
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
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        J = Jn;
        buf ^= 1;
    }
    // back to plain frame units
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[cb][i] *= gsc;

    // ------------------------------------------------------------ bf16 path
    const int n_items = 2 * ns;
    if (n_items > 0) {
        VStage vst;
        issue_bf(a, b, hk, sel[0] * KB, lds[0].b, w, l, tid, vst);
        store_bf(vst, lds[0].b, tid);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    buf = 0;
    const uint16_t* qh = (const uint16_t*)a.q_hi.p + b * a.q_hi.sB + hq * a.q_hi.sH + (int64_t)(row_ok ? qrow : 0) * a.q_hi.sN;
    for (int it = 0; it < n_items; ++it) {
        const int k0 = sel[it >> 1] * KB + HB * (it & 1);
        VStage vst;
        if (it + 1 < n_items) issue_bf(a, b, hk, sel[(it + 1) >> 1] * KB + HB * ((it + 1) & 1), lds[buf ^ 1].b, w, l,
                                       tid, vst);
        const LdsBf& L = lds[buf].b;
        // Q in bf16, only for the selected blocks: channels 16 s + 8 h .. + 7
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
        const float mx = __builtin_fmaxf(m, partner32f(m)) * c;
        if (__any(mx > m_ref + 64.0f)) {
            if (mx > m_ref) move_frame(oacc, l_run, m_ref, __builtin_ceilf(mx));
        }
        const float mu = m_ref == -__builtin_inff() ? 0.0f : m_ref;
        float ps[2] = {0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -mu));
            s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -mu));
            ps[0] += s0[i];
            ps[1] += s1[i];
        }
        l_run += ps[0] + ps[1];
        // P.V in bf16: step st covers keys 32 (st / 2) + 16 h + 8 (st % 2) + e
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
        if (it + 1 < n_items) store_bf(vst, lds[buf ^ 1].b, tid);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        buf ^= 1;
        (void)k0;
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
    if (a.lse && h == 0) a.lse[(int64_t)bh * a.Nq + qrow] = m_ref * 0.6931471805599453f + __logf(l_tot);
}

}  // namespace

hipError_t launch_thrift_fwd(const ThriftFwdArgs& a, hipStream_t st) {
    const int grid = a.B * a.Hq * ((a.Nq + BM - 1) / BM);
    thrift_fwd_kernel<<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace bqa
