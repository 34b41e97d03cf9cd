// attn_sage_fwd.hip — SageAttention INT8 forward for gfx950.
//
// "SageBwd: A Trainable Low-bit Attention", Methodology 1 (INT8 attention with
// per-block scales) and 4 (K-smoothing, which happens in the K quantiser):
//   S_int = Qhat Khat^T exactly in int32 (i8 matrix instructions), scores
//   s = S_int * s_q * s_k * tau; online softmax over key tiles of 64
//   (FlashAttention-2 style); P rounded for the P.V product as fp16 (V fp16),
//   e4m3(448 P) (V per-channel e4m3) or int8 per (row, tile) (V per-channel
//   int8); the row sum accumulates the unrounded P.
//
// Work decomposition: one workgroup of 4 wavefronts per 128 query rows of one
// (batch, head); each wavefront owns 32 rows.  The score tile is computed
// transposed, S^T = Khat Qhat^T (A = key rows from LDS, B = the wavefront's
// query rows held in registers), so the 32x32 accumulator puts one query row
// in each lane (32 keys per lane, the other 32 of the tile in lane l^32).
// Row max and row sum are then in-lane reductions plus one permlane32 swap,
// and the probabilities are already laid out as the B operand of
// O^T = V^T P^T, which therefore needs no LDS round trip.  K tiles and the
// channel-major V tiles are staged in LDS with XOR-swizzled 16-byte chunks
// (conflict-free 128-bit reads for 16 consecutive lanes), double-buffered
// through registers so the next tile's HBM/L2 loads overlap the current
// tile's math.  Causal workgroups are issued heaviest-first; consecutive
// workgroup ids take different heads, which keeps each head on one XCD.
#include "common.hpp"
#include "internal.hpp"

namespace bqa {

namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile (= INT8 K block)

// LDS byte offset of logical 16-byte chunk `c` of row `r` in a tile whose rows
// are `row_bytes` long; XOR swizzle so 16 consecutive rows read at one logical
// chunk land in 16 distinct 16-byte bank groups.
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int r, int c) {
    constexpr int rows_per_256 = 256 / ROW_BYTES;
    constexpr int nch = ROW_BYTES / 16;
    return r * ROW_BYTES + 16 * (c ^ ((r / rows_per_256) & (nch - 1)));
}

// S^T tile of 64 keys x 32 queries for one wavefront: acc0 keys 0..31,
// acc1 keys 32..63 (of the tile in LDS); lane (q = l%32, half h) register i
// holds key 8(i/4) + 4h + i%4 (+32 for acc1).
template <int D>
__device__ __forceinline__ void qk_tile(const uint8_t* k_lds, const v4i* qb, int lq, int h, v16i& acc0, v16i& acc1) {
    acc0 = v16i{};
    acc1 = v16i{};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        v4i a0 = *(const v4i*)(k_lds + swz<D>(lq, 2 * kk + h));
        v4i a1 = *(const v4i*)(k_lds + swz<D>(32 + lq, 2 * kk + h));
        acc0 = mfma_i8_32x32x32(a0, qb[kk], acc0);
        acc1 = mfma_i8_32x32x32(a1, qb[kk], acc1);
    }
}

template <int PV, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void sage_fwd_kernel(SageFwdArgs a) {
    constexpr int V_ROW = PV == PV_F16 ? BN * 2 : BN;          // bytes per V^T row in LDS
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][BN * D];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][D * V_ROW];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
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

    // ---- this lane's query codes: B operand, Q[qrow][16h + 32kk .. +16)
    v4i qb[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        qb[kk] = row_ok ? *(const v4i*)(a.qc + ((int64_t)bh * a.Nq + qrow) * D + 16 * h + 32 * kk) : v4i{};
    const float cq = row_ok ? a.qs[(int64_t)bh * (a.Nq / a.q_blk) + qrow / a.q_blk] * a.c_log2 : 0.0f;

    const int last_row = min(q0 + BM, a.Nq) - 1;
    const int n_tiles = CAUSAL ? min(a.Nk / BN, (last_row + off) / BN + 1) : a.Nk / BN;
    const int wave_row0 = q0 + 32 * w;

    // ---- staging: global -> registers -> LDS
    const int8_t* kbase = a.kc + (int64_t)bhk * a.Nk * D;
    constexpr int K_CHUNKS = BN * D / 16;                 // 16-byte chunks per K tile
    constexpr int KPT = K_CHUNKS / 256;                    // per thread (1 or 2)
    constexpr int V_CHUNKS = D * V_ROW / 16;
    constexpr int VPT = V_CHUNKS / 256;
    uint4 kreg[KPT], vreg[VPT];

    auto gload = [&](int j) {
        const int t0 = j * BN;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int g = tid + 256 * u, r = g / (D / 16), c = g % (D / 16);
            kreg[u] = *(const uint4*)(kbase + (int64_t)(t0 + r) * D + 16 * c);
        }
        if constexpr (PV == PV_F16) {
            const uint16_t* vb = (const uint16_t*)a.v16.p + b * a.v16.sB + hk * a.v16.sH;
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int g = tid + 256 * u, key = g / (D / 8), c8 = (g % (D / 8)) * 8;
                vreg[u] = *(const uint4*)(vb + (int64_t)(t0 + key) * a.v16.sN + c8);
            }
        } else {
            const uint8_t* vb = a.vc + (int64_t)bhk * D * a.Nk + t0;
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int g = tid + 256 * u, r = g / 4, q = g % 4;
                vreg[u] = *(const uint4*)(vb + (int64_t)r * a.Nk + 16 * q);
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int g = tid + 256 * u, r = g / (D / 16), c = g % (D / 16);
            *(uint4*)(&k_lds[buf][swz<D>(r, c)]) = kreg[u];
        }
        if constexpr (PV == PV_F16) {
            // transpose fp16 V into V^T [channel][key]
            uint16_t* vt = (uint16_t*)v_lds[buf];
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int g = tid + 256 * u, key = g / (D / 8), c8 = (g % (D / 8)) * 8;
                const uint16_t* e = (const uint16_t*)&vreg[u];
#pragma unroll
                for (int k = 0; k < 8; ++k) vt[(c8 + k) * BN + key] = e[k];
            }
        } else {
            // even dwords of a 64-key row first, odd dwords second (see the B
            // operand layout of the probabilities), then the 16-byte swizzle
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int g = tid + 256 * u, r = g / 4, q = g % 4;
                const uint32_t* dw = (const uint32_t*)&vreg[u];
                const int lo = 8 * q, hi = 32 + 8 * q;
                *(uint2*)(&v_lds[buf][swz<BN>(r, lo / 16) + lo % 16]) = make_uint2(dw[0], dw[2]);
                *(uint2*)(&v_lds[buf][swz<BN>(r, hi / 16) + hi % 16]) = make_uint2(dw[1], dw[3]);
            }
        }
    };

    // ---- running state: O^T accumulator (lane: query lq, channels 32cb + 8(i/4) + 4h + i%4)
    v16f oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = v16f{};
    float m_run = -__builtin_inff();
    float l_run = 0.0f;                                   // this lane-half's share of the row sum
    const float pbias = PV == PV_F8 ? 8.807354922057604f : 0.0f;     // log2(448): P scaled by 448

    if (n_tiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int buf = j & 1;
        if (j + 1 < n_tiles) gload(j + 1);
        const int t0 = j * BN;
        // wavefront-uniform: does any of this wave's rows see any key of this tile?
        const bool wave_live = !CAUSAL || (t0 <= wave_row0 + 31 + off);
        if (wave_live) {
            v16i s0, s1;
            qk_tile<D>(k_lds[buf], qb, lq, h, s0, s1);
            const bool diag = CAUSAL && (t0 + BN - 1 > wave_row0 + off);
            const int lim = qrow + off - t0;               // keys with tile index <= lim are visible
            int mx = INT32_MIN;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k0 = 8 * (i / 4) + 4 * h + (i % 4);
                if (diag) {
                    if (k0 > lim) s0[i] = INT32_MIN;
                    if (k0 + 32 > lim) s1[i] = INT32_MIN;
                }
                mx = max(mx, max(s0[i], s1[i]));
            }
            mx = max(mx, partner32(mx));
            const float c = cq * a.ks[(int64_t)bhk * (a.Nk / BN) + j];
            const float tmax = mx == INT32_MIN ? -__builtin_inff() : (float)mx * c;
            const float m_new = __builtin_fmaxf(m_run, tmax);
            const float alpha = m_run == m_new ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            const float bias = pbias - m_new;
            float p0[16], p1[16];
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p0[i] = s0[i] == INT32_MIN ? 0.0f : __builtin_amdgcn_exp2f(__builtin_fmaf((float)s0[i], c, bias));
                p1[i] = s1[i] == INT32_MIN ? 0.0f : __builtin_amdgcn_exp2f(__builtin_fmaf((float)s1[i], c, bias));
                psum += p0[i] + p1[i];
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
            }
            if constexpr (PV == PV_F8) {
                v8i pb;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(p0[4 * k], p0[4 * k + 1], 0, false);
                    pb[k] = __builtin_amdgcn_cvt_pk_fp8_f32(p0[4 * k + 2], p0[4 * k + 3], w0, true);
                    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(p1[4 * k], p1[4 * k + 1], 0, false);
                    pb[4 + k] = __builtin_amdgcn_cvt_pk_fp8_f32(p1[4 * k + 2], p1[4 * k + 3], w1, true);
                }
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb) {
                    const uint8_t* vrow = v_lds[buf];
                    const int r = 32 * cb + lq;
                    v4i lo = *(const v4i*)(vrow + swz<BN>(r, 2 * h));
                    v4i hi = *(const v4i*)(vrow + swz<BN>(r, 2 * h + 1));
                    v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    oacc[cb] = mfma_f8_32x32x64(av, pb, oacc[cb]);
                }
            } else if constexpr (PV == PV_I8) {
                // int8 P per (row, tile): r = the row's largest P in the tile
                const float r = mx == INT32_MIN ? 0.0f : __builtin_amdgcn_exp2f(__builtin_fmaf((float)mx, c, bias));
                float inv = r > 0.0f ? 127.0f / r : 0.0f;
                if (__builtin_isinf(inv)) inv = 0.0f;
                const float rs = r * (1.0f / 127.0f);
                v4i pb0, pb1;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t w0 = 0, w1 = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w0 |= (uint32_t)enc_i8(p0[4 * k + e], inv) << (8 * e);
                        w1 |= (uint32_t)enc_i8(p1[4 * k + e], inv) << (8 * e);
                    }
                    pb0[k] = (int)w0;
                    pb1[k] = (int)w1;
                }
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb) {
                    const uint8_t* vrow = v_lds[buf];
                    const int rr = 32 * cb + lq;
                    v4i v0 = *(const v4i*)(vrow + swz<BN>(rr, 2 * h));
                    v4i v1 = *(const v4i*)(vrow + swz<BN>(rr, 2 * h + 1));
                    v16i pv = mfma_i8_32x32x32(v0, pb0, v16i{});
                    pv = mfma_i8_32x32x32(v1, pb1, pv);
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[cb][i] = __builtin_fmaf((float)pv[i], rs, oacc[cb][i]);
                }
            } else {
                // fp16 P; the 64 keys go through four 16-deep steps
                const uint16_t* vt = (const uint16_t*)v_lds[buf];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    v8h pb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pb[e] = (_Float16)((s < 2 ? p0 : p1)[8 * (s % 2) + e]);
#pragma unroll
                    for (int cb = 0; cb < D / 32; ++cb) {
                        const int ch = 32 * cb + lq;
                        const uint16_t* row = vt + ch * BN + 16 * s + 4 * h;
                        uint2 x0 = *(const uint2*)row;
                        uint2 x1 = *(const uint2*)(row + 8);
                        v8h av = __builtin_bit_cast(v8h, make_uint4(x0.x, x0.y, x1.x, x1.y));
                        oacc[cb] = mfma_f16_32x32x16(av, pb, oacc[cb]);
                    }
                }
            }
        }
        if (j + 1 < n_tiles) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    const float l_tot = l_run + partner32f(l_run);
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
                float v = oacc[cb][4 * g + e] * inv_l;
                if constexpr (PV != PV_F16) v *= a.vs[(int64_t)bhk * D + ch0 + e];
                out[e] = PV == PV_F16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
            }
            *(uint2*)(orow + ch0) = make_uint2((uint32_t)out[0] | ((uint32_t)out[1] << 16),
                                               (uint32_t)out[2] | ((uint32_t)out[3] << 16));
        }
    }
    if (a.lse && h == 0) {
        // natural-log LSE; with P scaled by 448 the sum carries that factor
        const float ln2 = 0.6931471805599453f;
        float lse = m_run * ln2 + __logf(l_tot);
        if (PV == PV_F8) lse -= 6.104793232414985f;   // ln(448)
        a.lse[(int64_t)bh * a.Nq + qrow] = lse;
    }
}

// Raw int32 S tile (32 queries x 32 keys) through the same tile code.
template <int D>
__global__ __launch_bounds__(64) void debug_scores_i8_kernel(const int8_t* qc, const int8_t* kc, int32_t* out) {
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[BN * D];
    const int l = threadIdx.x, h = l >> 5, lq = l & 31;
    for (int g = l; g < 32 * D / 16; g += 64) {
        const int r = g / (D / 16), c = g % (D / 16);
        *(uint4*)(&k_lds[swz<D>(r, c)]) = *(const uint4*)(kc + (int64_t)r * D + 16 * c);
    }
    for (int g = l; g < 32 * D / 16; g += 64) {            // rows 32..63: zero
        const int r = 32 + g / (D / 16), c = g % (D / 16);
        *(uint4*)(&k_lds[swz<D>(r, c)]) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    v4i qb[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qb[kk] = *(const v4i*)(qc + (int64_t)lq * D + 16 * h + 32 * kk);
    v16i s0, s1;
    qk_tile<D>(k_lds, qb, lq, h, s0, s1);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[lq * 32 + 8 * (i / 4) + 4 * h + (i % 4)] = s0[i];
}

template <int PV, int D>
hipError_t launch_t(const SageFwdArgs& a, hipStream_t st) {
    const int grid = a.B * a.Hq * ((a.Nq + BM - 1) / BM);
    if (a.causal) sage_fwd_kernel<PV, D, true><<<grid, 256, 0, st>>>(a);
    else sage_fwd_kernel<PV, D, false><<<grid, 256, 0, st>>>(a);
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
