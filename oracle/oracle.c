/*
 * oracle.c — plain, slow CPU oracle for block-quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg are its only users.  It shares no code with the GPU
 * library.
 *
 * Sources (cited by page title and section):
 *  [SB]  "SageBwd: A Trainable Low-bit Attention" — Methodology items 1, 2
 *        and 4 (INT8 engine, INT8 backward with the softmax gradient kept in
 *        higher precision, QK-norm, K-smoothing with a small constant),
 *        Results (epsilon about 1e-3), Limitations (softmax gradient stays
 *        FP16/FP32).
 *  [AQ]  "Attn-QAT: 4-Bit Attention With Quantization-Aware Training" —
 *        technical summary §1 (FP4 has 15 values), §2 Principle 1 (the
 *        backward recomputes P at the forward's FP4 precision with fake
 *        quantisation), §2 Principle 2 (a high-precision auxiliary output O'
 *        used only for the dO.O' row term), §2 Implementation (FP4 GEMMs
 *        with no smoothing or two-level quantisation at inference).
 *  [TA]  "ThriftAttention" technical summary — Method step 1 (block means,
 *        importance q̄_i·k̄_j, top-k pairs), step 2 (selected pairs in
 *        16-bit, the rest in microscaled FP4 with two-level quantisation of
 *        the probability block, merged by FlashAttention-2 online softmax),
 *        the kernel paragraph (FP4 blocks first, then the 16-bit helper).
 *
 * Where the pages are silent the plainest reading is taken; each reading is
 * listed in the design notes.  Floating-point work is fp64 except at the
 * rounding points the kernels have (fp32 scale arithmetic, the storage
 * formats), which are reproduced exactly.  Build with -ffp-contract=off and
 * without fast-math.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ========================================================================
 * Scalar formats
 * ====================================================================== */

/* Round x to the value grid of a binary floating format with `mant_bits`
 * stored mantissa bits and minimum normal exponent `emin` (gradual underflow
 * below it).  Ties go to the even grid point.  Magnitudes above `maxval`
 * saturate to it, or become infinity when saturate == 0. */
double orc_round_grid(double x, int mant_bits, int emin, double maxval, int saturate) {
    if (x != x || x == 0.0) return x;
    double a = fabs(x);
    int E;
    frexp(a, &E);                     /* a = f * 2^E with f in [0.5, 1) */
    int e = E - 1;                    /* exponent of the leading bit */
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - mant_bits);
    double r = nearbyint(a / quantum) * quantum;   /* default mode: nearest-even */
    if (r > maxval) r = saturate ? maxval : INFINITY;
    return copysign(r, x);
}

/* Bits of a value that already lies on the grid of the format. */
static unsigned grid_bits(double v, int mant_bits, int exp_bits, int bias) {
    unsigned sign = signbit(v) ? 1u : 0u;
    double a = fabs(v);
    unsigned mag = 0;
    int emin = 1 - bias;
    if (isinf(a)) {
        mag = ((1u << exp_bits) - 1u) << mant_bits;
    } else if (a != 0.0) {
        int E;
        frexp(a, &E);
        int e = E - 1;
        if (e < emin) {
            mag = (unsigned)(a / ldexp(1.0, emin - mant_bits));        /* subnormal */
        } else {
            unsigned m = (unsigned)((a / ldexp(1.0, e) - 1.0) * (double)(1u << mant_bits));
            mag = ((unsigned)(e + bias) << mant_bits) | m;
        }
    }
    return (sign << (mant_bits + exp_bits)) | mag;
}

static double bits_value(unsigned c, int mant_bits, int exp_bits, int bias) {
    unsigned sign = (c >> (mant_bits + exp_bits)) & 1u;
    unsigned ef = (c >> mant_bits) & ((1u << exp_bits) - 1u);
    unsigned m = c & ((1u << mant_bits) - 1u);
    double v = ef == 0 ? ldexp((double)m, 1 - bias - mant_bits)
                       : ldexp(1.0 + (double)m / (double)(1u << mant_bits), (int)ef - bias);
    return sign ? -v : v;
}

/* OCP FP8 E4M3 ("fn"): bias 7, largest finite 448, no infinities, S.1111.111
 * is NaN.  Encoding rounds to nearest-even and saturates to +-448. */
uint8_t orc_e4m3_encode(double x) {
    if (x != x) return 0x7F;
    return (uint8_t)grid_bits(orc_round_grid(x, 3, -6, 448.0, 1), 3, 4, 7);
}
double orc_e4m3_decode(uint8_t c) {
    if ((c & 0x7F) == 0x7F) return NAN;
    return bits_value(c, 3, 4, 7);
}

/* OCP FP4 E2M1: bias 1, values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; the two zeros
 * make 15 distinct values ([AQ] §1).  Nearest-even, saturating to +-6. */
uint8_t orc_e2m1_encode(double x) {
    if (x != x) return 0x7;
    return (uint8_t)grid_bits(orc_round_grid(x, 1, 0, 6.0, 1), 1, 2, 1);
}
double orc_e2m1_decode(uint8_t c) { return bits_value(c & 0xF, 1, 2, 1); }

/* OCP MX shared scale: X = 2^e with e = floor(log2(amax)) - 2 (2 is the
 * exponent of e2m1's largest normal), clamped to the E8M0 range; amax == 0
 * gives the smallest scale.  frexp is exact on any float. */
int orc_e8m0_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    int E;
    frexp((double)amax, &E);
    int e = (E - 1) - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

uint16_t orc_bf16_bits(double x) {
    return (uint16_t)grid_bits(orc_round_grid(x, 7, -126, 0x1.FEp127, 0), 7, 8, 127);
}
uint16_t orc_f16_bits(double x) {
    return (uint16_t)grid_bits(orc_round_grid(x, 10, -14, 65504.0, 0), 10, 5, 15);
}
double orc_bf16_value(double x) { return orc_round_grid(x, 7, -126, 0x1.FEp127, 0); }
double orc_f16_value(double x) { return orc_round_grid(x, 10, -14, 65504.0, 0); }

/* Round n values to bf16 (fmt 0) or fp16 (fmt 1), nearest-even, as values. */
void orc_round_array(const double* x, int64_t n, int fmt, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = fmt == 0 ? orc_bf16_value(x[i]) : orc_f16_value(x[i]);
}

/* Symmetric INT8 with a per-block absmax scale: scale = amax/127 and
 * inv = 127/amax, both correctly-rounded fp32 divisions; the code is the
 * nearest-even integer of the fp32 product x*inv, clamped to [-127, 127].
 * amax == 0 gives scale 0 and all-zero codes. */
void orc_i8_scale(float amax, float* scale, float* inv) {
    float i = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (!(amax > 0.0f) || isinf(i)) { *scale = 0.0f; *inv = 0.0f; return; }
    *scale = amax / 127.0f;
    *inv = i;
}
int8_t orc_i8_encode(float x, float inv) {
    float p = x * inv;
    float r = rintf(p);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

/* ========================================================================
 * Quantisers
 * ====================================================================== */

/* Error-free transformation of a + b (Knuth's TwoSum). */
static double two_sum(double a, double b, double* err) {
    double s = a + b;
    double bb = s - a;
    *err = (a - (s - bb)) + (b - bb);
    return s;
}

/* K-smoothing ([SB] Methodology 4, Results): subtract the token-mean of every
 * key channel and add the small constant back, K_s = K - (mean - eps).  The
 * channel sum is accumulated in fp64; TwoSum certifies that every addition
 * was exact (then the sum does not depend on the order), and the number of
 * channels whose sum was not certified is returned.  mu_eff = fp32(S/N - eps). */
int orc_smooth_mean(const float* K, int BH, int N, int d, double eps, float* mu_eff) {
    int inexact = 0;
    for (int bh = 0; bh < BH; ++bh) {
        const float* k = K + (size_t)bh * N * d;
        for (int c = 0; c < d; ++c) {
            double s = 0.0, err;
            int bad = 0;
            for (int t = 0; t < N; ++t) {
                s = two_sum(s, (double)k[(size_t)t * d + c], &err);
                if (err != 0.0) bad = 1;
            }
            inexact += bad;
            mu_eff[(size_t)bh * d + c] = (float)(s / (double)N - eps);
        }
    }
    return inexact;
}

/* INT8 per token block ([SB] Methodology 1; per-block scales): one absmax
 * scale per `blk` consecutive tokens of a head.  With mu != NULL the rows are
 * first smoothed, x_s = fp32(x - mu[c]). */
void orc_quant_i8_tokblock(const float* X, const float* mu, int BH, int N, int d, int blk,
                           int8_t* codes, float* scales) {
    int nb = N / blk;
    for (int bh = 0; bh < BH; ++bh) {
        for (int b = 0; b < nb; ++b) {
            const float* x = X + ((size_t)bh * N + (size_t)b * blk) * d;
            const float* m = mu ? mu + (size_t)bh * d : NULL;
            float amax = 0.0f;
            for (int t = 0; t < blk; ++t)
                for (int c = 0; c < d; ++c) {
                    float v = m ? x[(size_t)t * d + c] - m[c] : x[(size_t)t * d + c];
                    float a = fabsf(v);
                    if (a > amax) amax = a;
                }
            float scale, inv;
            orc_i8_scale(amax, &scale, &inv);
            scales[(size_t)bh * nb + b] = scale;
            int8_t* o = codes + ((size_t)bh * N + (size_t)b * blk) * d;
            for (int t = 0; t < blk; ++t)
                for (int c = 0; c < d; ++c) {
                    float v = m ? x[(size_t)t * d + c] - m[c] : x[(size_t)t * d + c];
                    o[(size_t)t * d + c] = orc_i8_encode(v, inv);
                }
        }
    }
}

/* Per-channel V (fmt 0: INT8, fmt 1: FP8 E4M3).  One scale per channel over
 * all N tokens; codes are written channel-major, codes_t[bh][c][t]. */
void orc_quant_chan(const float* V, int BH, int N, int d, int fmt, uint8_t* codes_t, float* scales) {
    for (int bh = 0; bh < BH; ++bh) {
        const float* v = V + (size_t)bh * N * d;
        for (int c = 0; c < d; ++c) {
            float amax = 0.0f;
            for (int t = 0; t < N; ++t) {
                float a = fabsf(v[(size_t)t * d + c]);
                if (a > amax) amax = a;
            }
            float scale, inv;
            uint8_t* o = codes_t + ((size_t)bh * d + c) * N;
            if (fmt == 0) {
                orc_i8_scale(amax, &scale, &inv);
                for (int t = 0; t < N; ++t) o[t] = (uint8_t)orc_i8_encode(v[(size_t)t * d + c], inv);
            } else {
                inv = amax > 0.0f ? 448.0f / amax : 0.0f;
                scale = amax / 448.0f;
                if (!(amax > 0.0f) || isinf(inv)) { scale = 0.0f; inv = 0.0f; }
                for (int t = 0; t < N; ++t) {
                    float p = v[(size_t)t * d + c] * inv;
                    o[t] = orc_e4m3_encode((double)p);
                }
            }
            scales[(size_t)bh * d + c] = scale;
        }
    }
}

/* One MX block: 32 values sharing X = 2^e; element codes e2m1(x / X). */
static void mx_block(const float* x, int stride, uint8_t* codes /* 32 nibbles, one per byte */, uint8_t* e_biased) {
    float amax = 0.0f;
    for (int k = 0; k < 32; ++k) {
        float a = fabsf(x[(size_t)k * stride]);
        if (a > amax) amax = a;
    }
    int e = orc_e8m0_exponent(amax);
    *e_biased = (uint8_t)(e + 127);
    for (int k = 0; k < 32; ++k)
        codes[k] = orc_e2m1_encode(ldexp((double)x[(size_t)k * stride], -e));
}

/* MXFP4 along d (Q and K): codes[bh][t][c/2] (even c in the low nibble),
 * scales[bh][t][c/32] holding e + 127. */
void orc_quant_mx_rows(const float* X, int BH, int N, int d, uint8_t* codes, uint8_t* scales) {
    uint8_t nib[32];
    for (size_t r = 0; r < (size_t)BH * N; ++r) {
        for (int b = 0; b < d / 32; ++b) {
            mx_block(X + r * d + b * 32, 1, nib, &scales[r * (d / 32) + b]);
            for (int k = 0; k < 32; k += 2)
                codes[r * (d / 2) + (b * 32 + k) / 2] = (uint8_t)(nib[k] | (nib[k + 1] << 4));
        }
    }
}

/* MXFP4 along tokens (V): one scale per (channel, 32 tokens); codes are
 * channel-major, codes_t[bh][c][t/2], scales_t[bh][c][t/32]. */
void orc_quant_mx_cols(const float* X, int BH, int N, int d, uint8_t* codes_t, uint8_t* scales_t) {
    uint8_t nib[32];
    for (int bh = 0; bh < BH; ++bh)
        for (int c = 0; c < d; ++c)
            for (int b = 0; b < N / 32; ++b) {
                const float* x = X + ((size_t)bh * N + (size_t)b * 32) * d + c;
                mx_block(x, d, nib, &scales_t[((size_t)bh * d + c) * (N / 32) + b]);
                for (int k = 0; k < 32; k += 2)
                    codes_t[((size_t)bh * d + c) * (N / 2) + (b * 32 + k) / 2] =
                        (uint8_t)(nib[k] | (nib[k + 1] << 4));
            }
}

/* Block means ([TA] Method step 1): the mean of the `blk` token vectors of
 * each block, summed in fp64 and rounded once to fp32. */
void orc_block_means(const float* X, int BH, int N, int d, int blk, float* means) {
    for (int bh = 0; bh < BH; ++bh)
        for (int b = 0; b < N / blk; ++b)
            for (int c = 0; c < d; ++c) {
                double s = 0.0;
                for (int t = 0; t < blk; ++t) s += (double)X[((size_t)bh * N + (size_t)b * blk + t) * d + c];
                means[((size_t)bh * (N / blk) + b) * d + c] = (float)(s / (double)blk);
            }
}

/* ========================================================================
 * Textbook attention, fp64, two-pass softmax (no tiling, no quantisation)
 * ====================================================================== */

static int last_key(int i, int Nq, int Nk, int causal) {
    return causal ? i + (Nk - Nq) : Nk - 1;        /* bottom-right aligned mask */
}

void orc_ref_fwd(const float* Q, const float* K, const float* V, int Nq, int Nk, int d,
                 int causal, double tau, double* O, double* lse) {
#pragma omp parallel for schedule(dynamic)
    for (int i = 0; i < Nq; ++i) {
        int last = last_key(i, Nq, Nk, causal);
        double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
        double m = -INFINITY;
        for (int j = 0; j <= last; ++j) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += (double)Q[(size_t)i * d + c] * (double)K[(size_t)j * d + c];
            s[j] = tau * acc;
            if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (int j = 0; j <= last; ++j) { s[j] = exp(s[j] - m); l += s[j]; }
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j <= last; ++j) acc += s[j] * (double)V[(size_t)j * d + c];
            O[(size_t)i * d + c] = acc / l;
        }
        lse[i] = m + log(l);
        free(s);
    }
}

/* Gradients of O = softmax(tau Q K^T) V with respect to Q, K, V (FlashAttention
 * notation): dV = P^T dO, dP = dO V^T, dS = P o (dP - rowsum(P o dP)),
 * dQ = tau dS K, dK = tau dS^T Q. */
void orc_ref_bwd(const float* Q, const float* K, const float* V, const float* dO,
                 int Nq, int Nk, int d, int causal, double tau,
                 double* dQ, double* dK, double* dV) {
    double* P = (double*)calloc((size_t)Nq * Nk, sizeof(double));
    double* dS = (double*)calloc((size_t)Nq * Nk, sizeof(double));
    for (int i = 0; i < Nq; ++i) {
        int last = last_key(i, Nq, Nk, causal);
        double m = -INFINITY, l = 0.0;
        for (int j = 0; j <= last; ++j) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += (double)Q[(size_t)i * d + c] * (double)K[(size_t)j * d + c];
            P[(size_t)i * Nk + j] = tau * acc;
            if (tau * acc > m) m = tau * acc;
        }
        for (int j = 0; j <= last; ++j) { P[(size_t)i * Nk + j] = exp(P[(size_t)i * Nk + j] - m); l += P[(size_t)i * Nk + j]; }
        for (int j = 0; j <= last; ++j) P[(size_t)i * Nk + j] /= l;
        double rowdot = 0.0;
        for (int j = 0; j <= last; ++j) {
            double dp = 0.0;
            for (int c = 0; c < d; ++c) dp += (double)dO[(size_t)i * d + c] * (double)V[(size_t)j * d + c];
            dS[(size_t)i * Nk + j] = dp;
            rowdot += P[(size_t)i * Nk + j] * dp;
        }
        for (int j = 0; j <= last; ++j)
            dS[(size_t)i * Nk + j] = P[(size_t)i * Nk + j] * (dS[(size_t)i * Nk + j] - rowdot);
    }
    for (int i = 0; i < Nq; ++i)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < Nk; ++j) acc += dS[(size_t)i * Nk + j] * (double)K[(size_t)j * d + c];
            dQ[(size_t)i * d + c] = tau * acc;
        }
    for (int j = 0; j < Nk; ++j)
        for (int c = 0; c < d; ++c) {
            double ak = 0.0, av = 0.0;
            for (int i = 0; i < Nq; ++i) {
                ak += dS[(size_t)i * Nk + j] * (double)Q[(size_t)i * d + c];
                av += P[(size_t)i * Nk + j] * (double)dO[(size_t)i * d + c];
            }
            dK[(size_t)j * d + c] = tau * ak;
            dV[(size_t)j * d + c] = av;
        }
    free(P);
    free(dS);
}

/* ========================================================================
 * Online-softmax row state (FlashAttention-2 style merge, [TA] step 2)
 * ====================================================================== */

typedef struct {
    double m, l;
    double* acc;     /* d values: running sum of dequantised P times V */
    double* acc2;    /* d values: second output (Attn-QAT O'), may be NULL */
} row_state;

/* FlashAttention-2's merge step ([TA] step 2): the running maximum becomes
 * m_new = max(m, tile max), and the sums gathered so far are scaled by
 * exp(m - m_new) so that every later P = exp(s - m_new) joins them in the
 * same frame.  The largest P of the row so far is therefore exactly 1. */
static void row_update_max(row_state* st, double tile_max, int d) {
    double m_new = st->m > tile_max ? st->m : tile_max;
    if (m_new == st->m) return;
    double alpha = (st->m == -INFINITY) ? 0.0 : exp(st->m - m_new);
    st->l *= alpha;
    for (int c = 0; c < d; ++c) st->acc[c] *= alpha;
    if (st->acc2) for (int c = 0; c < d; ++c) st->acc2[c] *= alpha;
    st->m = m_new;
}

/* ========================================================================
 * SageAttention INT8 forward ([SB] Methodology 1, 4)
 * ====================================================================== */

static double sage_score(int qk_mode, const int8_t* qc, const float* qs, int q_blk,
                         const int8_t* kc, const float* ks, int k_blk,
                         const float* Qf, const float* Kf, int d, int i, int j, double tau) {
    if (qk_mode == ORC_QK_I8) {
        int64_t acc = 0;
        for (int c = 0; c < d; ++c) acc += (int64_t)qc[(size_t)i * d + c] * (int64_t)kc[(size_t)j * d + c];
        /* |acc| <= 127^2 d < 2^31: the int32 accumulator of the kernel is exact */
        return (double)acc * (double)qs[i / q_blk] * (double)ks[j / k_blk] * tau;
    }
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += (double)Qf[(size_t)i * d + c] * (double)Kf[(size_t)j * d + c];
    return acc * tau;
}

/* Rows [r0, r1) of one head.  Keys are visited in tiles of kv_tile in
 * ascending order (causal: up to the row's diagonal).  Per tile:
 * m_new = max(m, tile max) (FlashAttention-2's running maximum),
 * P = exp(s - m_new), l accumulates the unquantised P, and P is rounded for
 * the P.V product by pv_mode:
 *   ORC_PV_F16: fp16(P) times V given in fp16;
 *   ORC_PV_F8 : e4m3(448 P)/448 times e4m3 V codes times the channel scale;
 *   ORC_PV_I8 : int8 per (row, tile) with r = the row's tile max of P,
 *               code = rint(fp32(P * fp32(127/r))), value code*r/127,
 *               times int8 V codes times the channel scale;
 *   ORC_PV_NONE: P times V in fp64.
 * Output: O = acc / l (fp64, before the storage rounding), lse = m + ln l. */
void orc_sage_fwd(int qk_mode, const int8_t* qc, const float* qs, int q_blk,
                  const int8_t* kc, const float* ks, int k_blk,
                  const float* Qf, const float* Kf,
                  int pv_mode, const float* Vf, const uint8_t* vc_t, const float* vs,
                  int Nq, int Nk, int d, int causal, double tau, int kv_tile,
                  int r0, int r1, double* O, double* lse) {
#pragma omp parallel for schedule(dynamic)
    for (int i = r0; i < r1; ++i) {
        int last = last_key(i, Nq, Nk, causal);
        double* s = (double*)malloc(sizeof(double) * (size_t)kv_tile);
        double* p = (double*)malloc(sizeof(double) * (size_t)kv_tile);
        row_state st = {-INFINITY, 0.0, (double*)calloc((size_t)d, sizeof(double)), NULL};
        for (int t0 = 0; t0 <= last; t0 += kv_tile) {
            int n = kv_tile;
            if (t0 + n - 1 > last) n = last - t0 + 1;     /* keys past the diagonal are masked */
            double tmax = -INFINITY;
            for (int u = 0; u < n; ++u) {
                s[u] = sage_score(qk_mode, qc, qs, q_blk, kc, ks, k_blk, Qf, Kf, d, i, t0 + u, tau);
                if (s[u] > tmax) tmax = s[u];
            }
            row_update_max(&st, tmax, d);
            double r = 0.0;
            for (int u = 0; u < n; ++u) {
                p[u] = exp(s[u] - st.m);
                st.l += p[u];
                if (p[u] > r) r = p[u];
            }
            float inv_r = r > 0.0 ? (float)(127.0 / r) : 0.0f;
            if (isinf(inv_r)) inv_r = 0.0f;          /* degenerate tile: P rounds to zero */
            for (int u = 0; u < n; ++u) {
                int j = t0 + u;
                double pq;
                switch (pv_mode) {
                    case ORC_PV_F16: pq = orc_f16_value(p[u]); break;
                    case ORC_PV_F8: pq = orc_e4m3_decode(orc_e4m3_encode(448.0 * p[u])) / 448.0; break;
                    case ORC_PV_I8: pq = (double)rintf((float)(p[u] * (double)inv_r)) * r / 127.0; break;
                    default: pq = p[u];
                }
                for (int c = 0; c < d; ++c) {
                    double v;
                    switch (pv_mode) {
                        case ORC_PV_F8: v = orc_e4m3_decode(vc_t[(size_t)c * Nk + j]) * (double)vs[c]; break;
                        case ORC_PV_I8: v = (double)(int8_t)vc_t[(size_t)c * Nk + j] * (double)vs[c]; break;
                        default: v = (double)Vf[(size_t)j * d + c];
                    }
                    st.acc[c] += pq * v;
                }
            }
        }
        for (int c = 0; c < d; ++c) O[(size_t)(i - r0) * d + c] = st.acc[c] / st.l;
        lse[i - r0] = st.m + log(st.l);
        free(st.acc);
        free(s);
        free(p);
    }
}

/* ========================================================================
 * SageBwd INT8 backward ([SB] Methodology 2; Limitations)
 *
 * Of the five backward products, four are INT8 with one scale per operand
 * tile (P^T dO, dS K, dS^T Q and the recomputed Q K^T); dP = dO V^T stays in
 * 16-bit (fp64 here on the bf16 inputs), and dS = P o (dP - delta) is
 * formed in full precision before it is rounded to INT8 for dQ and dK.
 * delta = rowsum(dO o O) with the forward's stored O.
 * ====================================================================== */

typedef struct {
    const int8_t *qc, *kc;
    const float *qs, *ks, *V, *dO, *lse;
    const int8_t* doc;
    const float* dos;
    const double* delta;
    int N, d, causal, tq, tk, do_blk, quantize;
    double tau;
    const int8_t* vc;     /* fully INT8 backward: V codes per v_blk tokens; NULL: dP from bf16 V */
    const float* vs;
    int v_blk;
} sbwd_ctx;

/* Round a tile to INT8 with one scale (its absmax) and return the
 * dequantised values in place. */
static void tile_i8_fake(double* x, int n) {
    double a = 0.0;
    for (int u = 0; u < n; ++u) if (fabs(x[u]) > a) a = fabs(x[u]);
    float inv = a > 0.0 ? (float)(127.0 / a) : 0.0f;
    if (inv == 0.0f || isinf(inv)) { for (int u = 0; u < n; ++u) x[u] = 0.0; return; }
    for (int u = 0; u < n; ++u) {
        float r = rintf((float)(x[u] * (double)inv));
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        x[u] = (double)r * a / 127.0;
    }
}

static void sbwd_tile(const sbwd_ctx* c, int I, int J, double* dQ /* tile rows, or NULL */,
                      double* dK, double* dV /* tile keys, or NULL */) {
    int tq = c->tq, tk = c->tk, d = c->d;
    double* P = (double*)calloc((size_t)tq * tk, sizeof(double));
    double* dS = (double*)calloc((size_t)tq * tk, sizeof(double));
    double* Pq = (double*)calloc((size_t)tq * tk, sizeof(double));
    for (int a = 0; a < tq; ++a) {
        int i = I * tq + a;
        for (int b = 0; b < tk; ++b) {
            int j = J * tk + b;
            if (c->causal && j > i) continue;
            double s;
            int64_t acc = 0;
            for (int k = 0; k < d; ++k) acc += (int64_t)c->qc[(size_t)i * d + k] * (int64_t)c->kc[(size_t)j * d + k];
            s = (double)acc * (double)c->qs[i / tq] * (double)c->ks[j / tk] * c->tau;
            P[(size_t)a * tk + b] = exp(s - (double)c->lse[i]);
            double dp = 0.0;
            if (c->vc) {
                /* dP in INT8: the dO codes (per do_blk tokens) against the V
                 * codes (per v_blk tokens), exact integer sum, then both scales */
                int64_t di = 0;
                for (int k = 0; k < d; ++k)
                    di += (int64_t)c->doc[(size_t)i * d + k] * (int64_t)c->vc[(size_t)j * d + k];
                dp = (double)di * (double)c->dos[i / c->do_blk] * (double)c->vs[j / c->v_blk];
            } else {
                for (int k = 0; k < d; ++k) dp += (double)c->dO[(size_t)i * d + k] * (double)c->V[(size_t)j * d + k];
            }
            dS[(size_t)a * tk + b] = P[(size_t)a * tk + b] * (dp - c->delta[i]);
        }
    }
    memcpy(Pq, P, sizeof(double) * (size_t)tq * tk);
    if (c->quantize) { tile_i8_fake(Pq, tq * tk); tile_i8_fake(dS, tq * tk); }
    if (dV) {
        for (int b = 0; b < tk; ++b)
            for (int k = 0; k < d; ++k) {
                double acc = 0.0;
                for (int a = 0; a < tq; ++a) {
                    int i = I * tq + a;
                    double g = c->quantize ? (double)c->doc[(size_t)i * d + k] * (double)c->dos[i / c->do_blk]
                                           : (double)c->dO[(size_t)i * d + k];
                    acc += Pq[(size_t)a * tk + b] * g;
                }
                dV[(size_t)b * d + k] += acc;
            }
    }
    if (dK) {
        for (int b = 0; b < tk; ++b)
            for (int k = 0; k < d; ++k) {
                double acc = 0.0;
                for (int a = 0; a < tq; ++a) {
                    int i = I * tq + a;
                    acc += dS[(size_t)a * tk + b] * (double)c->qc[(size_t)i * d + k] * (double)c->qs[i / tq];
                }
                dK[(size_t)b * d + k] += c->tau * acc;
            }
    }
    if (dQ) {
        for (int a = 0; a < tq; ++a)
            for (int k = 0; k < d; ++k) {
                double acc = 0.0;
                for (int b = 0; b < tk; ++b) {
                    int j = J * tk + b;
                    acc += dS[(size_t)a * tk + b] * (double)c->kc[(size_t)j * d + k] * (double)c->ks[j / tk];
                }
                dQ[(size_t)a * d + k] += c->tau * acc;
            }
    }
    free(P);
    free(dS);
    free(Pq);
}

/* dQ for query tiles [qt0, qt1) and dK, dV for key tiles [kt0, kt1) of one
 * head (outputs hold only those rows).  Q codes are per 128-token block and
 * K codes per 64-token block (the forward's), dO is quantised here per
 * do_blk tokens.  With quantize == 0 every rounding is skipped (the codes
 * times their scales are then the operands).  With vc != NULL the fully
 * INT8 variant that [SB] Limitations leaves open: dP = dO V^T from the INT8
 * codes of dO and of V (vc, vs: V per v_blk tokens). */
void orc_sage_bwd_v(const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                    const float* V, const float* dO, const float* O, const float* lse,
                    int N, int d, int causal, double tau, int tile_q, int tile_k, int do_blk,
                    int quantize, int qt0, int qt1, int kt0, int kt1,
                    const int8_t* vc, const float* vs, int v_blk,
                    double* dQ, double* dK, double* dV) {
    double* delta = (double*)malloc(sizeof(double) * (size_t)N);
    for (int i = 0; i < N; ++i) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += (double)dO[(size_t)i * d + k] * (double)O[(size_t)i * d + k];
        delta[i] = acc;
    }
    int8_t* doc = (int8_t*)malloc((size_t)N * d);
    float* dos = (float*)malloc(sizeof(float) * (size_t)(N / do_blk));
    orc_quant_i8_tokblock(dO, NULL, 1, N, d, do_blk, doc, dos);
    sbwd_ctx c = {qc, kc, qs, ks, V, dO, lse, doc, dos, delta, N, d, causal, tile_q, tile_k, do_blk, quantize, tau,
                  vc, vs, v_blk};
    memset(dQ, 0, sizeof(double) * (size_t)(qt1 - qt0) * tile_q * d);
    memset(dK, 0, sizeof(double) * (size_t)(kt1 - kt0) * tile_k * d);
    memset(dV, 0, sizeof(double) * (size_t)(kt1 - kt0) * tile_k * d);
    int nkt = N / tile_k, nqt = N / tile_q;
#pragma omp parallel for schedule(dynamic)
    for (int I = qt0; I < qt1; ++I)
        for (int J = 0; J < nkt; ++J) {
            if (causal && J * tile_k > I * tile_q + tile_q - 1) break;
            sbwd_tile(&c, I, J, dQ + (size_t)(I - qt0) * tile_q * d, NULL, NULL);
        }
#pragma omp parallel for schedule(dynamic)
    for (int J = kt0; J < kt1; ++J)
        for (int I = 0; I < nqt; ++I) {
            if (causal && J * tile_k > I * tile_q + tile_q - 1) continue;
            sbwd_tile(&c, I, J, NULL, dK + (size_t)(J - kt0) * tile_k * d, dV + (size_t)(J - kt0) * tile_k * d);
        }
    free(delta);
    free(doc);
    free(dos);
}

void orc_sage_bwd(const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                  const float* V, const float* dO, const float* O, const float* lse,
                  int N, int d, int causal, double tau, int tile_q, int tile_k, int do_blk,
                  int quantize, int qt0, int qt1, int kt0, int kt1,
                  double* dQ, double* dK, double* dV) {
    orc_sage_bwd_v(qc, qs, kc, ks, V, dO, O, lse, N, d, causal, tau, tile_q, tile_k, do_blk, quantize, qt0, qt1,
                   kt0, kt1, NULL, NULL, 0, dQ, dK, dV);
}

/* ========================================================================
 * Attn-QAT FP4 ([AQ] §1, §2)
 * ====================================================================== */

static double mx_value(const uint8_t* codes, const uint8_t* scales, size_t elem, size_t blk_index) {
    uint8_t byte = codes[elem / 2];
    uint8_t nib = (elem & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
    return ldexp(orc_e2m1_decode(nib), (int)scales[blk_index] - 127);
}

/* Exact MX dot product of row i of Q and row j of K: per 32-channel block the
 * e2m1 products are multiples of 1/4 and their sum is an exact integer count
 * of quarters; the blocks are then joined with their power-of-two scales.
 * Returns 1 when every fp64 addition was exact (the result is then the exact
 * rational value), 0 otherwise. */
int orc_mx_scores(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                  int d, int i, int j, double* s) {
    double total = 0.0, err;
    int exact = 1;
    for (int b = 0; b < d / 32; ++b) {
        int64_t quarters = 0;
        for (int k = 0; k < 32; ++k) {
            size_t eq = (size_t)i * d + b * 32 + k, ek = (size_t)j * d + b * 32 + k;
            uint8_t nq = (eq & 1) ? (qc[eq / 2] >> 4) : (qc[eq / 2] & 0xF);
            uint8_t nk = (ek & 1) ? (kc[ek / 2] >> 4) : (kc[ek / 2] & 0xF);
            quarters += (int64_t)llround(4.0 * orc_e2m1_decode(nq) * orc_e2m1_decode(nk));
        }
        int e = (int)qs[(size_t)i * (d / 32) + b] - 127 + (int)ks[(size_t)j * (d / 32) + b] - 127;
        total = two_sum(total, ldexp((double)quarters, e - 2), &err);
        if (err != 0.0) exact = 0;
    }
    *s = total;
    return exact;
}

/* Fake-quantise 32 probabilities to MXFP4 (P rounded to fp32 first, as the
 * kernel holds it) and return the dequantised values in place. */
static void mx_fake32(double* p, int n) {
    float pf[32];
    float amax = 0.0f;
    for (int k = 0; k < n; ++k) { pf[k] = (float)p[k]; if (fabsf(pf[k]) > amax) amax = fabsf(pf[k]); }
    int e = orc_e8m0_exponent(amax);
    for (int k = 0; k < n; ++k) p[k] = ldexp(orc_e2m1_decode(orc_e2m1_encode(ldexp((double)pf[k], -e))), e);
}

static double vmx(const uint8_t* vc_t, const uint8_t* vs_t, int Nk, int j, int c) {
    return mx_value(vc_t, vs_t, (size_t)c * Nk + j, (size_t)c * (Nk / 32) + j / 32);
}
static double kmx(const uint8_t* kc, const uint8_t* ks, int d, int j, int c) {
    return mx_value(kc, ks, (size_t)j * d + c, (size_t)j * (d / 32) + c / 32);
}

/* Attn-QAT forward, rows [r0, r1) of one head, non-causal: s = tau * exact
 * MX dot product; key tiles of kv_tile ascending with FlashAttention-2's
 * running maximum; P = exp(s - m) fake-quantised to MXFP4 per 32 keys of the
 * row (no smoothing, no two-level step, [AQ] §2 Implementation) for O, and
 * rounded to bf16 for O' ([AQ] §2 Principle 2), both against the FP4 V;
 * l sums the unquantised P.  quantize_p == 0 uses P itself in both products.
 * Outputs O, O', lse = m + ln l and, when rowmax != NULL, the row's final
 * running maximum m (= the largest tau * s of the row). */
void orc_qat_fwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                 const uint8_t* vc_t, const uint8_t* vs_t, int Nq, int Nk, int d,
                 double tau, int kv_tile, int quantize_p, int r0, int r1,
                 double* O, double* O_aux, double* lse, double* rowmax) {
    (void)Nq;
#pragma omp parallel for schedule(dynamic)
    for (int i = r0; i < r1; ++i) {
        double* s = (double*)malloc(sizeof(double) * (size_t)kv_tile);
        double* p = (double*)malloc(sizeof(double) * (size_t)kv_tile);
        double* pq = (double*)malloc(sizeof(double) * (size_t)kv_tile);
        row_state st = {-INFINITY, 0.0, (double*)calloc((size_t)d, sizeof(double)),
                        (double*)calloc((size_t)d, sizeof(double))};
        for (int t0 = 0; t0 < Nk; t0 += kv_tile) {
            double tmax = -INFINITY;
            for (int u = 0; u < kv_tile; ++u) {
                orc_mx_scores(qc, qs, kc, ks, d, i, t0 + u, &s[u]);
                s[u] *= tau;
                if (s[u] > tmax) tmax = s[u];
            }
            row_update_max(&st, tmax, d);
            for (int u = 0; u < kv_tile; ++u) { p[u] = exp(s[u] - st.m); st.l += p[u]; pq[u] = p[u]; }
            if (quantize_p) for (int u = 0; u < kv_tile; u += 32) mx_fake32(pq + u, 32);
            for (int u = 0; u < kv_tile; ++u) {
                double pb = quantize_p ? orc_bf16_value(p[u]) : p[u];
                for (int c = 0; c < d; ++c) {
                    double v = vmx(vc_t, vs_t, Nk, t0 + u, c);
                    st.acc[c] += pq[u] * v;
                    st.acc2[c] += pb * v;
                }
            }
        }
        for (int c = 0; c < d; ++c) {
            O[(size_t)(i - r0) * d + c] = st.acc[c] / st.l;
            O_aux[(size_t)(i - r0) * d + c] = st.acc2[c] / st.l;
        }
        lse[i - r0] = st.m + log(st.l);
        if (rowmax) rowmax[i - r0] = st.m;
        free(st.acc); free(st.acc2); free(s); free(p); free(pq);
    }
}

/* Attn-QAT backward ([AQ] §2 Principles 1 and 2): P = exp(s - L) recomputed
 * from the same exact MX scores.  For dV = P^ dO, P is fake-quantised at the
 * forward's precision: the forward made MXFP4 codes of exp(s - m) per 32
 * keys, with m the running maximum, so the backward rounds exp(s - M) per 32
 * keys, M = the row's final maximum (rowmax, from the forward; NULL: taken
 * here over every key), and scales the result by exp(M - L) = 1/l.  The row's
 * largest P is then exactly 1/l, as in the forward, and every tile that the
 * forward visited once its maximum had reached M gets the forward's own
 * codes.  dP = dO V^T against the FP4 V; dS = P o (dP - delta') with
 * delta' = rowsum(dO o O') (the straight-through estimator keeps the
 * unquantised P in the softmax Jacobian); dS is rounded to bf16 where the
 * products take bf16 operands; dQ = tau dS K, dK = tau dS^T Q with the FP4
 * Q, K.  Outputs: dQ rows [q0, q1), dK and dV rows [k0, k1) of one head.
 * quantize_p == 0 skips the P and dS roundings. */
void orc_qat_bwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                 const uint8_t* vc_t, const uint8_t* vs_t, const float* dO, const float* O_aux,
                 const float* lse, const double* rowmax, int Nq, int Nk, int d, double tau, int quantize_p,
                 int q0, int q1, int k0, int k1, double* dQ, double* dK, double* dV) {
    double* delta = (double*)malloc(sizeof(double) * (size_t)Nq);
    for (int i = 0; i < Nq; ++i) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)dO[(size_t)i * d + c] * (double)O_aux[(size_t)i * d + c];
        delta[i] = acc;
    }
    memset(dQ, 0, sizeof(double) * (size_t)(q1 - q0) * d);
    memset(dK, 0, sizeof(double) * (size_t)(k1 - k0) * d);
    memset(dV, 0, sizeof(double) * (size_t)(k1 - k0) * d);
    /* rows needed: dQ rows, plus every row for the dK/dV columns */
    int need_all = (k1 > k0);
    int ra = need_all ? 0 : q0, rb = need_all ? Nq : q1;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* pq = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* ds = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* dk_loc = (double*)calloc((size_t)(k1 - k0) * d + 1, sizeof(double));
        double* dv_loc = (double*)calloc((size_t)(k1 - k0) * d + 1, sizeof(double));
#pragma omp for schedule(dynamic)
        for (int i = ra; i < rb; ++i) {
            int want_q = (i >= q0 && i < q1);
            int ja = want_q ? 0 : (k0 / 32) * 32, jb = want_q ? Nk : ((k1 + 31) / 32) * 32;
            double mrow = rowmax ? rowmax[i] : -INFINITY;
            if (!rowmax)
                for (int j = 0; j < Nk; ++j) {
                    double s;
                    orc_mx_scores(qc, qs, kc, ks, d, i, j, &s);
                    if (tau * s > mrow) mrow = tau * s;
                }
            for (int j = ja; j < jb; ++j) {
                double s;
                orc_mx_scores(qc, qs, kc, ks, d, i, j, &s);
                p[j] = exp(tau * s - (double)lse[i]);
                pq[j] = quantize_p ? exp(tau * s - mrow) : p[j];
            }
            if (quantize_p) {
                const double back = exp(mrow - (double)lse[i]);
                for (int j = ja; j < jb; j += 32) mx_fake32(pq + j, 32);
                for (int j = ja; j < jb; ++j) pq[j] *= back;
            }
            for (int j = ja; j < jb; ++j) {
                double dp = 0.0;
                for (int c = 0; c < d; ++c) dp += (double)dO[(size_t)i * d + c] * vmx(vc_t, vs_t, Nk, j, c);
                ds[j] = p[j] * (dp - delta[i]);
                if (quantize_p) ds[j] = orc_bf16_value(ds[j]);
            }
            if (want_q)
                for (int c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < Nk; ++j) acc += ds[j] * kmx(kc, ks, d, j, c);
                    dQ[(size_t)(i - q0) * d + c] = tau * acc;
                }
            for (int j = k0; j < k1; ++j)
                for (int c = 0; c < d; ++c) {
                    dk_loc[(size_t)(j - k0) * d + c] += ds[j] * kmx(qc, qs, d, i, c);
                    dv_loc[(size_t)(j - k0) * d + c] += pq[j] * (double)dO[(size_t)i * d + c];
                }
        }
#pragma omp critical
        {
            for (size_t u = 0; u < (size_t)(k1 - k0) * d; ++u) { dK[u] += tau * dk_loc[u]; dV[u] += dv_loc[u]; }
        }
        free(p); free(pq); free(ds); free(dk_loc); free(dv_loc);
    }
    free(delta);
}

/* ========================================================================
 * ThriftAttention ([TA] Method)
 * ====================================================================== */

/* Pairs kept in 16-bit for a query block with n valid key blocks:
 * max(1, ceil(n * budget)), never more than n; budget in parts per million. */
int orc_budget_count(int n_valid, int budget_ppm) {
    if (n_valid <= 0) return 0;
    int64_t k = ((int64_t)n_valid * budget_ppm + 999999) / 1000000;
    if (k < 1) k = 1;
    if (k > n_valid) k = n_valid;
    return (int)k;
}

typedef struct { double s; int j; } scored;
static int by_score(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);       /* equal scores: smaller j first */
}
static int by_int(const void* a, const void* b) {
    int x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Block selection ([TA] step 1): importance S_ij = qbar_i . kbar_j (fp64 on
 * the fp32 means) over the valid key blocks of query block i (causal:
 * j <= i + nkb - nqb); the top-k by score, ties to the smaller j, written in
 * ascending j.  Unused slots hold -1. */
void orc_select_blocks(const float* qbar, const float* kbar, int nqb, int nkb, int d,
                       int causal, int budget_ppm, int max_sel, int32_t* sel_idx, int32_t* sel_cnt) {
#pragma omp parallel for schedule(dynamic)
    for (int i = 0; i < nqb; ++i) {
        int nv = causal ? i + (nkb - nqb) + 1 : nkb;
        if (nv > nkb) nv = nkb;
        scored* sc = (scored*)malloc(sizeof(scored) * (size_t)(nv > 0 ? nv : 1));
        for (int j = 0; j < nv; ++j) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += (double)qbar[(size_t)i * d + c] * (double)kbar[(size_t)j * d + c];
            sc[j].s = acc;
            sc[j].j = j;
        }
        qsort(sc, (size_t)nv, sizeof(scored), by_score);
        int k = orc_budget_count(nv, budget_ppm);
        if (k > max_sel) k = max_sel;
        int32_t* out = sel_idx + (size_t)i * max_sel;
        for (int u = 0; u < max_sel; ++u) out[u] = -1;
        for (int u = 0; u < k; ++u) out[u] = sc[u].j;
        qsort(out, (size_t)k, sizeof(int32_t), by_int);
        sel_cnt[i] = k;
        free(sc);
    }
}

typedef struct {
    const uint8_t *qc, *qs, *kc, *ks, *vc_t, *vs_t;
    const float *Qh, *Kh, *Vh;
    int Nk, d, quantize;
    double tau;
    const double* bias;   /* FP4 path: added to key j's raw score (query smoothing); NULL: none */
    const float *Qn, *Kn, *Vn;   /* NVFP4 emulation (path 2): the dequantised NVFP4 rows */
} thrift_ctx;

/* One key block (keys [j0, j0+n)) through one path, for query row i (row
 * index into the codes / bf16 rows).  path 0: FP4 — exact MX scores, P
 * rounded to fp32, two-level MXFP4: the row's tile max r maps to 6,
 * P' = fp32(P * fp32(6/r)) is MXFP4-quantised per 32 keys and dequantised
 * as (r/6) deq(P'), times the FP4 V.  path 1: bf16 — scores from the bf16
 * Q and K, bf16(P) times the bf16 V.  quantize == 0: both paths use the
 * bf16 operands and unrounded P. */
static void nvfp4_p_tile(double* p, int n, double* out);

static void thrift_block(const thrift_ctx* c, row_state* st, int i, int j0, int n, int path) {
    int d = c->d;
    double s[256], p[256];
    double tmax = -INFINITY;
    const float* Qx = path == 2 ? c->Qn : c->Qh;
    const float* Kx = path == 2 ? c->Kn : c->Kh;
    for (int u = 0; u < n; ++u) {
        int j = j0 + u;
        if (path == 0 && c->quantize) {
            orc_mx_scores(c->qc, c->qs, c->kc, c->ks, d, i, j, &s[u]);
            if (c->bias) s[u] += c->bias[j];
            s[u] *= c->tau;
        } else {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += (double)Qx[(size_t)i * d + k] * (double)Kx[(size_t)j * d + k];
            s[u] = c->tau * acc;
        }
        if (s[u] > tmax) tmax = s[u];
    }
    row_update_max(st, tmax, d);
    if (path == 2) {
        /* NVFP4 emulation: P quantised in two levels to NVFP4, times the
         * dequantised NVFP4 V */
        double pq[256];
        for (int u = 0; u < n; ++u) { p[u] = exp(s[u] - st->m); st->l += p[u]; }
        nvfp4_p_tile(p, n, pq);
        for (int u = 0; u < n; ++u)
            for (int k = 0; k < d; ++k) st->acc[k] += pq[u] * (double)c->Vn[(size_t)(j0 + u) * d + k];
        return;
    }
    double r = 0.0;
    for (int u = 0; u < n; ++u) { p[u] = exp(s[u] - st->m); st->l += p[u]; if (p[u] > r) r = p[u]; }
    if (!c->quantize) {
        for (int u = 0; u < n; ++u)
            for (int k = 0; k < d; ++k) st->acc[k] += p[u] * (double)c->Vh[(size_t)(j0 + u) * d + k];
        return;
    }
    if (path == 1) {
        for (int u = 0; u < n; ++u) {
            double pb = orc_bf16_value(p[u]);
            for (int k = 0; k < d; ++k) st->acc[k] += pb * (double)c->Vh[(size_t)(j0 + u) * d + k];
        }
        return;
    }
    float rf = (float)r;
    if (rf == 0.0f) return;        /* every P of the block underflows fp32: nothing to add */
    float six_over_r = 6.0f / rf;
    double pp[256];
    for (int u = 0; u < n; ++u) pp[u] = (double)((float)p[u] * six_over_r);
    for (int u = n; u < ((n + 31) / 32) * 32; ++u) pp[u] = 0.0;      /* masked keys */
    for (int u = 0; u < n; u += 32) mx_fake32(pp + u, 32);
    for (int u = 0; u < n; ++u) {
        double pq = (double)rf / 6.0 * pp[u];
        for (int k = 0; k < d; ++k) st->acc[k] += pq * vmx(c->vc_t, c->vs_t, c->Nk, j0 + u, k);
    }
}

/* Thrift prefill for query blocks [qb0, qb1) of one head ([TA] step 2 and
 * the kernel paragraph): per query block, the unselected valid key blocks
 * go through the FP4 path in ascending order, then the selected blocks
 * through the bf16 path in ascending order, all merged in one online
 * softmax.  The diagonal block is masked in whichever path takes it.  An FP4
 * block is one tile of the online softmax (its two-level factor is per row
 * and block); a bf16 block is visited as tiles of hp_tile keys. */
void orc_thrift_fwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                    const uint8_t* vc_t, const uint8_t* vs_t,
                    const float* Qh, const float* Kh, const float* Vh,
                    const int32_t* sel_idx, const int32_t* sel_cnt, int max_sel,
                    int Nq, int Nk, int d, int blk, int hp_tile, int causal, double tau, int quantize,
                    int qb0, int qb1, double* O, double* lse) {
    thrift_ctx c = {qc, qs, kc, ks, vc_t, vs_t, Qh, Kh, Vh, Nk, d, quantize, tau, NULL, NULL, NULL, NULL};
    int nkb = Nk / blk;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int I = qb0; I < qb1; ++I)
        for (int a = 0; a < blk; ++a) {
            int i = I * blk + a;
            int last = last_key(i, Nq, Nk, causal);
            const int32_t* sel = sel_idx + (size_t)I * max_sel;
            int ns = sel_cnt[I];
            row_state st = {-INFINITY, 0.0, (double*)calloc((size_t)d, sizeof(double)), NULL};
            for (int pass = 0; pass < 2; ++pass)
                for (int J = 0; J < nkb && J * blk <= last; ++J) {
                    int picked = 0;
                    for (int u = 0; u < ns; ++u) if (sel[u] == J) picked = 1;
                    if (picked != pass) continue;
                    int tile = pass ? hp_tile : blk;
                    for (int t0 = J * blk; t0 < (J + 1) * blk && t0 <= last; t0 += tile) {
                        int n = tile;
                        if (t0 + n - 1 > last) n = last - t0 + 1;
                        thrift_block(&c, &st, i, t0, n, pass);
                    }
                }
            for (int k = 0; k < d; ++k) O[((size_t)(I - qb0) * blk + a) * d + k] = st.acc[k] / st.l;
            lse[(size_t)(I - qb0) * blk + a] = st.m + log(st.l);
            free(st.acc);
        }
}

/* Thrift decode for one (batch, query head): the single query sits after
 * the whole cache, so every key is visible.  The key blocks are cut into
 * num_splits contiguous ranges [s nb/S, (s+1) nb/S); each range runs its
 * FP4 blocks, then its selected bf16 blocks (as tiles of hp_tile keys), in
 * ascending order, giving a partial (m_s, l_s, acc_s); the partials are
 * merged by m = max m_s, l = sum e^(m_s - m) l_s, o = sum e^(m_s - m) acc_s / l. */
void orc_thrift_decode(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                       const uint8_t* vc_t, const uint8_t* vs_t,
                       const float* q, const float* Kh, const float* Vh,
                       const int32_t* sel, int nsel, int Nk, int d, int blk, int hp_tile, double tau,
                       int num_splits, int quantize, double* o, double* lse) {
    thrift_ctx c = {qc, qs, kc, ks, vc_t, vs_t, q, Kh, Vh, Nk, d, quantize, tau, NULL, NULL, NULL, NULL};
    int nb = Nk / blk;
    double* ms = (double*)malloc(sizeof(double) * (size_t)num_splits);
    double* ls = (double*)malloc(sizeof(double) * (size_t)num_splits);
    double* acc = (double*)calloc((size_t)num_splits * d, sizeof(double));
    for (int sp = 0; sp < num_splits; ++sp) {
        int b0 = (int)((int64_t)sp * nb / num_splits), b1 = (int)((int64_t)(sp + 1) * nb / num_splits);
        row_state st = {-INFINITY, 0.0, acc + (size_t)sp * d, NULL};
        for (int pass = 0; pass < 2; ++pass)
            for (int J = b0; J < b1; ++J) {
                int picked = 0;
                for (int u = 0; u < nsel; ++u) if (sel[u] == J) picked = 1;
                if (picked != pass) continue;
                int tile = pass ? hp_tile : blk;
                for (int t0 = J * blk; t0 < (J + 1) * blk; t0 += tile) thrift_block(&c, &st, 0, t0, tile, pass);
            }
        ms[sp] = st.m;
        ls[sp] = st.l;
    }
    double m = -INFINITY;
    for (int sp = 0; sp < num_splits; ++sp) if (ms[sp] > m) m = ms[sp];
    double l = 0.0;
    for (int k = 0; k < d; ++k) o[k] = 0.0;
    for (int sp = 0; sp < num_splits; ++sp) {
        if (ms[sp] == -INFINITY) continue;
        double w = exp(ms[sp] - m);
        l += w * ls[sp];
        for (int k = 0; k < d; ++k) o[k] += w * acc[(size_t)sp * d + k];
    }
    for (int k = 0; k < d; ++k) o[k] /= l;
    *lse = m + log(l);
    free(ms); free(ls); free(acc);
}

/* ========================================================================
 * Post-training FP4 baseline in the SageAttention3 style
 * ====================================================================== */

/* [AQ] §1 and §2 Implementation describe the post-training FP4 method that
 * Attn-QAT is measured against: FP4 attention with query and key smoothing
 * and two-level quantisation of P ([TA] step 2 uses the same two-level
 * scheme).  Reading: K is smoothed as in [SB] (its token mean is subtracted;
 * the shift is the same for every key of a row, so the softmax is
 * unchanged); Q is smoothed per block of blk rows: qbar_I, the block's mean
 * rounded to bf16, is subtracted before quantisation and its product with
 * the keys is added back, s_ij = tau (q^_s,i . k^_j + qbar_I . k^_j), both
 * dot products exact in fp64 (k^ the dequantised MXFP4 key).  The softmax
 * and P.V are those of the Thrift FP4 path with nothing selected: key
 * blocks of blk keys in ascending order (causal: up to the row's last key),
 * each one online-softmax tile with two-level P.  qc/qs hold the codes of
 * the smoothed Q, kc/ks those of the smoothed K; qbar is [nqb][d] with
 * nqb = ceil(Nq / blk); query blocks [qb0, qb1), the last one possibly
 * short.  O and lse hold the rows of those blocks that exist. */
void orc_ptq_fwd(const uint8_t* qc, const uint8_t* qs, const float* qbar, const uint8_t* kc, const uint8_t* ks,
                 const uint8_t* vc_t, const uint8_t* vs_t, int Nq, int Nk, int d, int blk, int causal, double tau,
                 int qb0, int qb1, double* O, double* lse) {
    int nkb = Nk / blk;
    double* bias = (double*)malloc(sizeof(double) * (size_t)Nk);
    size_t out_row = 0;
    for (int I = qb0; I < qb1; ++I) {
        for (int j = 0; j < Nk; ++j) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += (double)qbar[(size_t)I * d + c] * kmx(kc, ks, d, j, c);
            bias[j] = acc;
        }
        thrift_ctx ctx = {qc, qs, kc, ks, vc_t, vs_t, NULL, NULL, NULL, Nk, d, 1, tau, bias, NULL, NULL, NULL};
        int rows = Nq - I * blk < blk ? Nq - I * blk : blk;
#pragma omp parallel for schedule(dynamic)
        for (int a = 0; a < rows; ++a) {
            int i = I * blk + a;
            int last = last_key(i, Nq, Nk, causal);
            row_state st = {-INFINITY, 0.0, (double*)calloc((size_t)d, sizeof(double)), NULL};
            for (int J = 0; J < nkb && J * blk <= last; ++J) {
                int n = blk;
                if (J * blk + n - 1 > last) n = last - J * blk + 1;
                thrift_block(&ctx, &st, i, J * blk, n, 0);
            }
            for (int k = 0; k < d; ++k) O[(out_row + (size_t)a) * d + k] = st.acc[k] / st.l;
            lse[out_row + (size_t)a] = st.m + log(st.l);
            free(st.acc);
        }
        out_row += (size_t)rows;
    }
    free(bias);
}

/* ========================================================================
 * QK-norm ([SB] Methodology 4 and Practical implications: every query and
 * key row is scaled to unit L2 norm before the dot product)
 * ====================================================================== */

/* Forward, row by row: S = sum_c x_c^2 in fp64 (exact for bf16 rows),
 * r = fp32(1 / sqrt(S)) from the fp64 value (r = 0 for a zero row), and the
 * normalised row y_c = bf16(fp32(x_c r)), the bf16 output a model's QK-norm
 * layer would hand to the attention.  r is kept for the backward. */
void orc_qk_norm(const float* X, int64_t rows, int d, float* Y, float* r) {
    for (int64_t i = 0; i < rows; ++i) {
        const float* x = X + (size_t)i * d;
        double S = 0.0;
        for (int c = 0; c < d; ++c) S += (double)x[c] * (double)x[c];
        float ri = S > 0.0 ? (float)(1.0 / sqrt(S)) : 0.0f;
        r[i] = ri;
        for (int c = 0; c < d; ++c) Y[(size_t)i * d + c] = (float)orc_bf16_value((double)(x[c] * ri));
    }
}

/* Backward of y = x / |x| with the bf16 rounding of y passed straight
 * through: with y = x r (unrounded), dx = r (g - y (y . g)), in fp64. */
void orc_qk_norm_bwd(const float* X, const float* r, const double* G, int64_t rows, int d, double* dX) {
    for (int64_t i = 0; i < rows; ++i) {
        const float* x = X + (size_t)i * d;
        const double* g = G + (size_t)i * d;
        double ri = (double)r[i], t = 0.0;
        for (int c = 0; c < d; ++c) t += (double)x[c] * ri * g[c];
        for (int c = 0; c < d; ++c) dX[(size_t)i * d + c] = ri * (g[c] - (double)x[c] * ri * t);
    }
}

/* ========================================================================
 * NVFP4 format emulation ([TA] Method step 2: the FP4 path uses NVFP4
 * micro-scaling: e2m1 values in blocks of 16 with an E4M3 block scale)
 * ====================================================================== */

/* e4m3 value nearest to x (RNE, saturating at 448). */
static double e4m3_value(double x) { return orc_round_grid(x, 3, -6, 448.0, 1); }
/* e2m1 value nearest to x (RNE, saturating at 6). */
static double e2m1_value(double x) { return orc_round_grid(x, 1, 0, 6.0, 1); }

/* One block of 16 values with shared scale S (an fp32 value, the block
 * scale times the tensor scale): x_q = e2m1(fp32(x / S)) S; S == 0 gives
 * zeros. */
static void nv_block(const float* x, int stride, int n, float S, float* out, int ostride) {
    for (int u = 0; u < n; ++u) {
        double v = 0.0;
        if (S != 0.0f) v = e2m1_value((double)(x[(size_t)u * stride] / S)) * (double)S;
        out[(size_t)u * ostride] = (float)v;
    }
}

/* NVFP4 quantisation of one [N, d] slice, written back as the dequantised
 * values (exact in fp32 and in bf16): blocks of 16 along d (axis 0: Q, K)
 * or along the tokens of each channel (axis 1: V).  Reading of the
 * two-level scale: the tensor scale g of the slice is the power of two at
 * or above amax / (448 * 6) (1 for an all-zero slice), so that every block
 * scale fits E4M3; a block's scale is e4m3(fp32(amax_b / fp32(6 g))) and
 * its values e2m1(fp32(x / fp32(s_b g))) s_b g. */
void orc_nvfp4_fake(const float* X, int BH, int N, int d, int axis, float* out) {
    for (int bh = 0; bh < BH; ++bh) {
        const float* x = X + (size_t)bh * N * d;
        float* o = out + (size_t)bh * N * d;
        float amax = 0.0f;
        for (size_t t = 0; t < (size_t)N * d; ++t) if (fabsf(x[t]) > amax) amax = fabsf(x[t]);
        float g = 1.0f;
        if (amax > 0.0f) {
            int E;
            double q = (double)amax / 2688.0;
            double f = frexp(q, &E);          /* q = f 2^E, f in [0.5, 1) */
            g = (float)ldexp(1.0, f == 0.5 ? E - 1 : E);
        }
        float six_g = 6.0f * g;
        int nb = axis == 0 ? d / 16 : N / 16;
        int nrow = axis == 0 ? N : d;
        for (int r = 0; r < nrow; ++r)
            for (int b = 0; b < nb; ++b) {
                const float* xb = axis == 0 ? x + (size_t)r * d + 16 * b : x + (size_t)16 * b * d + r;
                float* ob = axis == 0 ? o + (size_t)r * d + 16 * b : o + (size_t)16 * b * d + r;
                int stride = axis == 0 ? 1 : d;
                float am = 0.0f;
                for (int u = 0; u < 16; ++u) if (fabsf(xb[(size_t)u * stride]) > am) am = fabsf(xb[(size_t)u * stride]);
                float sb = (float)e4m3_value((double)(am / six_g));
                nv_block(xb, stride, 16, sb * g, ob, stride);
            }
    }
}

/* Two-level NVFP4 quantisation of one row's probabilities in a tile of n
 * keys (n a multiple of 16): r = the tile's largest fp32(P); P' =
 * fp32(fp32(P) fp32(2688 / r)) puts it at 448 * 6; blocks of 16 keys get the
 * scale e4m3(fp32(amax / 6)) and values e2m1(fp32(P' / s_b)) s_b; the first
 * level is undone as bf16(fp32(P^' fp32(r / 2688))), the operand of the
 * bf16 P.V.  A tile whose P all underflow fp32 gives zeros. */
static void nvfp4_p_tile(double* p, int n, double* out) {
    float pf[256], pp[256];
    float r = 0.0f;
    for (int u = 0; u < n; ++u) { pf[u] = (float)p[u]; if (pf[u] > r) r = pf[u]; }
    if (r == 0.0f) { for (int u = 0; u < n; ++u) out[u] = 0.0; return; }
    float f_in = 2688.0f / r, f_out = r / 2688.0f;
    for (int u = 0; u < n; ++u) pp[u] = pf[u] * f_in;
    for (int b = 0; b < n; b += 16) {
        float am = 0.0f;
        for (int u = b; u < b + 16 && u < n; ++u) if (pp[u] > am) am = pp[u];
        float sb = (float)e4m3_value((double)(am / 6.0f));
        for (int u = b; u < b + 16 && u < n; ++u) {
            double q = sb != 0.0f ? e2m1_value((double)(pp[u] / sb)) * (double)sb : 0.0;
            out[u] = orc_bf16_value((double)((float)q * f_out));
        }
    }
}

/* Thrift prefill in NVFP4 emulation: as orc_thrift_fwd, except that the
 * unselected blocks take path 2 (the dequantised NVFP4 Q, K, V of Qn, Kn,
 * Vn, NVFP4 two-level P) in tiles of hp_tile keys. */
void orc_thrift_fwd_nv(const float* Qn, const float* Kn, const float* Vn, const float* Qh, const float* Kh,
                       const float* Vh, const int32_t* sel_idx, const int32_t* sel_cnt, int max_sel, int Nq, int Nk,
                       int d, int blk, int hp_tile, int causal, double tau, int qb0, int qb1, double* O,
                       double* lse) {
    thrift_ctx c = {NULL, NULL, NULL, NULL, NULL, NULL, Qh, Kh, Vh, Nk, d, 1, tau, NULL, Qn, Kn, Vn};
    int nkb = Nk / blk;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int I = qb0; I < qb1; ++I)
        for (int a = 0; a < blk; ++a) {
            int i = I * blk + a;
            int last = last_key(i, Nq, Nk, causal);
            const int32_t* sel = sel_idx + (size_t)I * max_sel;
            int ns = sel_cnt[I];
            row_state st = {-INFINITY, 0.0, (double*)calloc((size_t)d, sizeof(double)), NULL};
            for (int pass = 0; pass < 2; ++pass)
                for (int J = 0; J < nkb && J * blk <= last; ++J) {
                    int picked = 0;
                    for (int u = 0; u < ns; ++u) if (sel[u] == J) picked = 1;
                    if (picked != pass) continue;
                    for (int t0 = J * blk; t0 < (J + 1) * blk && t0 <= last; t0 += hp_tile) {
                        int n = hp_tile;
                        if (t0 + n - 1 > last) n = last - t0 + 1;
                        thrift_block(&c, &st, i, t0, n, pass ? 1 : 2);
                    }
                }
            for (int k = 0; k < d; ++k) O[((size_t)(I - qb0) * blk + a) * d + k] = st.acc[k] / st.l;
            lse[(size_t)(I - qb0) * blk + a] = st.m + log(st.l);
            free(st.acc);
        }
}

