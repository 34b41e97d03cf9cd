/*
 * Plain CPU oracle for block-quantized attention (test infrastructure only).
 *
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with
 * the GPU library: every encoder and every loop here is written out again
 * from the format definitions and from the method as the pages describe it.
 *
 * Conventions: one call covers one (batch, head) slice unless it says
 * otherwise; slices are row-major [N, d] fp32 arrays whose values are the
 * bf16/fp16 inputs converted exactly; floating-point work between the
 * rounding points the method prescribes is done in fp64.
 */
#ifndef BQA_ORACLE_H
#define BQA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar encoders (OCP 8-bit/4-bit formats, IEEE half formats) ---- */
double  orc_round_grid(double x, int mant_bits, int emin, double maxval, int saturate);
uint8_t orc_e4m3_encode(double x);          /* RNE, saturating to +-448 */
double  orc_e4m3_decode(uint8_t c);
uint8_t orc_e2m1_encode(double x);          /* RNE, saturating to +-6, 4-bit code */
double  orc_e2m1_decode(uint8_t c);
int     orc_e8m0_exponent(float amax);      /* clamp(floor(log2 amax) - 2, -127, 127) */
uint16_t orc_bf16_bits(double x);
uint16_t orc_f16_bits(double x);
double  orc_bf16_value(double x);           /* x rounded to bf16, as a value */
double  orc_f16_value(double x);
void    orc_round_array(const double* x, int64_t n, int fmt, double* out);
int8_t  orc_i8_encode(float x, float inv);  /* clamp(rint(fp32(x*inv)), -127, 127) */
void    orc_i8_scale(float amax, float* scale, float* inv);

/* ---- quantisers (arrays are one head unless BH is an argument) ---- */
int  orc_smooth_mean(const float* K, int BH, int N, int d, double eps, float* mu_eff);
void orc_quant_i8_tokblock(const float* X, const float* mu, int BH, int N, int d, int blk,
                           int8_t* codes, float* scales);
void orc_quant_chan(const float* V, int BH, int N, int d, int fmt, uint8_t* codes_t, float* scales);
void orc_quant_mx_rows(const float* X, int BH, int N, int d, uint8_t* codes, uint8_t* scales);
void orc_quant_mx_cols(const float* X, int BH, int N, int d, uint8_t* codes_t, uint8_t* scales_t);
void orc_block_means(const float* X, int BH, int N, int d, int blk, float* means);

/* ---- textbook attention in fp64 (two-pass softmax) ---- */
void orc_ref_fwd(const float* Q, const float* K, const float* V, int Nq, int Nk, int d,
                 int causal, double tau, double* O, double* lse);
void orc_ref_bwd(const float* Q, const float* K, const float* V, const float* dO,
                 int Nq, int Nk, int d, int causal, double tau,
                 double* dQ, double* dK, double* dV);

/* ---- SageAttention INT8 forward / SageBwd backward ---- */
enum { ORC_PV_NONE = 0, ORC_PV_F16 = 1, ORC_PV_F8 = 2, ORC_PV_I8 = 3 };
enum { ORC_QK_I8 = 0, ORC_QK_F64 = 1 };
void orc_sage_fwd(int qk_mode, const int8_t* qc, const float* qs, int q_blk,
                  const int8_t* kc, const float* ks, int k_blk,
                  const float* Qf, const float* Kf,
                  int pv_mode, const float* Vf, const uint8_t* vc_t, const float* vs,
                  int Nq, int Nk, int d, int causal, double tau, int kv_tile,
                  int r0, int r1, double* O, double* lse);
void orc_sage_bwd(const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                  const float* V, const float* dO, const float* O, const float* lse,
                  int N, int d, int causal, double tau, int tile_q, int tile_k, int do_blk,
                  int quantize, int qt0, int qt1, int kt0, int kt1,
                  double* dQ, double* dK, double* dV);
void orc_sage_bwd_v(const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                    const float* V, const float* dO, const float* O, const float* lse,
                    int N, int d, int causal, double tau, int tile_q, int tile_k, int do_blk,
                    int quantize, int qt0, int qt1, int kt0, int kt1,
                    const int8_t* vc, const float* vs, int v_blk,
                    double* dQ, double* dK, double* dV);

/* ---- Attn-QAT FP4 forward / backward ---- */
int  orc_mx_scores(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                   int d, int i, int j, double* s);
void orc_qat_fwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                 const uint8_t* vc_t, const uint8_t* vs_t, int Nq, int Nk, int d,
                 double tau, int kv_tile, int quantize_p, int r0, int r1,
                 double* O, double* O_aux, double* lse, double* rowmax);
void orc_qat_bwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                 const uint8_t* vc_t, const uint8_t* vs_t, const float* dO, const float* O_aux,
                 const float* lse, const double* rowmax, int Nq, int Nk, int d, double tau, int quantize_p,
                 int q0, int q1, int k0, int k1, double* dQ, double* dK, double* dV);

/* ---- ThriftAttention ---- */
int  orc_budget_count(int n_valid, int budget_ppm);
void orc_select_blocks(const float* qbar, const float* kbar, int nqb, int nkb, int d,
                       int causal, int budget_ppm, int max_sel, int32_t* sel_idx, int32_t* sel_cnt);
void orc_thrift_fwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                    const uint8_t* vc_t, const uint8_t* vs_t,
                    const float* Qh, const float* Kh, const float* Vh,
                    const int32_t* sel_idx, const int32_t* sel_cnt, int max_sel,
                    int Nq, int Nk, int d, int blk, int hp_tile, int causal, double tau, int quantize,
                    int qb0, int qb1, double* O, double* lse);
void orc_thrift_decode(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                       const uint8_t* vc_t, const uint8_t* vs_t,
                       const float* q, const float* Kh, const float* Vh,
                       const int32_t* sel, int nsel, int Nk, int d, int blk, int hp_tile, double tau,
                       int num_splits, int quantize, double* o, double* lse);
void orc_ptq_fwd(const uint8_t* qc, const uint8_t* qs, const float* qbar, const uint8_t* kc, const uint8_t* ks,
                 const uint8_t* vc_t, const uint8_t* vs_t, int Nq, int Nk, int d, int blk, int causal, double tau,
                 int qb0, int qb1, double* O, double* lse);
void orc_nvfp4_fake(const float* X, int BH, int N, int d, int axis, float* out);
void orc_thrift_fwd_nv(const float* Qn, const float* Kn, const float* Vn, const float* Qh, const float* Kh,
                       const float* Vh, const int32_t* sel_idx, const int32_t* sel_cnt, int max_sel, int Nq, int Nk,
                       int d, int blk, int hp_tile, int causal, double tau, int qb0, int qb1, double* O,
                       double* lse);
void orc_qk_norm(const float* X, int64_t rows, int d, float* Y, float* r);
void orc_qk_norm_bwd(const float* X, const float* r, const double* G, int64_t rows, int d, double* dX);

#ifdef __cplusplus
}
#endif
#endif
