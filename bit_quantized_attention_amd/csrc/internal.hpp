// internal.hpp — host-side declarations shared by the library's translation
// units (launchers and argument blocks).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace bqa {

// ---- quantisation (quant.hip)
size_t ws_kmean_bytes(int BH, int N, int d);
size_t ws_chan_bytes(int BH, int N, int d);
hipError_t launch_quant_i8_tokblock(const Dense& x, bool f16, int B, int H, int N, int d, int blk, bool smooth,
                                    double eps, float* mu, void* ws, int8_t* codes, float* scales,
                                    hipStream_t st);
hipError_t launch_quant_chan(const Dense& x, bool f16, int B, int H, int N, int d, int fmt, uint8_t* codes_t,
                             float* scales, void* ws, hipStream_t st);
size_t ws_kv_bytes(int BH, int N, int d);
hipError_t launch_quant_kv(const Dense& k, const Dense& v, bool f16, int B, int H, int N, int d, bool smooth,
                           double eps, float* mu, int8_t* kc, float* ks, int vfmt, uint8_t* vc, float* vs, void* ws,
                           hipStream_t st);
hipError_t launch_quant_mx(const Dense& x, bool f16, int B, int H, int N, int d, int axis, uint8_t* codes,
                           uint8_t* scales, float* means, hipStream_t st);
hipError_t launch_quant_i8_qknorm(const Dense& x, bool f16, int B, int H, int N, int d, int blk, bool smooth,
                                  double eps, float* mu, float* inv_norm, void* ws, int8_t* codes, float* scales,
                                  hipStream_t st);
size_t ws_nvfp4_bytes(int BH, int N, int d);
hipError_t launch_nvfp4(const Dense& x, bool f16, int B, int H, int N, int d, int axis, const Dense& out, void* ws,
                        hipStream_t st);
hipError_t launch_quant_mx_smooth(const Dense& x, bool f16, int B, int H, int N, int d, bool key, double eps,
                                  uint8_t* codes, uint8_t* scales, float* means, void* ws, hipStream_t st);

// ---- SageAttention INT8 forward (attn_sage_fwd.hip)
enum { PV_F16 = 0, PV_F8 = 1, PV_I8 = 2 };
struct SageFwdArgs {
    const int8_t* qc;  const float* qs;  int q_blk;     // Q codes [B,Hq,Nq,d], scales [B,Hq,Nq/q_blk]
    Dense q16;                                           // bf16 Q quantised in the kernel (p null: use qc/qs)
    int8_t* qc_out;    float* qs_out;                    // with q16: where its codes / scales go (or null)
    const int8_t* kc;  const float* ks;                  // K codes [B,Hkv,Nk,d], scales [B,Hkv,Nk/64]
    const uint8_t* vc; const float* vs;                  // V codes [B,Hkv,d,Nk], scales [B,Hkv,d]
    Dense v16;                                           // V fp16 (PV_F16)
    Dense o;                                             // O [B,Hq,Nq,d] bf16 (fp16 for PV_F16)
    float* lse;                                          // [B,Hq,Nq] or null
    int B, Hq, Hkv, Nq, Nk;
    int causal;
    float c_log2;                                        // tau * log2(e)
};
hipError_t launch_sage_fwd(const SageFwdArgs& a, int pv, int d, hipStream_t st);
hipError_t launch_debug_scores_i8(const int8_t* qc, const int8_t* kc, int d, int64_t q_row0, int64_t k_row0,
                                  int32_t* out, hipStream_t st);

// ---- Attn-QAT MXFP4 forward (attn_qat.hip); head dimension 128, non-causal
struct QatFwdArgs {
    const uint8_t* qc; const uint8_t* qs;                // Q codes [B,Hq,Nq,d/2], E8M0 [B,Hq,Nq,d/32]
    const uint8_t* kc; const uint8_t* ks;                // K codes [B,Hkv,Nk,d/2], E8M0 [B,Hkv,Nk,d/32]
    const uint8_t* vc; const uint8_t* vs;                // V codes [B,Hkv,d,Nk/2], E8M0 [B,Hkv,d,Nk/32]
    uint16_t* vdeq;                                      // workspace [B,Hkv,d,Nk] bf16; null: no O'
    Dense o, oa;                                         // O, O' [B,Hq,Nq,d] bf16
    float* lse;                                          // [B,Hq,Nq] or null
    float* row_max;                                      // [B,Hq,Nq] largest raw score of each row, or null
    int B, Hq, Hkv, Nq, Nk;
    float c_log2;                                        // tau * log2(e)
};
size_t ws_qat_fwd_bytes(int B, int Hkv, int Nk, int d);
// MXFP4 blocks (16 code bytes + 1 E8M0 byte each) -> 32 bf16 values each (the conversion of deq(V))
hipError_t launch_mx_dequant(const uint8_t* codes, const uint8_t* scales, int64_t nblocks, uint16_t* out,
                             hipStream_t st);
hipError_t launch_qat_fwd(const QatFwdArgs& a, hipStream_t st);
hipError_t launch_debug_scores_mx(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                  float* out, hipStream_t st);

// ---- SageBwd backward (attn_sage_bwd.hip); d = 128, Hq == Hkv, N a multiple of 128
struct SageBwdArgs {
    const int8_t* qc; const float* qs;                   // forward Q codes [B,H,N,d], scales per 128 tokens
    const int8_t* kc; const float* ks;                   // forward K codes [B,H,N,d], scales per 64 tokens
    Dense v, d_o;                                        // V, dO bf16 [B,H,N,d]
    const float* lse;                                    // forward log-sum-exp [B,H,N]
    float* delta; const float* dos;                      // workspace: delta [B,H,N], dO scales
    const int8_t* doT; const int8_t* qT; const int8_t* kT;   // workspace: channel-major codes [B,H,d,N]
    Dense dq, dk, dv;                                    // outputs bf16
    int B, H, N, causal;
    float c_log2, tau;
    // QK-norm backward in the dQ / dK epilogues (null: gradients of the
    // normalised rows): raw Q, K [B,H,N,d] bf16 and their inverse norms [B,H,N]
    Dense q_raw, k_raw;
    const float* q_rn; const float* k_rn;
    // fully INT8 variant (null: dP in bf16 from v): V's INT8 codes [B,H,N,d]
    // and scales per 64 tokens; doc: workspace, row-major dO codes
    const int8_t* vc8; const float* vs8;
    int8_t* doc;
};
size_t ws_sage_bwd_bytes(int B, int H, int N, int d);
hipError_t launch_sage_bwd(SageBwdArgs a, Dense o, void* ws, hipStream_t st);

// ---- Attn-QAT backward (attn_qat_bwd.hip); d = 128, Hq == Hkv, N a multiple of 128, non-causal
struct QatBwdArgs {
    const uint8_t* qc; const uint8_t* qs;                // MXFP4 Q [B,H,N,d/2], E8M0 [B,H,N,d/32]
    const uint8_t* kc; const uint8_t* ks;                // MXFP4 K
    const uint8_t* vc; const uint8_t* vs;                // MXFP4 V [B,H,d,N/2], E8M0 [B,H,d,N/32]
    Dense d_o;                                           // dO bf16
    const float* lse;                                    // forward log-sum-exp
    const float* row_max;                                // forward: largest raw score of each row
    float* delta;                                        // workspace: delta' [B,H,N]
    uint32_t* do_amax;                                   // workspace: largest |dO| per (b, h), fp32 bits
    uint16_t* vdeq; uint16_t* qT; uint16_t* kT; uint16_t* doT;   // workspace: bf16 copies (dO^T fp16, scaled)
    Dense dq, dk, dv;
    int B, H, N;
    float c_log2, tau;
};
size_t ws_qat_bwd_bytes(int B, int H, int N, int d);
hipError_t launch_qat_bwd(QatBwdArgs a, Dense o_aux, void* ws, hipStream_t st);

// ---- ThriftAttention mixed prefill (attn_thrift.hip); head dimension 128, 128-token blocks
struct ThriftFwdArgs {
    const uint8_t* qc; const uint8_t* qs;                // MXFP4 Q [B,Hq,Nq,d/2], E8M0 [B,Hq,Nq,d/32]
    const uint8_t* kc; const uint8_t* ks;                // MXFP4 K [B,Hkv,Nk,d/2], E8M0 [B,Hkv,Nk,d/32]
    const uint8_t* vc; const uint8_t* vs;                // MXFP4 V [B,Hkv,d,Nk/2], E8M0 [B,Hkv,d,Nk/32]
    Dense q_hi, k_hi, v_hi;                              // bf16 Q, K, V [B,H,N,d]
    const int32_t* sel_idx; const int32_t* sel_cnt;      // [B,Hq,nqb,max_sel], [B,Hq,nqb]
    int max_sel;
    Dense o;                                             // O [B,Hq,Nq,d] bf16
    float* lse;                                          // [B,Hq,Nq] or null
    int B, Hq, Hkv, Nq, Nk, causal;
    float c_log2;                                        // tau * log2(e)
    const float* sbias;                                  // post-training baseline: [B,Hq,nqb,Nk] score shifts
    Dense q_nv, k_nv, v_nv;                              // NVFP4 emulation: dequantised NVFP4 Q, K, V (bf16)
};
hipError_t launch_thrift_fwd(const ThriftFwdArgs& a, hipStream_t st);
// post-training FP4 baseline: score shifts from qbar [B,Hq,nqb,d] into ws, then the FP4 path
size_t ws_ptq_fwd_bytes(int B, int Hq, int Nq, int Nk);
// Thrift prefill with the FP4 path in NVFP4 emulation (bf16 instructions on q_nv, k_nv, v_nv)
hipError_t launch_thrift_nv(const ThriftFwdArgs& a, hipStream_t st);
hipError_t launch_ptq_fwd(ThriftFwdArgs a, const float* qbar, void* ws, hipStream_t st);

// ---- ThriftAttention decode (attn_thrift.hip): one query per (batch, query head)
struct ThriftDecArgs {
    const uint8_t* qc; const uint8_t* qs;                // MXFP4 q [B,Hq,1,d/2], E8M0 [B,Hq,1,d/32]
    const uint8_t* kc; const uint8_t* ks;                // MXFP4 K cache [B,Hkv,Nk,d/2], E8M0
    const uint8_t* vc; const uint8_t* vs;                // MXFP4 V cache [B,Hkv,d,Nk/2], E8M0 [B,Hkv,d,Nk/32],
    int v_tiled;                                         // or blocked by 128 keys: [B,Hkv,Nk/128,d,64], [..,d,4]
    Dense q_hi, k_hi, v_hi;                              // bf16 q [B,Hq,1,d]; caches [B,Hkv,Nk,d]
    const int32_t* sel_idx; const int32_t* sel_cnt;      // [B,Hq,1,max_sel], [B,Hq,1]
    int max_sel;
    float* part;                                         // workspace: [B,Hq,splits,d+4] partials
    int B, Hq, Hkv, Nk, splits;
    float c_log2;
};
int decode_splits(int B, int Hkv, int Nk, int requested);
size_t ws_decode_bytes(int B, int Hq, int Hkv, int Nk, int requested);
hipError_t launch_thrift_decode(const ThriftDecArgs& a, Dense o, float* lse, hipStream_t st);
size_t decode_scratch_bytes();
hipError_t decode_scratch(float** out);    // this device's static partials array

// ---- ThriftAttention block selection (select.hip)
int select_sort_len(int nkb);
hipError_t launch_select(const float* qbar, const float* kbar, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                         int causal, int budget_ppm, int max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                         hipStream_t st);

// ---- BQA_DEBUG=1 input scan (debug.hip)
struct DebugInput {
    enum Kind { BF16 = 0, F16 = 1, F32 = 2 };
    const void* p;        // null: skipped
    int kind;
    int64_t sB, sH, sN;   // 16-bit [B, H, N, d] views: element strides
    int B, H, N, d;
    int64_t n;            // fp32 arrays: element count
};
bool debug_enabled();
int debug_scan(hipStream_t st, const DebugInput* in, int n_in);   // 1 found, 0 clean, -1 HIP error

// ---- rate probes (probe.hip); the kinds are the BQA_PROBE_* values of bqa.h
enum { PROBE_MFMA_I8 = 0, PROBE_MFMA_F8 = 1, PROBE_MFMA_F4 = 2, PROBE_MFMA_BF16 = 3, PROBE_EXP = 4, PROBE_COPY = 5,
       PROBE_READ = 6, PROBE_READ_NT = 7, PROBE_ISSUE_MFMA = 8, PROBE_ISSUE_FMA = 9, PROBE_ISSUE_MFMA_FMA = 10,
       PROBE_ISSUE_EXP = 11, PROBE_ISSUE_MFMA_EXP = 12, PROBE_OP_MUL = 13, PROBE_OP_FMA = 14,
       PROBE_OP_CVT_F32_I32 = 15, PROBE_OP_MAX3 = 16, PROBE_OP_CVT_PK_FP8 = 17, PROBE_OP_CVT_PK_FP4 = 18,
       PROBE_OP_PERMLANE32 = 19, PROBE_ISSUE_EXP_FMA = 20, PROBE_LDS_SHARED_ROWS = 21, PROBE_LDS_SPANS = 22 };
hipError_t launch_probe(int kind, int grid, int64_t iters, const void* src, void* dst, size_t bytes, hipStream_t st);

}  // namespace bqa
