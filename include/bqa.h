/*
 * bqa.h — C ABI of the block-quantized attention library (libbqa.so, gfx950).
 *
 * The library implements fused, tiled FlashAttention-style attention whose
 * matrix products run on block-quantized operands, in the three variants
 * described by the source pages:
 *
 *  - SageAttention / SageBwd ("SageBwd: A Trainable Low-bit Attention",
 *    Methodology items 1, 2 and 4): K-smoothing, per-block INT8 Q and K with
 *    exact int32 Q K^T, online softmax, low-bit P.V, and an INT8 backward
 *    that keeps the softmax-gradient product dP = dO V^T in 16-bit.
 *  - Attn-QAT ("Attn-QAT: 4-Bit Attention With Quantization-Aware Training",
 *    technical summary §2, Principles 1 and 2): FP4 forward that also emits a
 *    high-precision auxiliary output O', and a backward that recomputes P at
 *    the forward's FP4 precision and uses delta = rowsum(dO o O').
 *  - ThriftAttention ("ThriftAttention" technical summary, Method steps 1 and
 *    2): block-mean importance scores, top-k query/key block pairs computed in
 *    bf16 and the rest in FP4, merged by online softmax; prefill and decode.
 *
 * FP4 here is OCP MXFP4 (e2m1 values with one E8M0 power-of-two scale per 32
 * elements), which the gfx950 scaled matrix instructions consume; it stands
 * in for the pages' NVFP4.  The bf16 path stands in for the pages' FP16.
 *
 * Conventions
 *  - Every tensor pointer is a device pointer on the current HIP device.
 *    The caller allocates and owns every buffer, including the workspace
 *    sized by bqa_workspace_size(); the library never allocates memory and
 *    keeps no state between calls.
 *  - Every call validates all of its arguments on the host before anything is
 *    enqueued and returns a negative bqa_status on the first violation; then
 *    nothing has been launched and no output has been written.  On success the
 *    work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting for it.
 *  - Dense tensors are [B, H, N, d] with element strides given per dimension;
 *    the innermost stride must be 1, rows must start on 16-byte boundaries.
 *    Quantized tensors are contiguous in the layouts listed at bqa_qtensor.
 *  - Outputs are overwritten, never accumulated into.
 *  - Calls that overlap on one stream are ordered by the stream; the library
 *    itself holds no locks and is safe to call from several host threads.
 */
#ifndef BQA_H
#define BQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQA_ABI_VERSION 3

typedef int32_t bqa_status;
enum {
    BQA_OK = 0,
    BQA_E_NULL = -1,          /* a required pointer is NULL */
    BQA_E_SHAPE = -2,         /* inconsistent or out-of-range sizes */
    BQA_E_UNSUPPORTED = -3,   /* a valid request the library does not implement */
    BQA_E_ALIGN = -4,         /* misaligned pointer or stride, or inner stride != 1 */
    BQA_E_WORKSPACE = -5,     /* workspace pointer NULL or smaller than bqa_workspace_size() */
    BQA_E_DEVICE = -6,        /* the current device is not gfx950, or no device */
    BQA_E_LAUNCH = -7,        /* a kernel launch reported an error */
    BQA_E_NONFINITE = -8,     /* BQA_DEBUG=1: an input holds a NaN or an infinity */
    BQA_E_TOO_LARGE = -9      /* bqa_attn_decode_static: the partials exceed its static scratch */
};

typedef enum {
    BQA_BF16 = 0,
    BQA_FP16 = 1,
    BQA_INT8 = 2,             /* symmetric int8 codes, fp32 scales */
    BQA_FP8E4M3 = 3,          /* OCP e4m3 ("fn") codes, fp32 scales */
    BQA_MXFP4 = 4             /* packed e2m1 codes (even element in the low nibble), E8M0 scales */
} bqa_dtype;

typedef enum {
    BQA_SAGE_I8_F16PV = 0,    /* INT8 Q K^T, P and V in fp16 for P.V (V given as fp16) */
    BQA_SAGE_I8_F8PV = 1,     /* INT8 Q K^T, P = e4m3(448 P) and per-channel e4m3 V */
    BQA_SAGE_I8_I8PV = 2,     /* INT8 Q K^T, P int8 per (row, key tile), per-channel int8 V; trainable */
    BQA_QAT_MXFP4 = 3,        /* Attn-QAT: MXFP4 Q, K, P, V; optional bf16 auxiliary output O' */
    BQA_THRIFT = 4,           /* ThriftAttention: selected block pairs in bf16, the rest MXFP4 */
    BQA_PTQ_MXFP4 = 5         /* post-training FP4 baseline: smoothed MXFP4 Q, K; two-level P; MXFP4 V */
} bqa_mode;

typedef enum {
    BQA_ROLE_Q = 0,
    BQA_ROLE_K = 1,
    BQA_ROLE_V = 2,
    BQA_ROLE_DO = 3
} bqa_role;

/* The attention problem.  Fields that a mode does not use are ignored. */
typedef struct bqa_problem {
    int32_t B, Hq, Hkv;       /* batch, query heads, key/value heads (Hq % Hkv == 0) */
    int32_t Nq, Nk;           /* query and key lengths */
    int32_t d;                /* head dimension: 64 or 128 */
    int32_t causal;           /* 1: key j is visible to query i iff j <= i + (Nk - Nq) */
    float sm_scale;           /* softmax scale tau; <= 0 selects 1/sqrt(d) */
    int32_t mode;             /* bqa_mode */
    int32_t q_block;          /* INT8 token block of Q and dO (64 or 128; Sage modes) */
    int32_t k_block;          /* INT8 token block of K (64; Sage modes); also the key tile */
    int32_t smooth_k;         /* Sage: subtract the per-channel token-mean of K ... */
    float smooth_eps;         /* ... and add this constant back (K-smoothing) */
    int32_t hp_budget_ppm;    /* Thrift: share of valid block pairs kept in bf16, parts per million */
    int32_t sel_block;        /* Thrift: selection block (128) */
    int32_t num_splits;       /* Thrift decode: key-range splits merged at the end; 0 = automatic */
} bqa_problem;

/* A dense [B, H, N, d] tensor; stride[] in elements, stride[3] must be 1. */
typedef struct bqa_tensor {
    void* data;
    int32_t dtype;            /* bqa_dtype: BQA_BF16 or BQA_FP16 */
    int64_t stride[4];
} bqa_tensor;

/*
 * A quantized tensor, contiguous, in one of these layouts (H = Hq for Q and
 * dO, Hkv for K and V):
 *   INT8 / FP8E4M3, token blocks (Q, K, dO): codes int8 [B, H, N, d],
 *       scales fp32 [B, H, N / block]                         (axis 0)
 *   INT8 / FP8E4M3, per channel (V):         codes [B, H, d, N] (channel-major),
 *       scales fp32 [B, H, d]                                  (axis 1)
 *   MXFP4 along d (Q, K):      codes u8 [B, H, N, d / 2], scales u8 [B, H, N, d / 32]  (axis 0)
 *   MXFP4 along tokens (V):    codes u8 [B, H, d, N / 2], scales u8 [B, H, d, N / 32]  (axis 1)
 *   MXFP4 along tokens, blocked by 128 tokens (V of a decode cache):
 *       codes u8 [B, H, N / 128, d, 64], scales u8 [B, H, N / 128, d, 4]      (axis 2)
 * E8M0 scale bytes hold e + 127 for the power of two 2^e.
 */
typedef struct bqa_qtensor {
    int32_t fmt;              /* bqa_dtype: BQA_INT8, BQA_FP8E4M3 or BQA_MXFP4 */
    int32_t axis;             /* 0: blocks along tokens of rows / along d; 1: per channel / along tokens */
    int32_t block;            /* token block for INT8 axis 0; 32 for MXFP4; N for per-channel */
    void* codes;
    void* scales;
} bqa_qtensor;

/* Operations, for bqa_workspace_size(). */
enum {
    BQA_OP_QUANTIZE_Q = 0, BQA_OP_QUANTIZE_K = 1, BQA_OP_QUANTIZE_V = 2, BQA_OP_QUANTIZE_DO = 3,
    BQA_OP_SELECT = 4, BQA_OP_FWD = 5, BQA_OP_BWD = 6, BQA_OP_QUANTIZE_KV = 7, BQA_OP_QUANTIZE_NVFP4 = 8
};

/* ABI version of the loaded library (BQA_ABI_VERSION it was built with). */
int32_t bqa_abi_version(void);

/* Static description of a status code; never NULL. */
const char* bqa_status_string(bqa_status status);

/* Bytes of workspace the operation `op` needs for problem `p`; 0 when it needs
 * none or the problem is invalid. */
size_t bqa_workspace_size(const bqa_problem* p, int32_t op);

/*
 * Quantize one operand into `out` (whose fmt/axis/block select the format;
 * codes and scales must be allocated by the caller in the layout above).
 *
 *  - Q, dO, INT8 axis 0: per token block of out->block tokens, scale =
 *    amax/127 and code = round-half-even(x * (127/amax)) clamped to +-127,
 *    both divisions correctly rounded in fp32 ("SageBwd", Methodology 1:
 *    per-block INT8).  V with INT8 axis 0 (block 64) is quantised the same
 *    way, for the fully INT8 backward of bqa_attn_bwd.
 *  - K, INT8 axis 0 with p->smooth_k: K-smoothing ("SageBwd", Methodology 4
 *    and Results): mu = fp32(sum_t K / N - eps) per (b, h, channel), summed
 *    in fp64, written to k_mean [B, Hkv, d] when k_mean is not NULL; the codes
 *    are those of fp32(K - mu).
 *  - V, INT8 or FP8E4M3 axis 1: one scale per (b, h, channel) over all tokens,
 *    amax/127 or amax/448; e4m3 codes round to nearest even and saturate.
 *  - Q, K, MXFP4 axis 0; V, MXFP4 axis 1 or 2: OCP MX blocks of 32 along d
 *    (Q, K) or along tokens (V) ("Attn-QAT", §1 Problem: FP4 has 15 values;
 *    "ThriftAttention", Method step 2: micro-scaled FP4): X = 2^e with
 *    e = floor(log2 amax) - 2 clamped to [-127, 127], codes e2m1(x / X),
 *    nearest-even, saturating at 6.  With block_means != NULL and role Q or K
 *    the means over each p->sel_block tokens are written as fp32
 *    [B, H, N / sel_block, d] ("ThriftAttention", Method step 1).
 *  - BQA_PTQ_MXFP4, Q and K (MXFP4 axis 0, d = 128): the smoothing of the
 *    post-training FP4 method that Attn-QAT is compared with ("Attn-QAT",
 *    technical summary §1 and §2 Implementation: SageAttention3-style Q/K
 *    smoothing).  Q: per block of 128 rows (the last may be short) the mean
 *    of its rows, summed in fp64, rounded to fp32 and then to bf16, is written
 *    to block_means (required, fp32 [B, Hq, ceil(Nq / 128), d], 16-byte
 *    aligned) and the codes are those of fp32(Q - mean).  K with
 *    p->smooth_k: mu = fp32(sum_t K / N - eps) as for the Sage modes, to
 *    k_mean when not NULL, codes of fp32(K - mu); workspace
 *    bqa_workspace_size(p, BQA_OP_QUANTIZE_K) bytes.  V as for MXFP4 V.
 *  A block whose amax is 0 (or whose inverse scale overflows fp32) gets
 *  scale 0 and all-zero codes.
 * `x` is [B, H, N, d] bf16 (fp16 for Q, K, V allowed in BQA_SAGE_I8_F16PV).
 */
bqa_status bqa_quantize_blocks(const bqa_problem* p, int32_t role, const bqa_tensor* x,
                               bqa_qtensor* out, float* k_mean, float* block_means,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * K and V of the Sage fp8 / int8 P.V modes in one call: the same codes,
 * scales and k_mean as bqa_quantize_blocks for role K (INT8 token blocks of
 * 64 tokens, K-smoothing per p->smooth_k and p->smooth_eps) and role V
 * (per-channel e4m3 for BQA_SAGE_I8_F8PV, int8 for BQA_SAGE_I8_I8PV).  With
 * d = 128, Nk a multiple of 256, a grid of B Hkv Nk / 256 workgroups that the
 * device holds at once and a stream that is not being captured, this is one
 * kernel launch that reads K and V once (the workgroups of a head exchange
 * their partial sums and maxima through the workspace); otherwise two
 * launches (the K token sums and the V channel maxima, then both encodings).
 * Either way the bytes equal those of the per-operand calls.  k and v are
 * [B, Hkv, Nk, d] of one dtype (bf16 or fp16); kq is INT8 axis 0 with block
 * 64, vq the per-channel layout with block Nk; Nk a multiple of 64.
 * Workspace: bqa_workspace_size(p, BQA_OP_QUANTIZE_KV) bytes, 16-byte
 * aligned, contents on entry arbitrary; two calls that run at the same time
 * must not share it.
 */
bqa_status bqa_quantize_kv(const bqa_problem* p, const bqa_tensor* k, const bqa_tensor* v, bqa_qtensor* kq,
                           bqa_qtensor* vq, float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/*
 * QK-norm fused into the INT8 quantisation ("SageBwd", Methodology 4 and the
 * recommended SageBwd + QK-norm + K-smoothing recipe): the raw rows x of Q
 * or K (bf16 or fp16, d = 128, a Sage mode) are scaled to unit L2 norm,
 * y = bf16(fp32(x r)) with r = fp32(1/sqrt(S)) from the fp64 sum of squares
 * S (r = 0 for a zero row), and y is quantised exactly as
 * bqa_quantize_blocks quantises its input for the same role: INT8 token
 * blocks of out->block (64 or 128) tokens; for K with p->smooth_k the
 * smoothing mean is taken over the normalised rows (to k_mean when not
 * NULL; workspace bqa_workspace_size(p, BQA_OP_QUANTIZE_K) bytes).  One pass
 * over x replaces a normalisation pass and the quantiser's read of its
 * output.  inv_norm (fp32 [B, H, N], required) receives r of every row, for
 * bqa_attn_bwd_qknorm.
 */
bqa_status bqa_quantize_qknorm(const bqa_problem* p, int32_t role, const bqa_tensor* x, bqa_qtensor* out,
                               float* inv_norm, float* k_mean, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * NVFP4 format emulation ("ThriftAttention", Method step 2: the FP4 path of
 * the pages uses NVFP4 micro-scaling, e2m1 values in blocks of 16 with an
 * E4M3 scale; gfx950's scaled matrix instructions take only power-of-two
 * scales, so NVFP4 is emulated).  x (Q: [B, Hq, Nq, d]; K, V: [B, Hkv, Nk,
 * d], bf16 or fp16, d = 128) is quantised to NVFP4 and the dequantised
 * values, exact in bf16, are written to out (bf16, same shape): per (b, h)
 * slice a tensor scale g, the power of two at or above amax / (448 * 6);
 * blocks of 16 along d (Q, K) or along the tokens of each channel (V, Nk a
 * multiple of 32) with the scale s_b = e4m3(fp32(amax_b / (6 g))) and
 * values e2m1(fp32(x / (s_b g))) s_b g (nearest-even, saturating).
 * Workspace: bqa_workspace_size(p, BQA_OP_QUANTIZE_NVFP4) bytes.
 */
bqa_status bqa_quantize_nvfp4(const bqa_problem* p, int32_t role, const bqa_tensor* x, bqa_tensor* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * ThriftAttention prefill (as bqa_attn_fwd in BQA_THRIFT mode, Nq > 1) with
 * its FP4 path in NVFP4 emulation: the unselected valid blocks run the bf16
 * matrix instructions on q_nv, k_nv, v_nv (from bqa_quantize_nvfp4) with P
 * quantised in two levels to NVFP4 (the row's largest P of the 64-key tile
 * scaled to 448 * 6, E4M3 scales per 16 keys, e2m1 values, the first level
 * undone into the bf16 operand); the selected blocks then run through the
 * bf16 path on q_hi, k_hi, v_hi; all in tiles of 64 keys merged by one
 * online softmax.  For measuring the pages' numerics, not their speed.
 */
bqa_status bqa_attn_fwd_thrift_nvfp4(const bqa_problem* p, const bqa_tensor* q_nv, const bqa_tensor* k_nv,
                                     const bqa_tensor* v_nv, const bqa_tensor* q_hi, const bqa_tensor* k_hi,
                                     const bqa_tensor* v_hi, const int32_t* sel_idx, const int32_t* sel_cnt,
                                     bqa_tensor* o, float* lse, void* stream);

/*
 * ThriftAttention block selection ("ThriftAttention", Method step 1): for
 * every (b, query head h, query block i) the importance of key block j is
 * qbar_i . kbar_j (kbar of KV head h / (Hq/Hkv)) over the valid key blocks
 * (causal: j <= i + nkb - nqb); the k_i = max(1, ceil(n_valid * budget))
 * highest-scoring blocks (equal scores: smaller j first) are written to
 * sel_idx [B, Hq, nqb, max_sel] in ascending order, unused slots -1, and k_i
 * to sel_cnt [B, Hq, nqb].  q_means [B, Hq, nqb, d], k_means [B, Hkv, nkb, d]
 * are fp32 block means; nqb = ceil(Nq / sel_block) (a decode query is its own
 * block), nkb = Nk / sel_block; max_sel = max(1, ceil(nkb * budget)).  A
 * causal prefill needs Nq a multiple of sel_block (BQA_E_UNSUPPORTED
 * otherwise): the block-level mask is defined for whole query blocks.
 */
bqa_status bqa_select_blocks(const bqa_problem* p, const float* q_means, const float* k_means,
                             int32_t* sel_idx, int32_t* sel_cnt,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention forward.  Output o [B, Hq, Nq, d] (bf16; fp16 in
 * BQA_SAGE_I8_F16PV) and, when lse is not NULL, the natural-log
 * log-sum-exp of every row, fp32 [B, Hq, Nq].
 *
 * Every mode runs FlashAttention-2's online softmax ("ThriftAttention",
 * Method step 2): keys are visited in tiles in a fixed order, the running
 * row maximum m is updated per tile, P = exp(s - m) is rounded for P.V as the
 * mode says (the row's largest P so far is 1, exactly representable in every
 * P format), the sums gathered before are scaled by exp(m_old - m_new), and
 * the row sum accumulates the unrounded P.
 *
 *  - Sage modes ("SageBwd", Methodology 1): q, k are the INT8 token-block
 *    codes (k of the smoothed K); v is per-channel e4m3 (F8PV) or int8
 *    (I8PV) codes, or for F16PV v_hi holds V in fp16 and v is unused.  In
 *    F8PV, q_hi (bf16 [B, Hq, Nq, d]) may be given instead: the kernel then
 *    quantises Q itself, with the codes and scales bqa_quantize_blocks gives
 *    for role Q, and writes them to q's buffers when q is not NULL (q may be
 *    NULL).
 *    Key tiles of k_block, ascending (causal: up to the row's diagonal).
 *  - BQA_QAT_MXFP4 ("Attn-QAT", §2): q, k MXFP4 along d, v MXFP4 along tokens;
 *    d = 128, non-causal, Nk a multiple of 128.  Key tiles of 128, ascending;
 *    P is made MXFP4 per 32 keys of the row for O (no smoothing or two-level
 *    step, §2 Implementation).  When o_aux is not NULL, O' = sum bf16(P) V / l
 *    is written too (Principle 2); this needs a workspace of
 *    bqa_workspace_size(p, BQA_OP_FWD) bytes (a bf16 copy of the dequantised
 *    V), else none.  When row_max is not NULL it receives the largest raw
 *    score q^.k^ (before the softmax scale) of every row, fp32 [B, Hq, Nq]:
 *    the backward rounds P against it.
 *  - BQA_THRIFT ("ThriftAttention", Method step 2 and kernel paragraph): per
 *    query block, the unselected valid key blocks go through the FP4 path
 *    (MXFP4 q, k, v; P quantised in two levels: scaled so its row max is 6,
 *    then MXFP4 per 32 keys), then the selected blocks (sel_idx, sel_cnt from
 *    bqa_select_blocks) through the bf16 path (q_hi, k_hi, v_hi), all merged
 *    by one online softmax.  Nq == 1 is decode: the key range is cut into
 *    p->num_splits parts whose partial results are merged at the end; its v
 *    may also be blocked by 128 tokens (axis 2), which lets each key
 *    block's V be read as one contiguous stretch.
 * row_max is used by BQA_QAT_MXFP4 only (NULL elsewhere).
 */
bqa_status bqa_attn_fwd(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                        const bqa_qtensor* v, const bqa_tensor* q_hi, const bqa_tensor* k_hi,
                        const bqa_tensor* v_hi, const int32_t* sel_idx, const int32_t* sel_cnt,
                        bqa_tensor* o, bqa_tensor* o_aux, float* lse, float* row_max,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Post-training FP4 attention in the SageAttention3 style, the baseline the
 * Attn-QAT pages compare against ("Attn-QAT", technical summary §1: PTQ with
 * Q/K smoothing and two-level quantisation; the two-level step as in
 * "ThriftAttention", Method step 2).  p->mode must be BQA_PTQ_MXFP4; d = 128,
 * Nk a multiple of 128; causal allowed (bottom-right); Hq a multiple of Hkv.
 * q, k: the MXFP4 codes bqa_quantize_blocks writes for the smoothed Q and K;
 * q_means: the bf16 block means it wrote for Q (fp32 [B, Hq, ceil(Nq/128), d],
 * 16-byte aligned); v: MXFP4 along tokens.  The score of query row i in
 * block I against key j is tau (q^_i . k^_j + qbar_I . k^_j): the smoothed
 * product on the scaled FP4 matrix instructions plus the block mean's
 * product with the dequantised key (bf16 products, fp32 sums, computed once
 * per call into the workspace).  Keys are visited in blocks of 128 in
 * ascending order; in each block P is quantised in two levels (scaled so the
 * row's largest P in the block is 6, then MXFP4 per 32 keys, the factor
 * undone in fp32) and merged by FlashAttention-2's online softmax.  Output
 * o [B, Hq, Nq, d] bf16; lse (fp32 [B, Hq, Nq]) when not NULL.  Workspace:
 * bqa_workspace_size(p, BQA_OP_FWD) = B Hq ceil(Nq/128) Nk 4 bytes, 16-byte
 * aligned; two calls that run at the same time must not share it.
 */
bqa_status bqa_attn_fwd_ptq(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                            const bqa_qtensor* v, const float* q_means, bqa_tensor* o, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * ThriftAttention decode for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and arguments as bqa_attn_fwd in BQA_THRIFT mode with
 * Nq == 1, without a workspace.  The per-split partial results live in a
 * static 16 MiB device array of the library (one per device, held until the
 * process ends); calls that would need more, B * Hq * splits * (d + 4) * 4
 * bytes > 16 MiB, return BQA_E_TOO_LARGE and launch nothing.  Every call on
 * a device shares that array: calls that overlap on one device (several
 * streams or host threads) race and must be serialised by the caller.  No
 * memory is allocated or freed by this call.
 */
bqa_status bqa_attn_decode_static(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                                  const bqa_qtensor* v, const bqa_tensor* q_hi, const bqa_tensor* k_hi,
                                  const bqa_tensor* v_hi, const int32_t* sel_idx, const int32_t* sel_cnt,
                                  bqa_tensor* o, float* lse, void* stream);

/*
 * Attention backward: dq, dk, dv [B, H, N, d] bf16 from the forward's codes,
 * its lse and d_o.
 *  - Sage modes ("SageBwd", Methodology 2, Limitations): d = 128,
 *    Hq == Hkv, Nq == Nk a multiple of 128, q_block 128, k_block 64.  delta =
 *    rowsum(dO o O) with o_for_delta = the forward's O; dO is quantized to
 *    INT8 per 128 tokens; tiles of 128 queries x 64 keys; P and dS are
 *    INT8 with one scale per tile; dV = P^T dO, dQ = tau dS K and
 *    dK = tau dS^T Q run as INT8 products, dP = dO V^T in bf16 from v_hi
 *    (bf16).  With v given (INT8 axis 0, block 64: V's token-block codes
 *    from bqa_quantize_blocks) dP runs in INT8 as well, the dO codes against
 *    the V codes times both scales: the fully INT8 backward the page's
 *    Limitations leave open (v_hi is still validated and read for nothing
 *    else; it may be the same V).  Otherwise v is unused.  Workspace:
 *    bqa_workspace_size(p, BQA_OP_BWD) bytes.
 *  - BQA_QAT_MXFP4 ("Attn-QAT", §2 Principles 1 and 2): o_for_delta = O';
 *    d = 128, Hq == Hkv, Nq == Nk a multiple of 128, non-causal.  P is
 *    recomputed from the same FP4 scores; for dV it is rounded at the
 *    forward's precision: MXFP4 per 32 keys of exp(s - M), M the row's
 *    maximum from the forward's row_max (required here), then scaled to
 *    exp(s - L); dS = P o (dP - delta) uses the unrounded P and is rounded to
 *    bf16; dP, dQ, dK run in bf16 against the FP4 operands; delta =
 *    rowsum(dO o O').  Workspace: bqa_workspace_size(p, BQA_OP_BWD) bytes.
 * row_max is used by BQA_QAT_MXFP4 only (NULL elsewhere).
 */
bqa_status bqa_attn_bwd(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                        const bqa_qtensor* v, const bqa_tensor* v_hi,
                        const bqa_tensor* o_for_delta, const float* lse, const float* row_max,
                        const bqa_tensor* d_o,
                        bqa_tensor* dq, bqa_tensor* dk, bqa_tensor* dv,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The SageBwd backward of bqa_attn_bwd (same arguments, requirements and
 * workspace) for a forward whose Q and K came from bqa_quantize_qknorm: the
 * QK-norm backward is applied in the dQ and dK epilogues, so dq and dk are
 * the gradients with respect to the raw rows: dx = r (g - y (y . g)) with
 * g the gradient with respect to the normalised row, y = x r (the bf16
 * rounding of the forward passed straight through).  K-smoothing adds no
 * term: its mean enters every score of a query row equally, and the key
 * gradients it would add sum, over all keys, to zero in exact arithmetic
 * (each query's dS row sums to zero).  q_raw, k_raw: the raw bf16 rows;
 * q_inv_norm, k_inv_norm: the r that bqa_quantize_qknorm wrote.
 */
bqa_status bqa_attn_bwd_qknorm(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                               const bqa_tensor* v_hi, const bqa_tensor* o_for_delta, const float* lse,
                               const bqa_tensor* d_o, const bqa_tensor* q_raw, const bqa_tensor* k_raw,
                               const float* q_inv_norm, const float* k_inv_norm, bqa_tensor* dq, bqa_tensor* dk,
                               bqa_tensor* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hook: the raw Q K^T accumulator of one tile as the forward kernel's
 * matrix-instruction code computes it — int32 [32 x 32] for INT8 codes
 * (exact integer dot products) or fp32 [32 x 32] for MXFP4 codes (the
 * instruction's fp32 result, before tau) — for query rows q_tile*32 .. +31
 * and key rows k_tile*32 .. +31 of (b, h), written row-major to out.
 */
bqa_status bqa_debug_qk_scores(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                               int32_t b, int32_t h, int32_t q_tile, int32_t k_tile, void* out,
                               void* stream);

/*
 * Test hook: the MXFP4 -> bf16 conversion that the Attn-QAT forward uses for
 * the bf16 copy of deq(V) behind O' and the backward for its bf16 operands
 * ("Attn-QAT", §2 Principle 2): nblocks blocks of 32 e2m1 values (16 code
 * bytes each, low nibble first, 16-byte aligned) with one E8M0 byte each
 * (scales[i]) to 32 bf16 values each (out, 16-byte aligned).  Every e2m1
 * value times 2^e that is a finite bf16 value is exact.
 */
bqa_status bqa_debug_mx_dequant(const void* codes, const void* scales, int64_t nblocks, void* out, void* stream);

/*
 * Measurement hook: rate probes for the roofline's denominators.  Each runs
 * `grid` workgroups of 256 threads and is timed by the caller (events on
 * `stream`).  Matrix probes: every wavefront issues iters x 8 dense matrix
 * instructions of one type on register operands (4 independent accumulator
 * chains): BQA_PROBE_MFMA_I8 (32x32x32 int8, 65536 ops each),
 * BQA_PROBE_MFMA_F8 (32x32x64 e4m3, 131072), BQA_PROBE_MFMA_F4 (32x32x64
 * scaled e2m1, 131072), BQA_PROBE_MFMA_BF16 (32x32x16 bf16, 32768).
 * BQA_PROBE_EXP: every thread runs iters x 8 v_exp_f32.  These write one
 * checksum word per workgroup to dst (bytes >= 4 grid, 4-byte aligned; src
 * unused).  BQA_PROBE_COPY: copies `bytes` (a multiple of 16, both pointers
 * 16-byte aligned) from src to dst with 16-byte accesses; iters unused.
 * BQA_PROBE_READ: reads `bytes` (a multiple of 16, src 16-byte aligned) with
 * 16-byte accesses and writes one checksum word per workgroup to dst (dst
 * 4-byte aligned and holding grid words, which the caller sizes: `bytes`
 * describes src here); BQA_PROBE_READ_NT the same with the non-temporal
 * cache policy.  Issue
 * probes (src unused, one checksum word per workgroup to dst, bytes >= 4
 * grid): every wavefront runs iters rounds of 8 int8 32x32x32 matrix
 * instructions (BQA_PROBE_ISSUE_MFMA), 64 fp32 fused multiply-adds
 * (BQA_PROBE_ISSUE_FMA), 32 v_exp_f32 (BQA_PROBE_ISSUE_EXP), or the matrix
 * instructions interleaved with the multiply-adds (BQA_PROBE_ISSUE_MFMA_FMA)
 * or with the exponentials (BQA_PROBE_ISSUE_MFMA_EXP).  Instruction probes
 * (same arguments): every lane runs iters rounds of 64 instances of one
 * vector instruction over 16 independent chains: fp32 multiply
 * (BQA_PROBE_OP_MUL), fused multiply-add (BQA_PROBE_OP_FMA), int->float
 * conversion (BQA_PROBE_OP_CVT_F32_I32), v_max3_f32 (BQA_PROBE_OP_MAX3), the
 * packed fp8 conversion (BQA_PROBE_OP_CVT_PK_FP8), the scaled packed fp4
 * conversion (BQA_PROBE_OP_CVT_PK_FP4), v_permlane32_swap
 * (BQA_PROBE_OP_PERMLANE32).  BQA_PROBE_ISSUE_EXP_FMA (same arguments): the
 * 64 multiply-adds and the 32 v_exp_f32 of a round interleaved, on chains of
 * their own.  LDS read probes (same arguments): every wavefront runs iters
 * rounds of 8 back-to-back 16-byte LDS reads; lane 16 g + q reads entry q of
 * its group's own 256-byte span (BQA_PROBE_LDS_SPANS) or chunk g ^ (q / 4) of
 * the 64-byte row q, the four groups sharing the rows
 * (BQA_PROBE_LDS_SHARED_ROWS).
 */
enum {
    BQA_PROBE_MFMA_I8 = 0, BQA_PROBE_MFMA_F8 = 1, BQA_PROBE_MFMA_F4 = 2, BQA_PROBE_MFMA_BF16 = 3,
    BQA_PROBE_EXP = 4, BQA_PROBE_COPY = 5, BQA_PROBE_READ = 6, BQA_PROBE_READ_NT = 7,
    BQA_PROBE_ISSUE_MFMA = 8, BQA_PROBE_ISSUE_FMA = 9, BQA_PROBE_ISSUE_MFMA_FMA = 10, BQA_PROBE_ISSUE_EXP = 11,
    BQA_PROBE_ISSUE_MFMA_EXP = 12, BQA_PROBE_OP_MUL = 13, BQA_PROBE_OP_FMA = 14, BQA_PROBE_OP_CVT_F32_I32 = 15,
    BQA_PROBE_OP_MAX3 = 16, BQA_PROBE_OP_CVT_PK_FP8 = 17, BQA_PROBE_OP_CVT_PK_FP4 = 18, BQA_PROBE_OP_PERMLANE32 = 19,
    BQA_PROBE_ISSUE_EXP_FMA = 20, BQA_PROBE_LDS_SHARED_ROWS = 21, BQA_PROBE_LDS_SPANS = 22
};
bqa_status bqa_debug_probe(int32_t kind, int32_t grid, int64_t iters, const void* src, void* dst, size_t bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BQA_H */
