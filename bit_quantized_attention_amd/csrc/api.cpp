// api.cpp — the C ABI declared in include/bqa.h: argument validation (host
// only, before anything touches the device), the once-per-device gfx950
// check, workspace sizing and dispatch to the kernels' launchers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "bqa.h"
#include "internal.hpp"

using namespace bqa;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

bqa_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BQA_E_DEVICE;
    if (dev >= kMaxDevices) return BQA_E_DEVICE;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BQA_E_DEVICE;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? BQA_OK : BQA_E_DEVICE;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// dense [B, H, N, d] half-precision tensor
bqa_status check_dense(const bqa_tensor* t, bool allow_f16, bool allow_bf16) {
    if (!t || !t->data) return BQA_E_NULL;
    if (!((t->dtype == BQA_BF16 && allow_bf16) || (t->dtype == BQA_FP16 && allow_f16))) return BQA_E_UNSUPPORTED;
    if (t->stride[3] != 1) return BQA_E_ALIGN;
    if (!aligned16(t->data)) return BQA_E_ALIGN;
    for (int i = 0; i < 3; ++i)
        if (t->stride[i] < 0 || (t->stride[i] * 2) % 16 != 0) return BQA_E_ALIGN;
    return BQA_OK;
}

Dense as_dense(const bqa_tensor* t) { return Dense{t->data, t->stride[0], t->stride[1], t->stride[2]}; }

bqa_status check_problem(const bqa_problem* p) {
    if (!p) return BQA_E_NULL;
    if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Nq < 1 || p->Nk < 1) return BQA_E_SHAPE;
    if (p->Hq % p->Hkv != 0) return BQA_E_SHAPE;
    if (p->d != 64 && p->d != 128) return BQA_E_UNSUPPORTED;
    if (p->mode < BQA_SAGE_I8_F16PV || p->mode > BQA_PTQ_MXFP4) return BQA_E_UNSUPPORTED;
    if (p->causal && p->Nq > p->Nk) return BQA_E_SHAPE;
    if ((int64_t)p->B * p->Hq * p->Nq * p->d > ((int64_t)1 << 40)) return BQA_E_SHAPE;
    return BQA_OK;
}

bool is_sage(int mode) { return mode == BQA_SAGE_I8_F16PV || mode == BQA_SAGE_I8_F8PV || mode == BQA_SAGE_I8_I8PV; }

bqa_status check_sage_blocks(const bqa_problem* p) {
    if (p->q_block != 64 && p->q_block != 128) return BQA_E_UNSUPPORTED;
    if (p->k_block != 64) return BQA_E_UNSUPPORTED;
    if (p->Nq % p->q_block != 0 || p->Nk % p->k_block != 0) return BQA_E_UNSUPPORTED;
    return BQA_OK;
}

bqa_status check_q(const bqa_qtensor* q, int fmt, int axis) {
    if (!q || !q->codes || !q->scales) return BQA_E_NULL;
    if (q->fmt != fmt || q->axis != axis) return BQA_E_UNSUPPORTED;
    if (!aligned16(q->codes)) return BQA_E_ALIGN;
    if (fmt != BQA_MXFP4 && ((uintptr_t)q->scales & 3u)) return BQA_E_ALIGN;
    return BQA_OK;
}

// slots per query block in sel_idx: max(1, ceil(nkb * budget)), at most nkb
int max_sel_of(const bqa_problem* p) {
    const int nkb = p->Nk / p->sel_block;
    int64_t k = ((int64_t)nkb * p->hp_budget_ppm + 999999) / 1000000;
    if (k < 1) k = 1;
    if (k > nkb) k = nkb;
    return (int)k;
}

float tau_of(const bqa_problem* p) { return p->sm_scale > 0.0f ? p->sm_scale : 1.0f / std::sqrt((float)p->d); }

bqa_status launched(hipError_t e) { return e == hipSuccess ? BQA_OK : BQA_E_LAUNCH; }

#define TRY(x)                           \
    do {                                 \
        bqa_status _s = (x);             \
        if (_s != BQA_OK) return _s;     \
    } while (0)

// Validation and argument block of a ThriftAttention decode call (everything
// but the partials buffer).
bqa_status check_decode(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k, const bqa_qtensor* v,
                        const bqa_tensor* q_hi, const bqa_tensor* k_hi, const bqa_tensor* v_hi,
                        const int32_t* sel_idx, const int32_t* sel_cnt, const bqa_tensor* o, ThriftDecArgs& a) {
    if (p->mode != BQA_THRIFT || p->Nq != 1) return BQA_E_UNSUPPORTED;
    if (p->d != 128 || p->sel_block != 128 || p->Nk % 128 != 0) return BQA_E_UNSUPPORTED;
    if (p->Hq / p->Hkv > 32) return BQA_E_UNSUPPORTED;
    if (p->num_splits < 0) return BQA_E_SHAPE;
    TRY(check_q(q, BQA_MXFP4, 0));
    TRY(check_q(k, BQA_MXFP4, 0));
    TRY(check_q(v, BQA_MXFP4, v && v->axis == 2 ? 2 : 1));
    if (q->block != 32 || k->block != 32 || v->block != 32) return BQA_E_UNSUPPORTED;
    TRY(check_dense(q_hi, false, true));
    TRY(check_dense(k_hi, false, true));
    TRY(check_dense(v_hi, false, true));
    TRY(check_dense(o, false, true));
    if (!sel_idx || !sel_cnt) return BQA_E_NULL;
    if (p->hp_budget_ppm < 0 || p->hp_budget_ppm > 1000000) return BQA_E_SHAPE;
    a.v_tiled = v->axis == 2;
    a.qc = (const uint8_t*)q->codes; a.qs = (const uint8_t*)q->scales;
    a.kc = (const uint8_t*)k->codes; a.ks = (const uint8_t*)k->scales;
    a.vc = (const uint8_t*)v->codes; a.vs = (const uint8_t*)v->scales;
    a.q_hi = as_dense(q_hi); a.k_hi = as_dense(k_hi); a.v_hi = as_dense(v_hi);
    a.sel_idx = sel_idx; a.sel_cnt = sel_cnt; a.max_sel = max_sel_of(p);
    a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nk = p->Nk;
    a.splits = decode_splits(p->B, p->Hkv, p->Nk, p->num_splits);
    a.c_log2 = tau_of(p) * 1.4426950408889634f;
    return BQA_OK;
}

// Validation and argument block of a SageBwd backward call.
bqa_status check_sage_bwd(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k, const bqa_tensor* v_hi,
                          const bqa_tensor* o_for_delta, const float* lse, const bqa_tensor* d_o, const bqa_tensor* dq,
                          const bqa_tensor* dk, const bqa_tensor* dv, const void* ws, size_t ws_bytes,
                          SageBwdArgs& a) {
    if (p->d != 128 || p->Hq != p->Hkv || p->Nq != p->Nk || p->Nq % 128 != 0) return BQA_E_UNSUPPORTED;
    if (p->q_block != 128 || p->k_block != 64) return BQA_E_UNSUPPORTED;
    TRY(check_q(q, BQA_INT8, 0));
    TRY(check_q(k, BQA_INT8, 0));
    if (q->block != 128 || k->block != 64) return BQA_E_UNSUPPORTED;
    TRY(check_dense(v_hi, false, true));
    TRY(check_dense(o_for_delta, false, true));
    TRY(check_dense(d_o, false, true));
    TRY(check_dense(dq, false, true));
    TRY(check_dense(dk, false, true));
    TRY(check_dense(dv, false, true));
    if (!lse) return BQA_E_NULL;
    if (!ws || ws_bytes < ws_sage_bwd_bytes(p->B, p->Hq, p->Nq, p->d)) return BQA_E_WORKSPACE;
    if (!aligned16(ws) || ((uintptr_t)lse & 15u)) return BQA_E_ALIGN;
    a.qc = (const int8_t*)q->codes; a.qs = (const float*)q->scales;
    a.kc = (const int8_t*)k->codes; a.ks = (const float*)k->scales;
    a.v = as_dense(v_hi); a.d_o = as_dense(d_o); a.lse = lse;
    a.dq = as_dense(dq); a.dk = as_dense(dk); a.dv = as_dense(dv);
    a.B = p->B; a.H = p->Hq; a.N = p->Nq; a.causal = p->causal;
    a.tau = tau_of(p);
    a.c_log2 = a.tau * 1.4426950408889634f;
    return BQA_OK;
}

// BQA_DEBUG=1: scan the call's floating-point inputs before it launches.
DebugInput dbg16(const bqa_tensor* t, int B, int H, int N, int d) {
    if (!t) return DebugInput{nullptr, DebugInput::BF16, 0, 0, 0, 0, 0, 0, 0, 0};
    return DebugInput{t->data, t->dtype == BQA_FP16 ? DebugInput::F16 : DebugInput::BF16, t->stride[0], t->stride[1],
                      t->stride[2], B, H, N, d, 0};
}
DebugInput dbg32(const float* p, int64_t n) { return DebugInput{p, DebugInput::F32, 0, 0, 0, 0, 0, 0, 0, n}; }

bqa_status debug_check(void* stream, std::initializer_list<DebugInput> in) {
    if (!debug_enabled()) return BQA_OK;
    TRY(check_device());
    const int r = debug_scan((hipStream_t)stream, in.begin(), (int)in.size());
    return r < 0 ? BQA_E_LAUNCH : (r > 0 ? BQA_E_NONFINITE : BQA_OK);
}

}  // namespace

extern "C" {

int32_t bqa_abi_version(void) { return BQA_ABI_VERSION; }

const char* bqa_status_string(bqa_status s) {
    switch (s) {
        case BQA_OK: return "ok";
        case BQA_E_NULL: return "a required pointer is NULL";
        case BQA_E_SHAPE: return "inconsistent or out-of-range sizes";
        case BQA_E_UNSUPPORTED: return "unsupported combination of mode, format or sizes";
        case BQA_E_ALIGN: return "misaligned pointer or stride, or inner stride != 1";
        case BQA_E_WORKSPACE: return "workspace missing or too small";
        case BQA_E_DEVICE: return "current device is not gfx950 (MI355X) or no device";
        case BQA_E_LAUNCH: return "kernel launch failed";
        case BQA_E_NONFINITE: return "an input holds a NaN or an infinity (BQA_DEBUG=1 scan)";
        case BQA_E_TOO_LARGE: return "request exceeds the static scratch of the allocation-free entry point";
        default: return "unknown status";
    }
}

size_t bqa_workspace_size(const bqa_problem* p, int32_t op) {
    if (check_problem(p) != BQA_OK) return 0;
    switch (op) {
        case BQA_OP_QUANTIZE_K:
            if ((is_sage(p->mode) || p->mode == BQA_PTQ_MXFP4) && p->smooth_k)
                return ws_kmean_bytes(p->B * p->Hkv, p->Nk, p->d);
            return 0;
        case BQA_OP_QUANTIZE_V:
            if (p->mode == BQA_SAGE_I8_F8PV || p->mode == BQA_SAGE_I8_I8PV) return ws_chan_bytes(p->B * p->Hkv, p->Nk, p->d);
            return 0;
        case BQA_OP_QUANTIZE_KV:
            if (p->mode == BQA_SAGE_I8_F8PV || p->mode == BQA_SAGE_I8_I8PV) return ws_kv_bytes(p->B * p->Hkv, p->Nk, p->d);
            return 0;
        case BQA_OP_BWD:
            if (is_sage(p->mode) && p->Nq == p->Nk) return ws_sage_bwd_bytes(p->B, p->Hq, p->Nq, p->d);
            if (p->mode == BQA_QAT_MXFP4 && p->Nq == p->Nk) return ws_qat_bwd_bytes(p->B, p->Hq, p->Nq, p->d);
            return 0;
        case BQA_OP_FWD:
            if (p->mode == BQA_QAT_MXFP4) return ws_qat_fwd_bytes(p->B, p->Hkv, p->Nk, p->d);
            if (p->mode == BQA_THRIFT && p->Nq == 1 && p->Nk % 128 == 0)
                return ws_decode_bytes(p->B, p->Hq, p->Hkv, p->Nk, p->num_splits);
            if (p->mode == BQA_PTQ_MXFP4) return ws_ptq_fwd_bytes(p->B, p->Hq, p->Nq, p->Nk);
            return 0;
        case BQA_OP_QUANTIZE_NVFP4: {
            const size_t a = ws_nvfp4_bytes(p->B * p->Hq, p->Nq, p->d), b = ws_nvfp4_bytes(p->B * p->Hkv, p->Nk, p->d);
            return a > b ? a : b;
        }
        default:
            return 0;
    }
}

bqa_status bqa_quantize_blocks(const bqa_problem* p, int32_t role, const bqa_tensor* x, bqa_qtensor* out,
                               float* k_mean, float* block_means, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_problem(p));
    if (role < BQA_ROLE_Q || role > BQA_ROLE_DO) return BQA_E_UNSUPPORTED;
    if (!out) return BQA_E_NULL;
    const bool kv = role == BQA_ROLE_K || role == BQA_ROLE_V;
    const int H = kv ? p->Hkv : p->Hq, N = kv ? p->Nk : p->Nq, d = p->d;
    TRY(check_dense(x, true, true));
    const bool f16 = x->dtype == BQA_FP16;
    hipStream_t st = (hipStream_t)stream;
    if (out->fmt != BQA_MXFP4 && out->fmt != BQA_INT8 && out->fmt != BQA_FP8E4M3) return BQA_E_UNSUPPORTED;
    if (out->fmt == BQA_MXFP4) {
        if (role == BQA_ROLE_DO) return BQA_E_UNSUPPORTED;
        // V: along tokens (axis 1) or blocked by 128 tokens (axis 2)
        const int axis = role == BQA_ROLE_V ? (out->axis == 2 ? 2 : 1) : 0;
        TRY(check_q(out, BQA_MXFP4, axis));
        if (out->block != 32) return BQA_E_UNSUPPORTED;
        if (axis >= 1 && N % 128 != 0) return BQA_E_UNSUPPORTED;
        if (p->mode == BQA_PTQ_MXFP4 && role != BQA_ROLE_V) {
            // the post-training baseline: Q less its bf16 block means (written to
            // block_means, required), K less its token mean when p->smooth_k
            if (d != 128) return BQA_E_UNSUPPORTED;
            const bool key = role == BQA_ROLE_K;
            if (key && block_means) return BQA_E_UNSUPPORTED;
            if (!key && !block_means) return BQA_E_NULL;
            if (!key || p->smooth_k) {
                if (key) {
                    if (!ws || ws_bytes < ws_kmean_bytes(p->B * H, N, d)) return BQA_E_WORKSPACE;
                    if (!std::isfinite(p->smooth_eps)) return BQA_E_SHAPE;
                }
                if (((uintptr_t)block_means & 15u) || ((uintptr_t)k_mean & 3u)) return BQA_E_ALIGN;
                TRY(check_device());
                TRY(debug_check(stream, {dbg16(x, p->B, H, N, d)}));
                return launched(launch_quant_mx_smooth(as_dense(x), f16, p->B, H, N, d, key, (double)p->smooth_eps,
                                                       (uint8_t*)out->codes, (uint8_t*)out->scales,
                                                       key ? k_mean : block_means, ws, st));
            }
        }
        if (block_means && (role == BQA_ROLE_V || p->sel_block != 128)) return BQA_E_UNSUPPORTED;
        if (block_means && N > 1 && N % 128 != 0) return BQA_E_UNSUPPORTED;
        TRY(check_device());
        TRY(debug_check(stream, {dbg16(x, p->B, H, N, d)}));
        return launched(launch_quant_mx(as_dense(x), f16, p->B, H, N, d, axis, (uint8_t*)out->codes,
                                        (uint8_t*)out->scales, block_means, st));
    }
    if (role == BQA_ROLE_V && out->axis == 1) {
        if (out->fmt != BQA_INT8 && out->fmt != BQA_FP8E4M3) return BQA_E_UNSUPPORTED;
        TRY(check_q(out, out->fmt, 1));
        if (out->block != N || N % 64 != 0) return BQA_E_UNSUPPORTED;
        const size_t need = ws_chan_bytes(p->B * H, N, d);
        if (!ws || ws_bytes < need) return BQA_E_WORKSPACE;
        TRY(check_device());
        TRY(debug_check(stream, {dbg16(x, p->B, H, N, d)}));
        return launched(launch_quant_chan(as_dense(x), f16, p->B, H, N, d, out->fmt == BQA_INT8 ? 0 : 1,
                                          (uint8_t*)out->codes, (float*)out->scales, ws, st));
    }
    // INT8 token blocks: Q, K, dO, and V for the fully INT8 backward
    TRY(check_q(out, BQA_INT8, 0));
    const int blk = out->block;
    if (blk != 64 && blk != 128) return BQA_E_UNSUPPORTED;
    if (N % blk != 0) return BQA_E_UNSUPPORTED;
    const bool smooth = role == BQA_ROLE_K && p->smooth_k;
    if (smooth) {
        const size_t need = ws_kmean_bytes(p->B * H, N, d);
        if (!ws || ws_bytes < need) return BQA_E_WORKSPACE;
        if (!std::isfinite(p->smooth_eps)) return BQA_E_SHAPE;
    }
    TRY(check_device());
    TRY(debug_check(stream, {dbg16(x, p->B, H, N, d)}));
    return launched(launch_quant_i8_tokblock(as_dense(x), f16, p->B, H, N, d, blk, smooth, (double)p->smooth_eps,
                                             k_mean, ws, (int8_t*)out->codes, (float*)out->scales, st));
}

bqa_status bqa_quantize_kv(const bqa_problem* p, const bqa_tensor* k, const bqa_tensor* v, bqa_qtensor* kq,
                           bqa_qtensor* vq, float* k_mean, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_problem(p));
    if (p->mode != BQA_SAGE_I8_F8PV && p->mode != BQA_SAGE_I8_I8PV) return BQA_E_UNSUPPORTED;
    TRY(check_sage_blocks(p));
    if (!kq || !vq) return BQA_E_NULL;
    TRY(check_dense(k, true, true));
    TRY(check_dense(v, true, true));
    if (k->dtype != v->dtype) return BQA_E_UNSUPPORTED;
    TRY(check_q(kq, BQA_INT8, 0));
    const int vfmt = p->mode == BQA_SAGE_I8_F8PV ? BQA_FP8E4M3 : BQA_INT8;
    TRY(check_q(vq, vfmt, 1));
    if (kq->block != 64 || p->k_block != 64 || vq->block != p->Nk || p->Nk % 64 != 0) return BQA_E_UNSUPPORTED;
    const int BH = p->B * p->Hkv;
    if (!ws || ws_bytes < ws_kv_bytes(BH, p->Nk, p->d)) return BQA_E_WORKSPACE;
    if (!aligned16(ws)) return BQA_E_ALIGN;
    if (p->smooth_k && !std::isfinite(p->smooth_eps)) return BQA_E_SHAPE;
    TRY(check_device());
    TRY(debug_check(stream, {dbg16(k, p->B, p->Hkv, p->Nk, p->d), dbg16(v, p->B, p->Hkv, p->Nk, p->d)}));
    return launched(launch_quant_kv(as_dense(k), as_dense(v), k->dtype == BQA_FP16, p->B, p->Hkv, p->Nk, p->d,
                                    p->smooth_k != 0, (double)p->smooth_eps, k_mean, (int8_t*)kq->codes,
                                    (float*)kq->scales, vfmt == BQA_INT8 ? 0 : 1, (uint8_t*)vq->codes,
                                    (float*)vq->scales, ws, (hipStream_t)stream));
}

bqa_status bqa_select_blocks(const bqa_problem* p, const float* q_means, const float* k_means, int32_t* sel_idx,
                             int32_t* sel_cnt, void* ws, size_t ws_bytes, void* stream) {
    (void)ws; (void)ws_bytes;
    TRY(check_problem(p));
    if (p->mode != BQA_THRIFT || p->sel_block != 128) return BQA_E_UNSUPPORTED;
    if (!q_means || !k_means || !sel_idx || !sel_cnt) return BQA_E_NULL;
    if (p->Nk % p->sel_block != 0) return BQA_E_UNSUPPORTED;
    // causal prefill: the block-level mask assumes whole query blocks
    if (p->causal && p->Nq > 1 && p->Nq % p->sel_block != 0) return BQA_E_UNSUPPORTED;
    if (p->hp_budget_ppm < 0 || p->hp_budget_ppm > 1000000) return BQA_E_SHAPE;
    const int nkb = p->Nk / p->sel_block, nqb = (p->Nq + p->sel_block - 1) / p->sel_block;
    if (nkb > 4096) return BQA_E_UNSUPPORTED;
    if (!aligned16(k_means) || ((uintptr_t)q_means & 3u) || ((uintptr_t)sel_idx & 3u) || ((uintptr_t)sel_cnt & 3u))
        return BQA_E_ALIGN;
    TRY(check_device());
    TRY(debug_check(stream, {dbg32(q_means, (int64_t)p->B * p->Hq * nqb * p->d),
                             dbg32(k_means, (int64_t)p->B * p->Hkv * nkb * p->d)}));
    return launched(launch_select(q_means, k_means, p->B, p->Hq, p->Hkv, nqb, nkb, p->d, p->causal,
                                  p->hp_budget_ppm, max_sel_of(p), sel_idx, sel_cnt, (hipStream_t)stream));
}

bqa_status bqa_attn_fwd(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k, const bqa_qtensor* v,
                        const bqa_tensor* q_hi, const bqa_tensor* k_hi, const bqa_tensor* v_hi,
                        const int32_t* sel_idx, const int32_t* sel_cnt, bqa_tensor* o, bqa_tensor* o_aux,
                        float* lse, float* row_max, void* ws, size_t ws_bytes, void* stream) {
    (void)q_hi; (void)k_hi; (void)sel_idx; (void)sel_cnt;
    TRY(check_problem(p));
    hipStream_t st = (hipStream_t)stream;
    // BQA_DEBUG=1 (after each mode's validation): the bf16 / fp16 inputs the mode reads
    auto dbg_fwd = [&]() {
        return debug_check(stream, {dbg16(q_hi, p->B, p->Hq, p->Nq, p->d), dbg16(k_hi, p->B, p->Hkv, p->Nk, p->d),
                                    dbg16(v_hi, p->B, p->Hkv, p->Nk, p->d)});
    };
    if (p->mode == BQA_QAT_MXFP4) {
        if (p->d != 128 || p->causal || p->Nk % 128 != 0) return BQA_E_UNSUPPORTED;
        TRY(check_q(q, BQA_MXFP4, 0));
        TRY(check_q(k, BQA_MXFP4, 0));
        TRY(check_q(v, BQA_MXFP4, 1));
        if (q->block != 32 || k->block != 32 || v->block != 32) return BQA_E_UNSUPPORTED;
        TRY(check_dense(o, false, true));
        QatFwdArgs a{};
        if (o_aux) {
            TRY(check_dense(o_aux, false, true));
            if (!ws || ws_bytes < ws_qat_fwd_bytes(p->B, p->Hkv, p->Nk, p->d)) return BQA_E_WORKSPACE;
            if (!aligned16(ws)) return BQA_E_ALIGN;
            a.vdeq = (uint16_t*)ws;
            a.oa = as_dense(o_aux);
        }
        a.qc = (const uint8_t*)q->codes; a.qs = (const uint8_t*)q->scales;
        a.kc = (const uint8_t*)k->codes; a.ks = (const uint8_t*)k->scales;
        a.vc = (const uint8_t*)v->codes; a.vs = (const uint8_t*)v->scales;
        a.o = as_dense(o); a.lse = lse; a.row_max = row_max;
        a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk;
        a.c_log2 = tau_of(p) * 1.4426950408889634f;
        TRY(check_device());
        TRY(dbg_fwd());
        return launched(launch_qat_fwd(a, st));
    }
    if (p->mode == BQA_THRIFT && p->Nq == 1) {
        ThriftDecArgs a{};
        TRY(check_decode(p, q, k, v, q_hi, k_hi, v_hi, sel_idx, sel_cnt, o, a));
        if (!ws || ws_bytes < ws_decode_bytes(p->B, p->Hq, p->Hkv, p->Nk, p->num_splits)) return BQA_E_WORKSPACE;
        if (!aligned16(ws)) return BQA_E_ALIGN;
        a.part = (float*)ws;
        TRY(check_device());
        TRY(dbg_fwd());
        return launched(launch_thrift_decode(a, as_dense(o), lse, st));
    }
    if (p->mode == BQA_THRIFT && p->Nq > 1) {
        if (p->d != 128 || p->sel_block != 128 || p->Nk % 128 != 0) return BQA_E_UNSUPPORTED;
        if (p->causal && p->Nq % 128 != 0) return BQA_E_UNSUPPORTED;   // selection is per whole query block
        TRY(check_q(q, BQA_MXFP4, 0));
        TRY(check_q(k, BQA_MXFP4, 0));
        TRY(check_q(v, BQA_MXFP4, 1));
        if (q->block != 32 || k->block != 32 || v->block != 32) return BQA_E_UNSUPPORTED;
        TRY(check_dense(q_hi, false, true));
        TRY(check_dense(k_hi, false, true));
        TRY(check_dense(v_hi, false, true));
        TRY(check_dense(o, false, true));
        if (!sel_idx || !sel_cnt) return BQA_E_NULL;
        if (p->hp_budget_ppm < 0 || p->hp_budget_ppm > 1000000) return BQA_E_SHAPE;
        ThriftFwdArgs a{};
        a.qc = (const uint8_t*)q->codes; a.qs = (const uint8_t*)q->scales;
        a.kc = (const uint8_t*)k->codes; a.ks = (const uint8_t*)k->scales;
        a.vc = (const uint8_t*)v->codes; a.vs = (const uint8_t*)v->scales;
        a.q_hi = as_dense(q_hi); a.k_hi = as_dense(k_hi); a.v_hi = as_dense(v_hi);
        a.sel_idx = sel_idx; a.sel_cnt = sel_cnt; a.max_sel = max_sel_of(p);
        a.o = as_dense(o); a.lse = lse;
        a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.causal = p->causal;
        a.c_log2 = tau_of(p) * 1.4426950408889634f;
        TRY(check_device());
        TRY(dbg_fwd());
        return launched(launch_thrift_fwd(a, st));
    }
    if (is_sage(p->mode)) {
        TRY(check_sage_blocks(p));
        // q_hi given (fp8 P.V): the kernel quantises Q itself; q, when given, receives its codes
        const bool q_in = q_hi != nullptr;
        if (q_in) {
            if (p->mode != BQA_SAGE_I8_F8PV) return BQA_E_UNSUPPORTED;
            TRY(check_dense(q_hi, false, true));
        }
        if (!q_in || q) {
            TRY(check_q(q, BQA_INT8, 0));
            if (q->block != p->q_block) return BQA_E_UNSUPPORTED;
        }
        TRY(check_q(k, BQA_INT8, 0));
        if (k->block != p->k_block) return BQA_E_UNSUPPORTED;
        SageFwdArgs a{};
        int pv;
        if (p->mode == BQA_SAGE_I8_F16PV) {
            TRY(check_dense(v_hi, true, false));
            pv = PV_F16;
            a.v16 = as_dense(v_hi);
        } else {
            const int fmt = p->mode == BQA_SAGE_I8_F8PV ? BQA_FP8E4M3 : BQA_INT8;
            TRY(check_q(v, fmt, 1));
            if (v->block != p->Nk) return BQA_E_UNSUPPORTED;
            pv = p->mode == BQA_SAGE_I8_F8PV ? PV_F8 : PV_I8;
            a.vc = (const uint8_t*)v->codes;
            a.vs = (const float*)v->scales;
        }
        TRY(check_dense(o, pv == PV_F16, pv != PV_F16));
        a.q_blk = p->q_block;
        if (q_in) {
            a.q16 = as_dense(q_hi);
            if (q) { a.qc_out = (int8_t*)q->codes; a.qs_out = (float*)q->scales; }
        } else {
            a.qc = (const int8_t*)q->codes; a.qs = (const float*)q->scales;
        }
        a.kc = (const int8_t*)k->codes; a.ks = (const float*)k->scales;
        a.o = as_dense(o); a.lse = lse;
        a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.causal = p->causal;
        a.c_log2 = tau_of(p) * 1.4426950408889634f;
        TRY(check_device());
        TRY(dbg_fwd());
        return launched(launch_sage_fwd(a, pv, p->d, st));
    }
    return BQA_E_UNSUPPORTED;
}

bqa_status bqa_attn_fwd_ptq(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k, const bqa_qtensor* v,
                            const float* q_means, bqa_tensor* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_problem(p));
    if (p->mode != BQA_PTQ_MXFP4) return BQA_E_UNSUPPORTED;
    if (p->d != 128 || p->Nk % 128 != 0) return BQA_E_UNSUPPORTED;
    TRY(check_q(q, BQA_MXFP4, 0));
    TRY(check_q(k, BQA_MXFP4, 0));
    TRY(check_q(v, BQA_MXFP4, 1));
    if (q->block != 32 || k->block != 32 || v->block != 32) return BQA_E_UNSUPPORTED;
    TRY(check_dense(o, false, true));
    if (!q_means) return BQA_E_NULL;
    if (!ws || ws_bytes < ws_ptq_fwd_bytes(p->B, p->Hq, p->Nq, p->Nk)) return BQA_E_WORKSPACE;
    if (!aligned16(ws) || !aligned16(q_means) || ((uintptr_t)k->scales & 3u)) return BQA_E_ALIGN;
    ThriftFwdArgs a{};
    a.qc = (const uint8_t*)q->codes; a.qs = (const uint8_t*)q->scales;
    a.kc = (const uint8_t*)k->codes; a.ks = (const uint8_t*)k->scales;
    a.vc = (const uint8_t*)v->codes; a.vs = (const uint8_t*)v->scales;
    a.o = as_dense(o); a.lse = lse;
    a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.causal = p->causal;
    a.c_log2 = tau_of(p) * 1.4426950408889634f;
    TRY(check_device());
    const int nqb = (p->Nq + 127) / 128;
    TRY(debug_check(stream, {dbg32(q_means, (int64_t)p->B * p->Hq * nqb * p->d)}));
    return launched(launch_ptq_fwd(a, q_means, ws, (hipStream_t)stream));
}

bqa_status bqa_quantize_qknorm(const bqa_problem* p, int32_t role, const bqa_tensor* x, bqa_qtensor* out,
                               float* inv_norm, float* k_mean, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_problem(p));
    if (!is_sage(p->mode) || p->d != 128) return BQA_E_UNSUPPORTED;
    if (role != BQA_ROLE_Q && role != BQA_ROLE_K) return BQA_E_UNSUPPORTED;
    if (!out || !inv_norm) return BQA_E_NULL;
    const bool key = role == BQA_ROLE_K;
    const int H = key ? p->Hkv : p->Hq, N = key ? p->Nk : p->Nq;
    TRY(check_dense(x, true, true));
    TRY(check_q(out, BQA_INT8, 0));
    const int blk = out->block;
    if ((blk != 64 && blk != 128) || N % blk != 0) return BQA_E_UNSUPPORTED;
    if ((uintptr_t)inv_norm & 3u) return BQA_E_ALIGN;
    const bool smooth = key && p->smooth_k;
    if (smooth) {
        if (!ws || ws_bytes < ws_kmean_bytes(p->B * H, N, p->d)) return BQA_E_WORKSPACE;
        if (!std::isfinite(p->smooth_eps)) return BQA_E_SHAPE;
    }
    TRY(check_device());
    TRY(debug_check(stream, {dbg16(x, p->B, H, N, p->d)}));
    return launched(launch_quant_i8_qknorm(as_dense(x), x->dtype == BQA_FP16, p->B, H, N, p->d, blk, smooth,
                                           (double)p->smooth_eps, smooth ? k_mean : nullptr, inv_norm, ws,
                                           (int8_t*)out->codes, (float*)out->scales, (hipStream_t)stream));
}

bqa_status bqa_attn_bwd_qknorm(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                               const bqa_tensor* v_hi, const bqa_tensor* o_for_delta, const float* lse,
                               const bqa_tensor* d_o, const bqa_tensor* q_raw, const bqa_tensor* k_raw,
                               const float* q_inv_norm, const float* k_inv_norm, bqa_tensor* dq, bqa_tensor* dk,
                               bqa_tensor* dv, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_problem(p));
    if (!is_sage(p->mode)) return BQA_E_UNSUPPORTED;
    SageBwdArgs a{};
    TRY(check_sage_bwd(p, q, k, v_hi, o_for_delta, lse, d_o, dq, dk, dv, ws, ws_bytes, a));
    TRY(check_dense(q_raw, false, true));
    TRY(check_dense(k_raw, false, true));
    if (!q_inv_norm || !k_inv_norm) return BQA_E_NULL;
    if (((uintptr_t)q_inv_norm & 3u) || ((uintptr_t)k_inv_norm & 3u)) return BQA_E_ALIGN;
    a.q_raw = as_dense(q_raw); a.k_raw = as_dense(k_raw);
    a.q_rn = q_inv_norm; a.k_rn = k_inv_norm;
    TRY(check_device());
    const int64_t bhn = (int64_t)p->B * p->Hq * p->Nq;
    TRY(debug_check(stream, {dbg16(v_hi, p->B, p->Hq, p->Nq, p->d), dbg16(o_for_delta, p->B, p->Hq, p->Nq, p->d),
                             dbg16(d_o, p->B, p->Hq, p->Nq, p->d), dbg32(lse, bhn),
                             dbg16(q_raw, p->B, p->Hq, p->Nq, p->d), dbg16(k_raw, p->B, p->Hq, p->Nq, p->d),
                             dbg32(q_inv_norm, bhn), dbg32(k_inv_norm, bhn)}));
    return launched(launch_sage_bwd(a, as_dense(o_for_delta), ws, (hipStream_t)stream));
}

bqa_status bqa_quantize_nvfp4(const bqa_problem* p, int32_t role, const bqa_tensor* x, bqa_tensor* out, void* ws,
                              size_t ws_bytes, void* stream) {
    TRY(check_problem(p));
    if (p->d != 128) return BQA_E_UNSUPPORTED;
    if (role != BQA_ROLE_Q && role != BQA_ROLE_K && role != BQA_ROLE_V) return BQA_E_UNSUPPORTED;
    const bool kv = role != BQA_ROLE_Q;
    const int H = kv ? p->Hkv : p->Hq, N = kv ? p->Nk : p->Nq;
    TRY(check_dense(x, true, true));
    TRY(check_dense(out, false, true));
    if (role == BQA_ROLE_V && N % 32 != 0) return BQA_E_UNSUPPORTED;
    if (!ws || ws_bytes < ws_nvfp4_bytes(p->B * H, N, p->d)) return BQA_E_WORKSPACE;
    if (!aligned16(ws)) return BQA_E_ALIGN;
    TRY(check_device());
    TRY(debug_check(stream, {dbg16(x, p->B, H, N, p->d)}));
    return launched(launch_nvfp4(as_dense(x), x->dtype == BQA_FP16, p->B, H, N, p->d, role == BQA_ROLE_V ? 1 : 0,
                                 as_dense(out), ws, (hipStream_t)stream));
}

bqa_status bqa_attn_fwd_thrift_nvfp4(const bqa_problem* p, const bqa_tensor* q_nv, const bqa_tensor* k_nv,
                                     const bqa_tensor* v_nv, const bqa_tensor* q_hi, const bqa_tensor* k_hi,
                                     const bqa_tensor* v_hi, const int32_t* sel_idx, const int32_t* sel_cnt,
                                     bqa_tensor* o, float* lse, void* stream) {
    TRY(check_problem(p));
    if (p->mode != BQA_THRIFT || p->Nq < 2) return BQA_E_UNSUPPORTED;
    if (p->d != 128 || p->sel_block != 128 || p->Nk % 128 != 0) return BQA_E_UNSUPPORTED;
    if (p->causal && p->Nq % 128 != 0) return BQA_E_UNSUPPORTED;
    TRY(check_dense(q_nv, false, true));
    TRY(check_dense(k_nv, false, true));
    TRY(check_dense(v_nv, false, true));
    TRY(check_dense(q_hi, false, true));
    TRY(check_dense(k_hi, false, true));
    TRY(check_dense(v_hi, false, true));
    TRY(check_dense(o, false, true));
    if (!sel_idx || !sel_cnt) return BQA_E_NULL;
    if (p->hp_budget_ppm < 0 || p->hp_budget_ppm > 1000000) return BQA_E_SHAPE;
    ThriftFwdArgs a{};
    a.q_nv = as_dense(q_nv); a.k_nv = as_dense(k_nv); a.v_nv = as_dense(v_nv);
    a.q_hi = as_dense(q_hi); a.k_hi = as_dense(k_hi); a.v_hi = as_dense(v_hi);
    a.sel_idx = sel_idx; a.sel_cnt = sel_cnt; a.max_sel = max_sel_of(p);
    a.o = as_dense(o); a.lse = lse;
    a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.causal = p->causal;
    a.c_log2 = tau_of(p) * 1.4426950408889634f;
    TRY(check_device());
    TRY(debug_check(stream, {dbg16(q_nv, p->B, p->Hq, p->Nq, p->d), dbg16(k_nv, p->B, p->Hkv, p->Nk, p->d),
                             dbg16(v_nv, p->B, p->Hkv, p->Nk, p->d), dbg16(q_hi, p->B, p->Hq, p->Nq, p->d),
                             dbg16(k_hi, p->B, p->Hkv, p->Nk, p->d), dbg16(v_hi, p->B, p->Hkv, p->Nk, p->d)}));
    return launched(launch_thrift_nv(a, (hipStream_t)stream));
}

bqa_status bqa_attn_decode_static(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k,
                                  const bqa_qtensor* v, const bqa_tensor* q_hi, const bqa_tensor* k_hi,
                                  const bqa_tensor* v_hi, const int32_t* sel_idx, const int32_t* sel_cnt,
                                  bqa_tensor* o, float* lse, void* stream) {
    TRY(check_problem(p));
    ThriftDecArgs a{};
    TRY(check_decode(p, q, k, v, q_hi, k_hi, v_hi, sel_idx, sel_cnt, o, a));
    if (ws_decode_bytes(p->B, p->Hq, p->Hkv, p->Nk, p->num_splits) > decode_scratch_bytes()) return BQA_E_TOO_LARGE;
    TRY(check_device());
    TRY(debug_check(stream, {dbg16(q_hi, p->B, p->Hq, 1, p->d), dbg16(k_hi, p->B, p->Hkv, p->Nk, p->d),
                             dbg16(v_hi, p->B, p->Hkv, p->Nk, p->d)}));
    float* part = nullptr;
    if (decode_scratch(&part) != hipSuccess) return BQA_E_DEVICE;
    a.part = part;
    return launched(launch_thrift_decode(a, as_dense(o), lse, (hipStream_t)stream));
}

bqa_status bqa_attn_bwd(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k, const bqa_qtensor* v,
                        const bqa_tensor* v_hi, const bqa_tensor* o_for_delta, const float* lse,
                        const float* row_max, const bqa_tensor* d_o, bqa_tensor* dq, bqa_tensor* dk, bqa_tensor* dv, void* ws,
                        size_t ws_bytes, void* stream) {
    TRY(check_problem(p));
    hipStream_t st = (hipStream_t)stream;
    if (is_sage(p->mode)) {
        SageBwdArgs a{};
        TRY(check_sage_bwd(p, q, k, v_hi, o_for_delta, lse, d_o, dq, dk, dv, ws, ws_bytes, a));
        if (v) {
            // the fully INT8 variant: dP from V's INT8 codes per 64 tokens
            TRY(check_q(v, BQA_INT8, 0));
            if (v->block != 64) return BQA_E_UNSUPPORTED;
            a.vc8 = (const int8_t*)v->codes;
            a.vs8 = (const float*)v->scales;
        }
        TRY(check_device());
        const int64_t bhn = (int64_t)p->B * p->Hq * p->Nq;
        TRY(debug_check(stream, {dbg16(v_hi, p->B, p->Hq, p->Nq, p->d), dbg16(o_for_delta, p->B, p->Hq, p->Nq, p->d),
                                 dbg16(d_o, p->B, p->Hq, p->Nq, p->d), dbg32(lse, bhn)}));
        return launched(launch_sage_bwd(a, as_dense(o_for_delta), ws, st));
    }
    if (p->mode == BQA_QAT_MXFP4) {
        if (p->d != 128 || p->Hq != p->Hkv || p->Nq != p->Nk || p->Nq % 128 != 0 || p->causal)
            return BQA_E_UNSUPPORTED;
        TRY(check_q(q, BQA_MXFP4, 0));
        TRY(check_q(k, BQA_MXFP4, 0));
        TRY(check_q(v, BQA_MXFP4, 1));
        if (q->block != 32 || k->block != 32 || v->block != 32) return BQA_E_UNSUPPORTED;
        TRY(check_dense(o_for_delta, false, true));
        TRY(check_dense(d_o, false, true));
        TRY(check_dense(dq, false, true));
        TRY(check_dense(dk, false, true));
        TRY(check_dense(dv, false, true));
        if (!lse || !row_max) return BQA_E_NULL;
        if (!ws || ws_bytes < ws_qat_bwd_bytes(p->B, p->Hq, p->Nq, p->d)) return BQA_E_WORKSPACE;
        if (!aligned16(ws) || ((uintptr_t)lse & 15u) || ((uintptr_t)row_max & 15u)) return BQA_E_ALIGN;
        QatBwdArgs a{};
        a.qc = (const uint8_t*)q->codes; a.qs = (const uint8_t*)q->scales;
        a.kc = (const uint8_t*)k->codes; a.ks = (const uint8_t*)k->scales;
        a.vc = (const uint8_t*)v->codes; a.vs = (const uint8_t*)v->scales;
        a.d_o = as_dense(d_o); a.lse = lse; a.row_max = row_max;
        a.dq = as_dense(dq); a.dk = as_dense(dk); a.dv = as_dense(dv);
        a.B = p->B; a.H = p->Hq; a.N = p->Nq;
        a.tau = tau_of(p);
        a.c_log2 = a.tau * 1.4426950408889634f;
        TRY(check_device());
        const int64_t bhn = (int64_t)p->B * p->Hq * p->Nq;
        TRY(debug_check(stream, {dbg16(o_for_delta, p->B, p->Hq, p->Nq, p->d), dbg16(d_o, p->B, p->Hq, p->Nq, p->d),
                                 dbg32(lse, bhn), dbg32(row_max, bhn)}));
        return launched(launch_qat_bwd(a, as_dense(o_for_delta), ws, st));
    }
    return BQA_E_UNSUPPORTED;
}

bqa_status bqa_debug_qk_scores(const bqa_problem* p, const bqa_qtensor* q, const bqa_qtensor* k, int32_t b,
                               int32_t h, int32_t q_tile, int32_t k_tile, void* out, void* stream) {
    TRY(check_problem(p));
    if (!out) return BQA_E_NULL;
    if (b < 0 || b >= p->B || h < 0 || h >= p->Hq) return BQA_E_SHAPE;
    if (q_tile < 0 || (int64_t)(q_tile + 1) * 32 > p->Nq || k_tile < 0 || (int64_t)(k_tile + 1) * 32 > p->Nk)
        return BQA_E_SHAPE;
    if (!q || !k) return BQA_E_NULL;
    if (q->fmt == BQA_INT8) {
        TRY(check_q(q, BQA_INT8, 0));
        TRY(check_q(k, BQA_INT8, 0));
        TRY(check_device());
        const int hk = h / (p->Hq / p->Hkv);
        const int64_t qrow = ((int64_t)b * p->Hq + h) * p->Nq + (int64_t)q_tile * 32;
        const int64_t krow = ((int64_t)b * p->Hkv + hk) * p->Nk + (int64_t)k_tile * 32;
        return launched(launch_debug_scores_i8((const int8_t*)q->codes, (const int8_t*)k->codes, p->d, qrow, krow,
                                               (int32_t*)out, (hipStream_t)stream));
    }
    if (q->fmt == BQA_MXFP4) {
        if (p->d != 128) return BQA_E_UNSUPPORTED;
        TRY(check_q(q, BQA_MXFP4, 0));
        TRY(check_q(k, BQA_MXFP4, 0));
        TRY(check_device());
        const int hk = h / (p->Hq / p->Hkv);
        const int64_t qrow = ((int64_t)b * p->Hq + h) * p->Nq + (int64_t)q_tile * 32;
        const int64_t krow = ((int64_t)b * p->Hkv + hk) * p->Nk + (int64_t)k_tile * 32;
        const uint8_t* qc = (const uint8_t*)q->codes + qrow * (p->d / 2);
        const uint8_t* qs = (const uint8_t*)q->scales + qrow * (p->d / 32);
        const uint8_t* kc = (const uint8_t*)k->codes + krow * (p->d / 2);
        const uint8_t* ks = (const uint8_t*)k->scales + krow * (p->d / 32);
        return launched(launch_debug_scores_mx(qc, qs, kc, ks, (float*)out, (hipStream_t)stream));
    }
    return BQA_E_UNSUPPORTED;
}

}  // extern "C"

extern "C" bqa_status bqa_debug_mx_dequant(const void* codes, const void* scales, int64_t nblocks, void* out,
                                           void* stream) {
    if (!codes || !scales || !out) return BQA_E_NULL;
    if (nblocks < 0 || nblocks > ((int64_t)1 << 31)) return BQA_E_SHAPE;
    if (!aligned16(codes) || !aligned16(out)) return BQA_E_ALIGN;
    TRY(check_device());
    return launched(launch_mx_dequant((const uint8_t*)codes, (const uint8_t*)scales, nblocks, (uint16_t*)out,
                                      (hipStream_t)stream));
}

extern "C" bqa_status bqa_debug_probe(int32_t kind, int32_t grid, int64_t iters, const void* src, void* dst,
                                      size_t bytes, void* stream) {
    if (kind < BQA_PROBE_MFMA_I8 || kind > BQA_PROBE_LDS_SPANS) return BQA_E_UNSUPPORTED;
    if (grid < 1 || grid > (1 << 20) || iters < 0 || iters > ((int64_t)1 << 30)) return BQA_E_SHAPE;
    if (!dst) return BQA_E_NULL;
    if (kind == BQA_PROBE_COPY) {
        if (!src) return BQA_E_NULL;
        if (!aligned16(src) || !aligned16(dst) || bytes % 16 != 0) return BQA_E_ALIGN;
    } else if (kind == BQA_PROBE_READ || kind == BQA_PROBE_READ_NT) {
        if (!src) return BQA_E_NULL;
        if (!aligned16(src) || bytes % 16 != 0 || ((uintptr_t)dst & 3u)) return BQA_E_ALIGN;
    } else {
        if ((uintptr_t)dst & 3u) return BQA_E_ALIGN;
        if (bytes < (size_t)grid * 4) return BQA_E_SHAPE;
    }
    TRY(check_device());
    return launched(launch_probe(kind, grid, iters, src, dst, bytes, (hipStream_t)stream));
}
