"""Python binding of libbqa.so, the gfx950 block-quantized attention library.

The functions here carry the C ABI's names (``include/bqa.h``) and only
marshal arguments: torch tensors are turned into the ABI's descriptors
(device pointers, element strides) and the current torch stream is passed
as the HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no fallback — if ``libbqa.so`` is missing or the device is
not gfx950 the calls raise.
"""
from __future__ import annotations

import ctypes as C
import os

__all__ = [
    "BQA_OK", "BqaError", "bqa_problem", "bqa_tensor", "bqa_qtensor", "lib", "problem",
    "bqa_abi_version", "bqa_status_string", "bqa_workspace_size", "bqa_quantize_blocks", "bqa_quantize_kv",
    "bqa_select_blocks", "bqa_attn_fwd", "bqa_attn_bwd", "bqa_debug_qk_scores", "bqa_attn_decode_static",
    "bqa_debug_mx_dequant",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbqa.so")

BQA_OK, BQA_E_NULL, BQA_E_SHAPE, BQA_E_UNSUPPORTED, BQA_E_ALIGN, BQA_E_WORKSPACE, BQA_E_DEVICE, BQA_E_LAUNCH = \
    0, -1, -2, -3, -4, -5, -6, -7
BQA_E_NONFINITE, BQA_E_TOO_LARGE = -8, -9
BQA_BF16, BQA_FP16, BQA_INT8, BQA_FP8E4M3, BQA_MXFP4 = range(5)
BQA_SAGE_I8_F16PV, BQA_SAGE_I8_F8PV, BQA_SAGE_I8_I8PV, BQA_QAT_MXFP4, BQA_THRIFT, BQA_PTQ_MXFP4 = range(6)
BQA_ROLE_Q, BQA_ROLE_K, BQA_ROLE_V, BQA_ROLE_DO = range(4)
BQA_OP_QUANTIZE_Q, BQA_OP_QUANTIZE_K, BQA_OP_QUANTIZE_V, BQA_OP_QUANTIZE_DO, BQA_OP_SELECT, BQA_OP_FWD, \
    BQA_OP_BWD, BQA_OP_QUANTIZE_KV, BQA_OP_QUANTIZE_NVFP4 = range(9)

EXPORTS = ["bqa_abi_version", "bqa_status_string", "bqa_workspace_size", "bqa_quantize_blocks", "bqa_quantize_kv",
           "bqa_select_blocks", "bqa_attn_fwd", "bqa_attn_bwd", "bqa_debug_qk_scores", "bqa_attn_decode_static",
           "bqa_debug_mx_dequant", "bqa_attn_fwd_ptq", "bqa_debug_probe", "bqa_quantize_qknorm",
           "bqa_attn_bwd_qknorm", "bqa_quantize_nvfp4", "bqa_attn_fwd_thrift_nvfp4"]
BQA_PROBE_MFMA_I8, BQA_PROBE_MFMA_F8, BQA_PROBE_MFMA_F4, BQA_PROBE_MFMA_BF16, BQA_PROBE_EXP, BQA_PROBE_COPY, \
    BQA_PROBE_READ, BQA_PROBE_READ_NT, BQA_PROBE_ISSUE_MFMA, BQA_PROBE_ISSUE_FMA, BQA_PROBE_ISSUE_MFMA_FMA, \
    BQA_PROBE_ISSUE_EXP, BQA_PROBE_ISSUE_MFMA_EXP, BQA_PROBE_OP_MUL, BQA_PROBE_OP_FMA, BQA_PROBE_OP_CVT_F32_I32, \
    BQA_PROBE_OP_MAX3, BQA_PROBE_OP_CVT_PK_FP8, BQA_PROBE_OP_CVT_PK_FP4, BQA_PROBE_OP_PERMLANE32, \
    BQA_PROBE_ISSUE_EXP_FMA, BQA_PROBE_LDS_SHARED_ROWS, BQA_PROBE_LDS_SPANS = range(23)


class BqaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({bqa_status_string(status)})")
        self.status = status


class bqa_problem(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("Nq", C.c_int32), ("Nk", C.c_int32),
                ("d", C.c_int32), ("causal", C.c_int32), ("sm_scale", C.c_float), ("mode", C.c_int32),
                ("q_block", C.c_int32), ("k_block", C.c_int32), ("smooth_k", C.c_int32),
                ("smooth_eps", C.c_float), ("hp_budget_ppm", C.c_int32), ("sel_block", C.c_int32),
                ("num_splits", C.c_int32)]


class bqa_tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("stride", C.c_int64 * 4)]


class bqa_qtensor(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("axis", C.c_int32), ("block", C.c_int32), ("codes", C.c_void_p),
                ("scales", C.c_void_p)]


_lib = None


def lib():
    """Load libbqa.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        P = C.POINTER
        vp = C.c_void_p
        L.bqa_abi_version.restype = C.c_int32
        L.bqa_abi_version.argtypes = []
        L.bqa_status_string.restype = C.c_char_p
        L.bqa_status_string.argtypes = [C.c_int32]
        L.bqa_workspace_size.restype = C.c_size_t
        L.bqa_workspace_size.argtypes = [P(bqa_problem), C.c_int32]
        L.bqa_quantize_blocks.restype = C.c_int32
        L.bqa_quantize_blocks.argtypes = [P(bqa_problem), C.c_int32, P(bqa_tensor), P(bqa_qtensor), vp, vp, vp,
                                          C.c_size_t, vp]
        L.bqa_quantize_kv.restype = C.c_int32
        L.bqa_quantize_kv.argtypes = [P(bqa_problem), P(bqa_tensor), P(bqa_tensor), P(bqa_qtensor), P(bqa_qtensor),
                                      vp, vp, C.c_size_t, vp]
        L.bqa_select_blocks.restype = C.c_int32
        L.bqa_select_blocks.argtypes = [P(bqa_problem), vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.bqa_attn_fwd.restype = C.c_int32
        L.bqa_attn_fwd.argtypes = [P(bqa_problem), P(bqa_qtensor), P(bqa_qtensor), P(bqa_qtensor), P(bqa_tensor),
                                   P(bqa_tensor), P(bqa_tensor), vp, vp, P(bqa_tensor), P(bqa_tensor), vp, vp, vp,
                                   C.c_size_t, vp]
        L.bqa_attn_bwd.restype = C.c_int32
        L.bqa_attn_bwd.argtypes = [P(bqa_problem), P(bqa_qtensor), P(bqa_qtensor), P(bqa_qtensor), P(bqa_tensor),
                                   P(bqa_tensor), vp, vp, P(bqa_tensor), P(bqa_tensor), P(bqa_tensor), P(bqa_tensor),
                                   vp, C.c_size_t, vp]
        L.bqa_attn_decode_static.restype = C.c_int32
        L.bqa_attn_decode_static.argtypes = [P(bqa_problem), P(bqa_qtensor), P(bqa_qtensor), P(bqa_qtensor),
                                             P(bqa_tensor), P(bqa_tensor), P(bqa_tensor), vp, vp, P(bqa_tensor), vp,
                                             vp]
        L.bqa_attn_fwd_ptq.restype = C.c_int32
        L.bqa_attn_fwd_ptq.argtypes = [P(bqa_problem), P(bqa_qtensor), P(bqa_qtensor), P(bqa_qtensor), vp,
                                       P(bqa_tensor), vp, vp, C.c_size_t, vp]
        L.bqa_quantize_qknorm.restype = C.c_int32
        L.bqa_quantize_qknorm.argtypes = [P(bqa_problem), C.c_int32, P(bqa_tensor), P(bqa_qtensor), vp, vp, vp,
                                          C.c_size_t, vp]
        L.bqa_attn_bwd_qknorm.restype = C.c_int32
        L.bqa_attn_bwd_qknorm.argtypes = [P(bqa_problem), P(bqa_qtensor), P(bqa_qtensor), P(bqa_tensor),
                                          P(bqa_tensor), vp, P(bqa_tensor), P(bqa_tensor), P(bqa_tensor), vp, vp,
                                          P(bqa_tensor), P(bqa_tensor), P(bqa_tensor), vp, C.c_size_t, vp]
        L.bqa_quantize_nvfp4.restype = C.c_int32
        L.bqa_quantize_nvfp4.argtypes = [P(bqa_problem), C.c_int32, P(bqa_tensor), P(bqa_tensor), vp, C.c_size_t, vp]
        L.bqa_attn_fwd_thrift_nvfp4.restype = C.c_int32
        L.bqa_attn_fwd_thrift_nvfp4.argtypes = [P(bqa_problem), P(bqa_tensor), P(bqa_tensor), P(bqa_tensor),
                                                P(bqa_tensor), P(bqa_tensor), P(bqa_tensor), vp, vp, P(bqa_tensor),
                                                vp, vp]
        L.bqa_debug_probe.restype = C.c_int32
        L.bqa_debug_probe.argtypes = [C.c_int32, C.c_int32, C.c_int64, vp, vp, C.c_size_t, vp]
        L.bqa_debug_mx_dequant.restype = C.c_int32
        L.bqa_debug_mx_dequant.argtypes = [vp, vp, C.c_int64, vp, vp]
        L.bqa_debug_qk_scores.restype = C.c_int32
        L.bqa_debug_qk_scores.argtypes = [P(bqa_problem), P(bqa_qtensor), P(bqa_qtensor), C.c_int32, C.c_int32,
                                          C.c_int32, C.c_int32, vp, vp]
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling
def problem(**kw) -> bqa_problem:
    """A bqa_problem with the given fields (others zero)."""
    p = bqa_problem()
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def max_sel(p: bqa_problem) -> int:
    """Slots per query block of the selection output, as include/bqa.h sizes
    it: max(1, ceil(nkb * budget)), at most nkb = Nk / sel_block."""
    nkb = p.Nk // p.sel_block
    return max(1, min(nkb, -(-nkb * p.hp_budget_ppm // 1_000_000)))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    """The HIP stream handle: the given one, else torch's current stream (0 without a GPU)."""
    if stream is not None:
        return stream
    import torch
    if not torch.cuda.is_available():
        return 0
    return torch.cuda.current_stream().cuda_stream


def dense(t) -> bqa_tensor:
    """bqa_tensor view of a 4-d torch tensor [B, H, N, d] (bf16 or fp16)."""
    import torch
    if t is None:
        return None
    if t.dim() != 4:
        raise ValueError("dense tensors are [B, H, N, d]")
    dt = {torch.bfloat16: BQA_BF16, torch.float16: BQA_FP16}[t.dtype]
    d = bqa_tensor()
    d.data = t.data_ptr()
    d.dtype = dt
    for i in range(4):
        d.stride[i] = t.stride(i)
    return d


def qtensor(fmt: int, axis: int, block: int, codes, scales) -> bqa_qtensor:
    q = bqa_qtensor()
    q.fmt, q.axis, q.block = fmt, axis, block
    q.codes = _ptr(codes)
    q.scales = _ptr(scales)
    return q


def _ref(x):
    return None if x is None else C.byref(x)


def _check(status: int, where: str):
    if status != BQA_OK:
        raise BqaError(status, where)


# ------------------------------------------------------------------ entry points
def bqa_abi_version() -> int:
    return int(lib().bqa_abi_version())


def bqa_status_string(status: int) -> str:
    return lib().bqa_status_string(int(status)).decode()


def bqa_workspace_size(p: bqa_problem, op: int) -> int:
    return int(lib().bqa_workspace_size(C.byref(p), int(op)))


def bqa_quantize_blocks(p, role, x, out: bqa_qtensor, k_mean=None, block_means=None, workspace=None,
                        workspace_bytes=None, stream=None, check=True) -> int:
    xd = x if isinstance(x, bqa_tensor) else dense(x)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_quantize_blocks(C.byref(p), int(role), _ref(xd), C.byref(out), _ptr(k_mean),
                                  _ptr(block_means), _ptr(workspace), wb,
                                  _stream(stream))
    if check:
        _check(s, "bqa_quantize_blocks")
    return s


def bqa_quantize_kv(p, k, v, kq: bqa_qtensor, vq: bqa_qtensor, k_mean=None, workspace=None, workspace_bytes=None,
                    stream=None, check=True) -> int:
    kd = k if isinstance(k, bqa_tensor) else dense(k)
    vd = v if isinstance(v, bqa_tensor) else dense(v)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_quantize_kv(C.byref(p), _ref(kd), _ref(vd), C.byref(kq), C.byref(vq), _ptr(k_mean),
                              _ptr(workspace), wb, _stream(stream))
    if check:
        _check(s, "bqa_quantize_kv")
    return s


def bqa_select_blocks(p, q_means, k_means, sel_idx, sel_cnt, workspace=None, workspace_bytes=None, stream=None,
                      check=True) -> int:
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_select_blocks(C.byref(p), _ptr(q_means), _ptr(k_means), _ptr(sel_idx), _ptr(sel_cnt),
                                _ptr(workspace), wb, _stream(stream))
    if check:
        _check(s, "bqa_select_blocks")
    return s


def bqa_attn_fwd(p, q=None, k=None, v=None, q_hi=None, k_hi=None, v_hi=None, sel_idx=None, sel_cnt=None, o=None,
                 o_aux=None, lse=None, row_max=None, workspace=None, workspace_bytes=None, stream=None,
                 check=True) -> int:
    def dd(t):
        return t if (t is None or isinstance(t, bqa_tensor)) else dense(t)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_attn_fwd(C.byref(p), _ref(q), _ref(k), _ref(v), _ref(dd(q_hi)), _ref(dd(k_hi)), _ref(dd(v_hi)),
                           _ptr(sel_idx), _ptr(sel_cnt), _ref(dd(o)), _ref(dd(o_aux)), _ptr(lse), _ptr(row_max),
                           _ptr(workspace),
                           wb, _stream(stream))
    if check:
        _check(s, "bqa_attn_fwd")
    return s


def bqa_attn_bwd(p, q=None, k=None, v=None, v_hi=None, o_for_delta=None, lse=None, row_max=None, d_o=None, dq=None,
                 dk=None, dv=None, workspace=None, workspace_bytes=None, stream=None, check=True) -> int:
    def dd(t):
        return t if (t is None or isinstance(t, bqa_tensor)) else dense(t)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_attn_bwd(C.byref(p), _ref(q), _ref(k), _ref(v), _ref(dd(v_hi)), _ref(dd(o_for_delta)), _ptr(lse),
                           _ptr(row_max), _ref(dd(d_o)), _ref(dd(dq)), _ref(dd(dk)), _ref(dd(dv)), _ptr(workspace), wb,
                           _stream(stream))
    if check:
        _check(s, "bqa_attn_bwd")
    return s


def bqa_attn_fwd_ptq(p, q=None, k=None, v=None, q_means=None, o=None, lse=None, workspace=None,
                     workspace_bytes=None, stream=None, check=True) -> int:
    od = o if (o is None or isinstance(o, bqa_tensor)) else dense(o)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_attn_fwd_ptq(C.byref(p), _ref(q), _ref(k), _ref(v), _ptr(q_means), _ref(od), _ptr(lse),
                               _ptr(workspace), wb, _stream(stream))
    if check:
        _check(s, "bqa_attn_fwd_ptq")
    return s


def bqa_attn_decode_static(p, q=None, k=None, v=None, q_hi=None, k_hi=None, v_hi=None, sel_idx=None, sel_cnt=None,
                           o=None, lse=None, stream=None, check=True) -> int:
    def dd(t):
        return t if (t is None or isinstance(t, bqa_tensor)) else dense(t)
    s = lib().bqa_attn_decode_static(C.byref(p), _ref(q), _ref(k), _ref(v), _ref(dd(q_hi)), _ref(dd(k_hi)),
                                     _ref(dd(v_hi)), _ptr(sel_idx), _ptr(sel_cnt), _ref(dd(o)), _ptr(lse),
                                     _stream(stream))
    if check:
        _check(s, "bqa_attn_decode_static")
    return s


def bqa_quantize_qknorm(p, role, x, out: bqa_qtensor, inv_norm=None, k_mean=None, workspace=None,
                        workspace_bytes=None, stream=None, check=True) -> int:
    xd = x if isinstance(x, bqa_tensor) else dense(x)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_quantize_qknorm(C.byref(p), int(role), _ref(xd), C.byref(out), _ptr(inv_norm), _ptr(k_mean),
                                  _ptr(workspace), wb, _stream(stream))
    if check:
        _check(s, "bqa_quantize_qknorm")
    return s


def bqa_attn_bwd_qknorm(p, q=None, k=None, v_hi=None, o_for_delta=None, lse=None, d_o=None, q_raw=None, k_raw=None,
                        q_inv_norm=None, k_inv_norm=None, dq=None, dk=None, dv=None, workspace=None,
                        workspace_bytes=None, stream=None, check=True) -> int:
    def dd(t):
        return t if (t is None or isinstance(t, bqa_tensor)) else dense(t)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_attn_bwd_qknorm(C.byref(p), _ref(q), _ref(k), _ref(dd(v_hi)), _ref(dd(o_for_delta)), _ptr(lse),
                                  _ref(dd(d_o)), _ref(dd(q_raw)), _ref(dd(k_raw)), _ptr(q_inv_norm),
                                  _ptr(k_inv_norm), _ref(dd(dq)), _ref(dd(dk)), _ref(dd(dv)), _ptr(workspace), wb,
                                  _stream(stream))
    if check:
        _check(s, "bqa_attn_bwd_qknorm")
    return s


def bqa_quantize_nvfp4(p, role, x, out, workspace=None, workspace_bytes=None, stream=None, check=True) -> int:
    def dd(t):
        return t if (t is None or isinstance(t, bqa_tensor)) else dense(t)
    wb = workspace_bytes if workspace_bytes is not None else (workspace.numel() * workspace.element_size()
                                                              if workspace is not None else 0)
    s = lib().bqa_quantize_nvfp4(C.byref(p), int(role), _ref(dd(x)), _ref(dd(out)), _ptr(workspace), wb,
                                 _stream(stream))
    if check:
        _check(s, "bqa_quantize_nvfp4")
    return s


def bqa_attn_fwd_thrift_nvfp4(p, q_nv=None, k_nv=None, v_nv=None, q_hi=None, k_hi=None, v_hi=None, sel_idx=None,
                              sel_cnt=None, o=None, lse=None, stream=None, check=True) -> int:
    def dd(t):
        return t if (t is None or isinstance(t, bqa_tensor)) else dense(t)
    s = lib().bqa_attn_fwd_thrift_nvfp4(C.byref(p), _ref(dd(q_nv)), _ref(dd(k_nv)), _ref(dd(v_nv)), _ref(dd(q_hi)),
                                        _ref(dd(k_hi)), _ref(dd(v_hi)), _ptr(sel_idx), _ptr(sel_cnt), _ref(dd(o)),
                                        _ptr(lse), _stream(stream))
    if check:
        _check(s, "bqa_attn_fwd_thrift_nvfp4")
    return s


def bqa_debug_probe(kind: int, grid: int, iters: int, src=None, dst=None, nbytes: int = 0, stream=None,
                    check=True) -> int:
    s = lib().bqa_debug_probe(int(kind), int(grid), int(iters), _ptr(src), _ptr(dst), int(nbytes), _stream(stream))
    if check:
        _check(s, "bqa_debug_probe")
    return s


def bqa_debug_mx_dequant(codes, scales, nblocks: int, out, stream=None, check=True) -> int:
    s = lib().bqa_debug_mx_dequant(_ptr(codes), _ptr(scales), int(nblocks), _ptr(out), _stream(stream))
    if check:
        _check(s, "bqa_debug_mx_dequant")
    return s


def bqa_debug_qk_scores(p, q: bqa_qtensor, k: bqa_qtensor, b: int, h: int, q_tile: int, k_tile: int, out,
                        stream=None, check=True) -> int:
    s = lib().bqa_debug_qk_scores(C.byref(p), C.byref(q), C.byref(k), b, h, q_tile, k_tile, _ptr(out),
                                  _stream(stream))
    if check:
        _check(s, "bqa_debug_qk_scores")
    return s
