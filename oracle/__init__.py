"""NumPy front end of the C oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (built from
``oracle.c`` by :func:`build`) with functions over NumPy arrays; every
computation happens in the C file, whose header comment names the passages
of the source pages each function follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]

PV_NONE, PV_F16, PV_F8, PV_I8 = 0, 1, 2, 3
QK_I8, QK_F64 = 0, 1


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C11 + OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = C.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _declare(L):
    vp, i, d, f = C.c_void_p, C.c_int, C.c_double, C.c_float
    sig = {
        "orc_round_grid": (d, [d, i, i, d, i]),
        "orc_e4m3_encode": (C.c_uint8, [d]),
        "orc_e4m3_decode": (d, [C.c_uint8]),
        "orc_e2m1_encode": (C.c_uint8, [d]),
        "orc_e2m1_decode": (d, [C.c_uint8]),
        "orc_e8m0_exponent": (i, [f]),
        "orc_bf16_bits": (C.c_uint16, [d]),
        "orc_f16_bits": (C.c_uint16, [d]),
        "orc_bf16_value": (d, [d]),
        "orc_f16_value": (d, [d]),
        "orc_i8_encode": (C.c_int8, [f, f]),
        "orc_round_array": (None, [vp, C.c_int64, i, vp]),
        "orc_i8_scale": (None, [f, vp, vp]),
        "orc_smooth_mean": (i, [vp, i, i, i, d, vp]),
        "orc_quant_i8_tokblock": (None, [vp, vp, i, i, i, i, vp, vp]),
        "orc_quant_chan": (None, [vp, i, i, i, i, vp, vp]),
        "orc_quant_mx_rows": (None, [vp, i, i, i, vp, vp]),
        "orc_quant_mx_cols": (None, [vp, i, i, i, vp, vp]),
        "orc_block_means": (None, [vp, i, i, i, i, vp]),
        "orc_ref_fwd": (None, [vp, vp, vp, i, i, i, i, d, vp, vp]),
        "orc_ref_bwd": (None, [vp, vp, vp, vp, i, i, i, i, d, vp, vp, vp]),
        "orc_sage_fwd": (None, [i, vp, vp, i, vp, vp, i, vp, vp, i, vp, vp, vp,
                                i, i, i, i, d, i, i, i, vp, vp]),
        "orc_sage_bwd_v": (None, [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, d, i, i, i, i,
                                  i, i, i, i, vp, vp, i, vp, vp, vp]),
        "orc_sage_bwd": (None, [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, d, i, i, i, i,
                                i, i, i, i, vp, vp, vp]),
        "orc_mx_scores": (i, [vp, vp, vp, vp, i, i, i, vp]),
        "orc_qat_fwd": (None, [vp, vp, vp, vp, vp, vp, i, i, i, d, i, i, i, i, vp, vp, vp, vp]),
        "orc_qat_bwd": (None, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, d, i,
                               i, i, i, i, vp, vp, vp]),
        "orc_budget_count": (i, [i, i]),
        "orc_select_blocks": (None, [vp, vp, i, i, i, i, i, i, vp, vp]),
        "orc_thrift_fwd": (None, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i,
                                  i, i, i, i, i, i, d, i, i, i, vp, vp]),
        "orc_thrift_decode": (None, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, d,
                                     i, i, vp, vp]),
        "orc_ptq_fwd": (None, [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, d, i, i, vp, vp]),
        "orc_qk_norm": (None, [vp, C.c_int64, i, vp, vp]),
        "orc_nvfp4_fake": (None, [vp, i, i, i, i, vp]),
        "orc_thrift_fwd_nv": (None, [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, d, i, i, vp, vp]),
        "orc_qk_norm_bwd": (None, [vp, vp, vp, C.c_int64, i, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- scalars
def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


def e2m1_encode(x: float) -> int:
    return int(lib().orc_e2m1_encode(float(x)))


def e2m1_decode(c: int) -> float:
    return float(lib().orc_e2m1_decode(int(c)))


def e8m0_exponent(amax: float) -> int:
    return int(lib().orc_e8m0_exponent(float(amax)))


def i8_scale(amax: float):
    s, v = C.c_float(), C.c_float()
    lib().orc_i8_scale(float(amax), C.byref(s), C.byref(v))
    return s.value, v.value


def i8_encode(x: float, inv: float) -> int:
    return int(lib().orc_i8_encode(float(x), float(inv)))


def bf16_value(x: float) -> float:
    return float(lib().orc_bf16_value(float(x)))


def f16_value(x: float) -> float:
    return float(lib().orc_f16_value(float(x)))


def round_to(a: np.ndarray, fmt: str) -> np.ndarray:
    """Round an array to bf16 or fp16 values (nearest-even) with the oracle's encoder."""
    x = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty_like(x)
    lib().orc_round_array(_p(x), x.size, 0 if fmt == "bf16" else 1, _p(out))
    return out


# ---------------------------------------------------------------- quantisers
def smooth_mean(K: np.ndarray, eps: float):
    """K [BH, N, d] -> (mu_eff [BH, d] fp32, number of uncertified channel sums)."""
    K = _f32(K)
    BH, N, d = K.shape
    mu = np.empty((BH, d), np.float32)
    bad = lib().orc_smooth_mean(_p(K), BH, N, d, float(eps), _p(mu))
    return mu, bad


def quant_i8_tokblock(X: np.ndarray, blk: int, mu: np.ndarray | None = None):
    X = _f32(X)
    BH, N, d = X.shape
    codes = np.empty((BH, N, d), np.int8)
    scales = np.empty((BH, N // blk), np.float32)
    lib().orc_quant_i8_tokblock(_p(X), _p(None if mu is None else _f32(mu)), BH, N, d, blk,
                                _p(codes), _p(scales))
    return codes, scales


def quant_chan(V: np.ndarray, fmt: str):
    """fmt 'i8' or 'e4m3'; codes channel-major [BH, d, N] (uint8 storage), scales [BH, d]."""
    V = _f32(V)
    BH, N, d = V.shape
    codes = np.empty((BH, d, N), np.uint8)
    scales = np.empty((BH, d), np.float32)
    lib().orc_quant_chan(_p(V), BH, N, d, 0 if fmt == "i8" else 1, _p(codes), _p(scales))
    return codes, scales


def quant_mx_rows(X: np.ndarray):
    X = _f32(X)
    BH, N, d = X.shape
    codes = np.empty((BH, N, d // 2), np.uint8)
    scales = np.empty((BH, N, d // 32), np.uint8)
    lib().orc_quant_mx_rows(_p(X), BH, N, d, _p(codes), _p(scales))
    return codes, scales


def quant_mx_cols(X: np.ndarray):
    X = _f32(X)
    BH, N, d = X.shape
    codes = np.empty((BH, d, N // 2), np.uint8)
    scales = np.empty((BH, d, N // 32), np.uint8)
    lib().orc_quant_mx_cols(_p(X), BH, N, d, _p(codes), _p(scales))
    return codes, scales


def smooth_q_blocks(Q: np.ndarray, blk: int = 128):
    """Query smoothing of the post-training FP4 baseline ("Attn-QAT"
    technical summary §1: the SageAttention3-style method smooths Q and K):
    per block of `blk` rows (the last block may be short) the mean of its
    rows, summed in fp64 and rounded to fp32 as the block means of
    block_means are, then rounded to bf16: qbar [BH, nqb, d] (bf16 values
    held as fp32).  Returns (qbar, Q_s) with Q_s = fp32(Q - qbar) row by row."""
    Q = _f32(Q)
    BH, N, d = Q.shape
    nqb = (N + blk - 1) // blk
    qbar = np.empty((BH, nqb, d), np.float32)
    for I in range(nqb):
        rows = Q[:, I * blk:(I + 1) * blk].astype(np.float64)
        s = np.zeros((BH, d))
        for t in range(rows.shape[1]):           # token order
            s += rows[:, t]
        qbar[:, I] = round_to((s / rows.shape[1]).astype(np.float32), "bf16")
    Qs = (Q - np.repeat(qbar, blk, axis=1)[:, :N]).astype(np.float32)
    return qbar, Qs


def qk_norm(X: np.ndarray):
    """QK-norm forward ("SageBwd" Methodology 4): X [..., d] -> (Y, r) with
    r = fp32(1/sqrt(sum x^2)) per row and Y = bf16(fp32(x r))."""
    X = _f32(X)
    d = X.shape[-1]
    rows = X.size // d
    Y = np.empty_like(X)
    r = np.empty(X.shape[:-1], np.float32)
    lib().orc_qk_norm(_p(X), rows, d, _p(Y), _p(r))
    return Y, r


def qk_norm_bwd(X: np.ndarray, r: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Gradient with respect to the raw rows X of y = x / |x| given dL/dy = G."""
    X = _f32(X)
    d = X.shape[-1]
    G = np.ascontiguousarray(G, dtype=np.float64)
    dX = np.empty(X.shape, np.float64)
    lib().orc_qk_norm_bwd(_p(X), _p(_f32(r)), _p(G), X.size // d, d, _p(dX))
    return dX


def smooth_k(K: np.ndarray, eps: float = 0.0):
    """Key smoothing as in the SageAttention path (token mean per channel,
    mu = fp32(S/N - eps)); returns (mu [BH, d], K_s = fp32(K - mu))."""
    K = _f32(K)
    mu, _ = smooth_mean(K, eps)
    return mu, (K - mu[:, None, :]).astype(np.float32)


def block_means(X: np.ndarray, blk: int) -> np.ndarray:
    X = _f32(X)
    BH, N, d = X.shape
    out = np.empty((BH, N // blk, d), np.float32)
    lib().orc_block_means(_p(X), BH, N, d, blk, _p(out))
    return out


# ---------------------------------------------------------------- attention
def ref_fwd(Q, K, V, causal: bool, tau: float):
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    Nq, d = Q.shape
    Nk = K.shape[0]
    O = np.empty((Nq, d), np.float64)
    lse = np.empty(Nq, np.float64)
    lib().orc_ref_fwd(_p(Q), _p(K), _p(V), Nq, Nk, d, int(causal), float(tau), _p(O), _p(lse))
    return O, lse


def ref_bwd(Q, K, V, dO, causal: bool, tau: float):
    Q, K, V, dO = _f32(Q), _f32(K), _f32(V), _f32(dO)
    Nq, d = Q.shape
    Nk = K.shape[0]
    dQ = np.empty((Nq, d)); dK = np.empty((Nk, d)); dV = np.empty((Nk, d))
    lib().orc_ref_bwd(_p(Q), _p(K), _p(V), _p(dO), Nq, Nk, d, int(causal), float(tau),
                      _p(dQ), _p(dK), _p(dV))
    return dQ, dK, dV


def sage_fwd(*, qk_mode=QK_I8, qc=None, qs=None, q_blk=128, kc=None, ks=None, k_blk=64,
             Qf=None, Kf=None, pv_mode=PV_F8, Vf=None, vc_t=None, vs=None,
             Nq, Nk, d, causal, tau, kv_tile=64, rows=None):
    r0, r1 = (0, Nq) if rows is None else rows
    O = np.empty((r1 - r0, d), np.float64)
    lse = np.empty(r1 - r0, np.float64)
    args = [_c(qc, np.int8) if qc is not None else None, _f32(qs) if qs is not None else None,
            _c(kc, np.int8) if kc is not None else None, _f32(ks) if ks is not None else None,
            _f32(Qf) if Qf is not None else None, _f32(Kf) if Kf is not None else None,
            _f32(Vf) if Vf is not None else None, _c(vc_t, np.uint8) if vc_t is not None else None,
            _f32(vs) if vs is not None else None]
    qc_, qs_, kc_, ks_, Qf_, Kf_, Vf_, vc_, vs_ = args
    lib().orc_sage_fwd(qk_mode, _p(qc_), _p(qs_), q_blk, _p(kc_), _p(ks_), k_blk, _p(Qf_), _p(Kf_),
                       pv_mode, _p(Vf_), _p(vc_), _p(vs_), Nq, Nk, d, int(causal), float(tau),
                       kv_tile, r0, r1, _p(O), _p(lse))
    return O, lse


def sage_bwd(*, qc, qs, kc, ks, V, dO, O, lse, causal, tau, tile_q=128, tile_k=64, do_blk=128,
             quantize=True, qtiles=None, ktiles=None, vc=None, vs=None, v_blk=64):
    """SageBwd backward of one head; with vc / vs (V's INT8 codes per v_blk
    tokens) dP = dO V^T runs in INT8 as well (the fully INT8 variant)."""
    N, d = V.shape
    qt0, qt1 = (0, N // tile_q) if qtiles is None else qtiles
    kt0, kt1 = (0, N // tile_k) if ktiles is None else ktiles
    dQ = np.empty(((qt1 - qt0) * tile_q, d)); dK = np.empty(((kt1 - kt0) * tile_k, d))
    dV = np.empty_like(dK)
    a = [_c(qc, np.int8), _f32(qs), _c(kc, np.int8), _f32(ks), _f32(V), _f32(dO), _f32(O), _f32(lse)]
    vcc = None if vc is None else _c(vc, np.int8)
    vss = None if vs is None else _f32(vs)
    lib().orc_sage_bwd_v(*[_p(x) for x in a], N, d, int(causal), float(tau), tile_q, tile_k, do_blk,
                         int(quantize), qt0, qt1, kt0, kt1, _p(vcc), _p(vss), int(v_blk), _p(dQ), _p(dK), _p(dV))
    return dQ, dK, dV


def mx_score(qc, qs, kc, ks, d, i, j):
    s = C.c_double()
    ok = lib().orc_mx_scores(_p(qc), _p(qs), _p(kc), _p(ks), d, i, j, C.byref(s))
    return s.value, bool(ok)


def qat_fwd(*, qc, qs, kc, ks, vc_t, vs_t, Nq, Nk, d, tau, kv_tile=128, quantize_p=True, rows=None,
            return_rowmax=False):
    """O, O', lse (and with return_rowmax the rows' final running maxima tau*s)."""
    r0, r1 = (0, Nq) if rows is None else rows
    O = np.empty((r1 - r0, d)); Oa = np.empty((r1 - r0, d)); lse = np.empty(r1 - r0); mrow = np.empty(r1 - r0)
    a = [_c(x, np.uint8) for x in (qc, qs, kc, ks, vc_t, vs_t)]
    lib().orc_qat_fwd(*[_p(x) for x in a], Nq, Nk, d, float(tau), kv_tile, int(quantize_p), r0, r1,
                      _p(O), _p(Oa), _p(lse), _p(mrow))
    return (O, Oa, lse, mrow) if return_rowmax else (O, Oa, lse)


def qat_bwd(*, qc, qs, kc, ks, vc_t, vs_t, dO, O_aux, lse, Nq, Nk, d, tau, quantize_p=True,
            qrows=None, krows=None, rowmax=None):
    """rowmax: the rows' final running maxima from the forward (fp64, all Nq
    rows); None takes them here from the scores of every key."""
    q0, q1 = (0, Nq) if qrows is None else qrows
    k0, k1 = (0, Nk) if krows is None else krows
    dQ = np.empty((q1 - q0, d)); dK = np.empty((k1 - k0, d)); dV = np.empty((k1 - k0, d))
    a = [_c(x, np.uint8) for x in (qc, qs, kc, ks, vc_t, vs_t)] + [_f32(dO), _f32(O_aux), _f32(lse)]
    mr = None if rowmax is None else _c(rowmax, np.float64)
    lib().orc_qat_bwd(*[_p(x) for x in a], _p(mr), Nq, Nk, d, float(tau), int(quantize_p), q0, q1, k0, k1,
                      _p(dQ), _p(dK), _p(dV))
    return dQ, dK, dV


def budget_count(n_valid: int, ppm: int) -> int:
    return int(lib().orc_budget_count(int(n_valid), int(ppm)))


def select_blocks(qbar, kbar, causal: bool, budget_ppm: int, max_sel: int):
    qbar, kbar = _f32(qbar), _f32(kbar)
    nqb, d = qbar.shape
    nkb = kbar.shape[0]
    idx = np.empty((nqb, max_sel), np.int32)
    cnt = np.empty(nqb, np.int32)
    lib().orc_select_blocks(_p(qbar), _p(kbar), nqb, nkb, d, int(causal), int(budget_ppm), max_sel,
                            _p(idx), _p(cnt))
    return idx, cnt


def thrift_fwd(*, qc, qs, kc, ks, vc_t, vs_t, Qh, Kh, Vh, sel_idx, sel_cnt, Nq, Nk, d, blk=128, hp_tile=None,
               causal=True, tau, quantize=True, qblocks=None):
    """hp_tile: keys per online-softmax tile of the bf16 path (default: the whole block)."""
    qb0, qb1 = (0, Nq // blk) if qblocks is None else qblocks
    O = np.empty(((qb1 - qb0) * blk, d)); lse = np.empty((qb1 - qb0) * blk)
    sel_idx = _c(sel_idx, np.int32)
    a = [_c(x, np.uint8) if x is not None else None for x in (qc, qs, kc, ks, vc_t, vs_t)]
    lib().orc_thrift_fwd(*[_p(x) for x in a], _p(_f32(Qh)), _p(_f32(Kh)), _p(_f32(Vh)),
                         _p(sel_idx), _p(_c(sel_cnt, np.int32)), sel_idx.shape[1], Nq, Nk, d, blk,
                         blk if hp_tile is None else hp_tile, int(causal), float(tau), int(quantize), qb0, qb1, _p(O), _p(lse))
    return O, lse


def thrift_decode(*, qc, qs, kc, ks, vc_t, vs_t, q, Kh, Vh, sel, Nk, d, blk=128, hp_tile=None, tau, num_splits,
                  quantize=True):
    o = np.empty(d)
    lse = C.c_double()
    sel = _c(sel, np.int32)
    a = [_c(x, np.uint8) if x is not None else None for x in (qc, qs, kc, ks, vc_t, vs_t)]
    lib().orc_thrift_decode(*[_p(x) for x in a], _p(_f32(q)), _p(_f32(Kh)), _p(_f32(Vh)), _p(sel),
                            len(sel), Nk, d, blk, blk if hp_tile is None else hp_tile, float(tau), int(num_splits),
                            int(quantize),
                            _p(o), C.byref(lse))
    return o, lse.value


def ptq_fwd(*, qc, qs, qbar, kc, ks, vc_t, vs_t, Nq, Nk, d, blk=128, causal=False, tau, qblocks=None):
    """Post-training FP4 forward (query and key smoothing, two-level P) of one
    head: qc/qs the MXFP4 codes of the smoothed Q, qbar [nqb, d] its bf16
    block means, kc/ks those of the smoothed K.  Returns (O, lse) for the rows
    of query blocks `qblocks` (default all)."""
    nqb = (Nq + blk - 1) // blk
    qb0, qb1 = (0, nqb) if qblocks is None else qblocks
    rows = min(Nq, qb1 * blk) - qb0 * blk
    O = np.empty((rows, d)); lse = np.empty(rows)
    a = [_c(x, np.uint8) for x in (qc, qs)]
    b = [_c(x, np.uint8) for x in (kc, ks, vc_t, vs_t)]
    lib().orc_ptq_fwd(_p(a[0]), _p(a[1]), _p(_f32(qbar)), *[_p(x) for x in b], Nq, Nk, d, blk, int(causal),
                      float(tau), qb0, qb1, _p(O), _p(lse))
    return O, lse


def nvfp4_fake(X: np.ndarray, axis: int) -> np.ndarray:
    """NVFP4 emulation ("ThriftAttention", Method step 2): X [BH, N, d] ->
    the dequantised NVFP4 values (blocks of 16 along d for axis 0, along the
    tokens of each channel for axis 1; E4M3 block scales; a power-of-two
    tensor scale per slice)."""
    X = _f32(X)
    BH, N, d = X.shape
    out = np.empty_like(X)
    lib().orc_nvfp4_fake(_p(X), BH, N, d, int(axis), _p(out))
    return out


def thrift_fwd_nv(*, Qn, Kn, Vn, Qh, Kh, Vh, sel_idx, sel_cnt, Nq, Nk, d, blk=128, hp_tile=64, causal=True, tau,
                  qblocks=None):
    """Thrift prefill with the FP4 path in NVFP4 emulation (dequantised NVFP4
    Qn, Kn, Vn; two-level NVFP4 P; tiles of hp_tile keys)."""
    qb0, qb1 = (0, Nq // blk) if qblocks is None else qblocks
    O = np.empty(((qb1 - qb0) * blk, d)); lse = np.empty((qb1 - qb0) * blk)
    sel_idx = _c(sel_idx, np.int32)
    lib().orc_thrift_fwd_nv(*[_p(_f32(x)) for x in (Qn, Kn, Vn, Qh, Kh, Vh)], _p(sel_idx),
                            _p(_c(sel_cnt, np.int32)), sel_idx.shape[1], Nq, Nk, d, blk, hp_tile, int(causal),
                            float(tau), qb0, qb1, _p(O), _p(lse))
    return O, lse

