"""Shared pieces of the GPU parity tests: the oracle side of each path (the
oracle quantises the generated inputs itself; nothing it sees comes from the
GPU) and the comparison rules."""
from __future__ import annotations

import math

import numpy as np

import oracle as orc

MAX_ABS = 2e-2          # output tolerance: max |gpu - oracle| after both are in bf16
MEAN_REL = 1e-3         # and sum |gpu - oracle| / sum |oracle|


def assert_same(gpu, ref, what: str):
    """Bit-exact equality with a short report of the first mismatches."""
    g, r = np.asarray(gpu), np.asarray(ref)
    assert g.shape == r.shape, f"{what}: shape {g.shape} != {r.shape}"
    if g.dtype.kind == "f":
        bad = g.view(np.uint32 if g.itemsize == 4 else np.uint64) != r.astype(g.dtype).view(
            np.uint32 if g.itemsize == 4 else np.uint64)
    else:
        bad = g != r
    n = int(bad.sum())
    if n:
        idx = np.argwhere(bad)[:5]
        ex = [(tuple(int(t) for t in i), g[tuple(i)].item(), r[tuple(i)].item()) for i in idx]
        raise AssertionError(f"{what}: {n} of {g.size} differ, e.g. {ex}")


def ulp(x: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of the storage format's grid at |x| (bf16: 8 significant bits,
    fp16: 11, with fp16's subnormal floor)."""
    mant, emin = {"bf16": (7, -126), "fp16": (10, -14)}[fmt]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - mant)


def compare_outputs(gpu: np.ndarray, ref64: np.ndarray, fmt: str = "bf16", what: str = "O"):
    """GPU output (already in its storage dtype, as float) against the oracle's
    fp64 output rounded to the same storage format.

    Max-abs bound: MAX_ABS on the values before their final rounding, so each
    element may differ by MAX_ABS plus one unit of the storage grid at the
    reference value (two nearly equal values can round to neighbouring grid
    points).  Mean-rel bound: MEAN_REL on the stored values."""
    ref = orc.round_to(ref64, fmt)
    g = np.asarray(gpu, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    diff = np.abs(g - ref)
    excess = diff - ulp(ref, fmt)
    max_abs = float(diff.max())
    worst = float(excess.max())
    mean_rel = float(diff.sum() / max(np.abs(ref).sum(), 1e-300))
    assert worst <= MAX_ABS and mean_rel <= MEAN_REL, \
        f"{what}: max_abs {max_abs:.3e} (beyond one grid unit: {worst:.3e}) mean_rel {mean_rel:.3e}"
    return max_abs, mean_rel


class SageOracle:
    """Oracle quantisation of a Sage workload's inputs ([B, H, N, d] fp32)."""

    def __init__(self, Q, K, V, *, q_block, k_block=64, eps=0.0, smooth=True, pv="f8"):
        B, Hq, Nq, d = Q.shape
        Hkv, Nk = K.shape[1], K.shape[2]
        self.B, self.Hq, self.Hkv, self.Nq, self.Nk, self.d = B, Hq, Hkv, Nq, Nk, d
        self.q_block, self.k_block, self.pv = q_block, k_block, pv
        self.V = V
        Qf, Kf, Vf = (x.reshape(-1, x.shape[2], d) for x in (Q, K, V))
        # the library takes eps as the fp32 value of the problem descriptor
        self.mu, self.uncertified = orc.smooth_mean(Kf, float(np.float32(eps))) if smooth else (None, 0)
        self.qc, self.qs = orc.quant_i8_tokblock(Qf, q_block)
        self.kc, self.ks = orc.quant_i8_tokblock(Kf, k_block, self.mu)
        self.vc = self.vs = None
        if pv in ("f8", "i8"):
            self.vc, self.vs = orc.quant_chan(Vf, "e4m3" if pv == "f8" else "i8")
        self.Vf = Vf

    def forward(self, b, h, causal, tau, rows=None):
        hk = h // (self.Hq // self.Hkv)
        iq, ik = b * self.Hq + h, b * self.Hkv + hk
        pv_mode = {"f16": orc.PV_F16, "f8": orc.PV_F8, "i8": orc.PV_I8}[self.pv]
        kw = dict(qk_mode=orc.QK_I8, qc=self.qc[iq], qs=self.qs[iq], q_blk=self.q_block, kc=self.kc[ik],
                  ks=self.ks[ik], k_blk=self.k_block, pv_mode=pv_mode, Nq=self.Nq, Nk=self.Nk, d=self.d,
                  causal=causal, tau=tau, kv_tile=self.k_block, rows=rows)
        if self.pv == "f16":
            kw["Vf"] = self.Vf[ik]
        else:
            kw["vc_t"], kw["vs"] = self.vc[ik], self.vs[ik]
        return orc.sage_fwd(**kw)


def tau_for(d: int) -> float:
    return float(np.float32(1.0) / np.float32(math.sqrt(d)))
