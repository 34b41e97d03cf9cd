"""Pins of the oracle's fully-INT8 SageBwd variant (dP = dO V^T from INT8
codes as well; "SageBwd: A Trainable Low-bit Attention", Limitations, names
it as open):

* where dO (per 128-token block) and V (per 64-token block, a different
  power-of-two scale in every block) are exact on their INT8 grids, the
  INT8 dP equals the 16-bit one, so every gradient equals the 16-bit-dP
  oracle's to rounding — a transposed operand or a misindexed block scale
  fails it;
* on generic inputs the INT8 dP only perturbs the gradients slightly."""
import numpy as np

import oracle as orc
import workloads as wl
from tests.helpers import SageOracle, tau_for


def _exact_int8(rng, N, d, blk, exps):
    """Rows whose blocks of `blk` tokens are int8 codes times 2^e (e from
    `exps`, cycled), each block holding a +-127 so that its absmax scale is
    exactly 2^e."""
    codes = rng.integers(-127, 128, (N, d)).astype(np.float32)
    X = np.empty((N, d), np.float32)
    for b in range(N // blk):
        codes[b * blk, 0] = 127.0
        X[b * blk:(b + 1) * blk] = codes[b * blk:(b + 1) * blk] * np.float32(2.0 ** exps[b % len(exps)])
    return X


def _setup(V, dO, N=256, d=128):
    w = wl.with_len(wl.WORKLOADS["c3"], N, hq=1, hkv=1)
    Q, K = wl.build(w, "q"), wl.build(w, "k")
    oc = SageOracle(Q, K, V[None, None], q_block=128, eps=1e-3, pv="i8")
    tau = tau_for(d)
    O, lse = oc.forward(0, 0, True, tau)
    return oc, tau, orc.round_to(O, "bf16"), lse.astype(np.float32)


def test_int8_dp_equals_16bit_dp_on_exact_grids():
    rng = np.random.default_rng(21)
    N, d = 256, 128
    V = _exact_int8(rng, N, d, 64, (-7, -5, -9, -6))
    dO = _exact_int8(rng, N, d, 128, (-10, -8))
    oc, tau, O, lse = _setup(V, dO)
    vc, vs = orc.quant_i8_tokblock(V[None], 64)
    assert np.array_equal(vs[0], [2.0 ** e for e in (-7, -5, -9, -6)])
    args = dict(qc=oc.qc[0], qs=oc.qs[0], kc=oc.kc[0], ks=oc.ks[0], V=V, dO=dO, O=O, lse=lse, causal=True, tau=tau)
    ref = orc.sage_bwd(**args)
    got = orc.sage_bwd(**args, vc=vc[0], vs=vs[0], v_blk=64)
    for r, g in zip(ref, got):
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-15 * np.abs(r).max())


def test_int8_dp_perturbs_gradients_slightly():
    w = wl.with_len(wl.WORKLOADS["c3"], 256, hq=1, hkv=1)
    V, dO = wl.build(w, "v")[0, 0], wl.build(w, "do")[0, 0]
    oc, tau, O, lse = _setup(V, dO)
    vc, vs = orc.quant_i8_tokblock(V[None], 64)
    args = dict(qc=oc.qc[0], qs=oc.qs[0], kc=oc.kc[0], ks=oc.ks[0], V=V, dO=dO, O=O, lse=lse, causal=True, tau=tau)
    ref = orc.sage_bwd(**args)
    got = orc.sage_bwd(**args, vc=vc[0], vs=vs[0], v_blk=64)
    for r, g in zip(ref[:2], got[:2]):                     # dQ, dK change; dV does not use dP
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        assert 0.0 < rel < 0.1, rel
    np.testing.assert_array_equal(got[2], ref[2])
