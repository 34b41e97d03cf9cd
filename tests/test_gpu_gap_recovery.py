"""Synthetic analogue of ThriftAttention's gap-recovery figures ("ThriftAttention"
technical summary, Results: the share of the FP4-to-16-bit quality gap that
the method recovers at 5, 10 and 25 % high-precision budgets).

The pages measure model quality; here the measure is the attention output
itself on the c5 recipe (low-rank, block-structured inputs, N = 131072,
causal, the first 8 query heads and 2 KV heads of the c5 workload): the
relative L2 error of O on sampled query rows against exact fp64 attention of
the bf16 inputs (the oracle), for
  * every pair through the FP4 path (selection counts forced to 0),
  * the Thrift selection at budgets 5, 10 and 25 %,
  * every valid pair through the bf16 path (budget 100 %).
Gap recovery at budget rho = (E_fp4 - E_rho) / (E_fp4 - E_bf16).  The
errors must fall as the budget grows and the recovery must be positive; the
figures are printed as one JSON line."""
import json

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.helpers import tau_for

pytestmark = pytest.mark.gpu

BUDGETS = (50_000, 100_000, 250_000)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _rel_err(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.slow
def test_gap_recovery_c5_recipe():
    from bit_quantized_attention_amd.runner import ThriftNvPath, ThriftPath, thrift_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c5"], 131072, hq=8, hkv=2)
    nw = wl.default_workers()
    Q, K, V = (wl.build(w, t, workers=nw) for t in ("q", "k", "v"))
    qd, kd, vd = (to_device(x, "bf16") for x in (Q, K, V))
    tau = tau_for(w.d)
    # sampled rows: 32-row blocks early, middle and late in the sequence, two query heads
    samples = [(h, r0) for h in (0, 5) for r0 in (8192 - 32, 65536 - 32, 131072 - 32)]
    exact = {}
    for h, r0 in samples:
        hk = h // (w.Hq // w.Hkv)
        O, _ = orc.ref_fwd(Q[0, h, r0:r0 + 32], K[0, hk, :r0 + 32], V[0, hk, :r0 + 32], True, tau)
        exact[(h, r0)] = O

    def run(ppm, force_fp4=False, nv=False):
        p = thrift_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, budget_ppm=ppm)
        path = (ThriftNvPath if nv else ThriftPath)(p, qd, kd, vd)
        path.quantize()
        path.select()
        if force_fp4:
            path.sel_cnt.zero_()
        path.forward()
        torch.cuda.synchronize()
        O = path.o.float().cpu().numpy()
        del path
        got = np.concatenate([O[0, h, r0:r0 + 32] for h, r0 in samples])
        ref = np.concatenate([exact[s] for s in samples])
        return _rel_err(got, ref)

    e_bf16 = run(1_000_000)
    out = {}
    for fmt, nv in (("mxfp4", False), ("nvfp4_emulated", True)):
        e_fp4 = run(0, force_fp4=True, nv=nv)
        e = {ppm: run(ppm, nv=nv) for ppm in BUDGETS}
        rec = {ppm: (e_fp4 - e[ppm]) / (e_fp4 - e_bf16) for ppm in BUDGETS}
        out[fmt] = {"rel_l2_error": {"fp4_only": e_fp4, "bf16_only": e_bf16,
                                     **{f"budget_{ppm / 1e4:g}%": e[ppm] for ppm in BUDGETS}},
                    "recovery": {f"budget_{ppm / 1e4:g}%": rec[ppm] for ppm in BUDGETS}}
        assert e_bf16 < e_fp4
        assert rec[BUDGETS[0]] > 0.0
        for a, b in zip(BUDGETS, BUDGETS[1:]):
            assert e[b] <= e[a] * 1.02, (fmt, a, b, e)
        assert e[BUDGETS[-1]] < e_fp4 and e[BUDGETS[-1]] > e_bf16 * 0.98
    print(json.dumps({"gap_recovery": {"workload": "c5 recipe, Hq=8 Hkv=2 N=131072 causal, 192 sampled rows",
                                       **out}}), flush=True)
