"""GPU parity of the fully INT8 SageBwd backward (dP = dO V^T from INT8 codes
too; "SageBwd: A Trainable Low-bit Attention", Limitations) against the
oracle's INT8-dP variant, through the C ABI: V's token-block codes bit for
bit, dQ / dK / dV at N = 512 and 1024 and on sampled tiles of the full c3
shape.  A last test measures what the INT8 dP costs in accuracy: the error
of dQ and dK against exact fp64 gradients of the same bf16 inputs, for the
16-bit and the INT8 dP, printed as one JSON line."""
import json

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.helpers import SageOracle, assert_same, compare_outputs, tau_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_quantized_attention_amd as bqa
    bqa.lib()


def _run(w, int8_dp=True):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SageTrainStep, sage_problem, to_device
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_I8PV, q_block=128,
                     smooth_k=True, smooth_eps=1e-3)
    step = SageTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"),
                         to_device(dO, "bf16"), int8_dp=int8_dp)
    step.step()
    torch.cuda.synchronize()
    return p, step, (Q, K, V, dO)


def _oracle(oc, V, dO, h, vc, vs, qtiles=None, ktiles=None):
    tau = tau_for(V.shape[-1])
    O, lse = oc.forward(0, h, True, tau)
    return orc.sage_bwd(qc=oc.qc[h], qs=oc.qs[h], kc=oc.kc[h], ks=oc.ks[h], V=V[0, h], dO=dO[0, h],
                        O=orc.round_to(O, "bf16"), lse=lse.astype(np.float32), causal=True, tau=tau,
                        qtiles=qtiles, ktiles=ktiles, vc=None if vc is None else vc[h],
                        vs=None if vs is None else vs[h])


@pytest.mark.parametrize("N", [512, 1024])
def test_int8_dp_backward_small(N):
    w = wl.with_len(wl.WORKLOADS["c3"], N, hq=2, hkv=2)
    p, step, (Q, K, V, dO) = _run(w)
    vc, vs = orc.quant_i8_tokblock(V.reshape(-1, N, w.d), 64)
    assert_same(step.vc8.cpu().numpy().reshape(vc.shape), vc, "V token-block codes")
    assert_same(step.vs8.cpu().numpy().reshape(vs.shape), vs, "V token-block scales")
    oc = SageOracle(Q, K, V, q_block=128, eps=1e-3, pv="i8")
    g = [t.float().cpu().numpy() for t in (step.dq, step.dk, step.dv)]
    for h in range(2):
        ref = _oracle(oc, V, dO, h, vc, vs)
        for name, gi, ri in zip(("dQ", "dK", "dV"), g, ref):
            compare_outputs(gi[0, h], ri, "bf16", what=f"{name}[h={h}]")


@pytest.mark.slow
def test_int8_dp_backward_full_size_sampled():
    w = wl.WORKLOADS["c3"]
    p, step, (Q, K, V, dO) = _run(w)
    h = 3
    oc = SageOracle(Q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1], q_block=128, eps=1e-3, pv="i8")
    vc, vs = orc.quant_i8_tokblock(V[0, h:h + 1], 64)
    g = [t.float().cpu().numpy()[0, h] for t in (step.dq, step.dk, step.dv)]
    nqt, nkt = w.Nq // 128, w.Nk // 64
    for qt, kt in ((0, nkt - 1), (nqt - 1, 0)):
        dQ, dK, dV = _oracle(oc, V[:, h:h + 1], dO[:, h:h + 1], 0, vc, vs, qtiles=(qt, qt + 1), ktiles=(kt, kt + 1))
        compare_outputs(g[0][128 * qt:128 * qt + 128], dQ, "bf16", what=f"dQ tile {qt}")
        compare_outputs(g[1][64 * kt:64 * kt + 64], dK, "bf16", what=f"dK tile {kt}")
        compare_outputs(g[2][64 * kt:64 * kt + 64], dV, "bf16", what=f"dV tile {kt}")


def test_int8_dp_error_growth():
    """Relative L2 error of the GPU's dQ, dK against the exact gradients of
    the bf16 inputs (oracle, fp64, no quantisation), with dP in 16-bit and
    in INT8 (c3 recipe, N = 2048, two heads)."""
    w = wl.with_len(wl.WORKLOADS["c3"], 2048, hq=2, hkv=2)
    res, exact = {}, {}
    for mode in (False, True):
        p, step, (Q, K, V, dO) = _run(w, int8_dp=mode)
        g = [t.float().cpu().numpy() for t in (step.dq, step.dk)]
        errs = {"dQ": [], "dK": []}
        for h in range(2):
            if h not in exact:
                exact[h] = orc.ref_bwd(Q[0, h], K[0, h], V[0, h], dO[0, h], True, tau_for(w.d))
            ex = exact[h]
            for name, gi, ei in zip(("dQ", "dK"), g, ex[:2]):
                errs[name].append(float(np.linalg.norm(gi[0, h] - ei) / np.linalg.norm(ei)))
        res["int8_dp" if mode else "bf16_dp"] = {k: float(np.mean(v)) for k, v in errs.items()}
    print(json.dumps({"int8_dp_error": {"workload": "c3 recipe, N=2048, 2 heads, causal", **res}}), flush=True)
    for k in ("dQ", "dK"):
        assert res["int8_dp"][k] < 0.2 and res["bf16_dp"][k] < 0.2
        assert res["int8_dp"][k] >= 0.9 * res["bf16_dp"][k]
