"""GPU parity of the SageBwd INT8 backward against the oracle, through the C
ABI: QK-norm inputs with K-smoothing (eps = 1e-3), INT8 Q/K/dO/P/dS with the
bf16 dP = dO V^T; dQ, dK, dV within max-abs 2e-2 and mean-rel 1e-3 of the
oracle rounded to bf16.  The oracle runs its own forward (O, log-sum-exp)
on its own quantisation of the same generated inputs."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.helpers import SageOracle, compare_outputs, tau_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_quantized_attention_amd as bqa
    bqa.lib()


def _run(w):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SageTrainStep, sage_problem, to_device
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_I8PV, q_block=128,
                     smooth_k=True, smooth_eps=1e-3)
    step = SageTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), to_device(dO, "bf16"))
    step.step()
    torch.cuda.synchronize()
    return p, step, (Q, K, V, dO)


def _oracle_grads(oc, Q, V, dO, h, causal, qtiles=None, ktiles=None):
    tau = tau_for(Q.shape[-1])
    O, lse = oc.forward(0, h, causal, tau)
    O16 = orc.round_to(O, "bf16")
    return orc.sage_bwd(qc=oc.qc[h], qs=oc.qs[h], kc=oc.kc[h], ks=oc.ks[h], V=V[0, h], dO=dO[0, h], O=O16,
                        lse=lse.astype(np.float32), causal=causal, tau=tau, qtiles=qtiles, ktiles=ktiles)


@pytest.mark.parametrize("N", [512, 1024])
def test_sage_backward_small(N):
    w = wl.with_len(wl.WORKLOADS["c3"], N, hq=2, hkv=2)
    p, step, (Q, K, V, dO) = _run(w)
    oc = SageOracle(Q, K, V, q_block=128, eps=1e-3, pv="i8")
    g = [t.float().cpu().numpy() for t in (step.dq, step.dk, step.dv)]
    for h in range(2):
        ref = _oracle_grads(oc, Q, V, dO, h, True)
        for name, gi, ri in zip(("dQ", "dK", "dV"), g, ref):
            compare_outputs(gi[0, h], ri, "bf16", what=f"{name}[h={h}]")


def test_sage_backward_zero_do_tile():
    """A query tile whose dO rows are all zero: its dO block quantises to
    scale 0 and zero codes, its dS tiles have maximum 0 (the zero-scale path
    of both product kernels: inverse scale 0, zero codes), so its dQ is
    exactly zero and it adds nothing to dK and dV.  All three against the
    oracle, which takes the same degenerate tiles."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SageTrainStep, sage_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c3"], 512, hq=1, hkv=1)
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    dO[0, 0, 128:256] = 0.0
    p = sage_problem(1, 1, 1, 512, 512, w.d, True, bqa.BQA_SAGE_I8_I8PV, q_block=128, smooth_k=True, smooth_eps=1e-3)
    step = SageTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), to_device(dO, "bf16"))
    step.step()
    torch.cuda.synchronize()
    assert not step.dq[0, 0, 128:256].any()
    oc = SageOracle(Q, K, V, q_block=128, eps=1e-3, pv="i8")
    ref = _oracle_grads(oc, Q, V, dO, 0, True)
    assert not ref[0][128:256].any()
    for name, gi, ri in zip(("dQ", "dK", "dV"), (step.dq, step.dk, step.dv), ref):
        compare_outputs(gi[0, 0].float().cpu().numpy(), ri, "bf16", what=f"{name} (zero dO tile)")


@pytest.mark.slow
def test_sage_backward_full_size_sampled():
    """Full c3 shape (B=1, H=16, N=8192, causal): the GPU runs the whole
    training step; the oracle runs its forward of one head and the backward
    of sampled tiles (dQ of the first and last query tiles, dK and dV of the
    first and last key tiles)."""
    w = wl.WORKLOADS["c3"]
    p, step, (Q, K, V, dO) = _run(w)
    h = 11
    oc = SageOracle(Q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1], q_block=128, eps=1e-3, pv="i8")
    g = [t.float().cpu().numpy()[0, h] for t in (step.dq, step.dk, step.dv)]
    nqt, nkt = w.Nq // 128, w.Nk // 64
    for qt, kt in ((0, nkt - 1), (nqt - 1, 0)):
        dQ, dK, dV = _oracle_grads(oc, Q[:, h:h + 1], V[:, h:h + 1], dO[:, h:h + 1], 0, True, qtiles=(qt, qt + 1),
                                   ktiles=(kt, kt + 1))
        compare_outputs(g[0][128 * qt:128 * qt + 128], dQ, "bf16", what=f"dQ tile {qt}")
        compare_outputs(g[1][64 * kt:64 * kt + 64], dK, "bf16", what=f"dK tile {kt}")
        compare_outputs(g[2][64 * kt:64 * kt + 64], dV, "bf16", what=f"dV tile {kt}")


def test_sage_backward_n2048_two_heads():
    """The c3 comparison length (B=1, H=16, N=2048), two heads checked whole."""
    w = wl.with_len(wl.WORKLOADS["c3"], 2048)
    p, step, (Q, K, V, dO) = _run(w)
    g = [t.float().cpu().numpy() for t in (step.dq, step.dk, step.dv)]
    for h in (0, 15):
        oc = SageOracle(Q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1], q_block=128, eps=1e-3, pv="i8")
        ref = _oracle_grads(oc, Q[:, h:h + 1], V[:, h:h + 1], dO[:, h:h + 1], 0, True)
        for name, gi, ri in zip(("dQ", "dK", "dV"), g, ref):
            compare_outputs(gi[0, h], ri, "bf16", what=f"{name}[h={h}]")
