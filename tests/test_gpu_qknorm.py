"""GPU parity of QK-norm fused into the SageBwd path ("SageBwd: A Trainable
Low-bit Attention", Methodology 4, and the recommended SageBwd + QK-norm +
K-smoothing recipe), through the C ABI: the fused quantiser's inverse norms,
codes, scales and smoothing mean bit for bit against the oracle's QK-norm
followed by its quantisers; then the whole training step, whose dQ and dK
are gradients of the raw rows (the oracle's backward on its normalised rows,
then its QK-norm backward)."""
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


def _run(w):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SageQkNormTrainStep, sage_problem, to_device
    Qr, Kr, V, dO = (wl.build(w, t) for t in ("qraw", "kraw", "v", "do"))
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_I8PV, q_block=128,
                     smooth_k=True, smooth_eps=1e-3)
    step = SageQkNormTrainStep(p, to_device(Qr, "bf16"), to_device(Kr, "bf16"), to_device(V, "bf16"),
                               to_device(dO, "bf16"))
    step.step()
    torch.cuda.synchronize()
    return p, step, (Qr, Kr, V, dO)


def _normalised(Qr, Kr):
    Yq, rq = orc.qk_norm(Qr)
    Yk, rk = orc.qk_norm(Kr)
    return Yq, rq, Yk, rk


def _grads(oc, Qr, Kr, rq, rk, V, dO, h, qtiles=None, ktiles=None):
    """The oracle's forward and backward on its normalised rows (head h of
    oc), then the QK-norm backward to the raw rows."""
    tau = tau_for(Qr.shape[-1])
    O, lse = oc.forward(0, h, True, tau)
    dQn, dKn, dV = orc.sage_bwd(qc=oc.qc[h], qs=oc.qs[h], kc=oc.kc[h], ks=oc.ks[h], V=V[0, h], dO=dO[0, h],
                                O=orc.round_to(O, "bf16"), lse=lse.astype(np.float32), causal=True, tau=tau,
                                qtiles=qtiles, ktiles=ktiles)
    q0, q1 = (0, Qr.shape[2]) if qtiles is None else (128 * qtiles[0], 128 * qtiles[1])
    k0, k1 = (0, Kr.shape[2]) if ktiles is None else (64 * ktiles[0], 64 * ktiles[1])
    dQ = orc.qk_norm_bwd(Qr[0, h, q0:q1], rq[0, h, q0:q1], dQn)
    dK = orc.qk_norm_bwd(Kr[0, h, k0:k1], rk[0, h, k0:k1], dKn)
    return dQ, dK, dV


def test_fused_quantisation_bit_exact():
    w = wl.with_len(wl.WORKLOADS["c3"], 512, hq=2, hkv=2)
    p, step, (Qr, Kr, V, dO) = _run(w)
    Yq, rq, Yk, rk = _normalised(Qr, Kr)
    assert_same(step.q_rn.cpu().numpy(), rq, "Q inverse norms")
    assert_same(step.k_rn.cpu().numpy(), rk, "K inverse norms")
    oc = SageOracle(Yq, Yk, V, q_block=128, eps=1e-3, pv="i8")
    assert oc.uncertified == 0
    assert_same(step.mu.cpu().numpy().reshape(oc.mu.shape), oc.mu, "smoothing mean of the normalised K")
    assert_same(step.qc.cpu().numpy().reshape(oc.qc.shape), oc.qc, "Q codes")
    assert_same(step.qs.cpu().numpy().reshape(oc.qs.shape), oc.qs, "Q scales")
    assert_same(step.kc.cpu().numpy().reshape(oc.kc.shape), oc.kc, "K codes")
    assert_same(step.ks.cpu().numpy().reshape(oc.ks.shape), oc.ks, "K scales")


def test_zero_rows_and_scaled_rows():
    """A zero row stays zero (inverse norm 0); a row scaled by 2^k gives the
    same codes and an inverse norm scaled by 2^-k."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import sage_problem, to_device
    rng = np.random.default_rng(2)
    N, d = 128, 128
    X = wl.round_to(rng.standard_normal((1, 1, N, d)).astype(np.float32), "bf16").reshape(1, 1, N, d)
    X[0, 0, 5] = 0.0
    X[0, 0, 9] = X[0, 0, 8] * 8.0
    p = sage_problem(1, 1, 1, N, N, d, True, bqa.BQA_SAGE_I8_I8PV, q_block=128)
    codes = torch.empty((1, 1, N, d), dtype=torch.int8, device="cuda")
    scl = torch.empty((1, 1, 1), dtype=torch.float32, device="cuda")
    rn = torch.empty((1, 1, N), dtype=torch.float32, device="cuda")
    bqa.bqa_quantize_qknorm(p, bqa.BQA_ROLE_Q, to_device(X, "bf16"), bqa.qtensor(bqa.BQA_INT8, 0, 128, codes, scl),
                            inv_norm=rn)
    torch.cuda.synchronize()
    c, r = codes.cpu().numpy()[0, 0], rn.cpu().numpy()[0, 0]
    assert r[5] == 0.0 and np.all(c[5] == 0)
    assert r[9] == r[8] / 8.0 and np.array_equal(c[9], c[8])


@pytest.mark.parametrize("N", [512, 1024])
def test_qknorm_training_step_small(N):
    w = wl.with_len(wl.WORKLOADS["c3"], N, hq=2, hkv=2)
    p, step, (Qr, Kr, V, dO) = _run(w)
    Yq, rq, Yk, rk = _normalised(Qr, Kr)
    oc = SageOracle(Yq, Yk, V, q_block=128, eps=1e-3, pv="i8")
    g = [t.float().cpu().numpy() for t in (step.dq, step.dk, step.dv)]
    for h in range(2):
        ref = _grads(oc, Qr, Kr, rq, rk, V, dO, h)
        for name, gi, ri in zip(("dQ", "dK", "dV"), g, ref):
            compare_outputs(gi[0, h], ri, "bf16", what=f"{name}[h={h}]")


@pytest.mark.slow
def test_qknorm_training_step_full_size_sampled():
    """Full c3 shape (B=1, H=16, N=8192, causal) from raw rows: sampled tiles
    of one head against the oracle."""
    w = wl.WORKLOADS["c3"]
    p, step, (Qr, Kr, V, dO) = _run(w)
    h = 6
    Yq, rq, Yk, rk = _normalised(Qr[:, h:h + 1], Kr[:, h:h + 1])
    oc = SageOracle(Yq, Yk, V[:, h:h + 1], q_block=128, eps=1e-3, pv="i8")
    g = [t.float().cpu().numpy()[0, h] for t in (step.dq, step.dk, step.dv)]
    nqt, nkt = w.Nq // 128, w.Nk // 64
    for qt, kt in ((0, nkt - 1), (nqt - 1, 0)):
        dQ, dK, dV = _grads(oc, Qr[:, h:h + 1], Kr[:, h:h + 1], rq, rk, V[:, h:h + 1], dO[:, h:h + 1], 0,
                            qtiles=(qt, qt + 1), ktiles=(kt, kt + 1))
        compare_outputs(g[0][128 * qt:128 * qt + 128], dQ, "bf16", what=f"dQ tile {qt}")
        compare_outputs(g[1][64 * kt:64 * kt + 64], dK, "bf16", what=f"dK tile {kt}")
        compare_outputs(g[2][64 * kt:64 * kt + 64], dV, "bf16", what=f"dV tile {kt}")
