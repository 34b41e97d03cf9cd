"""GPU parity of the Attn-QAT FP4 forward against the oracle, through the C ABI:
the MXFP4 scores of one tile, then O, O' and the log-sum-exp on the
heavy-tailed Student-t recipe (small, ragged, grouped heads, full size on
sampled rows)."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.helpers import assert_same, compare_outputs, tau_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_quantized_attention_amd as bqa
    bqa.lib()


def _run(w, Nq=None, aux=True):
    from bit_quantized_attention_amd.runner import QatPath, qat_problem, to_device
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    if Nq is not None:
        Q = np.ascontiguousarray(Q[:, :, :Nq])
    p = qat_problem(w.B, w.Hq, w.Hkv, Q.shape[2], K.shape[2], w.d)
    path = QatPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), aux=aux)
    path.step()
    torch.cuda.synchronize()
    return p, path, (Q, K, V)


class _Oracle:
    def __init__(self, Q, K, V):
        self.Hq, self.Hkv, self.Nq, self.Nk, self.d = Q.shape[1], K.shape[1], Q.shape[2], K.shape[2], Q.shape[3]
        self.qc, self.qs = orc.quant_mx_rows(Q.reshape(-1, self.Nq, self.d))
        self.kc, self.ks = orc.quant_mx_rows(K.reshape(-1, self.Nk, self.d))
        self.vc, self.vs = orc.quant_mx_cols(V.reshape(-1, self.Nk, self.d))

    def forward(self, b, h, rows=None, return_rowmax=False, kv_tile=64):
        """kv_tile: keys per online-softmax tile of the kernel compared against
        (64 for the forward with O', 128 for the inference forward)."""
        iq, ik = b * self.Hq + h, b * self.Hkv + h // (self.Hq // self.Hkv)
        return orc.qat_fwd(qc=self.qc[iq], qs=self.qs[iq], kc=self.kc[ik], ks=self.ks[ik], vc_t=self.vc[ik],
                           vs_t=self.vs[ik], Nq=self.Nq, Nk=self.Nk, d=self.d, tau=tau_for(self.d), kv_tile=kv_tile,
                           rows=rows, return_rowmax=return_rowmax)


def _check(path, oc, heads, rows=None):
    O = path.o.float().cpu().numpy()
    Oa = path.oa.float().cpu().numpy() if path.oa is not None else None
    L = path.lse.cpu().numpy()
    kv_tile = 64 if Oa is not None else 128
    for b, h in heads:
        r = rows or (0, oc.Nq)
        ref, ref_aux, lse = oc.forward(b, h, rows=r, kv_tile=kv_tile)
        compare_outputs(O[b, h, r[0]:r[1]], ref, "bf16", what=f"O[b={b},h={h},rows={r}]")
        if Oa is not None:
            compare_outputs(Oa[b, h, r[0]:r[1]], ref_aux, "bf16", what=f"O'[b={b},h={h},rows={r}]")
        assert np.abs(L[b, h, r[0]:r[1]] - lse).max() < 2e-3


def _fits_f32(x: float) -> bool:
    return float(np.float32(x)) == x


def test_mx_scores_tile():
    """One 32 x 32 tile of raw MXFP4 scores from the forward's tile code (one
    scaled 16x16x128 instruction per 16 keys over all 128 channels).  Where
    the oracle's exact rational score and its 64-channel partial sum are both
    fp32 values, the result is compared bit for bit; elsewhere within the
    rounding of one fp32 addition of two 64-channel partials."""
    import bit_quantized_attention_amd as bqa
    w = wl.with_len(wl.WORKLOADS["c4"], 256, hq=2, hkv=2)
    p, path, (Q, K, V) = _run(w)
    oc = _Oracle(Q, K, V)
    assert_same(path.qc.cpu().numpy().reshape(oc.qc.shape), oc.qc, "Q MX codes")
    assert_same(path.kc.cpu().numpy().reshape(oc.kc.shape), oc.kc, "K MX codes")
    out = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    n_exact = 0
    for (h, qt, kt) in ((0, 0, 0), (1, 3, 5), (1, 7, 2)):
        bqa.bqa_debug_qk_scores(p, path.qq, path.kq, 0, h, qt, kt, out)
        torch.cuda.synchronize()
        g = out.cpu().numpy()
        qch, qsh = np.ascontiguousarray(oc.qc[h][:, :32]), np.ascontiguousarray(oc.qs[h][:, :2])
        kch, ksh = np.ascontiguousarray(oc.kc[h][:, :32]), np.ascontiguousarray(oc.ks[h][:, :2])
        for i in range(32):
            for j in range(32):
                qi, kj = 32 * qt + i, 32 * kt + j
                ref, exact = orc.mx_score(oc.qc[h], oc.qs[h], oc.kc[h], oc.ks[h], 128, qi, kj)
                half, exact_h = orc.mx_score(qch, qsh, kch, ksh, 64, qi, kj)
                if exact and exact_h and _fits_f32(ref) and _fits_f32(half):
                    n_exact += 1
                    assert g[i, j] == np.float32(ref), (h, qt, kt, i, j, g[i, j], ref)
                else:
                    assert abs(float(g[i, j]) - ref) <= 2 * np.finfo(np.float32).eps * (abs(ref) + abs(half)), \
                        (h, qt, kt, i, j, g[i, j], ref)
    assert n_exact > 1000


@pytest.mark.parametrize("aux", [True, False], ids=["with_aux", "inference"])
@pytest.mark.parametrize("Nq,Nk,hq,hkv", [(512, 512, 2, 2), (1000, 1024, 4, 2), (64, 384, 1, 1), (200, 128, 2, 1)])
def test_qat_forward_small(Nq, Nk, hq, hkv, aux):
    """c4 recipe at sizes spanning several tiles: ragged query count, grouped
    heads, a single partial query tile, a single key tile; the forward with O'
    (tiles of 64 keys) and the inference forward (tiles of 128)."""
    w = wl.with_len(wl.WORKLOADS["c4"], Nk, hq=hq, hkv=hkv)
    p, path, (Q, K, V) = _run(w, Nq=Nq, aux=aux)
    oc = _Oracle(Q, K, V)
    assert_same(path.vc.cpu().numpy().reshape(oc.vc.shape), oc.vc, "V MX codes")
    _check(path, oc, [(0, h) for h in range(hq)])


@pytest.mark.parametrize("aux", [True, False], ids=["with_aux", "inference"])
def test_qat_forward_zero_blocks(aux):
    """Degenerate MXFP4 blocks: a whole query tile of zero rows (E8M0 scale
    byte 0, zero codes) scores exactly 0 against every key, so its rows have
    row maximum 0 and identical outputs; a key tile of zero rows scores 0
    against every query; a zero V channel gives exactly zero output.  O, O'
    and the log-sum-exp against the oracle."""
    from bit_quantized_attention_amd.runner import QatPath, qat_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c4"], 512, hq=1, hkv=1)
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    Q[0, 0, 128:256] = 0.0
    K[0, 0, 256:384] = 0.0
    V[0, 0, :, 5] = 0.0
    p = qat_problem(1, 1, 1, 512, 512, w.d)
    path = QatPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), aux=aux)
    path.step()
    torch.cuda.synchronize()
    oc = _Oracle(Q, K, V)
    assert_same(path.qc.cpu().numpy().reshape(oc.qc.shape), oc.qc, "Q MX codes")
    assert_same(path.qs.cpu().numpy().reshape(oc.qs.shape), oc.qs, "Q MX scales")
    assert not path.qc[0, 0, 128:256].any() and not path.qs[0, 0, 128:256].any()
    _check(path, oc, [(0, 0)])
    assert torch.equal(path.row_max[0, 0, 128:256], torch.zeros(128, device="cuda"))
    O = path.o[0, 0].float()
    assert torch.equal(O[128:256], O[128:129].expand(128, -1))
    assert not O[:, 5].any()
    if aux:
        assert not path.oa[0, 0, :, 5].float().any()


def test_qat_forward_variants_agree():
    """The inference forward and the forward with O' visit the keys in tiles
    of 128 and 64: their O differ by the MXFP4 rounding of P under different
    running maxima only, and their log-sum-exps by fp32 rounding."""
    w = wl.with_len(wl.WORKLOADS["c4"], 1024, hq=2, hkv=2)
    _, with_aux, _ = _run(w)
    _, no_aux, _ = _run(w, aux=False)
    a, b = with_aux.o.float().cpu().numpy(), no_aux.o.float().cpu().numpy()
    assert np.abs(a - b).sum() / np.abs(a).sum() < 2e-2
    assert torch.allclose(with_aux.lse, no_aux.lse, atol=2e-3, rtol=0)


@pytest.mark.slow
@pytest.mark.parametrize("aux", [True, False], ids=["with_aux", "inference"])
def test_qat_forward_full_size_sampled(aux):
    """Full c4 shape (B=1, H=32, N=16384, d=128, non-causal); the oracle checks
    sampled rows of sampled heads."""
    w = wl.WORKLOADS["c4"]
    p, path, (Q, K, V) = _run(w, aux=aux)
    oc = _Oracle(Q, K, V)
    for h in (0, 13, 31):
        for r0 in (0, 8191, 16384 - 16):
            _check(path, oc, [(0, h)], rows=(r0, r0 + 16))


def _train(w):
    from bit_quantized_attention_amd.runner import QatTrainStep, qat_problem, to_device
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    p = qat_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    step = QatTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), to_device(dO, "bf16"))
    step.step()
    torch.cuda.synchronize()
    return p, step, (Q, K, V, dO)


def _qat_grads(oc, dO, h, qrows=None, krows=None):
    """The oracle's own forward (O', log-sum-exp, stored as the GPU stores
    them: bf16 and fp32; the rows' maxima), then its backward."""
    _, Oa, lse, mrow = oc.forward(0, h, return_rowmax=True)
    return orc.qat_bwd(qc=oc.qc[h], qs=oc.qs[h], kc=oc.kc[h], ks=oc.ks[h], vc_t=oc.vc[h], vs_t=oc.vs[h],
                       dO=dO[0, h], O_aux=orc.round_to(Oa, "bf16"), lse=lse.astype(np.float32), rowmax=mrow,
                       Nq=oc.Nq, Nk=oc.Nk,
                       d=oc.d, tau=tau_for(oc.d), qrows=qrows, krows=krows)


@pytest.mark.parametrize("N", [256, 1024])
def test_qat_backward_small(N):
    """Attn-QAT backward on the Student-t recipe: dQ, dK, dV against the
    oracle's forward + backward on its own quantisation of the inputs."""
    w = wl.with_len(wl.WORKLOADS["c4"], N, hq=2, hkv=2)
    p, step, (Q, K, V, dO) = _train(w)
    oc = _Oracle(Q, K, V)
    g = [t.float().cpu().numpy() for t in (step.dq, step.dk, step.dv)]
    for h in range(2):
        ref = _qat_grads(oc, dO, h)
        for name, gi, ri in zip(("dQ", "dK", "dV"), g, ref):
            compare_outputs(gi[0, h], ri, "bf16", what=f"{name}[h={h}]")


@pytest.mark.slow
def test_qat_backward_full_size_sampled():
    """Full c4 training shape (B=1, H=32, N=16384): the oracle checks sampled
    query rows (dQ) and key rows (dK, dV) of one head."""
    w = wl.WORKLOADS["c4"]
    p, step, (Q, K, V, dO) = _train(w)
    h = 21
    oc = _Oracle(Q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1])
    g = [t.float().cpu().numpy()[0, h] for t in (step.dq, step.dk, step.dv)]
    for r0 in (0, 16384 - 32):
        dQ, dK, dV = _qat_grads(oc, dO[:, h:h + 1], 0, qrows=(r0, r0 + 32), krows=(r0, r0 + 32))
        compare_outputs(g[0][r0:r0 + 32], dQ, "bf16", what=f"dQ rows {r0}")
        compare_outputs(g[1][r0:r0 + 32], dK, "bf16", what=f"dK rows {r0}")
        compare_outputs(g[2][r0:r0 + 32], dV, "bf16", what=f"dV rows {r0}")


def test_qat_score_jump_rescales():
    """Keys after the first tile score more than 64 binades above it: the
    running maximum jumps (the first tile's sums scale to zero) and the
    result still matches."""
    from bit_quantized_attention_amd.runner import QatPath, qat_problem, to_device
    rng = np.random.default_rng(42)
    N, d = 256, 128
    Q, K, V = (rng.standard_t(3, (1, 1, N, d)).astype(np.float32) for _ in range(3))
    Q[..., 0] = 40.0
    K[0, 0, :64, 0] = -40.0
    K[0, 0, 64:, 0] = 40.0
    Q, K, V = (wl.round_to(x, "bf16").reshape(x.shape) for x in (Q, K, V))
    p = qat_problem(1, 1, 1, N, N, d)
    path = QatPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.step()
    torch.cuda.synchronize()
    oc = _Oracle(Q, K, V)
    ref, ref_aux, lse = oc.forward(0, 0)
    s0 = max(orc.mx_score(oc.qc[0], oc.qs[0], oc.kc[0], oc.ks[0], d, 10, j)[0] for j in range(64))
    s1 = max(orc.mx_score(oc.qc[0], oc.qs[0], oc.kc[0], oc.ks[0], d, 10, j)[0] for j in range(64, 128))
    assert (s1 - s0) * tau_for(d) / np.log(2) > 64
    compare_outputs(path.o[0, 0].float().cpu().numpy(), ref, "bf16", what="O (score jump)")
    compare_outputs(path.oa[0, 0].float().cpu().numpy(), ref_aux, "bf16", what="O' (score jump)")
    assert np.abs(path.lse[0, 0].cpu().numpy() - lse).max() < 2e-3


@pytest.mark.parametrize("k", [-17, 20])
def test_qat_backward_tiny_and_huge_do(k):
    """dO scaled by 2^k: values around 1e-7 (below fp16's normal range) and
    around 1e5 (above fp16's largest value).  The gradients are linear in dO,
    so 2^-k times the GPU's gradients must match the oracle's gradients for
    the unscaled dO: the fp16 dV product must lose nothing to the scale."""
    from bit_quantized_attention_amd.runner import QatTrainStep, qat_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c4"], 256, hq=2, hkv=2)
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    dOs = (dO * np.float32(2.0 ** k)).astype(np.float32)
    assert (np.abs(dOs).max() > 65504.0) if k > 0 else (np.abs(dOs).max() < 6.1e-5)
    p = qat_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    step = QatTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), to_device(dOs, "bf16"))
    step.step()
    torch.cuda.synchronize()
    oc = _Oracle(Q, K, V)
    g = [t.float().cpu().numpy() * 2.0 ** -k for t in (step.dq, step.dk, step.dv)]
    for h in range(2):
        ref = _qat_grads(oc, dO, h)
        for name, gi, ri in zip(("dQ", "dK", "dV"), g, ref):
            compare_outputs(gi[0, h], ri, "bf16", what=f"{name}[h={h}] (dO x 2^{k})")
