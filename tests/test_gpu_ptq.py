"""GPU parity of the post-training FP4 baseline (query and key smoothing plus
two-level P; "Attn-QAT" technical summary §1 and §2 Implementation) against
the oracle, through the C ABI: the smoothed quantisation bit for bit, then
O and the log-sum-exp at small ragged sizes with grouped heads, causal and
not, and at the full Attn-QAT shape on sampled rows."""
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


def _inputs(Nq, Nk, hq, hkv, offset=0.0):
    w = wl.with_len(wl.WORKLOADS["c4"], Nk, hq=hq, hkv=hkv)
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    Q = np.ascontiguousarray(Q[:, :, :Nq])
    if offset:
        # a shared per-channel component in Q and K (what smoothing removes)
        ch = np.where(np.arange(w.d) % 4 == 0, offset, -0.5 * offset).astype(np.float32)
        Q = wl.round_to(Q + ch, "bf16").reshape(Q.shape)
        K = wl.round_to(K + 2.0 * ch, "bf16").reshape(K.shape)
    return w, Q, K, V


def _run(Q, K, V, causal):
    from bit_quantized_attention_amd.runner import PtqPath, ptq_problem, to_device
    B, Hq, Nq, d = Q.shape
    Hkv, Nk = K.shape[1], K.shape[2]
    p = ptq_problem(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    path = PtqPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.step()
    torch.cuda.synchronize()
    return path


class _Oracle:
    def __init__(self, Q, K, V):
        self.Hq, self.Hkv, self.Nq, self.Nk, self.d = Q.shape[1], K.shape[1], Q.shape[2], K.shape[2], Q.shape[3]
        self.qbar, Qs = orc.smooth_q_blocks(Q.reshape(-1, self.Nq, self.d))
        self.mu, Ks = orc.smooth_k(K.reshape(-1, self.Nk, self.d))
        self.qc, self.qs = orc.quant_mx_rows(Qs)
        self.kc, self.ks = orc.quant_mx_rows(Ks)
        self.vc, self.vs = orc.quant_mx_cols(V.reshape(-1, self.Nk, self.d))

    def forward(self, b, h, causal, qblocks=None):
        iq, ik = b * self.Hq + h, b * self.Hkv + h // (self.Hq // self.Hkv)
        return orc.ptq_fwd(qc=self.qc[iq], qs=self.qs[iq], qbar=self.qbar[iq], kc=self.kc[ik], ks=self.ks[ik],
                           vc_t=self.vc[ik], vs_t=self.vs[ik], Nq=self.Nq, Nk=self.Nk, d=self.d, causal=causal,
                           tau=tau_for(self.d), qblocks=qblocks)


@pytest.mark.parametrize("Nq,Nk,hq,hkv", [(300, 512, 4, 2), (128, 128, 1, 1), (1, 256, 2, 1)])
def test_smoothed_quantisation_bit_exact(Nq, Nk, hq, hkv):
    """Q less its bf16 block means (ragged last block, a one-row problem),
    K less its token mean: codes, scales and means equal the oracle's."""
    w, Q, K, V = _inputs(Nq, Nk, hq, hkv, offset=3.0)
    path = _run(Q, K, V, causal=False)
    oc = _Oracle(Q, K, V)
    assert_same(path.qbar.cpu().numpy().reshape(oc.qbar.shape), oc.qbar, "Q block means")
    assert_same(path.mu.cpu().numpy().reshape(oc.mu.shape), oc.mu, "K token means")
    assert_same(path.qc.cpu().numpy().reshape(oc.qc.shape), oc.qc, "smoothed Q codes")
    assert_same(path.qs.cpu().numpy().reshape(oc.qs.shape), oc.qs, "smoothed Q scales")
    assert_same(path.kc.cpu().numpy().reshape(oc.kc.shape), oc.kc, "smoothed K codes")
    assert_same(path.ks.cpu().numpy().reshape(oc.ks.shape), oc.ks, "smoothed K scales")
    assert_same(path.vc.cpu().numpy().reshape(oc.vc.shape), oc.vc, "V codes")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,hq,hkv,offset", [(512, 512, 2, 2, 0.0), (300, 512, 4, 2, 3.0),
                                                 (1000, 1024, 2, 1, 1.0), (64, 384, 1, 1, 0.0)])
def test_ptq_forward_small(causal, Nq, Nk, hq, hkv, offset):
    """Several query and key blocks, a ragged query tail, grouped heads, a
    single short query block; with and without a shared offset in Q and K."""
    w, Q, K, V = _inputs(Nq, Nk, hq, hkv, offset)
    path = _run(Q, K, V, causal)
    oc = _Oracle(Q, K, V)
    O = path.o.float().cpu().numpy()
    L = path.lse.cpu().numpy()
    for h in range(hq):
        ref, lse = oc.forward(0, h, causal)
        compare_outputs(O[0, h], ref, "bf16", what=f"O[h={h}]")
        assert np.abs(L[0, h] - lse).max() < 2e-3


def test_ptq_smoothing_helps_on_offset_inputs():
    """Where Q and K share a large per-channel component, the smoothed FP4
    output is closer to exact attention than plain MXFP4 of the same inputs
    (the oracle's unsmoothed Attn-QAT forward)."""
    w, Q, K, V = _inputs(256, 256, 1, 1, offset=6.0)
    path = _run(Q, K, V, causal=False)
    tau = tau_for(w.d)
    exact, _ = orc.ref_fwd(Q[0, 0], K[0, 0], V[0, 0], False, tau)
    qc, qs = orc.quant_mx_rows(Q[0])
    kc, ks = orc.quant_mx_rows(K[0])
    vc, vs = orc.quant_mx_cols(V[0])
    plain, _, _ = orc.qat_fwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Nq=256, Nk=256,
                              d=w.d, tau=tau, kv_tile=64)
    err_ptq = np.abs(path.o[0, 0].float().cpu().numpy() - exact).mean()
    err_plain = np.abs(plain - exact).mean()
    assert err_ptq < err_plain, (err_ptq, err_plain)


@pytest.mark.slow
def test_ptq_forward_full_size_sampled():
    """The Attn-QAT shape (B=1, H=32, N=16384, d=128, non-causal, Student-t):
    sampled query blocks of sampled heads against the oracle."""
    w = wl.WORKLOADS["c4"]
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    path = _run(Q, K, V, causal=False)
    O = path.o.float().cpu().numpy()
    L = path.lse.cpu().numpy()
    for h in (0, 17, 31):
        oc = _Oracle(Q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1])
        for qb in (0, 63, 127):
            ref, lse = oc.forward(0, 0, False, qblocks=(qb, qb + 1))
            rows = slice(128 * qb, 128 * qb + 128)
            compare_outputs(O[0, h, rows], ref, "bf16", what=f"O[h={h}, block {qb}]")
            assert np.abs(L[0, h, rows] - lse).max() < 2e-3
