"""Pins of the oracle's post-training FP4 baseline (query and key smoothing
plus two-level P, "Attn-QAT" technical summary §1 and §2 Implementation;
the two-level step of "ThriftAttention", Method step 2).

* the bf16 query block mean, on values whose mean is known in closed form;
* the smoothing decomposition: where Q, its block mean and Q - mean are all
  exact on the MXFP4 grid, the smoothed scores equal the unsmoothed ones, so
  the baseline must reproduce the (separately pinned) Thrift FP4 path with
  nothing selected, bit for bit — a dropped, negated or misindexed bias term
  fails it;
* key smoothing: a per-channel offset added to every key leaves every
  output unchanged;
* a ragged last query block only changes its own rows."""
import numpy as np
import pytest

import oracle as orc
from tests.helpers import tau_for


def test_qbar_closed_form():
    Q = np.zeros((1, 131, 32), np.float32)
    Q[0, :128, 0] = np.arange(128)                 # mean 63.5, exact in bf16
    Q[0, :128, 1] = 1.0 + (np.arange(128) % 2)     # mean 1.5
    Q[0, 128:, 0] = [1.0, 2.0, 4.0]                # mean 7/3: fp32 then bf16 -> 149/64
    Q[0, 128:, 1] = [-3.0, 0.0, 0.0]               # mean -1
    qbar, Qs = orc.smooth_q_blocks(Q, 128)
    assert qbar.shape == (1, 2, 32)
    assert qbar[0, 0, 0] == 63.5 and qbar[0, 0, 1] == 1.5
    assert qbar[0, 1, 0] == 149.0 / 64.0 and qbar[0, 1, 1] == -1.0
    assert np.all(qbar[0, :, 2:] == 0.0)
    assert Qs[0, 0, 0] == -63.5 and Qs[0, 130, 0] == np.float32(4.0 - 149.0 / 64.0)


def _exact_q(rng, N, d):
    """Rows in +- pairs around a block mean qbar: Q_s entries +-1 with a +-4
    in the first channel of every 32-channel group (so the MX scale is 1 and
    every value is on the e2m1 grid), qbar entries in {-1, 0, 1} with 0 on
    the first channels: Q = Q_s + qbar lies on the grid too."""
    nb = N // 128
    Q = np.zeros((N, d), np.float32)
    qbars = np.zeros((nb, d), np.float32)
    for I in range(nb):
        qbar = rng.integers(-1, 2, d).astype(np.float32)
        qbar[::32] = 0.0
        half = rng.choice([-1.0, 1.0], (64, d)).astype(np.float32)
        half[:, ::32] = 4.0 * rng.choice([-1.0, 1.0], (64, d // 32))
        Qs = np.concatenate([half, -half])[rng.permutation(128)]
        Q[I * 128:(I + 1) * 128] = Qs + qbar
        qbars[I] = qbar
    return Q, qbars


@pytest.mark.parametrize("causal", [False, True])
def test_smoothing_is_exact_where_the_grid_is(causal):
    rng = np.random.default_rng(11)
    N, d = 256, 128
    Q, qbar_true = _exact_q(rng, N, d)
    K = (rng.standard_t(4, (N, d)) * 0.5).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    qbar, Qs = orc.smooth_q_blocks(Q[None], 128)
    assert np.array_equal(qbar[0], qbar_true)
    qc0, qs0 = orc.quant_mx_rows(Q[None])
    qc, qs = orc.quant_mx_rows(Qs)
    assert not np.array_equal(qc, qc0)                  # the smoothed codes are other codes
    kc, ks = orc.quant_mx_rows(K[None])
    vc, vs = orc.quant_mx_cols(V[None])
    tau = tau_for(d)
    O, lse = orc.ptq_fwd(qc=qc[0], qs=qs[0], qbar=qbar[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Nq=N, Nk=N,
                         d=d, causal=causal, tau=tau)
    none = -np.ones((N // 128, 1), np.int32)
    O2, lse2 = orc.thrift_fwd(qc=qc0[0], qs=qs0[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Qh=Q, Kh=K, Vh=V,
                              sel_idx=none, sel_cnt=np.zeros(N // 128, np.int32), Nq=N, Nk=N, d=d, blk=128,
                              causal=causal, tau=tau)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)


def test_key_offset_is_removed():
    rng = np.random.default_rng(5)
    N, d = 256, 128
    half = (rng.standard_normal((N // 2, d)) * 0.75).astype(np.float32)
    K = np.concatenate([half, -half])                  # token mean exactly 0
    off = np.where(np.arange(d) % 3 == 0, 3.0, -0.5).astype(np.float32)
    Q = (rng.standard_t(3, (N, d))).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    outs = []
    for Kx in (K, K + off):
        mu, Ks = orc.smooth_k(Kx[None])
        qbar, Qs = orc.smooth_q_blocks(Q[None])
        qc, qs = orc.quant_mx_rows(Qs)
        kc, ks = orc.quant_mx_rows(Ks)
        vc, vs = orc.quant_mx_cols(V[None])
        outs.append(orc.ptq_fwd(qc=qc[0], qs=qs[0], qbar=qbar[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0],
                                Nq=N, Nk=N, d=d, tau=tau_for(d)))
    assert np.array_equal(mu[0], off)
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_ragged_last_block():
    rng = np.random.default_rng(8)
    Nk, d = 256, 128
    Q = rng.standard_t(3, (200, d)).astype(np.float32)
    K = rng.standard_t(3, (Nk, d)).astype(np.float32)
    V = rng.standard_normal((Nk, d)).astype(np.float32)
    kc, ks = orc.quant_mx_rows(K[None])
    vc, vs = orc.quant_mx_cols(V[None])
    res = []
    for Nq in (200, 256):
        Qx = np.concatenate([Q, rng.standard_normal((Nq - 200, d)).astype(np.float32)]) if Nq > 200 else Q
        qbar, Qs = orc.smooth_q_blocks(Qx[None])
        qc, qs = orc.quant_mx_rows(Qs)
        res.append(orc.ptq_fwd(qc=qc[0], qs=qs[0], qbar=qbar[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0],
                               Nq=Nq, Nk=Nk, d=d, tau=tau_for(d)))
    (O1, l1), (O2, l2) = res
    assert O1.shape == (200, d)
    np.testing.assert_array_equal(O1[:128], O2[:128])          # block 0 is the same block
    assert not np.allclose(O1[128:], O2[128:200])              # block 1's mean differs
    # block 1 alone
    O3, l3 = orc.ptq_fwd(qc=orc.quant_mx_rows(orc.smooth_q_blocks(Q[None])[1])[0][0],
                         qs=orc.quant_mx_rows(orc.smooth_q_blocks(Q[None])[1])[1][0],
                         qbar=orc.smooth_q_blocks(Q[None])[0][0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0],
                         Nq=200, Nk=Nk, d=d, tau=tau_for(d), qblocks=(1, 2))
    np.testing.assert_array_equal(O3, O1[128:])
    np.testing.assert_array_equal(l3, l1[128:])
