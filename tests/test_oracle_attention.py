"""Pins of the oracle's attention paths (CPU only).

The unquantised paths are pinned to torch's fp64 scaled_dot_product_attention
and autograd, to central finite differences and to closed forms (rows of
softmax sum to one, tiling invariance, K-smoothing invariance, the
FlashAttention row identity).  The quantised paths are pinned through special
cases that reduce to library rounding (torch fp16 / float8_e4m3fn), exact
brute-force integer and MX dot products, and error bounds.
"""
import math

import numpy as np
import pytest
import torch

TAU = 1.0 / math.sqrt(16)


def _torch_attn(Q, K, V, causal, tau):
    q, k, v = (torch.from_numpy(np.asarray(x, np.float64)).clone().requires_grad_(True) for x in (Q, K, V))
    Nq, Nk = q.shape[0], k.shape[0]
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= i + (Nk - Nq)
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask,
                                                         scale=tau)[0]
    return o, (q, k, v)


def _rand(rng, *shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("Nq,Nk,causal", [(33, 33, False), (40, 40, True), (17, 50, True), (8, 29, False)])
def test_ref_fwd_matches_torch_sdpa(orc, Nq, Nk, causal):
    rng = np.random.default_rng(Nq * 100 + Nk)
    Q, K, V = _rand(rng, Nq, 16, scale=2), _rand(rng, Nk, 16, scale=2), _rand(rng, Nk, 16)
    O, lse = orc.ref_fwd(Q, K, V, causal, TAU)
    o, _ = _torch_attn(Q, K, V, causal, TAU)
    assert np.abs(O - o.detach().numpy()).max() < 1e-12
    # lse: log of the row normaliser
    s = TAU * Q.astype(np.float64) @ K.astype(np.float64).T
    if causal:
        s = np.where(np.arange(Nk)[None] <= np.arange(Nq)[:, None] + Nk - Nq, s, -np.inf)
    ref = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
    assert np.abs(lse - ref).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_ref_bwd_matches_autograd(orc, causal):
    rng = np.random.default_rng(7)
    Q, K, V, dO = _rand(rng, 24, 16), _rand(rng, 24, 16), _rand(rng, 24, 16), _rand(rng, 24, 16)
    dQ, dK, dV = orc.ref_bwd(Q, K, V, dO, causal, TAU)
    o, (q, k, v) = _torch_attn(Q, K, V, causal, TAU)
    o.backward(torch.from_numpy(dO.astype(np.float64)))
    for a, b in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-12


def test_ref_bwd_finite_differences(orc):
    rng = np.random.default_rng(8)
    N, d = 6, 4
    Q, K, V, dO = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d)
    tau = 0.7
    dQ, dK, dV = orc.ref_bwd(Q, K, V, dO, True, tau)

    def loss(Qx, Kx, Vx):
        q, k, v = (torch.from_numpy(x) for x in (Qx, Kx, Vx))
        mask = torch.arange(N)[None] <= torch.arange(N)[:, None]
        s = (tau * q @ k.T).masked_fill(~mask, -math.inf)
        return float((torch.softmax(s, -1) @ v * torch.from_numpy(dO.astype(np.float64))).sum())

    base = [x.astype(np.float64) for x in (Q, K, V)]
    h = 1e-6
    for which, grad in enumerate((dQ, dK, dV)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            plus = [b.copy() for b in base]; minus = [b.copy() for b in base]
            plus[which][idx] += h; minus[which][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.abs(num - grad).max() / np.abs(grad).max() < 1e-6


def test_rows_sum_to_one(orc):
    rng = np.random.default_rng(9)
    Q, K = _rand(rng, 32, 16, scale=3), _rand(rng, 32, 16, scale=3)
    ones = np.ones((32, 16), np.float32)
    O, _ = orc.ref_fwd(Q, K, ones, True, TAU)
    assert np.abs(O - 1).max() < 1e-13
    O2, _ = orc.sage_fwd(qk_mode=orc.QK_F64, Qf=Q, Kf=K, pv_mode=orc.PV_NONE, Vf=ones,
                         Nq=32, Nk=32, d=16, causal=True, tau=TAU, kv_tile=8)
    assert np.abs(O2 - 1).max() < 1e-13


@pytest.mark.parametrize("kv_tile", [1, 5, 16, 64, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_any_tiling(orc, kv_tile, causal):
    rng = np.random.default_rng(10)
    Q, K, V = _rand(rng, 48, 16, scale=3), _rand(rng, 48, 16, scale=3), _rand(rng, 48, 16)
    O, lse = orc.ref_fwd(Q, K, V, causal, TAU)
    O2, lse2 = orc.sage_fwd(qk_mode=orc.QK_F64, Qf=Q, Kf=K, pv_mode=orc.PV_NONE, Vf=V,
                            Nq=48, Nk=48, d=16, causal=causal, tau=TAU, kv_tile=kv_tile)
    assert np.abs(O - O2).max() < 1e-12 and np.abs(lse - lse2).max() < 1e-12


def test_k_smoothing_invariance(orc):
    """Subtracting a per-channel constant from every key (and adding eps back)
    leaves softmax(Q K^T), dQ and dK unchanged; sum_j dK_j = 0."""
    rng = np.random.default_rng(11)
    Q, K, V, dO = _rand(rng, 40, 16), _rand(rng, 40, 16) + 3.0, _rand(rng, 40, 16), _rand(rng, 40, 16)
    mu, _ = orc.smooth_mean(K[None], 1e-3)
    Ks = (K - mu[0]).astype(np.float64)
    O1, _ = orc.ref_fwd(Q, K, V, True, TAU)
    O2, _ = orc.ref_fwd(Q, Ks, V, True, TAU)
    assert np.abs(O1 - O2).max() < 1e-12
    g1 = orc.ref_bwd(Q, K, V, dO, True, TAU)
    g2 = orc.ref_bwd(Q, Ks, V, dO, True, TAU)
    for a, b in zip(g1, g2):
        assert np.abs(a - b).max() < 1e-11
    assert np.abs(g1[1].sum(axis=0)).max() < 1e-12


def _sage_inputs(orc, rng, N, d, q_blk=32, k_blk=16):
    Q, K, V = _rand(rng, N, d, scale=2), _rand(rng, N, d, scale=2) + 1.0, _rand(rng, N, d)
    mu, _ = orc.smooth_mean(K[None], 0.0)
    qc, qs = orc.quant_i8_tokblock(Q[None], q_blk)
    kc, ks = orc.quant_i8_tokblock(K[None], k_blk, mu)
    return Q, K, V, qc[0], qs[0], kc[0], ks[0]


def test_sage_int8_scores_are_exact(orc):
    """Integer scores times the two block scales reproduce fp64 attention on the
    dequantised operands (the int64 dot products are brute force here)."""
    rng = np.random.default_rng(12)
    N, d = 64, 32
    Q, K, V, qc, qs, kc, ks = _sage_inputs(orc, rng, N, d)
    S_int = qc.astype(np.int64) @ kc.astype(np.int64).T
    assert np.abs(S_int).max() <= 127 * 127 * d
    Qd = qc.astype(np.float64) * np.repeat(qs, 32)[:, None]
    Kd = kc.astype(np.float64) * np.repeat(ks, 16)[:, None]
    O, lse = orc.sage_fwd(qk_mode=orc.QK_I8, qc=qc, qs=qs, q_blk=32, kc=kc, ks=ks, k_blk=16,
                          pv_mode=orc.PV_NONE, Vf=V, Nq=N, Nk=N, d=d, causal=True, tau=TAU, kv_tile=16)
    o, _ = _torch_attn(Qd, Kd, V, True, TAU)        # fp64 library attention on the dequantised operands
    assert np.abs(O - o.detach().numpy()).max() < 1e-12


def _single_tile_ref(orc, s, Vd, rounding):
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return rounding(p) @ Vd / l


def test_sage_pv_rounding_single_tile(orc):
    """With one key tile the running max is the row max, so each P.V mode is a
    library rounding of exp(s - max): fp16, e4m3 at 448 P, int8 per tile at
    127 P / max P (max P = 1)."""
    rng = np.random.default_rng(13)
    N, d = 32, 16
    Q, K, V, qc, qs, kc, ks = _sage_inputs(orc, rng, N, d, q_blk=32, k_blk=32)
    s = TAU * (qc.astype(np.float64) * qs[0]) @ (kc.astype(np.float64) * ks[0]).T
    kw = dict(qk_mode=orc.QK_I8, qc=qc, qs=qs, q_blk=32, kc=kc, ks=ks, k_blk=32, Nq=N, Nk=N, d=d,
              causal=False, tau=TAU, kv_tile=32)
    V16 = V.astype(np.float16).astype(np.float32)
    O, _ = orc.sage_fwd(pv_mode=orc.PV_F16, Vf=V16, **kw)
    ref = _single_tile_ref(orc, s, V16.astype(np.float64),
                           lambda p: torch.from_numpy(p).to(torch.float16).double().numpy())
    assert np.abs(O - ref).max() < 1e-12
    vc, vs = orc.quant_chan(V[None], "e4m3")
    dec = torch.from_numpy(vc[0].T.copy()).view(torch.float8_e4m3fn).double().numpy() * vs[0][None]
    O, _ = orc.sage_fwd(pv_mode=orc.PV_F8, vc_t=vc[0], vs=vs[0], **kw)
    ref = _single_tile_ref(orc, s, dec, lambda p: torch.from_numpy(448 * p).to(torch.float8_e4m3fn).double().numpy() / 448)
    assert np.abs(O - ref).max() < 1e-12
    vc, vs = orc.quant_chan(V[None], "i8")
    deq = vc[0].T.view(np.int8).astype(np.float64) * vs[0][None]
    O, _ = orc.sage_fwd(pv_mode=orc.PV_I8, vc_t=vc[0], vs=vs[0], **kw)
    ref = _single_tile_ref(orc, s, deq, lambda p: np.rint((p * np.float32(127.0)).astype(np.float32)).astype(np.float64) / 127)
    assert np.abs(O - ref).max() < 1e-12


@pytest.mark.parametrize("pv", ["f16", "f8", "i8"])
def test_sage_quantised_error_bounded(orc, pv):
    """Multi-tile quantised attention stays within the rounding error of its
    P format of the exact attention on the same dequantised operands."""
    rng = np.random.default_rng(14)
    N, d = 256, 32
    Q, K, V, qc, qs, kc, ks = _sage_inputs(orc, rng, N, d)
    Qd = qc.astype(np.float64) * np.repeat(qs, 32)[:, None]
    Kd = kc.astype(np.float64) * np.repeat(ks, 16)[:, None]
    kw = dict(qk_mode=orc.QK_I8, qc=qc, qs=qs, q_blk=32, kc=kc, ks=ks, k_blk=16, Nq=N, Nk=N, d=d,
              causal=True, tau=TAU, kv_tile=16)
    if pv == "f16":
        O, _ = orc.sage_fwd(pv_mode=orc.PV_F16, Vf=V, **kw); Vd = V; rel = 2 ** -11
    elif pv == "f8":
        vc, vs = orc.quant_chan(V[None], "e4m3")
        Vd = torch.from_numpy(vc[0].T.copy()).view(torch.float8_e4m3fn).double().numpy() * vs[0][None]
        O, _ = orc.sage_fwd(pv_mode=orc.PV_F8, vc_t=vc[0], vs=vs[0], **kw); rel = 2 ** -4
    else:
        vc, vs = orc.quant_chan(V[None], "i8")
        Vd = vc[0].T.view(np.int8).astype(np.float64) * vs[0][None]
        O, _ = orc.sage_fwd(pv_mode=orc.PV_I8, vc_t=vc[0], vs=vs[0], **kw); rel = 1 / 127
    ref, _ = orc.ref_fwd(Qd, Kd, Vd, True, TAU)
    # |sum_j (P^_j - P_j) V_j| / l  <=  max|V| * rel   (rounding at most `rel` of each P, or of the tile max)
    assert np.abs(O - ref).max() <= np.abs(Vd).max() * rel * 1.01
    assert np.abs(O - ref).mean() < np.abs(Vd).max() * rel * 0.25


def _sage_bwd_setup(orc, rng, N=256, d=32):
    Q, K, V = _rand(rng, N, d), _rand(rng, N, d) + 0.5, _rand(rng, N, d)
    dO = _rand(rng, N, d, scale=0.1)
    mu, _ = orc.smooth_mean(K[None], 1e-3)
    qc, qs = orc.quant_i8_tokblock(Q[None], 128)
    kc, ks = orc.quant_i8_tokblock(K[None], 64, mu)
    Qd = qc[0].astype(np.float64) * np.repeat(qs[0], 128)[:, None]
    Kd = kc[0].astype(np.float64) * np.repeat(ks[0], 64)[:, None]
    return dict(Q=Q, K=K, V=V, dO=dO, qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], Qd=Qd, Kd=Kd)


def test_sage_bwd_unquantised_is_textbook(orc):
    """With the roundings off, the tiled backward (delta = rowsum(dO o O)) equals
    autograd-checked textbook gradients (delta = rowsum(P o dP)) on the same
    operands: this pins the tiling, the masks and the row identity."""
    rng = np.random.default_rng(15)
    t = _sage_bwd_setup(orc, rng)
    O, lse = orc.ref_fwd(t["Qd"], t["Kd"], t["V"], True, TAU)
    dQ, dK, dV = orc.sage_bwd(qc=t["qc"], qs=t["qs"], kc=t["kc"], ks=t["ks"], V=t["V"], dO=t["dO"],
                              O=O, lse=lse, causal=True, tau=TAU, quantize=False)
    rQ, rK, rV = orc.ref_bwd(t["Qd"], t["Kd"], t["V"], t["dO"], True, TAU)
    # O and lse pass through fp32 on the way in: compare at that precision
    for a, b in ((dQ, rQ), (dK, rK), (dV, rV)):
        assert np.abs(a - b).max() <= 1e-5 * np.abs(b).max()


def test_sage_bwd_quantised_close_and_tile_local(orc):
    rng = np.random.default_rng(16)
    t = _sage_bwd_setup(orc, rng)
    O, lse = orc.ref_fwd(t["Qd"], t["Kd"], t["V"], True, TAU)
    kw = dict(qc=t["qc"], qs=t["qs"], kc=t["kc"], ks=t["ks"], V=t["V"], dO=t["dO"], O=O, lse=lse,
              causal=True, tau=TAU)
    dQ, dK, dV = orc.sage_bwd(**kw)
    rQ, rK, rV = orc.ref_bwd(t["Qd"], t["Kd"], t["V"], t["dO"], True, TAU)
    for a, b in ((dQ, rQ), (dK, rK), (dV, rV)):
        cos = (a * b).sum() / np.linalg.norm(a) / np.linalg.norm(b)
        assert cos > 0.99
    sQ, sK, sV = orc.sage_bwd(qtiles=(1, 2), ktiles=(2, 3), **kw)
    assert np.array_equal(sQ, dQ[128:256]) and np.array_equal(sK, dK[128:192]) and np.array_equal(sV, dV[128:192])


def _mx_deq_rows(codes, scales):
    tab = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
    v = np.stack([tab[codes & 0xF], tab[codes >> 4]], -1).reshape(codes.shape[0], -1)
    return v * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=-1)


def _qat_setup(orc, rng, N=128, d=64):
    X = [rng.standard_t(3, (N, d)).astype(np.float32) for _ in range(3)]
    qc, qs = orc.quant_mx_rows(X[0][None]); kc, ks = orc.quant_mx_rows(X[1][None])
    vc, vs = orc.quant_mx_cols(X[2][None])
    t = dict(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0])
    deq = dict(Q=_mx_deq_rows(qc[0], qs[0]), K=_mx_deq_rows(kc[0], ks[0]), V=_mx_deq_rows(vc[0], vs[0]).T.copy())
    return t, deq


def test_mx_scores_exact(orc):
    rng = np.random.default_rng(17)
    t, deq = _qat_setup(orc, rng)
    for (i, j) in [(0, 0), (5, 77), (127, 3), (64, 64)]:
        s, exact = orc.mx_score(t["qc"], t["qs"], t["kc"], t["ks"], 64, i, j)
        terms = deq["Q"][i] * deq["K"][j]
        assert exact and s == math.fsum(terms)


def test_qat_unquantised_is_textbook(orc):
    rng = np.random.default_rng(18)
    t, deq = _qat_setup(orc, rng)
    tau = 1 / 8
    O, Oa, lse = orc.qat_fwd(Nq=128, Nk=128, d=64, tau=tau, kv_tile=32, quantize_p=False, **t)
    rO, rl = orc.ref_fwd(deq["Q"], deq["K"], deq["V"], False, tau)
    # the operands pass through fp32 on the way into the textbook reference
    assert np.abs(O - rO).max() < 1e-6 * np.abs(rO).max() and np.array_equal(O, Oa)
    assert np.abs(lse - rl).max() < 1e-9 * np.abs(rl).max() + 1e-12
    dO = (rng.standard_normal((128, 64)) * 0.1).astype(np.float32)
    dQ, dK, dV = orc.qat_bwd(dO=dO, O_aux=Oa, lse=lse, Nq=128, Nk=128, d=64, tau=tau, quantize_p=False, **t)
    r = orc.ref_bwd(deq["Q"], deq["K"], deq["V"], dO, False, tau)
    for a, b in zip((dQ, dK, dV), r):
        assert np.abs(a - b).max() <= 1e-5 * np.abs(b).max()


def test_qat_quantised_close_and_aux_identity(orc):
    rng = np.random.default_rng(19)
    t, deq = _qat_setup(orc, rng)
    tau = 1 / 8
    O, Oa, lse = orc.qat_fwd(Nq=128, Nk=128, d=64, tau=tau, kv_tile=32, **t)
    rO, _ = orc.ref_fwd(deq["Q"], deq["K"], deq["V"], False, tau)
    # O' only rounds P to bf16: close to the exact attention on the FP4 operands
    assert np.abs(Oa - rO).max() <= np.abs(deq["V"]).max() * 2 ** -8
    # O rounds P to MXFP4 (step 1/8 of the block max at worst)
    assert np.abs(O - rO).max() <= np.abs(deq["V"]).max() * 2 ** -3
    dO = (rng.standard_normal((128, 64)) * 0.1).astype(np.float32)
    dQ, dK, dV = orc.qat_bwd(dO=dO, O_aux=Oa, lse=lse, Nq=128, Nk=128, d=64, tau=tau, **t)
    r = orc.ref_bwd(deq["Q"], deq["K"], deq["V"], dO, False, tau)
    for a, b in zip((dQ, dK, dV), r):
        cos = (a * b).sum() / np.linalg.norm(a) / np.linalg.norm(b)
        assert cos > 0.98
    sub = orc.qat_bwd(dO=dO, O_aux=Oa, lse=lse, Nq=128, Nk=128, d=64, tau=tau, qrows=(10, 20),
                      krows=(32, 64), **t)
    assert np.array_equal(sub[0], dQ[10:20]) and np.allclose(sub[1], dK[32:64], rtol=1e-12, atol=1e-15)
    assert np.allclose(sub[2], dV[32:64], rtol=1e-12, atol=1e-15)


def test_qat_backward_reuses_forward_p(orc):
    """Attn-QAT §2 Principle 1: the backward's rounded P is the forward's.
    With dO one-hot on (row i, channel k), dV[:, k] is row i of the
    backward's P^.  For a row whose maximum sits in the first key tile, the
    forward's running maximum never moves, every tile's P^ is made against the
    final maximum, and P^ V gives back the forward's O row exactly --
    including peaked rows whose largest P is 1 (on an MXFP4 exponent step)."""
    rng = np.random.default_rng(23)
    N, d, tau, tile = 128, 64, 1 / 8, 32
    X = [rng.standard_t(3, (N, d)).astype(np.float32) for _ in range(3)]
    X[0][5] = X[1][3] * 4.0                      # row 5: key 3 (first tile) dominates
    qc, qs = orc.quant_mx_rows(X[0][None]); kc, ks = orc.quant_mx_rows(X[1][None]); vc, vs = orc.quant_mx_cols(X[2][None])
    t = dict(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0])
    O, Oa, lse, mrow = orc.qat_fwd(Nq=N, Nk=N, d=d, tau=tau, kv_tile=tile, return_rowmax=True, **t)
    S = np.array([[orc.mx_score(qc[0], qs[0], kc[0], ks[0], d, i, j)[0] for j in range(N)] for i in range(N)])
    assert np.array_equal(mrow, tau * S.max(axis=1))                 # the final running max is the row max
    first = [i for i in range(N) if S[i].argmax() < tile]
    assert 5 in first and len(first) >= 10
    Vd = _mx_deq_rows(vc[0], vs[0]).T                  # [N keys, d]
    for i in first[:8]:
        k = 3
        dO = np.zeros((N, d), np.float32)
        dO[i, k] = 1.0
        kw = dict(dO=dO, O_aux=Oa.astype(np.float32), lse=lse.astype(np.float32), Nq=N, Nk=N, d=d, tau=tau, **t)
        _, _, dV = orc.qat_bwd(rowmax=mrow, **kw)
        _, _, dV2 = orc.qat_bwd(**kw)                  # row max taken inside: the same
        assert np.array_equal(dV, dV2)
        prow = dV[:, k]
        assert prow[S[i].argmax()] == pytest.approx(np.exp(mrow[i] - np.float32(lse[i])), rel=1e-15)
        # the forward normalises by its own row sum; the backward by exp(L): equal up to L's fp32 storage
        assert np.abs(prow @ Vd - O[i]).max() <= 1e-5 * np.abs(O[i]).max()
    assert np.exp(tau * S[5, 3] - lse[5]) > 0.5


def test_qat_one_hot_row_is_exact(orc):
    """A row whose scores put all the mass on one key: that key's P is exactly
    1 (the running max), its MXFP4 code is exact and every other P rounds to
    zero, so O and O' equal that key's FP4 value row."""
    d, N = 32, 64
    Q = np.zeros((N, d), np.float32); K = np.zeros((N, d), np.float32)
    Q[:, 0] = 6.0
    K[:, 0] = -4.0
    K[7, 0] = 6.0
    rng = np.random.default_rng(20)
    V = rng.standard_t(3, (N, d)).astype(np.float32)
    qc, qs = orc.quant_mx_rows(Q[None]); kc, ks = orc.quant_mx_rows(K[None]); vc, vs = orc.quant_mx_cols(V[None])
    O, Oa, _ = orc.qat_fwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0],
                           Nq=N, Nk=N, d=d, tau=1.0, kv_tile=32)
    Vd = _mx_deq_rows(vc[0], vs[0]).T
    assert np.abs(O - Vd[7][None]).max() < 1e-12
    assert np.abs(Oa - Vd[7][None]).max() < 1e-12
