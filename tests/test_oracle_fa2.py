"""Closed-form pins of the oracle's online softmax and quantisation
granularities (CPU only).

FlashAttention-2's merge, which the "ThriftAttention" summary (Methodology
step 2) names for joining the two precision paths and which every variant
here follows, forms P against the running row maximum: in the key tile that
holds the row's maximum so far that P is exactly 1, and the sums gathered
before a larger maximum arrives are scaled by exp(m_old - m_new).  The cases
below use scores with one or two non-negligible keys per tile, so the
expected output is a short closed form with library roundings (torch fp16,
bf16, float8_e4m3fn casts) or hand-read e2m1 grid points.  A reference point
other than the running max (a power of two above it, or the final row max
of a two-pass softmax) or a missing rescale changes these values.

The backward cases pin the scale granularities of the SageBwd INT8
backward ("SageBwd", Methodology 2: per-block INT8 scales) and the bf16
rounding of dS in the Attn-QAT backward ("Attn-QAT", §2), through operands
that expose P^, dS^ and the dO codes in the outputs.
"""
import math

import numpy as np
import pytest
import torch

# e2m1 values of the 16 codes (OCP FP4): sign bit 3, then 0, 0.5, 1, 1.5, 2, 3, 4, 6
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def _deq_mx(codes, scales):
    """MXFP4 codes [R, C/2] + E8M0 bytes [R, C/32] -> values [R, C] (read off the grid)."""
    v = np.stack([E2M1[codes & 0xF], E2M1[codes >> 4]], -1).reshape(codes.shape[0], -1)
    return v * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=-1)


def _f16(x):
    return torch.tensor(x, dtype=torch.float64).to(torch.float16).double().item()


def _bf16(x):
    return torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).double().item()


def _e4m3(x):
    return torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn).double().item()


# ---------------------------------------------------------------------------
# SageAttention forward: two key tiles, the second raises the row maximum
# ---------------------------------------------------------------------------
A_, DELTA, B_ = 0.3, 0.7, 1.1     # scores: tile 0 keys (a, a - delta), tile 1 key b > a


def _two_tile_scores():
    """Qf rows [1, 0, 0, 0] and Kf rows [s_j, 0, 0, 0] with tau = 1: key 0 = a,
    key 1 = a - delta, key 4 = b; every other key -1000 (P = 0 exactly)."""
    Q = np.zeros((2, 4), np.float32); Q[:, 0] = 1.0
    K = np.zeros((8, 4), np.float32); K[:, 0] = -1000.0
    K[0, 0], K[1, 0], K[4, 0] = A_, A_ - DELTA, B_
    return Q, K


@pytest.mark.parametrize("pv", ["f16", "f8", "i8"])
def test_sage_two_tiles_running_max(orc, pv):
    """P^ of the first tile is made against m = a (its max P is exactly 1 in
    every format), then the first tile's sums are scaled by exp(a - b) when
    the second tile brings b: O = (alpha (V0 + R(e^-delta) V1) + V4) / l."""
    Q, K = _two_tile_scores()
    a32, d32, b32 = (float(np.float32(x)) for x in (A_, A_ - DELTA, B_))
    rng = np.random.default_rng(101)
    kw = dict(qk_mode=orc.QK_F64, Qf=Q, Kf=K, Nq=2, Nk=8, d=4, causal=False, tau=1.0, kv_tile=4)
    p1 = math.exp(d32 - a32)
    if pv == "f16":
        V = rng.standard_normal((8, 4)).astype(np.float16).astype(np.float32)
        O, lse = orc.sage_fwd(pv_mode=orc.PV_F16, Vf=V, **kw)
        Vd, R1 = V.astype(np.float64), _f16(p1)
    elif pv == "f8":
        codes = rng.integers(0, 0x7E, (4, 8)).astype(np.uint8) | (rng.integers(0, 2, (4, 8)) << 7).astype(np.uint8)
        vs = rng.uniform(0.5, 2.0, 4).astype(np.float32)
        O, lse = orc.sage_fwd(pv_mode=orc.PV_F8, vc_t=codes, vs=vs, **kw)
        Vd = torch.from_numpy(codes.T.copy()).view(torch.float8_e4m3fn).double().numpy() * vs[None]
        R1 = _e4m3(448 * p1) / 448
    else:
        codes = rng.integers(-127, 128, (4, 8)).astype(np.int8)
        vs = rng.uniform(0.5, 2.0, 4).astype(np.float32)
        O, lse = orc.sage_fwd(pv_mode=orc.PV_I8, vc_t=codes.view(np.uint8), vs=vs, **kw)
        Vd = codes.T.astype(np.float64) * vs[None]
        R1 = float(np.rint(np.float32(np.float32(p1) * np.float32(127.0)))) / 127   # tile max P = 1
    alpha = math.exp(a32 - b32)
    l = alpha * (1 + p1) + 1
    ref = (alpha * (Vd[0] + R1 * Vd[1]) + Vd[4]) / l
    assert np.abs(O - ref[None]).max() < 1e-12
    assert np.abs(lse - (b32 + math.log(l))).max() < 1e-12
    # the reading matters: against the final maximum the first tile would round e^(a - b)
    assert R1 != {"f16": _f16, "f8": lambda x: _e4m3(448 * x) / 448,
                  "i8": lambda x: x}[pv](p1 * alpha) / alpha or pv == "i8"


@pytest.mark.parametrize("pv", ["f16", "f8", "i8"])
def test_sage_row_max_is_exact(orc, pv):
    """A row whose whole mass is on one key: that key's P is exactly 1 and its
    rounded value too, so O is that key's (dequantised) V row exactly."""
    Q = np.zeros((3, 4), np.float32); Q[:, 0] = 1.0
    K = np.full((8, 4), 0.0, np.float32); K[:, 0] = -1000.0; K[5, 0] = 0.4567
    rng = np.random.default_rng(102)
    kw = dict(qk_mode=orc.QK_F64, Qf=Q, Kf=K, Nq=3, Nk=8, d=4, causal=False, tau=1.0, kv_tile=4)
    if pv == "f16":
        V = rng.standard_normal((8, 4)).astype(np.float16).astype(np.float32)
        O, _ = orc.sage_fwd(pv_mode=orc.PV_F16, Vf=V, **kw)
        Vd = V.astype(np.float64)
    elif pv == "f8":
        codes = rng.integers(0, 0x7E, (4, 8)).astype(np.uint8)
        vs = rng.uniform(0.5, 2.0, 4).astype(np.float32)
        O, _ = orc.sage_fwd(pv_mode=orc.PV_F8, vc_t=codes, vs=vs, **kw)
        Vd = torch.from_numpy(codes.T.copy()).view(torch.float8_e4m3fn).double().numpy() * vs[None]
    else:
        codes = rng.integers(-127, 128, (4, 8)).astype(np.int8)
        vs = rng.uniform(0.5, 2.0, 4).astype(np.float32)
        O, _ = orc.sage_fwd(pv_mode=orc.PV_I8, vc_t=codes.view(np.uint8), vs=vs, **kw)
        Vd = codes.T.astype(np.float64) * vs[None]
    assert np.abs(O - Vd[5][None]).max() < 1e-12


# ---------------------------------------------------------------------------
# Attn-QAT forward: MXFP4 P and bf16 P for O', two key tiles of 32
# ---------------------------------------------------------------------------
def _qat_two_tile(orc):
    """Q rows [6, 0, ...]; K rows key 0 = [4], key 1 = [3], key 32 = [6], the
    rest [-384]; each is one MX grid value, so the MX codes hold them exactly.
    With tau = 1/12 the scores are 2, 1.5, 3 and -192."""
    d, N = 32, 64
    Q = np.zeros((N, d), np.float32); Q[:, 0] = 6.0
    K = np.zeros((N, d), np.float32); K[:, 0] = -384.0
    K[0, 0], K[1, 0], K[32, 0] = 4.0, 3.0, 6.0
    rng = np.random.default_rng(103)
    V = rng.standard_t(3, (N, d)).astype(np.float32)
    qc, qs = orc.quant_mx_rows(Q[None]); kc, ks = orc.quant_mx_rows(K[None]); vc, vs = orc.quant_mx_cols(V[None])
    assert np.array_equal(_deq_mx(kc[0], ks[0]), K) and np.array_equal(_deq_mx(qc[0], qs[0]), Q)
    t = dict(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0])
    return t, _deq_mx(vc[0], vs[0]).T, N, d


def test_qat_two_tiles_running_max(orc):
    """Tile 0: m = 2, P = (1, e^-0.5): MXFP4 per 32 keys with the block max 1
    (scale 1/4) gives (1, 0.5) [e^-0.5 / (1/4) = 2.43 rounds to the grid
    point 2]; bf16 for O'.  Tile 1 raises m to 3 (alpha = e^-1) with P = 1."""
    t, Vd, N, d = _qat_two_tile(orc)
    O, Oa, lse, mrow = orc.qat_fwd(Nq=N, Nk=N, d=d, tau=1 / 12, kv_tile=32, return_rowmax=True, **t)
    p1, alpha = math.exp(-0.5), math.exp(-1.0)
    l = alpha * (1 + p1) + 1
    ref = (alpha * (Vd[0] + 0.5 * Vd[1]) + Vd[32]) / l
    ref_aux = (alpha * (Vd[0] + _bf16(p1) * Vd[1]) + Vd[32]) / l
    assert np.abs(O - ref[None]).max() < 1e-12 * np.abs(ref).max()
    assert np.abs(Oa - ref_aux[None]).max() < 1e-12 * np.abs(ref).max()
    assert np.abs(lse - (3 + math.log(l))).max() < 1e-12
    assert np.all(mrow == 3.0)


# ---------------------------------------------------------------------------
# ThriftAttention: per-row two-level P, FA2 merge across the two paths
# ---------------------------------------------------------------------------
def _thrift_case(orc):
    """d = 64, blocks of 32, causal, rows A = 40 and B = 50 (query block 1).
    Row A reads channel 0, row B channel 32 (separate MX blocks of K).
    Scores (tau = 1/12):      key 0   key 32   key 33   others
      row A                   1.5     3        2        -192
      row B                   3       2        1.5      -192
    Row A's maximum arrives in key block 1; row B's is in key block 0, so in
    block 1 its largest P is e^-1, not 1."""
    d, N = 64, 64
    Q = np.zeros((N, d), np.float32)
    Q[40, 0] = 6.0
    Q[50, 32] = 6.0
    K = np.full((N, d), 0.0, np.float32); K[:, 0] = -384.0; K[:, 32] = -384.0
    K[0, 0], K[32, 0], K[33, 0] = 3.0, 6.0, 4.0
    K[0, 32], K[32, 32], K[33, 32] = 6.0, 4.0, 3.0
    rng = np.random.default_rng(104)
    V = torch.from_numpy(rng.standard_normal((N, d)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    qc, qs = orc.quant_mx_rows(Q[None]); kc, ks = orc.quant_mx_rows(K[None]); vc, vs = orc.quant_mx_cols(V[None])
    assert np.array_equal(_deq_mx(kc[0], ks[0]), K)
    t = dict(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Qh=Q, Kh=K, Vh=V)
    return t, _deq_mx(vc[0], vs[0]).T, V.astype(np.float64), N, d


def test_thrift_two_level_is_per_row(orc):
    """Both key blocks through the FP4 path.  Two-level P scales each row of
    the block by 6 / (its own largest P): row A (block max P 1) rounds
    6 (1, e^-1) = (6, 2.21) to (6, 2); row B (block max P e^-1) rounds
    6 (1, e^-0.5) = (6, 3.64) to (6, 4).  A factor shared by the tile's
    rows (6 / 1) would round row B's P to (1.5, 1) / 6 instead.  The factor r
    is held in fp32, so row B's block dequantises as fp32(e^-1)/6 x codes."""
    t, Vf4, _, N, d = _thrift_case(orc)
    idx = np.full((2, 2), -1, np.int32); cnt = np.zeros(2, np.int32)
    O, lse = orc.thrift_fwd(sel_idx=idx, sel_cnt=cnt, Nq=N, Nk=N, d=d, blk=32, tau=1 / 12, **t)
    e = math.exp
    alpha_a = e(1.5 - 3)
    la = alpha_a + 1 + e(-1)
    ref_a = (alpha_a * Vf4[0] + Vf4[32] + (2 / 6) * Vf4[33]) / la
    lb = 1 + e(-1) + e(-1.5)
    rb = float(np.float32(e(-1)))
    ref_b = (Vf4[0] + rb * (Vf4[32] + (4 / 6) * Vf4[33])) / lb
    tol = 1e-12 * np.abs(Vf4).max()
    assert np.abs(O[40] - ref_a).max() < tol and np.abs(O[50] - ref_b).max() < tol
    assert abs(lse[40] - (3 + math.log(la))) < 1e-12 and abs(lse[50] - (3 + math.log(lb))) < 1e-12
    shared = (Vf4[0] + (1.5 / 6) * Vf4[32] + (1 / 6) * Vf4[33]) / lb
    assert np.abs(shared - ref_b).max() > 1e-3


def test_thrift_paths_merge_with_running_max(orc):
    """Key block 1 selected for query block 1: it runs second, in bf16, after
    the FP4 block 0, against the running max that block 0 left.  Row A:
    block 0 gives m = 1.5, block 1 moves it to 3 (alpha = e^-1.5) with
    bf16 P (1, e^-1); row B keeps m = 3 and rounds (e^-1, e^-1.5) to bf16."""
    t, Vf4, Vh, N, d = _thrift_case(orc)
    idx = np.array([[0, -1], [1, -1]], np.int32); cnt = np.array([1, 1], np.int32)
    O, _ = orc.thrift_fwd(sel_idx=idx, sel_cnt=cnt, Nq=N, Nk=N, d=d, blk=32, tau=1 / 12, **t)
    e = math.exp
    alpha_a = e(-1.5)
    ref_a = (alpha_a * Vf4[0] + Vh[32] + _bf16(e(-1)) * Vh[33]) / (alpha_a + 1 + e(-1))
    ref_b = (Vf4[0] + _bf16(e(-1)) * Vh[32] + _bf16(e(-1.5)) * Vh[33]) / (1 + e(-1) + e(-1.5))
    tol = 1e-12 * np.abs(Vh).max()
    assert np.abs(O[40] - ref_a).max() < tol and np.abs(O[50] - ref_b).max() < tol


# ---------------------------------------------------------------------------
# SageBwd: one INT8 scale per 128 x 64 tile for P^ and dS^, dO per 128 tokens
# ---------------------------------------------------------------------------
def _sbwd_identity_q(rng, N=128):
    """Q codes = identity (scale 1), so Q^ = I and s_ij = tau * kc[j, i] * ks[j / 64]:
    dK[j, c] = tau * dS_cj exposes dS (or dS^) and the scores are set by K."""
    d = N
    qc = np.eye(N, d, dtype=np.int8)
    qs = np.ones(1, np.float32)
    kc = rng.integers(-127, 128, (N, d)).astype(np.int8)
    ks = np.array([0.02, 0.03], np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    O = rng.standard_normal((N, d)).astype(np.float32)
    return qc, qs, kc, ks, V, O


def _tile_grid_check(exact, rounded, tiles):
    """Every rounded value of a tile is an integer multiple of (tile absmax)/127
    and within half a step of the exact value (the step may be held in fp32:
    a relative 1e-7 of slack)."""
    for sl in tiles:
        x, r = exact[sl], rounded[sl]
        a = np.abs(x).max()
        step = a / 127
        k = r / step
        assert np.abs(k - np.rint(k)).max() < 1e-6 * 127
        assert np.abs(r - x).max() <= step / 2 * (1 + 1e-5)


def test_sage_bwd_ds_one_scale_per_tile(orc):
    rng = np.random.default_rng(105)
    N, tau = 128, 0.05
    qc, qs, kc, ks, V, O = _sbwd_identity_q(rng, N)
    dO = (rng.standard_normal((N, N)) * 0.1).astype(np.float32)
    s = tau * kc.T.astype(np.float64) * np.repeat(ks, 64)[None, :]     # s[i, j]
    lse = (np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)).astype(np.float32)
    kw = dict(qc=qc, qs=qs, kc=kc, ks=ks, V=V, dO=dO, O=O, lse=lse, causal=False, tau=tau)
    _, dKu, _ = orc.sage_bwd(quantize=False, **kw)
    _, dKq, _ = orc.sage_bwd(quantize=True, **kw)
    dS, dSq = dKu.T / tau, dKq.T / tau                     # [query i, key j]
    _tile_grid_check(dS, dSq, [np.s_[:, 0:64], np.s_[:, 64:128]])
    # a per-row scale would put row i on the grid of its own absmax / 127: not so here
    i = int(np.argmin(np.abs(dS[:, :64]).max(1)))
    own = np.abs(dS[i, :64]).max() / 127
    assert np.abs(dSq[i, :64] / own - np.rint(dSq[i, :64] / own)).max() > 1e-3


def test_sage_bwd_p_one_scale_per_tile(orc):
    rng = np.random.default_rng(106)
    N, tau = 128, 0.05
    qc, qs, kc, ks, V, O = _sbwd_identity_q(rng, N)
    dO = np.eye(N, dtype=np.float32)                        # dV[j, c] = P^_cj (times the dO code scale)
    s = tau * kc.T.astype(np.float64) * np.repeat(ks, 64)[None, :]
    lse = (np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)).astype(np.float32)
    kw = dict(qc=qc, qs=qs, kc=kc, ks=ks, V=V, dO=dO, O=O, lse=lse, causal=False, tau=tau)
    _, _, dVu = orc.sage_bwd(quantize=False, **kw)
    _, _, dVq = orc.sage_bwd(quantize=True, **kw)
    kappa = 127.0 * float(np.float32(1.0) / np.float32(127.0))      # dO^ = 127 codes x fp32(1/127)
    P, Pq = dVu.T, dVq.T / kappa
    _tile_grid_check(P, Pq, [np.s_[:, 0:64], np.s_[:, 64:128]])
    i = int(np.argmin(P[:, :64].max(1)))
    own = P[i, :64].max() / 127
    assert np.abs(Pq[i, :64] / own - np.rint(Pq[i, :64] / own)).max() > 1e-3


def test_sage_bwd_do_blocks_of_128(orc):
    """With P one-hot (s_ii far above every other score) dV_j is the
    dequantised dO row j: its grid is the absmax of dO's 128-token block over
    127, although the second half of each block is 100x smaller than the
    first (a 64-token block would give that half a finer grid)."""
    rng = np.random.default_rng(107)
    N, d, tau = 256, 64, 8.0
    codes = rng.choice(np.array([-127, 127], np.int8), (N, d))
    G = codes.astype(np.int64) @ codes.astype(np.int64).T
    off = G - np.diag(np.diag(G))
    assert (np.diag(G) - off.max(1)).min() * tau / 127 ** 2 > 150       # other P below e^-150
    qs = np.full(2, 1 / 127, np.float32); ks = np.full(4, 1 / 127, np.float32)
    dO = rng.standard_normal((N, d)).astype(np.float32)
    for b in range(0, N, 128):
        dO[b + 64:b + 128] *= 0.01
    V = rng.standard_normal((N, d)).astype(np.float32); O = rng.standard_normal((N, d)).astype(np.float32)
    s = tau * G * float(np.float32(1 / 127)) ** 2
    lse = s.max(1).astype(np.float32)
    _, _, dV = orc.sage_bwd(qc=codes, qs=qs, kc=codes, ks=ks, V=V, dO=dO, O=O, lse=lse, causal=False, tau=tau,
                            quantize=True)
    # every diagonal P is within 1e-7 of its tile's largest, so its INT8 code is
    # 127 and P^_ii is that largest value a_T (one per 64-key tile)
    Pii = np.exp(np.diag(s) - lse.astype(np.float64))
    a_T = np.repeat(Pii.reshape(-1, 64).max(1), 64)
    assert (Pii / a_T).min() > 1 - 1e-6
    deq = dV / a_T[:, None]
    _tile_grid_check(dO.astype(np.float64), deq, [np.s_[0:128], np.s_[128:256]])
    half = np.abs(dO[64:128]).max() / 127
    assert np.abs(deq[64:128] / half - np.rint(deq[64:128] / half)).max() > 1e-3


# ---------------------------------------------------------------------------
# Attn-QAT backward: dS rounded to bf16 (the operand of the bf16 products)
# ---------------------------------------------------------------------------
def test_qat_bwd_ds_is_bf16(orc):
    """Q rows one-hot (Q^ = I in MXFP4: 1 = 4 x 2^-2), so dK[j, c] = tau dS_cj:
    the quantised backward's dS equals torch's bf16 cast of the unrounded dS
    (the straight-through estimator keeps the unrounded P in dS)."""
    rng = np.random.default_rng(108)
    N = d = 128
    tau = 0.1
    Q = np.eye(N, d, dtype=np.float32)
    K = rng.standard_t(3, (N, d)).astype(np.float32)
    V = rng.standard_t(3, (N, d)).astype(np.float32)
    qc, qs = orc.quant_mx_rows(Q[None]); kc, ks = orc.quant_mx_rows(K[None]); vc, vs = orc.quant_mx_cols(V[None])
    assert np.array_equal(_deq_mx(qc[0], qs[0]), Q)
    t = dict(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0])
    _, Oa, lse = orc.qat_fwd(Nq=N, Nk=N, d=d, tau=tau, kv_tile=64, **t)
    dO = (rng.standard_normal((N, d)) * 0.1).astype(np.float32)
    kw = dict(dO=dO, O_aux=Oa.astype(np.float32), lse=lse.astype(np.float32), Nq=N, Nk=N, d=d, tau=tau, **t)
    _, dKu, _ = orc.qat_bwd(quantize_p=False, **kw)
    _, dKq, _ = orc.qat_bwd(quantize_p=True, **kw)
    dS, dSq = dKu.T / tau, dKq.T / tau
    want = torch.from_numpy(dS).to(torch.bfloat16).double().numpy()
    assert np.abs(dSq - want).max() <= 1e-15 * np.abs(want).max()
    assert np.abs(dSq - dS).max() > 0
