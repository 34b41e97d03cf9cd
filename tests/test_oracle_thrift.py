"""Pins of the oracle's ThriftAttention paths (CPU only): the budget rule,
selection against a brute-force library sort, the online merge of the two
precision paths (exact for any selection once quantisation is off), split
invariance of decode, and special cases of the FP4 path."""
import json
import math
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
PPM = int(round(FACTS["thrift_budget"]["fraction"] * 1e6))


def test_budget_counts(orc):
    # ThriftAttention, Results: 5% block budget.  Per causal query block i the
    # valid key blocks number i + 1; at least one pair is always promoted.
    total = sum(orc.budget_count(i + 1, PPM) for i in range(1024))
    assert total == sum(max(1, math.ceil((i + 1) / 20)) for i in range(1024)) == 26728
    assert orc.budget_count(1024, PPM) == 52          # decode: one query row against 1024 blocks
    assert orc.budget_count(20, PPM) == 1 and orc.budget_count(21, PPM) == 2
    assert orc.budget_count(7, 0) == 1 and orc.budget_count(7, 1_000_000) == 7 and orc.budget_count(0, PPM) == 0


def test_selection_brute_force(orc):
    rng = np.random.default_rng(30)
    nqb, nkb, d = 40, 40, 16
    qbar = rng.standard_normal((nqb, d)).astype(np.float32)
    kbar = rng.standard_normal((nkb, d)).astype(np.float32)
    kbar[5] = kbar[6]                                   # an exact tie: the smaller index wins
    for causal, ppm in ((True, PPM), (True, 250_000), (False, 100_000)):
        idx, cnt = orc.select_blocks(qbar, kbar, causal, ppm, max_sel=16)
        S = qbar.astype(np.float64) @ kbar.astype(np.float64).T
        for i in range(nqb):
            nv = i + 1 if causal else nkb
            k = min(16, max(1, math.ceil(nv * ppm / 1e6 - 1e-12)))
            order = np.lexsort((np.arange(nv), -S[i, :nv]))    # score descending, then index
            want = np.sort(order[:k])
            assert cnt[i] == k and np.array_equal(idx[i, :k], want) and np.all(idx[i, k:] == -1)


def _thrift_inputs(orc, rng, N=256, d=32, blk=32):
    Q = (rng.standard_normal((N, d)) * 1.5).astype(np.float32)
    K = (rng.standard_normal((N, d)) * 1.5).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    qc, qs = orc.quant_mx_rows(Q[None]); kc, ks = orc.quant_mx_rows(K[None]); vc, vs = orc.quant_mx_cols(V[None])
    return dict(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Qh=Q, Kh=K, Vh=V)


def _random_selection(rng, nb, max_sel, mode):
    idx = np.full((nb, max_sel), -1, np.int32)
    cnt = np.zeros(nb, np.int32)
    for i in range(nb):
        pool = np.arange(i + 1)
        k = {"none": 0, "all": i + 1, "some": rng.integers(0, i + 2)}[mode]
        k = min(k, max_sel)
        pick = np.sort(rng.choice(pool, size=k, replace=False)) if k else np.array([], np.int32)
        idx[i, :k] = pick
        cnt[i] = k
    return idx, cnt


@pytest.mark.parametrize("mode", ["none", "all", "some"])
def test_thrift_merge_exact_without_quantisation(orc, mode):
    rng = np.random.default_rng(31)
    t = _thrift_inputs(orc, rng)
    idx, cnt = _random_selection(rng, 8, 8, mode)
    O, lse = orc.thrift_fwd(sel_idx=idx, sel_cnt=cnt, Nq=256, Nk=256, d=32, blk=32, tau=0.3,
                            quantize=False, **t)
    rO, rl = orc.ref_fwd(t["Qh"], t["Kh"], t["Vh"], True, 0.3)
    assert np.abs(O - rO).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12


def test_thrift_all_bf16_close(orc):
    """rho = 1: every valid pair takes the bf16 path; the only rounding is bf16(P)."""
    rng = np.random.default_rng(32)
    t = _thrift_inputs(orc, rng)
    idx, cnt = _random_selection(rng, 8, 8, "all")
    O, _ = orc.thrift_fwd(sel_idx=idx, sel_cnt=cnt, Nq=256, Nk=256, d=32, blk=32, tau=0.3, **t)
    rO, _ = orc.ref_fwd(t["Qh"], t["Kh"], t["Vh"], True, 0.3)
    assert np.abs(O - rO).max() <= np.abs(t["Vh"]).max() * 2 ** -8


def test_thrift_fp4_close_and_order(orc):
    """rho = 0: the FP4 path with two-level P stays within the FP4 error of the
    exact attention on the FP4 operands; promoting pairs moves it toward the
    bf16 result."""
    rng = np.random.default_rng(33)
    t = _thrift_inputs(orc, rng)
    tab = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])

    def deq(c, s):
        v = np.stack([tab[c & 0xF], tab[c >> 4]], -1).reshape(c.shape[0], -1)
        return v * np.repeat(2.0 ** (s.astype(np.int64) - 127), 32, axis=-1)

    Qd, Kd, Vd = deq(t["qc"], t["qs"]), deq(t["kc"], t["ks"]), deq(t["vc_t"], t["vs_t"]).T
    none = _random_selection(rng, 8, 8, "none")
    O0, _ = orc.thrift_fwd(sel_idx=none[0], sel_cnt=none[1], Nq=256, Nk=256, d=32, blk=32, tau=0.3, **t)
    o, = [torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(np.ascontiguousarray(x, np.float64))[None] for x in (Qd, Kd, Vd)),
        is_causal=True, scale=0.3)[0].numpy()]
    assert np.abs(O0 - o).max() <= np.abs(Vd).max() * 2 ** -3
    assert np.abs(O0 - o).mean() <= np.abs(Vd).max() * 2 ** -6
    rO, _ = orc.ref_fwd(t["Qh"], t["Kh"], t["Vh"], True, 0.3)
    allsel = _random_selection(rng, 8, 8, "all")
    O1, _ = orc.thrift_fwd(sel_idx=allsel[0], sel_cnt=allsel[1], Nq=256, Nk=256, d=32, blk=32, tau=0.3, **t)
    assert np.abs(O1 - rO).mean() < np.abs(O0 - rO).mean()


def test_thrift_fp4_one_hot_exact(orc):
    """All the mass on one key: its P is exactly 1 (the running max), two-level
    P puts it at exactly 6 (r/6 * 6 = 1), every other P rounds to zero, so the
    FP4 path returns that key's FP4 V row."""
    d, N, blk = 32, 64, 32
    Q = np.zeros((N, d), np.float32); K = np.zeros((N, d), np.float32)
    Q[:, 0] = 6.0; K[:, 0] = -6.0; K[3, 0] = 6.0
    rng = np.random.default_rng(34)
    V = rng.standard_normal((N, d)).astype(np.float32)
    qc, qs = orc.quant_mx_rows(Q[None]); kc, ks = orc.quant_mx_rows(K[None]); vc, vs = orc.quant_mx_cols(V[None])
    idx = np.full((2, 2), -1, np.int32); cnt = np.zeros(2, np.int32)
    O, _ = orc.thrift_fwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Qh=Q, Kh=K, Vh=V,
                          sel_idx=idx, sel_cnt=cnt, Nq=N, Nk=N, d=d, blk=blk, tau=1.0)
    tab = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
    c = vc[0][:, 1]                                       # tokens 2, 3 of every channel
    v3 = tab[c >> 4] * 2.0 ** (vs[0][:, 0].astype(np.int64) - 127)
    assert np.abs(O[3:] - v3[None]).max() < 1e-12


@pytest.mark.parametrize("splits", [1, 3, 8, 16])
def test_decode_exact_without_quantisation_any_split(orc, splits):
    rng = np.random.default_rng(35)
    t = _thrift_inputs(orc, rng, N=512)
    q = (rng.standard_normal(32) * 1.5).astype(np.float32)
    qc, qs = orc.quant_mx_rows(q[None, None])
    sel = np.array([2, 5, 11], np.int32)
    kw = {k: t[k] for k in ("kc", "ks", "vc_t", "vs_t")}
    o, lse = orc.thrift_decode(qc=qc[0], qs=qs[0], q=q, Kh=t["Kh"], Vh=t["Vh"], sel=sel, Nk=512, d=32, blk=32,
                               tau=0.3, num_splits=splits, quantize=False, **kw)
    rO, rl = orc.ref_fwd(q[None], t["Kh"], t["Vh"], False, 0.3)
    assert np.abs(o - rO[0]).max() < 1e-12 and abs(lse - rl[0]) < 1e-12


def test_decode_matches_prefill_last_row(orc):
    """With one split, decode of the last token runs the same block order as
    the last row of prefill given the same selection."""
    rng = np.random.default_rng(36)
    t = _thrift_inputs(orc, rng, N=256)
    sel = np.array([1, 4, 7], np.int32)
    idx = np.full((8, 8), -1, np.int32); cnt = np.ones(8, np.int32); idx[:, 0] = 0
    idx[7, :3] = sel; cnt[7] = 3
    O, lse = orc.thrift_fwd(sel_idx=idx, sel_cnt=cnt, Nq=256, Nk=256, d=32, blk=32, tau=0.3, qblocks=(7, 8), **t)
    qc, qs = t["qc"][255:256], t["qs"][255:256]
    o, l = orc.thrift_decode(qc=qc, qs=qs, kc=t["kc"], ks=t["ks"], vc_t=t["vc_t"], vs_t=t["vs_t"],
                             q=t["Qh"][255], Kh=t["Kh"], Vh=t["Vh"], sel=sel, Nk=256, d=32, blk=32, tau=0.3,
                             num_splits=1)
    assert np.abs(O[-1] - o).max() < 1e-12 and abs(lse[-1] - l) < 1e-12
