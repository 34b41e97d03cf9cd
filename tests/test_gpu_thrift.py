"""GPU parity of the ThriftAttention path against the oracle, through the C
ABI: block selection (bit-exact indices and counts)."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.helpers import assert_same, compare_outputs, tau_for

pytestmark = pytest.mark.gpu

PPM_5 = 50_000          # the pages' 5 % budget, in parts per million


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_quantized_attention_amd as bqa
    bqa.lib()


def _select_gpu(p, qbar, kbar):
    import bit_quantized_attention_amd as bqa
    B, Hq, nqb, d = qbar.shape
    ms = bqa.max_sel(p)
    idx = torch.full((B, Hq, nqb, ms), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
    bqa.bqa_select_blocks(p, torch.from_numpy(qbar).cuda(), torch.from_numpy(kbar).cuda(), idx, cnt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy(), ms


def _select_oracle(qbar, kbar, causal, ppm, ms):
    B, Hq, nqb, d = qbar.shape
    Hkv = kbar.shape[1]
    idx = np.empty((B, Hq, nqb, ms), np.int32)
    cnt = np.empty((B, Hq, nqb), np.int32)
    for b in range(B):
        for h in range(Hq):
            idx[b, h], cnt[b, h] = orc.select_blocks(qbar[b, h], kbar[b, h // (Hq // Hkv)], causal, ppm, ms)
    return idx, cnt


@pytest.mark.parametrize("ppm", [PPM_5, 250_000, 0, 1_000_000])
def test_selection_from_block_means(ppm):
    """c5 recipe (low-rank shared component, GQA 8/2) at N=4096: the GPU's
    own block means feed the GPU selection; the oracle computes its means
    from the same inputs."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import to_device
    w = wl.with_len(wl.WORKLOADS["c5"], 4096, hq=8, hkv=2)
    p = bqa.problem(B=1, Hq=8, Hkv=2, Nq=4096, Nk=4096, d=128, causal=1, mode=bqa.BQA_THRIFT, sel_block=128,
                    hp_budget_ppm=ppm)
    means = {}
    for name, role, H in (("q", bqa.BQA_ROLE_Q, 8), ("k", bqa.BQA_ROLE_K, 2)):
        X = wl.build(w, name)
        codes = torch.empty((1, H, 4096, 64), dtype=torch.uint8, device="cuda")
        scales = torch.empty((1, H, 4096, 4), dtype=torch.uint8, device="cuda")
        bm = torch.empty((1, H, 32, 128), dtype=torch.float32, device="cuda")
        bqa.bqa_quantize_blocks(p, role, to_device(X, "bf16"), bqa.qtensor(bqa.BQA_MXFP4, 0, 32, codes, scales),
                                block_means=bm)
        means[name] = (bm, orc.block_means(X.reshape(H, 4096, 128), 128).reshape(1, H, 32, 128))
    torch.cuda.synchronize()
    qg, kg = (means[n][0].cpu().numpy() for n in ("q", "k"))
    assert_same(qg, means["q"][1], "q block means")
    assert_same(kg, means["k"][1], "k block means")
    ms = bqa.max_sel(p)
    idx, cnt, _ = _select_gpu(p, means["q"][1], means["k"][1])
    ridx, rcnt = _select_oracle(means["q"][1], means["k"][1], True, ppm, ms)
    assert_same(cnt, rcnt, "selection counts")
    assert_same(idx, ridx, "selected blocks")


def _lowrank_means(rng, B, H, nb, d, rank=4):
    """Block means shaped like the c5 recipe's: a shared low-rank part per
    head plus the block-averaged noise of 128 tokens."""
    W = rng.standard_normal((H, rank, d)) / np.sqrt(d)
    a = rng.standard_normal((B, H, nb, rank)) * 0.5
    m = np.sqrt(d) * np.einsum("bhnr,hrd->bhnd", a, W) + rng.standard_normal((B, H, nb, d)) / np.sqrt(128)
    return m.astype(np.float32)


def test_selection_full_size_prefill():
    """Full c5 prefill shape: 32 query heads, 8 KV heads, 1024 x 1024 causal
    block pairs, 5 % budget (26,728 pairs per head)."""
    import bit_quantized_attention_amd as bqa
    rng = np.random.default_rng(51)
    qbar = _lowrank_means(rng, 1, 32, 1024, 128)
    kbar = _lowrank_means(rng, 1, 8, 1024, 128)
    kbar[0, 3, 10] = kbar[0, 3, 11]                       # an exact tie: the smaller index ranks first
    p = bqa.problem(B=1, Hq=32, Hkv=8, Nq=131072, Nk=131072, d=128, causal=1, mode=bqa.BQA_THRIFT, sel_block=128,
                    hp_budget_ppm=PPM_5)
    idx, cnt, ms = _select_gpu(p, qbar, kbar)
    assert ms == 52
    ridx, rcnt = _select_oracle(qbar, kbar, True, PPM_5, ms)
    assert_same(cnt, rcnt, "selection counts")
    assert int(cnt[0, 0].sum()) == 26728
    assert_same(idx, ridx, "selected blocks")


def test_selection_decode():
    """Decode: one query per (b, head) against 1024 key blocks, k = 52."""
    import bit_quantized_attention_amd as bqa
    rng = np.random.default_rng(52)
    qbar = _lowrank_means(rng, 16, 32, 1, 128)
    kbar = _lowrank_means(rng, 16, 8, 1024, 128)
    p = bqa.problem(B=16, Hq=32, Hkv=8, Nq=1, Nk=131072, d=128, causal=1, mode=bqa.BQA_THRIFT, sel_block=128,
                    hp_budget_ppm=PPM_5)
    idx, cnt, ms = _select_gpu(p, qbar, kbar)
    ridx, rcnt = _select_oracle(qbar, kbar, True, PPM_5, ms)
    assert np.all(cnt == 52)
    assert_same(cnt, rcnt, "selection counts")
    assert_same(idx, ridx, "selected blocks")


@pytest.mark.parametrize("nkb,ppm", [(1500, PPM_5), (1500, 1_000_000), (3000, 250_000), (1024, 1_000_000),
                                     (37, PPM_5), (1, PPM_5)])
def test_selection_row_lengths(nkb, ppm):
    """Rows of 1 to 3000 key blocks (the single-wavefront sort up to 1024,
    the workgroup sort beyond, with its narrower LDS pieces past 2048), two
    query blocks at the bottom-right end of the causal mask, exact ties."""
    import bit_quantized_attention_amd as bqa
    rng = np.random.default_rng(53 + nkb)
    nqb = min(2, nkb)
    qbar = _lowrank_means(rng, 1, 4, nqb, 128)
    kbar = _lowrank_means(rng, 1, 2, nkb, 128)
    if nkb > 8:
        kbar[0, 0, 7] = kbar[0, 0, 3]
        kbar[0, 1, nkb - 1] = kbar[0, 1, 0]
    p = bqa.problem(B=1, Hq=4, Hkv=2, Nq=128 * nqb, Nk=128 * nkb, d=128, causal=1, mode=bqa.BQA_THRIFT,
                    sel_block=128, hp_budget_ppm=ppm)
    idx, cnt, ms = _select_gpu(p, qbar, kbar)
    ridx, rcnt = _select_oracle(qbar, kbar, True, ppm, ms)
    assert_same(cnt, rcnt, "selection counts")
    assert_same(idx, ridx, "selected blocks")


class _ThriftOracle:
    """The oracle's own quantisation, block means and selection of the
    generated inputs (nothing from the GPU)."""

    def __init__(self, Q, K, V, ppm, causal=True):
        self.Hq, self.Hkv, self.Nq, self.Nk, self.d = Q.shape[1], K.shape[1], Q.shape[2], K.shape[2], Q.shape[3]
        self.Q, self.K, self.V = (x.reshape(-1, x.shape[2], x.shape[3]) for x in (Q, K, V))
        self.qc, self.qs = orc.quant_mx_rows(self.Q)
        self.kc, self.ks = orc.quant_mx_rows(self.K)
        self.vc, self.vs = orc.quant_mx_cols(self.V)
        nkb = self.Nk // 128
        self.ms = max(1, min(nkb, -(-nkb * ppm // 1_000_000)))
        qm = orc.block_means(self.Q, 128) if self.Nq > 1 else self.Q.copy()
        km = orc.block_means(self.K, 128)
        self.sel = [orc.select_blocks(qm[iq], km[iq // (self.Hq // self.Hkv)], causal, ppm, self.ms)
                    for iq in range(qm.shape[0])]
        self.causal = causal

    def forward(self, iq, qblocks=None):
        ik = iq // (self.Hq // self.Hkv)
        idx, cnt = self.sel[iq]
        return orc.thrift_fwd(qc=self.qc[iq], qs=self.qs[iq], kc=self.kc[ik], ks=self.ks[ik], vc_t=self.vc[ik],
                              vs_t=self.vs[ik], Qh=self.Q[iq], Kh=self.K[ik], Vh=self.V[ik], sel_idx=idx, sel_cnt=cnt,
                              Nq=self.Nq, Nk=self.Nk, d=self.d, blk=128, hp_tile=32, causal=self.causal,
                              tau=tau_for(self.d),
                              qblocks=qblocks)


def _thrift_run(w, ppm):
    import bit_quantized_attention_amd as bqa  # noqa: F401
    from bit_quantized_attention_amd.runner import ThriftPath, thrift_problem, to_device
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = thrift_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, budget_ppm=ppm)
    path = ThriftPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.step()
    torch.cuda.synchronize()
    return p, path, (Q, K, V)


@pytest.mark.parametrize("ppm", [PPM_5, 250_000, 1_000_000])
def test_thrift_prefill_small(ppm):
    """c5 recipe at N=1024 (8 x 8 causal blocks), GQA 4/2: FP4 blocks first,
    then the selected bf16 blocks, one online softmax; budgets 5 % (one
    bf16 block per query block), 25 % and 100 % (every pair in bf16)."""
    w = wl.with_len(wl.WORKLOADS["c5"], 1024, hq=4, hkv=2)
    p, path, (Q, K, V) = _thrift_run(w, ppm)
    oc = _ThriftOracle(Q, K, V, ppm)
    idx = path.sel_idx.cpu().numpy()
    for iq in range(4):
        assert_same(idx[0, iq], oc.sel[iq][0], f"selection of head {iq}")
    O = path.o.float().cpu().numpy()
    L = path.lse.cpu().numpy()
    for iq in range(4):
        ref, lse = oc.forward(iq)
        compare_outputs(O[0, iq], ref, "bf16", what=f"O[h={iq}]")
        assert np.abs(L[0, iq] - lse).max() < 2e-3


def _decode_run(w, ppm, splits, v_tiled=False):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import to_device
    q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    B, Hq, Hkv, Nk, d = w.B, w.Hq, w.Hkv, w.Nk, w.d
    p = bqa.problem(B=B, Hq=Hq, Hkv=Hkv, Nq=1, Nk=Nk, d=d, causal=1, mode=bqa.BQA_THRIFT, sel_block=128,
                    hp_budget_ppm=ppm, num_splits=splits)
    u8, dev = torch.uint8, "cuda"
    qt, kt, vt = to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    qc = torch.empty((B, Hq, 1, d // 2), dtype=u8, device=dev); qs = torch.empty((B, Hq, 1, d // 32), dtype=u8, device=dev)
    kc = torch.empty((B, Hkv, Nk, d // 2), dtype=u8, device=dev); ks = torch.empty((B, Hkv, Nk, d // 32), dtype=u8, device=dev)
    if v_tiled:      # the decode cache's V blocked by 128 keys
        vc = torch.empty((B, Hkv, Nk // 128, d, 64), dtype=u8, device=dev)
        vs = torch.empty((B, Hkv, Nk // 128, d, 4), dtype=u8, device=dev)
    else:
        vc = torch.empty((B, Hkv, d, Nk // 2), dtype=u8, device=dev); vs = torch.empty((B, Hkv, d, Nk // 32), dtype=u8, device=dev)
    qm = torch.empty((B, Hq, 1, d), dtype=torch.float32, device=dev)
    km = torch.empty((B, Hkv, Nk // 128, d), dtype=torch.float32, device=dev)
    qq, kq, vq = (bqa.qtensor(bqa.BQA_MXFP4, ax, 32, c, s)
                  for ax, c, s in ((0, qc, qs), (0, kc, ks), (2 if v_tiled else 1, vc, vs)))
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_Q, qt, qq, block_means=qm)
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_K, kt, kq, block_means=km)
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_V, vt, vq)
    ms = bqa.max_sel(p)
    idx = torch.empty((B, Hq, 1, ms), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq, 1), dtype=torch.int32, device=dev)
    bqa.bqa_select_blocks(p, qm, km, idx, cnt)
    o = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(bqa.bqa_workspace_size(p, bqa.BQA_OP_FWD), dtype=torch.uint8, device=dev)
    bqa.bqa_attn_fwd(p, q=qq, k=kq, v=vq, q_hi=qt, k_hi=kt, v_hi=vt, sel_idx=idx, sel_cnt=cnt, o=o, lse=lse,
                     workspace=ws)
    torch.cuda.synchronize()
    if v_tiled:
        # the blocked codes are the channel-major ones, key block by key block
        rc, rs = orc.quant_mx_cols(V.reshape(-1, Nk, d))
        g = vc.cpu().numpy().reshape(B * Hkv, Nk // 128, d, 64).transpose(0, 2, 1, 3).reshape(B * Hkv, d, Nk // 2)
        gs = vs.cpu().numpy().reshape(B * Hkv, Nk // 128, d, 4).transpose(0, 2, 1, 3).reshape(B * Hkv, d, Nk // 32)
        assert_same(g, rc, "blocked V codes")
        assert_same(gs, rs, "blocked V scales")
    return p, (q, K, V), idx.cpu().numpy(), o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("ppm,splits,v_tiled", [(PPM_5, 1, False), (PPM_5, 3, False), (250_000, 0, False),
                                                (1_000_000, 2, False), (PPM_5, 3, True), (250_000, 0, True)])
def test_thrift_decode_small(ppm, splits, v_tiled):
    """Decode recipe (batch 2, GQA 8/2) against a 4096-token cache: per split
    the FP4 blocks, then each head's selected blocks in bf16; partials merged."""
    w = wl.with_len(wl.WORKLOADS["c5d"], 4096, b=2, hq=8, hkv=2)
    p, (q, K, V), idx, O, L = _decode_run(w, ppm, splits, v_tiled)
    import bit_quantized_attention_amd as bqa
    ms = bqa.max_sel(p)
    B, Hq, Hkv, d = w.B, w.Hq, w.Hkv, w.d
    qf, Kf, Vf = q.reshape(B * Hq, d), K.reshape(B * Hkv, -1, d), V.reshape(B * Hkv, -1, d)
    qc, qs = orc.quant_mx_rows(qf[:, None])
    kc, ks = orc.quant_mx_rows(Kf)
    vc, vs = orc.quant_mx_cols(Vf)
    km = orc.block_means(Kf, 128)
    nb = w.Nk // 128
    S = splits if splits > 0 else min(nb, -(-2048 // (B * Hkv)))
    for bq in range(B * Hq):
        b, hq = divmod(bq, Hq)
        ik = b * Hkv + hq // (Hq // Hkv)
        ridx, rcnt = orc.select_blocks(qf[bq][None], km[ik], True, ppm, ms)
        assert_same(idx[b, hq, 0], ridx[0], f"decode selection (b={b}, h={hq})")
        ref, lse = orc.thrift_decode(qc=qc[bq], qs=qs[bq], kc=kc[ik], ks=ks[ik], vc_t=vc[ik], vs_t=vs[ik], q=qf[bq],
                                     Kh=Kf[ik], Vh=Vf[ik], sel=ridx[0, :rcnt[0]], Nk=w.Nk, d=d, blk=128, hp_tile=32,
                                     tau=tau_for(d), num_splits=S)
        compare_outputs(O[b, hq, 0], ref, "bf16", what=f"decode o (b={b}, h={hq})")
        assert abs(L[b, hq, 0] - lse) < 2e-3


@pytest.mark.slow
def test_thrift_prefill_full_size_sampled():
    """Full c5 prefill shape (B=1, Hq=32, Hkv=8, N=131072, 5 %): the GPU runs
    the whole problem; the oracle checks sampled query blocks of two heads
    (first, middle and last block, the last against all 1024 key blocks)."""
    from bit_quantized_attention_amd.runner import ThriftPath, thrift_problem, to_device
    w = wl.WORKLOADS["c5"]
    nw = wl.default_workers()
    Q, K, V = (wl.build(w, t, workers=nw) for t in ("q", "k", "v"))
    p = thrift_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, budget_ppm=PPM_5)
    path = ThriftPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.step()
    torch.cuda.synchronize()
    O = path.o[0].float().cpu().numpy()
    L = path.lse[0].cpu().numpy()
    cnt = path.sel_cnt[0].cpu().numpy()
    assert int(cnt[0].sum()) == 26728
    for h in (0, 29):
        hk = h // 4
        Qh, Kh, Vh = Q[0, h], K[0, hk], V[0, hk]
        qc, qs = orc.quant_mx_rows(Qh[None]); kc, ks = orc.quant_mx_rows(Kh[None]); vc, vs = orc.quant_mx_cols(Vh[None])
        idx, rc = orc.select_blocks(orc.block_means(Qh[None], 128)[0], orc.block_means(Kh[None], 128)[0], True, PPM_5, 52)
        assert_same(path.sel_idx[0, h].cpu().numpy(), idx, f"selection of head {h}")
        for qb in (0, 517, 1023):
            ref, lse = orc.thrift_fwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Qh=Qh, Kh=Kh, Vh=Vh,
                                      sel_idx=idx, sel_cnt=rc, Nq=w.Nq, Nk=w.Nk, d=w.d, blk=128, hp_tile=32,
                                      causal=True,
                                      tau=tau_for(w.d), qblocks=(qb, qb + 1))
            compare_outputs(O[h, 128 * qb:128 * qb + 128], ref, "bf16", what=f"O[h={h}, query block {qb}]")
            assert np.abs(L[h, 128 * qb:128 * qb + 128] - lse).max() < 2e-3


@pytest.mark.slow
def test_thrift_decode_full_size_sampled():
    """Full decode shape (B=16, Hq=32, Hkv=8, 131072-token cache, k = 52,
    automatic splits); the oracle checks sampled (batch, head) pairs with the
    same split count."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import ThriftDecodePath, thrift_problem, to_device
    w = wl.WORKLOADS["c5d"]
    nw = wl.default_workers()
    q, K, V = wl.build(w, "q"), wl.build(w, "k", workers=nw), wl.build(w, "v", workers=nw)
    p = thrift_problem(w.B, w.Hq, w.Hkv, 1, w.Nk, w.d, budget_ppm=PPM_5)
    path = ThriftDecodePath(p, to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.build_cache()
    path.step()
    torch.cuda.synchronize()
    O = path.o.float().cpu().numpy()
    L = path.lse.cpu().numpy()
    idx = path.sel_idx.cpu().numpy()
    S = min(1024, -(-2048 // (w.B * w.Hkv)))
    assert bqa.max_sel(p) == 52
    for b, hq in ((0, 0), (7, 13), (15, 31)):
        hk = hq // 4
        Kh, Vh, qh = K[b, hk], V[b, hk], q[b, hq]
        kc, ks = orc.quant_mx_rows(Kh[None]); vc, vs = orc.quant_mx_cols(Vh[None])
        qc, qs = orc.quant_mx_rows(qh[None])
        ridx, rcnt = orc.select_blocks(qh, orc.block_means(Kh[None], 128)[0], True, PPM_5, 52)
        assert_same(idx[b, hq], ridx, f"decode selection (b={b}, h={hq})")
        ref, lse = orc.thrift_decode(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], q=qh[0], Kh=Kh,
                                     Vh=Vh, sel=ridx[0, :rcnt[0]], Nk=w.Nk, d=w.d, blk=128, hp_tile=32, tau=tau_for(w.d),
                                     num_splits=S)
        compare_outputs(O[b, hq, 0], ref, "bf16", what=f"decode o (b={b}, h={hq})")
        assert abs(L[b, hq, 0] - lse) < 2e-3


def test_thrift_score_jump_rescales():
    """The first key blocks score far below the later ones (more than 64
    binades): the running maximum jumps in both the FP4 and the bf16 path."""
    from bit_quantized_attention_amd.runner import ThriftPath, thrift_problem, to_device
    rng = np.random.default_rng(43)
    N, d = 1024, 128
    Q, K, V = (rng.standard_normal((1, 2, N, d)).astype(np.float32) for _ in range(3))
    K = K[:, :1].copy(); V = V[:, :1].copy()
    Q[..., 0] = 30.0
    K[0, 0, :256, 0] = -30.0
    K[0, 0, 256:, 0] = 30.0
    Q, K, V = (wl.round_to(x, "bf16").reshape(x.shape) for x in (Q, K, V))
    for ppm in (PPM_5, 250_000):
        p = thrift_problem(1, 2, 1, N, N, d, budget_ppm=ppm)
        path = ThriftPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
        path.step()
        torch.cuda.synchronize()
        oc = _ThriftOracle(Q, K, V, ppm)
        O = path.o.float().cpu().numpy()
        for iq in range(2):
            assert_same(path.sel_idx[0, iq].cpu().numpy(), oc.sel[iq][0], f"selection h={iq}")
            ref, lse = oc.forward(iq)
            compare_outputs(O[0, iq], ref, "bf16", what=f"O[h={iq}] budget {ppm}")
            assert np.abs(path.lse[0, iq].cpu().numpy() - lse).max() < 2e-3
