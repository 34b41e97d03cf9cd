"""GPU parity of the SageAttention INT8 path (quantisers + forward) against the
oracle, through the C ABI.  Codes, scales, smoothing means and integer scores
must match bit for bit; outputs within max-abs 2e-2 and mean-rel 1e-3 of the
oracle rounded to the output format."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.helpers import SageOracle, assert_same, compare_outputs, tau_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_quantized_attention_amd as bqa
    bqa.lib()


def _run(w, mode_name, q_block, eps, Nq=None, **kw):
    """Generate the workload, run the GPU path, and build the oracle."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SagePath, sage_problem, to_device
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    if Nq is not None:
        Q = np.ascontiguousarray(Q[:, :, -Nq:])
    mode = {"f16": bqa.BQA_SAGE_I8_F16PV, "f8": bqa.BQA_SAGE_I8_F8PV, "i8": bqa.BQA_SAGE_I8_I8PV}[mode_name]
    p = sage_problem(w.B, w.Hq, w.Hkv, Q.shape[2], K.shape[2], w.d, w.causal, mode, q_block=q_block,
                     smooth_k=True, smooth_eps=eps)
    vdt = "fp16" if mode_name == "f16" else w.dtype
    path = SagePath(p, to_device(Q, w.dtype), to_device(K, w.dtype), to_device(V, vdt), **kw)
    path.step()
    torch.cuda.synchronize()
    orc = SageOracle(Q, K, V, q_block=q_block, eps=eps, pv=mode_name)
    return p, path, orc


def _check_codes(p, path, orc):
    assert orc.uncertified == 0
    B, Hq, Hkv, d = p.B, p.Hq, p.Hkv, p.d
    assert_same(path.mu.cpu().numpy().reshape(-1, d), orc.mu, "K token-mean")
    assert_same(path.qc.cpu().numpy().reshape(orc.qc.shape), orc.qc, "Q codes")
    assert_same(path.qs.cpu().numpy().reshape(orc.qs.shape), orc.qs, "Q scales")
    assert_same(path.kc.cpu().numpy().reshape(orc.kc.shape), orc.kc, "K codes")
    assert_same(path.ks.cpu().numpy().reshape(orc.ks.shape), orc.ks, "K scales")
    if orc.vc is not None:
        assert_same(path.vc.cpu().numpy().reshape(orc.vc.shape), orc.vc, "V codes")
        assert_same(path.vs.cpu().numpy().reshape(orc.vs.shape), orc.vs, "V scales")


def _check_heads(p, path, orc, heads, rows=None):
    tau = tau_for(p.d)
    O = path.o.float().cpu().numpy()
    L = path.lse.cpu().numpy()
    fmt = "fp16" if path.o.dtype == torch.float16 else "bf16"
    for (b, h) in heads:
        r = rows or (0, p.Nq)
        ref, lse = orc.forward(b, h, bool(p.causal), tau, rows=r)
        compare_outputs(O[b, h, r[0]:r[1]], ref, fmt, what=f"O[b={b},h={h},rows={r}]")
        assert np.abs(L[b, h, r[0]:r[1]] - lse).max() < 2e-3


def test_c1_tiny_fp16_pv():
    """Tiny INT8 forward (B=H=1, N=128, d=64, non-causal, fp16 P.V)."""
    w = wl.WORKLOADS["c1"]
    p, path, orc = _run(w, "f16", q_block=64, eps=0.0)
    _check_codes(p, path, orc)
    _check_heads(p, path, orc, [(0, 0)])


@pytest.mark.parametrize("N", [512, 1024])
def test_c2_recipe_small_causal(N):
    """c2 recipe (outlier channels, K bias, fp8 P.V) at sizes spanning many tiles."""
    w = wl.with_len(wl.WORKLOADS["c2"], N, b=1, hq=3, hkv=3)
    p, path, orc = _run(w, "f8", q_block=128, eps=0.0)
    _check_codes(p, path, orc)
    _check_heads(p, path, orc, [(0, 0), (0, 2)])


def test_c2_ragged_query_tail():
    """Nq not a multiple of the 128-row workgroup tile (q_block 64): last tile half full."""
    w = wl.with_len(wl.WORKLOADS["c2"], 320, b=1, hq=2, hkv=2)
    p, path, orc = _run(w, "f8", q_block=64, eps=0.0)
    _check_codes(p, path, orc)
    _check_heads(p, path, orc, [(0, 0), (0, 1)])


def test_c2_short_queries_bottom_right_causal():
    """Nq < Nk with causal masking aligned to the bottom-right corner."""
    w = wl.with_len(wl.WORKLOADS["c2"], 512, b=1, hq=2, hkv=2)
    p, path, orc = _run(w, "f8", q_block=128, eps=0.0, Nq=256)
    _check_heads(p, path, orc, [(0, 0), (0, 1)])


def test_c3_recipe_int8_pv():
    """SageBwd training forward (QK-norm inputs, eps=1e-3, int8 P.V)."""
    w = wl.with_len(wl.WORKLOADS["c3"], 512, hq=2, hkv=2)
    p, path, orc = _run(w, "i8", q_block=128, eps=1e-3)
    _check_codes(p, path, orc)
    _check_heads(p, path, orc, [(0, 0), (0, 1)])


def test_c2_full_size_sampled():
    """The full c2 workload (B=2, H=16, N=4096) in the launch configuration the
    benchmark times (Q quantised inside the attention kernel, its codes not
    kept); outputs on sampled query tiles, then every code (Q through the
    stand-alone quantiser)."""
    w = wl.WORKLOADS["c2"]
    p, path, orc = _run(w, "f8", q_block=128, eps=0.0, keep_q_codes=False)
    path.quantize_q()
    torch.cuda.synchronize()
    _check_codes(p, path, orc)
    for (b, h, r) in [(0, 0, (0, 128)), (1, 15, (3968, 4096)), (0, 7, (2048, 2176)), (1, 3, (1920, 2048))]:
        _check_heads(p, path, orc, [(b, h)], rows=r)


def test_debug_scores_bit_exact():
    """Integer Q K^T tiles through the forward kernel's tile code equal the
    oracle codes' exact integer dot products."""
    import bit_quantized_attention_amd as bqa
    w = wl.with_len(wl.WORKLOADS["c2"], 512, b=2, hq=2, hkv=2)
    p, path, orc = _run(w, "f8", q_block=128, eps=0.0)
    out = torch.empty((32, 32), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(0)
    for _ in range(6):
        b, h = int(rng.integers(2)), int(rng.integers(2))
        qt, kt = int(rng.integers(16)), int(rng.integers(16))
        bqa.bqa_debug_qk_scores(p, path.qq, path.kq, b, h, qt, kt, out)
        torch.cuda.synchronize()
        iq = b * 2 + h
        ref = orc.qc[iq, qt * 32:(qt + 1) * 32].astype(np.int64) @ orc.kc[iq, kt * 32:(kt + 1) * 32].astype(np.int64).T
        assert_same(out.cpu().numpy(), ref.astype(np.int32), f"S_int tile b={b} h={h} q={qt} k={kt}")


def test_deterministic_and_zero_block():
    """Two passes give identical bits; an all-zero Q block gets scale 0 and
    zero codes and its rows attend uniformly."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SagePath, sage_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c2"], 512, b=1, hq=2, hkv=2)
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    Q[0, 1, 128:256] = 0.0
    p = sage_problem(1, 2, 2, 512, 512, 128, False, bqa.BQA_SAGE_I8_F8PV)
    path = SagePath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    o1 = path.step().clone()
    c1 = path.qc.clone()
    o2 = path.step().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(c1, path.qc)
    assert path.qs[0, 1, 1].item() == 0.0 and not path.qc[0, 1, 128:256].any()
    orc = SageOracle(Q, K, V, q_block=128, pv="f8")
    ref, _ = orc.forward(0, 1, False, tau_for(128), rows=(128, 256))
    compare_outputs(o1[0, 1, 128:256].float().cpu().numpy(), ref)


@pytest.mark.parametrize("pv", ["f8", "i8"])
def test_score_jump_rescales(pv):
    """Keys after the first tile score far above it (more than 96 binades, in
    log2 units): the running maximum jumps, the rescale factor of the first
    tile's sums underflows to zero, and the result still matches the oracle."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SagePath, sage_problem, to_device
    rng = np.random.default_rng(41)
    N, d = 512, 128
    Q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    K = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    V = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    Q[..., 0] = 30.0
    K[0, 0, :64, 0] = -30.0
    K[0, 0, 64:, 0] = 30.0
    Q, K, V = (wl.round_to(x, "bf16").reshape(x.shape) for x in (Q, K, V))
    mode = bqa.BQA_SAGE_I8_F8PV if pv == "f8" else bqa.BQA_SAGE_I8_I8PV
    p = sage_problem(1, 1, 1, N, N, d, True, mode, q_block=128, smooth_k=True, smooth_eps=0.0)
    path = SagePath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.step()
    torch.cuda.synchronize()
    orc = SageOracle(Q, K, V, q_block=128, pv=pv)
    ref, lse = orc.forward(0, 0, True, tau_for(d))
    # the jump really is that large: log2-unit score difference across key tile 0 / 1
    s = (orc.qc[0].astype(np.float64) @ orc.kc[0].astype(np.float64).T) * np.repeat(orc.qs[0], 128)[:, None] \
        * np.repeat(orc.ks[0], 64)[None, :] * tau_for(d) / np.log(2)
    assert s[200, 64:128].max() - s[200, :64].max() > 96
    compare_outputs(path.o[0, 0].float().cpu().numpy(), ref, "bf16", what=f"O ({pv} P.V, score jump)")
    assert np.abs(path.lse[0, 0].cpu().numpy() - lse).max() < 2e-3


@pytest.mark.parametrize("N,d,causal,hq,hkv", [(128, 64, False, 2, 1), (192, 128, True, 2, 2), (384, 64, True, 4, 2),
                                               (512, 128, False, 4, 2), (640, 64, False, 1, 1)])
def test_f8_shapes(N, d, causal, hq, hkv):
    """fp8 P.V path over the shapes its kernel distinguishes: head dimension 64
    and 128, causal and not, grouped heads, sequences of fewer tiles than its
    LDS ring holds, odd and even query-tile counts (causal pairing), a half
    query tile (q_block 64)."""
    import dataclasses
    w = dataclasses.replace(wl.with_len(wl.WORKLOADS["c2"], N, b=1, hq=hq, hkv=hkv), d=d, causal=causal)
    p, path, orc = _run(w, "f8", q_block=64, eps=0.0)
    _check_codes(p, path, orc)
    _check_heads(p, path, orc, [(0, h) for h in range(hq)])


@pytest.mark.parametrize("N,d,causal,q_block", [(512, 128, True, 128), (320, 128, False, 64), (384, 64, True, 64)])
def test_q_quantised_in_kernel_matches_separate(N, d, causal, q_block):
    """fp8 P.V: Q quantised by the attention kernel gives the same codes and
    scales as the token-block quantiser and bit-identical O and LSE."""
    import dataclasses
    w = dataclasses.replace(wl.with_len(wl.WORKLOADS["c2"], N, b=1, hq=2, hkv=2), d=d, causal=causal)
    _, fused, _ = _run(w, "f8", q_block=q_block, eps=0.0, fuse_q=True)
    _, sep, _ = _run(w, "f8", q_block=q_block, eps=0.0, fuse_q=False)
    assert torch.equal(fused.qc, sep.qc) and torch.equal(fused.qs, sep.qs)
    assert torch.equal(fused.o, sep.o) and torch.equal(fused.lse, sep.lse)


# (N % 256 == 0 at d = 128 runs the one-launch resident kernel, the others the two launches)
KV_JOINT_CASES = [(512, 128, "f8", True, "bf16"), (320, 128, "i8", True, "bf16"), (384, 64, "f8", False, "bf16"),
                  (448, 128, "f8", True, "fp16"), (1024, 128, "i8", True, "fp16"), (768, 128, "f8", False, "bf16"),
                  (256, 128, "f8", True, "bf16")]


def _kv_joint_vs_separate(N, d, pv, smooth, dt, b=2, h=2):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SagePath, sage_problem, to_device
    import dataclasses
    w = dataclasses.replace(wl.with_len(wl.WORKLOADS["c2"], N, b=b, hq=h, hkv=h), d=d)
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    mode = bqa.BQA_SAGE_I8_F8PV if pv == "f8" else bqa.BQA_SAGE_I8_I8PV
    p = sage_problem(b, h, h, N, N, d, True, mode, q_block=64, smooth_k=smooth, smooth_eps=1e-3)
    paths = [SagePath(p, to_device(Q, "bf16"), to_device(K, dt), to_device(V, dt)) for _ in range(2)]
    paths[1].kv_joint = False
    for pa in paths:
        pa.mu.fill_(7.0)
        pa.ws.fill_(0xA5)          # the joint call must not rely on workspace contents
        pa.quantize()
    torch.cuda.synchronize()
    a, b_ = paths
    assert paths[0].kv_joint
    names = ("kc", "ks", "vc", "vs") + (("mu",) if smooth else ())
    for name in names:
        assert torch.equal(getattr(a, name), getattr(b_, name)), name
    # a second call on the same workspace with other inputs: nothing of the
    # first call (flags, partials) may leak into it
    for pa in paths:
        pa.k.mul_(-2.0).add_(0.5)
        pa.v.mul_(0.25)
        pa.quantize()
    torch.cuda.synchronize()
    for name in names:
        assert torch.equal(getattr(a, name), getattr(b_, name)), name + " (second call)"


@pytest.mark.parametrize("N,d,pv,smooth,dt", KV_JOINT_CASES)
def test_kv_joint_matches_separate(N, d, pv, smooth, dt):
    """bqa_quantize_kv gives the K codes, scales, mean and the V codes and
    scales of the per-operand calls bit for bit (bf16 and fp16 inputs, 64- and
    128-token V tiles, both the resident one-launch kernel and the two-launch
    path)."""
    _kv_joint_vs_separate(N, d, pv, smooth, dt)


def test_kv_resident_long_head():
    """One head of 65536 tokens: 256 workgroups meet on one head's flags
    (four per polling lane)."""
    _kv_joint_vs_separate(65536, 128, "f8", True, "bf16", b=1, h=1)


@pytest.mark.parametrize("limit", ["1", "3"])
def test_kv_resident_own_statistics(limit, monkeypatch):
    """With the resident kernel's wait cut to a few polls, workgroups that do
    not see the rest of their head in time take the head's statistics from HBM
    themselves: the bits are the same.  16 heads x 4 chunks of 256 tokens."""
    monkeypatch.setenv("BQA_KV_WAIT_LIMIT", limit)
    _kv_joint_vs_separate(1024, 128, "f8", True, "bf16", b=2, h=8)


def test_kv_joint_in_captured_graph():
    """bqa_quantize_kv captured in a graph (where the call takes the two-launch
    path) and replayed on new inputs matches the eager call on each of them,
    with eager work and synchronisations between the replays."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SagePath, sage_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c2"], 1024, b=2, hq=4, hkv=4)
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = sage_problem(2, 4, 4, 1024, 1024, 128, True, bqa.BQA_SAGE_I8_F8PV, q_block=128, smooth_k=True, smooth_eps=0.0)
    g_path = SagePath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    e_path = SagePath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g_path.quantize()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_path.quantize()
    torch.cuda.synchronize()
    names = ("kc", "ks", "vc", "vs", "mu")
    for rep in range(3):
        scale = 1.0 + 0.5 * rep
        for pa in (g_path, e_path):
            pa.k.copy_(to_device(K * scale - rep, "bf16"))
            pa.v.copy_(to_device(V / scale, "bf16"))
        e_path.quantize()                      # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in names:
            assert torch.equal(getattr(g_path, name), getattr(e_path, name)), f"{name} (replay {rep})"


@pytest.mark.parametrize("N", [384, 512])
def test_token_major_layouts(N):
    """Q, K, V stored token-major ([B, N, H, d] memory viewed as [B, H, N, d]):
    the in-kernel Q quantisation, the joint K/V call (two-launch and resident
    kernels) and the attention follow the strides and give the bits of
    contiguous inputs."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SagePath, sage_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c2"], N, b=2, hq=4, hkv=2)
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = sage_problem(2, 4, 2, N, N, 128, True, bqa.BQA_SAGE_I8_F8PV, q_block=128, smooth_k=True, smooth_eps=0.0)

    def token_major(x):
        t = to_device(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), "bf16")   # memory [B, N, H, d]
        return t.transpose(1, 2)                                                # view [B, H, N, d]
    dense = SagePath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    strided = SagePath(p, token_major(Q), token_major(K), token_major(V))
    assert not strided.q.is_contiguous()
    for pa in (dense, strided):
        pa.step()
    torch.cuda.synchronize()
    for name in ("qc", "qs", "kc", "ks", "vc", "vs", "mu", "o", "lse"):
        assert torch.equal(getattr(dense, name), getattr(strided, name)), name
