"""GPU parity of the quantisers against the oracle (bit-exact codes, scales,
smoothing means and block means), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.helpers import assert_same

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _mx_rows_gpu(p, role, x_t, means=False):
    import bit_quantized_attention_amd as bqa
    B, H, N, d = x_t.shape
    codes = torch.empty((B, H, N, d // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device="cuda")
    bm = torch.empty((B, H, (N + 127) // 128, d), dtype=torch.float32, device="cuda") if means else None
    q = bqa.qtensor(bqa.BQA_MXFP4, 0, 32, codes, scales)
    bqa.bqa_quantize_blocks(p, role, x_t, q, block_means=bm)
    return codes, scales, bm


def _mx_cols_gpu(p, x_t):
    import bit_quantized_attention_amd as bqa
    B, H, N, d = x_t.shape
    codes = torch.empty((B, H, d, N // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, d, N // 32), dtype=torch.uint8, device="cuda")
    q = bqa.qtensor(bqa.BQA_MXFP4, 1, 32, codes, scales)
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_V, x_t, q)
    return codes, scales


@pytest.mark.parametrize("wname,n", [("c4", 1024), ("c5", 2048)])
def test_mxfp4_quantisers_bit_exact(wname, n):
    """MXFP4 along d (Q, K, with 128-token block means) and along tokens (V):
    heavy-tailed Student-t inputs (Attn-QAT recipe) and the low-rank recipe."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import to_device
    w = wl.with_len(wl.WORKLOADS[wname], n, hq=4 if wname == "c4" else 8, hkv=4 if wname == "c4" else 2)
    p = bqa.problem(B=w.B, Hq=w.Hq, Hkv=w.Hkv, Nq=w.Nq, Nk=w.Nk, d=w.d, causal=int(w.causal),
                    mode=bqa.BQA_QAT_MXFP4 if wname == "c4" else bqa.BQA_THRIFT, sel_block=128)
    for name, role in (("q", bqa.BQA_ROLE_Q), ("k", bqa.BQA_ROLE_K)):
        X = wl.build(w, name)
        c, s, m = _mx_rows_gpu(p, role, to_device(X, "bf16"), means=True)
        torch.cuda.synchronize()
        Xf = X.reshape(-1, X.shape[2], X.shape[3])
        rc, rs = orc.quant_mx_rows(Xf)
        assert_same(c.cpu().numpy().reshape(rc.shape), rc, f"{name} MX codes")
        assert_same(s.cpu().numpy().reshape(rs.shape), rs, f"{name} MX scales")
        assert_same(m.cpu().numpy().reshape(-1, X.shape[2] // 128, X.shape[3]), orc.block_means(Xf, 128),
                    f"{name} block means")
    V = wl.build(w, "v")
    c, s = _mx_cols_gpu(p, to_device(V, "bf16"))
    torch.cuda.synchronize()
    rc, rs = orc.quant_mx_cols(V.reshape(-1, V.shape[2], V.shape[3]))
    assert_same(c.cpu().numpy().reshape(rc.shape), rc, "V MX codes (token axis)")
    assert_same(s.cpu().numpy().reshape(rs.shape), rs, "V MX scales (token axis)")


def test_mxfp4_edge_values():
    """Zero blocks, exact ties, saturation, tiny and huge magnitudes, and a
    single decode query (one-token block mean)."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import to_device
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((1, 2, 256, 128)) * 2.0 ** rng.integers(-30, 30, (1, 2, 256, 1))).astype(np.float32)
    X[0, 0, 3, :32] = 0.0
    X[0, 0, 5, :32] = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4)    # e2m1 ties, saturation at 7
    X[0, 1, 7, 32:64] = -np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4)
    X[0, 1, 9, 64:96] = 1e-38
    X = wl.round_to(X, "bf16").reshape(1, 2, 256, 128)
    p = bqa.problem(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, d=128, mode=bqa.BQA_QAT_MXFP4, sel_block=128)
    c, s, _ = _mx_rows_gpu(p, bqa.BQA_ROLE_Q, to_device(X, "bf16"))
    torch.cuda.synchronize()
    rc, rs = orc.quant_mx_rows(X.reshape(2, 256, 128))
    assert_same(c.cpu().numpy().reshape(rc.shape), rc, "edge MX codes")
    assert_same(s.cpu().numpy().reshape(rs.shape), rs, "edge MX scales")
    # one decode query: its block mean is the query itself
    q1 = X[:, :, :1].copy()
    p1 = bqa.problem(B=1, Hq=2, Hkv=2, Nq=1, Nk=256, d=128, causal=1, mode=bqa.BQA_THRIFT, sel_block=128)
    c, s, m = _mx_rows_gpu(p1, bqa.BQA_ROLE_Q, to_device(q1, "bf16"), means=True)
    torch.cuda.synchronize()
    assert_same(m.cpu().numpy().reshape(2, 128), q1.reshape(2, 128), "decode query mean")


@pytest.mark.parametrize("fmt", ["i8", "e4m3"])
def test_per_channel_v_odd_strides(fmt):
    """Per-channel V from a non-contiguous view (head-interleaved layout)."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import to_device
    w = wl.with_len(wl.WORKLOADS["c2"], 1024, b=2, hq=3, hkv=3)
    V = wl.build(w, "v")
    vt = to_device(np.ascontiguousarray(V.transpose(0, 2, 1, 3)), "bf16").transpose(1, 2)   # [B,H,N,d] view, strided
    p = bqa.problem(B=2, Hq=3, Hkv=3, Nq=1024, Nk=1024, d=128, mode=bqa.BQA_SAGE_I8_F8PV, q_block=128, k_block=64)
    codes = torch.empty((2, 3, 128, 1024), dtype=torch.uint8, device="cuda")
    scales = torch.empty((2, 3, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(bqa.bqa_workspace_size(p, bqa.BQA_OP_QUANTIZE_V), dtype=torch.uint8, device="cuda")
    q = bqa.qtensor(bqa.BQA_FP8E4M3 if fmt == "e4m3" else bqa.BQA_INT8, 1, 1024, codes, scales)
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_V, vt, q, workspace=ws)
    torch.cuda.synchronize()
    rc, rs = orc.quant_chan(V.reshape(6, 1024, 128), fmt)
    assert_same(codes.cpu().numpy().reshape(rc.shape), rc, "V codes")
    assert_same(scales.cpu().numpy().reshape(rs.shape), rs, "V scales")
