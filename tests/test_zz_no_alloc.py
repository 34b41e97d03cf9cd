"""The allocation-free decode entry point (bqa_attn_decode_static) against
the workspace one (bqa_attn_fwd, ThriftAttention decode) through the C ABI:
the same kernels, so the outputs must agree bit for bit -- on two calls in a
row, the second with a smaller problem (the static partials array keeps the
first call's contents)."""
import ctypes as C

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _decode_pair(B, Hq, Hkv, Nk, ppm, splits):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import ThriftDecodePath, thrift_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c5d"], Nk, b=B, hq=Hq, hkv=Hkv)
    q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = thrift_problem(B, Hq, Hkv, 1, Nk, 128, budget_ppm=ppm, num_splits=splits)
    path = ThriftDecodePath(p, to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.build_cache()
    path.quantize()
    path.forward()                                    # workspace entry point
    o_ws, lse_ws = path.o.clone(), path.lse.clone()
    o = torch.full_like(path.o, float("nan"))
    lse = torch.full_like(path.lse, float("nan"))
    st = bqa.lib().bqa_attn_decode_static(C.byref(p), C.byref(path.qq), C.byref(path.kq), C.byref(path.vq),
                                          C.byref(bqa.dense(path.q)), C.byref(bqa.dense(path.k)),
                                          C.byref(bqa.dense(path.v)), C.c_void_p(path.sel_idx.data_ptr()),
                                          C.c_void_p(path.sel_cnt.data_ptr()), C.byref(bqa.dense(o)),
                                          C.c_void_p(lse.data_ptr()),
                                          C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bqa.BQA_OK, bqa.bqa_status_string(st)
    torch.cuda.synchronize()
    return o_ws, lse_ws, o, lse


def test_static_decode_matches_workspace_twice():
    # first call: 4 x 8 heads against 8192 keys, 4 splits; second: smaller
    for (B, Hq, Hkv, Nk, ppm, splits) in ((4, 8, 2, 8192, 50_000, 4), (2, 4, 1, 2048, 250_000, 2)):
        o_ws, lse_ws, o, lse = _decode_pair(B, Hq, Hkv, Nk, ppm, splits)
        assert torch.equal(o, o_ws), (B, Hq, Nk)
        assert torch.equal(lse, lse_ws), (B, Hq, Nk)
        assert torch.isfinite(o.float()).all()
