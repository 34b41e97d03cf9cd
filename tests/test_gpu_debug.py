"""BQA_DEBUG=1: calls scan their floating-point inputs and return
BQA_E_NONFINITE on a NaN or an infinity (launching nothing else); clean
inputs pass, and without the variable no scan runs."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _sage(debug, bad=None):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SagePath, sage_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c2"], 256, hq=2, hkv=2)
    Q, K, V = (wl.build(w, t) for t in ("q", "k", "v"))
    if bad == "q":
        Q[0, 1, 77, 5] = np.nan
    if bad == "v":
        V[0, 0, 200, 100] = np.inf
    p = sage_problem(1, 2, 2, 256, 256, 128, True, bqa.BQA_SAGE_I8_F8PV, q_block=128, smooth_k=True)
    path = SagePath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), fuse_q=False)
    return bqa, p, path


def test_clean_inputs_pass(monkeypatch):
    monkeypatch.setenv("BQA_DEBUG", "1")
    bqa, p, path = _sage(True)
    path.step()
    torch.cuda.synchronize()
    assert torch.isfinite(path.o.float()).all()


def test_nan_in_q_is_reported(monkeypatch):
    monkeypatch.setenv("BQA_DEBUG", "1")
    bqa, p, path = _sage(True, bad="q")
    st = bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_Q, path._qd, path.qq, workspace=path.ws, check=False)
    assert st == bqa.BQA_E_NONFINITE


def test_inf_in_v_is_reported_by_the_kv_call(monkeypatch):
    monkeypatch.setenv("BQA_DEBUG", "1")
    bqa, p, path = _sage(True, bad="v")
    st = bqa.bqa_quantize_kv(p, path._kd, path._vd, path.kq, path.vq, k_mean=path.mu, workspace=path.ws,
                             check=False)
    assert st == bqa.BQA_E_NONFINITE


def test_nan_in_lse_is_reported_by_the_backward(monkeypatch):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import SageTrainStep, sage_problem, to_device
    w = wl.with_len(wl.WORKLOADS["c3"], 256, hq=1, hkv=1)
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    p = sage_problem(1, 1, 1, 256, 256, 128, True, bqa.BQA_SAGE_I8_I8PV, smooth_eps=1e-3)
    step = SageTrainStep(p, *(to_device(x, "bf16") for x in (Q, K, V, dO)))
    step.quantize()
    step.forward()
    torch.cuda.synchronize()
    monkeypatch.setenv("BQA_DEBUG", "1")
    step.lse[0, 0, 17] = float("nan")
    st = bqa.bqa_attn_bwd(step.p, q=step.qq, k=step.kq, v_hi=step._vd, o_for_delta=step._od, lse=step.lse,
                          d_o=step._dod, dq=step.dq, dk=step.dk, dv=step.dv, workspace=step.ws_bwd, check=False)
    assert st == bqa.BQA_E_NONFINITE
    step.lse[0, 0, 17] = 0.0
    assert bqa.bqa_attn_bwd(step.p, q=step.qq, k=step.kq, v_hi=step._vd, o_for_delta=step._od, lse=step.lse,
                            d_o=step._dod, dq=step.dq, dk=step.dk, dv=step.dv, workspace=step.ws_bwd,
                            check=False) == bqa.BQA_OK


def test_no_scan_without_the_variable(monkeypatch):
    monkeypatch.delenv("BQA_DEBUG", raising=False)
    bqa, p, path = _sage(False, bad="q")
    st = bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_Q, path._qd, path.qq, workspace=path.ws, check=False)
    assert st == bqa.BQA_OK
    torch.cuda.synchronize()
