"""GPU parity of the NVFP4 emulation ("ThriftAttention", Method step 2: the
FP4 path in NVFP4 micro-scaling) against the oracle, through the C ABI: the
NVFP4 fake-quantisation of Q, K (blocks of 16 channels) and V (blocks of 16
tokens) bit for bit, then the Thrift prefill with its FP4 path in NVFP4 (the
oracle's own quantisation, block means and selection) at budgets 5, 25 and
100 %."""
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


def _run(w, ppm, Q=None, K=None, V=None):
    from bit_quantized_attention_amd.runner import ThriftNvPath, thrift_problem, to_device
    if Q is None:
        Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = thrift_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, budget_ppm=ppm)
    path = ThriftNvPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    path.step()
    torch.cuda.synchronize()
    return p, path, (Q, K, V)


def test_nvfp4_fake_quantisation_bit_exact():
    w = wl.with_len(wl.WORKLOADS["c5"], 512, hq=4, hkv=2)
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    # a head with a wide dynamic range: one large channel, tiny values elsewhere
    Q[0, 1] *= np.float32(2.0 ** -20)
    Q[0, 1, :, 5] = 3072.0
    K[0, 1, ::7] *= np.float32(64.0)
    Q, K = (wl.round_to(x, "bf16").reshape(x.shape) for x in (Q, K))
    p, path, _ = _run(w, 50_000, Q, K, V)
    for name, x, got, axis in (("Q", Q, path.qn, 0), ("K", K, path.kn, 0), ("V", V, path.vn, 1)):
        ref = orc.nvfp4_fake(x.reshape(-1, x.shape[2], x.shape[3]), axis).reshape(x.shape)
        g = got.float().cpu().numpy()
        assert_same(g.view(np.uint32), ref.view(np.uint32), f"NVFP4 {name}")


@pytest.mark.parametrize("ppm", [50_000, 250_000, 1_000_000])
def test_thrift_nvfp4_prefill_small(ppm):
    w = wl.with_len(wl.WORKLOADS["c5"], 1024, hq=4, hkv=2)
    p, path, (Q, K, V) = _run(w, ppm)
    Qf, Kf, Vf = (x.reshape(-1, x.shape[2], x.shape[3]) for x in (Q, K, V))
    Qn, Kn, Vn = orc.nvfp4_fake(Qf, 0), orc.nvfp4_fake(Kf, 0), orc.nvfp4_fake(Vf, 1)
    nkb = w.Nk // 128
    ms = max(1, min(nkb, -(-nkb * ppm // 1_000_000)))
    qm, km = orc.block_means(Qf, 128), orc.block_means(Kf, 128)
    O = path.o.float().cpu().numpy()
    L = path.lse.cpu().numpy()
    for iq in range(4):
        ik = iq // 2
        idx, cnt = orc.select_blocks(qm[iq], km[ik], True, ppm, ms)
        assert_same(path.sel_idx.cpu().numpy()[0, iq], idx, f"selection of head {iq}")
        ref, lse = orc.thrift_fwd_nv(Qn=Qn[iq], Kn=Kn[ik], Vn=Vn[ik], Qh=Qf[iq], Kh=Kf[ik], Vh=Vf[ik], sel_idx=idx,
                                     sel_cnt=cnt, Nq=w.Nq, Nk=w.Nk, d=w.d, causal=True, tau=tau_for(w.d))
        compare_outputs(O[0, iq], ref, "bf16", what=f"O[h={iq}]")
        assert np.abs(L[0, iq] - lse).max() < 2e-3
