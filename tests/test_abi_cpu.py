"""The C-ABI library loads, exports every symbol bqa.h declares, and rejects
bad arguments on the host before touching a device (CPU only; with valid
arguments and no GPU the calls return BQA_E_DEVICE)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import bit_quantized_attention_amd as bqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bqa.LIB_PATH):
        pytest.fail("libbqa.so is not built (run __graft_entry__.build())")
    return bqa.lib()


def _declared():
    txt = open(os.path.join(ROOT, "include", "bqa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(bqa_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(bqa.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", bqa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (bqa_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_version_and_strings(L):
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "bqa.h")).read()
    assert bqa.bqa_abi_version() == int(re.search(r"#define BQA_ABI_VERSION (\d+)", hdr).group(1))
    for s in range(-7, 1):
        assert isinstance(bqa.bqa_status_string(s), str) and bqa.bqa_status_string(s)
    assert bqa.bqa_status_string(-99) == "unknown status"


class FakeTensor:
    """A host object posing as a device tensor (only pointer and strides are read)."""

    def __init__(self, ptr, shape, strides, dtype):
        self._p, self.shape, self._s, self.dtype = ptr, shape, strides, dtype

    def data_ptr(self):
        return self._p

    def dim(self):
        return 4

    def stride(self, i):
        return self._s[i]


def _dense(ptr=0x10000, strides=(4096 * 128 * 16, 4096 * 128, 128, 1), dtype=bqa.BQA_BF16):
    t = bqa.bqa_tensor()
    t.data, t.dtype = ptr, dtype
    for i, s in enumerate(strides):
        t.stride[i] = s
    return t


def _p(**kw):
    base = dict(B=2, Hq=16, Hkv=16, Nq=4096, Nk=4096, d=128, causal=1, mode=bqa.BQA_SAGE_I8_F8PV, q_block=128,
                k_block=64, smooth_k=1, smooth_eps=0.0)
    base.update(kw)
    return bqa.problem(**base)


def _q(fmt=bqa.BQA_INT8, axis=0, block=128, codes=0x20000, scales=0x30000):
    return bqa.qtensor(fmt, axis, block, codes, scales)


def _quant(p, role, x, out, ws=0x40000, wsb=1 << 30):
    return bqa.lib().bqa_quantize_blocks(C.byref(p), role, None if x is None else C.byref(x), C.byref(out), None,
                                         None, ws, wsb, None)


def test_quantize_validation(L):
    x = _dense()
    assert _quant(None if False else _p(d=96), bqa.BQA_ROLE_Q, x, _q()) == bqa.BQA_E_UNSUPPORTED
    assert _quant(_p(Hq=16, Hkv=3), bqa.BQA_ROLE_Q, x, _q()) == bqa.BQA_E_SHAPE
    assert _quant(_p(B=0), bqa.BQA_ROLE_Q, x, _q()) == bqa.BQA_E_SHAPE
    assert _quant(_p(), bqa.BQA_ROLE_Q, None, _q()) == bqa.BQA_E_NULL
    assert _quant(_p(), bqa.BQA_ROLE_Q, _dense(ptr=0x10008), _q()) == bqa.BQA_E_ALIGN
    assert _quant(_p(), bqa.BQA_ROLE_Q, _dense(strides=(1 << 20, 1 << 16, 130, 1)), _q()) == bqa.BQA_E_ALIGN
    assert _quant(_p(), bqa.BQA_ROLE_Q, _dense(strides=(1 << 20, 1 << 16, 128, 2)), _q()) == bqa.BQA_E_ALIGN
    assert _quant(_p(), bqa.BQA_ROLE_Q, x, _q(codes=0x20004)) == bqa.BQA_E_ALIGN
    assert _quant(_p(), bqa.BQA_ROLE_Q, x, _q(codes=0)) == bqa.BQA_E_NULL
    assert _quant(_p(), bqa.BQA_ROLE_Q, x, _q(block=96)) == bqa.BQA_E_UNSUPPORTED
    assert _quant(_p(Nq=4032), bqa.BQA_ROLE_Q, x, _q(block=128)) == bqa.BQA_E_UNSUPPORTED
    assert _quant(_p(), 7, x, _q()) == bqa.BQA_E_UNSUPPORTED
    # smoothing needs a workspace
    assert _quant(_p(), bqa.BQA_ROLE_K, x, _q(block=64), ws=0, wsb=0) == bqa.BQA_E_WORKSPACE
    need = bqa.bqa_workspace_size(_p(), bqa.BQA_OP_QUANTIZE_K)
    assert need > 0
    assert _quant(_p(), bqa.BQA_ROLE_K, x, _q(block=64), wsb=need - 1) == bqa.BQA_E_WORKSPACE
    assert bqa.bqa_workspace_size(_p(d=96), bqa.BQA_OP_QUANTIZE_K) == 0
    # per-channel V: block must be N
    assert _quant(_p(), bqa.BQA_ROLE_V, x, _q(fmt=bqa.BQA_FP8E4M3, axis=1, block=64)) == bqa.BQA_E_UNSUPPORTED
    # valid arguments: no GPU here, so the device check answers
    import torch
    if not torch.cuda.is_available():
        assert _quant(_p(), bqa.BQA_ROLE_Q, x, _q()) == bqa.BQA_E_DEVICE
        assert _quant(_p(), bqa.BQA_ROLE_V, x, _q(fmt=bqa.BQA_FP8E4M3, axis=1, block=4096)) == bqa.BQA_E_DEVICE


def test_quantize_kv_validation(L):
    k, v = _dense(), _dense(ptr=0x50000)
    kq, vq = _q(block=64), _q(fmt=bqa.BQA_FP8E4M3, axis=1, block=4096)

    def qkv(p, k=k, v=v, kq=kq, vq=vq, ws=0x40000, wsb=1 << 30):
        return bqa.lib().bqa_quantize_kv(C.byref(p), None if k is None else C.byref(k),
                                         None if v is None else C.byref(v), None if kq is None else C.byref(kq),
                                         None if vq is None else C.byref(vq), None, ws, wsb, None)
    assert qkv(_p(mode=bqa.BQA_SAGE_I8_F16PV)) == bqa.BQA_E_UNSUPPORTED
    assert qkv(_p(mode=bqa.BQA_QAT_MXFP4)) == bqa.BQA_E_UNSUPPORTED
    assert qkv(_p(), kq=None) == bqa.BQA_E_NULL
    assert qkv(_p(), v=None) == bqa.BQA_E_NULL
    assert qkv(_p(), v=_dense(ptr=0x50000, dtype=bqa.BQA_FP16)) == bqa.BQA_E_UNSUPPORTED   # K and V differ
    assert qkv(_p(), kq=_q(block=128)) == bqa.BQA_E_UNSUPPORTED
    assert qkv(_p(), vq=_q(fmt=bqa.BQA_INT8, axis=1, block=4096)) == bqa.BQA_E_UNSUPPORTED  # F8PV needs e4m3
    assert qkv(_p(mode=bqa.BQA_SAGE_I8_I8PV)) == bqa.BQA_E_UNSUPPORTED                      # I8PV needs int8
    assert qkv(_p(), vq=_q(fmt=bqa.BQA_FP8E4M3, axis=1, block=64)) == bqa.BQA_E_UNSUPPORTED
    need = bqa.bqa_workspace_size(_p(), bqa.BQA_OP_QUANTIZE_KV)
    assert need >= bqa.bqa_workspace_size(_p(), bqa.BQA_OP_QUANTIZE_K) + bqa.bqa_workspace_size(_p(), bqa.BQA_OP_QUANTIZE_V)
    assert qkv(_p(), wsb=need - 1) == bqa.BQA_E_WORKSPACE
    assert qkv(_p(), ws=0, wsb=0) == bqa.BQA_E_WORKSPACE
    assert qkv(_p(), ws=0x40008) == bqa.BQA_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert qkv(_p()) == bqa.BQA_E_DEVICE
        assert qkv(_p(mode=bqa.BQA_SAGE_I8_I8PV), vq=_q(fmt=bqa.BQA_INT8, axis=1, block=4096)) == bqa.BQA_E_DEVICE


def test_fwd_validation(L):
    o = _dense()
    q, k = _q(), _q(block=64)
    v = _q(fmt=bqa.BQA_FP8E4M3, axis=1, block=4096)

    def fwd(p, q=q, k=k, v=v, o=o, v_hi=None):
        return bqa.lib().bqa_attn_fwd(C.byref(p), C.byref(q), C.byref(k), None if v is None else C.byref(v), None,
                                      None, None if v_hi is None else C.byref(v_hi), None, None,
                                      None if o is None else C.byref(o), None, None, None, None, 0, None)
    assert fwd(_p(k_block=32)) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(q_block=32)) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(causal=1, Nq=8192)) == bqa.BQA_E_SHAPE
    assert fwd(_p(), q=_q(block=64)) == bqa.BQA_E_UNSUPPORTED          # block differs from q_block
    assert fwd(_p(), v=_q(fmt=bqa.BQA_INT8, axis=1, block=4096)) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(), o=None) == bqa.BQA_E_NULL
    assert fwd(_p(), o=_dense(dtype=bqa.BQA_FP16)) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(mode=bqa.BQA_SAGE_I8_F16PV), v=None) == bqa.BQA_E_NULL
    assert fwd(_p(mode=9)) == bqa.BQA_E_UNSUPPORTED
    # Attn-QAT: key tiles of 128, so Nk a multiple of 128
    assert fwd(_p(mode=bqa.BQA_QAT_MXFP4, causal=0, Nq=320, Nk=320)) == bqa.BQA_E_UNSUPPORTED

    def fwd_qhi(p, q=q, q_hi=_dense(ptr=0x60000)):
        return bqa.lib().bqa_attn_fwd(C.byref(p), None if q is None else C.byref(q), C.byref(k), C.byref(v),
                                      None if q_hi is None else C.byref(q_hi), None, None, None, None, C.byref(o),
                                      None, None, None, None, 0, None)
    # Q quantised inside the kernel: fp8 P.V and bf16 only; q optional, but checked when given
    assert fwd_qhi(_p(mode=bqa.BQA_SAGE_I8_I8PV)) == bqa.BQA_E_UNSUPPORTED
    assert fwd_qhi(_p(), q_hi=_dense(ptr=0x60000, dtype=bqa.BQA_FP16)) == bqa.BQA_E_UNSUPPORTED
    assert fwd_qhi(_p(), q_hi=_dense(ptr=0x60008)) == bqa.BQA_E_ALIGN
    assert fwd_qhi(_p(), q=_q(block=64)) == bqa.BQA_E_UNSUPPORTED
    assert fwd_qhi(_p(), q=_q(codes=0)) == bqa.BQA_E_NULL
    import torch
    if not torch.cuda.is_available():
        assert fwd_qhi(_p()) == bqa.BQA_E_DEVICE
        assert fwd_qhi(_p(), q=None) == bqa.BQA_E_DEVICE
        assert fwd(_p()) == bqa.BQA_E_DEVICE
        assert fwd(_p(mode=bqa.BQA_SAGE_I8_F16PV), v=None, v_hi=_dense(dtype=bqa.BQA_FP16),
                   o=_dense(dtype=bqa.BQA_FP16)) == bqa.BQA_E_DEVICE


def test_empty_and_inconsistent_shapes(L):
    """Empty inputs (a zero batch, head count or length) and head counts that
    do not group are refused before any device work, by every attention
    entry point."""
    g = _dense()
    q, k = _q(), _q(block=64)
    v = _q(fmt=bqa.BQA_FP8E4M3, axis=1, block=4096)

    def fwd(p):
        return bqa.lib().bqa_attn_fwd(C.byref(p), C.byref(q), C.byref(k), C.byref(v), None, None, None, None, None,
                                      C.byref(g), None, None, None, None, 0, None)

    def bwd(p):
        return bqa.lib().bqa_attn_bwd(C.byref(p), C.byref(q), C.byref(k), None, C.byref(g), C.byref(g), 0x50000, None,
                                      C.byref(g), C.byref(g), C.byref(g), C.byref(g), 0x40000, 1 << 34, None)
    for bad in (dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Nq=0), dict(Nk=0), dict(Nq=-128), dict(Hq=6, Hkv=4)):
        assert fwd(_p(**bad)) == bqa.BQA_E_SHAPE, bad
        assert bwd(_p(mode=bqa.BQA_SAGE_I8_I8PV, **dict(dict(Nq=4096, Nk=4096), **bad))) == bqa.BQA_E_SHAPE, bad


def test_debug_scores_validation(L):
    q, k = _q(), _q(block=64)
    f = bqa.lib().bqa_debug_qk_scores
    assert f(C.byref(_p()), C.byref(q), C.byref(k), 0, 0, 0, 0, None, None) == bqa.BQA_E_NULL
    assert f(C.byref(_p()), C.byref(q), C.byref(k), 2, 0, 0, 0, 0x1000, None) == bqa.BQA_E_SHAPE
    assert f(C.byref(_p()), C.byref(q), C.byref(k), 0, 0, 128, 0, 0x1000, None) == bqa.BQA_E_SHAPE
    assert f(C.byref(_p()), C.byref(q), C.byref(k), 0, 0, 0, -1, 0x1000, None) == bqa.BQA_E_SHAPE


def _nodev(st):
    """A call with valid arguments stops at the device check without a GPU."""
    import torch
    return torch.cuda.is_available() or st == bqa.BQA_E_DEVICE


def test_bwd_validation(L):
    g = _dense()
    q, k = _q(), _q(block=64)

    def bwd(p, q=q, k=k, v=None, v_hi=g, o=g, lse=0x50000, row_max=None, d_o=g, dq=g, ws=0x40000, wsb=1 << 34):
        return bqa.lib().bqa_attn_bwd(C.byref(p), None if q is None else C.byref(q), C.byref(k),
                                      None if v is None else C.byref(v), None if v_hi is None else C.byref(v_hi),
                                      C.byref(o), lse, row_max, C.byref(d_o), None if dq is None else C.byref(dq),
                                      C.byref(g), C.byref(g), ws, wsb, None)
    sage = dict(mode=bqa.BQA_SAGE_I8_I8PV, Nq=4096, Nk=4096)
    assert bwd(_p(d=64, **sage)) == bqa.BQA_E_UNSUPPORTED
    assert bwd(_p(Hkv=8, **sage)) == bqa.BQA_E_SHAPE or bwd(_p(Hkv=8, **sage)) == bqa.BQA_E_UNSUPPORTED
    assert bwd(_p(mode=bqa.BQA_SAGE_I8_I8PV, Nq=2048, Nk=4096)) == bqa.BQA_E_UNSUPPORTED
    assert bwd(_p(**sage), lse=None) == bqa.BQA_E_NULL
    assert bwd(_p(**sage), dq=None) == bqa.BQA_E_NULL
    assert bwd(_p(**sage), q=None) == bqa.BQA_E_NULL
    assert bwd(_p(**sage), wsb=16) == bqa.BQA_E_WORKSPACE
    assert bwd(_p(**sage), lse=0x50004) == bqa.BQA_E_ALIGN
    assert _nodev(bwd(_p(**sage)))
    mx = dict(mode=bqa.BQA_QAT_MXFP4, causal=0, Nq=4096, Nk=4096)
    qm, km, vm = _q(fmt=bqa.BQA_MXFP4, block=32), _q(fmt=bqa.BQA_MXFP4, block=32), _q(fmt=bqa.BQA_MXFP4, axis=1, block=32)
    assert bwd(_p(**mx), q=qm, k=km, v=vm, row_max=None) == bqa.BQA_E_NULL          # Attn-QAT needs row_max
    assert bwd(_p(**dict(mx, causal=1)), q=qm, k=km, v=vm, row_max=0x60000) == bqa.BQA_E_UNSUPPORTED
    assert bwd(_p(**mx), q=qm, k=km, v=vm, row_max=0x60008) == bqa.BQA_E_ALIGN
    assert _nodev(bwd(_p(**mx), q=qm, k=km, v=vm, row_max=0x60000))


def test_select_validation(L):
    def sel(p, qm=0x10000, km=0x20000, idx=0x30000, cnt=0x40000):
        return bqa.lib().bqa_select_blocks(C.byref(p), qm, km, idx, cnt, None, 0, None)
    th = dict(mode=bqa.BQA_THRIFT, Hq=32, Hkv=8, Nq=131072, Nk=131072, hp_budget_ppm=50_000, sel_block=128)
    assert sel(_p(**dict(th, mode=bqa.BQA_QAT_MXFP4))) == bqa.BQA_E_UNSUPPORTED
    assert sel(_p(**dict(th, sel_block=64))) == bqa.BQA_E_UNSUPPORTED
    assert sel(_p(**th), km=None) == bqa.BQA_E_NULL
    assert sel(_p(**th), cnt=None) == bqa.BQA_E_NULL
    assert sel(_p(**dict(th, hp_budget_ppm=1_000_001))) == bqa.BQA_E_SHAPE
    assert sel(_p(**dict(th, Nk=131072 - 64, Nq=131072 - 64))) == bqa.BQA_E_UNSUPPORTED
    assert sel(_p(**dict(th, Nq=200, Nk=1024))) == bqa.BQA_E_UNSUPPORTED         # ragged causal query blocks
    assert sel(_p(**th), km=0x20004) == bqa.BQA_E_ALIGN
    assert _nodev(sel(_p(**th)))
    assert _nodev(sel(_p(**dict(th, Nq=1, Nk=1024))))                             # decode: one query, any length
    assert _nodev(sel(_p(**dict(th, causal=0, Nq=200, Nk=1024))))


def test_decode_static_validation(L):
    d = _dense()
    qm, km, vm = _q(fmt=bqa.BQA_MXFP4, block=32), _q(fmt=bqa.BQA_MXFP4, block=32), _q(fmt=bqa.BQA_MXFP4, axis=1, block=32)

    def dec(p, idx=0x30000):
        return bqa.lib().bqa_attn_decode_static(C.byref(p), C.byref(qm), C.byref(km), C.byref(vm), C.byref(d),
                                                C.byref(d), C.byref(d), idx, 0x40000, C.byref(d), None, None)
    th = dict(mode=bqa.BQA_THRIFT, B=16, Hq=32, Hkv=8, Nq=1, Nk=131072, hp_budget_ppm=50_000, sel_block=128)
    assert dec(_p(**dict(th, Nq=128, Nk=1024))) == bqa.BQA_E_UNSUPPORTED
    assert dec(_p(**th), idx=None) == bqa.BQA_E_NULL
    # 64 batches x 32 heads x 128 splits x 132 floats = 138 MB of partials > the 16 MiB static array
    assert dec(_p(**dict(th, B=64, num_splits=128))) == bqa.BQA_E_TOO_LARGE
    assert _nodev(dec(_p(**th)))                                                  # c5d: 4.3 MB of partials


def test_ptq_validation(L):
    x = _dense()
    pt = dict(mode=bqa.BQA_PTQ_MXFP4, B=1, Hq=4, Hkv=2, Nq=300, Nk=512, causal=0, smooth_k=1)
    mq, mk, mv = _q(fmt=bqa.BQA_MXFP4, block=32), _q(fmt=bqa.BQA_MXFP4, block=32), \
        _q(fmt=bqa.BQA_MXFP4, axis=1, block=32)

    def quant(p, role, out, means=None, kmean=None, ws=0x40000, wsb=1 << 30):
        return bqa.lib().bqa_quantize_blocks(C.byref(p), role, C.byref(x), C.byref(out), kmean, means, ws, wsb, None)

    # Q smoothing writes its block means: required, 16-byte aligned
    assert quant(_p(**pt), bqa.BQA_ROLE_Q, mq) == bqa.BQA_E_NULL
    assert quant(_p(**pt), bqa.BQA_ROLE_Q, mq, means=0x50004) == bqa.BQA_E_ALIGN
    assert quant(_p(**dict(pt, d=64)), bqa.BQA_ROLE_Q, mq, means=0x50000) == bqa.BQA_E_UNSUPPORTED
    # K smoothing: token sums in the workspace; no block means for K
    need = bqa.bqa_workspace_size(_p(**pt), bqa.BQA_OP_QUANTIZE_K)
    assert need > 0 and bqa.bqa_workspace_size(_p(**dict(pt, smooth_k=0)), bqa.BQA_OP_QUANTIZE_K) == 0
    assert quant(_p(**pt), bqa.BQA_ROLE_K, mk, wsb=need - 1) == bqa.BQA_E_WORKSPACE
    assert quant(_p(**pt), bqa.BQA_ROLE_K, mk, means=0x50000) == bqa.BQA_E_UNSUPPORTED

    def fwd(p, qm=0x60000, ws=0x70000, wsb=None):
        wsb = bqa.bqa_workspace_size(p, bqa.BQA_OP_FWD) if wsb is None else wsb
        return bqa.lib().bqa_attn_fwd_ptq(C.byref(p), C.byref(mq), C.byref(mk), C.byref(mv), qm, C.byref(x), None,
                                          ws, wsb, None)
    # score shifts: B Hq ceil(Nq / 128) Nk fp32
    assert bqa.bqa_workspace_size(_p(**pt), bqa.BQA_OP_FWD) == 1 * 4 * 3 * 512 * 4
    assert fwd(_p(**dict(pt, mode=bqa.BQA_THRIFT))) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(**dict(pt, Nk=500))) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(**pt), qm=None) == bqa.BQA_E_NULL
    assert fwd(_p(**pt), qm=0x60008) == bqa.BQA_E_ALIGN
    assert fwd(_p(**pt), wsb=1000) == bqa.BQA_E_WORKSPACE
    # the plain forward does not take this mode
    assert bqa.lib().bqa_attn_fwd(C.byref(_p(**pt)), C.byref(mq), C.byref(mk), C.byref(mv), None, None, None, None,
                                  None, C.byref(x), None, None, None, 0x70000, 1 << 30, None) == bqa.BQA_E_UNSUPPORTED
    assert _nodev(fwd(_p(**pt)))
    assert _nodev(quant(_p(**pt), bqa.BQA_ROLE_Q, mq, means=0x50000))
    assert _nodev(quant(_p(**pt), bqa.BQA_ROLE_K, mk))


def test_probe_validation(L):
    P = bqa.lib().bqa_debug_probe
    assert P(23, 16, 10, None, 0x1000, 4096, None) == bqa.BQA_E_UNSUPPORTED
    assert P(-1, 16, 10, None, 0x1000, 4096, None) == bqa.BQA_E_UNSUPPORTED
    assert P(bqa.BQA_PROBE_MFMA_I8, 0, 10, None, 0x1000, 4096, None) == bqa.BQA_E_SHAPE
    assert P(bqa.BQA_PROBE_MFMA_I8, 16, -1, None, 0x1000, 4096, None) == bqa.BQA_E_SHAPE
    assert P(bqa.BQA_PROBE_MFMA_I8, 16, 10, None, None, 4096, None) == bqa.BQA_E_NULL
    assert P(bqa.BQA_PROBE_MFMA_I8, 16, 10, None, 0x1002, 4096, None) == bqa.BQA_E_ALIGN
    assert P(bqa.BQA_PROBE_EXP, 2048, 10, None, 0x1000, 4096, None) == bqa.BQA_E_SHAPE      # 4 bytes per workgroup
    assert P(bqa.BQA_PROBE_COPY, 16, 0, None, 0x1000, 4096, None) == bqa.BQA_E_NULL
    assert P(bqa.BQA_PROBE_COPY, 16, 0, 0x2008, 0x1000, 4096, None) == bqa.BQA_E_ALIGN
    assert P(bqa.BQA_PROBE_COPY, 16, 0, 0x2000, 0x1000, 4100, None) == bqa.BQA_E_ALIGN
    assert P(bqa.BQA_PROBE_READ, 16, 0, None, 0x1000, 4096, None) == bqa.BQA_E_NULL
    assert P(bqa.BQA_PROBE_READ, 16, 0, 0x2000, 0x1002, 4096, None) == bqa.BQA_E_ALIGN
    assert _nodev(P(bqa.BQA_PROBE_READ, 16, 0, 0x2000, 0x1000, 4096, None))
    assert P(bqa.BQA_PROBE_READ_NT, 16, 0, None, 0x1000, 4096, None) == bqa.BQA_E_NULL
    assert _nodev(P(bqa.BQA_PROBE_READ_NT, 16, 0, 0x2000, 0x1000, 4096, None))
    assert P(bqa.BQA_PROBE_ISSUE_MFMA_EXP, 2048, 10, None, 0x1000, 4096, None) == bqa.BQA_E_SHAPE
    for kind in range(bqa.BQA_PROBE_ISSUE_MFMA, bqa.BQA_PROBE_LDS_SPANS + 1):
        assert _nodev(P(kind, 16, 10, None, 0x1000, 4096, None))
    assert _nodev(P(bqa.BQA_PROBE_MFMA_F4, 16, 10, None, 0x1000, 4096, None))
    assert _nodev(P(bqa.BQA_PROBE_COPY, 16, 0, 0x2000, 0x1000, 4096, None))


def test_qknorm_validation(L):
    x = _dense()
    sage = dict(mode=bqa.BQA_SAGE_I8_I8PV, Nq=4096, Nk=4096, smooth_k=1, smooth_eps=1e-3)

    def quant(p, role, out, rn=0x70000, ws=0x40000, wsb=1 << 30):
        return bqa.lib().bqa_quantize_qknorm(C.byref(p), role, C.byref(x), C.byref(out), rn, None, ws, wsb, None)
    assert quant(_p(**sage), bqa.BQA_ROLE_V, _q()) == bqa.BQA_E_UNSUPPORTED
    assert quant(_p(**dict(sage, mode=bqa.BQA_QAT_MXFP4)), bqa.BQA_ROLE_Q, _q()) == bqa.BQA_E_UNSUPPORTED
    assert quant(_p(**dict(sage, d=64)), bqa.BQA_ROLE_Q, _q()) == bqa.BQA_E_UNSUPPORTED
    assert quant(_p(**sage), bqa.BQA_ROLE_Q, _q(), rn=None) == bqa.BQA_E_NULL
    assert quant(_p(**sage), bqa.BQA_ROLE_Q, _q(), rn=0x70002) == bqa.BQA_E_ALIGN
    assert quant(_p(**sage), bqa.BQA_ROLE_Q, _q(block=96)) == bqa.BQA_E_UNSUPPORTED
    assert quant(_p(**sage), bqa.BQA_ROLE_K, _q(block=64), wsb=8) == bqa.BQA_E_WORKSPACE
    assert _nodev(quant(_p(**sage), bqa.BQA_ROLE_Q, _q()))
    assert _nodev(quant(_p(**sage), bqa.BQA_ROLE_K, _q(block=64)))
    g = _dense()
    q, k = _q(), _q(block=64)

    def bwd(p, qraw=g, rq=0x71000, rk=0x72000):
        return bqa.lib().bqa_attn_bwd_qknorm(C.byref(p), C.byref(q), C.byref(k), C.byref(g), C.byref(g), 0x50000,
                                             C.byref(g), None if qraw is None else C.byref(qraw), C.byref(g), rq, rk,
                                             C.byref(g), C.byref(g), C.byref(g), 0x40000, 1 << 34, None)
    assert bwd(_p(**dict(sage, mode=bqa.BQA_QAT_MXFP4))) == bqa.BQA_E_UNSUPPORTED
    assert bwd(_p(**sage), qraw=None) == bqa.BQA_E_NULL
    assert bwd(_p(**sage), rk=None) == bqa.BQA_E_NULL
    assert bwd(_p(**sage), rq=0x71001) == bqa.BQA_E_ALIGN
    assert _nodev(bwd(_p(**sage)))


def test_nvfp4_validation(L):
    x = _dense()
    th = dict(mode=bqa.BQA_THRIFT, B=1, Hq=4, Hkv=2, Nq=1024, Nk=1024, hp_budget_ppm=50_000, sel_block=128)

    def quant(p, role, out=x, ws=0x40000, wsb=1 << 30):
        return bqa.lib().bqa_quantize_nvfp4(C.byref(p), role, C.byref(x), None if out is None else C.byref(out),
                                            ws, wsb, None)
    assert quant(_p(**dict(th, d=64)), bqa.BQA_ROLE_Q) == bqa.BQA_E_UNSUPPORTED
    assert quant(_p(**th), bqa.BQA_ROLE_DO) == bqa.BQA_E_UNSUPPORTED
    assert quant(_p(**th), bqa.BQA_ROLE_Q, out=None) == bqa.BQA_E_NULL
    assert quant(_p(**dict(th, Nk=1008, causal=0)), bqa.BQA_ROLE_V) == bqa.BQA_E_UNSUPPORTED
    need = bqa.bqa_workspace_size(_p(**th), bqa.BQA_OP_QUANTIZE_NVFP4)
    assert need > 0 and quant(_p(**th), bqa.BQA_ROLE_Q, wsb=need - 1) == bqa.BQA_E_WORKSPACE
    assert _nodev(quant(_p(**th), bqa.BQA_ROLE_V, wsb=need))

    def fwd(p, idx=0x30000):
        return bqa.lib().bqa_attn_fwd_thrift_nvfp4(C.byref(p), *[C.byref(x)] * 6, idx, 0x31000, C.byref(x), None,
                                                   None)
    assert fwd(_p(**dict(th, Nq=1, Nk=1024))) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(**dict(th, mode=bqa.BQA_QAT_MXFP4))) == bqa.BQA_E_UNSUPPORTED
    assert fwd(_p(**th), idx=None) == bqa.BQA_E_NULL
    assert _nodev(fwd(_p(**th)))
