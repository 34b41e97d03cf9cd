"""Conformance of the kernels' format conversions, bit for bit against the
oracle's encoders (which are pinned exhaustively over fp32 on the CPU):

* the MXFP4 -> bf16 conversion behind O' and the Attn-QAT backward, for every
  code byte under every E8M0 scale whose values are finite in bf16;
* the MXFP4 encoder (OCP rule: X = 2^(floor(log2 amax) - 2), e2m1
  nearest-even, saturating at 6), the per-channel e4m3 encoder and the INT8
  token-block encoder, each on every finite bf16 value below a block's
  anchor (the block's largest magnitude), for anchors that put the grid at
  many scales, that saturate (amax / X in [6, 8)), and whose inverse scale is
  not a power of two.  Exact ties of every grid are among the inputs.

Inputs reach the encoders through the library's own quantisation calls."""
import numpy as np
import pytest
import torch

import oracle as orc
from tests.helpers import assert_same

pytestmark = pytest.mark.gpu

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _finite_bf16():
    """Every finite bf16 value (both zeros included), as fp32."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


def _below(anchor):
    v = _finite_bf16()
    return v[np.abs(v) <= anchor]


def _bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


def _bf16(a):
    """The bf16 value nearest to a (anchors must be values the device sees)."""
    return np.float32(torch.tensor(float(a), dtype=torch.float32).to(torch.bfloat16).item())


def test_mx_dequant_every_code_and_scale():
    import bit_quantized_attention_amd as bqa
    scales = np.arange(0, 253, dtype=np.uint8)                       # 6 x 2^(s - 127) finite in bf16
    nb = 16 * len(scales)
    codes = np.tile(np.arange(256, dtype=np.uint8).reshape(16, 16), (len(scales), 1))    # [nb, 16]
    sc = np.repeat(scales, 16)
    cd, sd = torch.from_numpy(codes).cuda(), torch.from_numpy(sc).cuda()
    out = torch.empty((nb, 32), dtype=torch.bfloat16, device="cuda")
    bqa.bqa_debug_mx_dequant(cd, sd, nb, out)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().astype(np.uint16)
    nib = np.stack([codes & 0xF, codes >> 4], -1).reshape(nb, 32)
    val = E2M1[nib] * 2.0 ** (sc.astype(np.int64) - 127)[:, None]
    want = torch.from_numpy(val).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.all(np.isfinite(val))
    assert_same(got, want, "e2m1 x 2^e -> bf16")


def _anchored_rows(anchors, d, per_block):
    """Rows of d values made of blocks of `per_block`: each block starts with
    its anchor and holds finite bf16 values of magnitude <= the anchor (all of
    them, spread over as many blocks as they need), signs included."""
    blocks = []
    for a in anchors:
        vals = _below(a)
        n = per_block - 1
        for i in range(0, len(vals), n):
            chunk = vals[i:i + n]
            blk = np.zeros(per_block, np.float32)
            blk[0] = a
            blk[1:1 + len(chunk)] = chunk
            blocks.append(blk)
    x = np.concatenate(blocks)
    pad = (-len(x)) % d
    x = np.concatenate([x, np.zeros(pad, np.float32)])
    return x.reshape(-1, d)


def _pad_rows(x, mult):
    pad = (-x.shape[0]) % mult
    return np.concatenate([x, np.zeros((pad, x.shape[1]), np.float32)]) if pad else x


@pytest.mark.parametrize("k", [-120, -3, 0, 7, 100])
def test_mx_encode_every_bf16_value(k):
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import qat_problem
    # anchors 1, 1.25 (no saturation), 1.5, 1.75 (amax / X = 6, 7: the top of the grid saturates) times 2^k
    anchors = [_bf16(m * 2.0 ** k) for m in (1.0, 1.25, 1.5, 1.75)]
    X = _pad_rows(_anchored_rows(anchors, 128, 32), 128)
    N = X.shape[0]
    p = qat_problem(1, 1, 1, N, N, 128)
    codes = torch.empty((N, 64), dtype=torch.uint8, device="cuda")
    scl = torch.empty((N, 4), dtype=torch.uint8, device="cuda")
    xq = bqa.qtensor(bqa.BQA_MXFP4, 0, 32, codes, scl)
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_Q, _bf16_dev(X.reshape(1, 1, N, 128)), xq)
    torch.cuda.synchronize()
    rc, rs = orc.quant_mx_rows(X[None])
    assert_same(scl.cpu().numpy(), rs[0], f"E8M0 scales (2^{k} anchors)")
    assert_same(codes.cpu().numpy(), rc[0], f"e2m1 codes (2^{k} anchors)")


@pytest.mark.parametrize("anchors", [
    (448.0, 1.0, 448.0 * 2 ** -30, 448.0 * 2 ** 20),                    # inverse scale a power of two
    (3.140625, 1e-3, 7.5e-37, 2.5e30),                                   # inverse scale inexact in fp32
])
def test_e4m3_channel_encode_every_bf16_value(anchors):
    """Per-channel V (the fp8 P.V mode): channel c's first token is its
    anchor, the other tokens all finite bf16 values below it (a sample at
    most every 2nd value when they do not fit)."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import sage_problem
    d, N = 64, 32768
    V = np.zeros((N, d), np.float32)
    for c in range(d):
        a = _bf16(anchors[c % len(anchors)])
        vals = _below(a)
        vals = vals[(c // len(anchors)) % 2::2] if len(vals) > N - 1 else vals
        vals = vals[:N - 1]
        V[0, c] = a
        V[1:1 + len(vals), c] = vals
    p = sage_problem(1, 1, 1, N, N, d, False, bqa.BQA_SAGE_I8_F8PV)
    codes = torch.empty((d, N), dtype=torch.uint8, device="cuda")
    scl = torch.empty((d,), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(bqa.bqa_workspace_size(p, bqa.BQA_OP_QUANTIZE_V), 16), dtype=torch.uint8, device="cuda")
    vq = bqa.qtensor(bqa.BQA_FP8E4M3, 1, N, codes, scl)
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_V, _bf16_dev(V.reshape(1, 1, N, d)), vq, workspace=ws)
    torch.cuda.synchronize()
    rc, rs = orc.quant_chan(V[None], "e4m3")
    assert_same(scl.cpu().numpy(), rs[0], "e4m3 channel scales")
    assert_same(codes.cpu().numpy(), rc[0], "e4m3 codes")


@pytest.mark.parametrize("anchors", [(1.0, 127.0, 127.0 * 2 ** -40, 2 ** 90), (3.3, 0.1, 1e-30, 7e25)])
def test_int8_tokblock_encode_every_bf16_value(anchors):
    """INT8 token blocks of 64 tokens x 64 channels: each block's first value
    is its anchor, the rest finite bf16 values below it."""
    import bit_quantized_attention_amd as bqa
    from bit_quantized_attention_amd.runner import sage_problem
    d = 64
    X = _pad_rows(_anchored_rows([_bf16(a) for a in anchors], d, 64 * d), 64)
    N = X.shape[0]
    p = sage_problem(1, 1, 1, N, N, d, False, bqa.BQA_SAGE_I8_F8PV, q_block=64)
    codes = torch.empty((N, d), dtype=torch.int8, device="cuda")
    scl = torch.empty((N // 64,), dtype=torch.float32, device="cuda")
    xq = bqa.qtensor(bqa.BQA_INT8, 0, 64, codes, scl)
    bqa.bqa_quantize_blocks(p, bqa.BQA_ROLE_Q, _bf16_dev(X.reshape(1, 1, N, d)), xq)
    torch.cuda.synchronize()
    rc, rs = orc.quant_i8_tokblock(X[None], 64)
    assert_same(scl.cpu().numpy(), rs[0], "INT8 block scales")
    assert_same(codes.cpu().numpy(), rc[0], "INT8 codes")
