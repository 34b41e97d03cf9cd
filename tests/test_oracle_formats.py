"""Pins of the oracle's scalar encoders and quantisers (CPU only).

Each test checks the oracle against something other than itself: the
format definitions through an exhaustive brute-force search, library
conversions (NumPy fp16, torch bf16 / float8_e4m3fn), closed-form error
bounds and numbers the pages state.
"""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))


def test_e2m1_has_fifteen_values(orc):
    # Attn-QAT, technical summary §1: FP4 represents only 15 numbers (+0 and -0 coincide)
    vals = {orc.e2m1_decode(c) for c in range(16)}
    assert len(vals) == FACTS["fp4_distinct_values"]["value"]
    assert sorted(v for v in vals if v >= 0) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.fixture(scope="module")
def bruteforce(orc, tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("bf") / "enc_bruteforce")
    libdir = os.path.dirname(orc.lib()._name)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "pins", "enc_bruteforce.c"), "-L", libdir, "-loracle",
                    f"-Wl,-rpath,{libdir}", "-lm"], check=True)
    return exe


@pytest.mark.slow
@pytest.mark.parametrize("which", ["e2m1", "e4m3", "e8m0", "i8"])
def test_encoders_exhaustive(bruteforce, which):
    """Every finite fp32 input against a nearest-value search over the format's table."""
    out = subprocess.run([bruteforce, which, "1"], check=True, capture_output=True, text=True).stdout.split()
    assert out[0] == which
    checked, bad = int(out[1]), int(out[2])
    assert checked > 2_000_000_000 and bad == 0


def test_bf16_f16_match_library(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 4000),
                        np.float32([0.0, -0.0, 1e-40, -3e-42, 65504.0, 65519.0, 65520.0])]).astype(np.float32)
    t_bf = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    t_f16 = x.astype(np.float16).astype(np.float64)
    for i, v in enumerate(x):
        assert orc.bf16_value(float(v)) == t_bf[i] or (np.isinf(t_bf[i]) and np.isinf(orc.bf16_value(float(v))))
        o = orc.f16_value(float(v))
        assert o == t_f16[i] or (np.isinf(o) and np.isinf(t_f16[i]))


def test_e4m3_matches_torch_float8(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.standard_normal(3000) * 1e-2,
                        rng.standard_normal(1000) * 3e-3]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i, v in enumerate(x):
        assert orc.e4m3_encode(float(v)) == t[i], (v, orc.e4m3_encode(float(v)), t[i])
    for c in range(256):
        ref = torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
        got = orc.e4m3_decode(c)
        assert (np.isnan(ref) and np.isnan(got)) or ref == got


def test_i8_scale_degenerate(orc):
    assert orc.i8_scale(0.0) == (0.0, 0.0)
    assert orc.i8_scale(1e-38) == (0.0, 0.0)          # 127/amax overflows fp32: block is all-zero
    s, inv = orc.i8_scale(3.0)
    assert s == np.float32(np.float32(3.0) / np.float32(127.0)) and inv == np.float32(np.float32(127.0) / np.float32(3.0))
    assert orc.i8_encode(3.0, inv) == 127 and orc.i8_encode(-3.0, inv) == -127


def test_quant_i8_tokblock_bounds(orc):
    rng = np.random.default_rng(2)
    X = rng.standard_normal((2, 256, 64)).astype(np.float32) * 3
    X[1, 64:128] = 0.0                                # an all-zero block
    codes, scales = orc.quant_i8_tokblock(X, 64)
    assert codes.shape == X.shape and scales.shape == (2, 4)
    assert scales[1, 1] == 0 and not codes[1, 64:128].any()
    for bh in range(2):
        for b in range(4):
            blk = X[bh, b * 64:(b + 1) * 64]
            c = codes[bh, b * 64:(b + 1) * 64].astype(np.float64)
            s = float(scales[bh, b])
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            assert np.isclose(s, amax / 127, rtol=1e-6)
            assert np.abs(blk - c * s).max() <= 0.5 * s * (1 + 1e-5)      # nearest rounding
            assert np.abs(c).max() == 127                                  # the block max hits the top code
    c2, s2 = orc.quant_i8_tokblock(-X, 64)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scales)      # symmetric


def test_smooth_mean_certified_and_centres(orc):
    import workloads as wl
    w = wl.with_len(wl.WORKLOADS["c2"], 512, b=1, hq=2, hkv=2)
    K = wl.build(w, "k")[0]
    eps = 1e-3
    mu, bad = orc.smooth_mean(K, eps)
    assert bad == 0
    ref = (K.astype(np.float64).mean(axis=1) - eps).astype(np.float32)
    assert np.array_equal(mu, ref)
    Ks = (K - mu[:, None, :]).astype(np.float32)
    assert np.abs(Ks.astype(np.float64).mean(axis=1) - eps).max() < 1e-4


def test_quant_chan_bounds(orc):
    rng = np.random.default_rng(3)
    V = rng.standard_normal((2, 128, 32)).astype(np.float32)
    for fmt in ("i8", "e4m3"):
        codes, scales = orc.quant_chan(V, fmt)
        assert codes.shape == (2, 32, 128) and scales.shape == (2, 32)
        amax = np.abs(V).max(axis=1)
        top = 127 if fmt == "i8" else 448
        assert np.allclose(scales, amax / top, rtol=1e-6)
        if fmt == "i8":
            deq = codes.view(np.int8).astype(np.float64) * scales[:, :, None]
            assert np.all(np.abs(V.transpose(0, 2, 1) - deq) <= 0.5 * scales[:, :, None] * (1 + 1e-5))
        else:
            dec = np.array([orc.e4m3_decode(c) for c in range(256)])
            deq = dec[codes] * scales[:, :, None]
            err = np.abs(V.transpose(0, 2, 1) - deq)
            # e4m3: half an ulp of 3 mantissa bits (relative 1/16) or half the subnormal step
            bound = np.maximum(np.abs(V.transpose(0, 2, 1)) / 16.0, 2.0 ** -10 * scales[:, :, None]) * (1 + 1e-6)
            assert np.all(err <= bound)
            for bh in range(2):
                for c in range(32):
                    assert (codes[bh, c] & 0x7F).max() == 0x7E        # channel max encodes as 448


def _mx_decode(codes, scales, blk_axis_len):
    tab = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
    lo, hi = tab[codes & 0xF], tab[codes >> 4]
    v = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    e = scales.astype(np.int64) - 127
    return v * np.repeat(2.0 ** e, 32, axis=-1)


def test_mx_quant_bounds_and_layouts(orc):
    rng = np.random.default_rng(4)
    X = (rng.standard_t(3, (2, 64, 64)) * 2.0 ** rng.integers(-20, 20, (2, 64, 1))).astype(np.float32)
    X[0, 3, :32] = 0.0                               # zero block -> smallest scale, zero codes
    codes, scales = orc.quant_mx_rows(X)
    assert codes.shape == (2, 64, 32) and scales.shape == (2, 64, 2)
    assert scales[0, 3, 0] == 0 and not (codes[0, 3, :16] & 0x77).any()
    deq = _mx_decode(codes, scales, 32)
    xb = X.reshape(2, 64, 2, 32).astype(np.float64)
    e = scales.astype(np.int64) - 127
    amax = np.abs(xb).max(axis=-1)
    ok = amax > 0
    assert np.all((2.0 ** (e + 2) <= amax)[ok]) and np.all((amax < 2.0 ** (e + 3))[ok])
    y = np.abs(xb) / (2.0 ** e)[..., None]                         # magnitude on the e2m1 axis
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(xb - deq.reshape(2, 64, 2, 32)) / (2.0 ** e)[..., None]
    bound = np.where(y <= 6, step / 2, y - 6)
    assert np.all(err <= bound + 1e-12)
    # token-axis layout is the row layout of the transposed slice
    ct, st = orc.quant_mx_cols(X)
    cr, sr = orc.quant_mx_rows(np.ascontiguousarray(X.transpose(0, 2, 1)))
    assert np.array_equal(ct, cr) and np.array_equal(st, sr)


def test_block_means_library(orc):
    rng = np.random.default_rng(5)
    X = rng.standard_normal((3, 512, 16)).astype(np.float32)
    m = orc.block_means(X, 128)
    ref = X.astype(np.float64).reshape(3, 4, 128, 16).mean(axis=2).astype(np.float32)
    assert np.array_equal(m, ref)


def test_double_cache_overhead(orc):
    # ThriftAttention, Significance: double caching costs +28% KV memory.  NVFP4
    # (4-bit values, one 8-bit scale per 16) gives 4.5/16; the MXFP4 used here
    # (one 8-bit scale per 32) gives 4.25/16, measured from the quantiser output.
    page = FACTS["thrift_kv_memory_overhead"]["value"]
    assert abs(4.5 / 16 - page) < 0.005
    X = np.zeros((1, 256, 128), np.float32)
    c, s = orc.quant_mx_rows(X)
    ratio = (c.nbytes + s.nbytes) / (X.size * 2)
    assert ratio == 4.25 / 16
