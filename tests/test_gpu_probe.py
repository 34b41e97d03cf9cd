"""Rate probes behind bqa_debug_probe, run through the C ABI on small grids.

The read probes' checksum words are recomputed on the host from the same
buffer (one XOR fold per thread over the elements it loads, the low 16 bits
of the four folded words, the maximum over the first wavefront), which
checks that every 16-byte element of a ragged length is read exactly where
the probe's grid-stride loop and its tail say it is.  The copy probe must
reproduce its source; every compute probe must finish and write its word
for every workgroup."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _read_checksums(words: np.ndarray, grid: int) -> np.ndarray:
    """words: int32 [n16, 4]. Per workgroup: each thread t < 64 of wavefront 0
    loads elements b*2048 + t + 256 u + k * grid * 2048 (u = 0..7) below n16."""
    n16 = words.shape[0]
    fold = np.bitwise_xor.reduce(words, axis=1).astype(np.int64) & 0xFFFFFFFF
    out = np.zeros(grid, np.uint32)
    stride = grid * 2048
    for b in range(grid):
        best = 0
        for t in range(64):
            idx = np.arange(b * 2048 + t, n16, stride)[:, None] + 256 * np.arange(8)[None, :]
            idx = idx[idx < n16]
            acc = np.bitwise_xor.reduce(fold[idx]) if idx.size else 0
            best = max(best, int(acc) & 0xFFFF)
        out[b] = best
    return out


@pytest.mark.parametrize("nt", [False, True], ids=["default", "nontemporal"])
@pytest.mark.parametrize("grid,n16", [(4, 4 * 2048 * 3 + 777), (7, 5000), (3, 100), (2, 2048 * 2)])
def test_read_probe_checksum(nt, grid, n16):
    import bit_quantized_attention_amd as bqa
    rng = np.random.default_rng(grid * 100003 + n16)
    words = rng.integers(-2**31, 2**31, size=(n16, 4), dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(words).cuda()
    dst = torch.full((grid + 1,), -1, dtype=torch.int32, device="cuda")
    kind = bqa.BQA_PROBE_READ_NT if nt else bqa.BQA_PROBE_READ
    bqa.bqa_debug_probe(kind, grid, 0, src, dst, n16 * 16)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got[:grid], _read_checksums(words, grid))
    assert got[grid] == 0xFFFFFFFF                       # nothing past the grid's words


@pytest.mark.parametrize("grid,n16", [(5, 3 * 1280 + 11), (64, 100)])
def test_copy_probe(grid, n16):
    import bit_quantized_attention_amd as bqa
    rng = np.random.default_rng(n16)
    src = torch.from_numpy(rng.integers(0, 2**31, size=(n16 + 1, 4), dtype=np.int64).astype(np.int32)).cuda()
    dst = torch.full((n16 + 1, 4), -7, dtype=torch.int32, device="cuda")
    bqa.bqa_debug_probe(bqa.BQA_PROBE_COPY, grid, 0, src, dst, n16 * 16)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n16], src[:n16])
    assert (dst[n16] == -7).all()


def test_compute_probes_write_every_word():
    import bit_quantized_attention_amd as bqa
    kinds = [bqa.BQA_PROBE_MFMA_I8, bqa.BQA_PROBE_MFMA_F8, bqa.BQA_PROBE_MFMA_F4, bqa.BQA_PROBE_MFMA_BF16,
             bqa.BQA_PROBE_EXP] + list(range(bqa.BQA_PROBE_ISSUE_MFMA, bqa.BQA_PROBE_LDS_SPANS + 1))
    grid = 9
    for kind in kinds:
        dst = torch.full((grid + 1,), -1, dtype=torch.int32, device="cuda")
        bqa.bqa_debug_probe(kind, grid, 3, None, dst, grid * 4)
        torch.cuda.synchronize()
        got = dst.cpu().numpy().view(np.uint32)
        assert got[grid] == 0xFFFFFFFF, kind
        if kind in (bqa.BQA_PROBE_MFMA_I8, bqa.BQA_PROBE_MFMA_F8, bqa.BQA_PROBE_MFMA_F4,
                    bqa.BQA_PROBE_MFMA_BF16, bqa.BQA_PROBE_EXP):
            assert (got[:grid] != 0xFFFFFFFF).all(), kind
        else:
            assert (got[:grid] <= 0xFFFF).all(), kind  # the wavefront maximum of a 16-bit word
