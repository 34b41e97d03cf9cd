"""Seeded synthetic inputs shaped like the workloads on the source pages.

This module is shared by the CPU oracle's tests, the GPU parity tests and
the benchmark.  It holds only random-number recipes and the rounding of
fp32 draws to the storage dtype of each workload; none of the attention,
quantisation or selection arithmetic lives here.

Every tensor is produced in chunks of one (batch, head) slice, each from its
own ``SeedSequence([config_id, tensor_id, b, h])`` on NumPy's PCG64, so any
chunk can be regenerated on its own (the oracle samples chunks of the large
workloads).  Values are drawn in fp32 and rounded to nearest-even into the
workload dtype (bf16 or fp16); the arrays returned are fp32 arrays whose
values are exactly representable in that dtype.

Recipes (distributions written N(mean, variance)):

* ``c1``  B=1 H=1 N=128 d=64, fp16, non-causal.  Q, K, V ~ N(0,1); each K
  channel gets a bias ~ N(0,4) (the same for all tokens of a head).
* ``c2``  B=2 H=16 N=4096 d=128, bf16, causal.  Q, K, V ~ N(0,1); 20 of the
  16*128 (head, channel) pairs of Q, and 20 of K, drawn without replacement,
  are multiplied by 20 (outlier channels); K gets a channel bias ~ N(0,4).
* ``c3``  B=1 H=16 N=8192 (or 2048) d=128, bf16, causal.  Q, K, V ~ N(0,1);
  every row of Q and K is scaled to unit L2 norm (QK-norm) before rounding;
  dO ~ N(0, 0.01).  ``qraw`` / ``kraw`` are the same draws rounded to bf16
  without the normalisation (inputs of the fused QK-norm quantiser).
* ``c4``  B=1 H=32 N=16384 d=128, bf16, non-causal.  Q, K, V ~ Student-t
  with 3 degrees of freedom (heavy tails); dO ~ N(0, 0.01).
* ``c5``  B=1 Hq=32 Hkv=8 N=131072 d=128, bf16, causal, GQA.  Per KV head a
  basis W (4 x d, entries N(0,1/d)); per (head, 128-token block)
  coefficients a ~ N(0, 0.25 I4).  Q[h,t] = g + sqrt(d) a_q[h,blk(t)] W[h/4],
  K[h',t] = g' + sqrt(d) a_k[h',blk(t)] W[h'], with g, g', V ~ N(0,1): a
  shared rank-4 part that makes attention peaked and block-structured.
* ``c5d`` decode against a 131072-token cache: B=16, Hq=32, Hkv=8, one query
  token per (b, head).  The cache is built like c5's K and V for every b; the
  query row is built like a Q row with its own coefficients.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids used in the seed sequence
T_Q, T_K, T_V, T_DO, T_KBIAS, T_OUTLIER, T_W, T_AQ, T_AK, T_QDEC = range(10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: str          # "bf16" or "fp16"
    kind: str           # "sage" | "sagebwd" | "qat" | "thrift" | "thrift_decode"


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 1, 1, 128, 128, 64, False, "fp16", "sage"),
    "c2": Workload("c2", 2, 2, 16, 16, 4096, 4096, 128, True, "bf16", "sage"),
    "c3": Workload("c3", 3, 1, 16, 16, 8192, 8192, 128, True, "bf16", "sagebwd"),
    "c4": Workload("c4", 4, 1, 32, 32, 16384, 16384, 128, False, "bf16", "qat"),
    "c5": Workload("c5", 5, 1, 32, 8, 131072, 131072, 128, True, "bf16", "thrift"),
    "c5d": Workload("c5d", 6, 16, 32, 8, 1, 131072, 128, True, "bf16", "thrift_decode"),
}


def with_len(w: Workload, n: int, b: int | None = None, hq: int | None = None,
             hkv: int | None = None) -> Workload:
    """Same recipe and seeds at another sequence length / batch / head count."""
    nq = 1 if w.kind == "thrift_decode" else n
    hq = w.Hq if hq is None else hq
    hkv = (w.Hkv if hkv is None else hkv)
    return dataclasses.replace(w, Nq=nq, Nk=n, B=w.B if b is None else b, Hq=hq, Hkv=hkv)


def _rng(cfg_id: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, tensor, b, h])))


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to nearest-even bf16/fp16, returned as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32)
        r = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) & np.uint32(0xFFFF0000))
        return r.view(np.float32)
    if dtype == "fp32":
        return x
    raise ValueError(dtype)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 storage of an fp32 array whose values are bf16-exact."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _normal(g: np.random.Generator, shape, std=1.0) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _outlier_mask(w: Workload, tensor: int) -> np.ndarray:
    """c2: boolean [H, d] marking the 20 outlier (head, channel) pairs of Q or K."""
    g = _rng(w.cfg_id, T_OUTLIER, tensor, 0)
    n_out = int(round(0.01 * w.Hq * w.d))
    pick = g.choice(w.Hq * w.d, size=n_out, replace=False)
    m = np.zeros(w.Hq * w.d, dtype=bool)
    m[pick] = True
    return m.reshape(w.Hq, w.d)


def _basis(w: Workload, hkv: int) -> np.ndarray:
    """c5: rank-4 basis W of KV head hkv, entries N(0, 1/d)."""
    g = _rng(5, T_W, 0, hkv)   # shared by prefill and decode recipes
    return _normal(g, (4, w.d), 1.0 / math.sqrt(w.d))


def chunk(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One [N, d] slice (fp32 values, exact in the workload dtype)."""
    N = w.Nk if tensor in ("k", "v", "kraw") else w.Nq
    d = w.d
    if w.name == "c1" or w.name == "c2":
        tid = {"q": T_Q, "k": T_K, "v": T_V}[tensor]
        x = _normal(_rng(w.cfg_id, tid, b, h), (N, d))
        if w.name == "c2" and tensor in ("q", "k"):
            m = _outlier_mask(w, tid)[h]
            x[:, m] *= np.float32(20.0)
        if tensor == "k":
            bias = _normal(_rng(w.cfg_id, T_KBIAS, b, h), (d,), 2.0)
            x += bias[None, :]
        return round_to(x, w.dtype)
    if w.name == "c3":
        raw = tensor in ("qraw", "kraw")        # the same draws before QK-norm
        tensor = {"qraw": "q", "kraw": "k"}.get(tensor, tensor)
        tid = {"q": T_Q, "k": T_K, "v": T_V, "do": T_DO}[tensor]
        if tensor == "do":
            return round_to(_normal(_rng(w.cfg_id, tid, b, h), (N, d), 0.1), w.dtype)
        x = _normal(_rng(w.cfg_id, tid, b, h), (N, d))
        if tensor in ("q", "k") and not raw:       # QK-norm of the model layer, applied to the inputs
            x64 = x.astype(np.float64)
            x64 /= np.sqrt(np.sum(x64 * x64, axis=1, keepdims=True))
            x = x64.astype(np.float32)
        return round_to(x, w.dtype)
    if w.name == "c4":
        tid = {"q": T_Q, "k": T_K, "v": T_V, "do": T_DO}[tensor]
        g = _rng(w.cfg_id, tid, b, h)
        if tensor == "do":
            return round_to(_normal(g, (N, d), 0.1), w.dtype)
        return round_to(g.standard_t(3.0, size=(N, d)).astype(np.float32), w.dtype)
    if w.name in ("c5", "c5d"):
        blk = 128
        if tensor == "v":
            return round_to(_normal(_rng(5, T_V, b, h), (N, d)), w.dtype)
        if tensor == "k":
            gk = _normal(_rng(5, T_K, b, h), (N, d))
            a = _normal(_rng(5, T_AK, b, h), (N // blk, 4), 0.5)
            low = (math.sqrt(d) * (a @ _basis(w, h))).astype(np.float32)
            return round_to(gk + np.repeat(low, blk, axis=0), w.dtype)
        if tensor == "q" and w.name == "c5":
            gq = _normal(_rng(5, T_Q, b, h), (N, d))
            a = _normal(_rng(5, T_AQ, b, h), (N // blk, 4), 0.5)
            low = (math.sqrt(d) * (a @ _basis(w, h * w.Hkv // w.Hq))).astype(np.float32)
            return round_to(gq + np.repeat(low, blk, axis=0), w.dtype)
        if tensor == "q":                   # decode: one token, fresh coefficients
            g = _rng(6, T_QDEC, b, h)
            gq = _normal(g, (1, d))
            a = _normal(g, (1, 4), 0.5)
            low = (math.sqrt(d) * (a @ _basis(w, h * w.Hkv // w.Hq))).astype(np.float32)
            return round_to(gq + low, w.dtype)
    raise ValueError((w.name, tensor))


def heads_of(w: Workload, tensor: str) -> int:
    return w.Hkv if tensor in ("k", "v", "kraw") else w.Hq


def _chunk_job(args):
    w, tensor, b, h = args
    return b, h, chunk(w, tensor, b, h)


def build(w: Workload, tensor: str, workers: int = 0) -> np.ndarray:
    """Whole [B, H, N, d] tensor (fp32 values, exact in the workload dtype).

    workers > 1 generates the (b, h) chunks in that many fresh interpreter
    processes (each chunk has its own seed, so the result is the same)."""
    H = heads_of(w, tensor)
    N = w.Nk if tensor in ("k", "v", "kraw") else w.Nq
    out = np.empty((w.B, H, N, w.d), dtype=np.float32)
    jobs = [(w, tensor, b, h) for b in range(w.B) for h in range(H)]
    if workers > 1 and len(jobs) > 1:
        import concurrent.futures as cf
        import multiprocessing as mp
        with cf.ProcessPoolExecutor(max_workers=min(workers, len(jobs)), mp_context=mp.get_context("spawn")) as ex:
            for b, h, x in ex.map(_chunk_job, jobs, chunksize=1):
                out[b, h] = x
        return out
    for job in jobs:
        b, h, x = _chunk_job(job)
        out[b, h] = x
    return out


def default_workers() -> int:
    """Generator processes for full-size inputs: the CPUs this process may use,
    at most 16 (BQA_GEN_WORKERS overrides, e.g. 1 under a profiler)."""
    import os
    if os.environ.get("BQA_GEN_WORKERS"):
        return max(1, int(os.environ["BQA_GEN_WORKERS"]))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))
