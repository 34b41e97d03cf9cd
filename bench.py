"""Benchmark of the block-quantized attention hot path on one MI355X.

Workloads (``--workload``, default c2):

  c2  SageAttention INT8 forward at B=2, H=16, N=4096, d=128, causal, bf16
      inputs (outlier channels and a K channel bias): K-smoothing means, INT8
      Q/K, per-channel e4m3 V, fused attention with e4m3 P.V.
  c3  SageBwd training step at B=1, H=16, N=8192, d=128, causal, QK-norm
      inputs: K-smoothing (eps 1e-3), INT8 forward, INT8 backward with the
      bf16 dP = dO V^T; `value` counts forward + backward (14 B H N^2 d / 2)
      and the roofline covers the backward call.
  c3i the same step with the fully INT8 backward (dP = dO V^T in INT8 too).
  c3n the same step from raw (unnormalised) Q, K rows with QK-norm fused
      into the INT8 quantiser and its backward into the dQ / dK epilogues.
  c4  Attn-QAT FP4 forward at B=1, H=32, N=16384, d=128, non-causal,
      Student-t inputs: MXFP4 Q, K, V, fused attention with MXFP4 P.V and
      the bf16 auxiliary output O'.
  c4t the Attn-QAT training step on the same inputs: forward with O', then
      the backward; `value` counts forward + backward, the roofline the
      backward call.
  c4i the Attn-QAT inference forward on the same inputs: no O'.
  c4p the post-training FP4 baseline that Attn-QAT is compared with, on
      c4's inputs: Q smoothed by its bf16 128-row block means and K by its
      token mean before MXFP4, the means' score shifts, two-level P.
  c5  ThriftAttention prefill at B=1, Hq=32, Hkv=8, N=131072, d=128,
      causal, low-rank inputs: MXFP4 Q, K, V with block means, block
      selection (5 %), mixed FP4 / bf16 attention.
  c5d ThriftAttention decode, B=16, one query against a 131072-token
      cache: query quantisation, selection, split-K attention and merge.

One step = one pass of the whole path over the batch (quantisers and
attention).  Inputs are generated on the host and are resident in HBM
before timing starts.

Prints one JSON line.  `value` is effective attention TOPS of the whole step
(4*B*H*N^2*d, halved for causal, over the step time).  `roofline` reports the
attention call alone: its algorithmic operations per launch over its average
time, measured with HIP events on the stream it runs on, against the dense
matrix-core peak of its operand types.  `cpu_baseline` times the CPU oracle
on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--workload c2|c3|c3i|c3n|c4|c4t|c4i|c4p|c5|c5d] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_I8_TOPS = 5033.2          # MI355X dense INT8 (and FP8) MFMA peak, 256 CU x 2.4 GHz x 8192 ops/clk
PEAK_F4_TFLOPS = 10066.3       # dense MXFP4, twice the fp8 rate
PEAK_BF16_TFLOPS = 2516.6      # dense bf16, half the fp8 rate
METRIC = "attention TOPS (fwd, fwd+bwd) at d=128, N=4k-131k; % of i8/fp8/fp4 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _traffic_for(kernel: str):
    """Measured HBM bytes per launch of `kernel` from the committed counter
    summary, if it was taken on the current kernel source and build flags."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e:
        return None
    src = os.path.join(ROOT, e["source"])
    try:
        import hashlib
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != e["source_sha256"]:
            return None
    except OSError:
        return None
    from bit_quantized_attention_amd.csrc import build as _build
    if e.get("build_flags") != _build.EXTRA.get(os.path.basename(src), []):
        return None
    return e["bytes_per_launch"]


PROBES_FILE = os.path.join(ROOT, "profiles", "probes.json")


def _measured_peak(kinds):
    """The rate probes' measured figure for a roofline peak (committed from a
    `bench.py --probe` run): the matrix rates per operand type, weighted the
    way the spec peak is, or the HBM read rate."""
    try:
        with open(PROBES_FILE) as f:
            pr = json.load(f)["probes"]
    except (OSError, ValueError, KeyError):
        return None
    try:
        return {k: pr[k]["measured"] for k in kinds}
    except KeyError:
        return None


def cpu_baseline(w, budget_s: float = 20.0):
    """The oracle (as it stands) on a bounded sample: full quantisation and
    forward of whole (b, h) heads, as many as fit the time budget."""
    import numpy as np

    import oracle
    import workloads as wl
    from tests.helpers import tau_for
    oracle.lib()
    tau = tau_for(w.d)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    ops = 0.0
    heads = 0
    t0 = time.perf_counter()
    for idx in range(w.B * w.Hq):
        b, h = divmod(idx, w.Hq)
        Q, K, V = (wl.chunk(w, t, b, h)[None] for t in ("q", "k", "v"))
        mu, _ = oracle.smooth_mean(K, 0.0)
        qc, qs = oracle.quant_i8_tokblock(Q, 128)
        kc, ks = oracle.quant_i8_tokblock(K, 64, mu)
        vc, vs = oracle.quant_chan(V, "e4m3")
        oracle.sage_fwd(qc=qc[0], qs=qs[0], q_blk=128, kc=kc[0], ks=ks[0], k_blk=64, pv_mode=oracle.PV_F8,
                        vc_t=vc[0], vs=vs[0], Nq=w.Nq, Nk=w.Nk, d=w.d, causal=w.causal, tau=tau, kv_tile=64)
        ops += 4.0 * w.Nq * w.Nk * w.d / (2 if w.causal else 1)
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    _ = np
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.Hq} (b,h) heads, full quantisation + forward, N={w.Nk}, "
                      f"{dt:.1f} s"}


def cpu_baseline_qat(w, budget_s: float = 20.0, kv_tile: int = 64):
    """The oracle on a bounded sample of the Attn-QAT forward: MXFP4
    quantisation of one whole head, then its forward (O and O') over chunks of
    query rows until the time budget is spent; key tiles of kv_tile as the
    kernel timed (64 for the forward with O', 128 without)."""
    import oracle
    import workloads as wl
    from tests.helpers import tau_for
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V = (wl.chunk(w, t, 0, 0)[None] for t in ("q", "k", "v"))
    qc, qs = oracle.quant_mx_rows(Q)
    kc, ks = oracle.quant_mx_rows(K)
    vc, vs = oracle.quant_mx_cols(V)
    rows, r0, chunk = 0, 0, 16
    while r0 < w.Nq and time.perf_counter() - t0 < budget_s:
        oracle.qat_fwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Nq=w.Nq, Nk=w.Nk, d=w.d,
                       tau=tau_for(w.d), kv_tile=kv_tile, rows=(r0, r0 + chunk))
        rows += chunk
        r0 += chunk
    dt = time.perf_counter() - t0
    ops = 4.0 * rows * w.Nk * w.d
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"head (0,0): MXFP4 quantisation of Q, K, V, then O and O' for {rows} of {w.Nq} query "
                      f"rows against N={w.Nk} keys, {dt:.1f} s"}


def _sage_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import SagePath, attention_ops, sage_problem, to_device
    import workloads as wl
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_F8PV, q_block=128,
                     smooth_k=True, smooth_eps=0.0)
    path = SagePath(p, to_device(Q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype), keep_q_codes=False)
    ops = attention_ops(p)
    return dict(
        path=path, ops=ops, dtype="i8+e4m3",
        workload="SageAttention INT8 forward (c2): B=2 H=16 N=4096 d=128 causal, bf16 in, K-smoothing, "
                 "INT8 Q/K, e4m3 P.V; step = quantise K,V + attention (Q quantised inside the attention kernel)",
        roofline={"bound": "mfma", "kernel": "sage_fwd_f8_kernel (i8 QK^T + fp8 P.V, three-stage pipeline)",
                  "peak": PEAK_I8_TOPS, "ops_per_launch": ops},
        traffic_key="sage_fwd_f8_kernel<128,causal>", cpu=cpu_baseline)


def _qat_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import QatPath, attention_ops, qat_problem, to_device
    import workloads as wl
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = qat_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    path = QatPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), aux=True)
    ops = attention_ops(p)                       # the two MXFP4 products
    aux = ops / 2                                # O' = bf16(P) V, one more product of the P.V size
    # time at the two peaks: the fp4 products at the MXFP4 rate, O' at the bf16 rate
    t_peak = ops / (PEAK_F4_TFLOPS * 1e12) + aux / (PEAK_BF16_TFLOPS * 1e12)
    return dict(
        path=path, ops=ops, dtype="mxfp4+bf16",
        workload="Attn-QAT FP4 forward (c4): B=1 H=32 N=16384 d=128 non-causal, Student-t bf16 in, MXFP4 Q/K/V/P, "
                 "bf16 auxiliary output O'; step = quantise Q,K,V + attention",
        roofline={"bound": "mfma", "kernel": "attn_fwd QAT (vdeq_kernel + qat_aux_kernel): MXFP4 QK^T and "
                                             "P.V plus bf16 O'",
                  "peak": round((ops + aux) / t_peak / 1e12, 1), "peak_note": "fp4 and bf16 dense peaks "
                  "weighted by each product's share of the operations",
                  "ops_per_launch": ops + aux},
        traffic_key="qat_aux_kernel", cpu=cpu_baseline_qat)


def cpu_baseline_ptq(w, budget_s: float = 20.0):
    """The oracle on a bounded sample of the post-training baseline: smoothing
    and MXFP4 quantisation of one whole head, then its forward over query
    blocks until the time budget is spent."""
    import oracle
    import workloads as wl
    from tests.helpers import tau_for
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V = (wl.chunk(w, t, 0, 0)[None] for t in ("q", "k", "v"))
    qbar, Qs = oracle.smooth_q_blocks(Q)
    _, Ks = oracle.smooth_k(K)
    qc, qs = oracle.quant_mx_rows(Qs)
    kc, ks = oracle.quant_mx_rows(Ks)
    vc, vs = oracle.quant_mx_cols(V)
    qb = 0
    while qb * 128 < w.Nq and time.perf_counter() - t0 < budget_s:
        oracle.ptq_fwd(qc=qc[0], qs=qs[0], qbar=qbar[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Nq=w.Nq,
                       Nk=w.Nk, d=w.d, tau=tau_for(w.d), qblocks=(qb, qb + 1))
        qb += 1
    dt = time.perf_counter() - t0
    rows = min(w.Nq, 128 * qb)
    return {"value": 4.0 * rows * w.Nk * w.d / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"head (0,0): Q/K smoothing and MXFP4 quantisation, then the forward of {qb} of "
                      f"{(w.Nq + 127) // 128} query blocks against N={w.Nk} keys, {dt:.1f} s"}


def _ptq_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import PtqPath, attention_ops, ptq_problem, to_device
    import workloads as wl
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = ptq_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, causal=w.causal)
    path = PtqPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    ops = attention_ops(p)                       # the two MXFP4 products
    return dict(
        path=path, ops=ops, dtype="mxfp4",
        workload="post-training FP4 baseline on the Attn-QAT inputs (c4p): B=1 H=32 N=16384 d=128 non-causal, "
                 "Student-t bf16 in; Q less its bf16 128-row block means and K less its token mean, MXFP4 Q/K/V, "
                 "two-level MXFP4 P; step = smoothing quantisers + score shifts + attention",
        roofline={"bound": "mfma", "kernel": "attn_fwd_ptq (ptq_bias_kernel + thrift_fwd_kernel<PTQ>): MXFP4 QK^T "
                                             "and P.V; the bf16 score-shift product adds 0.02 % more operations",
                  "peak": PEAK_F4_TFLOPS, "ops_per_launch": ops},
        traffic_key="thrift_fwd_kernel<true>", cpu=cpu_baseline_ptq)


def _qat_infer_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import QatPath, attention_ops, qat_problem, to_device
    import workloads as wl
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = qat_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    path = QatPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), aux=False)
    ops = attention_ops(p)
    return dict(
        path=path, ops=ops, dtype="mxfp4",
        workload="Attn-QAT FP4 inference forward (c4i): B=1 H=32 N=16384 d=128 non-causal, Student-t bf16 in, MXFP4 "
                 "Q/K/V/P, no auxiliary output; step = quantise Q,K,V + attention",
        roofline={"bound": "mfma", "kernel": "attn_fwd QAT without O' (qat_fwd_kernel): MXFP4 QK^T and P.V",
                  "peak": PEAK_F4_TFLOPS, "ops_per_launch": ops},
        traffic_key="qat_fwd_kernel", cpu=lambda w: cpu_baseline_qat(w, kv_tile=128))


def _thrift_pairs(path, w):
    """(fp4 pairs, bf16 pairs) of (query, key) scores the prefill computes,
    from the selection the step made (diagonal blocks count their causal half)."""
    import numpy as np
    idx = path.sel_idx.cpu().numpy()
    cnt = path.sel_cnt.cpu().numpy()
    full, diag = 128 * 128, 128 * 129 // 2
    bf16 = 0
    for i in range(idx.shape[2]):
        sel = idx[:, :, i, :]
        n = cnt[:, :, i]
        on_diag = ((sel == i) & (np.arange(sel.shape[-1])[None, None, :] < n[..., None])).sum()
        bf16 += int(n.sum() - on_diag) * full + int(on_diag) * diag
    total = w.B * w.Hq * w.Nq * (w.Nq + 1) // 2
    return total - bf16, bf16


def cpu_baseline_thrift(w, budget_s: float = 20.0):
    """The oracle on a bounded sample of the Thrift prefill: MXFP4
    quantisation, block means and selection of head (0,0), then the mixed
    forward of its last query blocks (the longest rows) until the budget."""
    import numpy as np

    import oracle
    import workloads as wl
    from tests.helpers import tau_for
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V = (wl.chunk(w, t, 0, 0) for t in ("q", "k", "v"))
    qc, qs = oracle.quant_mx_rows(Q[None]); kc, ks = oracle.quant_mx_rows(K[None]); vc, vs = oracle.quant_mx_cols(V[None])
    nkb = w.Nk // 128
    ms = max(1, min(nkb, -(-nkb * 50_000 // 1_000_000)))
    idx, cnt = oracle.select_blocks(oracle.block_means(Q[None], 128)[0], oracle.block_means(K[None], 128)[0], True,
                                    50_000, ms)
    pairs, qb = 0, nkb
    while qb > 0 and time.perf_counter() - t0 < budget_s:
        qb -= 1
        oracle.thrift_fwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Qh=Q, Kh=K, Vh=V,
                          sel_idx=idx, sel_cnt=cnt, Nq=w.Nq, Nk=w.Nk, d=w.d, blk=128, hp_tile=32, causal=True,
                          tau=tau_for(w.d),
                          qblocks=(qb, qb + 1))
        pairs += sum(128 * qb + a + 1 for a in range(128))
    dt = time.perf_counter() - t0
    _ = np
    return {"value": 4.0 * pairs * w.d / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"head (0,0): MXFP4 quantisation, block means and selection, then the mixed forward of its "
                      f"last {nkb - qb} of {nkb} query blocks (N={w.Nk}), {dt:.1f} s"}


def _thrift_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import ThriftPath, thrift_problem, to_device
    import workloads as wl
    nw = wl.default_workers()
    Q, K, V = (wl.build(w, t, workers=nw) for t in ("q", "k", "v"))
    p = thrift_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, budget_ppm=50_000)
    path = ThriftPath(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    del Q, K, V
    path.step()
    torch.cuda.synchronize()
    f4, b16 = _thrift_pairs(path, w)
    ops_f4, ops_b16 = 4.0 * w.d * f4, 4.0 * w.d * b16
    t_peak = ops_f4 / (PEAK_F4_TFLOPS * 1e12) + ops_b16 / (PEAK_BF16_TFLOPS * 1e12)
    ops = 4.0 * w.B * w.Hq * w.Nq * w.Nk * w.d / 2
    return dict(
        path=path, ops=ops, dtype="mxfp4+bf16",
        workload="ThriftAttention prefill (c5): B=1 Hq=32 Hkv=8 N=131072 d=128 causal, low-rank bf16 in, 5 % of "
                 "128x128 block pairs in bf16, the rest MXFP4; step = quantise Q,K,V + block means + selection + "
                 "attention",
        roofline={"bound": "mfma", "kernel": "thrift_fwd_kernel: MXFP4 QK^T/P.V on unselected pairs, bf16 on "
                                             "selected pairs",
                  "peak": round((ops_f4 + ops_b16) / t_peak / 1e12, 1),
                  "peak_note": f"fp4 and bf16 dense peaks weighted by the pairs each path computed "
                               f"({100.0 * b16 / (f4 + b16):.2f} % bf16)",
                  "ops_per_launch": ops_f4 + ops_b16},
        traffic_key="thrift_fwd_kernel<false>", cpu=cpu_baseline_thrift)


def cpu_baseline_decode(w, budget_s: float = 20.0):
    """The oracle on a bounded sample of decode: per (b, KV head) the MXFP4
    cache and key means, then each query head's selection and decode, until
    the budget."""
    import oracle
    import workloads as wl
    from tests.helpers import tau_for
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    G = w.Hq // w.Hkv
    nkb = w.Nk // 128
    ms = max(1, min(nkb, -(-nkb * 50_000 // 1_000_000)))
    heads = 0
    for bk in range(w.B * w.Hkv):
        b, hk = divmod(bk, w.Hkv)
        K, V = wl.chunk(w, "k", b, hk), wl.chunk(w, "v", b, hk)
        kc, ks = oracle.quant_mx_rows(K[None]); vc, vs = oracle.quant_mx_cols(V[None])
        km = oracle.block_means(K[None], 128)[0]
        for g in range(G):
            q = wl.chunk(w, "q", b, hk * G + g)
            qc, qs = oracle.quant_mx_rows(q[None])
            idx, cnt = oracle.select_blocks(q, km, True, 50_000, ms)
            oracle.thrift_decode(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], q=q[0], Kh=K, Vh=V,
                                 sel=idx[0, :cnt[0]], Nk=w.Nk, d=w.d, blk=128, hp_tile=32, tau=tau_for(w.d),
                                 num_splits=1)
            heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": 4.0 * heads * w.Nk * w.d / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.Hq} (b, query head) decodes with their KV head's MXFP4 cache, key means "
                      f"and selection, Nk={w.Nk}, {dt:.1f} s"}


def _decode_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import ThriftDecodePath, thrift_problem, to_device
    import numpy as np
    import workloads as wl
    nw = wl.default_workers()
    q, K, V = wl.build(w, "q"), wl.build(w, "k", workers=nw), wl.build(w, "v", workers=nw)
    p = thrift_problem(w.B, w.Hq, w.Hkv, 1, w.Nk, w.d, budget_ppm=50_000)
    path = ThriftDecodePath(p, to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    del K, V
    path.build_cache()
    path.step()
    torch.cuda.synchronize()
    # algorithmic bytes of one attention call: the whole MXFP4 cache, the bf16
    # blocks that some head of the KV head selected, the queries and the output
    idx = path.sel_idx.cpu().numpy().reshape(w.B, w.Hkv, -1)
    union = sum(len(set(int(j) for j in idx[b, hk] if j >= 0)) for b in range(w.B) for hk in range(w.Hkv))
    fp4 = w.B * w.Hkv * w.Nk * 2 * (w.d // 2 + w.d // 32)
    b16 = union * 128 * w.d * 2 * 2
    qo = w.B * w.Hq * w.d * (2 + 0.5 + 2) + w.B * w.Hq * 4 * (idx.shape[-1] // (w.Hq // w.Hkv) + 1)
    nbytes = fp4 + b16 + qo
    ops = 4.0 * w.B * w.Hq * w.Nk * w.d
    _ = np
    return dict(
        path=path, ops=ops, dtype="mxfp4+bf16",
        workload="ThriftAttention decode (c5d): B=16 Hq=32 Hkv=8, one query against a 131072-token cache, d=128, "
                 "top 52 of 1024 blocks per head in bf16, the rest MXFP4; step = quantise q + block mean + "
                 "selection + attention (the double cache is built once, outside the step)",
        roofline={"bound": "hbm", "kernel": "thrift_decode_kernel + decode_combine_kernel", "peak": 8000.0,
                  "unit": "GB/s", "bytes_per_launch": nbytes,
                  "bytes_note": f"MXFP4 K/V cache {fp4 / 1e9:.3f} GB + bf16 blocks selected by some head of the KV "
                                f"head ({union} blocks, {b16 / 1e9:.3f} GB) + queries, selections and outputs"},
        traffic_key="thrift_decode_kernel", cpu=cpu_baseline_decode)


def cpu_baseline_sagebwd(w, budget_s: float = 25.0):
    """The oracle on a bounded sample of the SageBwd step: quantisation and
    the whole forward of head (0,0) (every row's O and log-sum-exp feed the
    backward), then its backward on the last query tile (dQ) and the first
    key tile (dK, dV), the two longest."""
    import oracle
    import workloads as wl
    from tests.helpers import tau_for
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V, dO = (wl.chunk(w, t, 0, 0) for t in ("q", "k", "v", "do"))
    tau = tau_for(w.d)
    mu, _ = oracle.smooth_mean(K[None], float(__import__("numpy").float32(1e-3)))
    qc, qs = oracle.quant_i8_tokblock(Q[None], 128)
    kc, ks = oracle.quant_i8_tokblock(K[None], 64, mu)
    vc, vs = oracle.quant_chan(V[None], "i8")
    O, lse = oracle.sage_fwd(qc=qc[0], qs=qs[0], q_blk=128, kc=kc[0], ks=ks[0], k_blk=64, pv_mode=oracle.PV_I8,
                             vc_t=vc[0], vs=vs[0], Nq=w.Nq, Nk=w.Nk, d=w.d, causal=True, tau=tau, kv_tile=64)
    nqt, nkt = w.Nq // 128, w.Nk // 64
    oracle.sage_bwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], V=V, dO=dO, O=oracle.round_to(O, "bf16"),
                    lse=lse.astype("float32"), causal=True, tau=tau, qtiles=(nqt - 1, nqt), ktiles=(0, 1))
    dt = time.perf_counter() - t0
    n = w.Nq
    fwd_pairs = n * (n + 1) // 2
    dq_pairs = sum(i + 1 for i in range(n - 128, n))             # last query tile, causal
    dkv_pairs = sum(n - j for j in range(64))                    # first key tile, causal
    ops = 4.0 * w.d * fwd_pairs + 6.0 * w.d * dq_pairs + 8.0 * w.d * dkv_pairs
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"head (0,0) at N={n}: quantisation and the full forward, then the backward of the last "
                      f"query tile (dQ) and the first key tile (dK, dV), {dt:.1f} s"}


def _sagebwd_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import SageTrainStep, sage_problem, to_device
    import workloads as wl
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_I8PV, q_block=128,
                     smooth_k=True, smooth_eps=1e-3)
    path = SageTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), to_device(dO, "bf16"))
    return dict(_sagebwd_roofline(w), path=path)


def _sagebwd_roofline(w):
    n_pairs = w.B * w.Hq * w.Nq * (w.Nq + 1) / 2
    bwd_ops = 10.0 * w.d * n_pairs          # S recompute, dP, dV, dQ, dK
    ops = 14.0 * w.B * w.Hq * w.Nq * w.Nk * w.d / 2
    # backward roofline: 4 of the 5 products at the i8 rate, dP at the bf16 rate
    t_peak = 0.8 * bwd_ops / (PEAK_I8_TOPS * 1e12) + 0.2 * bwd_ops / (PEAK_BF16_TFLOPS * 1e12)
    return dict(
        ops=ops, dtype="i8+bf16", timed="backward",
        workload="SageBwd training step (c3): B=1 H=16 N=8192 d=128 causal, QK-norm bf16 in, K-smoothing eps=1e-3, "
                 "INT8 Q/K/V/P forward; backward with INT8 dO/P/dS and bf16 dP; step = quantise + forward + backward",
        roofline={"bound": "mfma", "kernel": "attn_bwd (delta, dO quantiser, code transposes, sbwd_dkdv_kernel, "
                                             "sbwd_dq_kernel)",
                  "peak": round(bwd_ops / t_peak / 1e12, 1),
                  "peak_note": "i8 peak for 4 of the 5 backward products, bf16 for dP = dO V^T",
                  "ops_per_launch": bwd_ops},
        traffic_key="sbwd_dkdv_kernel<false>", cpu=cpu_baseline_sagebwd)


def _sagebwd_i8dp_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import SageTrainStep, sage_problem, to_device
    import workloads as wl
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_I8PV, q_block=128,
                     smooth_k=True, smooth_eps=1e-3)
    path = SageTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), to_device(dO, "bf16"),
                         int8_dp=True)
    case = _sagebwd_roofline(w)
    n_pairs = w.B * w.Hq * w.Nq * (w.Nq + 1) / 2
    bwd_ops = 10.0 * w.d * n_pairs
    case.update(path=path, dtype="i8",
                workload="fully INT8 SageBwd training step (c3i): B=1 H=16 N=8192 d=128 causal, QK-norm bf16 in, "
                         "K-smoothing eps=1e-3, INT8 forward; backward with all five products in INT8 (dP = dO V^T "
                         "from V's 64-token codes); step = quantise (V twice) + forward + backward")
    case["roofline"] = dict(case["roofline"], kernel="attn_bwd with INT8 dP (delta and row-major dO codes, code "
                                                     "transposes, sbwd_dkdv_kernel<I8DP>, sbwd_dq_kernel<I8DP>)",
                            peak=PEAK_I8_TOPS, peak_note="i8 peak for all five backward products",
                            ops_per_launch=bwd_ops)
    case["traffic_key"] = "sbwd_dkdv_kernel<true>"
    return case


def _sagebwd_qknorm_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import SageQkNormTrainStep, sage_problem, to_device
    import workloads as wl
    Qr, Kr, V, dO = (wl.build(w, t) for t in ("qraw", "kraw", "v", "do"))
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_I8PV, q_block=128,
                     smooth_k=True, smooth_eps=1e-3)
    path = SageQkNormTrainStep(p, to_device(Qr, "bf16"), to_device(Kr, "bf16"), to_device(V, "bf16"),
                               to_device(dO, "bf16"))
    case = _sagebwd_roofline(w)
    case.update(path=path, workload="SageBwd training step with QK-norm fused (c3n): B=1 H=16 N=8192 d=128 causal, "
                                    "raw bf16 Q/K rows normalised inside the INT8 quantiser, K-smoothing eps=1e-3, "
                                    "INT8 forward; backward with the QK-norm backward in the dQ/dK epilogues; step = "
                                    "fused quantise + forward + backward")
    case["roofline"] = dict(case["roofline"], kernel="attn_bwd_qknorm (delta, dO quantiser, code transposes, "
                                                      "sbwd_dkdv_kernel, sbwd_dq_kernel with the norm epilogues)")
    return case


def cpu_baseline_qat_train(w, budget_s: float = 25.0):
    """The oracle on a bounded sample of the Attn-QAT training step:
    quantisation and the whole forward (O, O', log-sum-exp) of head (0,0),
    then the backward for chunks of query rows (dQ) and key rows (dK, dV)
    until the budget."""
    import numpy as np

    import oracle
    import workloads as wl
    from tests.helpers import tau_for
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V, dO = (wl.chunk(w, t, 0, 0) for t in ("q", "k", "v", "do"))
    qc, qs = oracle.quant_mx_rows(Q[None]); kc, ks = oracle.quant_mx_rows(K[None]); vc, vs = oracle.quant_mx_cols(V[None])
    t = dict(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0])
    tau = tau_for(w.d)
    _, Oa, lse, mrow = oracle.qat_fwd(Nq=w.Nq, Nk=w.Nk, d=w.d, tau=tau, kv_tile=64, return_rowmax=True, **t)
    ops = 6.0 * w.Nq * w.Nk * w.d                    # forward: QK^T, P.V and O'
    r0 = 0
    while r0 < w.Nq and time.perf_counter() - t0 < budget_s:
        oracle.qat_bwd(dO=dO, O_aux=oracle.round_to(Oa, "bf16").astype(np.float32), lse=lse.astype(np.float32),
                       rowmax=mrow, Nq=w.Nq, Nk=w.Nk, d=w.d, tau=tau, qrows=(r0, r0 + 32), krows=(r0, r0 + 32), **t)
        ops += 2.0 * 32 * w.Nk * w.d * 3 + 2.0 * 32 * w.Nq * w.d * 4      # dQ rows; dK, dV key rows
        r0 += 32
    dt = time.perf_counter() - t0
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"head (0,0) at N={w.Nk}: MXFP4 quantisation and the full forward with O', then the backward "
                      f"of {r0} query rows (dQ) and {r0} key rows (dK, dV), {dt:.1f} s"}


def _qat_train_case(w, bqa, torch):
    from bit_quantized_attention_amd.runner import QatTrainStep, qat_problem, to_device
    import workloads as wl
    Q, K, V, dO = (wl.build(w, t) for t in ("q", "k", "v", "do"))
    p = qat_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    path = QatTrainStep(p, to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), to_device(dO, "bf16"))
    n = w.B * w.Hq * w.Nq * w.Nk * w.d
    bwd_f4, bwd_b16 = 2.0 * n, 8.0 * n          # S recompute in MXFP4; dP, dV, dQ, dK in 16-bit
    t_peak = bwd_f4 / (PEAK_F4_TFLOPS * 1e12) + bwd_b16 / (PEAK_BF16_TFLOPS * 1e12)
    return dict(
        path=path, ops=14.0 * n, dtype="mxfp4+bf16", timed="backward",
        workload="Attn-QAT training step (c4): B=1 H=32 N=16384 d=128 non-causal, Student-t bf16 in; MXFP4 forward "
                 "with O', backward with P recomputed at the forward's precision and delta' = rowsum(dO o O'); "
                 "step = quantise + forward + backward",
        roofline={"bound": "mfma", "kernel": "attn_bwd QAT (delta', bf16 copies, qbwd_dkdv_kernel, qbwd_dq_kernel)",
                  "peak": round((bwd_f4 + bwd_b16) / t_peak / 1e12, 1),
                  "peak_note": "MXFP4 peak for the score recompute, bf16 (fp16 for dV) peak for the other four",
                  "ops_per_launch": bwd_f4 + bwd_b16},
        traffic_key="qbwd_dkdv_kernel", cpu=cpu_baseline_qat_train)


def probe_main(torch, bqa):
    """Rate probes (bqa_debug_probe): the sustained dense matrix rate per
    operand type, the v_exp_f32 rate and the HBM copy bandwidth, each beside
    the published peak the roofline figures divide by.  Prints one JSON line."""
    dev = torch.device("cuda")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None or t < best else best
        return best

    res = {}
    grid = 4 * n_cu                      # 16 wavefronts per compute unit
    waves = grid * 4
    mm = [("mfma_i8", bqa.BQA_PROBE_MFMA_I8, 65536, PEAK_I8_TOPS, "TOPS"),
          ("mfma_fp8", bqa.BQA_PROBE_MFMA_F8, 131072, PEAK_I8_TOPS, "TFLOP/s"),
          ("mfma_mxfp4", bqa.BQA_PROBE_MFMA_F4, 131072, PEAK_F4_TFLOPS, "TFLOP/s"),
          ("mfma_bf16", bqa.BQA_PROBE_MFMA_BF16, 32768, PEAK_BF16_TFLOPS, "TFLOP/s")]
    iters = 20000
    for name, kind, per, peak, unit in mm:
        t = timed(lambda: bqa.bqa_debug_probe(kind, grid, iters, None, out, out.numel()))
        v = waves * iters * 8 * per / t / 1e12
        res[name] = {"measured": round(v, 1), "peak": peak, "unit": unit, "frac": round(v / peak, 4),
                     "time_ms": round(t * 1e3, 3)}
    it_exp = 100000
    t = timed(lambda: bqa.bqa_debug_probe(bqa.BQA_PROBE_EXP, grid, it_exp, None, out, out.numel()))
    v = grid * 256 * it_exp * 8 / t / 1e12
    # one v_exp_f32 per lane every 8 clocks on each SIMD (8 lanes / clock), 2.4 GHz
    spec = n_cu * 4 * 8 * 2.4e9 / 1e12
    res["v_exp_f32"] = {"measured": round(v, 3), "peak": round(spec, 3), "unit": "T exp/s",
                        "frac": round(v / spec, 4), "time_ms": round(t * 1e3, 3),
                        "peak_note": "8 lanes per clock per SIMD (a wavefront instruction every 8 clocks), "
                                     "4 SIMDs per CU, 2.4 GHz"}
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for name, kind, g in (("hbm_copy", bqa.BQA_PROBE_COPY, 8 * n_cu), ("hbm_copy_wide", bqa.BQA_PROBE_COPY, 32 * n_cu)):
        t = timed(lambda: bqa.bqa_debug_probe(kind, g, 0, src, dst, nbytes))
        v = 2 * nbytes / t / 1e9
        res[name] = {"measured": round(v, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(v / 8000.0, 4),
                     "time_ms": round(t * 1e3, 3), "grid": g, "note": "1 GiB read + 1 GiB written per launch"}
    assert torch.equal(dst[:4096], src[:4096])
    t = timed(lambda: dst.copy_(src))
    v = 2 * nbytes / t / 1e9
    res["hbm_copy_torch"] = {"measured": round(v, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(v / 8000.0, 4),
                             "time_ms": round(t * 1e3, 3), "note": "torch copy_ of the same buffers"}
    for name, g in (("hbm_read", 8 * n_cu), ("hbm_read_wide", 32 * n_cu)):
        t = timed(lambda: bqa.bqa_debug_probe(bqa.BQA_PROBE_READ, g, 0, src, out, nbytes))
        v = nbytes / t / 1e9
        res[name] = {"measured": round(v, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(v / 8000.0, 4),
                     "time_ms": round(t * 1e3, 3), "grid": g, "note": "1 GiB read per launch"}
    del src, dst
    torch.cuda.empty_cache()
    # 4 GiB, default and non-temporal policy (the decode kernel's copies are non-temporal)
    big = 4 << 30
    src = torch.ones(big, dtype=torch.uint8, device=dev)
    for name, kind in (("hbm_read_4g", bqa.BQA_PROBE_READ), ("hbm_read_nt", bqa.BQA_PROBE_READ_NT)):
        g = 8 * n_cu
        t = timed(lambda: bqa.bqa_debug_probe(kind, g, 0, src, out, big))
        v = big / t / 1e9
        res[name] = {"measured": round(v, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(v / 8000.0, 4),
                     "time_ms": round(t * 1e3, 3), "grid": g,
                     "note": "4 GiB read per launch" + (", non-temporal cache policy" if "nt" in name else "")}
    del src
    torch.cuda.empty_cache()
    # vector work under matrix work: time per round of each mix, 2 wavefronts per SIMD
    g2, it2 = 2 * n_cu, 20000
    iss = {}
    for name, kind in (("mfma", bqa.BQA_PROBE_ISSUE_MFMA), ("fma", bqa.BQA_PROBE_ISSUE_FMA),
                       ("mfma_fma", bqa.BQA_PROBE_ISSUE_MFMA_FMA), ("exp", bqa.BQA_PROBE_ISSUE_EXP),
                       ("mfma_exp", bqa.BQA_PROBE_ISSUE_MFMA_EXP)):
        t = timed(lambda: bqa.bqa_debug_probe(kind, g2, it2, None, out, out.numel()))
        iss[name] = t / it2 / 2 * 1e9                   # ns of SIMD time per wavefront round
    res["issue_overlap"] = {
        "unit": "ns per wavefront round (SIMD time, 2 wavefronts per SIMD)",
        "round": "8 i8 32x32x32 matrix instructions / 64 fp32 multiply-adds / 32 v_exp_f32, or the matrix "
                 "instructions interleaved with either",
        **{k: round(v, 2) for k, v in iss.items()},
        "hidden_fma_share": round((iss["mfma"] + iss["fma"] - iss["mfma_fma"]) / min(iss["mfma"], iss["fma"]), 3),
        "hidden_exp_share": round((iss["mfma"] + iss["exp"] - iss["mfma_exp"]) / min(iss["mfma"], iss["exp"]), 3),
        "note": "hidden share = (separate sum - mixed) / the shorter part: 1 if the shorter part runs entirely "
                "under the longer one, 0 if the two only add up"}
    # vector work under vector work: the multiply-adds and exponentials of a round interleaved
    t = timed(lambda: bqa.bqa_debug_probe(bqa.BQA_PROBE_ISSUE_EXP_FMA, g2, it2, None, out, out.numel()))
    ef = t / it2 / 2 * 1e9
    res["vector_overlap"] = {
        "unit": "ns per wavefront round (SIMD time, 2 wavefronts per SIMD)",
        "round": "64 fp32 multiply-adds and 32 v_exp_f32 on independent chains, interleaved",
        "fma": round(iss["fma"], 2), "exp": round(iss["exp"], 2), "fma_exp": round(ef, 2),
        "hidden_share": round((iss["fma"] + iss["exp"] - ef) / min(iss["fma"], iss["exp"]), 3)}
    # LDS: 16-byte reads with every 16-lane group on its own span, or the four groups on one set of rows
    lds = {}
    for name, kind in (("spans", bqa.BQA_PROBE_LDS_SPANS), ("shared_rows", bqa.BQA_PROBE_LDS_SHARED_ROWS)):
        t = timed(lambda: bqa.bqa_debug_probe(kind, g2, 20000, None, out, out.numel()))
        lds[name] = round(t / 20000 / 8 / 2 * 1e9, 3)      # per wavefront read, 2 wavefronts per SIMD
    res["lds_read_b128"] = {
        "unit": "ns per wavefront 16-byte read (SIMD time, 2 wavefronts per SIMD, 8 reads per round)",
        "layouts": "spans: lane 16 g + q reads entry q of group g's own 256-byte span; shared_rows: chunk "
                   "g ^ (q / 4) of 64-byte row q (the four groups read different chunks of the same rows); "
                   "every group of 16 lanes covers all 64 banks in both",
        **lds, "ratio": round(lds["shared_rows"] / lds["spans"], 3)}
    # issue cost of single vector instructions: ns of SIMD time per wavefront instruction
    ops = {}
    for name, kind in (("v_mul_f32", bqa.BQA_PROBE_OP_MUL), ("v_fma_f32", bqa.BQA_PROBE_OP_FMA),
                       ("v_cvt_f32_i32", bqa.BQA_PROBE_OP_CVT_F32_I32), ("v_max3_f32", bqa.BQA_PROBE_OP_MAX3),
                       ("v_cvt_pk_fp8_f32", bqa.BQA_PROBE_OP_CVT_PK_FP8),
                       ("v_cvt_scalef32_pk_fp4_f32", bqa.BQA_PROBE_OP_CVT_PK_FP4),
                       ("v_permlane32_swap", bqa.BQA_PROBE_OP_PERMLANE32)):
        t = timed(lambda: bqa.bqa_debug_probe(kind, g2, 2000, None, out, out.numel()))
        ops[name] = round(t / 2000 / 2 / 64 * 1e9, 3)
    ops["v_exp_f32"] = round(iss["exp"] / 32, 3)
    res["instruction_issue"] = {"unit": "ns of SIMD time per wavefront instruction (2 wavefronts per SIMD, 16 "
                                        "independent chains per lane)", **ops}
    print(json.dumps({"probes": res, "compute_units": n_cu, "grid_matrix": grid, "iters_matrix": iters}), flush=True)


CASES = {"c2": _sage_case, "c3": _sagebwd_case, "c3i": _sagebwd_i8dp_case, "c3n": _sagebwd_qknorm_case, "c4": _qat_case, "c4t": _qat_train_case, "c4i": _qat_infer_case,
         "c4p": _ptq_case, "c5": _thrift_case, "c5d": _decode_case}
INPUTS_OF = {"c3i": "c3", "c3n": "c3", "c4t": "c4", "c4i": "c4", "c4p": "c4"}        # workloads that reuse another's inputs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps; 0 (default): enough for about 0.1 s, at least 10")
    ap.add_argument("--warmup", type=int, default=0,
                    help="untimed warmup steps; the warmup runs at least this many steps and at least 0.5 s "
                         "(and 20 steps), which brings the GPU clocks up from idle; the JSON line reports "
                         "the number actually run")
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="minimum warmup time (profiler runs pass 0 to keep the number of dispatches small)")
    ap.add_argument("--workload", choices=sorted(CASES), default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe", action="store_true",
                    help="only run the rate probes (matrix rate per type, v_exp_f32, HBM copy) and print them "
                         "beside the published peaks")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(every kernel is independent per (batch, head), so the path shards by heads; "
              f"this benchmark measures one GPU's share)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_attention_amd as bqa
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    if args.probe:
        probe_main(torch, bqa)
        return
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "launches": 5}))
        return
    w = wl.WORKLOADS[INPUTS_OF.get(args.workload, args.workload)]
    case = CASES[args.workload](w, bqa, torch)
    path = case["path"]
    t_w = time.perf_counter()
    n_warm = 0
    warm_req = args.warmup
    min_steps = 20 if args.warmup_seconds > 0 else 1
    while n_warm < warm_req or n_warm < min_steps or time.perf_counter() - t_w < args.warmup_seconds:
        path.step()
        n_warm += 1
        if n_warm % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    args.warmup = n_warm
    if args.steps <= 0:
        est = (time.perf_counter() - t_w) / n_warm
        args.steps = int(min(1000, max(10, round(0.1 / est))))

    stream = torch.cuda.current_stream()
    # the timed kernel is bracketed by HIP events on its stream in every
    # `every`-th step (about 64 samples): each event is a marker the command
    # processor handles between kernels, and one pair per step would add
    # several microseconds to every step of a 0.1 ms workload
    every = max(1, args.steps // 64)
    n_ev = (args.steps + every - 1) // every
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timed_bwd = case.get("timed") == "backward"
    for i in range(args.steps):
        sample = i % every == 0
        path.quantize()
        if timed_bwd:
            path.forward()
        if sample:
            ev[i // every][0].record(stream)
        if timed_bwd:
            path.backward()
        else:
            path.forward()
        if sample:
            ev[i // every][1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / n_ev

    ops = case["ops"]
    ms_per_step = dt * 1e3 / args.steps
    value = ops / (ms_per_step * 1e-3) / 1e12
    rl = dict(case["roofline"])
    if rl["bound"] == "hbm":
        achieved = rl["bytes_per_launch"] / (kern_ms * 1e-3) / 1e9
    else:
        achieved = rl["ops_per_launch"] / (kern_ms * 1e-3) / 1e12
        rl["unit"] = "TFLOP/s"
    rl.update({"achieved": round(achieved, 1), "frac": round(achieved / rl["peak"], 4),
               "traffic": _traffic_for(case["traffic_key"]), "kernel_ms": round(kern_ms, 5)})
    # the probes' sustained rates of the same units, beside the published peak
    probes = {"hbm": ["hbm_read_wide", "hbm_read_nt"],
              "mfma": ["mfma_i8", "mfma_fp8", "mfma_mxfp4", "mfma_bf16"]}[rl["bound"]]
    mp = _measured_peak(probes)
    if mp is not None:
        rl["probe_rates"] = mp
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_rule": f"at least {warm_req} steps (requested), {min_steps} steps and {args.warmup_seconds} s",
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case["dtype"],
        "data": "synthetic",
        "config": {"workload": case["workload"], "global_batch": w.B, "seq_len": w.Nk, "heads": w.Hq,
                   "head_dim": w.d, "parallelism": "single GPU"},
        "roofline": rl,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = case["cpu"](w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
