"""Benchmark of the block-quantized attention hot path on one MI355X.

Default workload: the SageAttention INT8 forward at B=2, H=16, N=4096,
d=128, causal, bf16 inputs (outlier channels and a K channel bias), INT8
Q/K with K-smoothing, e4m3 P.V.  One step = one pass of the whole path over
the batch: K-smoothing means, INT8 quantisation of Q and K, per-channel e4m3
V, and the fused attention kernel.  Inputs are generated on the host and are
resident in HBM before timing starts.

Prints one JSON line.  `value` is effective attention TOPS of the whole step
(4*B*H*N^2*d, halved for causal, over the step time).  `roofline` reports the
attention kernel alone: its algorithmic ops per launch over its average
launch time, measured with HIP events on the stream it runs on, against the
i8/fp8 dense MFMA peak.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
METRIC = "attention TOPS (fwd, fwd+bwd) at d=128, N=4k-131k; % of i8/fp8/fp4 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _traffic_for(kernel: str):
    """Measured HBM bytes per launch of `kernel` from the committed counter
    summary, if it was taken on the current kernel source."""
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
    return e["bytes_per_launch"]


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(every kernel is independent per (batch, head); sharding is described in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_attention_amd as bqa
    import workloads as wl
    from bit_quantized_attention_amd.runner import SagePath, attention_ops, sage_problem, to_device

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "launches": 5}))
        return
    w = wl.WORKLOADS["c2"]
    Q, K, V = wl.build(w, "q"), wl.build(w, "k"), wl.build(w, "v")
    p = sage_problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, bqa.BQA_SAGE_I8_F8PV, q_block=128,
                     smooth_k=True, smooth_eps=0.0)
    path = SagePath(p, to_device(Q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype))
    del Q, K, V
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        path.quantize()
        ev[i][0].record(stream)
        path.forward()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps

    ops = attention_ops(p)
    ms_per_step = dt * 1e3 / args.steps
    value = ops / (ms_per_step * 1e-3) / 1e12
    achieved = ops / (kern_ms * 1e-3) / 1e12
    traffic = _traffic_for("sage_fwd_kernel<F8,128,causal>")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+e4m3",
        "data": "synthetic",
        "config": {"workload": "SageAttention INT8 forward (c2): B=2 H=16 N=4096 d=128 causal, bf16 in, "
                               "K-smoothing, INT8 Q/K, e4m3 P.V; step = quantise Q,K,V + attention",
                   "global_batch": w.B, "seq_len": w.Nk, "heads": w.Hq, "head_dim": w.d,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "sage_fwd_kernel (i8 QK^T + fp8 P.V)",
                     "achieved": round(achieved, 1), "peak": PEAK_I8_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_I8_TOPS, 4), "traffic": traffic,
                     "kernel_ms": round(kern_ms, 5), "ops_per_launch": ops},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
