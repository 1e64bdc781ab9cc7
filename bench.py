#!/usr/bin/env python3
"""Decode-step throughput of the TiDAR hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
36 layers of hybrid-mask attention (Qwen3-8B shape: 32 query heads, 8 KV
heads, head_dim 128, prefix P = 4096, k = 16 drafts, 17 pre-draft blocks of
16 mask tokens, 288 query rows), rejection sampling over a 151936-token
vocabulary, and the KV commit of the accepted drafts. Inputs are resident in
HBM before timing starts; every step re-reads the full 36-layer KV cache.

Prints one JSON line (see the keys below). `--gpus N` with N > 1 exits: this
build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid-mask decode steps/sec and KV-read HBM GB/s (% of peak) at P=4096,k=16"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0

# HBM traffic of one attention launch (main kernel + split merge), from
# rocprofv3 FETCH_SIZE / WRITE_SIZE passes scaled by the same counters' reading
# on a device copy of known size. Valid only for the attention source it was
# taken on (sha256 prefix of csrc/attn.hip); any other source reports null.
ATTN_TRAFFIC = {
    "b935db2740045bbe": 57081768,
}

SHAPE = dict(layers=36, batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, P=4096, k=16,
             vocab=151936)


def algorithmic_counts(L, B, Hq, Hkv, D, P, k, V):
    """Algorithmic bytes and FLOPs of one step (no re-reads, no partials)."""
    R = k + (k + 1) * k
    local_pairs = k * (k + 1) // 2 + sum(k * (j + k) for j in range(k + 1))   # visible step keys
    e = 2  # bf16
    attn_flops_layer = 4 * Hq * D * (R * P + local_pairs) * B
    kv_prefix = 2 * Hkv * P * D * e * B
    kv_step = 2 * R * Hkv * D * e * B
    qo = 2 * R * Hq * D * e * B
    return dict(R=R, attn_flops_layer=attn_flops_layer, kv_prefix_layer=kv_prefix, kv_step_layer=kv_step,
                qo_layer=qo, attn_bytes_layer=kv_prefix + kv_step + qo,
                sampler_bytes=(2 * k + 1) * V * 4 * B)


def attn_source_digest() -> str:
    import hashlib

    path = os.path.join(ROOT, "ar_self_speculative_amd", "csrc", "attn.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def copy_calibration(mib: int) -> None:
    """Device-to-device copies of a known size, for scaling HBM byte counters."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def cpu_baseline(seconds: float = 8.0) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from tidar_synth import commit_accept_lengths, config_attn, config_sampler

    c = config_attn(3, seed=0, layers=1, poison=False)
    R, Hq = c.rows, c.num_q_heads
    rng = np.random.default_rng(0)
    rows, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds or rows < 32:
        batch = [(0, int(rng.integers(R)), int(rng.integers(Hq))) for _ in range(16)]
        oracle.attn_rows(c.q[0], c.k_step[0], c.v_step[0], c.k_cache[0], c.v_cache[0], c.cache_len, batch,
                         k=c.k, num_blocks=c.num_blocks, block_len=c.block_len, sm_scale=c.sm_scale)
        rows += len(batch)
    t_row = (time.perf_counter() - t0) / rows
    sc = config_sampler(3, seed=0)
    t1 = time.perf_counter()
    oracle.reject_sample(sc.ar_logits, sc.diff_logits, sc.drafts, sc.uniforms)
    t_samp = time.perf_counter() - t1
    L, Hkv, D, cap = 36, c.num_kv_heads, c.head_dim, c.cache_capacity
    ks = np.zeros((L, 1, R, Hkv, D), np.uint16)
    kc = np.zeros((L, 1, Hkv, cap, D), np.uint16)
    t2 = time.perf_counter()
    oracle.kv_commit(ks, ks, kc, kc, commit_accept_lengths(1, c.k, 0), c.cache_len)
    t_commit = time.perf_counter() - t2
    t_step = L * R * Hq * t_row + t_samp + t_commit
    threads = 1
    for info in threadpool_info():
        if info.get("internal_api") in ("openblas", "mkl", "blis"):
            threads = max(threads, int(info.get("num_threads", 1)))
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"{rows} attention rows (b,r,h) of one Qwen3-8B layer at P=4096 "
                       f"({t_row * 1e3:.2f} ms/row, scaled to 36 layers x {R * Hq} rows), one full sampler "
                       f"call at V=151936 k=16 ({t_samp:.2f} s), one 36-layer commit ({t_commit:.3f} s)")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="force the prefix split count (0 = library plan)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run three device copies of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path is measured on a "
              "single MI355X and multi-GPU sharding is not part of this build.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import ar_self_speculative_amd as tidar
    from tidar_synth import fill_device_step

    s = SHAPE
    torch.cuda.set_device(0)
    step = tidar.DecodeStep(layers=s["layers"], batch=s["batch"], num_q_heads=s["num_q_heads"],
                            num_kv_heads=s["num_kv_heads"], head_dim=s["head_dim"], k=s["k"],
                            cache_capacity=s["P"] + s["k"], max_cache_len=s["P"], vocab=s["vocab"],
                            num_splits=args.splits)
    fill_device_step(step, seed=0, cache_len=s["P"])
    torch.cuda.synchronize()

    # The step is replayed from a HIP graph (one host launch per step): the
    # host cost of issuing 75 library calls would otherwise show up in the
    # GPU timeline once the kernels are fast.
    for _ in range(args.warmup):
        step.run()
    graph = step.capture()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    # Average duration of one attention launch (main kernel + split merge):
    # HIP events on the launch stream around a graph of the 36 layers'
    # attention calls, replayed back to back.
    attn_graph = step.capture(lambda: [step.attention(layer) for layer in range(s["layers"])])
    reps = max(1, min(args.steps, 10))
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    attn_graph.replay()
    a0.record()
    for _ in range(reps):
        attn_graph.replay()
    a1.record()
    torch.cuda.synchronize()
    attn_ms = a0.elapsed_time(a1) / (reps * s["layers"])
    status = int(step.dev_status.item())
    if status:
        print(f"device status flags set: {status}", file=sys.stderr)
        sys.exit(1)

    cnt = algorithmic_counts(s["layers"], s["batch"], s["num_q_heads"], s["num_kv_heads"], s["head_dim"],
                             s["P"], s["k"], s["vocab"])
    t_step = ms_step * 1e-3
    kv_bytes = s["layers"] * (cnt["kv_prefix_layer"] + cnt["kv_step_layer"])
    kv_gbps = kv_bytes / t_step / 1e9
    achieved_tflops = cnt["attn_flops_layer"] / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(1.0 / t_step, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b-shape 36-layer TiDAR decode step, batch 1, P=4096, k=16 "
                               "(288 query rows), vocab 151936",
                   "batch": s["batch"], "layers": s["layers"], "q_heads": s["num_q_heads"],
                   "kv_heads": s["num_kv_heads"], "head_dim": s["head_dim"], "prefix": s["P"], "k": s["k"],
                   "query_rows": cnt["R"], "vocab": s["vocab"]},
        "kv_read_gbps": round(kv_gbps, 1),
        "kv_read_frac_of_hbm_peak": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "attn_us_per_layer": round(attn_ms * 1e3, 2),
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel<128> (+ split merge)",
                     "achieved": round(achieved_tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": ATTN_TRAFFIC.get(attn_source_digest()),
                     "flops_per_launch": cnt["attn_flops_layer"]},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
