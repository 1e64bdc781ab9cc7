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

import numpy as np

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
    "9f896ed05fd7059d": 57159857,
}

# MFMA utilisation of the main attention kernel at this workload, from a
# rocprofv3 --pmc pass (SQ_VALU_MFMA_BUSY_CYCLES over 1024 * GRBM_GUI_ACTIVE / 8
# XCDs), beside the same ratio for the MFMA-only ceiling kernel (a dependent
# chain of v_mfma_f32_32x32x16_bf16, 96.7%). Keyed like ATTN_TRAFFIC; any other
# attention source reports null.
ATTN_COUNTERS = {
    "9f896ed05fd7059d": {"mfma_busy_frac": 0.2807, "ceiling_kernel_mfma_busy_frac": 0.9665,
                         "mfma_busy_frac_of_ceiling": 0.2904, "valu_insts_per_mfma": 5.74,
                         "mfma_coexec_frac": 0.4337, "wave_cycles_waiting_on_dependencies": 0.3364},
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
    """The fp64 oracle, as it stands, on a bounded sample of the same workload
    (all of the host's cores for the BLAS calls, then one core)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

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
    # the attention rows again with the BLAS pools held to one thread
    with threadpool_limits(limits=1):
        rows1, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds / 2 or rows1 < 16:
            batch = [(0, int(rng.integers(R)), int(rng.integers(Hq))) for _ in range(16)]
            oracle.attn_rows(c.q[0], c.k_step[0], c.v_step[0], c.k_cache[0], c.v_cache[0], c.cache_len, batch,
                             k=c.k, num_blocks=c.num_blocks, block_len=c.block_len, sm_scale=c.sm_scale)
            rows1 += len(batch)
        t_row1 = (time.perf_counter() - t0) / rows1
    t_step1 = L * R * Hq * t_row1 + t_samp + t_commit
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "value_1core": 1.0 / t_step1,
            "sample": (f"{rows} attention rows (b,r,h) of one Qwen3-8B layer at P=4096 "
                       f"({t_row * 1e3:.2f} ms/row, scaled to 36 layers x {R * Hq} rows), one full sampler "
                       f"call at V=151936 k=16 ({t_samp:.2f} s), one 36-layer commit ({t_commit:.3f} s)")}


def _rand_bf16(shape, gen):
    import torch

    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def _time_graph(g, reps: int) -> float:
    """Milliseconds per replay of graph g (HIP events on the launch stream)."""
    import torch

    g.replay()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def _capture(fn):
    import torch

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def ceilings_bench(args) -> dict:
    """Measured machine ceilings: HBM streaming read, bf16 MFMA rate, fp32
    exponential and FMA issue rates, LDS read rates (ds_read_b128 and the
    transposing ds_read_b64_tr_b16), and the cost of an empty kernel launched
    back to back (from a graph and from the stream). Each kernel is timed with
    HIP events on the stream it is launched on."""
    import torch

    import ar_self_speculative_amd as tidar

    dev = torch.device("cuda")
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3  # seconds per call

    out = {}
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    hbm = {}
    for grid in (1024, 2048, 4096, 8192):
        t = timed(lambda: tidar.ceiling("hbm_read", buf, grid, sink), 5)
        hbm[str(grid)] = round(nbytes / t / 1e9, 1)
    del buf
    out["hbm_read_gbps_by_grid"] = hbm
    out["hbm_read_gbps"] = max(hbm.values())
    out["hbm_read_bytes"] = nbytes
    grid, iters = 1024, 20000
    t = timed(lambda: tidar.ceiling("mfma_bf16", grid, iters, sink), 3)
    flops = grid * 4 * 4 * iters * 32768
    out["mfma_bf16_tflops"] = round(flops / t / 1e12, 1)
    # the nominal 2.5 PFLOP/s is 256 CUs x 4 SIMDs x 1024 flops per cycle at 2.4 GHz
    out["mfma_implied_clock_ghz"] = round(flops / t / (1024 * 1024) / 1e9, 3)
    grid, iters = 2048, 20000
    n = grid * 256 * 8 * iters
    t_exp = timed(lambda: tidar.ceiling("exp_f32", grid, iters, sink), 3)
    t_fma = timed(lambda: tidar.ceiling("fma_f32", grid, iters, sink), 3)
    out["exp_f32_gops"] = round(n / t_exp / 1e9, 1)
    out["fma_f32_gops"] = round(n / t_fma / 1e9, 1)
    # cycles one SIMD spends per wave64 instruction, at the clock implied by the MFMA run
    clk = out["mfma_implied_clock_ghz"] * 1e9
    out["exp_f32_cycles_per_wave_instr"] = round(1024 * clk * 64 / (n / t_exp), 2)
    out["fma_f32_cycles_per_wave_instr"] = round(1024 * clk * 64 / (n / t_fma), 2)
    # LDS reads: two 256-thread workgroups per CU (8 waves), bytes per clock
    # per CU at the clock implied by the MFMA run
    grid, iters = 512, 4096
    for kind, lane_bytes in (("lds_read_b128", 16), ("lds_read_tr16", 8)):
        t = timed(lambda: tidar.ceiling(kind, grid, iters, sink), 3)
        nb = grid * 256 * 8 * iters * lane_bytes
        out[f"{kind}_tbps"] = round(nb / t / 1e12, 1)
        out[f"{kind}_bytes_per_clk_per_cu"] = round(nb / t / (256 * clk), 1)
    for grid in (1, 512):
        def many():
            for _ in range(100):
                tidar.ceiling("empty", grid)
        g = _capture(many)
        out[f"empty_kernel_us_graph_grid{grid}"] = round(_time_graph(g, 5) * 1e3 / 100, 3)
        out[f"empty_kernel_us_stream_grid{grid}"] = round(timed(many, 3) * 1e6 / 100, 3)
    return out


def sampler_bench(args) -> None:
    """The sampler alone (tidar_reject_sample) at one shape, B:k[:V] (V
    defaults to the Qwen3 vocabulary 151936): 50 calls captured in a HIP
    graph and replayed, HIP events on the launch stream. Inputs are the
    sampler recipe drawn on the device (AR logits ~ N(0, 3), diffusion logits
    = AR + N(0, 0.162), drafts by Gumbel-max from the diffusion logits).
    Reports microseconds per call and the logit bytes the statistics pass
    must read ((2k+1) V fp32 rows per sequence) per call time."""
    import torch

    import ar_self_speculative_amd as tidar
    from tidar_synth import fill_verifier_device

    parts = [int(x) for x in args.sampler.split(":")]
    B, k = parts[0], parts[1]
    V = parts[2] if len(parts) > 2 else 151936
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    ar = torch.empty(B, k + 1, V, dtype=torch.float32, device=dev)
    diff = torch.empty(B, k, V, dtype=torch.float32, device=dev)
    drafts = torch.empty(B, k, dtype=torch.int32, device=dev)
    uni = torch.empty(B, k + 1, dtype=torch.float32, device=dev)
    fill_verifier_device(ar, diff, drafts, uni, g, ar_sigma=3.0, diff_sigma=0.162)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(tidar.reject_workspace_bytes(B, k, V), dtype=torch.uint8, device=dev)

    def call():
        tidar.reject_sample(ar_logits=ar, diff_logits=diff, drafts=drafts, uniforms=uni, accept_len=acc,
                            next_token=nxt, dev_status=status, workspace=ws)

    for _ in range(max(1, args.warmup)):
        call()
    calls = 50
    graph = _capture(lambda: [call() for _ in range(calls)])
    us = _time_graph(graph, max(1, args.steps // 5)) * 1e3 / calls
    if int(status.item()):
        print(f"device status flags set: {int(status.item())}", file=sys.stderr)
        sys.exit(1)
    logit_bytes = B * (2 * k + 1) * V * 4
    print(json.dumps({
        "metric": "sampler call time (tidar_reject_sample)", "value": round(us, 2), "unit": "us/call",
        "higher_is_better": False, "n_gpus": 1, "data": "synthetic", "dtype": "f32",
        "config": {"workload": f"rejection sampling, batch {B}, k={k}, vocab {V}", "batch": B, "k": k, "vocab": V},
        "logit_bytes": logit_bytes, "logit_read_gbps": round(logit_bytes / (us * 1e-6) / 1e9, 1),
        "mean_accept_len": round(float(acc.float().mean().item()), 3),
    }), flush=True)


def config5_bench(args) -> None:
    """Ragged batch at full depth: 8 sequences with prefixes from U{256..4096},
    k = 8 (80 query rows), 36 Qwen3-8B-shaped layers, 64 chained steps
    (attention of every layer -> sampler -> commit, each step attending over
    the prefixes the earlier steps grew). Every step's inputs are drawn on the
    device beforehand; the 64 steps are captured in one graph and timed with
    HIP events on the launch stream. The two cache-length buffers alternate,
    so no copy sits between steps."""
    import torch

    import ar_self_speculative_amd as tidar
    from tidar_synth import CONFIGS, config5_lengths, fill_device_step, fill_verifier_device

    c = CONFIGS[5]
    L, B, k, cap, n_steps = c["layers"], c["batch"], c["k"], c["cap"], c["steps"]
    Hq, Hkv, D, V = c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["vocab"]
    sigma = c["sampler"]["diff_sigma"]
    lens0 = config5_lengths(0)
    W = k * n_steps
    step = tidar.DecodeStep(layers=L, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, k=k,
                            cache_capacity=cap, max_cache_len=int(lens0.max()) + W, vocab=V,
                            num_splits=args.splits)
    R = step.R
    fill_device_step(step, seed=5, cache_len=lens0)
    dev = step.q.device
    g = torch.Generator(device=dev).manual_seed(77)
    bf = lambda shape: torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ins = []
    for _ in range(n_steps):
        d = dict(q=bf((L, B, R, Hq, D)), ks=bf((L, B, R, Hkv, D)), vs=bf((L, B, R, Hkv, D)),
                 ar=torch.empty((B, k + 1, V), device=dev), diff=torch.empty((B, k, V), device=dev),
                 drafts=torch.empty((B, k), dtype=torch.int32, device=dev),
                 u=torch.empty((B, k + 1), device=dev),
                 acc=torch.zeros(B, dtype=torch.int32, device=dev),
                 nxt=torch.zeros(B, dtype=torch.int32, device=dev),
                 ratio=torch.zeros((B, k), device=dev))
        fill_verifier_device(d["ar"], d["diff"], d["drafts"], d["u"], g, ar_sigma=3.0, diff_sigma=sigma)
        ins.append(d)
    lens = [torch.from_numpy(lens0.copy()).to(dev), torch.empty(B, dtype=torch.int32, device=dev)]
    status = step.dev_status

    def run_steps():
        for s_, d in enumerate(ins):
            lin, lout = lens[s_ % 2], lens[(s_ + 1) % 2]
            for layer in range(L):
                tidar.attn_step(step.desc, d["q"][layer], d["ks"][layer], d["vs"][layer], step.k_cache[layer],
                                step.v_cache[layer], lin, step.out[layer], None, status, step.attn_ws)
            tidar.reject_sample(ar_logits=d["ar"], diff_logits=d["diff"], drafts=d["drafts"], uniforms=d["u"],
                                accept_len=d["acc"], next_token=d["nxt"], ratio=d["ratio"], dev_status=status,
                                workspace=step.rej_ws)
            tidar.kv_commit(num_layers=L, batch=B, num_kv_heads=Hkv, head_dim=D, k=k, step_rows=R,
                            cache_capacity=cap, max_cache_len=step.max_len, dtype=tidar.DTYPE_BF16,
                            k_step=d["ks"], v_step=d["vs"], k_cache=step.k_cache, v_cache=step.v_cache,
                            accept_len=d["acc"], cache_len_in=lin, cache_len_out=lout, dev_status=status)

    reset = lambda: lens[0].copy_(torch.from_numpy(lens0.copy()).to(dev))
    run_steps()                                       # eager warm-up pass
    reset()
    graph = _capture(run_steps)
    times = []
    for _ in range(max(1, args.steps if args.steps < 10 else 3)):
        reset()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) * 1e-3)
    t = sorted(times)[len(times) // 2]
    if int(status.item()):
        print(f"device status flags set: {int(status.item())}", file=sys.stderr)
        sys.exit(1)
    acc = torch.stack([d["acc"] for d in ins]).cpu().numpy()          # [steps, B]
    ratio = torch.stack([d["ratio"] for d in ins]).cpu().numpy()
    uu = torch.stack([d["u"] for d in ins]).cpu().numpy()
    committed = acc + 1
    # acceptance tests within 1e-5 of their threshold (by the GPU's own ratios), among those consulted
    near = 0
    for s_ in range(n_steps):
        for b in range(B):
            n = int(acc[s_, b])
            tested = np.arange(min(n + 1, k))
            near += int(np.any(np.abs(uu[s_, b, tested] - np.minimum(1.0, ratio[s_, b, tested])) < 1e-5))
    # algorithmic bytes and flops, from the lengths each step attended over
    local = k * (k + 1) // 2 + sum(k * (j + k) for j in range(k + 1))
    lens_at = lens0[None, :] + np.concatenate([np.zeros((1, B), np.int64), np.cumsum(acc, axis=0)[:-1]])
    e = 2
    kv_bytes = float(L * (2 * Hkv * D * e * lens_at.sum() + n_steps * B * 2 * R * Hkv * D * e))
    qo_bytes = float(L * n_steps * B * 2 * R * Hq * D * e)
    samp_bytes = float(n_steps * B * (2 * k + 1) * V * 4)
    commit_bytes = float(2 * 2 * L * acc.sum() * Hkv * D * e)
    flops = float(L * 4 * Hq * D * (R * lens_at.sum() + n_steps * B * local))
    all_bytes = kv_bytes + qo_bytes + samp_bytes + commit_bytes
    t_hbm, t_mfma = all_bytes / (HBM_PEAK_GBPS * 1e9), flops / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    print(json.dumps({
        "metric": "ragged-batch TiDAR decode steps/sec (8 sequences, k=8, 36 layers, 64 chained steps)",
        "value": round(n_steps / t, 2), "unit": "steps/s", "n_gpus": 1, "steps": n_steps, "higher_is_better": True,
        "ms_per_step": round(t / n_steps * 1e3, 4), "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3-8b-shape ragged batch: 8 sequences, prefixes U{256..4096}, k=8 (80 query "
                               "rows), 36 layers, vocab 151936, 64 chained steps",
                   "batch": B, "layers": L, "k": k, "query_rows": R, "prefix_lengths": lens0.tolist(),
                   "diff_sigma": sigma},
        "tokens_per_s": round(float(committed.sum()) / t, 1),
        "tokens_per_step_mean": round(float(committed.mean()), 3),
        "tokens_per_step_hist": np.bincount(committed.ravel(), minlength=k + 2)[1:].tolist(),
        "accept_near_ties": near,
        "hbm_gbps_algorithmic": round(all_bytes / t / 1e9, 1),
        "kv_read_gbps": round(kv_bytes / t / 1e9, 1),
        "mfma_tflops_algorithmic": round(flops / t / 1e12, 1),
        "roofline": {"bound": "hbm" if t_hbm > t_mfma else "mfma",
                     "frac": round(max(t_hbm, t_mfma) / t, 4), "t_hbm_s": t_hbm, "t_mfma_s": t_mfma,
                     "bytes": all_bytes, "flops": flops},
    }), flush=True)


def likelihood_bench(args) -> None:
    """Likelihood mode: one causal forward scoring R tokens after a prefix P
    (36 attention layers with num_blocks = 0, then the log-probabilities of
    the R next tokens over the vocabulary)."""
    import math

    import torch

    import ar_self_speculative_amd as tidar

    s = SHAPE
    L, Hq, Hkv, D, P, V = s["layers"], s["num_q_heads"], s["num_kv_heads"], s["head_dim"], s["P"], s["vocab"]
    R = args.likelihood
    gen = torch.Generator(device="cuda").manual_seed(0)
    desc = tidar.make_attn_desc(batch=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, k=R, num_blocks=0,
                                block_len=1, cache_capacity=P + R, max_cache_len=P, sm_scale=1 / math.sqrt(D),
                                dtype=tidar.DTYPE_BF16)
    q = _rand_bf16((L, 1, R, Hq, D), gen)
    ks, vs = _rand_bf16((L, 1, R, Hkv, D), gen), _rand_bf16((L, 1, R, Hkv, D), gen)
    kc, vc = _rand_bf16((L, 1, Hkv, P + R, D), gen), _rand_bf16((L, 1, Hkv, P + R, D), gen)
    lens = torch.full((1,), P, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = tidar.attn_workspace(desc, torch.device("cuda"))
    logits = torch.randn((R, V), generator=gen, device="cuda", dtype=torch.float32) * 3.0
    targets = torch.randint(0, V, (R,), generator=gen, device="cuda", dtype=torch.int32)
    lp = torch.empty(R, dtype=torch.float32, device="cuda")
    lws = torch.empty(tidar.logprob_workspace_bytes(R, V), dtype=torch.uint8, device="cuda")

    def attention():
        for l in range(L):
            tidar.attn_step(desc, q[l], ks[l], vs[l], kc[l], vc[l], lens, out[l], None, status, ws)

    def scores():
        tidar.token_logprobs(logits=logits, targets=targets, logprobs=lp, workspace=lws, dev_status=status)

    for _ in range(args.warmup):
        attention()
        scores()
    g_all = _capture(lambda: (attention(), scores()))
    g_lp = _capture(scores)
    ms = _time_graph(g_all, args.steps)
    ms_lp = _time_graph(g_lp, args.steps)
    if int(status.item()):
        print(f"device status flags set: {int(status.item())}", file=sys.stderr)
        sys.exit(1)
    lp_gbps = R * V * 4 / (ms_lp * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"likelihood-mode scored tokens/s (one causal forward: {L} attention layers + log-probs) "
                  f"at P={P},R={R}",
        "value": round(R / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_forward": round(ms, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"qwen3-8b-shape causal scoring forward, batch 1, prefix {P}, {R} scored tokens, "
                               f"vocab {V}", "layers": L, "prefix": P, "rows": R, "vocab": V},
        "logprob_us": round(ms_lp * 1e3, 2),
        "logprob_roofline": {"bound": "hbm", "achieved": round(lp_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(lp_gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": R * V * 4},
    }), flush=True)


def knee_ceilings() -> dict:
    """The two ceilings the free-slot knee is computed from, measured on this machine:
    HBM streaming-read bandwidth and the bf16 MFMA rate (ceilings_bench's kernels)."""
    import torch

    import ar_self_speculative_amd as tidar

    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    hbm = max(nbytes / best(lambda: tidar.ceiling("hbm_read", buf, grid, sink)) / 1e9 for grid in (4096, 8192))
    del buf
    grid, iters = 1024, 20000
    mfma = grid * 4 * 4 * iters * 32768 / best(lambda: tidar.ceiling("mfma_bf16", grid, iters, sink), 3) / 1e12
    return {"hbm_read_gbps": round(hbm, 1), "mfma_bf16_tflops": round(mfma, 1)}


def stamps_bench(args) -> None:
    """Where one attention launch of the headline step spends its time: the
    timestamped instantiation of the main kernel (TIDAR_ATTN_STAMPS=1, the
    same computation with per-workgroup s_memtime / s_memrealtime records)
    launched eagerly --steps times on layer 0; medians over the launches."""
    import torch

    import ar_self_speculative_amd as tidar
    from tidar_synth import fill_device_step

    s = SHAPE
    torch.cuda.set_device(0)
    step = tidar.DecodeStep(layers=1, batch=s["batch"], num_q_heads=s["num_q_heads"],
                            num_kv_heads=s["num_kv_heads"], head_dim=s["head_dim"], k=s["k"],
                            cache_capacity=s["P"] + s["k"], max_cache_len=s["P"], vocab=s["vocab"])
    fill_device_step(step, seed=0, cache_len=s["P"])
    os.environ.pop("TIDAR_ATTN_STAMPS", None)
    step.attention(0)
    torch.cuda.synchronize()
    plain = step.out[0].clone()
    os.environ["TIDAR_ATTN_STAMPS"] = "1"
    per = []
    try:
        for _ in range(max(1, args.steps)):
            step.out.zero_()
            step.attention(0)
            torch.cuda.synchronize()
            r = tidar.attn_stamps(4096).astype(np.int64)
            nwg = int(r[0, 7] >> 32)
            if nwg <= 0 or nwg > 4096:
                print("no timestamped launch (the plan did not select it)", file=sys.stderr)
                sys.exit(1)
            r = r[:nwg]
            same = bool(torch.equal(step.out[0], plain))
            ghz = (r[:, 4] - r[:, 0]) / ((r[:, 5] - r[:, 1]) * 10.0)       # cycles per ns
            us = lambda cyc: cyc / ghz / 1e3                              # noqa: E731
            rt0, rt1 = r[:, 1], r[:, 5]
            xcc = (r[:, 6] >> 32) & 0xF
            xcc_start = [float((rt0[xcc == x].min() - rt0.min()) / 100.0) for x in range(8) if np.any(xcc == x)]
            per.append({
                "span_us": float((rt1.max() - rt0.min()) / 100.0),
                "last_start_after_first_us": float((rt0.max() - rt0.min()) / 100.0),
                "prologue_us_median": float(np.median(us(r[:, 2] - r[:, 0]))),
                "loop_us_median": float(np.median(us(r[:, 3] - r[:, 2]))),
                "epilogue_us_median": float(np.median(us(r[:, 4] - r[:, 3]))),
                "slowest_end_after_median_us": float((rt1.max() - np.median(rt1)) / 100.0),
                "shader_clock_ghz_median": float(np.median(ghz)),
                "xcd_first_start_us": xcc_start,
                "output_bitwise_equal_to_plain_launch": same,
                "workgroups": nwg,
                "tiles_per_workgroup": sorted(set(int(v) for v in (r[:, 7] & 0xFFFF))),
            })
    finally:
        os.environ.pop("TIDAR_ATTN_STAMPS", None)
    keys = [k for k, v in per[0].items() if isinstance(v, float)]
    med = {k: round(float(np.median([p[k] for p in per])), 3) for k in keys}
    print(json.dumps({
        "metric": "attention launch breakdown (timestamped main kernel)", "unit": "us", "n_gpus": 1,
        "data": "synthetic", "dtype": "bf16",
        "config": {"workload": "one Qwen3-8B-shaped layer of the decode step, P=4096, k=16, library plan",
                   "launches": len(per)},
        "median_over_launches": med,
        "output_bitwise_equal_to_plain_launch": all(p["output_bitwise_equal_to_plain_launch"] for p in per),
        "workgroups": per[0]["workgroups"], "tiles_per_workgroup": per[0]["tiles_per_workgroup"],
        "xcd_first_start_us_first_launch": [round(v, 3) for v in per[0]["xcd_first_start_us"]],
    }), flush=True)


def knee_bench(args) -> None:
    """Free-token-slot knee and the draft length it gives.

    The knee is where an append-prefill attention layer (64 query heads, 8 KV
    heads, head_dim 128) turns from HBM-bound to MFMA-bound: the roofline
    crossing at this box's measured HBM read rate and MFMA rate
    (draft_length.roofline_knee). The measured latency sweep over prefixes P
    and row counts R (32 rotated caches per timed graph) is reported beside
    it with its hinge fit t = c + max(a, b R) (draft_length.hinge_fit). The
    draft length for the Qwen3-8B step (4 query heads per KV head) is the
    largest k whose packed rows fit under the knee at P = 4096."""
    import math

    import torch

    import ar_self_speculative_amd as tidar
    from ar_self_speculative_amd import draft_length as dl

    Hq, Hkv, D = 64, 8, 128
    Ps, Rs = (512, 1024, 2048, 4096), (1, 8, 16, 32, 64, 128, 256, 512)
    if getattr(args, "knee_rows", ""):
        Rs = tuple(int(r) for r in args.knee_rows.split(","))
    ceil = knee_ceilings()
    gen = torch.Generator(device="cuda").manual_seed(0)
    nbuf = 32  # distinct caches per timed graph (32 x 16.8 MB at P=4096 > the 256 MB last-level cache)
    table = {}
    # The floor of one launch in this regime: a plain streaming read of the
    # prefix K/V bytes (fresh, uncached buffers) in one kernel, and an empty
    # kernel, each timed as graph nodes like the sweep.
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    floor = {}
    for P in Ps:
        nbytes = 2 * Hkv * P * D * 2
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(nbuf)]

        def read():
            for b in bufs:
                tidar.ceiling("hbm_read", b, 512, sink)

        read()
        floor[P] = _time_graph(_capture(read), 5) * 1e3 / nbuf
        del bufs

    def empty():
        for _ in range(nbuf):
            tidar.ceiling("empty", 1)

    empty()
    empty_us = _time_graph(_capture(empty), 5) * 1e3 / nbuf
    for P in Ps:
        kcs = [_rand_bf16((1, Hkv, P + 512, D), gen) for _ in range(nbuf)]
        vcs = [_rand_bf16((1, Hkv, P + 512, D), gen) for _ in range(nbuf)]
        lens = torch.full((1,), P, dtype=torch.int32, device="cuda")
        for R in Rs:
            desc = tidar.make_attn_desc(batch=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, k=R, num_blocks=0,
                                        block_len=1, cache_capacity=P + 512, max_cache_len=P,
                                        sm_scale=1 / math.sqrt(D), dtype=tidar.DTYPE_BF16)
            q = _rand_bf16((1, R, Hq, D), gen)
            ks, vs = _rand_bf16((1, R, Hkv, D), gen), _rand_bf16((1, R, Hkv, D), gen)
            out = torch.empty_like(q)
            ws = tidar.attn_workspace(desc, torch.device("cuda"))

            def run():
                for i in range(nbuf):
                    tidar.attn_step(desc, q, ks, vs, kcs[i], vcs[i], lens, out, None, None, ws)

            run()
            g = _capture(run)
            table[(P, R)] = _time_graph(g, 3) * 1e3 / nbuf
        del kcs, vcs
    g_sweep, g_step = Hq // Hkv, SHAPE["num_q_heads"] // SHAPE["num_kv_heads"]
    knees, fits = {}, {}
    for P in Ps:
        knees[P] = dl.roofline_knee(prefix=P, q_heads=Hq, kv_heads=Hkv, head_dim=D, hbm_gbps=ceil["hbm_read_gbps"],
                                    mfma_tflops=ceil["mfma_bf16_tflops"])
        if len(Rs) >= 3:
            # fitted to the printed (rounded) times, so the record reproduces its own fit
            f = dl.hinge_fit(Rs, [round(table[(P, R)], 2) for R in Rs])
            fits[P] = {key: round(v, 3) for key, v in f.items()}
        else:
            fits[P] = None  # too few row counts to fit
    k_pick = dl.draft_length(knees[4096], sweep_group=g_sweep, step_group=g_step)
    print(json.dumps({
        "metric": "free-token-slot knee (append-prefill attention, 64 q heads, 8 kv heads, d 128) and draft length",
        "unit": "us", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "one layer, batch 1, append-prefill sweep", "P": list(Ps), "R": list(Rs),
                   "caches_rotated": nbuf},
        "ceilings": ceil,
        "us": {str(P): [round(table[(P, R)], 2) for R in Rs] for P in Ps},
        "one_launch_floor": {
            "kv_read_us": {str(P): round(floor[P], 2) for P in Ps},
            "empty_kernel_us": round(empty_us, 2),
            "kv_bytes": {str(P): 2 * Hkv * P * D * 2 for P in Ps},
            "R1_over_read_floor": {str(P): round(table[(P, 1)] / floor[P], 2) for P in Ps} if 1 in Rs else None,
            "note": "a single launch streaming the prefix K/V of fresh buffers (512 workgroups) and an empty kernel, "
                    "graph nodes like the sweep; the sweep's points are two launches (attention and split merge)"},
        "knee_rule": "rows where MFMA time equals HBM time at the measured ceilings (roofline crossing)",
        "knee_rows": {str(P): round(knees[P], 2) for P in Ps},
        "sweep_hinge_fit": {str(P): fits[P] for P in Ps},
        "draft_length_at_P4096": {"rule": "largest k in (1, 2, 4, 8, 16) whose step's rows x 4 query heads per kv "
                                          "head fit under the knee's rows x 8",
                                  "k": k_pick, "rows": dl.step_rows(k_pick),
                                  "packed_rows": dl.step_rows(k_pick) * g_step},
    }), flush=True)


def loop_bench(args) -> None:
    """The TiDAR step loop with a random-weight Qwen3-8B-shaped decoder:
    time per step (one NFE: 36 layers of GEMMs + hybrid attention, the
    sampler, the commit and the next drafts), tokens per NFE, and the share of
    the step spent in the hybrid attention."""
    import torch

    import ar_self_speculative_amd as tidar
    from ar_self_speculative_amd.loop import TiDARLoop, TinyDecoder

    s = SHAPE
    L, Hq, Hkv, D, P, V = s["layers"], s["num_q_heads"], s["num_kv_heads"], s["head_dim"], s["P"], s["vocab"]
    k_rule = None
    if args.k == "auto":
        # the draft length from the free-slot knee at this box's measured ceilings
        from ar_self_speculative_amd import draft_length as dl

        ceil = knee_ceilings()
        knee = dl.roofline_knee(prefix=P, q_heads=Hq, kv_heads=Hkv, head_dim=D, hbm_gbps=ceil["hbm_read_gbps"],
                                mfma_tflops=ceil["mfma_bf16_tflops"])
        k = dl.draft_length(knee, sweep_group=Hq // Hkv, step_group=Hq // Hkv)
        k_rule = {"ceilings": ceil, "knee_rows": round(knee, 2), "k": k}
    else:
        k = int(args.k) if args.k else s["k"]
    model = TinyDecoder(vocab=V, hidden=4096, layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, mlp=12288,
                        seed=0)
    cap = P + 2048
    lp = TiDARLoop(model, batch=1, k=k, cache_capacity=cap)
    gen = torch.Generator(device="cuda").manual_seed(1)
    lp.k_cache.copy_(torch.randn(lp.k_cache.shape, generator=gen, device="cuda").to(torch.bfloat16))
    lp.v_cache.copy_(torch.randn(lp.v_cache.shape, generator=gen, device="cuda").to(torch.bfloat16))
    lp.region.copy_(torch.randint(0, V - 1, lp.region.shape, generator=gen, device="cuda", dtype=torch.int32))
    lp.q_logits.zero_()
    uv = torch.rand((1, k), generator=gen, device="cuda")
    ud = torch.rand((1, k - 1), generator=gen, device="cuda")
    emitted = torch.zeros(1, dtype=torch.int64, device="cuda")

    def one_step():
        lp.step(uv, ud)
        emitted.add_(lp.accept_len.long() + 1)

    lp.cache_len.fill_(P)
    for _ in range(args.warmup):
        one_step()
    lp.cache_len.fill_(P)
    g = _capture(one_step)
    reps = args.steps
    if P + (reps + 2) * k > cap - k:
        reps = (cap - k - P) // k - 2
    lp.cache_len.fill_(P)
    emitted.zero_()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    tokens_per_nfe = int(emitted.item()) / reps
    # the hybrid attention alone, on the same buffers and prefix length
    lp.cache_len.fill_(P)
    ga = _capture(lambda: [tidar.attn_step(lp.desc, lp.last_q, lp.k_step[l], lp.v_step[l], lp.k_cache[l],
                                           lp.v_cache[l], lp.cache_len, lp.attn_out, None, lp.status, lp.attn_ws)
                           for l in range(L)])
    ms_attn = _time_graph(ga, 5)
    if int(lp.status.item()):
        print(f"device status flags set: {int(lp.status.item())}", file=sys.stderr)
        sys.exit(1)
    print(json.dumps({
        "metric": f"TiDAR step loop NFE/s with a random-weight Qwen3-8B-shape decoder (k={k} region rows, P~4096)",
        "value": round(1e3 / ms, 2), "unit": "NFE/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic, random weights",
        "config": {"workload": f"qwen3-8b-shape decoder (hidden 4096, 36 layers, 32/8 heads, head_dim 128, "
                               f"MLP 12288, vocab 151936), batch 1, prefix 4096, k={k} region rows ({lp.R} rows)",
                   "layers": L, "prefix": P, "k": k, "rows": lp.R},
        "draft_length_rule": k_rule,
        "tokens_per_nfe": round(tokens_per_nfe, 3),
        "attention_ms_per_step": round(ms_attn, 4),
        "attention_share": round(ms_attn / ms, 4),
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="force the prefix split count (0 = library plan)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run three device copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--likelihood", type=int, default=0, metavar="R",
                    help="only time likelihood mode: one causal forward scoring R tokens (P=4096), and exit")
    ap.add_argument("--loop", action="store_true",
                    help="only time the TiDAR step loop with a random-weight Qwen3-8B-shaped decoder, and exit")
    ap.add_argument("--k", default="", metavar="K|auto",
                    help="draft length of --loop (default 16); 'auto' takes it from the free-slot knee at this "
                         "box's measured HBM and MFMA ceilings")
    ap.add_argument("--config5", action="store_true",
                    help="only time the ragged batch (8 sequences, k=8, 36 layers, 64 chained steps) and exit")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the machine ceilings (HBM read, MFMA, exp/FMA rates, empty kernel) and exit")
    ap.add_argument("--sampler", default="", metavar="B:k[:V]",
                    help="only time the sampler (tidar_reject_sample) at batch B, draft length k, vocab V, and exit")
    ap.add_argument("--stamps", action="store_true",
                    help="per-workgroup timestamps of one attention launch (timestamped main kernel)")
    ap.add_argument("--knee", action="store_true",
                    help="only run the append-prefill sweep, report its knee and the draft length it allows")
    ap.add_argument("--knee-rows", default="", metavar="R,R,...",
                    help="with --knee: time only these row counts (e.g. 1 for the decode regime under a tracer)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path is measured on a "
              "single MI355X and multi-GPU sharding is not part of this build.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.likelihood:
        likelihood_bench(args)
        return
    if args.config5:
        config5_bench(args)
        return
    if args.ceilings:
        print(json.dumps({"metric": "measured MI355X ceilings", "n_gpus": 1, "data": "synthetic",
                          **ceilings_bench(args)}), flush=True)
        return
    if args.sampler:
        sampler_bench(args)
        return
    if args.stamps:
        stamps_bench(args)
        return
    if args.knee:
        knee_bench(args)
        return
    if args.loop:
        loop_bench(args)
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
    # what the timed step decided: every replay verifies the same synthetic
    # drafts with the same uniforms, so it is one accept length (the
    # ragged-batch mode, --config5, reports the distribution over chained
    # steps); acceptance tests within 1e-5 of their threshold among those
    # the chain consulted, by the GPU's own ratios
    acc_n = int(step.accept_len[0].item())
    u0 = step.uniforms[0].float().cpu().numpy()
    r0 = step.ratio[0].float().cpu().numpy()
    tested = np.arange(min(acc_n + 1, s["k"]))
    near = int(np.sum(np.abs(u0[tested] - np.minimum(1.0, r0[tested])) < 1e-5))

    cnt = algorithmic_counts(s["layers"], s["batch"], s["num_q_heads"], s["num_kv_heads"], s["head_dim"],
                             s["P"], s["k"], s["vocab"])
    t_step = ms_step * 1e-3
    kv_bytes = s["layers"] * (cnt["kv_prefix_layer"] + cnt["kv_step_layer"])
    # every byte the step must move at least once: Q, K/V (prefix and step) and O of every layer, and
    # the logits the sampler reads (the commit's few MB depend on the accept lengths and are left out)
    comp_bytes = s["layers"] * cnt["attn_bytes_layer"] + cnt["sampler_bytes"]
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
        "compulsory_gbps": round(comp_bytes / t_step / 1e9, 1),
        "compulsory_frac_of_hbm_peak": round(comp_bytes / t_step / 1e9 / HBM_PEAK_GBPS, 4),
        "kv_read_frac_of_hbm_peak": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "attn_us_per_layer": round(attn_ms * 1e3, 2),
        "sampler": {"accept_len": acc_n, "tokens_per_step": acc_n + 1, "accept_near_ties": near,
                    "inputs": "one synthetic set (diffusion = AR + N(0,1) noise) replayed every step"},
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel<128> (+ split merge)",
                     "achieved": round(achieved_tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": ATTN_TRAFFIC.get(attn_source_digest()),
                     "flops_per_launch": cnt["attn_flops_layer"]},
        "mfma_util": ATTN_COUNTERS.get(attn_source_digest()),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
