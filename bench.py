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
    "8ca6ea5ef832f306": 57074936,
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


def knee_bench(args) -> None:
    """Append-prefill sweep (one layer, 64 query heads, 8 KV heads, head_dim
    128): attention time per launch for each prefix P and row count R, the
    knee where more rows stop being nearly free, and the largest draft length
    k whose hybrid step (k + (k+1)k rows) fits under it."""
    import math

    import torch

    import ar_self_speculative_amd as tidar

    Hq, Hkv, D = 64, 8, 128
    Ps, Rs = (512, 1024, 2048, 4096), (1, 8, 16, 32, 64, 128, 256, 512)
    gen = torch.Generator(device="cuda").manual_seed(0)
    nbuf = 32  # distinct caches per timed graph (32 x 16.8 MB at P=4096 > the 256 MB last-level cache)
    table = {}
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
    knee = {}
    for P in Ps:
        base = table[(P, 1)]
        knee[P] = max(R for R in Rs if table[(P, R)] <= 1.25 * base)
    g = Hq // Hkv
    # packed query rows (rows x group) at the knee; the Qwen3-8B decode step
    # packs k + (k+1)k rows x 4 query heads per KV head
    packed = knee[4096] * g
    g_step = SHAPE["num_q_heads"] // SHAPE["num_kv_heads"]
    k_pick = max([k for k in (1, 2, 4, 8, 16) if (k + (k + 1) * k) * g_step <= packed] or [1])
    print(json.dumps({
        "metric": "append-prefill attention us per launch (64 q heads, 8 kv heads, d 128) and its knee",
        "unit": "us", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "one layer, batch 1, append-prefill sweep", "P": list(Ps), "R": list(Rs),
                   "caches_rotated": nbuf},
        "us": {str(P): [round(table[(P, R)], 2) for R in Rs] for P in Ps},
        "knee_rule": "largest R with time <= 1.25 x time at R = 1",
        "knee_R": {str(P): knee[P] for P in Ps},
        "knee_rows_times_group": {str(P): knee[P] * g for P in Ps},
        "draft_length_at_P4096": {"rule": "largest k whose step packs at most the knee's rows x group",
                                  "k": k_pick, "rows": k_pick + (k_pick + 1) * k_pick,
                                  "packed_rows": (k_pick + (k_pick + 1) * k_pick) * g_step},
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
    L, Hq, Hkv, D, P, V, k = s["layers"], s["num_q_heads"], s["num_kv_heads"], s["head_dim"], s["P"], s["vocab"], \
        s["k"]
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
        "metric": "TiDAR step loop NFE/s with a random-weight Qwen3-8B-shape decoder (k=16 region rows, P~4096)",
        "value": round(1e3 / ms, 2), "unit": "NFE/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic, random weights",
        "config": {"workload": "qwen3-8b-shape decoder (hidden 4096, 36 layers, 32/8 heads, head_dim 128, "
                               "MLP 12288, vocab 151936), batch 1, prefix 4096, k=16 region rows (288 rows)",
                   "layers": L, "prefix": P, "k": k, "rows": lp.R},
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
    ap.add_argument("--knee", action="store_true",
                    help="only run the append-prefill sweep, report its knee and the draft length it allows")
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
