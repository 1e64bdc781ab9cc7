"""Draft length from the free-token-slot knee.

The TiDAR pages build on one observation: at small batch a forward's latency
stays nearly flat as more tokens ride along, until the forward turns
compute-bound, so those extra slots are free (TiDAR review on the
awesome-system-papers wiki, 关键观察 / 隐含假设, observation 1 and Fig. 1;
talk notes on notes.yuuk.io, フリートークンスロットの着想). The block length
is fixed at training time and the draft length can be adjusted zero-shot; the
pages list picking it per target GPU from that roofline as future work
(review, 局限与 Future Work, future work 2; talk notes, 制約と今後の課題,
バッチサイズ and システム最適化). This module is that choice, as host logic:

* ``hinge_fit`` reads the knee off a measured latency-vs-rows sweep by
  fitting t(R) = c + max(a, b R): c is the fixed cost of a launch, a the
  time to stream the K/V cache, b the per-row compute time. The knee
  R* = a / b is where compute overtakes the memory stream; the fixed cost c
  does not move it.
* ``roofline_knee`` predicts the same crossing from the attention layer's
  algorithmic bytes and flops at measured ceilings (HBM read bandwidth, MFMA
  rate).
* ``draft_length`` is the largest candidate k whose decode step, k drafts
  plus k + 1 pre-draft blocks of k rows, packs no more rows per KV head
  than the knee.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence


def step_rows(k: int) -> int:
    """Query rows of one TiDAR step: k drafts and k + 1 blocks of k masks."""
    return k + (k + 1) * k


def hinge_fit(rows: Sequence[float], times: Sequence[float], grid: int = 400) -> dict:
    """Least-squares fit of t(R) = c + b * max(R*, R) over the sweep.

    For a fixed knee R* the model is linear in (c, b); R* is scanned on a
    log grid between the smallest and largest swept row counts and the best
    fit kept. Returns the knee, c, b, the memory term a = b R* and the RMS
    residual (all in the units of `times`).
    """
    rows = [float(r) for r in rows]
    times = [float(t) for t in times]
    if len(rows) != len(times) or len(rows) < 3:
        raise ValueError("need at least three (rows, time) points")
    lo, hi = math.log(min(rows)), math.log(max(rows))
    best = None
    for i in range(grid + 1):
        knee = math.exp(lo + (hi - lo) * i / grid)
        x = [max(knee, r) for r in rows]
        n = len(x)
        sx, sy = sum(x), sum(times)
        sxx = sum(v * v for v in x)
        sxy = sum(v * t for v, t in zip(x, times))
        den = n * sxx - sx * sx
        if den <= 0:
            continue
        b = (n * sxy - sx * sy) / den
        c = (sy - b * sx) / n
        if b <= 0:
            continue
        rss = sum((c + b * v - t) ** 2 for v, t in zip(x, times))
        if best is None or rss < best[0] - 1e-12:
            best = (rss, knee, c, b)
    if best is None:
        raise ValueError("the sweep does not rise with the row count")
    rss, knee, c, b = best
    return {"knee_rows": knee, "fixed": c, "per_row": b, "memory": b * knee, "rms": math.sqrt(rss / len(rows))}


def roofline_knee(*, prefix: int, q_heads: int, kv_heads: int, head_dim: int, hbm_gbps: float, mfma_tflops: float,
                  elem_bytes: int = 2) -> float:
    """Rows R at which one append-prefill attention layer's MFMA time equals
    its HBM time: bytes(R) = 2 Hkv P D e + R (2 Hkv + 2 Hq) D e (prefix K/V,
    the rows' K/V, Q and O), flops(R) = 4 Hq D P R."""
    kv = 2.0 * kv_heads * prefix * head_dim * elem_bytes
    per_row_bytes = (2.0 * kv_heads + 2.0 * q_heads) * head_dim * elem_bytes
    per_row_flops = 4.0 * q_heads * head_dim * prefix
    bw, f = hbm_gbps * 1e9, mfma_tflops * 1e12
    slope = per_row_flops / f - per_row_bytes / bw
    if slope <= 0:
        return math.inf
    return (kv / bw) / slope


def draft_length(knee_rows: float, *, sweep_group: int, step_group: int,
                 candidates: Iterable[int] = (1, 2, 4, 8, 16)) -> int:
    """Largest k among `candidates` whose step packs at most the knee's rows
    per KV head: step_rows(k) * step_group <= knee_rows * sweep_group (each
    KV head serves its group of query heads, so packed rows are what the
    attention's matrix work scales with). At least the smallest candidate."""
    budget = knee_rows * sweep_group
    cands = sorted(candidates)
    ok = [k for k in cands if step_rows(k) * step_group <= budget]
    return ok[-1] if ok else cands[0]
