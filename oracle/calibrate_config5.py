"""Calibrate the diffusion-noise scale of the ragged-batch workload.

TEST INFRASTRUCTURE ONLY (see the package docstring). Run as a script:

    python oracle/calibrate_config5.py            # bisection, writes tests/golden/config5_sigma.json

The ragged batch (8 sequences, k = 8 drafts, vocabulary 151936) draws AR
logits ~ N(0, 3) and diffusion logits = AR + N(0, sigma) for each of its 64
steps (seeds 50..113). The pages report about 7 to 8.5 tokens per forward
for TiDAR 8B (talk notes on notes.yuuk.io, SGLang throughput section: 6.98
to 8.51 per task; TiDAR review, 实验与结果: 7.45 and 8.25), and the workload
asks for a mean of about 7 committed tokens per step. Committed tokens per
step are n + 1, and E[n] has the closed form of speculative sampling
(oracle.reject.expected_accept_len), which is smooth and increasing as sigma
falls, so sigma is found by bisection on the mean over every (step,
sequence) of 1 + E[n]. Only the oracle and the input generators are used.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.reject import expected_accept_len  # noqa: E402
from tidar_synth import CONFIG5_STEP_SEED0, CONFIGS, diffusion_logits, sampler_draws  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden", "config5_sigma.json")
TARGET = 7.0


def mean_committed(draws, sigma: float) -> float:
    """Mean over every (step, sequence) of 1 + E[n] at noise scale sigma."""
    tot, cnt = 0.0, 0
    for ar, z in draws:
        e = expected_accept_len(ar, diffusion_logits(ar, z, "noisy", sigma))
        tot += float(np.sum(1.0 + e))
        cnt += len(e)
    return tot / cnt


def step_draws(steps: int | None = None):
    c = CONFIGS[5]
    steps = c["steps"] if steps is None else steps
    out = []
    for it in range(steps):
        ar, z, _ = sampler_draws(batch=c["batch"], k=c["k"], vocab=c["vocab"], ar_sigma=3.0,
                                 seed=CONFIG5_STEP_SEED0 + it)
        out.append((ar, z))
    return out


def calibrate(tol: float = 1e-3) -> dict:
    draws = step_draws()
    lo, hi = 0.02, 1.0             # mean committed falls from ~9 to ~4 over this range
    m_lo, m_hi = mean_committed(draws, lo), mean_committed(draws, hi)
    assert m_lo > TARGET > m_hi, (m_lo, m_hi)
    while hi - lo > tol:
        mid = 0.5 * (lo + hi)
        m = mean_committed(draws, mid)
        print(f"sigma {mid:.5f}: mean committed {m:.4f}", flush=True)
        if m > TARGET:
            lo = mid
        else:
            hi = mid
    sigma = round(0.5 * (lo + hi), 3)
    return {"sigma": sigma, "mean_committed_expected": round(mean_committed(draws, sigma), 4),
            "target": TARGET, "steps": len(draws), "batch": CONFIGS[5]["batch"], "k": CONFIGS[5]["k"],
            "vocab": CONFIGS[5]["vocab"], "step_seeds": [CONFIG5_STEP_SEED0, CONFIG5_STEP_SEED0 + len(draws) - 1],
            "written_by": "python oracle/calibrate_config5.py"}


if __name__ == "__main__":
    res = calibrate()
    with open(GOLDEN, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))
