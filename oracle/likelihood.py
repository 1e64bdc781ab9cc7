"""Per-token log-likelihood in TiDAR's causal (AR) mode, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* yuuk.io talk notes, 尤度評価 (Table 3): with the attention mask set to
  causal, TiDAR scores a sequence as an AR model, directly and without
  Monte-Carlo sampling.
* TiDAR review (awesome-system-papers wiki), 实验与结果: likelihood tasks are
  evaluated with a pure causal mask in a single forward (one NFE), in line
  with AR evaluation.

The causal forward is the append-prefill mode of the attention
(``attn_step`` with ``num_blocks = 0``). What this module adds is the AR
log-likelihood of each next token from that forward's logits:

    log p(x_{t+1} | x_<=t) = logits[t, x_{t+1}] - log(sum_v exp(logits[t, v]))

Readings where the pages are silent: temperature 1 (no scaling); a target id
outside 0..V-1 has no probability and scores NaN.
"""
from __future__ import annotations

import math

import numpy as np


def log_normaliser(row) -> float:
    """log(sum_v exp(row[v])) in fp64, with the row maximum taken out first."""
    x = np.asarray(row, np.float64)
    m = float(x.max())
    if not math.isfinite(m):
        return m
    return m + math.log(float(np.exp(x - m).sum()))


def token_logprobs(logits, targets) -> np.ndarray:
    """logits [..., V], targets [...] int -> log-probabilities [...] (fp64)."""
    logits = np.asarray(logits)
    targets = np.asarray(targets)
    V = logits.shape[-1]
    flat = logits.reshape(-1, V)
    tf = targets.reshape(-1)
    out = np.empty(tf.shape[0], np.float64)
    for i in range(tf.shape[0]):
        t = int(tf[i])
        out[i] = float(flat[i, t]) - log_normaliser(flat[i]) if 0 <= t < V else math.nan
    return out.reshape(targets.shape)


def sequence_loglik(logits, targets) -> np.ndarray:
    """Sum of the per-token log-probabilities over the last axis of targets."""
    return token_logprobs(logits, targets).sum(axis=-1)
