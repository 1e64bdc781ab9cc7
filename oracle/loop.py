"""The TiDAR decode-step loop around the hot path: which rows a step feeds,
at which positions, and how one step's verification chooses the next
step's inputs (fp64, numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* TiDAR review (awesome-system-papers wiki), 核心方法 §3.2: one forward
  verifies the previous step's drafts with causal (AR) logits and, in the
  same pass, pre-drafts the next step for every possible accept length; the
  block matching the accept length is kept and the rejected drafts' KV is
  dropped without recomputation.
* yuuk.io talk notes, 推論パイプライン: the input is the prefix plus the
  tokens drafted last step; tokens after the first rejection are discarded;
  the next drafts come from the pre-drafted block.

Readings (the pages never align rows; this is the plainest scheme in which
every committed token gets its KV from a forward without recomputation):
* A step feeds k region rows [c, d_1 .. d_{k-1}]: c is the token the AR side
  sampled at the end of the last step (its KV is not cached yet) and d_i are
  the last step's drafts. Region row i sits at position len + i, len being
  the committed length (the KV cache length).
* Block j (j = 0..k) holds k mask tokens at positions len + j + m
  (m = 0..k-1): it sees region rows 0..j-1 and itself, so its mask m
  proposes the token at that position given c, d_1..d_{j-1}.
* Verification: region row i's AR logits are the target of region row i+1
  (i < k-1); row k-1 is the bonus row. The k-1 drafts were proposed by the
  diffusion logits carried from the last step. The sampler (oracle.reject
  .reject_sample) returns n accepted drafts and the next AR token c'.
* Commit: region rows 0..n (c and the n accepted drafts) join the cache.
* Next inputs: block j* = n + 1 saw exactly the committed rows; its mask
  m = 0 sits at c''s position (decided by the AR side), masks m = 1..k-1
  give the next drafts d'_m, drawn by inverse CDF from softmax(logits / T)
  with the draft uniforms, and their logits are carried as the proposals.
* Tokens emitted per step: d_1..d_n and c' (n + 1 tokens; c was emitted by
  the step before).
* The loop starts from a causal prefill of the prompt (the likelihood-mode
  forward): c_0 is drawn from the last prompt row, and the first drafts are
  drawn from the uniform distribution (any proposal keeps the sampler exact).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .reject import invcdf, reject_sample, softmax_t


def step_rows(k: int) -> int:
    """Rows of one step: k region rows and k + 1 blocks of k mask tokens."""
    return k + (k + 1) * k


def step_positions(k: int, cache_len: int) -> np.ndarray:
    """Position of every row of a step whose committed length is cache_len."""
    pos = np.empty(step_rows(k), np.int64)
    for i in range(k):
        pos[i] = cache_len + i
    for j in range(k + 1):
        for m in range(k):
            pos[k + j * k + m] = cache_len + j + m
    return pos


def block_row(k: int, j: int, m: int) -> int:
    """Row index of mask m of block j."""
    return k + j * k + m


@dataclasses.dataclass
class LoopState:
    region: np.ndarray     # [B, k] int: c, d_1..d_{k-1}
    q_logits: np.ndarray   # [B, k-1, V]: logits that proposed d_1..d_{k-1}
    cache_len: np.ndarray  # [B] int: committed length (KV rows cached)
    emitted: list          # per sequence: tokens emitted after the prompt


def start(last_prompt_logits, cache_len, k: int, u_first, u_drafts, temperature: float = 1.0) -> LoopState:
    """State after the causal prefill: c_0 from the last prompt row, uniform first drafts."""
    last_prompt_logits = np.asarray(last_prompt_logits, np.float64)
    B, V = last_prompt_logits.shape
    region = np.zeros((B, k), np.int64)
    q = np.zeros((B, k - 1, V))
    emitted = []
    for b in range(B):
        region[b, 0], _ = invcdf(softmax_t(last_prompt_logits[b], temperature), float(u_first[b]))
        for m in range(1, k):
            region[b, m], _ = invcdf(np.full(V, 1.0 / V), float(u_drafts[b, m - 1]))
        emitted.append([int(region[b, 0])])
    return LoopState(region, q, np.asarray(cache_len, np.int64).copy(), emitted)


def loop_step(logits, state: LoopState, u_verify, u_draft, temperature: float = 1.0, trust_ar: float = 1.0):
    """One step given the forward's logits [B, R, V] for the rows of step_positions.

    Returns (new_state, accept_n [B], next_token [B], sample_result).
    """
    logits = np.asarray(logits, np.float64)
    B, R, V = logits.shape
    k = state.region.shape[1]
    assert R == step_rows(k)
    ar = logits[:, :k]                       # row i verifies region row i+1; row k-1 = bonus row
    res = reject_sample(ar, state.q_logits, state.region[:, 1:], np.asarray(u_verify), temperature,
                        trust_ar=trust_ar)
    n = res.accept_len.astype(np.int64)
    c_next = res.next_token.astype(np.int64)
    region = np.zeros_like(state.region)
    q = np.zeros_like(state.q_logits)
    emitted = [list(e) for e in state.emitted]
    for b in range(B):
        j = int(n[b]) + 1                    # the block that saw c and the accepted drafts
        region[b, 0] = c_next[b]
        for m in range(1, k):
            row = logits[b, block_row(k, j, m)]
            region[b, m], _ = invcdf(softmax_t(row, temperature), float(u_draft[b, m - 1]))
            q[b, m - 1] = row
        emitted[b].extend(int(t) for t in state.region[b, 1:1 + n[b]])
        emitted[b].append(int(c_next[b]))
    new = LoopState(region, q, state.cache_len + n + 1, emitted)
    return new, n, c_next, res
