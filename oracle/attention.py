"""Hybrid-mask decode-step attention, fp64, by its plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* TiDAR review (awesome-system-papers wiki), "核心方法" -> "并行 self-speculative
  生成 (§3.2)": one forward holds three regions: the prefix reuses the causal KV
  of earlier steps; last step's drafts are verified with this step's causal
  logits; the next step's drafts are pre-drafted, conditioned on every possible
  accept prefix, so that any accept length has a matching next draft.
* Same review, "关键观察" observation 3: only the last block is bidirectional
  and the prefix stays causal, which is what keeps the KV cache exact.
* yuuk.io talk notes, "推論パイプライン" steps 1-4 (verify, discard rejected,
  pre-draft for the next step in the same forward).

Reading used here (the pages give no formula): for a query row r and a step
key c,

* draft row i (0 <= i < k, draft d_{i+1}) sees step keys c <= i (causal,
  itself included);
* mask row m of pre-draft block j (j = 0..num_blocks-1, accept length j) sees
  drafts d_1..d_j (step keys c < j) and all block_len keys of block j
  (bidirectional, itself included), and nothing of any other block;
* every row sees all cache_len[b] committed prefix keys.

Query head h reads KV head h // (Hq // Hkv) (contiguous GQA groups).
"""
from __future__ import annotations

import numpy as np


def local_keys(r: int, k: int, num_blocks: int, block_len: int) -> list[int]:
    """Indices of the step keys (0..R-1) that query row r may attend to."""
    if r < k:
        # region of last step's drafts: causal over the drafts
        return list(range(0, r + 1))
    j = (r - k) // block_len
    if j >= num_blocks:
        raise IndexError(r)
    first = k + j * block_len
    # drafts d_1..d_j, then the whole of block j
    return list(range(0, j)) + list(range(first, first + block_len))


def kv_head(h: int, g: int) -> int:
    """KV head read by query head h when g query heads share one KV head
    (contiguous groups)."""
    return h // g


def visible_local_count(k: int, num_blocks: int, block_len: int) -> int:
    """Number of (row, step key) pairs that are visible in one head."""
    R = k + num_blocks * block_len
    return sum(len(local_keys(r, k, num_blocks, block_len)) for r in range(R))


def attn_step(q, k_step, v_step, k_cache, v_cache, cache_len, *, k: int,
              num_blocks: int, block_len: int, sm_scale: float):
    """One layer of hybrid-mask attention.

    Shapes: q [B,R,Hq,D]; k_step/v_step [B,R,Hkv,D]; k_cache/v_cache
    [B,Hkv,cap,D]; cache_len [B]. Returns (out [B,R,Hq,D], lse [B,R,Hq]) in
    fp64, lse being the natural-log normaliser ln(sum_c exp(s_c)).

    Each output row is softmax(sm_scale * q . K_vis^T) V_vis over its visible
    keys, with the row maximum subtracted before exponentiation.
    """
    q = np.asarray(q, dtype=np.float64)
    k_step = np.asarray(k_step, dtype=np.float64)
    v_step = np.asarray(v_step, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, R, Hq, D = q.shape
    Hkv = k_step.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if R != k + num_blocks * block_len:
        raise ValueError("R != k + num_blocks * block_len")
    g = Hq // Hkv
    out = np.empty((B, R, Hq, D))
    lse = np.empty((B, R, Hq))
    locals_ = [local_keys(r, k, num_blocks, block_len) for r in range(R)]
    for b in range(B):
        n_pre = int(cache_len[b])
        for h in range(Hq):
            kvh = kv_head(h, g)
            pre_k = k_cache[b, kvh, :n_pre]
            pre_v = v_cache[b, kvh, :n_pre]
            for r in range(R):
                loc = locals_[r]
                keys = np.concatenate([pre_k, k_step[b, loc, kvh]], axis=0)
                vals = np.concatenate([pre_v, v_step[b, loc, kvh]], axis=0)
                s = sm_scale * (keys @ q[b, r, h])
                m = s.max()
                e = np.exp(s - m)
                z = e.sum()
                out[b, r, h] = (e @ vals) / z
                lse[b, r, h] = m + np.log(z)
    return out, lse


def attn_rows(q, k_step, v_step, k_cache, v_cache, cache_len, rows, *, k: int,
              num_blocks: int, block_len: int, sm_scale: float):
    """The same definition evaluated only at the given (b, r, h) triples.

    Lets the parity tests check sampled outputs of full-size workloads.
    Returns (out [N,D], lse [N]).
    """
    B, R, Hq, D = q.shape
    Hkv = k_step.shape[2]
    g = Hq // Hkv
    out = np.empty((len(rows), D))
    lse = np.empty(len(rows))
    for i, (b, r, h) in enumerate(rows):
        kvh = kv_head(h, g)
        n_pre = int(cache_len[b])
        loc = local_keys(r, k, num_blocks, block_len)
        keys = np.concatenate([np.asarray(k_cache[b, kvh, :n_pre], np.float64),
                               np.asarray(k_step[b, loc, kvh], np.float64)], axis=0)
        vals = np.concatenate([np.asarray(v_cache[b, kvh, :n_pre], np.float64),
                               np.asarray(v_step[b, loc, kvh], np.float64)], axis=0)
        s = sm_scale * (keys @ np.asarray(q[b, r, h], np.float64))
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        out[i] = (e @ vals) / z
        lse[i] = m + np.log(z)
    return out, lse
