"""Dense-mask brute force for the hybrid decode-step attention (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring). Written separately from
``attention.py`` and used only to pin it on tiny inputs: it builds the explicit
0/1 matrix M of shape R x (P + R) by enumerating every (row, key) pair against
the three region rules, then applies an ordinary masked softmax over the
concatenated key set [cache prefix; step keys].

Region rules (TiDAR review, awesome-system-papers wiki, "核心方法" §3.2; talk
notes on yuuk.io, "推論パイプライン"):
(a) the k drafted tokens attend causally over the prefix and each other;
(b) for each accept length j, a block of mask tokens attends to the prefix,
    the drafts d_1..d_j, and bidirectionally inside its own block;
every row attends to every committed prefix key.
"""
from __future__ import annotations

import numpy as np


def hybrid_mask_matrix(P: int, k: int, num_blocks: int, block_len: int) -> np.ndarray:
    """0/1 matrix over columns [prefix 0..P-1 | step keys P..P+R-1]."""
    R = k + num_blocks * block_len
    M = np.zeros((R, P + R), dtype=np.int8)
    for row in range(R):
        for col in range(P + R):
            if col < P:
                M[row, col] = 1                      # committed prefix: always visible
                continue
            key = col - P                            # step key index
            if row < k:                              # rule (a): drafts, causal
                key_is_draft = key < k
                M[row, col] = 1 if (key_is_draft and key <= row) else 0
            else:                                    # rule (b): pre-draft blocks
                blk = (row - k) // block_len
                if key < k:
                    M[row, col] = 1 if key < blk else 0          # drafts d_1..d_blk
                else:
                    key_blk = (key - k) // block_len
                    M[row, col] = 1 if key_blk == blk else 0     # own block only
    return M


def attn_dense(q, k_step, v_step, k_cache, v_cache, cache_len, *, k: int,
               num_blocks: int, block_len: int, sm_scale: float):
    """Masked softmax attention with the explicit matrix, per (b, head)."""
    q = np.asarray(q, np.float64)
    B, R, Hq, D = q.shape
    Hkv = k_step.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, R, Hq, D))
    lse = np.zeros((B, R, Hq))
    for b in range(B):
        P = int(cache_len[b])
        M = hybrid_mask_matrix(P, k, num_blocks, block_len).astype(bool)
        for h in range(Hq):
            kv = h // g
            K = np.concatenate([np.asarray(k_cache[b, kv, :P], np.float64),
                                np.asarray(k_step[b, :, kv], np.float64)])
            V = np.concatenate([np.asarray(v_cache[b, kv, :P], np.float64),
                                np.asarray(v_step[b, :, kv], np.float64)])
            S = sm_scale * (q[b, :, h] @ K.T)             # [R, P+R]
            S = np.where(M, S, -np.inf)
            mx = S.max(axis=1, keepdims=True)
            W = np.where(M, np.exp(S - mx), 0.0)
            Z = W.sum(axis=1, keepdims=True)
            out[b, :, h] = (W @ V) / Z
            lse[b, :, h] = (mx + np.log(Z))[:, 0]
    return out, lse
