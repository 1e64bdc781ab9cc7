"""Exact-KV commit after verification: append accepted drafts, evict the rest.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* TiDAR review (awesome-system-papers wiki), "核心方法" §3.2: when fewer drafts
  are accepted than were drafted, the surplus KV is evicted with no
  recomputation; §3.3: exact KV cache as in Block Diffusion.
* yuuk.io talk notes, "厳密 KV キャッシュ対応": the AR part of the cache is
  reused exactly, with no extra computation.

Reading: the KV of draft rows 0..n-1 of this step (computed causally in this
forward) is appended after the committed prefix; rejected draft rows and all
pre-draft rows are never written. Accepted rows are always a prefix of the
drafts, so the valid cache stays one contiguous run [0, len + n).
"""
from __future__ import annotations

import numpy as np


def kv_commit(k_step, v_step, k_cache, v_cache, accept_len, cache_len):
    """Return (new_k_cache, new_v_cache, new_cache_len); inputs are not modified.

    k_step/v_step [L, B, R, Hkv, D]; k_cache/v_cache [L, B, Hkv, cap, D];
    accept_len, cache_len [B]. Works on any dtype (bf16 as uint16 bits), so
    results are exact copies.
    """
    new_k = np.array(k_cache, copy=True)
    new_v = np.array(v_cache, copy=True)
    L, B, R, Hkv, D = k_step.shape
    for b in range(B):
        n = int(accept_len[b])
        start = int(cache_len[b])
        for layer in range(L):
            for h in range(Hkv):
                for i in range(n):
                    new_k[layer, b, h, start + i, :] = k_step[layer, b, i, h, :]
                    new_v[layer, b, h, start + i, :] = v_step[layer, b, i, h, :]
    new_len = np.asarray(cache_len, np.int64) + np.asarray(accept_len, np.int64)
    return new_k, new_v, new_len.astype(np.int32)
