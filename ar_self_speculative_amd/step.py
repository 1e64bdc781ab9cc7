"""One TiDAR decode step on device buffers: L x attention, verify, commit.

The call sequence of a step (TiDAR review, awesome-system-papers wiki,
核心方法 section 3.2; talk notes on notes.yuuk.io, 推論パイプライン): one
forward's hybrid-mask attention per layer, rejection sampling of the drafts
against the AR logits, then the exact-KV commit of the accepted drafts. The
accept length stays on the device between the sampler and the commit.
This class only owns buffers and issues library calls in order.
"""
from __future__ import annotations

import math

import torch

from . import _lib


class DecodeStep:
    def __init__(self, *, layers: int, batch: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, k: int, cache_capacity: int, max_cache_len: int, vocab: int,
                 dtype: int = _lib.DTYPE_BF16, sm_scale: float | None = None,
                 num_blocks: int | None = None, block_len: int | None = None,
                 num_splits: int = 0, device: str = "cuda", with_lse: bool = False,
                 trust_ar: float = 1.0):
        self.L, self.B, self.Hq, self.Hkv, self.D = layers, batch, num_q_heads, num_kv_heads, head_dim
        self.k = k
        self.trust_ar = trust_ar  # weight of the AR logits in the verification targets (1 = plain AR)
        self.num_blocks = k + 1 if num_blocks is None else num_blocks
        self.block_len = k if block_len is None else block_len
        self.R = k + self.num_blocks * self.block_len
        self.cap, self.max_len, self.V = cache_capacity, max_cache_len, vocab
        self.dtype = dtype
        tdt = torch.bfloat16 if dtype == _lib.DTYPE_BF16 else torch.float32
        scale = 1.0 / math.sqrt(head_dim) if sm_scale is None else sm_scale
        self.desc = _lib.make_attn_desc(
            batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
            k=k, num_blocks=self.num_blocks, block_len=self.block_len, cache_capacity=cache_capacity,
            max_cache_len=max_cache_len, sm_scale=scale, dtype=dtype, num_splits=num_splits)
        dev = torch.device(device)
        L, B, R, Hq, Hkv, D = layers, batch, self.R, num_q_heads, num_kv_heads, head_dim
        self.q = torch.empty((L, B, R, Hq, D), dtype=tdt, device=dev)
        self.k_step = torch.empty((L, B, R, Hkv, D), dtype=tdt, device=dev)
        self.v_step = torch.empty((L, B, R, Hkv, D), dtype=tdt, device=dev)
        self.k_cache = torch.empty((L, B, Hkv, cache_capacity, D), dtype=tdt, device=dev)
        self.v_cache = torch.empty((L, B, Hkv, cache_capacity, D), dtype=tdt, device=dev)
        self.out = torch.empty((L, B, R, Hq, D), dtype=tdt, device=dev)
        self.lse = torch.empty((L, B, R, Hq), dtype=torch.float32, device=dev) if with_lse else None
        self.cache_len = torch.zeros(B, dtype=torch.int32, device=dev)
        self.cache_len_out = torch.zeros(B, dtype=torch.int32, device=dev)
        self.ar_logits = torch.empty((B, k + 1, vocab), dtype=torch.float32, device=dev)
        self.diff_logits = torch.empty((B, max(k, 1), vocab), dtype=torch.float32, device=dev)[:, :k]
        self.drafts = torch.zeros((B, k), dtype=torch.int32, device=dev)
        self.uniforms = torch.zeros((B, k + 1), dtype=torch.float32, device=dev)
        self.accept_len = torch.zeros(B, dtype=torch.int32, device=dev)
        self.next_token = torch.zeros(B, dtype=torch.int32, device=dev)
        self.ratio = torch.zeros((B, k), dtype=torch.float32, device=dev)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.attn_ws = _lib.attn_workspace(self.desc, dev)
        rb = _lib.reject_workspace_bytes(B, k, vocab)
        self.rej_ws = torch.empty(max(rb, 256), dtype=torch.uint8, device=dev)

    def attention(self, layer: int, stream=None):
        _lib.attn_step(self.desc, self.q[layer], self.k_step[layer], self.v_step[layer],
                       self.k_cache[layer], self.v_cache[layer], self.cache_len, self.out[layer],
                       None if self.lse is None else self.lse[layer], self.dev_status,
                       self.attn_ws, stream)

    def verify(self, stream=None):
        _lib.reject_sample(ar_logits=self.ar_logits, diff_logits=self.diff_logits, drafts=self.drafts,
                           uniforms=self.uniforms, accept_len=self.accept_len, next_token=self.next_token,
                           ratio=self.ratio, dev_status=self.dev_status, workspace=self.rej_ws,
                           trust_ar=self.trust_ar, stream=stream)

    def commit(self, stream=None):
        _lib.kv_commit(num_layers=self.L, batch=self.B, num_kv_heads=self.Hkv, head_dim=self.D,
                       k=self.k, step_rows=self.R, cache_capacity=self.cap, max_cache_len=self.max_len,
                       dtype=self.dtype, k_step=self.k_step, v_step=self.v_step, k_cache=self.k_cache,
                       v_cache=self.v_cache, accept_len=self.accept_len, cache_len_in=self.cache_len,
                       cache_len_out=self.cache_len_out, dev_status=self.dev_status, stream=stream)

    def run(self, stream=None):
        """One whole step: every layer's attention, the verifier, the commit."""
        for layer in range(self.L):
            self.attention(layer, stream)
        self.verify(stream)
        self.commit(stream)

    def capture(self, fn=None):
        """Record fn (default: run) into a HIP graph and return it.

        The library calls only launch kernels on the given stream (no
        allocation, memset or synchronisation), so the whole step can be
        replayed with one launch from the host: g.replay().
        """
        fn = self.run if fn is None else fn
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g
