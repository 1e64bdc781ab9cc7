"""The TiDAR decode-step loop on the GPU, around the hot path.

A small Qwen-style decoder with random bf16 weights stands in for the model
(no trained weights are involved): token embedding, per layer RMSNorm ->
Q/K/V projections -> rotary position embedding -> hybrid-mask attention
(libtidar) -> output projection -> RMSNorm -> SwiGLU MLP, then a final
RMSNorm and the LM head. The dense layers use torch (hipBLASLt GEMMs); the
attention, the verification sampler and the exact-KV commit are the
library's kernels.

The loop follows the TiDAR review (awesome-system-papers wiki, 核心方法
§3.2) and the talk notes' 推論パイプライン (notes.yuuk.io): one forward
verifies the previous step's drafts with causal logits and pre-drafts the
next step for every accept length; the block for the actual accept length
supplies the next drafts; only the accepted rows' KV is committed. The pages
never align rows; the scheme used here is:

* a step feeds k region rows [c, d_1..d_{k-1}] at positions len + i, where c
  is the token the AR side sampled last step (its KV is computed now, with
  no recomputation) and d_i are the drafts, then k + 1 blocks of k mask
  tokens, block j at positions len + j + m and seeing region rows 0..j-1;
* region row i's logits verify region row i + 1, row k - 1 is the bonus row;
  the diffusion logits that proposed the drafts are carried from last step;
* region rows 0..n are committed (n accepted drafts), the sampler's token c'
  heads the next region, and masks 1..k-1 of block n + 1 give the next drafts
  (inverse CDF with their own uniforms);
* the loop starts from a causal prefill of the prompt (the attention's
  num_blocks = 0 mode): c_0 comes from the last prompt row and the first
  drafts from the uniform distribution.
"""
from __future__ import annotations

import math

import torch

from . import _lib


class TinyDecoder:
    """Random-weight Qwen-style decoder (bf16 weights, fp32 norms and rotary)."""

    def __init__(self, *, vocab: int = 512, hidden: int = 256, layers: int = 2, num_q_heads: int = 4,
                 num_kv_heads: int = 2, head_dim: int = 64, mlp: int = 512, rope_theta: float = 1e6,
                 eps: float = 1e-6, seed: int = 0, device: str = "cuda"):
        self.V, self.H, self.L = vocab, hidden, layers
        self.Hq, self.Hkv, self.D, self.mlp = num_q_heads, num_kv_heads, head_dim, mlp
        self.theta, self.eps = rope_theta, eps
        self.mask_id = vocab - 1
        dev = torch.device(device)
        gen = torch.Generator(device=dev).manual_seed(seed)

        def w(shape, fan_in):
            return (torch.randn(shape, generator=gen, device=dev) / math.sqrt(fan_in)).to(torch.bfloat16)

        def norm_w():
            return (1.0 + 0.1 * torch.randn(hidden, generator=gen, device=dev)).to(torch.bfloat16)

        self.emb = w((vocab, hidden), 1.0)
        self.layers = []
        for _ in range(layers):
            self.layers.append(dict(
                ln1=norm_w(), wq=w((hidden, num_q_heads * head_dim), hidden),
                wk=w((hidden, num_kv_heads * head_dim), hidden), wv=w((hidden, num_kv_heads * head_dim), hidden),
                wo=w((num_q_heads * head_dim, hidden), num_q_heads * head_dim), ln2=norm_w(),
                wg=w((hidden, mlp), hidden), wu=w((hidden, mlp), hidden), wd=w((mlp, hidden), mlp)))
        self.norm_f = norm_w()
        self.lm_head = w((hidden, vocab), hidden)
        half = head_dim // 2
        self.inv_freq = 1.0 / (rope_theta ** (torch.arange(half, device=dev, dtype=torch.float32) / half))

    def rmsnorm(self, x, w):
        xf = x.float()
        return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + self.eps) * w.float()).to(torch.bfloat16)

    def rope(self, x, pos):
        """Rotary embedding, rotate-half form, angle pos * theta^(-2i/D); x [B,R,H,D], pos [B,R]."""
        ang = pos.float()[..., None] * self.inv_freq          # [B, R, D/2]
        cos, sin = ang.cos()[:, :, None, :], ang.sin()[:, :, None, :]
        xf = x.float()
        x1, x2 = xf[..., : self.D // 2], xf[..., self.D // 2:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1).to(torch.bfloat16)

    def forward(self, tokens, positions, k_step, v_step, attend):
        """Logits [B, R, V] (fp32) for tokens [B, R] at positions [B, R].

        Writes each layer's rotated keys and values into k_step[l] / v_step[l]
        ([B, R, Hkv, D]); attend(l, q) returns the attention output
        [B, R, Hq, D] of layer l (it reads k_step[l] / v_step[l]).
        """
        B, R = tokens.shape
        x = self.emb[tokens]
        for l, p in enumerate(self.layers):
            h = self.rmsnorm(x, p["ln1"])
            q = self.rope((h @ p["wq"]).view(B, R, self.Hq, self.D), positions)
            k_step[l].copy_(self.rope((h @ p["wk"]).view(B, R, self.Hkv, self.D), positions))
            v_step[l].copy_((h @ p["wv"]).view(B, R, self.Hkv, self.D))
            o = attend(l, q.contiguous())
            x = x + o.view(B, R, self.Hq * self.D) @ p["wo"]
            h2 = self.rmsnorm(x, p["ln2"])
            x = x + (torch.nn.functional.silu(h2 @ p["wg"]) * (h2 @ p["wu"])) @ p["wd"]
        return (self.rmsnorm(x, self.norm_f) @ self.lm_head).float()


class TiDARLoop:
    """Batched TiDAR generation with k region rows per step (k - 1 drafts)."""

    def __init__(self, model: TinyDecoder, *, batch: int, k: int, cache_capacity: int,
                 temperature: float = 1.0, trust_ar: float = 1.0, device: str = "cuda"):
        if k < 1:
            raise ValueError("k must be >= 1")
        m = model
        self.m, self.B, self.k, self.cap = m, batch, k, cache_capacity
        self.R = k + (k + 1) * k
        self.T, self.trust_ar = temperature, trust_ar
        dev = self.dev = torch.device(device)
        self.k_cache = torch.zeros((m.L, batch, m.Hkv, cache_capacity, m.D), dtype=torch.bfloat16, device=dev)
        self.v_cache = torch.zeros_like(self.k_cache)
        self.cache_len = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.cache_len_out = torch.zeros_like(self.cache_len)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.k_step = torch.empty((m.L, batch, self.R, m.Hkv, m.D), dtype=torch.bfloat16, device=dev)
        self.v_step = torch.empty_like(self.k_step)
        self.attn_out = torch.empty((batch, self.R, m.Hq, m.D), dtype=torch.bfloat16, device=dev)
        self.desc = _lib.make_attn_desc(batch=batch, num_q_heads=m.Hq, num_kv_heads=m.Hkv, head_dim=m.D, k=k,
                                        num_blocks=k + 1, block_len=k, cache_capacity=cache_capacity,
                                        max_cache_len=cache_capacity - k, sm_scale=1.0 / math.sqrt(m.D),
                                        dtype=_lib.DTYPE_BF16)
        self.attn_ws = _lib.attn_workspace(self.desc, dev)
        # row offsets of a step: region row i at len + i, block j mask m at len + j + m
        offs = list(range(k)) + [j + mm for j in range(k + 1) for mm in range(k)]
        self.offsets = torch.tensor(offs, dtype=torch.int64, device=dev)
        self.block_m = torch.arange(1, k, dtype=torch.int64, device=dev)
        self.region = torch.zeros((batch, k), dtype=torch.int32, device=dev)
        self.q_logits = torch.zeros((batch, max(k - 1, 1), m.V), dtype=torch.float32, device=dev)[:, : k - 1]
        self.accept_len = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.next_token = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.rej_ws = torch.empty(max(_lib.reject_workspace_bytes(batch, k - 1, m.V), 256), dtype=torch.uint8,
                                  device=dev)
        nd = max(batch * (k - 1), 1)
        self.draft_ws = torch.empty(max(_lib.reject_workspace_bytes(nd, 0, m.V), 256), dtype=torch.uint8,
                                    device=dev)
        self.draft_tok = torch.zeros(nd, dtype=torch.int32, device=dev)
        self.draft_n = torch.zeros(nd, dtype=torch.int32, device=dev)
        self.last_logits = None

    # -- helpers ---------------------------------------------------------
    def _categorical(self, logits2d, uniforms, out_tok, out_n, ws):
        """Inverse-CDF draw from softmax(logits / T) per row: the sampler with no drafts."""
        n = logits2d.shape[0]
        _lib.reject_sample(ar_logits=logits2d.view(n, 1, -1), diff_logits=None, drafts=None,
                           uniforms=uniforms.reshape(n, 1).contiguous(), accept_len=out_n, next_token=out_tok,
                           dev_status=self.status, workspace=ws, temperature=self.T)

    def _commit(self, k_step, v_step, n_rows, rows_in_step, k_max):
        _lib.kv_commit(num_layers=self.m.L, batch=self.B, num_kv_heads=self.m.Hkv, head_dim=self.m.D, k=k_max,
                       step_rows=rows_in_step, cache_capacity=self.cap, max_cache_len=self.cap - k_max,
                       dtype=_lib.DTYPE_BF16, k_step=k_step, v_step=v_step, k_cache=self.k_cache,
                       v_cache=self.v_cache, accept_len=n_rows, cache_len_in=self.cache_len,
                       cache_len_out=self.cache_len_out, dev_status=self.status)
        self.cache_len.copy_(self.cache_len_out)

    # -- the loop --------------------------------------------------------
    def prefill(self, prompt, u_first, u_drafts):
        """Causal forward over prompt [B, P0] (int64), commit it, draw c_0 and the first drafts."""
        m, B, k = self.m, self.B, self.k
        P0 = prompt.shape[1]
        if P0 + 1 > self.cap - k:
            raise ValueError("prompt does not fit the cache")
        desc = _lib.make_attn_desc(batch=B, num_q_heads=m.Hq, num_kv_heads=m.Hkv, head_dim=m.D, k=P0,
                                   num_blocks=0, block_len=1, cache_capacity=self.cap,
                                   max_cache_len=self.cap - P0, sm_scale=1.0 / math.sqrt(m.D),
                                   dtype=_lib.DTYPE_BF16)
        ws = _lib.attn_workspace(desc, self.dev)
        ks = torch.empty((m.L, B, P0, m.Hkv, m.D), dtype=torch.bfloat16, device=self.dev)
        vs = torch.empty_like(ks)
        out = torch.empty((B, P0, m.Hq, m.D), dtype=torch.bfloat16, device=self.dev)
        self.cache_len.zero_()

        def attend(l, q):
            _lib.attn_step(desc, q, ks[l], vs[l], self.k_cache[l], self.v_cache[l], self.cache_len, out, None,
                           self.status, ws)
            return out

        pos = torch.arange(P0, device=self.dev, dtype=torch.int64).expand(B, P0)
        logits = m.forward(prompt, pos, ks, vs, attend)
        self._commit(ks, vs, torch.full((B,), P0, dtype=torch.int32, device=self.dev), P0, P0)
        c0 = torch.zeros(B, dtype=torch.int32, device=self.dev)
        n0 = torch.zeros(B, dtype=torch.int32, device=self.dev)
        ws0 = torch.empty(max(_lib.reject_workspace_bytes(B, 0, m.V), 256), dtype=torch.uint8, device=self.dev)
        self._categorical(logits[:, P0 - 1].contiguous(), u_first, c0, n0, ws0)
        self.region[:, 0] = c0
        if k > 1:
            self.q_logits.zero_()              # uniform proposals for the first drafts
            self._categorical(torch.zeros((B * (k - 1), m.V), device=self.dev), u_drafts, self.draft_tok,
                              self.draft_n, self.draft_ws)
            self.region[:, 1:] = self.draft_tok.view(B, k - 1)
        self.last_logits = logits
        return logits

    def step(self, u_verify, u_draft):
        """One TiDAR step: forward, verification, commit, next drafts (all on the device).

        u_verify [B, k] (k - 1 acceptance tests and the final draw), u_draft
        [B, k - 1]. Leaves accept_len (n), next_token (c') and the next
        region / proposals in place; returns the step's logits [B, R, V].
        """
        m, B, k, R = self.m, self.B, self.k, self.R
        tokens = torch.full((B, R), m.mask_id, dtype=torch.int64, device=self.dev)
        tokens[:, :k] = self.region.long()
        pos = self.cache_len.long()[:, None] + self.offsets[None, :]

        def attend(l, q):
            _lib.attn_step(self.desc, q, self.k_step[l], self.v_step[l], self.k_cache[l], self.v_cache[l],
                           self.cache_len, self.attn_out, None, self.status, self.attn_ws)
            self.last_q = q
            return self.attn_out

        self.last_tokens, self.last_pos = tokens, pos
        self.last_cache_len = self.cache_len.clone()

        logits = m.forward(tokens, pos, self.k_step, self.v_step, attend)
        ar = logits[:, :k].contiguous()
        _lib.reject_sample(ar_logits=ar, diff_logits=self.q_logits.contiguous() if k > 1 else None,
                           drafts=self.region[:, 1:].contiguous() if k > 1 else None,
                           uniforms=u_verify.contiguous(), accept_len=self.accept_len, next_token=self.next_token,
                           dev_status=self.status, workspace=self.rej_ws, temperature=self.T,
                           trust_ar=self.trust_ar)
        self._commit(self.k_step, self.v_step, self.accept_len + 1, R, k)
        if k > 1:
            rows = k + (self.accept_len.long()[:, None] + 1) * k + self.block_m[None, :]   # block n+1, masks 1..k-1
            self.q_logits.copy_(torch.gather(logits, 1, rows[:, :, None].expand(B, k - 1, m.V)))
            self._categorical(self.q_logits.reshape(B * (k - 1), m.V), u_draft, self.draft_tok, self.draft_n,
                              self.draft_ws)
            self.region[:, 1:] = self.draft_tok.view(B, k - 1)
        self.region[:, 0] = self.next_token
        self.last_logits = logits
        return logits
