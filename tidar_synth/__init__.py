"""Seeded synthetic inputs for the TiDAR decode-step hot path.

This module only draws random numbers and arranges them in the documented
layouts. It holds none of the decode step's arithmetic (no attention, no
softmax, no acceptance test, no cache update), so both the fp64 oracle and the
GPU path can take their inputs from here without sharing any method code.

Layouts (row-major, contiguous):

* ``q``            [B, R, Hq, D]
* ``k_step/v_step`` [B, R, Hkv, D]   (per layer; stacked as [L, B, R, Hkv, D])
* ``k_cache/v_cache`` [B, Hkv, cap, D] (per layer; stacked as [L, B, Hkv, cap, D])
* ``ar_logits``    [B, k+1, V] fp32, ``diff_logits`` [B, k, V] fp32
* ``drafts``       [B, k] int32, ``uniforms`` [B, k+1] fp32 in [0, 1)

Step query rows are ordered: rows 0..k-1 are the drafts d_1..d_k, then
``k + j*block_len + m`` is mask token m of the pre-draft block for accept
length j (TiDAR paper, section 3.2 "parallel self-speculative generation":
prefix, last step's drafts, next step's pre-drafts in one forward).

bf16 inputs are drawn in fp32 and rounded to bf16 with round-to-nearest-even
(``torch.Tensor.to(torch.bfloat16)``); ``*_bits`` hold the uint16 patterns the
GPU reads and the matching float32 arrays hold exactly the same values for the
oracle.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "AttnCase", "SamplerCase", "bf16_round", "attn_case", "sampler_case",
    "draft_from_logits", "CONFIGS", "config_attn", "config_sampler",
    "commit_accept_lengths", "BF16_NAN_BITS",
]

BF16_NAN_BITS = np.uint16(0x7FC0)


def bf16_round(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 ``x`` to bf16 (RNE). Returns (uint16 bits, float32 values)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    vals = t.to(torch.float32).numpy().copy()
    return bits, vals


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class AttnCase:
    """One hybrid-mask attention problem (possibly several layers).

    Float arrays are float32 holding exactly the values the GPU reads; for
    bf16 cases the ``bits`` dict holds the uint16 patterns of the same arrays.
    ``k_cache``/``v_cache`` rows at or beyond ``cache_len[b]`` are filled with
    NaN when ``poison`` was requested, so a kernel that lets an invalid slot
    into the softmax or the PV product produces NaN.
    """

    dtype: str                 # "f32" or "bf16"
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    k: int
    num_blocks: int
    block_len: int
    cache_capacity: int
    cache_len: np.ndarray      # int32 [B]
    sm_scale: float
    q: np.ndarray              # [L, B, R, Hq, D]
    k_step: np.ndarray         # [L, B, R, Hkv, D]
    v_step: np.ndarray
    k_cache: np.ndarray        # [L, B, Hkv, cap, D]
    v_cache: np.ndarray
    bits: dict | None = None   # name -> uint16 array (bf16 only)

    @property
    def rows(self) -> int:
        return self.k + self.num_blocks * self.block_len

    @property
    def max_cache_len(self) -> int:
        return int(self.cache_len.max()) if self.cache_len.size else 0


def attn_case(*, dtype: str, layers: int, batch: int, num_q_heads: int,
              num_kv_heads: int, head_dim: int, k: int, num_blocks: int,
              block_len: int, cache_len, cache_capacity: int,
              sm_scale: float | None = None, qkv_scale: float = 1.0,
              seed: int = 0, poison: bool = True) -> AttnCase:
    """Draw Q, step K/V and cache K/V ~ N(0, qkv_scale^2) from ``seed``.

    Generation order is fixed: Q, K_step, V_step, K_cache, V_cache.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    R = k + num_blocks * block_len
    L, B, Hq, Hkv, D, cap = layers, batch, num_q_heads, num_kv_heads, head_dim, cache_capacity
    cache_len = np.broadcast_to(np.asarray(cache_len, dtype=np.int32), (B,)).copy()
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if qkv_scale != 1.0:
            x *= np.float32(qkv_scale)
        return x

    arrs = {
        "q": draw((L, B, R, Hq, D)),
        "k_step": draw((L, B, R, Hkv, D)),
        "v_step": draw((L, B, R, Hkv, D)),
        "k_cache": draw((L, B, Hkv, cap, D)),
        "v_cache": draw((L, B, Hkv, cap, D)),
    }
    bits = None
    if dtype == "bf16":
        bits = {}
        for name in list(arrs):
            b_, v_ = bf16_round(arrs[name])
            bits[name] = b_
            arrs[name] = v_
    elif dtype != "f32":
        raise ValueError(dtype)
    if poison:
        for b in range(B):
            for name in ("k_cache", "v_cache"):
                arrs[name][:, b, :, cache_len[b]:, :] = np.nan
                if bits is not None:
                    bits[name][:, b, :, cache_len[b]:, :] = BF16_NAN_BITS
    return AttnCase(dtype=dtype, layers=L, batch=B, num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, k=k, num_blocks=num_blocks,
                    block_len=block_len, cache_capacity=cap, cache_len=cache_len,
                    sm_scale=float(sm_scale), bits=bits, **arrs)


@dataclasses.dataclass
class SamplerCase:
    batch: int
    k: int
    vocab: int
    ar_logits: np.ndarray      # float32 [B, k+1, V]
    diff_logits: np.ndarray    # float32 [B, k, V]
    drafts: np.ndarray         # int32 [B, k]
    uniforms: np.ndarray       # float32 [B, k+1]
    temperature: float = 1.0


def draft_from_logits(diff_logits: np.ndarray, rng: np.random.Generator,
                      temperature: float = 1.0) -> np.ndarray:
    """One draw per row from softmax(diff_logits / T) by the Gumbel-max trick.

    This stands in for the model's one-step diffusion drafting (each mask
    position sampled from its own marginal): argmax(x/T + G) with G i.i.d.
    standard Gumbel is an exact draw from the softmax distribution.
    """
    u = rng.random(diff_logits.shape)  # float64 in [0, 1)
    u = np.maximum(u, np.finfo(np.float64).tiny)
    g = -np.log(-np.log(u))
    return np.argmax(diff_logits.astype(np.float64) / temperature + g, axis=-1).astype(np.int32)


def sampler_draws(*, batch: int, k: int, vocab: int, ar_sigma: float, seed: int = 0):
    """The first two draws of the verifier recipe from ``seed``: AR logits
    ~ N(0, ar_sigma) [B, k+1, V] and unit-normal noise [B, k, V] (float32),
    plus the generator positioned for the draws that follow."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ar = rng.standard_normal((batch, k + 1, vocab), dtype=np.float32) * np.float32(ar_sigma)
    z = rng.standard_normal((batch, k, vocab), dtype=np.float32)
    return ar, z, rng


def diffusion_logits(ar: np.ndarray, z: np.ndarray, diff_mode: str, diff_sigma: float) -> np.ndarray:
    """Diffusion logits from the recipe's noise: ``"independent"``: z * sigma;
    ``"noisy"``: AR logits of rows 0..k-1 + z * sigma (float32)."""
    k = z.shape[1]
    noise = z * np.float32(diff_sigma)
    if diff_mode == "independent":
        return np.ascontiguousarray(noise)
    if diff_mode == "noisy":
        return np.ascontiguousarray((ar[:, :k, :] + noise).astype(np.float32))
    raise ValueError(diff_mode)


def sampler_case(*, batch: int, k: int, vocab: int, ar_sigma: float,
                 diff_mode: str, diff_sigma: float, seed: int = 0,
                 temperature: float = 1.0) -> SamplerCase:
    """Synthetic verifier inputs.

    ``diff_mode="independent"``: diffusion logits ~ N(0, diff_sigma) drawn
    independently of the AR logits. ``diff_mode="noisy"``: diffusion logits =
    AR logits of rows 0..k-1 + N(0, diff_sigma) noise. Generation order: AR
    logits, diffusion logits/noise, draft-sampling draws, verify uniforms.
    """
    ar, z, rng = sampler_draws(batch=batch, k=k, vocab=vocab, ar_sigma=ar_sigma, seed=seed)
    diff = diffusion_logits(ar, z, diff_mode, diff_sigma)
    drafts = draft_from_logits(diff, rng, temperature) if k > 0 else np.zeros((batch, 0), np.int32)
    uniforms = rng.random((batch, k + 1), dtype=np.float32)
    return SamplerCase(batch=batch, k=k, vocab=vocab, ar_logits=ar,
                       diff_logits=diff, drafts=drafts,
                       uniforms=uniforms, temperature=temperature)


def commit_accept_lengths(batch: int, k: int, seed: int) -> np.ndarray:
    """Accept lengths n ~ U{0..k} (inclusive) for the standalone commit runs."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    return rng.integers(0, k + 1, size=batch, dtype=np.int32)


# --------------------------------------------------------------------------
# The five workloads. Shapes are Qwen-like single layers / full depth.
# --------------------------------------------------------------------------
CONFIGS = {
    1: dict(name="tiny-hybrid-f32", dtype="f32", layers=1, batch=1, num_q_heads=2,
            num_kv_heads=1, head_dim=64, P=128, k=4, vocab=512,
            sampler=dict(ar_sigma=2.0, diff_mode="independent", diff_sigma=2.0)),
    2: dict(name="qwen2.5-1.5b-layer-bf16", dtype="bf16", layers=1, batch=1, num_q_heads=12,
            num_kv_heads=2, head_dim=128, P=1024, k=16, vocab=151936,
            sampler=dict(ar_sigma=3.0, diff_mode="noisy", diff_sigma=1.0)),
    3: dict(name="qwen3-8b-36L-bf16", dtype="bf16", layers=36, batch=1, num_q_heads=32,
            num_kv_heads=8, head_dim=128, P=4096, k=16, vocab=151936,
            sampler=dict(ar_sigma=3.0, diff_mode="noisy", diff_sigma=1.0)),
    4: dict(name="qwen3-32b-layer-sweep-bf16", dtype="bf16", layers=1, batch=1, num_q_heads=64,
            num_kv_heads=8, head_dim=128, P=(512, 1024, 2048, 4096),
            R=(1, 8, 16, 32, 64, 128, 256, 512)),
    5: dict(name="qwen3-8b-ragged-b8-bf16", dtype="bf16", layers=36, batch=8, num_q_heads=32,
            num_kv_heads=8, head_dim=128, P_range=(256, 4096), k=8, cap=4608,
            vocab=151936, steps=64,
            # diffusion noise scale for a mean of ~7 committed tokens per step, found by
            # bisection on the oracle's closed-form acceptance (tests/golden/config5_sigma.json)
            sampler=dict(ar_sigma=3.0, diff_mode="noisy", diff_sigma=0.162)),
}

# verifier inputs of step `it` of the ragged batch come from seed CONFIG5_STEP_SEED0 + it
CONFIG5_STEP_SEED0 = 50


def config5_lengths(seed: int = 0) -> np.ndarray:
    """Prefix lengths of the ragged batch, U{256..4096} per sequence."""
    c = CONFIGS[5]
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    return rng.integers(c["P_range"][0], c["P_range"][1] + 1, size=c["batch"]).astype(np.int32)


def config5_step_sampler(it: int, *, diff_sigma: float | None = None) -> SamplerCase:
    """Verifier inputs of step ``it`` of the ragged-batch workload."""
    c = CONFIGS[5]
    s = dict(c["sampler"])
    if diff_sigma is not None:
        s["diff_sigma"] = diff_sigma
    return sampler_case(batch=c["batch"], k=c["k"], vocab=c["vocab"], seed=CONFIG5_STEP_SEED0 + it, **s)


def config_attn(n: int, *, seed: int = 0, layers: int | None = None, P: int | None = None,
                R: int | None = None, poison: bool = True) -> AttnCase:
    """Attention inputs for workload ``n`` (``layers`` may cut a full-depth case)."""
    c = CONFIGS[n]
    L = c["layers"] if layers is None else layers
    if n in (1, 2, 3):
        k = c["k"]
        return attn_case(dtype=c["dtype"], layers=L, batch=c["batch"],
                         num_q_heads=c["num_q_heads"], num_kv_heads=c["num_kv_heads"],
                         head_dim=c["head_dim"], k=k, num_blocks=k + 1, block_len=k,
                         cache_len=c["P"], cache_capacity=c["P"] + k, seed=seed,
                         poison=poison)
    if n == 4:
        # Append-prefill: R new tokens, causal among themselves, over a prefix P.
        P = c["P"][-1] if P is None else P
        R = 32 if R is None else R
        return attn_case(dtype="bf16", layers=L, batch=1, num_q_heads=c["num_q_heads"],
                         num_kv_heads=c["num_kv_heads"], head_dim=c["head_dim"], k=R,
                         num_blocks=0, block_len=1, cache_len=P, cache_capacity=P + R,
                         seed=seed, poison=poison)
    if n == 5:
        lens = config5_lengths(seed)
        k = c["k"]
        return attn_case(dtype="bf16", layers=L, batch=c["batch"], num_q_heads=c["num_q_heads"],
                         num_kv_heads=c["num_kv_heads"], head_dim=c["head_dim"], k=k,
                         num_blocks=k + 1, block_len=k, cache_len=lens,
                         cache_capacity=c["cap"], seed=seed, poison=poison)
    raise KeyError(n)


def config_sampler(n: int, *, seed: int = 0, diff_sigma: float | None = None,
                   batch: int | None = None) -> SamplerCase:
    c = CONFIGS[n]
    s = dict(c.get("sampler", dict(ar_sigma=3.0, diff_mode="noisy", diff_sigma=1.0)))
    if diff_sigma is not None:
        s["diff_sigma"] = diff_sigma
    return sampler_case(batch=c["batch"] if batch is None else batch, k=c["k"],
                        vocab=c["vocab"], seed=seed + 1, **s)


def fill_verifier_device(ar_logits, diff_logits, drafts, uniforms, g, *, ar_sigma: float = 3.0,
                         diff_sigma: float = 1.0, temperature: float = 1.0) -> None:
    """Verifier inputs on the device from torch generator ``g``, same recipe
    as sampler_case: AR logits ~ N(0, ar_sigma), diffusion logits = AR of
    rows 0..k-1 + N(0, diff_sigma), drafts by Gumbel-max from the diffusion
    logits, uniforms in [0, 1). Buffers: [B, k+1, V], [B, k, V], [B, k], [B, k+1]."""
    import torch

    dev = ar_logits.device
    ar_logits.normal_(generator=g).mul_(ar_sigma)
    k = diff_logits.shape[1]
    if k:
        noise = torch.randn(diff_logits.shape, generator=g, device=dev) * diff_sigma
        diff_logits.copy_(ar_logits[:, :k] + noise)
        u = torch.rand(diff_logits.shape, generator=g, device=dev).clamp_min(1e-30)
        gumbel = -torch.log(-torch.log(u))
        drafts.copy_(torch.argmax(diff_logits / temperature + gumbel, dim=-1).to(torch.int32))
        del noise, u, gumbel
    uniforms.copy_(torch.rand(uniforms.shape, generator=g, device=dev))


def fill_device_step(step, *, seed: int, cache_len, ar_sigma: float = 3.0,
                     diff_sigma: float = 1.0, temperature: float = 1.0) -> None:
    """Fill the buffers of a decode step on its device with a seeded torch RNG.

    Same recipe as the numpy generators (Q/K/V ~ N(0, 1) rounded to the
    buffer dtype, AR logits ~ N(0, ar_sigma), diffusion logits = AR + N(0,
    diff_sigma), drafts by Gumbel-max from the diffusion logits, uniforms in
    [0, 1)), but drawn on the GPU so full-depth workloads set up in seconds.
    Cache rows at or beyond each sequence's length are left as NaN.
    """
    import torch

    dev = step.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def normal_(t):
        if t.dtype == torch.bfloat16:
            # draw in fp32, round once to bf16
            for i in range(t.shape[0]):
                t[i].copy_(torch.randn(t[i].shape, generator=g, device=dev, dtype=torch.float32))
        else:
            t.normal_(generator=g)

    for t in (step.q, step.k_step, step.v_step, step.k_cache, step.v_cache):
        normal_(t)
    lens = torch.as_tensor(np.broadcast_to(np.asarray(cache_len, np.int32), (step.B,)).copy())
    step.cache_len.copy_(lens.to(dev))
    step.cache_len_out.copy_(lens.to(dev))
    pos = torch.arange(step.cap, device=dev)
    invalid = pos[None, :] >= step.cache_len[:, None]          # [B, cap]
    mask = invalid[None, :, None, :, None]
    step.k_cache.masked_fill_(mask, float("nan"))
    step.v_cache.masked_fill_(mask, float("nan"))
    fill_verifier_device(step.ar_logits, step.diff_logits, step.drafts, step.uniforms, g,
                         ar_sigma=ar_sigma, diff_sigma=diff_sigma, temperature=temperature)
    step.accept_len.zero_()
    step.next_token.zero_()
    step.dev_status.zero_()
