"""Helpers shared by the GPU parity tests: upload synthetic cases, call the
library through the binding, bring results back as numpy."""
from __future__ import annotations

import numpy as np
import torch

import ar_self_speculative_amd as tidar


def dev_array(case, name, layer=None):
    """Device tensor holding exactly the values of case.<name> (bf16 bits or f32)."""
    if case.bits is not None:
        a = case.bits[name] if layer is None else case.bits[name][layer]
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        a = getattr(case, name) if layer is None else getattr(case, name)[layer]
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t


def attn_desc(case, num_splits=0, max_cache_len=None):
    return tidar.make_attn_desc(
        batch=case.batch, num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
        head_dim=case.head_dim, k=case.k, num_blocks=case.num_blocks, block_len=case.block_len,
        cache_capacity=case.cache_capacity,
        max_cache_len=case.max_cache_len if max_cache_len is None else max_cache_len,
        sm_scale=case.sm_scale, dtype=tidar.DTYPE_BF16 if case.dtype == "bf16" else tidar.DTYPE_F32,
        num_splits=num_splits)


def run_attn(case, layer=0, num_splits=0, cache_len=None, max_cache_len=None, with_status=False):
    desc = attn_desc(case, num_splits, max_cache_len)
    q = dev_array(case, "q", layer)
    ks = dev_array(case, "k_step", layer)
    vs = dev_array(case, "v_step", layer)
    kc = dev_array(case, "k_cache", layer)
    vc = dev_array(case, "v_cache", layer)
    lens = torch.from_numpy(np.asarray(case.cache_len if cache_len is None else cache_len, np.int32)).cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsb = tidar.attn_workspace_bytes(desc)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda") if wsb else None
    tidar.attn_step(desc, q, ks, vs, kc, vc, lens, out, lse, status, ws)
    torch.cuda.synchronize()
    res = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    if with_status:
        return res + (int(status.item()),)
    return res


def oracle_inputs(case, layer=0):
    return (case.q[layer], case.k_step[layer], case.v_step[layer], case.k_cache[layer],
            case.v_cache[layer])


NEAR = 1e-5  # near-tie band of the sampler comparison (fraction of the total mass / of the accept probability)


def draw_candidates(ar_logits, diff_logits, b, n, u_last, temperature=1.0, eps=NEAR, trust_ar=1.0):
    """Tokens whose inverse-CDF interval meets [target - eps*total, target + eps*total].

    For a draw the oracle flags as a near-tie, the GPU's token must be one of
    these: a different rounding of the running sum can only move the draw
    across a boundary that lies inside the band.
    """
    import oracle

    k = ar_logits.shape[1] - 1
    p = oracle.softmax_t(oracle.target_logits(ar_logits[b, n], diff_logits[b, n] if n < k else None, trust_ar),
                         temperature)
    if n < k:
        w = np.maximum(0.0, p - oracle.softmax_t(diff_logits[b, n], temperature))
        if w.sum() == 0.0:
            w = p
    else:
        w = p
    cs = np.cumsum(w)
    total = cs[-1]
    target = float(u_last) * total
    lo = cs - w
    return np.nonzero((cs > target - eps * total) & (lo < target + eps * total) & (w > 0))[0]


def check_samples(ref, acc, nxt, ar_logits, diff_logits, uniforms, temperature=1.0, trust_ar=1.0):
    """Compare GPU (accept_len, next_token) with the oracle's SampleResult.

    Accept lengths must match unless an acceptance test the oracle consulted
    is a near-tie. With equal accept lengths the token must match, or (for a
    draw the oracle flags as a near-tie) lie in the band of boundary tokens.
    Returns (number of accept near-ties excused, number of draw near-ties).
    """
    B = len(acc)
    k = ar_logits.shape[1] - 1
    excused = draw_near = 0
    for b in range(B):
        if ref.accept_margin[b] < NEAR:
            excused += 1
            continue
        assert acc[b] == ref.accept_len[b], (b, int(acc[b]), int(ref.accept_len[b]))
        if ref.draw_margin[b] < NEAR:
            draw_near += 1
            cand = draw_candidates(ar_logits, diff_logits, b, int(acc[b]), uniforms[b, k], temperature,
                                   trust_ar=trust_ar)
            assert nxt[b] in cand, (b, int(nxt[b]), cand[:8])
        else:
            assert nxt[b] == ref.next_token[b], (b, int(nxt[b]), int(ref.next_token[b]))
    return excused, draw_near
