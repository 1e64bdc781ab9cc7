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


def run_attn(case, layer=0, num_splits=0, cache_len=None, max_cache_len=None, with_status=False, with_lse=True):
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
    tidar.attn_step(desc, q, ks, vs, kc, vc, lens, out, lse if with_lse else None, status, ws)
    torch.cuda.synchronize()
    res = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64) if with_lse else None)
    if with_status:
        return res + (int(status.item()),)
    return res


def oracle_inputs(case, layer=0):
    return (case.q[layer], case.k_step[layer], case.v_step[layer], case.k_cache[layer],
            case.v_cache[layer])


NEAR = 1e-5  # acceptance near-tie band: |u_i - min(1, rho_i)| below it (the stated tolerance for accept draws)

# Draw band, in probability units (the draw weights normalised so that p sums
# to one). The GPU forms every weight in fp32 from per-row statistics
# (maximum, sum of exponentials over 151936 tokens in 4096-token chunks) and
# scans them in fp64. A weight's relative error is a few 1e-7 (the exponent
# y*log2(e)/T - m*log2(e) rounded in fp32 at |y*log2(e)| ~ 20, v_exp_f32, the
# reciprocal of the sum), so a running sum over weights that total at most
# one (p) or two (p and q of a residual) moves by at most ~1e-6 per
# distribution. A draw whose target lies closer than this to a CDF boundary
# may fall on the token across it.
DRAW_EPS = 2e-6


def draw_weights(ar_logits, diff_logits, b, n, temperature=1.0, trust_ar=1.0):
    """The oracle's (unnormalised) draw weights after accept length n: the
    residual max(0, p_n - q_n) (p_n when it vanishes), or p_k for the bonus."""
    import oracle

    k = ar_logits.shape[1] - 1
    p = oracle.softmax_t(oracle.target_logits(ar_logits[b, n], diff_logits[b, n] if n < k else None, trust_ar),
                         temperature)
    if n < k:
        w = np.maximum(0.0, p - oracle.softmax_t(diff_logits[b, n], temperature))
        if w.sum() == 0.0:
            w = p
        return w
    return p


def draw_candidates(w, u_last, eps_abs=DRAW_EPS):
    """Tokens an inverse-CDF draw with uniform u_last may return under weights
    w when the running sums carry an absolute error up to eps_abs: the
    oracle's token, and any token whose interval meets
    [target - eps_abs, target + eps_abs]."""
    import oracle

    t_ref, _ = oracle.invcdf(w, float(u_last))
    cs = np.cumsum(w)
    target = float(u_last) * cs[-1]
    lo = cs - w
    near = np.nonzero((cs > target - eps_abs) & (lo < target + eps_abs) & (w > 0))[0]
    return sorted(set(near.tolist()) | {int(t_ref)})


def accept_outcomes(ratio_b, u_b, n_ref, k):
    """Accept lengths the GPU may return for one sequence: the oracle's n, and
    for each consulted acceptance test that is a near-tie, the chain with that
    one test flipped (the later tests as the oracle evaluates them)."""
    outs = {int(n_ref)}
    a = np.minimum(1.0, ratio_b)
    for i in range(min(int(n_ref) + 1, k)):          # tests 0..n consulted (n = the rejecting one)
        if abs(float(u_b[i]) - a[i]) >= NEAR:
            continue
        if i < n_ref:                                 # an acceptance turned into the rejection
            outs.add(i)
        else:                                         # the rejection turned into an acceptance
            n = i + 1
            while n < k and float(u_b[n]) < a[n]:
                n += 1
            outs.add(n)
    return outs


def check_sequence(ref, b, acc_b, nxt_b, ar_logits, diff_logits, uniforms, temperature=1.0, trust_ar=1.0):
    """One sequence of check_samples. Returns (accept length differs from the
    oracle's, token differs from the oracle's draw at the GPU's accept length)."""
    import oracle

    k = ar_logits.shape[1] - 1
    outs = accept_outcomes(ref.ratio[b], uniforms[b], ref.accept_len[b], k)
    assert int(acc_b) in outs, (b, int(acc_b), int(ref.accept_len[b]), sorted(outs))
    n = int(acc_b)
    if n == ref.accept_len[b] and ref.draw_margin[b] * ref.residual_mass[b] >= DRAW_EPS:
        assert nxt_b == ref.next_token[b], (b, int(nxt_b), int(ref.next_token[b]))
        return False, False
    w = draw_weights(ar_logits, diff_logits, b, n, temperature, trust_ar)
    cand = draw_candidates(w, uniforms[b, k])
    assert int(nxt_b) in cand, (b, n, int(nxt_b), cand[:8])
    return n != ref.accept_len[b], int(nxt_b) != oracle.invcdf(w, float(uniforms[b, k]))[0]


def check_samples(ref, acc, nxt, ar_logits, diff_logits, uniforms, temperature=1.0, trust_ar=1.0):
    """Compare GPU (accept_len, next_token) with the oracle's SampleResult.

    The accept length must be the oracle's, or (where a consulted acceptance
    test is within NEAR of its threshold) the oracle's chain with that one
    test flipped. The token must be the oracle's inverse-CDF draw for the
    accept length the GPU returned, or a token whose interval lies within
    DRAW_EPS of that draw's target (the GPU's rounding of the running sums).
    Returns (accept lengths that differ from the oracle's, tokens that differ
    from the oracle's draw at the GPU's accept length).
    """
    B = len(acc)
    acc_diff = draw_diff = 0
    for b in range(B):
        a, d = check_sequence(ref, b, acc[b], nxt[b], ar_logits, diff_logits, uniforms, temperature, trust_ar)
        acc_diff += int(a)
        draw_diff += int(d)
    # a differing token needs a target within DRAW_EPS of a boundary; with
    # healthy arithmetic that is rare
    assert draw_diff <= max(2, B // 20), (draw_diff, B)
    return acc_diff, draw_diff
