"""AR rejection sampling of the diffusion drafts, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* TiDAR review (awesome-system-papers wiki), "核心方法" §3.2: last step's
  drafts are proposals from the diffusion marginals and are verified by
  rejection sampling against this step's causal (AR) logits; the pre-drafted
  block for the resulting accept length is taken for the next step.
* yuuk.io talk notes, "推論パイプライン" step 3: tokens after the first rejected
  one are discarded.
* The acceptance rule is that of speculative sampling (Leviathan et al., 2023;
  Chen et al., 2023): draft d_{i+1} ~ q_i is kept with probability
  min(1, p_i(d)/q_i(d)); at the first rejection a replacement is drawn from
  the normalised residual max(0, p_i - q_i); if every draft is kept, one bonus
  token is drawn from the last AR distribution p_k. The committed tokens are
  then distributed exactly as the AR chain.

* TiDAR review, "设计取舍" (trust AR vs trust diffusion, Fig. 6): at
  verification the AR and diffusion logits can be mixed with a weight lambda;
  the quality barely moves across lambda, which the review reads as the AR
  rejection-sampling step (not either mode's knowledge) setting the
  quality/speed trade-off.

Readings where the pages are silent:
* p_i = softmax(ar_logits[i] / T) for i = 0..k, q_i = softmax(diff_logits[i]/T)
  for i = 0..k-1; row i of the AR logits is the target for draft d_{i+1} and
  row k is the bonus row.
* uniforms[0..k-1] drive the acceptance tests (accept iff u_i < min(1, rho_i),
  strict), uniforms[k] drives the replacement / bonus draw.
* q_i(d) = 0 reads as rho = +inf (accept).
* An all-zero residual (possible only through rounding) falls back to p_n.
* invcdf(w, u): smallest token id t (scanning in id order) whose running sum
  of w exceeds u * sum(w); if rounding leaves none, the largest t with w_t > 0.
* Trust mixing (trust_ar = lambda): the target of draft d_{i+1} becomes
  softmax((lambda * ar_logits[i] + (1 - lambda) * diff_logits[i]) / T), mixed
  in logit space on the diffusion row that proposed the draft; the proposal
  q_i is unchanged, and the bonus row k has no diffusion counterpart so it
  stays pure AR. lambda = 1 is the plain sampler (trust AR) and lambda = 0
  takes the diffusion logits as the target (trust diffusion); these two end
  points use the respective logits as they are, so infinite logits need no
  0 * inf.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def softmax_t(logits, temperature: float = 1.0) -> np.ndarray:
    """softmax(logits / T) in fp64 with the maximum subtracted first."""
    z = np.asarray(logits, np.float64) / temperature
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def invcdf(w: np.ndarray, u: float) -> tuple[int, float]:
    """Inverse-CDF draw from the (unnormalised) weights ``w`` with uniform ``u``.

    Returns (token, margin) where margin is the distance of u*sum(w) to the
    nearest edge of the chosen token's CDF interval, divided by sum(w)
    (used to flag draws that sit on a boundary).
    """
    w = np.asarray(w, np.float64)
    cs = np.cumsum(w)                       # running sum in token-id order
    total = cs[-1]
    target = float(u) * total
    above = np.nonzero(cs > target)[0]
    if above.size:
        t = int(above[0])
    else:
        t = int(np.nonzero(w > 0)[0][-1])
    lo = cs[t] - w[t]
    hi = cs[t]
    margin = min(abs(target - lo), abs(hi - target)) / total if total > 0 else 0.0
    return t, margin


@dataclasses.dataclass
class SampleResult:
    accept_len: np.ndarray    # int32 [B]
    next_token: np.ndarray    # int32 [B]
    ratio: np.ndarray         # float64 [B, k]: p_i(d_{i+1}) / q_i(d_{i+1})
    accept_margin: np.ndarray  # float64 [B]: min |u_i - min(1, rho_i)| over consulted tests
    draw_margin: np.ndarray   # float64 [B]: invcdf boundary margin of the final draw
    residual_mass: np.ndarray  # float64 [B]: sum(max(0, p_n - q_n)), or 1 for the bonus draw


def target_logits(ar_row, diff_row, trust_ar: float = 1.0) -> np.ndarray:
    """Logits of the verification target for one draft position (fp64).

    diff_row is None for the bonus row. Mixing as in the review's trust
    AR / trust diffusion comparison: lambda * AR + (1 - lambda) * diffusion.
    """
    a = np.asarray(ar_row, np.float64)
    if diff_row is None or trust_ar == 1.0:
        return a
    d = np.asarray(diff_row, np.float64)
    if trust_ar == 0.0:
        return d
    return trust_ar * a + (1.0 - trust_ar) * d


def reject_sample(ar_logits, diff_logits, drafts, uniforms, temperature: float = 1.0,
                  trust_ar: float = 1.0) -> SampleResult:
    """Verify k drafts per sequence and draw the correction / bonus token.

    ar_logits [B, k+1, V], diff_logits [B, k, V], drafts [B, k] int,
    uniforms [B, k+1]; trust_ar in [0, 1] mixes the targets (1 = plain AR).
    Returns accept lengths n in 0..k and next_token c.
    """
    if not (0.0 <= trust_ar <= 1.0):
        raise ValueError("trust_ar must lie in [0, 1]")
    ar_logits = np.asarray(ar_logits)
    diff_logits = np.asarray(diff_logits)
    B, kp1, V = ar_logits.shape
    k = kp1 - 1
    acc = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    ratio = np.zeros((B, k))
    amarg = np.full(B, np.inf)
    dmarg = np.zeros(B)
    rmass = np.zeros(B)
    for b in range(B):
        p = [softmax_t(target_logits(ar_logits[b, i], diff_logits[b, i] if i < k else None, trust_ar),
                       temperature) for i in range(k + 1)]
        q = [softmax_t(diff_logits[b, i], temperature) for i in range(k)]
        for i in range(k):
            d = int(drafts[b, i])
            ratio[b, i] = p[i][d] / q[i][d] if q[i][d] > 0 else np.inf
        n = 0
        for i in range(k):
            a = min(1.0, ratio[b, i])
            u = float(uniforms[b, i])
            amarg[b] = min(amarg[b], abs(u - a))
            if u < a:
                n += 1
            else:
                break
        if n < k:
            resid = np.maximum(0.0, p[n] - q[n])
            if resid.sum() == 0.0:
                resid = p[n]
            c, dm = invcdf(resid, float(uniforms[b, k]))
            rmass[b] = resid.sum()
        else:
            c, dm = invcdf(p[k], float(uniforms[b, k]))
            rmass[b] = 1.0
        acc[b] = n
        nxt[b] = c
        dmarg[b] = dm
    return SampleResult(acc, nxt, ratio, amarg, dmarg, rmass)


def expected_accept_len(ar_logits, diff_logits, temperature: float = 1.0, trust_ar: float = 1.0) -> np.ndarray:
    """E[n] per sequence under the speculative-sampling rule, in closed form.

    A draft d ~ q_m is kept with probability min(1, p_m(d)/q_m(d)), so
    averaged over d the test passes with probability
    alpha_m = sum_t min(p_m(t), q_m(t)); the tests run in order and stop at
    the first rejection, so P(n >= i) = prod_{m < i} alpha_m and
    E[n] = sum_{i=1..k} prod_{m < i} alpha_m (Leviathan et al., 2023).
    Shapes as in reject_sample; returns float64 [B]. Committed tokens per step
    (the pages' tokens per forward) are E[n] + 1.
    """
    ar_logits = np.asarray(ar_logits)
    diff_logits = np.asarray(diff_logits)
    B, kp1, _ = ar_logits.shape
    k = kp1 - 1
    out = np.zeros(B)
    for b in range(B):
        reach = 1.0
        for m in range(k):
            p = softmax_t(target_logits(ar_logits[b, m], diff_logits[b, m], trust_ar), temperature)
            q = softmax_t(diff_logits[b, m], temperature)
            reach *= np.minimum(p, q).sum()
            out[b] += reach
    return out


def selected_block_rows(k: int, n: int) -> tuple[int, int]:
    """Step rows of the pre-drafted block chosen for accept length n.

    The block for accept length j occupies rows [k + j*k, k + (j+1)*k)
    (review §3.2: a pre-draft exists for every accept length).
    """
    return k + n * k, k + (n + 1) * k
