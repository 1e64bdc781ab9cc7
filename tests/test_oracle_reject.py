"""Pins for the fp64 rejection-sampling oracle (CPU only).

Checked against: hand-derived worked examples (tests/golden/reject_tiny.json),
special cases that reduce to plain categorical sampling, the closed-form
acceptance law of speculative sampling (P(n >= i) = prod_{m<i} alpha_m with
alpha_m = sum_t min(p_m(t), q_m(t))), and the empirical law of the committed
tokens, which must equal the AR distributions p_0 and p_1 (chi-square).
With trust mixing (TiDAR review, 设计取舍, Fig. 6) the same laws hold for the
mixed targets softmax(lambda * AR + (1 - lambda) * diffusion): lambda = 0
accepts every draft, and the first committed token follows the logit-space
mixture, not the probability-space one.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax as sp_softmax

import oracle
from tidar_synth import sampler_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _scan_invcdf(w, u):
    """Brute-force scan: first token whose running sum passes u * total."""
    total = 0.0
    for x in w:
        total += float(x)
    run = 0.0
    for t, x in enumerate(w):
        run += float(x)
        if run > u * total:
            return t
    return max(t for t, x in enumerate(w) if x > 0)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "reject_tiny.json")))["cases"],
                         ids=lambda c: c["name"])
def test_golden_hand_examples(case):
    ar = np.log(np.array(case["p"]))[None]
    diff = np.log(np.array(case["q"]))[None]
    res = oracle.reject_sample(ar, diff, np.array([case["drafts"]]), np.array([case["uniforms"]]),
                               trust_ar=case.get("trust_ar", 1.0))
    assert res.accept_len[0] == case["expect_n"]
    assert res.next_token[0] == case["expect_c"]
    np.testing.assert_allclose(res.ratio[0], case["ratio"], rtol=1e-12)


def test_identical_proposal_accepts_everything():
    c = sampler_case(batch=64, k=5, vocab=97, ar_sigma=2.0, diff_mode="independent",
                     diff_sigma=1.0, seed=3)
    diff = c.ar_logits[:, :5].copy()
    res = oracle.reject_sample(c.ar_logits, diff, c.drafts, c.uniforms)
    assert (res.accept_len == 5).all()
    for b in range(64):
        p = sp_softmax(c.ar_logits[b, 5].astype(np.float64))
        assert res.next_token[b] == _scan_invcdf(p, float(c.uniforms[b, 5]))


def test_zero_drafts_is_categorical_sampling():
    c = sampler_case(batch=200, k=0, vocab=50, ar_sigma=2.0, diff_mode="independent",
                     diff_sigma=1.0, seed=4)
    res = oracle.reject_sample(c.ar_logits, c.diff_logits, c.drafts, c.uniforms)
    assert (res.accept_len == 0).all()
    for b in range(200):
        p = sp_softmax(c.ar_logits[b, 0].astype(np.float64))
        assert res.next_token[b] == _scan_invcdf(p, float(c.uniforms[b, 0]))


def test_draft_impossible_under_ar_is_rejected():
    rng = np.random.default_rng(5)
    V, d = 20, 7
    ar = rng.normal(size=(1, 2, V))
    ar[0, 0, d] = -np.inf                       # p_0(d) = 0
    diff = np.full((1, 1, V), -np.inf)
    diff[0, 0, d] = 0.0                         # q_0 = delta_d
    for u in (0.0, 0.3, 0.999):
        res = oracle.reject_sample(ar, diff, np.array([[d]]), np.array([[u, 0.42]]))
        assert res.accept_len[0] == 0
        p0 = sp_softmax(ar[0, 0])
        assert res.next_token[0] == _scan_invcdf(p0, 0.42) and res.next_token[0] != d


def test_temperature_scales_logits():
    c = sampler_case(batch=16, k=3, vocab=64, ar_sigma=2.0, diff_mode="noisy", diff_sigma=0.5, seed=6)
    a = oracle.reject_sample(c.ar_logits, c.diff_logits, c.drafts, c.uniforms, temperature=1.0)
    b = oracle.reject_sample(c.ar_logits * 2.0, c.diff_logits * 2.0, c.drafts, c.uniforms, temperature=2.0)
    assert (a.accept_len == b.accept_len).all() and (a.next_token == b.next_token).all()


def _trials(V, k, N, seed):
    rng = np.random.default_rng(seed)
    ar = rng.normal(0, 1.5, size=(k + 1, V))
    diff = ar[:k] + rng.normal(0, 1.0, size=(k, V))
    p = sp_softmax(ar, axis=-1)
    q = sp_softmax(diff, axis=-1)
    drafts = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(k)], axis=1)
    u = rng.random((N, k + 1))
    res = oracle.reject_sample(np.broadcast_to(ar, (N, k + 1, V)), np.broadcast_to(diff, (N, k, V)),
                               drafts, u)
    return p, q, drafts, res


def test_acceptance_law_matches_closed_form():
    V, k, N = 16, 4, 20000
    p, q, _, res = _trials(V, k, N, seed=7)
    alpha = np.minimum(p[:k], q).sum(axis=1)
    for i in range(1, k + 1):
        expect = np.prod(alpha[:i])
        got = (res.accept_len >= i).mean()
        se = np.sqrt(expect * (1 - expect) / N)
        assert abs(got - expect) < 5 * se + 1e-9, (i, got, expect)
    e_n = sum(np.prod(alpha[:i]) for i in range(1, k + 1))
    assert abs(res.accept_len.mean() - e_n) < 0.05


def test_committed_tokens_follow_ar_chain():
    """First committed token ~ p_0; second committed token given the first was a kept draft ~ p_1."""
    V, k, N = 16, 3, 100_000
    p, q, drafts, res = _trials(V, k, N, seed=8)
    first = np.where(res.accept_len >= 1, drafts[:, 0], res.next_token)
    obs = np.bincount(first, minlength=V)
    chi = stats.chisquare(obs, N * p[0])
    assert chi.pvalue > 1e-3, chi
    sel = res.accept_len >= 1
    second = np.where(res.accept_len[sel] >= 2, drafts[sel, 1], res.next_token[sel])
    obs2 = np.bincount(second, minlength=V)
    chi2 = stats.chisquare(obs2, sel.sum() * p[1])
    assert chi2.pvalue > 1e-3, chi2
    # and the law is far from the proposal, so the test has power
    assert stats.chisquare(obs, N * q[0]).pvalue < 1e-6


def test_trust_diffusion_accepts_every_draft():
    c = sampler_case(batch=64, k=5, vocab=97, ar_sigma=2.0, diff_mode="independent",
                     diff_sigma=1.0, seed=9)
    res = oracle.reject_sample(c.ar_logits, c.diff_logits, c.drafts, c.uniforms, trust_ar=0.0)
    assert (res.accept_len == 5).all()
    np.testing.assert_allclose(res.ratio, 1.0, rtol=1e-12)
    for b in range(64):
        p = sp_softmax(c.ar_logits[b, 5].astype(np.float64))   # bonus row stays pure AR
        assert res.next_token[b] == _scan_invcdf(p, float(c.uniforms[b, 5]))


def test_trust_one_is_the_plain_sampler():
    c = sampler_case(batch=32, k=4, vocab=80, ar_sigma=2.0, diff_mode="noisy", diff_sigma=0.7, seed=10)
    a = oracle.reject_sample(c.ar_logits, c.diff_logits, c.drafts, c.uniforms)
    b = oracle.reject_sample(c.ar_logits, c.diff_logits, c.drafts, c.uniforms, trust_ar=1.0)
    assert (a.accept_len == b.accept_len).all() and (a.next_token == b.next_token).all()
    with pytest.raises(ValueError):
        oracle.reject_sample(c.ar_logits, c.diff_logits, c.drafts, c.uniforms, trust_ar=1.5)


def test_trust_mixture_laws():
    """lambda = 0.4: acceptance law and first-token law of the logit-space mixture."""
    V, k, N, lam = 12, 2, 100_000, 0.4
    rng = np.random.default_rng(11)
    ar = rng.normal(0, 2.0, size=(k + 1, V))
    diff = rng.normal(0, 2.0, size=(k, V))
    q = sp_softmax(diff, axis=-1)
    target = sp_softmax(lam * ar[:k] + (1 - lam) * diff, axis=-1)
    drafts = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(k)], axis=1)
    u = rng.random((N, k + 1))
    res = oracle.reject_sample(np.broadcast_to(ar, (N, k + 1, V)), np.broadcast_to(diff, (N, k, V)),
                               drafts, u, trust_ar=lam)
    alpha = np.minimum(target, q).sum(axis=1)
    for i in range(1, k + 1):
        expect = np.prod(alpha[:i])
        got = (res.accept_len >= i).mean()
        assert abs(got - expect) < 5 * np.sqrt(expect * (1 - expect) / N) + 1e-9, (i, got, expect)
    first = np.where(res.accept_len >= 1, drafts[:, 0], res.next_token)
    obs = np.bincount(first, minlength=V)
    assert stats.chisquare(obs, N * target[0]).pvalue > 1e-3
    # power: the law differs from the probability-space mixture and from both modes
    prob_mix = lam * sp_softmax(ar[0]) + (1 - lam) * q[0]
    for other in (prob_mix, sp_softmax(ar[0]), q[0]):
        assert stats.chisquare(obs, N * other / other.sum()).pvalue < 1e-6


def test_selected_block_rows():
    assert oracle.selected_block_rows(16, 0) == (16, 32)
    assert oracle.selected_block_rows(16, 16) == (16 + 256, 16 + 272)
    assert oracle.selected_block_rows(4, 2) == (12, 16)


def test_expected_accept_len_closed_form_pins():
    """expected_accept_len against Monte-Carlo of reject_sample, and its special
    cases: identical proposal -> k, proposal disjoint from the target -> 0,
    one draft -> alpha_0 = 1 - total variation distance."""
    V, k, N = 16, 4, 20000
    rng = np.random.default_rng(7)
    ar = rng.normal(0, 1.5, size=(k + 1, V))
    diff = ar[:k] + rng.normal(0, 1.0, size=(k, V))
    e = oracle.expected_accept_len(ar[None], diff[None])[0]
    _, _, _, res = _trials(V, k, N, seed=7)
    se = res.accept_len.std() / np.sqrt(N)
    assert abs(res.accept_len.mean() - e) < 5 * se, (res.accept_len.mean(), e)
    assert oracle.expected_accept_len(ar[None], ar[None, :k])[0] == pytest.approx(k, abs=1e-12)
    disjoint_ar = np.full((1, 2, 4), -np.inf)
    disjoint_ar[0, :, :2] = 0.0
    disjoint_q = np.full((1, 1, 4), -np.inf)
    disjoint_q[0, 0, 2:] = 0.0
    assert oracle.expected_accept_len(disjoint_ar, disjoint_q)[0] == 0.0
    p, q = sp_softmax(ar[0]), sp_softmax(diff[0])
    one = oracle.expected_accept_len(ar[None, :2], diff[None, :1])[0]
    assert one == pytest.approx(1.0 - 0.5 * np.abs(p - q).sum(), abs=1e-12)


def test_config5_noise_scale_gives_seven_committed_tokens():
    """The ragged batch's stored noise scale (written by oracle/calibrate_config5.py)
    gives a mean of 7 committed tokens per step by the oracle's closed form, over
    the exact verifier inputs of its 64 steps."""
    import json
    import os

    from oracle.calibrate_config5 import mean_committed, step_draws
    from tidar_synth import CONFIGS

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "config5_sigma.json")))
    assert CONFIGS[5]["sampler"]["diff_sigma"] == g["sigma"]
    m = mean_committed(step_draws(), g["sigma"])
    assert abs(m - 7.0) < 0.02, m
