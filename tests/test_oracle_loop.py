"""Pins for the step-loop logic of the oracle (CPU only).

A toy model stands in for the decoder: region rows predict the next token of
a position-dependent Markov chain, x_{t+1} ~ softmax(T[x_t, t]); mask rows
propose from an unrelated table. Checked against:
* k = 1 (no drafts): the loop is plain AR sampling of the chain with the same
  uniforms, token for token;
* k = 3: the joint law of the first emitted tokens equals the chain's, exactly
  computed (chi-square over 20 000 sequences) -- wrong AR-row alignment,
  positions, commit lengths or emission bookkeeping all change it;
* block selection: with delta proposals that name their block, the next
  drafts reveal that block n + 1 (the one that saw c and the n accepted
  drafts) is the one used;
* the closed-form positions of a step's rows.
"""
import numpy as np
from scipy import stats
from scipy.special import softmax as sp_softmax

import oracle
from oracle import loop as L


def toy_logits(T, D, state, k):
    """Logits of one step of the toy model for every row of step_positions
    (T [V, positions, V]: region rows; D [V, k, V]: mask rows, by the last
    visible region token and the mask index)."""
    B = state.region.shape[0]
    V = T.shape[-1]
    R = L.step_rows(k)
    out = np.zeros((B, R, V))
    for b in range(B):
        pos = L.step_positions(k, int(state.cache_len[b]))
        for i in range(k):
            out[b, i] = T[state.region[b, i], pos[i] % T.shape[1]]
        for j in range(k + 1):
            ctx = state.region[b, j - 1] if j >= 1 else 0
            for m in range(k):
                out[b, L.block_row(k, j, m)] = D[ctx, m % D.shape[1]]
    return out


def run_toy(T, D, k, prompt_last, P0, steps, rng, B):
    st = L.start(np.stack([T[prompt_last[b], (P0 - 1) % T.shape[1]] for b in range(B)]),
                 np.full(B, P0), k, rng.random(B), rng.random((B, max(k - 1, 0))))
    used = []
    for _ in range(steps):
        uv, ud = rng.random((B, k)), rng.random((B, max(k - 1, 0)))
        st_new, n, c, _ = L.loop_step(toy_logits(T, D, st, k), st, uv, ud)
        used.append((uv, n))
        assert (st_new.cache_len == st.cache_len + n + 1).all()
        st = st_new
    return st, used


def test_positions_closed_form():
    k, ln = 4, 100
    pos = L.step_positions(k, ln)
    assert L.step_rows(k) == 4 + 5 * 4 == len(pos)
    assert list(pos[:4]) == [100, 101, 102, 103]
    for j in range(5):
        assert list(pos[L.block_row(k, j, 0):L.block_row(k, j, 0) + 4]) == [100 + j + m for m in range(4)]


def test_k1_is_plain_ar_sampling():
    rng = np.random.default_rng(1)
    V, P0, B, steps = 7, 5, 16, 12
    T = rng.normal(0, 2, size=(V, 64, V))
    D = rng.normal(0, 2, size=(V, 4, V))
    last = rng.integers(0, V, size=B)
    u_first = rng.random(B)
    st = L.start(np.stack([T[last[b], P0 - 1] for b in range(B)]), np.full(B, P0), 1, u_first,
                 np.zeros((B, 0)))
    us = [rng.random((B, 1)) for _ in range(steps)]
    for s in range(steps):
        st, n, c, _ = L.loop_step(toy_logits(T, D, st, 1), st, us[s], np.zeros((B, 0)))
        assert (n == 0).all()
    for b in range(B):
        x, t = int(last[b]), P0 - 1
        expect = []
        for u in [u_first[b]] + [us[s][b, 0] for s in range(steps)]:
            x, _ = oracle.invcdf(sp_softmax(T[x, t]), float(u))
            expect.append(x)
            t += 1
        assert st.emitted[b] == expect


def test_k3_emitted_tokens_follow_the_chain():
    rng = np.random.default_rng(2)
    V, P0, B, k = 4, 3, 20000, 3
    T = rng.normal(0, 1.5, size=(V, 16, V))
    D = rng.normal(0, 1.0, size=(V, k, V))
    last = np.zeros(B, np.int64)
    st, used = run_toy(T, D, k, last, P0, steps=3, rng=rng, B=B)
    # exact law of the first three emitted tokens x_P0, x_P0+1, x_P0+2
    p = np.zeros((V, V, V))
    p0 = sp_softmax(T[0, P0 - 1])
    for a in range(V):
        p1 = sp_softmax(T[a, P0])
        for bb in range(V):
            p2 = sp_softmax(T[bb, P0 + 1])
            p[a, bb] = p0[a] * p1[bb] * p2
    obs = np.zeros((V, V, V))
    for e in st.emitted:
        obs[e[0], e[1], e[2]] += 1
    chi = stats.chisquare(obs.ravel(), B * p.ravel())
    assert chi.pvalue > 1e-3, chi
    mean_n = np.mean([n.mean() for _, n in used])
    assert mean_n > 0.2          # drafts do get accepted, so the test exercises them
    # power: shifting the positions by one changes the law
    p_shift = np.zeros((V, V, V))
    p0s = sp_softmax(T[0, P0])
    for a in range(V):
        for bb in range(V):
            p_shift[a, bb] = p0s[a] * sp_softmax(T[a, P0 + 1])[bb] * sp_softmax(T[bb, P0 + 2])
    assert stats.chisquare(obs.ravel(), B * p_shift.ravel()).pvalue < 1e-6


def test_next_drafts_come_from_block_n_plus_1():
    rng = np.random.default_rng(3)
    k, V, B = 4, 16, 64
    # region rows: targets that make the accept chain follow the uniforms; mask rows of
    # block j propose token j (delta), so the next drafts name the block they came from
    st = L.LoopState(region=rng.integers(0, V, size=(B, k)), q_logits=rng.normal(size=(B, k - 1, V)),
                     cache_len=np.full(B, 50), emitted=[[] for _ in range(B)])
    logits = rng.normal(0, 1, size=(B, L.step_rows(k), V))
    for j in range(k + 1):
        for m in range(k):
            row = np.full(V, -1e9)
            row[j] = 0.0
            logits[:, L.block_row(k, j, m)] = row
    new, n, c, _ = L.loop_step(logits, st, rng.random((B, k)), rng.random((B, k - 1)))
    assert set(n.tolist()) != {int(n[0])}        # several accept lengths occur
    for b in range(B):
        assert (new.region[b, 1:] == n[b] + 1).all()
        assert new.region[b, 0] == c[b]
        assert new.emitted[b] == [int(t) for t in st.region[b, 1:1 + n[b]]] + [int(c[b])]
        np.testing.assert_array_equal(new.q_logits[b], logits[b, [L.block_row(k, n[b] + 1, m) for m in range(1, k)]])
