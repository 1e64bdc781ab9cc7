"""Pins for the fp64 attention oracle (CPU only).

The oracle is checked against things other than itself:
* a hand-derived worked example (tests/golden/attn_tiny.json);
* the separately written dense 0/1-mask brute force (oracle/dense.py);
* torch's scaled_dot_product_attention (fp64, CPU) on the three textbook
  special cases the region rules reduce to: causal AR attention for the draft
  rows, prefix-LM attention for each pre-draft block, causal append-prefill
  when there are no blocks;
* closed forms and invariants: constant V, prefix permutation, logsumexp,
  visible-key counts.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy.special import logsumexp

import oracle
from oracle import attention as oatt
from tidar_synth import attn_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(x):
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(x[2:]))
        if "/" in x:
            a, b = x.split("/")
            return float(a) / float(b)
    return float(x)


def _arr(nested):
    if isinstance(nested, list):
        return np.array([_arr(x) for x in nested], dtype=np.float64)
    return _val(nested)


def _case(P, k, nb, bl, Hq, Hkv, D=8, B=1, seed=0, cache_len=None):
    cap = P + k + 3
    lens = P if cache_len is None else cache_len
    return attn_case(dtype="f32", layers=1, batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
                     head_dim=D, k=k, num_blocks=nb, block_len=bl, cache_len=lens,
                     cache_capacity=cap, seed=seed, poison=True)


def _run(c, fn=oracle.attn_step):
    return fn(c.q[0], c.k_step[0], c.v_step[0], c.k_cache[0], c.v_cache[0], c.cache_len,
              k=c.k, num_blocks=c.num_blocks, block_len=c.block_len, sm_scale=c.sm_scale)


def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "attn_tiny.json")))
    s = g["shape"]
    q = _arr(g["q"])[None]                 # [1, R, 1, D]
    ks = _arr(g["k_step"])[None]
    vs = _arr(g["v_step"])[None]
    kc = _arr(g["k_cache"])[None]          # [1, 1, P, D]
    vc = _arr(g["v_cache"])[None]
    out, lse = oracle.attn_step(q, ks, vs, kc, vc, np.array([s["P"]]), k=s["k"],
                                num_blocks=s["num_blocks"], block_len=s["block_len"],
                                sm_scale=s["sm_scale"])
    np.testing.assert_allclose(out[0], _arr(g["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], _arr(g["lse"]), rtol=0, atol=1e-14)


@settings(max_examples=60, deadline=None)
@given(P=st.integers(0, 40), k=st.integers(1, 6), extra_blocks=st.integers(-1, 0),
       gq=st.sampled_from([(1, 1), (2, 1), (4, 2), (4, 1), (6, 2)]),
       bl_same=st.booleans(), seed=st.integers(0, 10_000))
def test_matches_dense_bruteforce(P, k, extra_blocks, gq, bl_same, seed):
    nb = k + 1 + extra_blocks            # k+1 blocks (TiDAR) or fewer
    bl = k if bl_same else max(1, k - 1)
    Hq, Hkv = gq
    c = _case(P, k, nb, bl, Hq, Hkv, seed=seed)
    o1, l1 = _run(c)
    o2, l2 = _run(c, oracle.attn_dense)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def _sdpa(qh, kh, vh, mask, scale):
    """torch SDPA in fp64 on CPU; qh [Hq, M, D], kh/vh [Hq, N, D], mask [M, N] bool."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(qh), t(kh), t(vh), attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def _expand_kv(x, g):
    # [N, Hkv, D] -> [Hq, N, D] with query head h reading KV head h // g
    return np.repeat(np.transpose(x, (1, 0, 2)), g, axis=0)


@pytest.mark.parametrize("P,k,Hq,Hkv,B", [(0, 3, 2, 1, 1), (17, 4, 4, 2, 2), (33, 6, 6, 2, 1), (5, 1, 8, 8, 1)])
def test_draft_rows_are_causal_ar_attention(P, k, Hq, Hkv, B):
    lens = np.array([P, max(0, P - 3)][:B])
    c = _case(P, k, k + 1, k, Hq, Hkv, B=B, seed=P + k, cache_len=lens)
    out, _ = _run(c)
    g = Hq // Hkv
    for b in range(B):
        n = int(lens[b])
        keys = np.concatenate([np.transpose(c.k_cache[0, b, :, :n], (1, 0, 2)), c.k_step[0, b, :k]])
        vals = np.concatenate([np.transpose(c.v_cache[0, b, :, :n], (1, 0, 2)), c.v_step[0, b, :k]])
        mask = np.tril(np.ones((k, n + k), dtype=bool), k=n)   # bottom-right causal
        ref = _sdpa(np.transpose(c.q[0, b, :k], (1, 0, 2)), _expand_kv(keys, g), _expand_kv(vals, g),
                    mask, c.sm_scale)
        np.testing.assert_allclose(out[b, :k], np.transpose(ref, (1, 0, 2)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("P,k,Hq,Hkv", [(0, 2, 1, 1), (9, 4, 4, 2), (40, 5, 4, 1)])
def test_block_rows_are_prefix_lm_attention(P, k, Hq, Hkv):
    c = _case(P, k, k + 1, k, Hq, Hkv, seed=11 * P + k)
    out, _ = _run(c)
    g = Hq // Hkv
    for j in range(k + 1):
        rows = list(range(k + j * k, k + (j + 1) * k))
        # sequence [prefix; d_1..d_j; block j], fully visible to block j
        keys = np.concatenate([np.transpose(c.k_cache[0, 0, :, :P], (1, 0, 2)),
                               c.k_step[0, 0, :j], c.k_step[0, 0, rows]])
        vals = np.concatenate([np.transpose(c.v_cache[0, 0, :, :P], (1, 0, 2)),
                               c.v_step[0, 0, :j], c.v_step[0, 0, rows]])
        mask = np.ones((k, keys.shape[0]), dtype=bool)
        ref = _sdpa(np.transpose(c.q[0, 0, rows], (1, 0, 2)), _expand_kv(keys, g),
                    _expand_kv(vals, g), mask, c.sm_scale)
        np.testing.assert_allclose(out[0, rows], np.transpose(ref, (1, 0, 2)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("P,R", [(0, 5), (12, 8), (31, 1)])
def test_no_blocks_is_causal_append_prefill(P, R):
    c = _case(P, R, 0, 1, 4, 2, seed=P * 7 + R)
    out, _ = _run(c)
    keys = np.concatenate([np.transpose(c.k_cache[0, 0, :, :P], (1, 0, 2)), c.k_step[0, 0]])
    vals = np.concatenate([np.transpose(c.v_cache[0, 0, :, :P], (1, 0, 2)), c.v_step[0, 0]])
    mask = np.tril(np.ones((R, P + R), dtype=bool), k=P)
    ref = _sdpa(np.transpose(c.q[0, 0], (1, 0, 2)), _expand_kv(keys, 2), _expand_kv(vals, 2),
                mask, c.sm_scale)
    np.testing.assert_allclose(out[0], np.transpose(ref, (1, 0, 2)), rtol=0, atol=1e-12)


def test_constant_values_give_that_value():
    c = _case(23, 4, 5, 4, 4, 2, seed=3)
    c.v_cache[...] = 0.625
    c.v_step[...] = 0.625
    out, _ = _run(c)
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-15)


def test_prefix_permutation_invariance():
    c = _case(29, 3, 4, 3, 2, 1, seed=5)
    out, lse = _run(c)
    perm = np.random.default_rng(0).permutation(29)
    c.k_cache[0, :, :, :29] = c.k_cache[0][:, :, perm]
    c.v_cache[0, :, :, :29] = c.v_cache[0][:, :, perm]
    out2, lse2 = _run(c)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


def test_lse_is_logsumexp_of_visible_scores():
    c = _case(13, 3, 4, 3, 2, 2, seed=9)
    _, lse = _run(c)
    M = oracle.hybrid_mask_matrix(13, 3, 4, 3).astype(bool)
    for h in range(2):
        K = np.concatenate([c.k_cache[0, 0, h, :13], c.k_step[0, 0, :, h]]).astype(np.float64)
        S = c.sm_scale * (c.q[0, 0, :, h].astype(np.float64) @ K.T)
        for r in range(c.rows):
            assert abs(lse[0, r, h] - logsumexp(S[r, M[r]])) < 1e-12


@pytest.mark.parametrize("k", [1, 2, 4, 8, 16])
def test_visible_local_count_closed_form(k):
    # k draft rows see 1..k step keys; block j's k rows each see j drafts + k block keys
    expect = k * (k + 1) // 2 + sum(k * (j + k) for j in range(k + 1))
    assert oracle.visible_local_count(k, k + 1, k) == expect
    assert oracle.hybrid_mask_matrix(0, k, k + 1, k).sum() == expect
    if k == 16:
        assert expect == 6664


def test_poisoned_slots_are_never_read():
    # rows >= cache_len hold NaN in the synthetic cache; the output stays finite
    c = _case(10, 2, 3, 2, 2, 1, cache_len=7)
    out, lse = _run(c)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_planted_mask_mistake_is_caught(monkeypatch):
    """An off-by-one in the oracle's block rule must break the dense pin."""
    c = _case(6, 3, 4, 3, 2, 1, seed=2)
    good, _ = _run(c, oracle.attn_dense)
    real = oatt.local_keys

    def off_by_one(r, k, nb, bl):
        keys = real(r, k, nb, bl)
        if r >= k:
            j = (r - k) // bl
            if j < k:
                keys = sorted(set(keys) | {j})      # block j also sees d_{j+1}
        return keys

    monkeypatch.setattr(oatt, "local_keys", off_by_one)
    bad, _ = _run(c)
    assert np.abs(bad - good).max() > 1e-3


def _all_rows(c):
    return [(b, r, h) for b in range(c.batch) for r in range(c.rows) for h in range(c.num_q_heads)]


def _rows_vs_dense(c):
    """oracle.attn_rows at every (b, r, h) against the dense brute force."""
    rows = _all_rows(c)
    o1, l1 = oracle.attn_rows(c.q[0], c.k_step[0], c.v_step[0], c.k_cache[0], c.v_cache[0], c.cache_len, rows,
                              k=c.k, num_blocks=c.num_blocks, block_len=c.block_len, sm_scale=c.sm_scale)
    o2, l2 = _run(c, oracle.attn_dense)
    idx = tuple(np.array(rows).T)
    return np.abs(o1 - o2[idx]).max(), np.abs(l1 - l2[idx]).max()


@settings(max_examples=60, deadline=None)
@given(B=st.integers(2, 3), k=st.integers(1, 5), blocks=st.sampled_from(["none", "fewer", "all"]),
       g=st.sampled_from([1, 2, 4]), Hkv=st.integers(1, 2), seed=st.integers(0, 10_000),
       lens=st.lists(st.integers(0, 24), min_size=3, max_size=3))
def test_attn_rows_matches_dense_bruteforce(B, k, blocks, g, Hkv, seed, lens):
    """attn_rows (the sampled-row checker of the full-size parity tests) is
    pinned to the separately written dense brute force at every (b, r, h):
    several sequences with ragged prefix lengths (0 included), GQA groups of
    1, 2 and 4, and no blocks, fewer than k + 1 blocks, or all k + 1."""
    nb = {"none": 0, "fewer": max(0, k - 1), "all": k + 1}[blocks]
    cl = np.array(lens[:B], dtype=np.int32)
    c = _case(int(cl.max()), k, nb, k, g * Hkv, Hkv, B=B, seed=seed, cache_len=cl)
    e_out, e_lse = _rows_vs_dense(c)
    assert e_out <= 1e-12 and e_lse <= 1e-12, (e_out, e_lse)


def test_attn_rows_planted_head_map_mistake_is_caught(monkeypatch):
    """A wrong GQA head map (h % Hkv instead of h // g) in attn_rows breaks the pin."""
    c = _case(9, 3, 4, 3, 4, 2, B=2, seed=4, cache_len=np.array([9, 5], np.int32))
    assert max(_rows_vs_dense(c)) <= 1e-12
    monkeypatch.setattr(oatt, "kv_head", lambda h, g: h % 2)
    assert _rows_vs_dense(c)[0] > 1e-3


def test_attn_rows_planted_sequence_length_mistake_is_caught(monkeypatch):
    """Reading sequence 0's prefix length for every sequence breaks the pin."""
    c = _case(12, 2, 3, 2, 2, 1, B=2, seed=6, cache_len=np.array([12, 4], np.int32))
    good = _rows_vs_dense(c)
    assert max(good) <= 1e-12
    real = oracle.attn_rows

    def first_len_everywhere(q, ks, vs, kc, vc, cache_len, rows, **kw):
        return real(q, ks, vs, kc, vc, np.full_like(np.asarray(cache_len), np.asarray(cache_len)[0]), rows, **kw)

    monkeypatch.setattr(oracle, "attn_rows", first_len_everywhere)
    # the poisoned cache slots past sequence 1's length make the outputs NaN
    e = _rows_vs_dense(c)[0]
    assert not (e <= 1e-3), e
