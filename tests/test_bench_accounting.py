"""The bench's algorithmic accounting (the FLOPs and bytes its roofline
figures divide by) against the oracle's mask and hand-derived totals.

The FLOP count is 4 * Hq * D * (R * P + sum over rows of the visible step
keys) per layer: two multiply-adds per (row, visible key, dim) for Q K^T and
two for P V (TiDAR review, awesome-system-papers wiki, 核心方法 section 3.2,
for which keys each query region sees). The bytes are each operand moved
once: prefix K/V, step K/V, Q and O, and the sampler's 2k+1 fp32 logit rows.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle.dense import hybrid_mask_matrix

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("k", [1, 2, 4, 8, 16])
def test_visible_step_keys_match_the_brute_force_mask(k):
    """The closed form the bench uses for the visible step keys equals the
    count of ones in the step-key columns of the oracle's brute-force mask."""
    b = _bench()
    P = 3
    M = hybrid_mask_matrix(P, k, k + 1, k)
    brute = int(M[:, P:].sum())
    c = b.algorithmic_counts(1, 1, 1, 1, 1, P, k, 1)
    R = k + (k + 1) * k
    assert c["R"] == R == M.shape[0]
    # attn_flops_layer = 4 * Hq * D * (R * P + visible step keys) with Hq = D = B = 1
    assert c["attn_flops_layer"] == 4 * (R * P + brute)
    assert int(M[:, :P].sum()) == R * P  # every row sees the whole prefix


def test_bench_shape_totals():
    """Qwen3-8B step, P = 4096, k = 16: 6664 visible step-key pairs (16
    drafts see 1..16 of their own; each of the 17 blocks of 16 sees its j
    drafts and its 16 block keys, j = 0..16), 19.44 GFLOP per layer, and the
    operand bytes of one layer and of the sampler."""
    b = _bench()
    c = b.algorithmic_counts(36, 1, 32, 8, 128, 4096, 16, 151936)
    drafts = sum(range(1, 17))
    blocks = sum(16 * (j + 16) for j in range(17))
    assert drafts + blocks == 6664
    assert c["attn_flops_layer"] == 4 * 32 * 128 * (288 * 4096 + 6664) == 19436535808
    assert c["kv_prefix_layer"] == 2 * 8 * 4096 * 128 * 2 == 16777216
    assert c["kv_step_layer"] == 2 * 288 * 8 * 128 * 2 == 1179648
    assert c["qo_layer"] == 2 * 288 * 32 * 128 * 2 == 4718592
    assert c["attn_bytes_layer"] == 16777216 + 1179648 + 4718592
    assert c["sampler_bytes"] == 33 * 151936 * 4 == 20055552
    # arithmetic intensity of one layer, against the bf16 MFMA / HBM ridge of the nominal peaks
    ai = c["attn_flops_layer"] / c["attn_bytes_layer"]
    assert 850 < ai < 860 and ai > 2.5e15 / 8e12


def test_bench_shape_mask_count_by_brute_force():
    """The 6664 of the bench shape, counted from the oracle's mask itself."""
    M = hybrid_mask_matrix(1, 16, 17, 16)
    assert int(M[:, 1:].sum()) == 6664
    assert np.all(M[:, 0] == 1)
