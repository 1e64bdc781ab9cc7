"""GPU parity of the decode-regime attention kernel (few packed query rows per
KV head, head_dim 128: chosen by the planner for R * g <= 32 when its
workgroups fit one per CU, forced up to R * g <= 128 with TIDAR_ATTN_DECODE=1)
against the fp64 oracle.

The same inputs run three ways: splits merged inside the kernel by the
last-arriving split, merged by the separate merge kernel, and on the main
kernel (decode path off); each is compared with the oracle at every output
element (bf16: max-abs 2e-2, LSE 2^-8). Prefix lengths straddle the 128-key
split boundaries and include 0. Repeated launches on one workspace give
identical bits and leave its arrival counters at zero.
"""
import numpy as np
import pytest
import torch

import ar_self_speculative_amd as tidar
import oracle
from tidar_synth import attn_case, config_attn
from tests.gpu_util import attn_desc, dev_array, oracle_inputs, run_attn

pytestmark = pytest.mark.gpu

TOL, LSE_TOL = 2e-2, 2.0 ** -8

SHAPES = [
    # (B, lens, k, num_blocks, Hq, Hkv): TiDAR steps with small k, and append-prefill rows
    (3, [0, 1, 129], 1, 2, 32, 8),          # k = 1: R = 3, M = 12
    (2, [127, 128], 2, 3, 32, 8),           # k = 2: R = 8, M = 32
    (2, [256, 4096], 4, 5, 32, 8),          # k = 4: R = 24, M = 96
    (1, [4096], 1, 0, 64, 8),               # one decode row, Qwen3-32B heads: M = 8
    (2, [2049, 511], 4, 0, 64, 8),          # four append rows, M = 32
    (1, [1000], 16, 0, 64, 8),              # M = 128, the largest the kernel takes
    (2, [300, 5], 3, 4, 8, 2),              # g = 4, fewer blocks than k + 1
    (1, [70], 128, 0, 8, 8),                # g = 1, R = 128 step keys (two local tiles)
]


def _case(shape, seed):
    B, lens, k, nb, Hq, Hkv = shape
    cap = max(lens) + k + 8
    return attn_case(dtype="bf16", layers=1, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, k=k,
                     num_blocks=nb, block_len=k if nb else 1, cache_len=lens, cache_capacity=cap, seed=seed)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}-k{s[2]}-nb{s[3]}-Hq{s[4]}-Hkv{s[5]}")
def test_decode_kernel_matches_oracle(shape, monkeypatch):
    c = _case(shape, seed=sum(shape[1]) + shape[2])
    ref, rlse = oracle.attn_step(*oracle_inputs(c), c.cache_len, k=c.k, num_blocks=c.num_blocks,
                                 block_len=c.block_len, sm_scale=c.sm_scale)
    results = {}
    for mode, env in (("fused", {"TIDAR_ATTN_DECODE": "1", "TIDAR_ATTN_FUSED_MERGE": "1"}),
                      ("merge-kernel", {"TIDAR_ATTN_DECODE": "1", "TIDAR_ATTN_FUSED_MERGE": "0"}),
                      ("main-kernel", {"TIDAR_ATTN_DECODE": "0"})):
        with monkeypatch.context() as mp:
            for key, val in env.items():
                mp.setenv(key, val)
            out, lse = run_attn(c)
        err = float(np.abs(out - ref).max())
        lerr = float(np.abs(lse - rlse).max())
        print(f"[parity] decode {shape} {mode}: max-abs {err:.3e}, lse {lerr:.3e}", flush=True)
        assert np.isfinite(out).all() and err <= TOL and lerr <= LSE_TOL, (mode, err, lerr)
        results[mode] = out
    # the two merges of the same split partials agree closely
    assert np.abs(results["fused"] - results["merge-kernel"]).max() <= 2.0 ** -7


def test_config4_decode_rows_every_element(monkeypatch):
    """One decode row over P = 4096 with Qwen3-32B heads (64 query, 8 KV), every output element."""
    monkeypatch.setenv("TIDAR_ATTN_DECODE", "1")
    c = config_attn(4, P=4096, R=1, seed=11)
    out, lse = run_attn(c)
    ref, rlse = oracle.attn_step(*oracle_inputs(c), c.cache_len, k=c.k, num_blocks=0, block_len=1,
                                 sm_scale=c.sm_scale)
    err = float(np.abs(out - ref).max())
    print(f"[parity] cfg4 P=4096 R=1 all elements: max-abs {err:.3e}", flush=True)
    assert err <= TOL and np.abs(lse - rlse).max() <= LSE_TOL


@pytest.mark.parametrize("fused", ["1", "0"])
def test_repeated_launches_bitwise_equal_and_counters_reset(fused, monkeypatch):
    monkeypatch.setenv("TIDAR_ATTN_DECODE", "1")
    monkeypatch.setenv("TIDAR_ATTN_FUSED_MERGE", fused)
    c = _case((2, [1500, 77], 2, 3, 32, 8), seed=3)
    desc = attn_desc(c)
    args = [dev_array(c, n, 0) for n in ("q", "k_step", "v_step", "k_cache", "v_cache")]
    lens = torch.from_numpy(c.cache_len).cuda()
    ws = tidar.attn_workspace(desc)
    counters = ws[: 4 * c.batch * c.num_kv_heads].view(torch.int32)
    first = None
    for i in range(10):
        out = torch.empty_like(args[0])
        tidar.attn_step(desc, *args, lens, out, None, None, ws)
        torch.cuda.synchronize()
        assert int(counters.abs().sum().item()) == 0, i
        bits = out.view(torch.int16).cpu().numpy()
        if first is None:
            first = bits
        assert np.array_equal(bits, first), i
