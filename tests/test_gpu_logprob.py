"""GPU parity of tidar_token_logprobs (likelihood mode) against the fp64 oracle.

Tolerance: 1e-4 absolute on the log-probability. The GPU keeps fp32 chunk
statistics (maximum and sum of exp over 4096 tokens) merged in a fixed order;
the oracle is fp64. For rows of ~150k logits with values of a few units the
fp32 log-normaliser is good to a few 1e-6.
"""
import math

import numpy as np
import pytest
import torch

import ar_self_speculative_amd as tidar
import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-4


def gpu_logprobs(logits, targets, with_status=False):
    V = logits.shape[-1]
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    tg = torch.from_numpy(np.ascontiguousarray(targets, dtype=np.int32)).cuda()
    out = torch.full(targets.shape, -7.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(tidar.logprob_workspace_bytes(tg.numel(), V), 256), dtype=torch.uint8, device="cuda")
    tidar.token_logprobs(logits=lg, targets=tg, logprobs=out, workspace=ws, dev_status=status)
    torch.cuda.synchronize()
    res = out.cpu().numpy().astype(np.float64)
    return (res, int(status.item())) if with_status else res


@pytest.mark.parametrize("B,R,V,sigma", [(1, 16, 151936, 3.0), (2, 150, 5003, 2.0), (1, 512, 32000, 4.0),
                                          (3, 5, 3, 1.0), (1, 1, 4096, 1.0), (1, 7, 4097, 10.0)])
def test_parity(B, R, V, sigma):
    rng = np.random.default_rng(B * 1000 + R + V)
    logits = rng.normal(0, sigma, size=(B, R, V)).astype(np.float32)
    targets = rng.integers(0, V, size=(B, R))
    got = gpu_logprobs(logits, targets)
    ref = oracle.token_logprobs(logits, targets)
    err = float(np.abs(got - ref).max())
    print(f"[parity] logprobs B={B} R={R} V={V}: max-abs {err:.2e}", flush=True)
    assert err <= TOL


def test_uniform_rows_and_large_logits():
    V = 151936
    logits = np.full((2, V), 7.0, np.float32)
    logits[1] = 0.0
    logits[1, 5] = 80.0                       # exp(80) overflows fp32 without the maximum taken out
    got = gpu_logprobs(logits, np.array([123, 5]))
    assert abs(got[0] + math.log(V)) <= TOL
    assert abs(got[1] - oracle.token_logprobs(logits[1:], np.array([5]))[0]) <= TOL


def test_out_of_range_target_is_nan_and_flagged():
    rng = np.random.default_rng(9)
    logits = rng.normal(size=(3, 1000)).astype(np.float32)
    got, status = gpu_logprobs(logits, np.array([1, 1000, -2]), with_status=True)
    assert status & tidar._lib.DEV_TARGET_RANGE
    assert np.isfinite(got[0]) and np.isnan(got[1]) and np.isnan(got[2])


def test_likelihood_mode_attention_is_causal_single_forward():
    """The forward of likelihood mode is the append-prefill attention (num_blocks = 0):
    rows of a causal sequence must match the oracle's causal attention."""
    from tidar_synth import config_attn
    from tests.gpu_util import run_attn, oracle_inputs
    c = config_attn(4, seed=0, P=512, R=32)
    out, _ = run_attn(c)
    ref, _ = oracle.attn_step(*oracle_inputs(c), c.cache_len, k=c.k, num_blocks=c.num_blocks,
                              block_len=c.block_len, sm_scale=c.sm_scale)
    err = float(np.abs(out - ref).max())
    print(f"[parity] likelihood-mode causal forward P=512 R=32: max-abs {err:.2e}", flush=True)
    assert c.num_blocks == 0 and err <= 2e-2
