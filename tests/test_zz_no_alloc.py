"""The allocation-free sampler entry point (tidar_reject_sample_noalloc)
against the workspace entry point (tidar_reject_sample_trust), through the C
ABI: two calls in a row, the second with a smaller input. (Inputs beyond the
static scratch are rejected on the host: tests/test_abi.py.)"""
import numpy as np
import pytest
import torch

import ar_self_speculative_amd as tidar
from tidar_synth import sampler_case

pytestmark = pytest.mark.gpu


def _run(case, trust_ar, noalloc):
    B, kp1, V = case.ar_logits.shape
    k = kp1 - 1
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).cuda()
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ratio = torch.full((B, k), -1.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = dict(ar_logits=t(case.ar_logits, np.float32), diff_logits=t(case.diff_logits, np.float32),
                drafts=t(case.drafts, np.int32), uniforms=t(case.uniforms, np.float32), accept_len=acc,
                next_token=nxt, ratio=ratio, dev_status=status, trust_ar=trust_ar)
    if noalloc:
        tidar.reject_sample_noalloc(**args)
    else:
        ws = torch.empty(tidar.reject_workspace_bytes(B, k, V), dtype=torch.uint8, device="cuda")
        tidar.reject_sample(workspace=ws, **args)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy(), ratio.cpu().numpy(), int(status.item())


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    big = sampler_case(batch=8, k=16, vocab=151936, ar_sigma=3.0, diff_mode="noisy", diff_sigma=1.0, seed=31)
    small = sampler_case(batch=3, k=5, vocab=5003, ar_sigma=2.0, diff_mode="noisy", diff_sigma=0.5, seed=32)
    for case, trust in ((big, 1.0), (small, 0.5)):
        ref = _run(case, trust, noalloc=False)
        got = _run(case, trust, noalloc=True)
        print(f"[parity] noalloc B={case.batch} k={case.k} V={case.vocab}: accept {got[0].tolist()}", flush=True)
        # same kernels, same order of every reduction: identical bits
        for a, b in zip(ref[:3], got[:3]):
            np.testing.assert_array_equal(a, b)
        assert ref[3] == got[3] == 0
