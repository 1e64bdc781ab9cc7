"""GPU parity of tidar_reject_sample against the fp64 oracle.

Accept lengths and tokens must match bit for bit given the same uniforms.
Exceptions, counted and printed: a sequence whose consulted acceptance test
is a near-tie (|u - min(1, rho)| < 1e-5) is excused; a draw within 1e-5 of
the total mass of a CDF boundary must return one of the tokens whose interval
meets that band.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax as sp_softmax

import ar_self_speculative_amd as tidar
import oracle
from tidar_synth import config_sampler, sampler_case
from tests.gpu_util import check_samples

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEAR = 1e-5


def gpu_reject(ar, diff, drafts, u, temperature=1.0, with_status=False):
    B, kp1, V = ar.shape
    k = kp1 - 1
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).cuda()
    ar_d = t(ar, np.float32)
    diff_d = t(diff, np.float32) if k else torch.empty((B, 0, V), dtype=torch.float32, device="cuda")
    dr_d = t(drafts, np.int32) if k else torch.empty((B, 0), dtype=torch.int32, device="cuda")
    u_d = t(u, np.float32)
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ratio = torch.zeros((B, k), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(tidar.reject_workspace_bytes(B, k, V), dtype=torch.uint8, device="cuda")
    tidar.reject_sample(ar_logits=ar_d, diff_logits=diff_d, drafts=dr_d, uniforms=u_d, accept_len=acc,
                        next_token=nxt, ratio=ratio, dev_status=status, workspace=ws,
                        temperature=temperature)
    torch.cuda.synchronize()
    res = (acc.cpu().numpy(), nxt.cpu().numpy(), ratio.cpu().numpy())
    return res + (int(status.item()),) if with_status else res


def compare(case, name):
    ref = oracle.reject_sample(case.ar_logits, case.diff_logits, case.drafts, case.uniforms,
                               case.temperature)
    acc, nxt, ratio = gpu_reject(case.ar_logits, case.diff_logits, case.drafts, case.uniforms,
                                 case.temperature)
    mism = (acc != ref.accept_len) | (nxt != ref.next_token)
    excused, draw_near = check_samples(ref, acc, nxt, case.ar_logits, case.diff_logits, case.uniforms,
                                       case.temperature)
    print(f"[parity] {name}: B={case.batch} mismatches={int(mism.sum())} accept near-ties={excused} "
          f"draw near-ties={draw_near} mean accept={ref.accept_len.mean():.2f}", flush=True)
    finite = np.isfinite(ref.ratio)
    np.testing.assert_allclose(ratio[finite], ref.ratio[finite], rtol=2e-5)
    return ref


def test_golden_hand_examples():
    for c in json.load(open(os.path.join(GOLDEN, "reject_tiny.json")))["cases"]:
        ar = np.log(np.array(c["p"], np.float32))[None]
        diff = np.log(np.array(c["q"], np.float32))[None]
        acc, nxt, ratio = gpu_reject(ar, diff, np.array([c["drafts"]]), np.array([c["uniforms"]]))
        assert acc[0] == c["expect_n"] and nxt[0] == c["expect_c"], c["name"]
        np.testing.assert_allclose(ratio[0], c["ratio"], rtol=1e-5)


@pytest.mark.parametrize("seed", range(4))
def test_config1_many_sequences(seed):
    case = sampler_case(batch=512, k=4, vocab=512, ar_sigma=2.0, diff_mode="independent",
                        diff_sigma=2.0, seed=seed)
    compare(case, f"cfg1-like V=512 k=4 seed={seed}")


@pytest.mark.parametrize("seed", range(3))
def test_config2_qwen_vocab(seed):
    case = config_sampler(2, seed=seed, batch=4)
    compare(case, f"cfg2 V=151936 k=16 seed={seed}")


def test_ragged_vocab_and_k():
    case = sampler_case(batch=64, k=7, vocab=5003, ar_sigma=3.0, diff_mode="noisy", diff_sigma=1.5, seed=9)
    compare(case, "V=5003 k=7")
    case0 = sampler_case(batch=64, k=0, vocab=4097, ar_sigma=1.0, diff_mode="independent", diff_sigma=1.0,
                         seed=10)
    compare(case0, "k=0 V=4097")


def test_temperature():
    case = sampler_case(batch=128, k=3, vocab=1000, ar_sigma=2.0, diff_mode="noisy", diff_sigma=1.0, seed=11,
                        temperature=0.7)
    compare(case, "T=0.7")


def test_identical_proposal_accepts_all():
    case = sampler_case(batch=64, k=5, vocab=300, ar_sigma=2.0, diff_mode="noisy", diff_sigma=0.0, seed=12)
    acc, _, _ = gpu_reject(case.ar_logits, case.diff_logits, case.drafts, case.uniforms)
    assert (acc == 5).all()


def test_first_token_law_is_ar_on_gpu():
    """Empirical law of the first committed token over 10^6 GPU draws equals p_0."""
    V, k, N = 16, 3, 1_000_000
    rng = np.random.default_rng(21)
    ar = rng.normal(0, 1.5, size=(k + 1, V)).astype(np.float32)
    diff = (ar[:k] + rng.normal(0, 1.0, size=(k, V))).astype(np.float32)
    q = sp_softmax(diff.astype(np.float64), axis=-1)
    p = sp_softmax(ar.astype(np.float64), axis=-1)
    drafts = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(k)], axis=1).astype(np.int32)
    u = rng.random((N, k + 1), dtype=np.float32)
    acc, nxt, _ = gpu_reject(np.broadcast_to(ar, (N, k + 1, V)), np.broadcast_to(diff, (N, k, V)), drafts, u)
    first = np.where(acc >= 1, drafts[:, 0], nxt)
    obs = np.bincount(first, minlength=V)
    chi = stats.chisquare(obs, N * p[0])
    print(f"[stats] first-token chi2 p-value {chi.pvalue:.3g}", flush=True)
    assert chi.pvalue > 1e-3


def test_bad_draft_id_is_flagged():
    case = sampler_case(batch=2, k=2, vocab=100, ar_sigma=1.0, diff_mode="independent", diff_sigma=1.0, seed=3)
    drafts = case.drafts.copy()
    drafts[1, 0] = 100
    acc, _, _, status = gpu_reject(case.ar_logits, case.diff_logits, drafts, case.uniforms, with_status=True)
    assert status & 16
    assert acc[1] == 0
