"""GPU parity of tidar_reject_sample (and its trust-mixing variant,
tidar_reject_sample_trust) against the fp64 oracle.

Accept lengths and tokens must match bit for bit given the same uniforms.
Exceptions, counted and printed (tests/gpu_util.py::check_samples): where a
consulted acceptance test is a near-tie (|u - min(1, rho)| < 1e-5) the
accept length may be the oracle's chain with that one test flipped; a draw
whose target lies within 2e-6 (probability units) of a CDF boundary may
return the token across it.
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


def gpu_reject(ar, diff, drafts, u, temperature=1.0, with_status=False, trust_ar=1.0):
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
                        temperature=temperature, trust_ar=trust_ar)
    torch.cuda.synchronize()
    res = (acc.cpu().numpy(), nxt.cpu().numpy(), ratio.cpu().numpy())
    return res + (int(status.item()),) if with_status else res


def compare(case, name, trust_ar=1.0):
    ref = oracle.reject_sample(case.ar_logits, case.diff_logits, case.drafts, case.uniforms,
                               case.temperature, trust_ar=trust_ar)
    acc, nxt, ratio = gpu_reject(case.ar_logits, case.diff_logits, case.drafts, case.uniforms,
                                 case.temperature, trust_ar=trust_ar)
    mism = (acc != ref.accept_len) | (nxt != ref.next_token)
    acc_diff, draw_diff = check_samples(ref, acc, nxt, case.ar_logits, case.diff_logits, case.uniforms,
                                        case.temperature, trust_ar=trust_ar)
    print(f"[parity] {name}: B={case.batch} mismatches={int(mism.sum())} accept flips (near-tie)={acc_diff} "
          f"tokens across a boundary (near-tie)={draw_diff} mean accept={ref.accept_len.mean():.2f}", flush=True)
    finite = np.isfinite(ref.ratio)
    np.testing.assert_allclose(ratio[finite], ref.ratio[finite], rtol=2e-5)
    return ref


def test_golden_hand_examples():
    for c in json.load(open(os.path.join(GOLDEN, "reject_tiny.json")))["cases"]:
        ar = np.log(np.array(c["p"], np.float32))[None]
        diff = np.log(np.array(c["q"], np.float32))[None]
        acc, nxt, ratio = gpu_reject(ar, diff, np.array([c["drafts"]]), np.array([c["uniforms"]]),
                                     trust_ar=c.get("trust_ar", 1.0))
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


def test_max_k_and_statistics_past_the_lds_stage():
    """k = 128 (the largest the sampler takes) and a vocabulary whose (row, chunk)
    statistics exceed the LDS stage (257 rows x 25 chunks > 4096), so every row
    is merged straight from global memory."""
    case = sampler_case(batch=4, k=128, vocab=100003, ar_sigma=2.0, diff_mode="noisy", diff_sigma=0.3, seed=17)
    compare(case, "k=128 V=100003 (unstaged statistics)")
    # identical proposal: every draft accepted, the bonus token drawn from row 128
    same = sampler_case(batch=2, k=128, vocab=100003, ar_sigma=2.0, diff_mode="noisy", diff_sigma=0.0, seed=18)
    ref = compare(same, "k=128 V=100003 identical proposal")
    assert (ref.accept_len == 128).all()


@pytest.mark.parametrize("batch,k,vocab,path", [
    (2, 31, 262144, "registers, at their limit: 63 rows x 64 chunks"),
    (8, 40, 8192, "LDS stage: 81 rows"),
    (2, 8, 300000, "LDS stage: 74 chunks"),
], ids=["registers-limit", "lds-rows", "lds-chunks"])
def test_row_statistics_merge_paths(batch, k, vocab, path):
    """The draw pass merges each row's chunk statistics from registers (up to
    64 rows of up to 64 chunks), from an LDS stage (up to 4096 pairs), or one
    wave per row from global memory (the k = 128 test above): every path
    against the oracle."""
    case = sampler_case(batch=batch, k=k, vocab=vocab, ar_sigma=2.5, diff_mode="noisy", diff_sigma=0.5, seed=23 + k)
    compare(case, f"k={k} V={vocab} ({path})")


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


@pytest.mark.parametrize("lam", [0.0, 0.3, 0.5, 0.8])
def test_trust_mixing_config2(lam):
    case = config_sampler(2, seed=5, batch=4)
    ref = compare(case, f"cfg2 V=151936 k=16 trust_ar={lam}", trust_ar=lam)
    if lam == 0.0:
        assert (ref.accept_len == 16).all()


@pytest.mark.parametrize("lam", [0.25, 0.6])
def test_trust_mixing_many_sequences(lam):
    case = sampler_case(batch=256, k=6, vocab=3001, ar_sigma=2.5, diff_mode="noisy", diff_sigma=1.5, seed=13,
                        temperature=0.8)
    compare(case, f"V=3001 k=6 T=0.8 trust_ar={lam}", trust_ar=lam)


def test_trust_one_entry_matches_plain_entry():
    """tidar_reject_sample_trust with weight 1 is the plain sampler, bit for bit."""
    import ctypes
    from ar_self_speculative_amd import _lib
    case = config_sampler(2, seed=6, batch=3)
    B, kp1, V = case.ar_logits.shape
    k = kp1 - 1
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).cuda()
    ar, diff, dr, u = t(case.ar_logits, np.float32), t(case.diff_logits, np.float32), \
        t(case.drafts, np.int32), t(case.uniforms, np.float32)
    ws = torch.empty(tidar.reject_workspace_bytes(B, k, V), dtype=torch.uint8, device="cuda")
    outs = []
    for fn in ("plain", "trust"):
        acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        ratio = torch.zeros((B, k), dtype=torch.float32, device="cuda")
        head = (B, k, V, ar.data_ptr(), diff.data_ptr(), dr.data_ptr(), u.data_ptr(), 1.0)
        tail = (acc.data_ptr(), nxt.data_ptr(), ratio.data_ptr(), None, ws.data_ptr(), ws.numel(), None)
        st = (_lib._lib.tidar_reject_sample(*head, *tail) if fn == "plain"
              else _lib._lib.tidar_reject_sample_trust(*head, 1.0, *tail))
        assert st == 0
        torch.cuda.synchronize()
        outs.append((acc.cpu().numpy(), nxt.cpu().numpy(), ratio.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_trust_mixture_law_on_gpu():
    """lambda = 0.5: first committed token over 10^6 GPU draws follows softmax of the mixed logits."""
    V, k, N, lam = 16, 2, 1_000_000, 0.5
    rng = np.random.default_rng(22)
    ar = rng.normal(0, 2.0, size=(k + 1, V)).astype(np.float32)
    diff = rng.normal(0, 2.0, size=(k, V)).astype(np.float32)
    q = sp_softmax(diff.astype(np.float64), axis=-1)
    target = sp_softmax(lam * ar[:k].astype(np.float64) + (1 - lam) * diff.astype(np.float64), axis=-1)
    drafts = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(k)], axis=1).astype(np.int32)
    u = rng.random((N, k + 1), dtype=np.float32)
    acc, nxt, _ = gpu_reject(np.broadcast_to(ar, (N, k + 1, V)), np.broadcast_to(diff, (N, k, V)), drafts, u,
                             trust_ar=lam)
    first = np.where(acc >= 1, drafts[:, 0], nxt)
    obs = np.bincount(first, minlength=V)
    chi = stats.chisquare(obs, N * target[0])
    print(f"[stats] trust 0.5 first-token chi2 p-value {chi.pvalue:.3g}", flush=True)
    assert chi.pvalue > 1e-3


def test_bitwise_deterministic_over_ten_calls():
    case = config_sampler(2, seed=9, batch=4)
    outs = [gpu_reject(case.ar_logits, case.diff_logits, case.drafts, case.uniforms, trust_ar=lam)
            for lam in (1.0, 0.4) for _ in range(5)]
    for i in (1, 2, 3, 4):
        for a, b in zip(outs[0], outs[i]):
            assert np.array_equal(a, b)
    for i in (6, 7, 8, 9):
        for a, b in zip(outs[5], outs[i]):
            assert np.array_equal(a, b)
