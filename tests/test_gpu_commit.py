"""GPU parity of tidar_kv_commit: bit-exact against the oracle's append."""
import numpy as np
import pytest
import torch

import ar_self_speculative_amd as tidar
import oracle
from tidar_synth import commit_accept_lengths

pytestmark = pytest.mark.gpu


def _rand_bits(rng, shape):
    return rng.integers(0, 2 ** 16, size=shape, dtype=np.uint16)


def run_commit(ks, vs, kc, vc, acc, lens, k, cap, max_len, dtype=tidar.DTYPE_BF16):
    L, B, R, Hkv, D = ks.shape
    if dtype == tidar.DTYPE_BF16:
        t = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        t = lambda a: torch.from_numpy(a).cuda()
    ks_d, vs_d, kc_d, vc_d = t(ks), t(vs), t(kc.copy()), t(vc.copy())
    acc_d = torch.from_numpy(acc.astype(np.int32)).cuda()
    lin = torch.from_numpy(lens.astype(np.int32)).cuda()
    lout = torch.full_like(lin, -1)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    tidar.kv_commit(num_layers=L, batch=B, num_kv_heads=Hkv, head_dim=D, k=k, step_rows=R, cache_capacity=cap,
                    max_cache_len=max_len, dtype=dtype, k_step=ks_d, v_step=vs_d, k_cache=kc_d, v_cache=vc_d,
                    accept_len=acc_d, cache_len_in=lin, cache_len_out=lout, dev_status=status)
    torch.cuda.synchronize()
    back = (lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)) if dtype == tidar.DTYPE_BF16 else \
        (lambda x: x.cpu().numpy())
    return back(kc_d), back(vc_d), lout.cpu().numpy(), int(status.item())


def test_config3_full_depth_uniform_accept():
    """36 layers, 8 KV heads, D=128, P=4096, cap 4112; n ~ U{0..16} per seed."""
    rng = np.random.default_rng(0)
    L, B, R, Hkv, D, cap, P, k = 36, 1, 288, 8, 128, 4112, 4096, 16
    ks, vs = _rand_bits(rng, (L, B, R, Hkv, D)), _rand_bits(rng, (L, B, R, Hkv, D))
    kc, vc = _rand_bits(rng, (L, B, Hkv, cap, D)), _rand_bits(rng, (L, B, Hkv, cap, D))
    lens = np.array([P], np.int32)
    for seed in range(3):
        acc = commit_accept_lengths(B, k, seed)
        nk, nv, nl, st = run_commit(ks, vs, kc, vc, acc, lens, k, cap, P)
        ek, ev, el = oracle.kv_commit(ks, vs, kc, vc, acc, lens)
        assert st == 0
        assert np.array_equal(nl, el)
        assert np.array_equal(nk, ek) and np.array_equal(nv, ev)


@pytest.mark.parametrize("seed", range(3))
def test_ragged_batch(seed):
    rng = np.random.default_rng(100 + seed)
    L, B, k, Hkv, D, cap = 3, 8, 8, 8, 128, 4608
    R = k + (k + 1) * k
    ks, vs = _rand_bits(rng, (L, B, R, Hkv, D)), _rand_bits(rng, (L, B, R, Hkv, D))
    kc, vc = _rand_bits(rng, (L, B, Hkv, cap, D)), _rand_bits(rng, (L, B, Hkv, cap, D))
    lens = rng.integers(256, 4097, size=B).astype(np.int32)
    acc = rng.integers(0, k + 1, size=B).astype(np.int32)
    acc[0], acc[1] = 0, k
    nk, nv, nl, st = run_commit(ks, vs, kc, vc, acc, lens, k, cap, int(lens.max()))
    ek, ev, el = oracle.kv_commit(ks, vs, kc, vc, acc, lens)
    assert st == 0 and np.array_equal(nl, el)
    assert np.array_equal(nk, ek) and np.array_equal(nv, ev)


def test_f32_commit():
    rng = np.random.default_rng(7)
    L, B, k, Hkv, D, cap = 1, 2, 4, 1, 64, 140
    R = k + (k + 1) * k
    f = lambda s: rng.standard_normal(s).astype(np.float32)
    ks, vs, kc, vc = f((L, B, R, Hkv, D)), f((L, B, R, Hkv, D)), f((L, B, Hkv, cap, D)), f((L, B, Hkv, cap, D))
    lens = np.array([128, 3], np.int32)
    acc = np.array([4, 2], np.int32)
    nk, nv, nl, st = run_commit(ks, vs, kc, vc, acc, lens, k, cap, 128, dtype=tidar.DTYPE_F32)
    ek, ev, el = oracle.kv_commit(ks, vs, kc, vc, acc, lens)
    assert st == 0 and np.array_equal(nl, el) and np.array_equal(nk, ek) and np.array_equal(nv, ev)


def test_out_of_range_accept_and_capacity_are_flagged_not_written():
    rng = np.random.default_rng(8)
    L, B, k, Hkv, D, cap = 2, 3, 4, 2, 64, 32
    R = k + (k + 1) * k
    ks, vs = _rand_bits(rng, (L, B, R, Hkv, D)), _rand_bits(rng, (L, B, R, Hkv, D))
    kc, vc = _rand_bits(rng, (L, B, Hkv, cap, D)), _rand_bits(rng, (L, B, Hkv, cap, D))
    lens = np.array([10, 10, 28], np.int32)
    acc = np.array([5, -1, 4], np.int32)        # > k, < 0, and 28 + 4 = 32 <= cap (fine)
    nk, nv, nl, st = run_commit(ks, vs, kc, vc, acc, lens, k, cap, 28)
    assert st & 2
    assert nl[0] == 10 and nl[1] == 10 and nl[2] == 32
    assert np.array_equal(nk[:, :2], kc[:, :2]) and np.array_equal(nv[:, :2], vc[:, :2])
    lens2 = np.array([10, 10, 30], np.int32)     # device length above the host bound: 30 + 4 > cap
    _, _, nl2, st2 = run_commit(ks, vs, kc, vc, np.array([1, 1, 4], np.int32), lens2, k, cap, 28)
    assert st2 & 4 and nl2[2] == 30
