"""Pins for the KV-commit oracle (CPU only): invariants of an exact append."""
import numpy as np
import pytest

import oracle


def _case(L=3, B=4, R=7, Hkv=2, D=5, cap=16, seed=0):
    rng = np.random.default_rng(seed)
    ks = rng.integers(0, 2**16, size=(L, B, R, Hkv, D), dtype=np.uint16)
    vs = rng.integers(0, 2**16, size=(L, B, R, Hkv, D), dtype=np.uint16)
    kc = rng.integers(0, 2**16, size=(L, B, Hkv, cap, D), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(L, B, Hkv, cap, D), dtype=np.uint16)
    return ks, vs, kc, vc


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_append_invariants(seed):
    ks, vs, kc, vc = _case(seed=seed)
    k = 3
    lens = np.array([0, 5, 9, 13], np.int32)
    acc = np.array([3, 0, 2, 1], np.int32)
    nk, nv, nl = oracle.kv_commit(ks, vs, kc, vc, acc, lens)
    assert (nl == lens + acc).all()
    for b in range(4):
        s, n = lens[b], acc[b]
        # committed prefix untouched
        assert (nk[:, b, :, :s] == kc[:, b, :, :s]).all() and (nv[:, b, :, :s] == vc[:, b, :, :s]).all()
        # accepted draft rows appended in order, per layer and head
        for i in range(n):
            assert (nk[:, b, :, s + i] == ks[:, b, i]).all()
            assert (nv[:, b, :, s + i] == vs[:, b, i]).all()
        # slots past the new length untouched (rejected drafts and pre-drafts never written)
        assert (nk[:, b, :, s + n:] == kc[:, b, :, s + n:]).all()
        assert (nv[:, b, :, s + n:] == vc[:, b, :, s + n:]).all()
    assert k >= acc.max()


def test_zero_accept_is_noop():
    ks, vs, kc, vc = _case(seed=9)
    lens = np.array([4, 4, 4, 4], np.int32)
    nk, nv, nl = oracle.kv_commit(ks, vs, kc, vc, np.zeros(4, np.int32), lens)
    assert (nk == kc).all() and (nv == vc).all() and (nl == lens).all()


def test_inputs_not_modified():
    ks, vs, kc, vc = _case(seed=3)
    kc0 = kc.copy()
    oracle.kv_commit(ks, vs, kc, vc, np.array([2, 2, 2, 2], np.int32), np.array([1, 2, 3, 4], np.int32))
    assert (kc == kc0).all()
