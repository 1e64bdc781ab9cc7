"""The C-ABI library loads without a GPU, exports every declared symbol, and
rejects bad arguments on the host before any HIP call (no compute here)."""
import ctypes
import os
import re

import pytest

from ar_self_speculative_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
lib = _lib._lib
FAKE = 0x10000  # aligned non-null address; every call below fails validation before using it


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            names |= set(re.findall(r"\b(tidar_[a-z0-9_]+)\s*\(", open(os.path.join(inc, h)).read()))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert lib.tidar_status_string(0) == b"TIDAR_OK"
    assert lib.tidar_status_string(-4) == b"TIDAR_E_CAPACITY"
    assert lib.tidar_version() >= 100


def _desc(**kw):
    d = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, k=16, num_blocks=17,
             block_len=16, cache_capacity=4112, max_cache_len=4096, sm_scale=0.088, dtype=1,
             num_splits=0)
    d.update(kw)
    return _lib.make_attn_desc(**d)


def _attn(desc, ws=FAKE, ws_bytes=1 << 30, **ptrs):
    p = dict(q=FAKE, ks=FAKE, vs=FAKE, kc=FAKE, vc=FAKE, cl=FAKE, out=FAKE)
    p.update(ptrs)
    return lib.tidar_attn_step(ctypes.byref(desc), p["q"], p["ks"], p["vs"], p["kc"], p["vc"], p["cl"],
                               p["out"], None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=30), _lib.TIDAR_E_INVALID),            # Hq % Hkv != 0
    (dict(num_kv_heads=0), _lib.TIDAR_E_INVALID),
    (dict(dtype=7), _lib.TIDAR_E_INVALID),
    (dict(head_dim=96), _lib.TIDAR_E_UNSUPPORTED),           # bf16 needs 64/128
    (dict(num_blocks=18), _lib.TIDAR_E_INVALID),             # more blocks than accept lengths
    (dict(k=0, num_blocks=0), _lib.TIDAR_E_INVALID),         # no rows
    (dict(max_cache_len=5000), _lib.TIDAR_E_CAPACITY),       # max_cache_len > cap
    (dict(sm_scale=0.0), _lib.TIDAR_E_INVALID),
    (dict(sm_scale=float("nan")), _lib.TIDAR_E_INVALID),
    (dict(num_splits=-1), _lib.TIDAR_E_INVALID),
    (dict(block_len=0), _lib.TIDAR_E_INVALID),
    (dict(dtype=0, head_dim=6), _lib.TIDAR_E_UNSUPPORTED),   # f32 needs multiple of 4
])
def test_attn_rejects_bad_descriptors(kw, status):
    d = _desc(**kw)
    assert _attn(d) == status
    assert lib.tidar_last_error()
    assert lib.tidar_attn_workspace_bytes(ctypes.byref(d)) == 0


def test_attn_rejects_null_and_misaligned_pointers():
    d = _desc()
    assert _attn(d, q=None) == _lib.TIDAR_E_INVALID
    assert _attn(d, out=None) == _lib.TIDAR_E_INVALID
    assert _attn(d, kc=FAKE + 2) == _lib.TIDAR_E_INVALID
    assert lib.tidar_attn_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None) \
        == _lib.TIDAR_E_INVALID


def test_attn_workspace_query_and_check():
    d = _desc()
    need = lib.tidar_attn_workspace_bytes(ctypes.byref(d))
    assert need > 0                          # the prefix is split at this shape
    assert _attn(d, ws=None, ws_bytes=0) == _lib.TIDAR_E_WORKSPACE
    assert _attn(d, ws_bytes=need - 1) == _lib.TIDAR_E_WORKSPACE
    one = _desc(num_splits=1)
    assert lib.tidar_attn_workspace_bytes(ctypes.byref(one)) == 0


def test_commit_rejects_bad_arguments():
    def call(**kw):
        a = dict(L=36, B=1, H=8, D=128, k=16, rows=288, cap=4112, maxlen=4096, dtype=1,
                 ks=FAKE, vs=FAKE, kc=FAKE, vc=FAKE, acc=FAKE, lin=FAKE, lout=FAKE + 64)
        a.update(kw)
        return lib.tidar_kv_commit(a["L"], a["B"], a["H"], a["D"], a["k"], a["rows"], a["cap"],
                                   a["maxlen"], a["dtype"], a["ks"], a["vs"], a["kc"], a["vc"],
                                   a["acc"], a["lin"], a["lout"], None, None)
    assert call(maxlen=4100) == _lib.TIDAR_E_CAPACITY        # 4100 + 16 > 4112
    assert call(lout=FAKE) == _lib.TIDAR_E_INVALID           # aliasing in/out lengths
    assert call(rows=8) == _lib.TIDAR_E_INVALID              # fewer step rows than drafts
    assert call(acc=None) == _lib.TIDAR_E_INVALID
    assert call(dtype=3) == _lib.TIDAR_E_INVALID
    assert call(D=4) == _lib.TIDAR_E_UNSUPPORTED             # 8-byte rows
    assert call(kc=FAKE + 8) == _lib.TIDAR_E_INVALID


def test_reject_rejects_bad_arguments():
    def call(**kw):
        a = dict(B=1, k=16, V=151936, ar=FAKE, diff=FAKE, drafts=FAKE, u=FAKE, T=1.0, acc=FAKE,
                 nxt=FAKE, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.tidar_reject_sample(a["B"], a["k"], a["V"], a["ar"], a["diff"], a["drafts"], a["u"],
                                       a["T"], a["acc"], a["nxt"], None, None, a["ws"], a["wsb"], None)
    assert call(T=0.0) == _lib.TIDAR_E_INVALID
    assert call(T=-1.0) == _lib.TIDAR_E_INVALID
    assert call(V=0) == _lib.TIDAR_E_INVALID
    assert call(drafts=None) == _lib.TIDAR_E_INVALID
    assert call(wsb=16) == _lib.TIDAR_E_WORKSPACE
    assert call(k=1000) == _lib.TIDAR_E_UNSUPPORTED
    assert call(ar=FAKE + 4) == _lib.TIDAR_E_INVALID
    need = lib.tidar_reject_workspace_bytes(1, 16, 151936)
    assert need > 0 and call(wsb=need - 1) == _lib.TIDAR_E_WORKSPACE


@pytest.mark.parametrize("lam", [-0.25, 1.5, float("nan"), float("inf")])
def test_reject_trust_rejects_bad_weight(lam):
    st = lib.tidar_reject_sample_trust(1, 16, 151936, FAKE, FAKE, FAKE, FAKE, 1.0, lam, FAKE, FAKE, None, None,
                                       FAKE, 1 << 30, None)
    assert st == _lib.TIDAR_E_INVALID
    assert b"trust_ar" in lib.tidar_last_error()


def test_logprob_rejects_bad_arguments():
    def call(**kw):
        a = dict(rows=4, V=151936, lg=FAKE, tg=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.tidar_token_logprobs(a["rows"], a["V"], a["lg"], a["tg"], a["out"], None, a["ws"], a["wsb"], None)
    assert call(rows=0) == _lib.TIDAR_E_INVALID
    assert call(V=0) == _lib.TIDAR_E_INVALID
    assert call(lg=None) == _lib.TIDAR_E_INVALID
    assert call(tg=None) == _lib.TIDAR_E_INVALID
    assert call(lg=FAKE + 4) == _lib.TIDAR_E_INVALID
    assert call(rows=1 << 20) == _lib.TIDAR_E_UNSUPPORTED
    need = lib.tidar_logprob_workspace_bytes(4, 151936)
    assert need >= 4 * 38 * 8 and call(wsb=need - 1) == _lib.TIDAR_E_WORKSPACE
    assert call(ws=FAKE + 16) == _lib.TIDAR_E_INVALID
    assert lib.tidar_logprob_workspace_bytes(0, 10) == 0


def test_noalloc_sampler_rejects_inputs_beyond_its_scratch():
    """The allocation-free sampler checks its static scratch size on the host,
    before any HIP call: a shape that needs more returns TIDAR_E_WORKSPACE."""
    cap = int(lib.tidar_reject_noalloc_max_bytes())
    assert cap == 1 << 20
    B, k, V = 64, 128, 151936
    assert _lib.reject_workspace_bytes(B, k, V) > cap
    st = lib.tidar_reject_sample_noalloc(B, k, V, FAKE, FAKE, FAKE, FAKE, 1.0, 1.0, FAKE, FAKE, None, None, None)
    assert st == _lib.TIDAR_E_WORKSPACE
    assert b"scratch" in lib.tidar_last_error()
    # and the ordinary argument checks come first
    assert lib.tidar_reject_sample_noalloc(B, k, V, FAKE, FAKE, FAKE, FAKE, 0.0, 1.0, FAKE, FAKE, None, None,
                                           None) == _lib.TIDAR_E_INVALID


def test_decode_regime_workspace_layout(monkeypatch):
    """With TIDAR_ATTN_DECODE=1, few packed rows per KV head select the decode
    kernel: 128-key prefix splits plus one split of step keys, arrival
    counters first (256-byte padded), then the bf16 split outputs and fp32
    split log-sum-exps."""
    monkeypatch.setenv("TIDAR_ATTN_DECODE", "1")
    d = _desc(num_q_heads=64, num_kv_heads=8, k=1, num_blocks=0, block_len=1, cache_capacity=4104,
              max_cache_len=4096)
    S, rows = 4096 // 128 + 1, 1 * 1 * 64
    expect = 256 + (S * rows * 128 * 2 + 255) // 256 * 256 + S * rows * 4
    assert lib.tidar_attn_workspace_bytes(ctypes.byref(d)) == expect
    # forcing a split count keeps the main kernel (no counters)
    f = _desc(num_q_heads=64, num_kv_heads=8, k=1, num_blocks=0, block_len=1, cache_capacity=4104,
              max_cache_len=4096, num_splits=4)
    assert lib.tidar_attn_workspace_bytes(ctypes.byref(f)) == 4 * rows * 128 * 2 + 4 * rows * 4


def _is_decode_plan(d, rows):
    """The decode plan's workspace: counters, then ceil(max_len / 128) + 1 splits."""
    S = (d.max_cache_len + 127) // 128 + 1
    counters = (d.batch * d.num_kv_heads * 4 + 255) // 256 * 256
    return lib.tidar_attn_workspace_bytes(ctypes.byref(d)) == \
        counters + (S * rows * 128 * 2 + 255) // 256 * 256 + S * rows * 4


@pytest.mark.parametrize("P,R,expect", [(512, 1, True), (2048, 1, True), (2048, 4, True),
                                        (2048, 8, False),    # 64 packed rows per KV head
                                        (4096, 1, False)])   # 8 x 33 workgroups > 256
def test_decode_regime_chosen_by_itself(P, R, expect, monkeypatch):
    """Without the environment switch the decode kernel serves up to 32 packed
    rows per KV head when its workgroups fit one per CU; otherwise the main
    kernel's plan stands. TIDAR_ATTN_DECODE=0 turns it off."""
    monkeypatch.delenv("TIDAR_ATTN_DECODE", raising=False)
    d = _desc(num_q_heads=64, num_kv_heads=8, k=R, num_blocks=0, block_len=1, cache_capacity=P + 8,
              max_cache_len=P)
    assert _is_decode_plan(d, R * 64) == expect
    monkeypatch.setenv("TIDAR_ATTN_DECODE", "0")
    assert not _is_decode_plan(d, R * 64)


def test_attn_stamps_rejects_bad_arguments():
    """The timestamp reader checks its arguments on the host before any copy."""
    assert lib.tidar_attn_stamps(None, 1) == -1
    buf = (ctypes.c_uint64 * 8)()
    assert lib.tidar_attn_stamps(ctypes.addressof(buf), -1) == -1
