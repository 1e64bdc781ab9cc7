"""GPU parity of tidar_attn_step against the fp64 oracle.

Tolerances: max-abs 1e-5 for fp32 inputs and 2e-2 for bf16 inputs, on the
stored output. LSE: 1e-5 for fp32 and 1e-4 for bf16 (when the LSE is asked
for, the bf16 kernel sums each row's probabilities in fp32 before they are
rounded for the P.V product; without it the sum is taken over the rounded
values, which the full-layer test below exercises on the output).
"""
import numpy as np
import pytest
import torch

import oracle
from tidar_synth import attn_case, config_attn
from tests.gpu_util import run_attn, oracle_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
LSE_TOL = {"f32": 1e-5, "bf16": 1e-4}


def _oracle_full(case, layer=0, cache_len=None):
    lens = case.cache_len if cache_len is None else cache_len
    return oracle.attn_step(*oracle_inputs(case, layer), lens, k=case.k, num_blocks=case.num_blocks,
                            block_len=case.block_len, sm_scale=case.sm_scale)


def _report(name, out, ref, tol):
    err = np.abs(out - ref).max()
    print(f"[parity] {name}: max-abs {err:.3e} (tol {tol})", flush=True)
    return err


@pytest.mark.parametrize("splits", [0, 1, 2, 3])
def test_config1_f32(splits):
    c = config_attn(1, seed=0)
    out, lse = run_attn(c, num_splits=splits)
    ref, rlse = _oracle_full(c)
    assert _report(f"cfg1 f32 splits={splits}", out, ref, TOL["f32"]) <= TOL["f32"]
    assert np.abs(lse - rlse).max() <= 1e-5


@pytest.mark.parametrize("seed", [0, 1])
def test_config2_bf16(seed):
    c = config_attn(2, seed=seed)
    out, lse = run_attn(c)
    ref, rlse = _oracle_full(c)
    assert _report(f"cfg2 bf16 seed={seed}", out, ref, TOL["bf16"]) <= TOL["bf16"]
    assert np.abs(lse - rlse).max() <= LSE_TOL["bf16"]


@pytest.mark.parametrize("waves", ["8"])
def test_workgroup_shape_knob_matches_oracle(waves, monkeypatch):
    """The 8-wave workgroup layout (a tuning knob, TIDAR_ATTN_WAVES) gives the
    same results within tolerance, including a half-filled last query tile
    (the decode-regime kernel is switched off, as by default, so the small case runs it too),
    and head_dim 64, which the knob leaves on four waves."""
    monkeypatch.setenv("TIDAR_ATTN_WAVES", waves)
    monkeypatch.setenv("TIDAR_ATTN_DECODE", "0")
    c = config_attn(2, seed=5)
    out, lse = run_attn(c)
    ref, rlse = _oracle_full(c)
    assert _report(f"cfg2 bf16 waves={waves}", out, ref, TOL["bf16"]) <= TOL["bf16"]
    assert np.abs(lse - rlse).max() <= LSE_TOL["bf16"]
    small = attn_case(dtype="bf16", layers=1, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, k=4,
                      num_blocks=5, block_len=4, cache_len=[65, 200], cache_capacity=232, seed=6)
    out2, _ = run_attn(small)
    ref2, _ = _oracle_full(small)
    assert _report(f"small bf16 waves={waves}", out2, ref2, TOL["bf16"]) <= TOL["bf16"]
    d64 = attn_case(dtype="bf16", layers=1, batch=1, num_q_heads=8, num_kv_heads=1, head_dim=64, k=16,
                    num_blocks=17, block_len=16, cache_len=[333], cache_capacity=350, seed=7)
    out3, _ = run_attn(d64)
    ref3, _ = _oracle_full(d64)
    assert np.isfinite(out3).all()
    assert _report(f"D=64 bf16 waves={waves}", out3, ref3, TOL["bf16"]) <= TOL["bf16"]


SMALL = [
    # (B, lens, k, num_blocks, block_len, Hq, Hkv, D)
    (1, [0], 4, 5, 4, 4, 1, 128),            # empty prefix: local keys only
    (1, [1], 3, 4, 3, 2, 2, 64),
    (2, [65, 200], 4, 5, 4, 8, 2, 128),      # ragged lengths, partial tiles
    (3, [130, 7, 64], 5, 4, 3, 6, 2, 128),   # fewer blocks, other block length
    (1, [300], 16, 17, 16, 4, 1, 128),       # R*g spans several 128-row tiles
    (1, [129], 12, 0, 1, 8, 8, 128),         # append-prefill (no blocks), g = 1
    (2, [513, 1000], 8, 9, 8, 32, 8, 128),   # Qwen3-8B heads, k = 8
    (1, [77], 2, 3, 2, 1, 1, 64),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"B{s[0]}-k{s[2]}-nb{s[3]}-g{s[5] // s[6]}-D{s[7]}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [0, 1])
def test_small_shapes(shape, dtype, splits):
    B, lens, k, nb, bl, Hq, Hkv, D = shape
    cap = max(lens) + k + 5
    c = attn_case(dtype=dtype, layers=1, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, k=k,
                  num_blocks=nb, block_len=bl, cache_len=lens, cache_capacity=cap, seed=sum(lens) + k)
    out, lse = run_attn(c, num_splits=splits)
    ref, rlse = _oracle_full(c)
    assert np.isfinite(out).all()
    assert _report(f"small {shape} {dtype} S={splits}", out, ref, TOL[dtype]) <= TOL[dtype]
    assert np.abs(lse - rlse).max() <= LSE_TOL[dtype]


def _sample_rows(case, n, seed):
    rng = np.random.default_rng(seed)
    R = case.rows
    edge_r = [0, case.k - 1, case.k, case.k + case.block_len - 1, R - case.block_len, R - 1]
    rows = []
    for i in range(n):
        b = int(rng.integers(case.batch))
        r = int(edge_r[i % len(edge_r)] if i < 2 * len(edge_r) else rng.integers(R))
        h = int(rng.integers(case.num_q_heads))
        rows.append((b, max(0, min(R - 1, r)), h))
    return rows


def test_config3_full_depth_sampled():
    """All 36 layers at the full Qwen3-8B step shape (P = 4096, k = 16), split plan as in the bench."""
    c = config_attn(3, seed=0)
    rng = np.random.default_rng(1)
    worst = 0.0
    for layer in range(c.layers):
        out, lse = run_attn(c, layer=layer)
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        if layer % 5 == 0 or layer == c.layers - 1:
            rows = _sample_rows(c, 24, seed=layer)
            ref, rlse = oracle.attn_rows(*oracle_inputs(c, layer), c.cache_len, rows, k=c.k,
                                         num_blocks=c.num_blocks, block_len=c.block_len,
                                         sm_scale=c.sm_scale)
            got = np.stack([out[b, r, h] for b, r, h in rows])
            glse = np.array([lse[b, r, h] for b, r, h in rows])
            worst = max(worst, np.abs(got - ref).max())
            assert np.abs(glse - rlse).max() <= LSE_TOL["bf16"]
    print(f"[parity] cfg3 36 layers sampled: max-abs {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]
    del rng


def test_config3_one_layer_every_element_at_the_bench_launch():
    """One full Qwen3-8B-shaped layer (P = 4096, k = 16, 288 rows x 32 query
    heads) compared with the oracle at every output element, launched exactly
    as the bench times it: the library's split plan, no LSE requested."""
    c = config_attn(3, seed=2, layers=1)
    out, _ = run_attn(c, with_lse=False)
    ref, _ = _oracle_full(c)
    assert np.isfinite(out).all()
    assert _report("cfg3 one layer, every element, bench launch", out, ref, TOL["bf16"]) <= TOL["bf16"]


@pytest.mark.parametrize("lens", [[131072], [131072, 70001]], ids=["one", "ragged"])
def test_long_prefix_sampled(lens):
    """A TiDAR step (k = 4, 5 blocks of 4) over a 131072-key prefix (Qwen3-8B
    heads): alone (the planner's split count over 2048 key tiles, merged by
    several lanes per output vector) and beside a 70001-key sequence (the
    ragged apportionment of 64 split slots). Offsets run far into the cache.
    Sampled rows against the oracle."""
    c = attn_case(dtype="bf16", layers=1, batch=len(lens), num_q_heads=32, num_kv_heads=8, head_dim=128, k=4,
                  num_blocks=5, block_len=4, cache_len=lens, cache_capacity=max(lens) + 8, seed=7)
    out, lse = run_attn(c)
    rows = _sample_rows(c, 48, seed=5)
    ref, rlse = oracle.attn_rows(*oracle_inputs(c), c.cache_len, rows, k=c.k, num_blocks=c.num_blocks,
                                 block_len=c.block_len, sm_scale=c.sm_scale)
    got = np.stack([out[b, r, h] for b, r, h in rows])
    assert np.isfinite(out).all()
    assert _report(f"P={lens}, k=4", got, ref, TOL["bf16"]) <= TOL["bf16"]
    got_lse = np.array([lse[b, r, h] for b, r, h in rows])
    assert np.abs(got_lse - rlse).max() <= LSE_TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_draft_block_layout_sampled(dtype):
    """k = 64: 64 drafts and 65 blocks of 64 masks (R = 4224 rows), so a query
    tile spans several blocks and the local key ranges of one tile are far
    apart; sampled rows (every region's first and last rows included)."""
    c = attn_case(dtype=dtype, layers=1, batch=2, num_q_heads=4, num_kv_heads=1, head_dim=128, k=64,
                  num_blocks=65, block_len=64, cache_len=[300, 77], cache_capacity=320, seed=21)
    out, lse = run_attn(c)
    rows = _sample_rows(c, 40, seed=21)
    ref, rlse = oracle.attn_rows(*oracle_inputs(c), c.cache_len, rows, k=c.k, num_blocks=c.num_blocks,
                                 block_len=c.block_len, sm_scale=c.sm_scale)
    got = np.stack([out[b, r, h] for b, r, h in rows])
    assert _report(f"k=64 R=4224 {dtype}", got, ref, TOL[dtype]) <= TOL[dtype]
    got_lse = np.array([lse[b, r, h] for b, r, h in rows])
    assert np.abs(got_lse - rlse).max() <= LSE_TOL[dtype]


@pytest.mark.parametrize("P", [512, 1024, 2048, 4096])
@pytest.mark.parametrize("R", [1, 8, 16, 32, 64, 128, 256, 512])
def test_config4_points_sampled(P, R):
    """Append-prefill sweep (Qwen3-32B heads): R causal rows over a prefix P."""
    c = config_attn(4, P=P, R=R, seed=P + R)
    out, lse = run_attn(c)
    rows = _sample_rows(c, 12, seed=R)
    ref, rlse = oracle.attn_rows(*oracle_inputs(c), c.cache_len, rows, k=c.k, num_blocks=0,
                                 block_len=1, sm_scale=c.sm_scale)
    got = np.stack([out[b, r, h] for b, r, h in rows])
    assert _report(f"cfg4 P={P} R={R}", got, ref, TOL["bf16"]) <= TOL["bf16"]


def test_deterministic_and_split_independent():
    c = config_attn(2, seed=3)
    a, la = run_attn(c)
    b, lb = run_attn(c)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    one, _ = run_attn(c, num_splits=1)
    many, _ = run_attn(c, num_splits=8)
    assert np.abs(one - a).max() <= 2 ** -7 and np.abs(many - a).max() <= 2 ** -7


def test_forced_splits_past_short_sequences_on_a_nan_workspace():
    """Ragged batch with forced splits of 512 keys (one split count for every
    sequence): the splits of the short sequences that lie past their lengths
    hold no keys. The workspace is filled with NaN bytes first, so an empty
    split that left its partial slot unwritten, or a merge that mixed one in,
    would put NaN in the output."""
    import ar_self_speculative_amd as tidar
    from tests.gpu_util import attn_desc, dev_array, oracle_inputs
    lens = [0, 5, 64, 700, 3000]
    c = attn_case(dtype="bf16", layers=1, batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128, k=4,
                  num_blocks=5, block_len=4, cache_len=lens, cache_capacity=max(lens) + 8, seed=21)
    desc = attn_desc(c, num_splits=6)
    args = [dev_array(c, n, 0) for n in ("q", "k_step", "v_step", "k_cache", "v_cache")]
    ws = tidar.attn_workspace(desc)
    ws.fill_(0xFF)
    out = torch.empty_like(args[0])
    lse = torch.empty(out.shape[:-1], dtype=torch.float32, device=out.device)
    tidar.attn_step(desc, *args, torch.from_numpy(c.cache_len).cuda(), out, lse, None, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref, rlse = oracle.attn_step(*oracle_inputs(c), c.cache_len, k=c.k, num_blocks=c.num_blocks,
                                 block_len=c.block_len, sm_scale=c.sm_scale)
    assert np.isfinite(got).all()
    assert _report("ragged, empty splits, NaN workspace", got, ref, TOL["bf16"]) <= TOL["bf16"]
    assert np.abs(lse.cpu().numpy() - rlse).max() <= LSE_TOL["bf16"]


@pytest.mark.parametrize("splits", [9, 40, 100, 200])
def test_many_splits_merge_matches_oracle(splits):
    """Forced split counts past 8 make the merge spread each output vector's
    splits over 2, 8 or 16 lanes, all of whose loads go out in one round;
    200 splits over 16 lanes take two rounds. Prefixes of 12800 keys (200 key
    tiles, so every count is kept as asked) and 3000 (its later splits hold
    no keys); every element and log-sum-exp against the oracle, on a
    workspace filled with NaN bytes first."""
    import ar_self_speculative_amd as tidar
    from tests.gpu_util import attn_desc, dev_array, oracle_inputs
    lens = [12800, 3000]
    c = attn_case(dtype="bf16", layers=1, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, k=1,
                  num_blocks=2, block_len=1, cache_len=lens, cache_capacity=max(lens) + 8, seed=splits)
    desc = attn_desc(c, num_splits=splits)
    rows = c.batch * (c.k + c.num_blocks * c.block_len) * c.num_q_heads
    assert tidar.attn_workspace_bytes(desc) == (splits * rows * 256 + 255) // 256 * 256 + splits * rows * 4
    args = [dev_array(c, n, 0) for n in ("q", "k_step", "v_step", "k_cache", "v_cache")]
    ws = tidar.attn_workspace(desc)
    ws.fill_(0xFF)
    out = torch.empty_like(args[0])
    lse = torch.empty(out.shape[:-1], dtype=torch.float32, device=out.device)
    tidar.attn_step(desc, *args, torch.from_numpy(c.cache_len).cuda(), out, lse, None, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref, rlse = oracle.attn_step(*oracle_inputs(c), c.cache_len, k=c.k, num_blocks=c.num_blocks,
                                 block_len=c.block_len, sm_scale=c.sm_scale)
    assert np.isfinite(got).all()
    assert _report(f"{splits} forced splits, NaN workspace", got, ref, TOL["bf16"]) <= TOL["bf16"]
    assert np.abs(lse.cpu().numpy() - rlse).max() <= LSE_TOL["bf16"]


def _ragged_table(lens, slots, local_tiles, max_len):
    """Host restatement of the device's split apportionment (start, count) per
    sequence: weights of prefix tiles plus twice the step-key tiles, and the
    smallest weight per split c whose counts fit the slots."""
    w = [(min(max(l, 0), max_len) + 63) // 64 + 2 * local_tiles for l in lens]
    count = lambda c: sum(max(1, -(-wi // c)) for wi in w)
    if len(lens) <= 64:
        c = next(c for c in range(1, sum(w) + 1) if count(c) <= slots)
    else:  # more sequences than a wave's lanes: c = ceil(sum w / (slots - B))
        c = -(-sum(w) // (slots - len(lens)))
    tab, start = [], 0
    for wi in w:
        si = max(1, -(-wi // c))
        tab.append((start, si))
        start += si
    assert start <= slots
    return tab


_MANY = [int(x) for x in np.random.default_rng(70).integers(0, 400, size=70)]


@pytest.mark.parametrize("lens", [[0, 5, 64, 700, 3000, 129, 1, 2048], [4096, 4096], [0, 0, 0], _MANY],
                         ids=["mixed", "equal", "empty", "70seq"])
def test_ragged_batch_split_apportionment(lens, monkeypatch):
    """Batches of several sequences share the split slots out in proportion to
    each sequence's key tiles. Checked: the split table the kernel leaves in the
    workspace, every output row against the oracle (workspace filled with NaN
    bytes first, so an unwritten partial that the merge read would show), and
    agreement with one split count for all sequences (TIDAR_ATTN_RAGGED=0)."""
    import ar_self_speculative_amd as tidar
    from tests.gpu_util import attn_desc, dev_array
    k, nb, bl = 4, 5, 4
    c = attn_case(dtype="bf16", layers=1, batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128, k=k,
                  num_blocks=nb, block_len=bl, cache_len=lens, cache_capacity=max(lens) + 8, seed=len(lens))
    args = [dev_array(c, n, 0) for n in ("q", "k_step", "v_step", "k_cache", "v_cache")]
    dlens = torch.from_numpy(c.cache_len).cuda()
    outs = {}
    for mode in ("ragged", "static"):
        with monkeypatch.context() as mp:
            mp.setenv("TIDAR_ATTN_RAGGED", "1" if mode == "ragged" else "0")
            desc = attn_desc(c)
            ws = tidar.attn_workspace(desc)  # None when one split needs no partials
            if ws is not None:
                ws.fill_(0xFF)
            out = torch.empty_like(args[0])
            lse = torch.empty(out.shape[:-1], dtype=torch.float32, device=out.device)
            tidar.attn_step(desc, *args, dlens, out, lse, None, ws)
            torch.cuda.synchronize()
        if mode == "ragged":
            # 512 slots over Hkv = 2 KV heads x 1 query tile, at most B x (tiles + local) of them
            R = k + nb * bl
            local = (k + 63) // 64 + (bl + 63) // 64
            tiles = (max(lens) + 63) // 64
            slots = min(512 // 2, len(lens) * (tiles + local))
            tab = ws[: 8 * len(lens)].view(torch.int32).cpu().numpy().reshape(-1, 2)
            assert [tuple(t) for t in tab.tolist()] == _ragged_table(lens, slots, local, max(lens))
        outs[mode] = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy())
    ref, rlse = oracle.attn_step(*oracle_inputs(c), c.cache_len, k=c.k, num_blocks=c.num_blocks,
                                 block_len=c.block_len, sm_scale=c.sm_scale)
    for mode, (got, glse) in outs.items():
        assert np.isfinite(got).all(), mode
        assert _report(f"ragged {lens} {mode}", got, ref, TOL["bf16"]) <= TOL["bf16"]
        assert np.abs(glse - rlse).max() <= LSE_TOL["bf16"]
    # the two plans merge differently rounded bf16 partials: they agree to a
    # bf16 ulp or two of each output (2^-7 relative per ulp)
    diff = np.abs(outs["ragged"][0] - outs["static"][0])
    assert (diff <= 2 ** -6 * np.maximum(1.0, np.abs(ref))).all(), float(diff.max())


def test_cache_len_beyond_bound_is_clamped_and_flagged():
    c = attn_case(dtype="bf16", layers=1, batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, k=4,
                  num_blocks=5, block_len=4, cache_len=100, cache_capacity=120, seed=5, poison=False)
    out, _, status = run_attn(c, cache_len=[110], max_cache_len=100, with_status=True)
    ref, _ = _oracle_full(c, cache_len=[100])
    assert status & 1
    assert np.abs(out - ref).max() <= TOL["bf16"]


@pytest.mark.parametrize("cfg", [1, 2])
def test_ten_calls_on_one_workspace_bitwise_equal(cfg):
    """Ten launches on one workspace: outputs and LSEs equal bit for bit (an LDS
    or partial-buffer race would show as run-to-run differences)."""
    import ar_self_speculative_amd as tidar
    from tests.gpu_util import attn_desc, dev_array
    c = config_attn(cfg, seed=4)
    desc = attn_desc(c, num_splits=4)
    args = [dev_array(c, n, 0) for n in ("q", "k_step", "v_step", "k_cache", "v_cache")]
    lens = torch.from_numpy(c.cache_len).cuda()
    ws = tidar.attn_workspace(desc)
    outs, lses = [], []
    for _ in range(10):
        out = torch.empty_like(args[0])
        lse = torch.empty(out.shape[:-1], dtype=torch.float32, device=out.device)
        tidar.attn_step(desc, *args, lens, out, lse, None, ws)
        outs.append(out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32).cpu().numpy())
        lses.append(lse.view(torch.int32).cpu().numpy())
    for i in range(1, 10):
        assert np.array_equal(outs[0], outs[i]) and np.array_equal(lses[0], lses[i])


def test_timestamped_launch_is_the_same_computation(monkeypatch):
    """TIDAR_ATTN_STAMPS=1 selects the timestamped instantiation of the main
    kernel (bench.py --stamps): at the Qwen3-8B step's launch its output
    equals the plain launch's bit for bit, and every workgroup's record is
    ordered (entry <= first scores <= loop end <= stores acknowledged)."""
    import ar_self_speculative_amd as tidar
    c = config_attn(3, seed=2, layers=1)
    monkeypatch.delenv("TIDAR_ATTN_STAMPS", raising=False)
    base, _ = run_attn(c, with_lse=False)
    monkeypatch.setenv("TIDAR_ATTN_STAMPS", "1")
    out, _ = run_attn(c, with_lse=False)
    assert np.array_equal(out, base)
    r = tidar.attn_stamps(4096).astype(np.int64)
    nwg = int(r[0, 7] >> 32)
    assert 0 < nwg <= 4096
    r = r[:nwg]
    assert np.all(r[:, 0] <= r[:, 2]) and np.all(r[:, 2] <= r[:, 3]) and np.all(r[:, 3] <= r[:, 4])
    assert np.all(r[:, 1] <= r[:, 5])
    assert np.all((r[:, 7] & 0xFFFF) > 0)  # every workgroup of this launch had tiles
