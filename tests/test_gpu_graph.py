"""A whole decode step recorded into a HIP graph replays to the eager result.

The graph is replayed several times with unrelated eager device work and
host synchronisations in between; every replay must reproduce the eager
step bit for bit (attention output, accept length, next token, the
committed cache and the new lengths).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _snapshot(step):
    bits = lambda t: t.view(torch.int16).cpu().numpy().copy() if t.dtype == torch.bfloat16 else t.cpu().numpy().copy()
    return dict(out=bits(step.out), acc=bits(step.accept_len), nxt=bits(step.next_token),
                kc=bits(step.k_cache), vc=bits(step.v_cache), len_out=bits(step.cache_len_out),
                status=bits(step.dev_status))


@pytest.mark.parametrize("lens", [[200, 77], [256, 256]])
def test_step_graph_replays_match_eager(lens):
    import ar_self_speculative_amd as tidar
    from tidar_synth import fill_device_step

    step = tidar.DecodeStep(layers=2, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, k=4,
                            cache_capacity=300, max_cache_len=256, vocab=4096)
    fill_device_step(step, seed=11, cache_len=lens)
    step.run()
    torch.cuda.synchronize()
    ref = _snapshot(step)
    assert ref["status"].item() == 0
    graph = step.capture()
    for i in range(3):
        step.out.zero_()
        step.accept_len.fill_(-1)
        step.next_token.fill_(-1)
        x = torch.randn(1 << 16, device="cuda")
        assert torch.isfinite(x.sum()).item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(step)
        for name in ref:
            assert np.array_equal(got[name], ref[name]), (i, name)


@pytest.mark.parametrize("P,R,decode", [(2048, 1, True),    # decode-regime kernel (chosen by the planner)
                                        (4096, 1, False),   # main kernel, 22 splits: merge lanes share a vector
                                        (1024, 4, True)])
def test_few_rows_attention_graph_replays_match_eager(P, R, decode, monkeypatch):
    """Append-prefill attention with few rows (64 query heads, 8 KV heads):
    a graph of several launches on rotating caches replays to the eager
    outputs and log-sum-exps bit for bit, with eager work in between."""
    import math

    import ar_self_speculative_amd as tidar

    monkeypatch.delenv("TIDAR_ATTN_DECODE", raising=False)
    monkeypatch.delenv("TIDAR_ATTN_FUSED_MERGE", raising=False)
    Hq, Hkv, D, n = 64, 8, 128, 3
    g = torch.Generator(device="cuda").manual_seed(P + R)
    rnd = lambda *s: torch.randn(s, generator=g, device="cuda").to(torch.bfloat16)
    desc = tidar.make_attn_desc(batch=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, k=R, num_blocks=0,
                                block_len=1, cache_capacity=P + 64, max_cache_len=P, sm_scale=1 / math.sqrt(D),
                                dtype=tidar.DTYPE_BF16)
    # the planner's choice, read from the workspace layout (the decode plan has one split per 128 keys + 1)
    S = P // 128 + 1
    rows = R * Hq
    dec_bytes = 256 + (S * rows * D * 2 + 255) // 256 * 256 + S * rows * 4
    assert (tidar.attn_workspace_bytes(desc) == dec_bytes) == decode
    lens = torch.full((1,), P - 37, dtype=torch.int32, device="cuda")
    q = [rnd(1, R, Hq, D) for _ in range(n)]
    ks, vs = rnd(1, R, Hkv, D), rnd(1, R, Hkv, D)
    kc = [rnd(1, Hkv, P + 64, D) for _ in range(n)]
    vc = [rnd(1, Hkv, P + 64, D) for _ in range(n)]
    out = [torch.empty_like(q[0]) for _ in range(n)]
    lse = [torch.empty((1, R, Hq), dtype=torch.float32, device="cuda") for _ in range(n)]
    ws = tidar.attn_workspace(desc, torch.device("cuda"))

    def run():
        for i in range(n):
            tidar.attn_step(desc, q[i], ks, vs, kc[i], vc[i], lens, out[i], lse[i], None, ws)

    run()
    torch.cuda.synchronize()
    ref = [(o.view(torch.int16).cpu().numpy().copy(), l.cpu().numpy().copy()) for o, l in zip(out, lse)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in out:
            o.zero_()
        x = torch.randn(1 << 16, device="cuda")
        assert torch.isfinite(x.sum()).item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, l) in enumerate(zip(out, lse)):
            assert np.array_equal(o.view(torch.int16).cpu().numpy(), ref[i][0]), (rep, i)
            assert np.array_equal(l.cpu().numpy(), ref[i][1]), (rep, i)
