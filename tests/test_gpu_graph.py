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
