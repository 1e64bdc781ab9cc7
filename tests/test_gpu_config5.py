"""Ragged batch, 64 decode steps end to end (attention -> sampler -> commit).

Eight sequences with prefix lengths drawn from U{256..4096}, k = 8 (R = 80
query rows), Qwen3-8B heads (32 query, 8 KV, D = 128), cache capacity 4608,
two layers of the 36 (every layer runs the same kernels on its own slice).
Each step draws fresh queries, step keys/values and verifier inputs. The
oracle keeps its own cache and lengths and is compared after every step:

* attention on sampled rows of every layer, every 8th step (max-abs 2e-2, bf16),
* accept lengths and next tokens (bit-exact except oracle-flagged near-ties),
* the committed caches and the new lengths (bit-exact), after which the
  next step attends over the grown prefixes.
"""
import numpy as np
import pytest
import torch

import oracle
from tidar_synth import bf16_bits_to_f32, bf16_round, config_attn, sampler_case
from tests.gpu_util import check_samples

pytestmark = pytest.mark.gpu


def _to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(400)
def test_config5_ragged_multistep():
    import ar_self_speculative_amd as tidar

    L, steps = 2, 64
    c = config_attn(5, seed=0, layers=L)
    B, k, R, cap = c.batch, c.k, c.rows, c.cache_capacity
    Hq, Hkv, D = c.num_q_heads, c.num_kv_heads, c.head_dim
    V = 151936
    max_len = int(c.cache_len.max()) + k * steps
    assert max_len <= cap
    step = tidar.DecodeStep(layers=L, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, k=k,
                            cache_capacity=cap, max_cache_len=max_len, vocab=V)
    assert step.R == R and abs(step.desc.sm_scale - c.sm_scale) < 1e-7
    kc_bits, vc_bits = c.bits["k_cache"].copy(), c.bits["v_cache"].copy()
    step.k_cache.copy_(_to_dev_bf16(kc_bits))
    step.v_cache.copy_(_to_dev_bf16(vc_bits))
    lens = c.cache_len.astype(np.int32).copy()
    step.cache_len.copy_(torch.from_numpy(lens).cuda())

    rng = np.random.default_rng(5)
    committed = []
    near_ties = 0
    for it in range(steps):
        # fresh step inputs
        qb, qf = bf16_round(rng.standard_normal((L, B, R, Hq, D), dtype=np.float32))
        kb, kf = bf16_round(rng.standard_normal((L, B, R, Hkv, D), dtype=np.float32))
        vb, vf = bf16_round(rng.standard_normal((L, B, R, Hkv, D), dtype=np.float32))
        step.q.copy_(_to_dev_bf16(qb))
        step.k_step.copy_(_to_dev_bf16(kb))
        step.v_step.copy_(_to_dev_bf16(vb))
        sc = sampler_case(batch=B, k=k, vocab=V, ar_sigma=3.0, diff_mode="noisy", diff_sigma=0.5, seed=50 + it)
        step.ar_logits.copy_(torch.from_numpy(sc.ar_logits).cuda())
        step.diff_logits.copy_(torch.from_numpy(sc.diff_logits).cuda())
        step.drafts.copy_(torch.from_numpy(sc.drafts).cuda())
        step.uniforms.copy_(torch.from_numpy(sc.uniforms).cuda())
        step.run()
        torch.cuda.synchronize()
        assert int(step.dev_status.item()) == 0

        # attention on sampled rows of every layer, against the oracle's own cache
        out = step.out.float().cpu().numpy()
        srng = np.random.default_rng(1000 + it)
        for layer in (range(L) if it % 8 == 0 or it == steps - 1 else ()):
            rows = [(int(srng.integers(B)), int(r), int(srng.integers(Hq)))
                    for r in (0, k - 1, k, k + k - 1, R - 1, *srng.integers(R, size=19))]
            kcf = bf16_bits_to_f32(kc_bits[layer])
            vcf = bf16_bits_to_f32(vc_bits[layer])
            ref, _ = oracle.attn_rows(qf[layer], kf[layer], vf[layer], kcf, vcf, lens, rows, k=k,
                                      num_blocks=k + 1, block_len=k, sm_scale=c.sm_scale)
            got = np.stack([out[layer, b, r, h] for b, r, h in rows])
            err = float(np.abs(got - ref).max())
            if it % 16 == 0 or it == steps - 1:
                print(f"[parity] cfg5 step {it} layer {layer}: max-abs {err:.3e}", flush=True)
            assert err <= 2e-2

        # sampler
        acc = step.accept_len.cpu().numpy()
        nxt = step.next_token.cpu().numpy()
        ref = oracle.reject_sample(sc.ar_logits, sc.diff_logits, sc.drafts, sc.uniforms)
        excused, draw_near = check_samples(ref, acc, nxt, sc.ar_logits, sc.diff_logits, sc.uniforms)
        near_ties += excused + draw_near
        committed.extend((acc + 1).tolist())

        # commit: the oracle appends the accepted drafts the GPU chose
        ek, ev, el = oracle.kv_commit(kb, vb, kc_bits, vc_bits, acc, lens)
        assert np.array_equal(step.cache_len_out.cpu().numpy(), el)
        assert np.array_equal(_bits(step.k_cache), ek) and np.array_equal(_bits(step.v_cache), ev)
        kc_bits, vc_bits, lens = ek, ev, el.astype(np.int32)
        step.cache_len.copy_(step.cache_len_out)
    print(f"[cfg5] committed tokens per step: mean {np.mean(committed):.2f}; near-ties {near_ties}", flush=True)
