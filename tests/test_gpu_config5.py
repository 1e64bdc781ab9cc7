"""Ragged batch at full depth, 64 decode steps end to end (attention ->
sampler -> commit), against the oracle.

Eight sequences with prefix lengths drawn from U{256..4096}, k = 8 (R = 80
query rows), Qwen3-8B heads (32 query, 8 KV, D = 128), all 36 layers, cache
capacity 4608. The cache and every step's queries and step keys/values are
drawn on the device from seeded generators and copied back where the oracle
needs them; the verifier inputs of step `it` are the recipe's numpy draws
with the calibrated noise scale (mean ~7 committed tokens per step). The
oracle keeps its own copy of the rows the commits may write and is compared
after every step:

* attention on sampled rows of four layers every 8th step and at the last
  step, so that every layer is checked (max-abs 2e-2, bf16), against the
  oracle's own view of the cache (the initial cache plus its own commits);
* accept lengths and next tokens (bit-exact apart from the counted near-ties,
  tests/gpu_util.py::check_samples);
* the new lengths and the rows the step may have written, bit-exact; at the
  end, every committed row of every layer, and every row outside the
  appended range unchanged.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tidar_synth import CONFIGS, config5_lengths, config5_step_sampler, fill_device_step
from tests.gpu_util import check_samples

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "config5_sigma.json")


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.timeout(600)
def test_config5_ragged_full_depth_64_steps():
    import ar_self_speculative_amd as tidar

    c = CONFIGS[5]
    L, B, k, cap, steps = c["layers"], c["batch"], c["k"], c["cap"], c["steps"]
    Hq, Hkv, D, V = c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["vocab"]
    R = k + (k + 1) * k
    assert c["sampler"]["diff_sigma"] == json.load(open(GOLDEN))["sigma"]
    lens0 = config5_lengths(0)
    W = k * steps                                   # rows the commits may append per sequence
    assert int(lens0.max()) + W <= cap
    step = tidar.DecodeStep(layers=L, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, k=k,
                            cache_capacity=cap, max_cache_len=int(lens0.max()) + W, vocab=V)
    sm_scale = step.desc.sm_scale
    fill_device_step(step, seed=5, cache_len=lens0)
    torch.cuda.synchronize()
    k0, v0 = step.k_cache.clone(), step.v_cache.clone()   # the initial cache (device copy)
    # the oracle's copy of each sequence's appendable rows [P0_b, P0_b + W)
    win_k = np.stack([_bits(k0[:, b, :, lens0[b]:lens0[b] + W]) for b in range(B)], axis=1)
    win_v = np.stack([_bits(v0[:, b, :, lens0[b]:lens0[b] + W]) for b in range(B)], axis=1)
    rel = np.zeros(B, np.int32)                      # committed rows past P0_b
    gen = torch.Generator(device="cuda").manual_seed(1234)

    committed, acc_flips, draw_flips, checked_layers, n_checks = [], 0, 0, set(), 0
    for it in range(steps):
        for t in (step.q, step.k_step, step.v_step):
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda", dtype=torch.float32))
        sc = config5_step_sampler(it)
        step.ar_logits.copy_(torch.from_numpy(sc.ar_logits).cuda())
        step.diff_logits.copy_(torch.from_numpy(sc.diff_logits).cuda())
        step.drafts.copy_(torch.from_numpy(sc.drafts).cuda())
        step.uniforms.copy_(torch.from_numpy(sc.uniforms).cuda())
        if it % 16 == 0:
            print(f"[cfg5] step {it}", flush=True)
        step.run()
        torch.cuda.synchronize()
        assert int(step.dev_status.item()) == 0
        lens = lens0 + rel

        # attention on sampled rows of four layers, against the oracle's view of the cache
        if it % 8 == 0 or it == steps - 1:
            srng = np.random.default_rng(1000 + it)
            n_checks += 1
            for layer in ((4 * (n_checks - 1) + j) % L for j in range(4)):
                checked_layers.add(layer)
                kc = _f32(_bits(k0[layer]))
                vc = _f32(_bits(v0[layer]))
                for b in range(B):
                    kc[b, :, lens0[b]:lens0[b] + W] = _f32(win_k[layer, b])
                    vc[b, :, lens0[b]:lens0[b] + W] = _f32(win_v[layer, b])
                rows = [(int(srng.integers(B)), int(r), int(srng.integers(Hq)))
                        for r in (0, k - 1, k, 2 * k - 1, R - 1, *srng.integers(R, size=7))]
                ref, _ = oracle.attn_rows(_f32(_bits(step.q[layer])), _f32(_bits(step.k_step[layer])),
                                          _f32(_bits(step.v_step[layer])), kc, vc, lens, rows, k=k,
                                          num_blocks=k + 1, block_len=k, sm_scale=sm_scale)
                out = step.out[layer].float().cpu().numpy()
                err = float(np.abs(np.stack([out[b, r, h] for b, r, h in rows]) - ref).max())
                print(f"[parity] cfg5 step {it} layer {layer}: max-abs {err:.3e}", flush=True)
                assert err <= 2e-2, (it, layer, err)

        # sampler
        acc = step.accept_len.cpu().numpy()
        nxt = step.next_token.cpu().numpy()
        ref = oracle.reject_sample(sc.ar_logits, sc.diff_logits, sc.drafts, sc.uniforms)
        a, d = check_samples(ref, acc, nxt, sc.ar_logits, sc.diff_logits, sc.uniforms)
        acc_flips += a
        draw_flips += d
        committed.extend((acc + 1).tolist())

        # commit: the oracle appends the accepted drafts (those the GPU chose) to its own rows
        ks = _bits(step.k_step[:, :, :k])
        vs = _bits(step.v_step[:, :, :k])
        win_k, win_v, new_rel = oracle.kv_commit(ks, vs, win_k, win_v, acc, rel)
        assert np.array_equal(step.cache_len_out.cpu().numpy(), lens0 + new_rel)
        for b in range(B):
            lo = int(lens[b])
            np.testing.assert_array_equal(_bits(step.k_cache[:, b, :, lo:lo + k]), win_k[:, b, :, rel[b]:rel[b] + k])
            np.testing.assert_array_equal(_bits(step.v_cache[:, b, :, lo:lo + k]), win_v[:, b, :, rel[b]:rel[b] + k])
        rel = new_rel.astype(np.int32)
        step.cache_len.copy_(step.cache_len_out)

    # every appendable row of every layer, and everything else unchanged
    for b in range(B):
        lo = int(lens0[b])
        np.testing.assert_array_equal(_bits(step.k_cache[:, b, :, lo:lo + W]), win_k[:, b])
        np.testing.assert_array_equal(_bits(step.v_cache[:, b, :, lo:lo + W]), win_v[:, b])
        for cur, init in ((step.k_cache, k0), (step.v_cache, v0)):
            assert torch.equal(cur[:, b, :, :lo].view(torch.int16), init[:, b, :, :lo].view(torch.int16))
            assert torch.equal(cur[:, b, :, lo + W:].view(torch.int16), init[:, b, :, lo + W:].view(torch.int16))
    assert checked_layers == set(range(L))
    mean = float(np.mean(committed))
    hist = np.bincount(np.asarray(committed), minlength=k + 2)[1:].tolist()
    print(f"[cfg5] committed tokens per step: mean {mean:.3f}, histogram n+1=1..{k + 1}: {hist}; "
          f"accept near-tie flips {acc_flips}, draws across a boundary {draw_flips}; "
          f"final lengths {(lens0 + rel).tolist()}", flush=True)
    assert 6.5 <= mean <= 7.5, mean
