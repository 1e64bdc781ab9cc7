"""Host logic of the draft-length rule (ar_self_speculative_amd/draft_length.py):
the hinge fit, the roofline crossing, the choice of k, and that the rule
reproduces the draft length recorded in the committed knee profile from the
ceilings recorded there."""
import json
import os
import re

import pytest

from ar_self_speculative_amd import draft_length as dl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILE = os.path.join(ROOT, "profiles", "append_prefill_knee_h64_kv8_d128.md")


def test_step_rows():
    assert [dl.step_rows(k) for k in (1, 2, 4, 8, 16)] == [3, 8, 24, 80, 288]


def test_hinge_fit_recovers_a_planted_hinge():
    rows = [1, 8, 16, 32, 64, 128, 256, 512]
    c, b, knee = 9.0, 0.15, 40.0
    times = [c + b * max(knee, r) for r in rows]
    f = dl.hinge_fit(rows, times, grid=2000)
    assert f["knee_rows"] == pytest.approx(knee, rel=0.01)
    assert f["fixed"] == pytest.approx(c, rel=1e-3) and f["per_row"] == pytest.approx(b, rel=1e-3)
    assert f["rms"] < 0.01
    # the fixed cost does not move the knee
    f2 = dl.hinge_fit(rows, [t + 20.0 for t in times], grid=2000)
    assert f2["knee_rows"] == pytest.approx(knee, rel=0.01)


def test_roofline_knee_is_where_the_two_times_meet():
    P, Hq, Hkv, D, bw, f = 4096, 64, 8, 128, 6500.0, 1950.0
    r = dl.roofline_knee(prefix=P, q_heads=Hq, kv_heads=Hkv, head_dim=D, hbm_gbps=bw, mfma_tflops=f)
    t_hbm = (2 * Hkv * P * D * 2 + r * (2 * Hkv + 2 * Hq) * D * 2) / (bw * 1e9)
    t_mfma = 4 * Hq * D * P * r / (f * 1e12)
    assert t_hbm == pytest.approx(t_mfma, rel=1e-12)
    # at the nominal ceilings (8 TB/s, 2.5 PFLOP/s) the crossing is near 43 rows: 2.10 us of K/V
    # streaming against 0.0537 us of MFMA per row less 0.0046 us of per-row bytes
    assert dl.roofline_knee(prefix=P, q_heads=Hq, kv_heads=Hkv, head_dim=D, hbm_gbps=8000.0,
                            mfma_tflops=2500.0) == pytest.approx(42.7, abs=0.1)


def test_draft_length_boundaries():
    # Qwen3-8B step packs 4 query heads per KV head; the sweep has 8
    assert dl.draft_length(40.0, sweep_group=8, step_group=4) == 8      # 80 rows x 4 = 320 <= 320
    assert dl.draft_length(39.9, sweep_group=8, step_group=4) == 4
    assert dl.draft_length(144.0, sweep_group=8, step_group=4) == 16   # 288 x 4 = 1152
    assert dl.draft_length(0.5, sweep_group=8, step_group=4) == 1       # never below the smallest


def _profile_record():
    text = open(PROFILE).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    assert m, "the knee profile holds its bench line as a json block"
    return json.loads(m.group(1))


def test_rule_reproduces_the_committed_choice():
    rec = _profile_record()
    ceil = rec["ceilings"]
    knee = dl.roofline_knee(prefix=4096, q_heads=64, kv_heads=8, head_dim=128, hbm_gbps=ceil["hbm_read_gbps"],
                            mfma_tflops=ceil["mfma_bf16_tflops"])
    assert knee == pytest.approx(rec["knee_rows"]["4096"], abs=0.01)
    assert dl.draft_length(knee, sweep_group=8, step_group=4) == rec["draft_length_at_P4096"]["k"]
    # and the hinge fits recorded beside it come from the recorded sweep
    rows = rec["config"]["R"]
    for P, times in rec["us"].items():
        f = dl.hinge_fit(rows, times)
        assert f["knee_rows"] == pytest.approx(rec["sweep_hinge_fit"][P]["knee_rows"], abs=1e-3)
