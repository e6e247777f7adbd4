"""The synthetic error-accumulation study (study_error_accumulation.py): its summary on the CPU, and a
short run on the GPU through the quantise / append / decode entry points."""
import json
import math
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import study_error_accumulation as study  # noqa: E402


def test_summary_averages_over_seeds_and_keeps_every_run():
    args = study.parse(["--prefix", "128", "--steps", "64", "--seeds", "1,2", "--report", "32,64"])
    keys = [("free", "kvarn_k4v2_g128", 8), ("forced", "kvarn_k4v2_g128", 8)]
    per_seed = []
    for sd in (1, 2):
        out = {keys[0]: {"o": [0.1 * sd, 0.2 * sd], "o_all": 0.3 * sd, "x": [0.01 * sd, 0.02 * sd], "x_all": 0.03 * sd},
               keys[1]: {"o": [1.0 * sd, 2.0 * sd], "o_all": 3.0 * sd}}
        per_seed.append(([32, 64], out))
    s = study.summarise(args, [1, 2], per_seed)
    json.dumps(s)
    assert s["steps"] == 64 and s["prefix"] == 128 and s["seeds"] == [1, 2]
    free, forced = s["rows"]
    assert (free["run"], free["format"], free["sinkhorn_iters"]) == keys[0]
    assert free["o_rel_l2"] == pytest.approx({32: 0.15, 64: 0.3})
    assert free["o_rel_l2_steps_after_256"] == pytest.approx(0.45)
    assert free["x_rel_l2"] == pytest.approx({32: 0.015, 64: 0.03})
    assert "x_rel_l2" not in forced and forced["o_rel_l2"] == pytest.approx({32: 1.5, 64: 3.0})


@pytest.mark.gpu
def test_short_study_runs_and_orders_formats_by_bits():
    """128-token prefix and 96 decode steps, one seed: every run reports finite errors, 8-bit K/V stays
    within a few percent of the fp16 reference, and the one-step error falls as V gains bits."""
    pytest.importorskip("torch")
    print("case: study prefix 128, 96 steps, seed 11", flush=True)
    s = study.main(["--prefix", "128", "--steps", "96", "--seeds", "11", "--report", "64,96"])
    rows = {(r["run"], r["format"], r["sinkhorn_iters"]): r for r in s["rows"]}
    assert len(rows) == 2 * len(study.CONFIGS)
    for r in s["rows"]:
        for v in list(r["o_rel_l2"].values()) + list(r.get("x_rel_l2", {}).values()):
            assert math.isfinite(v) and v >= 0.0
    f = {fmt: rows[("forced", fmt, 8)]["o_rel_l2"][96]
         for fmt in ("kvarn_k8v8_g128", "kvarn_k4v8_g128", "kvarn_k4v2_g128", "kvarn_k2v2_g128")}
    assert f["kvarn_k8v8_g128"] < 0.05
    assert f["kvarn_k8v8_g128"] < f["kvarn_k4v8_g128"] < f["kvarn_k4v2_g128"] < f["kvarn_k2v2_g128"]
    x88 = rows[("free", "kvarn_k8v8_g128", 8)]["x_rel_l2"]
    assert np.all(np.asarray(list(x88.values())) < 0.02)
