"""The oracle against the hand-worked cases in tests/golden/hand_worked.json.

Those values were derived by hand from the definitions (each case names the
passage it follows); no program wrote them.
"""

import json
import os

import numpy as np
import pytest

from oracle import attend_block, attended_keys, build_pyramid, descend

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))
BS = 2  # tokens per block in the hand-worked descents


def _levels(case):
    k = np.repeat(np.asarray(case["block_means"], np.float32), BS)[None, None, :, None]
    return [p[0, 0] for p in build_pyramid(k, BS, case["fanout"], case["levels"])]


@pytest.mark.parametrize("case", GOLDEN["descents"], ids=lambda c: c["name"])
def test_hand_worked_descent(case):
    tr = []
    sel = descend(_levels(case), np.array([float(case["qbar"])]), case["query_block"], case["top_k"],
                  case["sink_blocks"] * BS, BS, case["fanout"], tr, case.get("causal", True))
    assert sel == case["selected"]
    assert [t["pool"] for t in tr] == case["pools"]


def test_hand_worked_exhaustive_differs():
    case = next(c for c in GOLDEN["descents"] if "exhaustive_top_k" in c)
    means = np.asarray(case["block_means"], np.float64) * case["qbar"]
    cand = list(range(case["sink_blocks"], case["query_block"]))
    best = sorted(sorted(cand, key=lambda j: (-means[j], j))[:case["top_k"]])
    assert best == case["exhaustive_top_k"] != case["selected"]


@pytest.mark.parametrize("case", GOLDEN["attention"], ids=lambda c: c["name"])
def test_hand_worked_attended_set_and_output(case):
    bs, s, i = case["block_size"], case["sink_len"], case["query_position"]
    assert attended_keys(i, case["selected"], s, bs).tolist() == case["attended"]
    n = (i // bs + 1) * bs
    k = np.zeros((n, 1))
    v = np.arange(n, dtype=np.float64)[:, None]
    q = np.ones((1, 1))
    o, _ = attend_block(q, k, v, i, case["selected"], s, bs, 1.0)
    assert o[0, 0] == pytest.approx(case["output_if_value_is_position"], abs=1e-12)


@pytest.mark.parametrize("case", GOLDEN["pyramids"], ids=lambda c: c["name"])
def test_hand_worked_max_pyramid(case):
    k = np.asarray(case["rows"], np.float32)[None, None, :, None]
    lv = build_pyramid(k, case["block_size"], case["fanout"], case["levels"], pool="max")
    assert [x[0, 0, :, 0].tolist() for x in lv] == case["levels_max"]
