"""Oracle against the hand-worked example in tests/golden/ (closed forms)."""

import json
import math
import os

import numpy as np

import oracle
from oracle.attention import SKIPPED

HERE = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_prefill_example():
    fx = json.load(open(os.path.join(HERE, "hand_worked_prefill.json")))
    x = np.array(fx["x"])
    L, d = 4, 4
    q = np.zeros((1, 1, L, d))
    q[..., 0] = 2.0
    k = np.zeros((1, 1, L, d))
    k[0, 0, :, 0] = x
    v = np.array(fx["v"], dtype=np.float64)[None, None]
    env = {"E": math.exp(4), "a": math.exp(-6), "b": math.exp(-1), "log": math.log}
    for case in fx["cases"]:
        res = oracle.prefill(q, k, v, case["lambda"], fx["Br"], fx["Bc"], fx["causal"])
        assert res["margin"][0, 0, 1, 1] == float(fx["margin_tile_1_1"])
        sk = sorted([int(i), int(j)] for i, j in zip(*np.nonzero(res["decision"][0, 0] == SKIPPED)))
        assert sk == case["skipped"]
        for r in range(L):
            assert abs(res["lse"][0, 0, r] - eval(case["lse"][r], {}, env)) < 1e-13
            assert abs(res["out"][0, 0, r, 0] - eval(case["out_col0"][r], {}, env)) < 1e-13
            # columns 1 and 3 are constant over keys; column 2 is minus column 0
            assert abs(res["out"][0, 0, r, 1] - 1.0) < 1e-14
            assert abs(res["out"][0, 0, r, 2] + res["out"][0, 0, r, 0]) < 1e-14
