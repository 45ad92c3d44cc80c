"""Pin the oracle to hand-computed 3x3 cases (tests/golden/hand_cases.json).

The cases distinguish cross-correlation from a flipped convolution (H2), fix
the sign of the tap offset (H4, H5c), the bias (H3c) and the bias gradient
(H6), and tie the three passes together through the adjoint value (H7)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _load():
    with open(GOLDEN) as f:
        d = json.load(f)
    mats = {k: np.array(v, dtype=np.float64).reshape(1, 1, 3, 3) for k, v in d["matrices"].items()}
    return d, mats


def test_hand_cases_exact():
    d, m = _load()
    assert len(d["cases"]) == 12
    for case in d["cases"]:
        exp = np.array(case["expected"], dtype=np.float64)
        if case["pass"] == "fwd":
            got = oracle.conv3x3_fwd(m[case["x"]], m[case["w"]], np.array([case["b"]]))[0, 0]
        elif case["pass"] == "bwd_data":
            got = oracle.conv3x3_bwd_data(m[case["g"]], m[case["w"]])[0, 0]
        else:
            dw, db = oracle.conv3x3_bwd_weight(m[case["x"]], m[case["g"]])
            got = dw[0, 0]
            assert db[0] == case["expected_db"], case["name"]
        assert np.array_equal(got, exp), (case["name"], got, exp)


def test_hand_adjoint_value():
    d, m = _load()
    A = m["A"]
    v = d["adjoint"]["value"]
    assert np.sum(oracle.conv3x3_fwd(A, A) * A) == v
    assert np.sum(A * oracle.conv3x3_bwd_data(A, A)) == v
    assert np.sum(oracle.conv3x3_bwd_weight(A, A)[0] * A) == v


def test_fwd_no_bias_equals_zero_bias():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 3, 5, 6))
    w = rng.standard_normal((4, 3, 3, 3))
    assert np.array_equal(oracle.conv3x3_fwd(x, w, None), oracle.conv3x3_fwd(x, w, np.zeros(4)))


def test_sampled_entry_points_match_whole_tensor():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 5, 6, 7))
    w = rng.standard_normal((3, 5, 3, 3))
    b = rng.standard_normal(3)
    g = rng.standard_normal((2, 3, 6, 7))
    y = oracle.conv3x3_fwd(x, w, b)
    dx = oracle.conv3x3_bwd_data(g, w)
    dw, db = oracle.conv3x3_bwd_weight(x, g)
    i = rng.integers(0, y.size, 50)
    assert np.array_equal(oracle.conv3x3_fwd_at(x, w, b, i), y.ravel()[i])
    i = rng.integers(0, dx.size, 50)
    assert np.array_equal(oracle.conv3x3_bwd_data_at(g, w, i), dx.ravel()[i])
    i = rng.integers(0, dw.size, 50)
    assert np.array_equal(oracle.conv3x3_bwd_weight_at(x, g, i), dw.ravel()[i])
    assert np.array_equal(oracle.conv3x3_bias_grad_at(g, [0, 1, 2]), db)
