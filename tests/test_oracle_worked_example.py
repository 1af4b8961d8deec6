"""Pin the oracle's masked-set attention against the page's printed worked
example ("Story of Attention -- Part 4: Sparse Attention, Then and Now",
section 1, "Worked example"; fixture tests/golden/worked_example_strided.txt).
"""
import math
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def load_fixture():
    blocks, cur = {}, None
    with open(os.path.join(HERE, "golden", "worked_example_strided.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                blocks[cur] = []
                continue
            blocks[cur].append([float(x) for x in line.split()])
    return {k: np.array(v) for k, v in blocks.items()}


def test_mask_is_causal_stride_two():
    fx = load_fixture()
    n = 4
    expect = np.array([[1.0 if (c <= r and (r - c) % 2 == 0) else 0.0 for c in range(n)] for r in range(n)])
    assert np.array_equal(fx["mask"], expect)


def test_scores_and_masked_scores_exact():
    fx = load_fixture()
    qkt = fx["Q"] @ fx["K"].T
    assert np.array_equal(qkt, fx["QKT"])
    masked = np.where(fx["mask"] > 0, qkt, -np.inf)
    assert np.array_equal(masked, fx["masked"])


def test_dense_oracle_weights_and_output():
    fx = load_fixture()
    mask = fx["mask"] > 0
    out, lse, p = oracle.masked_attention_dense(fx["Q"], fx["K"], fx["V"], mask)  # scale 1/sqrt(4)
    assert np.max(np.abs(p - fx["A_sparse"])) <= 1e-3
    printed = fx["output"]
    diff = np.abs(out - printed)
    diff_wo = diff.copy()
    diff_wo[3, 3] = 0.0
    assert np.max(diff_wo) <= 1e-3
    # cell (4, 4): the page multiplied the rounded weight 0.622 by 5
    assert abs(out[3, 3] - 3.112297) <= 1e-6
    assert abs(out[3, 3] - printed[3, 3]) <= 2.5e-3
    assert abs((fx["A_sparse"] @ fx["V"])[3, 3] - printed[3, 3]) <= 1e-9
    # exact values of the softmax rows with two keys
    s = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(p[2, 0] - s) < 1e-15 and abs(p[3, 3] - 1.0 / (1.0 + math.exp(-0.5))) < 1e-15
    # LSE (derived): row 1 = 1/2, row 2 = 1, row 3 = ln(e^1 + e^0), row 4 = ln(e^0.5 + e^1)
    assert np.allclose(lse, [0.5, 1.0, math.log(math.e + 1.0), math.log(math.exp(0.5) + math.e)], atol=1e-14)


def test_multiplying_scale_is_rejected_by_the_example():
    """The page's 'after scaling by 2' must mean divide: multiplying gives
    weights far from the printed ones."""
    fx = load_fixture()
    mask = fx["mask"] > 0
    _, _, p_mul = oracle.masked_attention_dense(fx["Q"], fx["K"], fx["V"], mask, scale=2.0)
    assert np.max(np.abs(p_mul - fx["A_sparse"])) > 0.2


def test_literal_oracle_matches_example():
    fx = load_fixture()
    mask = fx["mask"] > 0
    out, lse = oracle.masked_attention_literal(fx["Q"], fx["K"], fx["V"], lambda i, j: bool(mask[i, j]))
    out_d, lse_d, _ = oracle.masked_attention_dense(fx["Q"], fx["K"], fx["V"], mask)
    assert np.max(np.abs(out - out_d)) < 1e-14 and np.max(np.abs(lse - lse_d)) < 1e-14
