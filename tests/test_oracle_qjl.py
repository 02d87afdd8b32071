"""Pins of the oracle's 1-bit QJL residual sketch (TurboQuant-prod; "TurboQuant: paper
algorithm and vLLM engineering" diagram, paper column: the residual box and the QJL box):
a hand-worked example, the unbiasedness of the inner-product estimate and its variance
(closed form) by Monte Carlo over the Gaussian matrix, the key-logit estimate through
the full encode -> record -> packed-logit path unbiased for q . k, and the record layout."""
from __future__ import annotations

import math

import numpy as np

from gtq_inputs import head_rotations, qjl_matrix
from oracle import gtq_oracle as O


def test_hand_example():
    # S = I (2 x 2), r = (3, -4): gamma = 5, signs (+, -); y = (2, 1): S y = (2, 1), so the
    # estimate is 5 * sqrt(pi/2) / 2 * (2 - 1) = 3.13328534328875...
    S = np.eye(2, dtype=np.float32)
    gamma, bits, proj = O.qjl_encode(np.array([[3.0, -4.0]]), S)
    assert gamma[0] == np.float32(5.0) and bits.tolist() == [[1, 0]]
    est = O.qjl_inner(np.array([[2.0, 1.0]], np.float32), bits, gamma, S)
    assert abs(est[0, 0] - 3.13328534328875) < 1e-12
    # a projection of exactly zero counts as +
    _, b0, _ = O.qjl_encode(np.array([[0.0, 1.0]]), np.array([[1.0, 0.0]], np.float32))
    assert b0.tolist() == [[1]]


def test_estimate_unbiased_with_closed_form_variance():
    """E over S ~ N(0,1)^{m x d} of gamma sqrt(pi/2)/m sum_j (S y)_j sign((S r)_j) is y . r,
    with variance (pi / (2 m)) |r|^2 |y|^2 - (y . r)^2 / m."""
    rng = np.random.default_rng(7)
    d = m = 16
    r = rng.standard_normal(d)
    y = rng.standard_normal(d).astype(np.float32)
    n = 40000
    est = np.empty(n)
    for i in range(n):
        S = rng.standard_normal((m, d)).astype(np.float32)
        g, bits, _ = O.qjl_encode(r, S)
        est[i] = O.qjl_inner(y, bits, g, S)[0, 0]
    # with S fixed per draw, the estimator's target is y . r for the fp32 inputs it saw
    yr = float(np.dot(y.astype(np.float64), r))
    var = math.pi / (2 * m) * np.dot(r, r) * np.dot(y.astype(np.float64), y) - yr ** 2 / m
    se = math.sqrt(var / n)
    assert abs(est.mean() - yr) < 4 * se, (est.mean(), yr, se)
    assert abs(est.var() / var - 1) < 0.05, (est.var(), var)


def test_key_logit_unbiased_through_the_record():
    """A K2-prod key (K1 MSE part + sketch) of a real head plan: the logit q . k_hat +
    sketch estimate from the packed record, averaged over matrices S, is q . k."""
    rng = np.random.default_rng(11)
    scores = np.exp(2 * rng.standard_normal(64))
    rates = O.greedy_allocate(scores, O.rate_distortion(), 1, 4, 64)
    kr, vr = head_rotations(3, 0, 0, [len(c) for _, c in O.groups_from_rates(rates, O.HALF)])
    k = rng.standard_normal((1, 128)).astype(np.float32)
    v = rng.standard_normal((1, 128)).astype(np.float32)
    mse_plan = O.HeadPlan(rates, kr, vr, 2)
    e0 = O.encode_kv(mse_plan, k, v)
    # the query along the key's residual: the MSE logit then misses q . r = |r|^2
    q = (k.astype(np.float64) - O.dequantized_keys(mse_plan, e0["k_words"], e0["k_norms"])).astype(np.float32)
    exact = float((q.astype(np.float64) @ k.astype(np.float64).T)[0, 0])
    mse_logit = O.packed_logits(mse_plan, q, e0["k_words"], e0["k_norms"], 1.0)[0, 0]
    n = 3000
    vals = np.empty(n)
    for i in range(n):
        S = rng.standard_normal((128, 128)).astype(np.float32)
        plan = O.HeadPlan(rates, kr, vr, 2, qjl=S)
        e = O.encode_kv(plan, k, v)
        vals[i] = O.packed_logits(plan, q, e["k_words"], e["k_norms"], 1.0)[0, 0]
    se = vals.std() / math.sqrt(n)
    assert abs(vals.mean() - exact) < 4 * se, (vals.mean(), exact, se)
    # and the MSE logit alone is off by more than that: the sketch removes a real bias
    assert abs(mse_logit - exact) > 8 * se, (mse_logit, exact, se)


def test_record_layout():
    rng = np.random.default_rng(5)
    rates = O.greedy_allocate(np.exp(rng.standard_normal(64)), O.rate_distortion(), 1, 4, 128)
    kr, vr = head_rotations(5, 0, 0, [len(c) for _, c in O.groups_from_rates(rates, O.HALF)])
    S = qjl_matrix(5, 0, 0)
    k = rng.standard_normal((9, 128)).astype(np.float32)
    k[4] = 0.0
    v = rng.standard_normal((9, 128)).astype(np.float32)
    plan = O.HeadPlan(rates, kr, vr, 2, qjl=S)
    e = O.encode_kv(plan, k, v)
    e0 = O.encode_kv(O.HeadPlan(rates, kr, vr, 2), k, v)
    mw = plan.mse_words
    assert e["k_words"].shape == (9, mw + 5) and mw == 8
    assert np.array_equal(e["k_words"][:, :mw], e0["k_words"])
    bits, gamma = O.qjl_fields(plan, e["k_words"])
    assert np.array_equal(bits, e["qjl_bits"]) and np.array_equal(gamma, e["qjl_gamma"])
    # bit j of the sketch is bit j % 32 of word mw + j // 32
    assert ((e["k_words"][:, mw + 1] >> 5) & 1).tolist() == e["qjl_bits"][:, 37].tolist()
    # the zero key: zero residual, gamma 0, every projection 0 -> every sign +
    assert gamma[4] == 0.0 and bits[4].all()
    # the residual is the key minus its decoded MSE record
    r = k.astype(np.float64) - O.dequantized_keys(plan, e["k_words"], e["k_norms"])
    assert np.allclose(np.sqrt((r * r).sum(1)).astype(np.float32), gamma, rtol=0, atol=0)
