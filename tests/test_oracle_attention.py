"""Pins of the oracle's packed-cache attention (decode and chunked prefill).

Checks: packed-path logits equal logits of dequantized keys (two independent
evaluation orders); the packed decode equals a library softmax attention over the
dequantized cache; the blockwise logit-error bound of the Block-GTQ abstract holds
against exact (unquantized) logits; closed-form special cases (one token,
identical keys); prefill reduces to decode and is causal."""
import math

import numpy as np
import pytest
from scipy.special import softmax

from gtq_inputs import head_inputs, head_rotations
from oracle import gtq_oracle as O


def _plan_and_cache(seed=0, n=300, g=4, k_budget=128, v_bits=2, n_q=2):
    inp = head_inputs(seed, 0, 0, g, n, n_dec_q=n_q)
    s = O.energy_scores(inp["calib_q"], inp["calib_k"])
    rates = O.greedy_allocate(s, O.rate_distortion(), 1, 4, k_budget)
    dims = [len(c) for _, c in O.groups_from_rates(rates)]
    krots, vrot = head_rotations(seed, 0, 0, dims)
    plan = O.HeadPlan(rates, krots, vrot, v_bits)
    enc = O.encode_kv(plan, inp["k"], inp["v"])
    return inp, plan, enc


def test_packed_logits_equal_dequantized_key_logits():
    inp, plan, enc = _plan_and_cache()
    q = inp["q"].reshape(-1, 128)
    sc = 1 / math.sqrt(128)
    lp = O.packed_logits(plan, q, enc["k_words"], enc["k_norms"], sc)
    kh = O.dequantized_keys(plan, enc["k_words"], enc["k_norms"])
    ld = sc * q.astype(np.float64) @ kh.T
    assert np.allclose(lp, ld, rtol=1e-12, atol=1e-12 * np.abs(ld).max())


def test_decode_equals_library_attention_on_dequantized_cache():
    inp, plan, enc = _plan_and_cache(n=257)
    q = inp["q"].reshape(-1, 128)
    sc = 1 / math.sqrt(128)
    _, out = O.decode_attention(plan, q, enc["k_words"], enc["k_norms"], enc["v_words"],
                                enc["v_norms"], sc)
    kh = O.dequantized_keys(plan, enc["k_words"], enc["k_norms"])
    vh = O.dequantized_values(plan, enc["v_words"], enc["v_norms"])
    p = softmax(sc * q.astype(np.float64) @ kh.T, axis=1)
    assert np.allclose(out, p @ vh, rtol=1e-10, atol=1e-12)


def test_blockwise_logit_error_bound():
    """|q.k - q.k_hat| <= sum_j ||q_j|| ||k_j - k_hat_j|| over RoPE blocks j."""
    inp, plan, enc = _plan_and_cache(n=400)
    q = inp["q"].reshape(-1, 128).astype(np.float64)
    k = inp["k"].astype(np.float64)
    lp = O.packed_logits(plan, q, enc["k_words"], enc["k_norms"], 1.0)
    kh = O.dequantized_keys(plan, enc["k_words"], enc["k_norms"])
    exact = q @ k.T
    bound = np.zeros_like(exact)
    for j in range(64):
        a, b = O.block_coords(j)
        qn = np.sqrt(q[:, a] ** 2 + q[:, b] ** 2)
        en = np.sqrt((k[:, a] - kh[:, a]) ** 2 + (k[:, b] - kh[:, b]) ** 2)
        bound += qn[:, None] * en[None, :]
    assert np.all(np.abs(lp - exact) <= bound * (1 + 1e-9) + 1e-9)
    # and the key reconstruction error is of the codec's size, not arbitrary
    rel = np.sum((k - kh) ** 2, axis=1) / np.sum(k ** 2, axis=1)
    assert 0.005 < np.mean(rel) < 0.3


def test_single_token_cache_returns_its_value():
    inp, plan, enc = _plan_and_cache(n=5)
    q = inp["q"].reshape(-1, 128)
    _, out = O.decode_attention(plan, q, enc["k_words"], enc["k_norms"], enc["v_words"],
                                enc["v_norms"], 0.1, length=1)
    vh = O.dequantized_values(plan, enc["v_words"][:1], enc["v_norms"][:1])
    assert np.allclose(out, np.repeat(vh, q.shape[0], axis=0), rtol=1e-12, atol=1e-12)


def test_identical_keys_average_values():
    inp, plan, enc = _plan_and_cache(n=40)
    kw = np.repeat(enc["k_words"][:1], 40, axis=0)
    kn = np.repeat(enc["k_norms"][:1], 40, axis=0)
    q = inp["q"].reshape(-1, 128)
    logits, out = O.decode_attention(plan, q, kw, kn, enc["v_words"], enc["v_norms"], 0.3)
    vh = O.dequantized_values(plan, enc["v_words"], enc["v_norms"])
    assert np.allclose(out, np.repeat(vh.mean(axis=0, keepdims=True), q.shape[0], axis=0),
                       rtol=1e-10, atol=1e-12)
    assert np.allclose(logits, logits[:, :1])


def test_rotated_basis_accumulation_matches_plain_basis():
    """Accumulating values in the rotated basis and rotating back once equals averaging
    fully dequantized values (Pi^T is linear)."""
    inp, plan, enc = _plan_and_cache(n=64)
    q = inp["q"].reshape(-1, 128)
    logits, out = O.decode_attention(plan, q, enc["k_words"], enc["k_norms"], enc["v_words"],
                                     enc["v_norms"], 0.05)
    p = softmax(logits, axis=1)
    vh = O.dequantized_values(plan, enc["v_words"], enc["v_norms"])
    assert np.allclose(out, p @ vh, rtol=1e-10, atol=1e-12)
    assert np.allclose(p.sum(axis=1), 1.0)


def test_prefill_reduces_to_decode_and_is_causal():
    inp, plan, enc = _plan_and_cache(n=48)
    rng = np.random.default_rng(1)
    T, pos0 = 6, 40
    q = rng.standard_normal((T, 3, 128)).astype(np.float32)
    sc = 1 / math.sqrt(128)
    out = O.prefill_attention(plan, q, pos0, enc["k_words"], enc["k_norms"], enc["v_words"],
                              enc["v_norms"], sc)
    for t in range(T):
        _, o = O.decode_attention(plan, q[t], enc["k_words"][:pos0 + t + 1], enc["k_norms"][:pos0 + t + 1],
                                  enc["v_words"][:pos0 + t + 1], enc["v_norms"][:pos0 + t + 1], sc)
        assert np.allclose(out[t], o, rtol=1e-12, atol=1e-14)
    # changing a future token leaves earlier queries untouched
    kw = enc["k_words"].copy()
    kw[pos0 + 3] ^= np.uint32(0xFFFFFFFF)
    out2 = O.prefill_attention(plan, q, pos0, kw, enc["k_norms"], enc["v_words"], enc["v_norms"], sc)
    assert np.array_equal(out2[:3], out[:3])
    assert not np.allclose(out2[3:], out[3:])


# ---------------------------------------------------------------- fp16 sink + recent window

def test_window_positions_by_hand():
    """Length 20, 3 sink and 5 recent positions: 0, 1, 2 and 15..19 read the fp16
    buffers; a window longer than the sequence covers everything; none when both are 0."""
    assert np.flatnonzero(O.window_positions(20, 3, 5)).tolist() == [0, 1, 2, 15, 16, 17, 18, 19]
    assert O.window_positions(6, 4, 4).all()
    assert not O.window_positions(9, 0, 0).any()
    assert np.flatnonzero(O.window_positions(10, 0, 1)).tolist() == [9]


def test_window_without_buffers_is_the_packed_decode():
    inp, plan, enc = _plan_and_cache(n=150)
    q = inp["q"].reshape(-1, 128)
    sc = 1 / math.sqrt(128)
    args = (enc["k_words"], enc["k_norms"], enc["v_words"], enc["v_norms"])
    lg0, o0 = O.decode_attention(plan, q, *args, sc, length=150)
    lg1, o1 = O.decode_attention_window(plan, q, *args, inp["k"], inp["v"], 0, 0, sc, 150)
    assert np.array_equal(lg0, lg1)
    assert np.allclose(o0, o1, rtol=1e-13, atol=1e-15)


def test_window_covering_everything_is_fp16_attention():
    """Sink + recent >= length: plain softmax attention over the binary16-rounded K, V."""
    inp, plan, enc = _plan_and_cache(n=96)
    q = inp["q"].reshape(-1, 128).astype(np.float64)
    sc = 0.07
    args = (enc["k_words"], enc["k_norms"], enc["v_words"], enc["v_norms"])
    for ns, nr in ((96, 0), (0, 96), (40, 60)):
        _, o = O.decode_attention_window(plan, q, *args, inp["k"], inp["v"], ns, nr, sc, 96)
        k16 = inp["k"].astype(np.float16).astype(np.float64)
        v16 = inp["v"].astype(np.float16).astype(np.float64)
        ref = softmax(sc * q @ k16.T, axis=1) @ v16
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-14)


def test_window_brute_force_small():
    """Position by position in plain Python: fp16 key/value inside the window,
    dequantized packed key/value outside; softmax with math.exp."""
    inp, plan, enc = _plan_and_cache(n=23, n_q=1)
    q = inp["q"].reshape(-1, 128)[:2].astype(np.float64)
    sc = 0.09
    n, ns, nr = 23, 2, 6
    kh = O.dequantized_keys(plan, enc["k_words"], enc["k_norms"])
    vh = O.dequantized_values(plan, enc["v_words"], enc["v_norms"])
    lg, o = O.decode_attention_window(plan, q, enc["k_words"], enc["k_norms"], enc["v_words"], enc["v_norms"],
                                      inp["k"], inp["v"], ns, nr, sc, n)
    for r in range(2):
        logit, val = [], []
        for pos in range(n):
            if pos < ns or pos >= n - nr:
                kk = [float(np.float16(x)) for x in inp["k"][pos]]
                vv = [float(np.float16(x)) for x in inp["v"][pos]]
            else:
                kk, vv = list(kh[pos]), list(vh[pos])
            logit.append(sc * sum(a * b for a, b in zip(q[r], kk)))
            val.append(vv)
        mx = max(logit)
        w = [math.exp(x - mx) for x in logit]
        tot = sum(w)
        ref = [sum(w[p] * val[p][c] for p in range(n)) / tot for c in range(128)]
        assert np.allclose(lg[r], logit, rtol=1e-12, atol=1e-12)
        assert np.allclose(o[r], ref, rtol=1e-11, atol=1e-13)
