"""Property tests (hypothesis) over the oracle and the library's host ABI: the allocation
is the exact optimum of the separable proxy for any budget, rate range and score vector
(checked against dynamic programming, an independent exact solver); the library's
allocation, layouts and workspace sizing agree with the oracle and the record format for
arbitrary rates, head counts, GQA ratios, lengths and split sizes; the bit packing is a
bijection; the packed decode is a softmax average that splits over query heads and over
token chunks (log-sum-exp merge). No GPU is used."""
from __future__ import annotations

import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from gtq_inputs import HALF, INTERLEAVED, head_inputs, head_rotations
from oracle import gtq_oracle as O

G = pytest.importorskip("packed_cache_attention_tq_amd")

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
DIST = O.rate_distortion()


def _dp_min(scores, b_min, b_max, budget):
    """min sum_j s_j D(b_j) over b_j in [b_min, b_max] with sum_j b_j = budget, by dynamic
    programming over (blocks seen, bits spent)."""
    inf = math.inf
    best = {0: 0.0}
    for s in scores:
        nxt = {}
        for spent, val in best.items():
            for b in range(b_min, b_max + 1):
                t = spent + b
                v = val + float(s) * DIST[b]
                if v < nxt.get(t, inf):
                    nxt[t] = v
        best = nxt
    return best[budget]


@st.composite
def alloc_problem(draw, n_blocks=64):
    b_min = draw(st.integers(1, 4))
    b_max = draw(st.integers(b_min, 4))
    budget = draw(st.integers(n_blocks * b_min, n_blocks * b_max))
    kind = draw(st.sampled_from(["lognormal", "ties", "zeros", "spiky"]))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    if kind == "lognormal":
        s = np.exp(3 * rng.standard_normal(n_blocks))
    elif kind == "ties":
        s = rng.integers(1, 4, n_blocks).astype(np.float64)
    elif kind == "zeros":
        s = np.where(rng.random(n_blocks) < 0.5, 0.0, rng.random(n_blocks))
    else:
        s = np.full(n_blocks, 1e-3)
        s[rng.integers(0, n_blocks, 3)] = 1e3
    return s, b_min, b_max, budget


@SETTINGS
@given(alloc_problem(n_blocks=16))
def test_greedy_is_the_exact_optimum_for_any_budget(prob):
    """Block-GTQ abstract, 4th sentence: the largest-marginal-gain allocation solves the
    separable proxy exactly for arbitrary budgets (D is convex in the rate)."""
    s, b_min, b_max, budget = prob
    r = O.greedy_allocate(s, DIST, b_min, b_max, budget)
    assert int(r.sum()) == budget and r.min() >= b_min and r.max() <= b_max
    assert O.proxy(s, DIST, r) == pytest.approx(_dp_min(s, b_min, b_max, budget), rel=1e-12, abs=1e-300)


@SETTINGS
@given(alloc_problem())
def test_greedy_has_no_improving_exchange(prob):
    s, b_min, b_max, budget = prob
    r = O.greedy_allocate(s, DIST, b_min, b_max, budget)
    p = O.proxy(s, DIST, r)
    down = [j for j in range(64) if r[j] > b_min]
    up = [j for j in range(64) if r[j] < b_max]
    for i in down:
        for j in up:
            if i != j:
                gain_j = s[j] * (DIST[r[j]] - DIST[r[j] + 1])
                loss_i = s[i] * (DIST[r[i] - 1] - DIST[r[i]])
                assert loss_i >= gain_j - 1e-12 * max(p, 1e-300)


@SETTINGS
@given(seed=st.integers(0, 2**16), n_q=st.integers(1, 6), n_k=st.integers(1, 9),
       layout=st.sampled_from([HALF, INTERLEAVED]), prob=alloc_problem())
def test_library_allocation_equals_the_oracle(seed, n_q, n_k, layout, prob):
    _, b_min, b_max, budget = prob
    rng = np.random.default_rng(seed)
    spread = np.exp(2 * rng.standard_normal(128)).astype(np.float32)
    q = (rng.standard_normal((n_q, 128)) * spread).astype(np.float32)
    k = (rng.standard_normal((n_k, 128)) * spread[::-1]).astype(np.float32)
    r, s, p = G.gtq_alloc_rates(q, k, b_min, b_max, budget, rope_layout=layout)
    so = O.energy_scores(q, k, layout)
    ro = O.greedy_allocate(so, DIST, b_min, b_max, budget)
    assert np.allclose(s, so, rtol=1e-12, atol=0)
    # a near-tie of two gains can be decided differently by the last bit of a score; then
    # both allocations must reach the same proxy
    if not np.array_equal(r, ro):
        assert O.proxy(so, DIST, r) == pytest.approx(O.proxy(so, DIST, ro), rel=1e-12)
    assert int(r.sum()) == budget


rates_st = st.lists(st.integers(1, 4), min_size=64, max_size=64)


@SETTINGS
@given(rates=rates_st, layout=st.sampled_from([HALF, INTERLEAVED]))
def test_library_layout_equals_the_oracle_groups(rates, layout):
    rates = np.array(rates, np.uint8)
    lay = G.gtq_head_layout_from_rates(rates, layout)
    groups = O.groups_from_rates(rates, layout)
    assert lay["rate"] == [r for r, _ in groups]
    assert lay["dim"] == [len(c) for _, c in groups]
    assert lay["coord"] == [int(x) for _, c in groups for x in c]
    assert lay["k_words"] == (2 * int(rates.sum()) + 31) // 32
    assert sorted(lay["coord"]) == list(range(128))


@SETTINGS
@given(rates=rates_st, n=st.integers(1, 5), seed=st.integers(0, 2**16))
def test_packing_is_a_bijection(rates, n, seed):
    groups = O.groups_from_rates(np.array(rates), HALF)
    dims, rs = [len(c) for _, c in groups], [r for r, _ in groups]
    rng = np.random.default_rng(seed)
    codes = [rng.integers(0, 2**r, (n, d)) for d, r in zip(dims, rs)]
    words = O.pack_codes(codes, rs)
    assert words.shape == (n, (2 * sum(rates) + 31) // 32)
    back = O.unpack_codes(words, dims, rs)
    for a, b in zip(codes, back):
        assert np.array_equal(a, b)
    # one flipped code bit changes exactly one code by a power of two
    j = int(rng.integers(0, 2 * sum(rates)))
    w2 = words.copy()
    w2[0, j // 32] ^= np.uint32(1 << (j % 32))
    diff = sum(int((a != b).sum()) for a, b in zip(codes, O.unpack_codes(w2, dims, rs)))
    assert diff == 1


def _host_plan(H, g, budget, v_bits, seed):
    rng = np.random.default_rng(seed)
    rates = np.zeros((1, H, 64), np.uint8)
    krot, vrot = [[]], []
    for h in range(H):
        r = O.greedy_allocate(np.exp(2 * rng.standard_normal(64)), DIST, 1, 4, budget)
        rates[0, h] = r
        krot[0].append([np.eye(len(c), dtype=np.float32) for _, c in O.groups_from_rates(r, HALF)])
        vrot.append(np.eye(128, dtype=np.float32))
    return G.Plan(1, H, H * g, budget, v_bits, rates, krot, np.array([vrot]), host_only=True)


@SETTINGS
@given(H=st.integers(1, 8), g=st.sampled_from([1, 2, 3, 4, 5, 7, 8, 16]), batch=st.integers(1, 40),
       max_len=st.integers(1, 70000), chunk_blocks=st.integers(0, 64),
       budget=st.sampled_from([64, 128, 192, 256]), v_bits=st.integers(1, 4))
def test_decode_workspace_covers_every_split(H, g, batch, max_len, chunk_blocks, budget, v_bits):
    """The workspace the library asks for holds one partial (128 accumulators, m, l and
    padding) per query row and split; split sizes must be whole 32-token blocks and give
    at most 256 splits."""
    p = _host_plan(H, g, budget, v_bits, seed=H * 131 + g)
    chunk = 32 * chunk_blocks
    n_chunks = 1 if chunk == 0 else -(-max_len // chunk)
    if chunk and n_chunks > 256:
        with pytest.raises(G.GtqError):
            G.gtq_decode_workspace_bytes(p, batch, max_len, chunk)
    else:
        ws = G.gtq_decode_workspace_bytes(p, batch, max_len, chunk)
        rows = batch * H * g
        assert ws >= rows * n_chunks * 128 * 4
        if chunk:
            assert ws >= rows * n_chunks * 130 * 4
        for bad in (16, 33, -32):
            with pytest.raises(G.GtqError):
                G.gtq_decode_workspace_bytes(p, batch, max_len, bad)
    p.destroy()


@settings(max_examples=15, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**16), n=st.integers(1, 90), g=st.integers(1, 6),
       budget=st.sampled_from([64, 128, 192]), v_bits=st.integers(1, 4),
       cuts=st.lists(st.integers(1, 89), max_size=4))
def test_packed_decode_splits_over_heads_and_chunks(seed, n, g, budget, v_bits, cuts):
    """The oracle's decode is a softmax average: its weights sum to one, every output lies
    in the convex hull of the decoded values, query heads are independent, and any split of
    the tokens into chunks recombines exactly by the log-sum-exp merge."""
    inp = head_inputs(seed, 0, 0, g, n)
    r = O.greedy_allocate(O.energy_scores(inp["calib_q"], inp["calib_k"], HALF), DIST, 1, 4, budget)
    kr, vr = head_rotations(seed, 0, 0, [len(c) for _, c in O.groups_from_rates(r, HALF)])
    plan = O.HeadPlan(r, kr, vr, v_bits)
    rec = O.encode_kv(plan, inp["k"], inp["v"])
    q = inp["q"][0]
    scale = 1 / math.sqrt(128)
    lg, out = O.decode_attention(plan, q, rec["k_words"], rec["k_norms"], rec["v_words"], rec["v_norms"], scale)
    vals = O.dequantized_values(plan, rec["v_words"], rec["v_norms"])
    assert np.all(out <= vals.max(axis=0) + 1e-12) and np.all(out >= vals.min(axis=0) - 1e-12)
    for h in range(g):
        _, oh = O.decode_attention(plan, q[h:h + 1], rec["k_words"], rec["k_norms"], rec["v_words"],
                                   rec["v_norms"], scale)
        # (a different BLAS blocking moves logits of size ~100 by an ulp: compare at the scale of the outputs)
        assert np.abs(oh[0] - out[h]).max() <= 1e-11 * max(1.0, np.abs(out).max())
    bounds = sorted({0, n, *[c for c in cuts if c < n]})
    ms, ls, accs = [], [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        x = lg[:, a:b]
        m = x.max(axis=1)
        e = np.exp(x - m[:, None])
        ms.append(m)
        ls.append(e.sum(axis=1))
        accs.append(e @ vals[a:b])
    M = np.max(ms, axis=0)
    w = [np.exp(m - M) for m in ms]
    L = sum(wi * li for wi, li in zip(w, ls))
    merged = sum(wi[:, None] * ai for wi, ai in zip(w, accs)) / L[:, None]
    assert np.abs(merged - out).max() <= 1e-11 * max(1.0, np.abs(out).max())
