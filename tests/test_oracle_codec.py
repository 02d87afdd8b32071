"""Pins of the oracle's codec: Lloyd-Max codebooks, encode, dequantize, bit packing.

Each check is fixed by something other than the oracle itself: closed forms, a
published table, scipy quadrature of the optimality conditions, Monte Carlo,
hand-worked bit patterns, or invariants (rotation/permutation equivariance)."""
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from gtq_inputs import haar_rotation
from oracle import gtq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_max():
    rows = {}
    for line in open(os.path.join(GOLD, "lloyd_max_gaussian.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        rows[int(f[0])] = (float(f[1]), [float(x) for x in f[2:]])
    return rows


def test_one_bit_closed_form():
    c, mse = O.lloyd_max_gaussian(1)
    assert c[1] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-14)
    assert c[0] == pytest.approx(-math.sqrt(2 / math.pi), abs=1e-14)
    assert mse == pytest.approx(1 - 2 / math.pi, abs=1e-14)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_matches_published_table(bits):
    mse_t, cent_t = _golden_max()[bits]
    c, mse = O.lloyd_max_gaussian(bits)
    pos = c[len(c) // 2:]
    for a, b in zip(pos, cent_t):
        assert abs(a - b) <= 6e-4 * max(1.0, abs(b))
    assert abs(mse - mse_t) <= 1e-3 * mse_t


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_optimality_conditions_by_quadrature(bits):
    """Centroid condition (each centroid is its cell's conditional mean) and the
    distortion, recomputed with scipy quadrature on the Gaussian density."""
    c, mse = O.lloyd_max_gaussian(bits)
    edges = [-np.inf] + list((c[:-1] + c[1:]) / 2) + [np.inf]
    pdf = stats.norm.pdf
    tot = 0.0
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        m0 = stats.norm.cdf(b) - stats.norm.cdf(a)
        m1 = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert m1 / m0 == pytest.approx(c[k], rel=1e-9, abs=1e-10)
        tot += integrate.quad(lambda x: (x - c[k]) ** 2 * pdf(x), a, b, epsabs=1e-14, epsrel=1e-12)[0]
    assert tot == pytest.approx(mse, rel=1e-8)


def test_monte_carlo_distortion():
    rng = np.random.default_rng(123)
    x = rng.standard_normal(2_000_000)
    for b in range(1, 5):
        c16, t = O.codebook(b)
        q = c16[np.searchsorted(t, x, side="right")]
        assert np.mean((x - q) ** 2) == pytest.approx(O.rate_distortion()[b], rel=0.01)


def test_rate_penalties_diminishing_gains():
    d = O.rate_distortion()
    gains = d[:-1] - d[1:]
    assert np.all(gains[1:] < gains[:-1])          # strictly diminishing (b >= 1)
    assert np.all(gains > 0)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_stored_codebook(bits):
    c, _ = O.lloyd_max_gaussian(bits)
    c16, t = O.codebook(bits)
    # every entry is a binary16 value within half an ulp of the fp64 centroid
    assert np.all(c16.astype(np.float16).astype(np.float64) == c16)
    ulp = np.spacing(np.abs(c).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(c16 - c) <= 0.5 * ulp + 1e-18)
    assert np.all(c16 == -c16[::-1])                # symmetric
    assert t[len(t) // 2] == 0.0                    # middle threshold at zero
    assert np.all(t == (c16[:-1] + c16[1:]) / 2)


# ---------------------------------------------------------------- encode

def test_zero_vector():
    rot = haar_rotation(16, np.random.default_rng(0))
    nu, codes, _ = O.encode(np.zeros((1, 16), np.float32), rot, 3)
    assert nu[0] == 0.0
    assert np.all(codes == 4)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_identity_rotation_is_scalar_quantizer(bits):
    """Special case Pi = I: codes are the scalar cell indices of sqrt(d) x / ||x||,
    cross-checked with numpy.searchsorted (upper cell on a tie)."""
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((50, 32)).astype(np.float32)
    nu, codes, _ = O.encode(x, np.eye(32, dtype=np.float32), bits)
    x64 = x.astype(np.float64)
    z = math.sqrt(32) * x64 / np.linalg.norm(x64, axis=1, keepdims=True)
    _, t = O.codebook(bits)
    assert np.array_equal(codes, np.searchsorted(t, z, side="right"))
    assert np.allclose(nu, np.linalg.norm(x64, axis=1), rtol=1e-7)
    # a value exactly on a threshold goes up
    if len(t) > 1:
        xe = np.zeros((1, 2), np.float32)
        xe[0, 0] = 1.0            # z = (sqrt 2, 0): coordinate 1 sits on the middle threshold 0
        _, ce, _ = O.encode(xe, np.eye(2, dtype=np.float32), bits)
        assert ce[0, 1] == (1 << (bits - 1))


def test_permutation_equivariance():
    """With Pi a permutation P, codes(x; P) = P applied to codes(x; I). A transposed
    rotation in encode would permute the wrong way and fail."""
    rng = np.random.default_rng(7)
    d = 24
    perm = rng.permutation(d)
    P = np.eye(d, dtype=np.float32)[perm]         # (P u)_i = u_{perm[i]}
    x = rng.standard_normal((40, d)).astype(np.float32)
    _, c_id, _ = O.encode(x, np.eye(d, dtype=np.float32), 2)
    _, c_p, _ = O.encode(x, P, 2)
    assert np.array_equal(c_p, c_id[:, perm])
    assert not np.array_equal(c_p, c_id[:, np.argsort(perm)])


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_unit_vector_distortion_near_gaussian(bits):
    """At d = 128 the rotated, sqrt(d)-scaled coordinates of a random unit vector are
    nearly N(0,1): E||u - u_hat||^2 is within 3% of D(b)."""
    rng = np.random.default_rng(100 + bits)
    d = 128
    rot = haar_rotation(d, rng)
    x = rng.standard_normal((3000, d)).astype(np.float32) * 3.0
    nu, codes, _ = O.encode(x, rot, bits)
    xh = O.dequantize(nu, codes, rot, bits)
    x64 = x.astype(np.float64)
    err = np.sum((x64 - xh) ** 2, axis=1) / np.sum(x64 ** 2, axis=1)
    assert np.mean(err) == pytest.approx(O.rate_distortion()[bits], rel=0.03)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_norm_corrected_reconstruction_keeps_the_norm(bits):
    """Norm-corrected variant: the decoded vector has the input's norm (up to the fp32
    rounding of the stored norm), the codes are those of the plain variant, and the
    plain variant's reconstruction is shorter on average (a Lloyd-Max quantizer keeps
    E[C^2] = 1 - D(b) of the energy)."""
    rng = np.random.default_rng(200 + bits)
    d = 40
    rot = haar_rotation(d, rng)
    x = (rng.standard_normal((200, d)) * 2.5).astype(np.float32)
    nu_p, c_p, _ = O.encode(x, rot, bits)
    nu_c, c_c, _ = O.encode(x, rot, bits, nc=True)
    assert np.array_equal(c_p, c_c)
    x64 = x.astype(np.float64)
    true = np.linalg.norm(x64, axis=1)
    rec_c = np.linalg.norm(O.dequantize(nu_c, c_c, rot, bits), axis=1)
    rec_p = np.linalg.norm(O.dequantize(nu_p, c_p, rot, bits), axis=1)
    assert np.allclose(rec_c, true, rtol=2e-7, atol=0)
    assert np.mean(rec_p ** 2 / true ** 2) == pytest.approx(1 - O.rate_distortion()[bits], abs=0.04)


def test_norm_corrected_one_bit_closed_form():
    """At 1 bit every centroid has magnitude c1, so ||C[code]|| = sqrt(d) c1 and the
    stored norm is nu / c1 whatever the codes are."""
    rng = np.random.default_rng(9)
    d = 24
    rot = haar_rotation(d, rng)
    x = rng.standard_normal((64, d)).astype(np.float32)
    nu_c, _, _ = O.encode(x, rot, 1, nc=True)
    c1 = O.codebook(1)[0][1]
    ref = (np.linalg.norm(x.astype(np.float64), axis=1) / c1).astype(np.float32)
    d_ulp = np.abs(nu_c.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert d_ulp.max() <= 1
    assert O.encode(np.zeros((1, d), np.float32), rot, 1, nc=True)[0][0] == 0.0


def test_haar_rotations_orthogonal():
    rng = np.random.default_rng(5)
    for d in (2, 6, 40, 128):
        r = haar_rotation(d, rng).astype(np.float64)
        assert np.max(np.abs(r @ r.T - np.eye(d))) <= 2e-6
        assert abs(abs(np.linalg.det(r)) - 1) <= 1e-5
        x, y = rng.standard_normal(d), rng.standard_normal(d)
        assert (r @ x) @ (r @ y) == pytest.approx(x @ y, rel=1e-5, abs=1e-5)


# ---------------------------------------------------------------- packing

def _pack_cases():
    for line in open(os.path.join(GOLD, "pack_examples.txt")):
        if line.startswith("#") or not line.strip():
            continue
        r, d, c, w = [p.split() for p in line.split(";")]
        yield [int(x) for x in r], [int(x) for x in d], [int(x) for x in c], [int(x, 16) for x in w]


@pytest.mark.parametrize("case", list(_pack_cases()))
def test_pack_hand_examples(case):
    rates, dims, codes, words = case
    groups, p = [], 0
    for d in dims:
        groups.append(np.array([codes[p:p + d]]))
        p += d
    got = O.pack_codes(groups, rates)
    assert got.tolist() == [words]
    back = O.unpack_codes(got, dims, rates)
    assert [g.tolist() for g in back] == [g.tolist() for g in groups]


def test_pack_round_trip_and_record_size():
    rng = np.random.default_rng(11)
    for budget in (128, 192, 100):
        s = np.exp(rng.standard_normal(64))
        rates = O.greedy_allocate(s, O.rate_distortion(), 1, 4, budget)
        gs = O.groups_from_rates(rates)
        cg = [rng.integers(0, 1 << r, size=(9, len(c))) for r, c in gs]
        w = O.pack_codes(cg, [r for r, _ in gs])
        assert sum(len(c) * r for r, c in gs) == 2 * budget          # 128 * average bits
        assert w.shape == (9, (2 * budget + 31) // 32)
        back = O.unpack_codes(w, [len(c) for _, c in gs], [r for r, _ in gs])
        for a, b in zip(cg, back):
            assert np.array_equal(a, b)


def test_hadamard_rotation_is_sylvester_times_signs():
    """The randomized Hadamard generator: scipy's Sylvester Hadamard matrix with a +-1
    column scaling, entries exactly +-fp32(1/sqrt(128)), orthogonal."""
    from scipy.linalg import hadamard
    from gtq_inputs import hadamard_rotation
    r = hadamard_rotation(128, np.random.default_rng(3))
    c = np.float32(1 / np.sqrt(128))
    h = hadamard(128)
    s = np.sign(r[0])
    assert np.array_equal(r, (h * s[None, :]).astype(np.float32) * c)
    assert set(np.unique(np.abs(r)).tolist()) == {float(c)}
    r64 = r.astype(np.float64)
    assert np.max(np.abs(r64 @ r64.T - np.eye(128))) < 1e-6
