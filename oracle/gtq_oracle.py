"""CPU oracle for the Block-GTQ packed-cache path (numpy, fp64).

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library never
calls it and shares no code with it.

Sources (cited as [short tag] in each function):
  [BGTQ sN]  "Block-GTQ: RoPE-Block Rate Allocation for KV-Cache Quantization"
             (ai-club.cn frontier article), abstract, N-th sentence:
             s2 RoPE 2-D frequency blocks carry the key precision; s3 blockwise
             logit-error bound -> label-free query-key energy score combined with
             codec-dependent rate penalties; s4 largest-marginal-gain allocation
             is exact for the separable integer proxy under equal costs and
             diminishing gains; s5 TQ-MSE instantiation, equal-rate blocks grouped,
             attention over packed caches with no decoded fp16 cache; s7 "K2V2"
             means 2 average logical bits per K/V coordinate.
  [TQ-diag X] "TurboQuant: paper algorithm and vLLM engineering" pipeline
             diagram (hsthanb4.github.io kvcache_quant_tutorial_2026,
             01_turboquant_pipeline), left ("paper") column, box X:
             input (vector x of a head's K or V), rotate (random rotation /
             Hadamard), scalar-MSE (per-coordinate MSE scalar quantization with a
             few centroids), residual (r = x - x_hat: the MSE-optimal code is not
             inner-product unbiased), QJL (a 1-bit sign sketch of the residual that
             corrects the attention inner products; TQ-MSE is the variant without
             it, TurboQuant-prod the one with it).

Readings where the pages are silent (each also listed in the design notes):
  R1  RoPE pairing: half-split, block j = coordinates (j, j+64); interleaved
      (2j, 2j+1) as an option.
  R2  energy score s_j = mean over calibration queries (all g heads of the KV
      group) of ||q_j||^2  times  mean over calibration keys of ||k_j||^2.
  R4  rate penalty D(b) = MSE of the b-bit Lloyd-Max quantizer of N(0,1).
  R5  per-rate codebook: the N(0,1) Lloyd-Max centroids, stored rounded to
      binary16; a group of dimension d is quantized as sqrt(d) * Pi * x/||x||.
  R6  one norm per group sub-vector (each group is its own TQ-MSE instance).
  R11 a value on a threshold goes to the upper cell; a zero vector has norm 0
      and every code 2^(b-1).
  R12 greedy ties go to the smallest block index.
  R13 the budget counts code bits only: sum_j b_j = (average key bits) * 64.
  R22 fp16 sink and recent-token buffers ([BGTQ s8] names the variant as one its K3V2
      result does without): the first n_sink positions and the last n_recent
      positions of a sequence attend through fp16 copies of their K and V (binary16,
      round to nearest even), every other position through the packed cache.
  R24 QJL residual sketch (TurboQuant-prod): keys only (it corrects q . k); the
      residual is r = k - k_hat in head coordinates, k_hat the TQ-MSE reconstruction of
      the stored record (fp64); S is an m x 128 matrix of N(0,1) entries (m = 128, one
      bit per coordinate), drawn per (layer, KV head) and passed in like the rotations;
      the sketch stores sign(S r) (a zero projection counts as +) and gamma = ||r||
      (fp64, stored fp32); the estimate is q . k_hat + gamma sqrt(pi/2) / m *
      sum_j (S q)_j sign_j, unbiased over S. The sketch bits and gamma's fp32 bits
      follow the MSE words of the key record (4 + 1 words). A prod key at b bits is the
      MSE key at b - 1 bits plus the sketch.
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128
N_BLOCKS = 64
HALF, INTERLEAVED = 0, 1


# --------------------------------------------------------------------------
# Lloyd-Max quantizer of N(0,1)  [TQ-diag scalar-MSE], [BGTQ s3] (rate penalty)
# --------------------------------------------------------------------------

def _phi(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _mass(a: float, b: float) -> float:
    """P(a < X < b) for X ~ N(0,1), accurate in both tails."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / math.sqrt(2.0)) - math.erfc(b / math.sqrt(2.0)))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / math.sqrt(2.0)) - math.erfc(-a / math.sqrt(2.0)))
    return 1.0 - 0.5 * math.erfc(-a / math.sqrt(2.0)) - 0.5 * math.erfc(b / math.sqrt(2.0))


def lloyd_max_gaussian(bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Lloyd iteration for the MSE-optimal 2^bits-level quantizer of N(0,1).

    Alternates the two optimality conditions: cell edges at centroid midpoints,
    centroids at the conditional means E[X | cell] = (phi(a)-phi(b))/P(a<X<b).
    Returns (centroids ascending, fp64; mse = E[(X - Q(X))^2])."""
    n = 1 << bits
    c = np.array([(-1.0 + (2.0 * k + 1.0) / n) * 2.0 for k in range(n)])
    for _ in range(max_iter):
        edges = [-math.inf] + [(c[k] + c[k + 1]) / 2.0 for k in range(n - 1)] + [math.inf]
        new = np.array([(_phi(edges[k]) - _phi(edges[k + 1])) / _mass(edges[k], edges[k + 1])
                        for k in range(n)])
        delta = float(np.max(np.abs(new - c)))
        c = new
        if delta < tol:
            break
    edges = [-math.inf] + [(c[k] + c[k + 1]) / 2.0 for k in range(n - 1)] + [math.inf]
    # E[X^2] = 1; for centroids at conditional means, E[(X-c_k)^2 ; cell k]
    # = E[X^2 ; cell] - P_k c_k^2, so mse = 1 - sum_k P_k c_k^2.
    mse = 1.0 - sum(_mass(edges[k], edges[k + 1]) * c[k] * c[k] for k in range(n))
    return c, mse


def rate_distortion(b_max: int = 4) -> np.ndarray:
    """D[b] for b = 0..b_max: D[0] = 1 (no bits: reconstruct 0), D[b] = Lloyd-Max MSE.
    [BGTQ s3] 'codec-dependent rate penalties' read as the codec's distortion-rate table (R4)."""
    d = np.ones(b_max + 1)
    for b in range(1, b_max + 1):
        d[b] = lloyd_max_gaussian(b)[1]
    return d


def codebook(bits: int):
    """Stored codebook of rate `bits` (R5): Lloyd-Max centroids rounded to binary16,
    returned as fp64 values, plus the 2^bits - 1 decision thresholds (midpoints)."""
    c, _ = lloyd_max_gaussian(bits)
    c16 = np.array([float(np.float16(v)) for v in c])
    t = (c16[:-1] + c16[1:]) / 2.0
    return c16, t


# --------------------------------------------------------------------------
# RoPE blocks and the energy score  [BGTQ s2], [BGTQ s3]
# --------------------------------------------------------------------------

def block_coords(j: int, layout: int = HALF, d: int = HEAD_DIM) -> tuple[int, int]:
    """The two coordinates of RoPE frequency block j (R1)."""
    if layout == HALF:
        return j, j + d // 2
    return 2 * j, 2 * j + 1


def energy_scores(q_cal: np.ndarray, k_cal: np.ndarray, layout: int = HALF) -> np.ndarray:
    """s_j = mean_rows ||q_{.,j}||^2 * mean_rows ||k_{.,j}||^2 (R2), fp64.

    The blockwise logit-error bound |q.k - q.k_hat| <= sum_j ||q_j|| ||k_j - k_hat_j||
    with ||k_j - k_hat_j||^2 ~ ||k_j||^2 D(b_j) makes the expected error separate
    into sum_j s_j D(b_j) [BGTQ s3, s4]."""
    q = np.asarray(q_cal, dtype=np.float64)
    k = np.asarray(k_cal, dtype=np.float64)
    s = np.empty(N_BLOCKS)
    for j in range(N_BLOCKS):
        a, b = block_coords(j, layout)
        eq = math.fsum((q[:, a] ** 2 + q[:, b] ** 2).tolist()) / q.shape[0]
        ek = math.fsum((k[:, a] ** 2 + k[:, b] ** 2).tolist()) / k.shape[0]
        s[j] = eq * ek
    return s


# --------------------------------------------------------------------------
# Largest-marginal-gain allocation  [BGTQ s4]
# --------------------------------------------------------------------------

def greedy_allocate(scores, dist, b_min: int, b_max: int, budget: int) -> np.ndarray:
    """Start every block at b_min; while the bit total is below the budget, give one
    more bit to the block with the largest gain s_j * (D(b_j) - D(b_j + 1)) among
    blocks below b_max (ties: smallest j, R12)."""
    s = list(map(float, scores))
    n = len(s)
    if not (1 <= b_min <= b_max):
        raise ValueError("need 1 <= b_min <= b_max")
    if not (n * b_min <= budget <= n * b_max):
        raise ValueError("budget outside [n*b_min, n*b_max]")
    b = [b_min] * n
    total = n * b_min
    while total < budget:
        best, best_gain = -1, -math.inf
        for j in range(n):
            if b[j] < b_max:
                gain = s[j] * (dist[b[j]] - dist[b[j] + 1])
                if gain > best_gain:
                    best, best_gain = j, gain
        b[best] += 1
        total += 1
    return np.array(b, dtype=np.int64)


def proxy(scores, dist, rates) -> float:
    """The separable integer proxy sum_j s_j D(b_j) [BGTQ s4]."""
    return float(sum(float(s) * dist[int(b)] for s, b in zip(scores, rates)))


# --------------------------------------------------------------------------
# Equal-rate groups  [BGTQ s5]
# --------------------------------------------------------------------------

def groups_from_rates(rates, layout: int = HALF) -> list[tuple[int, np.ndarray]]:
    """[(rate, coordinate indices)] in ascending rate; blocks ascending inside a group,
    each block contributing its two coordinates in order."""
    out = []
    for r in sorted(set(int(x) for x in rates)):
        coords = []
        for j, bj in enumerate(rates):
            if int(bj) == r:
                coords.extend(block_coords(j, layout))
        out.append((r, np.array(coords, dtype=np.int64)))
    return out


# --------------------------------------------------------------------------
# TQ-MSE encode / dequantize  [TQ-diag input -> rotate -> scalar-MSE], [BGTQ s5]
# --------------------------------------------------------------------------

def encode(x: np.ndarray, rot: np.ndarray, bits: int, nc: bool = False):
    """Encode rows of x [n, d] (fp32 input) with rotation rot [d, d] (fp32 entries).

    nu = sqrt(sum x_i^2) in fp64, stored fp32; u = x / nu; z = sqrt(d) * rot @ u;
    code_i = #{k : z_i >= t_k}. Returns (stored norm fp32 [n], codes int64 [n, d],
    z fp64 [n, d]).

    nc (the norm-corrected variant named in the TurboQuant page's vLLM preset column):
    the stored norm is nu * sqrt(d) / ||C[code]|| instead of nu, so that the decoded
    vector nu_stored * rot^T C[code] / sqrt(d) has norm nu exactly (rot is orthogonal).
    It is evaluated in fp64 as (nu * sqrt(d)) / sqrt(sum_i C[code_i]^2) and rounded to
    fp32; the sum is exact in any order (binary16 centroids, at most 128 terms)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    n, d = x64.shape
    nu = np.sqrt(np.sum(x64 * x64, axis=1))
    safe = np.where(nu > 0.0, nu, 1.0)
    u = np.where(nu[:, None] > 0.0, x64 / safe[:, None], 0.0)
    y = u @ np.asarray(rot, dtype=np.float32).astype(np.float64).T
    z = math.sqrt(d) * y
    _, t = codebook(bits)
    codes = np.zeros((n, d), dtype=np.int64)
    for tk in t:
        codes += (z >= tk)
    if nc:
        c16, _ = codebook(bits)
        ssq = np.sum(c16[codes] ** 2, axis=1)
        stored = np.where(nu > 0.0, nu * math.sqrt(d) / np.sqrt(ssq), 0.0)
        return stored.astype(np.float32), codes, z
    return nu.astype(np.float32), codes, z


def dequantize(nu32: np.ndarray, codes: np.ndarray, rot: np.ndarray, bits: int) -> np.ndarray:
    """x_hat = nu * rot^T @ C[code] / sqrt(d), fp64 [n, d] (the decoded vector that the
    packed path never materialises; used here only to check the packed-path logits)."""
    c16, _ = codebook(bits)
    d = codes.shape[1]
    vals = c16[codes] / math.sqrt(d)
    return np.asarray(nu32, dtype=np.float64)[:, None] * (vals @ np.asarray(rot, np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# Bit packing (the canonical little-endian record)
# --------------------------------------------------------------------------

def pack_codes(code_groups: list[np.ndarray], rates: list[int]) -> np.ndarray:
    """Concatenate the groups' codes (ascending-rate order) into one little-endian bit
    stream: code i of group g takes bits [off_g + i*b_g, off_g + (i+1)*b_g), with bit p
    stored as bit (p mod 32) of word p // 32. code_groups: list of [n, d_g] arrays.
    Returns uint32 words [n, ceil(total_bits / 32)]."""
    n = code_groups[0].shape[0]
    total = sum(cg.shape[1] * b for cg, b in zip(code_groups, rates))
    nwords = (total + 31) // 32
    bits = np.zeros((n, nwords * 32), dtype=np.uint64)
    pos = 0
    for cg, b in zip(code_groups, rates):
        for i in range(cg.shape[1]):
            for k in range(b):
                bits[:, pos + k] = (cg[:, i].astype(np.uint64) >> np.uint64(k)) & np.uint64(1)
            pos += b
    words = np.zeros((n, nwords), dtype=np.uint64)
    for w in range(nwords):
        for k in range(32):
            words[:, w] |= bits[:, 32 * w + k] << np.uint64(k)
    return words.astype(np.uint32)


def unpack_codes(words: np.ndarray, dims: list[int], rates: list[int]) -> list[np.ndarray]:
    """Inverse of pack_codes."""
    w = np.asarray(words, dtype=np.uint64)
    if w.ndim == 1:
        w = w[None, :]
    out = []
    pos = 0
    for d, b in zip(dims, rates):
        cg = np.zeros((w.shape[0], d), dtype=np.int64)
        for i in range(d):
            for k in range(b):
                p = pos + k
                bit = (w[:, p // 32] >> np.uint64(p % 32)) & np.uint64(1)
                cg[:, i] |= (bit.astype(np.int64) << k)
            pos += b
        out.append(cg)
    return out


# --------------------------------------------------------------------------
# 1-bit QJL residual sketch (TurboQuant-prod)  [TQ-diag residual, QJL], R24
# --------------------------------------------------------------------------

QJL_M = 128  # sketch rows: one sign bit per key coordinate


def qjl_encode(r: np.ndarray, S: np.ndarray):
    """Residual rows r [n, d] (fp64) and S [m, d] (fp32 entries): (gamma = ||r|| fp64
    stored fp32 [n], sign bits [n, m] (1 where (S r)_j >= 0), the projections S r fp64)."""
    r64 = np.asarray(r, np.float64)
    if r64.ndim == 1:
        r64 = r64[None, :]
    gamma = np.sqrt(np.sum(r64 * r64, axis=1))
    proj = r64 @ np.asarray(S, np.float32).astype(np.float64).T
    bits = (proj >= 0.0).astype(np.int64)
    return gamma.astype(np.float32), bits, proj


def qjl_inner(y: np.ndarray, bits, gamma, S: np.ndarray) -> np.ndarray:
    """The sketch's estimate of y . r for rows y [k, d] and sketches (bits [n, m],
    gamma [n]): gamma sqrt(pi/2) / m * sum_j (S y)_j (2 bit_j - 1), fp64 [k, n]."""
    y64 = np.atleast_2d(np.asarray(y, np.float32)).astype(np.float64)
    S64 = np.asarray(S, np.float32).astype(np.float64)
    m = S64.shape[0]
    sy = y64 @ S64.T                                   # [k, m]
    sigma = 2.0 * np.asarray(bits, np.float64) - 1.0   # [n, m]
    g = np.asarray(gamma, np.float32).astype(np.float64)
    return (sy @ sigma.T) * (g * math.sqrt(math.pi / 2.0) / m)[None, :]


def qjl_fields(plan, k_words):
    """The sketch bits [n, m] and gamma (fp32) [n] stored after the MSE words of key
    records [n, words]."""
    w = np.atleast_2d(np.asarray(k_words, np.uint32))
    mw = plan.mse_words
    (bits,) = unpack_codes(w[:, mw:mw + QJL_M // 32], [QJL_M], [1])
    gamma = np.ascontiguousarray(w[:, mw + QJL_M // 32]).view(np.float32)
    return bits, gamma


# --------------------------------------------------------------------------
# A head's plan and its packed cache
# --------------------------------------------------------------------------

class HeadPlan:
    """Rates, groups, rotations and V rate of one (layer, KV head); qjl: the residual
    sketch matrix S [128, 128] (R24) or None."""

    def __init__(self, rates, k_rots: list[np.ndarray], v_rot: np.ndarray, v_bits: int,
                 layout: int = HALF, nc: bool = False, qjl=None):
        self.rates = np.asarray(rates, dtype=np.int64)
        self.layout = layout
        self.nc = bool(nc)  # norm-corrected stored norms (see encode)
        self.groups = groups_from_rates(self.rates, layout)
        if len(k_rots) != len(self.groups):
            raise ValueError("one K rotation per group")
        for (r, coords), rot in zip(self.groups, k_rots):
            if rot.shape != (len(coords), len(coords)):
                raise ValueError("K rotation shape does not match its group")
        self.k_rots = [np.asarray(r, np.float32) for r in k_rots]
        self.v_rot = np.asarray(v_rot, np.float32)
        self.v_bits = int(v_bits)
        self.qjl = None if qjl is None else np.asarray(qjl, np.float32)
        if self.qjl is not None and self.qjl.shape != (QJL_M, HEAD_DIM):
            raise ValueError("the QJL matrix is 128 x 128")

    @property
    def mse_words(self):
        """Words of the MSE part of a key record."""
        return (sum(len(c) * r for r, c in self.groups) + 31) // 32

    @property
    def group_rates(self):
        return [r for r, _ in self.groups]

    @property
    def group_dims(self):
        return [len(c) for _, c in self.groups]


def encode_kv(plan: HeadPlan, k: np.ndarray, v: np.ndarray) -> dict:
    """Encode tokens k, v [n, 128] of one KV head into the packed record
    (K words, K norms per group, V words, V norm) [BGTQ s5], [TQ-diag]. With a QJL plan
    the key record goes on with the residual's sketch words and gamma's bits (R24)
    [TQ-diag residual, QJL]."""
    kn, kc, kz = [], [], []
    for (r, coords), rot in zip(plan.groups, plan.k_rots):
        nu, codes, z = encode(np.asarray(k)[:, coords], rot, r, nc=plan.nc)
        kn.append(nu)
        kc.append(codes)
        kz.append(z)
    vn, vc, vz = encode(v, plan.v_rot, plan.v_bits, nc=plan.nc)
    k_words = pack_codes(kc, plan.group_rates)
    k_norms = np.stack(kn, axis=1)
    out = dict(k_norms=k_norms, v_words=pack_codes([vc], [plan.v_bits]), v_norms=vn,
               k_codes=kc, k_z=kz, v_codes=vc, v_z=vz)
    if plan.qjl is not None:
        k64 = np.asarray(k, np.float32).astype(np.float64)
        r = k64 - dequantized_keys(plan, k_words, k_norms)
        gamma, bits, proj = qjl_encode(r, plan.qjl)
        k_words = np.concatenate([k_words, pack_codes([bits], [1]), gamma.view(np.uint32)[:, None]], axis=1)
        out.update(qjl_bits=bits, qjl_gamma=gamma, qjl_proj=proj)
    out["k_words"] = k_words
    return out


def rotate_query(plan: HeadPlan, q: np.ndarray) -> list[np.ndarray]:
    """r_g = Pi_g @ q[G_g] for each group (fp64), q [..., 128]."""
    q64 = np.asarray(q, np.float32).astype(np.float64)
    return [q64[..., coords] @ rot.astype(np.float64).T for (_, coords), rot in zip(plan.groups, plan.k_rots)]


def packed_logits(plan: HeadPlan, q: np.ndarray, k_words, k_norms, scale: float) -> np.ndarray:
    """Logits straight from the packed record: for each group,
    nu_g / sqrt(d_g) * sum_i r_{g,i} * C_b[code_i], summed over groups, plus (QJL plans)
    the sketch's estimate of q . r, times scale. q [m, 128] -> [m, n]."""
    q = np.atleast_2d(q)
    codes = unpack_codes(k_words, plan.group_dims, plan.group_rates)
    r = rotate_query(plan, q)
    kn = np.asarray(k_norms, np.float32).astype(np.float64)
    out = np.zeros((q.shape[0], codes[0].shape[0]))
    for g, ((b, coords), cg) in enumerate(zip(plan.groups, codes)):
        c16, _ = codebook(b)
        vals = c16[cg]                                   # [n, d_g]
        out += (r[g] @ vals.T) * (kn[:, g] / math.sqrt(len(coords)))[None, :]
    if plan.qjl is not None:
        bits, gamma = qjl_fields(plan, k_words)
        out += qjl_inner(q, bits, gamma, plan.qjl)
    return scale * out


def dequantized_keys(plan: HeadPlan, k_words, k_norms) -> np.ndarray:
    codes = unpack_codes(k_words, plan.group_dims, plan.group_rates)
    n = codes[0].shape[0]
    khat = np.zeros((n, HEAD_DIM))
    for g, ((b, coords), cg, rot) in enumerate(zip(plan.groups, codes, plan.k_rots)):
        khat[:, coords] = dequantize(np.asarray(k_norms)[:, g], cg, rot, b)
    return khat


def dequantized_values(plan: HeadPlan, v_words, v_norms) -> np.ndarray:
    (vc,) = unpack_codes(v_words, [HEAD_DIM], [plan.v_bits])
    return dequantize(v_norms, vc, plan.v_rot, plan.v_bits)


def decode_attention(plan: HeadPlan, q: np.ndarray, k_words, k_norms, v_words, v_norms,
                     scale: float, length: int | None = None):
    """Attention of queries q [m, 128] over the first `length` packed tokens, without a
    decoded key cache: logits from packed_logits, softmax in fp64, values accumulated in
    the rotated V basis (sum_n p_n nu_n C[code_n] / sqrt(128)) and rotated back once
    (o = Pi_V^T o_rot) [BGTQ s5]. Returns (logits [m, n], out [m, 128])."""
    n = np.asarray(k_words).shape[0] if length is None else int(length)
    kw, kn = np.asarray(k_words)[:n], np.asarray(k_norms)[:n]
    vw, vn = np.asarray(v_words)[:n], np.asarray(v_norms)[:n]
    logits = packed_logits(plan, q, kw, kn, scale)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=1, keepdims=True)
    (vc,) = unpack_codes(vw, [HEAD_DIM], [plan.v_bits])
    c16, _ = codebook(plan.v_bits)
    vrot = c16[vc] * (np.asarray(vn, np.float32).astype(np.float64)[:, None] / math.sqrt(HEAD_DIM))
    o_rot = p @ vrot
    out = o_rot @ plan.v_rot.astype(np.float64)          # (Pi^T o_rot^T)^T
    return logits, out


def window_positions(length: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Boolean mask [length]: True where position p reads the fp16 buffers (R22): the
    sink p < n_sink, or the recent window p >= length - n_recent."""
    p = np.arange(int(length))
    return (p < n_sink) | (p >= int(length) - n_recent)


def decode_attention_window(plan: HeadPlan, q: np.ndarray, k_words, k_norms, v_words, v_norms,
                            k_full, v_full, n_sink: int, n_recent: int, scale: float, length: int):
    """Decode attention with fp16 sink and recent-token buffers (R22) [BGTQ s8]: the
    logit of a window position is scale * q . fp16(k) and its value fp16(v); every
    other position uses the packed cache (packed_logits, and the value decoded as
    nu Pi_V^T C[code] / sqrt(128)). Softmax over all `length` positions in fp64.
    k_full, v_full [>= length, 128] are the fp32 inputs the buffers were filled from.
    Returns (logits [m, length], out [m, 128])."""
    n = int(length)
    win = window_positions(n, n_sink, n_recent)
    q64 = np.asarray(q, np.float32).astype(np.float64)
    k16 = np.asarray(k_full, np.float32)[:n].astype(np.float16).astype(np.float64)
    v16 = np.asarray(v_full, np.float32)[:n].astype(np.float16).astype(np.float64)
    logits = np.empty((q64.shape[0], n))
    if (~win).any():
        logits[:, ~win] = packed_logits(plan, q, np.asarray(k_words)[:n][~win], np.asarray(k_norms)[:n][~win], scale)
    if win.any():
        logits[:, win] = scale * (q64 @ k16[win].T)
    values = np.empty((n, HEAD_DIM))
    if (~win).any():
        values[~win] = dequantized_values(plan, np.asarray(v_words)[:n][~win], np.asarray(v_norms)[:n][~win])
    values[win] = v16[win]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=1, keepdims=True)
    return logits, p @ values


def prefill_attention(plan: HeadPlan, q: np.ndarray, pos0: int, k_words, k_norms, v_words,
                      v_norms, scale: float) -> np.ndarray:
    """Causal attention of a chunk of queries q [T, m, 128] at positions pos0..pos0+T-1
    over the packed cache (whose slots 0..pos0+T-1 already hold the chunk's own
    tokens): query at position p sees cached positions 0..p. Returns [T, m, 128]."""
    T = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for t in range(T):
        _, o = decode_attention(plan, q[t], k_words, k_norms, v_words, v_norms, scale,
                                length=pos0 + t + 1)
        out[t] = o
    return out
