"""Helpers for the GPU parity tests: building matching plans for the oracle and the
library from the seeded generator, and converting between the canonical per-token
code stream and the library's physical cache layout (bit marshalling only)."""
from __future__ import annotations

import math

import numpy as np

from gtq_inputs import head_inputs, head_rotations, qjl_matrix
from oracle import gtq_oracle as O

TOL_REL, TOL_ABS = 2e-3, 1e-4     # |gpu - ref| <= TOL_ABS + TOL_REL * |ref|
TIE_WINDOW = 1e-6

# running totals of what the parity checks compared (printed at the end of the session)
STATS = {"attn_values": 0, "attn_checks": 0, "codes": 0, "code_ties": 0, "norms": 0, "norm_mismatches": 0}


def assert_close(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    lim = TOL_ABS + TOL_REL * np.abs(ref)
    bad = ~(err <= lim)
    STATS["attn_checks"] += 1
    STATS["attn_values"] += int(err.size)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}")
    return float((err / (TOL_ABS + TOL_REL * np.abs(ref))).max()) if err.size else 0.0


class Case:
    """Plans (oracle + library) and per-sequence inputs for n_layers x h_kv heads."""

    def __init__(self, seed, n_layers, h_kv, g, n_cache, k_budget, v_bits, batch=1, layout=O.HALF,
                 n_dec_q=1, b_min=1, b_max=4, nc=False, v_hadamard=False, qjl=False):
        import packed_cache_attention_tq_amd as G
        self.seed, self.L, self.H, self.g = seed, n_layers, h_kv, g
        self.HQ = h_kv * g
        self.n, self.k_budget, self.v_bits, self.batch, self.layout = n_cache, k_budget, v_bits, batch, layout
        self.nc = nc
        self.qjl = np.stack([np.stack([qjl_matrix(seed, l, h) for h in range(h_kv)]) for l in range(n_layers)]) \
            if qjl else None
        self.rates = np.zeros((n_layers, h_kv, 64), np.uint8)
        self.heads = {}
        k_rot_all, v_rot_all = [], []
        self.inputs = {}
        for l in range(n_layers):
            kl, vl = [], []
            for h in range(h_kv):
                inp = [head_inputs(seed, l, h, g, n_cache, n_dec_q=n_dec_q, layout=layout, seq=b)
                       for b in range(batch)]
                self.inputs[l, h] = inp
                # the oracle allocates for itself; the library's allocation must agree
                s = O.energy_scores(inp[0]["calib_q"], inp[0]["calib_k"], layout)
                r = O.greedy_allocate(s, O.rate_distortion(), b_min, b_max, k_budget)
                r_lib, _, _ = G.gtq_alloc_rates(inp[0]["calib_q"], inp[0]["calib_k"], b_min, b_max,
                                                k_budget, rope_layout=layout)
                assert np.array_equal(r_lib, r), f"rate allocation differs at layer {l} head {h}"
                self.rates[l, h] = r_lib
                dims = [len(c) for _, c in O.groups_from_rates(r, layout)]
                kr, vr = head_rotations(seed, l, h, dims, v_hadamard=v_hadamard)
                self.heads[l, h] = O.HeadPlan(r, kr, vr, v_bits, layout, nc=nc,
                                              qjl=None if self.qjl is None else self.qjl[l, h])
                kl.append(kr)
                vl.append(vr)
            k_rot_all.append(kl)
            v_rot_all.append(vl)
        self.k_rot, self.v_rot = k_rot_all, np.array(v_rot_all)

    def plan(self, host_only=False):
        import packed_cache_attention_tq_amd as G
        return G.Plan(self.L, self.H, self.HQ, self.k_budget, self.v_bits, self.rates, self.k_rot,
                      self.v_rot, rope_layout=self.layout, host_only=host_only, norm_correct=self.nc,
                      qjl=self.qjl)

    def kv(self, l, b, lo=0, hi=None):
        """k, v [n_tok, H_kv, 128] of sequence b, tokens lo..hi-1."""
        hi = self.n if hi is None else hi
        k = np.stack([self.inputs[l, h][b]["k"][lo:hi] for h in range(self.H)], axis=1)
        v = np.stack([self.inputs[l, h][b]["v"][lo:hi] for h in range(self.H)], axis=1)
        return np.ascontiguousarray(k), np.ascontiguousarray(v)

    def q(self, l, b, qi=0):
        """decode query [H_q, 128] of sequence b (query heads of KV head h are h*g .. h*g+g-1)."""
        return np.concatenate([self.inputs[l, h][b]["q"][qi] for h in range(self.H)], axis=0)


# ---------------------------------------------------------------- layout marshalling

def v_codes_from_physical(words: np.ndarray, n_tok: int, vb: int) -> np.ndarray:
    """Physical value blocks [n_blocks][32*vb] u32 -> codes [n_tok][128]."""
    w = np.asarray(words, np.uint32).astype(np.uint64)
    s = np.arange(n_tok)[:, None]
    c = np.arange(128)[None, :]
    blk, j = s // 8, s % 8
    bit = 8 * vb * c + vb * j
    wi, sh = bit // 32, (bit % 32).astype(np.uint64)
    lo = w[blk, wi]
    hi = np.where(wi + 1 < w.shape[1], w[blk, np.minimum(wi + 1, w.shape[1] - 1)], np.uint64(0))
    val = lo | (hi << np.uint64(32))
    return ((val >> sh) & np.uint64((1 << vb) - 1)).astype(np.int64)


def v_codes_to_physical(codes: np.ndarray, vb: int, n_blocks: int) -> np.ndarray:
    """codes [n_tok][128] -> physical blocks [n_blocks][32*vb] u32 (unwritten bits 0)."""
    words = np.zeros((n_blocks, 32 * vb + 1), np.uint64)
    n = codes.shape[0]
    s = np.arange(n)[:, None]
    c = np.arange(128)[None, :]
    blk, j = np.broadcast_arrays(s // 8, s % 8)
    bit = 8 * vb * c + vb * j
    wi, sh = bit // 32, (bit % 32).astype(np.uint64)
    v = np.asarray(codes, np.uint64) << sh
    np.bitwise_or.at(words, (blk, wi), v & np.uint64(0xFFFFFFFF))
    np.bitwise_or.at(words, (blk, wi + 1), v >> np.uint64(32))
    return words[:, :32 * vb].astype(np.uint32)


def unpack_key_record(words, plan: O.HeadPlan):
    return O.unpack_codes(np.asarray(words, np.uint32), plan.group_dims, plan.group_rates)


def tie_mask(z: np.ndarray, bits: int) -> np.ndarray:
    """True where z lies within TIE_WINDOW of one of the codebook thresholds."""
    _, t = O.codebook(bits)
    return (np.abs(z[..., None] - t[None, :]) < TIE_WINDOW).any(axis=-1)


def compare_codes(gpu_codes, ref_codes, ref_z, bits, what):
    """Codes must be equal except where the oracle's z is within the tie window of a
    threshold; returns the number of such tie mismatches."""
    gpu_codes = np.asarray(gpu_codes)
    mism = gpu_codes != ref_codes
    ties = tie_mask(ref_z, bits)
    hard = mism & ~ties
    STATS["codes"] += int(mism.size)
    STATS["code_ties"] += int((mism & ties).sum())
    if hard.any():
        i = tuple(np.argwhere(hard)[0])
        raise AssertionError(f"{what}: {hard.sum()} code mismatches outside the tie window; first at {i}: "
                             f"gpu={gpu_codes[i]} ref={ref_codes[i]} z={ref_z[i]!r}")
    return int((mism & ties).sum())


def compare_qjl(gpu_words, gpu_norms, k, enc, plan, what, rel_window=1e-9):
    """The residual sketch of GPU records [n, words] against the oracle's encoding: sign
    bits equal except where the oracle's projection lies within rel_window * |S| |r| of
    zero (both sides compute S r in fp64, in different orders), gamma bit for bit. A token
    whose MSE codes took the other side of a tie has another residual: for such tokens
    the oracle sketches k minus the key decoded from the GPU's own MSE record (k [n, 128]
    the fp32 keys, gpu_norms [n, groups]). Returns the number of near-zero sign
    differences."""
    gpu_words = np.asarray(gpu_words, np.uint32)
    mw = plan.mse_words
    bits_ref = enc["qjl_bits"].copy()
    gamma_ref = enc["qjl_gamma"].copy()
    proj_ref = enc["qjl_proj"].copy()
    moved = np.flatnonzero((gpu_words[:, :mw] != enc["k_words"][:, :mw]).any(axis=1))
    if moved.size:
        k64 = np.asarray(k, np.float32)[moved].astype(np.float64)
        r = k64 - O.dequantized_keys(plan, gpu_words[moved, :mw], np.asarray(gpu_norms)[moved])
        gamma_ref[moved], bits_ref[moved], proj_ref[moved] = O.qjl_encode(r, plan.qjl)
    bits, gamma = O.qjl_fields(plan, gpu_words)
    mism = bits != bits_ref
    scale = np.abs(plan.qjl).max() * np.maximum(gamma_ref.astype(np.float64), 1e-30) * 128
    near = np.abs(proj_ref) < rel_window * scale[:, None]
    hard = mism & ~near
    STATS["codes"] += int(mism.size)
    STATS["code_ties"] += int((mism & near).sum())
    if hard.any():
        i = tuple(np.argwhere(hard)[0])
        raise AssertionError(f"{what}: {hard.sum()} sketch bits differ; first at {i}: proj={proj_ref[i]!r}")
    compare_norms(gamma, gamma_ref, f"{what} gamma")
    return int((mism & near).sum())


def compare_norms(gpu, ref, what):
    """Stored fp32 norms must equal the oracle's bit for bit (both sides accumulate in
    fp64 and round once to fp32). Returns 0, the number of norms off (kept so that the
    callers' summaries print it)."""
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    d = np.abs(gpu.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    STATS["norms"] += int(d.size)
    STATS["norm_mismatches"] += int((d > 0).sum())
    if (d > 0).any():
        i = tuple(np.argwhere(d > 0)[0])
        raise AssertionError(f"{what}: {(d > 0).sum()} norms differ; first off by {d[i]} ulp at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r}")
    return 0


def scale_default():
    return 1.0 / math.sqrt(128)
