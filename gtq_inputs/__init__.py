"""Seeded synthetic inputs for the Block-GTQ packed-cache path.

This module only draws random inputs: per-block key/query scales, Gaussian
keys/queries/values, the rotary position embedding that a model applies before
caching, and Haar-random rotation matrices (the random rotations of the
TurboQuant codec are drawn here and handed to both sides as plan inputs). It
holds none of the method's arithmetic (no scores, allocation, codebooks,
quantization, packing or attention), so both the oracle and the GPU path may
import it.

Recipe (shapes follow the model shapes named on the Block-GTQ page, abstract):
  * per (layer, KV head): block std sigma_j = exp(N(0,1)) for the 64 RoPE
    blocks, two distinct blocks (uniform draw) multiplied by 8 (outliers);
  * pre-RoPE keys and queries: coordinate pair of block j ~ sigma_j * N(0,1);
    one sigma vector per KV head, shared by its keys and its g query heads;
  * values ~ N(0,1);
  * RoPE, half-split pairing (j, j+64), theta_j = 500000^(-2j/128); cached keys
    at positions 0..N-1, decode queries at position N;
  * calibration set: 256 fresh tokens (keys and g query heads per token),
    pre-RoPE, from a stream disjoint from the cache's.
Seeds: numpy SeedSequence([cfg_seed, layer, kv_head, stream]).
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
N_BLOCKS = 64
ROPE_BASE = 500000.0
N_CALIB = 256

# stream ids of the SeedSequence tuple
S_SIGMA, S_CACHE_K, S_CACHE_V, S_DEC_Q, S_CAL_Q, S_CAL_K, S_LENGTHS, S_ROT, S_QJL = range(9)

HALF, INTERLEAVED = 0, 1


def rng_for(cfg_seed: int, layer: int, kv_head: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_seed, layer, kv_head, stream])))


def seed_int(cfg_seed: int, layer: int, kv_head: int, stream: int) -> int:
    """A 63-bit integer seed derived from the same tuple (for torch device generators)."""
    st = np.random.SeedSequence([cfg_seed, layer, kv_head, stream]).generate_state(2, dtype=np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def block_std(rng: np.random.Generator, n_blocks: int = N_BLOCKS, n_outliers: int = 2,
              outlier_mult: float = 8.0) -> np.ndarray:
    sig = np.exp(rng.standard_normal(n_blocks))
    out = rng.choice(n_blocks, size=n_outliers, replace=False)
    sig[out] *= outlier_mult
    return sig


def coord_std(sig: np.ndarray, layout: int = HALF) -> np.ndarray:
    """Expand a per-block std vector to the 128 coordinates of a head."""
    j = len(sig)
    s = np.empty(2 * j)
    if layout == HALF:
        s[:j] = sig
        s[j:] = sig
    else:
        s[0::2] = sig
        s[1::2] = sig
    return s


def apply_rope(x: np.ndarray, positions: np.ndarray, base: float = ROPE_BASE,
               layout: int = HALF) -> np.ndarray:
    """Rotary embedding on the last axis (fp64 math, fp32 result). x: [..., n, D]."""
    d = x.shape[-1]
    j = d // 2
    theta = base ** (-2.0 * np.arange(j) / d)
    ang = positions.astype(np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    xd = x.astype(np.float64)
    if layout == HALF:
        a, b = xd[..., :j], xd[..., j:]
    else:
        a, b = xd[..., 0::2], xd[..., 1::2]
    ra = a * c - b * s
    rb = a * s + b * c
    out = np.empty_like(xd)
    if layout == HALF:
        out[..., :j], out[..., j:] = ra, rb
    else:
        out[..., 0::2], out[..., 1::2] = ra, rb
    return out.astype(np.float32)


def haar_rotation(d: int, rng: np.random.Generator) -> np.ndarray:
    """Haar-distributed orthogonal d x d matrix (QR of a Gaussian matrix with the
    sign of diag(R) folded into Q), rounded to fp32."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


def head_inputs(cfg_seed: int, layer: int, kv_head: int, g: int, n_cache: int,
                n_dec_q: int = 1, layout: int = HALF, qk_std: str = "shared", seq: int = 0) -> dict:
    """All inputs of one (layer, KV head): calibration (pre-RoPE), cache K (post-RoPE),
    cache V, decode queries (post-RoPE, position n_cache), as fp32 numpy arrays.
    `seq` selects the batch row: it changes the cache and query streams, not the
    per-head scales or the calibration set."""
    D = HEAD_DIM
    sig = block_std(rng_for(cfg_seed, layer, kv_head, S_SIGMA))
    sc = coord_std(sig, layout)
    if qk_std == "shared":
        sq = sc
    else:
        sq = coord_std(block_std(rng_for(cfg_seed, layer, kv_head, S_SIGMA + 100)), layout)
    so = 16 * seq
    rk = rng_for(cfg_seed, layer, kv_head, S_CACHE_K + so)
    k_pre = (rk.standard_normal((n_cache, D)) * sc).astype(np.float32)
    k = apply_rope(k_pre, np.arange(n_cache), layout=layout)
    v = rng_for(cfg_seed, layer, kv_head, S_CACHE_V + so).standard_normal((n_cache, D)).astype(np.float32)
    q_pre = (rng_for(cfg_seed, layer, kv_head, S_DEC_Q + so).standard_normal((n_dec_q, g, D)) * sq).astype(np.float32)
    q = apply_rope(q_pre.reshape(n_dec_q * g, D), np.full(n_dec_q * g, n_cache), layout=layout)
    q = q.reshape(n_dec_q, g, D)
    cq = (rng_for(cfg_seed, layer, kv_head, S_CAL_Q).standard_normal((N_CALIB, g, D)) * sq).astype(np.float32)
    ck = (rng_for(cfg_seed, layer, kv_head, S_CAL_K).standard_normal((N_CALIB, D)) * sc).astype(np.float32)
    return dict(sigma=sig, k=k, v=v, q=q, calib_q=cq.reshape(N_CALIB * g, D), calib_k=ck,
                k_pre=k_pre)


def head_inputs_device(cfg_seed: int, layer: int, kv_head: int, g: int, n_cache: int, device,
                       seq: int = 0, pos0: int = 0, n_q_tok: int = 1, q_positions=None, layout: int = HALF,
                       with_q: bool = True) -> dict:
    """The same recipe as head_inputs for large workloads, drawn on `device` with torch
    generators seeded from the same (cfg_seed, layer, kv_head, stream) tuples (so the
    numbers differ from head_inputs'): cache keys (post-RoPE, positions pos0 ..
    pos0 + n_cache - 1), values, and n_q_tok x g queries (post-RoPE at q_positions,
    default: position pos0 + n_cache). The calibration set is the small numpy one of
    head_inputs (n_cache = 0)."""
    import torch

    D = HEAD_DIM
    small = head_inputs(cfg_seed, layer, kv_head, g, 0, layout=layout)
    sc = torch.tensor(coord_std(small["sigma"], layout), dtype=torch.float32, device=device)
    so = 16 * seq

    def gen(stream):
        gg = torch.Generator(device=device)
        gg.manual_seed(seed_int(cfg_seed, layer, kv_head, stream + so))
        return gg

    def rope(x, pos):
        j = D // 2
        theta = ROPE_BASE ** (-2.0 * torch.arange(j, dtype=torch.float64, device=device) / D)
        ang = pos.to(torch.float64)[:, None] * theta[None, :]
        c, sn = torch.cos(ang), torch.sin(ang)
        xd = x.to(torch.float64)
        if layout == HALF:
            a, b = xd[..., :j], xd[..., j:]
        else:
            a, b = xd[..., 0::2], xd[..., 1::2]
        out = torch.empty_like(xd)
        if layout == HALF:
            out[..., :j], out[..., j:] = a * c - b * sn, a * sn + b * c
        else:
            out[..., 0::2], out[..., 1::2] = a * c - b * sn, a * sn + b * c
        return out.to(torch.float32)

    pos = torch.arange(pos0, pos0 + n_cache, device=device)
    k = rope(torch.randn(n_cache, D, generator=gen(S_CACHE_K), device=device) * sc, pos)
    v = torch.randn(n_cache, D, generator=gen(S_CACHE_V), device=device)
    out = dict(k=k, v=v, calib_q=small["calib_q"], calib_k=small["calib_k"], sigma=small["sigma"])
    if with_q:
        qp = torch.randn(n_q_tok, g, D, generator=gen(S_DEC_Q), device=device) * sc
        if q_positions is None:
            q_positions = torch.full((n_q_tok,), pos0 + n_cache, device=device)
        qpos = torch.as_tensor(q_positions, device=device).repeat_interleave(g)
        out["q"] = rope(qp.reshape(n_q_tok * g, D), qpos).reshape(n_q_tok, g, D)
    return out


def hadamard_rotation(d: int, rng: np.random.Generator) -> np.ndarray:
    """Randomized Hadamard rotation H_d diag(s) / sqrt(d) (d a power of two): H_d the
    Sylvester matrix, H[i][j] = (-1)^popcount(i & j), s a seeded random sign vector;
    entries +-fp32(1/sqrt(d))."""
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    h = np.where(np.vectorize(lambda x: bin(x).count("1") % 2)(i[:, None] & i[None, :]) == 1, -1.0, 1.0)
    s = np.where(rng.integers(0, 2, size=d) == 1, -1.0, 1.0)
    c = np.float32(1.0 / np.sqrt(d))
    return (h * s[None, :]).astype(np.float32) * c


def head_rotations(cfg_seed: int, layer: int, kv_head: int, group_dims: list[int],
                   v_hadamard: bool = False) -> tuple[list[np.ndarray], np.ndarray]:
    """Haar rotations for the K groups (in the order given) and the V rotation (Haar, or
    a randomized Hadamard one with v_hadamard)."""
    rng = rng_for(cfg_seed, layer, kv_head, S_ROT)
    k_rots = [haar_rotation(d, rng) for d in group_dims]
    v_rot = hadamard_rotation(HEAD_DIM, rng) if v_hadamard else haar_rotation(HEAD_DIM, rng)
    return k_rots, v_rot


def qjl_matrix(cfg_seed: int, layer: int, kv_head: int, m: int = HEAD_DIM) -> np.ndarray:
    """The residual sketch's matrix of one (layer, KV head): m x 128 entries N(0, 1), fp32."""
    return rng_for(cfg_seed, layer, kv_head, S_QJL).standard_normal((m, HEAD_DIM)).astype(np.float32)


def ragged_lengths(cfg_seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths uniform on the integers [lo, hi]."""
    return rng_for(cfg_seed, 0, 0, S_LENGTHS).integers(lo, hi + 1, size=batch).astype(np.int32)


# Workload shapes (the model shapes of the Block-GTQ page's experiments).
CONFIGS = {
    0: dict(name="tiny-1head-k2v2", layers=1, h_q=1, h_kv=1, batch=1, n=1024, n_dec_q=4,
            k_bits=2, v_bits=2),
    1: dict(name="llama3.1-8b-layer-k2v2", layers=1, h_q=32, h_kv=8, batch=1, n=32768, n_dec_q=1,
            k_bits=2, v_bits=2),
    2: dict(name="qwen2.5-3b-36L-k3v3", layers=36, h_q=16, h_kv=2, batch=1, n=131072, n_dec_q=1,
            k_bits=3, v_bits=3),
    3: dict(name="llama3-70b-80L-b32-ragged-k2v2", layers=80, h_q=64, h_kv=8, batch=32,
            n=(8192, 16384), n_dec_q=1, k_bits=2, v_bits=2),
    4: dict(name="qwen2.5-32b-prefill-k3v2", layers=64, h_q=40, h_kv=8, batch=1, n=65536,
            chunk=4096, k_bits=3, v_bits=2),
}
