"""Python binding of libgtq (Block-GTQ packed mixed-rate TQ-MSE KV cache for MI355X).

Argument marshalling only: every step of the path runs in libgtq's host code and
HIP kernels. PyTorch supplies device memory and streams. The functions carry the
names of the C entry points declared in include/gtq.h.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch  # loads the HIP runtime that libgtq links against (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgtq.so")

HEAD_DIM = 128
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
PLAN_HOST_ONLY, PLAN_NORM_CORRECT, PLAN_QJL = 1, 2, 4
STATUS = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "ENOMEM", 4: "EDEVICE", 5: "ECAPACITY"}


class GtqError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class HeadLayout(C.Structure):
    _fields_ = [("n_groups", C.c_int32), ("rate", C.c_int32 * 4), ("dim", C.c_int32 * 4),
                ("bit_offset", C.c_int32 * 4), ("rot_offset", C.c_int32 * 4),
                ("k_words", C.c_int32), ("coord", C.c_int32 * 128), ("v_hadamard", C.c_int32)]

    def as_dict(self) -> dict:
        n = self.n_groups
        return dict(n_groups=n, rate=list(self.rate)[:n], dim=list(self.dim)[:n],
                    bit_offset=list(self.bit_offset)[:n], rot_offset=list(self.rot_offset)[:n],
                    k_words=self.k_words, coord=list(self.coord), v_hadamard=self.v_hadamard)


class PlanDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_kv_heads", C.c_int32), ("n_q_heads", C.c_int32),
                ("head_dim", C.c_int32), ("rope_layout", C.c_int32), ("k_budget", C.c_int32),
                ("v_bits", C.c_int32), ("flags", C.c_int32),
                ("k_rates", C.POINTER(C.c_uint8)), ("k_rot", C.POINTER(C.c_float)),
                ("v_rot", C.POINTER(C.c_float)), ("qjl", C.POINTER(C.c_float))]


class CacheView(C.Structure):
    _fields_ = [("k_codes", C.c_void_p), ("k_norms", C.c_void_p), ("v_codes", C.c_void_p),
                ("v_norms", C.c_void_p), ("batch", C.c_int32), ("capacity", C.c_int64),
                ("block_table", C.c_void_p), ("page_tokens", C.c_int32), ("n_pages", C.c_int32),
                ("table_stride", C.c_int32)]


class WindowView(C.Structure):
    _fields_ = [("k_sink", C.c_void_p), ("v_sink", C.c_void_p), ("k_recent", C.c_void_p),
                ("v_recent", C.c_void_p), ("batch", C.c_int32), ("n_sink", C.c_int32), ("n_recent", C.c_int32)]


class CacheSizes(C.Structure):
    _fields_ = [("k_codes_bytes", C.c_size_t), ("k_norms_bytes", C.c_size_t),
                ("v_codes_bytes", C.c_size_t), ("v_norms_bytes", C.c_size_t),
                ("k_words", C.c_int32), ("v_words_per_block", C.c_int32),
                ("logical_bits_per_token", C.c_int32), ("bytes_per_token", C.c_int32)]


_LIB = None

# (name, restype, argtypes) of every exported entry point
_SIGS = [
    ("gtq_last_error", C.c_char_p, []),
    ("gtq_rate_distortion", C.c_int32, [C.c_int32, C.POINTER(C.c_double)]),
    ("gtq_codebook", C.c_int32, [C.c_int32, C.POINTER(C.c_float), C.POINTER(C.c_float)]),
    ("gtq_alloc_rates", C.c_int32, [C.POINTER(C.c_float), C.c_int64, C.POINTER(C.c_float), C.c_int64,
                                    C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.POINTER(C.c_uint8), C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    ("gtq_head_layout_from_rates", C.c_int32, [C.POINTER(C.c_uint8), C.c_int32, C.POINTER(HeadLayout)]),
    ("gtq_plan_create", C.c_int32, [C.POINTER(PlanDesc), C.POINTER(C.c_void_p)]),
    ("gtq_plan_destroy", C.c_int32, [C.c_void_p]),
    ("gtq_plan_layout", C.c_int32, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(HeadLayout)]),
    ("gtq_plan_overflow_count", C.c_int32, [C.c_void_p, C.POINTER(C.c_int64)]),
    ("gtq_cache_bytes", C.c_int32, [C.c_void_p, C.c_int32, C.c_int64, C.POINTER(CacheSizes)]),
    ("gtq_quantize_append", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]),
    ("gtq_quantize_append_chunk", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p,
                                              C.c_void_p, C.c_int32, C.c_int64, C.c_int64, C.c_void_p]),
    ("gtq_decode_workspace_bytes", C.c_int32, [C.c_void_p, C.c_int32, C.c_int64, C.c_int32,
                                               C.POINTER(C.c_size_t)]),
    ("gtq_decode_attn", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p, C.c_void_p,
                                    C.c_int64, C.c_float, C.c_int32, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_size_t, C.c_void_p]),
    ("gtq_decode_attn_static", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p, C.c_void_p,
                                           C.c_int64, C.c_float, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    ("gtq_decode_prepare", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_int64, C.c_float, C.c_int32, C.c_void_p,
                                       C.c_size_t, C.c_void_p]),
    ("gtq_decode_step", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_int64, C.c_float, C.c_int32, C.c_void_p,
                                    C.c_void_p, C.c_size_t, C.c_void_p]),
    ("gtq_decode_rotate_queries", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p,
                                              C.c_int64, C.c_float, C.c_int32, C.c_void_p, C.c_size_t,
                                              C.c_void_p]),
    ("gtq_decode_attn_partials", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p,
                                             C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t,
                                             C.c_void_p]),
    ("gtq_decode_attn_merge", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p, C.c_int64,
                                          C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    ("gtq_prefill_workspace_bytes", C.c_int32, [C.c_void_p, C.c_int64, C.c_int64, C.c_int32,
                                                C.POINTER(C.c_size_t)]),
    ("gtq_prefill_attn", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.c_void_p, C.c_int32,
                                     C.c_int64, C.c_int64, C.c_float, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.c_size_t, C.c_void_p]),
    ("gtq_window_append", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(WindowView), C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]),
    ("gtq_decode_window_workspace_bytes", C.c_int32, [C.c_void_p, C.c_int32, C.c_int64, C.c_int32,
                                                      C.POINTER(C.c_size_t)]),
    ("gtq_decode_attn_window", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.POINTER(WindowView),
                                           C.c_void_p, C.c_void_p, C.c_int64, C.c_float, C.c_int32, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    ("gtq_decode_step_window", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(CacheView), C.POINTER(WindowView),
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_float,
                                           C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
]
EXPORTS = [s[0] for s in _SIGS]


def lib():
    """The loaded libgtq (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m packed_cache_attention_tq_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, res, args in _SIGS:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(st: int, fn: str):
    if st != 0:
        raise GtqError(st, fn, lib().gtq_last_error().decode())


def _fptr(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_float))


def _dev(t: torch.Tensor | None, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


def _need(t, numel: int, name: str, at_least: bool = False):
    """Host-side size check before a tensor's pointer reaches a kernel: the C ABI takes
    plain pointers and cannot see how much memory lies behind them."""
    if t is None:
        return
    n = t.numel()
    if (n < numel) if at_least else (n != numel):
        raise ValueError(f"{name} holds {n} elements, {'at least ' if at_least else ''}{numel} expected "
                         f"(shape {tuple(t.shape)})")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ host math

def gtq_rate_distortion(b_max: int = 4) -> np.ndarray:
    out = np.zeros(b_max + 1, np.float64)
    _check(lib().gtq_rate_distortion(b_max, out.ctypes.data_as(C.POINTER(C.c_double))), "gtq_rate_distortion")
    return out


def gtq_codebook(bits: int):
    c = np.zeros(1 << bits, np.float32)
    t = np.zeros(max(1, (1 << bits) - 1), np.float32)
    _check(lib().gtq_codebook(bits, _fptr(c), _fptr(t)), "gtq_codebook")
    return c, t[: (1 << bits) - 1]


def gtq_alloc_rates(q_cal, k_cal, b_min: int, b_max: int, budget: int, rope_layout: int = ROPE_HALF,
                    head_dim: int = HEAD_DIM):
    """Returns (rates uint8[64], scores float64[64], proxy float)."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    k = np.ascontiguousarray(k_cal, dtype=np.float32)
    rates = np.zeros(64, np.uint8)
    scores = np.zeros(64, np.float64)
    proxy = C.c_double(0.0)
    st = lib().gtq_alloc_rates(_fptr(q), q.shape[0], _fptr(k), k.shape[0], head_dim, rope_layout,
                               b_min, b_max, budget, rates.ctypes.data_as(C.POINTER(C.c_uint8)),
                               scores.ctypes.data_as(C.POINTER(C.c_double)), C.byref(proxy))
    _check(st, "gtq_alloc_rates")
    return rates, scores, proxy.value


def gtq_head_layout_from_rates(rates, rope_layout: int = ROPE_HALF) -> dict:
    r = np.ascontiguousarray(rates, dtype=np.uint8)
    lay = HeadLayout()
    _check(lib().gtq_head_layout_from_rates(r.ctypes.data_as(C.POINTER(C.c_uint8)), rope_layout,
                                            C.byref(lay)), "gtq_head_layout_from_rates")
    return lay.as_dict()


# ------------------------------------------------------------------ plans

class Plan:
    """Owner of a gtq_plan*. k_rot[l][h] is the list of group rotations (ascending
    rate) of (layer l, KV head h); v_rot is [L][H_kv][128][128]. norm_correct selects
    the norm-corrected stored norms (GTQ_PLAN_NORM_CORRECT); qjl, [L][H_kv][128][128]
    sketch matrices, the QJL residual sketch of the keys (GTQ_PLAN_QJL)."""

    def __init__(self, n_layers, n_kv_heads, n_q_heads, k_budget, v_bits, k_rates, k_rot, v_rot,
                 rope_layout=ROPE_HALF, host_only=False, head_dim=HEAD_DIM, norm_correct=False, qjl=None):
        self.n_layers, self.n_kv, self.n_q = n_layers, n_kv_heads, n_q_heads
        self.k_budget, self.v_bits = k_budget, v_bits
        self.norm_correct = bool(norm_correct)
        rates = np.ascontiguousarray(k_rates, dtype=np.uint8).reshape(-1)
        flat = [np.asarray(m, np.float32).reshape(-1) for lh in k_rot for hh in lh for m in hh]
        krot = np.ascontiguousarray(np.concatenate(flat) if flat else np.zeros(1, np.float32))
        vrot = np.ascontiguousarray(v_rot, dtype=np.float32).reshape(-1)
        self.qjl = qjl is not None
        qm = None if qjl is None else np.ascontiguousarray(qjl, dtype=np.float32).reshape(-1)
        self._keep = (rates, krot, vrot, qm)
        d = PlanDesc(n_layers, n_kv_heads, n_q_heads, head_dim, rope_layout, k_budget, v_bits,
                     (PLAN_HOST_ONLY if host_only else 0) | (PLAN_NORM_CORRECT if norm_correct else 0)
                     | (PLAN_QJL if qjl is not None else 0),
                     rates.ctypes.data_as(C.POINTER(C.c_uint8)), _fptr(krot), _fptr(vrot),
                     _fptr(qm) if qm is not None else None)
        h = C.c_void_p()
        self._h = None
        _check(lib().gtq_plan_create(C.byref(d), C.byref(h)), "gtq_plan_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def layout(self, layer: int, kv_head: int) -> dict:
        lay = HeadLayout()
        _check(lib().gtq_plan_layout(self._h, layer, kv_head, C.byref(lay)), "gtq_plan_layout")
        return lay.as_dict()

    def overflow_count(self) -> int:
        v = C.c_int64(0)
        _check(lib().gtq_plan_overflow_count(self._h, C.byref(v)), "gtq_plan_overflow_count")
        return v.value

    def cache_sizes(self, batch: int, capacity: int) -> CacheSizes:
        s = CacheSizes()
        _check(lib().gtq_cache_bytes(self._h, batch, capacity, C.byref(s)), "gtq_cache_bytes")
        return s

    def destroy(self):
        if self._h is not None and _LIB is not None:
            _LIB.gtq_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def gtq_plan_create(*args, **kw) -> Plan:
    return Plan(*args, **kw)


class PackedCache:
    """One layer's packed cache as caller-owned torch tensors (see gtq_cache_view)."""

    def __init__(self, plan: Plan, batch: int, capacity: int, device="cuda"):
        s = plan.cache_sizes(batch, capacity)
        self.batch, self.capacity, self.sizes = batch, capacity, s
        self.k_codes = torch.zeros(s.k_codes_bytes // 4, dtype=torch.int32, device=device)
        self.k_norms = torch.zeros(s.k_norms_bytes // 4, dtype=torch.float32, device=device)
        self.v_codes = torch.zeros(s.v_codes_bytes // 4, dtype=torch.int32, device=device)
        self.v_norms = torch.zeros(s.v_norms_bytes // 4, dtype=torch.float32, device=device)

    def clone(self) -> "PackedCache":
        c = PackedCache.__new__(PackedCache)
        c.batch, c.capacity, c.sizes = self.batch, self.capacity, self.sizes
        c.k_codes, c.k_norms = self.k_codes.clone(), self.k_norms.clone()
        c.v_codes, c.v_norms = self.v_codes.clone(), self.v_norms.clone()
        return c

    def view(self) -> CacheView:
        return CacheView(self.k_codes.data_ptr(), self.k_norms.data_ptr(), self.v_codes.data_ptr(),
                         self.v_norms.data_ptr(), self.batch, self.capacity)

    def nbytes(self) -> int:
        s = self.sizes
        return s.k_codes_bytes + s.k_norms_bytes + s.v_codes_bytes + s.v_norms_bytes


class PagedCache(PackedCache):
    """One layer's paged cache: a pool of n_pages pages of page_tokens tokens (each laid
    out like a contiguous cache of batch n_pages and capacity page_tokens) and a block
    table [batch, max_pages] int32 (entry -1 = absent); sequence capacity
    max_pages * page_tokens."""

    def __init__(self, plan: Plan, batch: int, n_pages: int, page_tokens: int, max_pages: int, device="cuda"):
        super().__init__(plan, n_pages, page_tokens, device)
        self.n_pages, self.page_tokens, self.max_pages = n_pages, page_tokens, max_pages
        self.batch, self.capacity = batch, max_pages * page_tokens
        self.block_table = torch.full((batch, max_pages), -1, dtype=torch.int32, device=device)

    def clone(self) -> "PagedCache":
        c = PagedCache.__new__(PagedCache)
        c.__dict__.update(self.__dict__)
        c.k_codes, c.k_norms = self.k_codes.clone(), self.k_norms.clone()
        c.v_codes, c.v_norms = self.v_codes.clone(), self.v_norms.clone()
        c.block_table = self.block_table.clone()
        return c

    def view(self) -> CacheView:
        return CacheView(self.k_codes.data_ptr(), self.k_norms.data_ptr(), self.v_codes.data_ptr(),
                         self.v_norms.data_ptr(), self.batch, self.capacity, self.block_table.data_ptr(),
                         self.page_tokens, self.n_pages, self.max_pages)


# ------------------------------------------------------------------ GPU calls

def gtq_quantize_append(plan: Plan, layer: int, cache: PackedCache, k, v, seq_idx, slot, stream=None):
    n = k.shape[0]
    for t, nm in ((k, "k"), (v, "v")):
        _need(t, n * plan.n_kv * HEAD_DIM, nm)
    _need(seq_idx, n, "seq_idx")
    _need(slot, n, "slot")
    cv = cache.view()
    st = lib().gtq_quantize_append(plan.handle, layer, C.byref(cv), _dev(k, torch.float32, "k"),
                                   _dev(v, torch.float32, "v"), _dev(seq_idx, torch.int32, "seq_idx"),
                                   _dev(slot, torch.int64, "slot"), n, _stream(stream))
    _check(st, "gtq_quantize_append")


def gtq_quantize_append_chunk(plan: Plan, layer: int, cache: PackedCache, k, v, seq: int, pos0: int,
                              stream=None):
    n = k.shape[0]
    for t, nm in ((k, "k"), (v, "v")):
        _need(t, n * plan.n_kv * HEAD_DIM, nm)
    cv = cache.view()
    st = lib().gtq_quantize_append_chunk(plan.handle, layer, C.byref(cv), _dev(k, torch.float32, "k"),
                                         _dev(v, torch.float32, "v"), seq, pos0, n, _stream(stream))
    _check(st, "gtq_quantize_append_chunk")


def gtq_decode_workspace_bytes(plan: Plan, batch: int, max_len: int, chunk: int = 0) -> int:
    out = C.c_size_t(0)
    _check(lib().gtq_decode_workspace_bytes(plan.handle, batch, max_len, chunk, C.byref(out)),
           "gtq_decode_workspace_bytes")
    return out.value


def _decode_sizes(plan, cache, q, seq_len, max_len, logits=None, k_new=None, v_new=None):
    B = cache.batch
    if q is not None:
        _need(q, B * plan.n_q * HEAD_DIM, "q")
    _need(seq_len, B, "seq_len")
    if logits is not None:
        _need(logits, B * plan.n_q * max(int(max_len), 0), "logits")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, B * plan.n_kv * HEAD_DIM, nm)


def gtq_decode_attn(plan: Plan, layer: int, cache: PackedCache, q, seq_len, max_len: int, scale: float,
                    chunk: int = 0, out=None, logits=None, workspace=None, stream=None):
    _decode_sizes(plan, cache, q, seq_len, max_len, logits)
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.numel(), "out")
    if workspace is None:
        nb = gtq_decode_workspace_bytes(plan, cache.batch, max_len, chunk)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    cv = cache.view()
    st = lib().gtq_decode_attn(plan.handle, layer, C.byref(cv), _dev(q, torch.float32, "q"),
                               _dev(seq_len, torch.int32, "seq_len"), max_len, float(scale), chunk,
                               _dev(out, torch.float32, "out"), _dev(logits, torch.float32, "logits"),
                               _dev(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(st, "gtq_decode_attn")
    return out


def gtq_decode_attn_static(plan: Plan, layer: int, cache: PackedCache, q, seq_len, max_len: int, scale: float,
                           out, chunk: int = 0, logits=None, stream=None):
    """gtq_decode_attn on the library's static scratch (no workspace); `out` is the
    caller's [batch][n_q][128] fp32 tensor."""
    _decode_sizes(plan, cache, q, seq_len, max_len, logits)
    _need(out, q.numel(), "out")
    cv = cache.view()
    st = lib().gtq_decode_attn_static(plan.handle, layer, C.byref(cv), _dev(q, torch.float32, "q"),
                                      _dev(seq_len, torch.int32, "seq_len"), max_len, float(scale), chunk,
                                      _dev(out, torch.float32, "out"), _dev(logits, torch.float32, "logits"),
                                      _stream(stream))
    _check(st, "gtq_decode_attn_static")
    return out


def gtq_decode_prepare(plan: Plan, layer: int, cache: PackedCache, k_new, v_new, q, seq_len, max_len: int,
                       scale: float, workspace, chunk: int = 0, stream=None):
    _decode_sizes(plan, cache, q, seq_len, max_len, k_new=k_new, v_new=v_new)
    cv = cache.view()
    st = lib().gtq_decode_prepare(plan.handle, layer, C.byref(cv), _dev(k_new, torch.float32, "k_new"),
                                  _dev(v_new, torch.float32, "v_new"), _dev(q, torch.float32, "q"),
                                  _dev(seq_len, torch.int32, "seq_len"), max_len, float(scale), chunk,
                                  _dev(workspace, None, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gtq_decode_prepare")


def gtq_decode_step(plan: Plan, layer: int, cache: PackedCache, k_new, v_new, q, seq_len, max_len: int,
                    scale: float, chunk: int = 0, out=None, workspace=None, stream=None):
    _decode_sizes(plan, cache, q, seq_len, max_len, k_new=k_new, v_new=v_new)
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.numel(), "out")
    if workspace is None:
        workspace = torch.empty(gtq_decode_workspace_bytes(plan, cache.batch, max_len, chunk), dtype=torch.uint8,
                                device=q.device)
    cv = cache.view()
    st = lib().gtq_decode_step(plan.handle, layer, C.byref(cv), _dev(k_new, torch.float32, "k_new"),
                               _dev(v_new, torch.float32, "v_new"), _dev(q, torch.float32, "q"),
                               _dev(seq_len, torch.int32, "seq_len"), max_len, float(scale), chunk,
                               _dev(out, torch.float32, "out"), _dev(workspace, None, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gtq_decode_step")
    return out


def gtq_decode_rotate_queries(plan: Plan, layer: int, cache: PackedCache, q, max_len: int, scale: float,
                              workspace, chunk: int = 0, stream=None):
    _decode_sizes(plan, cache, q, None, max_len)
    cv = cache.view()
    st = lib().gtq_decode_rotate_queries(plan.handle, layer, C.byref(cv), _dev(q, torch.float32, "q"), max_len,
                                         float(scale), chunk, _dev(workspace, None, "workspace"),
                                         workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gtq_decode_rotate_queries")


def gtq_decode_attn_partials(plan: Plan, layer: int, cache: PackedCache, seq_len, max_len: int, workspace,
                             chunk: int = 0, logits=None, stream=None):
    _decode_sizes(plan, cache, None, seq_len, max_len, logits)
    cv = cache.view()
    st = lib().gtq_decode_attn_partials(plan.handle, layer, C.byref(cv), _dev(seq_len, torch.int32, "seq_len"),
                                        max_len, chunk, _dev(logits, torch.float32, "logits"),
                                        _dev(workspace, None, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gtq_decode_attn_partials")


def gtq_decode_attn_merge(plan: Plan, layer: int, cache: PackedCache, seq_len, max_len: int, out, workspace,
                          chunk: int = 0, stream=None):
    _decode_sizes(plan, cache, None, seq_len, max_len)
    _need(out, cache.batch * plan.n_q * HEAD_DIM, "out")
    cv = cache.view()
    st = lib().gtq_decode_attn_merge(plan.handle, layer, C.byref(cv), _dev(seq_len, torch.int32, "seq_len"),
                                     max_len, chunk, _dev(out, torch.float32, "out"),
                                     _dev(workspace, None, "workspace"),
                                     workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gtq_decode_attn_merge")
    return out


def gtq_prefill_workspace_bytes(plan: Plan, pos0: int, n_tok: int, chunk: int = 0) -> int:
    out = C.c_size_t(0)
    _check(lib().gtq_prefill_workspace_bytes(plan.handle, pos0, n_tok, chunk, C.byref(out)),
           "gtq_prefill_workspace_bytes")
    return out.value


def gtq_prefill_attn(plan: Plan, layer: int, cache: PackedCache, q, seq: int, pos0: int, scale: float,
                     chunk: int = 0, out=None, workspace=None, stream=None):
    n = q.shape[0]
    _need(q, n * plan.n_q * HEAD_DIM, "q")
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.numel(), "out")
    if workspace is None:
        nb = gtq_prefill_workspace_bytes(plan, pos0, n, chunk)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    cv = cache.view()
    st = lib().gtq_prefill_attn(plan.handle, layer, C.byref(cv), _dev(q, torch.float32, "q"), seq, pos0, n,
                                float(scale), chunk, _dev(out, torch.float32, "out"),
                                _dev(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(st, "gtq_prefill_attn")
    return out


# ------------------------------------------------------------------ fp16 window

class WindowCache:
    """One layer's fp16 sink and recent-token buffers (see gtq_window_view): binary16
    K [batch, n_kv, slots, 128] token-major, V [batch, n_kv, slots / 8, 128, 8] in
    8-token blocks; sink slots = n_sink rounded up to 32, the recent ring has n_recent
    slots (position p at p % n_recent)."""

    def __init__(self, plan: Plan, batch: int, n_sink: int, n_recent: int, device="cuda"):
        self.batch, self.n_sink, self.n_recent = batch, n_sink, n_recent
        ss = (n_sink + 31) // 32 * 32
        h = plan.n_kv
        # never-written slots are masked by the kernels; fill with NaN so a test notices
        # any read of them into a result
        nan = float("nan")
        self.k_sink = torch.full((batch, h, max(ss, 1), 128), nan, dtype=torch.float16, device=device)
        self.v_sink = torch.full((batch, h, max(ss, 8) // 8, 128, 8), nan, dtype=torch.float16, device=device)
        self.k_recent = torch.full((batch, h, max(n_recent, 1), 128), nan, dtype=torch.float16, device=device)
        self.v_recent = torch.full((batch, h, max(n_recent, 8) // 8, 128, 8), nan, dtype=torch.float16,
                                   device=device)

    def view(self) -> WindowView:
        return WindowView(self.k_sink.data_ptr(), self.v_sink.data_ptr(), self.k_recent.data_ptr(),
                          self.v_recent.data_ptr(), self.batch, self.n_sink, self.n_recent)


def gtq_window_append(plan: Plan, layer: int, win: WindowCache, k, v, seq_idx, pos, stream=None):
    n = k.shape[0]
    for t, nm in ((k, "k"), (v, "v")):
        _need(t, n * plan.n_kv * HEAD_DIM, nm)
    _need(seq_idx, n, "seq_idx")
    _need(pos, n, "pos")
    wv = win.view()
    st = lib().gtq_window_append(plan.handle, layer, C.byref(wv), _dev(k, torch.float32, "k"),
                                 _dev(v, torch.float32, "v"), _dev(seq_idx, torch.int32, "seq_idx"),
                                 _dev(pos, torch.int64, "pos"), k.shape[0], _stream(stream))
    _check(st, "gtq_window_append")


def gtq_decode_window_workspace_bytes(plan: Plan, batch: int, max_len: int, chunk: int = 0) -> int:
    out = C.c_size_t(0)
    _check(lib().gtq_decode_window_workspace_bytes(plan.handle, batch, max_len, chunk, C.byref(out)),
           "gtq_decode_window_workspace_bytes")
    return out.value


def gtq_decode_attn_window(plan: Plan, layer: int, cache: PackedCache, win: WindowCache, q, seq_len,
                           max_len: int, scale: float, chunk: int = 0, out=None, logits=None, workspace=None,
                           stream=None):
    _decode_sizes(plan, cache, q, seq_len, max_len, logits)
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.numel(), "out")
    if workspace is None:
        nb = gtq_decode_window_workspace_bytes(plan, cache.batch, max_len, chunk)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    cv, wv = cache.view(), win.view()
    st = lib().gtq_decode_attn_window(plan.handle, layer, C.byref(cv), C.byref(wv), _dev(q, torch.float32, "q"),
                                      _dev(seq_len, torch.int32, "seq_len"), max_len, float(scale), chunk,
                                      _dev(out, torch.float32, "out"), _dev(logits, torch.float32, "logits"),
                                      _dev(workspace, None, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gtq_decode_attn_window")
    return out


def gtq_decode_step_window(plan: Plan, layer: int, cache: PackedCache, win: WindowCache, k_new, v_new, q, seq_len,
                           max_len: int, scale: float, chunk: int = 0, out=None, workspace=None, stream=None):
    """One decode step with the fp16 window: append at seq_len - 1 (packed and fp16), then attend."""
    _decode_sizes(plan, cache, q, seq_len, max_len, k_new=k_new, v_new=v_new)
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.numel(), "out")
    if workspace is None:
        nb = gtq_decode_window_workspace_bytes(plan, cache.batch, max_len, chunk)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    cv, wv = cache.view(), win.view()
    st = lib().gtq_decode_step_window(plan.handle, layer, C.byref(cv), C.byref(wv),
                                      _dev(k_new, torch.float32, "k_new"), _dev(v_new, torch.float32, "v_new"),
                                      _dev(q, torch.float32, "q"), _dev(seq_len, torch.int32, "seq_len"), max_len,
                                      float(scale), chunk, _dev(out, torch.float32, "out"),
                                      _dev(workspace, None, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gtq_decode_step_window")
    return out
