"""gtq_decode_attn_static (decode attention on the library's static scratch, no
workspace and no allocation) against gtq_decode_attn on the same inputs: two calls in a
row, the second on a smaller input, at the automatic split and at an explicit one; and
the host-side refusal of a batch whose workspace exceeds the scratch."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from gtq_testutil import Case, assert_close, scale_default

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import packed_cache_attention_tq_amd as G
    G.lib()
    return G


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cache(G, case, plan, lens, cap):
    cache = G.PackedCache(plan, len(lens), cap)
    for b, n in enumerate(lens):
        k, v = case.kv(0, b, 0, n)
        G.gtq_quantize_append_chunk(plan, 0, cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), b, 0)
    return cache


def test_static_scratch_matches_workspace_path(G):
    case = Case(11, 1, 4, 4, 600, 128, 2, batch=3)
    plan = case.plan()
    sc = scale_default()
    runs = [([1, 333, 600], 608, 600), ([5, 250], 256, 250)]  # the second: a smaller input
    for chunk in (0, 64):
        for lens, cap, max_len in runs:
            _say(f"case: static-scratch decode, lens={lens} chunk={chunk}")
            cache = _cache(G, case, plan, lens, cap)
            q = torch.from_numpy(np.stack([case.q(0, b) for b in range(len(lens))])).cuda()
            sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
            ref = G.gtq_decode_attn(plan, 0, cache, q, sl, max_len, sc, chunk=chunk)
            out = torch.full_like(q, float("nan"))
            G.gtq_decode_attn_static(plan, 0, cache, q, sl, max_len, sc, out, chunk=chunk)
            torch.cuda.synchronize()
            got, want = out.cpu().numpy(), ref.cpu().numpy()
            assert np.isfinite(got).all()
            assert_close(got, want, f"static vs workspace lens={lens} chunk={chunk}")
            _say(f"  max |static - workspace| = {np.abs(got - want).max():.3g}")


def test_static_scratch_refuses_a_workspace_beyond_it(G):
    case = Case(12, 1, 4, 4, 32, 128, 2, batch=1)
    plan = case.plan()
    big = G.PackedCache(plan, 1024, 32)  # 4096 row tiles: about 68 MB of workspace
    q = torch.zeros((1024, case.HQ, 128), device="cuda")
    sl = torch.zeros(1024, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(G.GtqError, match="static scratch"):
        G.gtq_decode_attn_static(plan, 0, big, q, sl, 32, scale_default(), out)
