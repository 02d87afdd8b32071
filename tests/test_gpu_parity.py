"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Append: codes bit-exact except values whose oracle z lies within 1e-6 of a
threshold (counted and printed), fp32 norms bit-exact. Attention: logits and outputs
within 1e-4 + 2e-3 |ref| element-wise. Decode-only tests feed the GPU the oracle's
own packed cache (written into the library's layout). The end-to-end tests (append
then decode) compare the decode with the oracle's decode over the records the GPU
itself wrote, read back and converted to the canonical stream: every such comparison
runs, whether or not the append produced tie codes.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import gtq_oracle as O
from gtq_testutil import (Case, assert_close, compare_codes, compare_norms, compare_qjl, scale_default,
                          unpack_key_record, v_codes_from_physical, v_codes_to_physical)

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


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def _cache_arrays(cache, case):
    s = cache.sizes
    B, H, cap = cache.batch, case.H, cache.capacity
    kc = cache.k_codes.cpu().numpy().view(np.uint32).reshape(B, H, cap, s.k_words)
    kn = cache.k_norms.cpu().numpy().reshape(B, H, cap, 4)
    vc = cache.v_codes.cpu().numpy().view(np.uint32).reshape(B, H, cap // 8, s.v_words_per_block)
    vn = cache.v_norms.cpu().numpy().reshape(B, H, cap)
    return kc, kn, vc, vn


def _check_append(case, cache, l, b, n, enc_by_head, what):
    kc, kn, vc, vn = _cache_arrays(cache, case)
    ties = ulps = 0
    for h in range(case.H):
        hp = case.heads[l, h]
        enc = enc_by_head[h]
        got = unpack_key_record(kc[b, h, :n], hp)
        for gi, (r, _) in enumerate(hp.groups):
            ties += compare_codes(got[gi], enc["k_codes"][gi], enc["k_z"][gi], r, f"{what} K group {gi} h{h}")
            ulps += compare_norms(kn[b, h, :n, gi], enc["k_norms"][:, gi], f"{what} K norm g{gi} h{h}")
        assert np.all(kn[b, h, :n, len(hp.groups):] == 0)
        vg = v_codes_from_physical(vc[b, h], n, case.v_bits)
        ties += compare_codes(vg, enc["v_codes"], enc["v_z"], case.v_bits, f"{what} V h{h}")
        ulps += compare_norms(vn[b, h, :n], enc["v_norms"], f"{what} V norm h{h}")
    return ties, ulps


def _upload_oracle_cache(case, cache, l, b, n, enc_by_head):
    """Write the oracle's packed records into the library's cache layout."""
    s = cache.sizes
    B, H, cap = cache.batch, case.H, cache.capacity
    kc = cache.k_codes.cpu().numpy().view(np.uint32).reshape(B, H, cap, s.k_words).copy()
    kn = cache.k_norms.cpu().numpy().reshape(B, H, cap, 4).copy()
    vc = cache.v_codes.cpu().numpy().view(np.uint32).reshape(B, H, cap // 8, s.v_words_per_block).copy()
    vn = cache.v_norms.cpu().numpy().reshape(B, H, cap).copy()
    for h in range(H):
        e = enc_by_head[h]
        kc[b, h, :n] = e["k_words"]
        kn[b, h, :n] = 0
        kn[b, h, :n, :e["k_norms"].shape[1]] = e["k_norms"]
        vc[b, h] = v_codes_to_physical(e["v_codes"], case.v_bits, cap // 8)
        vn[b, h, :n] = e["v_norms"]
    cache.k_codes.copy_(torch.from_numpy(kc.view(np.int32).reshape(-1)))
    cache.k_norms.copy_(torch.from_numpy(kn.reshape(-1)))
    cache.v_codes.copy_(torch.from_numpy(vc.view(np.int32).reshape(-1)))
    cache.v_norms.copy_(torch.from_numpy(vn.reshape(-1)))


def _oracle_decode(case, l, b, n, enc_by_head, q, scale):
    """q [HQ, 128] -> (logits [HQ, n], out [HQ, 128])."""
    lg = np.zeros((case.HQ, n))
    out = np.zeros((case.HQ, 128))
    for h in range(case.H):
        e = enc_by_head[h]
        sl = slice(h * case.g, (h + 1) * case.g)
        lg[sl], out[sl] = O.decode_attention(case.heads[l, h], q[sl], e["k_words"], e["k_norms"],
                                             e["v_words"], e["v_norms"], scale, length=n)
    return lg, out


def _records_from_gpu(case, cache, l, b, n):
    """The packed records of sequence b, positions 0..n-1, as the GPU wrote them, in the
    oracle's canonical form (key words, key norms per group, value words, value norms)."""
    kc, kn, vc, vn = _cache_arrays(cache, case)
    recs = []
    for h in range(case.H):
        ng = len(case.heads[l, h].groups)
        vcodes = v_codes_from_physical(vc[b, h], n, case.v_bits)
        recs.append(dict(k_words=kc[b, h, :n].copy(), k_norms=kn[b, h, :n, :ng].copy(),
                         v_words=O.pack_codes([vcodes], [case.v_bits]), v_norms=vn[b, h, :n].copy()))
    return recs


def _encode(case, l, b, n):
    return [O.encode_kv(case.heads[l, h], case.inputs[l, h][b]["k"][:n], case.inputs[l, h][b]["v"][:n])
            for h in range(case.H)]


# ------------------------------------------------------------------------ tests

def test_config0_tiny_single_head(G):
    """1 head, 1024 tokens, K2V2, 4 queries at position 1024 (queries go to 4 batch rows
    holding the same cache)."""
    _say("case: config0 tiny single head, K2V2, N=1024, 4 queries")
    case = Case(0, 1, 1, 1, 1024, 128, 2, batch=1, n_dec_q=4)
    plan = case.plan()
    cache = G.PackedCache(plan, 4, 1024)
    k, v = case.kv(0, 0)
    kk = np.concatenate([k] * 4)
    vv = np.concatenate([v] * 4)
    seq_idx = np.repeat(np.arange(4, dtype=np.int32), 1024)
    slot = np.tile(np.arange(1024, dtype=np.int64), 4)
    G.gtq_quantize_append(plan, 0, cache, _dev(kk), _dev(vv), _dev(seq_idx), _dev(slot))
    torch.cuda.synchronize()
    enc = _encode(case, 0, 0, 1024)
    ties = ulps = 0
    for b in range(4):
        t, u = _check_append(case, cache, 0, b, 1024, enc, f"config0 b{b}")
        ties, ulps = ties + t, ulps + u
    _say(f"  append ties={ties} norm-ulps={ulps}")
    q = np.stack([case.inputs[0, 0][0]["q"][i, 0] for i in range(4)])[:, None, :]     # [4, 1, 128]
    sc = scale_default()
    logits = torch.full((4, 1, 1024), float("nan"), device="cuda")
    out = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.full(4, 1024, np.int32)), 1024, sc,
                            logits=logits)
    torch.cuda.synchronize()
    for b in range(4):
        rec = _records_from_gpu(case, cache, 0, b, 1024)[0]
        lg_ref, out_ref = O.decode_attention(case.heads[0, 0], q[b], rec["k_words"], rec["k_norms"],
                                             rec["v_words"], rec["v_norms"], sc)
        assert_close(logits[b].cpu().numpy(), lg_ref, f"config0 logits q{b}")
        assert_close(out[b].cpu().numpy(), out_ref, f"config0 out q{b}")
    _say(f"  config0: decode of 4 queries compared (append ties={ties})")


@pytest.mark.parametrize("chunk", [32, 96, 512, 0])
def test_gqa_ragged_decode_on_oracle_cache(G, chunk):
    """4 KV heads x g=4, batch 3 with lengths 1, 333, 600; split sizes 32..auto."""
    _say(f"case: gqa ragged decode, chunk={chunk}")
    case = Case(1, 1, 4, 4, 600, 128, 2, batch=3)
    plan = case.plan()
    cap = 608
    lens = [1, 333, 600]
    cache = G.PackedCache(plan, 3, cap)
    encs = []
    for b, n in enumerate(lens):
        e = _encode(case, 0, b, n)
        encs.append(e)
        _upload_oracle_cache(case, cache, 0, b, n, e)
    q = np.stack([case.q(0, b) for b in range(3)])
    sc = scale_default()
    logits = torch.zeros((3, case.HQ, 600), device="cuda")
    out = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.array(lens, np.int32)), 600, sc, chunk=chunk,
                            logits=logits)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        lg_ref, out_ref = _oracle_decode(case, 0, b, n, encs[b], q[b], sc)
        assert_close(logits[b, :, :n].cpu().numpy(), lg_ref, f"logits b{b}")
        assert_close(out[b].cpu().numpy(), out_ref, f"out b{b}")


@pytest.mark.parametrize("nc", [False, True])
def test_decode_step_fused(G, nc):
    """gtq_decode_step: every sequence appends its newest token at slot seq_len - 1 and
    attends to seq_len tokens (lengths 1, 0, 300, 129; 4 KV heads x g=4, K2V2): cache
    records and outputs against the oracle, and the same outputs as the separate
    append + decode calls; plain and norm-corrected stored norms."""
    _say(f"case: fused decode step (append + rotate, partials, merge), nc={nc}")
    case = Case(5, 1, 4, 4, 300, 128, 2, batch=4, nc=nc)
    plan = case.plan()
    cap, lens = 320, [1, 0, 300, 129]
    cache = G.PackedCache(plan, 4, cap)
    for b, n in enumerate(lens):     # the prompt: all tokens but the step's newest
        if n > 1:
            k, v = case.kv(0, b, 0, n - 1)
            G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k), _dev(v), b, 0)
    ref_cache = cache.clone()
    knew = np.zeros((4, case.H, 128), np.float32)
    vnew = np.zeros((4, case.H, 128), np.float32)
    for b, n in enumerate(lens):
        if n > 0:
            k, v = case.kv(0, b, n - 1, n)
            knew[b], vnew[b] = k[0], v[0]
    q = np.stack([case.q(0, b) for b in range(4)])
    sl = _dev(np.array(lens, np.int32))
    sc = scale_default()
    out = G.gtq_decode_step(plan, 0, cache, _dev(knew), _dev(vnew), _dev(q), sl, cap, sc)
    # the same step as separate calls
    live = [b for b, n in enumerate(lens) if n > 0]
    G.gtq_quantize_append(plan, 0, ref_cache, _dev(knew[live]), _dev(vnew[live]),
                          _dev(np.array(live, np.int32)), _dev(np.array([lens[b] - 1 for b in live], np.int64)))
    out_sep = G.gtq_decode_attn(plan, 0, ref_cache, _dev(q), sl, cap, sc)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        assert torch.equal(getattr(cache, name), getattr(ref_cache, name)), name
    assert torch.equal(out, out_sep)
    assert plan.overflow_count() == 1          # the sequence of length 0 appends nothing
    ties = 0
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[b]) == 0
            continue
        enc = _encode(case, 0, b, n)
        t, _ = _check_append(case, cache, 0, b, n, enc, f"step b{b}")
        ties += t
        _, out_ref = _oracle_decode(case, 0, b, n, _records_from_gpu(case, cache, 0, b, n), q[b], sc)
        assert_close(out[b].cpu().numpy(), out_ref, f"step out b{b}")
    _say(f"  append ties={ties}; decode of 3 sequences compared")


@pytest.mark.parametrize("nc,v_hadamard", [(False, False), (True, False), (False, True)])
def test_decode_step_one_round_prepare(G, nc, v_hadamard):
    """gtq_decode_step with as many token-heads as the chip has compute units and one row
    tile per KV head (32 sequences x 4 KV heads, g = 8): the prepare launch gives each
    workgroup one token append and one tile's query rotation. Caches and outputs equal the
    separate append + decode calls bit for bit; records and outputs of sampled sequences
    against the oracle; a sequence of length 0 appends nothing and is counted once."""
    _say(f"case: decode step, one-round prepare (32 x 4 token-heads), nc={nc} v_hadamard={v_hadamard}")
    B, H, g, cap = 32, 4, 8, 96
    case = Case(41, 1, H, g, cap, 128, 2, batch=B, nc=nc, v_hadamard=v_hadamard)
    plan = case.plan()
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(1, cap + 1, B)]
    lens[5] = 0
    lens[9] = cap
    cache = G.PackedCache(plan, B, cap)
    knew = np.zeros((B, H, 128), np.float32)
    vnew = np.zeros((B, H, 128), np.float32)
    for b, n in enumerate(lens):
        if n > 1:
            k, v = case.kv(0, b, 0, n - 1)
            G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k), _dev(v), b, 0)
        if n > 0:
            k, v = case.kv(0, b, n - 1, n)
            knew[b], vnew[b] = k[0], v[0]
    ref_cache = cache.clone()
    q = np.stack([case.q(0, b) for b in range(B)])
    sl = _dev(np.array(lens, np.int32))
    sc = scale_default()
    out = G.gtq_decode_step(plan, 0, cache, _dev(knew), _dev(vnew), _dev(q), sl, cap, sc)
    live = [b for b, n in enumerate(lens) if n > 0]
    G.gtq_quantize_append(plan, 0, ref_cache, _dev(knew[live]), _dev(vnew[live]),
                          _dev(np.array(live, np.int32)), _dev(np.array([lens[b] - 1 for b in live], np.int64)))
    out_sep = G.gtq_decode_attn(plan, 0, ref_cache, _dev(q), sl, cap, sc)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        assert torch.equal(getattr(cache, name), getattr(ref_cache, name)), name
    assert torch.equal(out, out_sep)
    assert plan.overflow_count() == 1
    assert torch.count_nonzero(out[5]) == 0
    ties = 0
    for b in (0, 9, 17, 31):
        n = lens[b]
        enc = _encode(case, 0, b, n)
        t, _ = _check_append(case, cache, 0, b, n, enc, f"one-round step b{b}")
        ties += t
        _, out_ref = _oracle_decode(case, 0, b, n, _records_from_gpu(case, cache, 0, b, n), q[b], sc)
        assert_close(out[b].cpu().numpy(), out_ref, f"one-round step out b{b}")
    _say(f"  append ties={ties}; 4 sampled sequences compared")


def test_decode_step_one_round_prepare_paged(G):
    """The one-round decode-step prepare (32 sequences x 4 KV heads, g = 8) over a paged
    cache (32-token pages, pool pages shuffled): the same records as over a contiguous
    cache, and the outputs of both against the oracle (sampled sequences)."""
    _say("case: decode step, one-round prepare, paged cache (32 x 4 token-heads)")
    B, H, g, P, maxp = 32, 4, 8, 32, 3
    cap = P * maxp
    case = Case(43, 1, H, g, cap, 128, 2, batch=B)
    plan = case.plan()
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(1, cap + 1, B)]
    cont = G.PackedCache(plan, B, cap)
    pc = G.PagedCache(plan, B, B * maxp, P, maxp)
    pc.block_table.copy_(torch.from_numpy(rng.permutation(B * maxp).astype(np.int32).reshape(B, maxp)))
    knew = np.zeros((B, H, 128), np.float32)
    vnew = np.zeros((B, H, 128), np.float32)
    for b, n in enumerate(lens):
        k, v = case.kv(0, b, 0, n)
        if n > 1:
            for c in (cont, pc):
                G.gtq_quantize_append_chunk(plan, 0, c, _dev(k[:n - 1]), _dev(v[:n - 1]), b, 0)
        knew[b], vnew[b] = k[n - 1], v[n - 1]
    q = np.stack([case.q(0, b) for b in range(B)])
    sl = _dev(np.array(lens, np.int32))
    sc = scale_default()
    o_c = G.gtq_decode_step(plan, 0, cont, _dev(knew), _dev(vnew), _dev(q), sl, cap, sc)
    o_p = G.gtq_decode_step(plan, 0, pc, _dev(knew), _dev(vnew), _dev(q), sl, cap, sc)
    torch.cuda.synchronize()
    # (a paged cache decodes every K-block slot through the generic path, so its outputs
    # round differently from the contiguous kernel's specialized slots: both are compared
    # with the oracle, and with each other at the same tolerance)
    assert_close(o_p.cpu().numpy(), o_c.cpu().numpy(), "one-round step paged vs contiguous")
    assert plan.overflow_count() == 0
    kc, kn, vc, vn = _cache_arrays(cont, case)
    for b in (0, 13, 31):
        n = lens[b]
        for h, (kw, knn, vcodes, vnn) in enumerate(_gather_paged(case, pc, b, n)):
            assert np.array_equal(kw, kc[b, h, :n]), f"paged K codes b{b} h{h}"
            assert np.array_equal(knn, kn[b, h, :n]), f"paged K norms b{b} h{h}"
            assert np.array_equal(vnn, vn[b, h, :n]), f"paged V norms b{b} h{h}"
            assert np.array_equal(vcodes, v_codes_from_physical(vc[b, h], n, case.v_bits)), f"paged V b{b} h{h}"
        _, ref = _oracle_decode(case, 0, b, n, _records_from_gpu(case, cont, 0, b, n), q[b], sc)
        assert_close(o_p[b].cpu().numpy(), ref, f"one-round paged step out b{b}")
        assert_close(o_c[b].cpu().numpy(), ref, f"one-round contiguous step out b{b}")
    _say("  paged one-round step: records and outputs of 3 sequences compared")


@pytest.mark.parametrize("k_budget,v_bits,g,layout", [(128, 1, 8, 0), (192, 3, 8, 0), (160, 4, 2, 0),
                                                      (64, 2, 8, 0), (256, 2, 4, 0), (192, 3, 2, 1),
                                                      (96, 1, 1, 1)])
def test_append_and_decode_rates(G, k_budget, v_bits, g, layout):
    """Chunked append (partial and whole value blocks) then decode, several rate mixes."""
    _say(f"case: append+decode budget={k_budget} v_bits={v_bits} g={g} layout={layout}")
    n = 203
    case = Case(2, 1, 2, g, n, k_budget, v_bits, batch=1, layout=layout)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, 224)
    k, v = case.kv(0, 0)
    for lo, hi in [(0, 5), (5, 77), (77, 80), (80, 203)]:
        G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k[lo:hi]), _dev(v[lo:hi]), 0, lo)
    torch.cuda.synchronize()
    enc = _encode(case, 0, 0, n)
    ties, ulps = _check_append(case, cache, 0, 0, n, enc, "chunked append")
    _say(f"  append ties={ties} norm-ulps={ulps}")
    _upload_oracle_cache(case, cache, 0, 0, n, enc)
    q = case.q(0, 0)[None]
    sc = 0.11
    logits = torch.zeros((1, case.HQ, n), device="cuda")
    out = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.array([n], np.int32)), n, sc, chunk=64,
                            logits=logits)
    torch.cuda.synchronize()
    lg_ref, out_ref = _oracle_decode(case, 0, 0, n, enc, q[0], sc)
    assert_close(logits[0].cpu().numpy(), lg_ref, "logits")
    assert_close(out[0].cpu().numpy(), out_ref, "out")


@pytest.mark.parametrize("H,n,splits", [(3, 300, (0, 37, 300)), (5, 2100, (0, 1000, 2100))])
def test_chunk_append_head_counts(G, H, n, splits):
    """Chunked append with KV-head counts that do not divide the eight dies: the append's
    one-dimensional grid gives workgroup w the KV head w mod H, and with 5 heads over 66
    tiles some workgroups take two tiles. Every head's codes (up to counted threshold
    ties) and norms (bit for bit) against the oracle, ragged tails included."""
    _say(f"case: chunked append with {H} KV heads, {n} tokens in chunks at {splits}")
    case = Case(4, 1, H, 2, n, 128, 2, batch=1)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, (n + 31) // 32 * 32)
    k, v = case.kv(0, 0)
    for lo, hi in zip(splits[:-1], splits[1:]):
        G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k[lo:hi]), _dev(v[lo:hi]), 0, lo)
    torch.cuda.synchronize()
    enc = _encode(case, 0, 0, n)
    ties, ulps = _check_append(case, cache, 0, 0, n, enc, f"chunked append H={H}")
    _say(f"  append ties={ties} norm-ulps={ulps}")


def test_scatter_append_random_order_and_overflow(G):
    _say("case: scatter append in random order + overflow counting")
    n = 150
    case = Case(3, 2, 2, 2, n, 128, 2, batch=2)
    plan = case.plan()
    rng = np.random.default_rng(0)
    for l in range(2):
        cache = G.PackedCache(plan, 2, 160)
        ks, vs, sq, sl = [], [], [], []
        for b in range(2):
            k, v = case.kv(l, b)
            ks.append(k)
            vs.append(v)
            sq.append(np.full(n, b, np.int32))
            sl.append(np.arange(n, dtype=np.int64))
        k, v, sq, sl = map(np.concatenate, (ks, vs, sq, sl))
        perm = rng.permutation(len(sq))
        k, v, sq, sl = k[perm], v[perm], sq[perm], sl[perm]
        before = plan.overflow_count()
        # three extra tokens that must be skipped: bad slot, bad sequence, negative slot
        k = np.concatenate([k, k[:3]])
        v = np.concatenate([v, v[:3]])
        sq = np.concatenate([sq, np.array([0, 2, 1], np.int32)])
        sl = np.concatenate([sl, np.array([160, 3, -1], np.int64)])
        G.gtq_quantize_append(plan, l, cache, _dev(k), _dev(v), _dev(sq), _dev(sl))
        torch.cuda.synchronize()
        assert plan.overflow_count() - before == 3
        for b in range(2):
            ties, _ = _check_append(case, cache, l, b, n, _encode(case, l, b, n), f"scatter l{l} b{b}")
            q = case.q(l, b)[None]
            lens = np.array([n, n], np.int32)
            out = G.gtq_decode_attn(plan, l, cache, _dev(np.concatenate([q, q])), _dev(lens), n,
                                    scale_default())
            torch.cuda.synchronize()
            _, out_ref = _oracle_decode(case, l, b, n, _records_from_gpu(case, cache, l, b, n), q[0],
                                        scale_default())
            assert_close(out[b].cpu().numpy(), out_ref, f"end-to-end out l{l} b{b}")
            _say(f"  scatter l{l} b{b}: append ties={ties}; decode compared")


def test_norm_corrected_append(G):
    """Norm-corrected stored norms through both append kernels (the tiled chunk kernel and
    the per-token scatter kernel): codes as in the plain variant, norms bit-exact to the
    oracle's corrected norms, and the decode over the corrected cache matching the
    oracle's."""
    _say("case: norm-corrected append (chunk + scatter)")
    n = 150
    case = Case(4, 1, 2, 4, n, 160, 2, batch=2, nc=True)
    plain = Case(4, 1, 2, 4, n, 160, 2, batch=2)
    plan = case.plan()
    cache = G.PackedCache(plan, 2, 160)
    # sequence 0: chunks (one tile-aligned, one ragged); sequence 1: scatter in random order
    k, v = case.kv(0, 0)
    for lo, hi in [(0, 64), (64, 101), (101, n)]:
        G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k[lo:hi]), _dev(v[lo:hi]), 0, lo)
    k1, v1 = case.kv(0, 1)
    perm = np.random.default_rng(5).permutation(n)
    G.gtq_quantize_append(plan, 0, cache, _dev(k1[perm]), _dev(v1[perm]), _dev(np.ones(n, np.int32)),
                          _dev(perm.astype(np.int64)))
    torch.cuda.synchronize()
    for b, what in ((0, "nc chunk"), (1, "nc scatter")):
        enc = _encode(case, 0, b, n)
        enc_plain = _encode(plain, 0, b, n)
        ties, ulps = _check_append(case, cache, 0, b, n, enc, what)
        _say(f"  {what}: ties={ties} norm-ulps={ulps}")
        for h in range(case.H):  # the correction changes the norms only
            for gi in range(len(enc[h]["k_codes"])):
                assert np.array_equal(enc[h]["k_codes"][gi], enc_plain[h]["k_codes"][gi])
            assert not np.array_equal(enc[h]["v_norms"], enc_plain[h]["v_norms"])
        q = case.q(0, b)[None]
        qq = np.concatenate([q, q])
        out = G.gtq_decode_attn(plan, 0, cache, _dev(qq), _dev(np.array([n, n], np.int32)), n,
                                scale_default())
        torch.cuda.synchronize()
        _, out_ref = _oracle_decode(case, 0, b, n, _records_from_gpu(case, cache, 0, b, n), q[0], scale_default())
        assert_close(out[b].cpu().numpy(), out_ref, f"{what} decode out")


@pytest.mark.parametrize("T", [60, 61, 7])
def test_prefill_chunk(G, T):
    """g = 5 (Qwen2.5-32B ratio): append 176 tokens, then a T-token chunk appended and
    attended causally over the packed cache (T g = 300, 305, 35 query rows per KV head: the
    last 16-row tile holds 12, 1 and 3 rows)."""
    _say(f"case: chunked prefill g=5 T={T}")
    n0 = 176
    case = Case(4, 1, 2, 5, n0 + T, 192, 2, batch=1)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, 256)
    k, v = case.kv(0, 0)
    enc = _encode(case, 0, 0, n0 + T)
    _upload_oracle_cache(case, cache, 0, 0, n0 + T, enc)
    rng = np.random.default_rng(5)
    q = (rng.standard_normal((T, case.HQ, 128)) * 3).astype(np.float32)
    sc = scale_default()
    out = G.gtq_prefill_attn(plan, 0, cache, _dev(q), 0, n0, sc, chunk=64)
    torch.cuda.synchronize()
    for h in range(case.H):
        sl = slice(h * 5, h * 5 + 5)
        ref = O.prefill_attention(case.heads[0, h], q[:, sl], n0, enc[h]["k_words"], enc[h]["k_norms"],
                                  enc[h]["v_words"], enc[h]["v_norms"], sc)
        assert_close(out[:, sl].cpu().numpy(), ref, f"prefill out h{h}")
    # and the same after the library's own chunk append of the prompt chunk
    G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k[n0:]), _dev(v[n0:]), 0, n0)
    torch.cuda.synchronize()
    ties, _ = _check_append(case, cache, 0, 0, n0 + T, enc, "prefill-chunk append")
    _say(f"  prefill chunk append ties={ties}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_binary16_operand_ranges(G, mode):
    """Operands that leave the binary16 range unless rescaled: value norms near 1e5 (p *
    nu_V above 65504 without the moved softmax reference) and a softmax scale of 2e4 on
    keys shrunk by 1e-5 (scaled rotated queries above 16384 without the per-tile power
    of two), against the oracle on the same records; decode (ragged batch, explicit and
    automatic split) and causal prefill. Outputs are compared in units of the value scale
    (divided by 1e4): the bar's absolute term is meant for values of order one, and an
    output that cancels terms of order 1e5 carries their fp32 rounding."""
    _say(f"case: binary16 operand ranges, {mode}")
    n = 300
    case = Case(21, 1, 2, 4, n, 128, 2, batch=2)
    for h in range(case.H):
        for b in range(2):
            inp = case.inputs[0, h][b]
            inp["k"] = (inp["k"] * 1e-5).astype(np.float32)
            inp["v"] = (inp["v"] * 1e4).astype(np.float32)
    plan = case.plan()
    sc = 2e4
    if mode == "decode":
        lens = [n, 157]
        cache = G.PackedCache(plan, 2, 320)
        encs = [_encode(case, 0, b, lens[b]) for b in range(2)]
        for b in range(2):
            _upload_oracle_cache(case, cache, 0, b, lens[b], encs[b])
        q = np.stack([case.q(0, b) for b in range(2)])
        assert np.abs(q).max() * sc > 16384 * 4
        for chunk in (64, 0):
            out = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.array(lens, np.int32)), n, sc, chunk=chunk)
            torch.cuda.synchronize()
            for b in range(2):
                _, ref = _oracle_decode(case, 0, b, lens[b], encs[b], q[b], sc)
                assert np.abs(ref).max() > 1e3
                assert_close(out[b].cpu().numpy() / 1e4, ref / 1e4, f"decode b{b} chunk={chunk}")
    else:
        n0, T = 240, 60
        cache = G.PackedCache(plan, 1, 320)
        enc = _encode(case, 0, 0, n0 + T)
        _upload_oracle_cache(case, cache, 0, 0, n0 + T, enc)
        rng = np.random.default_rng(21)
        q = (rng.standard_normal((T, case.HQ, 128)) * 3).astype(np.float32)
        out = G.gtq_prefill_attn(plan, 0, cache, _dev(q), 0, n0, sc, chunk=64)
        torch.cuda.synchronize()
        for h in range(case.H):
            sl = slice(h * case.g, (h + 1) * case.g)
            ref = O.prefill_attention(case.heads[0, h], q[:, sl], n0, enc[h]["k_words"], enc[h]["k_norms"],
                                      enc[h]["v_words"], enc[h]["v_norms"], sc)
            assert np.abs(ref).max() > 1e3
            assert_close(out[:, sl].cpu().numpy() / 1e4, ref / 1e4, f"prefill out h{h}")


@pytest.mark.parametrize("k_budget", [64, 128])
def test_qjl_residual_sketch(G, k_budget):
    """TurboQuant-prod keys (QJL residual sketch, GTQ_PLAN_QJL) at 2 and 3 bits (K1 / K2
    MSE part + one sketch bit per coordinate): records from the chunk append (through the
    per-token kernel) and from the fused decode step against the oracle (MSE codes, norms
    and gamma bit-exact, sketch signs except at near-zero projections), then decode over
    the GPU's records against the oracle: ragged batch, explicit and automatic split."""
    _say(f"case: QJL residual sketch, k_budget={k_budget}")
    case = Case(31, 1, 2, 4, 300, k_budget, 2, batch=2, qjl=True)
    plan = case.plan()
    lens = [300, 171]
    cache = G.PackedCache(plan, 2, 320)
    ties = 0
    for b, n in enumerate(lens):
        k, v = case.kv(0, b, 0, n - 1)
        G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k), _dev(v), b, 0)
    # the newest token through the fused step (decode_prep's per-token append)
    knew = np.stack([case.kv(0, b, n - 1, n)[0][0] for b, n in enumerate(lens)])
    vnew = np.stack([case.kv(0, b, n - 1, n)[1][0] for b, n in enumerate(lens)])
    q = np.stack([case.q(0, b) for b in range(2)])
    sc = scale_default()
    out_step = G.gtq_decode_step(plan, 0, cache, _dev(knew), _dev(vnew), _dev(q),
                                 _dev(np.array(lens, np.int32)), 320, sc)
    torch.cuda.synchronize()
    kc, kn, vc, vn = _cache_arrays(cache, case)
    for b, n in enumerate(lens):
        encs = _encode(case, 0, b, n)
        t, _ = _check_append(case, cache, 0, b, n, encs, f"qjl append b{b}")
        ties += t
        for h in range(case.H):
            ng = len(case.heads[0, h].groups)
            ties += compare_qjl(kc[b, h, :n], kn[b, h, :n, :ng], case.inputs[0, h][b]["k"][:n], encs[h],
                                case.heads[0, h], f"qjl sketch b{b} h{h}")
    recs = [_records_from_gpu(case, cache, 0, b, n) for b, n in enumerate(lens)]
    for chunk in (64, 0):
        out = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.array(lens, np.int32)), 320, sc, chunk=chunk)
        torch.cuda.synchronize()
        for b, n in enumerate(lens):
            _, ref = _oracle_decode(case, 0, b, n, recs[b], q[b], sc)
            assert_close(out[b].cpu().numpy(), ref, f"qjl decode b{b} chunk={chunk}")
    for b, n in enumerate(lens):
        _, ref = _oracle_decode(case, 0, b, n, recs[b], q[b], sc)
        assert_close(out_step[b].cpu().numpy(), ref, f"qjl decode step b{b}")
    _say(f"  qjl: sketch sign ties={ties}")
    with pytest.raises(G.GtqError, match="decode only"):
        G.gtq_prefill_attn(plan, 0, cache, _dev(np.zeros((4, case.HQ, 128), np.float32)), 0, 100, sc)


def test_qjl_wide_window_paged(G):
    """QJL keys with 16 query heads per KV head (two row tiles per head), 13-word records
    (8 key words per lane) and 3-bit values: decode over the GPU's records against the
    oracle; the fp16-window decode against the oracle's window decode; a paged cache (64-token
    pages, shuffled) filled the same way gives the same records and decode outputs."""
    _say("case: QJL, g=16, window and paged")
    lens, P, maxp = [200, 90], 64, 4
    case = Case(33, 1, 2, 16, 200, 128, 3, batch=2, qjl=True)
    plan = case.plan()
    cont = G.PackedCache(plan, 2, P * maxp)
    pc = G.PagedCache(plan, 2, 8, P, maxp)
    perm = np.random.default_rng(5).permutation(8)
    tab = np.full((2, maxp), -1, np.int32)
    tab[0, :4] = perm[:4]
    tab[1, :2] = perm[4:6]
    pc.block_table.copy_(torch.from_numpy(tab))
    for c in (cont, pc):
        for b, n in enumerate(lens):
            k, v = case.kv(0, b, 0, n)
            G.gtq_quantize_append_chunk(plan, 0, c, _dev(k), _dev(v), b, 0)
    q = np.stack([case.q(0, b) for b in range(2)])
    sl = _dev(np.array(lens, np.int32))
    sc = scale_default()
    out = G.gtq_decode_attn(plan, 0, cont, _dev(q), sl, P * maxp, sc)
    out_p = G.gtq_decode_attn(plan, 0, pc, _dev(q), sl, P * maxp, sc)
    win = G.WindowCache(plan, 2, 4, 32)
    for b, n in enumerate(lens):
        k, v = case.kv(0, b, 0, n)
        pos = _window_positions_to_fill(n, 4, 32)
        G.gtq_window_append(plan, 0, win, _dev(k[pos]), _dev(v[pos]), _dev(np.full(len(pos), b, np.int32)),
                            _dev(pos))
    out_w = G.gtq_decode_attn_window(plan, 0, cont, win, _dev(q), sl, P * maxp, sc, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(out, out_p)
    ties = 0
    for b, n in enumerate(lens):
        encs = _encode(case, 0, b, n)
        t, _ = _check_append(case, cont, 0, b, n, encs, f"qjl wide b{b}")
        ties += t
        recs = _records_from_gpu(case, cont, 0, b, n)
        _, ref = _oracle_decode(case, 0, b, n, recs, q[b], sc)
        assert_close(out[b].cpu().numpy(), ref, f"qjl wide decode b{b}")
        for h in range(case.H):
            e = recs[h]
            sl_ = slice(h * case.g, (h + 1) * case.g)
            inp = case.inputs[0, h][b]
            _, o_ref = O.decode_attention_window(case.heads[0, h], q[b, sl_], e["k_words"], e["k_norms"],
                                                 e["v_words"], e["v_norms"], inp["k"], inp["v"], 4, 32, sc, n)
            assert_close(out_w[b, sl_].cpu().numpy(), o_ref, f"qjl window decode b{b} h{h}")
    _say(f"  qjl wide: append ties={ties}")
    plan.destroy()


def test_edge_cases(G):
    """Zero vectors (norm 0, codes 2^(b-1)), sequences of length 0 and 1, determinism."""
    _say("case: edge cases")
    n = 40
    case = Case(5, 1, 1, 4, n, 128, 3, batch=3)
    plan = case.plan()
    cache = G.PackedCache(plan, 3, 64)
    k, v = case.kv(0, 0)
    k[7] = 0
    v[9] = 0
    k[11, :, :] = 0
    G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k), _dev(v), 0, 0)
    G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k[:1]), _dev(v[:1]), 2, 0)
    torch.cuda.synchronize()
    kc, kn, vc, vn = _cache_arrays(cache, case)
    assert np.all(kn[0, 0, 7] == 0) and np.all(vn[0, 0, 9] == 0)
    hp = case.heads[0, 0]
    codes = unpack_key_record(kc[0, 0, 7:8], hp)
    for (r, _), cg in zip(hp.groups, codes):
        assert np.all(cg == (1 << (r - 1)))
    assert np.all(v_codes_from_physical(vc[0, 0], 10, 3)[9] == 4)
    q = np.stack([case.q(0, 0)] * 3)
    lens = np.array([n, 0, 1], np.int32)
    o1 = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(lens), 64, scale_default(), chunk=32)
    o2 = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(lens), 64, scale_default(), chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.all(o1[1] == 0)
    vhat = O.dequantized_values(hp, O.encode_kv(hp, k[:1, 0], v[:1, 0])["v_words"],
                                O.encode_kv(hp, k[:1, 0], v[:1, 0])["v_norms"])
    assert_close(o1[2].cpu().numpy(), np.repeat(vhat, 4, axis=0), "length-1 sequence returns its value")
    _, ref = _oracle_decode(case, 0, 0, n, [O.encode_kv(hp, k[:, 0], v[:, 0])], q[0], scale_default())
    assert_close(o1[0].cpu().numpy(), ref, "zero-vector sequence")


def test_capacity_limit_and_merge_paths(G):
    """A cache view above 2^25 tokens is refused before any launch (no memory behind it
    is touched); both merge kernels (at most 8 splits per row: one workgroup per row
    tile; more: one per row) give the oracle's outputs on the same cache."""
    _say("case: capacity limit, merge paths")
    import ctypes as C
    case = Case(6, 1, 2, 8, 700, 128, 2, batch=2)
    plan = case.plan()
    big = G.CacheView(16, 16, 16, 16, 1, (1 << 25) + 32)  # dummy non-null pointers, never read
    out = torch.empty(1, case.HQ, 128, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    q1 = torch.zeros(1, case.HQ, 128, device="cuda")
    sl1 = torch.full((1,), 8, dtype=torch.int32, device="cuda")
    st = G.lib().gtq_decode_attn(plan.handle, 0, C.byref(big), q1.data_ptr(), sl1.data_ptr(), 8, 0.1, 0,
                                 out.data_ptr(), None, ws.data_ptr(), ws.numel(), None)
    assert st == 2  # GTQ_EUNSUPPORTED
    cache = G.PackedCache(plan, 2, 704)
    lens = [700, 333]
    encs = []
    for b, n in enumerate(lens):
        e = _encode(case, 0, b, n)
        encs.append(e)
        _upload_oracle_cache(case, cache, 0, b, n, e)
    q = np.stack([case.q(0, b) for b in range(2)])
    sc = scale_default()
    for chunk in (96, 32):  # 8 splits (tile merge) and 22 splits (row merge) at 700 tokens
        out = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.array(lens, np.int32)), 700, sc, chunk=chunk)
        torch.cuda.synchronize()
        for b, n in enumerate(lens):
            _, ref = _oracle_decode(case, 0, b, n, encs[b], q[b], sc)
            assert_close(out[b].cpu().numpy(), ref, f"chunk {chunk} out b{b}")


def _window_positions_to_fill(L, ns, nr):
    pos = [p for p in range(min(ns, L))] + [p for p in range(max(ns, L - nr), L)]
    return np.array(sorted(set(pos)), np.int64)


@pytest.mark.parametrize("ns,nr,chunk", [(4, 64, 0), (4, 64, 64), (0, 96, 0), (40, 32, 96), (0, 0, 0)])
def test_window_decode(G, ns, nr, chunk):
    """fp16 sink + recent buffers beside the packed cache: sequences shorter than the
    window, one that wraps the ring (filled in two calls, the second overwriting), and a
    plain one; logits of every position and outputs against the oracle; the buffers
    hold binary16 of the inputs exactly; unfilled slots (NaN) never reach a result."""
    _say(f"case: fp16 window decode n_sink={ns} n_recent={nr} chunk={chunk}")
    lens = [300, 37, 150]
    case = Case(6, 1, 2, 4, 300, 128, 2, batch=3)
    plan = case.plan()
    cap = 320
    cache = G.PackedCache(plan, 3, cap)
    win = G.WindowCache(plan, 3, ns, nr)
    encs = []
    for b, L in enumerate(lens):
        enc = _encode(case, 0, b, L)
        _upload_oracle_cache(case, cache, 0, b, L, enc)
        encs.append(enc)
        k, v = case.kv(0, b, 0, L)
        pos = _window_positions_to_fill(L, ns, nr)
        if b == 0 and nr:  # ring wrap: positions nr earlier first, then the real window
            early = np.arange(max(ns, L - nr - 20), L - 20, dtype=np.int64)
            G.gtq_window_append(plan, 0, win, _dev(k[early]), _dev(v[early]), _dev(np.full(len(early), b, np.int32)),
                                _dev(early))
        if len(pos):
            G.gtq_window_append(plan, 0, win, _dev(k[pos]), _dev(v[pos]), _dev(np.full(len(pos), b, np.int32)),
                                _dev(pos))
    torch.cuda.synchronize()
    # buffer contents: binary16 of the inputs, bit for bit
    for b, L in enumerate(lens):
        k, v = case.kv(0, b, 0, L)
        for p in _window_positions_to_fill(L, ns, nr):
            if p < ns:
                kb, vb = win.k_sink[b, :, p], win.v_sink[b, :, p // 8, :, p % 8]
            else:
                s_ = p % nr
                kb, vb = win.k_recent[b, :, s_], win.v_recent[b, :, s_ // 8, :, s_ % 8]
            assert np.array_equal(kb.cpu().numpy().view(np.uint16), k[p].astype(np.float16).view(np.uint16))
            assert np.array_equal(vb.cpu().numpy().view(np.uint16), v[p].astype(np.float16).view(np.uint16))
    q = np.stack([case.q(0, b) for b in range(3)])
    sc = scale_default()
    logits = torch.full((3, case.HQ, cap), float("nan"), device="cuda")
    out = G.gtq_decode_attn_window(plan, 0, cache, win, _dev(q), _dev(np.array(lens, np.int32)), cap, sc,
                                   chunk=chunk, logits=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    for b, L in enumerate(lens):
        for h in range(case.H):
            e = encs[b][h]
            sl = slice(h * case.g, (h + 1) * case.g)
            inp = case.inputs[0, h][b]
            lg_ref, o_ref = O.decode_attention_window(case.heads[0, h], q[b, sl], e["k_words"], e["k_norms"],
                                                      e["v_words"], e["v_norms"], inp["k"], inp["v"], ns, nr,
                                                      sc, L)
            assert_close(lg[b, sl, :L], lg_ref, f"window logits b{b} h{h}")
            assert_close(o[b, sl], o_ref, f"window out b{b} h{h}")
    if ns == 0 and nr == 0:  # no window: the plain decode
        ref = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.array(lens, np.int32)), cap, sc, chunk=chunk)
        torch.cuda.synchronize()
        assert_close(o, ref.cpu().numpy(), "empty window vs plain decode")
    plan.destroy()


@pytest.mark.parametrize("ns,nr", [(4, 64), (0, 96), (40, 32)])
def test_window_decode_step(G, ns, nr):
    """gtq_decode_step_window: each sequence appends its newest token at seq_len - 1 to
    the packed cache and the fp16 buffers and attends (lengths 300, 1, 0, 150; ring wrap
    for the 300 one): packed cache and fp16 buffers identical to the separate appends,
    outputs identical to gtq_decode_attn_window after them, and against the oracle."""
    _say(f"case: fused fp16 window decode step n_sink={ns} n_recent={nr}")
    lens = [300, 1, 0, 150]
    case = Case(8, 1, 2, 4, 300, 128, 2, batch=4)
    plan = case.plan()
    cap = 320
    caches = [G.PackedCache(plan, 4, cap) for _ in range(2)]
    wins = [G.WindowCache(plan, 4, ns, nr) for _ in range(2)]
    for b, L in enumerate(lens):   # the prompt: every token but the step's newest
        if L <= 1:
            continue
        k, v = case.kv(0, b, 0, L - 1)
        pos = _window_positions_to_fill(L - 1, ns, nr)
        for c, w in zip(caches, wins):
            G.gtq_quantize_append_chunk(plan, 0, c, _dev(k), _dev(v), b, 0)
            if len(pos):
                G.gtq_window_append(plan, 0, w, _dev(k[pos]), _dev(v[pos]), _dev(np.full(len(pos), b, np.int32)),
                                    _dev(pos))
    knew = np.zeros((4, case.H, 128), np.float32)
    vnew = np.zeros((4, case.H, 128), np.float32)
    for b, L in enumerate(lens):
        if L > 0:
            k, v = case.kv(0, b, L - 1, L)
            knew[b], vnew[b] = k[0], v[0]
    q = np.stack([case.q(0, b) for b in range(4)])
    sl = _dev(np.array(lens, np.int32))
    sc = scale_default()
    ov0 = plan.overflow_count()
    out = G.gtq_decode_step_window(plan, 0, caches[0], wins[0], _dev(knew), _dev(vnew), _dev(q), sl, cap, sc)
    torch.cuda.synchronize()
    assert plan.overflow_count() == ov0 + 1     # the sequence of length 0 appends nothing
    live = [b for b, L in enumerate(lens) if L > 0]
    lb = _dev(np.array(live, np.int32))
    pos = _dev(np.array([lens[b] - 1 for b in live], np.int64))
    G.gtq_quantize_append(plan, 0, caches[1], _dev(knew[live]), _dev(vnew[live]), lb, pos)
    G.gtq_window_append(plan, 0, wins[1], _dev(knew[live]), _dev(vnew[live]), lb, pos)
    out_sep = G.gtq_decode_attn_window(plan, 0, caches[1], wins[1], _dev(q), sl, cap, sc)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), name
    for name in ("k_sink", "v_sink", "k_recent", "v_recent"):
        a0, a1 = getattr(wins[0], name), getattr(wins[1], name)
        assert torch.equal(a0.view(torch.int16), a1.view(torch.int16)), name
    assert torch.equal(out, out_sep)
    o = out.cpu().numpy()
    assert np.count_nonzero(o[2]) == 0
    for b, L in enumerate(lens):
        if L == 0:
            continue
        recs = _records_from_gpu(case, caches[0], 0, b, L)
        for h in range(case.H):
            e = recs[h]
            sl_ = slice(h * case.g, (h + 1) * case.g)
            inp = case.inputs[0, h][b]
            _, o_ref = O.decode_attention_window(case.heads[0, h], q[b, sl_], e["k_words"], e["k_norms"],
                                                 e["v_words"], e["v_norms"], inp["k"], inp["v"], ns, nr, sc, L)
            assert_close(o[b, sl_], o_ref, f"window step out b{b} h{h}")
    plan.destroy()


def test_window_errors(G):
    _say("case: fp16 window argument errors")
    case = Case(7, 1, 2, 4, 64, 128, 2, batch=1)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, 64)
    q = _dev(np.stack([case.q(0, 0)]))
    sl = _dev(np.array([64], np.int32))
    for ns, nr, what in ((0, 48, "multiple of 32"), (300, 32, "n_sink"), (0, 8224, "n_recent")):
        win = G.WindowCache(plan, 1, 4, 32)
        win.n_sink, win.n_recent = ns, nr
        with pytest.raises(G.GtqError) as e:
            G.gtq_decode_attn_window(plan, 0, cache, win, q, sl, 64, 0.1)
        assert e.value.status == 1 and what in str(e.value)
    win = G.WindowCache(plan, 2, 4, 32)
    with pytest.raises(G.GtqError) as e:
        G.gtq_decode_attn_window(plan, 0, cache, win, q, sl, 64, 0.1)
    assert "batch" in str(e.value)
    plan.destroy()


def _gather_paged(case, pc, b, n):
    """Records of sequence b, positions 0..n-1, gathered from a paged cache through its
    block table: (k words, k norms, v codes [n][128], v norms)."""
    s = pc.sizes
    P, H = pc.page_tokens, case.H
    kc = pc.k_codes.cpu().numpy().view(np.uint32).reshape(pc.n_pages, H, P, s.k_words)
    kn = pc.k_norms.cpu().numpy().reshape(pc.n_pages, H, P, 4)
    vc = pc.v_codes.cpu().numpy().view(np.uint32).reshape(pc.n_pages, H, P // 8, s.v_words_per_block)
    vn = pc.v_norms.cpu().numpy().reshape(pc.n_pages, H, P)
    tab = pc.block_table.cpu().numpy()
    out = []
    for h in range(H):
        pages = [tab[b, p // P] for p in range(n)]
        kw = np.stack([kc[pg, h, p % P] for p, pg in zip(range(n), pages)])
        knn = np.stack([kn[pg, h, p % P] for p, pg in zip(range(n), pages)])
        vnn = np.array([vn[pg, h, p % P] for p, pg in zip(range(n), pages)])
        vcodes = np.concatenate([v_codes_from_physical(vc[tab[b, j], h], P, case.v_bits)
                                 for j in range((n + P - 1) // P)])[:n]
        out.append((kw, knn, vcodes, vnn))
    return out


def test_paged_cache(G):
    """A paged cache (64-token pages, shuffled pool pages, absent entries -1) filled by
    the chunk append (across page boundaries), the scatter append and the fused decode
    step holds the same records as a contiguous cache filled the same way; decode,
    window decode and prefill give the same outputs, and match the oracle; appends into
    an absent page are skipped and counted."""
    _say("case: paged cache (block table) vs contiguous")
    lens, P, maxp = [300, 150], 64, 5
    case = Case(8, 1, 2, 4, 300, 128, 2, batch=2)
    plan = case.plan()
    cont = G.PackedCache(plan, 2, P * maxp)
    pc = G.PagedCache(plan, 2, 12, P, maxp)
    perm = np.random.default_rng(3).permutation(12)
    tab = np.full((2, maxp), -1, np.int32)
    tab[0, :5] = perm[:5]
    tab[1, :3] = perm[5:8]
    pc.block_table.copy_(torch.from_numpy(tab))
    k0, v0 = case.kv(0, 0)
    k1, v1 = case.kv(0, 1)
    for c in (cont, pc):
        for lo, hi in [(0, 77), (77, 200)]:  # chunks across page boundaries
            G.gtq_quantize_append_chunk(plan, 0, c, _dev(k0[lo:hi]), _dev(v0[lo:hi]), 0, lo)
        idx = np.concatenate([np.stack([np.zeros(99, int), np.arange(200, 299)], 1),
                              np.stack([np.ones(149, int), np.arange(149)], 1)])
        idx = idx[np.random.default_rng(9).permutation(len(idx))]
        kk = np.stack([(k0 if b == 0 else k1)[p] for b, p in idx])
        vv = np.stack([(v0 if b == 0 else v1)[p] for b, p in idx])
        G.gtq_quantize_append(plan, 0, c, _dev(kk), _dev(vv), _dev(idx[:, 0].astype(np.int32)),
                              _dev(idx[:, 1].astype(np.int64)))
    before = plan.overflow_count()
    # positions 192.. of sequence 1 lie in its absent page 3
    G.gtq_quantize_append(plan, 0, pc, _dev(k1[250:251]), _dev(v1[250:251]), _dev(np.ones(1, np.int32)),
                          _dev(np.array([250], np.int64)))
    G.gtq_quantize_append_chunk(plan, 0, pc, _dev(k1[192:200]), _dev(v1[192:200]), 1, 192)
    torch.cuda.synchronize()
    assert plan.overflow_count() - before == 1 + 8
    # the step: both sequences append their last token and attend (fused prepare)
    q = np.stack([case.q(0, 0), case.q(0, 1)])
    knew = np.stack([k0[299], k1[149]])
    vnew = np.stack([v0[299], v1[149]])
    sl = _dev(np.array(lens, np.int32))
    sc = scale_default()
    o_c = G.gtq_decode_step(plan, 0, cont, _dev(knew), _dev(vnew), _dev(q), sl, P * maxp, sc)
    o_p = G.gtq_decode_step(plan, 0, pc, _dev(knew), _dev(vnew), _dev(q), sl, P * maxp, sc)
    torch.cuda.synchronize()
    kc, kn, vc, vn = _cache_arrays(cont, case)
    for b, n in enumerate(lens):
        for h, (kw, knn, vcodes, vnn) in enumerate(_gather_paged(case, pc, b, n)):
            assert np.array_equal(kw, kc[b, h, :n]), f"paged K codes b{b} h{h}"
            assert np.array_equal(knn, kn[b, h, :n]), f"paged K norms b{b} h{h}"
            assert np.array_equal(vnn, vn[b, h, :n]), f"paged V norms b{b} h{h}"
            assert np.array_equal(vcodes, v_codes_from_physical(vc[b, h], n, case.v_bits)), f"paged V b{b} h{h}"
    assert torch.equal(o_c, o_p)
    for b, n in enumerate(lens):
        enc = _encode(case, 0, b, n)
        t, _ = _check_append(case, cont, 0, b, n, enc, f"contiguous b{b}")
        _, ref = _oracle_decode(case, 0, b, n, _records_from_gpu(case, cont, 0, b, n), q[b], sc)
        assert_close(o_p[b].cpu().numpy(), ref, f"paged step out b{b}")
        _say(f"  paged b{b}: append ties={t}; step output compared")
    # window decode and prefill over the paged cache equal the contiguous ones
    win = G.WindowCache(plan, 2, 4, 64)
    for b, n in enumerate(lens):
        kx, vx = case.kv(0, b, 0, n)
        pos = _window_positions_to_fill(n, 4, 64)
        G.gtq_window_append(plan, 0, win, _dev(kx[pos]), _dev(vx[pos]), _dev(np.full(len(pos), b, np.int32)),
                            _dev(pos))
    w_c = G.gtq_decode_attn_window(plan, 0, cont, win, _dev(q), sl, P * maxp, sc, chunk=64)
    w_p = G.gtq_decode_attn_window(plan, 0, pc, win, _dev(q), sl, P * maxp, sc, chunk=64)
    qp = (np.random.default_rng(4).standard_normal((40, case.HQ, 128)) * 2).astype(np.float32)
    p_c = G.gtq_prefill_attn(plan, 0, cont, _dev(qp), 0, 260, sc, chunk=64)
    p_p = G.gtq_prefill_attn(plan, 0, pc, _dev(qp), 0, 260, sc, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(w_c, w_p)
    assert torch.equal(p_c, p_p)
    plan.destroy()


@pytest.mark.parametrize("chunk", [0, 32])
def test_hadamard_value_rotation(G, chunk):
    """Randomized Hadamard value rotations (detected at plan creation): the chunk append
    (dense split rotation), the scatter append and the decode step (fast transform), and
    the merge's inverse rotation (fast transform; tile merge and row merge) against the
    oracle's dense Pi_V."""
    _say(f"case: Hadamard value rotation, chunk={chunk}")
    lens = [290, 64]
    case = Case(10, 1, 2, 4, 290, 128, 2, batch=2, v_hadamard=True)
    plan = case.plan()
    assert all(plan.layout(0, h)["v_hadamard"] == 1 for h in range(case.H))
    cache = G.PackedCache(plan, 2, 320)
    k0, v0 = case.kv(0, 0)
    k1, v1 = case.kv(0, 1)
    G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k0[:200]), _dev(v0[:200]), 0, 0)
    idx = np.random.default_rng(2).permutation(89) + 200
    G.gtq_quantize_append(plan, 0, cache, _dev(k0[idx]), _dev(v0[idx]), _dev(np.zeros(89, np.int32)), _dev(idx))
    G.gtq_quantize_append_chunk(plan, 0, cache, _dev(k1[:63]), _dev(v1[:63]), 1, 0)
    q = np.stack([case.q(0, 0), case.q(0, 1)])
    sl = _dev(np.array(lens, np.int32))
    sc = scale_default()
    out = G.gtq_decode_step(plan, 0, cache, _dev(np.stack([k0[289], k1[63]])), _dev(np.stack([v0[289], v1[63]])),
                            _dev(q), sl, 320, sc, chunk=chunk)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        enc = _encode(case, 0, b, n)
        ties, ulps = _check_append(case, cache, 0, b, n, enc, f"hadamard b{b}")
        _say(f"  b{b}: ties={ties} norm-ulps={ulps}; decode compared")
        _, ref = _oracle_decode(case, 0, b, n, _records_from_gpu(case, cache, 0, b, n), q[b], sc)
        assert_close(out[b].cpu().numpy(), ref, f"hadamard out b{b}")
    plan.destroy()


def test_paged_view_errors(G):
    """Paged views that the host rejects before any launch: a page size that is not a
    power of two of at least 32, an empty pool, a capacity beyond the table."""
    _say("case: paged view argument errors")
    case = Case(11, 1, 2, 4, 64, 128, 2, batch=1)
    plan = case.plan()
    q = _dev(np.stack([case.q(0, 0)]))
    sl = _dev(np.array([64], np.int32))
    for P, n_pages, maxp in ((48, 4, 2), (16, 4, 4), (64, 4, 2)):
        pc = G.PagedCache(plan, 1, n_pages, P if P % 32 == 0 else 64, maxp)
        pc.page_tokens = P
        if P == 64:
            pc.capacity = 64 * maxp + 64  # beyond table_stride * page_tokens
        with pytest.raises(G.GtqError) as e:
            G.gtq_decode_attn(plan, 0, pc, q, sl, 64, 0.1)
        assert e.value.status == 1 and "paged cache" in str(e.value)
    plan.destroy()


@pytest.mark.parametrize("g", [12, 16])
def test_wide_gqa_groups(G, g):
    """More than 8 query heads per KV head (two row tiles per KV head): append, decode
    (tile and row merges), the fused step and the fp16 window decode against the oracle."""
    _say(f"case: GQA group of {g} query heads")
    n = 170
    case = Case(12, 1, 2, g, n, 128, 2, batch=1)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, 192)
    enc = _encode(case, 0, 0, n)
    _upload_oracle_cache(case, cache, 0, 0, n, enc)
    q = case.q(0, 0)[None]
    sc = scale_default()
    for chunk in (0, 32):
        lg = torch.zeros((1, case.HQ, n), device="cuda")
        out = G.gtq_decode_attn(plan, 0, cache, _dev(q), _dev(np.array([n], np.int32)), n, sc, chunk=chunk,
                                logits=lg)
        torch.cuda.synchronize()
        lg_ref, out_ref = _oracle_decode(case, 0, 0, n, enc, q[0], sc)
        assert_close(lg[0].cpu().numpy(), lg_ref, f"g{g} logits chunk {chunk}")
        assert_close(out[0].cpu().numpy(), out_ref, f"g{g} out chunk {chunk}")
    win = G.WindowCache(plan, 1, 4, 32)
    k, v = case.kv(0, 0)
    pos = _window_positions_to_fill(n, 4, 32)
    G.gtq_window_append(plan, 0, win, _dev(k[pos]), _dev(v[pos]), _dev(np.zeros(len(pos), np.int32)), _dev(pos))
    ow = G.gtq_decode_attn_window(plan, 0, cache, win, _dev(q), _dev(np.array([n], np.int32)), n, sc)
    torch.cuda.synchronize()
    for h in range(case.H):
        e = enc[h]
        sl = slice(h * g, (h + 1) * g)
        inp = case.inputs[0, h][0]
        _, o_ref = O.decode_attention_window(case.heads[0, h], q[0, sl], e["k_words"], e["k_norms"], e["v_words"],
                                             e["v_norms"], inp["k"], inp["v"], 4, 32, sc, n)
        assert_close(ow[0, sl].cpu().numpy(), o_ref, f"g{g} window out h{h}")
    plan.destroy()
