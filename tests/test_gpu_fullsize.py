"""GPU parity at the full workload sizes, in the launch configurations bench.py times
(automatic split size, the fused decode step, chunked appends), on sampled rows.

Every test appends the prompt on the GPU and checks the resulting codes and norms of the
sampled (sequence, KV head) slices against the oracle's encoding of the same seeded
inputs (bit-exact, ties within 1e-6 of a threshold counted). At these sizes some ties do
occur, so before the attention is compared the sampled slices are overwritten with the
oracle's own records; the attention then runs exactly as in the benchmark and its sampled
rows are compared with the oracle's attention over the oracle's records.
Slices that are not sampled hold inputs drawn on the GPU with the same recipe
(head_inputs_device); they only shape the launch.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import gtq_oracle as O
from gtq_inputs import head_inputs, head_inputs_device, ragged_lengths
from gtq_testutil import (Case, assert_close, compare_codes, compare_norms, scale_default,
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


class Slices:
    """Host views of a cache for per-(sequence, KV head) checks and uploads."""

    def __init__(self, cache, h_kv):
        s = cache.sizes
        self.c, self.s, self.H = cache, s, h_kv
        B, cap = cache.batch, cache.capacity
        self.kc = cache.k_codes.view(B, h_kv, cap, s.k_words)
        self.kn = cache.k_norms.view(B, h_kv, cap, 4)
        self.vc = cache.v_codes.view(B, h_kv, cap // 8, s.v_words_per_block)
        self.vn = cache.v_norms.view(B, h_kv, cap)

    def check(self, hp, enc, b, h, n, what, lo=0):
        """Codes and norms of tokens lo..n-1 of slice (b, h) against the oracle's."""
        kc = self.kc[b, h, lo:n].cpu().numpy().view(np.uint32)
        kn = self.kn[b, h, lo:n].cpu().numpy()
        ties = ulps = 0
        got = unpack_key_record(kc, hp)
        for gi, (r, _) in enumerate(hp.groups):
            ties += compare_codes(got[gi], enc["k_codes"][gi][lo:n], enc["k_z"][gi][lo:n], r, f"{what} K g{gi}")
            ulps += compare_norms(kn[:, gi], enc["k_norms"][lo:n, gi], f"{what} K norm g{gi}")
        b0 = lo // 8
        nb = (n + 7) // 8
        vg = v_codes_from_physical(self.vc[b, h, b0:nb].cpu().numpy().view(np.uint32), n - 8 * b0, hp.v_bits)
        vg = vg[lo - 8 * b0:]
        ties += compare_codes(vg, enc["v_codes"][lo:n], enc["v_z"][lo:n], hp.v_bits, f"{what} V")
        ulps += compare_norms(self.vn[b, h, lo:n].cpu().numpy(), enc["v_norms"][lo:n], f"{what} V norm")
        return ties, ulps

    def upload(self, enc, b, h, n):
        """Overwrite tokens 0..n-1 of slice (b, h) with the oracle's records."""
        dev = self.c.k_codes.device
        self.kc[b, h, :n] = torch.from_numpy(enc["k_words"][:n].view(np.int32)).to(dev)
        kn = np.zeros((n, 4), np.float32)
        kn[:, :enc["k_norms"].shape[1]] = enc["k_norms"][:n]
        self.kn[b, h, :n] = torch.from_numpy(kn).to(dev)
        nb = self.c.capacity // 8
        blocks = v_codes_to_physical(enc["v_codes"][:n], self.s.v_words_per_block // 32, nb)
        m = (n + 7) // 8
        self.vc[b, h, :m] = torch.from_numpy(blocks[:m].view(np.int32)).to(dev)
        self.vn[b, h, :n] = torch.from_numpy(enc["v_norms"][:n]).to(dev)


def _plan_case(seed, h_kv, g, k_budget, v_bits):
    """Rates and rotations (library and oracle) from the calibration sets only."""
    return Case(seed, 1, h_kv, g, 1, k_budget, v_bits)


def test_fullsize_decode_8b_layer(G):
    """Llama-3.1-8B-shaped layer: 8 KV heads x g=4, batch 1, 32768 tokens, K2V2; the
    benchmark's step (prepare = append token n-1 + rotate queries, partials, merge) with
    the automatic split size; all 8 KV heads checked."""
    _say("case: full-size decode, 8 KV heads x g=4, 32768 tokens, K2V2")
    n, H, g = 32768, 8, 4
    case = Case(0, 1, H, g, n, 128, 2)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, n)
    k, v = case.kv(0, 0)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    G.gtq_quantize_append_chunk(plan, 0, cache, kd[: n - 1].contiguous(), vd[: n - 1].contiguous(), 0, 0)
    q = torch.from_numpy(case.q(0, 0)[None]).cuda()
    sl = torch.full((1,), n, dtype=torch.int32, device="cuda")
    sc = scale_default()
    ws = torch.empty(G.gtq_decode_workspace_bytes(plan, 1, n, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty(1, H * g, 128, device="cuda")
    G.gtq_decode_prepare(plan, 0, cache, kd[n - 1:].contiguous(), vd[n - 1:].contiguous(), q, sl, n, sc, ws)
    torch.cuda.synchronize()
    S = Slices(cache, H)
    ties = ulps = 0
    encs = []
    for h in range(H):
        e = O.encode_kv(case.heads[0, h], case.inputs[0, h][0]["k"], case.inputs[0, h][0]["v"])
        encs.append(e)
        t, u = S.check(case.heads[0, h], e, 0, h, n, f"8b h{h}")
        ties, ulps = ties + t, ulps + u
        S.upload(e, 0, h, n)
    _say(f"  append ties={ties} norm-ulps={ulps}")
    # the prepared queries stay in the workspace: partials and merge as in the benchmark
    G.gtq_decode_attn_partials(plan, 0, cache, sl, n, ws)
    G.gtq_decode_attn_merge(plan, 0, cache, sl, n, out, ws)
    torch.cuda.synchronize()
    qn = case.q(0, 0)
    for h in range(H):
        e = encs[h]
        sl_h = slice(h * g, (h + 1) * g)
        _, ref = O.decode_attention(case.heads[0, h], qn[sl_h], e["k_words"], e["k_norms"], e["v_words"],
                                    e["v_norms"], sc, length=n)
        assert_close(out[0, sl_h].cpu().numpy(), ref, f"8b out h{h}")


def test_fullsize_decode_3b_layer(G):
    """Qwen2.5-3B-shaped layer: 2 KV heads x g=8, batch 1, 131072 tokens, K3V3, fused step
    (gtq_decode_step, automatic split size: 128 splits, the per-row merge)."""
    _say("case: full-size decode, 2 KV heads x g=8, 131072 tokens, K3V3")
    n, H, g = 131072, 2, 8
    case = Case(1, 1, H, g, n, 192, 3)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, n)
    k, v = case.kv(0, 0)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    G.gtq_quantize_append_chunk(plan, 0, cache, kd[: n - 1].contiguous(), vd[: n - 1].contiguous(), 0, 0)
    torch.cuda.synchronize()
    S = Slices(cache, H)
    ties = 0
    encs = []
    for h in range(H):
        e = O.encode_kv(case.heads[0, h], case.inputs[0, h][0]["k"], case.inputs[0, h][0]["v"])
        encs.append(e)
        ties += S.check(case.heads[0, h], e, 0, h, n - 1, f"3b h{h}")[0]
        S.upload(e, 0, h, n)
    _say(f"  append ties={ties}")
    q = torch.from_numpy(case.q(0, 0)[None]).cuda()
    sl = torch.full((1,), n, dtype=torch.int32, device="cuda")
    sc = scale_default()
    out = G.gtq_decode_step(plan, 0, cache, kd[n - 1:].contiguous(), vd[n - 1:].contiguous(), q, sl, n, sc)
    torch.cuda.synchronize()
    # the step appended token n-1 itself; it must agree with the oracle's record
    tie_last = 0
    for h in range(H):
        tie_last += S.check(case.heads[0, h], encs[h], 0, h, n, f"3b step token h{h}", lo=n - 1)[0]
    if tie_last:  # a tie in the step's own token: restore the oracle's record and attend again
        for h in range(H):
            S.upload(encs[h], 0, h, n)
        ws = torch.empty(G.gtq_decode_workspace_bytes(plan, 1, n, 0), dtype=torch.uint8, device="cuda")
        out = G.gtq_decode_attn(plan, 0, cache, q, sl, n, sc, workspace=ws)
        torch.cuda.synchronize()
    qn = case.q(0, 0)
    for h in range(H):
        e = encs[h]
        sl_h = slice(h * g, (h + 1) * g)
        _, ref = O.decode_attention(case.heads[0, h], qn[sl_h], e["k_words"], e["k_norms"], e["v_words"],
                                    e["v_norms"], sc, length=n)
        assert_close(out[0, sl_h].cpu().numpy(), ref, f"3b out h{h}")


def test_fullsize_decode_70b_batch(G):
    """Llama-3-70B-shaped layer: 8 KV heads x g=8, batch 32 with lengths U[8192, 16384]
    (the benchmark's draw), K2V2, fused step with the automatic split (the tile merge).
    Sequences 0 and 31 are checked for all 8 KV heads."""
    seed, H, g, B = 0, 8, 8, 32
    lengths = ragged_lengths(seed, B, 8192, 16384)
    _say(f"case: full-size batched decode, 8 KV heads x g=8, batch 32, lengths {lengths.min()}..{lengths.max()}")
    case = _plan_case(seed, H, g, 128, 2)
    plan = case.plan()
    cap = int((lengths.max() + 31) // 32 * 32)
    cache = G.PackedCache(plan, B, cap)
    sampled = (0, B - 1)
    q = torch.zeros(B, H * g, 128, device="cuda")
    knew = torch.zeros(B, H, 128, device="cuda")
    vnew = torch.zeros(B, H, 128, device="cuda")
    host = {}
    for b in range(B):
        n = int(lengths[b])
        if b in sampled:
            ins = [head_inputs(seed, 0, h, g, n, seq=b) for h in range(H)]
            host[b] = ins
            k = torch.from_numpy(np.stack([d["k"] for d in ins], 1)).cuda()
            v = torch.from_numpy(np.stack([d["v"] for d in ins], 1)).cuda()
            qb = torch.from_numpy(np.concatenate([d["q"][0] for d in ins], 0)).cuda()
        else:
            ins = [head_inputs_device(seed, 0, h, g, n, "cuda", seq=b) for h in range(H)]
            k = torch.stack([d["k"] for d in ins], 1)
            v = torch.stack([d["v"] for d in ins], 1)
            qb = torch.cat([d["q"][0] for d in ins], 0)
        G.gtq_quantize_append_chunk(plan, 0, cache, k[: n - 1].contiguous(), v[: n - 1].contiguous(), b, 0)
        knew[b], vnew[b], q[b] = k[n - 1], v[n - 1], qb
    torch.cuda.synchronize()
    S = Slices(cache, H)
    encs = {}
    ties = 0
    for b in sampled:
        n = int(lengths[b])
        for h in range(H):
            d = host[b][h]
            e = O.encode_kv(case.heads[0, h], d["k"], d["v"])
            encs[b, h] = e
            ties += S.check(case.heads[0, h], e, b, h, n - 1, f"70b b{b} h{h}")[0]
            S.upload(e, b, h, n)
    _say(f"  append ties={ties}")
    sl = torch.from_numpy(lengths.astype(np.int32)).cuda()
    ml = int(lengths.max())
    sc = scale_default()
    out = G.gtq_decode_step(plan, 0, cache, knew, vnew, q, sl, ml, sc)
    torch.cuda.synchronize()
    tie_last = 0
    for b in sampled:
        for h in range(H):
            n = int(lengths[b])
            tie_last += S.check(case.heads[0, h], encs[b, h], b, h, n, f"70b step b{b} h{h}", lo=n - 1)[0]
    if tie_last:
        for b in sampled:
            for h in range(H):
                S.upload(encs[b, h], b, h, int(lengths[b]))
        out = G.gtq_decode_attn(plan, 0, cache, q, sl, ml, sc)
        torch.cuda.synchronize()
    for b in sampled:
        n = int(lengths[b])
        qn = q[b].cpu().numpy()
        for h in range(H):
            e = encs[b, h]
            sl_h = slice(h * g, (h + 1) * g)
            _, ref = O.decode_attention(case.heads[0, h], qn[sl_h], e["k_words"], e["k_norms"], e["v_words"],
                                        e["v_norms"], sc, length=n)
            assert_close(out[b, sl_h].cpu().numpy(), ref, f"70b out b{b} h{h}")


def test_fullsize_append_and_prefill_32b(G):
    """Qwen2.5-32B-shaped: 8 KV heads x g=5, K3V2, a 65536-token prompt appended in
    4096-token chunks (the append benchmark's calls), then causal prefill of the last
    4096-token chunk (the prefill benchmark's call, automatic split). KV heads 0 and 5
    are checked: every code and norm, and 8 query tokens of the chunk x 5 query heads."""
    seed, H, g, total, chunk = 3, 8, 5, 65536, 4096
    pos0 = total - chunk
    _say("case: full-size append 16 x 4096 tokens + prefill 4096 over 65536, 8 KV heads x g=5, K3V2")
    case = _plan_case(seed, H, g, 192, 2)
    plan = case.plan()
    cache = G.PackedCache(plan, 1, total)
    sampled = (0, 5)
    host = {}
    ks, vs = [], []
    for h in range(H):
        if h in sampled:
            d = head_inputs(seed, 0, h, g, total)
            host[h] = d
            ks.append(torch.from_numpy(d["k"]).cuda())
            vs.append(torch.from_numpy(d["v"]).cuda())
        else:
            d = head_inputs_device(seed, 0, h, g, total, "cuda", with_q=False)
            ks.append(d["k"])
            vs.append(d["v"])
    k = torch.stack(ks, 1)
    v = torch.stack(vs, 1)
    del ks, vs
    for m in range(total // chunk):
        G.gtq_quantize_append_chunk(plan, 0, cache, k[m * chunk:(m + 1) * chunk].contiguous(),
                                    v[m * chunk:(m + 1) * chunk].contiguous(), 0, m * chunk)
    torch.cuda.synchronize()
    del k, v
    S = Slices(cache, H)
    encs = {}
    ties = ulps = 0
    for h in sampled:
        e = O.encode_kv(case.heads[0, h], host[h]["k"], host[h]["v"])
        encs[h] = e
        t, u = S.check(case.heads[0, h], e, 0, h, total, f"32b h{h}")
        ties, ulps = ties + t, ulps + u
        S.upload(e, 0, h, total)
    _say(f"  append ties={ties} norm-ulps={ulps}")
    rng = np.random.default_rng(11)
    qn = (rng.standard_normal((chunk, H * g, 128)) * 2).astype(np.float32)
    sc = scale_default()
    out = G.gtq_prefill_attn(plan, 0, cache, torch.from_numpy(qn).cuda(), 0, pos0, sc)
    torch.cuda.synchronize()
    for t in (0, 1, 255, 1024, 2047, 3000, 4094, 4095):
        for h in sampled:
            e = encs[h]
            sl_h = slice(h * g, (h + 1) * g)
            _, ref = O.decode_attention(case.heads[0, h], qn[t, sl_h], e["k_words"], e["k_norms"], e["v_words"],
                                        e["v_norms"], sc, length=pos0 + t + 1)
            assert_close(out[t, sl_h].cpu().numpy(), ref, f"32b prefill t{t} h{h}")
