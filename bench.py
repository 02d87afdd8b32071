"""Benchmark: packed-KV decode attention over a Block-GTQ (mixed-rate TQ-MSE) cache.

One step = one decode step of one Llama-3.1-8B-shaped attention layer at batch 1:
quantize-append the step's new key/value token (8 KV heads) into the packed cache,
then split-K packed decode attention of the 32 query heads over the 32768 cached
tokens: one launch appends the token and rotates the queries, one computes the
per-split online-softmax partials, one does the log-sum-exp merge with the inverse
value rotation. Inputs are seeded synthetic tensors with the pages' distributions,
resident in HBM before timing. The cache is replicated into --copies layer caches
that the steps cycle through (as a 32-layer stack would), so that each step reads
its cache from HBM rather than from the 256 MB last-level cache.

Prints one JSON line (metric, value = KV tokens/s, roofline of the attention
(partials) kernel measured with HIP events around each of its launches in the timed
region, cpu_baseline = the
fp64 oracle timed on a bounded slice of the same workload on this host).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--copies", type=int, default=32, help="layer caches the steps cycle through")
    p.add_argument("--chunk", type=int, default=0, help="split size (0 = automatic)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--workload", default="decode-8b",
                   choices=["decode-8b", "decode-3b-36L", "decode-70b-b32", "append-32b", "prefill-32b",
                            "logit-mae", "decode-8b-window"],
                   help="decode-8b (default, the headline): Llama-3.1-8B-shaped layer decode; the others "
                        "measure the other workload shapes (one JSON line each)")
    p.add_argument("--norm-correct", action="store_true",
                   help="append-32b: plan with norm-corrected stored norms (GTQ_PLAN_NORM_CORRECT)")
    p.add_argument("--paged", type=int, default=0,
                   help="decode-8b: a paged cache of this many tokens per page (pool pages in shuffled order)")
    p.add_argument("--v-hadamard", action="store_true",
                   help="decode-8b: randomized Hadamard value rotations (applied as fast transforms)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after timing, run a plain device copy (torch.neg) of this many MiB three "
                        "times: a kernel of known traffic that calibrates the HBM byte counters")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_partials_k2v2_32k_traffic.txt")
KERNEL_SRC = os.path.join(ROOT, "packed_cache_attention_tq_amd", "csrc", "gtq_device.hip")


def measured_traffic():
    """HBM bytes per launch of the attention (partials) kernel from the committed counter
    summary, or None when the kernel source has changed since the counters were taken."""
    import hashlib
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE).read().splitlines()
                  if ":" in line and not line.startswith("#"))
        sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
        if kv["kernel_source_sha256"].strip() != sha:
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def build_workload(seed, n_ctx=32768, h_kv=8, g=4, k_budget=128, v_bits=2, v_hadamard=False):
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs, head_rotations

    rates = np.zeros((1, h_kv, 64), np.uint8)
    krot, vrot, inps = [[]], [[]], []
    for h in range(h_kv):
        inp = head_inputs(seed, 0, h, g, n_ctx)   # the last token is the step's new token
        r, _, _ = G.gtq_alloc_rates(inp["calib_q"], inp["calib_k"], 1, 4, k_budget)
        rates[0, h] = r
        lay = G.gtq_head_layout_from_rates(r)
        kr, vr = head_rotations(seed, 0, h, lay["dim"], v_hadamard=v_hadamard)
        krot[0].append(kr)
        vrot[0].append(vr)
        inps.append(inp)
    plan = G.Plan(1, h_kv, h_kv * g, k_budget, v_bits, rates, krot, np.array(vrot))
    k = np.stack([i["k"] for i in inps], axis=1)          # [n_ctx+1, H, 128]
    v = np.stack([i["v"] for i in inps], axis=1)
    q = np.concatenate([i["q"][0] for i in inps])[None]   # [1, 32, 128]
    return dict(plan=plan, k=k, v=v, q=q, rates=rates, krot=krot, vrot=vrot, inps=inps,
                n_ctx=n_ctx, h_kv=h_kv, g=g, k_budget=k_budget, v_bits=v_bits)


def partials_kernel_name(plan, layer, h_kv, v_bits):
    """The partials kernel instance a decode of this layer launches: value bits, key words
    per lane (4 up to 8 key words, else 8) and the layer's largest K-block count."""
    lays = [plan.layout(layer, h) for h in range(h_kv)]
    nkb = max(sum((d + 31) // 32 for d in lay["dim"]) for lay in lays)
    kwl = 4 if lays[0]["k_words"] <= 8 else 8
    return f"attn_partials_kernel<{v_bits}, {kwl}, {nkb}>"


def make_plan(seed, n_layers, h_kv, g, k_budget, v_bits, share_layer0=False, nc=False):
    """A plan with library-allocated rates (from each head's calibration set) and Haar
    rotations; with share_layer0 every layer reuses layer 0's rates and rotations."""
    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs, head_rotations

    rates = np.zeros((n_layers, h_kv, 64), np.uint8)
    krot, vrot = [], []
    for l in range(n_layers):
        if share_layer0 and l > 0:
            rates[l] = rates[0]
            krot.append(krot[0])
            vrot.append(vrot[0])
            continue
        kl, vl = [], []
        for h in range(h_kv):
            inp = head_inputs(seed, l, h, g, 0)
            r, _, _ = G.gtq_alloc_rates(inp["calib_q"], inp["calib_k"], 1, 4, k_budget)
            rates[l, h] = r
            kr, vr = head_rotations(seed, l, h, G.gtq_head_layout_from_rates(r)["dim"])
            kl.append(kr)
            vl.append(vr)
        krot.append(kl)
        vrot.append(vl)
    return G.Plan(n_layers, h_kv, h_kv * g, k_budget, v_bits, rates, krot, np.array(vrot), norm_correct=nc)


def fill_layer(plan, layer, cache, seed, h_kv, g, lengths, gen_layer=None):
    """Append seeded synthetic keys/values of every sequence (token n - 1 excluded: the
    step appends it) and return the step's new tokens and queries."""
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs_device

    dev = torch.device("cuda")
    gl = layer if gen_layer is None else gen_layer
    B = len(lengths)
    knew = torch.zeros(B, h_kv, 128, device=dev)
    vnew = torch.zeros(B, h_kv, 128, device=dev)
    q = torch.zeros(B, h_kv * g, 128, device=dev)
    for b, n in enumerate(lengths):
        ks, vs = [], []
        for h in range(h_kv):
            d = head_inputs_device(seed, gl, h, g, int(n), dev, seq=b)
            ks.append(d["k"])
            vs.append(d["v"])
            q[b, h * g:(h + 1) * g] = d["q"][0]
        k = torch.stack(ks, 1)
        v = torch.stack(vs, 1)
        if n > 1:
            G.gtq_quantize_append_chunk(plan, layer, cache, k[: n - 1].contiguous(), v[: n - 1].contiguous(), b, 0)
        knew[b], vnew[b] = k[n - 1], v[n - 1]
        del ks, vs, k, v
    return knew, vnew, q


def timed_graph(fn, steps, warmup):
    """Capture fn (one step of kernel launches on the current stream) in a HIP graph,
    replay it warmup + steps times; returns ms per step."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager run before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def bench_decode_stack(args, name):
    """Multi-layer decode steps as one HIP graph per step: decode-3b-36L (Qwen2.5-3B shape:
    36 layers, 16 query / 2 KV heads, batch 1, 131072 tokens, K3V3) or decode-70b-b32
    (Llama-3-70B shape: 80 layers, 64 query / 8 KV heads, batch 32 with ragged lengths
    uniform in [8192, 16384], K2V2; the 80 layer caches hold copies of one generated layer
    and every layer uses that layer's rates and rotations)."""
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import ragged_lengths

    if name == "decode-3b-36L":
        L, h_kv, g, kb, vb, lengths, share = 36, 2, 8, 192, 3, np.array([131072]), False
    else:
        L, h_kv, g, kb, vb, share = 80, 8, 8, 128, 2, True
        lengths = ragged_lengths(args.seed, 32, 8192, 16384)
    B, cap = len(lengths), int((lengths.max() + 31) // 32 * 32)
    t_setup = time.perf_counter()
    plan = make_plan(args.seed, L, h_kv, g, kb, vb, share_layer0=share)
    caches, steps_in = [], []
    for l in range(L):
        if share and l > 0:
            caches.append(caches[0].clone())
            steps_in.append(steps_in[0])
            continue
        c = G.PackedCache(plan, B, cap)
        steps_in.append(fill_layer(plan, l, c, args.seed, h_kv, g, lengths))
        caches.append(c)
    torch.cuda.synchronize()
    sl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    max_len = int(lengths.max())
    ws = [torch.empty(G.gtq_decode_workspace_bytes(plan, B, max_len, 0), dtype=torch.uint8, device="cuda")
          for _ in range(2)]
    outs = [torch.empty(B, h_kv * g, 128, device="cuda") for _ in range(L)]
    scale = 1.0 / math.sqrt(128)
    log(f"{name}: setup {time.perf_counter() - t_setup:.1f}s, {L} layers, cache "
        f"{sum(c.nbytes() for c in caches) / 1e9:.2f} GB")

    def step():
        for l in range(L):
            kn, vn, q = steps_in[l]
            G.gtq_decode_step(plan, l, caches[l], kn, vn, q, sl, max_len, scale,
                              out=outs[l], workspace=ws[l & 1])

    ms = timed_graph(step, args.steps, args.warmup)
    kv_tok = L * int(lengths.sum())
    sizes = caches[0].sizes
    alg = L * (int(lengths.sum()) * h_kv * sizes.bytes_per_token)
    return {
        "metric": "packed-KV decode attention: KV tokens/s + achieved HBM GB/s (% of peak)",
        "value": round(kv_tok / (ms / 1e3), 1), "unit": "KV tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 (fp16 hi/lo split MFMA operands, fp32 accumulation; u32 packed codes)",
        "data": "synthetic",
        "config": {"workload": name, "layers": L, "global_batch": B, "kv_heads": h_kv, "q_heads": h_kv * g,
                   "seq_len": [int(lengths.min()), int(lengths.max())], "k_bits_avg": kb / 64, "v_bits": vb,
                   "graph": "one HIP graph per step (append + rotate, partials, merge per layer)"},
        "step_hbm_gbs": round(alg / (ms / 1e3) / 1e9, 1), "step_hbm_frac": round(alg / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
    }


def bench_append(args):
    """append-32b: Qwen2.5-32B-shaped chunk append, 4096-token chunks x 8 KV heads, K3V2,
    the 16 chunks of a 65536-token prompt in turn (one call = one chunk-layer)."""
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs_device

    h_kv, g, kb, vb, chunk, total = 8, 5, 192, 2, 4096, 65536
    plan = make_plan(args.seed, 1, h_kv, g, kb, vb, nc=args.norm_correct)
    cache = G.PackedCache(plan, 1, total)
    ks = torch.stack([head_inputs_device(args.seed, 0, h, g, total, "cuda", with_q=False)["k"] for h in range(h_kv)], 1)
    vs = torch.stack([head_inputs_device(args.seed, 0, h, g, total, "cuda", with_q=False)["v"] for h in range(h_kv)], 1)
    chunks = [(ks[m * chunk:(m + 1) * chunk].contiguous(), vs[m * chunk:(m + 1) * chunk].contiguous())
              for m in range(total // chunk)]
    for m, (k, v) in enumerate(chunks):
        G.gtq_quantize_append_chunk(plan, 0, cache, k, v, 0, m * chunk)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_steps = max(args.steps, 16)
    t0.record()
    for i in range(n_steps):
        m = i % len(chunks)
        G.gtq_quantize_append_chunk(plan, 0, cache, chunks[m][0], chunks[m][1], 0, m * chunk)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n_steps
    per_tok = 2 * 128 * 4 + cache.sizes.bytes_per_token  # fp32 key + value in, packed record out
    alg = chunk * h_kv * per_tok
    return {
        "metric": "fused rotate+quantize+pack append: tokens/s + achieved HBM GB/s (% of peak)",
        "value": round(chunk / (ms / 1e3), 1), "unit": "tokens/s (x 8 KV heads)", "n_gpus": 1, "steps": n_steps,
        "warmup": 16, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 in; binary16 hi/lo split MFMA; u32 packed codes", "data": "synthetic",
        "config": {"workload": "append-32b", "chunk_tokens": chunk, "kv_heads": h_kv, "k_bits_avg": kb / 64,
                   "v_bits": vb, "prompt": total, "norm_correct": bool(args.norm_correct)},
        "roofline": {"bound": "hbm", "achieved": round(alg / (ms / 1e3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(alg / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "append_gemm_kernel", "alg_bytes_per_launch": int(alg)},
    }


def bench_prefill(args):
    """prefill-32b: causal chunked-prefill attention of the last 4096-token chunk of a
    65536-token prompt (Qwen2.5-32B shape: 40 query / 8 KV heads, K3V2) over the packed
    cache; reported as TFLOP/s of the attention products (2 x 2 x 128 flop per visible
    (query, key) pair and head)."""
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs_device

    h_kv, g, kb, vb, chunk, total = 8, 5, 192, 2, 4096, 65536
    pos0 = total - chunk
    plan = make_plan(args.seed, 1, h_kv, g, kb, vb)
    cache = G.PackedCache(plan, 1, total)
    qpos = torch.arange(pos0, total, device="cuda")
    ds = [head_inputs_device(args.seed, 0, h, g, total, "cuda", n_q_tok=chunk, q_positions=qpos) for h in range(h_kv)]
    k = torch.stack([d["k"] for d in ds], 1)
    v = torch.stack([d["v"] for d in ds], 1)
    G.gtq_quantize_append_chunk(plan, 0, cache, k.contiguous(), v.contiguous(), 0, 0)
    q = torch.cat([d["q"] for d in ds], 1).contiguous()  # [chunk, 40, 128]
    del ds, k, v
    ws = torch.empty(G.gtq_prefill_workspace_bytes(plan, pos0, chunk), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(128)
    G.gtq_prefill_attn(plan, 0, cache, q, 0, pos0, scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_steps = max(1, min(args.steps, 5))
    t0.record()
    for _ in range(n_steps):
        G.gtq_prefill_attn(plan, 0, cache, q, 0, pos0, scale, out=out, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n_steps
    pairs = sum(pos0 + t + 1 for t in range(chunk)) * h_kv * g
    flop = 4.0 * 128 * pairs
    return {
        "metric": "chunked prefill attention over the packed cache: TFLOP/s",
        "value": round(flop / (ms / 1e3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": n_steps,
        "warmup": 1, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 (fp16 hi/lo split MFMA operands, fp32 accumulation)", "data": "synthetic",
        "config": {"workload": "prefill-32b", "chunk": chunk, "pos0": pos0, "q_heads": h_kv * g, "kv_heads": h_kv,
                   "k_bits_avg": kb / 64, "v_bits": vb},
    }


def bench_logit_mae(args):
    """K-only logit error of Block-GTQ (greedy per-block rates) against uniform TQ-MSE
    (every block at the same rate), at 2 and 3 average key bits: one Llama-3.1-8B-shaped
    layer (8 KV heads, g = 4), 8192 cached tokens. The logits come from the packed-cache
    decode kernel's logits output and are compared with exact fp32 logits of the
    unquantized keys (mean absolute error over queries and tokens)."""
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs, head_inputs_device, head_rotations

    h_kv, g, n, vb = 8, 4, 8192, 2
    scale = 1.0 / math.sqrt(128)
    D = G.gtq_rate_distortion(4)
    out = {}
    for bits in (2, 3):
        for mode in ("block-gtq", "uniform"):
            rates, krot, vrot, prox = [], [], [], 0.0
            for h in range(h_kv):
                inp = head_inputs(args.seed, 0, h, g, 0)
                r, sc, px = G.gtq_alloc_rates(inp["calib_q"], inp["calib_k"], 1, 4, 64 * bits)
                if mode == "uniform":
                    r = np.full(64, bits, np.uint8)
                    px = float(np.sum(sc * D[bits]))
                prox += px
                kr, vr = head_rotations(args.seed, 0, h, G.gtq_head_layout_from_rates(r)["dim"])
                rates.append(r)
                krot.append(kr)
                vrot.append(vr)
            plan = G.Plan(1, h_kv, h_kv * g, 64 * bits, vb, np.array(rates)[None], [krot], np.array(vrot)[None])
            cache = G.PackedCache(plan, 1, n)
            ds = [head_inputs_device(args.seed, 0, h, g, n, "cuda") for h in range(h_kv)]
            k = torch.stack([d["k"] for d in ds], 1).contiguous()
            v = torch.stack([d["v"] for d in ds], 1).contiguous()
            q = torch.cat([d["q"][0] for d in ds], 0)[None].contiguous()
            G.gtq_quantize_append_chunk(plan, 0, cache, k, v, 0, 0)
            logits = torch.zeros(1, h_kv * g, n, device="cuda")
            G.gtq_decode_attn(plan, 0, cache, q, torch.full((1,), n, dtype=torch.int32, device="cuda"), n, scale,
                              logits=logits)
            exact = torch.cat([(q[0, h * g:(h + 1) * g] @ k[:, h].T) * scale for h in range(h_kv)], 0)
            err = (logits[0] - exact).abs()
            out[f"K{bits}_{mode}"] = {"logit_mae": round(float(err.mean()), 6),
                                      "logit_max_err": round(float(err.max()), 5),
                                      "proxy_sum_s_D": round(prox, 6)}
            del cache, k, v, logits, exact
            plan.destroy()
    ratio = out["K2_uniform"]["logit_mae"] / out["K2_block-gtq"]["logit_mae"]
    return {
        "metric": "K-only logit MAE, Block-GTQ rates vs uniform TQ-MSE (ratio uniform / Block-GTQ at 2 bits)",
        "value": round(ratio, 4), "unit": "x", "n_gpus": 1, "steps": 1, "warmup": 0, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 logits from the packed cache vs f32 exact", "data": "synthetic",
        "config": {"workload": "logit-mae", "kv_heads": h_kv, "q_heads": h_kv * g, "tokens": n},
        "results": out,
    }


def bench_window(args, n_sink=4, n_recent=128):
    """decode-8b-window: the Llama-3.1-8B-shaped layer decode (32768 cached tokens, K2V2,
    32 query / 8 KV heads) with fp16 sink and recent-token buffers: a step appends its
    token to the packed cache and to the fp16 ring, then attends (window split in the
    query-rotation launch, packed partials over positions [n_sink, L - n_recent), merge)."""
    import torch

    import packed_cache_attention_tq_amd as G

    w = build_workload(args.seed)
    plan, n, h_kv, g = w["plan"], w["n_ctx"], w["h_kv"], w["g"]
    dev = torch.device("cuda")
    k_all = torch.from_numpy(w["k"]).to(dev)
    v_all = torch.from_numpy(w["v"]).to(dev)
    base = G.PackedCache(plan, 1, n)
    G.gtq_quantize_append_chunk(plan, 0, base, k_all[: n - 1].contiguous(), v_all[: n - 1].contiguous(), 0, 0)
    win = G.WindowCache(plan, 1, n_sink, n_recent)
    pos = torch.cat([torch.arange(n_sink), torch.arange(n - 1 - n_recent, n - 1)]).to(dev)
    G.gtq_window_append(plan, 0, win, k_all[pos].contiguous(), v_all[pos].contiguous(),
                        torch.zeros(len(pos), dtype=torch.int32, device=dev), pos.to(torch.int64))
    caches = [base] + [base.clone() for _ in range(args.copies - 1)]
    k_new, v_new = k_all[n - 1: n].contiguous(), v_all[n - 1: n].contiguous()
    q = torch.from_numpy(w["q"]).to(dev)
    seq_len = torch.full((1,), n, dtype=torch.int32, device=dev)
    sidx = torch.zeros(1, dtype=torch.int32, device=dev)
    slot = torch.full((1,), n - 1, dtype=torch.int64, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(G.gtq_decode_window_workspace_bytes(plan, 1, n, args.chunk), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(128)
    stream = torch.cuda.current_stream()

    def step(i):
        c = caches[i % len(caches)]
        G.gtq_quantize_append(plan, 0, c, k_new, v_new, sidx, slot, stream=stream)
        G.gtq_window_append(plan, 0, win, k_new, v_new, sidx, slot, stream=stream)
        G.gtq_decode_attn_window(plan, 0, c, win, q, seq_len, n, scale, chunk=args.chunk, out=out, workspace=ws,
                                 stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    packed = n - n_sink - n_recent
    alg = packed * h_kv * base.sizes.bytes_per_token + (n_sink + n_recent) * h_kv * 512
    return {
        "metric": "packed-KV decode attention with fp16 sink + recent window: KV tokens/s",
        "value": round(n / (ms / 1e3), 1), "unit": "KV tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 (fp16 hi/lo split MFMA operands; binary16 window K/V)",
        "data": "synthetic",
        "config": {"workload": "decode-8b-window", "seq_len": n, "n_sink": n_sink, "n_recent": n_recent,
                   "k_bits_avg": w["k_budget"] / 64, "v_bits": w["v_bits"], "cache_copies": len(caches),
                   "step": "packed append + window append (1 token) + window decode (3 launches)"},
        "step_hbm_gbs": round(alg / (ms / 1e3) / 1e9, 1),
    }


def cpu_baseline(w, seed, min_seconds=10.0):
    """The fp64 oracle on the whole step (1-token encode + decode of all 32 query heads over
    every cached token, 8 KV heads), repeated until at least min_seconds of CPU time."""
    from oracle import gtq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    n, g, h_kv = w["n_ctx"], w["g"], w["h_kv"]
    heads, caches = [], []
    for h in range(h_kv):                                    # cache fill (untimed setup)
        inp = w["inps"][h]
        hp = O.HeadPlan(w["rates"][0, h], w["krot"][0][h], w["vrot"][0][h], w["v_bits"])
        heads.append(hp)
        caches.append(O.encode_kv(hp, inp["k"][: n - 1], inp["v"][: n - 1]))
    reps, t_total = 0, 0.0
    while t_total < min_seconds and reps < 100:
        t0 = time.perf_counter()
        for h in range(h_kv):
            inp, enc, hp = w["inps"][h], caches[h], heads[h]
            new = O.encode_kv(hp, inp["k"][n - 1: n], inp["v"][n - 1: n])
            kw = np.concatenate([enc["k_words"], new["k_words"]])
            kn = np.concatenate([enc["k_norms"], new["k_norms"]])
            vw = np.concatenate([enc["v_words"], new["v_words"]])
            vn = np.concatenate([enc["v_norms"], new["v_norms"]])
            O.decode_attention(hp, inp["q"][0], kw, kn, vw, vn, 1 / math.sqrt(128))
        t_total += time.perf_counter() - t0
        reps += 1
    t_step = t_total / reps
    return {"value": n / t_step, "unit": "KV tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole step (1-token encode + decode of {h_kv * g} query heads over {n} tokens, "
                      f"{h_kv} KV heads), {reps} step(s), {t_total:.1f} s",
            "seconds": round(t_total, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the decode shards by KV head or sequence with no exchange; see the design notes). "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch

    import packed_cache_attention_tq_amd as G
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a HIP device")
    G.lib()
    torch.cuda.set_device(0)
    if args.workload != "decode-8b":
        fn = {"decode-3b-36L": lambda: bench_decode_stack(args, "decode-3b-36L"),
              "decode-70b-b32": lambda: bench_decode_stack(args, "decode-70b-b32"),
              "append-32b": lambda: bench_append(args), "prefill-32b": lambda: bench_prefill(args),
              "logit-mae": lambda: bench_logit_mae(args),
              "decode-8b-window": lambda: bench_window(args)}[args.workload]
        print(json.dumps(fn()), flush=True)
        return
    t_setup = time.perf_counter()
    w = build_workload(args.seed, v_hadamard=args.v_hadamard)
    plan, n, h_kv, g = w["plan"], w["n_ctx"], w["h_kv"], w["g"]
    hq = h_kv * g
    dev = torch.device("cuda")
    k_all = torch.from_numpy(w["k"]).to(dev)
    v_all = torch.from_numpy(w["v"]).to(dev)
    if args.paged:
        n_pages = (n + args.paged - 1) // args.paged
        base = G.PagedCache(plan, 1, n_pages, args.paged, n_pages)
        base.block_table.copy_(torch.from_numpy(
            np.random.default_rng(args.seed).permutation(n_pages).astype(np.int32)[None]))
    else:
        base = G.PackedCache(plan, 1, n)
    # fill the cache: tokens 0..n-2 as one prompt; the step appends token n-1
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    G.gtq_quantize_append_chunk(plan, 0, base, k_all[: n - 1].contiguous(), v_all[: n - 1].contiguous(), 0, 0)
    t1.record()
    torch.cuda.synchronize()
    fill_ms = t0.elapsed_time(t1)
    sizes = base.sizes
    caches = [base] + [base.clone() for _ in range(args.copies - 1)]
    k_new = k_all[n - 1: n].contiguous()
    v_new = v_all[n - 1: n].contiguous()
    q = torch.from_numpy(w["q"]).to(dev)
    seq_len = torch.full((1,), n, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(G.gtq_decode_workspace_bytes(plan, 1, n, args.chunk), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(128)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        c = caches[i % len(caches)]
        if ev is None:  # the fused step: prepare + partials + merge in one library call
            G.gtq_decode_step(plan, 0, c, k_new, v_new, q, seq_len, n, scale, chunk=args.chunk, out=out,
                              workspace=ws, stream=stream)
            return
        # the same three launches as separate calls, with timing events around the partials:
        # append the step's token at slot n - 1 and rotate the queries (one launch)
        G.gtq_decode_prepare(plan, 0, c, k_new, v_new, q, seq_len, n, scale, ws, chunk=args.chunk, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        G.gtq_decode_attn_partials(plan, 0, c, seq_len, n, ws, chunk=args.chunk, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        G.gtq_decode_attn_merge(plan, 0, c, seq_len, n, out, ws, chunk=args.chunk, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f}s; cache fill (append of {n - 1} tokens x {h_kv} heads) "
        f"{fill_ms:.3f} ms; cache {base.nbytes() / 1e6:.2f} MB x {len(caches)} copies")

    # the partials kernel's duration is sampled with HIP events on every EVERY-th timed step
    # (events and separate calls on every step would make the loop host-bound)
    EVERY = 8
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range((args.steps + EVERY - 1) // EVERY)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i // EVERY] if i % EVERY == 0 else None)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    kern_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_per_step = total_ms / args.steps
    value = n / (ms_per_step / 1e3)

    # algorithmic bytes of one launch of the attention (partials) kernel: the packed
    # records of every attended (token, KV head), the key-group rotations, the queries
    krot_bytes = sum(sum(int(np.prod(m.shape)) for m in hh) for hh in w["krot"][0]) * 4
    alg_bytes = n * h_kv * sizes.bytes_per_token + krot_bytes + hq * 128 * 4
    kern_avg = float(kern_ms.mean())
    achieved = alg_bytes / (kern_avg / 1e3) / 1e9
    res = {
        "metric": "packed-KV decode attention: KV tokens/s + achieved HBM GB/s (% of peak)",
        "value": round(value, 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (fp16 hi/lo split MFMA operands, fp32 accumulation; u32 packed codes)",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b-shaped layer decode, batch 1, 32768 cached tokens, K2V2 "
                               "packed cache, 32 query / 8 KV heads, head_dim 128",
                   "global_batch": 1, "seq_len": n, "parallelism": "none (1 GPU)",
                   "k_bits_avg": w["k_budget"] / 64, "v_bits": w["v_bits"], "cache_copies": len(caches),
                   **({"page_tokens": args.paged} if args.paged else {}),
                   **({"v_rotation": "randomized Hadamard"} if args.v_hadamard else {})},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "kernel": partials_kernel_name(plan, 0, h_kv, w["v_bits"]),
                     "kernel_avg_us": round(kern_avg * 1e3, 3),
                     "kernel_p10_us": round(float(np.percentile(kern_ms, 10)) * 1e3, 3),
                     "kernel_p90_us": round(float(np.percentile(kern_ms, 90)) * 1e3, 3),
                     "alg_bytes_per_launch": int(alg_bytes)},
    }
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded slice ...")
        res["cpu_baseline"] = cpu_baseline(w, args.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
