"""Benchmark: packed-KV decode attention over a Block-GTQ (mixed-rate TQ-MSE) cache.

Default workload (the headline): one decode step of a Llama-3-70B-shaped model on one
GPU: 80 layers, 64 query / 8 KV heads, head_dim 128, batch 32 sequences with ragged
lengths uniform in [8192, 16384], K2V2 packed cache (about 28 GB resident). A step runs,
for every layer, the three launches of gtq_decode_step: prepare (append each sequence's
new token into the packed cache + rotate the queries), split-K packed decode partials,
log-sum-exp merge with the inverse value rotation. The 80 layers are captured in one
HIP graph; the graph is replayed --steps times after --warmup replays.

Inputs are seeded synthetic tensors with the pages' distributions, resident in HBM
before timing. The 80 layer caches are copies of one generated layer (same rates and
rotations; every layer reads its own copy from HBM).

Prints one JSON line: value = KV tokens/s (layers x cached positions attended per
second), roofline = the split-K partials kernel (algorithmic bytes of one launch, i.e.
the packed records of every attended (token, KV head), over its average duration,
measured with HIP events around a graph of back-to-back partials launches on the same
stream), cpu_baseline = the fp64 CPU oracle timed on a bounded slice of the same
workload on this host (all BLAS threads, and one thread).

Other workloads (--workload NAME) print one line each: decode-8b (Llama-3.1-8B layer,
batch 1, 32768 tokens, K2V2), decode-3b-36L (Qwen2.5-3B, 36 layers, batch 1, 131072
tokens, K3V3), append-32b, prefill-32b, logit-mae, decode-8b-window.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0   # dense fp16 MFMA
METRIC = "packed-KV decode attention: KV tokens/s + achieved HBM GB/s (% of peak)"
KERNEL_SRC = os.path.join(ROOT, "packed_cache_attention_tq_amd", "csrc", "gtq_device.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--chunk", type=int, default=0, help="split size (0 = automatic)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="CPU time of each oracle leg (all threads, one thread)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--workload", default="decode-70b-b32",
                   choices=["decode-70b-b32", "decode-8b", "decode-3b-36L", "append-32b", "prefill-32b",
                            "logit-mae", "decode-8b-window"])
    p.add_argument("--copies", type=int, default=32, help="decode-8b: layer caches the steps cycle through")
    p.add_argument("--norm-correct", action="store_true",
                   help="append-32b: plan with norm-corrected stored norms (GTQ_PLAN_NORM_CORRECT)")
    p.add_argument("--paged", type=int, default=0,
                   help="decode-8b: a paged cache of this many tokens per page (pool pages in shuffled order)")
    p.add_argument("--v-hadamard", action="store_true",
                   help="decode-8b: randomized Hadamard value rotations (applied as fast transforms)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="decode, append and prefill workloads: after timing, run a plain device copy "
                        "(torch.neg) of this many MiB three times: a kernel of known traffic that "
                        "calibrates the HBM byte counters")
    return p.parse_args()


# ---------------------------------------------------------------- measured traffic

def measured_traffic(name):
    """Calibrated HBM bytes per launch of a workload's dominant kernel from its committed
    counter summary profiles/<name>_traffic.txt, or None when the kernel source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    try:
        kv = dict(line.split(":", 1) for line in open(path).read().splitlines()
                  if ":" in line and not line.startswith("#"))
        sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
        if kv["kernel_source_sha256"].strip() != sha:
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def hbm_roofline(kernel, alg_bytes, avg_ms, traffic_name, extra=None):
    achieved = alg_bytes / (avg_ms / 1e3) / 1e9
    r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(traffic_name),
         "kernel": kernel, "kernel_avg_us": round(avg_ms * 1e3, 3), "alg_bytes_per_launch": int(alg_bytes)}
    if extra:
        r.update(extra)
    return r


# ---------------------------------------------------------------- plans and caches

def make_plan(seed, n_layers, h_kv, g, k_budget, v_bits, share_layer0=False, nc=False, v_hadamard=False):
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
            kr, vr = head_rotations(seed, l, h, G.gtq_head_layout_from_rates(r)["dim"], v_hadamard=v_hadamard)
            kl.append(kr)
            vl.append(vr)
        krot.append(kl)
        vrot.append(vl)
    plan = G.Plan(n_layers, h_kv, h_kv * g, k_budget, v_bits, rates, krot, np.array(vrot), norm_correct=nc)
    return plan, rates, krot, vrot


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


def graph_ms(fn, reps, warmup, per=1):
    """Capture fn (kernel launches on the current stream) in a HIP graph, replay it
    warmup + reps times; returns ms per replay / per (HIP events around the replays)."""
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
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps / per
    del g
    return ms


def partials_kernel_name(plan, layer, h_kv, v_bits, paged=False):
    """The decode partials kernel instance a decode of this layer launches: value bits, key
    words per lane (4 up to 8 key words, else 8) and the layer's specialized K-block slot
    counts (leading rate-1 and rate-4 blocks common to every head, at most 3 each and 4
    together; none for paged caches)."""
    lays = [plan.layout(layer, h) for h in range(h_kv)]
    kwl = 4 if lays[0]["k_words"] <= 8 else 8
    n1 = min((lay["dim"][0] + 31) // 32 if lay["rate"][0] == 1 else 0 for lay in lays)
    n4 = min((lay["dim"][-1] + 31) // 32 if lay["rate"][-1] == 4 else 0 for lay in lays)
    n1 = min(n1, 3)
    n4 = min(n4, 3, 4 - n1)
    if paged:
        n1 = n4 = 0
    return f"attn_decode_kernel<{v_bits}, {kwl}, {n1}, {n4}, {'true' if paged else 'false'}, false>"


# ---------------------------------------------------------------- decode workloads

DECODE = {
    # name: layers, KV heads, g, key budget, value bits, lengths, shared layer plan, cache copies
    "decode-70b-b32": dict(L=80, h_kv=8, g=8, kb=128, vb=2, batch=32, lens=(8192, 16384), share=True,
                           desc="Llama-3-70B-shaped decode step: 80 layers, 64 query / 8 KV heads, head_dim 128, "
                                "batch 32, ragged lengths U[8192, 16384], K2V2 packed cache"),
    "decode-3b-36L": dict(L=36, h_kv=2, g=8, kb=192, vb=3, batch=1, lens=131072, share=False,
                          desc="Qwen2.5-3B-shaped decode step: 36 layers, 16 query / 2 KV heads, head_dim 128, "
                               "batch 1, 131072 cached tokens per layer, K3V3 packed cache"),
    "decode-8b": dict(L=1, h_kv=8, g=4, kb=128, vb=2, batch=1, lens=32768, share=False,
                      desc="Llama-3.1-8B-shaped layer decode: 32 query / 8 KV heads, head_dim 128, batch 1, "
                           "32768 cached tokens, K2V2 packed cache"),
}


def bench_decode(args, name):
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import ragged_lengths

    c = DECODE[name]
    L, h_kv, g, kb, vb = c["L"], c["h_kv"], c["g"], c["kb"], c["vb"]
    if isinstance(c["lens"], tuple):
        lengths = ragged_lengths(args.seed, c["batch"], *c["lens"])
    else:
        lengths = np.full(c["batch"], c["lens"], np.int32)
    B = len(lengths)
    cap = int((lengths.max() + 31) // 32 * 32)
    t_setup = time.perf_counter()
    plan, rates, krot, vrot = make_plan(args.seed, L, h_kv, g, kb, vb, share_layer0=c["share"],
                                        v_hadamard=args.v_hadamard)
    # cache entries: one per layer; the single-layer shape cycles through --copies copies of
    # its layer (a step is one layer-step, the graph holds one step per copy)
    n_ent = L if L > 1 else args.copies
    caches, step_in = [], []
    for i in range(n_ent):
        li = i if L > 1 else 0
        if i > 0 and (c["share"] or L == 1):
            caches.append(caches[0].clone())
            step_in.append(step_in[0])
            continue
        if args.paged and L == 1:
            n_pages = (cap + args.paged - 1) // args.paged
            cc = G.PagedCache(plan, B, n_pages * B, args.paged, n_pages)
            perm = np.random.default_rng(args.seed).permutation(n_pages * B).astype(np.int32).reshape(B, n_pages)
            cc.block_table.copy_(torch.from_numpy(perm))
        else:
            cc = G.PackedCache(plan, B, cap)
        step_in.append(fill_layer(plan, li, cc, args.seed, h_kv, g, lengths))
        caches.append(cc)
    torch.cuda.synchronize()
    sl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    max_len = int(lengths.max())
    wsb = G.gtq_decode_workspace_bytes(plan, B, max_len, args.chunk)
    ws = [torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(n_ent)]
    outs = [torch.empty(B, h_kv * g, 128, device="cuda") for _ in range(n_ent)]
    scale = 1.0 / math.sqrt(128)
    log(f"{name}: setup {time.perf_counter() - t_setup:.1f}s, {n_ent} cache entries, "
        f"{sum(x.nbytes() for x in caches) / 1e9:.2f} GB")

    def layer_of(i):
        return i if L > 1 else 0

    def step():
        for i in range(n_ent):
            kn, vn, q = step_in[i]
            G.gtq_decode_step(plan, layer_of(i), caches[i], kn, vn, q, sl, max_len, scale, chunk=args.chunk,
                              out=outs[i], workspace=ws[i])

    def partials_only():
        for i in range(n_ent):
            G.gtq_decode_attn_partials(plan, layer_of(i), caches[i], sl, max_len, ws[i], chunk=args.chunk)

    per_step = n_ent if L == 1 else 1            # graph replays hold this many model steps
    ms = graph_ms(step, args.steps, args.warmup, per=per_step)
    part_ms = graph_ms(partials_only, args.steps, min(args.warmup, 2), per=n_ent)
    tok_per_step = (L if L > 1 else 1) * int(lengths.sum())
    bpt = caches[0].sizes.bytes_per_token
    alg_launch = int(lengths.sum()) * h_kv * bpt      # packed records one partials launch reads
    step_alg = (L if L > 1 else 1) * alg_launch
    res = {
        "metric": METRIC, "value": round(tok_per_step / (ms / 1e3), 1), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32 packed codes; f16 hi/lo MFMA operands, f32 accumulation",
        "data": "synthetic",
        "config": {"workload": c["desc"], "layers": L, "global_batch": B, "q_heads": h_kv * g, "kv_heads": h_kv,
                   "head_dim": 128, "seq_len": [int(lengths.min()), int(lengths.max())],
                   "k_bits_avg": kb / 64, "v_bits": vb, "parallelism": "none (1 GPU)",
                   "step": "one HIP graph: per layer prepare (token append + query rotation), partials, merge",
                   **({"cache_copies": n_ent} if L == 1 else {}),
                   **({"page_tokens": args.paged} if args.paged else {}),
                   **({"v_rotation": "randomized Hadamard"} if args.v_hadamard else {})},
        "roofline": hbm_roofline(partials_kernel_name(plan, 0, h_kv, vb, bool(args.paged)), alg_launch, part_ms, name,
                                 {"timing": "HIP events around a graph of back-to-back partials launches"}),
        "step_hbm_gbs": round(step_alg / (ms / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_alg / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
    }
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded slice ...")
        res["cpu_baseline"] = cpu_baseline_decode(args, c, lengths, rates, krot, vrot)
    return res


def calib_copy(mib):
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- CPU oracle baselines

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _two_legs(run_leg, seconds):
    """run_leg(seconds) -> (units, elapsed, detail) with all BLAS threads, then one."""
    from threadpoolctl import threadpool_limits
    out = {}
    u, t, det = run_leg(seconds)
    out["all"] = (u / t, _blas_threads(), det, t)
    with threadpool_limits(1):
        u, t, det = run_leg(seconds)
        out["one"] = (u / t, 1, det, t)
    return out


def cpu_baseline_decode(args, c, lengths, rates, krot, vrot):
    """The fp64 oracle on slices of one (layer, sequence, KV head): the step's one-token
    encode plus the decode of the KV head's g query heads over the sequence's cached
    tokens, repeated over sequences (and heads) until `seconds` of CPU time. KV tokens/s
    = attended positions / (KV heads x time), since a KV token holds all KV heads."""
    from gtq_inputs import head_inputs
    from oracle import gtq_oracle as O

    h_kv, g, vb = c["h_kv"], c["g"], c["vb"]
    scale = 1 / math.sqrt(128)
    order = [(b % len(lengths), (b // len(lengths) + b) % h_kv) for b in range(128)]
    prepared = {}

    def slice_inputs(b, h):        # generation and the cache's encode are setup (untimed, shared by the legs)
        if (b, h) not in prepared:
            n = int(lengths[b])
            inp = head_inputs(args.seed, 0, h, g, n, seq=b)
            hp = O.HeadPlan(rates[0, h], krot[0][h], vrot[0][h], vb)
            prepared[b, h] = (n, inp, hp, O.encode_kv(hp, inp["k"][: n - 1], inp["v"][: n - 1]))
        return prepared[b, h]

    def leg(seconds):
        done, t_total, slices = 0, 0.0, 0
        for b, h in order:
            n, inp, hp, enc = slice_inputs(b, h)
            t0 = time.perf_counter()
            new = O.encode_kv(hp, inp["k"][n - 1: n], inp["v"][n - 1: n])
            O.decode_attention(hp, inp["q"][0], np.concatenate([enc["k_words"], new["k_words"]]),
                               np.concatenate([enc["k_norms"], new["k_norms"]]),
                               np.concatenate([enc["v_words"], new["v_words"]]),
                               np.concatenate([enc["v_norms"], new["v_norms"]]), scale)
            t_total += time.perf_counter() - t0
            done += n
            slices += 1
            if t_total >= seconds:
                break
        return done / h_kv, t_total, f"{slices} slice(s) of 1 layer x 1 sequence x 1 KV head ({g} query heads)"

    legs = _two_legs(leg, args.cpu_seconds)
    v, cores, det, t = legs["all"]
    v1, _, det1, t1 = legs["one"]
    return {"value": round(v, 1), "unit": "KV tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{det}, encode of the step's token + decode, {t:.1f} s; extrapolated to the step by "
                      f"rate (the work is linear in tokens and heads)",
            "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(v1, 1), "cores": 1, "sample": f"{det1}, {t1:.1f} s"}}


# ---------------------------------------------------------------- append / prefill

def bench_append(args):
    """append-32b: Qwen2.5-32B-shaped chunk append, 4096-token chunks x 8 KV heads, K3V2,
    the 16 chunks of a 65536-token prompt in turn (one call = one chunk-layer)."""
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs_device

    h_kv, g, kb, vb, chunk, total = 8, 5, 192, 2, 4096, 65536
    plan, rates, krot, vrot = make_plan(args.seed, 1, h_kv, g, kb, vb, nc=args.norm_correct)
    cache = G.PackedCache(plan, 1, total)
    ks = torch.stack([head_inputs_device(args.seed, 0, h, g, total, "cuda", with_q=False)["k"] for h in range(h_kv)], 1)
    vs = torch.stack([head_inputs_device(args.seed, 0, h, g, total, "cuda", with_q=False)["v"] for h in range(h_kv)], 1)
    chunks = [(ks[m * chunk:(m + 1) * chunk].contiguous(), vs[m * chunk:(m + 1) * chunk].contiguous())
              for m in range(total // chunk)]

    def run():
        for m, (k, v) in enumerate(chunks):
            G.gtq_quantize_append_chunk(plan, 0, cache, k, v, 0, m * chunk)

    ms = graph_ms(run, max(1, args.steps // 4), 1, per=len(chunks))
    per_tok = 2 * 128 * 4 + cache.sizes.bytes_per_token  # fp32 key + value in, packed record out
    alg = chunk * h_kv * per_tok
    res = {
        "metric": "fused rotate+quantize+pack append: tokens/s + achieved HBM GB/s (% of peak)",
        "value": round(chunk / (ms / 1e3), 1), "unit": "tokens/s (x 8 KV heads)", "n_gpus": 1,
        "steps": max(1, args.steps // 4) * len(chunks), "warmup": len(chunks), "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 in; f16 hi/lo split MFMA rotation; u32 packed codes", "data": "synthetic",
        "config": {"workload": "Qwen2.5-32B-shaped prompt append: 4096-token chunk x 8 KV heads, K3V2 "
                               "(the 16 chunks of a 65536-token prompt in turn)",
                   "chunk_tokens": chunk, "kv_heads": h_kv, "k_bits_avg": kb / 64, "v_bits": vb, "prompt": total,
                   "norm_correct": bool(args.norm_correct)},
        "roofline": hbm_roofline("append_gemm_kernel", alg, ms, "append-32b",
                                 {"timing": "HIP events around a graph of the 16 chunk launches"}),
    }
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_append(args, rates, krot, vrot, kb, vb, chunk, h_kv, g)
    return res


def cpu_baseline_append(args, rates, krot, vrot, kb, vb, chunk, h_kv, g):
    """The oracle's encode + pack of one chunk of one KV head, repeated over heads until
    `seconds`; tokens/s of the whole 8-head chunk = tokens / (heads x time)."""
    from gtq_inputs import head_inputs
    from oracle import gtq_oracle as O

    def leg(seconds):
        done, t_total, n_sl = 0, 0.0, 0
        for i in range(64):
            h = i % h_kv
            inp = head_inputs(args.seed, 0, h, g, chunk)
            hp = O.HeadPlan(rates[0, h], krot[0][h], vrot[0][h], vb, nc=args.norm_correct)
            t0 = time.perf_counter()
            O.encode_kv(hp, inp["k"], inp["v"])
            t_total += time.perf_counter() - t0
            done += chunk
            n_sl += 1
            if t_total >= seconds:
                break
        return done / h_kv, t_total, f"{n_sl} chunk(s) of {chunk} tokens x 1 KV head"

    legs = _two_legs(leg, args.cpu_seconds)
    v, cores, det, t = legs["all"]
    v1, _, det1, t1 = legs["one"]
    return {"value": round(v, 1), "unit": "tokens/s (x 8 KV heads)", "cores": int(cores), "kind": "oracle",
            "sample": f"{det}, {t:.1f} s", "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(v1, 1), "cores": 1, "sample": f"{det1}, {t1:.1f} s"}}


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
    plan, rates, krot, vrot = make_plan(args.seed, 1, h_kv, g, kb, vb)
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
    tf = flop / (ms / 1e3) / 1e12
    res = {
        "metric": "chunked prefill attention over the packed cache: TFLOP/s",
        "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": n_steps,
        "warmup": 1, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 hi/lo split MFMA operands, f32 accumulation", "data": "synthetic",
        "config": {"workload": "Qwen2.5-32B-shaped chunked prefill: the last 4096-token chunk of a 65536-token "
                               "prompt, 40 query / 8 KV heads, K3V2", "chunk": chunk, "pos0": pos0,
                   "q_heads": h_kv * g, "kv_heads": h_kv, "k_bits_avg": kb / 64, "v_bits": vb},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_F16_TFLOPS, 4), "traffic": None,
                     "kernel": "gtq_prefill_attn (query rotation, partials, merge)",
                     "alg_flop_per_call": flop, "note": "algorithmic flop: 4 x 128 per visible (query, key) pair and "
                                                        "query head; the split operands execute twice that"},
    }
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(args, rates, krot, vrot, vb, g, pos0, chunk)
    return res


def cpu_baseline_prefill(args, rates, krot, vrot, vb, g, pos0, chunk):
    """The oracle's causal attention of a few query tokens of the chunk (one KV head, its g
    query heads) over the packed cache; TFLOP/s of the attention products."""
    from gtq_inputs import head_inputs
    from oracle import gtq_oracle as O

    total = pos0 + chunk
    inp = head_inputs(args.seed, 0, 0, g, total)
    hp = O.HeadPlan(rates[0, 0], krot[0][0], vrot[0][0], vb)
    enc = O.encode_kv(hp, inp["k"], inp["v"])
    q = np.random.default_rng(args.seed).standard_normal((chunk, g, 128)).astype(np.float32)

    def leg(seconds):
        fl, t_total, n = 0.0, 0.0, 0
        for t in range(chunk):
            p = pos0 + t
            t0 = time.perf_counter()
            O.decode_attention(hp, q[t], enc["k_words"], enc["k_norms"], enc["v_words"], enc["v_norms"],
                               1 / math.sqrt(128), length=p + 1)
            t_total += time.perf_counter() - t0
            fl += 4.0 * 128 * (p + 1) * g
            n += 1
            if t_total >= seconds:
                break
        return fl / 1e12, t_total, f"{n} query token(s) x {g} query heads of one KV head over ~{total} positions"

    legs = _two_legs(leg, args.cpu_seconds)
    v, cores, det, t = legs["all"]
    v1, _, det1, t1 = legs["one"]
    return {"value": round(v, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{det}, {t:.1f} s", "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(v1, 6), "cores": 1, "sample": f"{det1}, {t1:.1f} s"}}


# ---------------------------------------------------------------- diagnostics

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
    32 query / 8 KV heads) with fp16 sink and recent-token buffers: a step
    (gtq_decode_step_window) appends its token to the packed cache and to the fp16 ring
    and rotates the queries in one launch, whose window-split workgroups also write the
    token to the ring first; then the packed partials over positions [n_sink, L - n_recent)
    and the merge."""
    import torch

    import packed_cache_attention_tq_amd as G
    from gtq_inputs import head_inputs, head_rotations

    h_kv, g, n, kb, vb = 8, 4, 32768, 128, 2
    plan, rates, krot, vrot = make_plan(args.seed, 1, h_kv, g, kb, vb)
    dev = torch.device("cuda")
    inps = [head_inputs(args.seed, 0, h, g, n) for h in range(h_kv)]
    k_all = torch.from_numpy(np.stack([i["k"] for i in inps], axis=1)).to(dev)
    v_all = torch.from_numpy(np.stack([i["v"] for i in inps], axis=1)).to(dev)
    base = G.PackedCache(plan, 1, n)
    G.gtq_quantize_append_chunk(plan, 0, base, k_all[: n - 1].contiguous(), v_all[: n - 1].contiguous(), 0, 0)
    win = G.WindowCache(plan, 1, n_sink, n_recent)
    pos = torch.cat([torch.arange(n_sink), torch.arange(n - 1 - n_recent, n - 1)]).to(dev)
    G.gtq_window_append(plan, 0, win, k_all[pos].contiguous(), v_all[pos].contiguous(),
                        torch.zeros(len(pos), dtype=torch.int32, device=dev), pos.to(torch.int64))
    caches = [base] + [base.clone() for _ in range(args.copies - 1)]
    k_new, v_new = k_all[n - 1: n].contiguous(), v_all[n - 1: n].contiguous()
    q = torch.from_numpy(np.concatenate([i["q"][0] for i in inps])[None]).to(dev)
    seq_len = torch.full((1,), n, dtype=torch.int32, device=dev)
    sidx = torch.zeros(1, dtype=torch.int32, device=dev)
    slot = torch.full((1,), n - 1, dtype=torch.int64, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(G.gtq_decode_window_workspace_bytes(plan, 1, n, args.chunk), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(128)

    def run():
        for c in caches:
            G.gtq_decode_step_window(plan, 0, c, win, k_new, v_new, q, seq_len, n, scale, chunk=args.chunk, out=out,
                                     workspace=ws)

    def attend():
        for c in caches:
            G.gtq_decode_attn_window(plan, 0, c, win, q, seq_len, n, scale, chunk=args.chunk, out=out, workspace=ws)

    ms = graph_ms(run, args.steps, args.warmup, per=len(caches))
    att_ms = graph_ms(attend, args.steps, min(args.warmup, 2), per=len(caches))
    packed = n - n_sink - n_recent
    alg = packed * h_kv * base.sizes.bytes_per_token + (n_sink + n_recent) * h_kv * 512
    res = {
        "metric": "packed-KV decode attention with fp16 sink + recent window: KV tokens/s",
        "value": round(n / (ms / 1e3), 1), "unit": "KV tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32 packed codes; f16 hi/lo MFMA operands; binary16 window K/V",
        "data": "synthetic",
        "config": {"workload": "decode-8b-window", "seq_len": n, "n_sink": n_sink, "n_recent": n_recent,
                   "k_bits_avg": kb / 64, "v_bits": vb, "cache_copies": len(caches),
                   "step": "gtq_decode_step_window: prepare (packed append, window append + window split, "
                           "query rotation), partials, merge (3 launches)"},
        "roofline": hbm_roofline("gtq_decode_attn_window (window split + query rotation, partials, merge)", alg,
                                 att_ms, "decode-8b-window",
                                 {"timing": "HIP events around a graph of back-to-back gtq_decode_attn_window "
                                            "calls (3 launches each)"}),
        "step_hbm_gbs": round(alg / (ms / 1e3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded slice ...")
        res["cpu_baseline"] = cpu_baseline_window(args, rates, krot, vrot, h_kv, g, n, kb, vb, n_sink, n_recent)
    return res


def cpu_baseline_window(args, rates, krot, vrot, h_kv, g, n, kb, vb, n_sink, n_recent):
    """The fp64 oracle on one KV head of the step: encode of the step's token, then the
    window decode of its g query heads over n positions (packed records + binary16 window),
    repeated over the KV heads until `seconds` of CPU time; KV tokens/s = positions /
    (KV heads x time)."""
    from gtq_inputs import head_inputs
    from oracle import gtq_oracle as O

    scale = 1 / math.sqrt(128)
    prepared = {}

    def head(h):
        if h not in prepared:
            inp = head_inputs(args.seed, 0, h, g, n)
            hp = O.HeadPlan(rates[0, h], krot[0][h], vrot[0][h], vb)
            prepared[h] = (inp, hp, O.encode_kv(hp, inp["k"][: n - 1], inp["v"][: n - 1]))
        return prepared[h]

    def leg(seconds):
        done, t_total, slices = 0, 0.0, 0
        for i in range(64):
            inp, hp, enc = head(i % h_kv)
            t0 = time.perf_counter()
            new = O.encode_kv(hp, inp["k"][n - 1: n], inp["v"][n - 1: n])
            O.decode_attention_window(hp, inp["q"][0], np.concatenate([enc["k_words"], new["k_words"]]),
                                      np.concatenate([enc["k_norms"], new["k_norms"]]),
                                      np.concatenate([enc["v_words"], new["v_words"]]),
                                      np.concatenate([enc["v_norms"], new["v_norms"]]), inp["k"], inp["v"],
                                      n_sink, n_recent, scale, n)
            t_total += time.perf_counter() - t0
            done += n
            slices += 1
            if t_total >= seconds:
                break
        return done / h_kv, t_total, f"{slices} slice(s) of 1 KV head ({g} query heads) x {n} positions"

    legs = _two_legs(leg, args.cpu_seconds)
    v, cores, det, t = legs["all"]
    v1, _, det1, t1 = legs["one"]
    return {"value": round(v, 1), "unit": "KV tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{det}, encode of the step's token + window decode, {t:.1f} s; extrapolated to the step "
                      f"by rate (the work is linear in heads)",
            "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(v1, 1), "cores": 1, "sample": f"{det1}, {t1:.1f} s"}}


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
    if args.workload in DECODE:
        res = bench_decode(args, args.workload)
    else:
        res = {"append-32b": lambda: bench_append(args), "prefill-32b": lambda: bench_prefill(args),
               "logit-mae": lambda: bench_logit_mae(args),
               "decode-8b-window": lambda: bench_window(args)}[args.workload]()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
