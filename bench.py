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


def build_workload(seed, n_ctx=32768, h_kv=8, g=4, k_budget=128, v_bits=2):
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
        kr, vr = head_rotations(seed, 0, h, lay["dim"])
        krot[0].append(kr)
        vrot[0].append(vr)
        inps.append(inp)
    plan = G.Plan(1, h_kv, h_kv * g, k_budget, v_bits, rates, krot, np.array(vrot))
    k = np.stack([i["k"] for i in inps], axis=1)          # [n_ctx+1, H, 128]
    v = np.stack([i["v"] for i in inps], axis=1)
    q = np.concatenate([i["q"][0] for i in inps])[None]   # [1, 32, 128]
    return dict(plan=plan, k=k, v=v, q=q, rates=rates, krot=krot, vrot=vrot, inps=inps,
                n_ctx=n_ctx, h_kv=h_kv, g=g, k_budget=k_budget, v_bits=v_bits)


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
    t_setup = time.perf_counter()
    w = build_workload(args.seed)
    plan, n, h_kv, g = w["plan"], w["n_ctx"], w["h_kv"], w["g"]
    hq = h_kv * g
    dev = torch.device("cuda")
    k_all = torch.from_numpy(w["k"]).to(dev)
    v_all = torch.from_numpy(w["v"]).to(dev)
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

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
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
                   "k_bits_avg": w["k_budget"] / 64, "v_bits": w["v_bits"], "cache_copies": len(caches)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "attn_partials_kernel<2, 4>", "kernel_avg_us": round(kern_avg * 1e3, 3),
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
