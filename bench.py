#!/usr/bin/env python3
"""Throughput of one CSA2 decode stack step on one MI355X.

Workload (default decoder_stack_128k): 16 sequences, each with its own shared
global KV of 131072 entries (FP4 main KV + FP8 indexer K), 20 layers planned
F RRR X RRR X RRR X RRR X RRR (1 Full, 4 Reindex, 15 Reuse), 64 query heads,
top-512, pool of 2048 blocks x 8, every layer with its own FP8 128-token
window.  One step = the write path of the new token (FP4 main KV entry after
RoPE + FP8 indexer key, for every sequence) + the Full-layer scan, block pool
and top-K + 4 Reindex selections + 20 sparse attentions.  All inputs are
resident in HBM before timing; `cache_sets` identical copies of the caches at
different addresses are used in rotation so that consecutive steps cannot be
served from the 256 MB last-level cache.

Prints ONE JSON line on stdout (progress goes to stderr):
  value       = sequences (decode queries) per second through the whole stack
  rooflines   = per timed kernel: algorithmic bytes per launch over its mean
                duration from HIP events recorded around its own dispatch,
                against 8 TB/s -- the sparse attention (launched once per
                layer) and the Full-layer scan (the only kernel whose work
                grows with context)
  roofline    = the entry of `rooflines` that takes the most time per step;
                `traffic` = measured HBM bytes per launch (FETCH_SIZE +
                WRITE_SIZE counters scaled by a copy kernel of known size, from
                profiles/traffic.json), or null when those counters were taken
                on a different version of the kernel's source
  cpu_baseline= the CPU oracle on a bounded sample of the same workload
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "CSA2 decode queries/s per layer stack at 128K ctx; achieved HBM GB/s vs peak"
# the arithmetic the path computes in: fp32 indexer scores (sequential FMA
# chains over E4M3 / E2M1 values), attention on fp16 MFMA with fp32
# accumulation (dequantised FP4 / FP8 operands exact in fp16, q split into fp16
# hi + lo), fp32 online softmax; storage is FP4 (E2M1 + E4M3 scales) and FP8
DTYPE = "f32+f16mfma"
DTYPE_DETAIL = ("indexer scores fp32 (exact-order FMA chains over E4M3/E2M1 values); attention "
                "fp16 MFMA with fp32 accumulate (FP4/FP8 operands exact in fp16, q as fp16 hi+lo "
                "= 22 bits), fp32 online softmax; cache storage FP4 E2M1+E4M3 scales, FP8 E4M3")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decoder_stack_128k")
    p.add_argument("--cache-sets", type=int, default=3)
    p.add_argument("--no-graph", action="store_true", help="time eager launches, no HIP graph")
    p.add_argument("--cpu-seqs", type=int, default=0,
                   help="sequences in the CPU-oracle sample (0 = one whole batch)")
    p.add_argument("--skip-cpu-baseline", action="store_true")
    p.add_argument("--contexts", default="4096,16384,65536,131072,262144,1048576",
                   help="model_step workload: context lengths (tokens) of the sweep")
    p.add_argument("--batches", default="1,4,16,64,256,1024",
                   help="attn_batch_sweep workload: batch sizes (sequences, one query each)")
    p.add_argument("--model-batch", type=int, default=4,
                   help="model_step workload: sequences per step")
    p.add_argument("--replay-tokens", type=int, default=0,
                   help="replay_stack_128k workload: tokens per replay chunk (default 128; 2560 "
                        "is the exact replay of a 20-layer stack)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the measurements beside the headline workload (copy and read "
                        "ceilings, large-batch attention, the 1M-entry stack)")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="also run one device-to-device copy of this many MiB (a known-size "
                        "kernel for scaling hardware byte counters)")
    return p.parse_args()


# --------------------------------------------------------------------------- bytes
def attn_bytes(n_sel, n_swa, H):
    """Algorithmic bytes of one query's attention in one layer: 144 B per
    selected FP4 entry, 264 B per window token (2 x 128 E4M3 + 2 fp32 scales),
    fp32 q and out."""
    return 144 * n_sel + 264 * n_swa + 2 * H * 128 * 4


def percentile(sorted_vals, f):
    """Nearest-rank percentile of an ascending list."""
    i = min(len(sorted_vals) - 1, max(0, int(round(f * (len(sorted_vals) - 1)))))
    return sorted_vals[i]


def idx_key_bytes(wl):
    """Bytes of one position's indexer key: FP8 (64 codes + fp32 sigma) or FP4
    (32 code bytes + 4 E4M3 scales)."""
    return 36 if wl.idx_fp4 else 68


def step_bytes(wl):
    """Algorithmic HBM bytes of one stack step (all queries)."""
    B, N, H = wl.B, wl.n_ent, wl.H
    key = idx_key_bytes(wl)
    scan = key * N * B
    n_x = wl.plan.count("X")
    reindex = n_x * key * min(wl.pool_blocks * 8, N) * B
    attn = len(wl.plan) * B * attn_bytes(min(wl.topk, N), 128, H)
    write = B * (2 * 128 * 4 + 144 + 64 * 4 + 68)
    return scan + reindex + attn + write, scan


# --------------------------------------------------------------------------- GPU side
class StepSet:
    """One complete, independent copy of a step's device inputs."""

    def __init__(self, csa2, DecodeStack, cache, wl, dev_inputs):
        self.cache, self.ratio = cache, wl.ratio
        self.stack = DecodeStack(cache, wl.plan, wl.B, wl.H, topk=wl.topk,
                                 pool_blocks=wl.pool_blocks)
        self.inp = {k: v.clone() for k, v in dev_inputs.items()}
        self.csa2 = csa2

    def run(self, scan_timer=None, attn_timer=None, index_events=None):
        i = self.inp
        # write path of the new token of every sequence (position n_ent - 1),
        # in one launch: its FP4 record, its indexer key projected on the
        # device from its K, and every layer's window token at its ring slot
        self.stack.write(i["k_new"], i["v_new"], i["rows_new"], i["proj"], i["win_k"],
                         i["win_v"], i["win_rows"], i["swk"], i["swv"], i["sks"], i["svs"],
                         ratio=self.ratio, rope_cs=i.get("rope_new"))
        self.stack.step(i["iq"], i["iw"], i["n_vis"], i["q"], i["swk"], i["swv"], i["sks"],
                        i["svs"], i["swa_len"], scan_timer=scan_timer, attn_timer=attn_timer,
                        index_events=index_events)


def build_sets(args, wl, inp):
    import numpy as np
    import torch

    import compressed_kv_cache_decode_amd as csa2
    from compressed_kv_cache_decode_amd.stack import DecodeStack

    B, N = wl.B, wl.n_ent
    cap = (N + 63) // 64 * 64
    log(f"writing the caches with the library: B={B} entries={N} ratio={wl.ratio}")
    cache0 = csa2.Cache(B, cap, idx_fp4=wl.idx_fp4)
    for b in range(B):
        rows = cache0.rows(b, np.arange(N))
        k = torch.from_numpy(inp.k_tok[b]).cuda()
        v = torch.from_numpy(inp.v_tok[b]).cuda()
        cs = torch.from_numpy(csa2.rope_table(np.arange(N))).cuda() if wl.ratio == 1 else None
        csa2.quant_fp4(k, v, cache0.kv_codes, cache0.kv_scales, ratio=wl.ratio, rope_cs=cs,
                       dst_rows=rows)
        ik = torch.from_numpy(inp.idx_k[b]).cuda()
        if wl.idx_fp4:
            csa2.quant_idx_fp4(ik, cache0.ik_codes, cache0.ik_scales4, dst_rows=rows)
        else:
            csa2.quant_fp8(ik, cache0.ik_codes, cache0.ik_sigma, layout=csa2.FP8_IDX_TILED,
                           dst_rows=rows)
        del k, v, cs
    L = len(wl.plan)
    swk = torch.empty((L, B, 128, 128), dtype=torch.uint8, device="cuda")
    swv = torch.empty_like(swk)
    sks = torch.empty((L, B, 128), dtype=torch.float32, device="cuda")
    svs = torch.empty_like(sks)
    csa2.quant_fp8(torch.from_numpy(inp.swa_k.reshape(-1, 128)).cuda(), swk, sks)
    csa2.quant_fp8(torch.from_numpy(inp.swa_v.reshape(-1, 128)).cuda(), swv, svs)
    last = N - 1
    tok = last * wl.ratio  # the new token (pair) of every sequence
    slot = (tok + wl.ratio - 1) % 128  # window ring slot of the newest token
    if wl.ratio == 1:
        k_new, v_new = inp.k_tok[:, last], inp.v_tok[:, last]
    else:  # the newest pair is re-averaged by the write path
        k_new = inp.k_tok[:, tok:tok + 2].reshape(-1, 128)
        v_new = inp.v_tok[:, tok:tok + 2].reshape(-1, 128)
    dev_inputs = {
        "k_new": torch.from_numpy(np.ascontiguousarray(k_new)).cuda(),
        "v_new": torch.from_numpy(np.ascontiguousarray(v_new)).cuda(),
        "proj": torch.from_numpy(inp.proj).cuda(),
        # the newest token's window row of every layer, at its ring slot
        "win_k": torch.from_numpy(np.ascontiguousarray(inp.swa_k[:, :, slot].reshape(-1, 128))).cuda(),
        "win_v": torch.from_numpy(np.ascontiguousarray(inp.swa_v[:, :, slot].reshape(-1, 128))).cuda(),
        "win_rows": torch.from_numpy(((np.arange(L)[:, None] * B + np.arange(B)[None, :]) * 128
                                      + slot).reshape(-1).astype(np.int64)).cuda(),
        "rope_new": (torch.from_numpy(csa2.rope_table(np.full(B, last))).cuda()
                     if wl.ratio == 1 else None),
        "rows_new": torch.arange(B, dtype=torch.int64, device="cuda") * cap + last,
        "iq": torch.from_numpy(inp.iq[:, :, None]).cuda(),
        "iw": torch.from_numpy(inp.iw[:, :, None]).cuda(),
        "n_vis": torch.full((B, 1), N, dtype=torch.int32, device="cuda"),
        "q": torch.from_numpy(inp.q).cuda(),
        "swk": swk, "swv": swv, "sks": sks, "svs": svs,
        "swa_len": torch.from_numpy(inp.swa_len).cuda(),
    }
    if dev_inputs["rope_new"] is None:
        del dev_inputs["rope_new"]
    sets = []
    for s in range(args.cache_sets):
        cache = cache0 if s == 0 else csa2.Cache(B, cap, idx_fp4=wl.idx_fp4)
        if s:
            for name in ("kv_codes", "kv_scales", "ik_codes"):
                getattr(cache, name).copy_(getattr(cache0, name))
            cache.ik_aux.copy_(cache0.ik_aux)
        ss = StepSet(csa2, DecodeStack, cache, wl, dev_inputs)
        if "rope_new" not in ss.inp:
            ss.inp["rope_new"] = None
        sets.append(ss)
    torch.cuda.synchronize()
    log(f"{len(sets)} cache sets of {cache0.nbytes / 1e6:.1f} MB each")
    return csa2, sets


def time_gpu(args, wl, csa2, sets):
    import torch
    stream = torch.cuda.Stream()
    graphs = None
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, 1)):
            sets[i % len(sets)].run()
        torch.cuda.synchronize()
        if not args.no_graph:
            graphs = []
            for s in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    s.run()
                graphs.append(g)
            for i in range(args.warmup):
                graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()

        log(f"timing {args.steps} steps ({'graph replay' if graphs else 'eager'})")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                sets[i % len(sets)].run()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

        # the same replays once more with an event between consecutive steps:
        # the distribution of single-step times
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                sets[i % len(sets)].run()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))

        # per-kernel durations, HIP events recorded around each kernel's own
        # dispatch.  A bounded spin kernel first lets the host queue the eager
        # launches ahead of the GPU, so that they run back to back as in the
        # graph replays instead of waiting for the host between kernels
        timer = csa2.KernelTimer(args.steps)
        attn_timer = csa2.KernelTimer(args.steps * len(wl.plan))
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(3e6 * args.steps))  # about 1.2 ms of spinning per step
        index_events = []
        for i in range(args.steps):
            sets[i % len(sets)].run(scan_timer=timer, attn_timer=attn_timer,
                                    index_events=index_events)
        torch.cuda.synchronize()
        full_ms = [a.elapsed_time(b) for m, a, b in index_events if m == "F"]
        reindex_ms = [a.elapsed_time(b) for m, a, b in index_events if m == "X"]
        scan_ms = timer.durations_ms()
        attn_ms = attn_timer.durations_ms()
        timer.close()
        attn_timer.close()
        t1 = time.perf_counter()
        for i in range(args.steps):
            sets[i % len(sets)].run()
        torch.cuda.synchronize()
        eager_elapsed = time.perf_counter() - t1
    return elapsed, {"scan": scan_ms, "attn": attn_ms, "step": step_ms, "full_call": full_ms,
                     "reindex_call": reindex_ms}, eager_elapsed


# --------------------------------------------------------------------------- replay chunk
def run_chunk_bench(args, wl):
    """Bounded-replay chunk (one layer): the chunk's 128 new entries through the
    write path (RoPE + FP4, FP8 indexer keys, FP8 window), the Full-layer top-512
    of every query over positions [0, N-128+i], and the chunk attention."""
    import numpy as np
    import torch

    import compressed_kv_cache_decode_amd as csa2
    from compressed_kv_cache_decode_amd import synth

    inp = synth.chunk_inputs(wl)
    B, N, Q, H = wl.B, wl.n_ent, wl.Q, wl.H
    cap = (N + 63) // 64 * 64
    log(f"chunk: writing {args.cache_sets} cache sets of {N} entries")
    pos_new = np.arange(N - Q, N)
    dev_in = {
        "k_new": torch.from_numpy(np.ascontiguousarray(inp.k_tok[0, N - Q:])).cuda(),
        "v_new": torch.from_numpy(np.ascontiguousarray(inp.v_tok[0, N - Q:])).cuda(),
        "rope_new": torch.from_numpy(csa2.rope_table(pos_new)).cuda(),
        "proj": torch.from_numpy(inp.proj).cuda(),
        "swa_k": torch.from_numpy(inp.swa_k.reshape(-1, 128)).cuda(),
        "swa_v": torch.from_numpy(inp.swa_v.reshape(-1, 128)).cuda(),
        "iq": torch.from_numpy(inp.iq).cuda(), "iw": torch.from_numpy(inp.iw).cuda(),
        "n_vis": torch.from_numpy(np.arange(N - Q + 1, N + 1, dtype=np.int32)[None]).cuda(),
        "q": torch.from_numpy(inp.q).cuda(),
    }
    caches = []
    for s_ in range(args.cache_sets):
        cache = csa2.Cache(B, cap, idx_fp4=wl.idx_fp4)
        if s_ == 0:
            pre = np.arange(N - Q)
            csa2.quant_fp4(torch.from_numpy(inp.k_tok[0, :N - Q]).cuda(),
                           torch.from_numpy(inp.v_tok[0, :N - Q]).cuda(), cache.kv_codes,
                           cache.kv_scales, rope_cs=torch.from_numpy(csa2.rope_table(pre)).cuda(),
                           dst_rows=cache.rows(0, pre))
            ik = torch.from_numpy(inp.idx_k[0, :N - Q]).cuda()
            if wl.idx_fp4:
                csa2.quant_idx_fp4(ik, cache.ik_codes, cache.ik_scales4, dst_rows=cache.rows(0, pre))
            else:
                csa2.quant_fp8(ik, cache.ik_codes, cache.ik_sigma, layout=csa2.FP8_IDX_TILED,
                               dst_rows=cache.rows(0, pre))
        else:
            for name in ("kv_codes", "kv_scales", "ik_codes"):
                getattr(cache, name).copy_(getattr(caches[0], name))
            cache.ik_aux.copy_(caches[0].ik_aux)
        caches.append(cache)
    rows_new = caches[0].rows(0, pos_new)
    swk = torch.empty((B, Q, 128), dtype=torch.uint8, device="cuda")
    swv = torch.empty_like(swk)
    sks = torch.empty((B, Q), dtype=torch.float32, device="cuda")
    svs = torch.empty_like(sks)
    tk = torch.empty((B, Q, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Q, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, H), dtype=torch.float32, device="cuda")
    ws = csa2.alloc_workspace(csa2.workspace_size(csa2.OP_INDEX_FULL, B, Q, cap, wl.topk, 0, 0))
    d = dev_in

    def step(cache, scan_timer=None):
        # the chunk's 128 entries (RoPE + FP4), their indexer keys projected
        # on the device from their K, and the window's K and V, in one launch
        csa2.write_entries(d["k_new"], d["v_new"], cache.kv_codes, cache.kv_scales,
                           rope_cs=d["rope_new"], dst_rows=rows_new, idx_proj=d["proj"],
                           ik_codes=cache.ik_codes, ik_sigma=cache.ik_sigma,
                           ik_scales4=cache.ik_scales4,
                           fp8_jobs=[dict(x=d["swa_k"], codes=swk, sigma=sks),
                                     dict(x=d["swa_v"], codes=swv, sigma=svs)])
        csa2.index_full(cache, d["iq"], d["iw"], d["n_vis"], tk, None, topk=wl.topk,
                        pool_blocks=0, ws=ws, scan_timer=scan_timer)
        csa2.sparse_attn_chunk(d["q"], cache, tk, swk, swv, sks, svs, out, lse)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, 1)):
            step(caches[i % len(caches)])
        torch.cuda.synchronize()
        graphs = []
        if not args.no_graph:
            for c in caches:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(c)
                graphs.append(g)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                step(caches[i % len(caches)])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        timer = csa2.KernelTimer(args.steps)
        if hasattr(torch.cuda, "_sleep"):  # queue the eager launches ahead of the GPU
            torch.cuda._sleep(int(3e6 * args.steps))
        for i in range(args.steps):
            step(caches[i % len(caches)], scan_timer=timer)
        torch.cuda.synchronize()
        scan_ms = timer.durations_ms()
        timer.close()
    ms_per_step = elapsed / args.steps * 1e3
    scan_mean = sum(scan_ms) / len(scan_ms)
    # the chunk's scan is a dense (queries x 256) . (256 x positions) contraction
    # on fp16 MFMA: 4 heads x 64 multiply-adds per (query, position) pair,
    # counted as 2 flops, against the dense fp16 matrix peak
    flops = 2.0 * 256 * Q * N
    scan_tfs = flops / (scan_mean * 1e-3) / 1e12
    peak = 2500.0
    rl = {"bound": "mfma", "achieved": round(scan_tfs, 2), "peak": peak, "unit": "TFLOP/s",
          "frac": round(scan_tfs / peak, 4), "traffic": load_traffic(wl.name).get("k_scan_mma"),
          "kernel": "k_scan_mma (Full-layer indexer bounds of 128 chunk queries, fp16 MFMA"
                    + (", FP4 keys)" if wl.idx_fp4 else ")"),
          "flops_per_launch": flops, "mean_us": round(scan_mean * 1e3, 2)}
    return {
        "metric": "CSA2 bounded-replay chunk queries/s (128 replayed tokens over 128K entries, one layer)",
        "value": round(Q * B * args.steps / elapsed, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": wl.name, "sequences": B, "entries": N, "queries": Q, "heads": H,
                   "indexer_key": "fp4" if wl.idx_fp4 else "fp8",
                   "topk": wl.topk, "cache_sets": args.cache_sets,
                   "launch": "eager" if args.no_graph else "hip-graph"},
        "roofline": rl,
    }


# --------------------------------------------------------------------------- replay chunk stack
def run_chunk_stack_bench(args, wl):
    """Bounded-replay chunk through the whole decoder stack: the chunk's 128
    new entries (RoPE + FP4), their indexer keys and every layer's window K and
    V in one write launch, then the 20 layers (Full with per-token pools, 4
    Reindex, 15 Reuse), each with the chunk attention of its 128 tokens."""
    import numpy as np
    import torch

    import compressed_kv_cache_decode_amd as csa2
    from compressed_kv_cache_decode_amd import synth
    from compressed_kv_cache_decode_amd.stack import ChunkStack

    Q = args.replay_tokens or wl.Q  # 128: bounded replay; 2560 = 20 x 128: exact replay
    inp = synth.chunk_stack_inputs(wl, Q=Q)
    B, N, H, L = wl.B, wl.n_ent, wl.H, len(wl.plan)
    cap = (N + 63) // 64 * 64
    log(f"chunk stack: writing {args.cache_sets} cache sets of {N} entries, plan {wl.plan}")
    caches = []
    for s_ in range(args.cache_sets):
        cache = csa2.Cache(B, cap)
        if s_ == 0:
            pre = np.arange(N - Q)
            csa2.quant_fp4(torch.from_numpy(inp.k_tok[0, :N - Q]).cuda(),
                           torch.from_numpy(inp.v_tok[0, :N - Q]).cuda(), cache.kv_codes,
                           cache.kv_scales, rope_cs=torch.from_numpy(csa2.rope_table(pre)).cuda(),
                           dst_rows=cache.rows(0, pre))
            csa2.quant_fp8(torch.from_numpy(inp.idx_k[0, :N - Q]).cuda(), cache.ik_codes,
                           cache.ik_sigma, layout=csa2.FP8_IDX_TILED, dst_rows=cache.rows(0, pre))
        else:
            for name in ("kv_codes", "kv_scales", "ik_codes", "ik_sigma"):
                getattr(cache, name).copy_(getattr(caches[0], name))
        caches.append(cache)
    d = {
        "k_new": torch.from_numpy(np.ascontiguousarray(inp.k_tok[0, N - Q:])).cuda(),
        "v_new": torch.from_numpy(np.ascontiguousarray(inp.v_tok[0, N - Q:])).cuda(),
        "rope_new": torch.from_numpy(csa2.rope_table(inp.positions)).cuda(),
        "proj": torch.from_numpy(inp.proj).cuda(),
        "swa_k": torch.from_numpy(inp.swa_k.reshape(-1, 128)).cuda(),
        "swa_v": torch.from_numpy(inp.swa_v.reshape(-1, 128)).cuda(),
        "iq": torch.from_numpy(inp.iq).cuda(), "iw": torch.from_numpy(inp.iw).cuda(),
        "n_vis": torch.from_numpy(np.arange(N - Q + 1, N + 1, dtype=np.int32)[None]).cuda(),
        "q": torch.from_numpy(inp.q).cuda(),
    }
    rows_new = caches[0].rows(0, inp.positions)
    swk = torch.empty((L, B, Q, 128), dtype=torch.uint8, device="cuda")
    swv = torch.empty_like(swk)
    sks = torch.empty((L, B, Q), dtype=torch.float32, device="cuda")
    svs = torch.empty_like(sks)
    stacks = [ChunkStack(c, wl.plan, B, Q, H, topk=wl.topk, pool_blocks=wl.pool_blocks)
              for c in caches]

    def step(i, scan_timer=None):
        cache, st = caches[i], stacks[i]
        csa2.write_entries(d["k_new"], d["v_new"], cache.kv_codes, cache.kv_scales,
                           rope_cs=d["rope_new"], dst_rows=rows_new, idx_proj=d["proj"],
                           ik_codes=cache.ik_codes, ik_sigma=cache.ik_sigma,
                           fp8_jobs=[dict(x=d["swa_k"], codes=swk, sigma=sks),
                                     dict(x=d["swa_v"], codes=swv, sigma=svs)])
        st.step(d["iq"], d["iw"], d["n_vis"], d["q"], swk, swv, sks, svs, scan_timer=scan_timer)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, 1)):
            step(i % len(caches))
        torch.cuda.synchronize()
        graphs = []
        if not args.no_graph:
            for i in range(len(caches)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(i)
                graphs.append(g)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                step(i % len(caches))
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        timer = csa2.KernelTimer(args.steps)
        if hasattr(torch.cuda, "_sleep"):  # queue the eager launches ahead of the GPU
            torch.cuda._sleep(int(3e6 * args.steps))
        for i in range(args.steps):
            step(i % len(caches), scan_timer=timer)
        torch.cuda.synchronize()
        scan_ms = timer.durations_ms()
        timer.close()
    scan_mean = sum(scan_ms) / len(scan_ms)
    # 4 heads x 64 channels per (token, position) pair, 2 flops each; with at
    # most 16384 blocks the Full layer with pools scores on fp16 MFMA
    # (k_scan_mma, bounds + exact rescore), otherwise on the exact VALU scan
    flops = 2.0 * 256 * Q * N
    tfs = flops / (scan_mean * 1e-3) / 1e12
    mma = Q >= 4 and cap // 8 <= 16384
    peak = 2500.0 if mma else 157.3
    kname = ("k_scan_mma (Full-layer indexer bounds of the chunk's tokens, fp16 MFMA)" if mma
             else "k_scan_multi (Full-layer exact scan of the chunk's tokens)")
    return {
        "metric": f"CSA2 replay chunk through the decoder stack, queries/s ({Q} replayed "
                  "tokens over 128K entries, 20 layers)",
        "value": round(Q * B * args.steps / elapsed, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": wl.name, "sequences": B, "entries": N, "queries": Q, "heads": H,
                   "plan": wl.plan, "topk": wl.topk, "pool_blocks": wl.pool_blocks,
                   "cache_sets": args.cache_sets,
                   "launch": "eager" if args.no_graph else "hip-graph"},
        "roofline": {"bound": "mfma" if mma else "alu", "achieved": round(tfs, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(tfs / peak, 4),
                     "traffic": None, "kernel": kname, "flops_per_launch": flops,
                     "mean_us": round(scan_mean * 1e3, 2)},
    }


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(args, wl, inp):
    """The oracle as it stands, on its own caches (built before timing), for a
    sample of the batch's sequences: one whole stack step per sequence."""
    import concurrent.futures as cf

    import numpy as np

    sys.path.insert(0, ROOT)
    import oracle

    S = min(args.cpu_seqs or wl.B, wl.B)
    N = wl.n_ent
    threads = oracle.num_threads()
    log(f"cpu baseline: oracle caches for {S} sequences ({threads} threads)")

    quant_ik = oracle.idx4_quant_rows if wl.idx_fp4 else oracle.quant_fp8_rows
    full_batch = oracle.index_full4_batch if wl.idx_fp4 else oracle.index_full_batch
    reindex_batch = oracle.index_reindex4_batch if wl.idx_fp4 else oracle.index_reindex_batch

    def prep(b):
        cs = oracle.rope_table(np.arange(N)) if wl.ratio == 1 else None
        c, s = oracle.quant_fp4(inp.k_tok[b], inp.v_tok[b], wl.ratio, cs)
        ik, iks = quant_ik(inp.idx_k[b])
        return c, s, ik, iks

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(prep, range(S)))
    codes = np.stack([p[0] for p in parts])
    scales = np.stack([p[1] for p in parts])
    ikc = np.stack([p[2] for p in parts])
    iks = np.stack([p[3] for p in parts])
    L = len(wl.plan)
    swk, sks = oracle.quant_fp8_rows(inp.swa_k[:, :S])
    swv, svs = oracle.quant_fp8_rows(inp.swa_v[:, :S])
    nv = np.full((S, 1), N, np.int32)
    sm = 1.0 / math.sqrt(128.0)
    r = wl.ratio
    tok = (N - 1) * r
    slot = (tok + r - 1) % 128
    cs_new = oracle.rope_table(np.array([N - 1])) if r == 1 else None
    log("cpu baseline: timing stack steps of the sample (at least 10 s)")

    def one_step():
        # write path: each sequence's new entry (FP4 record, projected indexer
        # key) and every layer's window token at its ring slot (the same slot
        # and values on every repetition)
        for b in range(S):
            c1, s1 = oracle.quant_fp4(inp.k_tok[b, tok:tok + r], inp.v_tok[b, tok:tok + r], r,
                                      cs_new)
            ik1, is1 = quant_ik(oracle.project_idx(
                oracle.entry_k(inp.k_tok[b, tok:tok + r], r, cs_new), inp.proj))
            codes[b, N - 1], scales[b, N - 1], ikc[b, N - 1], iks[b, N - 1] = c1[0], s1[0], ik1[0], is1[0]
        swk[:, :, slot], sks[:, :, slot] = oracle.quant_fp8_rows(inp.swa_k[:, :S, slot])
        swv[:, :, slot], svs[:, :, slot] = oracle.quant_fp8_rows(inp.swa_v[:, :S, slot])
        pool, cur, k = None, None, 0
        for layer, mode in enumerate(wl.plan):
            if mode == "F":
                cur, pool = full_batch(ikc, iks, inp.iq[k, :S, None], inp.iw[k, :S, None], nv,
                                       wl.topk, wl.pool_blocks)
                k += 1
            elif mode == "X":
                cur = reindex_batch(ikc, iks, inp.iq[k, :S, None], inp.iw[k, :S, None], nv, pool,
                                    wl.topk)
                k += 1
            oracle.attn_decode_batch(inp.q[layer, :S], codes, scales, cur[:, 0], swk[layer],
                                     swv[layer], sks[layer], svs[layer], inp.swa_len[:S], sm)

    t0 = time.perf_counter()
    reps = 0
    while reps < 20 and (reps == 0 or time.perf_counter() - t0 < 10.0):
        one_step()
        reps += 1
    dt = time.perf_counter() - t0
    del L
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    return {"value": S * reps / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"{S} of the {wl.B} sequences, {reps} full {len(wl.plan)}-layer stack "
                      f"step(s) each ({N} entries), repeated until at least 10 s had passed; "
                      f"oracle caches built before timing",
            "seconds": dt}


def roofline_entry(name, what, ms_list, bytes_per_launch, launches_per_step, ms_per_step,
                   traffic):
    mean_ms = sum(ms_list) / len(ms_list)
    gbs = bytes_per_launch / (mean_ms * 1e-3) / 1e9
    t = traffic.get(name)
    return {"kernel": f"{name} ({what})", "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": t, "bytes_per_launch": bytes_per_launch,
            "mean_us": round(mean_ms * 1e3, 2), "launches_per_step": launches_per_step,
            "us_per_step": round(mean_ms * 1e3 * launches_per_step, 1),
            "share_of_step": round(mean_ms * launches_per_step / ms_per_step, 3)}


# sources each kernel's counters depend on (the counters are void once these change)
KERNEL_SOURCES = {
    "k_attn": ["csa2_attn.hip", "csa2_device.hpp", "csa2_internal.hpp"],
    "k_scan": ["csa2_index.hip", "csa2_device.hpp", "csa2_internal.hpp"],
    "k_scan_fp4": ["csa2_index.hip", "csa2_device.hpp", "csa2_internal.hpp"],
    "k_scan_mma": ["csa2_chunk.hip", "csa2_device.hpp", "csa2_internal.hpp"],
}


def kernel_source_hash(name):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "compressed_kv_cache_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_traffic(workload=None):
    """Measured HBM bytes per launch from profiles/traffic.json, per kernel, kept
    only where the kernel's sources still hash to what was profiled and, when
    `workload` is given, the counters were taken on that workload."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as fh:
        data = json.load(fh)
    out = {}
    for name, rec in data.get("kernels", {}).items():
        if workload is not None and rec.get("workload") != workload:
            continue
        if name in KERNEL_SOURCES and rec.get("source_sha256") == kernel_source_hash(name):
            out[name] = rec["bytes_per_launch"]
    return out


# --------------------------------------------------------------------------- whole model
MODEL_METRIC = ("CSA2 whole-model decode step (40 layers: 2 window-only, 3 encoder groups "
                "F+5R over 2:1 entries, decoder F+4X+15R), queries/s vs context")


def build_model_set(csa2, T, B, H, topk, pool, seed):
    """Caches, windows and inputs of one model step at context T tokens (T
    even): the step's token is T - 1, which completes encoder pair T/2 - 1.
    Every global KV is written by the library's write path (FP4 records and
    device-projected FP8 indexer keys) from N(0, 1) K and V drawn on the
    device; the step writes the last entry of each."""
    import numpy as np
    import torch

    from compressed_kv_cache_decode_amd import stack as S
    from compressed_kv_cache_decode_amd import synth

    gen = synth.device_generator(seed)
    rnd = lambda *shape: synth.device_normal(gen, shape)
    proj = rnd(64, 128) / math.sqrt(128.0)
    n_enc, n_dec = T // 2, T
    up = lambda n: (n + 63) // 64 * 64
    enc_caches = [csa2.Cache(B, up(n_enc)) for _ in range(S.ENCODER_GROUPS)]
    dec_cache = csa2.Cache(B, up(n_dec))
    CH = 1 << 16
    for b in range(B):
        for c in enc_caches:
            for t0 in range(0, 2 * (n_enc - 1), CH):
                n = min(CH, 2 * (n_enc - 1) - t0)
                csa2.write_entries(rnd(n, 128), rnd(n, 128), c.kv_codes, c.kv_scales, ratio=2,
                                   dst_rows=c.rows(b, np.arange(t0 // 2, (t0 + n) // 2)),
                                   idx_proj=proj, ik_codes=c.ik_codes, ik_sigma=c.ik_sigma)
        for t0 in range(0, n_dec - 1, CH):
            n = min(CH, n_dec - 1 - t0)
            pos = np.arange(t0, t0 + n)
            csa2.write_entries(rnd(n, 128), rnd(n, 128), dec_cache.kv_codes, dec_cache.kv_scales,
                               rope_cs=torch.from_numpy(csa2.rope_table(pos)).cuda(),
                               dst_rows=dec_cache.rows(b, pos), idx_proj=proj,
                               ik_codes=dec_cache.ik_codes, ik_sigma=dec_cache.ik_sigma)
    slot = (T - 1) % 128

    def windows(L):
        k8 = torch.empty((L, B, 128, 128), dtype=torch.uint8, device="cuda")
        v8 = torch.empty_like(k8)
        ks = torch.empty((L, B, 128), dtype=torch.float32, device="cuda")
        vs = torch.empty_like(ks)
        csa2.quant_fp8(rnd(L * B * 128, 128), k8, ks)
        csa2.quant_fp8(rnd(L * B * 128, 128), v8, vs)
        rows = torch.from_numpy(((np.arange(L)[:, None] * B + np.arange(B)[None, :]) * 128
                                 + slot).reshape(-1).astype(np.int64)).cuda()
        return dict(swk=k8, swv=v8, sks=ks, svs=vs), rows

    def group_args(plan, n_vis):
        L, n_idx = len(plan), sum(m in "FX" for m in plan)
        w, rows = windows(L)
        a = dict(iq=rnd(n_idx, B, 1, 4, 64),
                 iw=torch.rand((n_idx, B, 1, 4), generator=gen, device="cuda"),
                 n_vis=torch.full((B, 1), n_vis, dtype=torch.int32, device="cuda"),
                 q=rnd(L, B, H, 128), swa_len=torch.full((B,), 128, dtype=torch.int32,
                                                         device="cuda"), **w)
        return a, rows

    enc_args, new = [], []
    for c in enc_caches:
        a, rows = group_args(S.ENCODER_GROUP_PLAN, n_enc)
        enc_args.append(a)
        new.append(dict(k_new=rnd(2 * B, 128), v_new=rnd(2 * B, 128),
                        rows_new=torch.arange(B, device="cuda") * c.cap + (n_enc - 1),
                        idx_proj=proj, win_k=rnd(len(S.ENCODER_GROUP_PLAN) * B, 128),
                        win_v=rnd(len(S.ENCODER_GROUP_PLAN) * B, 128), win_rows=rows, ratio=2,
                        rope_cs=None))
    dec_args, rows = group_args(S.DECODER_PLAN, n_dec)
    new.append(dict(k_new=rnd(B, 128), v_new=rnd(B, 128),
                    rows_new=torch.arange(B, device="cuda") * dec_cache.cap + (n_dec - 1),
                    idx_proj=proj, win_k=rnd(len(S.DECODER_PLAN) * B, 128),
                    win_v=rnd(len(S.DECODER_PLAN) * B, 128), win_rows=rows, ratio=1,
                    rope_cs=torch.from_numpy(csa2.rope_table(np.full(B, n_dec - 1))).cuda()))
    W = S.ENCODER_WINDOW_ONLY
    w, rows = windows(W)
    win = dict(q=rnd(W, B, H, 128), swa_len=torch.full((B,), 128, dtype=torch.int32, device="cuda"),
               win_k=rnd(W * B, 128), win_v=rnd(W * B, 128), win_rows=rows, **w)
    model = S.ModelStep(enc_caches, dec_cache, B, H, topk=topk, pool_blocks=pool)
    nbytes = dec_cache.nbytes + sum(c.nbytes for c in enc_caches)
    return model, (new, win, enc_args, dec_args), nbytes


def run_model_sweep(args):
    """Whole-model decode step at each context of --contexts (HIP-graph
    replay, two cache sets rotated)."""
    import torch

    import compressed_kv_cache_decode_amd as csa2
    B, H, topk, pool = args.model_batch, 64, 512, 2048
    sweep = []
    for T in [int(x) for x in args.contexts.split(",")]:
        if T % 2 or T < 256:
            raise SystemExit("contexts must be even and at least 256 tokens")
        log(f"model step: context {T} tokens, B={B}: writing the caches")
        sets = [build_model_set(csa2, T, B, H, topk, pool, 2000 + 7 * i + T)
                for i in range(2)]
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for i in range(max(args.warmup, 1)):
                m, a, _ = sets[i % 2]
                m.step(*a)
            torch.cuda.synchronize()
            graphs = []
            for m, a, _ in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    m.step(*a)
                graphs.append(g)
            for i in range(args.warmup):
                graphs[i % 2].replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                graphs[i % 2].replay()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / args.steps
        sweep.append({"context": T, "ms_per_step": round(dt * 1e3, 4),
                      "queries_per_s": round(B / dt, 1),
                      "cache_MB_per_set": round(sets[0][2] / 1e6, 1)})
        log(f"model step: context {T}: {dt * 1e3:.4f} ms per step")
        del sets, graphs
        torch.cuda.empty_cache()
    head = next((r for r in sweep if r["context"] == 131072), sweep[0])
    return {
        "metric": MODEL_METRIC, "value": head["queries_per_s"], "unit": "queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": "model_step", "sequences": B, "context": head["context"],
                   "layers": 40, "heads": H, "topk": topk, "pool_blocks": pool, "window": 128,
                   "cache_sets": 2, "launch": "hip-graph"},
        "roofline": None, "sweep": sweep,
        "step_time_growth_first_to_last": round(sweep[-1]["ms_per_step"] / sweep[0]["ms_per_step"], 3),
    }


# --------------------------------------------------------------------------- gather sweep
def attn_sweep_points(batches, n_launch):
    """The gathering sparse attention (csa2_sparse_attn_decode: 512 selected
    FP4 records and a 128-token FP8 window per query, 64 heads) at each batch
    of `batches`, timed with HIP events around its dispatch.  Each sequence's
    cache holds 16384 entries written by the library from N(0, 1) K and V
    drawn on the device; three sets of indices, queries and windows rotate so
    that consecutive launches gather different records."""
    import torch

    import compressed_kv_cache_decode_amd as csa2
    from compressed_kv_cache_decode_amd import synth
    H, topk, cap = 64, 512, 16384
    sweep = []
    for B in batches:
        gen = synth.device_generator(4000 + B)
        rnd = lambda *shape: synth.device_normal(gen, shape)
        cache = csa2.Cache(B, cap)
        CH = 1 << 18
        for r0 in range(0, B * cap, CH):
            n = min(CH, B * cap - r0)
            csa2.quant_fp4(rnd(n, 128), rnd(n, 128), cache.kv_codes, cache.kv_scales,
                           dst_rows=torch.arange(r0, r0 + n, dtype=torch.int64, device="cuda"))
        sets = []
        for _ in range(3):
            idx = torch.rand((B, cap), generator=gen, device="cuda").topk(topk).indices
            swk = torch.empty((B, 128, 128), dtype=torch.uint8, device="cuda")
            swv = torch.empty_like(swk)
            sks = torch.empty((B, 128), dtype=torch.float32, device="cuda")
            svs = torch.empty_like(sks)
            csa2.quant_fp8(rnd(B * 128, 128), swk, sks)
            csa2.quant_fp8(rnd(B * 128, 128), swv, svs)
            sets.append(dict(q=rnd(B, H, 128), idx=idx.sort().values.int().contiguous(),
                             swk=swk, swv=swv, sks=sks, svs=svs,
                             swa_len=torch.full((B,), 128, dtype=torch.int32, device="cuda"),
                             out=torch.empty((B, H, 128), dtype=torch.float32, device="cuda"),
                             lse=torch.empty((B, H), dtype=torch.float32, device="cuda")))
        timer = csa2.KernelTimer(n_launch)
        for rep in range(2):  # the first pass warms up
            if rep:
                timer.reset()
                if hasattr(torch.cuda, "_sleep"):  # queue the timed launches back to back
                    torch.cuda._sleep(int(2e5 * n_launch))
            for i in range(n_launch):
                d = sets[i % 3]
                csa2.sparse_attn_decode(d["q"], cache, d["idx"], d["swk"], d["swv"], d["sks"],
                                        d["svs"], d["swa_len"], d["out"], d["lse"],
                                        timer=timer if rep else None)
            torch.cuda.synchronize()
        ms = sorted(timer.durations_ms())
        # the same launches with no arithmetic: csa2_gather_probe reads the
        # same bytes (records, window, q) and writes the same row count
        timer.reset()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(2e5 * n_launch))
        for i in range(n_launch):
            d = sets[i % 3]
            csa2.gather_probe(d["q"], cache, d["idx"], d["swk"], d["swv"], d["sks"], d["svs"],
                              d["out"], timer=timer)
        torch.cuda.synchronize()
        gms = sorted(timer.durations_ms())
        timer.close()
        mean = sum(ms) / len(ms)
        gmean = sum(gms) / len(gms)
        nbytes = B * attn_bytes(topk, 128, H)
        sweep.append({"batch": B, "mean_us": round(mean * 1e3, 2),
                      "median_us": round(percentile(ms, 0.5) * 1e3, 2),
                      "bytes_per_launch": nbytes,
                      "achieved_GBps": round(nbytes / (mean * 1e-3) / 1e9, 1),
                      "frac": round(nbytes / (mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "gather_probe_us": round(gmean * 1e3, 2),
                      "gather_probe_GBps": round(nbytes / (gmean * 1e-3) / 1e9, 1),
                      "frac_of_gather": round(gmean / mean, 4)})
        log(f"attention sweep: B={B}: {mean * 1e3:.2f} us, "
            f"{nbytes / (mean * 1e-3) / 1e9:.0f} GB/s; memory-only gather probe "
            f"{gmean * 1e3:.2f} us, {nbytes / (gmean * 1e-3) / 1e9:.0f} GB/s")
        del cache, sets
        torch.cuda.empty_cache()
    return sweep


def run_attn_sweep(args):
    """Batch sweep of the gathering attention: where the kernel leaves the
    latency regime (attn_sweep_points over --batches)."""
    H, topk, cap = 64, 512, 16384
    n_launch = max(args.steps, 30)
    sweep = attn_sweep_points([int(x) for x in args.batches.split(",")], n_launch)
    best = max(sweep, key=lambda r: r["achieved_GBps"])
    return {"metric": "CSA2 sparse attention (gathering, 512 FP4 records + 128 FP8 window tokens "
                      "per query, 64 heads): HBM GB/s vs batch",
            "value": best["achieved_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": n_launch,
            "warmup": n_launch, "higher_is_better": True, "vs_baseline": None,
            "dtype": DTYPE, "dtype_detail": DTYPE_DETAIL, "data": "synthetic",
            "config": {"workload": "attn_batch_sweep", "heads": H, "topk": topk, "window": 128,
                       "entries_per_sequence": cap, "launch": "eager, HIP events per dispatch"},
            "roofline": {"bound": "hbm", "achieved": best["achieved_GBps"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": best["frac"], "traffic": None,
                         "kernel": f"k_attn (batch {best['batch']})",
                         "bytes_per_launch": best["bytes_per_launch"],
                         "mean_us": best["mean_us"]},
            "sweep": sweep}


# the read probes that cover the buffer with one grid (the others grid-stride)
PROBE_FORM = {2: "one load per thread", 3: "one 16 KB chunk per workgroup"}


def measure_ceilings(mib=1024, reps=10):
    """Streaming ceilings of this GPU, measured in the same run with the
    library's probe kernels (csa2_stream_probe): a read-only pass over `mib`
    MiB and a copy of `mib` MiB (reads and writes `mib` MiB each), 16-byte
    non-temporal loads, best of a few grid sizes, each the mean of `reps`
    back-to-back launches timed with events (queued behind a bounded spin, so
    that the host's launch path is not inside the interval)."""
    import torch

    import compressed_kv_cache_decode_amd as csa2
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    best = {}
    configs = [(0, b) for b in (1024, 2048, 4096, 8192)] + [(2, 1), (3, 1)] + \
              [(1, b) for b in (1024, 2048, 4096, 8192)]
    for mode, blocks in configs:
        probe = (lambda: csa2.stream_probe(1, src, dst, n_blocks=blocks)) if mode == 1 else \
                (lambda: csa2.stream_probe(mode, src, sink=sink, n_blocks=blocks))
        for _ in range(2):
            probe()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(1e6 * reps))  # lets the host queue every launch
        ev[0].record()
        for _ in range(reps):
            probe()
        ev[1].record()
        torch.cuda.synchronize()
        sec = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
        kind = 1 if mode == 1 else 0
        gbs = (2 * n if kind else n) / sec / 1e9
        if gbs > best.get(kind, (0, ""))[0]:
            best[kind] = (gbs, PROBE_FORM.get(mode, f"{blocks} workgroups"))
    del src, dst
    torch.cuda.empty_cache()
    out = {"read_GBps": round(best[0][0], 1), "copy_GBps": round(best[1][0], 1), "bytes": n,
           "how": f"csa2_stream_probe over {mib} MiB (read; copy = reads + writes), best of "
                  f"grid-stride 1024-8192 workgroups, one load per thread and 16 KB chunks per "
                  f"workgroup (read: "
                  f"{best[0][1]}; copy: {best[1][1]}), mean of {reps} launches"}
    log(f"ceilings: read {out['read_GBps']} GB/s, copy {out['copy_GBps']} GB/s")
    return out


def measure_read_at(nbytes, copies=3, reps=12):
    """The streaming-read ceiling at one transfer size: csa2_stream_probe
    reading `nbytes` (rounded up to 16) from one of `copies` buffers in turn
    (together larger than the last-level cache, so reads come from HBM),
    each launch timed by the events recorded just before and after it, with
    the launches queued behind a bounded spin so that the host's launch path
    is not inside any interval (the GPU runs them back to back, as the scan
    is timed); the best of one load per thread, 16 KB chunks per workgroup
    (the scan's own access) and grid-stride 2048-8192 workgroups, median over
    `reps` launches.  A small transfer does not reach the large-transfer
    ceiling (ramp-up and tail), so a kernel moving that many bytes is compared
    with this."""
    import statistics

    import torch

    import compressed_kv_cache_decode_amd as csa2
    n = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    best = (0.0, "")
    for mode, blocks in ((2, 1), (3, 1), (0, 2048), (0, 4096), (0, 8192)):
        for b in bufs:
            csa2.stream_probe(mode, b, sink=sink, n_blocks=blocks)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(1e6 * reps))  # lets the host queue every launch
        ev[0].record()
        for i in range(reps):
            csa2.stream_probe(mode, bufs[i % copies], sink=sink, n_blocks=blocks)
            ev[i + 1].record()
        torch.cuda.synchronize()
        us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]
        gbs = n / statistics.median(us) / 1e3
        if gbs > best[0]:
            best = (gbs, PROBE_FORM.get(mode, f"{blocks} workgroups"))
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": n, "read_GBps": round(best[0], 1),
            "how": f"csa2_stream_probe reading {n} bytes from one of {copies} buffers in turn, "
                   f"launches queued back to back behind a spin, each timed by the events "
                   f"around it, median of {reps} ({best[1]})"}


def with_same_size_read(entry, cache):
    """A scan entry with the read ceiling at its own bytes per launch."""
    if not entry["kernel"].startswith("k_scan"):
        return entry
    n = entry["bytes_per_launch"]
    if n not in cache:
        cache[n] = measure_read_at(n)
        log(f"read ceiling at {n} bytes: {cache[n]['read_GBps']} GB/s")
    e = dict(entry)
    e["read_same_bytes_GBps"] = cache[n]["read_GBps"]
    e["frac_of_read_same_bytes"] = round(e["achieved"] / cache[n]["read_GBps"], 4)
    return e


def with_ceilings(entry, ceil):
    """A roofline entry with its fraction of the measured copy and read ceilings."""
    e = dict(entry)
    e["frac_of_copy"] = round(e["achieved"] / ceil["copy_GBps"], 4)
    e["frac_of_read"] = round(e["achieved"] / ceil["read_GBps"], 4)
    return e


def copy_calibration(mib):
    """One device-to-device copy of `mib` MiB: a kernel of known traffic
    (reads and writes mib MiB each) for scaling the hardware byte counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {mib} MiB device-to-device")
    del src, dst


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the path is "
              "data-parallel over sequences and is measured on one GPU's share.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    from compressed_kv_cache_decode_amd import synth
    if args.workload == "model_step":
        print(json.dumps(run_model_sweep(args)), flush=True)
        return
    if args.workload == "attn_batch_sweep":
        print(json.dumps(run_attn_sweep(args)), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb)
    if wl.Q != 1:
        run = run_chunk_bench if wl.plan == "F" else run_chunk_stack_bench
        print(json.dumps(run(args, wl)), flush=True)
        return
    result = measure_decode(args, wl, cpu=not args.skip_cpu_baseline)
    if wl.name == "decoder_stack_128k" and not args.no_extras:
        extras(args, result)
    print(json.dumps(result), flush=True)


def measure_decode(args, wl, cpu=True):
    """One decode workload: HIP-graph step time, per-kernel rooflines and the
    Full / Reindex call times, and (cpu) the oracle on a sample."""
    import torch

    from compressed_kv_cache_decode_amd import synth
    log(f"workload {wl.name}: drawing inputs (seed {wl.seed})")
    inp = synth.decode_inputs(wl)
    csa2, sets = build_sets(args, wl, inp)
    elapsed, kernel_ms, eager_elapsed = time_gpu(args, wl, csa2, sets)
    del sets
    torch.cuda.empty_cache()

    total_bytes, scan_bytes = step_bytes(wl)
    ms_per_step = elapsed / args.steps * 1e3
    value = wl.B * args.steps / elapsed
    attn_launch_bytes = wl.B * attn_bytes(min(wl.topk, wl.n_ent), 128, wl.H)
    traffic = load_traffic(wl.name)
    rooflines = [
        roofline_entry("k_attn", "sparse attention, one launch per layer", kernel_ms["attn"],
                       attn_launch_bytes, len(wl.plan), ms_per_step, traffic),
        roofline_entry("k_scan_fp4" if wl.idx_fp4 else "k_scan",
                       "Full-layer indexer scan" + (", FP4 keys" if wl.idx_fp4 else ""),
                       kernel_ms["scan"], scan_bytes, 1, ms_per_step, traffic),
    ]
    dominant = max(rooflines, key=lambda r: r["us_per_step"])
    mean = lambda xs: sum(xs) / len(xs) if xs else None
    full_us = mean(kernel_ms["full_call"]) * 1e3
    scan_us = mean(kernel_ms["scan"]) * 1e3
    reindex_us = mean(kernel_ms["reindex_call"])
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "dtype_detail": DTYPE_DETAIL,
        "data": "synthetic",
        "config": {"workload": wl.name, "sequences": wl.B, "entries": wl.n_ent,
                   "indexer_key": "fp4" if wl.idx_fp4 else "fp8",
                   "layers": len(wl.plan), "plan": wl.plan, "heads": wl.H, "topk": wl.topk,
                   "pool_blocks": wl.pool_blocks, "window": 128, "cache_sets": args.cache_sets,
                   "launch": "eager" if args.no_graph else "hip-graph"},
        "roofline": {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                               "traffic", "kernel", "bytes_per_launch",
                                               "mean_us")},
        "rooflines": rooflines,
        "step": {"algorithmic_bytes": total_bytes,
                 "achieved_GBps": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                 "frac_of_hbm_peak": round(total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "eager_ms_per_step": round(eager_elapsed / args.steps * 1e3, 4),
                 "ms_p10_median_p90": [round(percentile(kernel_ms["step"], f), 4)
                                       for f in (0.1, 0.5, 0.9)]},
        # eager call times (HIP events around each library call, queued back to
        # back): the Full layer's index call is the query prep, the scan and the
        # pool + top-K selection; a Reindex call is the pool rescore and its
        # selection
        "index": {"full_call_us": round(full_us, 2), "scan_us": round(scan_us, 2),
                  "full_select_and_prep_us": round(full_us - scan_us, 2),
                  "reindex_call_us": round(reindex_us * 1e3, 2) if reindex_us else None},
    }
    if cpu:
        cb = cpu_baseline(args, wl, inp)
        result["cpu_baseline"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                  for k, v in cb.items()}
    return result


def extras(args, result):
    """Beside the headline: the copy and read ceilings of this GPU (every
    roofline entry also as a fraction of them), the gathering attention at
    large batches (where it is bandwidth- rather than latency-bound) beside
    the memory-only gather probe over the same bytes, and the 1M-entry
    decoder stack as a secondary workload."""
    import torch

    from compressed_kv_cache_decode_amd import synth
    ceil = measure_ceilings()
    result["ceilings"] = ceil
    same = {}
    result["rooflines"] = [with_same_size_read(with_ceilings(r, ceil), same)
                           for r in result["rooflines"]]
    for B, pt in zip((256, 1024), attn_sweep_points([256, 1024], 30)):
        result["rooflines"].append(with_ceilings({
            "kernel": f"k_attn (sparse attention, gathering, batch {B}, 64 heads, top-512 + "
                      f"128-token window)", "bound": "hbm", "achieved": pt["achieved_GBps"],
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": pt["frac"], "traffic": None,
            "bytes_per_launch": pt["bytes_per_launch"], "mean_us": pt["mean_us"],
            # the same bytes read and written by csa2_gather_probe, no arithmetic:
            # the access pattern's own ceiling (random 144-byte records)
            "gather_probe_us": pt["gather_probe_us"],
            "gather_probe_GBps": pt["gather_probe_GBps"],
            "frac_of_gather": pt["frac_of_gather"]}, ceil))
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup, sub.cache_sets = min(args.steps, 30), min(args.warmup, 5), 2
    r1m = measure_decode(sub, synth.WORKLOADS["decoder_stack_1m"], cpu=False)
    torch.cuda.empty_cache()
    result["secondary"] = {
        "decoder_stack_1m": {k: r1m[k] for k in ("value", "unit", "ms_per_step", "steps",
                                                  "warmup", "config", "step", "index")}}
    result["secondary"]["decoder_stack_1m"]["rooflines"] = [
        with_same_size_read(with_ceilings(r, ceil), same) for r in r1m["rooflines"]]
    result["ceilings"]["read_at_scan_bytes"] = [same[n] for n in sorted(same)]


if __name__ == "__main__":
    main()
