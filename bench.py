"""Benchmark: paged decode attention on one MI355X.

One step = one decode step of one attention layer for the whole batch:
  1. append each sequence's newest K/V token into its slot (quantize-on-write
     for INT4/FP8 pools; with --fused-step the split kernel writes it
     itself: pa_decode_step),
  2. split-K decode over all cached tokens (gathered through block tables),
     including the log-sum-exp merge of split segments (fused into the
     matrix-core kernels; a second launch for the generic kernel and for
     segments split over many workgroups).
Inputs are seeded synthetic data already resident in HBM when timing starts.

`value` is KV GB/s: the algorithmic K/V bytes one decode step must read
(sum over sequences of L * Hkv * 2 * D * bytes/element, or the packed
INT4/FP8 bytes plus their fp16 scales) divided by the measured step time.
`roofline` prices the dominant kernel (the split kernel) against 8 TB/s with
its own launch durations, measured with HIP events on the launch stream;
`roofline.traffic` is the HBM bytes rocprofv3 counted for one launch
(profiles/hbm_traffic.json) over the same duration.  `stream_read_gbs` is a
plain streaming read of the same byte count (the achievable rate);
`paged_read` a plain read of exactly the slabs the attention reads, through
the same tables (the paged access pattern without the arithmetic): its time,
bytes (whole slabs), rate and the split launch's time over it.
`cpu_baseline` times the CPU oracle (logical rebuild through the tables +
float64 attention) on a bounded sample of the same batch.  `warm` and `cold`
give the median / p10 / p90 of per-step HIP-event times, each step timed on
its own: warm behind a spin kernel (no memory traffic), cold after a 512 MiB
device read that evicts the 256 MB Infinity Cache and the L2s.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config llama3-8b]
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "llama3-8b": "Llama-3-8B-shaped decode layer: batch 64, lengths U[512,4096], 32 q / 8 kv heads, "
                 "head_dim 128, bf16, block 16, shuffled tables, pool +10%",
    "long-context": "long-context decode: 4 sequences x 65,536 tokens, 32 q / 8 kv heads, head_dim 128, "
                    "bf16, block 16, shuffled tables",
    "mixed-int4": "mixed precision: 1 x 65,536 (+64 appended) tokens, FP16 sink block, INT4 g128 body, "
                  "32 q / 8 kv heads, head_dim 128, 1% outlier channels x10",
    "mixed-fp8": "mixed precision: 1 x 65,536 (+64 appended) tokens, FP16 sink block, FP8 E4M3 body, "
                 "32 q / 8 kv heads, head_dim 128, 1% outlier channels x10",
    "mixed-window": "mixed precision with a local window: 1 x 65,536 (+64 appended, each settled) "
                    "tokens, FP16 sink block and last-128-token FP16 window, INT4 g64 body, 32 q / 8 kv "
                    "heads, head_dim 128, 1% outlier channels x10",
    "shared-prefix": "shared prefix: 32 forks of a 2,000-token prompt + U[0,512] suffixes, 64 q / 8 kv "
                     "heads, head_dim 128, bf16",
    "shared-prefix-partial": "shared prefix (1,992-token prompt, one CoW clone per writing fork), 64 q / "
                             "8 kv heads, head_dim 128, bf16",
    "spec-verify": "speculative verify step (gamma = 5: 6 causal queries per sequence) on the "
                   "Llama-3-8B-shaped batch: 64 sequences, lengths U[512,4096], 32 q / 8 kv heads, "
                   "head_dim 128, bf16, shuffled tables",
    "spec-verify-int4": "speculative verify step (gamma = 5: 6 causal queries) on the mixed-precision "
                        "sequence: 1 x 65,536 (+64 appended) tokens, FP16 sink block, INT4 g128 body, "
                        "32 q / 8 kv heads, head_dim 128, 1% outlier channels x10",
    "spec-verify-window": "speculative verify step (gamma = 5: 6 causal queries) on the pages' scheme: "
                          "1 x 65,536 (+64 appended, each settled) tokens, FP16 sink block and "
                          "last-128-token FP16 window, INT4 g64 body, 32 q / 8 kv heads, head_dim 128",
    "llama3-8b-bs8": "the Llama-3-8B-shaped decode batch in a pool of 8-token blocks",
    "llama3-8b-bs32": "the Llama-3-8B-shaped decode batch in a pool of 32-token blocks",
    "prefill-chunk": "chunked paged prefill: the last 512-token chunk of 4 prompts of 4,096 tokens "
                     "(causal over the cached prefix and the chunk), 32 q / 8 kv heads, head_dim 128, "
                     "bf16, prompts reserved chunk by chunk",
}
N_QUERY = {"spec-verify": 6, "spec-verify-int4": 6, "spec-verify-window": 6, "prefill-chunk": 512}   # queries per sequence of the step (1 = decode)
# configs whose dominant launch is a matrix-core contraction: roofline in
# TFLOP/s against the dense bf16 peak
MFMA_BOUND = {"prefill-chunk"}
MFMA_PEAK_TFLOPS = 2500.0


def queries(wl, config, nq):
    """The step's queries: decode, verify (gamma + 1) or the last prefill chunk."""
    if nq == 1:
        return wl.q()
    if config == "prefill-chunk":
        return wl.q_chunk(max(wl.extra["lengths"]) // nq - 1, nq)
    return wl.q_verify(nq)


def causal_flops(lens, nq, n_q_heads, head_dim):
    """Q K^T and P V multiply-adds of a step whose query i (of nq) sees
    L - nq + i + 1 tokens: 4 * Hq * D flops per (query, visible token)."""
    vis = sum(sum(max(0, L - nq + i + 1) for i in range(nq)) for L in lens)
    return 4.0 * n_q_heads * head_dim * vis


def kv_bytes_per_token(wl):
    D, H = wl.head_dim, wl.n_kv_heads
    if wl.kv_dtype == "int4":
        per = D // 2 + 4 * (D // wl.group_size)   # codes + fp16 scale and zero per group
    elif wl.kv_dtype == "fp8":
        per = D + 2
    else:
        per = D * {"f32": 4, "f16": 2, "bf16": 2}[wl.kv_dtype]
    return 2 * H * per


def algorithmic_bytes(wl, lens, tables):
    """K/V bytes the decode must read: quantized body tokens at their packed
    size, tokens of FP16 blocks (sink and window: table ids >= num_blocks) at
    fp16."""
    per = kv_bytes_per_token(wl)
    if not wl.num_sink_blocks:
        return int(sum(lens) * per)
    raw = 2 * wl.n_kv_heads * wl.head_dim * 2
    total = 0
    for row, L in zip(tables, lens):
        nb = (L + 15) // 16
        fp16 = np.asarray(row[:nb]) >= wl.num_blocks
        tok = np.minimum(16, L - 16 * np.arange(nb))
        total += int(tok[fp16].sum()) * raw + int(tok[~fp16].sum()) * per
    return int(total)


def paged_bytes(kv, wl, lens, tables):
    """Bytes pa_paged_read reads: every block of each table up to its length,
    whole slabs of every array of the block's arena, for every KV head."""
    from paged_kv_cache_18_amd import binding as B
    lay = B.pa_pool_layout(kv.pool)["slab_bytes"]
    body = sum(lay.get(a, 0) for a in ("K", "V", "KS", "KZ", "VS", "VZ"))
    sink = sum(lay.get(a, 0) for a in ("SK", "SV"))
    total = 0
    for row, L in zip(tables, lens):
        ids = np.asarray(row[:-(-int(L) // wl.block_size)])
        nb_body = int(((ids >= 0) & (ids < wl.num_blocks)).sum())
        nb_sink = int(((ids >= wl.num_blocks) & (ids < wl.num_blocks + wl.num_sink_blocks)).sum())
        total += (nb_body * body + nb_sink * sink) * wl.n_kv_heads
    return int(total)


def cpu_baseline(kv, wl, t, l, budget_s, nq=1, config=""):
    """Time the oracle's decode on the first sequences of the batch: rebuild the
    logical K/V through the table from the copied-back pool bytes, then float64
    attention.  Stops after ~budget_s seconds."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import attention as AT
    from paged_kv_cache_18_amd.binding import DTYPES

    pool_bytes = kv.pool_host_bytes()
    desc = dict(kv_dtype=DTYPES[wl.kv_dtype], n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                group_size=wl.group_size or wl.head_dim, num_blocks=wl.num_blocks,
                num_sink_blocks=wl.num_sink_blocks, block_size=wl.block_size)
    view = AT.PoolView(pool_bytes, desc)
    import torch
    qsrc = queries(wl, config, nq)
    q = torch.from_numpy(qsrc).to({"f32": torch.float32, "f16": torch.float16,
                                   "bf16": torch.bfloat16}[wl.q_dtype]).double().numpy()
    done, secs = 0, 0.0
    while done < wl.batch and secs < budget_s:
        t0 = time.perf_counter()
        K, V = view.logical_kv(t[done], int(l[done]))
        if nq == 1:
            AT.attention_one(q[done], K, V, wl.scale)
        else:
            AT.verify_attention_one(q[done], K, V, wl.scale)
        secs += time.perf_counter() - t0
        done += 1
    byts = algorithmic_bytes(wl, [int(x) for x in l[:done]], t[:done])
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    return {"value": round(byts / secs / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {wl.batch} sequences ({int(sum(l[:done]))} tokens): logical "
                      f"rebuild from the pool bytes + float64 attention, {secs:.1f} s",
            "queries_per_s": round(done * nq / secs, 3),
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama3-8b", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed one by one after a 512 MiB cache flush (0 = skip)")
    ap.add_argument("--identity-tables", action="store_true",
                    help="physical blocks in logical order (free order 0..N-1): the contiguous "
                         "comparator for the paging overhead")
    ap.add_argument("--fused-step", action="store_true",
                    help="decode steps through pa_decode_step (the split kernel writes the new "
                         "tokens itself)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_18_amd import binding as B
    from paged_kv_cache_18_amd import workloads as W
    from paged_kv_cache_18_amd.session import PagedKV, torch_dtype

    dev = "cuda"
    torch.cuda.set_device(0)
    wl = W.by_name(args.config)
    print(f"[bench] {args.config}: prefill ...", file=sys.stderr, flush=True)
    order = np.arange(wl.num_blocks) if args.identity_tables else None
    kv = PagedKV(wl, dev, body_free_order=order)
    kv.replay()
    tdev, ldev, t, l = kv.device_tables()
    lens = [int(x) for x in l]
    max_len = max(lens)
    nq = N_QUERY.get(args.config, 1)
    if nq == 1:
        q = torch.from_numpy(wl.q()).to(torch_dtype(wl.q_dtype)).to(dev)
        ws_bytes = B.pa_decode_workspace_bytes(kv.pool, wl.batch, wl.n_q_heads, max_len)
    else:
        q = torch.from_numpy(queries(wl, args.config, nq)).to(torch_dtype(wl.q_dtype)).to(dev)
        ws_bytes = B.pa_verify_workspace_bytes(kv.pool, wl.batch, wl.n_q_heads, nq, max_len)
    out = torch.empty_like(q)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    # the step's append: every sequence's nq newest tokens, rewritten in their
    # slots (the work per step stays constant)
    k_new, v_new, slots = [], [], []
    for b, (s, L) in enumerate(zip(wl.decode_seqs, lens)):
        K, V = wl.seq_tokens(s)
        for p in range(max(L - nq, 0), L):
            k_new.append(K[p])
            v_new.append(V[p])
            slots.append(t[b, p // wl.block_size] * wl.block_size + p % wl.block_size)
        del K, V
    k_new, v_new = np.stack(k_new), np.stack(v_new)
    n_new = len(slots)
    in_dt = torch_dtype(wl.in_dtype)
    k_new = torch.from_numpy(k_new).to(in_dt).to(dev)
    v_new = torch.from_numpy(v_new).to(in_dt).to(dev)
    slots_dev = torch.from_numpy(np.array(slots, dtype=np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    dargs = (q, kv.pool, tdev, ldev, wl.batch, wl.n_q_heads, wl.q_dtype, tdev.shape[1], max_len,
             wl.scale, out, ws, ws.numel(), sh)
    vargs = (q, kv.pool, tdev, ldev, wl.batch, wl.n_q_heads, nq, wl.q_dtype, tdev.shape[1],
             max_len, wl.scale, out, ws, ws.numel(), sh)

    # --fused-step: the step through pa_decode_step, whose split kernel writes
    # the new tokens itself (16-bit pools with inputs of the pool's dtype;
    # INT4/FP8 pools quantize them), one launch fewer per step and a longer
    # split launch; the roofline then times that launch
    fused = (args.fused_step and nq == 1
             and (wl.kv_dtype in ("int4", "fp8") or wl.in_dtype == wl.kv_dtype))

    def attn_split():   # the dominant launch (prefill: the only one at these shapes)
        if fused:
            B.pa_decode_step_split(q, k_new, v_new, wl.in_dtype, *dargs[1:])
        elif nq == 1:
            B.pa_decode_split(*dargs)
        elif args.config == "prefill-chunk":
            B.pa_prefill_attention(*vargs)
        else:
            B.pa_verify_split(*vargs)

    def attn_rest():    # the merge launch, where the split leaves one
        if nq == 1:
            B.pa_decode_combine(*dargs)
        elif args.config != "prefill-chunk":
            B.pa_verify_combine(*vargs)

    def step():
        if not fused:
            B.pa_append_kv(kv.pool, k_new, v_new, wl.in_dtype, slots_dev, n_new, sh)
        attn_split()
        attn_rest()

    # the workload generator leaves millions of small Python objects; a full
    # collection over them takes tens of milliseconds and, landing inside a
    # timed loop, would be counted as GPU time: move them out of the
    # collector's reach before timing
    gc.collect()
    gc.freeze()
    print(f"[bench] warmup {args.warmup} ...", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps ...", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps

    # the dominant kernel's average launch duration: as many split launches
    # again, back to back on the launch stream between two HIP events (an
    # event pair around every launch would add its own few microseconds to
    # each; back to back, only the gaps between launches are counted)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        attn_split()
    e1.record(stream)
    torch.cuda.synchronize()
    split_avg = e0.elapsed_time(e1) / args.steps
    attn_rest()

    byts = algorithmic_bytes(wl, lens, t)
    kv_gbs = byts / (ms_step * 1e-3) / 1e9
    achieved = byts / (split_avg * 1e-3) / 1e9

    extra = {}

    def one_by_one(n, pre):
        """Per-step event times (us) of n steps and of their split launches,
        each step preceded by `pre` (queued GPU work, so the host has
        enqueued the step's launches before the GPU reaches them)."""
        ev = []
        for _ in range(n):
            pre()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            B.pa_append_kv(kv.pool, k_new, v_new, wl.in_dtype, slots_dev, n_new, sh)
            e[1].record(stream)
            attn_split()
            e[2].record(stream)
            attn_rest()
            e[3].record(stream)
            ev.append(e)
        torch.cuda.synchronize()
        step = [1e3 * e[0].elapsed_time(e[3]) for e in ev]
        split = [1e3 * e[1].elapsed_time(e[2]) for e in ev]
        return step, split

    def dist(x):
        p10, p50, p90 = np.percentile(np.asarray(x), [10, 50, 90])
        return {"median": round(float(p50), 2), "p10": round(float(p10), 2),
                "p90": round(float(p90), 2), "n": len(x)}

    # warm: a spin kernel (no memory traffic) ahead of each step
    warm_step, warm_split = one_by_one(args.steps, lambda: torch.cuda._sleep(300_000))
    extra["fused_step"] = fused
    extra["warm"] = {"step_us": dist(warm_step), "split_us": dist(warm_split)}
    if args.cold_steps > 0:
        # evict the caches by *reading* 512 MiB (more than the 256 MB
        # Infinity Cache plus the L2s); a write would leave dirty lines whose
        # write-back would compete with the timed kernel
        flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        cold_step, cold_split = one_by_one(args.cold_steps, lambda: flush.sum())
        med = float(np.median(cold_split))
        extra["cold"] = {"step_us": dist(cold_step), "split_us": dist(cold_split),
                         "split_gbs_median": round(byts / (med * 1e-6) / 1e9, 1),
                         "flush": "512 MiB device read before each step"}
        if args.config in MFMA_BOUND:
            tfl = causal_flops(lens, nq, wl.n_q_heads, wl.head_dim) / (med * 1e-6) / 1e12
            extra["cold"]["split_frac_median"] = round(tfl / MFMA_PEAK_TFLOPS, 4)
        else:
            extra["cold"]["split_frac_median"] = round(byts / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        del flush
    # achievable read rate: the library's plain streaming-read kernel over a
    # buffer of the same byte count (reported beside the result; the roofline
    # denominator stays the 8 TB/s spec)
    ceil_buf = torch.ones(byts // 4 + 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    nread = (byts // 16) * 16
    B.pa_stream_read(ceil_buf, nread, sink, sh)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        B.pa_stream_read(ceil_buf, nread, sink, sh)
    c1.record(stream)
    torch.cuda.synchronize()
    extra["stream_read_gbs"] = round(nread / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9, 1)
    del ceil_buf
    # the paged read: the library's plain read of exactly the slabs this
    # step's attention reads, through the same tables (the paged access
    # pattern with none of the arithmetic); its bytes are whole slabs
    B.pa_paged_read(kv.pool, tdev, ldev, wl.batch, tdev.shape[1], max_len, sink, sh)
    c0.record(stream)
    for _ in range(10):
        B.pa_paged_read(kv.pool, tdev, ldev, wl.batch, tdev.shape[1], max_len, sink, sh)
    c1.record(stream)
    torch.cuda.synchronize()
    pr_us = c0.elapsed_time(c1) / 10 * 1e3
    pbytes = paged_bytes(kv, wl, lens, t)
    extra["paged_read"] = {"us": round(pr_us, 2), "bytes": pbytes, "gbs": round(pbytes / (pr_us * 1e-6) / 1e9, 1),
                           "split_over_paged_read": round(split_avg * 1e3 / pr_us, 3)}
    if args.copy_calibration:
        a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = 1 << 30

    cpu = None
    if args.cpu_budget > 0:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(kv, wl, t, l, args.cpu_budget, nq, args.config)

    split_blocks = B.pa_decode_split_blocks(kv.pool, wl.batch, wl.n_q_heads, max_len)
    # HBM bytes per split launch from the committed rocprofv3 counters, while
    # the library sources are the ones they were taken from
    from paged_kv_cache_18_amd.profiling import traffic_bytes
    tb = None if args.identity_tables else traffic_bytes(args.config)
    traffic = round(tb / (split_avg * 1e-3) / 1e9, 1) if tb else None
    if args.config in MFMA_BOUND:
        # algorithmic flops of the causal chunk (masked tokens not counted)
        flops = causal_flops(lens, nq, wl.n_q_heads, wl.head_dim)
        tfl = flops / (split_avg * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tfl, 1), "peak": MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tfl / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                    "traffic_unit": "GB/s", "traffic_bytes_per_launch": tb,
                    "flops_per_launch": flops, "kernel": "prefill_tile",
                    "avg_launch_ms": round(split_avg, 5)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "traffic_bytes_per_launch": tb, "kernel": "decode_split",
                    "avg_launch_ms": round(split_avg, 5)}
    res = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) and queries/s, 1 MI355X",
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int4": "int4+f16", "fp8": "fp8e4m3+f16"}.get(wl.kv_dtype, wl.kv_dtype),
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": WORKLOADS[args.config]
                   + (", identity block order" if args.identity_tables else ""), "batch": wl.batch,
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "kv_dtype": wl.kv_dtype,
                   "total_tokens": int(sum(lens)), "max_seq_len": max_len, "n_query": nq,
                   **({} if nq > 1 else {"split_blocks": split_blocks} if split_blocks > 0
                      else {"persistent_workgroups": -split_blocks})},
        "queries_per_s": round(wl.batch * nq / (ms_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * kv_gbs / HBM_PEAK_GBS, 2),
        "kv_bytes_per_step": byts,
        # the block-size trade: slots held per cached token (last-block padding)
        "block_size": wl.block_size,
        "slots_per_token": round(sum(-(-L // wl.block_size) * wl.block_size for L in lens) / max(sum(lens), 1), 5),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    res.update(extra)
    print(json.dumps(res), flush=True)
    kv.close()


if __name__ == "__main__":
    main()
