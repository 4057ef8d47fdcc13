#!/usr/bin/env python3
"""Benchmark of the paged-decode hot path on one MI355X.

Workload: the qwen3-0.6b-shaped decode batch -- 28 layers, 8 sequences x 4096
visible tokens, block 32, 32 blocks per slab, 16 query / 8 kv heads, head_dim
128, bf16, N(0,1) K/V/Q from fixed seeds, rows allocated monotonically per
sequence (4 same-slab runs each).

A step is one decode step of the whole batch: for each of the 28 layers,
write_block stores each sequence's newest token (position len-1) into its
row's slab, then paged_decode attends over all len tokens.  Inputs are
resident in HBM before timing starts.  The 28-layer step touches 3.5 GiB of
KV, far more than the last-level cache, so every layer is read from HBM.

Prints one JSON line.  `value` is the step's algorithmic HBM bytes (KV read
by paged_decode, q in, out, block table, lens, plus write_block's bytes)
divided by the measured step time; `roofline` is paged_decode's dominant kernel
(the split stage): its algorithmic bytes per launch over its average launch
duration, measured live with HIP events on the launch stream around 28-launch
runs of that stage (the combine stage is timed the same way and reported
beside).  `cpu_baseline` times the CPU oracle (numpy, fp64) on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
CALIB_COPY_BYTES = 256 << 20
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "paged_decode_qwen3_0p6b_8x4k_traffic.md")
DECODE_SOURCES = ("paged_decode_row.hip", "device_common.h")


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "decode_memory_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per paged_decode launch from the committed counter profile,
    or None when the profile is missing or the kernel changed since."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != decode_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_bytes(lengths, n_kv, n_q, D, block_size, kv_bytes_per_token_head=None):
    """Algorithmic bytes of one paged_decode launch."""
    kvb = 4 * D if kv_bytes_per_token_head is None else kv_bytes_per_token_head
    nb = sum(-(-int(n) // block_size) for n in lengths)
    B = len(lengths)
    return int(sum(lengths)) * n_kv * kvb + B * n_q * D * 2 * 2 + nb * 4 + 4 * B


def write_bytes(n_tokens, n_kv, D):
    """Algorithmic bytes of one write_block launch (read src, write slabs, rows, slots)."""
    return n_tokens * n_kv * D * 2 * 2 * 2 + n_tokens * 8


def cpu_baseline(w, target_s: float):
    """The oracle's fp64 decode over whole layers of the workload, until about
    target_s seconds of CPU work have been timed."""
    from oracle.attention import decode_attention_bits
    from synth import kv_bits_for_sequence, q_bits

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    lengths = [w.length] * w.batch
    elapsed, layers = 0.0, 0
    while elapsed < target_s and layers < w.n_layers:
        ks, vs = zip(*[kv_bits_for_sequence(w.seed, layers, b, w.length, w.n_kv_heads,
                                            w.head_dim, w.dtype) for b in range(w.batch)])
        q = q_bits(w.seed, layers, w.batch, w.n_q_heads, w.head_dim, w.dtype)
        t0 = time.perf_counter()
        decode_attention_bits(q, ks, vs, w.dtype, w.scale)
        elapsed += time.perf_counter() - t0
        layers += 1
    nbytes = decode_bytes(lengths, w.n_kv_heads, w.n_q_heads, w.head_dim, w.block_size) * layers
    return {
        "value": round(nbytes / elapsed / 1e9, 3),
        "unit": "GB/s",
        "tokens_attended_per_s": round(sum(lengths) * layers / elapsed, 1),
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{layers} of {w.n_layers} layers of the same batch ({w.batch} x {w.length} "
                  f"tokens), numpy fp64 decode_attention, {elapsed:.1f} s",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-oracle work to time for cpu_baseline (0 disables)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-decode path here runs on a single "
              "MI355X (a multi-GPU layout would shard sequences or kv heads with no exchange).",
              file=sys.stderr)
        return 2

    import torch

    import decode_memory_amd as pd
    from synth import WORKLOADS, kv_bits_for_sequence, make_block_table, monotone_rows, q_bits

    w = WORKLOADS["qwen3_0p6b_8x4k"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, L, n, bs = w.batch, w.n_layers, w.length, w.block_size
    n_kv, n_q, D = w.n_kv_heads, w.n_q_heads, w.head_dim
    lengths = [n] * B
    rows = monotone_rows(lengths, bs)
    table = torch.as_tensor(make_block_table(rows), device=dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)

    def dev_bits(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    pool = pd.SlabPool(L, bs, n_kv, D, w.slab_blocks, 64, "bf16", device=dev)
    pool.reserve_rows(int(max(r.max() for r in rows)) + 1)
    t_tok = np.arange(n)
    all_rows = torch.as_tensor(np.concatenate([r[t_tok // bs] for r in rows]).astype(np.int32), device=dev)
    all_slots = torch.as_tensor(np.tile((t_tok % bs).astype(np.int32), B), device=dev)
    new_rows = torch.as_tensor(np.array([r[(n - 1) // bs] for r in rows], np.int32), device=dev)
    new_slots = torch.full((B,), (n - 1) % bs, dtype=torch.int32, device=dev)
    qs, outs, k_new, v_new = [], [], [], []
    for layer in range(L):
        ks, vs = zip(*[kv_bits_for_sequence(w.seed, layer, b, n, n_kv, D, w.dtype) for b in range(B)])
        kd, vd = dev_bits(np.concatenate(ks)), dev_bits(np.concatenate(vs))
        pool.write_block(layer, all_rows, all_slots, kd, vd)
        k_new.append(kd.view(B, n, n_kv, D)[:, n - 1].contiguous())
        v_new.append(vd.view(B, n, n_kv, D)[:, n - 1].contiguous())
        del kd, vd
        qs.append(dev_bits(q_bits(w.seed, layer, B, n_q, D, w.dtype)))
        outs.append(torch.empty_like(qs[-1]))
    ws = pool.workspace(B, n_q, n)
    torch.cuda.synchronize()
    if pool.check_error():
        raise RuntimeError("device error while filling the pool")

    stream = torch.cuda.current_stream()

    def step():
        for layer in range(L):
            pool.write_block(layer, new_rows, new_slots, k_new[layer], v_new[layer])
            pool.paged_decode(layer, qs[layer], table, lens, n, w.scale, outs[layer], ws)

    def stage_pass(stage):
        for layer in range(L):
            pool.paged_decode(layer, qs[layer], table, lens, n, w.scale, outs[layer], ws,
                              stage=stage)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # microseconds per call of fn

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` full steps between two synchronised events
    step_ms = timed(step, args.steps) / 1e3
    if pool.check_error():
        raise RuntimeError("device error during the timed steps")

    # per-kernel durations, live: the split stage (the dominant kernel) of all
    # 28 layers back to back, then the combine stage, each between two events
    for _ in range(2):
        stage_pass("split")
        stage_pass("combine")
    split_us = timed(lambda: stage_pass("split"), args.steps) / L
    combine_us = timed(lambda: stage_pass("combine"), args.steps) / L
    stage_pass("split")
    stage_pass("combine")
    torch.cuda.synchronize()

    d_bytes = decode_bytes(lengths, n_kv, n_q, D, bs)
    w_bytes = write_bytes(B, n_kv, D)
    step_bytes = L * (d_bytes + w_bytes)
    achieved = d_bytes / (split_us * 1e-6) / 1e9

    # gather_visible of one layer to contiguous [B, n_kv, T, D] (reported beside)
    gk = torch.empty((B, n_kv, n, D), dtype=torch.bfloat16, device=dev)
    gv = torch.empty_like(gk)
    for _ in range(3):
        pool.gather_visible(0, table, lens, n, gk, gv)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g_iters = 10
    g0.record(stream)
    for i in range(g_iters):
        pool.gather_visible(i % L, table, lens, n, gk, gv)
    g1.record(stream)
    torch.cuda.synchronize()
    g_us = g0.elapsed_time(g1) * 1e3 / g_iters
    g_bytes = 2 * 2 * B * n * n_kv * D * 2 + B * (n // bs) * 4

    # A plain device copy of known size: the scale for HBM byte counters read
    # by a profiler over this same run (outside every timed region).
    calib = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib)
    calib_dst.copy_(calib)
    torch.cuda.synchronize()
    del calib, calib_dst

    result = {
        "metric": "paged_decode achieved HBM GB/s (% of peak) + KV tokens attended/sec",
        "value": round(step_bytes / (step_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-0.6b-shaped decode batch", "layers": L, "batch": B,
                   "seq_len": n, "block_size": bs, "slab_blocks": w.slab_blocks,
                   "n_q_heads": n_q, "n_kv_heads": n_kv, "head_dim": D,
                   "row_layout": "monotone, 4 same-slab runs per sequence"},
        "pct_of_peak": round(100.0 * step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "kv_tokens_attended_per_s": round(sum(lengths) * L / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "paged_decode_row_kernel<128,2,true,2> (split stage)",
                     "kernel_source_sha256": decode_source_hash(),
                     "algorithmic_bytes_per_launch": d_bytes,
                     "avg_launch_us": round(split_us, 3)},
        "paged_decode": {"split_us": round(split_us, 3), "combine_us": round(combine_us, 3),
                         "achieved_gbs_both_stages": round(d_bytes / ((split_us + combine_us) * 1e-6) / 1e9, 1)},
        "write_block": {"bytes_per_launch": w_bytes},
        "gather_visible": {"us_per_layer": round(g_us, 2), "bytes_per_layer": g_bytes,
                           "achieved_gbs": round(g_bytes / (g_us * 1e-6) / 1e9, 1)},
    }
    pool.close()
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
