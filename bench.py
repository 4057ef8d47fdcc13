#!/usr/bin/env python3
"""Benchmark of the paged-decode hot path on one MI355X.

Default workload: the qwen3-0.6b-shaped decode batch -- 28 layers, 8
sequences x 4096 visible tokens, block 32, 32 blocks per slab, 16 query / 8
kv heads, head_dim 128, bf16, N(0,1) K/V/Q from fixed seeds, rows allocated
monotonically per sequence (4 same-slab runs each).

A step is one decode step of the whole batch: for each of the 28 layers,
paged_decode_append stores each sequence's newest token (position len-1) into
its row's slab and attends over all len tokens, in the split kernel's launch
(then the combine).  The unfused form -- write_block, then paged_decode --
does the same work in three launches per layer; it is checked bit-equal and
timed beside.  Inputs are resident in HBM before timing starts.  The 28-layer step touches 3.5 GiB of
KV, far more than the last-level cache, so every layer is read from HBM.

The timed step is captured once into a HIP graph and replayed, as a serving
loop would run it (every replay is checked bit-equal to the eager step, whose
time is reported beside).  Prints one JSON line.  `value` is the step's
algorithmic HBM bytes (KV read by paged_decode, q in, out, block table, lens,
plus write_block's bytes) divided by the measured step time; `roofline` is paged_decode's dominant kernel
(the split stage): its algorithmic bytes per launch over its average launch
duration, measured live with HIP events on the launch stream around runs of
that stage over every layer (the combine stage is timed the same way and
reported beside).  `cpu_baseline` times the CPU oracle (numpy, fp64) on a
bounded sample of the same workload.

`--workload` selects one of the other workloads instead, each printed as its
own JSON line of the same form:
  fragmented_64      64 sequences of U{512..16384} tokens on rows popped from a
                     shuffled free list; a step writes one new token per
                     sequence (a fresh row at each block boundary) and decodes.
  qwen3_1p7b_32x16k  28 layers x 32 sequences x 16384 tokens (56 GiB of KV); a
                     write_block + paged_decode step, plus gather_visible of a
                     layer to [32, 8, 16384, 128] per tensor.
  footprint_8x4k     8 distinct ~4.2k-token prompts prefilled one after another
                     (qwen3-0.6b KV shape): peak HBM of the slab pool over the
                     dense backend's (its own metric; lower is better).
  packed_16x16k      16 sequences x 16384 tokens, 8 kv / 32 q heads, head_dim 64
                     and 256, bf16 and the packed formats K8V8, K8V4, K4V4;
                     decode calls rotate over enough pool layers that the
                     last-level cache cannot serve repeats.
Their K/V come from the seeded device generator (the parity tests use the
host generator at the same shapes).
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
TRACE_PROFILE = os.path.join(ROOT, "profiles", "paged_decode_qwen3_0p6b_8x4k_kernel_trace.md")
DECODE_SOURCES = ("paged_decode_row.hip", "device_common.h")
METRIC = "paged_decode achieved HBM GB/s (% of peak) + KV tokens attended/sec"
MALL_BYTES = 256 << 20  # last-level cache of the MI355X


def decode_source_hash(sources=DECODE_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in sources:
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


def traced_launch_us(kernel_prefix: str):
    """Average duration of `kernel_prefix` in the committed rocprofv3 kernel
    trace of this benchmark, or None when the trace is missing or was taken
    from another version of the decode kernel's source."""
    try:
        text = open(TRACE_PROFILE).read()
    except OSError:
        return None
    if f"source hash `{decode_source_hash()}`" not in text:
        return None
    for line in text.splitlines():
        cells = [c.strip().strip("`") for c in line.split("|")]
        if len(cells) > 4 and cells[1].startswith(kernel_prefix):
            try:
                return float(cells[3])
            except ValueError:
                return None
    return None


PACKED_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "paged_decode_packed_16x16k_traffic.md")
PACKED_SOURCES = ("paged_decode_packed_mfma.hip", "pack_vector.h", "device_common.h")


def measured_packed_traffic(case: str):
    """HBM bytes per launch of the packed decode kernel for `case` (e.g.
    "k4v4_d64") from the committed counter profile, or None when the profile
    is missing or the kernel changed since."""
    try:
        text = open(PACKED_TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != decode_source_hash(PACKED_SOURCES):
        return None
    try:
        return int(fields[f"hbm_bytes_per_launch {case}"])
    except (KeyError, ValueError):
        return None


def decode_bytes(lengths, n_kv, n_q, D, block_size, kv_bytes_per_token_head=None):
    """Algorithmic bytes of one paged_decode launch: K+V of the visible
    tokens, q in, out, the block-table entries in use and the lengths."""
    kvb = 4 * D if kv_bytes_per_token_head is None else kv_bytes_per_token_head
    nb = sum(-(-int(n) // block_size) for n in lengths)
    B = len(lengths)
    return int(sum(lengths)) * n_kv * kvb + B * n_q * D * 2 * 2 + nb * 4 + 4 * B


def write_bytes(n_tokens, n_kv, D, k_rec=None, v_rec=None):
    """Algorithmic bytes of one write_block launch (read the 16-bit source,
    write the records, rows, slots)."""
    k_rec = 2 * D if k_rec is None else k_rec
    v_rec = 2 * D if v_rec is None else v_rec
    return n_tokens * n_kv * (2 * D * 2 + k_rec + v_rec) + n_tokens * 8


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count()


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and logical CPU count, for
    the record beside a CPU timing."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def cpu_baseline(w, target_s: float):
    """The oracle's fp64 decode over whole layers of the workload, until about
    target_s seconds of CPU work have been timed."""
    from oracle.attention import decode_attention_bits
    from synth import kv_bits_for_sequence, q_bits

    lengths = [w.length] * w.batch
    elapsed, layers, calls, reps = 0.0, 0, 0, 1
    while elapsed < target_s and layers < w.n_layers:
        ks, vs = zip(*[kv_bits_for_sequence(w.seed, layers, b, w.length, w.n_kv_heads,
                                            w.head_dim, w.dtype) for b in range(w.batch)])
        q = q_bits(w.seed, layers, w.batch, w.n_q_heads, w.head_dim, w.dtype)
        for _ in range(reps):
            t0 = time.perf_counter()
            decode_attention_bits(q, ks, vs, w.dtype, w.scale)
            elapsed += time.perf_counter() - t0
            calls += 1
        if layers == 0:
            # when every layer once takes less than target_s, each layer is
            # timed several times so that the sample still spans target_s
            reps = max(1, min(10, int(np.ceil(target_s / (elapsed * w.n_layers)))))
        layers += 1
    nbytes = decode_bytes(lengths, w.n_kv_heads, w.n_q_heads, w.head_dim, w.block_size) * calls
    return {
        "value": round(nbytes / elapsed / 1e9, 3),
        "unit": "GB/s",
        "tokens_attended_per_s": round(sum(lengths) * calls / elapsed, 1),
        "cores": int(blas_threads()),
        **host_cpu(),
        "kind": "oracle",
        "sample": f"{layers} of {w.n_layers} layers of the same batch ({w.batch} x {w.length} "
                  f"tokens), {calls} timed layer decodes (layers after the first repeated "
                  f"{reps}x), numpy fp64 decode_attention, {elapsed:.1f} s",
    }


def cpu_baseline_sequences(w, lengths, target_s: float):
    """The oracle's fp64 decode one sequence at a time (layer 0 of the
    workload's seeded data), until about target_s seconds have been timed."""
    from oracle.attention import decode_attention_bits
    from synth import kv_bits_for_sequence, q_bits

    q = q_bits(w.seed, 0, len(lengths), w.n_q_heads, w.head_dim, w.dtype)
    elapsed, done = 0.0, []
    for b, n in enumerate(lengths):
        if elapsed >= target_s:
            break
        k, v = kv_bits_for_sequence(w.seed, 0, b, int(n), w.n_kv_heads, w.head_dim, w.dtype)
        t0 = time.perf_counter()
        decode_attention_bits(q[b:b + 1], [k], [v], w.dtype, w.scale)
        elapsed += time.perf_counter() - t0
        done.append(int(n))
    nbytes = decode_bytes(done, w.n_kv_heads, w.n_q_heads, w.head_dim, w.block_size)
    return {
        "value": round(nbytes / elapsed / 1e9, 3),
        "unit": "GB/s",
        "tokens_attended_per_s": round(sum(done) / elapsed, 1),
        "cores": int(blas_threads()),
        **host_cpu(),
        "kind": "oracle",
        "sample": f"{len(done)} of {len(lengths)} sequences of layer 0 ({sum(done)} tokens), "
                  f"numpy fp64 decode_attention, {elapsed:.1f} s",
    }


class Timer:
    """Microseconds per call of fn, between two events recorded on the
    stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def __call__(self, fn, reps):
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(reps):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps


class Graph:
    """fn captured once into a HIP graph (torch.cuda.CUDAGraph; the library
    launches on the capturing stream, which torch makes current) and replayed
    on the current stream.  fn must not allocate or synchronise."""

    def __init__(self, torch, fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()
        torch.cuda.synchronize()

    def __call__(self):
        self.graph.replay()


def check_graph_replays(torch, step, graph, outs, rounds=2):
    """Every replay of the captured step gives the eager step's outputs, bit
    for bit, with eager work and synchronisations between the replays."""
    for _ in range(rounds):
        step()
        torch.cuda.synchronize()
        eager = [o.clone() for o in outs]
        for o in outs:
            o.zero_()
        graph()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(eager, outs)):
            raise RuntimeError("a graph replay of the decode step differs from the eager step")


def stage_times(timer, decode_call, layers, reps, torch=None):
    """Per-launch durations of the split and combine stages: each stage of
    every listed layer back to back (the list repeated to at least 16
    launches), between two events on the launch stream.  With torch given,
    the combine run is captured into a HIP graph and replayed, so that host
    launch overhead does not count: issued from Python, the short combine
    would be timed at the rate the host can issue it."""
    layers = list(layers)
    layers = layers * max(1, -(-16 // len(layers)))

    def run(stage):
        for layer in layers:
            decode_call(layer, stage)
    for _ in range(2):
        run("split")
        run("combine")
    # The split stage is launched eagerly, as a serving loop issues it: it
    # runs far longer than the host takes to issue it (except under a
    # profiler's per-dispatch overhead), and graph replays add gaps of their
    # own between kernels.  It is timed before any graph is captured: the
    # launches right after a capture run slower for a while.
    split_us = timer(lambda: run("split"), reps) / len(layers)
    combine_fn = lambda: run("combine")  # noqa: E731
    if torch is not None:
        combine_fn = Graph(torch, combine_fn)
        for _ in range(4):
            combine_fn()
    combine_us = timer(combine_fn, reps) / len(layers)
    run("split")
    run("combine")
    return split_us, combine_us


def roofline(d_bytes, split_us, kernel, traffic=None, bound="hbm"):
    achieved = d_bytes / (split_us * 1e-6) / 1e9
    return {"bound": bound, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "algorithmic_bytes_per_launch": int(d_bytes), "avg_launch_us": round(split_us, 3)}


def base_result(args, value, ms_per_step, dtype, config):
    return {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic", "config": config,
    }


# ---------------------------------------------------------------------------
# default: the qwen3-0.6b-shaped batch
# ---------------------------------------------------------------------------

def run_qwen3_0p6b(args, torch, pd):
    from synth import WORKLOADS, kv_bits_for_sequence, make_block_table, monotone_rows, q_bits

    w = WORKLOADS["qwen3_0p6b_8x4k"]
    dev = torch.device("cuda:0")
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
        if layer == L - 1:
            prefill_src = (kd, vd)  # kept for the prefill-size write_block timing
        del kd, vd
        qs.append(dev_bits(q_bits(w.seed, layer, B, n_q, D, w.dtype)))
        outs.append(torch.empty_like(qs[-1]))
    ws = pool.workspace(B, n_q, n)
    torch.cuda.synchronize()
    if pool.check_error():
        raise RuntimeError("device error while filling the pool")

    timer = Timer(torch)

    # A decode step: every layer appends the sequences' newest token (position
    # n - 1) and attends over all n tokens, in one launch of the split kernel
    # plus the combine (pd_paged_decode_append).  The unfused step (write_block,
    # then paged_decode) does the same work in three launches per layer; it
    # is timed beside and must give the same bits.
    def step():
        for layer in range(L):
            pool.paged_decode_append(layer, qs[layer], k_new[layer], v_new[layer], table, lens, n,
                                     w.scale, outs[layer], ws)

    def step_unfused():
        for layer in range(L):
            pool.write_block(layer, new_rows, new_slots, k_new[layer], v_new[layer])
            pool.paged_decode(layer, qs[layer], table, lens, n, w.scale, outs[layer], ws)

    def decode_call(layer, stage):
        pool.paged_decode(layer, qs[layer], table, lens, n, w.scale, outs[layer], ws, stage=stage)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-stage launch durations first, right after the warm-up steps
    split_us, combine_us = stage_times(timer, decode_call, range(L), args.steps, torch)

    step_unfused()
    torch.cuda.synchronize()
    unfused_out = [o.clone() for o in outs]
    step()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(unfused_out, outs)):
        raise RuntimeError("the fused append step differs from write_block + paged_decode")
    del unfused_out

    # The step as a serving loop runs it: captured once into a HIP graph and
    # replayed (28 x append-and-split + combine, no host work per launch).
    graph = Graph(torch, step)
    check_graph_replays(torch, step, graph, outs)
    for _ in range(args.warmup):
        graph()
    # timed region: exactly `steps` full steps between two synchronised events
    step_ms = timer(graph, args.steps) / 1e3
    if pool.check_error():
        raise RuntimeError("device error during the timed steps")
    eager_ms = timer(step, args.steps) / 1e3
    graph_unfused = Graph(torch, step_unfused)
    check_graph_replays(torch, step_unfused, graph_unfused, outs)
    for _ in range(args.warmup):
        graph_unfused()
    unfused_ms = timer(graph_unfused, args.steps) / 1e3
    del graph_unfused

    d_bytes = decode_bytes(lengths, n_kv, n_q, D, bs)
    w_bytes = write_bytes(B, n_kv, D)
    step_bytes = L * (d_bytes + w_bytes)

    # write_block of a whole layer's prefill (8 x 4096 tokens; it rewrites the
    # same values), reported beside: K and V read from the sources, written
    # into their rows' slabs, plus the rows and slots
    for _ in range(2):
        pool.write_block(L - 1, all_rows, all_slots, *prefill_src)
    wb_us = timer(lambda: pool.write_block(L - 1, all_rows, all_slots, *prefill_src), 5)
    wb_bytes = 2 * 2 * B * n * n_kv * D * 2 + B * n * 8
    del prefill_src

    # gather_visible of one layer to contiguous [B, n_kv, T, D] (reported beside)
    gk = torch.empty((B, n_kv, n, D), dtype=torch.bfloat16, device=dev)
    gv = torch.empty_like(gk)
    for _ in range(3):
        pool.gather_visible(0, table, lens, n, gk, gv)
    it = iter(range(1 << 30))
    g_us = timer(lambda: pool.gather_visible(next(it) % L, table, lens, n, gk, gv), 10)
    g_bytes = 2 * 2 * B * n * n_kv * D * 2 + B * (n // bs) * 4

    # A plain device copy of known size: the scale for HBM byte counters read
    # by a profiler over this same run (outside every timed region).
    calib = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib)
    calib_dst.copy_(calib)
    torch.cuda.synchronize()
    del calib, calib_dst

    value = step_bytes / (step_ms * 1e-3) / 1e9
    result = base_result(args, value, step_ms, "bf16", {
        "workload": "qwen3-0.6b-shaped decode batch", "layers": L, "batch": B, "seq_len": n,
        "block_size": bs, "slab_blocks": w.slab_blocks, "n_q_heads": n_q, "n_kv_heads": n_kv,
        "head_dim": D, "row_layout": "monotone, 4 same-slab runs per sequence"})
    rl = roofline(d_bytes, split_us, "paged_decode_row_kernel<128,2,true,2> (split stage)",
                  measured_traffic())
    rl["kernel_source_sha256"] = decode_source_hash()
    # the whole paged_decode call (split + combine) against the same bytes
    rl["frac_call"] = round(d_bytes / ((split_us + combine_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    # the same kernel in the committed rocprofv3 trace of this benchmark
    # (another box, the same command; null when the kernel changed since)
    t_us = traced_launch_us("paged_decode_row_kernel<128, 2, true, 2>")
    rl["trace"] = None if t_us is None else {
        "avg_launch_us": t_us, "frac": round(d_bytes / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "profile": os.path.relpath(TRACE_PROFILE, ROOT)}
    result.update({
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_attended_per_s": round(sum(lengths) * L / (step_ms * 1e-3), 1),
        "roofline": rl,
        "step_timing": ("HIP graph of the 28-layer step (per layer: append the newest token and attend, "
                        "then combine), replayed; every replay checked bit-equal to the eager step, and "
                        "the step bit-equal to write_block + paged_decode"),
        "eager_ms_per_step": round(eager_ms, 4),
        "unfused_ms_per_step": round(unfused_ms, 4),
        "paged_decode": {"split_us": round(split_us, 3), "combine_us": round(combine_us, 3),
                         "achieved_gbs_both_stages": round(d_bytes / ((split_us + combine_us) * 1e-6) / 1e9, 1)},
        "write_block": {"decode_step_bytes_per_launch": w_bytes,
                        "prefill_layer_us": round(wb_us, 2), "prefill_layer_bytes": wb_bytes,
                        "prefill_layer_gbs": round(wb_bytes / (wb_us * 1e-6) / 1e9, 1)},
        "gather_visible": {"us_per_layer": round(g_us, 2), "bytes_per_layer": g_bytes,
                           "achieved_gbs": round(g_bytes / (g_us * 1e-6) / 1e9, 1)},
    })
    pool.close()
    result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    return result


# ---------------------------------------------------------------------------
# fragmented pool: 64 sequences, shuffled rows, one new token per step
# ---------------------------------------------------------------------------

def run_fragmented(args, torch, pd):
    from synth import WORKLOADS, make_block_table, normal_device, q_bits, shuffled_rows, workload_lengths

    w = WORKLOADS["fragmented_64"]
    dev = torch.device("cuda:0")
    B, bs, S = w.batch, w.block_size, w.slab_blocks
    n_kv, n_q, D = w.n_kv_heads, w.n_q_heads, w.head_dim
    lengths0 = [int(x) for x in workload_lengths(w)]
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 1 << 23]))
    rows, free, R = shuffled_rows(rng, lengths0, bs, S, spare_rows=64)
    n_steps = args.warmup + args.steps

    # every step's new rows, slots, tables and lengths, decided up front
    rows = [list(r) for r in rows]
    free = list(free)
    grow = 0
    step_rows, step_slots, step_lens = [], [], []
    lens_now = list(lengths0)
    for _ in range(n_steps):
        r_s, s_s = [], []
        for b in range(B):
            pos = lens_now[b]
            if pos % bs == 0:
                if not free:  # the free list ran dry: one more slab of rows
                    free = list(range(R + grow * S, R + (grow + 1) * S))
                    grow += 1
                rows[b].append(free.pop(0))
            r_s.append(rows[b][pos // bs])
            s_s.append(pos % bs)
            lens_now[b] = pos + 1
        step_rows.append(r_s)
        step_slots.append(s_s)
        step_lens.append(list(lens_now))
    table = make_block_table([np.asarray(r, np.int32) for r in rows])
    # the table of step i holds exactly the blocks in use after its write
    tables = []
    for i in range(n_steps):
        t = table.copy()
        for b in range(B):
            t[b, -(-step_lens[i][b] // bs):] = -1
        tables.append(torch.as_tensor(t, device=dev))
    max_len = max(step_lens[-1])

    pool = pd.SlabPool(1, bs, n_kv, D, S, -(-(R + grow * S) // S) + 1, "bf16", device=dev)
    pool.reserve_rows(R + grow * S)
    # fill: every sequence's first lengths0[b] tokens
    all_r, all_s = [], []
    for b in range(B):
        t = np.arange(lengths0[b])
        all_r.append(np.asarray(rows[b], np.int32)[t // bs])
        all_s.append((t % bs).astype(np.int32))
    all_r = torch.as_tensor(np.concatenate(all_r), device=dev)
    all_s = torch.as_tensor(np.concatenate(all_s), device=dev)
    n_tok = int(sum(lengths0))
    k = normal_device((w.seed, 0, 0), (n_tok, n_kv, D), w.dtype, dev)
    v = normal_device((w.seed, 0, 1), (n_tok, n_kv, D), w.dtype, dev)
    pool.write_block(0, all_r, all_s, k, v)
    del k, v
    k_new = normal_device((w.seed, 1, 0), (n_steps, B, n_kv, D), w.dtype, dev)
    v_new = normal_device((w.seed, 1, 1), (n_steps, B, n_kv, D), w.dtype, dev)
    new_r = [torch.tensor(r, dtype=torch.int32, device=dev) for r in step_rows]
    new_s = [torch.tensor(s, dtype=torch.int32, device=dev) for s in step_slots]
    lens_d = [torch.tensor(x, dtype=torch.int32, device=dev) for x in step_lens]
    q = torch.from_numpy(q_bits(w.seed, 0, B, n_q, D, w.dtype).view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty_like(q)
    ws = pool.workspace(B, n_q, max_len)
    torch.cuda.synchronize()
    if pool.check_error():
        raise RuntimeError("device error while filling the pool")

    timer = Timer(torch)
    cur = [0]

    def step():
        i = cur[0]
        pool.write_block(0, new_r[i], new_s[i], k_new[i], v_new[i])
        pool.paged_decode(0, q, tables[i], lens_d[i], max_len, w.scale, out, ws)
        cur[0] += 1

    for _ in range(args.warmup):
        step()
    t_steps = timer(step, args.steps)
    if pool.check_error():
        raise RuntimeError("device error during the timed steps")
    last = n_steps - 1
    step_bytes = sum(decode_bytes(step_lens[i], n_kv, n_q, D, bs) + write_bytes(B, n_kv, D)
                     for i in range(args.warmup, n_steps)) / args.steps

    def decode_call(layer, stage):
        pool.paged_decode(0, q, tables[last], lens_d[last], max_len, w.scale, out, ws, stage=stage)

    split_us, combine_us = stage_times(timer, decode_call, [0], args.steps, torch)
    d_bytes = decode_bytes(step_lens[last], n_kv, n_q, D, bs)
    stats = pool.stats()
    pool.close()
    value = step_bytes / (t_steps * 1e-6) / 1e9
    result = base_result(args, value, t_steps / 1e3, "bf16", {
        "workload": "fragmented pool, 64 sequences U{512..16384} tokens", "layers": 1, "batch": B,
        "total_tokens": int(sum(step_lens[last])), "block_size": bs, "slab_blocks": S,
        "n_q_heads": n_q, "n_kv_heads": n_kv, "head_dim": D,
        "row_layout": "rows popped from a seeded shuffled free list"})
    result.update({
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_attended_per_s": round(sum(step_lens[last]) / (t_steps * 1e-6), 1),
        "roofline": roofline(d_bytes, split_us, "paged_decode_row_kernel<128,2,true,2> (split stage)"),
        "paged_decode": {"split_us": round(split_us, 3), "combine_us": round(combine_us, 3)},
        "pool": {"n_slabs": stats["n_slabs"], "slabs_appended_for_steps": grow},
    })
    result["cpu_baseline"] = (cpu_baseline_sequences(w, step_lens[last], args.cpu_seconds)
                              if args.cpu_seconds > 0 else None)
    return result


# ---------------------------------------------------------------------------
# long context: 28 layers x 32 sequences x 16384 tokens
# ---------------------------------------------------------------------------

def run_long_context(args, torch, pd):
    from synth import WORKLOADS, make_block_table, monotone_rows, normal_device

    w = WORKLOADS["qwen3_1p7b_32x16k"]
    dev = torch.device("cuda:0")
    B, L, n, bs, S = w.batch, w.n_layers, w.length, w.block_size, w.slab_blocks
    n_kv, n_q, D = w.n_kv_heads, w.n_q_heads, w.head_dim
    lengths = [n] * B
    rows = monotone_rows(lengths, bs)
    cap = int(rows[-1].max()) + 1
    table = torch.as_tensor(make_block_table(rows), device=dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    pool = pd.SlabPool(L, bs, n_kv, D, S, -(-cap // S) + 1, "bf16", device=dev)
    pool.reserve_rows(cap)
    t_tok = np.arange(n)
    all_rows = torch.as_tensor(np.concatenate([r[t_tok // bs] for r in rows]).astype(np.int32), device=dev)
    all_slots = torch.as_tensor(np.tile((t_tok % bs).astype(np.int32), B), device=dev)
    new_rows = torch.as_tensor(np.array([r[(n - 1) // bs] for r in rows], np.int32), device=dev)
    new_slots = torch.full((B,), (n - 1) % bs, dtype=torch.int32, device=dev)
    qs, outs, k_new, v_new = [], [], [], []
    for layer in range(L):
        k = normal_device((w.seed, layer, 0), (B * n, n_kv, D), w.dtype, dev)
        v = normal_device((w.seed, layer, 1), (B * n, n_kv, D), w.dtype, dev)
        pool.write_block(layer, all_rows, all_slots, k, v)
        k_new.append(k.view(B, n, n_kv, D)[:, n - 1].contiguous())
        v_new.append(v.view(B, n, n_kv, D)[:, n - 1].contiguous())
        del k, v
        qs.append(normal_device((w.seed, layer, 2), (B, n_q, D), w.dtype, dev))
        outs.append(torch.empty_like(qs[-1]))
    ws = pool.workspace(B, n_q, n)
    torch.cuda.synchronize()
    if pool.check_error():
        raise RuntimeError("device error while filling the pool")

    timer = Timer(torch)

    def step():
        for layer in range(L):
            pool.write_block(layer, new_rows, new_slots, k_new[layer], v_new[layer])
            pool.paged_decode(layer, qs[layer], table, lens, n, w.scale, outs[layer], ws)

    def decode_call(layer, stage):
        pool.paged_decode(layer, qs[layer], table, lens, n, w.scale, outs[layer], ws, stage=stage)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager_ms = timer(step, max(2, args.steps // 4)) / 1e3
    graph = Graph(torch, step)
    check_graph_replays(torch, step, graph, outs, rounds=1)
    graph()
    step_ms = timer(graph, args.steps) / 1e3
    if pool.check_error():
        raise RuntimeError("device error during the timed steps")
    split_us, combine_us = stage_times(timer, decode_call, range(L), max(2, args.steps // 4), torch)
    d_bytes = decode_bytes(lengths, n_kv, n_q, D, bs)
    step_bytes = L * (d_bytes + write_bytes(B, n_kv, D))

    gk = torch.empty((B, n_kv, n, D), dtype=torch.bfloat16, device=dev)
    gv = torch.empty_like(gk)
    pool.gather_visible(0, table, lens, n, gk, gv)
    it = iter(range(1 << 30))
    g_us = timer(lambda: pool.gather_visible(next(it) % L, table, lens, n, gk, gv), 5)
    g_bytes = 2 * 2 * B * n * n_kv * D * 2 + B * (n // bs) * 4
    del gk, gv
    pool.close()
    value = step_bytes / (step_ms * 1e-3) / 1e9
    result = base_result(args, value, step_ms, "bf16", {
        "workload": "qwen3-1.7b-shaped long-context batch", "layers": L, "batch": B, "seq_len": n,
        "block_size": bs, "slab_blocks": S, "n_q_heads": n_q, "n_kv_heads": n_kv, "head_dim": D,
        "row_layout": "monotone"})
    result.update({
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_attended_per_s": round(sum(lengths) * L / (step_ms * 1e-3), 1),
        "roofline": roofline(d_bytes, split_us, "paged_decode_row_kernel<128,2,true,2> (split stage)"),
        "step_timing": "HIP graph of the 28-layer step, replayed; replays checked bit-equal to the eager step",
        "eager_ms_per_step": round(eager_ms, 4),
        "paged_decode": {"split_us": round(split_us, 3), "combine_us": round(combine_us, 3)},
        "gather_visible": {"us_per_layer": round(g_us, 2), "bytes_per_layer": g_bytes,
                           "achieved_gbs": round(g_bytes / (g_us * 1e-6) / 1e9, 1),
                           "pct_of_peak": round(100.0 * g_bytes / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)},
    })
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_sequences(w, [n] * B, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    return result


# ---------------------------------------------------------------------------
# packed formats: 16 sequences x 16384 tokens, head_dim 64 and 256
# ---------------------------------------------------------------------------

def run_packed(args, torch, pd):
    from synth import WORKLOADS, hadamard_signs, make_block_table, monotone_rows, normal_device

    w = WORKLOADS["packed_16x16k"]
    dev = torch.device("cuda:0")
    B, n, bs, S = w.batch, w.length, w.block_size, w.slab_blocks
    n_kv, n_q = w.n_kv_heads, w.n_q_heads
    lengths = [n] * B
    rows = monotone_rows(lengths, bs)
    cap = int(rows[-1].max()) + 1
    table = torch.as_tensor(make_block_table(rows), device=dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    t_tok = np.arange(n)
    all_rows = torch.as_tensor(np.concatenate([r[t_tok // bs] for r in rows]).astype(np.int32), device=dev)
    all_slots = torch.as_tensor(np.tile((t_tok % bs).astype(np.int32), B), device=dev)
    timer = Timer(torch)

    def measure(D, fmt, group):
        """One pool of one format and group size: fill, time write_block, the
        whole decode call and its two stages."""
        scale = 1.0 / float(np.sqrt(D))
        signs = hadamard_signs(w.seed, D) if fmt != "bf16" else None
        k_rec, v_rec = pd.record_bytes(pd.FORMAT_NAMES[fmt], D, group)
        kv_bytes = B * n * n_kv * (k_rec + v_rec)
        copies = max(2, -(-3 * MALL_BYTES // kv_bytes))  # rotate past the last-level cache
        pool = pd.SlabPool(copies, bs, n_kv, D, S, -(-cap // S) + 1, fmt, hadamard_signs=signs,
                           device=dev, group_size=group)
        pool.reserve_rows(cap)
        for layer in range(copies):
            k = normal_device((w.seed, D, layer, 0), (B * n, n_kv, D), "bf16", dev)
            v = normal_device((w.seed, D, layer, 1), (B * n, n_kv, D), "bf16", dev)
            pool.write_block(layer, all_rows, all_slots, k, v)
            if layer < copies - 1:
                del k, v
        # the write of a whole layer (16 x 16384 tokens; packed formats
        # rotate K and quantise K and V here), rewriting the same values
        wb_us = timer(lambda: pool.write_block(copies - 1, all_rows, all_slots, k, v), 3)
        wb_bytes = 2 * B * n * n_kv * D * 2 + kv_bytes + B * n * 8
        del k, v
        q = normal_device((w.seed, D, 2), (B, n_q, D), "bf16", dev)
        out = torch.empty_like(q)
        ws = pool.workspace(B, n_q, n)
        torch.cuda.synchronize()
        if pool.check_error():
            raise RuntimeError(f"device error while filling the {fmt} D={D} group {group} pool")
        it = iter(range(1 << 30))

        def call():
            pool.paged_decode(next(it) % copies, q, table, lens, n, scale, out, ws)

        # the same call with each sequence's newest token (position n - 1)
        # appended in the split launch: packed pools rotate and quantise it there
        k_new = normal_device((w.seed, D, 3), (B, n_kv, D), "bf16", dev)
        v_new = normal_device((w.seed, D, 4), (B, n_kv, D), "bf16", dev)

        def call_append():
            pool.paged_decode_append(next(it) % copies, q, k_new, v_new, table, lens, n, scale, out, ws)

        for _ in range(args.warmup):
            call()
            call_append()
        # alternate blocks of the two, so that both see the same clocks (the
        # GPU slows by up to about 10% over the first milliseconds of load)
        blocks, per_block = 3, max(args.steps, copies)
        us = append_us = 0.0
        for _ in range(blocks):
            us += timer(call, per_block) / blocks
            append_us += timer(call_append, per_block) / blocks

        def decode_call(layer, stage):
            pool.paged_decode(layer, q, table, lens, n, scale, out, ws, stage=stage)

        split_us, combine_us = stage_times(timer, decode_call, range(copies),
                                           max(2, args.steps // copies), torch)
        if pool.check_error():
            raise RuntimeError(f"device error during the {fmt} D={D} group {group} timing")
        pool.close()
        d_bytes = decode_bytes(lengths, n_kv, n_q, D, bs, k_rec + v_rec)
        return {
            "us_per_call": round(us, 2), "append_us_per_call": round(append_us, 2),
            "split_us": round(split_us, 2),
            "combine_us": round(combine_us, 2), "kv_bytes": kv_bytes,
            "algorithmic_bytes": d_bytes,
            "bits_per_value": round(8 * (k_rec + v_rec) / (2 * D), 3),
            "split_gbs": round(d_bytes / (split_us * 1e-6) / 1e9, 1),
            "split_pct_of_peak": round(100.0 * d_bytes / (split_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "call_gbs": round(d_bytes / (us * 1e-6) / 1e9, 1),
            "kv_tokens_attended_per_s": round(B * n / (us * 1e-6), 1),
            "pool_copies": copies,
            "write_block_us": round(wb_us, 2), "write_block_bytes": wb_bytes,
            "write_block_gbs": round(wb_bytes / (wb_us * 1e-6) / 1e9, 1),
        }

    # the workload: every head_dim, bf16 and the packed formats with groups of 32
    per, tot_bytes, tot_us = {}, 0, 0.0
    for D in w.head_dims:
        for fmt in ("bf16",) + tuple(w.formats):
            r = measure(D, fmt, 0 if fmt == "bf16" else 32)
            per[f"{fmt}_d{D}"] = r
            tot_bytes += r["algorithmic_bytes"]
            tot_us += r["us_per_call"]
    # beside it: groups of 64 at head_dim 256 (K4/V4 at five bits per value)
    group64 = {f"{fmt}_d256": measure(256, fmt, 64) for fmt in w.formats} if 256 in w.head_dims else {}
    value = tot_bytes / (tot_us * 1e-6) / 1e9
    worst = min((k for k in per if not k.startswith("bf16")), key=lambda k: per[k]["split_gbs"])
    result = base_result(args, value, tot_us / 1e3, "bf16 q, packed K/V, fp32 accumulate", {
        "workload": "packed KV batch, 16 sequences x 16384 tokens", "layers": 1, "batch": B,
        "seq_len": n, "block_size": bs, "slab_blocks": S, "n_q_heads": n_q, "n_kv_heads": n_kv,
        "head_dims": list(w.head_dims), "formats": ["bf16"] + list(w.formats)})
    p = per[worst]
    result.update({
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_attended_per_s": round(len(per) * B * n / (tot_us * 1e-6), 1),
        "roofline": {"bound": "hbm", "achieved": p["split_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(p["split_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": measured_packed_traffic(worst),
                     "kernel": f"paged_decode_packed_mfma_kernel ({worst}, split stage; the slowest packed case)",
                     "algorithmic_bytes_per_launch": p["algorithmic_bytes"],
                     "avg_launch_us": p["split_us"]},
        "formats": per,
        "group64_formats": group64,
    })
    result["cpu_baseline"] = cpu_baseline_packed(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    return result


# ---------------------------------------------------------------------------
# footprint: 8 sequential distinct ~4.2k-token prefills, slab pool vs dense
# ---------------------------------------------------------------------------

def run_footprint(args, torch, pd):
    """Peak HBM of the KV cache over 8 distinct prompts of ~4.2k tokens
    (qwen3-0.6b KV shape, 28 layers), three ways, each measured on the torch
    allocator (peak reserved bytes):
      - dense: each sequence in K/V tensors of exactly its length;
      - slab pool: grows by appending slabs as the prompts extend it;
      - growth by copy (the pool before slabs, mlxcel #235 "Problem"): one
        tensor per layer for K and one for V, grown to the rows in use
        rounded up to 32 blocks by allocating a larger zeroed tensor, copying
        and freeing the old one, so the allocator keeps the freed ladder.
    Twice: prefilled one after another (sequential), and concurrently (every
    round extends all 8 prompts by up to 512 tokens, so rows interleave).
    All arms write the same tokens from the same transient per-layer sources."""
    from synth import WORKLOADS, normal_device, workload_lengths

    w = WORKLOADS["footprint_8x4k"]
    dev = torch.device("cuda:0")
    L, bs, S, n_kv, D = w.n_layers, w.block_size, w.slab_blocks, w.n_kv_heads, w.head_dim
    lengths = [int(x) for x in workload_lengths(w)]
    token_bytes = L * n_kv * D * 2 * 2  # K + V, every layer
    chunk_tokens, grow_blocks = 512, 32

    def measure(fn):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base_a, base_r = torch.cuda.memory_allocated(), torch.cuda.memory_reserved()
        t0 = time.perf_counter()
        keep = fn()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        peak_a = torch.cuda.max_memory_allocated() - base_a
        peak_r = torch.cuda.max_memory_reserved() - base_r
        return keep, peak_a, peak_r, dt

    def source(i, layer, t0, t1):
        """Tokens [t0, t1) of prompt i in `layer` (drawn whole, then sliced)."""
        n = lengths[i]
        ks = normal_device((w.seed, layer, i, 0), (n, n_kv, D), w.dtype, dev)[t0:t1].contiguous()
        vs = normal_device((w.seed, layer, i, 1), (n, n_kv, D), w.dtype, dev)[t0:t1].contiguous()
        return ks, vs

    def spans(concurrent):
        """(prompt, first token, end token) in the order the prefills write them."""
        if not concurrent:
            return [(i, 0, n) for i, n in enumerate(lengths)]
        out, t = [], 0
        while t < max(lengths):
            out += [(i, t, min(n, t + chunk_tokens)) for i, n in enumerate(lengths) if t < n]
            t += chunk_tokens
        return out

    def dense(concurrent):
        cache = []
        for i, n in enumerate(lengths):
            k = torch.empty((L, n, n_kv, D), dtype=torch.bfloat16, device=dev)
            cache.append((k, torch.empty_like(k)))
        for i, t0, t1 in spans(concurrent):
            for layer in range(L):
                ks, vs = source(i, layer, t0, t1)
                cache[i][0][layer, t0:t1].copy_(ks)
                cache[i][1][layer, t0:t1].copy_(vs)
                del ks, vs
        return cache

    def slab(concurrent):
        pool = pd.SlabPool(L, bs, n_kv, D, S, 64, "bf16", device=dev)
        rows = [[] for _ in lengths]
        next_row = 0
        for i, t0, t1 in spans(concurrent):
            nb_have, nb_need = len(rows[i]), -(-t1 // bs)
            rows[i] += list(range(next_row, next_row + nb_need - nb_have))
            next_row += nb_need - nb_have
            pool.reserve_rows(next_row)  # presize for the span: whole slabs appended
            t = np.arange(t0, t1)
            r = torch.as_tensor(np.asarray(rows[i], np.int32)[t // bs], device=dev)
            sl = torch.as_tensor((t % bs).astype(np.int32), device=dev)
            for layer in range(L):
                ks, vs = source(i, layer, t0, t1)
                pool.write_block(layer, r, sl, ks, vs)
                del ks, vs
        return pool

    def by_copy(concurrent):
        # K and V of every layer in one tensor each, [capacity blocks, bs, n_kv, D]
        cap = 0
        pool = [[None, None] for _ in range(L)]
        rows = [[] for _ in lengths]
        next_row = 0
        for i, t0, t1 in spans(concurrent):
            nb_have, nb_need = len(rows[i]), -(-t1 // bs)
            rows[i] += list(range(next_row, next_row + nb_need - nb_have))
            next_row += nb_need - nb_have
            need = -(-next_row // grow_blocks) * grow_blocks
            if need > cap:
                for layer in range(L):
                    for kv in range(2):
                        new = torch.zeros((need, bs, n_kv, D), dtype=torch.bfloat16, device=dev)
                        if cap:
                            new[:cap].copy_(pool[layer][kv])
                        pool[layer][kv] = new  # the old tensor is freed into the allocator's cache
                        del new
                cap = need
            t = np.arange(t0, t1)
            r = torch.as_tensor(np.asarray(rows[i], np.int64)[t // bs], device=dev)
            sl = torch.as_tensor(t % bs, device=dev)
            for layer in range(L):
                ks, vs = source(i, layer, t0, t1)
                pool[layer][0][r, sl] = ks
                pool[layer][1][r, sl] = vs
                del ks, vs
        return pool

    arms = {}
    for mode in ("sequential", "concurrent"):
        conc = mode == "concurrent"
        cache, dense_a, dense_r, _ = measure(lambda: dense(conc))
        dense_storage = sum(k.numel() * 2 * 2 for k, _ in cache)
        del cache
        pool, slab_a, slab_r, slab_s = measure(lambda: slab(conc))
        if pool.check_error():
            raise RuntimeError("device error during the prefills")
        st = pool.stats()
        pool.close()
        del pool
        grown, copy_a, copy_r, _ = measure(lambda: by_copy(conc))
        del grown
        arms[mode] = {
            "dense": {"storage_bytes": dense_storage, "peak_allocated_bytes": dense_a,
                      "peak_reserved_bytes": dense_r},
            "slab_pool": {"bytes_reserved": st["bytes_reserved"], "n_slabs": st["n_slabs"],
                          "slab_append_events": st["slab_append_events"],
                          "bytes_copied_on_growth": st["bytes_copied_on_growth"],
                          "peak_allocated_bytes": slab_a, "peak_reserved_bytes": slab_r,
                          "prefill_s": round(slab_s, 3)},
            "growth_by_copy": {"peak_allocated_bytes": copy_a, "peak_reserved_bytes": copy_r},
            "ratio_reserved": round(slab_r / dense_r, 4),
            "ratio_allocated": round(slab_a / dense_a, 4),
            "growth_by_copy_ratio_reserved": round(copy_r / dense_r, 4),
        }
    seq = arms["sequential"]
    result = {
        "metric": "peak KV-cache HBM of 8 distinct ~4.2k-token prefills, slab pool / dense",
        "value": seq["ratio_reserved"], "unit": "x", "n_gpus": 1, "steps": 1, "warmup": 0,
        "ms_per_step": round(seq["slab_pool"]["prefill_s"] * 1e3, 2), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "footprint: 8 distinct prompts U{4096..4300} tokens, prefilled one after another "
                               "(value) and concurrently in 512-token rounds",
                   "layers": L, "block_size": bs, "slab_blocks": S, "n_kv_heads": n_kv, "head_dim": D,
                   "lengths": lengths, "growth_chunk_blocks": grow_blocks, "concurrent_chunk_tokens": chunk_tokens},
        "sequential": seq, "concurrent": arms["concurrent"],
        "gate": "within about 1.15x of the dense backend",
        "token_bytes_all_layers": token_bytes,
    }
    return result


def cpu_baseline_packed(w, target_s):
    """The oracle's packed decode (K4V4, head_dim 64) one sequence at a time."""
    from oracle.packed import k_records, packed_decode_attention, record_bytes, v_records
    from synth import hadamard_signs, kv_bits_for_sequence, q_bits

    D = 64
    signs = hadamard_signs(w.seed, D)
    q = q_bits(w.seed, 0, w.batch, w.n_q_heads, D, "bf16")
    elapsed, done = 0.0, 0
    for b in range(w.batch):
        if elapsed >= target_s:
            break
        k, v = kv_bits_for_sequence(w.seed, 0, b, w.length, w.n_kv_heads, D, "bf16")
        kr, vr = k_records(k, signs, 4), v_records(v, 4)
        t0 = time.perf_counter()
        packed_decode_attention(q[b:b + 1], [kr], [vr], signs, "k4v4", D, 1.0 / np.sqrt(D))
        elapsed += time.perf_counter() - t0
        done += 1
    rec = record_bytes(D, 4) * 2
    nbytes = decode_bytes([w.length] * done, w.n_kv_heads, w.n_q_heads, D, w.block_size, rec)
    return {"value": round(nbytes / elapsed / 1e9, 3), "unit": "GB/s",
            "tokens_attended_per_s": round(done * w.length / elapsed, 1),
            "cores": int(blas_threads()), **host_cpu(), "kind": "oracle",
            "sample": f"{done} of {w.batch} sequences, K4V4 head_dim 64, numpy fp64 "
                      f"packed_decode_attention, {elapsed:.1f} s"}


RUNNERS = {
    "qwen3_0p6b_8x4k": run_qwen3_0p6b,
    "fragmented_64": run_fragmented,
    "qwen3_1p7b_32x16k": run_long_context,
    "packed_16x16k": run_packed,
    "footprint_8x4k": run_footprint,
}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-oracle work to time for cpu_baseline (0 disables)")
    ap.add_argument("--workload", default="qwen3_0p6b_8x4k", choices=sorted(RUNNERS))
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-decode path here runs on a single "
              "MI355X (a multi-GPU layout would shard sequences or kv heads with no exchange).",
              file=sys.stderr)
        return 2

    import torch

    import decode_memory_amd as pd

    torch.cuda.set_device(torch.device("cuda:0"))
    result = RUNNERS[args.workload](args, torch, pd)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
