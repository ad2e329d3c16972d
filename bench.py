"""Benchmark of the ResidualQuant hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the hot path over one batch of synthetic input:
rq_encode_kv, the encode of K and of V in one launch (every non-final loop
against the bf16 final-loop reference), then rq_decode_attn for every loop
over the just-encoded cache.
K steps are timed between two device synchronisations. `value` is KV tokens
through the hot path per second: batch * seq_len * n_loops / step time.

Timed in the same run, each alone and outside the timed steps, with the
256 MB last-level cache flushed before every repetition by reading a 1 GiB
buffer (a read leaves no dirty lines whose write-back would compete with the
measured kernel):
* rq_decode_attn alone: KV tokens/s, algorithmic GB/s and the fraction of the
  8 TB/s HBM peak;
* the bf16-KV baseline decode (rq_decode_attn_bf16) over the same loops;
* one call per loop (per-loop mode);
* rq_reconstruct of one loop;
* rq_encode_refit of K with 0, 1 and 2 code / LS-scale refits: encode rate
  and reconstruction error per residual loop;
* a serving step: rq_decode_attn_varlen over ragged prefixes plus one bf16
  tail position per loop, then rq_encode_append of that position (K and V);
* the rotation-only baseline (rq_encode_rotonly of every loop of K with no
  reference): its encode rate, and its per-loop reconstruction error and
  cache bytes beside those of the residual codec.
* first of all, the peak-batch workload (8 loops, 4 / 16 heads, 16K tokens):
  the batch grows until the cache fills about 200 GB of HBM, for the residual
  cache and for the bf16-KV baseline at its own largest batch; decode tokens/s
  of both (one decode call = the next token of every sequence).

`roofline` covers the kernel that takes the largest share of the step (the
encoder, one launch for K and V). Its achieved rate is algorithmic bytes per launch divided by the
launch's average duration, timed with HIP events on the stream the kernel
runs on over a run of back-to-back launches (no event marker between two
launches). `traffic` comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary
under profiles/, but only while the kernel source still matches the hash
recorded there. Otherwise it is null.

`cpu_baseline` is the fp64 NumPy oracle on the host cores, timed on a fixed
sample of (batch, kv_head) rows of the same workload. It is a reported
baseline, not a target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "decode-attn KV tokens/s & achieved HBM GB/s (% of peak); encode GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
_CSRC = os.path.join(ROOT, "looped_transformer_kv_rq_amd", "csrc")
# sources each counted kernel is built from (a change to any of them voids its traffic figure)
KERNEL_SOURCES = {
    "encode": [os.path.join(_CSRC, f) for f in ("rq_codec.hip", "rq_device.h", "rq_internal.h")],
    "decode_attn": [os.path.join(_CSRC, f) for f in ("rq_decode_mfma.hip", "rq_combine.hip", "rq_api.hip",
                                                      "rq_device.h", "rq_internal.h")],
}


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method must move; nothing it avoids)
# ---------------------------------------------------------------------------

def encode_bytes(w, bits):
    """One rq_encode launch (one tensor): ref once + per loop x_l, codes, scales."""
    n = w.batch * w.n_kv_heads * w.seq_len * w.head_dim
    return n * (2 + sum(2 + b / 8 + 2 / 32 for b in bits))


def decode_bytes(w, bits_per_loop):
    """One rq_decode_attn call over the given loops: bf16 K/V ref once, each
    residual loop's K and V codes + scales, the queries and the outputs."""
    th = w.batch * w.n_kv_heads * w.seq_len
    d = w.head_dim
    per = 4 * d + sum(2 * (d * b / 8 + d / 32 * 2) for b in bits_per_loop if b)
    return th * per + len(bits_per_loop) * w.batch * w.n_q_heads * d * (2 + 4)


def bf16_decode_bytes(w, n_loops):
    th = w.batch * w.n_kv_heads * w.seq_len
    return n_loops * th * 4 * w.head_dim + n_loops * w.batch * w.n_q_heads * w.head_dim * (2 + 4)


def rotonly_encode_bytes(w, bits):
    """One rq_encode_rotonly launch: per state x, codes, scales (no reference)."""
    n = w.batch * w.n_kv_heads * w.seq_len * w.head_dim
    return n * sum(2 + b / 8 + 2 / 32 for b in bits)


def cache_bytes_per_token_head(w, bits_per_loop, with_reference):
    """K and V bytes one cached position of one KV head takes across all loops."""
    d = w.head_dim
    per = sum(d * b / 8 + 2 * d / 32 for b in bits_per_loop if b)
    return 2 * ((2 * d if with_reference else 0) + per)


def reconstruct_bytes(w, bits):
    n = w.batch * w.n_kv_heads * w.seq_len * w.head_dim
    return n * (2 + bits / 8 + 2 / 32 + 4)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on host cores (run before the GPU is touched)
# ---------------------------------------------------------------------------

def _oracle_row(args):
    """Encode every non-final loop of K and V and decode all loops, for one
    (batch, kv_head) row, with the fp64 oracle."""
    name, b, h = args
    from threadpoolctl import threadpool_limits

    import oracle

    w = workloads.WORKLOADS[name]
    with threadpool_limits(1):
        khat, vhat = [], []
        for tensor, sink in ((workloads.TENSOR_K, khat), (workloads.TENSOR_V, vhat)):
            xs = workloads.kv_rows_all_loops(w, b, h, tensor)
            for l in range(w.n_loops):
                if w.bits[l]:
                    words, scales = oracle.encode(xs[l], xs[-1], w.bits[l])
                    sink.append(oracle.reconstruct(xs[-1], words, scales, w.bits[l]))
                else:
                    sink.append(oracle.bf16_to_f64(xs[-1]))
        g = w.group_size
        scale = 1.0 / math.sqrt(w.head_dim)
        for l in range(w.n_loops):
            q = np.stack([oracle.bf16_to_f64(workloads.q_row(w, b, h * g + j, l)) for j in range(g)])
            oracle.attention(q, khat[l], vhat[l], scale)
    return 1


def cpu_baseline(w, rows_per_worker=8):
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    workers = max(1, min(16, avail))
    all_rows = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    n = min(len(all_rows), workers * rows_per_worker)
    sample = [(w.name, b, h) for (b, h) in all_rows[:n]]
    ctx = mp.get_context("fork")  # before any GPU use in this process
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_row, sample[:workers])  # warm the workers (imports)
        t0 = time.perf_counter()
        pool.map(_oracle_row, sample)
        dt = time.perf_counter() - t0
    kv_tokens = n * w.seq_len * w.n_loops / w.n_kv_heads  # same unit as `value`
    return {
        "value": kv_tokens / dt, "unit": "KV tokens/s", "cores": workers, "kind": "oracle",
        "sample": f"{n} of {len(all_rows)} (batch, kv_head) rows of {w.name}: oracle encode of K and V "
                  f"(all non-final loops) + decode of all {w.n_loops} loops, {dt:.1f} s wall on {workers} "
                  f"processes x 1 BLAS thread",
    }


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------

def _sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, workload_name):
    """HBM bytes per launch (per call for decode_attn) from the committed PMC summary, if the
    kernel sources are unchanged since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("workload") != workload_name or rec.get("source_sha") != _sha(KERNEL_SOURCES[kernel_key]):
        return None
    return rec.get("bytes_per_launch")


COPY_PROBE_BYTES = 256 * 2 ** 20


def copy_probe():
    """Five copies of COPY_PROBE_BYTES between two device buffers: each reads and
    writes exactly that many bytes, so a counter's reading per copy gives its
    scale factor (bytes per reported unit)."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 5}))


def peak_batch_leg(rq, torch, dev, reps):
    """The peak-batch workload: the batch grows until the cache fills about
    200 GB of HBM (less if the device has less free), for the residual cache
    (INT4 loop 0, INT2 loops 1-6, bf16 reference) and for the bf16-KV baseline
    at its own largest batch. One decode call produces the next token of every
    sequence (all 8 loops), so tokens/s = batch / call time. The batch repeats
    eight host-drawn entries (decode time does not depend on the values)."""
    w8 = workloads.WORKLOADS["peak_batch"].with_batch(workloads.PEAK_TILE)
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    budget = min(workloads.PEAK_CACHE_BUDGET, free - 16 * 2**30)
    b_rq = workloads.peak_batch(workloads.cache_bytes_per_sequence(w8, w8.bits), budget)
    b_bf = workloads.peak_batch(workloads.bf16_cache_bytes_per_sequence(w8, w8.n_loops), budget)
    if b_bf < workloads.PEAK_TILE:
        return {"skipped": f"{free / 1e9:.0f} GB free on the device"}

    def dev16(bits_u16, dtype=torch.bfloat16):
        return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(dev).view(dtype)

    def words(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev)

    tile = workloads.tile_batch
    kref8 = dev16(workloads.ref_tensor(w8, workloads.TENSOR_K))
    vref8 = dev16(workloads.ref_tensor(w8, workloads.TENSOR_V))
    q8 = workloads.q_tensor(w8)
    stream = torch.cuda.current_stream(dev)
    Ev = torch.cuda.Event

    def timed(fn):
        fn(); fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = Ev(enable_timing=True), Ev(enable_timing=True)
            a.record(stream); fn(); b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts)

    def q_for(batch):
        return torch.stack([tile(dev16(q8[l]), batch) for l in range(w8.n_loops)])

    out = {"workload": "peak_batch", "cache_budget_GB": budget / 1e9}
    # residual cache
    kref, vref = tile(kref8, b_rq), tile(vref8, b_rq)
    views = []
    for l in range(w8.n_loops):
        if w8.bits[l]:
            (kw, ksc), (vw, vsc) = workloads.packed_tensors(w8, 0, l), workloads.packed_tensors(w8, 1, l)
            views.append(rq.LoopView(w8.bits[l], tile(words(kw), b_rq), tile(dev16(ksc, torch.float16), b_rq),
                                     tile(words(vw), b_rq), tile(dev16(vsc, torch.float16), b_rq)))
        else:
            views.append(rq.LoopView(0))
    q = q_for(b_rq)
    o = torch.empty((w8.n_loops, b_rq, w8.n_q_heads, w8.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(rq.decode_workspace_bytes(b_rq, w8.n_kv_heads, w8.seq_len, w8.head_dim, w8.n_q_heads,
                                               w8.n_loops), dtype=torch.uint8, device=dev)
    ms = timed(lambda: rq.decode_attn(q, kref, vref, views, out=o, workspace=ws, stream=stream))
    wb = w8.with_batch(b_rq)
    nbytes = decode_bytes(wb, list(w8.bits))
    out["rq"] = {"batch": b_rq, "cache_GB": b_rq * workloads.cache_bytes_per_sequence(w8, w8.bits) / 1e9,
                 "ms": ms, "tokens_per_s": b_rq / (ms * 1e-3), "GBps": nbytes / (ms * 1e-3) / 1e9,
                 "frac_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del kref, vref, views, q, o, ws
    torch.cuda.empty_cache()
    # bf16-KV baseline: every loop's K and V in its own allocation
    ks = [tile(kref8, b_bf) for _ in range(w8.n_loops)]
    vs = [tile(vref8, b_bf) for _ in range(w8.n_loops)]
    q = q_for(b_bf)
    o = torch.empty((w8.n_loops, b_bf, w8.n_q_heads, w8.head_dim), dtype=torch.float32, device=dev)
    ms = timed(lambda: rq.decode_attn_bf16(q, ks, vs, out=o, stream=stream))
    nbytes = bf16_decode_bytes(w8.with_batch(b_bf), w8.n_loops)
    out["bf16"] = {"batch": b_bf, "cache_GB": b_bf * workloads.bf16_cache_bytes_per_sequence(w8, w8.n_loops) / 1e9,
                   "ms": ms, "tokens_per_s": b_bf / (ms * 1e-3), "GBps": nbytes / (ms * 1e-3) / 1e9,
                   "frac_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del ks, vs, q, o
    torch.cuda.empty_cache()
    out["rq_over_bf16_tokens_per_s"] = out["rq"]["tokens_per_s"] / out["bf16"]["tokens_per_s"]
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps first: the clocks settle within about 20")
    ap.add_argument("--workload", default="l4_b16_s4k", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--reps", type=int, default=20, help="repetitions of each side measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-step", action="store_true", help="time the step only (for profiling runs)")
    ap.add_argument("--no-peak-batch", action="store_true", help="skip the peak-batch leg (about 200 GB of HBM)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 256 MiB device-to-device copy, five times: the reference kernel "
                         "whose FETCH_SIZE / WRITE_SIZE readings calibrate the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the ResidualQuant hot path has no cross-GPU step; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return

    w = workloads.WORKLOADS[args.workload]
    if w.name == "peak_batch":
        print("the peak-batch workload does not fit bf16 loop states for encode on one GPU; "
              "it is covered by the parity tests", file=sys.stderr)
        sys.exit(2)
    cpu = None if (args.no_cpu_baseline or args.only_step) else cpu_baseline(w)

    import torch

    import looped_transformer_kv_rq_amd as rq

    rq._load()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # first, while nothing else holds device memory
    peak = None if (args.only_step or args.no_peak_batch) else peak_batch_leg(rq, torch, dev, 5)

    def up(bits_u16):
        return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(dev).view(torch.bfloat16)

    res_loops = [l for l in range(w.n_loops) if w.bits[l]]
    bits = [w.bits[l] for l in res_loops]
    kx = [up(x) for x in workloads.kv_tensors(w, workloads.TENSOR_K)]
    vx = [up(x) for x in workloads.kv_tensors(w, workloads.TENSOR_V)]
    q = up(workloads.q_tensor(w))
    shp = (w.batch, w.n_kv_heads, w.seq_len)
    kc = [torch.empty(shp + (w.head_dim * b // 32,), dtype=torch.int32, device=dev) for b in bits]
    vc = [torch.empty_like(t) for t in kc]
    ks = [torch.empty(shp + (w.head_dim // 32,), dtype=torch.float16, device=dev) for _ in bits]
    vs = [torch.empty_like(t) for t in ks]
    views = []
    for l in range(w.n_loops):
        if w.bits[l]:
            i = res_loops.index(l)
            views.append(rq.LoopView(w.bits[l], kc[i], ks[i], vc[i], vs[i]))
        else:
            views.append(rq.LoopView(0))
    out = torch.empty((w.n_loops, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(rq.decode_workspace_bytes(w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.n_q_heads,
                                               w.n_loops), dtype=torch.uint8, device=dev)
    kref, vref = kx[-1], vx[-1]
    stream = torch.cuda.current_stream(dev)

    def enc_k():
        rq.encode_into([kx[l] for l in res_loops], kref, bits, kc, ks, stream=stream)

    def enc_kv():  # K and V in one launch (the step's encode)
        rq.encode_kv_into([kx[l] for l in res_loops], [vx[l] for l in res_loops], kref, vref, bits, kc, ks, vc, vs,
                          stream=stream)

    def dec():
        rq.decode_attn(q, kref, vref, views, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        enc_kv(); dec()
    torch.cuda.synchronize()

    # The timed steps: one pair of events around all of them and nothing
    # between the launches.
    Ev = torch.cuda.Event
    start, stop = Ev(enable_timing=True), Ev(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        enc_kv(); dec()
    stop.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    step_ms = start.elapsed_time(stop) / args.steps

    # Per-kernel split of a step, from a separate pass with an event between
    # every two launches (each marker adds a drain, so this pass runs slower).
    marks = [[Ev(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        m = marks[k]
        m[0].record(stream); enc_kv()
        m[1].record(stream); dec()
        m[2].record(stream)
    torch.cuda.synchronize()
    enc_in_step_ms = statistics.mean([m[0].elapsed_time(m[1]) for m in marks])
    dec_in_step_ms = statistics.mean([m[1].elapsed_time(m[2]) for m in marks])
    marked_step_ms = statistics.mean([m[0].elapsed_time(m[2]) for m in marks])

    # The encoder's roofline figure: back-to-back K+V launches bracketed by
    # one pair of events, so no event marker sits between two launches (a
    # marker between kernels adds its own drain to the interval).
    enc_reps = max(10, args.steps // 2)
    e0, e1 = Ev(enable_timing=True), Ev(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(enc_reps):
        enc_kv()
    e1.record(stream)
    torch.cuda.synchronize()
    enc_ms = e0.elapsed_time(e1) / enc_reps

    kv_tokens = w.batch * w.seq_len * w.n_loops
    enc_b = encode_bytes(w, bits)  # one tensor
    enc_kv_b = 2 * enc_b
    dec_b = decode_bytes(w, list(w.bits))
    result = {
        "metric": METRIC,
        "value": kv_tokens / (step_ms * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "n_loops": w.n_loops, "batch": w.batch, "n_kv_heads": w.n_kv_heads,
            "n_q_heads": w.n_q_heads, "head_dim": w.head_dim, "seq_len": w.seq_len, "bits": list(w.bits),
            "step": "rq_encode_kv (K and V, one launch) + rq_decode_attn (all loops)",
            "storage": "bf16 reference, int2/int4 residual codes, fp16 scales per 32",
        },
    }
    enc_gbps = enc_kv_b / (enc_ms * 1e-3) / 1e9
    result["roofline"] = {
        "kernel": f"rq_encode_kernel<{w.head_dim}> (K and V, {len(bits)} loops each, one launch)",
        "bound": "hbm", "achieved": enc_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": enc_gbps / HBM_PEAK_GBPS, "traffic": _traffic("encode", w.name),
        "algorithmic_bytes_per_launch": enc_kv_b, "launch_ms": enc_ms, "launches_timed": enc_reps,
    }
    result["wall_s_timed"] = wall_s

    if not args.only_step:
        flush = torch.ones(2 ** 28, dtype=torch.float32, device=dev)  # 1 GiB, read to evict the caches

        def timed(fn, reps):
            ts = []
            for _ in range(reps):
                flush.amax()
                a, b = Ev(enable_timing=True), Ev(enable_timing=True)
                a.record(stream); fn(); b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return statistics.median(ts)

        dec_ms = timed(dec, args.reps)
        dec_gbps = dec_b / (dec_ms * 1e-3) / 1e9
        result["roofline_decode"] = {
            "kernel": "rq_decode_attn (split-S partial + combine), all loops, cache flushed",
            "bound": "hbm", "achieved": dec_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": dec_gbps / HBM_PEAK_GBPS, "traffic": _traffic("decode_attn", w.name),
            "algorithmic_bytes_per_call": dec_b,
        }
        out_b = torch.empty_like(out)
        ws_b = torch.empty_like(ws)

        def dec_bf16():
            rq.decode_attn_bf16(q, kx, vx, out=out_b, workspace=ws_b, stream=stream)

        bf_ms = timed(dec_bf16, args.reps)
        bf_b = bf16_decode_bytes(w, w.n_loops)
        per_loop = []
        for l in range(w.n_loops):
            ql = q[l:l + 1].contiguous()
            ol = torch.empty_like(out[:1])

            def dec_one(ql=ql, ol=ol, l=l):
                rq.decode_attn(ql, kref, vref, [views[l]], out=ol, stream=stream)

            ms = timed(dec_one, max(5, args.reps // 2))
            per_loop.append({"loop": l, "bits": w.bits[l], "ms": ms,
                             "GBps": decode_bytes(w, [w.bits[l]]) / (ms * 1e-3) / 1e9})
        rec = torch.empty(kref.shape, dtype=torch.float32, device=dev)

        def recon():
            rq.reconstruct(kref, kc[0], ks[0], bits[0], out=rec, stream=stream)

        rc_ms = timed(recon, max(5, args.reps // 2))
        per_loop_total = sum(p["ms"] for p in per_loop)
        result["decode_attn"] = {
            "kv_tokens_per_s": kv_tokens / (dec_ms * 1e-3), "ms": dec_ms, "GBps": dec_gbps,
            "frac_peak": dec_gbps / HBM_PEAK_GBPS, "ms_in_step": dec_in_step_ms,
        }
        result["encode"] = {"GBps": enc_gbps, "ms_per_launch": enc_ms, "ms_per_launch_in_step": enc_in_step_ms,
                            "launches_per_step": 1, "tensors_per_launch": 2}
        result["step_split"] = {"encode_ms": enc_in_step_ms, "decode_ms": dec_in_step_ms,
                                "step_ms_with_markers": marked_step_ms,
                                "what": "a separate pass with an event between launches"}
        result["bf16_baseline"] = {
            "kv_tokens_per_s": kv_tokens / (bf_ms * 1e-3), "ms": bf_ms,
            "GBps": bf_b / (bf_ms * 1e-3) / 1e9, "frac_peak": bf_b / (bf_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        }
        result["rq_vs_bf16_decode_tokens_per_s"] = bf_ms / dec_ms
        result["per_loop_mode"] = {"calls": per_loop, "total_ms": per_loop_total,
                                   "vs_bf16_all_loop": bf_ms / per_loop_total}
        result["reconstruct"] = {"loop": res_loops[0], "bits": bits[0], "ms": rc_ms,
                                 "GBps": reconstruct_bytes(w, bits[0]) / (rc_ms * 1e-3) / 1e9}

        # Code / LS-scale refits (rq_encode_refit): encode rate of K and the
        # residual-relative reconstruction error |x_hat - x| / |x - x_ref| per
        # residual loop, for 0, 1 and 2 refits.
        refit = []
        for k in (0, 1, 2):
            rc_c = [torch.empty_like(t) for t in kc]
            rc_s = [torch.empty_like(t) for t in ks]

            def enc_rf(k=k, rc_c=rc_c, rc_s=rc_s):
                rq.encode_into([kx[l] for l in res_loops], kref, bits, rc_c, rc_s, stream=stream, refits=k)

            rf_ms = timed(enc_rf, max(5, args.reps // 2))
            errs = []
            for i, l in enumerate(res_loops):
                xq = rq.reconstruct(kref, rc_c[i], rc_s[i], bits[i], stream=stream)
                xl = kx[l].float()
                errs.append(torch.linalg.vector_norm(xq - xl).item() /
                            torch.linalg.vector_norm(xl - kref.float()).item())
                del xq, xl
            refit.append({"refits": k, "encode_ms": rf_ms, "encode_GBps": enc_b / (rf_ms * 1e-3) / 1e9,
                          "residual_rel_error_per_loop": errs})
            del rc_c, rc_s
        result["encode_refits"] = refit

        # Rotation-only baseline (no reference: every loop, the final one
        # included, quantized directly after the rotation) at the same widths,
        # the final loop at the table's INT2. K tensor; errors |x_hat - x| / |x|
        # per loop, from the GPU reconstructions.
        ro_bits = [b if b else 2 for b in w.bits]
        ro = {}

        def enc_ro():
            ro["out"] = rq.encode_rotonly(kx, ro_bits, stream=stream)

        ro_ms = timed(enc_ro, max(5, args.reps // 2))
        ro_codes, ro_scales = ro["out"]
        err_rq, err_ro = [], []
        for l in range(w.n_loops):
            xl = kx[l].float()
            nx = torch.linalg.vector_norm(xl).item()
            xr = rq.reconstruct_rotonly(ro_codes[l], ro_scales[l], ro_bits[l], stream=stream)
            err_ro.append(torch.linalg.vector_norm(xr - xl).item() / nx)
            if w.bits[l]:
                i = res_loops.index(l)
                xq = rq.reconstruct(kref, kc[i], ks[i], w.bits[l], stream=stream)
                err_rq.append(torch.linalg.vector_norm(xq - xl).item() / nx)
            else:
                err_rq.append(0.0)
            del xl, xr
        ro_b = rotonly_encode_bytes(w, ro_bits)
        result["rotation_only_baseline"] = {
            "bits": ro_bits, "encode_ms": ro_ms, "encode_GBps": ro_b / (ro_ms * 1e-3) / 1e9,
            "encode_frac_peak": ro_b / (ro_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "rel_error_per_loop": err_ro, "rq_rel_error_per_loop": err_rq,
            "bytes_per_token_head": cache_bytes_per_token_head(w, ro_bits, False),
            "rq_bytes_per_token_head": cache_bytes_per_token_head(w, list(w.bits), True),
            "bf16_bytes_per_token_head": 2 * 2 * w.head_dim * w.n_loops,
        }

        # Per-(layer, loop) width table (rq_encode_layers, then each layer's
        # decode with its row): LAYER_BITS_L4 over four layers that share the
        # states above, so only the widths differ from layer to layer. Encode of
        # K and V for all layers, decode per layer (cache flushed), and the
        # residual-relative K error per (layer, loop).
        if w.n_loops == len(workloads.LAYER_BITS_L4[0]):
            table = workloads.LAYER_BITS_L4
            lt = {}
            n_lay = len(table)

            def enc_layers():
                lt["k"] = rq.encode_layers([[kx[l] for l in res_loops]] * n_lay, [kref] * n_lay,
                                           [row[:-1] for row in table], stream=stream)
                lt["v"] = rq.encode_layers([[vx[l] for l in res_loops]] * n_lay, [vref] * n_lay,
                                           [row[:-1] for row in table], stream=stream)

            lt_enc_ms = timed(enc_layers, max(5, args.reps // 2))
            lt_enc_b = 2 * sum(encode_bytes(w, row[:-1]) for row in table)
            layers = []
            for li_, row in enumerate(table):
                (lkc, lks), (lvc, lvs) = (lt["k"][0][li_], lt["k"][1][li_]), (lt["v"][0][li_], lt["v"][1][li_])
                lviews = [rq.LoopView(bl, lkc[i], lks[i], lvc[i], lvs[i]) for i, bl in enumerate(row[:-1])]
                lviews.append(rq.LoopView(0))

                def dec_layer(lviews=lviews):
                    rq.decode_attn(q, kref, vref, lviews, out=out, workspace=ws, stream=stream)

                ms = timed(dec_layer, max(5, args.reps // 2))
                gbps = decode_bytes(w, list(row)) / (ms * 1e-3) / 1e9
                errs = []
                for i, bl in enumerate(row[:-1]):
                    xq = rq.reconstruct(kref, lkc[i], lks[i], bl, stream=stream)
                    xl = kx[res_loops[i]].float()
                    errs.append(torch.linalg.vector_norm(xq - xl).item() /
                                torch.linalg.vector_norm(xl - kref.float()).item())
                    del xq, xl
                layers.append({"layer": li_, "bits": list(row), "decode_ms": ms, "decode_GBps": gbps,
                               "decode_frac_peak": gbps / HBM_PEAK_GBPS,
                               "kv_tokens_per_s": kv_tokens / (ms * 1e-3),
                               "bytes_per_token_head": cache_bytes_per_token_head(w, list(row), True),
                               "k_residual_rel_error_per_loop": errs})
            result["layer_table"] = {
                "table": [list(r) for r in table], "encode_all_layers_ms": lt_enc_ms,
                "encode_GBps": lt_enc_b / (lt_enc_ms * 1e-3) / 1e9, "layers": layers,
                "what": f"rq_encode_layers of K and V over {n_lay} layers sharing the {w.name} states, then "
                        "rq_decode_attn per layer with its row of the table",
            }
            del lt

        # Serving step (rq_decode_attn_varlen + rq_encode_append): ragged prefix
        # lengths drawn in [S/2, S), every loop's current position as a one-position
        # bf16 tail, then that position appended to the K and V caches. Runs last:
        # the appends overwrite one position per sequence of the cache above.
        lrng = np.random.default_rng(w.seed)
        lens = lrng.integers(w.seq_len // 2, w.seq_len, size=w.batch).astype(np.int32)
        lens_d = torch.from_numpy(lens).to(dev)
        tk = [x[:, :, :1].contiguous() for x in kx]
        tv = [x[:, :, :1].contiguous() for x in vx]
        ws_v = torch.empty(rq.decode_varlen_workspace_bytes(w.batch, w.n_kv_heads, w.seq_len, w.head_dim,
                                                            w.n_q_heads, w.n_loops, 0, 1),
                           dtype=torch.uint8, device=dev)

        def serve():
            rq.decode_attn_varlen(q, kref, vref, views, seq_lens=lens_d, tail_k=tk, tail_v=tv, out=out,
                                  workspace=ws_v, stream=stream)
            rq.encode_append_kv([tk[l] for l in res_loops], [tv[l] for l in res_loops], tk[-1], tv[-1], bits, lens_d,
                                kref, vref, kc, ks, vc, vs, stream=stream)

        sv_ms = timed(serve, args.reps)
        per_tok = decode_bytes(w, list(w.bits)) / (w.batch * w.seq_len)  # cache bytes per (b, position)
        sv_bytes = per_tok * float(lens.sum()) + w.batch * w.n_kv_heads * w.n_loops * 4 * w.head_dim
        result["serving_step"] = {
            "ms": sv_ms, "prefix_tokens": int(lens.sum()), "tail_positions_per_loop": 1,
            "decode_GBps": sv_bytes / (sv_ms * 1e-3) / 1e9,
            "kv_tokens_per_s": float(lens.sum() + w.batch) * w.n_loops / (sv_ms * 1e-3),
            "what": "rq_decode_attn_varlen (ragged prefixes + 1 tail position) + rq_encode_append_kv (K and V)",
        }

        # The same serving step over a block-paged copy of the cache: blocks of
        # 128 positions in a shuffled order, the table mapping each sequence's
        # blocks (rq_decode_attn_paged + rq_encode_append_paged).
        P = 128
        nbs = w.seq_len // P
        perm = torch.from_numpy(np.random.default_rng(w.seed + 1).permutation(w.batch * nbs)).to(dev)
        table = perm.view(w.batch, nbs).to(torch.int32).contiguous()

        def paged(t):  # [B, H, S, row] -> [B*S/P, H, P, row], logical block n at physical perm[n]
            blocks = t.view(w.batch, w.n_kv_heads, nbs, P, t.shape[-1]).permute(0, 2, 1, 3, 4)
            blocks = blocks.reshape(w.batch * nbs, w.n_kv_heads, P, t.shape[-1])
            out_t = torch.empty_like(blocks)
            out_t[perm] = blocks
            return out_t

        kref_p, vref_p = paged(kref), paged(vref)
        kc_p, ks_p = [paged(t) for t in kc], [paged(t) for t in ks]
        vc_p, vs_p = [paged(t) for t in vc], [paged(t) for t in vs]
        views_p = [rq.LoopView(bl, kc_p[i], ks_p[i], vc_p[i], vs_p[i]) for i, bl in enumerate(bits)]
        views_p.append(rq.LoopView(0))

        def serve_paged():
            rq.decode_attn_paged(q, kref_p, vref_p, views_p, table, seq_lens=lens_d, tail_k=tk, tail_v=tv, out=out,
                                 workspace=ws_v, stream=stream)
            rq.encode_append_paged_kv([tk[l] for l in res_loops], [tv[l] for l in res_loops], tk[-1], tv[-1], bits,
                                      lens_d, table, kref_p, vref_p, kc_p, ks_p, vc_p, vs_p, stream=stream)

        svp_ms = timed(serve_paged, args.reps)
        result["serving_step_paged"] = {
            "ms": svp_ms, "block_size": P, "blocks": w.batch * nbs, "prefix_tokens": int(lens.sum()),
            "decode_GBps": sv_bytes / (svp_ms * 1e-3) / 1e9,
            "kv_tokens_per_s": float(lens.sum() + w.batch) * w.n_loops / (svp_ms * 1e-3),
            "what": "serving_step over a block-paged cache (shuffled blocks of 128 positions)",
        }
        del kref_p, vref_p, kc_p, ks_p, vc_p, vs_p
    if peak is not None:
        result["peak_batch"] = peak
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
