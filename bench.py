"""Benchmark of the ResidualQuant hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the hot path over one batch of synthetic input:
rq_encode_kv, the encode of K and of V in one launch (every non-final loop
against the bf16 final-loop reference), then rq_decode_attn for every loop
over the just-encoded cache. The default workload is mixed_s32k: 4 loops
(INT4, INT2, INT2, bf16 reference), batch 8, 8 KV / 32 query heads, head_dim
128, 32K tokens. `value` is KV tokens through the hot path per second:
batch * seq_len * n_loops / step time, with K steps timed between two device
synchronisations after W untimed ones.

Every input of every leg is drawn on the host and uploaded before the first
GPU work, so the device is not idle while the host draws inputs. The main
step runs first: its W warm-up steps, the K timed steps, the marked pass and
the roofline calls, on a device that has run nothing but its own warm-up;
the other legs follow.

`roofline` covers the fused decode (rq_decode_attn: the split-S partial
kernel plus the small combine), the kernel the method is about. Its achieved
rate is algorithmic bytes per call divided by the call's mean duration over
the marked pass: the timed steps' own launch sequence (encode, then the decode
over the codes it just wrote) repeated with a HIP event between launches, on
the stream the kernels run on. Calls of the decode alone, back to back between
one pair of events, are reported beside it (`back_to_back_ms`); there no call
finds any of its cache in the 256 MB last-level cache. `roofline_encode` is
the same for the encoder (one launch for K and V). `traffic` comes from the
rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/, but only while the
kernel sources still match the hash recorded there; otherwise it is null.

Side legs in the same run, each repetition timed with its own pair of events
(median, p10, p90); the single-kernel legs flush the 256 MB last-level cache
first by reading a 1 GiB buffer (a read leaves no dirty lines):
* the peak-batch workload (8 loops, 4 / 16 heads, 16K tokens): the batch grows
  until the cache fills about 200 GB of HBM, for the residual cache and for
  the bf16-KV baseline at its own largest batch (one decode call = the next
  token of every sequence);
* the l4_b16_s4k and heavy_tail workloads: their own step (encode of K and V
  plus the all-loop decode), the decode alone and the bf16 baseline;
* on the main workload: the decode alone, the bf16-KV baseline, one call per
  loop, rq_reconstruct of one loop, rq_encode_refit with 0, 1 and 2 refits,
  the rotation-only baseline, a per-(layer, loop) width table and the serving
  step (ragged prefixes plus one bf16 tail position, dense and paged).

`cpu_baseline` is the fp64 NumPy oracle on the host cores, timed on a fixed
sample of (batch, kv_head) rows of the same workload, before the GPU is
touched. It is a reported baseline, not a target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import platform
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
DEFAULT_WORKLOAD = "mixed_s32k"
SIDE_WORKLOADS = ("l4_b16_s4k", "heavy_tail")


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


def stats(ts):
    """Median, p10 and p90 of per-repetition times (ms)."""
    q = np.percentile(np.asarray(ts, dtype=np.float64), [10, 50, 90])
    return {"ms": float(q[1]), "p10_ms": float(q[0]), "p90_ms": float(q[2]), "reps": len(ts)}


def rate(nbytes, ms):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"GBps": gbps, "frac_peak": gbps / HBM_PEAK_GBPS}


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


def _warm(_):
    from threadpoolctl import threadpool_limits

    import oracle

    with threadpool_limits(1):
        oracle.attention(np.ones((2, 64)), np.ones((8, 64)), np.ones((8, 64)), 0.125)
    return 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, max_workers=16):
    """The oracle on a fixed sample of rows: one row alone on one process (the
    single-core rate), then one row per worker process in parallel. The pool
    is capped at 16 processes (the host share of one GPU on the box); the
    host's own core count is reported beside it."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    workers = max(1, min(max_workers, avail))
    all_rows = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    n = min(len(all_rows), workers)
    sample = [(w.name, b, h) for (b, h) in all_rows[:n]]
    kv_per_row = w.seq_len * w.n_loops / w.n_kv_heads  # KV tokens (the unit of `value`) per row
    ctx = mp.get_context("fork")  # before any GPU use in this process
    with ctx.Pool(workers) as pool:
        pool.map(_warm, range(workers))  # imports and BLAS set-up in every worker
        t0 = time.perf_counter()
        pool.map(_oracle_row, sample[:1])
        t_one = time.perf_counter() - t0
        t0 = time.perf_counter()
        pool.map(_oracle_row, sample, chunksize=1)
        dt = time.perf_counter() - t0
    return {
        "value": n * kv_per_row / dt, "unit": "KV tokens/s", "cores": workers, "kind": "oracle",
        "sample": f"{n} of {len(all_rows)} (batch, kv_head) rows of {w.name}, one per process: oracle encode of "
                  f"K and V (all non-final loops) + decode of all {w.n_loops} loops; {dt:.1f} s wall on {workers} "
                  f"processes x 1 BLAS thread, scaled to the whole workload's KV tokens",
        "cpu_model": _cpu_model(), "host_cores": os.cpu_count(), "cores_available": avail,
        "single_core": {"value": kv_per_row / t_one, "unit": "KV tokens/s", "s_per_row": t_one},
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


def host_states(w):
    """Every loop of K and V (bf16 bits) and the queries of one workload."""
    return {"k": workloads.kv_tensors(w, workloads.TENSOR_K), "v": workloads.kv_tensors(w, workloads.TENSOR_V),
            "q": workloads.q_tensor(w)}


def host_peak_tiles():
    """The peak-batch workload's eight host-drawn batch entries: references,
    queries and random packed residual loops."""
    w8 = workloads.WORKLOADS["peak_batch"].with_batch(workloads.PEAK_TILE)
    packed = {l: (workloads.packed_tensors(w8, 0, l), workloads.packed_tensors(w8, 1, l))
              for l in range(w8.n_loops) if w8.bits[l]}
    return {"w": w8, "kref": workloads.ref_tensor(w8, workloads.TENSOR_K),
            "vref": workloads.ref_tensor(w8, workloads.TENSOR_V), "q": workloads.q_tensor(w8), "packed": packed,
            "k_states": workloads.kv_tensors(w8, workloads.TENSOR_K),
            "v_states": workloads.kv_tensors(w8, workloads.TENSOR_V)}


class Gpu:
    """Device helpers bound to one stream."""

    def __init__(self, torch, rq, dev):
        self.torch, self.rq, self.dev = torch, rq, dev
        self.stream = torch.cuda.current_stream(dev)
        self.flush_buf = None

    def bf16(self, bits_u16):
        t = self.torch
        return t.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(self.dev).view(t.bfloat16)

    def f16(self, bits_u16):
        t = self.torch
        return t.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(self.dev).view(t.float16)

    def words(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(self.dev)

    def flush(self):
        if self.flush_buf is None:
            self.flush_buf = self.torch.ones(2 ** 28, dtype=self.torch.float32, device=self.dev)  # 1 GiB
        self.flush_buf.amax()

    def reps(self, fn, n, flush=True):
        """Per-repetition times (ms), each between its own pair of events."""
        Ev = self.torch.cuda.Event
        fn()
        self.torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            if flush:
                self.flush()
            a, b = Ev(enable_timing=True), Ev(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            self.torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return ts

    def back_to_back(self, fn, n):
        """Average time (ms) of n back-to-back calls between one pair of events."""
        Ev = self.torch.cuda.Event
        fn()
        self.torch.cuda.synchronize()
        a, b = Ev(enable_timing=True), Ev(enable_timing=True)
        a.record(self.stream)
        for _ in range(n):
            fn()
        b.record(self.stream)
        self.torch.cuda.synchronize()
        return a.elapsed_time(b) / n


class Case:
    """One workload's device tensors and its step: rq_encode_kv + rq_decode_attn."""

    def __init__(self, g, w, host):
        t, rq = g.torch, g.rq
        self.g, self.w = g, w
        self.res_loops = [l for l in range(w.n_loops) if w.bits[l]]
        self.bits = [w.bits[l] for l in self.res_loops]
        self.kx = [g.bf16(x) for x in host["k"]]
        self.vx = [g.bf16(x) for x in host["v"]]
        self.q = g.bf16(host["q"])
        shp = (w.batch, w.n_kv_heads, w.seq_len)
        self.kc = [t.empty(shp + (w.head_dim * b // 32,), dtype=t.int32, device=g.dev) for b in self.bits]
        self.vc = [t.empty_like(x) for x in self.kc]
        self.ks = [t.empty(shp + (w.head_dim // 32,), dtype=t.float16, device=g.dev) for _ in self.bits]
        self.vs = [t.empty_like(x) for x in self.ks]
        self.views = []
        for l in range(w.n_loops):
            if w.bits[l]:
                i = self.res_loops.index(l)
                self.views.append(rq.LoopView(w.bits[l], self.kc[i], self.ks[i], self.vc[i], self.vs[i]))
            else:
                self.views.append(rq.LoopView(0))
        self.out = t.empty((w.n_loops, w.batch, w.n_q_heads, w.head_dim), dtype=t.float32, device=g.dev)
        self.ws = t.empty(rq.decode_workspace_bytes(w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.n_q_heads,
                                                    w.n_loops), dtype=t.uint8, device=g.dev)
        self.kref, self.vref = self.kx[-1], self.vx[-1]
        self.kv_tokens = w.batch * w.seq_len * w.n_loops
        self.enc_b = 2 * encode_bytes(w, self.bits)  # K and V
        self.dec_b = decode_bytes(w, list(w.bits))
        self.bf_b = bf16_decode_bytes(w, w.n_loops)

    def enc_kv(self):
        self.g.rq.encode_kv_into([self.kx[l] for l in self.res_loops], [self.vx[l] for l in self.res_loops],
                                 self.kref, self.vref, self.bits, self.kc, self.ks, self.vc, self.vs,
                                 stream=self.g.stream)

    def dec(self):
        self.g.rq.decode_attn(self.q, self.kref, self.vref, self.views, out=self.out, workspace=self.ws,
                              stream=self.g.stream)

    def step(self):
        self.enc_kv()
        self.dec()

    def dec_bf16_fn(self):
        out_b = self.g.torch.empty_like(self.out)
        ws_b = self.g.torch.empty_like(self.ws)

        def f():
            self.g.rq.decode_attn_bf16(self.q, self.kx, self.vx, out=out_b, workspace=ws_b, stream=self.g.stream)
        return f

    def config(self):
        w = self.w
        return {"workload": w.name, "n_loops": w.n_loops, "batch": w.batch, "n_kv_heads": w.n_kv_heads,
                "n_q_heads": w.n_q_heads, "head_dim": w.head_dim, "seq_len": w.seq_len, "bits": list(w.bits)}


def side_workload_leg(g, case, reps):
    """A side workload: its step (per-repetition events, no flush), the decode
    and the bf16 baseline alone (cache flushed)."""
    step = stats(g.reps(case.step, reps, flush=False))
    dec = stats(g.reps(case.dec, reps))
    bf = stats(g.reps(case.dec_bf16_fn(), reps))
    enc_ms = g.back_to_back(case.enc_kv, 10)
    return {
        "config": case.config(),
        "step": {**step, "kv_tokens_per_s": case.kv_tokens / (step["ms"] * 1e-3)},
        "decode_attn": {**dec, **rate(case.dec_b, dec["ms"]), "kv_tokens_per_s": case.kv_tokens / (dec["ms"] * 1e-3),
                        "algorithmic_bytes_per_call": case.dec_b},
        "encode_kv": {"ms_per_launch": enc_ms, **rate(case.enc_b, enc_ms), "algorithmic_bytes_per_launch": case.enc_b},
        "bf16_baseline": {**bf, **rate(case.bf_b, bf["ms"]), "kv_tokens_per_s": case.kv_tokens / (bf["ms"] * 1e-3)},
        "rq_vs_bf16_decode_tokens_per_s": bf["ms"] / dec["ms"],
    }


def peak_batch_leg(g, tiles, reps):
    """The peak-batch workload: the batch grows until the cache fills about
    200 GB of HBM (less if the device has less free), for the residual cache
    (INT4 loop 0, INT2 loops 1-6, bf16 reference) and for the bf16-KV baseline
    at its own largest batch. One decode call produces the next token of every
    sequence (all 8 loops), so tokens/s = batch / call time. The batch repeats
    eight host-drawn entries (decode time does not depend on the values).
    Then the encode of the seven residual loops of K and V (one rq_encode_kv
    launch) at the largest batch whose bf16 states and outputs fit the budget."""
    torch, rq = g.torch, g.rq
    w8 = tiles["w"]
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    budget = min(workloads.PEAK_CACHE_BUDGET, free - 16 * 2**30)
    b_rq = workloads.peak_batch(workloads.cache_bytes_per_sequence(w8, w8.bits), budget)
    b_bf = workloads.peak_batch(workloads.bf16_cache_bytes_per_sequence(w8, w8.n_loops), budget)
    if b_bf < workloads.PEAK_TILE:
        return {"skipped": f"{free / 1e9:.0f} GB free on the device"}
    tile = workloads.tile_batch
    kref8, vref8 = g.bf16(tiles["kref"]), g.bf16(tiles["vref"])
    q8 = [g.bf16(tiles["q"][l]) for l in range(w8.n_loops)]

    def q_for(batch):
        return torch.stack([tile(q8[l], batch) for l in range(w8.n_loops)])

    out = {"workload": "peak_batch", "cache_budget_GB": budget / 1e9}
    kref, vref = tile(kref8, b_rq), tile(vref8, b_rq)
    views = []
    for l in range(w8.n_loops):
        if w8.bits[l]:
            (kw, ksc), (vw, vsc) = tiles["packed"][l]
            views.append(rq.LoopView(w8.bits[l], tile(g.words(kw), b_rq), tile(g.f16(ksc), b_rq),
                                     tile(g.words(vw), b_rq), tile(g.f16(vsc), b_rq)))
        else:
            views.append(rq.LoopView(0))
    q = q_for(b_rq)
    o = torch.empty((w8.n_loops, b_rq, w8.n_q_heads, w8.head_dim), dtype=torch.float32, device=g.dev)
    ws = torch.empty(rq.decode_workspace_bytes(b_rq, w8.n_kv_heads, w8.seq_len, w8.head_dim, w8.n_q_heads,
                                               w8.n_loops), dtype=torch.uint8, device=g.dev)
    st = stats(g.reps(lambda: rq.decode_attn(q, kref, vref, views, out=o, workspace=ws, stream=g.stream), reps,
                      flush=False))
    nbytes = decode_bytes(w8.with_batch(b_rq), list(w8.bits))
    out["rq"] = {"batch": b_rq, "cache_GB": b_rq * workloads.cache_bytes_per_sequence(w8, w8.bits) / 1e9, **st,
                 "tokens_per_s": b_rq / (st["ms"] * 1e-3), **rate(nbytes, st["ms"])}
    del kref, vref, views, q, o, ws
    torch.cuda.empty_cache()
    # bf16-KV baseline: every loop's K and V in its own allocation
    ks = [tile(kref8, b_bf) for _ in range(w8.n_loops)]
    vs = [tile(vref8, b_bf) for _ in range(w8.n_loops)]
    q = q_for(b_bf)
    o = torch.empty((w8.n_loops, b_bf, w8.n_q_heads, w8.head_dim), dtype=torch.float32, device=g.dev)
    st = stats(g.reps(lambda: rq.decode_attn_bf16(q, ks, vs, out=o, stream=g.stream), reps, flush=False))
    nbytes = bf16_decode_bytes(w8.with_batch(b_bf), w8.n_loops)
    out["bf16"] = {"batch": b_bf, "cache_GB": b_bf * workloads.bf16_cache_bytes_per_sequence(w8, w8.n_loops) / 1e9,
                   **st, "tokens_per_s": b_bf / (st["ms"] * 1e-3), **rate(nbytes, st["ms"])}
    del ks, vs, q, o
    torch.cuda.empty_cache()
    out["rq_over_bf16_tokens_per_s"] = out["rq"]["tokens_per_s"] / out["bf16"]["tokens_per_s"]
    # encode of all seven residual loops, K and V in one launch, at the largest
    # batch whose bf16 states and packed outputs fit the same budget
    b_enc = workloads.peak_batch(workloads.encode_bytes_per_sequence(w8), budget)
    res = [l for l in range(w8.n_loops) if w8.bits[l]]
    bits = [w8.bits[l] for l in res]
    kx = [tile(g.bf16(x), b_enc) for x in tiles["k_states"]]
    vx = [tile(g.bf16(x), b_enc) for x in tiles["v_states"]]
    shp = (b_enc, w8.n_kv_heads, w8.seq_len)
    kc = [torch.empty(shp + (w8.head_dim * b // 32,), dtype=torch.int32, device=g.dev) for b in bits]
    vc = [torch.empty_like(x) for x in kc]
    ksc = [torch.empty(shp + (w8.head_dim // 32,), dtype=torch.float16, device=g.dev) for _ in bits]
    vsc = [torch.empty_like(x) for x in ksc]

    def enc():
        rq.encode_kv_into([kx[l] for l in res], [vx[l] for l in res], kx[-1], vx[-1], bits, kc, ksc, vc, vsc,
                          stream=g.stream)
    st = stats(g.reps(enc, reps, flush=False))
    nbytes = 2 * encode_bytes(w8.with_batch(b_enc), bits)
    out["encode_kv"] = {"batch": b_enc, "device_GB": b_enc * workloads.encode_bytes_per_sequence(w8) / 1e9, **st,
                        **rate(nbytes, st["ms"]), "algorithmic_bytes_per_launch": nbytes}
    del kx, vx, kc, vc, ksc, vsc
    torch.cuda.empty_cache()
    return out


def layer_table_leg(g, c, reps):
    """Per-(layer, loop) width table: LAYER_BITS_L4 over four layers sharing
    the case's states, so only the widths differ between layers: one
    rq_encode_layers call per tensor, then each layer's decode."""
    rq, torch, w = g.rq, g.torch, c.w
    table = workloads.LAYER_BITS_L4
    lt = {}
    n_lay = len(table)

    def enc_layers():
        lt["k"] = rq.encode_layers([[c.kx[l] for l in c.res_loops]] * n_lay, [c.kref] * n_lay,
                                   [row[:-1] for row in table], stream=g.stream)
        lt["v"] = rq.encode_layers([[c.vx[l] for l in c.res_loops]] * n_lay, [c.vref] * n_lay,
                                   [row[:-1] for row in table], stream=g.stream)

    st = stats(g.reps(enc_layers, max(5, reps // 4)))
    lt_enc_b = 2 * sum(encode_bytes(w, row[:-1]) for row in table)
    layers = []
    for li_, row in enumerate(table):
        (lkc, lks), (lvc, lvs) = (lt["k"][0][li_], lt["k"][1][li_]), (lt["v"][0][li_], lt["v"][1][li_])
        lviews = [rq.LoopView(bl, lkc[i], lks[i], lvc[i], lvs[i]) for i, bl in enumerate(row[:-1])]
        lviews.append(rq.LoopView(0))

        def dec_layer(lviews=lviews):
            rq.decode_attn(c.q, c.kref, c.vref, lviews, out=c.out, workspace=c.ws, stream=g.stream)

        dst = stats(g.reps(dec_layer, max(5, reps // 2)))
        errs = []
        for i, bl in enumerate(row[:-1]):
            xq = rq.reconstruct(c.kref, lkc[i], lks[i], bl, stream=g.stream)
            xl = c.kx[c.res_loops[i]].float()
            errs.append(torch.linalg.vector_norm(xq - xl).item() /
                        torch.linalg.vector_norm(xl - c.kref.float()).item())
            del xq, xl
        layers.append({"layer": li_, "bits": list(row), "decode": {**dst, **rate(decode_bytes(w, list(row)),
                                                                                   dst["ms"])},
                       "kv_tokens_per_s": c.kv_tokens / (dst["ms"] * 1e-3),
                       "bytes_per_token_head": cache_bytes_per_token_head(w, list(row), True),
                       "k_residual_rel_error_per_loop": errs})
    del lt
    return {
        "table": [list(r) for r in table], "encode_all_layers": {**st, **rate(lt_enc_b, st["ms"])},
        "layers": layers,
        "what": f"rq_encode_layers of K and V over {n_lay} layers sharing the {w.name} states, then "
                "rq_decode_attn per layer with its row of the table",
    }


def main_side_legs(g, c, reps):
    """Side measurements on the main workload's cache (encoded once here)."""
    torch, rq, w = g.torch, g.rq, c.w
    res = {}
    c.enc_kv()
    torch.cuda.synchronize()
    dec = stats(g.reps(c.dec, reps))
    res["decode_attn_flushed"] = {**dec, **rate(c.dec_b, dec["ms"]),
                                  "kv_tokens_per_s": c.kv_tokens / (dec["ms"] * 1e-3)}
    bf = stats(g.reps(c.dec_bf16_fn(), reps))
    res["bf16_baseline"] = {**bf, **rate(c.bf_b, bf["ms"]), "kv_tokens_per_s": c.kv_tokens / (bf["ms"] * 1e-3),
                            "algorithmic_bytes_per_call": c.bf_b}
    res["rq_vs_bf16_decode_tokens_per_s"] = bf["ms"] / dec["ms"]
    per_loop = []
    for l in range(w.n_loops):
        ql = c.q[l:l + 1].contiguous()
        ol = torch.empty_like(c.out[:1])

        def dec_one(ql=ql, ol=ol, l=l):
            rq.decode_attn(ql, c.kref, c.vref, [c.views[l]], out=ol, stream=g.stream)

        st = stats(g.reps(dec_one, max(5, reps // 2)))
        per_loop.append({"loop": l, "bits": w.bits[l], **st, **rate(decode_bytes(w, [w.bits[l]]), st["ms"])})
    per_loop_total = sum(p["ms"] for p in per_loop)
    res["per_loop_mode"] = {"calls": per_loop, "total_ms": per_loop_total, "vs_bf16_all_loop": bf["ms"] / per_loop_total}
    rec = torch.empty(c.kref.shape, dtype=torch.float32, device=g.dev)
    st = stats(g.reps(lambda: rq.reconstruct(c.kref, c.kc[0], c.ks[0], c.bits[0], out=rec, stream=g.stream),
                      max(5, reps // 2)))
    res["reconstruct"] = {"loop": c.res_loops[0], "bits": c.bits[0], **st,
                          **rate(reconstruct_bytes(w, c.bits[0]), st["ms"])}
    del rec

    # Code / LS-scale refits (rq_encode_refit) of K: encode rate and the
    # residual-relative reconstruction error |x_hat - x| / |x - x_ref| per loop.
    refit = []
    enc_b = encode_bytes(w, c.bits)
    for k in (0, 1, 2):
        rc_c = [torch.empty_like(t) for t in c.kc]
        rc_s = [torch.empty_like(t) for t in c.ks]

        def enc_rf(k=k, rc_c=rc_c, rc_s=rc_s):
            rq.encode_into([c.kx[l] for l in c.res_loops], c.kref, c.bits, rc_c, rc_s, stream=g.stream, refits=k)

        st = stats(g.reps(enc_rf, max(5, reps // 2)))
        errs = []
        for i, l in enumerate(c.res_loops):
            xq = rq.reconstruct(c.kref, rc_c[i], rc_s[i], c.bits[i], stream=g.stream)
            xl = c.kx[l].float()
            errs.append(torch.linalg.vector_norm(xq - xl).item() / torch.linalg.vector_norm(xl - c.kref.float()).item())
            del xq, xl
        refit.append({"refits": k, **st, **rate(enc_b, st["ms"]), "residual_rel_error_per_loop": errs})
        del rc_c, rc_s
    res["encode_refits"] = refit

    # Rotation-only baseline (no reference: every loop, the final one included,
    # quantized directly after the rotation), the final loop at INT2; K tensor.
    ro_bits = [b if b else 2 for b in w.bits]
    ro = {}

    def enc_ro():
        ro["out"] = rq.encode_rotonly(c.kx, ro_bits, stream=g.stream)

    st = stats(g.reps(enc_ro, max(5, reps // 2)))
    ro_codes, ro_scales = ro["out"]
    err_rq, err_ro = [], []
    for l in range(w.n_loops):
        xl = c.kx[l].float()
        nx = torch.linalg.vector_norm(xl).item()
        xr = rq.reconstruct_rotonly(ro_codes[l], ro_scales[l], ro_bits[l], stream=g.stream)
        err_ro.append(torch.linalg.vector_norm(xr - xl).item() / nx)
        if w.bits[l]:
            i = c.res_loops.index(l)
            xq = rq.reconstruct(c.kref, c.kc[i], c.ks[i], w.bits[l], stream=g.stream)
            err_rq.append(torch.linalg.vector_norm(xq - xl).item() / nx)
            del xq
        else:
            err_rq.append(0.0)
        del xl, xr
    res["rotation_only_baseline"] = {
        "bits": ro_bits, **st, **rate(rotonly_encode_bytes(w, ro_bits), st["ms"]),
        "rel_error_per_loop": err_ro, "rq_rel_error_per_loop": err_rq,
        "bytes_per_token_head": cache_bytes_per_token_head(w, ro_bits, False),
        "rq_bytes_per_token_head": cache_bytes_per_token_head(w, list(w.bits), True),
        "bf16_bytes_per_token_head": 2 * 2 * w.head_dim * w.n_loops,
    }
    del ro

    if w.n_loops == len(workloads.LAYER_BITS_L4[0]):
        res["layer_table"] = layer_table_leg(g, c, reps)


    # Serving step (rq_decode_attn_varlen + rq_encode_append_kv): ragged prefix
    # lengths drawn in [S/2, S), every loop's current position as a one-position
    # bf16 tail, then that position appended to copies of the K and V caches.
    lrng = np.random.default_rng(w.seed)
    lens = lrng.integers(w.seq_len // 2, w.seq_len, size=w.batch).astype(np.int32)
    lens_d = torch.from_numpy(lens).to(g.dev)
    tk = [x[:, :, :1].contiguous() for x in c.kx]
    tv = [x[:, :, :1].contiguous() for x in c.vx]
    kref_s, vref_s = c.kref.clone(), c.vref.clone()
    kc_s, ks_s = [t.clone() for t in c.kc], [t.clone() for t in c.ks]
    vc_s, vs_s = [t.clone() for t in c.vc], [t.clone() for t in c.vs]
    views_s = [rq.LoopView(bl, kc_s[i], ks_s[i], vc_s[i], vs_s[i]) for i, bl in enumerate(c.bits)] + [rq.LoopView(0)]
    ws_v = torch.empty(rq.decode_varlen_workspace_bytes(w.batch, w.n_kv_heads, w.seq_len, w.head_dim,
                                                        w.n_q_heads, w.n_loops, 0, 1), dtype=torch.uint8, device=g.dev)

    def serve():
        rq.decode_attn_varlen(c.q, kref_s, vref_s, views_s, seq_lens=lens_d, tail_k=tk, tail_v=tv, out=c.out,
                              workspace=ws_v, stream=g.stream)
        rq.encode_append_kv([tk[l] for l in c.res_loops], [tv[l] for l in c.res_loops], tk[-1], tv[-1], c.bits,
                            lens_d, kref_s, vref_s, kc_s, ks_s, vc_s, vs_s, stream=g.stream)

    st = stats(g.reps(serve, reps))
    per_tok = decode_bytes(w, list(w.bits)) / (w.batch * w.seq_len)  # cache bytes per (b, position)
    sv_bytes = per_tok * float(lens.sum()) + w.batch * w.n_kv_heads * w.n_loops * 4 * w.head_dim
    res["serving_step"] = {
        **st, "prefix_tokens": int(lens.sum()), "tail_positions_per_loop": 1, **rate(sv_bytes, st["ms"]),
        "kv_tokens_per_s": float(lens.sum() + w.batch) * w.n_loops / (st["ms"] * 1e-3),
        "what": "rq_decode_attn_varlen (ragged prefixes + 1 tail position) + rq_encode_append_kv (K and V)",
    }
    del kref_s, vref_s, kc_s, ks_s, vc_s, vs_s, views_s

    # The same serving step over a block-paged copy of the cache: blocks of 128
    # positions in a shuffled order (rq_decode_attn_paged + rq_encode_append_paged_kv).
    P = 128
    nbs = w.seq_len // P
    perm = torch.from_numpy(np.random.default_rng(w.seed + 1).permutation(w.batch * nbs)).to(g.dev)
    table = perm.view(w.batch, nbs).to(torch.int32).contiguous()

    def paged(t):  # [B, H, S, row] -> [B*S/P, H, P, row], logical block n at physical perm[n]
        blocks = t.view(w.batch, w.n_kv_heads, nbs, P, t.shape[-1]).permute(0, 2, 1, 3, 4)
        blocks = blocks.reshape(w.batch * nbs, w.n_kv_heads, P, t.shape[-1])
        out_t = torch.empty_like(blocks)
        out_t[perm] = blocks
        return out_t

    kref_p, vref_p = paged(c.kref), paged(c.vref)
    kc_p, ks_p = [paged(t) for t in c.kc], [paged(t) for t in c.ks]
    vc_p, vs_p = [paged(t) for t in c.vc], [paged(t) for t in c.vs]
    views_p = [rq.LoopView(bl, kc_p[i], ks_p[i], vc_p[i], vs_p[i]) for i, bl in enumerate(c.bits)]
    views_p.append(rq.LoopView(0))

    def serve_paged():
        rq.decode_attn_paged(c.q, kref_p, vref_p, views_p, table, seq_lens=lens_d, tail_k=tk, tail_v=tv, out=c.out,
                             workspace=ws_v, stream=g.stream)
        rq.encode_append_paged_kv([tk[l] for l in c.res_loops], [tv[l] for l in c.res_loops], tk[-1], tv[-1], c.bits,
                                  lens_d, table, kref_p, vref_p, kc_p, ks_p, vc_p, vs_p, stream=g.stream)

    st = stats(g.reps(serve_paged, reps))
    res["serving_step_paged"] = {
        **st, "block_size": P, "blocks": w.batch * nbs, "prefix_tokens": int(lens.sum()), **rate(sv_bytes, st["ms"]),
        "kv_tokens_per_s": float(lens.sum() + w.batch) * w.n_loops / (st["ms"] * 1e-3),
        "what": "serving_step over a block-paged cache (shuffled blocks of 128 positions)",
    }
    del kref_p, vref_p, kc_p, ks_p, vc_p, vs_p, views_p, ws_v
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps first")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--reps", type=int, default=20, help="repetitions of each side measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="the main step, the decode calls and the encode launches only (for profiling runs)")
    ap.add_argument("--no-peak-batch", action="store_true", help="skip the peak-batch leg (about 200 GB of HBM)")
    ap.add_argument("--only-peak-batch", action="store_true",
                    help="run only the peak-batch leg and print its figures (for profiling runs)")
    ap.add_argument("--only-layer-table", action="store_true",
                    help="run only the per-(layer, loop) width table leg and print its figures (for profiling runs)")
    ap.add_argument("--no-side-workloads", action="store_true", help="skip the l4_b16_s4k and heavy_tail legs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 256 MiB device-to-device copy, five times: the reference kernel "
                         "whose FETCH_SIZE / WRITE_SIZE readings calibrate the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the ResidualQuant hot path has no cross-GPU step, and this build "
              "runs on one GPU; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    if args.only_peak_batch:
        tiles = host_peak_tiles()
        import torch

        import looped_transformer_kv_rq_amd as rq

        rq._load()
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps({"peak_batch": peak_batch_leg(Gpu(torch, rq, dev), tiles, args.reps)}), flush=True)
        return

    w = workloads.WORKLOADS[args.workload]
    if w.name == "peak_batch":
        print("the peak-batch workload does not fit bf16 loop states for encode on one GPU; "
              "its decode is the peak-batch leg", file=sys.stderr)
        sys.exit(2)
    if args.only_layer_table:
        if w.n_loops != len(workloads.LAYER_BITS_L4[0]):
            print(f"the width table has {len(workloads.LAYER_BITS_L4[0])} loops per layer; {w.name} has "
                  f"{w.n_loops}", file=sys.stderr)
            sys.exit(2)
        host = host_states(w)
        import torch

        import looped_transformer_kv_rq_amd as rq

        rq._load()
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        g = Gpu(torch, rq, dev)
        case = Case(g, w, host)
        del host
        print(json.dumps({"layer_table": layer_table_leg(g, case, args.reps)}), flush=True)
        return
    cpu = None if (args.no_cpu_baseline or args.only_step) else cpu_baseline(w)

    # every input of every leg, drawn on the host before the GPU is used
    side_names = [] if (args.only_step or args.no_side_workloads) else [n for n in SIDE_WORKLOADS if n != w.name]
    host_main = host_states(w)
    host_side = {n: host_states(workloads.WORKLOADS[n]) for n in side_names}
    peak_tiles = None if (args.only_step or args.no_peak_batch) else host_peak_tiles()

    import torch

    import looped_transformer_kv_rq_amd as rq

    rq._load()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = Gpu(torch, rq, dev)
    main_case = Case(g, w, host_main)
    side_cases = {n: Case(g, workloads.WORKLOADS[n], host_side[n]) for n in side_names}
    del host_main, host_side
    torch.cuda.synchronize()

    # ---- the main step: W untimed steps, then K steps between one pair of
    # events with nothing between the launches
    Ev = torch.cuda.Event
    for _ in range(args.warmup):
        main_case.step()
    torch.cuda.synchronize()
    start, stop = Ev(enable_timing=True), Ev(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(g.stream)
    for _ in range(args.steps):
        main_case.step()
    stop.record(g.stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    step_ms = start.elapsed_time(stop) / args.steps

    # Per-kernel split of a step, from a separate pass with an event between
    # every two launches (each marker adds a drain, so this pass runs slower).
    marks = [[Ev(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        m = marks[k]
        m[0].record(g.stream); main_case.enc_kv()
        m[1].record(g.stream); main_case.dec()
        m[2].record(g.stream)
    torch.cuda.synchronize()
    enc_times = [m[0].elapsed_time(m[1]) for m in marks]
    dec_times = [m[1].elapsed_time(m[2]) for m in marks]
    enc_split = stats(enc_times)
    dec_split = stats(dec_times)
    marked = stats([m[0].elapsed_time(m[2]) for m in marks])

    # Roofline figures: each kernel's mean duration over the marked pass, which
    # repeats the timed steps' sequence (encode, then decode over the codes it
    # just wrote) with an event between launches, on the step's stream. Calls of
    # one kernel alone, back to back between one pair of events, are reported
    # beside them.
    dec_ms = statistics.mean(dec_times)
    enc_ms = statistics.mean(enc_times)
    n_rl = max(10, args.steps // 2)
    dec_b2b = g.back_to_back(main_case.dec, n_rl)
    enc_b2b = g.back_to_back(main_case.enc_kv, n_rl)

    # The other legs after the main step's figures, so that the step runs on a
    # device that has only run its own warm-up.
    result_side = {}
    peak = None
    if not args.only_step:
        if peak_tiles is not None:
            peak = peak_batch_leg(g, peak_tiles, 7)
        for n, case in side_cases.items():
            result_side[n] = side_workload_leg(g, case, args.reps)
            del case
        side_cases.clear()
        torch.cuda.empty_cache()
        main_side = main_side_legs(g, main_case, args.reps)

    c = main_case
    dec_gbps = c.dec_b / (dec_ms * 1e-3) / 1e9
    enc_gbps = c.enc_b / (enc_ms * 1e-3) / 1e9
    dec_traffic = _traffic("decode_attn", w.name)
    enc_traffic = _traffic("encode", w.name)
    result = {
        "metric": METRIC,
        "value": c.kv_tokens / (step_ms * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "decode: bf16 (reference) and fp16 (residual) matrix-core operands, fp32 accumulation and "
                        "softmax; encode: fp32; storage: bf16 reference, int2/int4 codes, fp16 scales",
        "data": "synthetic",
        "config": {**c.config(),
                   "step": "rq_encode_kv (K and V, one launch) + rq_decode_attn (all loops)",
                   "storage": "bf16 reference, int2/int4 residual codes, fp16 scales per 32"},
        "roofline": {
            "kernel": f"rq_decode_attn: rq_decode_partial_mfma<{w.head_dim}> + rq_combine_kernel, all "
                      f"{w.n_loops} loops in one call",
            "bound": "hbm", "achieved": dec_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": dec_gbps / HBM_PEAK_GBPS, "traffic": dec_traffic,
            "traffic_frac": None if dec_traffic is None else dec_traffic / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": c.dec_b, "launch_ms": dec_ms, "launches_timed": args.steps,
            "launch_ms_is": "mean over the marked pass (the timed steps' launch sequence, an event between launches)",
            "back_to_back_ms": dec_b2b, "back_to_back_frac": c.dec_b / (dec_b2b * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "back_to_back_calls": n_rl,
        },
        "roofline_encode": {
            "kernel": f"rq_encode_kernel<{w.head_dim}> (K and V, {len(c.bits)} loops each, one launch)",
            "bound": "hbm", "achieved": enc_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": enc_gbps / HBM_PEAK_GBPS, "traffic": enc_traffic,
            "algorithmic_bytes_per_launch": c.enc_b, "launch_ms": enc_ms, "launches_timed": args.steps,
            "back_to_back_ms": enc_b2b, "back_to_back_frac": c.enc_b / (enc_b2b * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        },
        "wall_s_timed": wall_s,
        "step_split": {"encode": enc_split, "decode": dec_split, "step_with_markers": marked,
                       "what": "a separate pass with an event between launches, per step"},
    }
    if not args.only_step:
        result.update(main_side)
        result["side_workloads"] = result_side
    if peak is not None:
        result["peak_batch"] = peak
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
