#!/usr/bin/env python3
"""Benchmark of the paged-attention step (KV append + forward) on one GPU.

A step is the whole hot path over one batch: token -> request resolution,
slot derivation, rotary (when the workload has it), the KV append, the
split-KV decode + merge and the MFMA prefill.  Inputs are synthetic and
already resident in device memory when the timed region starts.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--prefill-config NAME|none]
                    [--no-cpu-baseline] [--no-flush] [--copy-calibration-mib N]
                    [--cache int8|fp8 [--k-quant tensor|channel] [--v-quant tensor|channel]]
                    [--head-sink | --smooth-softmax] [--qk-norm]
    python bench.py --summarize-pmc counter_collection.csv ...
    python bench.py --summarize-mfma KERNEL counter_collection.csv

Prints ONE JSON line.  By default it is quoted on the decode-heavy batch
(``decode_heavy_256``: 256 requests, past U[1024, 16384], H=32, Hkv=8,
D=128, block 32; 9.09 GB of K/V per step): ``value`` is the decode KV
throughput of the whole step (algorithmic decode bytes / median step time).
The same line carries a ``prefill`` object for the windowed, softcapped
prefill batch (``gemma2_prefill_window``: 8 x 2048 new tokens on 2048 past,
H=16, Hkv=8, D=256; 824.8 GFLOP per step) with its own TFLOP/s, roofline and
oracle baseline.

Timing protocol, per workload: W untimed warm-up steps, then K steps each
bracketed by its own event pair on the launch stream, with a 1 GiB scratch
write and then a 1 GiB read of another buffer (not timed) before every step:
neither the L2s nor the 256 MB memory-side cache hold the step's inputs, and
the caches hold no dirty lines whose write-back the step would pay for
("cold"; the median and p10/p90 are reported).  Then K steps after the
scratch write alone ("cold_dirty", which includes that write-back), K
back-to-back steps without either (``warm``), and K cold steps with every
launch's dispatch timestamped on its stream (the per-kernel durations behind
``roofline``).  ``hbm_ceiling`` is a plain streaming read of a 4 GiB buffer,
the practical ceiling set beside the 8 TB/s figure; ``roofline.ceiling_at_size``
is the same read over the decode's own byte count under the cold protocol.
``cpu_baseline`` times the fp64 oracle on a bounded sample of the workload on
the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV GB/s (% HBM peak); prefill attention TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16 MFMA
DEFAULT_CONFIG = "decode_heavy_256"
DEFAULT_PREFILL_CONFIG = "gemma2_prefill_window"
FLUSH_BYTES = 1 << 30          # scratch written between cold steps (> 256 MB MALL + L2s)
CEILING_BYTES = 4 << 30        # streaming-read ceiling buffer
WARMUP_SECONDS = 0.5           # default warm-up: at least this long (and 10 steps)
STAGES = ("append", "decode", "merge", "prefill", "prefill_merge", "plan", "q_norm")


def algorithmic_work(w, kv_elem_bytes=2):
    """Decode bytes (K+V of every decode row's admitted keys, once per kv head,
    at ``kv_elem_bytes`` per element, plus its fp16 Q and O rows) and prefill
    FLOPs (4*D*H per admitted pair)."""
    H, Hkv, D = w.num_heads, w.kv_num_heads, w.head_size
    q_lens = w.q_lens
    dec_bytes = 0
    pf_pairs = 0
    n_dec = 0
    W = w.local_window_size
    for b in range(w.batch_size):
        ql = int(q_lens[b])
        past = int(w.past[b])
        if ql == 1:
            kv = past + 1
            if W > 0:
                kv = min(kv, W)
            dec_bytes += kv * Hkv * D * kv_elem_bytes * 2 + 2 * H * D * 2
            n_dec += 1
        elif ql > 1:
            for j in range(ql):
                pos = past + j
                lo = max(0, pos - W + 1) if W > 0 else 0
                pf_pairs += pos + 1 - lo
    return dec_bytes, 4.0 * D * H * pf_pairs, n_dec


def traffic_from_profiles(kernel_tag: str, src_hash: str):
    """HBM bytes per launch measured by rocprofv3 counters (committed summary),
    or None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(kernel_tag)
        if not ent or ent.get("source_sha256") != src_hash:
            return None
        return ent.get("bytes_per_launch")
    except Exception:
        return None


KERNEL_SOURCES = {
    "mla": ("mla.hip", "decode_rows.h", "pa_api.hip", "pa_device.h", "pa_internal.h"),
    "decode": ("decode.hip", "decode_rows.h", "pa_api.hip", "pa_device.h", "pa_internal.h"),
    "prefill": ("prefill.hip", "prefill16.hip", "prefill32.hip", "prefill_common.h", "pa_api.hip",
                "pa_device.h", "pa_internal.h"),
}


def kernel_source_hash(kind: str) -> str:
    """Hash of the sources that decide one kernel's memory traffic (its own
    file, the shared device helpers and the host planning code)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_append_amd", "csrc")
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()


def host_cpu():
    """CPU model and the host CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def blas_threads():
    import threadpoolctl
    return sum(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
               if i.get("user_api") == "blas") or 1


def _cpu_entry(value, unit, sample):
    model, n = host_cpu()
    return {"value": round(value, 4), "unit": unit, "cores": int(blas_threads()), "kind": "oracle",
            "sample": sample, "cpu_model": model, "host_cpus": n}


def cpu_baseline(w, gpu_out, decode_rows_sample=64, prefill_rows_sample=1024,
                 target_seconds=10.0, quant=None, feat=None):
    """fp64 oracle on a bounded sample of the workload: the decode requests
    (GB/s of decode K/V bytes) or, for a prefill-only batch, the last rows of
    the first request (GFLOP/s).  Also returns the max-abs error of the GPU
    rows the sample covers.  ``quant`` = (cache dtype, K quant type, V quant
    type, K scales, V scales) runs it on the quantized pool; ``feat`` holds
    the sink / QK-Norm inputs (host arrays) of the GPU run."""
    import oracle
    from paged_kv_cache_append_amd import workloads as wl
    dec = [b for b in range(w.batch_size) if int(w.q_lens[b]) == 1][:decode_rows_sample]
    prefill = not dec
    seqs = dec if dec else [0]
    sub = wl.subset(w, seqs)
    qkw = {}
    if quant:
        cd, kq, vq, ks, vs = quant
        qkw = dict(cache_dtype=cd, k_quant_type=kq, v_quant_type=vq, k_scale=ks, v_scale=vs)
        kc = sub.code_blocks(wl.KIND_K, range(sub.num_blocks), cd)
        vc = sub.code_blocks(wl.KIND_V, range(sub.num_blocks), cd)
    else:
        kc = sub.pool_blocks(wl.KIND_K, range(sub.num_blocks))
        vc = sub.pool_blocks(wl.KIND_V, range(sub.num_blocks))
    rot = dict(cos_cache=sub.cos_cache, sin_cache=sub.sin_cache,
               rotary_interleaved=bool(sub.rotary_interleaved)) if sub.do_rotary else {}
    feat = feat or {}
    akw, fkw = {}, {}
    if "k_norm_weight" in feat:
        akw = dict(k_norm_weight=feat["k_norm_weight"], qk_norm_epsilon=feat["qk_norm_epsilon"])
        fkw = dict(q_norm_weight=feat["q_norm_weight"], qk_norm_epsilon=feat["qk_norm_epsilon"])
    if "head_sink" in feat:
        fkw["head_sink"] = feat["head_sink"]
    if feat.get("use_smooth_softmax"):
        fkw["use_smooth_softmax"] = True
    nk, nv = oracle.append_kv(kc, vc, sub.key, sub.value, sub.cum, sub.past, sub.block_table,
                              kv_num_heads=sub.kv_num_heads, head_size=sub.head_size, **rot,
                              **qkw, **akw)
    rows = None
    if prefill:
        ql = int(sub.q_lens[0])
        rows = list(range(max(0, ql - prefill_rows_sample), ql))
    # the same sample is run until about target_seconds of CPU work have passed
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref = oracle.forward(sub.query, nk, nv, sub.cum, sub.past, sub.block_table,
                             num_heads=sub.num_heads, kv_num_heads=sub.kv_num_heads,
                             head_size=sub.head_size, scale=sub.scale, softcap=sub.softcap,
                             local_window_size=sub.local_window_size, rows=rows, **rot, **qkw,
                             **fkw)
        reps += 1
        if time.perf_counter() - t0 >= target_seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    prow = sub.extra["parent_rows"]
    if prefill:
        W = sub.local_window_size
        pairs = 0
        for j in rows:
            pos = int(sub.past[0]) + j
            pairs += pos + 1 - (max(0, pos - W + 1) if W > 0 else 0)
        flops = 4.0 * sub.head_size * sub.num_heads * pairs
        err = float(np.max(np.abs(gpu_out[prow[rows]].astype(np.float64) - ref)))
        return _cpu_entry(flops / dt / 1e9, "GFLOP/s",
                          f"last {len(rows)} query rows of request 0 of {w.name} "
                          f"({flops / 1e9:.2f} GFLOP over admitted pairs), full fp64 score "
                          f"rows + softmax + PV, {dt:.2f} s per pass, {reps} passes"), err
    nbytes, _, _ = algorithmic_work(sub, 1 if quant else 2)
    err = float(np.max(np.abs(gpu_out[prow].astype(np.float64) - ref)))
    return _cpu_entry(nbytes / dt / 1e9, "GB/s",
                      f"{len(dec)} decode requests of {w.name} ({nbytes / 1e6:.1f} MB of K/V+Q/O"
                      f"{', quantized pool dequantized on gather' if quant else ''}), "
                      f"gather + full scores + softmax + PV in fp64, {dt:.2f} s per pass, "
                      f"{reps} passes"), err


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries (no GPU use)
# ---------------------------------------------------------------------------

def _strip_params(name: str) -> str:
    """Kernel name without its trailing parameter list."""
    if not name.endswith(")"):
        return name
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        depth += {")": 1, "(": -1}.get(name[i], 0)
        if depth == 0:
            return name[:i]
    return name


COPY_KERNEL = "neg_kernel"


def _pmc_means(path):
    import csv
    from collections import defaultdict
    acc = defaultdict(list)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            acc[(_strip_params(row.get("Kernel_Name", "?")), row["Counter_Name"])].append(
                float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def record_traffic(tag, kernel, fetch_csv, write_csv, copy_mib):
    """HBM bytes per launch = FETCH_SIZE * (copy bytes / copy FETCH_SIZE)
    + WRITE_SIZE * (copy bytes / copy WRITE_SIZE), each counter in KiB per
    dispatch, the copy kernel reading and writing COPY_MIB MiB."""
    copy_kib = float(copy_mib) * 1024.0
    out = {}
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        means = _pmc_means(path)
        cal = [v for (k, c), v in means.items() if COPY_KERNEL in k and c == ctr]
        val = [v for (k, c), v in means.items() if kernel in k and c == ctr]
        if len(cal) != 1 or len(val) != 1:
            raise SystemExit(f"{path}: expected one copy kernel and one '{kernel}' kernel "
                             f"with {ctr}, found {len(cal)} and {len(val)}")
        out[ctr] = (val[0], copy_kib / cal[0])
    nbytes = sum(v * f for v, f in out.values()) * 1024.0
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[tag] = {"source_sha256": kernel_source_hash(tag.split(":")[0]),
                 "bytes_per_launch": round(nbytes),
                 "fetch_kib": round(out["FETCH_SIZE"][0], 1),
                 "fetch_scale": round(out["FETCH_SIZE"][1], 5),
                 "write_kib": round(out["WRITE_SIZE"][0], 1),
                 "write_scale": round(out["WRITE_SIZE"][1], 5)}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({tag: data[tag]}))


def summarize_pmc(paths):
    """Mean of each counter per kernel over the dispatches of rocprofv3
    ``counter_collection.csv`` files (values as the profiler reports them)."""
    import csv
    from collections import defaultdict
    acc = defaultdict(list)
    for path in paths:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                short = _strip_params(row.get("Kernel_Name", "?"))[:90]
                acc[(short, row["Counter_Name"])].append(float(row["Counter_Value"]))
    print(f"{'kernel':90s} {'counter':28s} {'dispatches':>10s} {'mean':>16s}")
    for (k, c), v in sorted(acc.items()):
        print(f"{k:90s} {c:28s} {len(v):10d} {sum(v) / len(v):16.1f}")


def summarize_mfma(kernel, path, simds=1024, xcds=8, clock_ghz=2.4):
    """MFMA utilisation of one kernel from a rocprofv3 counter run holding
    SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs), GRBM_GUI_ACTIVE (GPU
    cycles while busy, which the profiler sums over the XCDs of the chip)
    and SQ_INSTS_VALU_MFMA_MOPS_F16 (units of 512 FLOPs): busy cycles over
    (active cycles of one XCD * SIMDs), and the FLOPs the matrix cores
    executed per dispatch with the rate they imply over the active time."""
    means = {c: v for (k, c), v in _pmc_means(path).items() if kernel in k}
    busy = means.get("SQ_VALU_MFMA_BUSY_CYCLES")
    active = means.get("GRBM_GUI_ACTIVE")
    mops = means.get("SQ_INSTS_VALU_MFMA_MOPS_F16")
    out = {"kernel": kernel, "counters": means}
    if active:
        out["active_cycles_per_xcd"] = active / xcds
        out["active_us_at_clock"] = active / xcds / (clock_ghz * 1e3)
    if busy is not None and active:
        out["mfma_util"] = busy / (active / xcds * simds)
    if mops is not None:
        out["mfma_flops_per_dispatch"] = mops * 512.0
        if active:
            out["mfma_tflops_over_active"] = mops * 512.0 / (active / xcds / (clock_ghz * 1e9)) / 1e12
    print(json.dumps(out, indent=1))


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def stats(ms):
    a = np.asarray(ms, np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5),
            "reps": int(a.size)}


class Flusher:
    """Run before each cold step, outside its timing: writes FLUSH_BYTES of
    scratch (afterwards neither the L2s nor the 256 MB memory-side cache hold
    the step's inputs), then, unless ``dirty``, reads FLUSH_BYTES of another
    buffer, so the caches hold clean unrelated lines: the step then pays for
    no write-back of the scratch's dirty lines, which a write alone leaves
    behind (up to the size of the memory-side cache)."""

    def __init__(self, nbytes=FLUSH_BYTES, dirty=False):
        import torch
        self.buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
        self.clean = None if dirty else torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        self.n = 0

    def __call__(self):
        import paged_kv_cache_append_amd as pa
        self.n += 1
        self.buf.fill_(self.n)
        if self.clean is not None:
            pa.stream_read(self.clean, self.sink)

    def dirty(self):
        """The scratch write alone (caches left holding dirty lines)."""
        self.n += 1
        self.buf.fill_(self.n)


def _reps(step, reps, flush):
    """``reps`` steps, each between its own pair of events on the current
    stream; ``flush`` (or None) runs before each, outside the pair."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if flush is not None:
            flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def measure(step, steps, warmup, flush):
    """Warm-up, then cold steps (scratch write + clean read before each),
    cold steps after the scratch write alone ("cold_dirty"), warm steps (back
    to back) and cold steps with every kernel's dispatch timestamped.  With
    ``warmup`` None the warm-up runs until at least WARMUP_SECONDS have passed
    (and 10 steps): an idle GPU's clocks take that long to settle."""
    import torch

    import paged_kv_cache_append_amd as pa
    if warmup is None:
        warmup = 0
        t0 = time.perf_counter()
        while warmup < 10 or time.perf_counter() - t0 < WARMUP_SECONDS:
            for _ in range(10):
                step()
            warmup += 10
            torch.cuda.synchronize()
    else:
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()
    cold = _reps(step, steps, flush)
    dirty = _reps(step, steps, getattr(flush, "dirty", None))
    warm = _reps(step, steps, None)
    pa.timing_enable(8 * steps + 16)
    _reps(step, steps, flush)
    stages = {s: pa.timing_read(s) for s in STAGES}
    pa.timing_disable()
    return {"cold": cold, "cold_dirty": dirty, "warm": warm, "stages": stages, "warmup": warmup}


def stream_ceiling(nbytes, flush, reps=10):
    """A plain streaming read of ``nbytes`` (rounded up to 16 KiB) under the
    cold protocol: the practical HBM ceiling for a read of the step's size
    (ramp-up and drain included)."""
    import torch

    import paged_kv_cache_append_amd as pa
    nbytes = max(16384, (nbytes + 16383) // 16384 * 16384)
    buf = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    pa.stream_read(buf, sink)
    ms = float(np.median(_reps(lambda: pa.stream_read(buf, sink), reps, flush)))
    del buf
    return {"bytes": nbytes, "us": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def hbm_ceiling(reps=10):
    """Streaming read of a CEILING_BYTES buffer (larger than every cache):
    median GB/s over ``reps`` back-to-back reads, after WARMUP_SECONDS of
    reads (an idle GPU's clocks take that long to settle)."""
    import torch

    import paged_kv_cache_append_amd as pa
    buf = torch.ones(CEILING_BYTES // 2, dtype=torch.float16, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARMUP_SECONDS:
        for _ in range(10):
            pa.stream_read(buf, sink)
        torch.cuda.synchronize()
    ms = _reps(lambda: pa.stream_read(buf, sink), reps, None)
    del buf
    gbs = CEILING_BYTES / (float(np.median(ms)) * 1e-3) / 1e9
    return {"gbs": round(gbs, 1), "bytes": CEILING_BYTES, "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4),
            "protocol": f"pa_bench_stream_read of a 4 GiB buffer after {WARMUP_SECONDS} s of reads, "
                        f"median of {reps} back-to-back reads, each between its own event pair"}


# ---------------------------------------------------------------------------
# one workload
# ---------------------------------------------------------------------------

def run_workload(name, args, flush, ceiling):
    """Append + forward steps of one workload under the timing protocol;
    returns the fields of its JSON object."""
    import torch

    import paged_kv_cache_append_amd as pa
    from paged_kv_cache_append_amd import workloads as wl

    w = wl.make_workload(name)
    cd = {"fp16": wl.CACHE_FP16, "int8": wl.CACHE_INT8, "fp8": wl.CACHE_FP8}[args.cache]
    quant = None
    sc = {}
    if cd != wl.CACHE_FP16:
        qt = {"tensor": wl.QUANT_PER_TENSOR, "channel": wl.QUANT_PER_CHANNEL}
        kq, vq = qt[args.k_quant], qt[args.v_quant]
        ks = wl.draw_scales(w, wl.KIND_K, cd, kq, 7)
        vs = wl.draw_scales(w, wl.KIND_V, cd, vq, 7)
        quant = (cd, kq, vq, ks, vs)
        sc = dict(k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(vs).cuda())
    dev = wl.to_device(w, cache_dtype=cd)
    feat = {}
    frng = np.random.default_rng([w.seed, 31])
    if args.head_sink:
        feat["head_sink"] = torch.from_numpy(
            frng.uniform(-2.0, 3.0, w.num_heads).astype(np.float16)).cuda()
    if args.smooth_softmax:
        feat["use_smooth_softmax"] = 1
    if args.qk_norm:
        for k in ("q_norm_weight", "k_norm_weight"):
            feat[k] = torch.from_numpy(frng.uniform(0.5, 1.5, w.head_size).astype(np.float16)).cuda()
        feat["qk_norm_epsilon"] = 1e-6
    a = pa.Attn(num_heads=w.num_heads, kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                block_size=w.block_size, scale=w.scale, softcap=w.softcap,
                local_window_size=w.local_window_size, do_rotary=w.do_rotary,
                rotary_interleaved=w.rotary_interleaved, cache_dtype=cd,
                k_quant_type=quant[1] if quant else 0, v_quant_type=quant[2] if quant else 0,
                **feat)
    T = w.token_count
    out = torch.empty((T, w.num_heads * w.head_size), dtype=torch.float16, device="cuda")
    nws = pa.forward_workspace_bytes(a, dev["key_cache"], dev["value_cache"], dev["block_table"],
                                     dev["cum"], dev["past"], T, **sc)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    plan = pa.describe_plan(a, dev["key_cache"], dev["value_cache"], dev["block_table"],
                            dev["cum"], dev["past"], T, **sc)

    def step():
        pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                     dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"], **sc)
        pa.forward(a, dev["query"], dev["key_cache"], dev["value_cache"], dev["block_table"],
                   dev["cum"], dev["past"], dev["cos"], dev["sin"], workspace=ws, out=out, **sc)

    m = measure(step, args.steps, args.warmup, flush)
    cold, warm = stats(m["cold"]), stats(m["warm"])

    # the append alone with an explicit slot mapping (distinct slots scattered
    # over the pool, as a scheduler that owns placement hands them out): the
    # same bytes moved as the derived append of the steps above.  Runs after
    # the timed steps; the output checked below is the last step's.
    sm = torch.from_numpy(wl.random_slot_mapping(w, 4242)).to("cuda")
    pa.timing_enable(args.steps + 16)
    for _ in range(args.steps):
        flush()
        pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                     dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"],
                     slot_mapping=sm, **sc)
    torch.cuda.synchronize()
    slots_ms, slots_n = pa.timing_read("append")
    pa.timing_disable()

    kv_elem = 1 if quant else 2
    dec_bytes, pf_flops, n_dec = algorithmic_work(w, kv_elem)
    per = {s: (ms / n * 1e3 if n else 0.0) for s, (ms, n) in m["stages"].items()}  # us / launch
    ms_step = cold["median"]
    if dec_bytes:
        value, unit = dec_bytes / (ms_step * 1e-3) / 1e9, "GB/s"
        warm_value = dec_bytes / (warm["median"] * 1e-3) / 1e9
    else:
        value, unit = pf_flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
        warm_value = pf_flops / (warm["median"] * 1e-3) / 1e12
    kernels = {f"{s}_us": round(v, 3) for s, v in per.items()}
    app_bytes = 2 * T * w.kv_num_heads * w.head_size * (2 + kv_elem)
    append = {"algorithmic_bytes_per_launch": app_bytes,
              "derived_slots_us": round(per["append"], 3),
              "derived_slots_gbs": round(app_bytes / (per["append"] * 1e-6) / 1e9, 1)
              if per["append"] else None,
              "slot_mapping_us": round(slots_ms / slots_n * 1e3, 3) if slots_n else None,
              "slot_mapping_gbs": round(app_bytes / (slots_ms / slots_n * 1e-3) / 1e9, 1)
              if slots_n else None}
    if per["q_norm"]:   # the QK-Norm prologue: Q read and staged once
        kernels["q_norm_gbs"] = round(2 * T * w.num_heads * w.head_size * 2 /
                                      (per["q_norm"] * 1e-6) / 1e9, 1)
    if per["decode"]:
        kernels["decode_kernel_gbs"] = round(dec_bytes / (per["decode"] * 1e-6) / 1e9, 1)
        dm = per["decode"] + per["merge"] + per["plan"]
        kernels["decode_plan_merge_gbs"] = round(dec_bytes / (dm * 1e-6) / 1e9, 1)
        kernels["decode_plan_merge_frac"] = round(dec_bytes / (dm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    if per["prefill"] and pf_flops:
        kernels["prefill_kernel_tflops"] = round(pf_flops / (per["prefill"] * 1e-6) / 1e12, 2)
    step_frac = (dec_bytes / (HBM_PEAK_GBS * 1e9) + pf_flops / (MFMA_F16_PEAK_TFS * 1e12)) / \
        (ms_step * 1e-3)

    # dominant kernel: the one with the larger roofline time
    if dec_bytes / (HBM_PEAK_GBS * 1e9) >= pf_flops / (MFMA_F16_PEAK_TFS * 1e12):
        achieved = dec_bytes / (per["decode"] * 1e-6) / 1e9 if per["decode"] else None
        roof = {"bound": "hbm", "kernel": "decode", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                "traffic": traffic_from_profiles(
                    f"decode:{w.name}" + (f":{args.cache}" if quant else ""),
                    kernel_source_hash("decode")),
                "algorithmic_bytes_per_launch": dec_bytes, "kernel_us": round(per["decode"], 3)}
        if achieved and ceiling:
            roof["frac_of_ceiling"] = round(achieved / ceiling["gbs"], 4)
        if achieved and not args.no_flush:
            at = stream_ceiling(dec_bytes, flush)
            roof["ceiling_at_size"] = at
            roof["frac_of_ceiling_at_size"] = round(achieved / at["gbs"], 4)
    else:
        achieved = pf_flops / (per["prefill"] * 1e-6) / 1e12 if per["prefill"] else None
        roof = {"bound": "mfma", "kernel": "prefill", "achieved": achieved,
                "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": (achieved / MFMA_F16_PEAK_TFS) if achieved else None,
                "traffic": traffic_from_profiles(f"prefill:{w.name}", kernel_source_hash("prefill")),
                "algorithmic_flops_per_launch": pf_flops, "kernel_us": round(per["prefill"], 3)}
    for k in ("achieved", "frac"):
        if roof[k] is not None:
            roof[k] = round(roof[k], 4)

    cpu, err = (None, None)
    if not args.no_cpu_baseline:
        cpu, err = cpu_baseline(w, out.cpu().numpy(), quant=quant,
                                feat={k: (v.cpu().numpy() if hasattr(v, "cpu") else v)
                                      for k, v in feat.items()})
    del dev
    torch.cuda.empty_cache()
    return {
        "value": round(value, 2), "unit": unit, "ms_per_step": ms_step,
        "config": {"workload": w.name, "batch": w.batch_size, "tokens": T,
                   "num_heads": w.num_heads, "kv_num_heads": w.kv_num_heads,
                   "head_size": w.head_size, "block_size": w.block_size,
                   "cache": args.cache,
                   "k_quant": args.k_quant if quant else "none",
                   "v_quant": args.v_quant if quant else "none",
                   "head_sink": "drawn" if args.head_sink else
                   ("zero (smooth softmax)" if args.smooth_softmax else "none"),
                   "qk_norm": bool(args.qk_norm),
                   "decode_requests": n_dec, "decode_bytes": dec_bytes,
                   "prefill_flops": pf_flops, "plan": plan},
        "timing": {"cold_ms": cold, "cold_dirty_ms": stats(m["cold_dirty"]), "warm_ms": warm,
                   "warmup": m["warmup"],
                   "cold_warm_ratio": round(cold["median"] / warm["median"], 4)},
        "warm": {"value": round(warm_value, 2), "unit": unit, "ms_per_step": warm["median"],
                 "note": "back-to-back steps, caches holding what the previous step left"},
        "roofline": roof,
        "step_roofline_frac": round(step_frac, 4),
        "kernels": kernels,
        "append": append,
        "cpu_baseline": cpu,
        "parity_max_abs_err_sampled": err,
    }


# ---------------------------------------------------------------------------
# latent attention (MLA) workloads
# ---------------------------------------------------------------------------

def mla_work(w):
    """Latent attention: bytes (each admitted 576-channel row once -- V is a
    view of K -- plus the fp16 Q and O rows of every query token) and FLOPs
    (2 * H * (D + DV) per admitted key of every query token)."""
    from paged_kv_cache_append_amd import workloads as wl
    H, D, DV = w.num_heads, w.head_size, wl.MLA_V_HEAD_SIZE
    W = w.local_window_size
    nbytes = 0
    keys = 0
    for b in range(w.batch_size):
        for j in range(int(w.q_lens[b])):
            pos = int(w.past[b]) + j
            kv = pos + 1 - (max(0, pos - W + 1) if W > 0 else 0)
            nbytes += kv * D * 2 + H * D * 2 + H * DV * 2
            keys += kv
    return nbytes, 2.0 * H * (D + DV) * keys


def mla_cpu_baseline(w, gpu_out, sample=16, target_seconds=10.0):
    """The oracle on the first ``sample`` requests of a latent workload, for
    about target_seconds: GB/s of the same algorithmic bytes, and the max-abs
    error of the GPU rows it covers."""
    import oracle
    from paged_kv_cache_append_amd import workloads as wl
    sub = wl.subset(w, list(range(min(sample, w.batch_size))))
    rot = dict(cos_cache=sub.cos_cache, sin_cache=sub.sin_cache,
               rotary_interleaved=bool(sub.rotary_interleaved),
               rotary_offset=wl.MLA_ROTARY_OFFSET)
    kc = sub.pool_blocks(wl.KIND_K, range(sub.num_blocks))
    nk, _ = oracle.append_kv(kc, None, sub.key, None, sub.cum, sub.past, sub.block_table,
                             kv_num_heads=1, head_size=sub.head_size,
                             kv_cache_layout=oracle.LAYOUT_LATENT, **rot)
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref = oracle.forward(sub.query, nk, None, sub.cum, sub.past, sub.block_table,
                             num_heads=sub.num_heads, kv_num_heads=1, head_size=sub.head_size,
                             scale=sub.scale, softcap=sub.softcap,
                             local_window_size=sub.local_window_size,
                             kv_cache_layout=oracle.LAYOUT_LATENT,
                             v_head_size=wl.MLA_V_HEAD_SIZE, **rot)
        reps += 1
        if time.perf_counter() - t0 >= target_seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes, _ = mla_work(sub)
    err = float(np.max(np.abs(gpu_out[sub.extra["parent_rows"]].astype(np.float64) - ref)))
    return _cpu_entry(nbytes / dt / 1e9, "GB/s",
                      f"{sub.batch_size} requests of {w.name} ({nbytes / 1e6:.1f} MB of latent "
                      f"rows + Q/O), gather + full scores + softmax + PV in fp64, {dt:.2f} s "
                      f"per pass, {reps} passes"), err


def run_mla(name, args, flush, ceiling):
    """Latent attention (MLA) step: append of the latent rows + forward on the
    latent kernel, over an absorbed DeepSeek-shaped decode batch."""
    import torch

    import paged_kv_cache_append_amd as pa
    from paged_kv_cache_append_amd import workloads as wl
    w = wl.make_mla_workload(name)
    dev = wl.to_device(w)
    a = pa.Attn(num_heads=w.num_heads, kv_num_heads=1, head_size=w.head_size,
                block_size=w.block_size, scale=w.scale, do_rotary=1,
                rotary_interleaved=w.rotary_interleaved, kv_cache_layout=pa.LAYOUT_LATENT,
                v_head_size=wl.MLA_V_HEAD_SIZE, rotary_offset=wl.MLA_ROTARY_OFFSET)
    T = w.token_count
    out = torch.empty((T, w.num_heads * wl.MLA_V_HEAD_SIZE), dtype=torch.float16, device="cuda")
    nws = pa.forward_workspace_bytes(a, dev["key_cache"], None, dev["block_table"], dev["cum"],
                                     dev["past"], T)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    plan = pa.describe_plan(a, dev["key_cache"], None, dev["block_table"], dev["cum"],
                            dev["past"], T)

    def step():
        pa.append_kv(a, dev["key"], None, dev["key_cache"], None, dev["block_table"], dev["cum"],
                     dev["past"], dev["cos"], dev["sin"])
        pa.forward(a, dev["query"], dev["key_cache"], None, dev["block_table"], dev["cum"],
                   dev["past"], dev["cos"], dev["sin"], workspace=ws, out=out)

    m = measure(step, args.steps, args.warmup, flush)
    cold, warm = stats(m["cold"]), stats(m["warm"])
    per = {s: (ms / n * 1e3 if n else 0.0) for s, (ms, n) in m["stages"].items()}
    nbytes, flops = mla_work(w)
    t = per["decode"] * 1e-6
    gbs, tfs = nbytes / t / 1e9, flops / t / 1e12
    hbm_bound = nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_F16_PEAK_TFS * 1e12)
    roof = {"bound": "hbm" if hbm_bound else "mfma", "kernel": "mla",
            "achieved": round(gbs if hbm_bound else tfs, 4),
            "peak": HBM_PEAK_GBS if hbm_bound else MFMA_F16_PEAK_TFS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round(gbs / HBM_PEAK_GBS if hbm_bound else tfs / MFMA_F16_PEAK_TFS, 4),
            "traffic": traffic_from_profiles(f"mla:{w.name}", kernel_source_hash("mla")),
            "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
            "kernel_us": round(per["decode"], 3),
            "other_unit_frac": round(tfs / MFMA_F16_PEAK_TFS if hbm_bound
                                     else gbs / HBM_PEAK_GBS, 4)}
    if hbm_bound and ceiling:
        roof["frac_of_ceiling"] = round(gbs / ceiling["gbs"], 4)
    if hbm_bound and not args.no_flush:
        at = stream_ceiling(nbytes, flush)
        roof["ceiling_at_size"] = at
        roof["frac_of_ceiling_at_size"] = round(gbs / at["gbs"], 4)
    kernels = {f"{s}_us": round(v, 3) for s, v in per.items()}
    kernels["mla_kernel_gbs"] = round(gbs, 1)
    kernels["mla_kernel_tflops"] = round(tfs, 2)
    cpu, err = (None, None)
    if not args.no_cpu_baseline:
        cpu, err = mla_cpu_baseline(w, out.cpu().numpy())
    return {
        "value": round(nbytes / (cold["median"] * 1e-3) / 1e9, 2), "unit": "GB/s",
        "ms_per_step": cold["median"],
        "config": {"workload": w.name, "batch": w.batch_size, "tokens": T,
                   "num_heads": w.num_heads, "kv_num_heads": 1, "head_size": w.head_size,
                   "v_head_size": wl.MLA_V_HEAD_SIZE, "block_size": w.block_size,
                   "kv_cache_layout": "latent", "rotary_offset": wl.MLA_ROTARY_OFFSET,
                   "latent_bytes": nbytes, "flops": flops, "plan": plan},
        "timing": {"cold_ms": cold, "cold_dirty_ms": stats(m["cold_dirty"]), "warm_ms": warm,
                   "warmup": m["warmup"],
                   "cold_warm_ratio": round(cold["median"] / warm["median"], 4)},
        "warm": {"value": round(nbytes / (warm["median"] * 1e-3) / 1e9, 2), "unit": "GB/s",
                 "ms_per_step": warm["median"]},
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "parity_max_abs_err_sampled": err,
    }


def copy_calibration(mib):
    """A plain fp16 copy kernel over ``mib`` MiB (read N, write N), three
    times: the reference the HBM byte counters are scaled by."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for i in range(3):
        ev[i].record()
        torch.neg(src, out=dst)
    ev[3].record()
    torch.cuda.synchronize()
    ms = ev[2].elapsed_time(ev[3])   # the last launch, caches warm
    print(f"copy calibration: {mib} MiB read + {mib} MiB written per launch, "
          f"{2 * n * 2 / (ms * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50,
                    help="timed steps per pass (cold, warm and per-kernel passes)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least "
                         f"{WARMUP_SECONDS} s of steps, and 10; the count is reported)")
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--prefill-config", default=None,
                    help=f"workload of the 'prefill' object (default {DEFAULT_PREFILL_CONFIG} "
                         "with the default --config; 'none' to leave it out)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="no scratch write between the 'cold' steps (they are then warm too)")
    ap.add_argument("--cache", choices=("fp16", "int8", "fp8"), default="fp16",
                    help="element type of the paged pools (int8 / fp8: codes + fp32 scales)")
    ap.add_argument("--k-quant", choices=("tensor", "channel"), default="channel")
    ap.add_argument("--v-quant", choices=("tensor", "channel"), default="channel")
    ap.add_argument("--head-sink", action="store_true",
                    help="a sink logit per head (drawn from U[-2, 3])")
    ap.add_argument("--smooth-softmax", action="store_true", help="a zero sink for every head")
    ap.add_argument("--qk-norm", action="store_true",
                    help="QK-Norm of Q and new K with drawn weights (U[0.5, 1.5]), eps 1e-6")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain fp16 copy kernel over this many MiB (read N, "
                         "write N), three times, to scale HBM byte counters")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print per-kernel mean counter values of rocprofv3 counter "
                         "CSV files and exit (no GPU use)")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("KERNEL", "CSV"),
                    help="print the MFMA utilisation of KERNEL from a counter CSV and exit")
    ap.add_argument("--record-traffic", nargs=5,
                    metavar=("TAG", "KERNEL", "FETCH_CSV", "WRITE_CSV", "COPY_MIB"),
                    help="store HBM bytes per launch of KERNEL (substring of the kernel "
                         "name) under TAG in profiles/traffic.json, from a FETCH_SIZE and a "
                         "WRITE_SIZE counter run that both include the copy calibration of "
                         "COPY_MIB MiB, and exit (no GPU use)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    from paged_kv_cache_append_amd import workloads as wl
    latent = args.config in wl.MLA_CONFIG_NAMES
    if latent and (args.cache != "fp16" or args.head_sink or args.smooth_softmax or args.qk_norm):
        print("bench.py: the latent workloads run with an fp16 cache and no sink or QK-Norm "
              "(section 12.10)", file=sys.stderr)
        sys.exit(2)
    # a quantized pool with multi-token requests runs every token as a row of
    # the decode kernel (there is no quantized prefill kernel): measurable, and
    # reported like any other prefill batch (TFLOP/s of admitted pairs)
    pf_name = args.prefill_config
    if pf_name is None:
        pf_name = DEFAULT_PREFILL_CONFIG if (args.config == DEFAULT_CONFIG and
                                             args.cache == "fp16") else "none"

    import torch
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
    ceiling = hbm_ceiling()
    flush = (lambda: None) if args.no_flush else Flusher()
    res = run_mla(args.config, args, flush, ceiling) if latent else \
        run_workload(args.config, args, flush, ceiling)
    line = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": res["timing"]["warmup"],
            "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16", "data": "synthetic"}
    line.update({k: v for k, v in res.items() if k not in ("value", "unit", "ms_per_step")})
    line["timing"]["protocol"] = (
        "per step: its own event pair on the launch stream; 'cold' steps follow a "
        f"{FLUSH_BYTES >> 20} MiB scratch write and a {FLUSH_BYTES >> 20} MiB read of a clean "
        "buffer (outside the pair: the step's inputs are in no cache and the caches hold no "
        "dirty lines); 'cold_dirty' steps follow the scratch write alone, and so also pay "
        "for writing back the dirty lines it leaves in the 256 MB memory-side cache"
        if not args.no_flush else "per step: its own event pair; no scratch write (warm)")
    line["hbm_ceiling"] = ceiling
    if pf_name != "none":
        if pf_name in wl.MLA_CONFIG_NAMES:
            raise SystemExit("--prefill-config takes a prefill workload")
        args_pf = argparse.Namespace(**vars(args))
        args_pf.cache, args_pf.head_sink, args_pf.smooth_softmax, args_pf.qk_norm = \
            "fp16", False, False, False
        pf = run_workload(pf_name, args_pf, flush, ceiling)
        line["prefill"] = {"workload": pf_name, "value": pf["value"], "unit": pf["unit"],
                           "ms_per_step": pf["ms_per_step"],
                           **{k: v for k, v in pf.items()
                              if k not in ("value", "unit", "ms_per_step")}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
