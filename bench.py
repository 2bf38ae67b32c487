"""Benchmark of paged FP8-KV attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one forward of the whole path (block-table gather, FP8 dequant,
GQA QK^T, online softmax, PV in the attention kernel; log-sum-exp merge of
split segments in a second, small kernel) over one batch of synthetic
input.  Default workload: the LLaMA-3-8B-shaped decode
batch (32 sequences, 32 query / 8 KV heads, head_dim 128, contexts uniform in
512..4096, FP8 E4M3 KV in 16-token pages of a shuffled pool).  Inputs are
resident in HBM before timing starts; each forward reads a different copy of
the KV pool from a rotation set of >= 1 GiB so that neither L2 nor the
256 MB Infinity Cache can serve the KV.  Forwards are launched as one HIP
graph of K nodes (``--eager`` launches them one by one from Python).
``--workload prefill_mqa_mix`` makes a step of two forwards enqueued back to
back on one stream: the 8 x 512-token prefill chunk, then the 64-sequence
MQA decode batch (two plans, since their head counts differ).

Prints one JSON line (rank 0): metric/value (algorithmic HBM GB/s of the
whole step), query tokens/s, the roofline of the attention kernel (its own
duration, from HIP events the library records around it on the forward's
stream), and the CPU oracle's rate on a bounded sample of the same workload
(``cpu_baseline``).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged FP8-KV GQA attention: KV HBM GB/s (% of peak), query-tokens/s at bs=32"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
ROTATION_BYTES = 1 << 30
KERNEL_SOURCE = os.path.join(ROOT, "paged_fp8_kv_attn_amd", "csrc", "attn_stream.hip")
APPEND_SOURCE = os.path.join(ROOT, "paged_fp8_kv_attn_amd", "csrc", "attn_append.hip")
ACCEPT_SOURCE = os.path.join(ROOT, "paged_fp8_kv_attn_amd", "csrc", "attn_accept.hip")
PROFILES = os.path.join(ROOT, "profiles")
# workloads made of several forwards per step, enqueued back to back on one
# stream: the chunked-prefill chunk and the MQA decode batch of one serving
# step (two plans: their head counts differ)
COMPOSITE = {"prefill_mqa_mix": ["prefill_chunk", "mqa_decode"]}


def algorithmic_counts(w) -> dict:
    """Bytes and flops the method itself must move/do per forward."""
    L = w.ctx_lens.astype(np.int64)
    Q = w.q_lens.astype(np.int64)
    pages = (L + w.page_size - 1) // w.page_size
    code_bytes = 0.5 if getattr(w, "kv_format", "e4m3") == "int4" else 1  # two INT4 codes per byte
    kv = int((L * w.num_kv_heads * w.head_dim * 2 * code_bytes).sum())
    scales = int((pages * w.num_kv_heads * 8).sum())
    bt = int((pages * 4).sum())
    qb = 4 if w.q_dtype == "f32" else 2
    ob = 4 if w.out_dtype == "f32" else 2
    q_bytes = int(Q.sum()) * w.num_q_heads * w.head_dim * qb
    out_bytes = int(Q.sum()) * w.num_q_heads * w.head_dim * ob
    lens = 8 * w.num_seqs
    pairs = int(sum(int(Q[b]) * (int(L[b]) - int(Q[b])) + int(Q[b]) * (int(Q[b]) + 1) // 2 for b in range(w.num_seqs)))
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    return dict(bytes=kv + scales + bt + q_bytes + out_bytes + lens, kv_bytes=kv, flops=flops, pairs=pairs,
                query_tokens=int(Q.sum()))


APPEND_WORKLOADS = ("append_decode", "append_prefill")


def append_counts(c) -> dict:
    """Bytes the append itself must move: the new rows read, their bytes
    written, the cached bytes of every touched page read (the page absmax
    covers them), the touched pages' scales read and written, their
    block-table entries and the lengths."""
    S = 16
    elt = 4 if c.new_dtype == "f32" else 2
    L = c.ctx_lens.astype(np.int64)
    Q = c.q_lens.astype(np.int64)
    n0 = L - Q
    touched = (L - 1) // S - n0 // S + 1
    cached_in_touched = n0 - (n0 // S) * S  # cached slots of the first touched page
    hd = c.num_kv_heads * c.head_dim
    rows = int(Q.sum()) * hd * 2 * elt
    written = int(Q.sum()) * hd * 2
    cached = int(cached_in_touched.sum()) * hd * 2
    scales = int(touched.sum()) * c.num_kv_heads * 2 * 8
    bt = int(touched.sum()) * 4
    return dict(bytes=rows + written + cached + scales + bt + 8 * c.num_seqs, kv_bytes=written, flops=0, pairs=0,
                query_tokens=int(Q.sum()))


def append_config(c) -> dict:
    return {
        "workload": c.name,
        "batch": c.num_seqs,
        "kv_heads": c.num_kv_heads,
        "head_dim": c.head_dim,
        "page_size": 16,
        "new_tokens": sorted(set(int(x) for x in c.q_lens))[:4],
        "ctx_min": int(c.ctx_lens.min()),
        "ctx_max": int(c.ctx_lens.max()),
        "new_dtype": c.new_dtype,
        "kv_format": ("int8 (two's complement), fp32 scale per (page, kv head)" if c.kv_format == "int8"
                      else "fp8_e4m3 (OCP), fp32 scale per (page, kv head)"),
        "seed": c.seed,
    }


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def append_cpu_baseline(c, counts, budget_s: float) -> dict:
    """Time the append oracle (as it stands) on the host over whole calls."""
    import oracle

    ncpu = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    calls = 0
    while True:
        oracle.paged_kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.kv_scales, c.block_table, c.ctx_lens,
                               c.q_lens, kv_format=c.kv_format)
        calls += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    return {
        "value": counts["bytes"] * calls / wall / 1e9,
        "unit": "GB/s",
        "cores": max(1, int(math.ceil(cpu / wall - 0.05))),
        "kind": "oracle",
        "sample": (f"{calls} whole append calls of the same workload (copying the pools each call), {wall:.1f} s "
                   f"wall, {cpu:.1f} s CPU on {ncpu} allowed threads; numpy oracle"),
        "threads_allowed": ncpu,
        "cpu_model": cpu_model(),
    }


ACCEPT_WORKLOADS = ("mtp_accept",)


def accept_counts(c) -> dict:
    """Bytes greedy acceptance must move: the logits, the drafts, the target
    tokens and accepted counts written."""
    B, K, V = c.num_seqs, c.num_drafts, c.vocab
    elt = c.logits.element_size()
    return dict(bytes=B * (K + 1) * V * elt + B * K * 4 + B * (K + 1) * 4 + B * 4, kv_bytes=0, flops=0, pairs=0,
                query_tokens=B * (K + 1))


def accept_config(c) -> dict:
    return {"workload": c.name, "batch": c.num_seqs, "drafts": c.num_drafts, "vocab": c.vocab,
            "logits_dtype": str(c.logits.dtype).replace("torch.", ""), "seed": c.seed}


def accept_cpu_baseline(c, counts, budget_s: float) -> dict:
    """Time the acceptance oracle (as it stands) on the host over whole calls."""
    import oracle

    ncpu = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    calls = 0
    while True:
        oracle.greedy_accept(c.logits, c.drafts)
        calls += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    return {"value": counts["bytes"] * calls / wall / 1e9, "unit": "GB/s",
            "cores": max(1, int(math.ceil(cpu / wall - 0.05))), "kind": "oracle",
            "sample": (f"{calls} whole acceptance calls of the same workload, {wall:.1f} s wall, {cpu:.1f} s CPU "
                       f"on {ncpu} allowed threads; numpy oracle"), "threads_allowed": ncpu, "cpu_model": cpu_model()}


def workload_config(w) -> dict:
    return {
        "workload": w.name,
        "batch": w.num_seqs,
        "q_heads": w.num_q_heads,
        "kv_heads": w.num_kv_heads,
        "head_dim": w.head_dim,
        "page_size": w.page_size,
        "q_len": sorted(set(int(x) for x in w.q_lens))[:4],
        "ctx_min": int(w.ctx_lens.min()),
        "ctx_max": int(w.ctx_lens.max()),
        "ctx_mean": float(w.ctx_lens.mean()),
        "kv_format": {"int8": "int8 (two's complement), fp32 scale per (page, kv head)",
                      "int4": "int4 (two's complement, two per byte), fp32 scale per (page, kv head)"}.get(
                          w.kv_format, "fp8_e4m3 (OCP), fp32 scale per (page, kv head)"),
        "q_dtype": w.q_dtype,
        "out_dtype": w.out_dtype,
        "seed": w.seed,
    }


def source_hash(path: str = KERNEL_SOURCE) -> str:
    """Hash of a kernel's source and of the local headers it includes
    (``#include "..."``, followed transitively), so a counter summary taken
    on an older kernel is not applied to a newer one."""
    h = hashlib.sha256()
    seen = set()

    def add(fp: str):
        fp = os.path.normpath(fp)
        if fp in seen:
            return
        seen.add(fp)
        with open(fp, "rb") as f:
            data = f.read()
        h.update(data)
        for m in re.finditer(rb'^\s*#\s*include\s+"([^"]+)"', data, re.M):
            add(os.path.join(os.path.dirname(fp), m.group(1).decode()))

    add(path)
    return h.hexdigest()[:16]


def attention_kernel_name(info: dict) -> str:
    """The attention kernel the plan launches: the shared-KV tile kernel for
    blocks of more than 16 query columns, the streaming kernel otherwise."""
    return "attn_tile_kernel" if info.get("shared_kv") else "attn_stream_kernel"


def counter_summary_path(workload: str, kernel: str = "attn_stream_kernel") -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload}_hbm_counters.txt")


def profile_name(w) -> str:
    """Workload name of a counter summary: INT8-KV runs have their own."""
    fmt = getattr(w, "kv_format", "e4m3")
    return w.name + ("" if fmt == "e4m3" else "_" + fmt)


def committed_traffic(workload: str, kernel: str = "attn_stream_kernel"):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE per dispatch, each
    scaled by what the same counter reads for a plain device copy of known
    size), if it was taken on the current kernel source; otherwise None."""
    path = counter_summary_path(workload, kernel)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    src = {"kv_append_kernel": APPEND_SOURCE, "argmax_partial_kernel": ACCEPT_SOURCE}.get(kernel, KERNEL_SOURCE)
    if vals.get("kernel_source_sha256_16") != source_hash(src):
        return None
    try:
        fetch = float(vals["attn_FETCH_SIZE_KiB_per_dispatch"])
        write = float(vals["attn_WRITE_SIZE_KiB_per_dispatch"])
        copy_bytes = float(vals["copy_bytes"])
        cf = float(vals["copy_FETCH_SIZE_KiB_per_dispatch"])
        cw = float(vals["copy_WRITE_SIZE_KiB_per_dispatch"])
    except (KeyError, ValueError):
        return None
    return fetch * (copy_bytes / cf) + write * (copy_bytes / cw)


STREAM_CEILING = os.path.join(PROFILES, "stream_read_ceiling.txt")


def committed_sq_counters(workload: str, kernel: str):
    """MFMA and VALU busy fractions of the attention kernel from the committed
    rocprofv3 SQ counter summary, if it was taken on the current kernel
    source; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_sq_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_hash(KERNEL_SOURCE):
        return None
    try:
        return {"mfma_busy_frac": float(vals["mfma_busy_frac"]), "valu_busy_frac": float(vals["valu_busy_frac"]),
                "coexec_frac_of_mfma_busy": float(vals["coexec_frac_of_mfma_busy"]),
                "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


def committed_stream_ceiling(w):
    """The measured streaming-read ceiling for chunks of one (page, kv head)
    of the workload (16 * head_dim bytes: 2 KB at D = 128), from the
    committed calibration summary; None when it has no such line."""
    if not os.path.exists(STREAM_CEILING) or not hasattr(w, "head_dim"):
        return None
    want = 16 * w.head_dim
    with open(STREAM_CEILING) as f:
        for line in f:
            if line.startswith("chunk_bytes"):
                parts = dict(kv.split("=") for kv in line.split())
                if int(parts["chunk_bytes"]) == want:
                    return {"GB/s": float(parts["best_GBps"]), "chunk_bytes": want,
                            "source": "profiles/stream_read_ceiling.txt"}
    return None


def stream_calibration(dev, args):
    """Streaming-read ceiling: random distinct chunks of a 2 GiB pool, 1-64 KB
    each, ~150 MB per launch (the batch-32 decode's KV bytes), read by the
    library's attn_calib_stream_read; each repetition reads another slice of
    a random permutation of the pool's chunks, so no chunk is read twice in
    a row and the 256 MB Infinity Cache cannot hold what the next launch
    reads.  Also a contiguous read of the same size (ids in order), and the
    2 KB random read with half of 16 lines per load instruction (the access
    a plain [16 slots][128 bytes] page layout would give)."""
    import torch

    from paged_fp8_kv_attn_amd import calib_stream_read, load_library

    load_library()
    pool_bytes = 2 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pool.fill_(0x5A)
    target = 150_000_000
    reps = max(5, args.reps)
    rng = np.random.default_rng(7)
    rows = []
    hipt = HipGraph()
    for chunk in (1024, 2048, 4096, 8192, 16384, 65536):
        nchunks = target // chunk
        pool_chunks = pool_bytes // chunk
        perm = rng.permutation(pool_chunks).astype(np.int32)
        for order in ("random", "sequential", "half_lines"):
            if order == "sequential" and chunk != 65536:
                continue
            if order == "half_lines" and chunk != 2048:
                continue
            for waves in (1024, 2048, 4096):
                sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
                times = []
                for r in range(reps + 1):
                    if order != "sequential":
                        lo = (r * nchunks) % (pool_chunks - nchunks)
                        ids = torch.from_numpy(perm[lo:lo + nchunks].copy()).to(dev)
                    else:
                        start = (r * nchunks) % (pool_chunks - nchunks)
                        ids = torch.arange(start, start + nchunks, dtype=torch.int32, device=dev)
                    a, b = hipt.event(), hipt.event()
                    torch.cuda.synchronize()
                    calib_stream_read(pool, ids, chunk, waves, sink, kernel_events=(a, b),
                                      access=1 if order == "half_lines" else 0)
                    torch.cuda.synchronize()
                    if r > 0:  # the first launch is a warm-up
                        times.append(hipt.elapsed_ms(a, b))
                    hipt.destroy_event(a)
                    hipt.destroy_event(b)
                med = float(np.median(times))
                rows.append({"chunk_bytes": chunk, "order": order, "waves": waves, "bytes": nchunks * chunk,
                             "median_us": med * 1e3, "GBps": nchunks * chunk / (med * 1e-3) / 1e9,
                             "min_us": float(np.min(times)) * 1e3, "max_us": float(np.max(times)) * 1e3})
                print(json.dumps(rows[-1]), flush=True)
    best = {}
    for r in rows:
        key = (r["chunk_bytes"], r["order"])
        if key not in best or r["GBps"] > best[key]["GBps"]:
            best[key] = r
    if args.summary_out:
        lines = ["# Streaming-read ceiling on MI355X (gfx950): attn_calib_stream_read reading distinct random",
                 "# chunks of a 2 GiB pool (a different slice of one random permutation per launch), ~150 MB per",
                 "# launch, 16-byte non-temporal loads, 16 lines of 1 KB in flight per wave, waves streaming equal",
                 "# contiguous shares of the chunk list; the best of 1024/2048/4096 waves, median of "
                 f"{reps} launches",
                 "# timed with HIP events attached to the kernel's dispatch.  'sequential' reads consecutive chunks;",
                 "# 'half_line' reads the 2 KB random chunks as 16 rows of 128 bytes, each load instruction touching",
                 "# half of 16 lines (32 bytes of a row per lane in two 16-byte loads).",
                 "# command: python bench.py --stream-calibration --summary-out profiles/stream_read_ceiling.txt"]
        for (chunk, order), r in sorted(best.items()):
            tag = {"random": "chunk_bytes", "sequential": "sequential_chunk_bytes",
                   "half_lines": "half_line_chunk_bytes"}[order]
            lines.append(f"{tag}={chunk} best_GBps={r['GBps']:.1f} waves={r['waves']} median_us={r['median_us']:.2f} "
                         f"bytes={r['bytes']}")
        lines.append("# all runs:")
        lines += ["# " + json.dumps(r) for r in rows]
        with open(args.summary_out, "w") as f:
            f.write("\n".join(lines) + "\n")
    print(json.dumps({"stream_ceiling": {f"{c}_{o}": round(r["GBps"], 1) for (c, o), r in sorted(best.items())}}))


class HipGraph:
    """A HIP graph captured in global capture mode straight through the HIP
    runtime (only library calls run inside the capture), so that the event
    records the library makes around its attention kernel become event nodes
    of the graph."""

    def __init__(self):
        import ctypes

        self._c = ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        vp = ctypes.c_void_p
        hip.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
        hip.hipStreamEndCapture.argtypes = [vp, ctypes.POINTER(vp)]
        hip.hipGraphInstantiate.argtypes = [ctypes.POINTER(vp), vp, vp, vp, ctypes.c_size_t]
        hip.hipGraphLaunch.argtypes = [vp, vp]
        hip.hipGraphExecDestroy.argtypes = [vp]
        hip.hipGraphDestroy.argtypes = [vp]
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        hip.hipEventDestroy.argtypes = [vp]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self._hip = hip
        self._graph = vp()
        self._exec = vp()

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with hipError {rc}")

    def capture(self, stream, body):
        c = self._c
        st = c.c_void_p(stream.cuda_stream)
        self._ok(self._hip.hipStreamBeginCapture(st, 0), "hipStreamBeginCapture")  # global mode
        try:
            body()
        finally:
            rc = self._hip.hipStreamEndCapture(st, c.byref(self._graph))
        self._ok(rc, "hipStreamEndCapture")
        self._ok(self._hip.hipGraphInstantiate(c.byref(self._exec), self._graph, None, None, 0),
                 "hipGraphInstantiate")

    def launch(self, stream):
        self._ok(self._hip.hipGraphLaunch(self._exec, self._c.c_void_p(stream.cuda_stream)), "hipGraphLaunch")

    def event(self):
        """A timing-enabled hipEvent_t made by the HIP runtime itself."""
        e = self._c.c_void_p()
        self._ok(self._hip.hipEventCreateWithFlags(self._c.byref(e), 0), "hipEventCreateWithFlags")
        return e

    def elapsed_ms(self, a, b) -> float:
        ms = self._c.c_float(0)
        self._ok(self._hip.hipEventElapsedTime(self._c.byref(ms), a, b), "hipEventElapsedTime")
        return float(ms.value)

    def destroy_event(self, e):
        self._hip.hipEventDestroy(e)

    def close(self):
        if self._exec:
            self._hip.hipGraphExecDestroy(self._exec)
            self._exec = self._c.c_void_p()
        if self._graph:
            self._hip.hipGraphDestroy(self._graph)
            self._graph = self._c.c_void_p()


def timeline_stats(a: np.ndarray, info: dict) -> dict:
    """Summary of one forward's timeline rows (int64 [rows][TIMELINE_WORDS],
    attn_plan_set_timeline): the unit of the schedule is a wave of the packed
    decode or a workgroup otherwise (its wave 0 stands for it); times in us
    from the first wave's start."""
    words = a.shape[1]
    u = a.view(np.uint64)
    typ = (u & np.uint64(15)).astype(np.int64)
    tim = (u >> np.uint64(4)).astype(np.int64)
    per_us = info["wallclock_khz"] / 1e3
    wpg = info["waves_per_group"]
    packed = info["packed"] > 0
    ran = typ[:, 0] == 1
    t0 = tim[ran, 0].min()
    us = lambda x: (x - t0) / per_us  # noqa: E731
    units = []
    for r in np.nonzero(ran)[0]:
        if not packed and r % wpg:
            continue
        ev = [(int(typ[r, i]), us(tim[r, i])) for i in range(words - 1) if typ[r, i] != 0]
        steps = [t for k, t in ev if k == 4]
        pieces, cur = [], None
        for k, t in ev:
            if k == 3:
                cur = {"start": t, "steps": []}
            elif k == 4 and cur is not None:
                cur["steps"].append(t)
            elif k == 5 and cur is not None:
                cur["end"] = t
                pieces.append(cur)
                cur = None
        entry = ev[0][1] if ev and ev[0][0] == 1 else np.nan
        sched = next((t for k, t in ev if k == 2), np.nan)
        lens = next((t for k, t in ev if k == 6), np.nan)
        first_piece = pieces[0] if pieces else None
        gaps = [b - a_ for p_ in pieces for a_, b in zip(p_["steps"], p_["steps"][1:])]
        restarts = [nx["steps"][0] - pv["end"] for pv, nx in zip(pieces, pieces[1:]) if nx["steps"]]
        units.append({"slot": (r // wpg) // max(1, info["compute_units"]), "xcd": (r // wpg) % 8,
                      "first": steps[0] if steps else np.nan,
                      "end": us(tim[r, -1]) if typ[r, -1] == 7 else np.nan, "steps": len(steps),
                      "pieces": len(pieces), "gap": float(np.median(gaps)) if gaps else np.nan,
                      "restarts": restarts, "full": len(ev) >= words - 1,
                      # the start, split: dispatch, schedule, piece set-up, first chunk's data
                      "entry": entry, "lengths": lens - entry, "sched": sched - lens,
                      "setup": (first_piece["start"] - sched) if first_piece else np.nan,
                      "first_data": (first_piece["steps"][0] - first_piece["start"])
                      if first_piece and first_piece["steps"] else np.nan})
    busy = [x for x in units if x["steps"] > 0]
    f = np.array([x["first"] for x in busy])
    e = np.array([x["end"] for x in busy])
    g = np.array([x["gap"] for x in busy if np.isfinite(x["gap"])])
    rs = np.array([t for x in busy for t in x["restarts"]])
    pct = lambda v, q: float(np.percentile(v, q)) if len(v) else None  # noqa: E731

    def corr(key):
        v = np.array([x[key] for x in busy], dtype=float)
        return float(np.corrcoef(v, e)[0, 1]) if len(v) > 2 and np.std(v) > 0 and np.std(e) > 0 else None

    slots = sorted({x["slot"] for x in busy})
    return {
        "units": len(units), "units_with_chunks": len(busy),
        "rows_full": int(sum(x["full"] for x in units)),
        "span_us": float(np.nanmax([x["end"] for x in units])),
        "first_step_us": {"p10": pct(f, 10), "median": pct(f, 50), "p90": pct(f, 90)},
        "step_interval_us": {"p10": pct(g, 10), "median": pct(g, 50), "p90": pct(g, 90)},
        "end_us": {"min": pct(e, 0), "median": pct(e, 50), "max": pct(e, 100)},
        "restart_us": {"count": int(len(rs)), "median": pct(rs, 50)},
        "start_split_us": {k: pct([x[k] for x in busy if np.isfinite(x[k])], 50)
                           for k in ("entry", "lengths", "sched", "setup", "first_data")},
        "end_corr": {"dispatch_slot": corr("slot"), "first_step": corr("first"), "pieces": corr("pieces"),
                     "steps": corr("steps"), "step_interval": corr("gap")},
        "by_slot": {str(sl): {"units": int(sum(x["slot"] == sl for x in busy)),
                              "first_step_median_us": pct([x["first"] for x in busy if x["slot"] == sl], 50),
                              "end_median_us": pct([x["end"] for x in busy if x["slot"] == sl], 50)}
                    for sl in slots},
        # workgroups go to the 8 XCDs in turn: workgroup % 8
        "by_xcd": {str(xc): {"units": int(sum(x["xcd"] == xc for x in busy)),
                             "step_interval_median_us": pct([x["gap"] for x in busy
                                                             if x["xcd"] == xc and np.isfinite(x["gap"])], 50),
                             "end_median_us": pct([x["end"] for x in busy if x["xcd"] == xc], 50),
                             "end_max_us": pct([x["end"] for x in busy if x["xcd"] == xc], 100)}
                   for xc in range(8)},
    }


def record_timelines(pt, graph, stream, graph_ms: float, args, n: int = 3) -> dict:
    """Three more forwards of part `pt`, each with the timeline hook on and
    queued behind replays of the timed steps (so the GPU is in the timed
    state when it starts); returns their summaries and the per-key medians,
    and writes the text summary to args.timeline_summary."""
    import torch
    from paged_fp8_kv_attn_amd import TIMELINE_WORDS

    info = pt.plan.info()
    rows = torch.zeros(info["grid_size"] * info["waves_per_group"] * TIMELINE_WORDS, dtype=torch.int64,
                       device=pt.q.device)
    runs = []
    for i in range(n):
        rows.zero_()
        torch.cuda.synchronize()
        if graph is not None:
            for _ in range(max(1, math.ceil(2.0 / max(graph_ms, 1e-6)))):
                graph.launch(stream)
        pt.plan.set_timeline(rows)
        pt.forward(i + 1, stream)
        pt.plan.set_timeline(None)
        torch.cuda.synchronize()
        runs.append(timeline_stats(rows.view(-1, TIMELINE_WORDS).cpu().numpy(), info))

    def med(path):
        vals = []
        for r in runs:
            v = r
            for k in path:
                v = v.get(k) if isinstance(v, dict) else None
            if v is not None:
                vals.append(v)
        return float(np.median(vals)) if vals else None

    keys = [("span_us",), ("first_step_us", "p10"), ("first_step_us", "median"), ("first_step_us", "p90"),
            ("step_interval_us", "p10"), ("step_interval_us", "median"), ("step_interval_us", "p90"),
            ("end_us", "min"), ("end_us", "median"), ("end_us", "max"), ("restart_us", "median"),
            ("start_split_us", "entry"), ("start_split_us", "lengths"), ("start_split_us", "sched"),
            ("start_split_us", "setup"),
            ("start_split_us", "first_data"),
            ("end_corr", "dispatch_slot"), ("end_corr", "first_step"), ("end_corr", "pieces"),
            ("end_corr", "steps"), ("end_corr", "step_interval")]
    medians = {".".join(k): med(k) for k in keys}
    kern = attention_kernel_name(info)
    xf = f" --kv-format {args.kv_format}" if args.kv_format != "e4m3" else ""
    lines = [f"# Per-wave timeline of {kern}, workload {args.workload} (MI355X, gfx950), recorded by the kernels "
             f"through attn_plan_set_timeline",
             f"# command: python bench.py --workload {args.workload}{xf} --steps {args.steps} --warmup {args.warmup} "
             f"--reps {args.reps} --no-cpu-baseline --timeline-summary <this file>",
             f"# kernel_source_sha256_16: {source_hash(KERNEL_SOURCE)}",
             f"# counter: s_memrealtime at {info['wallclock_khz']} kHz; {n} forwards, each queued behind replays "
             f"of the timed steps; times in us from the kernel's first wave start; a unit is a wave (packed "
             f"decode) or a workgroup (its wave 0); dispatch slot = workgroup // compute units; first step = the "
             f"unit's first chunk step; step interval = median gap between consecutive chunk steps of a piece; "
             f"restart = from a piece's end to the next piece's first step; start_split = the start's parts: "
             f"wave start (entry), lengths read and summed (lengths), from there its unit's range known "
             f"(sched), the first piece's set-up, and from there to the first chunk step (first_data); "
             f"end_corr = correlation of the "
             f"units' end times with each quantity; the recording runs copies of the kernels with the "
             f"recording compiled in, whose counter reads and stores (an event's word is stored at the "
             f"next event) make them slower than the kernels forwards otherwise run (up to 19% on the "
             f"decode, long-context, MTP, MQA and prefill workloads)",
             f"plan: grid {info['grid_size']} waves_per_group {info['waves_per_group']} packed {info['packed']} "
             f"shared_kv {info['shared_kv']} units {runs[0]['units']} with chunks {runs[0]['units_with_chunks']} "
             f"rows full {runs[0]['rows_full']}"]
    for k, v in medians.items():
        lines.append(f"median_{k}: {v:.3f}" if v is not None else f"median_{k}: none")
    for sl, d in runs[0]["by_slot"].items():
        fs = d["first_step_median_us"]
        en = d["end_median_us"]
        lines.append(f"forward0_slot{sl}: units {d['units']} first_step_median_us "
                     f"{fs:.2f} end_median_us {en:.2f}" if fs is not None and en is not None
                     else f"forward0_slot{sl}: units {d['units']}")
    for xc, d in runs[0]["by_xcd"].items():
        if d["units"]:
            lines.append(f"forward0_xcd{xc} (workgroup % 8): units {d['units']} step_interval_median_us "
                         f"{d['step_interval_median_us'] or float('nan'):.3f} end_median_us {d['end_median_us']:.2f} "
                         f"end_max_us {d['end_max_us']:.2f}")
    with open(args.timeline_summary, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return {"medians": medians, "forwards": runs}


def cpu_baseline(w, counts, budget_s: float) -> dict:
    """Time the oracle (as it stands) on the host over whole passes of the
    workload's sequences until about budget_s seconds have been spent."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
        ncpu = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(limits=ncpu)
    except Exception:  # pragma: no cover
        ncpu, limiter = os.cpu_count() or 1, None
    # sequences sampled in order; whole sequences, all heads
    done_seqs = 0
    done_bytes = 0
    done_tokens = 0
    per_seq_bytes = None
    t0 = time.perf_counter()
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    row0 = np.concatenate([[0], np.cumsum(w.q_lens)]).astype(np.int64)
    L = w.ctx_lens.astype(np.int64)
    pages = (L + w.page_size - 1) // w.page_size
    qb = 4 if w.q_dtype == "f32" else 2
    ob = 4 if w.out_dtype == "f32" else 2
    code_bytes = 0.5 if getattr(w, "kv_format", "e4m3") == "int4" else 1
    per_seq_bytes = (L * w.num_kv_heads * w.head_dim * 2 * code_bytes + pages * w.num_kv_heads * 8 + pages * 4
                     + w.q_lens.astype(np.int64) * w.num_q_heads * w.head_dim * (qb + ob) + 8)
    b = 0
    while True:
        rows = list(range(int(row0[b]), int(row0[b + 1])))
        oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens, w.q_lens,
                               num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, rows=rows)
        done_seqs += 1
        done_bytes += int(per_seq_bytes[b])
        done_tokens += int(w.q_lens[b])
        b = (b + 1) % w.num_seqs
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {
        "value": done_bytes / wall / 1e9,
        "unit": "GB/s",
        "cores": max(1, int(math.ceil(cpu / wall - 0.05))),
        "kind": "oracle",
        "sample": (f"{done_seqs} sequence forwards (whole sequences in order, all heads) of the same workload, "
                   f"{wall:.1f} s wall, {cpu:.1f} s CPU on {ncpu} allowed threads; fp64 numpy oracle; "
                   f"{done_tokens / wall:.1f} query-tokens/s"),
        "query_tokens_per_s": done_tokens / wall,
        "threads_allowed": ncpu,
        "cpu_model": cpu_model(),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--reps", type=int, default=5,
                    help="timed repetitions of the K steps (each one graph launch); value from the median")
    ap.add_argument("--workload", default="llama3_8b_decode")
    ap.add_argument("--eager", action="store_true", help="launch forwards one by one instead of one HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--stream-calibration", action="store_true",
                    help="measure the streaming-read ceiling over random chunks of 1-64 KB (attn_calib_stream_read)")
    ap.add_argument("--summary-out", default=None, help="with --stream-calibration: write the text summary here")
    ap.add_argument("--kv-format", default="e4m3", choices=["e4m3", "int8", "int4"],
                    help="KV format of the attention workloads (INT8: two's-complement bytes times the page "
                         "scale; INT4: two 4-bit codes per byte, attention workloads of head_dim 128 only)")
    ap.add_argument("--kv-piece-len", type=int, default=0,
                    help="attention workloads: plans with this kv_piece_len (batch-invariant fixed pieces of "
                         "this many keys, a multiple of 32; 0: the balanced split)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--timeline-summary", default=None,
                    help="attention workloads: record per-wave timelines of three more forwards "
                         "(attn_plan_set_timeline) and write their summary here")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention path runs whole on a single MI355X "
              "and this library has no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "reps": 5}))
        return

    if args.stream_calibration:
        stream_calibration(dev, args)
        return

    from paged_fp8_kv_attn_amd import Plan, load_library
    from synth import make_workload

    load_library()
    names = COMPOSITE.get(args.workload, [args.workload])
    stream = torch.cuda.current_stream()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731

    class Part:
        """One forward of the step: a workload, its plan, its inputs in HBM
        and a rotation of KV pool copies of >= 1 GiB."""

        def __init__(self, name):
            w = make_workload(name, keep_logical=False, kv_format=args.kv_format)
            self.w = w
            self.counts = algorithmic_counts(w)
            self.plan = Plan(num_seqs=w.num_seqs, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                             head_dim=w.head_dim, num_pages=w.num_pages, max_pages_per_seq=w.max_pages_per_seq,
                             max_q_len=w.max_q_len, max_ctx_len=w.max_ctx_len, q_dtype=w.q_dtype,
                             out_dtype=w.out_dtype, sm_scale=w.sm_scale,
                             num_kv_splits=0 if args.kv_piece_len else w.num_kv_splits,
                             kv_format=w.kv_format, kv_piece_len=args.kv_piece_len)
            self.q = w.q.to(dev)
            self.bt = t(w.block_table)
            self.ctx = t(w.ctx_lens)
            self.ql = t(w.q_lens)
            k0, v0, s0 = t(w.k_pages), t(w.v_pages), t(w.kv_scales)
            pool_bytes = k0.numel() + v0.numel() + s0.numel() * 4
            self.copies = max(2, math.ceil(ROTATION_BYTES / pool_bytes))
            self.pools = [(k0, v0, s0)] + [(k0.clone(), v0.clone(), s0.clone()) for _ in range(self.copies - 1)]
            out_dt = torch.float32 if w.out_dtype == "f32" else torch.bfloat16
            self.out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=out_dt, device=dev)
            self.kernel = attention_kernel_name(self.plan.info())

        def forward(self, i, st):
            k, v, s_ = self.pools[i % self.copies]
            self.plan.forward(self.q, k, v, s_, self.bt, self.ctx, self.ql, self.out, stream=st)

    class AppendPart:
        """One append call per step (attn_kv_append) on a rotation of pool
        copies of >= 1 GiB; the same rows are appended at the same positions
        every time a copy comes round."""

        def __init__(self, name):
            from synth.append import make_append_case

            c = make_append_case(name, kv_format=args.kv_format)
            self.w = c
            self.counts = append_counts(c)
            self.plan = Plan(num_seqs=c.num_seqs, num_q_heads=c.num_kv_heads, num_kv_heads=c.num_kv_heads,
                             head_dim=c.head_dim, num_pages=c.num_pages, max_pages_per_seq=c.max_pages_per_seq,
                             max_q_len=c.max_q_len, max_ctx_len=c.max_ctx_len, kv_format=c.kv_format)
            self.k_new = c.k_new.to(dev).contiguous()
            self.v_new = c.v_new.to(dev).contiguous()
            self.bt = t(c.block_table)
            self.ctx = t(c.ctx_lens)
            self.ql = t(c.q_lens)
            k0, v0, s0 = t(c.k_pages), t(c.v_pages), t(c.kv_scales)
            pool_bytes = k0.numel() + v0.numel() + s0.numel() * 4
            self.copies = max(2, math.ceil(ROTATION_BYTES / pool_bytes))
            self.pools = [(k0, v0, s0)] + [(k0.clone(), v0.clone(), s0.clone()) for _ in range(self.copies - 1)]
            self.kernel = "kv_append_kernel"

        def forward(self, i, st):
            k, v, s_ = self.pools[i % self.copies]
            self.plan.kv_append(self.k_new, self.v_new, k, v, s_, self.bt, self.ctx, self.ql, stream=st)

    class AcceptPart:
        """One greedy acceptance call per step (attn_mtp_accept) on a
        rotation of >= 1 GiB of logits copies."""

        def __init__(self, name):
            from paged_fp8_kv_attn_amd import mtp_accept, mtp_accept_workspace_size
            from synth.accept import make_accept_case

            c = make_accept_case(name)
            self.w = c
            self.counts = accept_counts(c)
            self._accept = mtp_accept
            B, K, V = c.num_seqs, c.num_drafts, c.vocab
            l0 = c.logits.to(dev).contiguous()
            self.copies = max(2, math.ceil(ROTATION_BYTES / (l0.numel() * l0.element_size())))
            self.pools = [l0] + [l0.clone() for _ in range(self.copies - 1)]
            self.drafts = t(c.drafts)
            self.targets = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
            self.n = torch.empty((B,), dtype=torch.int32, device=dev)
            self.ws = torch.empty(mtp_accept_workspace_size(B, K, V), dtype=torch.uint8, device=dev)
            self.kernel = "argmax_partial_kernel"
            self.events = None
            outer = self

            class _EvPlan:
                def set_kernel_events(self, a, b):
                    outer.events = None if a is None else (a, b)

                def info(self):
                    return {"segments_per_row": mtp_accept_workspace_size(B, K, V) // (8 * B * (K + 1))}

                def close(self):
                    pass

            self.plan = _EvPlan()

        def forward(self, i, st):
            self._accept(self.pools[i % self.copies], self.drafts, self.targets, self.n, self.ws,
                         kernel_events=self.events, stream=st)

    if args.workload in APPEND_WORKLOADS:
        parts = [AppendPart(args.workload)]
    elif args.workload in ACCEPT_WORKLOADS:
        parts = [AcceptPart(args.workload)]
    else:
        parts = [Part(n) for n in names]
    counts = {key: sum(pt.counts[key] for pt in parts) for key in parts[0].counts}

    def fwd(i, st=stream):
        for pt in parts:
            pt.forward(i, st)

    for i in range(args.warmup):
        fwd(i)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        graph = HipGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        torch.cuda.synchronize()

        def body():
            for i in range(args.steps):
                fwd(i, cap)

        graph.capture(cap, body)
        graph.launch(stream)  # one untimed launch of the captured steps
        torch.cuda.synchronize()

    # Timed region 1: R repetitions of the K steps (one graph launch each, or
    # eager launches), each bracketed by a device synchronisation on both
    # sides and timed with HIP events; the headline is the median repetition.
    rep_ms = []
    for _ in range(max(1, args.reps)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        if graph is not None:
            graph.launch(stream)
        else:
            for i in range(args.steps):
                fwd(i)
        e1.record(stream)
        torch.cuda.synchronize()
        rep_ms.append(e0.elapsed_time(e1) / args.steps)
    ms = float(np.median(rep_ms))

    # Timed region 2: the same K steps launched one by one, each attention
    # kernel (and merge kernel) with a pair of HIP events that the library
    # attaches to that kernel's own dispatch (they take its start and end
    # timestamps).  Replays of the captured graph queued in front keep the
    # GPU busy, in the same state as in region 1, while the host enqueues
    # every step, so the steps run back to back as in region 1 (eager mode:
    # a sleep kernel does the same).
    hipt = HipGraph()
    ev = [([hipt.event() for _ in range(args.steps)], [hipt.event() for _ in range(args.steps)]) for _ in parts]
    # the attention forward launches a merge kernel; the append and the
    # acceptance do not (their events would never be recorded)
    has_merge = [isinstance(pt, Part) for pt in parts]
    mev = [([hipt.event() for _ in range(args.steps)], [hipt.event() for _ in range(args.steps)]) if hm else None
           for hm in has_merge]
    torch.cuda.synchronize()
    head_start_ms = 5.0 + 0.05 * args.steps * len(parts)  # generous: ~50 us of host time per forward
    if graph is not None:
        for _ in range(max(1, math.ceil(head_start_ms / max(ms * args.steps, 1e-6)))):
            graph.launch(stream)
    else:
        cal0 = torch.cuda.Event(enable_timing=True)
        cal1 = torch.cuda.Event(enable_timing=True)
        cal0.record(stream)
        torch.cuda._sleep(1 << 20)
        cal1.record(stream)
        torch.cuda.synchronize()
        sleep_ms_per_unit = cal0.elapsed_time(cal1) / (1 << 20)
        torch.cuda._sleep(int(head_start_ms / max(sleep_ms_per_unit, 1e-9)))
    for i in range(args.steps):
        for pt, (starts, stops), me in zip(parts, ev, mev):
            pt.plan.set_kernel_events(starts[i], stops[i])
            if me is not None:
                pt.plan.set_merge_events(me[0][i], me[1][i])
            pt.forward(i, stream)
    for pt, me in zip(parts, mev):
        pt.plan.set_kernel_events(None, None)
        if me is not None:
            pt.plan.set_merge_events(None, None)
    torch.cuda.synchronize()
    # span of the eager, back-to-back steps: from the first attention kernel's
    # start to the last step's last kernel end
    eager_span_ms = hipt.elapsed_ms(ev[0][0][0], ev[-1][1][-1]) if mev[-1] is None else \
        hipt.elapsed_ms(ev[0][0][0], mev[-1][1][-1])
    eager_step_ms = eager_span_ms / args.steps
    for pt, (starts, stops), me in zip(parts, ev, mev):
        pt.kernel_ms = [hipt.elapsed_ms(a, b) for a, b in zip(starts, stops)]
        pt.attn_ms = float(np.mean(pt.kernel_ms))
        pt.merge_ms = [hipt.elapsed_ms(a, b) for a, b in zip(*me)] if me is not None else []
        for e in starts + stops + (me[0] + me[1] if me is not None else []):
            hipt.destroy_event(e)

    timeline = None
    if args.timeline_summary and all(isinstance(pt, Part) for pt in parts):
        timeline = record_timelines(parts[0], graph, stream, ms * args.steps, args)

    def roofline(pt, traffic):
        c = pt.counts
        k_gbs = c["bytes"] / (pt.attn_ms * 1e-3) / 1e9
        k_tflops = c["flops"] / (pt.attn_ms * 1e-3) / 1e12
        if c["flops"] / max(1, c["bytes"]) > 312:  # above the bf16 ridge point
            roof = {"bound": "mfma", "achieved": k_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": k_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic}
        else:
            roof = {"bound": "hbm", "achieved": k_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": k_gbs / HBM_PEAK_GBS, "traffic": traffic}
        if roof["bound"] == "hbm":
            ceil = committed_stream_ceiling(pt.w)
            if ceil is not None:
                roof["stream_ceiling"] = {"GB/s": ceil["GB/s"], "chunk_bytes": ceil["chunk_bytes"],
                                          "frac": k_gbs / ceil["GB/s"], "source": ceil["source"]}
        sq = None if args.kv_piece_len else committed_sq_counters(profile_name(pt.w), pt.kernel)
        if sq is not None:
            roof["sq_counters"] = sq
        if pt.merge_ms:
            roof["merge_avg_us"] = float(np.mean(pt.merge_ms)) * 1e3
        roof.update({"kernel": pt.kernel, "kernel_avg_us": pt.attn_ms * 1e3,
                     "kernel_median_us": float(np.median(pt.kernel_ms)) * 1e3,
                     "kernel_min_us": float(np.min(pt.kernel_ms)) * 1e3,
                     "kernel_max_us": float(np.max(pt.kernel_ms)) * 1e3,
                     "algorithmic_bytes_per_launch": c["bytes"],
                     "algorithmic_flops_per_launch": c["flops"], "launches_per_step": 1})
        return roof

    # the dominant kernel: the attention kernel with the largest share of the step
    dom = max(parts, key=lambda pt: pt.attn_ms)
    # the committed counters were taken with the balanced split, not fixed pieces
    traffic_of = lambda pt: None if args.kv_piece_len else committed_traffic(profile_name(pt.w), pt.kernel)  # noqa: E731
    roof = roofline(dom, traffic_of(dom))
    if len(parts) > 1:
        roof["workload_part"] = dom.w.name

    gbs = counts["bytes"] / (ms * 1e-3) / 1e9
    tflops = counts["flops"] / (ms * 1e-3) / 1e12
    qtok = counts["query_tokens"] / (ms * 1e-3)
    if args.workload in APPEND_WORKLOADS:
        config = append_config(parts[0].w)
    elif args.workload in ACCEPT_WORKLOADS:
        config = accept_config(parts[0].w)
    elif len(parts) == 1:
        config = workload_config(parts[0].w)
    else:
        config = {"workload": args.workload, "parts": [workload_config(pt.w) for pt in parts],
                  "order": "back to back on one stream, in the order listed"}
    if args.kv_piece_len:
        config["kv_piece_len"] = args.kv_piece_len
    res = {
        "metric": METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "reps": len(rep_ms),
        "rep_ms_per_step": rep_ms,
        "rep_spread": (max(rep_ms) - min(rep_ms)) / ms if ms > 0 else None,
        "eager_ms_per_step": eager_step_ms,
        "query_tokens_per_s": qtok,
        "tflops": tflops,
        "launch": "graph" if graph is not None else "eager",
        "kv_pool_copies": [pt.copies for pt in parts] if len(parts) > 1 else parts[0].copies,
        "plan": [pt.plan.info() for pt in parts] if len(parts) > 1 else parts[0].plan.info(),
        "kernel_source_sha256_16": source_hash(APPEND_SOURCE if args.workload in APPEND_WORKLOADS else
                                               ACCEPT_SOURCE if args.workload in ACCEPT_WORKLOADS else KERNEL_SOURCE),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if len(parts) > 1:
        res["parts"] = [{"workload": pt.w.name, "roofline": roofline(pt, traffic_of(pt))}
                        for pt in parts]
    if args.workload in APPEND_WORKLOADS:
        res["dtype"] = "f32 (correctly rounded divide) -> " + ("int8" if args.kv_format == "int8" else "fp8 e4m3")
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = append_cpu_baseline(dom.w, dom.counts, args.cpu_seconds)
    elif args.workload in ACCEPT_WORKLOADS:
        res["dtype"] = "bf16 compare, int32 tokens"
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = accept_cpu_baseline(dom.w, dom.counts, args.cpu_seconds)
    elif not args.no_cpu_baseline:
        # the oracle on the first part (the dominant one for the mixed workload)
        res["cpu_baseline"] = cpu_baseline(dom.w, dom.counts, args.cpu_seconds)
        if len(parts) > 1:
            res["cpu_baseline"]["sample"] += f" (workload part {dom.w.name})"
    if timeline is not None:
        res["timeline"] = timeline
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    hipt.close()
    if graph is not None:
        graph.close()
    for pt in parts:
        pt.plan.close()


if __name__ == "__main__":
    main()
