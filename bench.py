"""Benchmark: low-bit MLA decode serving step on one MI355X.

One step = the whole hot path over one batch:
  1. mla_decode_append_partial: the new token of every sequence (position
     L_b - 1) is quantized and packed into the paged cache by the decode
     kernel's workgroup that reads that page, then split-KV attention runs
     over the packed cache, the batch's pages cut into one equal share per
     compute unit (num_splits = 0);
  2. mla_decode_combine: log-sum-exp merge of the pieces.
With --unfused the append is a separate mla_quant_append launch.
The default workload is the long-context C4R4 decode: 8 sequences x 131072
tokens, 128 heads (d_c = 512 latent + d_r = 64 RoPE key), 64-token pages.
Inputs are synthetic and resident in HBM before timing; the cache is
replicated so consecutive steps read different copies (no reuse through the
256 MB last-level cache).

Prints ONE JSON line on stdout.  `value` = packed cache bytes read by the
decode per step / step time (GB/s).  `roofline` describes the split-KV decode
kernel (its average duration from HIP events on its stream), `cpu_baseline`
the CPU oracle on a bounded sample of the same workload.
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

METRIC = "decode attn cache GB/s + % HBM peak (C4R4/C2R4, 128 heads, 32K–128K ctx)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_workload(w, device, replicas):
    import torch
    import bit_mla_kv_decode_amd as mla
    from bit_mla_kv_decode_amd import workloads as W
    lens = W.seq_lens(w)
    bt, npages = W.page_table(w, lens)
    caches = [mla.alloc_cache(w.fmt, npages, device) for _ in range(replicas)]
    for b, L in enumerate(lens):
        # rows are generated on the GPU in 32K-token pieces and packed by the library
        for t0 in range(0, int(L), 32768):
            t1 = min(int(L), t0 + 32768)
            lat, rope = W.sequence_rows(w, b, t0, t1, device)
            slots = torch.from_numpy(W.slots_for(bt, b, t0, t1)).to(device)
            for c in caches:
                mla.mla_quant_append(w.fmt, lat, rope, slots, c)
    torch.cuda.synchronize()
    q = W.queries(w, device)
    new_lat, new_rope = W.new_token_rows(w, lens, device)
    new_slots = torch.from_numpy(np.array([W.slots_for(bt, b, int(L) - 1, int(L))[0]
                                           for b, L in enumerate(lens)], dtype=np.int32)).to(device)
    return lens, bt, npages, caches, q, new_lat, new_rope, new_slots


KERNEL_SOURCES = ("bit_mla_kv_decode_amd/csrc/decode.hip", "bit_mla_kv_decode_amd/csrc/common.h",
                  "bit_mla_kv_decode_amd/csrc/kernels.h", "bit_mla_kv_decode_amd/csrc/append.h")


def kernel_source_sha256():
    """SHA-256 of the decode kernel's sources with comments, blank lines and
    trailing spaces removed: edits to comments keep the counted traffic valid,
    any change to the code drops it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            txt = f.read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", "", txt)
        lines = [l.rstrip() for l in txt.split("\n")]
        h.update("\n".join(l for l in lines if l).encode())
    return h.hexdigest()


def traffic_tag(workload, fmt_override="", heads_override=0):
    """Name of a decode launch's traffic summary: the workload, then the cache
    format if it is not the workload's own, then the head count if not its own."""
    tag = workload
    if fmt_override:
        tag += "_" + fmt_override.lower()
    if heads_override:
        tag += "_h%d" % heads_override
    return tag


def counted_traffic(tag, fmt=None):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary `profiles/traffic_k_decode_flat_<tag>.md`, or None when there is none or
    the kernel sources have changed since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", "traffic_k_decode_flat_%s.md" % tag)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", txt)
    val = re.search(r"traffic_bytes_per_launch:\s*(\d+)", txt)
    if not sha or not val or sha.group(1) != kernel_source_sha256():
        return None
    return int(val.group(1))


def _cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, seqs=8):
    """Oracle decode (fp64) on the first `seqs` sequences, all heads, on the host cores."""
    import oracle
    from bit_mla_kv_decode_amd import workloads as W
    lens = W.seq_lens(w)[:seqs]
    wq = W.derive(w, batch=len(lens))
    bt, npages = W.page_table(W.derive(w, pages="contiguous"), lens)
    fmt = {"C4R4": oracle.C4R4, "C2R4": oracle.C2R4, "BF16": oracle.BF16}[w.fmt]
    cache = np.zeros(npages * oracle.page_bytes(fmt), dtype=np.uint8)
    for b, L in enumerate(lens):
        lat, rope = W.sequence_rows(w, b, 0, int(L), "cpu")
        oracle.quant_append(fmt, lat, rope, W.slots_for(bt, b, 0, int(L)), cache, npages)
    q = W.queries(wq, "cpu")
    threads = min(16, os.cpu_count() or 1)
    t = time.perf_counter()
    oracle.decode(fmt, q, cache, npages, bt, lens, w.softmax_scale, nthreads=threads)
    dt = time.perf_counter() - t
    tokens = int(lens.sum())
    from bit_mla_kv_decode_amd import mla_token_bytes
    tb = mla_token_bytes(w.fmt)
    gbs = tokens * tb / dt / 1e9
    # one thread, on the first 4096 tokens of the first sequence
    n1 = min(4096, int(lens[0]))
    t = time.perf_counter()
    oracle.decode(fmt, q[:1], cache, npages, bt[:1], np.array([n1], np.int32), w.softmax_scale, nthreads=1)
    dt1 = time.perf_counter() - t
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host": {"cpu_model": _cpu_model(), "cpus_visible": os.cpu_count()},
            "sample": "%d of %d sequences (%d tokens), all %d heads, decode only (fp64), %.1f s"
                      % (len(lens), w.batch, tokens, w.heads, dt),
            "single_thread": {"value": round(n1 * tb / dt1 / 1e9, 6), "unit": "GB/s",
                              "sample": "%d tokens of one sequence, all heads, %.2f s" % (n1, dt1)}}


def time_case(w, args, fused, S, dev, label=None, tag=None):
    """Build `w`'s caches on the GPU and time the decode step on them: returns
    the step time, the decode kernel's average time (HIP events on its stream),
    packed GB/s and the kernel's roofline block."""
    import torch
    import bit_mla_kv_decode_amd as mla
    tok_bytes = mla.mla_token_bytes(w.fmt)
    lens_all = W_seq_lens(w)
    cache_bytes = int(((lens_all.astype(np.int64) + 63) // 64).sum()) * mla.mla_page_bytes(w.fmt)
    replicas = max(1, min(4, math.ceil(1.0e9 / cache_bytes)))
    log("building %s: B=%d H=%d fmt=%s, %.1f MB packed cache x %d replicas"
        % (label or w.name, w.batch, w.heads, w.fmt, cache_bytes / 1e6, replicas))
    lens, bt, npages, caches, q, new_lat, new_rope, new_slots = build_workload(w, dev, replicas)
    B, H = w.batch, w.heads
    max_len = int(lens.max())
    ws = torch.empty(mla.mla_decode_workspace_bytes(w.fmt, B, H, S), dtype=torch.uint8, device=dev)
    out = torch.empty(B, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    bt_d = torch.from_numpy(bt).to(dev)
    sl_d = torch.from_numpy(lens).to(dev)
    stream = torch.cuda.current_stream()
    tokens = int(lens.sum())
    packed_bytes = tokens * tok_bytes
    flops = tokens * 2.0 * H * (576 + 512)          # algorithmic: Q.K^T over 576 + P.V over 512

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def decode(c):
        if fused:
            mla.mla_decode_append_partial(w.fmt, new_lat, new_rope, q, c, bt_d, sl_d, w.softmax_scale, S, ws,
                                          max_seq_len=max_len, stream=stream)
        else:
            mla.mla_decode_partial(w.fmt, q, c, bt_d, sl_d, w.softmax_scale, S, ws, max_seq_len=max_len,
                                   stream=stream)

    def step(i, timed=None):
        c = caches[i % replicas]
        if not fused:
            mla.mla_quant_append(w.fmt, new_lat, new_rope, new_slots, c, stream=stream)
        if timed is not None:
            timed[0].record(stream)
        decode(c)
        if timed is not None:
            timed[1].record(stream)
        mla.mla_decode_combine(w.fmt, B, H, S, ws, out, lse, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    ms_step = total * 1e3 / args.steps
    k_ms_step = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # the decode kernel's average launch duration: the same launches back to
    # back between two events on its stream, so that the events' own dispatch
    # gap (several us per pair) is paid once, not per launch
    burst = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    burst[0].record(stream)
    for i in range(args.steps):
        decode(caches[i % replicas])
    burst[1].record(stream)
    torch.cuda.synchronize()
    k_ms = burst[0].elapsed_time(burst[1]) / args.steps
    value = packed_bytes / (ms_step * 1e-3) / 1e9
    k_gbs = packed_bytes / (k_ms * 1e-3) / 1e9
    k_tflops = flops / (k_ms * 1e-3) / 1e12
    log("%s: step %.3f ms, decode kernel %.3f ms: %.1f GB/s packed per step (%.1f%% of HBM), kernel %.1f GB/s, "
        "%.1f TFLOP/s (%.1f%% of bf16 MFMA)" % (label or w.name, ms_step, k_ms, value, 100 * value / HBM_PEAK_GBS,
                                             k_gbs, k_tflops, 100 * k_tflops / BF16_MFMA_PEAK_TFLOPS))
    # the decode kernel's binding roof: MFMA when its algorithmic intensity is
    # above the MI355X ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/B), else HBM
    intensity = flops / packed_bytes
    if intensity > BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        bound, achieved, peak, unit = "mfma", k_tflops, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", k_gbs, HBM_PEAK_GBS, "GB/s"
    roofline = {"kernel": ("k_decode_flat (balanced split-KV partial" if S == 0 else "k_decode (split-KV partial") +
                          (", fused append)" if fused else ")"),
                "bound": bound, "achieved": round(achieved, 2),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": counted_traffic(tag) if (tag and S == 0 and fused) else None,
                "kernel_ms": round(k_ms, 4), "kernel_ms_events_per_step": round(k_ms_step, 4),
                "flops_per_launch": flops, "packed_bytes_per_launch": packed_bytes,
                "intensity_flop_per_byte": round(intensity, 1),
                "kernel_packed_gbs": round(k_gbs, 2), "kernel_hbm_peak_frac": round(k_gbs / HBM_PEAK_GBS, 4)}
    res = {"workload": w.name, "format": w.fmt, "batch": B, "heads": H, "ctx": max_len, "tokens": tokens,
           "cache_replicas": replicas, "ms_per_step": round(ms_step, 4), "value": round(value, 2), "unit": "GB/s",
           "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
           "partition": ("balanced (%d equal page shares)" % (mla.mla_decode_partial_slots(w.fmt, B, H, 0) - B)
                         if S == 0 else "%d splits per sequence" % S),
           "roofline": roofline}
    del caches, ws
    torch.cuda.empty_cache()
    return res


def W_seq_lens(w):
    from bit_mla_kv_decode_amd import workloads as W
    return W.seq_lens(w)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU's clocks take the first ~50 ms of back-to-back decode launches to
    # settle (the first launches run up to 1.6x slower); 400 untimed steps
    # cover that for every case of the default run
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="c4r4_128k")
    ap.add_argument("--splits", type=int, default=0,
                    help="0 = balanced partition over the batch; 1..64 = fixed splits per sequence")
    ap.add_argument("--heads", type=int, default=0, help="override the workload's head count (head sweep)")
    ap.add_argument("--format", default="", help="override the cache format: C4R4, C2R4 or BF16 (same data)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time the headline workload only (no C2R4 / BF16 / 16-head records)")
    ap.add_argument("--unfused", action="store_true", help="separate append launch before the decode")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by sequence; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_mla_kv_decode_amd as mla
    from bit_mla_kv_decode_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    mla.load_library()
    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    if args.heads:
        w = W.derive(w, heads=args.heads)
    if args.format:
        w = W.derive(w, fmt=args.format)
    S = args.splits
    head = time_case(w, args, not args.unfused, S, dev,
                     tag=traffic_tag(args.workload, args.format, args.heads))
    roofline = head["roofline"]

    # the other formats the metric names, each with its own roofline block:
    # C2R4 on its 64 x 32768 workload (5% outlier channels), the unquantized
    # BF16 cache on the same data (the in-house baseline kernel), BF16 on the
    # headline's data, the 16-head share of the headline cache (the HBM-bound
    # regime of a head-sharded deployment) and the mixed C2R4 serving step
    # (128 sequences of 1K-128K tokens on random pages, one token appended each)
    extra = {}
    if not args.no_extra and not args.heads and not args.format and args.workload == "c4r4_128k":
        c2 = W.WORKLOADS["c2r4_32k_outliers"]
        extra["c2r4_32k_outliers"] = time_case(c2, args, not args.unfused, S, dev,
                                               tag=traffic_tag("c2r4_32k_outliers"))
        extra["bf16_on_c2r4_32k_outliers"] = time_case(W.derive(c2, fmt="BF16"), args, not args.unfused, S, dev,
                                                       label="bf16 cache, c2r4_32k_outliers data",
                                                       tag=traffic_tag("c2r4_32k_outliers", "BF16"))
        extra["bf16_on_c4r4_128k"] = time_case(W.derive(w, fmt="BF16"), args, not args.unfused, S, dev,
                                               label="bf16 cache, c4r4_128k data", tag=traffic_tag(w.name, "BF16"))
        extra["c4r4_128k_16_heads"] = time_case(W.derive(w, heads=16), args, not args.unfused, S, dev,
                                                label="c4r4_128k, 16 heads", tag=traffic_tag(w.name, "", 16))
        extra["mixed_c2r4_serving"] = time_case(W.WORKLOADS["mixed_c2r4_serving"], args, not args.unfused, S, dev,
                                                tag=traffic_tag("mixed_c2r4_serving"))
        for lo, bf in (("c2r4_32k_outliers", "bf16_on_c2r4_32k_outliers"), (None, "bf16_on_c4r4_128k")):
            lo_ms = extra[lo]["roofline"]["kernel_ms"] if lo else roofline["kernel_ms"]
            lo_step = extra[lo]["ms_per_step"] if lo else head["ms_per_step"]
            extra[bf]["lowbit_speedup_kernel"] = round(extra[bf]["roofline"]["kernel_ms"] / lo_ms, 3)
            extra[bf]["lowbit_speedup_step"] = round(extra[bf]["ms_per_step"] / lo_step, 3)
            extra[bf]["compared_with"] = lo or w.name

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(w)
        log("cpu baseline: %s" % cpu)

    tok_bytes = mla.mla_token_bytes(w.fmt)
    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "format": w.fmt, "batch": head["batch"], "heads": head["heads"],
                   "ctx": head["ctx"], "tokens": head["tokens"], "page_size": 64,
                   "cache_replicas": head["cache_replicas"], "partition": head["partition"],
                   "step": ("quant_append(1 token/seq) + split-KV decode + LSE combine" if args.unfused else
                            "fused append(1 token/seq) + split-KV decode, then LSE combine"),
                   "hbm_peak_frac": head["hbm_peak_frac"],
                   "compression_vs_bf16": round(1152.0 / tok_bytes, 3)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if extra:
        rec["formats"] = extra
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
