"""Measurements of the low-bit MLA decode path on one GPU.

  python -m bit_mla_kv_decode_amd.measure [--only peaks,configs,bf16,heads,pages,...]
      JSON lines on stdout, one per measured row (progress on stderr):
      - peaks:   practical peaks from the microbenchmarks (streaming HBM read,
                 plain copy, dense bf16 MFMA loop)
      - configs: every workload: decode partial / combine / append times
                 (median over bursts of back-to-back launches, each burst
                 timed by HIP events, after a warm-up), packed GB/s, TFLOP/s
                 and the roofline fraction max(t_HBM, t_MFMA) / t; balanced
                 and fixed-split partitions
      - bf16:    the unquantized-cache kernel on the C2R4 workload's data
      - heads:   head-count sweep at the 8 x 131072 C4R4 shape
      - pages:   contiguous vs randomly permuted page tables
      - multi:   multi-token decode (s_q query tokens per sequence) on the
                 8 x 131072 C4R4 cache: 16 heads x s_q 1..8, 128 heads x 2
      - proj:    the absorbed projections (mla_absorb_q, mla_project_out) at
                 128 heads, batch 8..128: weight GB/s
      - recompute: full-size cost of the fixed-reference softmax's second pass
      - power:   socket power and GFX clocks (amd-smi) under back-to-back
                 decode launches and the dense MFMA loop
  python -m bit_mla_kv_decode_amd.measure --counters [--workload W] [--format F] [--heads H]
      the launches a rocprofv3 --pmc run counts: a 1 GiB plain copy three
      times, then the decode of workload W (default the 8 x 131072 C4R4 cache;
      its data in format F if given) in the bench configuration (fused append +
      balanced partial; with --heads, the first H of its heads) three times
  python -m bit_mla_kv_decode_amd.measure --parse-counters FETCH.csv WRITE.csv
      per-launch HBM bytes of the decode kernel from FETCH_SIZE / WRITE_SIZE,
      each scaled by what the counter reads for the copy of known size
  python -m bit_mla_kv_decode_amd.measure --parse-pmc A.csv [B.csv ...]
      the decode kernel's other counters (median over its dispatches) and
      the ratios derived from them: MFMA busy share of the SIMD-cycles,
      VALU/MFMA co-execution, instructions per MFMA, LDS bank conflicts, L2 hits
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import sys

import numpy as np

HBM_PEAK = 8.0e12
MFMA_BF16_PEAK = 2.5e15


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def emit(rec):
    print(json.dumps(rec), flush=True)
    return rec


def flops_per_token(heads):
    return 2.0 * heads * (576 + 512)


# ------------------------------------------------------------------ timing helpers

def _events(fn, iters, warmup, stream, burst=10):
    """Per-launch times (ms) of fn: after at least `warmup` calls and 60 ms of
    back-to-back launches (the clocks settle within ~50 ms), `iters` bursts of
    `burst` launches, each timed by a pair of HIP events on `stream`."""
    import time
    import torch
    t0, n = time.perf_counter(), 0
    while n < warmup or time.perf_counter() - t0 < 0.06:
        fn(n)
        n += 1
        if n % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        for j in range(burst):
            fn(i * burst + j + 1)
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) / burst for a, b in ev])


class Case:
    """A workload's caches (replicated past the 256 MB last-level cache) and decode buffers.
    Timings are per-launch averages of back-to-back bursts after a warm-up (see _events)."""

    def __init__(self, w, min_total=1.0e9, rows_hook=None):
        import torch
        import bit_mla_kv_decode_amd as mla
        from bit_mla_kv_decode_amd import workloads as W
        self.w = w
        self.lens = W.seq_lens(w)
        self.bt, self.npages = W.page_table(w, self.lens)
        first = mla.alloc_cache(w.fmt, self.npages)
        hold = w.append_new
        for b, L in enumerate(self.lens):
            end = int(L) - 1 if hold else int(L)
            for t0 in range(0, end, 32768):
                t1 = min(end, t0 + 32768)
                lat, rope = W.sequence_rows(w, b, t0, t1, "cuda")
                if rows_hook is not None:
                    rows_hook(b, t0, t1, lat)
                mla.mla_quant_append(w.fmt, lat, rope, torch.from_numpy(W.slots_for(self.bt, b, t0, t1)).cuda(), first)
        self.new_lat, self.new_rope = W.new_token_rows(w, self.lens, "cuda")
        self.new_slots = torch.from_numpy(np.array([W.slots_for(self.bt, b, int(L) - 1, int(L))[0]
                                                    for b, L in enumerate(self.lens)], np.int32)).cuda()
        if hold:
            mla.mla_quant_append(w.fmt, self.new_lat, self.new_rope, self.new_slots, first)
        used = int(((self.lens.astype(np.int64) + 63) // 64).sum()) * mla.mla_page_bytes(w.fmt)
        self.packed = int(self.lens.sum()) * mla.mla_token_bytes(w.fmt)
        self.pool_bytes = first.numel()
        reps = max(1, min(12, math.ceil(min_total / max(self.pool_bytes, 1))))
        self.caches = [first] + [first.clone() for _ in range(reps - 1)]
        self.used_page_bytes = used
        self.q = W.queries(w, "cuda")
        self.btd = torch.from_numpy(self.bt).cuda()
        self.sld = torch.from_numpy(self.lens).cuda()
        self.out = torch.empty(w.batch, w.heads, 512, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(w.batch, w.heads, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def time(self, splits=0, iters=20, warmup=5, q=None):
        import torch
        import bit_mla_kv_decode_amd as mla
        w, B = self.w, self.w.batch
        q = self.q if q is None else q
        H = int(q.shape[1])
        out = self.out if H == self.w.heads else torch.empty(B, H, 512, dtype=torch.bfloat16, device="cuda")
        lse = self.lse if H == self.w.heads else torch.empty(B, H, dtype=torch.float32, device="cuda")
        ws = torch.empty(mla.mla_decode_workspace_bytes(w.fmt, B, H, splits), dtype=torch.uint8, device="cuda")
        st = torch.cuda.current_stream()
        R = len(self.caches)
        mx = int(self.lens.max())
        part = _events(lambda i: mla.mla_decode_partial(w.fmt, q, self.caches[i % R], self.btd, self.sld,
                                                          w.softmax_scale, splits, ws, max_seq_len=mx, stream=st),
                       iters, warmup, st)
        comb = _events(lambda i: mla.mla_decode_combine(w.fmt, B, H, splits, ws, out, lse, stream=st),
                       iters, warmup, st)
        app = _events(lambda i: mla.mla_quant_append(w.fmt, self.new_lat, self.new_rope, self.new_slots,
                                                      self.caches[i % R], stream=st), iters, warmup, st)
        return float(np.median(part)), float(np.median(comb)), float(np.median(app))

    def row(self, label, splits=0, q=None, **extra):
        w = self.w
        H = w.heads if q is None else int(q.shape[1])
        tp, tc, ta = self.time(splits, q=q)
        tok = int(self.lens.sum())
        fl = tok * flops_per_token(H)
        t_hbm, t_mfma = self.packed / HBM_PEAK, fl / MFMA_BF16_PEAK
        return emit({"row": label, "workload": w.name, "format": w.fmt, "batch": w.batch, "heads": H,
                     "tokens": tok, "pages": w.pages, "partition": "balanced" if splits == 0 else "S=%d" % splits,
                     "decode_ms": round(tp, 4), "combine_ms": round(tc, 4), "append_ms": round(ta, 4),
                     "step_ms": round(tp + tc + ta, 4),
                     "packed_GBps": round(self.packed / (tp * 1e-3) / 1e9, 1),
                     "hbm_frac": round(self.packed / (tp * 1e-3) / HBM_PEAK, 4),
                     "TFLOPs": round(fl / (tp * 1e-3) / 1e12, 1),
                     "mfma_frac": round(fl / (tp * 1e-3) / MFMA_BF16_PEAK, 4),
                     "roofline_frac": round(max(t_hbm, t_mfma) / (tp * 1e-3), 4),
                     "bound": "mfma" if t_mfma > t_hbm else "hbm", "replicas": len(self.caches), **extra})


# ------------------------------------------------------------------ sections

def section_peaks():
    import torch
    from bit_mla_kv_decode_amd import peaks
    st = torch.cuda.current_stream()
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    dst = torch.empty_like(src)
    sink = torch.zeros(4096 * 256, dtype=torch.float32, device="cuda")
    best = 0.0
    for g in (1024, 2048, 4096):
        t = _events(lambda i: peaks.read(src, sink, g, st), 10, 2, st)
        best = max(best, n / (np.median(t) * 1e-3))
    emit({"row": "peak_hbm_read", "GBps": round(best / 1e9, 1), "frac_of_8TBps": round(best / HBM_PEAK, 4)})
    t = _events(lambda i: peaks.copy(src, dst, st), 10, 2, st)
    cp = 2 * n / (np.median(t) * 1e-3)
    emit({"row": "peak_copy", "GBps_read_plus_write": round(cp / 1e9, 1)})
    fl = peaks.mfma_bf16(2048, 4000, sink, st)
    t = _events(lambda i: peaks.mfma_bf16(2048, 4000, sink, st), 5, 1, st)
    mf = fl / (np.median(t) * 1e-3)
    emit({"row": "peak_mfma_bf16_32x32x16", "TFLOPs": round(mf / 1e12, 1), "frac_of_2p5PF": round(mf / MFMA_BF16_PEAK, 4)})
    del src, dst
    torch.cuda.empty_cache()
    # cycle costs, one wavefront per SIMD on every compute unit (256 workgroups)
    G = 256
    cyc = torch.zeros(2 * G, dtype=torch.int64, device="cuda")
    for chains in (1, 2):
        for nv in ((0,) if chains == 1 else (0, 2, 4, 6, 8, 12)):
            iters = 20000 // chains
            peaks.mfma_cycles(G, iters, chains, nv, cyc, sink, st)  # warm-up
            peaks.mfma_cycles(G, iters, chains, nv, cyc, sink, st)
            torch.cuda.synchronize()
            c = cyc.view(G, 2).double().cpu().numpy()
            per = float(np.median(c[:, 0])) / (iters * chains)
            ghz = float(np.median(c[:, 0] / c[:, 1])) * 0.1
            emit({"row": "mfma_cycles", "chains": chains, "valu_per_mfma": nv,
                  "cycles_per_mfma": round(per, 1), "shader_clock_GHz": round(ghz, 2)})
    lsink = torch.zeros(G * 512, dtype=torch.int32, device="cuda")
    for write in (False, True):
        for width in (4, 8, 16):
            for waves in (1, 2):
                peaks.lds(G, waves, write, 20000, cyc, lsink, st, width=width)
                by = peaks.lds(G, waves, write, 20000, cyc, lsink, st, width=width)
                torch.cuda.synchronize()
                c = float(np.median(cyc[:G].double().cpu().numpy()))
                emit({"row": "lds_bandwidth", "op": ("write_b%d" if write else "read_b%d") % (8 * width),
                      "waves_per_simd": waves, "bytes_per_cycle_per_cu": round(by / c, 1)})


def section_configs():
    import torch
    import bit_mla_kv_decode_amd as mla
    from bit_mla_kv_decode_amd import workloads as W
    for name in ("tiny_c4r4", "dsv3_c4r4_8k", "c2r4_32k_outliers", "c4r4_128k", "mixed_c2r4_serving"):
        log("config %s" % name)
        c = Case(W.WORKLOADS[name])
        extra = {}
        if name == "c4r4_128k":
            extra["compression_vs_bf16"] = round(int(c.lens.sum()) * 1152 / c.used_page_bytes, 3)
        c.row("config", 0, **extra)
        S = mla.mla_decode_num_splits(c.w.fmt, c.w.batch, c.w.heads, int(c.lens.max()))
        c.row("config_fixed_splits", S)
        del c
        torch.cuda.empty_cache()


def section_bf16():
    import torch
    from bit_mla_kv_decode_amd import workloads as W
    w = W.WORKLOADS["c2r4_32k_outliers"]
    log("bf16 baseline on %s data" % w.name)
    c = Case(W.derive(w, fmt="BF16"), min_total=0)
    c.row("bf16_baseline", 0)
    del c
    torch.cuda.empty_cache()


def section_heads():
    import torch
    from bit_mla_kv_decode_amd import workloads as W
    w = W.WORKLOADS["c4r4_128k"]
    log("head sweep on %s" % w.name)
    c = Case(w)
    for H in (16, 32, 64, 128):
        c.row("head_sweep", 0, q=c.q[:, :H].contiguous())
    del c
    torch.cuda.empty_cache()


def section_pages():
    import torch
    from bit_mla_kv_decode_amd import workloads as W
    for name in ("dsv3_c4r4_8k", "c2r4_32k_outliers", "c4r4_128k"):
        log("random pages: %s" % name)
        c = Case(W.derive(W.WORKLOADS[name], pages="random"))
        c.row("random_pages", 0)
        del c
        torch.cuda.empty_cache()


def section_multi():
    import torch
    import bit_mla_kv_decode_amd as mla
    from bit_mla_kv_decode_amd import workloads as W
    w = W.WORKLOADS["c4r4_128k"]
    log("multi-token decode on %s" % w.name)
    c = Case(w)
    B = w.batch
    st = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(5)
    for H, s_q in ((16, 1), (16, 2), (16, 4), (16, 8), (32, 4), (128, 1), (128, 2)):
        q = torch.randn(B, s_q, H, 576, device="cuda", generator=g).to(torch.bfloat16)
        ws = torch.empty(mla.mla_decode_workspace_bytes(w.fmt, B, s_q * H, 0), dtype=torch.uint8, device="cuda")
        R = len(c.caches)
        t = _events(lambda i: mla.mla_decode_multi_partial(w.fmt, q, c.caches[i % R], c.btd, c.sld, w.softmax_scale,
                                                           0, ws, max_seq_len=int(c.lens.max()), stream=st),
                    20, 5, st)
        tp = float(np.median(t))
        tok = int(c.lens.sum())
        fl = tok * flops_per_token(s_q * H)
        emit({"row": "multi_token", "workload": w.name, "heads": H, "queries": s_q, "rows": s_q * H,
              "decode_ms": round(tp, 4), "packed_GBps": round(c.packed / (tp * 1e-3) / 1e9, 1),
              "TFLOPs": round(fl / (tp * 1e-3) / 1e12, 1),
              "roofline_frac": round(max(c.packed / HBM_PEAK, fl / MFMA_BF16_PEAK) / (tp * 1e-3), 4)})
    del c
    torch.cuda.empty_cache()


def section_proj():
    import torch
    import bit_mla_kv_decode_amd as mla
    from bit_mla_kv_decode_amd import workloads as W
    st = torch.cuda.current_stream()
    H = 128
    for B in (8, 32, 128):
        q_nope, q_pe, w_uk, w_uv = (t.cuda() for t in W.absorb_inputs(B, H, seed=B))
        # several weight copies so repeats read HBM, not the last-level cache
        n = 24
        wuks = [w_uk.clone() for _ in range(n)]
        wuvs = [w_uv.clone() for _ in range(n)]
        q = torch.empty(B, H, 576, dtype=torch.bfloat16, device="cuda")
        lat = torch.randn(B, H, 512, device="cuda").to(torch.bfloat16)
        o = torch.empty(B, H, 128, dtype=torch.bfloat16, device="cuda")
        ta = float(np.median(_events(lambda i: mla.mla_absorb_q(q_nope, q_pe, wuks[i % n], q, stream=st), 20, 5, st)))
        tp = float(np.median(_events(lambda i: mla.mla_project_out(lat, wuvs[i % n], o, stream=st), 20, 5, st)))
        wbytes = H * 512 * 128 * 2
        for name, t in (("absorb_q", ta), ("project_out", tp)):
            emit({"row": "projection", "op": name, "batch": B, "heads": H, "ms": round(t, 4),
                  "weight_GBps": round(wbytes / (t * 1e-3) / 1e9, 1),
                  "TFLOPs": round(2.0 * B * H * 512 * 128 / (t * 1e-3) / 1e12, 2)})
        del wuks, wuvs
        torch.cuda.empty_cache()


def section_recompute():
    """Cost of the fixed-reference recompute: the 8 x 131072 C4R4 cache with
    keys far above the rest a few tiles into every 4096-token balanced share
    (channel 0 = 60 .. 63 at share offsets 300, 332, 364, 396, so every
    wavefront of the <= 16-row kernel meets one after its first tile).  With
    q[:, :, 0] = 0 those keys are harmless; with q[:, :, 0] in [30, 40) their
    logits rise more than kRefLift + kMaxLift = 120 log2 units above each
    piece's first tile, so every piece is computed twice.  `share` selects
    every share (worst case) or one share in 32 (one per sequence)."""
    import torch
    from bit_mla_kv_decode_amd import workloads as W
    for every in (1, 32):
        def hook(b, t0, t1, lat, every=every):
            for s0 in range(0, int(W.seq_lens(W.WORKLOADS["c4r4_128k"])[b]), 4096 * every):
                for j in range(4):
                    t = s0 + 300 + 32 * j
                    if t0 <= t < t1:
                        lat[t - t0, 0] = 60.0 + j
        case = Case(W.WORKLOADS["c4r4_128k"], rows_hook=hook)
        g = torch.Generator(device="cuda").manual_seed(7)
        for H in (128, 16):
            q = case.q[:, :H].contiguous()
            q_off = q.clone()
            q_off[:, :, 0] = 0
            q_on = q.clone()
            q_on[:, :, 0] = (30.0 + 10.0 * torch.rand(q.shape[0], H, device="cuda", generator=g)).to(q.dtype)
            t_off = case.time(0, iters=20, warmup=50, q=q_off)[0]
            t_on = case.time(0, iters=20, warmup=50, q=q_on)[0]
            emit({"row": "recompute", "heads": H, "shares_with_jump": "all" if every == 1 else "1 of 32",
                  "decode_ms_no_jump": round(t_off, 4), "decode_ms_jump": round(t_on, 4),
                  "slowdown": round(t_on / t_off, 3)})
        del case
        torch.cuda.empty_cache()


def _smi_sample():
    """Socket power (W) and the GFX clocks (MHz) amd-smi reports, or None."""
    import re
    import subprocess
    try:
        t = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    p = re.findall(r"SOCKET_POWER: (\d+) W", t)
    c = [int(x) for x in re.findall(r"^\s+CLK: (\d+) MHz", t, re.M)][:8]
    return {"socket_power_W": int(p[0]) if p else None, "gfx_clk_MHz": c}


def section_power(seconds=14.0):
    """Socket power and GFX clocks while one kind of launch runs back to back:
    the decode of three workloads (and the BF16 cache) and the dense MFMA loop
    of the peaks section.  Samples are taken after 8 and 11 seconds, once the
    power controller has settled; the board's cap is 1400 W."""
    import threading
    import time
    import torch
    import bit_mla_kv_decode_amd as mla
    from bit_mla_kv_decode_amd import peaks
    from bit_mla_kv_decode_amd import workloads as W
    st = torch.cuda.current_stream()
    emit({"row": "power_idle", **(_smi_sample() or {})})
    runs = [("c4r4_128k", 128, ""), ("c4r4_128k", 16, ""), ("c2r4_32k_outliers", 128, ""),
            ("c2r4_32k_outliers", 128, "BF16"), ("mfma", 0, "")]
    for name, H, fmt in runs:
        if name == "mfma":
            sink = torch.zeros(2048 * 256, dtype=torch.float32, device="cuda")
            fl = peaks.mfma_bf16(2048, 4000, sink, st)
            launch = lambda i: peaks.mfma_bf16(2048, 4000, sink, st)
            per, unit = fl / 1e12, "TFLOP"
        else:
            w = W.WORKLOADS[name]
            if fmt:
                w = W.derive(w, fmt=fmt)
            c = Case(w)
            q = c.q[:, :H].contiguous()
            ws = torch.empty(mla.mla_decode_workspace_bytes(w.fmt, w.batch, H, 0), dtype=torch.uint8, device="cuda")
            mx = int(c.lens.max())
            launch = lambda i, c=c, q=q, ws=ws, w=w, mx=mx: mla.mla_decode_partial(
                w.fmt, q, c.caches[i % len(c.caches)], c.btd, c.sld, w.softmax_scale, 0, ws, max_seq_len=mx, stream=st)
            per, unit = c.packed / 1e9, "GB"
        samples = []
        timer = [threading.Timer(d, lambda: samples.append(_smi_sample())) for d in (8.0, 11.0)]
        t0 = time.time()
        for tm in timer:
            tm.start()
        n = 0
        while time.time() - t0 < seconds:
            for i in range(10):
                launch(i)
            torch.cuda.synchronize()
            n += 10
        dt = time.time() - t0
        for tm in timer:
            tm.join()
        emit({"row": "power", "run": name if name == "mfma" else "%s %s %d heads" % (name, fmt or W.WORKLOADS[name].fmt, H),
              "us_per_launch": round(dt / n * 1e6, 1), "rate": round(per * n / dt, 1), "rate_unit": unit + "/s",
              "samples": samples})
        launch = None
        torch.cuda.empty_cache()


SECTIONS = {"peaks": section_peaks, "configs": section_configs, "bf16": section_bf16,
            "heads": section_heads, "pages": section_pages, "multi": section_multi, "proj": section_proj,
            "recompute": section_recompute, "power": section_power}


# ------------------------------------------------------------------ counters

def run_counters(heads=0, workload="c4r4_128k", fmt=""):
    """The launches one rocprofv3 --pmc pass counts (kernel names tell them apart):
    a plain copy, then the bench step's decode launch on `workload` (its cache
    in format `fmt` if given); heads > 0 decodes with the first `heads` heads
    of the workload's queries."""
    import torch
    import bit_mla_kv_decode_amd as mla
    from bit_mla_kv_decode_amd import peaks
    from bit_mla_kv_decode_amd import workloads as W
    st = torch.cuda.current_stream()
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        peaks.copy(src, dst, st)
    torch.cuda.synchronize()
    del src, dst
    log("copy: 3 x %d bytes" % n)
    w0 = W.WORKLOADS[workload]
    c = Case(W.derive(w0, fmt=fmt) if fmt else w0)
    w, B = c.w, c.w.batch
    H = heads if heads > 0 else w.heads
    q = c.q[:, :H].contiguous()
    ws = torch.empty(mla.mla_decode_workspace_bytes(w.fmt, B, H, 0), dtype=torch.uint8, device="cuda")
    for i in range(3):  # the bench step's decode launch: fused append + balanced partial
        mla.mla_decode_append_partial(w.fmt, c.new_lat, c.new_rope, q, c.caches[i % len(c.caches)], c.btd, c.sld,
                                      w.softmax_scale, 0, ws, max_seq_len=int(c.lens.max()), stream=st)
    torch.cuda.synchronize()
    log("decode: 3 launches, %s %s, %d heads, %d packed bytes each, %d replicas"
        % (w.name, w.fmt, H, c.packed, len(c.caches)))
    print(json.dumps({"copy_bytes": n, "packed_bytes": c.packed}), flush=True)


def _counter_rows(path):
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def _is_kernel(name, short):
    # demangled "(anonymous namespace)::k_copy(...)" / "mla::k_decode_flat<0>(...)",
    # or mangled "...6k_copy..." / "...13k_decode_flat..."
    return ("::%s(" % short in name or "::%s<" % short in name or name.startswith(short + "(")
            or ("%d%s" % (len(short), short)) in name)


def _per_dispatch(rows, short, counter):
    return [v for k, c, v in rows if _is_kernel(k, short) and c == counter]


def parse_counters(fetch_csv, write_csv, copy_bytes=1 << 30, packed_bytes=None):
    """Per-launch HBM bytes of the decode kernel, each counter scaled by its reading on the copy."""
    fr, wr = _counter_rows(fetch_csv), _counter_rows(write_csv)
    cf = _per_dispatch(fr, "k_copy", "FETCH_SIZE")
    cw = _per_dispatch(wr, "k_copy", "WRITE_SIZE")
    df = _per_dispatch(fr, "k_decode_flat", "FETCH_SIZE")
    dw = _per_dispatch(wr, "k_decode_flat", "WRITE_SIZE")
    if not (cf and cw and df and dw):
        raise SystemExit("counter files lack the copy or decode dispatches")
    f_scale = copy_bytes / float(np.median(cf))   # bytes per counted unit (nominally 1024)
    w_scale = copy_bytes / float(np.median(cw))
    rec = {"copy_FETCH_SIZE": float(np.median(cf)), "copy_WRITE_SIZE": float(np.median(cw)),
           "fetch_scale_bytes_per_unit": round(f_scale, 2), "write_scale_bytes_per_unit": round(w_scale, 2),
           "decode_FETCH_SIZE": [round(v, 1) for v in df], "decode_WRITE_SIZE": [round(v, 1) for v in dw],
           "decode_read_bytes": int(np.median(df) * f_scale), "decode_write_bytes": int(np.median(dw) * w_scale)}
    rec["decode_traffic_bytes"] = rec["decode_read_bytes"] + rec["decode_write_bytes"]
    if packed_bytes:
        rec["read_over_packed"] = round(rec["decode_read_bytes"] / packed_bytes, 4)
    return rec


SIMDS = 256 * 4  # MI355X: 256 compute units x 4 SIMDs
XCDS = 8         # GRBM_GUI_ACTIVE is reported summed over the 8 XCDs


def parse_pmc(paths):
    vals = {}
    for p in paths:
        for k, c, v in _counter_rows(p):
            if _is_kernel(k, "k_decode_flat"):
                vals.setdefault(c, []).append(v)
    m = {c: float(np.median(v)) for c, v in vals.items()}
    d = {"counters": {c: round(v, 1) for c, v in sorted(m.items())}}
    g = m.get("GRBM_GUI_ACTIVE")
    if g and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        # SQ_VALU_MFMA_BUSY_CYCLES sums all SIMDs; GUI-active cycles per XCD times the SIMD count
        d["gpu_active_cycles"] = round(g / XCDS)
        d["mfma_busy_share"] = round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / XCDS * SIMDS), 4)
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and m.get("SQ_VALU_MFMA_BUSY_CYCLES"):
        d["coexec_share_of_mfma_busy"] = round(m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
    if m.get("SQ_INSTS_MFMA"):
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS"):
            if c in m:
                d[c.lower().replace("sq_insts_", "") + "_per_mfma"] = round(m[c] / m["SQ_INSTS_MFMA"], 3)
    if m.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in m:
        d["lds_bank_conflict_per_active_lds_cycle"] = round(m["SQ_LDS_BANK_CONFLICT"] / m["SQ_ACTIVE_INST_LDS"], 4)
    h, mi = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
    if h is not None and mi is not None and h + mi > 0:
        d["l2_hit_rate"] = round(h / (h + mi), 4)
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", default=",".join(SECTIONS))
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--heads", type=int, default=0, help="with --counters: decode this many heads (default all 128)")
    ap.add_argument("--workload", default="c4r4_128k", help="with --counters: the workload whose decode is counted")
    ap.add_argument("--format", default="", help="with --counters: its cache in this format instead (same data)")
    ap.add_argument("--parse-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--packed-bytes", type=int, default=None)
    ap.add_argument("--parse-pmc", nargs="+", metavar="CSV")
    args = ap.parse_args()
    if args.parse_pmc:
        print(json.dumps(parse_pmc(args.parse_pmc)))
        return
    if args.parse_counters:
        print(json.dumps(parse_counters(*args.parse_counters, packed_bytes=args.packed_bytes)))
        return
    import torch
    import bit_mla_kv_decode_amd as mla
    if not torch.cuda.is_available():
        raise SystemExit("measure needs a GPU")
    mla.load_library()
    if args.counters:
        run_counters(args.heads, args.workload, args.format)
        return
    for s in args.only.split(","):
        SECTIONS[s]()


if __name__ == "__main__":
    main()
