"""The serving step (append of one new row per sequence, decode, combine)
captured in a HIP graph and replayed: every replay must give the eager call's
outputs and log-sum-exps bit for bit, for the workspace and the
no-allocation entry points.  Between replays the test runs eager work of its
own, rewrites the queries in place (a serving loop's next step) and
synchronizes; the appended row lands at the same slot on every replay, so the
cache bytes stay those of the eager call."""
import math

import numpy as np
import pytest
import torch

import bit_mla_kv_decode_amd as mla
from bit_mla_kv_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _setup(fmt, lens, heads, seed):
    w = W.Workload("graph", fmt, batch=len(lens), heads=heads, pages="random", seed=seed, outliers=fmt == "C2R4")
    lens = np.asarray(lens, np.int32)
    bt, npages = W.page_table(w, lens, 2)
    cache = mla.alloc_cache(fmt, npages)
    for b, L in enumerate(lens):
        if L > 1:   # the last token of every sequence comes with the step
            lat, rope = W.sequence_rows(w, b, 0, int(L) - 1, "cuda")
            mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(W.slots_for(bt, b, 0, int(L) - 1)).cuda(), cache)
    g = torch.Generator().manual_seed(seed)
    new_lat = torch.randn(len(lens), 512, generator=g).to(torch.bfloat16).cuda()
    new_rope = torch.randn(len(lens), 64, generator=g).to(torch.bfloat16).cuda()
    return w, lens, bt, npages, cache, new_lat, new_rope


@pytest.mark.parametrize("fmt,heads,splits,noalloc", [
    ("C4R4", 128, 0, False), ("C2R4", 16, 0, False), ("C4R4", 32, 3, False), ("BF16", 48, 0, False),
    ("C2R4", 128, 0, True), ("C4R4", 16, 2, True)])
def test_replayed_step_equals_eager(fmt, heads, splits, noalloc):
    print("graph step %s H=%d S=%d noalloc=%s" % (fmt, heads, splits, noalloc), flush=True)
    w, lens, bt, npages, cache, new_lat, new_rope = _setup(fmt, [2100, 1, 700, 65, 4200], heads, 11 + heads)
    B = len(lens)
    btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
    g = torch.Generator().manual_seed(99)
    qs = [torch.randn(B, heads, 576, generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
    q = qs[0].clone()
    ws = None if noalloc else torch.empty(max(1, mla.mla_decode_workspace_bytes(fmt, B, heads, splits)),
                                          dtype=torch.uint8, device="cuda")

    slots = torch.from_numpy(np.array([W.slots_for(bt, b, int(L) - 1, int(L))[0] for b, L in enumerate(lens)],
                                      np.int32)).cuda()

    def step(out, lse):
        if noalloc:   # append first (the no-allocation call has no fused append), then decode
            mla.mla_quant_append(fmt, new_lat, new_rope, slots, cache)
            mla.mla_decode_lowbit_noalloc(fmt, q, cache, btd, sld, SCALE, max_seq_len=int(lens.max()),
                                          num_splits=splits, out=out, lse=lse)
        else:
            mla.mla_decode_append_lowbit(fmt, new_lat, new_rope, q, cache, btd, sld, SCALE,
                                         max_seq_len=int(lens.max()), num_splits=splits, out=out, lse=lse,
                                         workspace=ws)

    # eager results for each query set
    want = []
    for qi in qs:
        q.copy_(qi)
        out = torch.empty(B, heads, 512, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, heads, dtype=torch.float32, device="cuda")
        step(out, lse)
        torch.cuda.synchronize()
        want.append((out.clone(), lse.clone()))
    cache_eager = cache.clone()

    out_g = torch.empty(B, heads, 512, dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty(B, heads, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        step(out_g, lse_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out_g, lse_g)
    torch.cuda.synchronize()

    junk = torch.randn(512, 512, device="cuda")
    for rep in range(6):
        i = rep % 3
        q.copy_(qs[i])
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        junk = (junk @ junk).tanh()   # eager work of the program between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, want[i][0]), "replay %d: outputs differ from the eager call" % rep
        assert torch.equal(lse_g, want[i][1]), "replay %d: log-sum-exps differ from the eager call" % rep
        assert torch.equal(cache, cache_eager), "replay %d: cache bytes differ" % rep
