"""Decode at the edges of the accepted sizes, against the CPU oracle.

- The largest batch the boundary accepts (65535 sequences of one page or
  less, a few of them empty): the balanced partition then gives every
  workgroup hundreds of pieces and walks a thousand 64-sequence chunks, the
  combine merges 65535 sequences, and the fixed splits launch a grid of
  65535 rows.
- One sequence of 2^20 + 37 tokens: every workgroup of the balanced
  partition takes a share of that one sequence, and the combine merges 256
  slots of it (more than it loads in one round); fixed splits at their
  maximum of 64.  All heads against the oracle at 16 heads; 8 sampled heads
  at 128 (the oracle computes every head on its own, so a subset of the
  query heads gives those heads' outputs).
Tolerance as everywhere: |out - ref| <= 2e-3 + 1e-2 |ref|."""
import numpy as np
import pytest
import torch

import bit_mla_kv_decode_amd as mla
import oracle
from bit_mla_kv_decode_amd import workloads as W
from test_gpu_parity import OFMT, SCALE, _say, assert_close, assert_lse

pytestmark = pytest.mark.gpu


def _fill(fmt, w, lens, bt, cache, block=32768):
    """Append every sequence's rows (the workload's generator) in blocks of
    32768 tokens."""
    for b, L in enumerate(lens):
        for t0 in range(0, int(L), block):
            t1 = min(int(L), t0 + block)
            lat, rope = W.sequence_rows(w, b, t0, t1, "cuda")
            mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(W.slots_for(bt, b, t0, t1)).cuda(), cache)


@pytest.mark.parametrize("fmt,splits", [("C4R4", 0), ("C2R4", 0), ("C4R4", 2)])
def test_largest_batch(fmt, splits):
    B, H = 65535, 8
    _say("largest batch %s B=%d H=%d S=%d" % (fmt, B, H, splits))
    rng = np.random.default_rng(17 + splits)
    lens = rng.integers(1, 65, size=B).astype(np.int32)
    lens[rng.choice(B, size=40, replace=False)] = 0
    w = W.Workload("maxbatch", fmt, batch=B, heads=H, outliers=fmt == "C2R4", pages="random", seed=23)
    bt, npages = W.page_table(w, lens, 1)
    cache = mla.alloc_cache(fmt, npages)
    # rows: one draw for the whole batch (per-sequence draws would take minutes
    # at this batch), with the workload's per-channel spread and RoPE rows
    # rotated by their positions
    g = torch.Generator(device="cuda").manual_seed(29)
    n = int(lens.sum())
    lat = (torch.randn(n, 512, generator=g, device="cuda") * W.channel_sigma(w).cuda()).to(torch.bfloat16)
    pos = torch.from_numpy(np.concatenate([np.arange(L) for L in lens if L]).astype(np.float64)).cuda()
    inv = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -torch.arange(0, 64, 2, dtype=torch.float64) / 64).cuda()
    ang = pos[:, None] * inv[None, :]
    r = torch.randn(n, 32, 2, generator=g, device="cuda", dtype=torch.float64)
    rope = torch.stack([r[..., 0] * torch.cos(ang) - r[..., 1] * torch.sin(ang),
                        r[..., 0] * torch.sin(ang) + r[..., 1] * torch.cos(ang)], -1).reshape(n, 64)
    rope = rope.float().to(torch.bfloat16)
    slots = np.concatenate([W.slots_for(bt, b, 0, int(L)) for b, L in enumerate(lens) if L])
    mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(slots).cuda(), cache)
    q = torch.randn(B, H, 576, generator=g, device="cuda").to(torch.bfloat16)
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    out, _ = mla.mla_decode_lowbit(fmt, q, cache, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), SCALE,
                                   max_seq_len=int(lens.max()), num_splits=splits, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(OFMT[fmt], q.cpu(), cache.cpu().numpy(), npages, bt, lens, SCALE)
    o = out.float().cpu().numpy()
    assert_close(o, ref, "%s B=%d S=%d" % (fmt, B, splits))
    assert_lse(lse.cpu().numpy(), ref_lse)
    assert (o[lens == 0] == 0).all()


@pytest.mark.parametrize("fmt,heads,splits", [("C4R4", 16, 0), ("C2R4", 16, 64), ("C4R4", 128, 0), ("C2R4", 128, 0)])
def test_one_long_sequence(fmt, heads, splits):
    L = (1 << 20) + 37
    _say("one long sequence %s L=%d H=%d S=%d" % (fmt, L, heads, splits))
    w = W.Workload("long", fmt, batch=1, heads=heads, outliers=fmt == "C2R4", pages="random", seed=31)
    lens = np.array([L], np.int32)
    bt, npages = W.page_table(w, lens, 2)
    cache = mla.alloc_cache(fmt, npages)
    _fill(fmt, w, lens, bt, cache)
    q = W.queries(w, "cuda")
    lse = torch.empty(1, heads, dtype=torch.float32, device="cuda")
    out, _ = mla.mla_decode_lowbit(fmt, q, cache, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), SCALE,
                                   max_seq_len=L, num_splits=splits, lse=lse)
    torch.cuda.synchronize()
    if splits == 0:
        assert mla.mla_decode_partial_slots(fmt, 1, heads, 0) - 1 == 256   # every share a slot of this sequence
    sample = np.arange(heads) if heads <= 16 else np.sort(np.random.default_rng(5).choice(heads, 8, replace=False))
    qs = q.cpu()[:, torch.from_numpy(sample)].contiguous()
    ref, ref_lse = oracle.decode(OFMT[fmt], qs, cache.cpu().numpy(), npages, bt, lens, SCALE)
    assert_close(out.float().cpu().numpy()[:, sample], ref, "%s L=%d H=%d" % (fmt, L, heads))
    assert_lse(lse.cpu().numpy()[:, sample], ref_lse)
