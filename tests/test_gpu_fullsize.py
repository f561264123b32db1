"""GPU parity at the full workload sizes, in the launch configuration bench.py
uses (balanced partition, num_splits = 0, partial + combine).  The 32 x 8192
C4R4 workload is checked on every element (whole cache bytes, every output
and LSE); the larger ones on sampled sequences, all heads of each, that the
CPU oracle computes one by one."""
import math

import numpy as np
import pytest
import torch

import bit_mla_kv_decode_amd as mla
import oracle
from bit_mla_kv_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2
OFMT = {"C4R4": oracle.C4R4, "C2R4": oracle.C2R4, "BF16": oracle.BF16}


def _say(msg):
    print(msg, flush=True)


def _build(w, fmt, hold_back_last=False):
    """Full cache on the GPU; with hold_back_last the last token of every
    sequence is appended in one batched call afterwards (the serving step)."""
    lens = W.seq_lens(w)
    bt, npages = W.page_table(w, lens)
    cache = mla.alloc_cache(fmt, npages)
    for b, L in enumerate(lens):
        end = int(L) - 1 if hold_back_last else int(L)
        for t0 in range(0, end, 32768):
            t1 = min(end, t0 + 32768)
            lat, rope = W.sequence_rows(w, b, t0, t1, "cuda")
            mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(W.slots_for(bt, b, t0, t1)).cuda(), cache)
    if hold_back_last:
        lat, rope = W.new_token_rows(w, lens, "cuda")
        slots = np.array([W.slots_for(bt, b, int(L) - 1, int(L))[0] for b, L in enumerate(lens)], np.int32)
        mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    return lens, bt, npages, cache


def _decode(w, fmt, lens, bt, cache):
    B, H = w.batch, w.heads
    q = W.queries(w, "cuda")
    max_len = int(lens.max())
    S = 0
    ws = torch.empty(mla.mla_decode_workspace_bytes(fmt, B, H, S), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
    mla.mla_decode_partial(fmt, q, cache, btd, sld, w.softmax_scale, S, ws, max_seq_len=max_len)
    mla.mla_decode_combine(fmt, B, H, S, ws, out, lse)
    torch.cuda.synchronize()
    return q.cpu(), out.float().cpu().numpy(), lse.cpu().numpy(), S


def _assert_outputs(o, ref, what):
    err = np.abs(o - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d of %d outputs outside tolerance (max err %.3g)" % (
        what, int(bad.sum()), bad.size, float(err.max()))


def _check_sequence(w, fmt, b, lens, bt, cache, q, out, lse):
    L = int(lens[b])
    npg = (L + 63) // 64
    pb = mla.mla_page_bytes(fmt)
    pages = torch.from_numpy(bt[b, :npg].astype(np.int64)).cuda()
    got_pages = cache.view(-1, pb)[pages].cpu().numpy().reshape(-1)
    # bit-exact append on this sequence's pages
    lat, rope = W.sequence_rows(w, b, 0, L, "cuda")
    ref_cache = np.zeros(npg * pb, dtype=np.uint8)
    slots = np.arange(L, dtype=np.int32)
    oracle.quant_append(OFMT[fmt], lat.cpu(), rope.cpu(), slots, ref_cache, npg)
    assert np.array_equal(got_pages, ref_cache), "sequence %d: %d cache bytes differ" % (b, int((got_pages != ref_cache).sum()))
    # decode, every head of the sequence
    ref, ref_lse = oracle.decode(OFMT[fmt], q[b:b + 1].contiguous(), got_pages, npg,
                                 np.arange(npg, dtype=np.int32)[None], np.array([L], np.int32), w.softmax_scale)
    _assert_outputs(out[b], ref[0], "sequence %d" % b)
    assert np.allclose(lse[b], ref_lse[0], rtol=1e-5, atol=1e-4)


def test_fullsize_every_element_dsv3_8k():
    """32 x 8192 tokens, 128 heads, C4R4: the whole cache bit-exact against the
    oracle's quantizer and every output and LSE against the oracle's decode."""
    w = W.WORKLOADS["dsv3_c4r4_8k"]
    _say("full-size %s, every element: B=%d H=%d" % (w.name, w.batch, w.heads))
    lens, bt, npages, cache = _build(w, w.fmt)
    q, out, lse, S = _decode(w, w.fmt, lens, bt, cache)
    host = cache.cpu().numpy()
    ref_cache = np.zeros_like(host)
    for b, L in enumerate(lens):
        lat, rope = W.sequence_rows(w, b, 0, int(L), "cuda")   # the draws the cache was built from
        oracle.quant_append(OFMT[w.fmt], lat.cpu(), rope.cpu(), W.slots_for(bt, b, 0, int(L)), ref_cache, npages)
    assert np.array_equal(host, ref_cache), "%d cache bytes differ" % int((host != ref_cache).sum())
    _say("  cache bit-exact; oracle decode of all %d sequences" % w.batch)
    ref, ref_lse = oracle.decode(OFMT[w.fmt], q, host, npages, bt, lens, w.softmax_scale)
    _assert_outputs(out, ref, w.name)
    assert np.allclose(lse, ref_lse, rtol=1e-5, atol=1e-4)
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["c2r4_32k_outliers", "c4r4_128k", "mixed_c2r4_serving"])
def test_fullsize_sampled(name):
    w = W.WORKLOADS[name]
    _say("full-size %s: B=%d H=%d fmt=%s" % (name, w.batch, w.heads, w.fmt))
    lens, bt, npages, cache = _build(w, w.fmt, hold_back_last=w.append_new)
    q, out, lse, S = _decode(w, w.fmt, lens, bt, cache)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    for b in sorted({0, w.batch - 1, int(np.argmax(lens))}):
        _say("  check sequence %d (L=%d)" % (b, int(lens[b])))
        _check_sequence(w, w.fmt, b, lens, bt, cache, q, out, lse)
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["c4r4_128k", "c2r4_32k_outliers"])
def test_fullsize_16_heads(name):
    """The 16-head share of the full-size workloads (the bench's 16-head record):
    sampled sequences, every head, against the oracle."""
    w = W.derive(W.WORKLOADS[name], heads=16)
    _say("full-size %s at 16 heads: B=%d fmt=%s" % (name, w.batch, w.fmt))
    lens, bt, npages, cache = _build(w, w.fmt)
    q, out, lse, S = _decode(w, w.fmt, lens, bt, cache)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    for b in sorted({0, w.batch - 1}):
        _say("  check sequence %d (L=%d)" % (b, int(lens[b])))
        _check_sequence(w, w.fmt, b, lens, bt, cache, q, out, lse)
    del cache
    torch.cuda.empty_cache()


def test_fullsize_bf16_baseline_on_c2r4_data():
    """The unquantized-cache kernel on the C2R4 workload's data (the baseline
    the low-bit path is compared with)."""
    w = W.WORKLOADS["c2r4_32k_outliers"]
    _say("full-size bf16 baseline on %s" % w.name)
    lens, bt, npages, cache = _build(w, "BF16")
    q, out, lse, S = _decode(w, "BF16", lens, bt, cache)
    for b in (0, w.batch - 1):
        _check_sequence(w, "BF16", b, lens, bt, cache, q, out, lse)
    del cache
    torch.cuda.empty_cache()


def test_fullsize_fused_serving_step():
    """The mixed serving batch through the fused append + decode (bench's step):
    the appended rows land bit-exact and sampled outputs match the oracle."""
    w = W.WORKLOADS["mixed_c2r4_serving"]
    _say("full-size fused step on %s" % w.name)
    lens = W.seq_lens(w)
    bt, npages = W.page_table(w, lens)
    cache = mla.alloc_cache(w.fmt, npages)
    for b, L in enumerate(lens):
        for t0 in range(0, int(L) - 1, 32768):
            t1 = min(int(L) - 1, t0 + 32768)
            lat, rope = W.sequence_rows(w, b, t0, t1, "cuda")
            mla.mla_quant_append(w.fmt, lat, rope, torch.from_numpy(W.slots_for(bt, b, t0, t1)).cuda(), cache)
    new_lat, new_rope = W.new_token_rows(w, lens, "cuda")
    q = W.queries(w, "cuda")
    B, H = w.batch, w.heads
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    out, _ = mla.mla_decode_append_lowbit(w.fmt, new_lat, new_rope, q, cache, torch.from_numpy(bt).cuda(),
                                          torch.from_numpy(lens).cuda(), w.softmax_scale,
                                          max_seq_len=int(lens.max()), lse=lse)
    torch.cuda.synchronize()
    outn, lsen = out.float().cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(outn).all() and np.isfinite(lsen).all()
    for b in sorted({0, B - 1, int(np.argmin(lens))}):
        _say("  check sequence %d (L=%d)" % (b, int(lens[b])))
        _check_sequence(w, w.fmt, b, lens, bt, cache, q.cpu(), outn, lsen)
    del cache
    torch.cuda.empty_cache()
