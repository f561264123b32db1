"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

mla_quant_append must be bit-exact (codes, scales, zeros: whole pages);
decode outputs must satisfy |out - ref| <= 2e-3 + 1e-2 |ref| elementwise
against the fp64 oracle run on the same quantized cache.
"""
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
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _say(msg):
    print(msg, flush=True)


def build(fmt, lens, heads, seed, outliers=False, pages="random", extra_pages=3):
    """Host rows + page table for a batch of sequences of the given lengths."""
    w = W.Workload("case", fmt, batch=len(lens), heads=heads, outliers=outliers, pages=pages, seed=seed)
    lens = np.asarray(lens, dtype=np.int32)
    bt, npages = W.page_table(w, lens, extra_pages)
    lat, rope, slots = [], [], []
    for b, L in enumerate(lens):
        if L == 0:
            continue
        l, r = W.sequence_rows(w, b, 0, int(L), "cpu")
        lat.append(l)
        rope.append(r)
        slots.append(W.slots_for(bt, b, 0, int(L)))
    lat = torch.cat(lat) if lat else torch.zeros(0, 512, dtype=torch.bfloat16)
    rope = torch.cat(rope) if rope else torch.zeros(0, 64, dtype=torch.bfloat16)
    slots = np.concatenate(slots) if slots else np.zeros(0, np.int32)
    q = W.queries(w, "cpu")
    return w, lens, bt, npages, lat, rope, slots, q


def gpu_cache(fmt, npages, lat, rope, slots):
    cache = mla.alloc_cache(fmt, npages)
    if len(slots):
        mla.mla_quant_append(fmt, lat.cuda(), rope.cuda(), torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    return cache


def oracle_cache(fmt, npages, lat, rope, slots):
    cache = np.zeros(npages * oracle.page_bytes(OFMT[fmt]), dtype=np.uint8)
    if len(slots):
        oracle.quant_append(OFMT[fmt], lat, rope, slots, cache, npages)
    return cache


def gpu_decode(fmt, q, cache, bt, lens, splits=0, heads=None):
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    out, _ = mla.mla_decode_lowbit(fmt, q.cuda(), cache, torch.from_numpy(bt).cuda(),
                                   torch.from_numpy(lens).cuda(), SCALE, max_seq_len=int(lens.max()),
                                   num_splits=splits, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def assert_close(out, ref, what=""):
    err = np.abs(out - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), "%s: %d of %d outside tolerance, worst err %.3g at ref %.3g" % (
        what, int(bad.sum()), bad.size, float(err.max()), float(ref.flat[int(np.argmax(err - bound))]))


def assert_lse(lse, ref):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref))
    assert np.allclose(lse[fin], ref[fin], rtol=1e-5, atol=1e-4)


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "BF16"])
def test_quant_append_bit_exact(fmt):
    _say("append %s" % fmt)
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, [700, 129, 1, 64], 8, seed=11, outliers=True)
    # special rows: constant groups, signed zeros, exact ties and a skipped slot
    lat = lat.clone()
    lat[0] = 0.0
    lat[1, :64] = -0.0
    lat[1, 64:] = 1.5
    lat[2] = torch.arange(512, dtype=torch.float32).remainder(16).to(torch.bfloat16)
    lat[3, :32] = torch.tensor([0.0, 3.0] + [0.5, 1.5, 2.5] * 10, dtype=torch.float32).to(torch.bfloat16)
    slots = slots.copy()
    slots[5] = -1
    g = gpu_cache(fmt, npages, lat, rope, slots).cpu().numpy()
    o = oracle_cache(fmt, npages, lat, rope, slots)
    assert np.array_equal(g, o), "%d bytes differ" % int((g != o).sum())


def test_quant_append_skips_out_of_pool_slots():
    fmt = "C4R4"
    lat = torch.randn(3, 512).to(torch.bfloat16)
    rope = torch.randn(3, 64).to(torch.bfloat16)
    slots = np.array([5, 2 * 64 + 1, 70], dtype=np.int32)     # middle one is past a 2-page pool
    g = gpu_cache(fmt, 2, lat, rope, slots).cpu().numpy()
    o = oracle_cache(fmt, 2, lat[[0, 2]], rope[[0, 2]], slots[[0, 2]])
    assert np.array_equal(g, o)


# ------------------------------------------------------------------ decode

CASES = [
    ("C4R4", [256], 16, 0),                         # tiny decode shape
    ("C4R4", [1, 31, 32, 33, 64, 65, 200, 1000], 128, 0),
    ("C4R4", [1, 31, 32, 33, 64, 65, 200, 1000], 128, 1),
    ("C4R4", [1000, 130, 7], 128, 5),
    ("C2R4", [1, 33, 95, 640, 999], 128, 0),
    ("C2R4", [500, 64], 33, 3),
    ("BF16", [1, 33, 95, 640], 128, 0),
    ("BF16", [300], 48, 2),
    ("C4R4", [77, 512], 1, 0),
    ("C2R4", [2048], 64, 0),
]


@pytest.mark.parametrize("fmt,lens,heads,splits", CASES)
def test_decode_matches_oracle(fmt, lens, heads, splits):
    _say("decode %s lens=%s H=%d S=%d" % (fmt, lens, heads, splits))
    outl = fmt == "C2R4"
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, lens, heads, seed=len(lens) + heads, outliers=outl)
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    host = cache.cpu().numpy()
    assert np.array_equal(host, oracle_cache(fmt, npages, lat, rope, slots))
    out, lse = gpu_decode(fmt, q, cache, bt, lens, splits)
    ref, ref_lse = oracle.decode(OFMT[fmt], q, host, npages, bt, lens, SCALE)
    assert_close(out, ref, "%s %s" % (fmt, list(lens)))
    assert_lse(lse, ref_lse)


@pytest.mark.parametrize("splits", [0, 1, 4])
def test_empty_sequences(splits):
    fmt = "C4R4"
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, [0, 100, 0, 64], 128, seed=3)
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    out, lse = gpu_decode(fmt, q, cache, bt, lens, splits)
    ref, ref_lse = oracle.decode(OFMT[fmt], q, cache.cpu().numpy(), npages, bt, lens, SCALE)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert np.isneginf(lse[0]).all() and np.isneginf(lse[2]).all()
    assert_close(out, ref)
    assert_lse(lse, ref_lse)


@pytest.mark.parametrize("heads", [128, 48, 16])
@pytest.mark.parametrize("qmax", [40.0, 11.0])
def test_large_logit_jump(qmax, heads):
    """Logits that rise far above the first tile's after it: with qmax = 40 the
    rise (up to ~250 in log2 units) exceeds the kernel's fixed-reference range
    and the split is recomputed; with qmax = 11 (rises up to ~70-110) it stays
    inside the range.  Both must give the exact softmax, with one head group
    per wavefront (128 heads), two wavefronts per group (48) and four (16)."""
    _say("logit jump qmax=%g H=%d" % (qmax, heads))
    fmt = "C4R4"
    L = 300
    g = torch.Generator().manual_seed(5)
    lat = (torch.randn(L, 512, generator=g) * 0.05)
    lat[100:110, 0] = 60.0 + torch.arange(10, dtype=torch.float32)   # huge keys late in the sequence
    lat[250, 7] = -40.0
    lat = lat.to(torch.bfloat16)
    rope = torch.randn(L, 64, generator=g).to(torch.bfloat16)
    q = torch.randn(1, heads, 576, generator=g)
    q[0, :, 0] = qmax * torch.rand(heads, generator=g)
    q = q.to(torch.bfloat16)
    bt = np.arange(5, dtype=np.int32)[None]
    lens = np.array([L], np.int32)
    slots = np.arange(L, dtype=np.int32)
    cache = gpu_cache(fmt, 5, lat, rope, slots)
    ref, ref_lse = oracle.decode(OFMT[fmt], q, cache.cpu().numpy(), 5, bt, lens, SCALE)
    for splits in (1, 2):
        out, lse = gpu_decode(fmt, q, cache, bt, lens, splits)
        assert_close(out, ref, "splits=%d" % splits)
        assert_lse(lse, ref_lse)


def test_invariances_bitwise():
    """Same split count -> bit-identical across runs and page placements; other
    split counts agree with the oracle."""
    fmt = "C2R4"
    lens = [900, 333, 64]
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, lens, 128, seed=9, outliers=True)
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    a1, l1 = gpu_decode(fmt, q, cache, bt, lens, 3)
    a2, l2 = gpu_decode(fmt, q, cache, bt, lens, 3)
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2)
    # place the same tokens into a different page permutation (appended one token per call)
    w2 = W.derive(w, pages="random", seed=w.seed + 100)
    bt2, np2 = W.page_table(w2, lens, 7)
    slots2 = np.concatenate([W.slots_for(bt2, b, 0, int(L)) for b, L in enumerate(lens)])
    cache2 = mla.alloc_cache(fmt, np2)
    lat_d, rope_d, s_d = lat.cuda(), rope.cuda(), torch.from_numpy(slots2).cuda()
    for i0 in range(0, len(slots2), 97):
        mla.mla_quant_append(fmt, lat_d[i0:i0 + 97], rope_d[i0:i0 + 97], s_d[i0:i0 + 97], cache2)
    b1, m1 = gpu_decode(fmt, q, cache2, bt2, lens, 3)
    assert np.array_equal(a1, b1) and np.array_equal(l1, m1)
    ref, _ = oracle.decode(OFMT[fmt], q, cache.cpu().numpy(), npages, bt, lens, SCALE)
    for s in (1, 2, 7, 64):
        o, _ = gpu_decode(fmt, q, cache, bt, lens, s)
        assert_close(o, ref, "splits=%d" % s)


def test_partial_then_combine_equals_fused():
    fmt = "C4R4"
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, [700, 90], 128, seed=21)
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    S = 4
    ws = torch.empty(mla.mla_decode_workspace_bytes(fmt, 2, 128, S), dtype=torch.uint8, device="cuda")
    qd, btd, sld = q.cuda(), torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
    mla.mla_decode_partial(fmt, qd, cache, btd, sld, SCALE, S, ws, max_seq_len=700)
    out = torch.empty(2, 128, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(2, 128, dtype=torch.float32, device="cuda")
    mla.mla_decode_combine(fmt, 2, 128, S, ws, out, lse)
    o_part, l_part = mla.workspace_views(fmt, ws, 2, 128, S)
    # every partial matches the oracle on its own token range
    host = cache.cpu().numpy()
    pps = -(-((700 + 63) // 64) // S)
    for s in range(S):
        t0, t1 = s * pps * 64, ((s + 1) * pps * 64 if s < S - 1 else 10**9)
        ro, rl = oracle.decode(OFMT[fmt], q, host, npages, bt, lens, SCALE, t_begin=t0, t_end=t1)
        got = o_part[:, s].cpu().numpy()
        gl = l_part[:, s].cpu().numpy()
        for b in range(2):
            if np.isneginf(rl[b]).all():
                assert np.isneginf(gl[b]).all()
                continue
            assert np.allclose(got[b], ro[b], rtol=1e-4, atol=1e-4)
            assert np.allclose(gl[b], rl[b], rtol=1e-5, atol=1e-4)
    fused, flse = gpu_decode(fmt, q, cache, bt, lens, S)
    assert np.array_equal(out.float().cpu().numpy(), fused)
    assert np.array_equal(lse.cpu().numpy(), flse)


# ------------------------------------------------------------------ balanced partition

def balanced_pieces(lens, groups=256):
    """The documented num_splits = 0 cut: T pages in sequence order, G = min(groups, T)
    shares, share w = pages [w T / G, (w + 1) T / G); returns {slot: (b, first page,
    end page)} and per-sequence (first slot, count)."""
    n = [(int(L) + 63) // 64 for L in lens]
    T = sum(n)
    G = min(groups, T)
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    pieces, meta = {}, [(0, 0)] * len(lens)
    for w in range(G):
        s0, s1 = w * T // G, (w + 1) * T // G
        for b in range(len(lens)):
            lo, hi = max(off[b], s0), min(off[b + 1], s1)
            if lo < hi:
                pieces[w + b] = (b, int(lo - off[b]), int(hi - off[b]))
    for b in range(len(lens)):
        sl = sorted(k for k, v in pieces.items() if v[0] == b)
        if sl:
            assert sl == list(range(sl[0], sl[0] + len(sl)))
            meta[b] = (sl[0], len(sl))
    return pieces, np.array(meta, dtype=np.int32).reshape(-1, 2)


@pytest.mark.parametrize("fmt,lens,heads", [
    ("C4R4", [100, 0, 700, 5], 128),                               # 14 pages < 256 shares
    ("C2R4", [0] * 3 + [1, 64, 65, 3000, 129] * 30 + [0, 2000], 16),  # 152 sequences, spans chunks of 64
    ("BF16", [640, 1, 6000, 70], 40),
])
def test_balanced_partition_pieces(fmt, lens, heads):
    """Every (workgroup, sequence) piece of the balanced partition against the
    oracle on that piece's pages, the slot records against the documented cut,
    and the merged output against the oracle."""
    _say("balanced %s B=%d H=%d" % (fmt, len(lens), heads))
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, lens, heads, seed=len(lens) * 7 + heads)
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    host = cache.cpu().numpy()
    B, H = len(lens), heads
    ws = torch.full((mla.mla_decode_workspace_bytes(fmt, B, H, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    qd, btd, sld = q.cuda(), torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
    mla.mla_decode_partial(fmt, qd, cache, btd, sld, SCALE, 0, ws, max_seq_len=int(lens.max()))
    out = torch.empty(B, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    mla.mla_decode_combine(fmt, B, H, 0, ws, out, lse)
    torch.cuda.synchronize()
    o_part, l_part, meta = (t.cpu().numpy() for t in mla.balanced_workspace_views(fmt, ws, B, H))
    groups = mla.mla_decode_partial_slots(fmt, B, H, 0) - B   # 512 where two workgroups share a unit
    assert groups == (512 if fmt != "BF16" and 16 < H <= 32 else 256)
    pieces, want_meta = balanced_pieces(lens, groups)
    assert np.array_equal(meta, want_meta)
    for slot, (b, p0, p1) in sorted(pieces.items()):
        ro, rl = oracle.decode(OFMT[fmt], q[b:b + 1], host, npages, bt[b:b + 1], lens[b:b + 1], SCALE,
                               t_begin=p0 * 64, t_end=p1 * 64)
        assert np.allclose(o_part[slot], ro[0], rtol=1e-4, atol=1e-4), "slot %d (b=%d pages %d..%d)" % (slot, b, p0, p1)
        assert np.allclose(l_part[slot], rl[0], rtol=1e-5, atol=1e-4)
    ref, ref_lse = oracle.decode(OFMT[fmt], q, host, npages, bt, lens, SCALE)
    assert_close(out.float().cpu().numpy(), ref, "balanced")
    assert_lse(lse.cpu().numpy(), ref_lse)
    fused, flse = gpu_decode(fmt, q, cache, bt, lens, 0)
    assert np.array_equal(out.float().cpu().numpy(), fused) and np.array_equal(lse.cpu().numpy(), flse)


def test_balanced_all_empty():
    fmt = "C4R4"
    lens = np.zeros(5, np.int32)
    q = torch.randn(5, 8, 576).to(torch.bfloat16)
    cache = mla.alloc_cache(fmt, 2)
    bt = np.zeros((5, 2), np.int32)
    out, lse = gpu_decode(fmt, q, cache, bt, lens, 0)
    assert (out == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4"])
@pytest.mark.parametrize("heads", [1, 16, 31, 32, 33, 63, 64, 65, 100])
@pytest.mark.parametrize("splits", [0, 3])
def test_head_counts(fmt, heads, splits):
    """Every head-count regime of the decode: 4, 2 or 1 wavefronts per
    32-head group (channel split), with ragged lengths and a partial tile."""
    _say("heads %s H=%d S=%d" % (fmt, heads, splits))
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, [1500, 70, 0, 333], heads, seed=heads + 17,
                                                     outliers=fmt == "C2R4")
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    out, lse = gpu_decode(fmt, q, cache, bt, lens, splits)
    ref, ref_lse = oracle.decode(OFMT[fmt], q, cache.cpu().numpy(), npages, bt, lens, SCALE)
    assert_close(out, ref, "%s H=%d S=%d" % (fmt, heads, splits))
    assert_lse(lse, ref_lse)


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "BF16"])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("heads", [16, 64])
def test_fused_append_decode_equals_separate(fmt, splits, heads):
    """mla_decode_append_lowbit == mla_quant_append of the new rows (at position
    L - 1) followed by mla_decode_lowbit: same cache bytes, bitwise the same
    output and LSE; and the output matches the oracle on that cache."""
    lens = [1, 64, 65, 300, 0, 1000, 129]
    _say("fused append %s S=%d H=%d" % (fmt, splits, heads))
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, lens, heads, seed=splits + heads, outliers=fmt == "C2R4")
    # rows of every token except each sequence's last; the last rows are the new ones
    keep, last_rows = [], []
    off = 0
    for b, L in enumerate(lens):
        L = int(L)
        keep.extend(range(off, off + max(L - 1, 0)))
        last_rows.append(off + L - 1 if L > 0 else -1)
        off += L
    keep = np.array(keep, dtype=np.int64)
    base = gpu_cache(fmt, npages, lat[keep], rope[keep], slots[keep])
    B = len(lens)
    new_lat = torch.zeros(B, 512, dtype=torch.bfloat16)
    new_rope = torch.zeros(B, 64, dtype=torch.bfloat16)
    new_slots = np.full(B, -1, np.int32)
    for b, r in enumerate(last_rows):
        if r >= 0:
            new_lat[b], new_rope[b], new_slots[b] = lat[r], rope[r], slots[r]
    qd, btd, sld = q.cuda(), torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
    # separate
    c1 = base.clone()
    mla.mla_quant_append(fmt, new_lat.cuda(), new_rope.cuda(), torch.from_numpy(new_slots).cuda(), c1)
    l1 = torch.empty(B, heads, dtype=torch.float32, device="cuda")
    o1, _ = mla.mla_decode_lowbit(fmt, qd, c1, btd, sld, SCALE, max_seq_len=int(lens.max()), num_splits=splits, lse=l1)
    # fused
    c2 = base.clone()
    l2 = torch.empty(B, heads, dtype=torch.float32, device="cuda")
    o2, _ = mla.mla_decode_append_lowbit(fmt, new_lat.cuda(), new_rope.cuda(), qd, c2, btd, sld, SCALE,
                                         max_seq_len=int(lens.max()), num_splits=splits, lse=l2)
    torch.cuda.synchronize()
    h1, h2 = c1.cpu().numpy(), c2.cpu().numpy()
    assert np.array_equal(h1, h2), "%d cache bytes differ" % int((h1 != h2).sum())
    assert np.array_equal(h2, oracle_cache(fmt, npages, lat, rope, slots))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref, ref_lse = oracle.decode(OFMT[fmt], q, h2, npages, bt, lens, SCALE)
    assert_close(o2.float().cpu().numpy(), ref, "fused %s" % fmt)
    assert_lse(l2.cpu().numpy(), ref_lse)



@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "BF16"])
@pytest.mark.parametrize("s_q,heads", [(2, 64), (4, 8), (2, 24), (3, 100), (16, 16), (2, 8), (3, 5)])
@pytest.mark.parametrize("splits", [0, 3])
def test_multi_token_decode(fmt, s_q, heads, splits):
    """Several query tokens per sequence (causal among themselves): 128 rows in
    one workgroup, 32 rows (channel split), <= 16 rows (independent wavefronts),
    and rows split into head chunks;
    a sequence shorter than the query count; against oracle.decode_multi."""
    _say("multi-token %s s_q=%d H=%d S=%d" % (fmt, s_q, heads, splits))
    lens = [1500, 3, 70, 0, 64, 333]
    w, lens, bt, npages, lat, rope, slots, _ = build(fmt, lens, heads, seed=s_q * 7 + heads, outliers=fmt == "C2R4")
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    g = torch.Generator().manual_seed(s_q + heads + splits)
    q = torch.randn(len(lens), s_q, heads, 576, generator=g).to(torch.bfloat16)
    lse = torch.empty(len(lens), s_q, heads, dtype=torch.float32, device="cuda")
    out, _ = mla.mla_decode_multi_lowbit(fmt, q.cuda(), cache, torch.from_numpy(bt).cuda(),
                                         torch.from_numpy(lens).cuda(), SCALE, max_seq_len=int(lens.max()),
                                         num_splits=splits, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_multi(OFMT[fmt], q, cache.cpu().numpy(), npages, bt, lens, SCALE)
    assert_close(out.float().cpu().numpy(), ref, "multi %s s_q=%d H=%d" % (fmt, s_q, heads))
    assert_lse(lse.cpu().numpy(), ref_lse)


def test_multi_token_single_query_equals_decode():
    fmt = "C4R4"
    w, lens, bt, npages, lat, rope, slots, q = build(fmt, [900, 65, 1], 48, seed=77)
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
    for S in (0, 1, 4):
        o1, _ = mla.mla_decode_lowbit(fmt, q.cuda(), cache, btd, sld, SCALE, num_splits=S)
        o2, _ = mla.mla_decode_multi_lowbit(fmt, q.cuda()[:, None].contiguous(), cache, btd, sld, SCALE, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2[:, 0])


@pytest.mark.parametrize("fmt,heads,splits", [("C4R4", 16, 0), ("C2R4", 24, 0), ("C4R4", 48, 2), ("C2R4", 128, 0),
                                              ("BF16", 128, 0)])
def test_large_batch(fmt, heads, splits):
    """700 short ragged sequences (empty, single-token, partial-tile, up to a
    few pages): more sequences than the balanced partition has workgroups, so
    shares hold many pieces; the walk reads lengths beyond the first 256 from
    global memory and crosses many 64-sequence chunks; the combine merges
    every sequence's slots."""
    B = 700
    _say("large batch %s H=%d S=%d B=%d" % (fmt, heads, splits, B))
    rng = np.random.default_rng(heads + 31 * splits)
    kind = rng.integers(0, 10, size=B)
    lens = np.where(kind == 0, 0, np.where(kind == 1, 1, np.where(kind < 5, rng.integers(2, 64, size=B),
                                                                   rng.integers(64, 400, size=B)))).astype(np.int32)
    w = W.Workload("batch", fmt, batch=B, heads=heads, outliers=fmt == "C2R4", pages="random", seed=heads)
    bt, npages = W.page_table(w, lens, 2)
    cache = mla.alloc_cache(fmt, npages)
    for b, L in enumerate(lens):
        if L:
            lat, rope = W.sequence_rows(w, b, 0, int(L), "cuda")
            mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(W.slots_for(bt, b, 0, int(L))).cuda(), cache)
    q = W.queries(w, "cpu")
    out, lse = gpu_decode(fmt, q, cache, bt, lens, splits)
    ref, ref_lse = oracle.decode(OFMT[fmt], q, cache.cpu().numpy(), npages, bt, lens, SCALE)
    assert_close(out, ref, "%s H=%d B=%d" % (fmt, heads, B))
    assert_lse(lse, ref_lse)
    assert (out[lens == 0] == 0).all()
