"""GPU closed forms of the decode, checked bit for bit.

With one token in context, or with every token of a sequence carrying the
same dequantized row, the softmax gives all of its weight to that row, so the
exact output is the row's first 512 dequantized values.  Each of them is a
bf16 value (the canonical dequantized value bf16(fma(code, S, Z)) of the
quantized formats, the stored value of the BF16 cache), so the kernel's bf16
output must equal it bit for bit: the kernel's only rounding error is a few
fp32 ulps in the weights and their sum, far below half a bf16 ulp.  This
pins the in-kernel dequantization (code extraction, scale and zero, fused
multiply-add and bf16 rounding) against the oracle's canonical value, which
the tolerance of the general parity tests cannot do.

The rows below use every INT4 / INT2 code, zero-range groups (S = 0), fp16
subnormal scales, negative zeros and a zero of -0 (canonicalized to +0), and
go through every decode kernel variant (<= 16, 17..32, 33..64 and > 64 rows
per sequence) in both partitions (balanced, fixed splits, one split written
directly).
"""
import math

import numpy as np
import pytest
import torch

import bit_mla_kv_decode_amd as mla
import oracle

pytestmark = pytest.mark.gpu

OFMT = {"C4R4": oracle.C4R4, "C2R4": oracle.C2R4, "BF16": oracle.BF16}
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _say(msg):
    print(msg, flush=True)


def _bf16_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _grid(levels, z, s, n):
    """n values z + (i mod levels) * s (exact in bf16 for the choices below)."""
    return np.float32(z) + np.float32(s) * (np.arange(n) % levels).astype(np.float32)


def special_rows(fmt):
    """Latent [R, 512] and RoPE [R, 64] rows (float32, bf16-exact) whose groups
    cover every code, S = 0, subnormal fp16 S and negative / -0 zeros."""
    gsize = 32 if fmt == "C2R4" else 64
    levels = 4 if fmt == "C2R4" else 16
    ng = 512 // gsize
    rng = np.random.default_rng(1234)
    kinds = [
        lambda n: _grid(levels, 1.0, 0.25, n),                     # every code, positive Z
        lambda n: np.full(n, 3.0, np.float32),                      # zero range: S = 0, value = Z
        lambda n: _grid(levels, 0.0, 2.0 ** -20, n),                # fp16 subnormal S = 2^-20
        lambda n: _grid(levels, -5.0, 0.5, n),                      # negative Z
        lambda n: np.concatenate([[np.float32(-0.0)], _grid(levels, 0.0, 0.125, n)[1:]]),  # min is -0
        lambda n: _bf16_round(rng.standard_normal(n) * 2.0),        # codes off the grid
        lambda n: _grid(levels, 100.0, 8.0, n),                     # large values
        lambda n: -_grid(levels, 0.0, 2.0 ** -22, n),               # subnormal S, -0 as the maximum
    ]
    rows_lat, rows_rope = [], []
    for r in range(4):
        lat = np.concatenate([kinds[(g + r) % len(kinds)](gsize) for g in range(ng)])
        # a row of every code in reversed order within each group, so codes do not line up with channels
        if r == 3:
            lat = lat.reshape(ng, gsize)[:, ::-1].reshape(-1).copy()
        rope = kinds[(3 * r) % len(kinds)](64) if r != 1 else _grid(16, -1.0, 0.125, 64)
        rows_lat.append(lat)
        rows_rope.append(rope)
    lat = torch.from_numpy(np.stack(rows_lat)).to(torch.bfloat16)
    rope = torch.from_numpy(np.stack(rows_rope)).to(torch.bfloat16)
    assert torch.equal(lat.float(), torch.from_numpy(np.stack(rows_lat))), "rows must be bf16-exact"
    return lat, rope


def _bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


# (heads, expected kernel variant): rows per sequence pick the decode kernel
HEAD_CASES = [8, 24, 48, 128]


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "BF16"])
@pytest.mark.parametrize("heads", HEAD_CASES)
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_single_token_and_identical_rows_bit_exact(fmt, heads, splits):
    """out[b, h] == dequantized row (bit for bit) for ctx = 1 sequences and for
    sequences whose tokens all share one row; lse = logit (+ ln L)."""
    _say("closed forms %s H=%d S=%d" % (fmt, heads, splits))
    lat_s, rope_s = special_rows(fmt)
    R = lat_s.shape[0]
    # sequences: R of length 1 (one special row each), then R of identical rows
    # (lengths spanning partial tiles and pages), then one empty sequence
    ident_lens = [33, 64, 200, 1000][:R]
    lens = [1] * R + ident_lens + [0]
    B = len(lens)
    npg = [(L + 63) // 64 for L in lens]
    pool = np.random.default_rng(heads + splits).permutation(sum(npg) + 2).astype(np.int32)
    bt = np.full((B, max(npg)), -1, np.int32)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = pool[off:off + n]
        off += n
    num_pages = len(pool)
    lat_rows, rope_rows, slots = [], [], []
    for b, L in enumerate(lens):
        if L == 0:
            continue
        r = b % R
        lat_rows.append(lat_s[r:r + 1].expand(L, 512))
        rope_rows.append(rope_s[r:r + 1].expand(L, 64))
        t = np.arange(L)
        slots.append(bt[b, t // 64] * 64 + t % 64)
    lat = torch.cat(lat_rows).contiguous()
    rope = torch.cat(rope_rows).contiguous()
    slots = np.concatenate(slots).astype(np.int32)
    cache = mla.alloc_cache(fmt, num_pages)
    mla.mla_quant_append(fmt, lat.cuda(), rope.cuda(), torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    host = cache.cpu().numpy()
    ref_cache = np.zeros_like(host)
    oracle.quant_append(OFMT[fmt], lat, rope, slots, ref_cache, num_pages)
    assert np.array_equal(host, ref_cache)
    lens = np.array(lens, np.int32)
    deq = oracle.dequant_cache(OFMT[fmt], host, num_pages, bt, lens)   # [B, max_len, 576] float32

    g = torch.Generator().manual_seed(heads * 3 + splits)
    q = torch.randn(B, heads, 576, generator=g).to(torch.bfloat16)
    lse = torch.empty(B, heads, dtype=torch.float32, device="cuda")
    out, _ = mla.mla_decode_lowbit(fmt, q.cuda(), cache, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                   SCALE, max_seq_len=int(lens.max()), num_splits=splits, lse=lse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    _, ref_lse = oracle.decode(OFMT[fmt], q, host, num_pages, bt, lens, SCALE)
    for b, L in enumerate(lens):
        if L == 0:
            assert (got[b] == 0).all() and np.isneginf(got_lse[b]).all()
            continue
        want = deq[b, 0, :512]
        # every token of the sequence carries the same dequantized row
        assert np.array_equal(_bits(deq[b, :L]), np.broadcast_to(_bits(deq[b, 0]), (L, 576)))
        # bit for bit, except that a zero may come out as +0 for a stored -0
        # (the BF16 cache keeps -0; a weighted sum that starts from +0 gives +0)
        bad = (_bits(got[b]) != _bits(want)[None, :]) & ~((got[b] == 0) & (want[None, :] == 0))
        assert not bad.any(), "%s H=%d S=%d seq %d (L=%d): %d of %d outputs differ from the row, e.g. head %d ch %d: %r vs %r" % (
            fmt, heads, splits, b, L, int(bad.sum()), bad.size, *np.argwhere(bad)[0],
            float(got[b][tuple(np.argwhere(bad)[0])]), float(want[np.argwhere(bad)[0][1]]))
        assert np.allclose(got_lse[b], ref_lse[b], rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4"])
@pytest.mark.parametrize("heads", [8, 16, 48, 128])
def test_piece_longer_than_page_window(fmt, heads):
    """One piece covering more than 64 pages (the kernels keep a 64-page window
    of the block table in lanes and refill it): sequences above 4096 tokens
    with one split per sequence, through every kernel variant, on random
    page placements; against the oracle."""
    import bit_mla_kv_decode_amd.workloads as W
    _say("page window %s H=%d" % (fmt, heads))
    lens = [5000, 4097, 8300]
    w = W.Workload("window", fmt, batch=len(lens), heads=heads, outliers=fmt == "C2R4", pages="random",
                   seed=heads + 50)
    lens = np.array(lens, np.int32)
    bt, npages = W.page_table(w, lens, 3)
    cache = mla.alloc_cache(fmt, npages)
    for b, L in enumerate(lens):
        la, ro = W.sequence_rows(w, b, 0, int(L), "cuda")
        mla.mla_quant_append(fmt, la, ro, torch.from_numpy(W.slots_for(bt, b, 0, int(L))).cuda(), cache)
    q = W.queries(w, "cpu")
    host = cache.cpu().numpy()
    ref, ref_lse = oracle.decode(OFMT[fmt], q, host, npages, bt, lens, SCALE)
    for splits in (1, 2):
        lse = torch.empty(len(lens), heads, dtype=torch.float32, device="cuda")
        out, _ = mla.mla_decode_lowbit(fmt, q.cuda(), cache, torch.from_numpy(bt).cuda(),
                                       torch.from_numpy(lens).cuda(), SCALE, max_seq_len=int(lens.max()),
                                       num_splits=splits, lse=lse)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        err = np.abs(o - ref)
        bad = err > 2e-3 + 1e-2 * np.abs(ref)
        assert not bad.any(), "splits=%d: %d of %d outside tolerance (max err %.3g)" % (
            splits, int(bad.sum()), bad.size, float(err.max()))
        l = lse.cpu().numpy()
        assert np.allclose(l, ref_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "BF16"])
@pytest.mark.parametrize("heads", [8, 24, 48, 128])
def test_invalid_page_ids_read_as_zero_rows(fmt, heads):
    """Block-table entries outside [0, num_pages) inside a sequence's length
    read as rows of zeros (logit 0, value 0) in every kernel variant: the
    same result as pointing them at an all-zero page, which the oracle
    dequantizes to exact zeros."""
    import bit_mla_kv_decode_amd.workloads as W
    _say("invalid pages %s H=%d" % (fmt, heads))
    lens = np.array([700, 300, 2100], np.int32)
    w = W.Workload("badpages", fmt, batch=len(lens), heads=heads, outliers=fmt == "C2R4", pages="random",
                   seed=heads + 70)
    bt, npages = W.page_table(w, lens, 2)
    cache = mla.alloc_cache(fmt, npages + 1)   # page npages stays zero
    for b, L in enumerate(lens):
        la, ro = W.sequence_rows(w, b, 0, int(L), "cuda")
        mla.mla_quant_append(fmt, la, ro, torch.from_numpy(W.slots_for(bt, b, 0, int(L))).cuda(), cache)
    bad = bt.copy()
    bad[0, 3] = -1
    bad[2, 1] = npages + 7
    bad[2, 20] = -5
    zero_bt = bad.copy()
    zero_bt[(bad < 0) | (bad >= npages + 1)] = npages
    q = W.queries(w, "cpu")
    host = cache.cpu().numpy()
    ref, ref_lse = oracle.decode(OFMT[fmt], q, host, npages + 1, zero_bt, lens, SCALE)
    for splits in (0, 1, 3):
        lse = torch.empty(len(lens), heads, dtype=torch.float32, device="cuda")
        out, _ = mla.mla_decode_lowbit(fmt, q.cuda(), cache, torch.from_numpy(bad).cuda(),
                                       torch.from_numpy(lens).cuda(), SCALE, max_seq_len=int(lens.max()),
                                       num_splits=splits, lse=lse, num_pages=npages + 1)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        err = np.abs(o - ref)
        bad_el = err > 2e-3 + 1e-2 * np.abs(ref)
        assert not bad_el.any(), "splits=%d: %d outside tolerance (max err %.3g)" % (splits, int(bad_el.sum()), float(err.max()))
        assert np.allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-4)
