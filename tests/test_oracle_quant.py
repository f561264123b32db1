"""Pins for the oracle's number formats, quantizer, packing and dequantizer.

None of these re-types the oracle's own formula: each checks it against an
independent fact (a library conversion routine, exact rational arithmetic,
exact grids and ties, brute-force search, or hand-derived bytes of the page
layout).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.Generator(np.random.PCG64(1234))


def _f16_bits_numpy(x: np.ndarray) -> np.ndarray:
    return x.astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------- number formats

def test_f16_rounding_matches_numpy():
    # numpy's float32 -> float16 cast rounds to nearest even, with subnormals.
    bits = RNG.integers(0, 2**32, size=40000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    keep = np.isfinite(x) & (np.abs(x) < 65504.0)
    x = x[keep]
    # add exact ties and the subnormal range
    extra = []
    for e in range(-26, 16):
        for m in (0x000, 0x001, 0x3FF, 0x155):
            base = np.float32(2.0 ** e * (1 + m / 1024.0))
            extra += [base, np.float32(base * (1 + 2.0 ** -11)), np.float32(base * (1 + 3 * 2.0 ** -12))]
    x = np.concatenate([x, np.array(extra, dtype=np.float32), -np.array(extra, dtype=np.float32),
                        np.array([0.0, -0.0, 65504.0, 65519.99, 5.96e-8, 2.98e-8, 2.99e-8], dtype=np.float32)])
    x = x[np.abs(x) < 65520.0]
    ref = _f16_bits_numpy(x)
    got = np.array([oracle.f32_to_f16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    # and back: every fp16 pattern widens exactly
    allh = np.arange(0, 0x7C00, dtype=np.uint16)
    wide = np.array([oracle.f16_to_f32(int(h)) for h in allh[::7]], dtype=np.float32)
    assert np.array_equal(wide, allh[::7].view(np.float16).astype(np.float32))


def test_f16_overflow_is_an_error():
    assert oracle.f32_to_f16(65520.0) is None
    assert oracle.f32_to_f16(float("inf")) is None
    assert oracle.f32_to_f16(float("nan")) is None
    assert oracle.f32_to_f16(65519.0) == 0x7BFF


def test_bf16_rounding_matches_torch():
    bits = RNG.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[::3] = (bits[::3] & 0xFFFF0000) | 0x8000      # exact ties
    bits[1::5] = (bits[1::5] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3e38)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lib = oracle.lib()
    got = np.array([lib.oracle_f32_to_bf16(float(v)) for v in x[:50000]], dtype=np.uint16)
    assert np.array_equal(got, ref[:50000])


# ----------------------------------------------------------------- quantizer

@pytest.mark.parametrize("bits,G", [(4, 64), (2, 32), (4, 32), (2, 64)])
def test_exact_grid_gives_exact_codes(bits, G):
    """x = Z + k*S with power-of-two S and Z, group spanning 0..qmax: codes == k."""
    qmax = 2**bits - 1
    for S, Z in [(0.25, -2.0), (2.0 ** -6, 1.0), (4.0, -64.0), (1.0, 0.0)]:
        k = RNG.integers(0, qmax + 1, size=G)
        k[0], k[1] = 0, qmax
        RNG.shuffle(k)
        x = (Z + k * S).astype(np.float32)
        codes, s16, z16 = oracle.quant_group(x, bits)
        assert oracle.f16_to_f32(s16) == S and oracle.f16_to_f32(z16) == Z
        assert np.array_equal(codes, k.astype(np.uint8))


@pytest.mark.parametrize("bits", [2, 4])
def test_ties_round_half_to_even(bits):
    qmax = 2**bits - 1
    ties = np.arange(qmax, dtype=np.float64) + 0.5          # 0.5, 1.5, ...
    x = np.concatenate([[0.0, float(qmax)], ties]).astype(np.float32)
    codes, s16, z16 = oracle.quant_group(x, bits)
    assert oracle.f16_to_f32(s16) == 1.0 and oracle.f16_to_f32(z16) == 0.0
    # k + 1/2 goes to whichever of k, k + 1 is even
    expect = [0, qmax] + [int(v) if int(v) % 2 == 0 else int(v) + 1 for v in ties]
    assert codes.tolist() == expect
    if bits == 4:
        assert codes[2:5].tolist() == [0, 2, 2]          # 0.5 -> 0, 1.5 -> 2, 2.5 -> 2


def _bf16_group(G, scale, shift=0.0):
    x = (RNG.standard_normal(G) * scale + shift).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("bits,G", [(4, 64), (2, 32)])
def test_round_trip_and_brute_force(bits, G):
    """Round trip within half a step, and codes equal the brute-force nearest level."""
    qmax = 2**bits - 1
    near_tie = 0
    for it in range(300):
        scale = float(np.exp(RNG.uniform(np.log(0.05), np.log(64))))
        x = _bf16_group(G, scale, shift=float(RNG.uniform(-1, 1)) * scale * (it % 3))
        codes, s16, z16 = oracle.quant_group(x, bits)
        S = Fraction(oracle.f16_to_f32(s16))
        Z = Fraction(oracle.f16_to_f32(z16))
        mn = Fraction(float(x.min()))
        if S == 0:
            assert not codes.any()
            continue
        for xi, c in zip(x, codes):
            X = Fraction(float(xi))
            # brute force over all levels (ties to even), exact arithmetic
            dists = [abs(X - (k * S + Z)) for k in range(qmax + 1)]
            best = min(dists)
            cands = [k for k in range(qmax + 1) if dists[k] == best]
            bf = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
            t_exact = (X - Z) / S
            frac = t_exact - math.floor(t_exact)
            if abs(frac - Fraction(1, 2)) < Fraction(1, 2**20):
                near_tie += 1
                assert c in (bf, bf - 1, bf + 1)
            else:
                assert int(c) == bf, (float(X), float(S), float(Z))
            # round trip: exact bound with the stored S, Z
            err = abs(X - (int(c) * S + Z))
            if Z == mn:
                assert err <= S / 2
            s32 = Fraction(float(np.float32(np.float32(float(x.max())) - np.float32(float(x.min()))) / np.float32(qmax)))
            assert err <= S / 2 + qmax * abs(s32 - S) + abs(mn - Z)
    assert near_tie < 50


def test_signed_zero_and_constant_groups():
    x = np.zeros(64, dtype=np.float32)
    x[3] = -0.0
    x[10] = 1.0
    codes, s16, z16 = oracle.quant_group(x, 4)
    assert z16 == 0x0000                      # -0 minimum stored as +0
    x = np.full(64, -0.0, dtype=np.float32)
    codes, s16, z16 = oracle.quant_group(x, 4)
    assert (s16, z16) == (0, 0) and not codes.any()
    x = np.full(32, 3.25, dtype=np.float32)
    codes, s16, z16 = oracle.quant_group(x, 2)
    assert s16 == 0 and oracle.f16_to_f32(z16) == 3.25 and not codes.any()
    assert oracle.dequant_value(0, s16, z16) == 3.25


def test_quantizer_rejects_unrepresentable_groups():
    with pytest.raises(ValueError):
        oracle.quant_group(np.array([-1e6, 1e6] * 16, dtype=np.float32), 4)
    with pytest.raises(ValueError):
        oracle.quant_group(np.array([np.inf] + [0.0] * 31, dtype=np.float32), 2)


def test_dequant_is_single_fma_then_bf16():
    """bf16_rne(fma(code, S, Z)): exact code*S+Z (float64 holds it exactly here),
    one rounding to float32 (numpy), then bf16 (torch)."""
    for _ in range(3000):
        code = int(RNG.integers(0, 16))
        s16 = int(oracle.f32_to_f16(float(np.exp(RNG.uniform(-8, 4)))))
        z16 = int(oracle.f32_to_f16(float(RNG.standard_normal() * 8)))
        exact = code * float(np.uint16(s16).view(np.float16)) + float(np.uint16(z16).view(np.float16))
        f32 = np.float32(exact)
        ref = torch.tensor([float(f32)], dtype=torch.float32).to(torch.bfloat16).float().item()
        assert oracle.dequant_value(code, s16, z16) == ref


# ----------------------------------------------------------------- packing / layout

def test_page_sizes():
    assert oracle.page_bytes(oracle.C4R4) == 20736 == 64 * 324
    assert oracle.page_bytes(oracle.C2R4) == 14592 == 64 * 228
    assert oracle.page_bytes(oracle.BF16) == 73728 == 64 * 1152


def _load_golden():
    import os
    p = os.path.join(os.path.dirname(__file__), "golden", "pack_bytes.txt")
    out = {}
    for line in open(p):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        out[k.strip()] = bytes.fromhex(v.strip())
    return out


def test_golden_bytes_int4_and_int2():
    gold = _load_golden()
    tok = 5
    # C4R4: content channel c has value c % 16 inside every 64-channel group; RoPE = 15 - (c % 16)
    lat = np.array([c % 16 for c in range(512)], dtype=np.float32)
    rope = np.array([15 - (c % 16) for c in range(64)], dtype=np.float32)
    cache = np.zeros(2 * 20736, dtype=np.uint8)
    lat16 = torch.from_numpy(lat[None]).to(torch.bfloat16)
    rope16 = torch.from_numpy(rope[None]).to(torch.bfloat16)
    oracle.quant_append(oracle.C4R4, lat16, rope16, np.array([64 + tok]), cache, 2)
    page = cache[20736:]
    # region A, chunk j, token 5 at (j*64 + 5)*16
    for j in range(16):
        off = (j * 64 + tok) * 16
        assert bytes(page[off:off + 16]) == gold["int4_chunk_0_15"]
    # region B at 16384: group g, token 5 at 16384 + (g*64+5)*4: S16 = fp16(1.0), Z16 = 0
    for g in range(8):
        off = 16384 + (g * 64 + tok) * 4
        assert bytes(page[off:off + 4]) == gold["sz_s1_z0"]
    # region C (RoPE codes) at 18432, region D at 20480
    for j in range(2):
        off = 18432 + (j * 64 + tok) * 16
        assert bytes(page[off:off + 16]) == gold["int4_chunk_15_0"]
    assert bytes(page[20480 + tok * 4:20480 + tok * 4 + 4]) == gold["sz_s1_z0"]
    # nothing else in the page was touched
    touched = np.zeros(20736, dtype=bool)
    for j in range(16):
        touched[(j * 64 + tok) * 16:(j * 64 + tok) * 16 + 16] = True
    for g in range(8):
        touched[16384 + (g * 64 + tok) * 4:16384 + (g * 64 + tok) * 4 + 4] = True
    for j in range(2):
        touched[18432 + (j * 64 + tok) * 16:18432 + (j * 64 + tok) * 16 + 16] = True
    touched[20480 + tok * 4:20480 + tok * 4 + 4] = True
    assert not page[~touched].any()
    assert not cache[:20736].any()

    # C2R4: content value c % 4 in 32-channel groups -> INT2 bytes E4 repeated
    lat = np.array([c % 4 for c in range(512)], dtype=np.float32)
    cache = np.zeros(14592, dtype=np.uint8)
    oracle.quant_append(oracle.C2R4, torch.from_numpy(lat[None]).to(torch.bfloat16), rope16,
                        np.array([tok]), cache, 1)
    for j in range(8):
        off = (j * 64 + tok) * 16
        assert bytes(cache[off:off + 16]) == gold["int2_chunk_0123"]
    s_gold = gold["sz_s1_z0"]
    for g in range(16):
        off = 8192 + (g * 64 + tok) * 4
        assert bytes(cache[off:off + 4]) == s_gold
    assert bytes(cache[12288 + tok * 16:12288 + tok * 16 + 16]) == gold["int4_chunk_15_0"]
    assert bytes(cache[14336 + tok * 4:14336 + tok * 4 + 4]) == s_gold


def test_channel_to_byte_positions():
    """Changing one channel changes exactly the nibble / bit pair the layout assigns to it."""
    for fmt, bits in ((oracle.C4R4, 4), (oracle.C2R4, 2)):
        pb = oracle.page_bytes(fmt)
        G = fmt[1]
        for ch in (0, 1, 31, 32, 63, 64, 200, 511):
            lat = np.zeros(512, dtype=np.float32)
            g0 = (ch // G) * G
            lat[g0] = 0.0
            lat[g0 + (1 if ch == g0 else 0)] = float(2**bits - 1)   # fixes S = 1, Z = 0
            lat[ch] = 1.0 if ch != g0 + (1 if ch == g0 else 0) else lat[ch]
            rope = np.zeros(64, dtype=np.float32)
            c1 = np.zeros(pb, dtype=np.uint8)
            oracle.quant_append(fmt, torch.from_numpy(lat[None]).to(torch.bfloat16),
                                torch.from_numpy(rope[None]).to(torch.bfloat16), np.array([0]), c1, 1)
            per_chunk = 128 // bits
            chunk, e = ch // per_chunk, ch % per_chunk
            byte = chunk * 64 * 16 + (e * bits) // 8
            code = (c1[byte] >> ((e * bits) % 8)) & (2**bits - 1)
            assert code == int(lat[ch]), (bits, ch)


def test_append_matches_group_quantizer_and_dequant():
    """The page written by quant_append decodes to bf16(fma(code, S, Z)) with the
    codes/scales of quant_group applied group by group."""
    for fmt in (oracle.C4R4, oracle.C2R4):
        bits, G, rbits, rG = fmt[0], fmt[1], fmt[2], fmt[3]
        n = 70
        lat = torch.randn(n, 512) * torch.exp(torch.empty(512).uniform_(-1.4, 1.4))
        rope = torch.randn(n, 64)
        lat16, rope16 = lat.to(torch.bfloat16), rope.to(torch.bfloat16)
        num_pages = 3
        cache = np.zeros(num_pages * oracle.page_bytes(fmt), dtype=np.uint8)
        perm = np.array([2, 0], dtype=np.int32)
        slots = np.array([perm[t // 64] * 64 + t % 64 for t in range(n)], dtype=np.int32)
        oracle.quant_append(fmt, lat16, rope16, slots, cache, num_pages)
        bt = perm[None, :]
        deq = oracle.dequant_cache(fmt, cache, num_pages, bt, np.array([n]))[0]
        for t in (0, 1, 63, 64, 69):
            xs = lat16[t].float().numpy()
            xr = rope16[t].float().numpy()
            for x, off, bb, gg in ((xs, 0, bits, G), (xr, 512, rbits, rG)):
                for g in range(len(x) // gg):
                    codes, s16, z16 = oracle.quant_group(x[g * gg:(g + 1) * gg], bb)
                    ref = [oracle.dequant_value(int(c), s16, z16) for c in codes]
                    assert np.array_equal(deq[t, off + g * gg:off + (g + 1) * gg], np.array(ref, dtype=np.float32))


def test_bf16_format_is_a_plain_copy():
    n = 5
    lat16 = torch.randn(n, 512).to(torch.bfloat16)
    rope16 = torch.randn(n, 64).to(torch.bfloat16)
    cache = np.zeros(73728, dtype=np.uint8)
    oracle.quant_append(oracle.BF16, lat16, rope16, np.arange(n, dtype=np.int32) + 3, cache, 1)
    rows = cache.view(np.uint16).reshape(64, 576)
    ref = torch.cat([lat16, rope16], 1).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rows[3:8], ref)
    assert not rows[:3].any() and not rows[8:].any()


def test_compression_ratio_of_the_layout():
    """The pages report 3.59x physical compression at 128K for the low-bit cache
    (C4R4 context) but give no byte breakdown; this layout gives 1152/324."""
    import os
    p = os.path.join(os.path.dirname(__file__), "golden", "compression.txt")
    vals = {}
    for line in open(p):
        if line.strip() and not line.startswith("#"):
            k, v = line.split(":")
            vals[k.strip()] = float(v)
    ctx = 131072
    bf16_bytes = ctx * 576 * 2
    for name, fmt in (("c4r4", oracle.C4R4), ("c2r4", oracle.C2R4)):
        packed = (ctx // 64) * oracle.page_bytes(fmt)
        ratio = bf16_bytes / packed
        assert abs(ratio - vals["layout_" + name]) < 1e-3
    # the pages' figure sits within 1% of this layout's C4R4 ratio (parity unpinned: no breakdown)
    assert abs(vals["pages_reported"] / vals["layout_c4r4"] - 1) < 0.01
