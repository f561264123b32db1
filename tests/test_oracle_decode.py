"""Pins for the oracle's decode attention (fp64) and its split/combine algebra.

Each test checks the oracle against something other than itself: PyTorch's
scaled-dot-product attention (a library routine), unabsorbed naive MLA (the
absorbed form must agree by associativity), exact closed forms, and a
50-digit mpmath brute force on tiny inputs.
"""
import math

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _build(fmt, lens, H=3, seed=0, sig=None, perm=True):
    """Random bf16 rows appended through the oracle into a shuffled page pool."""
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    npg = [(L + 63) // 64 for L in lens]
    total = sum(npg) + 1
    pool = torch.randperm(total, generator=g).numpy().astype(np.int32) if perm else np.arange(total, dtype=np.int32)
    MP = max(max(npg), 1)
    bt = np.full((B, MP), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(npg):
        bt[b, :n] = pool[pos:pos + n]
        pos += n
    pb = oracle.page_bytes(fmt)
    cache = np.zeros(total * pb, dtype=np.uint8)
    lat_all, rope_all = [], []
    for b, L in enumerate(lens):
        s = sig if sig is not None else torch.exp(torch.empty(512).uniform_(-1.4, 1.4, generator=g))
        lat = (torch.randn(L, 512, generator=g) * s).to(torch.bfloat16)
        rope = torch.randn(L, 64, generator=g).to(torch.bfloat16)
        t = np.arange(L)
        slots = (bt[b, t // 64].astype(np.int64) * 64 + t % 64).astype(np.int32)
        oracle.quant_append(fmt, lat, rope, slots, cache, total)
        lat_all.append(lat)
        rope_all.append(rope)
    q = torch.randn(B, H, 576, generator=g).to(torch.bfloat16)
    return cache, total, bt, np.array(lens, dtype=np.int32), q, lat_all, rope_all


@pytest.mark.parametrize("fmt", [oracle.BF16, oracle.C4R4, oracle.C2R4])
def test_decode_equals_torch_sdpa(fmt):
    """out = softmax(scale q [c|k_r]^T) c, lse = logsumexp: against F.scaled_dot_product_attention in fp64."""
    lens = [70, 1, 130, 64]
    cache, npages, bt, sl, q, lat, rope = _build(fmt, lens, H=3, seed=1)
    out, lse = oracle.decode(fmt, q, cache, npages, bt, sl, SCALE)
    deq = oracle.dequant_cache(fmt, cache, npages, bt, sl)
    for b, L in enumerate(lens):
        if fmt == oracle.BF16:
            K = torch.cat([lat[b], rope[b]], 1).double()
            assert np.array_equal(deq[b, :L], K.float().numpy())
        else:
            K = torch.from_numpy(deq[b, :L]).double()
        V = K[:, :512]
        qd = q[b].double()                                    # [H, 576]
        ref = F.scaled_dot_product_attention(qd[None, :, None, :], K[None, None].expand(1, 3, L, 576),
                                             V[None, None].expand(1, 3, L, 512), scale=SCALE)[0, :, 0]
        assert np.allclose(out[b], ref.numpy(), rtol=0, atol=1e-12 * max(1.0, float(V.abs().max())))
        ref_lse = torch.logsumexp(SCALE * (qd @ K.T), dim=1)
        assert np.allclose(lse[b], ref_lse.numpy(), rtol=1e-13, atol=1e-13)


def test_absorbed_equals_naive_unabsorbed_mla():
    """Per head, naive MLA with up-projections W_UK [128 x 512] and W_UV [128 x 512]
    (keys k_t = W_UK c_t, values v_t = W_UV c_t) equals W_UV applied to the
    absorbed output with q_c = W_UK^T q_nope.  Integer-valued W_UK and q_nope keep
    q_c exact in bf16."""
    g = torch.Generator().manual_seed(7)
    H, L = 4, 150
    cache, npages, bt, sl, _, lat, rope = _build(oracle.BF16, [L], H=H, seed=3)
    W_UK = torch.randint(-1, 2, (H, 128, 512), generator=g).double()
    W_UK[torch.rand(W_UK.shape, generator=g) < 0.6] = 0
    W_UV = torch.randn(H, 128, 512, generator=g).double()
    q_nope = torch.randint(-1, 2, (H, 128), generator=g).double()
    q_rope = torch.randn(H, 64, generator=g).to(torch.bfloat16).double()
    q_c = torch.einsum("hdc,hd->hc", W_UK, q_nope)
    assert q_c.abs().max() <= 128
    q = torch.cat([q_c, q_rope], 1).to(torch.bfloat16)
    assert torch.equal(q.double()[:, :512], q_c)
    out, lse = oracle.decode(oracle.BF16, q[None], cache, npages, bt, sl, SCALE)
    c = lat[0].double()
    kr = rope[0].double()
    for h in range(H):
        k_nope = c @ W_UK[h].T                                # [L, 128]
        logits = SCALE * (k_nope @ q_nope[h] + kr @ q_rope[h])
        p = torch.softmax(logits, 0)
        v = c @ W_UV[h].T                                     # [L, 128]
        naive = p @ v
        absorbed = W_UV[h] @ torch.from_numpy(out[0, h])
        assert torch.allclose(absorbed, naive, rtol=1e-10, atol=1e-10)


def test_softmax_weights_sum_to_one():
    cache, npages, bt, sl, q, _, _ = _build(oracle.C2R4, [200, 3, 64], H=2, seed=4)
    out, lse, w = oracle.decode(oracle.C2R4, q, cache, npages, bt, sl, SCALE, want_weights=True)
    for b, L in enumerate(sl):
        s = w[b, :, :L].sum(axis=1)
        assert np.allclose(s, 1.0, rtol=0, atol=1e-12)
        assert (w[b, :, L:] == 0).all()


def test_closed_forms():
    # one token: the output is that token's dequantized latent, exactly
    cache, npages, bt, sl, q, _, _ = _build(oracle.C4R4, [1], H=5, seed=5)
    out, lse = oracle.decode(oracle.C4R4, q, cache, npages, bt, sl, SCALE)
    deq = oracle.dequant_cache(oracle.C4R4, cache, npages, bt, sl)
    assert np.array_equal(out[0], np.broadcast_to(deq[0, 0, :512].astype(np.float64), (5, 512)))
    # zero query: every logit is 0, so the output is the mean row and lse = log L
    L = 97
    cache, npages, bt, sl, q, _, _ = _build(oracle.C2R4, [L], H=2, seed=6)
    q = torch.zeros_like(q)
    out, lse = oracle.decode(oracle.C2R4, q, cache, npages, bt, sl, SCALE)
    deq = oracle.dequant_cache(oracle.C2R4, cache, npages, bt, sl)
    assert np.allclose(out[0], deq[0, :L, :512].astype(np.float64).mean(0), rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, math.log(L), rtol=1e-15, atol=1e-15)
    # identical keys: output equals that row whatever the query
    row_lat = torch.randn(1, 512).to(torch.bfloat16).repeat(40, 1)
    row_rope = torch.randn(1, 64).to(torch.bfloat16).repeat(40, 1)
    cache = np.zeros(oracle.page_bytes(oracle.C4R4), dtype=np.uint8)
    oracle.quant_append(oracle.C4R4, row_lat, row_rope, np.arange(40, dtype=np.int32), cache, 1)
    qq = torch.randn(1, 3, 576).to(torch.bfloat16)
    out, lse = oracle.decode(oracle.C4R4, qq, cache, 1, np.zeros((1, 1), np.int32), np.array([40], np.int32), SCALE)
    deq = oracle.dequant_cache(oracle.C4R4, cache, 1, np.zeros((1, 1), np.int32), np.array([40], np.int32))
    assert np.allclose(out[0], deq[0, 0, :512].astype(np.float64), rtol=1e-14, atol=1e-14)
    # an empty sequence: zeros and lse = -inf
    cache, npages, bt, sl, q, _, _ = _build(oracle.C4R4, [0, 5], H=2, seed=8)
    out, lse = oracle.decode(oracle.C4R4, q, cache, npages, bt, sl, SCALE)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all() and np.isfinite(lse[1]).all()


def test_mpmath_brute_force_tiny():
    mpmath.mp.dps = 50
    for seed, (fmt, lens, H) in enumerate([(oracle.C4R4, [5, 8], 2), (oracle.C2R4, [3], 1),
                                          (oracle.BF16, [7], 2)]):
        cache, npages, bt, sl, q, _, _ = _build(fmt, lens, H=H, seed=20 + seed)
        out, lse = oracle.decode(fmt, q, cache, npages, bt, sl, SCALE)
        deq = oracle.dequant_cache(fmt, cache, npages, bt, sl)
        qf = q.float().numpy()
        sc = mpmath.mpf(SCALE)
        for b, L in enumerate(lens):
            for h in range(H):
                logits = [sc * mpmath.fsum(mpmath.mpf(float(qf[b, h, i])) * mpmath.mpf(float(deq[b, t, i]))
                                           for i in range(576)) for t in range(L)]
                m = max(logits)
                e = [mpmath.exp(x - m) for x in logits]
                Z = mpmath.fsum(e)
                for c in range(0, 512, 37):
                    ref = mpmath.fsum(e[t] * mpmath.mpf(float(deq[b, t, c])) for t in range(L)) / Z
                    assert abs(float(ref) - out[b, h, c]) <= 1e-12 * max(1.0, abs(float(ref)))
                assert abs(float(m + mpmath.log(Z)) - lse[b, h]) <= 1e-12 * max(1.0, abs(lse[b, h]))


def test_split_combine_equals_unsplit():
    lens = [300, 64, 1, 129]
    cache, npages, bt, sl, q, _, _ = _build(oracle.C4R4, lens, H=3, seed=9)
    full, lse = oracle.decode(oracle.C4R4, q, cache, npages, bt, sl, SCALE)
    for bounds in ([0, 64, 128, 192, 256, 320], [0, 1, 100, 400], [0, 200, 200, 1000]):
        parts, lses = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            o, l = oracle.decode(oracle.C4R4, q, cache, npages, bt, sl, SCALE, t_begin=a, t_end=b)
            parts.append(o)
            lses.append(l)
        out, l2 = oracle.combine(np.stack(parts), np.stack(lses))
        assert np.allclose(out, full, rtol=1e-12, atol=1e-12)
        assert np.allclose(l2, lse, rtol=1e-12, atol=1e-12)
    # all partials empty -> zeros, -inf
    out, l2 = oracle.combine(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert (out == 0).all() and np.isneginf(l2).all()


def test_decode_detects_page_errors():
    cache, npages, bt, sl, q, _, _ = _build(oracle.C4R4, [70], H=1, seed=10)
    bad = bt.copy()
    bad[0, 1] = npages + 5
    with pytest.raises(ValueError):
        oracle.decode(oracle.C4R4, q, cache, npages, bad, sl, SCALE)


def test_multi_token_decode_is_causal_attention():
    """decode_multi (queries of the last s_q tokens, each seeing itself and the
    tokens before it) against PyTorch SDPA with an explicit causal mask on the
    raw bf16 rows (the 16-bit path), with a sequence shorter than s_q."""
    s_q, H = 3, 2
    fmt = oracle.BF16
    lens = [70, 2, 5]
    cache, total, bt, lens_a, _, lat_all, rope_all = _build(fmt, lens, H=H, seed=21)
    g = torch.Generator().manual_seed(22)
    q = torch.randn(len(lens), s_q, H, 576, generator=g).to(torch.bfloat16)
    out, lse = oracle.decode_multi(fmt, q, cache, total, bt, lens_a, SCALE)
    for b, L in enumerate(lens):
        k = torch.cat([lat_all[b], rope_all[b]], 1).double()
        v = lat_all[b].double()
        for i in range(s_q):
            pos = L - s_q + i                     # position of query i; it sees tokens 0..pos
            if pos < 0:
                assert (out[b, i] == 0).all() and np.isneginf(lse[b, i]).all()
                continue
            mask = torch.arange(L) <= pos
            qi = q[b, i].double()                 # [H, 576]
            ref = F.scaled_dot_product_attention(qi[None], k[None], v[None], attn_mask=mask[None, None, :],
                                                 scale=SCALE)[0]
            logits = (qi @ k.T) * SCALE
            ref_lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
            assert np.allclose(out[b, i], ref.numpy(), rtol=1e-12, atol=1e-12)
            assert np.allclose(lse[b, i], ref_lse.numpy(), rtol=1e-12, atol=1e-12)
    # one query is the single-token decode
    o1, l1 = oracle.decode_multi(fmt, q[:, -1:], cache, total, bt, lens_a, SCALE)
    o2, l2 = oracle.decode(fmt, q[:, -1], cache, total, bt, lens_a, SCALE)
    assert np.array_equal(o1[:, 0], o2) and np.array_equal(l1[:, 0], l2)
