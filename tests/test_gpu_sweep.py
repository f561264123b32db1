"""Seeded random sweep of decode configurations against the CPU oracle.

Each case draws a format, a head count from every kernel variant's range
(<= 16, 17..32, 33..64 and > 64 heads, at most 128), a query count (more
than 128 rows of queries x heads go into head chunks), a partition (balanced or
1..5 fixed splits) and a batch whose lengths mix empty sequences, single
tokens, partial tiles and pages, and a longer context, on a random page
placement.  The output must lie within |out - ref| <= 2e-3 + 1e-2 |ref| of
the fp64 oracle on the same quantized cache, and the log-sum-exps within
1e-5 relative."""
import numpy as np
import pytest
import torch

import bit_mla_kv_decode_amd as mla
import oracle
from test_gpu_parity import OFMT, SCALE, _say, assert_close, assert_lse, build, gpu_cache

pytestmark = pytest.mark.gpu

HEAD_RANGES = [(1, 16), (17, 32), (33, 64), (65, 128), (48, 128)]   # the last with 2 or 3 queries: head chunks


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    fmt = ["C4R4", "C2R4", "BF16"][seed % 3]
    lo, hi = HEAD_RANGES[(seed // 3) % len(HEAD_RANGES)]
    heads = int(rng.integers(lo, hi + 1))
    s_q = int(rng.choice([2, 3])) if (seed // 3) % len(HEAD_RANGES) == 4 else int(rng.choice([1, 1, 2, 3]))
    batch = int(rng.integers(1, 9))
    kinds = rng.integers(0, 5, size=batch)
    lens = []
    for k in kinds:
        lens.append([0, 1, int(rng.integers(2, 64)), int(rng.integers(65, 700)), int(rng.integers(700, 2600))][k])
    if max(lens) == 0:
        lens[0] = int(rng.integers(1, 300))
    splits = int(rng.choice([0, 0, 1, 2, 5]))
    return fmt, heads, s_q, lens, splits


@pytest.mark.parametrize("seed", range(195))   # 13 rounds of the 3 formats x 5 head ranges
def test_random_configuration(seed):
    fmt, heads, s_q, lens, splits = draw_case(seed)
    _say("sweep %d: %s H=%d s_q=%d splits=%d lens=%s" % (seed, fmt, heads, s_q, splits, lens))
    w, lens, bt, npages, lat, rope, slots, _ = build(fmt, lens, heads, seed=5000 + seed, outliers=fmt == "C2R4")
    cache = gpu_cache(fmt, npages, lat, rope, slots)
    host = cache.cpu().numpy()
    g = torch.Generator().manual_seed(7000 + seed)
    B = len(lens)
    btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
    if s_q == 1:
        q = torch.randn(B, heads, 576, generator=g).to(torch.bfloat16)
        lse = torch.empty(B, heads, dtype=torch.float32, device="cuda")
        out, _ = mla.mla_decode_lowbit(fmt, q.cuda(), cache, btd, sld, SCALE, max_seq_len=int(lens.max()),
                                       num_splits=splits, lse=lse)
        ref, ref_lse = oracle.decode(OFMT[fmt], q, host, npages, bt, lens, SCALE)
    else:
        q = torch.randn(B, s_q, heads, 576, generator=g).to(torch.bfloat16)
        lse = torch.empty(B, s_q, heads, dtype=torch.float32, device="cuda")
        out, _ = mla.mla_decode_multi_lowbit(fmt, q.cuda(), cache, btd, sld, SCALE, max_seq_len=int(lens.max()),
                                             num_splits=splits, lse=lse)
        ref, ref_lse = oracle.decode_multi(OFMT[fmt], q, host, npages, bt, lens, SCALE)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), ref, "sweep %d" % seed)
    assert_lse(lse.cpu().numpy(), ref_lse)
