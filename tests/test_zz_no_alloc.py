"""The no-allocation decode entry point (mla_decode_lowbit_noalloc) against
the workspace entry point it mirrors (mla_decode_lowbit): bitwise the same
outputs and log-sum-exps, through the C ABI, on two no-allocation calls in a
row, the second with a smaller input than the first (the scratch keeps the
first call's contents), for every cache format and both partitions; the first
case also against the oracle."""
import math

import numpy as np
import pytest
import torch

import bit_mla_kv_decode_amd as mla
import oracle
from bit_mla_kv_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

OFMT = {"C4R4": oracle.C4R4, "C2R4": oracle.C2R4, "BF16": oracle.BF16}
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _case(fmt, lens, heads, seed):
    w = W.Workload("noalloc", fmt, batch=len(lens), heads=heads, pages="random", seed=seed,
                   outliers=fmt == "C2R4")
    lens = np.asarray(lens, np.int32)
    bt, npages = W.page_table(w, lens, 2)
    cache = mla.alloc_cache(fmt, npages)
    for b, L in enumerate(lens):
        if L:
            lat, rope = W.sequence_rows(w, b, 0, int(L), "cuda")
            mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(W.slots_for(bt, b, 0, int(L))).cuda(), cache)
    q = W.queries(w, "cuda")
    return lens, bt, npages, cache, q, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()


@pytest.mark.parametrize("fmt,splits", [("C4R4", 0), ("C2R4", 0), ("BF16", 0), ("C4R4", 3), ("C2R4", 1)])
def test_noalloc_equals_workspace_entry_point(fmt, splits):
    print("no-alloc decode %s S=%d" % (fmt, splits), flush=True)
    cases = [_case(fmt, [3000, 70, 0, 1500, 129], 128, 1), _case(fmt, [300, 5], 16, 2)]   # second one smaller
    want = []
    for lens, bt, npages, cache, q, btd, sld in cases:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
        out, _ = mla.mla_decode_lowbit(fmt, q, cache, btd, sld, SCALE, max_seq_len=int(lens.max()),
                                       num_splits=splits, lse=lse)
        want.append((out, lse))
    got = []
    for lens, bt, npages, cache, q, btd, sld in cases:   # two no-allocation calls in a row
        out = torch.full((q.shape[0], q.shape[1], 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
        mla.mla_decode_lowbit_noalloc(fmt, q, cache, btd, sld, SCALE, max_seq_len=int(lens.max()),
                                      num_splits=splits, out=out, lse=lse)
        got.append((out, lse))
    torch.cuda.synchronize()
    for i, ((o1, l1), (o2, l2)) in enumerate(zip(want, got)):
        assert torch.equal(o1, o2), "call %d: outputs differ" % i
        assert torch.equal(l1, l2), "call %d: log-sum-exps differ" % i
    lens, bt, npages, cache, q, btd, sld = cases[0]
    ref, ref_lse = oracle.decode(OFMT[fmt], q.cpu(), cache.cpu().numpy(), npages, bt, lens, SCALE)
    o = got[0][0].float().cpu().numpy()
    assert not (np.abs(o - ref) > 2e-3 + 1e-2 * np.abs(ref)).any()
    l = got[0][1].cpu().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse))
    assert np.allclose(l[fin], ref_lse[fin], rtol=1e-5, atol=1e-4)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """A batch whose partials exceed the scratch is refused before any launch."""
    fmt = "C4R4"
    B = 600   # (256 + 600) balanced slots x 128 heads x 2 KiB > 128 MiB
    assert mla.mla_decode_workspace_bytes(fmt, B, 128, 0) > 128 << 20
    q = torch.zeros(B, 128, 576, dtype=torch.bfloat16, device="cuda")
    cache = mla.alloc_cache(fmt, 1)
    bt = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_lowbit_noalloc(fmt, q, cache, bt, sl, SCALE, num_splits=0)
    assert e.value.status == mla.MLA_ERR_WORKSPACE and "scratch" in str(e.value)
