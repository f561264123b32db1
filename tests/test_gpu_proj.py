"""GPU parity of the absorbed projections (mla_absorb_q, mla_project_out) and
of one MLA decode attention step built from them, against the CPU oracle.

The projections are bf16 outputs of fp32-accumulated products: each element
is within 2^-8 of the fp64 value relative to it (one bf16 rounding plus the
fp32 sums), plus a tiny absolute term for cancelling sums.  The chained step
is held to the decode's tolerance carried through the value projection.
"""
import math

import numpy as np
import pytest
import torch

import bit_mla_kv_decode_amd as mla
import oracle
from bit_mla_kv_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _close(got, ref, rtol=2.0 ** -8, atol=1e-5):
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), "%d of %d outside tolerance, worst %.3g" % (int(bad.sum()), bad.size, float(err.max()))


@pytest.mark.parametrize("B,H", [(1, 128), (8, 128), (33, 16), (130, 7)])
def test_absorb_and_project(B, H):
    print("projections B=%d H=%d" % (B, H), flush=True)
    q_nope, q_pe, w_uk, w_uv = W.absorb_inputs(B, H, seed=B * 31 + H)
    q = mla.mla_absorb_q(q_nope.cuda(), q_pe.cuda(), w_uk.cuda())
    lat = torch.randn(B, H, 512, generator=torch.Generator().manual_seed(B + H)).to(torch.bfloat16)
    o = mla.mla_project_out(lat.cuda(), w_uv.cuda())
    torch.cuda.synchronize()
    qh = q.cpu()
    _close(qh[:, :, :512].float().numpy(), oracle.absorb_q(q_nope, w_uk))
    assert torch.equal(qh[:, :, 512:], q_pe)                    # RoPE part copied bit for bit
    _close(o.float().cpu().numpy(), oracle.project_out(lat, w_uv))


def test_decode_attention_step():
    """absorb -> low-bit decode -> value projection, against the oracle chain
    on the same quantized cache (the absorbed query rounded to bf16 as the
    decode consumes it)."""
    fmt, B, H = "C4R4", 3, 128
    w = W.Workload("step", fmt, batch=B, heads=H, pages="random", seed=9)
    lens = np.array([700, 65, 1], np.int32)
    bt, npages = W.page_table(w, lens, 2)
    cache = mla.alloc_cache(fmt, npages)
    for b, L in enumerate(lens):
        lat, rope = W.sequence_rows(w, b, 0, int(L), "cuda")
        mla.mla_quant_append(fmt, lat, rope, torch.from_numpy(W.slots_for(bt, b, 0, int(L))).cuda(), cache)
    q_nope, q_pe, w_uk, w_uv = W.absorb_inputs(B, H, seed=10)
    q = mla.mla_absorb_q(q_nope.cuda(), q_pe.cuda(), w_uk.cuda())
    latent, _ = mla.mla_decode_lowbit(fmt, q, cache, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                      SCALE)
    o = mla.mla_project_out(latent, w_uv.cuda())
    torch.cuda.synchronize()
    q_ref = torch.from_numpy(oracle.absorb_q(q_nope, w_uk)).float().to(torch.bfloat16)
    q_ref = torch.cat([q_ref, q_pe], -1)
    lat_ref, _ = oracle.decode(oracle.C4R4, q_ref, cache.cpu().numpy(), npages, bt, lens, SCALE)
    o_ref = oracle.project_out(lat_ref, w_uv)
    # the decode's own tolerance (2e-3 + 1e-2 |latent|, which covers its bf16
    # output rounding) pushed through the linear map |W_UV|, plus the final
    # bf16 rounding of the projection
    wabs = np.abs(w_uv.double().numpy())
    bound = np.einsum("bhc,hjc->bhj", 2e-3 + 1e-2 * np.abs(lat_ref), wabs) + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    got = o.float().cpu().numpy()
    err = np.abs(got - o_ref)
    bad = err > bound
    assert not bad.any(), "%d of %d outside tolerance (worst %.3g)" % (int(bad.sum()), bad.size, float(err.max()))
    # and the latent itself meets the decode tolerance
    lat_err = np.abs(latent.float().cpu().numpy() - lat_ref)
    assert (lat_err <= 2e-3 + 1e-2 * np.abs(lat_ref)).all()
