"""Pins for the oracle's absorbed projections (absorb_q, project_out).

An explicit summation over sampled elements, and the MLA identity the
absorption rests on: attention with the absorbed query, followed by the value
projection, equals unabsorbed attention with explicit per-head keys
W_UK c and values W_UV c.
"""
import math

import numpy as np
import torch

import oracle
from bit_mla_kv_decode_amd import workloads as W


def _bf(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def test_projections_match_explicit_sums():
    q_nope, q_pe, w_uk, w_uv = W.absorb_inputs(3, 4, seed=1)
    qc = oracle.absorb_q(q_nope, w_uk)
    lat = _bf(np.random.default_rng(2).standard_normal((3, 4, 512)))
    o = oracle.project_out(lat, w_uv)
    qn, wk, wv, lt = (t.double().numpy() for t in (q_nope, w_uk, w_uv, lat))
    rng = np.random.default_rng(3)
    for _ in range(40):
        b, h, n, j = rng.integers(3), rng.integers(4), rng.integers(512), rng.integers(128)
        assert math.isclose(qc[b, h, n], math.fsum(qn[b, h, k] * wk[h, n, k] for k in range(128)),
                            rel_tol=1e-12, abs_tol=1e-12)
        assert math.isclose(o[b, h, j], math.fsum(lt[b, h, c] * wv[h, j, c] for c in range(512)),
                            rel_tol=1e-12, abs_tol=1e-12)


def test_absorbed_attention_equals_unabsorbed_mla():
    B, H, L = 2, 3, 40
    q_nope, q_pe, w_uk, w_uv = W.absorb_inputs(B, H, seed=4)
    g = torch.Generator().manual_seed(5)
    c = torch.randn(B, L, 512, generator=g).double()          # latents
    kr = torch.randn(B, L, 64, generator=g).double()           # RoPE keys
    scale = 1.0 / math.sqrt(192.0)
    qc = torch.from_numpy(oracle.absorb_q(q_nope, w_uk))      # [B, H, 512]
    qn, qp, wk, wv = (t.double() for t in (q_nope, q_pe, w_uk, w_uv))
    for b in range(B):
        # absorbed: logits over the latent, aggregate the latent, project once
        logits_a = (qc[b] @ c[b].T + qp[b] @ kr[b].T) * scale              # [H, L]
        lat = torch.softmax(logits_a, -1) @ c[b]                           # [H, 512]
        out_a = oracle.project_out(lat[None].numpy(), w_uv)[0]
        # unabsorbed: explicit keys and values per head
        keys = torch.einsum("hnk,ln->hlk", wk, c[b])                       # [H, L, 128]
        vals = torch.einsum("hjc,lc->hlj", wv, c[b])                       # [H, L, 128]
        logits_u = (torch.einsum("hk,hlk->hl", qn[b], keys) + qp[b] @ kr[b].T) * scale
        out_u = torch.einsum("hl,hlj->hj", torch.softmax(logits_u, -1), vals)
        assert torch.allclose(logits_a, logits_u, rtol=1e-12, atol=1e-10)
        assert np.allclose(out_a, out_u.numpy(), rtol=1e-11, atol=1e-12)
