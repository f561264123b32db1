"""Seeded synthetic inputs for the low-bit MLA decode path.

This module only draws random numbers and lays out page tables.  It holds
none of the method's arithmetic (no quantization, no attention), so both the
GPU path and the CPU oracle can be fed from it.

Value distributions follow the QuantMLA decode workloads used for testing
and benchmarking (the pages name no dataset; everything is synthetic):
  * content latent c[t, ch] = sigma_ch * N(0, 1), sigma_ch log-uniform in
    [0.25, 4]; optionally 5% of the content channels (26 of 512, drawn
    without replacement) are outliers with sigma multiplied by 16;
  * RoPE key: N(0, 1) pairs (2i, 2i+1), i < 32, rotated by the angle
    pos * 10000^(-2i/64) where pos is the token's position in its sequence;
  * queries: N(0, 1) for all d_c + d_r = 576 entries of every head (the
    absorbed content query followed by the rotated RoPE query);
  * every tensor is rounded to bfloat16 (round to nearest even) once drawn.

Each sequence's rows come from their own generator, seeded from
(workload seed, sequence index), so one sequence can be regenerated without
the others.  Draws are reproducible for a given seed and device type.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

D_C = 512
D_R = 64
PAGE = 64


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str                 # "C4R4", "C2R4" or "BF16"
    batch: int
    heads: int
    ctx: int = 0             # fixed context length per sequence (0: drawn, see ctx_range)
    ctx_range: tuple = ()    # (lo, hi): lengths round(exp(U[ln lo, ln hi]))
    outliers: bool = False
    pages: str = "contiguous"  # or "random": a random permutation of the page pool
    seed: int = 0
    max_splits: int = 64
    append_new: bool = False   # one new token per sequence is appended before decode
    note: str = ""

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(128 + 64): the q/k head dimension of a DeepSeek-V3-shaped MLA layer
        return float(np.float32(1.0 / math.sqrt(192.0)))


WORKLOADS = {
    "tiny_c4r4": Workload("tiny_c4r4", "C4R4", batch=1, heads=16, ctx=256, seed=0,
                          note="tiny decode, C4R4, 16 heads, 256 tokens"),
    "dsv3_c4r4_8k": Workload("dsv3_c4r4_8k", "C4R4", batch=32, heads=128, ctx=8192, seed=1,
                             note="DeepSeek-V3-shaped decode, C4R4, 32 x 8K"),
    "c2r4_32k_outliers": Workload("c2r4_32k_outliers", "C2R4", batch=64, heads=128, ctx=32768,
                                  outliers=True, seed=2,
                                  note="C2R4 with 5% outlier channels, 64 x 32K"),
    "c4r4_128k": Workload("c4r4_128k", "C4R4", batch=8, heads=128, ctx=131072, seed=3,
                          max_splits=64, note="long-context C4R4, 8 x 128K, split-KV"),
    "mixed_c2r4_serving": Workload("mixed_c2r4_serving", "C2R4", batch=128, heads=128,
                                   ctx_range=(1024, 131072), pages="random", seed=4,
                                   append_new=True,
                                   note="mixed serving step, C2R4, 128 sequences, 1K-128K, random pages"),
}


def derive(w: Workload, **kw) -> Workload:
    """A copy of `w` with some fields replaced (e.g. fewer sequences for a test)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


# --------------------------------------------------------------------- host-side draws

def seq_lens(w: Workload) -> np.ndarray:
    """Context length of every sequence (tokens, including an appended one)."""
    if w.ctx_range:
        rng = np.random.Generator(np.random.PCG64(w.seed))
        lo, hi = w.ctx_range
        u = rng.uniform(math.log(lo), math.log(hi), size=w.batch)
        return np.rint(np.exp(u)).astype(np.int32)
    return np.full(w.batch, w.ctx, dtype=np.int32)


def page_table(w: Workload, lens: np.ndarray, extra_pages: int = 0):
    """Block table [batch, max_pages] (int32, -1 past each sequence) and pool size.

    "contiguous": sequence b owns consecutive pages in sequence order.
    "random": the pool's pages are handed out in a random order."""
    npg = (lens.astype(np.int64) + PAGE - 1) // PAGE
    max_pages = int(max(1, npg.max() if npg.size else 1))
    total = int(npg.sum()) + extra_pages
    if w.pages == "random":
        rng = np.random.Generator(np.random.PCG64(w.seed + 7919))
        pool = rng.permutation(total).astype(np.int32)
    else:
        pool = np.arange(total, dtype=np.int32)
    bt = np.full((len(lens), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(npg):
        bt[b, :n] = pool[pos:pos + n]
        pos += int(n)
    return bt, max(total, 1)


def slots_for(block_table: np.ndarray, b: int, t0: int, t1: int) -> np.ndarray:
    """Physical slots (page * PAGE + offset) of tokens [t0, t1) of sequence b."""
    t = np.arange(t0, t1, dtype=np.int64)
    return (block_table[b, t // PAGE].astype(np.int64) * PAGE + t % PAGE).astype(np.int32)


# --------------------------------------------------------------------- tensor draws

def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def channel_sigma(w: Workload) -> torch.Tensor:
    """Per-channel std of the content latent (float32 [D_C], host)."""
    rng = np.random.Generator(np.random.PCG64(w.seed * 1000 + 17))
    sig = np.exp(rng.uniform(math.log(0.25), math.log(4.0), size=D_C))
    if w.outliers:
        idx = rng.choice(D_C, size=int(round(0.05 * D_C)), replace=False)
        sig[idx] *= 16.0
    return torch.from_numpy(sig.astype(np.float32))


def sequence_rows(w: Workload, b: int, t0: int, t1: int, device="cpu"):
    """bf16 latent [t1-t0, D_C] and RoPE key [t1-t0, D_R] for tokens [t0, t1) of sequence b.

    Rows of one sequence are drawn in blocks of 4096 positions, each block from
    its own generator, so any sub-range is reproducible on its own."""
    sig = channel_sigma(w).to(device)
    lat_parts, rope_parts = [], []
    blk = 4096
    i = (t0 // blk) * blk
    inv = torch.pow(torch.tensor(10000.0, dtype=torch.float64),
                    -torch.arange(0, D_R, 2, dtype=torch.float64) / D_R).to(device)
    while i < t1:
        j = i + blk
        g = _gen(((w.seed * 1_000_003 + b) * 65_537 + i // blk) & 0x7FFF_FFFF_FFFF, device)
        z = torch.randn((blk, D_C), generator=g, device=device, dtype=torch.float32)
        r = torch.randn((blk, D_R // 2, 2), generator=g, device=device, dtype=torch.float32)
        lo, hi = max(t0, i) - i, min(t1, j) - i
        z = z[lo:hi] * sig
        r = r[lo:hi].double()
        pos = torch.arange(i + lo, i + hi, dtype=torch.float64, device=device)
        ang = pos[:, None] * inv[None, :]
        c, s = torch.cos(ang), torch.sin(ang)
        x0, x1 = r[..., 0], r[..., 1]
        rot = torch.stack([x0 * c - x1 * s, x0 * s + x1 * c], dim=-1).reshape(hi - lo, D_R)
        lat_parts.append(z.to(torch.bfloat16))
        rope_parts.append(rot.float().to(torch.bfloat16))
        i = j
    return torch.cat(lat_parts, 0), torch.cat(rope_parts, 0)


def queries(w: Workload, device="cpu", heads: int | None = None) -> torch.Tensor:
    """bf16 [batch, heads, D_C + D_R] absorbed queries (RoPE part already rotated)."""
    h = w.heads if heads is None else heads
    g = _gen(w.seed * 31 + 5, device)
    return torch.randn((w.batch, h, D_C + D_R), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def new_token_rows(w: Workload, lens: np.ndarray, device="cpu"):
    """Rows of the token appended at position L_b - 1 of every sequence."""
    lat, rope = [], []
    for b, L in enumerate(lens):
        l, r = sequence_rows(w, b, int(L) - 1, int(L), device)
        lat.append(l)
        rope.append(r)
    return torch.cat(lat, 0), torch.cat(rope, 0)


def absorb_inputs(batch: int, heads: int, seed: int, device="cpu"):
    """Synthetic weights and queries of the absorbed projections: q_nope
    [B, H, 128] and q_pe [B, H, 64] ~ N(0, 1); w_uk [H, 512, 128] ~ N(0, 1/128)
    and w_uv [H, 128, 512] ~ N(0, 1/512) (unit-variance outputs); bf16."""
    g = np.random.Generator(np.random.PCG64(seed))
    def bf(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(device)
    q_nope = bf(g.standard_normal((batch, heads, 128)))
    q_pe = bf(g.standard_normal((batch, heads, 64)))
    w_uk = bf(g.standard_normal((heads, 512, 128)) / np.sqrt(128.0))
    w_uv = bf(g.standard_normal((heads, 128, 512)) / np.sqrt(512.0))
    return q_nope, q_pe, w_uk, w_uv
