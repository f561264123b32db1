"""CPU oracle for the low-bit MLA cache and its decode attention.

TEST INFRASTRUCTURE ONLY: the plain, slow reference that the GPU library is
checked against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library (``bit_mla_kv_decode_amd``) and never imports it.

The arithmetic lives in ``mla_oracle.c`` (C, fp32 IEEE quantizer, fp64
attention); this module compiles it with gcc and wraps it with ctypes over
numpy arrays.  Each function cites the passage of the QuantMLA pages it
follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Format descriptors as 7 ints: c_bits, c_group, r_bits, r_group, d_c, d_r, page_size.
C4R4 = (4, 64, 4, 64, 512, 64, 64)
C2R4 = (2, 32, 4, 64, 512, 64, 64)
BF16 = (16, 0, 16, 0, 512, 64, 64)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float, ctypes.POINTER(ctypes.c_uint16)]
        L.oracle_f32_to_f16.restype = ctypes.c_int
        L.oracle_quant_group.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P]
        L.oracle_quant_group.restype = ctypes.c_int
        L.oracle_dequant_value.argtypes = [ctypes.c_int, ctypes.c_uint16, ctypes.c_uint16]
        L.oracle_dequant_value.restype = ctypes.c_float
        L.oracle_page_bytes.argtypes = [P]
        L.oracle_page_bytes.restype = ctypes.c_int64
        L.oracle_quant_append.argtypes = [P, P, P, P, ctypes.c_int32, P, ctypes.c_int64]
        L.oracle_quant_append.restype = ctypes.c_int
        L.oracle_dequant_cache.argtypes = [P, P, ctypes.c_int64, P, P, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, P]
        L.oracle_dequant_cache.restype = ctypes.c_int
        L.oracle_decode_range.argtypes = [P, P, P, ctypes.c_int64, P, P, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                          P, P, P, ctypes.c_int32, ctypes.c_int]
        L.oracle_decode_range.restype = ctypes.c_int
        L.oracle_combine.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P, P, P]
        L.oracle_combine.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _fmt(fmt) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(fmt, dtype=np.int32))


def _u16(a) -> np.ndarray:
    """bf16 data as its uint16 bit patterns (accepts torch bf16 tensors)."""
    if hasattr(a, "view") and hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        a = a.detach().cpu().contiguous().view(torch.int16).numpy()
    return np.ascontiguousarray(np.asarray(a).view(np.uint16))


# ---------------------------------------------------------------------- formats

def f32_to_bf16(x: float) -> int:
    return int(lib().oracle_f32_to_bf16(ctypes.c_float(x)))


def bf16_to_f32(h: int) -> float:
    return float(lib().oracle_bf16_to_f32(h))


def f32_to_f16(x: float):
    out = ctypes.c_uint16(0)
    rc = lib().oracle_f32_to_f16(ctypes.c_float(x), ctypes.byref(out))
    return None if rc != 0 else int(out.value)


def f16_to_f32(h: int) -> float:
    return float(lib().oracle_f16_to_f32(h))


# ---------------------------------------------------------------------- quantizer

def quant_group(x, bits: int):
    """Quantize one group (float32 values).  Returns (codes uint8, S16, Z16)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    codes = np.zeros(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint16)
    z = np.zeros(1, dtype=np.uint16)
    rc = lib().oracle_quant_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(z))
    if rc != 0:
        raise ValueError("group not quantizable (non-finite input or fp16 overflow)")
    return codes, int(s[0]), int(z[0])


def dequant_value(code: int, s16: int, z16: int) -> float:
    return float(lib().oracle_dequant_value(int(code), s16, z16))


def page_bytes(fmt) -> int:
    return int(lib().oracle_page_bytes(_ptr(_fmt(fmt))))


def quant_append(fmt, latent, rope, slot_mapping, cache: np.ndarray, num_pages: int) -> None:
    """Quantize and write bf16 rows into `cache` (uint8 [num_pages * page_bytes]) in place."""
    lat = _u16(latent)
    rp = _u16(rope)
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int32))
    assert cache.dtype == np.uint8 and cache.flags["C_CONTIGUOUS"]
    rc = lib().oracle_quant_append(_ptr(_fmt(fmt)), _ptr(lat), _ptr(rp), _ptr(sm), sm.size, _ptr(cache), num_pages)
    if rc != 0:
        raise ValueError("oracle_quant_append failed: %d" % rc)


def dequant_cache(fmt, cache, num_pages, block_table, seq_lens, max_len=None) -> np.ndarray:
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B, MP = bt.shape
    f = _fmt(fmt)
    if max_len is None:
        max_len = int(sl.max()) if sl.size else 0
    out = np.zeros((B, max_len, int(f[4] + f[5])), dtype=np.float32)
    rc = lib().oracle_dequant_cache(_ptr(f), _ptr(np.ascontiguousarray(cache)), num_pages, _ptr(bt), _ptr(sl),
                                    B, MP, max_len, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequant_cache failed: %d" % rc)
    return out


def decode(fmt, q, cache, num_pages, block_table, seq_lens, softmax_scale,
           t_begin=0, t_end=2**31 - 1, want_weights=False, nthreads=0):
    """Attention over the dequantized cache in fp64.

    Returns (out [B, H, d_c] float64, lse [B, H] float64[, weights [B, H, max_len]])."""
    f = _fmt(fmt)
    qq = _u16(q)
    B, H, D = qq.shape
    assert D == f[4] + f[5]
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert bt.shape[0] == B and sl.shape == (B,)
    out = np.zeros((B, H, int(f[4])), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    max_len = int(sl.max()) if (want_weights and sl.size) else 0
    w = np.zeros((B, H, max(max_len, 1)), dtype=np.float64) if want_weights else None
    rc = lib().oracle_decode_range(_ptr(f), _ptr(qq), _ptr(np.ascontiguousarray(cache)), num_pages, _ptr(bt),
                                   _ptr(sl), B, H, bt.shape[1], ctypes.c_float(softmax_scale),
                                   int(t_begin), int(t_end), _ptr(out), _ptr(lse),
                                   _ptr(w) if w is not None else None, max_len, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode_range failed: %d" % rc)
    if want_weights:
        return out, lse, w[:, :, :max_len]
    return out, lse


def decode_multi(fmt, q, cache, num_pages, block_table, seq_lens, softmax_scale, nthreads=0):
    """Multi-token decode: q [B, s_q, H, d_c + d_r] holds the queries of the
    last s_q tokens of every sequence (already in the cache); query i sees
    tokens [0, L - s_q + 1 + i) (itself and those before it, causal), none
    when that count is <= 0 (output 0, lse -inf).  Each query is the
    single-token decode of the sequence cut at its own position.

    Returns (out [B, s_q, H, d_c], lse [B, s_q, H]) in float64."""
    qq = _u16(q)
    B, s_q, H, D = qq.shape
    sl = np.asarray(seq_lens, dtype=np.int64)
    out = np.zeros((B, s_q, H, int(_fmt(fmt)[4])), dtype=np.float64)
    lse = np.zeros((B, s_q, H), dtype=np.float64)
    for i in range(s_q):
        lens_i = np.maximum(sl - (s_q - 1) + i, 0).astype(np.int32)
        o, l = decode(fmt, np.ascontiguousarray(qq[:, i]), cache, num_pages, block_table, lens_i, softmax_scale,
                      nthreads=nthreads)
        out[:, i], lse[:, i] = o, l
    return out, lse


def _f64(a) -> np.ndarray:
    """bf16 tensor / uint16 bit patterns -> float64 values."""
    u = _u16(a).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def absorb_q(q_nope, w_uk) -> np.ndarray:
    """Absorbed query in latent space, per head (fp64): the latent is the
    shared source of every head's key (QuantMLA pages: [P2] TL;DR and
    flowchart), key_h = W_UK[h] c, so <q_nope, W_UK[h] c> = <W_UK[h]^T q_nope, c>.
    q_nope [B, H, 128], w_uk [H, 512, 128] (n-major) -> [B, H, 512]."""
    q = _f64(q_nope)
    w = _f64(w_uk)
    return np.einsum("bhk,hnk->bhn", q, w)


def project_out(latent, w_uv) -> np.ndarray:
    """Value projection applied after attention, per head (fp64): value_h =
    W_UV[h] c, so sum_t p_t W_UV[h] c_t = W_UV[h] sum_t p_t c_t.
    latent [B, H, 512] (bf16 or float64), w_uv [H, 128, 512] -> [B, H, 128]."""
    x = latent if (isinstance(latent, np.ndarray) and latent.dtype == np.float64) else _f64(latent)
    w = _f64(w_uv)
    return np.einsum("bhc,hjc->bhj", x, w)


def combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge partials o_parts [S, rows..., d] / lse_parts [S, rows...] (float64)."""
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    l = np.ascontiguousarray(lse_parts, dtype=np.float64)
    S = o.shape[0]
    d = o.shape[-1]
    rows = int(np.prod(o.shape[1:-1]))
    out = np.zeros(o.shape[1:], dtype=np.float64)
    lse = np.zeros(l.shape[1:], dtype=np.float64)
    lib().oracle_combine(S, rows, d, _ptr(o), _ptr(l), _ptr(out), _ptr(lse))
    return out, lse
