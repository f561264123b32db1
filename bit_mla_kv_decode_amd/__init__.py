"""Python binding of the gfx950 low-bit MLA cache library (libmla_lowbit.so).

Thin argument marshalling over the C ABI declared in include/mla_lowbit.h:
every entry point keeps its C name, takes torch tensors that already live on
the GPU, checks their dtype/shape/device, and passes raw device pointers and
the current HIP stream.  All computation happens in the library's HIP
kernels; there is no fallback path: if the library is missing or the tensors
are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "FORMATS", "MlaError", "format_struct", "load_library",
    "mla_token_bytes", "mla_page_bytes", "mla_quant_append", "mla_decode_num_splits",
    "mla_decode_workspace_bytes", "mla_decode_partial_slots", "mla_decode_lowbit", "mla_decode_lowbit_noalloc",
    "mla_decode_partial", "mla_decode_combine",
    "mla_decode_append_lowbit", "mla_decode_append_partial", "mla_decode_multi_lowbit",
    "mla_decode_multi_partial", "mla_absorb_q", "mla_project_out",
    "mla_last_error", "alloc_cache",
]

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_lowbit.so")

# name -> (c_bits, c_group, r_bits, r_group, d_c, d_r, page_size)
FORMATS = {
    "C4R4": (4, 64, 4, 64, 512, 64, 64),
    "C2R4": (2, 32, 4, 64, 512, 64, 64),
    "BF16": (16, 0, 16, 0, 512, 64, 64),
}

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
_STATUS = {1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), msg))
        self.status = status


class mla_format_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("c_bits", "c_group", "r_bits", "r_group", "d_c", "d_r", "page_size")]


def format_struct(fmt) -> mla_format_t:
    """mla_format_t from a name ("C4R4", "C2R4", "BF16") or a 7-tuple."""
    vals = FORMATS[fmt] if isinstance(fmt, str) else tuple(int(v) for v in fmt)
    return mla_format_t(*vals)


_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libmla_lowbit.so is not built (run __graft_entry__.build()); "
                           "there is no fallback implementation")
    L = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    FP = ctypes.POINTER(mla_format_t)
    sig = {
        "mla_token_bytes": (SZ, [FP]),
        "mla_page_bytes": (SZ, [FP]),
        "mla_quant_append": (ctypes.c_int, [FP, P, P, P, I32, P, I64, P]),
        "mla_decode_num_splits": (I32, [FP, I32, I32, I32]),
        "mla_decode_workspace_bytes": (SZ, [FP, I32, I32, I32]),
        "mla_decode_partial_slots": (I64, [FP, I32, I32, I32]),
        "mla_decode_lowbit": (ctypes.c_int, [FP, P, P, I64, P, P, I32, I32, I32, I32, F, I32, P, SZ, P, P, P]),
        "mla_decode_lowbit_noalloc": (ctypes.c_int, [FP, P, P, I64, P, P, I32, I32, I32, I32, F, I32, P, P, P]),
        "mla_decode_partial": (ctypes.c_int, [FP, P, P, I64, P, P, I32, I32, I32, I32, F, I32, P, SZ, P]),
        "mla_decode_combine": (ctypes.c_int, [FP, I32, I32, I32, P, SZ, P, P, P]),
        "mla_decode_append_lowbit": (ctypes.c_int, [FP, P, P, P, P, I64, P, P, I32, I32, I32, I32, F, I32, P, SZ,
                                                    P, P, P]),
        "mla_decode_append_partial": (ctypes.c_int, [FP, P, P, P, P, I64, P, P, I32, I32, I32, I32, F, I32, P, SZ,
                                                     P]),
        "mla_decode_multi_lowbit": (ctypes.c_int, [FP, P, I32, P, I64, P, P, I32, I32, I32, I32, F, I32, P, SZ,
                                                   P, P, P]),
        "mla_decode_multi_partial": (ctypes.c_int, [FP, P, I32, P, I64, P, P, I32, I32, I32, I32, F, I32, P, SZ,
                                                    P]),
        "mla_absorb_q": (ctypes.c_int, [P, P, P, I32, I32, P, P]),
        "mla_project_out": (ctypes.c_int, [P, P, I32, I32, P, P]),
        "mla_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def mla_last_error() -> str:
    return load_library().mla_last_error().decode()


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, mla_last_error())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name, dtype=None):
    return ctypes.c_void_p(0) if t is None else _dev(t, name, dtype)


# ---------------------------------------------------------------------- entry points

def mla_token_bytes(fmt) -> int:
    return int(load_library().mla_token_bytes(ctypes.byref(format_struct(fmt))))


def mla_page_bytes(fmt) -> int:
    return int(load_library().mla_page_bytes(ctypes.byref(format_struct(fmt))))


def alloc_cache(fmt, num_pages: int, device="cuda"):
    """Zeroed paged cache: uint8 [num_pages * page_bytes] on `device`."""
    import torch
    return torch.zeros(num_pages * mla_page_bytes(fmt), dtype=torch.uint8, device=device)


def mla_quant_append(fmt, latent, rope, slot_mapping, cache, num_pages=None, stream=None) -> None:
    """Quantize and pack bf16 rows latent [n, 512] / rope [n, 64] into `cache` at `slot_mapping` [n] int32."""
    import torch
    n = int(latent.shape[0]) if latent.dim() == 2 else -1
    if latent.dim() != 2 or rope.dim() != 2 or rope.shape[0] != n or slot_mapping.shape != (n,):
        raise ValueError("latent [n, 512], rope [n, 64] and slot_mapping [n] expected")
    pb = mla_page_bytes(fmt)
    if num_pages is None:
        num_pages = cache.numel() // pb if pb else 0
    if pb and cache.numel() < num_pages * pb:
        raise ValueError("cache holds fewer than num_pages pages")
    _check(load_library().mla_quant_append(
        ctypes.byref(format_struct(fmt)), _dev(latent, "latent", torch.bfloat16), _dev(rope, "rope", torch.bfloat16),
        _dev(slot_mapping, "slot_mapping", torch.int32), n, _dev(cache, "cache", torch.uint8), int(num_pages),
        _stream(stream)))


def mla_decode_num_splits(fmt, batch: int, num_heads: int, max_seq_len: int) -> int:
    return int(load_library().mla_decode_num_splits(ctypes.byref(format_struct(fmt)), batch, num_heads, max_seq_len))


def mla_decode_workspace_bytes(fmt, batch: int, num_heads: int, num_splits: int) -> int:
    return int(load_library().mla_decode_workspace_bytes(ctypes.byref(format_struct(fmt)), batch, num_heads,
                                                         num_splits))


def mla_decode_partial_slots(fmt, batch: int, num_heads: int, num_splits: int) -> int:
    """Partial slots of the decode workspace: batch * num_splits, or the balanced
    partition's workgroups + batch for num_splits = 0."""
    return int(load_library().mla_decode_partial_slots(ctypes.byref(format_struct(fmt)), batch, num_heads,
                                                       num_splits))


def _decode_shapes(q, cache, block_table, seq_lens, fmt, num_pages):
    if q.dim() != 3 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("q [B, H, 576], block_table [B, max_pages] and seq_lens [B] expected")
    B, H, D = (int(v) for v in q.shape)
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("batch sizes of q, block_table and seq_lens differ")
    pb = mla_page_bytes(fmt)
    if num_pages is None:
        num_pages = cache.numel() // pb if pb else 0
    return B, H, int(block_table.shape[1]), int(num_pages)


def mla_decode_lowbit(fmt, q, cache, block_table, seq_lens, softmax_scale, max_seq_len=None, num_splits=0,
                      out=None, lse=None, workspace=None, num_pages=None, stream=None):
    """Decode attention over the packed cache; returns (out bf16 [B, H, 512], lse fp32 [B, H] or None).

    num_splits = 0 balances the batch's pages over all compute units; 1..64
    splits every sequence into that many page ranges (1: no workspace).
    `max_seq_len` is the host-side bound on seq_lens (default: capacity)."""
    import torch
    B, H, MP, NP = _decode_shapes(q, cache, block_table, seq_lens, fmt, num_pages)
    if max_seq_len is None:
        max_seq_len = MP * 64
    S = int(num_splits)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q.device)
    if workspace is None and S != 1:
        workspace = torch.empty(mla_decode_workspace_bytes(fmt, B, H, S), dtype=torch.uint8, device=q.device)
    _check(load_library().mla_decode_lowbit(
        ctypes.byref(format_struct(fmt)), _dev(q, "q", torch.bfloat16), _dev(cache, "cache", torch.uint8), NP,
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), B, H, MP,
        int(max_seq_len), float(softmax_scale), int(num_splits),
        _opt(workspace, "workspace", torch.uint8), workspace.numel() if workspace is not None else 0,
        _dev(out, "out", torch.bfloat16), _opt(lse, "lse", torch.float32), _stream(stream)))
    return out, lse


def mla_decode_lowbit_noalloc(fmt, q, cache, block_table, seq_lens, softmax_scale, max_seq_len=None, num_splits=0,
                              out=None, lse=None, num_pages=None, stream=None):
    """mla_decode_lowbit whose partial results live in the library's per-device
    scratch (no workspace argument; the C call allocates nothing).  Pass `out`
    (and `lse`) to allocate nothing on this side either.  Returns (out, lse)."""
    import torch
    B, H, MP, NP = _decode_shapes(q, cache, block_table, seq_lens, fmt, num_pages)
    if max_seq_len is None:
        max_seq_len = MP * 64
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q.device)
    _check(load_library().mla_decode_lowbit_noalloc(
        ctypes.byref(format_struct(fmt)), _dev(q, "q", torch.bfloat16), _dev(cache, "cache", torch.uint8), NP,
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), B, H, MP,
        int(max_seq_len), float(softmax_scale), int(num_splits),
        _dev(out, "out", torch.bfloat16), _opt(lse, "lse", torch.float32), _stream(stream)))
    return out, lse


def mla_decode_append_lowbit(fmt, latent_new, rope_new, q, cache, block_table, seq_lens, softmax_scale,
                             max_seq_len=None, num_splits=0, out=None, lse=None, workspace=None, num_pages=None,
                             stream=None):
    """The serving step in one call: row b of latent_new [B, 512] / rope_new [B, 64] (bf16) is
    appended at position seq_lens[b] - 1, then decode over all seq_lens[b] tokens; returns
    (out, lse) as mla_decode_lowbit.  `cache` is written."""
    import torch
    B, H, MP, NP = _decode_shapes(q, cache, block_table, seq_lens, fmt, num_pages)
    if tuple(latent_new.shape) != (B, 512) or tuple(rope_new.shape) != (B, 64):
        raise ValueError("latent_new [B, 512] and rope_new [B, 64] expected")
    if max_seq_len is None:
        max_seq_len = MP * 64
    S = int(num_splits)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q.device)
    if workspace is None and S != 1:
        workspace = torch.empty(mla_decode_workspace_bytes(fmt, B, H, S), dtype=torch.uint8, device=q.device)
    _check(load_library().mla_decode_append_lowbit(
        ctypes.byref(format_struct(fmt)), _dev(latent_new, "latent_new", torch.bfloat16),
        _dev(rope_new, "rope_new", torch.bfloat16), _dev(q, "q", torch.bfloat16), _dev(cache, "cache", torch.uint8),
        NP, _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), B, H, MP,
        int(max_seq_len), float(softmax_scale), S,
        _opt(workspace, "workspace", torch.uint8), workspace.numel() if workspace is not None else 0,
        _dev(out, "out", torch.bfloat16), _opt(lse, "lse", torch.float32), _stream(stream)))
    return out, lse


def mla_decode_append_partial(fmt, latent_new, rope_new, q, cache, block_table, seq_lens, softmax_scale, num_splits,
                              workspace, max_seq_len=None, num_pages=None, stream=None) -> None:
    """First stage of mla_decode_append_lowbit (append + partial results); complete with mla_decode_combine."""
    import torch
    B, H, MP, NP = _decode_shapes(q, cache, block_table, seq_lens, fmt, num_pages)
    if tuple(latent_new.shape) != (B, 512) or tuple(rope_new.shape) != (B, 64):
        raise ValueError("latent_new [B, 512] and rope_new [B, 64] expected")
    if max_seq_len is None:
        max_seq_len = MP * 64
    _check(load_library().mla_decode_append_partial(
        ctypes.byref(format_struct(fmt)), _dev(latent_new, "latent_new", torch.bfloat16),
        _dev(rope_new, "rope_new", torch.bfloat16), _dev(q, "q", torch.bfloat16), _dev(cache, "cache", torch.uint8),
        NP, _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), B, H, MP,
        int(max_seq_len), float(softmax_scale), int(num_splits), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(stream)))


def _multi_shapes(q, cache, block_table, seq_lens, fmt, num_pages):
    if q.dim() != 4 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("q [B, s_q, H, 576], block_table [B, max_pages] and seq_lens [B] expected")
    B, s_q, H, D = (int(v) for v in q.shape)
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("batch sizes of q, block_table and seq_lens differ")
    pb = mla_page_bytes(fmt)
    if num_pages is None:
        num_pages = cache.numel() // pb if pb else 0
    return B, s_q, H, int(block_table.shape[1]), int(num_pages)


def mla_decode_multi_lowbit(fmt, q, cache, block_table, seq_lens, softmax_scale, max_seq_len=None, num_splits=0,
                            out=None, lse=None, workspace=None, num_pages=None, stream=None):
    """Multi-token decode: q [B, s_q, H, 576] are the queries of the last s_q tokens of every
    sequence (already in the cache); query i sees tokens [0, L - s_q + 1 + i).  Returns
    (out bf16 [B, s_q, H, 512], lse fp32 [B, s_q, H] or None)."""
    import torch
    B, s_q, H, MP, NP = _multi_shapes(q, cache, block_table, seq_lens, fmt, num_pages)
    if max_seq_len is None:
        max_seq_len = MP * 64
    S = int(num_splits)
    if out is None:
        out = torch.empty((B, s_q, H, 512), dtype=torch.bfloat16, device=q.device)
    if workspace is None and S != 1:
        workspace = torch.empty(mla_decode_workspace_bytes(fmt, B, s_q * H, S), dtype=torch.uint8, device=q.device)
    _check(load_library().mla_decode_multi_lowbit(
        ctypes.byref(format_struct(fmt)), _dev(q, "q", torch.bfloat16), s_q, _dev(cache, "cache", torch.uint8), NP,
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), B, H, MP,
        int(max_seq_len), float(softmax_scale), S,
        _opt(workspace, "workspace", torch.uint8), workspace.numel() if workspace is not None else 0,
        _dev(out, "out", torch.bfloat16), _opt(lse, "lse", torch.float32), _stream(stream)))
    return out, lse


def mla_decode_multi_partial(fmt, q, cache, block_table, seq_lens, softmax_scale, num_splits, workspace,
                             max_seq_len=None, num_pages=None, stream=None) -> None:
    """First stage of mla_decode_multi_lowbit; complete with mla_decode_combine(fmt, B, s_q * H, ...)."""
    import torch
    B, s_q, H, MP, NP = _multi_shapes(q, cache, block_table, seq_lens, fmt, num_pages)
    if max_seq_len is None:
        max_seq_len = MP * 64
    _check(load_library().mla_decode_multi_partial(
        ctypes.byref(format_struct(fmt)), _dev(q, "q", torch.bfloat16), s_q, _dev(cache, "cache", torch.uint8), NP,
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), B, H, MP,
        int(max_seq_len), float(softmax_scale), int(num_splits), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(stream)))


def mla_decode_partial(fmt, q, cache, block_table, seq_lens, softmax_scale, num_splits, workspace,
                       max_seq_len=None, num_pages=None, stream=None) -> None:
    import torch
    B, H, MP, NP = _decode_shapes(q, cache, block_table, seq_lens, fmt, num_pages)
    if max_seq_len is None:
        max_seq_len = MP * 64
    _check(load_library().mla_decode_partial(
        ctypes.byref(format_struct(fmt)), _dev(q, "q", torch.bfloat16), _dev(cache, "cache", torch.uint8), NP,
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), B, H, MP,
        int(max_seq_len), float(softmax_scale), int(num_splits), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(stream)))


def mla_decode_combine(fmt, batch, num_heads, num_splits, workspace, out, lse=None, stream=None) -> None:
    import torch
    _check(load_library().mla_decode_combine(
        ctypes.byref(format_struct(fmt)), int(batch), int(num_heads), int(num_splits),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _dev(out, "out", torch.bfloat16),
        _opt(lse, "lse", torch.float32), _stream(stream)))


def workspace_views(fmt, workspace, batch, num_heads, num_splits):
    """fp32 views (o_part [B, S, H, 512], lse_part [B, S, H]) of a workspace
    written with num_splits = S >= 1 per-sequence splits."""
    import torch
    if num_splits < 1:
        raise ValueError("workspace_views needs the per-sequence split layout (num_splits >= 1)")
    n_o = batch * num_splits * num_heads * 512
    o_bytes = (n_o * 4 + 255) // 256 * 256
    o = workspace[:n_o * 4].view(torch.float32).view(batch, num_splits, num_heads, 512)
    l = workspace[o_bytes:o_bytes + batch * num_splits * num_heads * 4].view(torch.float32)
    return o, l.view(batch, num_splits, num_heads)


def balanced_workspace_views(fmt, workspace, batch, num_heads):
    """Views of a workspace written with num_splits = 0: fp32 o_part
    [G + B, H, 512], fp32 lse_part [G + B, H] (slot w + b holds workgroup
    w's piece of sequence b; G + B from mla_decode_partial_slots) and int32
    meta [B, 2] (first slot, slot count)."""
    import torch
    slots = mla_decode_partial_slots(fmt, batch, num_heads, 0)
    n_o = slots * num_heads * 512
    o_bytes = (n_o * 4 + 255) // 256 * 256
    l_bytes = (slots * num_heads * 4 + 255) // 256 * 256
    o = workspace[:n_o * 4].view(torch.float32).view(slots, num_heads, 512)
    l = workspace[o_bytes:o_bytes + slots * num_heads * 4].view(torch.float32).view(slots, num_heads)
    m = workspace[o_bytes + l_bytes:o_bytes + l_bytes + batch * 8].view(torch.int32).view(batch, 2)
    return o, l, m


def mla_absorb_q(q_nope, q_pe, w_uk, q_out=None, stream=None):
    """q [B, H, 576] = [per-head q_nope [B, H, 128] times w_uk [H, 512, 128] | q_pe [B, H, 64]] (bf16)."""
    import torch
    B, H, K = (int(v) for v in q_nope.shape)
    if K != 128 or tuple(q_pe.shape) != (B, H, 64) or tuple(w_uk.shape) != (H, 512, 128):
        raise ValueError("q_nope [B, H, 128], q_pe [B, H, 64], w_uk [H, 512, 128] expected")
    if q_out is None:
        q_out = torch.empty(B, H, 576, dtype=torch.bfloat16, device=q_nope.device)
    _check(load_library().mla_absorb_q(_dev(q_nope, "q_nope", torch.bfloat16), _dev(q_pe, "q_pe", torch.bfloat16),
                                       _dev(w_uk, "w_uk", torch.bfloat16), B, H,
                                       _dev(q_out, "q_out", torch.bfloat16), _stream(stream)))
    return q_out


def mla_project_out(latent, w_uv, out=None, stream=None):
    """o [B, H, 128] = per-head latent [B, H, 512] times w_uv [H, 128, 512] (bf16)."""
    import torch
    B, H, C = (int(v) for v in latent.shape)
    if C != 512 or tuple(w_uv.shape) != (H, 128, 512):
        raise ValueError("latent [B, H, 512] and w_uv [H, 128, 512] expected")
    if out is None:
        out = torch.empty(B, H, 128, dtype=torch.bfloat16, device=latent.device)
    _check(load_library().mla_project_out(_dev(latent, "latent", torch.bfloat16), _dev(w_uv, "w_uv", torch.bfloat16),
                                          B, H, _dev(out, "out", torch.bfloat16), _stream(stream)))
    return out
