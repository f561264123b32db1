"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol the header declares, answers the format/size queries, and rejects bad
host-visible arguments before anything is launched."""
import ctypes
import os
import re

import pytest

import bit_mla_kv_decode_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_lowbit.h")

# fake, 256-byte-aligned device addresses: validation never dereferences them
A = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20000)


def _declared(header=HEADER, prefix="mla_"):
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(%s[a-z0-9_]+)\s*\(" % prefix, txt)))


def test_header_symbols_are_exported():
    lib = mla.load_library()
    names = _declared()
    assert {"mla_quant_append", "mla_decode_lowbit", "mla_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_peaks_header_symbols_are_exported():
    from bit_mla_kv_decode_amd import peaks
    lib = peaks.load_library()
    names = _declared(os.path.join(ROOT, "include", "mla_peaks.h"), "peak_")
    assert names == ["peak_copy", "peak_lds", "peak_mfma_bf16", "peak_mfma_cycles", "peak_read"]
    for n in names:
        assert hasattr(lib, n), n
    # host-side argument checks (no launch): misaligned or ragged sizes, unsupported shapes are refused
    assert lib.peak_copy(A, A2, 17, None) != 0
    assert lib.peak_read(A, 1000, 256, A2, None) != 0
    assert lib.peak_mfma_bf16(0, 10, A2, None) != 0
    assert lib.peak_mfma_cycles(256, 10, 3, 0, A, A2, None) != 0     # 1 or 2 chains
    assert lib.peak_mfma_cycles(256, 10, 2, 5, A, A2, None) != 0     # 0, 2, 4, 6, 8 or 12 FMAs
    assert lib.peak_mfma_cycles(0, 10, 2, 0, A, A2, None) != 0
    assert lib.peak_lds(256, 3, 0, 16, 10, A, A2, None) != 0         # 1 or 2 wavefronts per SIMD
    assert lib.peak_lds(0, 1, 0, 16, 10, A, A2, None) != 0
    assert lib.peak_lds(256, 1, 0, 12, 10, A, A2, None) != 0         # widths 4, 8, 16 only


def test_format_queries():
    assert mla.mla_page_bytes("C4R4") == 20736 and mla.mla_token_bytes("C4R4") == 324
    assert mla.mla_page_bytes("C2R4") == 14592 and mla.mla_token_bytes("C2R4") == 228
    assert mla.mla_page_bytes("BF16") == 73728 and mla.mla_token_bytes("BF16") == 1152
    for bad in [(4, 32, 4, 64, 512, 64, 64), (8, 64, 4, 64, 512, 64, 64), (4, 64, 4, 64, 512, 64, 32),
                (4, 64, 2, 64, 512, 64, 64), (4, 64, 4, 64, 256, 64, 64)]:
        assert mla.mla_page_bytes(bad) == 0 and mla.mla_token_bytes(bad) == 0


def test_split_heuristic_and_workspace():
    f = "C4R4"
    assert mla.mla_decode_num_splits(f, 1, 16, 256) == 4
    assert mla.mla_decode_num_splits(f, 32, 128, 8192) == 8
    assert mla.mla_decode_num_splits(f, 64, 128, 32768) == 4
    assert mla.mla_decode_num_splits(f, 8, 128, 131072) == 32
    assert mla.mla_decode_num_splits(f, 128, 128, 131072) == 16
    assert mla.mla_decode_num_splits(f, 1, 128, 64) == 1
    assert mla.mla_decode_num_splits(f, 0, 128, 1000) == 1
    for B, H, S in [(8, 128, 32), (1, 1, 1), (3, 17, 5)]:
        n = B * S * H
        expect = (n * 512 * 4 + 255) // 256 * 256 + (n * 4 + 255) // 256 * 256
        assert mla.mla_decode_workspace_bytes(f, B, H, S) == expect
    # balanced partition: G + B slots, then int32 (first slot, count) per sequence; G = 512
    # workgroups (two per compute unit) where the quantized formats split channels (17..32 rows),
    # else 256 (one per unit; at <= 16 rows a unit holds one 512-thread workgroup)
    for fm, B, H, G in [(f, 8, 128, 256), (f, 1, 1, 256), (f, 4, 16, 256), (f, 300, 17, 512), ("C2R4", 4, 32, 512),
                        ("C2R4", 4, 33, 256), ("BF16", 1, 1, 256), ("BF16", 8, 128, 256)]:
        n = (G + B) * H
        expect = (n * 512 * 4 + 255) // 256 * 256 + (n * 4 + 255) // 256 * 256 + (B * 8 + 255) // 256 * 256
        assert mla.mla_decode_workspace_bytes(fm, B, H, 0) == expect, (fm, B, H)
        assert mla.mla_decode_partial_slots(fm, B, H, 0) == G + B
    assert mla.mla_decode_partial_slots(f, 8, 128, 32) == 256
    assert mla.mla_decode_partial_slots(f, 8, 0, 0) == 0
    # fixed splits fill the resident workgroups: 512 at 17..32 heads
    assert mla.mla_decode_num_splits(f, 8, 17, 131072) == 64
    assert mla.mla_decode_num_splits(f, 16, 32, 131072) == 32
    assert mla.mla_decode_num_splits(f, 8, 16, 131072) == 32
    assert mla.mla_decode_num_splits("BF16", 16, 16, 131072) == 16
    assert mla.mla_decode_workspace_bytes(f, 8, 0, 4) == 0
    assert mla.mla_decode_workspace_bytes(f, 8, 128, -1) == 0
    assert mla.mla_decode_workspace_bytes(f, 8, 128, 65) == 0


def _fmt(name="C4R4"):
    return ctypes.byref(mla.format_struct(name))


def test_quant_append_argument_errors():
    L = mla.load_library()
    assert L.mla_quant_append(_fmt((4, 64, 4, 64, 512, 64, 32)), A, A, A, 4, A, 4, None) == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_quant_append(_fmt(), A, A, A, -1, A, 4, None) == mla.MLA_ERR_INVALID_ARG
    assert "n_new" in mla.mla_last_error()
    assert L.mla_quant_append(_fmt(), None, A, A, 4, A, 4, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_quant_append(_fmt(), A, A, A, 4, A, 0, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_quant_append(_fmt(), ctypes.c_void_p(0x10008), A, A, 4, A, 4, None) == mla.MLA_ERR_INVALID_ARG
    assert "aligned" in mla.mla_last_error()
    # nothing to do: OK without touching a device
    assert L.mla_quant_append(_fmt(), None, None, None, 0, None, 0, None) == mla.MLA_OK


def _decode(fmt="C4R4", q=A, cache=A, num_pages=10, bt=A, sl=A, batch=2, heads=128, max_pages=4, max_len=256,
            scale=0.07, splits=0, ws=A2, ws_bytes=1 << 30, out=A, lse=None):
    L = mla.load_library()
    return L.mla_decode_lowbit(_fmt(fmt), q, cache, num_pages, bt, sl, batch, heads, max_pages, max_len, scale,
                               splits, ws, ws_bytes, out, lse, None)


def test_decode_argument_errors():
    assert _decode(fmt=(2, 64, 4, 64, 512, 64, 64)) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(heads=0) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(heads=129) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(batch=-1) == mla.MLA_ERR_INVALID_ARG
    assert _decode(batch=70000) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(max_pages=0) == mla.MLA_ERR_INVALID_ARG
    assert _decode(num_pages=0) == mla.MLA_ERR_INVALID_ARG
    assert _decode(splits=65) == mla.MLA_ERR_INVALID_ARG
    assert _decode(splits=-1) == mla.MLA_ERR_INVALID_ARG
    assert _decode(scale=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert _decode(q=None) == mla.MLA_ERR_INVALID_ARG
    assert _decode(q=ctypes.c_void_p(0x10002)) == mla.MLA_ERR_INVALID_ARG
    assert _decode(out=None) == mla.MLA_ERR_INVALID_ARG
    # 4 splits need a workspace of the documented size
    need = mla.mla_decode_workspace_bytes("C4R4", 2, 128, 4)
    assert _decode(splits=4, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE
    assert _decode(splits=4, ws=None) == mla.MLA_ERR_INVALID_ARG
    assert _decode(splits=4, ws=ctypes.c_void_p(0x10010)) == mla.MLA_ERR_INVALID_ARG
    # so does the balanced partition (num_splits = 0)
    need0 = mla.mla_decode_workspace_bytes("C4R4", 2, 128, 0)
    assert _decode(splits=0, ws_bytes=need0 - 1) == mla.MLA_ERR_WORKSPACE
    assert _decode(splits=0, ws=None) == mla.MLA_ERR_INVALID_ARG
    # empty batch: nothing launched
    assert _decode(batch=0, q=None, cache=None, bt=None, sl=None, out=None) == mla.MLA_OK


def test_combine_argument_errors():
    L = mla.load_library()
    need = mla.mla_decode_workspace_bytes("C4R4", 2, 8, 3)
    assert L.mla_decode_combine(_fmt(), 2, 8, -1, A2, need, A, None, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_decode_combine(_fmt(), 2, 8, 65, A2, need, A, None, None) == mla.MLA_ERR_INVALID_ARG
    need0 = mla.mla_decode_workspace_bytes("C4R4", 2, 8, 0)
    assert L.mla_decode_combine(_fmt(), 2, 8, 0, A2, need0 - 1, A, None, None) == mla.MLA_ERR_WORKSPACE
    assert L.mla_decode_combine(_fmt(), 2, 8, 3, A2, need - 4, A, None, None) == mla.MLA_ERR_WORKSPACE
    assert L.mla_decode_combine(_fmt(), 2, 0, 3, A2, need, A, None, None) == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_decode_combine(_fmt(), 2, 8, 3, A2, need, None, None, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_decode_combine(_fmt(), 0, 8, 3, None, 0, None, None, None) == mla.MLA_OK


def test_python_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 512, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        mla.mla_quant_append("C4R4", x, torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, dtype=torch.int32),
                             torch.zeros(20736, dtype=torch.uint8))


def test_fused_append_argument_errors():
    L = mla.load_library()
    A3 = ctypes.c_void_p(0x30000)

    def call(lat=A3, rope=A3, batch=2, splits=0, ws_bytes=1 << 30):
        return L.mla_decode_append_lowbit(_fmt(), lat, rope, A, A, 10, A, A, batch, 128, 4, 256, 0.07, splits, A2,
                                          ws_bytes, A, None, None)
    assert call(lat=None) == mla.MLA_ERR_INVALID_ARG
    assert call(rope=None) == mla.MLA_ERR_INVALID_ARG
    assert call(lat=ctypes.c_void_p(0x30008)) == mla.MLA_ERR_INVALID_ARG
    assert "aligned" in mla.mla_last_error()
    assert call(ws_bytes=10) == mla.MLA_ERR_WORKSPACE
    assert call(splits=65) == mla.MLA_ERR_INVALID_ARG
    assert call(batch=0, lat=None, rope=None) == mla.MLA_OK
    assert L.mla_decode_append_partial(_fmt(), None, A3, A, A, 10, A, A, 2, 128, 4, 256, 0.07, 0, A2, 1 << 30,
                                       None) == mla.MLA_ERR_INVALID_ARG


def test_multi_token_argument_errors():
    L = mla.load_library()

    def call(nq=2, heads=64, splits=0, ws_bytes=1 << 30):
        return L.mla_decode_multi_lowbit(_fmt(), A, nq, A, 10, A, A, 2, heads, 4, 256, 0.07, splits, A2, ws_bytes,
                                         A, None, None)
    assert call(nq=0) == mla.MLA_ERR_INVALID_ARG
    assert call(nq=17) == mla.MLA_ERR_INVALID_ARG
    assert call(heads=129) == mla.MLA_ERR_UNSUPPORTED
    need = mla.mla_decode_workspace_bytes("C4R4", 2, 2 * 64, 0)
    assert call(ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE
    # the combine takes rows = num_queries * num_heads (up to 2048)
    assert L.mla_decode_combine(_fmt(), 2, 2049, 0, A2, 1 << 40, A, None, None) == mla.MLA_ERR_UNSUPPORTED


def test_noalloc_decode_argument_errors():
    """The no-allocation decode validates like mla_decode_lowbit and refuses a
    shape whose partial results exceed its per-device scratch (128 MiB) before
    looking up any device memory."""
    L = mla.load_library()

    def call(batch=2, heads=128, splits=0, out=A, q=A):
        return L.mla_decode_lowbit_noalloc(_fmt(), q, A, 10, A, A, batch, heads, 4, 256, 0.07, splits, out, None,
                                           None)
    assert call(heads=129) == mla.MLA_ERR_UNSUPPORTED
    assert call(splits=65) == mla.MLA_ERR_INVALID_ARG
    assert call(q=None) == mla.MLA_ERR_INVALID_ARG
    assert call(batch=0, q=None, out=None) == mla.MLA_OK
    assert mla.mla_decode_workspace_bytes("C4R4", 600, 128, 0) > 128 << 20
    assert call(batch=600) == mla.MLA_ERR_WORKSPACE
    assert "scratch" in mla.mla_last_error()
    assert call(batch=600, splits=1, out=None) == mla.MLA_ERR_INVALID_ARG   # one split needs no scratch: out checked

