"""ctypes binding of libmla_peaks.so: the practical-peak microbenchmarks
(streaming HBM read, plain copy, dense bf16 MFMA loop, MFMA cycle costs with
VALU work between the MFMAs, LDS bandwidth) the decode kernels are measured
against."""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_peaks.so")
_lib = None


def load_library():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmla_peaks.so is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        L.peak_copy.argtypes, L.peak_copy.restype = [vp, vp, sz, vp], i32
        L.peak_read.argtypes, L.peak_read.restype = [vp, sz, i32, vp, vp], i32
        L.peak_mfma_bf16.argtypes, L.peak_mfma_bf16.restype = [i32, i32, vp, vp], i32
        L.peak_mfma_cycles.argtypes, L.peak_mfma_cycles.restype = [i32, i32, i32, i32, vp, vp, vp], i32
        L.peak_lds.argtypes, L.peak_lds.restype = [i32, i32, i32, i32, i32, vp, vp, vp], i32
        _lib = L
    return _lib


def _ck(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed (HIP error %d)" % (what, rc))


def _s(stream):
    return ctypes.c_void_p(stream.cuda_stream) if stream is not None else None


def copy(src, dst, stream=None):
    """dst[:] = src[:] (uint8 device tensors of equal size, a multiple of 16 bytes)."""
    assert src.is_cuda and dst.is_cuda and src.numel() == dst.numel()
    _ck(load_library().peak_copy(src.data_ptr(), dst.data_ptr(), src.numel(), _s(stream)), "peak_copy")


def read(src, sink, groups=2048, stream=None):
    """Stream-read the uint8 device tensor src (a multiple of 16 KiB)."""
    _ck(load_library().peak_read(src.data_ptr(), src.numel(), groups, sink.data_ptr(), _s(stream)), "peak_read")


def mfma_bf16(groups, iters, sink, stream=None):
    """Dense 32x32x16 bf16 MFMA loop; returns the flops it executes."""
    assert sink.numel() >= groups * 256
    _ck(load_library().peak_mfma_bf16(groups, iters, sink.data_ptr(), _s(stream)), "peak_mfma_bf16")
    return groups * 4 * iters * 4 * 32768


def mfma_cycles(groups, iters, chains, valu_per_mfma, cycles, sink, stream=None):
    """Time `iters` rounds of `chains` MFMA chains, `valu_per_mfma` FMAs after each
    MFMA; cycles (int64 device tensor of 2 * groups) receives per workgroup the
    shader-clock cycles and the 100 MHz reference ticks of the loop."""
    assert cycles.numel() >= 2 * groups and sink.numel() >= groups * 256
    _ck(load_library().peak_mfma_cycles(groups, iters, chains, valu_per_mfma, cycles.data_ptr(), sink.data_ptr(),
                                        _s(stream)), "peak_mfma_cycles")


def lds(groups, waves_per_simd, write, iters, cycles, sink, stream=None, width=16):
    """LDS read (write=False) or write bandwidth loop with `width`-byte accesses
    (4, 8 or 16); cycles (int64 device tensor of groups) receives each
    workgroup's shader-clock cycles.  Returns the bytes one workgroup moves."""
    assert cycles.numel() >= groups and sink.numel() >= groups * 256 * waves_per_simd
    _ck(load_library().peak_lds(groups, waves_per_simd, int(write), width, iters, cycles.data_ptr(),
                                sink.data_ptr(), _s(stream)), "peak_lds")
    return iters * 8 * width * 256 * waves_per_simd
