"""Binding of ``libkvc_ceiling.so`` (include/kvc_ceiling.h): streaming
kernels that move the compressor's and the gather's bytes with no work
attached, which the benchmark times under the same cache conditions as the
kernels themselves.  Measurement aid only; not part of the compressed-KV
path.  Argument marshalling and size checks only."""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvc_ceiling.so")

COMPRESS_ITEM_READ, COMPRESS_ITEM_WRITES = 8192, (2048, 512, 64)
GATHER_ROW_READ, GATHER_ROW_WRITE = 528, 1024

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m fp8_fp4_quantized_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.kvc_ceiling_compress_shape.argtypes = [C.c_void_p] * 4 + [C.c_int64, C.c_void_p]
        L.kvc_ceiling_gather_shape.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
        _lib = L
    return _lib


def _dev(t, nbytes: int, name: str) -> int:
    if not (t.is_cuda and t.is_contiguous() and t.numel() * t.element_size() >= nbytes):
        raise ValueError(f"{name}: need a contiguous device tensor of at least {nbytes} bytes")
    return t.data_ptr()


def compress_shape(src, latent, data, scale, items: int):
    """A callable launching the compressor-shaped stream over ``items``
    two-row items (8 KB read, 2 KB + 512 B + 64 B written each)."""
    args = (_dev(src, items * COMPRESS_ITEM_READ, "src"),
            _dev(latent, items * COMPRESS_ITEM_WRITES[0], "latent"),
            _dev(data, items * COMPRESS_ITEM_WRITES[1], "data"),
            _dev(scale, items * COMPRESS_ITEM_WRITES[2], "scale"), items)
    keep = (src, latent, data, scale)

    def call(stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        if lib().kvc_ceiling_compress_shape(*args, s.cuda_stream) != 0:
            raise RuntimeError("kvc_ceiling_compress_shape failed")
    call.keep = keep
    return call


def gather_shape(src, out, rows: int):
    """A callable launching the gather-shaped stream over ``rows`` rows
    (528 B read, 1024 B written each, contiguous)."""
    args = (_dev(src, rows * GATHER_ROW_READ, "src"), _dev(out, rows * GATHER_ROW_WRITE, "out"),
            rows)
    keep = (src, out)

    def call(stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        if lib().kvc_ceiling_gather_shape(*args, s.cuda_stream) != 0:
            raise RuntimeError("kvc_ceiling_gather_shape failed")
    call.keep = keep
    return call
