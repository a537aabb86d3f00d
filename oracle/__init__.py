"""CPU oracle of the DeepSeek-V4.1 low-ratio compressed-KV path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
(``fp8_fp4_quantized_amd``) never imports it and shares no code with it.

A thin ctypes wrapper over ``libkvc_oracle.so`` (plain C, fp64, see
``kvc_oracle.c`` for the definitions and the page citations).  All arrays are
numpy host arrays; bf16 data are ``uint16`` bit patterns.  A cache is a
``uint8`` array of shape ``[num_pages, page_stride]``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libkvc_oracle.so")

LAYOUTS = {"V4": 0, "V41": 1, "V41_FP4": 2}
PREFILL, DECODE, VERIFY = 0, 1, 2
ST_ID_RANGE, ST_PAGE_RANGE, ST_PT_RANGE, ST_LATENT_RANGE, ST_POS_RANGE = 1, 2, 4, 8, 16
ST_REQ_RANGE, ST_TOKEN_RANGE = 32, 64

_lib = None


class _Cache(C.Structure):
    _fields_ = [("base", C.c_void_p), ("layout", C.c_int32), ("page_size", C.c_int32),
                ("page_stride", C.c_int64), ("num_pages", C.c_int64)]


class _CompressArgs(C.Structure):
    _fields_ = [
        ("ratio", C.c_int32), ("mode", C.c_int32),
        ("kv", C.c_void_p), ("kv_stride", C.c_int64),
        ("score", C.c_void_p), ("score_stride", C.c_int64),
        ("num_slots", C.c_int32),
        ("offsets", C.c_void_p), ("start_pos", C.c_void_p),
        ("page_table", C.c_void_p), ("pt_stride", C.c_int64),
        ("out_loc", C.c_void_p), ("state", C.c_void_p),
        ("norm_w", C.c_void_p), ("eps", C.c_float),
        ("freqs", C.c_void_p), ("max_pos", C.c_int64),
        ("latent", C.c_void_p), ("latent_stride", C.c_int64), ("max_out_rows", C.c_int64),
        ("prequant", C.c_void_p), ("prequant_stride", C.c_int64),
        ("cache", _Cache), ("status", C.c_void_p),
        ("draft_len", C.c_int32), ("ring_slots", C.c_int32),
        ("dcp_world", C.c_int32), ("dcp_rank", C.c_int32), ("dcp_interleave", C.c_int32),
        ("kv_rows", C.c_int64),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("oracle library not built: run oracle/build.py")
        L = C.CDLL(_LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        sig = {
            "kvo_layout_bytes": (C.c_int, [i32, vp, vp, vp, vp]),
            "kvo_e4m3_decode": (C.c_double, [C.c_uint8]),
            "kvo_e2m1_decode": (C.c_double, [C.c_uint8]),
            "kvo_e4m3_encode": (C.c_uint8, [C.c_double, C.c_int]),
            "kvo_e2m1_encode": (C.c_uint8, [C.c_double]),
            "kvo_bf16_encode": (C.c_uint16, [C.c_double]),
            "kvo_ue8m0": (C.c_int, [C.c_float]),
            "kvo_fp4_scale": (C.c_uint8, [C.c_float]),
            "kvo_e4m3_encode_n": (None, [vp, i64, C.c_int, vp]),
            "kvo_e2m1_encode_n": (None, [vp, i64, vp]),
            "kvo_bf16_encode_n": (None, [vp, i64, vp]),
            "kvo_ue8m0_n": (None, [vp, i64, vp]),
            "kvo_fp4_scale_n": (None, [vp, i64, vp]),
            "kvo_fp8_code_n": (None, [vp, vp, i64, vp]),
            "kvo_fp4_code_n": (None, [vp, vp, i64, vp]),
            "kvo_store_row_n": (None, [i32, vp, i64, vp, vp]),
            "kvo_dequant_row_n": (None, [i32, vp, vp, i64, vp]),
            "kvo_store_rows": (None, [C.POINTER(_Cache), vp, i64, vp, i64, vp]),
            "kvo_dequant_gather": (None, [C.POINTER(_Cache), vp, i64, vp, i64, vp, i64, vp]),
            "kvo_compress": (None, [C.POINTER(_CompressArgs)]),
            "kvo_count_rows": (i64, [C.POINTER(_CompressArgs)]),
            "kvo_num_threads": (C.c_int, []),
            "kvo_store_rows_rope": (None, [C.POINTER(_Cache), vp, i64, vp, vp, i64, vp, i64, vp, vp]),
            "kvo_dcp_owner": (i32, [i64, i32, i32, C.POINTER(C.c_int64)]),
            "kvo_dcp_filter_ids": (None, [vp, i64, i32, i64, vp, i32, vp, i64, vp, i32, i64,
                                          i32, i32, i32, vp, i64, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def num_threads() -> int:
    return lib().kvo_num_threads()


# ---------------------------------------------------------------- layouts
def layout_bytes(layout: str):
    """(data_bytes, scale_bytes, row_bytes, group) of a layout."""
    v = [C.c_int32() for _ in range(4)]
    rc = lib().kvo_layout_bytes(LAYOUTS[layout], *[C.byref(x) for x in v])
    if rc:
        raise ValueError(layout)
    return tuple(x.value for x in v)


# ---------------------------------------------------------------- formats
def e4m3_encode(v, satfinite=False) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().kvo_e4m3_encode_n(_p(v), v.size, int(satfinite), _p(out))
    return out


def e2m1_encode(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().kvo_e2m1_encode_n(_p(v), v.size, _p(out))
    return out


def bf16_encode(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().kvo_bf16_encode_n(_p(v), v.size, _p(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    f = lib().kvo_e4m3_decode
    return np.array([f(int(x)) for x in np.asarray(c, np.uint8).ravel()]).reshape(np.shape(c))


def e2m1_decode(c) -> np.ndarray:
    f = lib().kvo_e2m1_decode
    return np.array([f(int(x)) for x in np.asarray(c, np.uint8).ravel()]).reshape(np.shape(c))


def ue8m0(amax) -> np.ndarray:
    a = _c(amax, np.float32)
    out = np.empty(a.shape, np.int32)
    lib().kvo_ue8m0_n(_p(a), a.size, _p(out))
    return out


def fp4_scale(amax) -> np.ndarray:
    a = _c(amax, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().kvo_fp4_scale_n(_p(a), a.size, _p(out))
    return out


def fp8_code(x, E) -> np.ndarray:
    """fp8 code of bf16 elements ``x`` under ue8m0 exponents ``E`` (same shape)."""
    x = _c(x, np.uint16)
    E = _c(np.broadcast_to(E, x.shape), np.int32)
    out = np.empty(x.shape, np.uint8)
    lib().kvo_fp8_code_n(_p(x), _p(E), x.size, _p(out))
    return out


def fp4_code(x, sc) -> np.ndarray:
    """e2m1 code of bf16 elements ``x`` under e4m3 scale codes ``sc``."""
    x = _c(x, np.uint16)
    sc = _c(np.broadcast_to(sc, x.shape), np.uint8)
    out = np.empty(x.shape, np.uint8)
    lib().kvo_fp4_code_n(_p(x), _p(sc), x.size, _p(out))
    return out


# ---------------------------------------------------------------- rows
def store_row(layout: str, x) -> tuple[np.ndarray, np.ndarray]:
    """bf16 rows ``[n, 512]`` -> (data ``[n, data_bytes]``, scale ``[n, scale_bytes]``)."""
    x = _c(x, np.uint16).reshape(-1, 512)
    db, sb, _, _ = layout_bytes(layout)
    data = np.zeros((x.shape[0], db), np.uint8)
    scale = np.zeros((x.shape[0], sb), np.uint8)
    lib().kvo_store_row_n(LAYOUTS[layout], _p(x), x.shape[0], _p(data), _p(scale))
    return data, scale


def dequant_row(layout: str, data, scale) -> np.ndarray:
    db, sb, _, _ = layout_bytes(layout)
    data = _c(data, np.uint8).reshape(-1, db)
    scale = _c(scale, np.uint8).reshape(-1, sb)
    out = np.zeros((data.shape[0], 512), np.uint16)
    lib().kvo_dequant_row_n(LAYOUTS[layout], _p(data), _p(scale), data.shape[0], _p(out))
    return out


# ---------------------------------------------------------------- paged cache
def _cache(cache: np.ndarray, layout: str, page_size: int) -> _Cache:
    assert cache.dtype == np.uint8 and cache.ndim == 2 and cache.flags.c_contiguous
    return _Cache(cache.ctypes.data, LAYOUTS[layout], page_size, cache.shape[1], cache.shape[0])


def store_rows(cache: np.ndarray, layout: str, page_size: int, rows, out_loc) -> int:
    """Quantize bf16 ``rows [n, 512]`` into ``cache`` (in place) at ``out_loc``."""
    rows = _c(rows, np.uint16).reshape(-1, 512)
    out_loc = _c(out_loc, np.int32)
    st = np.zeros(1, np.int32)
    cd = _cache(cache, layout, page_size)
    lib().kvo_store_rows(C.byref(cd), _p(rows), 512, _p(out_loc), rows.shape[0], _p(st))
    return int(st[0])


def store_rows_rope(cache: np.ndarray, layout: str, page_size: int, rows, positions, freqs,
                    out_loc):
    """Rotate the rope dims of bf16 ``rows [n, 512]`` at ``positions`` and
    quantize them into ``cache`` (in place).  -> (rotated rows ``[n, 512]``,
    zero for rows not stored; status)."""
    rows = _c(rows, np.uint16).reshape(-1, 512)
    positions = _c(positions, np.int32)
    out_loc = _c(out_loc, np.int32)
    freqs = _c(freqs, np.float32)
    rot = np.zeros_like(rows)
    st = np.zeros(1, np.int32)
    cd = _cache(cache, layout, page_size)
    lib().kvo_store_rows_rope(C.byref(cd), _p(rows), 512, _p(positions), _p(freqs),
                              freqs.shape[0], _p(out_loc), rows.shape[0], _p(rot), _p(st))
    return rot, int(st[0])


def dcp_owner(c: int, world: int, interleave: int) -> tuple[int, int]:
    """(owner rank, ordinal among the owner's rows) of compressed row ``c``."""
    local = C.c_int64(0)
    r = lib().kvo_dcp_owner(int(c), int(world), int(interleave), C.byref(local))
    return int(r), int(local.value)


def dcp_filter_ids(ids, token_to_req, block_table, *, page_size, num_pages, world, rank,
                   interleave, valid=None):
    """One rank's share of global ids ``[T, k]`` -> (slots ``[T, k]`` with a
    -1 tail, lens ``[T]``, status)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    t2r = _c(token_to_req, np.int32)
    bt = _c(block_table, np.int32)
    va = None if valid is None else _c(valid, np.int32)
    slots = np.zeros((T, k), np.int32)
    lens = np.zeros(T, np.int32)
    st = np.zeros(1, np.int32)
    lib().kvo_dcp_filter_ids(_p(ids), T, k, k, _p(t2r), bt.shape[0], _p(bt), bt.shape[1],
                             _p(va), page_size, num_pages, world, rank, interleave,
                             _p(slots), k, _p(lens), _p(st))
    return slots, lens, int(st[0])


def dequant_gather(cache: np.ndarray, layout: str, page_size: int, page_table, ids):
    """-> (bf16 rows ``[n, 512]``, status)."""
    ids = _c(ids, np.int32)
    pt = None if page_table is None else _c(page_table, np.int32)
    out = np.zeros((ids.size, 512), np.uint16)
    st = np.zeros(1, np.int32)
    cd = _cache(cache, layout, page_size)
    lib().kvo_dequant_gather(C.byref(cd), _p(pt), 0 if pt is None else pt.size,
                             _p(ids), ids.size, _p(out), 512, _p(st))
    return out, int(st[0])


# ---------------------------------------------------------------- compressor
def compress(*, ratio, mode, kv, score=None, fused=False, offsets=None, start_pos,
             page_table=None, out_loc=None, state, norm_w, eps, freqs, cache,
             layout, page_size, max_out_rows=None, want_prequant=True, draft_len=1,
             ring_slots=1, dcp_world=1, dcp_rank=0, dcp_interleave=1):
    """Run the compressor.  ``kv`` is ``[T, 512]`` (or ``[T, 1024]`` with
    ``fused=True``: kv in columns 0..511, score in 512..1023).  ``state`` and
    ``cache`` are updated in place.  Returns (latent, prequant, status,
    n_rows); latent / prequant have ``max_out_rows`` rows (default: the
    number of rows the plan emits in prefill, the token count in decode and
    verify) and untouched rows stay zero.  ``state`` is ``[S, ring_slots, 2,
    512]`` (``[S, 2, 512]`` for one entry)."""
    kv = _c(kv, np.uint16)
    S = int(np.asarray(start_pos).size)
    if fused:
        assert kv.shape[1] == 1024
        kv_p, kv_stride = kv.ctypes.data, 1024
        sc_p, sc_stride = kv.ctypes.data + 512 * 2, 1024
    else:
        kv_p, kv_stride = kv.ctypes.data, kv.shape[1]
        if score is not None:
            score = _c(score, np.uint16)
            sc_p, sc_stride = score.ctypes.data, score.shape[1]
        else:
            sc_p, sc_stride = None, 0
    offsets = None if offsets is None else _c(offsets, np.int32)
    start_pos = _c(start_pos, np.int32)
    pt = None if page_table is None else _c(page_table, np.int32)
    ol = None if out_loc is None else _c(out_loc, np.int32)
    assert state.dtype == np.uint16 and state.flags.c_contiguous
    norm_w = _c(norm_w, np.uint16)
    freqs = _c(freqs, np.float32)
    st = np.zeros(1, np.int32)
    a = _CompressArgs()
    a.ratio, a.mode = ratio, mode
    a.kv, a.kv_stride, a.score, a.score_stride = kv_p, kv_stride, sc_p, sc_stride
    a.num_slots = S
    a.offsets, a.start_pos = _p(offsets), _p(start_pos)
    a.page_table = _p(pt)
    a.pt_stride = 0 if pt is None else pt.shape[-1]
    a.out_loc, a.state = _p(ol), state.ctypes.data
    a.norm_w, a.eps = _p(norm_w), eps
    a.freqs, a.max_pos = _p(freqs), freqs.shape[0]
    a.cache = _cache(cache, layout, page_size)
    a.status = _p(st)
    a.draft_len, a.ring_slots = draft_len, ring_slots
    a.dcp_world, a.dcp_rank, a.dcp_interleave = dcp_world, dcp_rank, dcp_interleave
    a.kv_rows = kv.shape[0] if score is None or fused else min(kv.shape[0], score.shape[0])
    if mode != PREFILL:
        assert a.kv_rows >= S * (draft_len if mode == VERIFY else 1), "token rows"
    n_rows = lib().kvo_count_rows(C.byref(a))
    if max_out_rows is None:
        max_out_rows = n_rows if mode == PREFILL else S * (draft_len if mode == VERIFY else 1)
    latent = np.zeros((max(max_out_rows, 1), 512), np.uint16)
    pre = np.zeros_like(latent) if want_prequant else None
    a.latent, a.latent_stride, a.max_out_rows = latent.ctypes.data, 512, max_out_rows
    a.prequant, a.prequant_stride = _p(pre), 512
    lib().kvo_compress(C.byref(a))
    return latent[:max_out_rows], (None if pre is None else pre[:max_out_rows]), int(st[0]), int(n_rows)
