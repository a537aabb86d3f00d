"""Python binding of ``libkvc.so``: the MI355X (gfx950) compressed-KV store
and gather for DeepSeek-V4.1 low-ratio layers (C ABI in ``include/kvc.h``).

Argument marshalling only.  Every step of the path runs in the HIP kernels of
``libkvc.so``; PyTorch provides device memory and the current stream.  There
is no fallback: importing this package without the built library raises.

Function names are those of the C ABI.  Tensors are CUDA (HIP) tensors:
bf16 rows may be ``torch.bfloat16`` or ``int16``/``uint16`` bit patterns;
caches are ``uint8`` tensors ``[num_pages, page_stride]``.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch  # noqa: F401  (loads the HIP runtime that libkvc.so then binds to)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvc.so")

KVC_OK, KVC_EINVAL, KVC_EUNSUPPORTED, KVC_ELAUNCH = 0, -1, -2, -3
LAYOUT_V4, LAYOUT_V41, LAYOUT_V41_FP4 = 0, 1, 2
LAYOUTS = {"V4": LAYOUT_V4, "V41": LAYOUT_V41, "V41_FP4": LAYOUT_V41_FP4}
MODE_PREFILL, MODE_DECODE, MODE_VERIFY = 0, 1, 2
STATUS_ID_RANGE, STATUS_PAGE_RANGE, STATUS_PT_RANGE = 1, 2, 4
STATUS_LATENT_RANGE, STATUS_POS_RANGE, STATUS_REQ_RANGE = 8, 16, 32
STATUS_TOKEN_RANGE = 64


class KvcError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"kvc error {code}: {msg}")
        self.code = code


class kvc_layout_info(C.Structure):
    _fields_ = [("data_bytes", C.c_int32), ("scale_bytes", C.c_int32),
                ("row_bytes", C.c_int32), ("group", C.c_int32), ("quant_dims", C.c_int32)]


class kvc_cache(C.Structure):
    _fields_ = [("base", C.c_void_p), ("layout", C.c_int32), ("page_size", C.c_int32),
                ("page_stride", C.c_int64), ("num_pages", C.c_int64)]


class kvc_compress_args(C.Structure):
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
        ("latent_out", C.c_void_p), ("latent_stride", C.c_int64), ("max_out_rows", C.c_int64),
        ("prequant_out", C.c_void_p), ("prequant_stride", C.c_int64),
        ("cache", kvc_cache), ("status", C.c_void_p),
        ("draft_len", C.c_int32), ("ring_slots", C.c_int32),
        ("dcp_world", C.c_int32), ("dcp_rank", C.c_int32), ("dcp_interleave", C.c_int32),
        ("tile_rows", C.c_int32), ("kv_rows", C.c_int64), ("pt_width", C.c_int64),
    ]


# symbol -> (restype, argtypes); the same list as include/kvc.h
_VP, _I32, _I64 = C.c_void_p, C.c_int32, C.c_int64
SIGNATURES = {
    "kvc_layout_query": (C.c_int, [_I32, C.POINTER(kvc_layout_info)]),
    "kvc_store_rows": (C.c_int, [C.POINTER(kvc_cache), _VP, _I64, _VP, _I64, _VP, _VP]),
    "kvc_store_rows_rope": (C.c_int, [C.POINTER(kvc_cache), _VP, _I64, _VP, _VP, _I64, _VP, _I64,
                                      _VP, _VP]),
    "kvc_dcp_filter_ids": (C.c_int, [_VP, _I64, _I32, _I64, _VP, _I32, _VP, _I64, _I64, _VP, _I32,
                                     _I64, _I32, _I32, _I32, _VP, _I64, _VP, _VP, _VP]),
    "kvc_compress_store": (C.c_int, [C.POINTER(kvc_compress_args), _VP]),
    "kvc_dequant_gather": (C.c_int, [C.POINTER(kvc_cache), _VP, _I64, _VP, _I64, _VP, _I64, _VP, _VP]),
    "kvc_kvbuf_create": (_VP, []),
    "kvc_kvbuf_destroy": (None, [_VP]),
    "kvc_kvbuf_forget": (None, [_VP]),
    "kvc_kvbuf_begin_forward": (None, [_VP]),
    "kvc_dequant_gather_reuse": (C.c_int, [_VP, C.POINTER(kvc_cache), _VP, _I64, _VP, _I64, _VP,
                                           _I64, _VP, _VP, _VP]),
    "kvc_last_error": (C.c_char_p, []),
    "kvc_version": (C.c_int, []),
}

_lib = None


def lib():
    """The loaded ``libkvc.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m fp8_fp4_quantized_amd.build` or __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


lib()   # fail loudly at import when the HIP library is missing


def _check(rc: int) -> None:
    if rc != KVC_OK:
        raise KvcError(rc, lib().kvc_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


_I32_T = (torch.int32,)
_F32_T = (torch.float32,)
_B16_T = (torch.bfloat16, torch.int16, torch.uint16)


def _dense(t, dtypes, name: str) -> int:
    """Pointer of a contiguous device tensor of one of ``dtypes``."""
    if not (t.is_cuda and t.dtype in dtypes and t.is_contiguous()):
        raise ValueError(f"{name}: expected a contiguous device tensor of {dtypes}, got "
                         f"{t.dtype} {tuple(t.shape)} strides {t.stride()} on {t.device}")
    return t.data_ptr()


def _rows(t, dtypes, name: str) -> int:
    """Pointer of a 2-D device tensor of ``dtypes`` whose rows are contiguous
    (any row stride)."""
    if not (t.is_cuda and t.dtype in dtypes and t.dim() == 2 and t.stride(1) == 1):
        raise ValueError(f"{name}: expected a 2-D device tensor of {dtypes} with contiguous "
                         f"rows, got {t.dtype} {tuple(t.shape)} strides {t.stride()}")
    return t.data_ptr()


def _opt(t, check, dtypes, name: str) -> int | None:
    return None if t is None else check(t, dtypes, name)


def _need(ok: bool, msg: str) -> None:
    """A size the library would trust (it reads or writes that many entries)
    that the tensor does not have: refused before anything is launched."""
    if not ok:
        raise ValueError(msg)


def _rows_of(t, name: str, min_cols: int = 512) -> int:
    """Row count of a 2-D row buffer holding at least ``min_cols`` columns."""
    _need(t.dim() == 2, f"{name}: expected a 2-D tensor, got shape {tuple(t.shape)}")
    _need(t.shape[1] >= min_cols, f"{name}: rows hold {t.shape[1]} columns, need {min_cols}")
    return t.shape[0]


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


@dataclass
class Cache:
    """A paged cache: ``data`` is a uint8 tensor ``[num_pages, page_stride]``."""
    data: torch.Tensor
    layout: int
    page_size: int

    def desc(self) -> kvc_cache:
        assert self.data.dtype == torch.uint8 and self.data.dim() == 2 and self.data.is_contiguous()
        lay = LAYOUTS[self.layout] if isinstance(self.layout, str) else int(self.layout)
        return kvc_cache(self.data.data_ptr(), lay, self.page_size,
                         self.data.shape[1], self.data.shape[0])


# --------------------------------------------------------------------- calls
def kvc_version() -> int:
    return lib().kvc_version()


def kvc_last_error() -> str:
    return lib().kvc_last_error().decode()


def kvc_layout_query(layout) -> kvc_layout_info:
    info = kvc_layout_info()
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    _check(lib().kvc_layout_query(lay, C.byref(info)))
    return info


def kvc_store_rows(cache: Cache, rows: torch.Tensor, out_loc: torch.Tensor,
                   status: torch.Tensor | None = None, stream=None) -> None:
    """Quantize bf16 ``rows [n, >=512]`` into ``cache`` at ``out_loc [n]``."""
    n = _rows_of(rows, "rows")
    _need(out_loc.numel() >= n, f"out_loc: {out_loc.numel()} entries for {n} rows")
    d = cache.desc()
    _check(lib().kvc_store_rows(C.byref(d), _rows(rows, _B16_T, "rows"), rows.stride(0),
                                _dense(out_loc, _I32_T, "out_loc"), rows.shape[0],
                                _opt(status, _dense, _I32_T, "status"), _stream(stream)))


def kvc_store_rows_rope(cache: Cache, rows: torch.Tensor, positions: torch.Tensor,
                        freqs: torch.Tensor, out_loc: torch.Tensor,
                        status: torch.Tensor | None = None, stream=None) -> None:
    """Rotate the rope dims of bf16 ``rows [n, >=512]`` at ``positions [n]``
    (table ``freqs [max_pos, 64]`` fp32) and quantize them at ``out_loc``."""
    n = _rows_of(rows, "rows")
    _need(out_loc.numel() >= n, f"out_loc: {out_loc.numel()} entries for {n} rows")
    _need(positions.numel() >= n, f"positions: {positions.numel()} entries for {n} rows")
    _need(freqs.dim() == 2 and freqs.shape[1] == 64, f"freqs: shape {tuple(freqs.shape)}, "
                                                     "expected [max_pos, 64]")
    d = cache.desc()
    _check(lib().kvc_store_rows_rope(C.byref(d), _rows(rows, _B16_T, "rows"), rows.stride(0),
                                     _dense(positions, _I32_T, "positions"),
                                     _dense(freqs, _F32_T, "freqs"), freqs.shape[0],
                                     _dense(out_loc, _I32_T, "out_loc"), rows.shape[0],
                                     _opt(status, _dense, _I32_T, "status"), _stream(stream)))


def kvc_dcp_filter_ids(ids: torch.Tensor, token_to_req: torch.Tensor, block_table: torch.Tensor,
                       out_slots: torch.Tensor, out_lens: torch.Tensor, *, page_size: int,
                       num_pages: int, world: int, rank: int, interleave: int,
                       valid: torch.Tensor | None = None, status: torch.Tensor | None = None,
                       stream=None) -> None:
    """This rank's share of global compressed ids ``[T, k]``: physical slots
    compacted into ``out_slots [T, k]`` (-1 tail), counts into ``out_lens [T]``."""
    _need(ids.dim() == 2, f"ids: expected [T, k], got shape {tuple(ids.shape)}")
    T, k = ids.shape
    _need(token_to_req.numel() >= T, f"token_to_req: {token_to_req.numel()} entries for {T} rows")
    _need(valid is None or valid.numel() >= T, f"valid: fewer than {T} entries")
    _need(out_slots.dim() == 2 and out_slots.shape[0] >= T and out_slots.shape[1] >= k,
          f"out_slots: shape {tuple(out_slots.shape)}, need at least [{T}, {k}]")
    _need(out_lens.numel() >= T, f"out_lens: {out_lens.numel()} entries for {T} rows")
    _need(block_table.dim() == 2, f"block_table: expected [n_req, pages], got "
                                  f"{tuple(block_table.shape)}")
    _check(lib().kvc_dcp_filter_ids(_rows(ids, _I32_T, "ids"), T, k, ids.stride(0),
                                    _dense(token_to_req, _I32_T, "token_to_req"),
                                    block_table.shape[0], _rows(block_table, _I32_T, "block_table"),
                                    block_table.stride(0), block_table.shape[1],
                                    _opt(valid, _dense, _I32_T, "valid"),
                                    page_size, num_pages, world, rank, interleave,
                                    _rows(out_slots, _I32_T, "out_slots"), out_slots.stride(0),
                                    _dense(out_lens, _I32_T, "out_lens"),
                                    _opt(status, _dense, _I32_T, "status"), _stream(stream)))


def kvc_dequant_gather(cache: Cache, page_table: torch.Tensor | None, ids: torch.Tensor,
                       out: torch.Tensor, status: torch.Tensor | None = None, stream=None) -> None:
    """``out[j] = bf16 row of ids[j]`` (through ``page_table`` when given)."""
    _need(_rows_of(out, "out") >= ids.numel(), f"out: {out.shape[0]} rows for {ids.numel()} ids")
    d = cache.desc()
    n_pages = 0 if page_table is None else page_table.numel()
    _check(lib().kvc_dequant_gather(C.byref(d), _opt(page_table, _dense, _I32_T, "page_table"),
                                    n_pages, _dense(ids, _I32_T, "ids"), ids.numel(),
                                    _rows(out, _B16_T, "out"), out.stride(0),
                                    _opt(status, _dense, _I32_T, "status"), _stream(stream)))


class KVBuf:
    """Dequant-reuse head (``kvc_kvbuf``): a gather whose arguments match the
    last one it ran is skipped."""

    def __init__(self):
        self._h = lib().kvc_kvbuf_create()
        if not self._h:
            raise MemoryError("kvc_kvbuf_create")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.kvc_kvbuf_destroy(h)

    def forget(self) -> None:
        lib().kvc_kvbuf_forget(self._h)

    def begin_forward(self) -> None:
        lib().kvc_kvbuf_begin_forward(self._h)

    def kvc_dequant_gather_reuse(self, cache: Cache, page_table, ids, out, status=None,
                                 stream=None) -> bool:
        _need(_rows_of(out, "out") >= ids.numel(),
              f"out: {out.shape[0]} rows for {ids.numel()} ids")
        d = cache.desc()
        hit = C.c_int32(0)
        n_pages = 0 if page_table is None else page_table.numel()
        _check(lib().kvc_dequant_gather_reuse(
            self._h, C.byref(d), _opt(page_table, _dense, _I32_T, "page_table"), n_pages,
            _dense(ids, _I32_T, "ids"), ids.numel(), _rows(out, _B16_T, "out"), out.stride(0),
            _opt(status, _dense, _I32_T, "status"), C.byref(hit), _stream(stream)))
        return bool(hit.value)


def _compress_args(*, ratio: int, mode: int, kv: torch.Tensor, score: torch.Tensor | None,
                       start_pos: torch.Tensor, cache: Cache, norm_w: torch.Tensor, eps: float,
                       freqs: torch.Tensor, latent_out: torch.Tensor, max_out_rows: int | None = None,
                       offsets: torch.Tensor | None = None, page_table: torch.Tensor | None = None,
                       out_loc: torch.Tensor | None = None, state: torch.Tensor | None = None,
                       prequant_out: torch.Tensor | None = None, status: torch.Tensor | None = None,
                       draft_len: int = 1, ring_slots: int = 1, dcp_world: int = 1,
                       dcp_rank: int = 0, dcp_interleave: int = 1,
                       tile_rows: int = 0) -> kvc_compress_args:
    """The argument block of kvc_compress_store (every check done here).
    The fused compressor.  ``kv``/``score`` are 2-D views whose row stride
    is passed through (a fused ``|kv|score|`` buffer ``proj [T, 1024]`` is
    ``kv=proj[:, :512], score=proj[:, 512:]``).  ``state`` is ``[S,
    ring_slots, 2, 512]`` bf16 (``[S, 2, 512]`` for one entry).  A page
    table may be a column slice of a wider table: its width bounds the
    logical pages, its row stride addresses the rows."""
    S = start_pos.numel()
    D = draft_len if mode == MODE_VERIFY else 1
    kv_rows = _rows_of(kv, "kv")
    if score is not None:
        kv_rows = min(kv_rows, _rows_of(score, "score"))
    lat_rows = _rows_of(latent_out, "latent_out")
    if max_out_rows is None:
        max_out_rows = lat_rows
    _need(0 <= max_out_rows <= lat_rows,
          f"max_out_rows {max_out_rows}: latent_out holds {lat_rows} rows")
    _need(prequant_out is None or _rows_of(prequant_out, "prequant_out") >= max_out_rows,
          f"prequant_out: fewer than max_out_rows = {max_out_rows} rows")
    if mode != MODE_PREFILL:
        _need(max_out_rows >= S * D, f"max_out_rows {max_out_rows}: decode / verify write "
                                     f"latent rows up to {S * D}")
        _need(kv_rows >= S * D, f"kv: {kv_rows} token rows for {S} slots x {D} tokens")
        _need(out_loc is None or out_loc.numel() >= S * D,
              f"out_loc: {out_loc.numel() if out_loc is not None else 0} entries for {S * D} "
              "tokens")
    else:
        _need(offsets is not None and offsets.numel() >= 2 * S,
              f"offsets: expected [2, {S}] entries")
    if page_table is not None:
        _need(page_table.dim() == 2 and page_table.shape[0] >= S,
              f"page_table: shape {tuple(page_table.shape)}, need {S} rows")
    if ratio == 2:
        _need(state is not None and state.numel() >= S * max(ring_slots, 1) * 1024,
              f"state: need [{S}, {max(ring_slots, 1)}, 2, 512] bf16")
    _need(norm_w.numel() >= 512, "norm_w: expected 512 entries")
    _need(freqs.dim() == 2 and freqs.shape[1] == 64,
          f"freqs: shape {tuple(freqs.shape)}, expected [max_pos, 64]")
    a = kvc_compress_args()
    a.ratio, a.mode = ratio, mode
    a.kv, a.kv_stride = _rows(kv, _B16_T, "kv"), kv.stride(0)
    a.score = _opt(score, _rows, _B16_T, "score")
    a.score_stride = 0 if score is None else score.stride(0)
    a.num_slots = S
    a.kv_rows = kv_rows
    a.offsets = _opt(offsets, _dense, _I32_T, "offsets")
    a.start_pos = _dense(start_pos, _I32_T, "start_pos")
    a.page_table = _opt(page_table, _rows, _I32_T, "page_table")
    a.pt_stride = 0 if page_table is None else page_table.stride(0)
    a.pt_width = 0 if page_table is None else page_table.shape[1]
    a.out_loc = _opt(out_loc, _dense, _I32_T, "out_loc")
    a.state = _opt(state, _dense, _B16_T, "state")
    a.norm_w, a.eps = _dense(norm_w, _B16_T, "norm_w"), eps
    a.freqs, a.max_pos = _dense(freqs, _F32_T, "freqs"), freqs.shape[0]
    a.latent_out = _rows(latent_out, _B16_T, "latent_out")
    a.latent_stride = latent_out.stride(0)
    a.max_out_rows = max_out_rows
    a.prequant_out = _opt(prequant_out, _rows, _B16_T, "prequant_out")
    a.prequant_stride = 0 if prequant_out is None else prequant_out.stride(0)
    a.cache = cache.desc()
    a.status = _opt(status, _dense, _I32_T, "status")
    a.draft_len, a.ring_slots = draft_len, ring_slots
    a.dcp_world, a.dcp_rank, a.dcp_interleave = dcp_world, dcp_rank, dcp_interleave
    a.tile_rows = tile_rows
    return a


def kvc_compress_store(*, stream=None, **kw) -> None:
    """The fused compressor; keyword arguments as ``_compress_args``."""
    _check(lib().kvc_compress_store(C.byref(_compress_args(**kw)), _stream(stream)))


class Prepared:
    """A call whose arguments were checked and packed once: calling it
    launches on the given stream (default: the current one) with no Python
    work beyond the foreign call.  It keeps the tensors it points to alive;
    their contents may change between calls, their storage must not."""

    __slots__ = ("_fn", "_args", "_keep")

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def prepare_compress_store(**kw) -> Prepared:
    """kvc_compress_store with its argument block built once."""
    a = _compress_args(**kw)
    return Prepared(lib().kvc_compress_store, (C.byref(a),), (a, kw))


def prepare_dequant_gather(cache: Cache, page_table: torch.Tensor | None, ids: torch.Tensor,
                           out: torch.Tensor, status: torch.Tensor | None = None) -> Prepared:
    """kvc_dequant_gather with its arguments checked and packed once."""
    _need(_rows_of(out, "out") >= ids.numel(), f"out: {out.shape[0]} rows for {ids.numel()} ids")
    d = cache.desc()
    n_pages = 0 if page_table is None else page_table.numel()
    args = (C.byref(d), _opt(page_table, _dense, _I32_T, "page_table"), n_pages,
            _dense(ids, _I32_T, "ids"), ids.numel(), _rows(out, _B16_T, "out"), out.stride(0),
            _opt(status, _dense, _I32_T, "status"))
    return Prepared(lib().kvc_dequant_gather, args, (d, cache, page_table, ids, out, status))
