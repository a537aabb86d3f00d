"""The C-ABI library: it loads, exports every symbol include/kvc.h declares,
and its host-side checks and reuse head behave as documented.  No GPU: only
calls that return before any launch are made."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(kvc_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def kvc():
    import fp8_fp4_quantized_amd as k
    return k


def test_every_declared_symbol_is_exported(kvc):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(kvc.lib(), n), n
    # the binding covers the same list
    assert set(names) == set(kvc.SIGNATURES)


def test_ceiling_library_exports_its_header():
    """libkvc_ceiling.so (the benchmark's streaming yardstick) loads and
    exports every function include/kvc_ceiling.h declares; a bad argument is
    refused before any launch."""
    path = os.path.join(ROOT, "fp8_fp4_quantized_amd", "libkvc_ceiling.so")
    L = C.CDLL(path)
    names = declared_functions(os.path.join(ROOT, "include", "kvc_ceiling.h"))
    assert names == ["kvc_ceiling_compress_shape", "kvc_ceiling_gather_shape"]
    for n in names:
        assert hasattr(L, n), n
    L.kvc_ceiling_compress_shape.argtypes = [C.c_void_p] * 4 + [C.c_int64, C.c_void_p]
    L.kvc_ceiling_gather_shape.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    assert L.kvc_ceiling_compress_shape(None, None, None, None, 0, None) == 0
    assert L.kvc_ceiling_compress_shape(None, FAKE, FAKE, FAKE, 4, None) == -1
    assert L.kvc_ceiling_compress_shape(FAKE, FAKE, FAKE, FAKE, -1, None) == -1
    assert L.kvc_ceiling_gather_shape(FAKE, None, 4, None) == -1


def test_version_and_layouts(kvc):
    assert kvc.kvc_version() == 3
    want = {"V4": (576, 8, 584, 64, 448), "V41": (512, 16, 528, 32, 512),
            "V41_FP4": (256, 32, 288, 16, 512)}
    for name, w in want.items():
        i = kvc.kvc_layout_query(name)
        assert (i.data_bytes, i.scale_bytes, i.row_bytes, i.group, i.quant_dims) == w
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_layout_query(7)
    assert e.value.code == kvc.KVC_EUNSUPPORTED


def test_layouts_agree_with_oracle(kvc):
    import oracle
    for name in ("V4", "V41", "V41_FP4"):
        i = kvc.kvc_layout_query(name)
        assert oracle.layout_bytes(name) == (i.data_bytes, i.scale_bytes, i.row_bytes, i.group)


FAKE = 0x7F0000000000   # never dereferenced: every call below returns before a launch


def _cache(kvc, layout=1, page_size=64, stride=None, pages=4, base=FAKE):
    rb = kvc.kvc_layout_query(layout).row_bytes if layout in (0, 1, 2) else 1024
    return kvc.kvc_cache(base, layout, page_size,
                         page_size * rb if stride is None else stride, pages)


def test_cache_descriptor_checks(kvc):
    L = kvc.lib()
    bad = [
        _cache(kvc, base=0),                      # NULL
        _cache(kvc, base=FAKE + 8),               # misaligned
        _cache(kvc, page_size=48),                # not a power of two
        _cache(kvc, page_size=8192),              # too large
        _cache(kvc, stride=64 * 528 - 16),        # too small a page stride
        _cache(kvc, stride=64 * 528 + 8),         # not a multiple of 16
        _cache(kvc, pages=0),
    ]
    for c in bad:
        rc = L.kvc_store_rows(C.byref(c), FAKE, 512, FAKE, 1, None, None)
        assert rc == kvc.KVC_EINVAL, kvc.kvc_last_error()
        assert kvc.kvc_last_error()
    c = _cache(kvc, layout=9)
    assert L.kvc_store_rows(C.byref(c), FAKE, 512, FAKE, 1, None, None) == kvc.KVC_EUNSUPPORTED
    assert L.kvc_store_rows(None, FAKE, 512, FAKE, 1, None, None) == kvc.KVC_EINVAL


def test_store_and_gather_argument_checks(kvc):
    L = kvc.lib()
    c = _cache(kvc)
    assert L.kvc_store_rows(C.byref(c), FAKE, 512, FAKE, 0, None, None) == kvc.KVC_OK  # n = 0
    assert kvc.kvc_last_error() == ""
    assert L.kvc_store_rows(C.byref(c), FAKE, 512, FAKE, -1, None, None) == kvc.KVC_EINVAL
    assert L.kvc_store_rows(C.byref(c), None, 512, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert L.kvc_store_rows(C.byref(c), FAKE, 500, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert L.kvc_store_rows(C.byref(c), FAKE + 2, 512, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert L.kvc_dequant_gather(C.byref(c), None, 0, FAKE, 0, FAKE, 512, None, None) == kvc.KVC_OK
    assert L.kvc_dequant_gather(C.byref(c), None, 0, None, 5, FAKE, 512, None, None) == kvc.KVC_EINVAL
    assert L.kvc_dequant_gather(C.byref(c), FAKE, 0, FAKE, 5, FAKE, 512, None, None) == kvc.KVC_EINVAL
    assert L.kvc_dequant_gather(C.byref(c), None, 0, FAKE, 5, FAKE, 500, None, None) == kvc.KVC_EINVAL
    assert L.kvc_dequant_gather(C.byref(c), None, 0, FAKE, 5, FAKE + 8, 512, None, None) == kvc.KVC_EINVAL
    assert L.kvc_dequant_gather(C.byref(c), None, 0, FAKE, 5, FAKE, (1 << 25) + 8, None,
                                None) == kvc.KVC_EINVAL
    # the rotary store: same checks plus positions and the table
    rope = L.kvc_store_rows_rope
    assert rope(C.byref(c), FAKE, 512, FAKE, FAKE, 16, FAKE, 0, None, None) == kvc.KVC_OK
    assert rope(C.byref(c), FAKE, 512, None, FAKE, 16, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert rope(C.byref(c), FAKE, 512, FAKE, None, 16, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert rope(C.byref(c), FAKE, 512, FAKE, FAKE + 4, 16, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert rope(C.byref(c), FAKE, 512, FAKE, FAKE, 0, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert rope(C.byref(c), FAKE, 500, FAKE, FAKE, 16, FAKE, 3, None, None) == kvc.KVC_EINVAL
    assert rope(C.byref(_cache(kvc, page_size=3)), FAKE, 512, FAKE, FAKE, 16, FAKE, 3, None,
                None) == kvc.KVC_EINVAL


def test_dcp_filter_argument_checks(kvc):
    L = kvc.lib()

    def call(T=4, k=8, ids_stride=8, t2r=FAKE, n_req=2, bt=FAKE, bt_stride=4, bt_width=4,
             valid=None, page_size=64, num_pages=10, world=2, rank=1, inter=4, out=FAKE,
             out_stride=8, lens=FAKE):
        return L.kvc_dcp_filter_ids(FAKE, T, k, ids_stride, t2r, n_req, bt, bt_stride, bt_width,
                                    valid, page_size, num_pages, world, rank, inter, out,
                                    out_stride, lens, None, None)

    assert call(T=0) == kvc.KVC_OK
    for kw in (dict(T=-1), dict(k=-1), dict(k=65537, ids_stride=65537, out_stride=65537),
               dict(page_size=48), dict(page_size=8192), dict(world=0), dict(world=1025),
               dict(rank=2), dict(rank=-1), dict(inter=0), dict(inter=3), dict(inter=128),
               dict(t2r=None), dict(out=None), dict(lens=None), dict(ids_stride=7),
               dict(out_stride=4), dict(n_req=-1), dict(bt=None), dict(bt_stride=0),
               dict(bt_width=0), dict(bt_width=5),
               dict(num_pages=0), dict(num_pages=1 << 30), dict(out=FAKE + 2)):
        assert call(**kw) == kvc.KVC_EINVAL, kw
        assert kvc.kvc_last_error()


def _args(kvc, **kw):
    a = kvc.kvc_compress_args()
    a.ratio, a.mode = 2, kvc.MODE_PREFILL
    a.kv, a.kv_stride, a.score, a.score_stride = FAKE, 1024, FAKE + 1024, 1024
    a.num_slots = 4
    a.offsets, a.start_pos, a.page_table, a.pt_stride, a.pt_width = FAKE, FAKE, FAKE, 8, 8
    a.kv_rows = 64
    a.state, a.norm_w, a.eps, a.freqs, a.max_pos = FAKE, FAKE, 1e-6, FAKE, 100
    a.latent_out, a.latent_stride, a.max_out_rows = FAKE, 512, 10
    a.cache = _cache(kvc, layout=2, page_size=128)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_compress_argument_checks(kvc):
    L = kvc.lib()
    bad_inval = [
        dict(kv=0), dict(kv_stride=500), dict(kv=FAKE + 4), dict(score=0), dict(score_stride=4),
        dict(state=0), dict(offsets=0), dict(start_pos=0), dict(page_table=0),
        dict(pt_stride=0), dict(pt_width=0), dict(pt_width=9), dict(norm_w=0), dict(freqs=0),
        dict(max_pos=0), dict(latent_out=0),
        dict(latent_stride=256), dict(max_out_rows=-1), dict(num_slots=-1),
        dict(num_slots=8192), dict(eps=-1.0), dict(prequant_out=FAKE, prequant_stride=3),
        dict(kv_rows=0), dict(tile_rows=3), dict(tile_rows=8), dict(tile_rows=-1),
        # decode / verify read token rows 0 .. num_slots * D - 1
        dict(mode=kvc.MODE_DECODE, kv_rows=3),
        dict(mode=kvc.MODE_VERIFY, draft_len=4, kv_rows=15),
    ]
    for kw in bad_inval:
        a = _args(kvc, **kw)
        assert L.kvc_compress_store(C.byref(a), None) == kvc.KVC_EINVAL, kw
    for kw in (dict(ratio=3), dict(ratio=0), dict(mode=5)):
        a = _args(kvc, **kw)
        assert L.kvc_compress_store(C.byref(a), None) == kvc.KVC_EUNSUPPORTED, kw
    # decode and verify need out_loc or a page table
    a = _args(kvc, mode=kvc.MODE_DECODE, page_table=0, out_loc=0)
    assert L.kvc_compress_store(C.byref(a), None) == kvc.KVC_EINVAL
    a = _args(kvc, mode=kvc.MODE_VERIFY, draft_len=4, page_table=0, out_loc=0)
    assert L.kvc_compress_store(C.byref(a), None) == kvc.KVC_EINVAL
    # verify draft length, ring size and the context-parallel group
    for kw in (dict(mode=kvc.MODE_VERIFY, draft_len=0), dict(mode=kvc.MODE_VERIFY, draft_len=65),
               dict(mode=kvc.MODE_VERIFY, draft_len=64, num_slots=1 << 25),
               dict(ring_slots=-1), dict(ring_slots=1025), dict(dcp_world=-1),
               dict(dcp_world=2, dcp_rank=2, dcp_interleave=1),
               dict(dcp_world=2, dcp_rank=-1, dcp_interleave=1),
               dict(dcp_world=1025, dcp_rank=0, dcp_interleave=1),
               dict(dcp_world=2, dcp_rank=0, dcp_interleave=0),
               dict(dcp_world=2, dcp_rank=0, dcp_interleave=3),
               dict(dcp_world=2, dcp_rank=0, dcp_interleave=256)):
        a = _args(kvc, **kw)
        assert L.kvc_compress_store(C.byref(a), None) == kvc.KVC_EINVAL, kw
    # nothing to do is fine
    a = _args(kvc, num_slots=0)
    assert L.kvc_compress_store(C.byref(a), None) == kvc.KVC_OK
    assert L.kvc_compress_store(None, None) == kvc.KVC_EINVAL


def test_reuse_head_semantics(kvc):
    """Head reuse (sglang PR #45909, summary): same (source cache, ids, row
    count) hits; a plain get (forget), a reallocation (new output or cache
    pointer) or a new forward forgets the head.  n = 0 keeps every call off
    the GPU, the key logic is the same."""
    L = kvc.lib()
    kb = L.kvc_kvbuf_create()
    assert kb
    c = _cache(kvc)
    hit = C.c_int32(-1)

    def call(cache=c, pt=None, ids=FAKE, n=0, out=FAKE, stride=512):
        rc = L.kvc_dequant_gather_reuse(kb, C.byref(cache), pt, 0 if pt is None else 16, ids, n,
                                        out, stride, None, C.byref(hit), None)
        assert rc == kvc.KVC_OK
        return hit.value

    assert call() == 0
    assert call() == 1
    assert call() == 1
    assert call(ids=FAKE + 64) == 0          # other ids
    assert call(ids=FAKE + 64) == 1
    assert call(out=FAKE + 4096) == 0        # output reallocated
    assert call(out=FAKE + 4096) == 1
    L.kvc_kvbuf_forget(kb)                   # a plain get
    assert call(out=FAKE + 4096) == 0
    L.kvc_kvbuf_begin_forward(kb)            # a new forward
    assert call(out=FAKE + 4096) == 0
    assert call(out=FAKE + 4096) == 1
    c2 = _cache(kvc, base=FAKE + 1 << 20)    # another source cache
    assert call(cache=c2, out=FAKE + 4096) == 0
    assert call(cache=c2, pt=FAKE, out=FAKE + 4096) == 0   # with a page table
    assert call(cache=c2, pt=FAKE, out=FAKE + 4096) == 1
    assert call(cache=c2, pt=FAKE, out=FAKE + 4096, stride=1024) == 0
    # a failed call leaves no head
    bad = _cache(kvc, page_size=3)
    rc = L.kvc_dequant_gather_reuse(kb, C.byref(bad), None, 0, FAKE, 0, FAKE, 512, None,
                                    C.byref(hit), None)
    assert rc == kvc.KVC_EINVAL and hit.value == 0
    assert call(cache=c2, pt=FAKE, out=FAKE + 4096, stride=1024) == 0
    L.kvc_kvbuf_destroy(kb)


def test_binding_rejects_host_and_mistyped_tensors(kvc):
    """The Python binding checks every tensor it passes as a raw pointer
    (device, dtype, contiguity) before calling the library: host tensors and
    int64 ids are refused with ValueError, and nothing is launched."""
    import torch
    cache = kvc.Cache(torch.zeros((2, 64 * 528), dtype=torch.uint8), "V41", 64)
    ids = torch.zeros(4, dtype=torch.int32)
    out = torch.zeros((4, 512), dtype=torch.int16)
    with pytest.raises(ValueError, match="ids"):
        kvc.kvc_dequant_gather(cache, None, ids, out)
    with pytest.raises(ValueError, match="page_table"):
        kvc.kvc_dequant_gather(cache, torch.zeros(4, dtype=torch.int64), ids, out)
    with pytest.raises(ValueError, match="rows"):
        kvc.kvc_store_rows(cache, out, ids)
    with pytest.raises(ValueError, match="kv"):
        kvc.kvc_compress_store(ratio=1, mode=kvc.MODE_PREFILL, kv=out, score=None,
                               start_pos=ids, cache=cache, norm_w=out[0], eps=1e-6,
                               freqs=torch.zeros((4, 64)), latent_out=out,
                               offsets=torch.zeros((2, 4), dtype=torch.int32),
                               page_table=torch.zeros((4, 2), dtype=torch.int32))


def test_binding_checks_sizes_against_counts(kvc):
    """Every count the binding hands the library (rows, ids, slots, tokens,
    table rows, output capacity) is checked against the tensors' shapes on
    the host before any launch: a mismatch that would let a kernel read or
    write past an allocation raises ValueError.  Host tensors reach these
    checks first, so no GPU is needed."""
    import torch
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    b16 = lambda *s: torch.zeros(s, dtype=torch.int16)
    cache = kvc.Cache(torch.zeros((4, 64 * 528), dtype=torch.uint8), "V41", 64)
    # gather: output rows against ids
    with pytest.raises(ValueError, match="out: 3 rows for 4 ids"):
        kvc.kvc_dequant_gather(cache, None, i32(4), b16(3, 512))
    with pytest.raises(ValueError, match="columns"):
        kvc.kvc_dequant_gather(cache, None, i32(4), b16(4, 256))
    buf = kvc.KVBuf()
    with pytest.raises(ValueError, match="out: 3 rows"):
        buf.kvc_dequant_gather_reuse(cache, None, i32(4), b16(3, 512))
    # stores: out_loc and positions against rows, the rotary table's width
    with pytest.raises(ValueError, match="out_loc: 2 entries for 3 rows"):
        kvc.kvc_store_rows(cache, b16(3, 512), i32(2))
    with pytest.raises(ValueError, match="positions"):
        kvc.kvc_store_rows_rope(cache, b16(3, 512), i32(2), torch.zeros((8, 64)), i32(3))
    with pytest.raises(ValueError, match="freqs"):
        kvc.kvc_store_rows_rope(cache, b16(3, 512), i32(3), torch.zeros((8, 32)), i32(3))
    # DCP filter: outputs and per-row inputs against [T, k]
    ids = i32(5, 8)
    good = dict(token_to_req=i32(5), block_table=i32(2, 4), out_slots=i32(5, 8),
                out_lens=i32(5), page_size=64, num_pages=10, world=2, rank=0, interleave=4)
    for key, bad in (("out_slots", i32(5, 7)), ("out_slots", i32(4, 8)), ("out_lens", i32(4)),
                     ("token_to_req", i32(4)), ("valid", i32(4)), ("block_table", i32(8))):
        kw = dict(good, **{key: bad})
        with pytest.raises(ValueError, match=key):
            kvc.kvc_dcp_filter_ids(ids, **kw)

    # compressor
    S = 4

    def comp(**kw):
        base = dict(ratio=2, mode=kvc.MODE_PREFILL, kv=b16(64, 1024)[:, :512],
                    score=b16(64, 1024)[:, 512:], start_pos=i32(S), cache=cache,
                    norm_w=b16(512), eps=1e-6, freqs=torch.zeros((64, 64)),
                    latent_out=b16(16, 512), offsets=i32(2, S), page_table=i32(S, 2),
                    state=b16(S, 2, 512))
        base.update(kw)
        kvc.kvc_compress_store(**base)

    cases = [
        (dict(max_out_rows=17), "max_out_rows 17"),              # past latent_out
        (dict(prequant_out=b16(8, 512)), "prequant_out"),          # fewer rows than max_out_rows
        (dict(prequant_out=b16(16, 512), max_out_rows=20), "max_out_rows 20"),
        (dict(state=b16(S, 2, 256)), "state"),                     # too small a ring
        (dict(state=b16(S, 2, 512), ring_slots=2), "state"),
        (dict(offsets=i32(2, S - 1)), "offsets"),
        (dict(offsets=None), "offsets"),
        (dict(page_table=i32(S - 1, 2)), "page_table"),
        (dict(page_table=i32(S * 2)), "page_table"),
        (dict(norm_w=b16(256)), "norm_w"),
        (dict(freqs=torch.zeros((64, 32))), "freqs"),
        (dict(kv=b16(64, 256)), "kv"),
        (dict(latent_out=b16(16, 128)), "latent_out"),
        # decode / verify: token rows, out_loc entries and latent rows per token
        (dict(mode=kvc.MODE_VERIFY, draft_len=4, latent_out=b16(15, 512), offsets=None,
              kv=b16(16, 512), score=b16(16, 512)), "max_out_rows"),
        (dict(mode=kvc.MODE_VERIFY, draft_len=4, latent_out=b16(16, 512), offsets=None,
              kv=b16(15, 512), score=b16(16, 512)), "kv: 15 token rows"),
        (dict(mode=kvc.MODE_DECODE, offsets=None, kv=b16(4, 512), score=b16(4, 512),
              out_loc=i32(3)), "out_loc"),
    ]
    for kw, msg in cases:
        with pytest.raises(ValueError, match=msg):
            comp(**kw)
