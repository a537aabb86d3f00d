"""Helpers for the GPU parity tests: host <-> device copies and the
comparison rules for the fused compressor's outputs."""
from __future__ import annotations

import hashlib

import numpy as np
import torch

import oracle
from tests import spec


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor with the same bits (uint16 as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def row_parts(cache: np.ndarray, layout: str, page_size: int, slot: int):
    db, sb, _, _ = oracle.layout_bytes(layout)
    p, r = divmod(int(slot), page_size)
    d = cache[p, r * db:(r + 1) * db]
    s = cache[p, page_size * db + r * sb: page_size * db + (r + 1) * sb]
    return d, s


def written_mask(cache_shape, layout: str, page_size: int, slots) -> np.ndarray:
    db, sb, _, _ = oracle.layout_bytes(layout)
    m = np.zeros(cache_shape, bool)
    for slot in slots:
        p, r = divmod(int(slot), page_size)
        m[p, r * db:(r + 1) * db] = True
        m[p, page_size * db + r * sb: page_size * db + (r + 1) * sb] = True
    return m


# --------------------------------------------------------------- tolerances
REL = 2e-2


def assert_latent_close(g: np.ndarray, o: np.ndarray, what="latent"):
    """|g - o| <= 2e-2 |o| + 2e-2 * 2^-6 * rms(o_row), elementwise (bf16 rows)."""
    gv, ov = spec.bf16_value(g), spec.bf16_value(o)
    rms = np.sqrt(np.mean(ov * ov, axis=-1, keepdims=True))
    tol = REL * np.abs(ov) + REL * 2.0 ** -6 * rms
    bad = np.abs(gv - ov) > tol
    assert not bad.any(), (what, np.argwhere(bad)[:5], gv[bad][:5], ov[bad][:5])


def _ordinal_fp8(c):
    c = c.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def _ordinal_fp4(n):
    n = n.astype(np.int64)
    mag = n & 7
    return np.where(n & 8, -mag, mag)


def assert_rows_close(layout: str, gd, gs, od, os_, ref_vals):
    """Fused-path cache rows: where the scale bytes agree every code is
    within one step of the oracle's; where a scale differs the dequantized
    values agree within the latent tolerance plus one quantization step.
    gd/gs/od/os_: [n, data], [n, scale] byte arrays; ref_vals: the oracle's
    fp64 values of the rows (bf16 of z) for the tolerance."""
    n = gd.shape[0]
    gq = oracle.dequant_row(layout, gd, gs)
    oq = oracle.dequant_row(layout, od, os_)
    gv, ov = spec.bf16_value(gq), spec.bf16_value(oq)
    t8 = spec.e4m3_table()
    if layout == "V41_FP4":
        nib = lambda d: np.stack([d & 0xF, d >> 4], -1).reshape(n, 512)
        gc, oc = _ordinal_fp4(nib(gd)), _ordinal_fp4(nib(od))
        same = np.repeat(gs == os_, 16, axis=1)
        step = np.repeat(np.abs(t8[np.maximum(gs, os_)]), 16, axis=1) * 2.0
        nq = 512
    else:
        nq = 512 if layout == "V41" else 448
        g = 32 if layout == "V41" else 64
        gc, oc = _ordinal_fp8(gd[:, :nq]), _ordinal_fp8(od[:, :nq])
        same = np.repeat(gs[:, : nq // g] == os_[:, : nq // g], g, axis=1)
        E = np.maximum(gs[:, : nq // g], os_[:, : nq // g]).astype(np.float64)
        step = np.repeat(2.0 ** (E - 127) * 32.0, g, axis=1)     # one step near 448 s
    dc = np.abs(gc - oc)
    assert np.all(dc[same[:, :nq]] <= 1), ("code step", np.argwhere((dc > 1) & same[:, :nq])[:5])
    rv = np.abs(ref_vals[:, :nq])
    rms = np.sqrt(np.mean(ref_vals * ref_vals, axis=-1, keepdims=True))
    tol = REL * rv + REL * 2.0 ** -6 * rms + step
    diff = np.abs(gv[:, :nq] - ov[:, :nq])
    bad = (~same[:, :nq]) & (diff > tol)
    assert not bad.any(), ("scale-differs rows", np.argwhere(bad)[:5])
    if layout == "V4":
        assert_latent_close(gq[:, 448:], oq[:, 448:], "v4 rope part")


# --------------------------------------------------------------- compressor runs
def _pt_view(pt, spare_cols, num_pages):
    """device copy of page table ``pt`` [S, W]; with spare columns, a [:, :W]
    slice of a [S, W + spare] table whose extra entries are valid pages"""
    if not spare_cols:
        return dev(pt)
    S, Wd = pt.shape
    wide = np.empty((S, Wd + spare_cols), np.int32)
    wide[:, :Wd] = pt
    wide[:, Wd:] = np.random.default_rng(7).integers(1, num_pages, size=(S, spare_cols))
    return dev(wide)[:, :Wd]


def run_compress(K, case, layout, ratio, mode, fused=True, eps=None, max_out_rows=None,
                 out_loc=None, page_table="case", want_state=True, cache_fill=0xA5,
                 page_stride=None, tile_rows=0, pt_spare_cols=0, **extra):
    """run oracle and GPU on the same inputs; returns dict of both sides.
    ``extra``: draft_len, ring_slots and dcp_* arguments, passed to both.
    ``tile_rows`` (rows per prefill work item) goes to the GPU only.
    ``pt_spare_cols``: the GPU's page table is a column slice of a wider
    table whose extra columns hold valid pages (the slice's width, not its
    row stride, must bound the lookups)."""
    ps = case["page_size"]
    db, sb, rb, _ = oracle.layout_bytes(layout)
    eps = case["eps"] if eps is None else eps
    hc = np.full((case["num_pages"], page_stride or ps * rb), cache_fill, np.uint8)
    dc = dev(hc)
    state_h = case["state"].copy()
    state_d = dev(case["state"])
    pt = case["page_table"] if isinstance(page_table, str) else page_table
    start = case["start_pos"] if mode == oracle.PREFILL else case["pos"]
    kv = case["kv"]
    if fused:
        o_kw = dict(kv=kv, fused=True)
    else:
        o_kw = dict(kv=kv, score=case["score"], fused=False)
    lat_o, pre_o, st_o, n_rows = oracle.compress(
        ratio=ratio, mode=mode, offsets=case.get("offsets"), start_pos=start, page_table=pt,
        out_loc=out_loc, state=state_h, norm_w=case["norm_w"], eps=eps, freqs=case["freqs"],
        cache=hc, layout=layout, page_size=ps, max_out_rows=max_out_rows, **o_kw, **extra)
    nlat = lat_o.shape[0]
    lat = torch.zeros((max(nlat, 1), 512), dtype=torch.int16, device="cuda")
    pre = torch.zeros_like(lat)
    kvd = dev(kv)
    if fused:
        kv_v, sc_v = kvd[:, :512], kvd[:, 512:]
    else:
        kv_v = kvd
        sc_v = dev(case["score"]) if case["score"] is not None else None
    s = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvc_compress_store(
        ratio=ratio, mode=mode, kv=kv_v, score=sc_v if ratio == 2 else None,
        start_pos=dev(start), cache=K.Cache(dc, layout, ps), norm_w=dev(case["norm_w"]), eps=eps,
        freqs=dev(case["freqs"]), latent_out=lat, max_out_rows=nlat,
        offsets=None if case.get("offsets") is None or mode != oracle.PREFILL else dev(case["offsets"]),
        page_table=None if pt is None else _pt_view(pt, pt_spare_cols, case["num_pages"]),
        out_loc=None if out_loc is None else dev(out_loc),
        state=state_d if ratio == 2 else None, prequant_out=pre, status=s, tile_rows=tile_rows,
        **extra)
    torch.cuda.synchronize()
    return dict(lat_o=lat_o, pre_o=pre_o, st_o=st_o, n_rows=n_rows, cache_o=hc, state_o=state_h,
                lat_g=host(lat, np.uint16)[:nlat], pre_g=host(pre, np.uint16)[:nlat],
                st_g=int(s.item()), cache_g=host(dc), state_g=host(state_d, np.uint16),
                cache_fill=cache_fill)


def check_compress(r, layout, ps, touched_slots, emitted):
    """emitted: latent indices that carry rows; touched_slots: their slots
    (0 = none), same order."""
    assert r["st_g"] == r["st_o"], (r["st_g"], r["st_o"])
    em = np.asarray(emitted, np.int64)
    if em.size:
        assert_latent_close(r["lat_g"][em], r["lat_o"][em])
        assert_latent_close(r["pre_g"][em], r["pre_o"][em], "prequant")
    # untouched cache bytes identical (sentinel)
    slots = [s for s in touched_slots if s != 0]
    m = written_mask(r["cache_g"].shape, layout, ps, slots)
    assert np.array_equal(r["cache_g"][~m], r["cache_o"][~m])
    # the kernel's quantizer is bit-exact given its own pre-quant rows,
    # and the fused rows are within one code step of the oracle's
    idx = [i for i, s in zip(emitted, touched_slots) if s != 0]
    if idx:
        gd = np.stack([row_parts(r["cache_g"], layout, ps, s)[0] for s in slots])
        gs = np.stack([row_parts(r["cache_g"], layout, ps, s)[1] for s in slots])
        od = np.stack([row_parts(r["cache_o"], layout, ps, s)[0] for s in slots])
        os_ = np.stack([row_parts(r["cache_o"], layout, ps, s)[1] for s in slots])
        qd, qs = oracle.store_row(layout, r["pre_g"][idx])
        assert np.array_equal(qd, gd) and np.array_equal(qs, gs), "quantizer not bit-exact"
        assert_rows_close(layout, gd, gs, od, os_, spec.bf16_value(r["pre_o"][idx]))
    # pending state: an exact copy
    assert np.array_equal(r["state_g"], r["state_o"])


