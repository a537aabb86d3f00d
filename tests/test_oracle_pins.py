"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU.  Each test checks the oracle against something other than itself:
the byte counts and the exponent formula printed on the pages, format grids
rebuilt from their bit fields with a nearest-value search, closed forms,
invariants and a differently written fp64 pipeline on tiny inputs.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from tests import spec

LAYOUTS = ["V4", "V41", "V41_FP4"]


@pytest.fixture(scope="module", autouse=True)
def _built():
    from oracle import build
    if not __import__("os").path.exists(oracle._LIB_PATH):
        build.build()


# --------------------------------------------------------------- layout bytes
def test_layout_bytes_match_pages():
    """584 / 528 / 288 bytes per token (sglang PR #39652, Summary) and the
    split they come from: bits per dim over 512 dims plus one byte per group."""
    assert oracle.layout_bytes("V4")[2] == 584
    assert oracle.layout_bytes("V41")[2] == 528
    assert oracle.layout_bytes("V41_FP4")[2] == 288
    # V41: 512 fp8 + one scale per 32;  FP4: 512 x 4 bit + one scale per 16
    assert oracle.layout_bytes("V41") == (512 * 8 // 8, 512 // 32, 528, 32)
    assert oracle.layout_bytes("V41_FP4") == (512 * 4 // 8, 512 // 16, 288, 16)
    # V4: 448 fp8 nope + 64 bf16 rope in the data part; 7 ue8m0 + 1 pad
    assert oracle.layout_bytes("V4") == (448 + 64 * 2, 448 // 64 + 1, 584, 64)


# --------------------------------------------------------------- ue8m0
def test_ue8m0_closed_form_all_bf16():
    """The pages' closed form equals the definition on every positive finite
    bf16 amax (sglang PR #39652, Review: exhaustive over bf16, 0 mismatches)."""
    b = spec.all_bf16()
    b = b[(b & 0x8000) == 0]
    amax = spec.bf16_value(b).astype(np.float32)
    got = oracle.ue8m0(amax)
    ref = spec.closed_form_ue8m0(amax)
    assert np.array_equal(got, ref)
    assert got.min() == 114 and got.max() == 247


def test_ue8m0_closed_form_fp32_samples_and_boundaries():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 0x7F800000, size=2_000_000, dtype=np.uint32)
    amax = bits.view(np.float32)
    assert np.array_equal(oracle.ue8m0(amax), spec.closed_form_ue8m0(amax))
    # +-64 ulp around every finite 448 * 2^k, zero and denormals
    near = []
    for k in range(-160, 120):
        c = np.float32(448.0 * 2.0 ** k)
        if not np.isfinite(c) or c == 0:
            continue
        cb = np.array([c], np.float32).view(np.uint32)[0].astype(np.int64)
        near.append(np.arange(max(cb - 64, 0), min(cb + 65, 0x7F800000), dtype=np.int64))
    near = np.concatenate(near).astype(np.uint32).view(np.float32)
    assert np.array_equal(oracle.ue8m0(near), spec.closed_form_ue8m0(near))
    den = np.arange(0, 1 << 16, dtype=np.uint32).view(np.float32)
    assert np.all(oracle.ue8m0(den) == 114)


def test_ue8m0_closed_form_every_positive_fp32():
    """The closed form against the oracle's definition (the smallest k >= -13
    with 448 * 2^k >= amax) on every positive finite fp32 amax, 2^31 - 2^23
    values in chunks (small enough to reuse warm memory)."""
    step = 1 << 20
    for lo in range(0, 0x7F800000, step):
        amax = np.arange(lo, min(lo + step, 0x7F800000), dtype=np.uint32).view(np.float32)
        got = oracle.ue8m0(amax)
        ref = spec.closed_form_ue8m0(amax)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (hex(lo + int(bad[0])), int(got[bad[0]]), int(ref[bad[0]]))


def test_ue8m0_against_log2_formula():
    """Against ceil(log2(max(amax/448, 1e-4))) evaluated by math.log2 on
    values away from exact powers of two, and hand-worked values."""
    assert list(oracle.ue8m0([0.0, 1.0, 448.0, 448.0001, 896.0, 896.1, 0.0448])) == [
        114, 127 + math.ceil(math.log2(1 / 448)), 127, 128, 128, 129,
        127 + math.ceil(math.log2(0.0448 / 448))]
    rng = np.random.default_rng(3)
    a = np.exp(rng.uniform(-20, 80, size=20000)).astype(np.float32)
    ref = np.array([127 + math.ceil(math.log2(max(float(x) / 448.0, 1e-4))) for x in a])
    assert np.array_equal(oracle.ue8m0(a), ref)


def _golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_golden_layout_bytes():
    for lay, total, qd, bits, grp, keep in _golden("layout_bytes.txt"):
        db, sb, rb, g = oracle.layout_bytes(lay)
        assert rb == int(total)
        assert g == int(grp)
        assert db == int(qd) * int(bits) // 8 + int(keep) * 2
        assert sb >= int(qd) // int(grp)


def test_golden_ue8m0_points():
    rows = _golden("ue8m0_points.txt")
    amax = np.array([float(a) for a, _ in rows], np.float32)
    want = np.array([int(e) for _, e in rows])
    assert np.array_equal(oracle.ue8m0(amax), want)


# --------------------------------------------------------------- fp8 e4m3
def test_e4m3_decode_matches_field_definition():
    t = spec.e4m3_table()
    got = oracle.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(got[ok], t[ok])
    assert t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x38] == 1.0


def test_e4m3_encode_round_trip_and_ties():
    t = spec.e4m3_table()
    finite = np.array([c for c in range(256) if not np.isnan(t[c])])
    assert np.array_equal(oracle.e4m3_encode(t[finite]), finite.astype(np.uint8))
    # ties go to the even mantissa; -0 keeps its sign; overflow rules
    assert list(oracle.e4m3_encode([2 ** -10, 3 * 2 ** -10, 1.0625, 1.1875, -0.0, -2 ** -11])) == [
        0x00, 0x02, 0x38, 0x3A, 0x80, 0x80]
    assert oracle.e4m3_encode([464.0], True)[0] == 0x7E
    assert oracle.e4m3_encode([500.0], True)[0] == 0x7E
    assert oracle.e4m3_encode([500.0], False)[0] == 0x7F


def test_fp8_code_exhaustive_vs_nearest_search():
    """fp8 code of every bf16 element under every exponent the quantizer can
    pick for it, against a nearest-grid search."""
    b = spec.all_bf16()
    x = spec.bf16_value(b)
    for E in range(114, 248):
        y = x * 2.0 ** (127 - E)
        ok = np.abs(y) <= 448.0
        got = oracle.fp8_code(b[ok], E)
        ref = spec.e4m3_nearest(y[ok])
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (E, b[ok][bad[:5]], got[bad[:5]], ref[bad[:5]])


# --------------------------------------------------------------- fp4 e2m1
def test_e2m1_decode_and_ties():
    t = spec.e2m1_table()
    assert np.array_equal(oracle.e2m1_decode(np.arange(16)), t)
    assert list(t[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert list(oracle.e2m1_encode(ties)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(oracle.e2m1_encode([7.0, 100.0, -100.0, -0.0, -0.2])) == [7, 7, 15, 8, 8]
    v = np.linspace(-8, 8, 100001)
    assert np.array_equal(oracle.e2m1_encode(v), spec.e2m1_nearest(v))


def test_fp4_scale_vs_exact_quotient():
    """The e4m3 scale taken from amax/6 in fp32 equals the nearest e4m3 value
    (clamped at 448) to the exact quotient, for every positive bf16 amax."""
    b = spec.all_bf16()
    b = b[(b & 0x8000) == 0]
    amax = spec.bf16_value(b)
    got = oracle.fp4_scale(amax.astype(np.float32))
    ref = spec.e4m3_nearest(amax / 6.0)
    assert np.array_equal(got, ref)


def test_fp4_code_exhaustive_vs_nearest_search():
    """e2m1 code of every bf16 element under every finite positive e4m3
    scale: fp32 division then rounding equals the nearest grid point of
    x / s found by exact search (products g*s are exact in fp64)."""
    b = spec.all_bf16()
    x = spec.bf16_value(b)
    t4 = spec.e2m1_table()[:8]
    t8 = spec.e4m3_table()
    for sc in range(1, 0x7F):
        s = t8[sc]
        got = oracle.fp4_code(b, sc)
        d = np.abs(np.abs(x)[:, None] - t4[None, :] * s)
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        # ties: the even code (lowest bit 0) among the nearest
        even = cand & ((np.arange(8) & 1) == 0)[None, :]
        code = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
        # beyond 6 s every grid point lies below |x| and the top one is nearest
        # (the fp64 differences would all round to |x| there)
        code = np.where(np.abs(x) >= 6 * s, 7, code)
        ref = (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (sc, b[bad[:5]], got[bad[:5]], ref[bad[:5]])
    assert np.all(oracle.fp4_code(b[:100], 0) == 0)


# --------------------------------------------------------------- bf16
def test_bf16_encode_vs_nearest_and_torch():
    import torch
    rng = np.random.default_rng(11)
    f = (rng.standard_normal(200000) * np.exp(rng.uniform(-90, 87, 200000))).astype(np.float32)
    f = np.concatenate([f, np.array([0.0, -0.0, 1e-45, 3.3e38, 3.4e38, -3.39e38], np.float32)])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_encode(f.astype(np.float64)), want)
    assert oracle.bf16_encode([2.0 ** 128])[0] == 0x7F80
    assert oracle.bf16_encode([(2 - 2 ** -8) * 2.0 ** 127])[0] == 0x7F80   # tie rounds up to inf
    assert oracle.bf16_encode([2.0 ** -134])[0] == 0x0000                  # half of min subnormal
    assert oracle.bf16_encode([3 * 2.0 ** -134])[0] == 0x0002


# --------------------------------------------------------------- rows
def _rows(seed=5, n=2048):
    rng = np.random.default_rng(seed)
    return W.outlier_rows(rng, n)


def test_zero_row_encoding():
    z = np.zeros((1, 512), np.uint16)
    for lay in ("V41", "V4"):
        d, s = oracle.store_row(lay, z)
        assert np.all(d[:, :448] == 0)
        assert np.all(s[:, : (16 if lay == "V41" else 7)] == 114)
    d, s = oracle.store_row("V41_FP4", z)
    assert np.all(d == 0) and np.all(s == 0)


@pytest.mark.parametrize("layout", ["V41", "V4"])
def test_fp8_round_trip_error_bound(layout):
    """|x - dq(q(x))| <= 2^-4 |x| in the fp8 normal range and <= 2^-10 s in
    the subnormal range (3 mantissa bits, spacing 2^-9 s below 2^-6 s)."""
    x = _rows()
    d, s = oracle.store_row(layout, x)
    y = spec.bf16_value(oracle.dequant_row(layout, d, s))
    xv = spec.bf16_value(x)
    nd = 512 if layout == "V41" else 448
    g = 32 if layout == "V41" else 64
    sc = 2.0 ** (s[:, : nd // g].astype(np.float64) - 127)
    sc = np.repeat(sc, g, axis=1)
    err = np.abs(xv[:, :nd] - y[:, :nd])
    normal = np.abs(xv[:, :nd]) / sc >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xv[:, :nd][normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * sc[~normal])
    if layout == "V4":
        assert np.array_equal(oracle.dequant_row(layout, d, s)[:, 448:], x[:, 448:])
        assert np.all(s[:, 7] == 0)


def test_v41_idempotent_and_code_reconstruction():
    # power-of-two scales: re-quantizing a dequantized row gives back the
    # same values (codes may move to a smaller exponent when the group's top
    # value rounded down onto 224 s)
    x = _rows(6)
    d, s = oracle.store_row("V41", x)
    y = oracle.dequant_row("V41", d, s)
    d2, s2 = oracle.store_row("V41", y)
    assert np.array_equal(oracle.dequant_row("V41", d2, s2), y)
    assert np.all((s2 == s) | (s2 == s - 1))
    # rows built from chosen codes with a group maximum in (224, 448] come back
    rng = np.random.default_rng(9)
    t = spec.e4m3_table()
    codes = rng.integers(0, 0x7F, size=(64, 512)).astype(np.uint8)
    codes[:, ::32] = rng.integers(0x77, 0x7F, size=(64, 16))   # 240..448 in each group
    codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    E = rng.integers(114, 200, size=(64, 16)).astype(np.uint8)
    vals = t[codes] * 2.0 ** (np.repeat(E, 32, axis=1).astype(np.float64) - 127)
    xb = oracle.bf16_encode(vals)
    d3, s3 = oracle.store_row("V41", xb)
    assert np.array_equal(s3, E) and np.array_equal(d3, codes)


def test_fp4_round_trip_bound():
    x = _rows(8)
    d, s = oracle.store_row("V41_FP4", x)
    y = spec.bf16_value(oracle.dequant_row("V41_FP4", d, s))
    xv = spec.bf16_value(x)
    sv = np.repeat(spec.e4m3_table()[s], 16, axis=1)
    q = np.abs(xv) / np.where(sv == 0, 1, sv)
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    sat = q > 6
    err = np.abs(xv - y)
    ok = (~sat) & (sv > 0)
    assert np.all(err[ok] <= 0.5 * step[ok] * sv[ok] * (1 + 1e-12))
    # dequant is the product of the two decoded values, exactly
    t4 = spec.e2m1_table()
    lo, hi = d & 0xF, d >> 4
    q4 = np.empty((d.shape[0], 512), np.uint8)
    q4[:, 0::2], q4[:, 1::2] = lo, hi
    assert np.array_equal(y, t4[q4] * sv)


def test_dequant_nan_conventions():
    d = np.zeros((1, 512), np.uint8)
    s = np.full((1, 16), 127, np.uint8)
    d[0, 0], d[0, 1] = 0x7F, 0xFF
    s[0, 1] = 255
    y = spec.bf16_value(oracle.dequant_row("V41", d, s))
    assert np.isnan(y[0, 0]) and np.isnan(y[0, 1]) and np.all(np.isnan(y[0, 32:64]))
    assert np.all(y[0, 2:32] == 0)


# --------------------------------------------------------------- paged cache
def _decode_cache_rows(cache, layout, page_size):
    """every row of a cache, dequantized with numpy from the format tables."""
    db, sb, rb, g = oracle.layout_bytes(layout)
    P = cache.shape[0]
    data = cache[:, : page_size * db].reshape(P * page_size, db)
    scale = cache[:, page_size * db: page_size * db + page_size * sb].reshape(P * page_size, sb)
    t8, t4 = spec.e4m3_table(), spec.e2m1_table()
    if layout == "V41":
        v = t8[data] * 2.0 ** (np.repeat(scale, 32, axis=1).astype(np.float64) - 127)
    elif layout == "V41_FP4":
        q = np.empty((data.shape[0], 512), np.uint8)
        q[:, 0::2], q[:, 1::2] = data & 0xF, data >> 4
        v = t4[q] * np.repeat(t8[scale], 16, axis=1)
    else:
        v = np.empty((data.shape[0], 512))
        v[:, :448] = t8[data[:, :448]] * 2.0 ** (np.repeat(scale[:, :7], 64, axis=1).astype(np.float64) - 127)
        v[:, 448:] = spec.bf16_value(data[:, 448:].copy().view(np.uint16))
    import torch
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gather_is_index_select_of_dequantized_cache(layout):
    db, sb, rb, g = oracle.layout_bytes(layout)
    ps = 16
    c = W.gather_case(123, 12, ps, 150, rb, db, sb,
                      scale_lo=(114 if layout != "V41_FP4" else None),
                      scale_hi=140)
    cache = c["cache"]
    full = _decode_cache_rows(cache, layout, ps)
    ids = c["ids"].copy()
    ids[::17] = -1
    got, st = oracle.dequant_gather(cache, layout, ps, c["page_table"], ids)
    assert st == 0
    pt = c["page_table"]
    slot = pt[np.maximum(ids, 0) // ps] * ps + np.maximum(ids, 0) % ps
    want = np.where((ids >= 0)[:, None], full[slot], 0)
    assert np.array_equal(got, want)
    # physical-slot ids (no page table) and out-of-range ids
    ids2 = np.array([ps * 3 + 1, ps * 13, -5, ps * 13 + 2], np.int32)
    got2, st2 = oracle.dequant_gather(cache, layout, ps, None, ids2)
    assert np.array_equal(got2[0], full[ps * 3 + 1]) and np.all(got2[1:] == 0)
    assert st2 == oracle.ST_ID_RANGE
    pt_bad = pt.copy()
    pt_bad[0] = 99
    _, st3 = oracle.dequant_gather(cache, layout, ps, pt_bad, np.array([0, 1], np.int32))
    assert st3 == oracle.ST_PAGE_RANGE


@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_rows_writes_exactly_the_slots(layout):
    db, sb, rb, g = oracle.layout_bytes(layout)
    c = W.store_case(77, [40, 3, 70], page_size=16)
    rows, out_loc = c["rows"], c["out_loc"].copy()
    out_loc[5] = 0                                   # a padded row
    cache = np.full((c["num_pages"], 16 * rb), 0xA5, np.uint8)
    st = oracle.store_rows(cache, layout, 16, rows, out_loc)
    assert st == 0
    d, s = oracle.store_row(layout, rows)
    touched = np.zeros(cache.shape, bool)
    for i, loc in enumerate(out_loc):
        if loc == 0:
            continue
        p, r = divmod(int(loc), 16)
        assert np.array_equal(cache[p, r * db:(r + 1) * db], d[i])
        assert np.array_equal(cache[p, 16 * db + r * sb: 16 * db + (r + 1) * sb], s[i])
        touched[p, r * db:(r + 1) * db] = True
        touched[p, 16 * db + r * sb: 16 * db + (r + 1) * sb] = True
    assert np.all(cache[~touched] == 0xA5)
    st = oracle.store_rows(cache, layout, 16, rows[:1], np.array([c["num_pages"] * 16], np.int32))
    assert st == oracle.ST_PAGE_RANGE


# --------------------------------------------------------------- compressor
def _plan(lengths, P, ratio):
    """Brute-force row plan: (slot, c, p, token_a, token_b) where token_a is
    -1 for the pending state, plus the list of tail tokens."""
    rows, tails, first = [], [], 0
    for b, (n, p0) in enumerate(zip(lengths, P)):
        toks = list(range(first, first + n))
        poss = list(range(p0, p0 + n))
        if ratio == 1:
            rows += [(b, q, q, None, t) for q, t in zip(poss, toks)]
        else:
            for i, q in enumerate(poss):
                if q % 2 == 1:
                    a = toks[i - 1] if i > 0 else -1
                    rows.append((b, q // 2, q - 1, a, toks[i]))
            if n > 0 and poss[-1] % 2 == 0:
                tails.append((b, toks[-1]))
        first += n
    return rows, tails


@pytest.mark.parametrize("ratio,eps", [(1, None), (2, None), (2, 0.5)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_compress_prefill_against_spec(ratio, layout, eps):
    lengths = [7, 0, 12, 1, 33]
    P = [0, 0, 3, 4, 9]                              # odd prefixes included
    case = W.compress_case(31 + ratio, lengths, start_pos=P, ratio=ratio, page_size=4,
                           fused=True)
    if eps is not None:                              # large enough to show in bf16
        case["eps"] = eps
    db, sb, rb, g = oracle.layout_bytes(layout)
    cache = np.full((case["num_pages"], 4 * rb), 0x5A, np.uint8)
    state0 = case["state"].copy()
    state = case["state"].copy()
    lat, pre, st, n_rows = oracle.compress(
        ratio=ratio, mode=oracle.PREFILL, kv=case["kv"], fused=True, offsets=case["offsets"],
        start_pos=case["start_pos"], page_table=case["page_table"], state=state,
        norm_w=case["norm_w"], eps=case["eps"], freqs=case["freqs"], cache=cache,
        layout=layout, page_size=4)
    assert st == 0
    rows, tails = _plan(lengths, P, ratio)
    assert n_rows == len(rows)
    kv, sc = case["kv"][:, :512], case["kv"][:, 512:]
    for i, (b, c, p, ta, tb) in enumerate(rows):
        if ta is None:
            k0 = s0 = None
        elif ta < 0:
            k0, s0 = state0[b, 0], state0[b, 1]
        else:
            k0, s0 = kv[ta], sc[ta]
        y, z = spec.pool_norm_rope(k0, s0, kv[tb], sc[tb], case["norm_w"], case["eps"],
                                   case["freqs"][p])
        ly, lz = spec.bf16_value(lat[i]), spec.bf16_value(pre[i])
        assert np.all(np.abs(ly - y) <= 0.5 * spec.bf16_ulp(y) * (1 + 1e-9) + 1e-300), i
        assert np.all(np.abs(lz - z) <= 0.5 * spec.bf16_ulp(z) * (1 + 1e-9) + 1e-300), i
        # cache row at the slot the page table gives; bytes = store_row(prequant)
        phys = case["page_table"][b, c // 4]
        d, s = oracle.store_row(layout, pre[i])
        r = c % 4
        assert np.array_equal(cache[phys, r * db:(r + 1) * db], d[0])
        assert np.array_equal(cache[phys, 4 * db + r * sb:4 * db + (r + 1) * sb], s[0])
    # every other cache byte untouched
    written = sum(1 for _ in rows)
    assert (cache != 0x5A).sum() <= written * rb
    # pending state: tails written, others unchanged
    tail_slots = {b for b, _ in tails}
    for b, t in tails:
        assert np.array_equal(state[b, 0], kv[t]) and np.array_equal(state[b, 1], sc[t])
    for b in range(len(lengths)):
        if b not in tail_slots:
            assert np.array_equal(state[b], state0[b])


def test_compress_decode_explicit_out_loc():
    case = W.decode_case(41, 64, ratio=2, page_size=16, max_pos=300)
    db, sb, rb, g = oracle.layout_bytes("V4")
    cache = np.full((case["num_pages"], 16 * rb), 0x11, np.uint8)
    state0 = case["state"].copy()
    state = case["state"].copy()
    lat, pre, st, n_rows = oracle.compress(
        ratio=2, mode=oracle.DECODE, kv=case["kv"], fused=True, start_pos=case["pos"],
        out_loc=case["out_loc"], state=state, norm_w=case["norm_w"], eps=case["eps"],
        freqs=case["freqs"], cache=cache, layout="V4", page_size=16)
    assert st == 0
    pos = case["pos"]
    kv, sc = case["kv"][:, :512], case["kv"][:, 512:]
    for b in range(64):
        if pos[b] % 2 == 1:
            y, z = spec.pool_norm_rope(state0[b, 0], state0[b, 1], kv[b], sc[b],
                                       case["norm_w"], case["eps"], case["freqs"][pos[b] - 1])
            ly = spec.bf16_value(lat[b])
            assert np.all(np.abs(ly - y) <= 0.5 * spec.bf16_ulp(y) * (1 + 1e-9))
            p, r = divmod(int(case["out_loc"][b]), 16)
            d, s = oracle.store_row("V4", pre[b])
            assert np.array_equal(cache[p, r * db:(r + 1) * db], d[0])
            assert np.array_equal(state[b], state0[b])
        else:
            assert case["out_loc"][b] == 0 and np.all(lat[b] == 0)
            assert np.array_equal(state[b, 0], kv[b]) and np.array_equal(state[b, 1], sc[b])


def test_pooling_special_cases_and_norm_rope_properties():
    rng = np.random.default_rng(4)
    k0, k1 = W.normal_bf16(rng, (2, 512))
    s = W.normal_bf16(rng, 512)
    w1 = W.bf16_bits(np.ones(512, np.float32))
    freqs = W.rope_freqs(8)
    base = dict(ratio=2, mode=oracle.PREFILL, fused=True, offsets=np.array([[0], [2]], np.int32),
                start_pos=np.array([0], np.int32), page_table=np.array([[1]], np.int32),
                norm_w=w1, eps=0.0, freqs=freqs, layout="V41", page_size=64)

    def run(kv0, sc0, kv1, sc1, **kw):
        a = dict(base)
        a.update(kw)
        proj = np.stack([np.concatenate([kv0, sc0]), np.concatenate([kv1, sc1])])
        cache = np.zeros((2, 64 * 528), np.uint8)
        st = np.zeros((1, 2, 512), np.uint16)
        lat, pre, status, n = oracle.compress(kv=proj, state=st, cache=cache, **a)
        return spec.bf16_value(lat[0]), spec.bf16_value(pre[0])

    # equal scores: plain mean; normalised with w = 1 -> unit RMS
    y, z = run(k0, s, k1, s)
    v = (spec.bf16_value(k0) + spec.bf16_value(k1)) / 2
    assert np.allclose(y, v / np.sqrt(np.mean(v * v)), rtol=2 ** -8, atol=0)
    assert abs(np.sqrt(np.mean(y * y)) - 1) < 1e-2
    # position 0: rotation by the identity, z == y
    assert np.array_equal(y, z)
    # a score far larger on the first token selects it
    big = W.bf16_bits(np.full(512, 80.0, np.float32))
    small = W.bf16_bits(np.full(512, -80.0, np.float32))
    y2, _ = run(k0, big, k1, small)
    v0 = spec.bf16_value(k0)
    assert np.allclose(y2, v0 / np.sqrt(np.mean(v0 * v0)), rtol=2 ** -8)
    # rotation keeps each rope pair's norm (position 2 of the second pair)
    a = dict(base)
    a["offsets"] = np.array([[0], [4]], np.int32)
    proj = np.stack([np.concatenate([k0, s]), np.concatenate([k1, s])] * 2)
    cache = np.zeros((2, 64 * 528), np.uint8)
    lat, pre, _, n = oracle.compress(kv=proj, state=np.zeros((1, 2, 512), np.uint16),
                                     cache=cache, **a)
    assert n == 2
    y, z = spec.bf16_value(lat[1]), spec.bf16_value(pre[1])
    ny = np.hypot(y[448::2], y[449::2])
    nz = np.hypot(z[448::2], z[449::2])
    assert np.allclose(ny, nz, rtol=2 ** -7)
    assert not np.array_equal(y[448:], z[448:])


def test_eps_perturbation_changes_output():
    """Negative control: a 1% change of eps must change the outputs."""
    case = W.compress_case(55, [16], ratio=2, page_size=16, fused=True)
    outs = []
    for eps in (1e-2, 1.01e-2):
        cache = np.zeros((case["num_pages"], 16 * 288), np.uint8)
        lat, pre, st, n = oracle.compress(
            ratio=2, mode=oracle.PREFILL, kv=case["kv"], fused=True, offsets=case["offsets"],
            start_pos=case["start_pos"], page_table=case["page_table"],
            state=case["state"].copy(), norm_w=case["norm_w"], eps=eps, freqs=case["freqs"],
            cache=cache, layout="V41_FP4", page_size=16)
        outs.append((lat.copy(), cache.copy()))
    assert not np.array_equal(outs[0][0], outs[1][0])
    assert not np.array_equal(outs[0][1], outs[1][1])


def test_compress_status_bits():
    case = W.compress_case(56, [10], ratio=2, page_size=4, fused=True, pt_slack=0)
    cache = np.zeros((case["num_pages"], 4 * 528), np.uint8)
    pt = case["page_table"].copy()
    pt[0, 1] = 10_000                                 # physical page outside the cache
    _, _, st, _ = oracle.compress(
        ratio=2, mode=oracle.PREFILL, kv=case["kv"], fused=True, offsets=case["offsets"],
        start_pos=case["start_pos"], page_table=pt, state=case["state"].copy(),
        norm_w=case["norm_w"], eps=1e-6, freqs=case["freqs"], cache=cache, layout="V41",
        page_size=4, max_out_rows=3)
    assert st == oracle.ST_PAGE_RANGE | oracle.ST_LATENT_RANGE
    # rows 4.. need a second page-table entry that is not there
    _, _, st, _ = oracle.compress(
        ratio=2, mode=oracle.PREFILL, kv=case["kv"], fused=True, offsets=case["offsets"],
        start_pos=case["start_pos"], page_table=case["page_table"][:, :1].copy(),
        state=case["state"].copy(), norm_w=case["norm_w"], eps=1e-6, freqs=case["freqs"],
        cache=cache, layout="V41", page_size=4)
    assert st == oracle.ST_PT_RANGE
    # rotary positions 4, 6, 8 lie outside a 4-entry table: rows skipped
    lat, _, st, _ = oracle.compress(
        ratio=2, mode=oracle.PREFILL, kv=case["kv"], fused=True, offsets=case["offsets"],
        start_pos=case["start_pos"], page_table=case["page_table"],
        state=case["state"].copy(), norm_w=case["norm_w"], eps=1e-6, freqs=case["freqs"][:4],
        cache=cache, layout="V41", page_size=4)
    assert st == oracle.ST_POS_RANGE
    assert np.all(lat[2:] == 0) and np.any(lat[:2] != 0)
