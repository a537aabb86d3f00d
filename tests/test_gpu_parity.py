"""HIP path vs the CPU oracle, through the C ABI (``fp8_fp4_quantized_amd``).

Bar: bit-exact for quantized bytes (store, and the fused kernel's quantizer
applied to its own pre-quant rows), dequantized values, pending state and
untouched cache bytes; 2e-2 relative (codes within one step) for the fused
compressor's outputs against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import spec
from tests.gpu_util import (assert_latent_close, assert_rows_close, check_compress, dev, host,
                            row_parts, run_compress, sha, written_mask)

pytestmark = pytest.mark.gpu

LAYOUTS = ["V4", "V41", "V41_FP4"]


@pytest.fixture(scope="module")
def K():
    import fp8_fp4_quantized_amd as k
    return k


def _say(*a):
    print("[case]", *a, flush=True)


def _status():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _cache_pair(num_pages, page_size, layout, fill=0xA5):
    db, sb, rb, _ = oracle.layout_bytes(layout)
    host_c = np.full((num_pages, page_size * rb), fill, np.uint8)
    return host_c, dev(host_c)


# ===================================================================== decode
def test_fp8_dequant_all_codes_all_exponents(K):
    """every e4m3fn code under every ue8m0 byte (0..255), V41 rows."""
    _say("fp8 dequant exhaustive")
    ps = 16
    codes = np.tile(np.arange(256, dtype=np.uint8), 256)           # per E: 256 codes
    E = np.repeat(np.arange(256, dtype=np.uint8), 8)                # 8 groups of 32 per E
    rows = codes.size // 512                                        # 128 rows
    data = codes.reshape(rows, 512)
    scale = E.reshape(rows, 16)
    npages = rows // ps + 1
    cache = np.zeros((npages, ps * 528), np.uint8)
    for i in range(rows):
        p, r = divmod(i + ps, ps)                                   # skip page 0
        cache[p, r * 512:(r + 1) * 512] = data[i]
        cache[p, ps * 512 + r * 16: ps * 512 + (r + 1) * 16] = scale[i]
    ids = np.arange(ps, ps + rows, dtype=np.int32)
    want, _ = oracle.dequant_gather(cache, "V41", ps, None, ids)
    out = torch.zeros((rows, 512), dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(cache), "V41", ps), None, dev(ids), out)
    got = host(out, np.uint16)
    gv, wv = spec.bf16_value(got), spec.bf16_value(want)
    nan = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_fp4_dequant_all_codes_all_scales(K):
    _say("fp4 dequant exhaustive")
    ps = 8
    nib = np.tile(np.arange(16, dtype=np.uint8), 256)              # per scale: 16 codes
    data = (nib[0::2] | (nib[1::2] << 4)).reshape(8, 256)
    scale = np.arange(256, dtype=np.uint8).reshape(8, 32)
    cache = np.zeros((2, ps * 288), np.uint8)
    for i in range(8):
        cache[1, i * 256:(i + 1) * 256] = data[i]
        cache[1, ps * 256 + i * 32: ps * 256 + (i + 1) * 32] = scale[i]
    ids = np.arange(ps, 2 * ps, dtype=np.int32)
    want, _ = oracle.dequant_gather(cache, "V41_FP4", ps, None, ids)
    out = torch.zeros((8, 512), dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(cache), "V41_FP4", ps), None, dev(ids), out)
    got = host(out, np.uint16)
    gv, wv = spec.bf16_value(got), spec.bf16_value(want)
    nan = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ===================================================================== store
@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_rows_c2(K, layout):
    """Ratio-1 store of 8 requests (extend lengths in [512, 4096], outlier
    rows, 1% zero rows), page 64: bit-exact cache image; then the dequant of
    every stored row by its physical slot (no page table): bit-exact bf16."""
    _say("store C2", layout)
    c = W.workload_c2()
    rows, out_loc = c["rows"], c["out_loc"].copy()
    out_loc[3] = 0                                    # a padded row
    hc, dc = _cache_pair(c["num_pages"], 64, layout)
    st = oracle.store_rows(hc, layout, 64, rows, out_loc)
    s = _status()
    cache = K.Cache(dc, layout, 64)
    K.kvc_store_rows(cache, dev(rows), dev(out_loc), s)
    got = host(dc)
    assert st == 0 and int(s.item()) == 0
    assert sha(got) == sha(hc), np.argwhere(got != hc)[:5]
    # dequant by slot; the padded row's id is -1 (a zero row)
    ids = np.where(out_loc == 0, -1, out_loc).astype(np.int32)
    want, gst = oracle.dequant_gather(hc, layout, 64, None, ids)
    out = torch.empty((ids.size, 512), dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(cache, None, dev(ids), out, s)
    assert gst == 0 and int(s.item()) == 0
    assert sha(host(out).view(np.uint16)) == sha(want)


def test_store_rows_status_and_stride(K):
    _say("store status")
    rng = np.random.default_rng(1)
    rows = W.outlier_rows(rng, 10)
    wide = np.zeros((10, 768), np.uint16)
    wide[:, :512] = rows
    loc = np.array([65, 66, 0, 10 ** 6, -3, 67, 68, 69, 70, 71], np.int32)
    hc, dc = _cache_pair(3, 64, "V41")
    st = oracle.store_rows(hc, "V41", 64, rows, loc)
    s = _status()
    K.kvc_store_rows(K.Cache(dc, "V41", 64), dev(wide)[:, :512], dev(loc), s)
    assert int(s.item()) == st == K.STATUS_PAGE_RANGE
    assert np.array_equal(host(dc), hc)


# ===================================================================== gather
@pytest.mark.parametrize("layout", LAYOUTS)
def test_gather_c4_full(K, layout):
    """cache of 1,048,576 rows (16384 pages x 64, random page table),
    262,144 distinct ids -> bf16 [262144, 512]: bit-exact, every row.  V41
    is the bench's C4; V4 and V41_FP4 are the same shape in their layouts."""
    _say("gather C4 full", layout)
    if layout == "V41":
        c = W.workload_c4()
    else:
        db, sb, rb, _ = oracle.layout_bytes(layout)
        c = W.gather_case(W.BASE_SEED + 4, 16384, 64, 262144, rb, db, sb,
                          scale_lo=None if layout == "V41_FP4" else 114, scale_hi=140)
    ids = c["ids"]
    want, st = oracle.dequant_gather(c["cache"], layout, 64, c["page_table"], ids)
    out = torch.empty((ids.size, 512), dtype=torch.int16, device="cuda")
    s = _status()
    dc = dev(c["cache"])
    K.kvc_dequant_gather(K.Cache(dc, layout, 64), dev(c["page_table"]), dev(ids), out, s)
    got = host(out, np.uint16)
    del dc
    assert st == 0 and int(s.item()) == 0
    assert sha(got) == sha(want)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gather_small_all_layouts(K, layout):
    """random valid codes (scales random too for FP4), ragged id count,
    negative ids, physical-slot mode, out-of-range ids and pages."""
    _say("gather small", layout)
    db, sb, rb, _ = oracle.layout_bytes(layout)
    ps = 32
    c = W.gather_case(99, 40, ps, 1001, rb, db, sb,
                      scale_lo=None if layout == "V41_FP4" else 100,
                      scale_hi=160)
    ids = c["ids"].copy()
    ids[::13] = -1
    dcache = K.Cache(dev(c["cache"]), layout, ps)
    want, st = oracle.dequant_gather(c["cache"], layout, ps, c["page_table"], ids)
    out = torch.full((ids.size, 512), 7, dtype=torch.int16, device="cuda")
    s = _status()
    K.kvc_dequant_gather(dcache, dev(c["page_table"]), dev(ids), out, s)
    got = host(out, np.uint16)
    gv, wv = spec.bf16_value(got), spec.bf16_value(want)
    nan = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), nan) and np.array_equal(got[~nan], want[~nan])
    assert int(s.item()) == st == 0
    # physical slots, strided output, bad ids
    ids2 = np.array([ps + 3, 41 * ps, -7, 5 * ps + 1, 2 ** 30], np.int32)
    want2, st2 = oracle.dequant_gather(c["cache"], layout, ps, None, ids2)
    out2 = torch.full((5, 640), 7, dtype=torch.int16, device="cuda")
    s2 = _status()
    K.kvc_dequant_gather(dcache, None, dev(ids2), out2[:, :512], s2)
    g2 = host(out2, np.uint16)
    assert np.array_equal(g2[:, :512], want2) and np.all(g2[:, 512:] == 7)
    assert int(s2.item()) == st2 == K.STATUS_ID_RANGE
    pt = c["page_table"].copy()
    pt[1] = 10 ** 6
    ids3 = np.array([ps + 1, 2, 10 ** 6], np.int32)
    want3, st3 = oracle.dequant_gather(c["cache"], layout, ps, pt, ids3)
    out3 = torch.full((3, 512), 7, dtype=torch.int16, device="cuda")
    s3 = _status()
    K.kvc_dequant_gather(dcache, dev(pt), dev(ids3), out3, s3)
    assert np.array_equal(host(out3, np.uint16), want3)
    assert int(s3.item()) == st3 == K.STATUS_PAGE_RANGE | K.STATUS_ID_RANGE


def test_gather_reuse_head(K):
    """A reused dequant equals a fresh one and launches nothing (sglang PR
    #45909, verification); forget / begin_forward force a fresh gather."""
    _say("gather reuse")
    c = W.gather_case(5, 64, 64, 4096, 528, 512, 16)
    cache = K.Cache(dev(c["cache"]), "V41", 64)
    pt, ids = dev(c["page_table"]), dev(c["ids"])
    out = torch.empty((4096, 512), dtype=torch.int16, device="cuda")
    fresh = torch.empty_like(out)
    K.kvc_dequant_gather(cache, pt, ids, fresh)
    kb = K.KVBuf()
    kb.begin_forward()
    assert kb.kvc_dequant_gather_reuse(cache, pt, ids, out) is False
    torch.cuda.synchronize()
    assert torch.equal(out, fresh)
    for _ in range(7):                               # the other layers of the source
        assert kb.kvc_dequant_gather_reuse(cache, pt, ids, out) is True
    out.zero_()                                      # a hit must not touch the buffer
    assert kb.kvc_dequant_gather_reuse(cache, pt, ids, out) is True
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0
    kb.forget()
    assert kb.kvc_dequant_gather_reuse(cache, pt, ids, out) is False
    torch.cuda.synchronize()
    assert torch.equal(out, fresh)
    kb.begin_forward()
    assert kb.kvc_dequant_gather_reuse(cache, pt, ids, out) is False


def test_gather_reuse_head_follows_the_oracle_model(K):
    """A random sequence of layers over three sources (V41, V41_FP4, V4
    caches), three id lists and two row counts, with plain gets, output
    reallocations and new forwards: every hit flag of kvc_dequant_gather_reuse
    equals the oracle model's (sglang PR #45909, summary), and after every
    operation the output buffer holds exactly the model's rows (the oracle's
    gather of the head's ids)."""
    from oracle.reuse_head import SparsePrefillKVBuffer
    _say("gather reuse vs the oracle model")
    rng = np.random.default_rng(9300)
    geo = {"V41": (528, 512, 16), "V41_FP4": (288, 256, 32), "V4": (584, 576, 8)}
    srcs = []
    for s, layout in enumerate(geo):
        c = W.gather_case(9301 + s, 24, 32, 64, *geo[layout],
                          scale_lo=None if layout == "V41_FP4" else 114)
        srcs.append((c, layout, K.Cache(dev(c["cache"]), layout, 32), dev(c["page_table"])))
    id_lists = [rng.choice(24 * 32, size=700, replace=False).astype(np.int32) for _ in range(3)]
    counts = (700, 513)
    ids_dev = {(j, n): dev(id_lists[j][:n]) for j in range(3) for n in counts}

    def fresh(s, j, n):
        c, layout = srcs[s][0], srcs[s][1]
        rows, st = oracle.dequant_gather(c["cache"], layout, 32, c["page_table"], id_lists[j][:n])
        assert st == 0
        return rows

    model = SparsePrefillKVBuffer(fresh)
    kb = K.KVBuf()
    out = torch.zeros((700, 512), dtype=torch.int16, device="cuda")
    hits = 0
    for step in range(120):
        op = rng.choice(["reuse", "reuse", "same", "same", "get", "realloc", "forward"])
        if op == "same" and model.head is not None:
            s, j, n = model.head
            op = "reuse"
        else:
            s, j, n = int(rng.integers(0, 3)), int(rng.integers(0, 3)), counts[rng.integers(0, 2)]
        c, layout, cache, pt = srcs[s]
        if op == "reuse":
            rows, want = model.get_with_head(s, j, n)
            got = kb.kvc_dequant_gather_reuse(cache, pt, ids_dev[(j, n)], out[:n])
            assert got == want, step
            hits += got
        elif op == "get":
            rows = model.get(s, j, n)
            K.kvc_dequant_gather(cache, pt, ids_dev[(j, n)], out[:n])
            kb.forget()
        elif op == "realloc":
            model.reallocate()
            out = torch.zeros((700, 512), dtype=torch.int16, device="cuda")
            continue
        else:
            model.begin_forward()
            kb.begin_forward()
            continue
        torch.cuda.synchronize()
        assert np.array_equal(host(out[:n], np.uint16), rows), step
    assert hits >= 10


# ===================================================================== compress
_run_compress = run_compress
_check_compress = check_compress


def _prefill_slots(case, ratio):
    """(latent index, slot) of every emitted row, from the plan."""
    S = case["S"]
    off, P, pt, ps = case["offsets"], case["start_pos"], case["page_table"], case["page_size"]
    lat, slots = [], []
    L = 0
    for b in range(S):
        n, p0 = int(off[1, b]), int(P[b])
        if n <= 0 or p0 < 0:
            continue
        qs = range(p0, p0 + n) if ratio == 1 else [q for q in range(p0, p0 + n) if q % 2 == 1]
        for q in qs:
            c = q if ratio == 1 else q // 2
            slots.append(int(pt[b, c // ps]) * ps + c % ps)
            lat.append(L)
            L += 1
    return lat, slots


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ratio", [1, 2])
def test_compress_prefill_ragged(K, layout, ratio):
    """ragged batch: odd lengths, odd prefixes (first pair from the pending
    state), an empty slot, padding tokens between requests, several pages."""
    _say("compress ragged", layout, ratio)
    lengths = [37, 0, 1, 2, 130, 65, 300, 3]
    P = [0, 0, 5, 7, 3, 0, 64, 1]
    case = W.compress_case(70 + ratio, lengths, start_pos=P, ratio=ratio, page_size=16,
                           fused=True, gap=3, extra_slots=2)
    r = _run_compress(K, case, layout, ratio, oracle.PREFILL)
    lat, slots = _prefill_slots(case, ratio)
    assert r["n_rows"] == len(lat)
    _check_compress(r, layout, 16, slots, lat)


@pytest.mark.parametrize("slots", [65, 150, 256, 300])
@pytest.mark.parametrize("layout,ratio", [("V41_FP4", 2), ("V41", 1), ("V4", 2)])
def test_compress_prefill_many_slots(K, layout, ratio, slots):
    """more slots than a wave has lanes, with lengths 0..40 and random (odd
    and even) start positions: 65 and 150 / 256 slots (two / four slots per
    lane, found by ballots) and 300 (LDS tables and a binary search)."""
    _say("compress many slots", layout, ratio, slots)
    rng = np.random.default_rng(123 + ratio + slots)
    lengths = rng.integers(0, 41, size=slots)
    P = rng.integers(0, 200, size=slots)
    case = W.compress_case(90 + ratio, lengths, start_pos=P, ratio=ratio, page_size=8,
                           fused=True, gap=1)
    r = _run_compress(K, case, layout, ratio, oracle.PREFILL)
    lat, slots = _prefill_slots(case, ratio)
    assert r["n_rows"] == len(lat)
    _check_compress(r, layout, 8, slots, lat)


def test_compress_c1(K):
    """one request of 64 tokens, ratio 2, separate kv / score buffers, V41,
    page 64 -> 32 rows; then a gather of the 32 rows."""
    _say("compress C1")
    case = W.workload_c1()
    r = _run_compress(K, case, "V41", 2, oracle.PREFILL, fused=False)
    lat, slots = _prefill_slots(case, 2)
    assert len(lat) == 32
    _check_compress(r, "V41", 64, slots, lat)
    ids = np.arange(32, dtype=np.int32)
    pt = case["page_table"][0]
    want, _ = oracle.dequant_gather(r["cache_g"], "V41", 64, pt, ids)
    out = torch.empty((32, 512), dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(r["cache_g"]), "V41", 64), dev(pt), dev(ids), out)
    assert np.array_equal(host(out, np.uint16), want)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compress_c3_full(K, layout):
    """16 requests totalling 32768 tokens, fused |kv|score| [32768, 1024],
    page 128, in the bench's launch configuration (the bench stores
    V41_FP4; V41 and V4 run the same batch in their layouts)."""
    _say("compress C3 full", layout)
    case = W.workload_c3()
    r = _run_compress(K, case, layout, 2, oracle.PREFILL)
    lat, slots = _prefill_slots(case, 2)
    assert r["n_rows"] == int((case["lengths"] // 2).sum()) == len(lat)
    _check_compress(r, layout, 128, slots, lat)


@pytest.mark.parametrize("requests", [128, 256])
def test_compress_many_requests_full(K, requests):
    """the C3 batch size (32768 tokens, fused buffer, page 128, V41_FP4) cut
    into 128 or 256 ragged requests, odd lengths included: the two- and
    four-slots-per-lane lookups with many items per wave."""
    _say("compress many requests full", requests)
    rng = np.random.default_rng(W.BASE_SEED + 30 + requests)
    lengths = W.ragged_lengths(rng, 32768, requests)
    case = W.compress_case(W.BASE_SEED + 31 + requests, lengths, ratio=2, page_size=128,
                           fused=True, state_random=False)
    r = _run_compress(K, case, "V41_FP4", 2, oracle.PREFILL)
    lat, slots = _prefill_slots(case, 2)
    assert r["n_rows"] == int((lengths // 2).sum()) == len(lat)
    _check_compress(r, "V41_FP4", 128, slots, lat)


@pytest.mark.parametrize("requests", [16, 100, 300])
def test_compress_prefill_many_passes(K, requests):
    """twice the C3 batch (65,536 tokens, fused buffer, page 128, V41_FP4)
    in 16, 100 or 300 ragged requests: about 16,380 work items on a grid of
    4096 waves, so every wave takes four passes, the last one partial, through
    the one-ballot, two-slots-per-lane and LDS-table kernels."""
    _say("compress many passes", requests)
    rng = np.random.default_rng(W.BASE_SEED + 50 + requests)
    lengths = W.ragged_lengths(rng, 65536, requests)
    case = W.compress_case(W.BASE_SEED + 51 + requests, lengths, ratio=2, page_size=128,
                           fused=True, state_random=False)
    r = _run_compress(K, case, "V41_FP4", 2, oracle.PREFILL)
    lat, slots = _prefill_slots(case, 2)
    assert r["n_rows"] == int((lengths // 2).sum()) == len(lat)
    _check_compress(r, "V41_FP4", 128, slots, lat)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compress_ratio1_c2(K, layout):
    """fused ratio-1 compress (norm + rope) of the C2 rows, then a gather of
    every row by physical slot."""
    _say("compress ratio-1 C2", layout)
    c2 = W.workload_c2()
    lengths = c2["lengths"]
    case = W.compress_case(W.BASE_SEED + 22, lengths, ratio=1, page_size=64, fused=False)
    case["kv"] = c2["rows"]
    r = _run_compress(K, case, layout, 1, oracle.PREFILL, fused=False)
    lat, slots = _prefill_slots(case, 1)
    _check_compress(r, layout, 64, slots, lat)
    ids = np.array(slots, np.int32)
    want, _ = oracle.dequant_gather(r["cache_g"], layout, 64, None, ids)
    out = torch.empty((ids.size, 512), dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(r["cache_g"]), layout, 64), None, dev(ids), out)
    assert np.array_equal(host(out, np.uint16), want)


def test_compress_decode_c5(K):
    """1024 slots x 1 token, ratio 2, V4, explicit out_loc (0 at even
    positions): rows at odd positions, pending state at even ones."""
    _say("compress decode C5")
    case = W.workload_c5()
    r = _run_compress(K, case, "V4", 2, oracle.DECODE, out_loc=case["out_loc"], page_table=None)
    odd = np.nonzero(case["pos"] % 2 == 1)[0]
    _check_compress(r, "V4", 64, [int(case["out_loc"][b]) for b in odd], list(odd))
    even = np.nonzero(case["pos"] % 2 == 0)[0]
    assert np.all(r["lat_g"][even] == 0)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ratio", [1, 2])
def test_compress_decode_page_table(K, layout, ratio):
    _say("compress decode page-table", layout, ratio)
    case = W.decode_case(91 + ratio, 300, ratio=ratio, page_size=32, max_pos=5000,
                         explicit_out_loc=False)
    case["pos"][::37] = -1                           # inactive slots
    r = _run_compress(K, case, layout, ratio, oracle.DECODE)
    pos = case["pos"]
    rows = np.nonzero((pos >= 0) & ((pos % 2 == 1) if ratio == 2 else True))[0]
    c = pos[rows] // ratio
    slots = [int(case["page_table"][b, cc // 32]) * 32 + int(cc % 32) for b, cc in zip(rows, c)]
    _check_compress(r, layout, 32, slots, list(rows))


def test_compress_status_bits(K):
    _say("compress status")
    case = W.compress_case(57, [10, 6], ratio=2, page_size=4, fused=True, pt_slack=0)
    pt = case["page_table"].copy()
    pt[0, 1] = 10 ** 6
    r = _run_compress(K, case, "V41", 2, oracle.PREFILL, max_out_rows=4, page_table=pt)
    assert r["st_g"] == r["st_o"] == K.STATUS_PAGE_RANGE | K.STATUS_LATENT_RANGE
    case2 = W.compress_case(58, [10], ratio=2, page_size=4, fused=True, pt_slack=0)
    case2["freqs"] = case2["freqs"][:4].copy()
    r2 = _run_compress(K, case2, "V41", 2, oracle.PREFILL)
    assert r2["st_g"] == r2["st_o"] == K.STATUS_POS_RANGE
    assert np.array_equal(r2["cache_g"], r2["cache_o"])


def test_negative_control_eps(K):
    """A 1% eps change must change the GPU's outputs (the harness really
    runs the kernel with the arguments it is given)."""
    _say("negative control")
    case = W.compress_case(59, [64, 33], ratio=2, page_size=16, fused=True)
    case["eps"] = 1e-2
    a = _run_compress(K, case, "V41", 2, oracle.PREFILL)
    b = _run_compress(K, case, "V41", 2, oracle.PREFILL, eps=1.01e-2)
    assert sha(a["cache_g"]) != sha(b["cache_g"])
    assert sha(a["lat_g"]) != sha(b["lat_g"])
    c = _run_compress(K, case, "V41", 2, oracle.PREFILL)
    assert sha(a["cache_g"]) == sha(c["cache_g"]) and sha(a["lat_g"]) == sha(c["lat_g"])
