"""Edge cases of the HIP path against the oracle, through the C ABI: the
largest prefill batch, the smallest and largest pages, strided buffers,
ragged gather counts, a gather and stores several grid rounds long, the
longest draft, decode context parallelism at a wide group and the widest
DCP id rows.  Same bar as the other parity tests (bytes bit-exact; fused
outputs within the stated tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import check_compress, dev, host, run_compress

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import fp8_fp4_quantized_amd as k
    return k


def _say(*a):
    print("[case]", *a, flush=True)


def _prefill_rows(case, ratio, lengths, P, ps):
    lat, slots, L = [], [], 0
    for b in range(len(lengths)):
        n, p0 = int(lengths[b]), int(P[b])
        if n <= 0 or p0 < 0:
            continue
        qs = range(p0, p0 + n) if ratio == 1 else [q for q in range(p0, p0 + n) if q % 2 == 1]
        for q in qs:
            c = q if ratio == 1 else q // 2
            slots.append(int(case["page_table"][b, c // ps]) * ps + c % ps)
            lat.append(L)
            L += 1
    return lat, slots


@pytest.mark.parametrize("ratio", [1, 2])
def test_prefill_largest_slot_count(K, ratio):
    """8191 request slots (the largest prefill batch: two LDS tables of 8192
    ints), lengths 0..3, odd and even starts."""
    _say("prefill 8191 slots", ratio)
    rng = np.random.default_rng(400 + ratio)
    S = 8191
    lengths = rng.integers(0, 4, size=S)
    P = rng.integers(0, 9, size=S)
    case = W.compress_case(401 + ratio, lengths, start_pos=P, ratio=ratio, page_size=4,
                           fused=True, pt_slack=0, spare_pages=1)
    r = run_compress(K, case, "V41_FP4", ratio, oracle.PREFILL)
    lat, slots = _prefill_rows(case, ratio, lengths, P, 4)
    assert r["n_rows"] == len(lat)
    check_compress(r, "V41_FP4", 4, slots, lat)


@pytest.mark.parametrize("ps", [1, 4096])
@pytest.mark.parametrize("layout", ["V4", "V41", "V41_FP4"])
def test_page_size_extremes(K, ps, layout):
    """page_size 1 (every row its own page; V4's 584-byte page padded to a
    592-byte stride) and 4096: store, compress and gather."""
    _say("page size", ps, layout)
    rng = np.random.default_rng(410 + ps)
    lengths = [300, 0, 77, 1]
    P = [0, 0, 3, 10]
    db, sb, rb, _ = oracle.layout_bytes(layout)
    stride = -(-ps * rb // 16) * 16
    case = W.compress_case(411, lengths, start_pos=P, ratio=2, page_size=ps, fused=True)
    r = run_compress(K, case, layout, 2, oracle.PREFILL, page_stride=stride)
    lat, slots = _prefill_rows(case, 2, lengths, P, ps)
    check_compress(r, layout, ps, slots, lat)
    # plain store + gather back through the physical slots just written
    rows = W.outlier_rows(rng, len(slots))
    loc = np.asarray(slots, np.int32)
    hc = np.zeros((case["num_pages"], stride), np.uint8)
    dc = dev(hc)
    assert oracle.store_rows(hc, layout, ps, rows, loc) == 0
    K.kvc_store_rows(K.Cache(dc, layout, ps), dev(rows), dev(loc))
    torch.cuda.synchronize()
    assert np.array_equal(host(dc), hc)
    ids = np.concatenate([loc[::-1], [-1, 0]]).astype(np.int32)
    want, st = oracle.dequant_gather(hc, layout, ps, None, ids)
    out = torch.empty((ids.size, 512), dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(K.Cache(dc, layout, ps), None, dev(ids), out)
    torch.cuda.synchronize()
    assert st == 0 and np.array_equal(host(out, np.uint16), want)


def test_strided_buffers(K):
    """separate kv and score buffers with row strides 640 and 768, latent
    and pre-quant outputs with strides 520 and 1024, gather output stride
    1032: the padding columns stay untouched."""
    _say("strided buffers")
    lengths, P = [45, 8, 0, 19], [0, 1, 0, 6]
    case = W.compress_case(420, lengths, start_pos=P, ratio=2, page_size=16, fused=False)
    T = case["T"]
    kv = np.full((T, 640), 0x7F7F, np.uint16)
    kv[:, :512] = case["kv"]
    sc = np.full((T, 768), 0x7F7F, np.uint16)
    sc[:, :512] = case["score"]
    hc = np.zeros((case["num_pages"], 16 * 528), np.uint8)
    state = case["state"].copy()
    lat_o, pre_o, st, n = oracle.compress(
        ratio=2, mode=oracle.PREFILL, kv=case["kv"], score=case["score"],
        offsets=case["offsets"], start_pos=case["start_pos"], page_table=case["page_table"],
        state=state, norm_w=case["norm_w"], eps=case["eps"], freqs=case["freqs"], cache=hc,
        layout="V41", page_size=16)
    dc = dev(np.zeros_like(hc))
    lat = torch.full((n, 520), 3, dtype=torch.int16, device="cuda")
    pre = torch.full((n, 1024), 3, dtype=torch.int16, device="cuda")
    sd = dev(case["state"])
    K.kvc_compress_store(ratio=2, mode=K.MODE_PREFILL, kv=dev(kv)[:, :512], score=dev(sc)[:, :512],
                         start_pos=dev(case["start_pos"]), offsets=dev(case["offsets"]),
                         page_table=dev(case["page_table"]), state=sd,
                         norm_w=dev(case["norm_w"]), eps=case["eps"], freqs=dev(case["freqs"]),
                         latent_out=lat[:, :512], prequant_out=pre[:, :512],
                         cache=K.Cache(dc, "V41", 16))
    torch.cuda.synchronize()
    lg, pg = host(lat, np.uint16), host(pre, np.uint16)
    assert np.all(lg[:, 512:] == 3) and np.all(pg[:, 512:] == 3)
    r = dict(lat_o=lat_o, pre_o=pre_o, st_o=st, st_g=st, lat_g=lg[:, :512], pre_g=pg[:, :512],
             cache_o=hc, cache_g=host(dc), state_o=state, state_g=host(sd, np.uint16))
    lat_i, slots = _prefill_rows(case, 2, lengths, P, 16)
    check_compress(r, "V41", 16, slots, lat_i)
    ids = np.asarray(slots[:37], np.int32)
    want, _ = oracle.dequant_gather(hc, "V41", 16, None, ids)
    out = torch.full((ids.size, 1032), 5, dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(hc), "V41", 16), None, dev(ids), out[:, :512])
    torch.cuda.synchronize()
    g = host(out, np.uint16)
    assert np.array_equal(g[:, :512], want) and np.all(g[:, 512:] == 5)


@pytest.mark.parametrize("n", [1, 15, 17, 31, 33, 97, 65537, 131071, 131072, 131085])
@pytest.mark.parametrize("layout", ["V4", "V41", "V41_FP4"])
def test_gather_ragged_counts(K, n, layout):
    """id counts that are not a multiple of the id batch or of the rows a
    wave expands per trip, through a page table.  Up to 65,535 ids the batch
    is 8 and a trip 8 rows; 65,537 and 131,071 ids take 16-id batches and
    8-row trips, the last batch short; from 131,072 ids (the large-gather
    form: streamed codes, 16-row trips except V4) 32-id batches, and
    131,085 ids end on a batch of 13."""
    _say("gather ragged", n, layout)
    db, sb, rb, _ = oracle.layout_bytes(layout)
    c = W.gather_case(430 + n, 8 if n <= 128 else n // 16 + 8, 16, n, rb, db, sb,
                      scale_lo=None if layout == "V41_FP4" else 110, scale_hi=140)
    want, st = oracle.dequant_gather(c["cache"], layout, 16, c["page_table"], c["ids"])
    out = torch.full((n + 1, 512), 9, dtype=torch.int16, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(c["cache"]), layout, 16), dev(c["page_table"]),
                         dev(c["ids"]), out[:n])
    torch.cuda.synchronize()
    g = host(out, np.uint16)
    assert st == 0 and np.array_equal(g[:n], want) and np.all(g[n] == 9)


@pytest.mark.parametrize("layout", ["V4", "V41", "V41_FP4"])
def test_gather_large_strided_output(K, layout):
    """a gather in the large form (140,001 ids, 32-id batches, streamed codes)
    into a strided output (rows 640 elements apart), ids with -1 and ids past
    the page table: rows and status equal the oracle's, the columns between
    rows are untouched."""
    _say("gather large strided", layout)
    n = 140001
    db, sb, rb, _ = oracle.layout_bytes(layout)
    c = W.gather_case(470, n // 16 + 8, 16, n, rb, db, sb,
                      scale_lo=None if layout == "V41_FP4" else 110, scale_hi=140)
    ids = c["ids"].copy()
    ids[::17] = -1
    ids[5::1001] = (n // 16 + 8) * 16 + 3               # past the page table
    want, st = oracle.dequant_gather(c["cache"], layout, 16, c["page_table"], ids)
    out = torch.full((n, 640), 11, dtype=torch.int16, device="cuda")
    s = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(c["cache"]), layout, 16), dev(c["page_table"]), dev(ids),
                         out[:, :512], s)
    torch.cuda.synchronize()
    g = host(out, np.uint16)
    assert np.array_equal(g[:, :512], want) and np.all(g[:, 512:] == 11)
    assert int(s.item()) == st == K.STATUS_ID_RANGE


def test_gather_grid_stride_sampled(K):
    """3,000,017 ids (random, 1% of them -1) from a 262,144-row V41 cache into
    a 3 GB output: past the gather grid's one-round capacity of 2^20 ids, so
    every wave takes about three batches and the last batch is ragged.  The
    first and last 256 rows and 8192 sampled rows are compared with the
    oracle; the guard row after the output is untouched."""
    _say("gather grid stride", 3000017)
    n = 3000017
    c = W.gather_case(W.BASE_SEED + 40, 4096, 64, 1, 528, 512, 16)
    rng = np.random.default_rng(W.BASE_SEED + 41)
    ids = rng.integers(0, 4096 * 64, size=n).astype(np.int32)
    ids[rng.random(n) < 0.01] = -1
    out = torch.full((n + 1, 512), 9, dtype=torch.int16, device="cuda")
    s = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvc_dequant_gather(K.Cache(dev(c["cache"]), "V41", 64), dev(c["page_table"]), dev(ids),
                         out[:n], s)
    pick = np.unique(np.concatenate([np.arange(256), np.arange(n - 256, n),
                                     rng.integers(0, n, size=8192)]))
    got = out[torch.from_numpy(pick).cuda()].cpu().numpy().view(np.uint16)
    want, st = oracle.dequant_gather(c["cache"], "V41", 64, c["page_table"], ids[pick])
    assert st == 0 and int(s.item()) == 0
    assert np.array_equal(got, want)
    assert np.all(out[n].cpu().numpy() == 9)
    del out


@pytest.mark.parametrize("layout,rope", [("V41_FP4", False), ("V41", True)])
def test_store_grid_stride(K, layout, rope):
    """200,003 rows into one cache: past the store grid's one-round capacity
    of 65,536 rows, so every wave takes about three trips and the last one is
    ragged; N(0, 1) rows, 1% padded (out_loc 0).  Plain store and RoPE store
    (positions across a 65,536-entry table): every cache byte equals the
    oracle's."""
    _say("store grid stride", layout, rope)
    n, ps = 200003, 64
    rng = np.random.default_rng(W.BASE_SEED + 42 + rope)
    rows = W.normal_bf16(rng, (n, 512))
    pages = n // ps + 3
    loc = (W.random_pages(rng, pages - 1, pages).astype(np.int64)[:, None] * ps
           + np.arange(ps)[None, :]).reshape(-1)[:n]
    loc = rng.permutation(loc).astype(np.int32)
    loc[rng.random(n) < 0.01] = 0
    rb = oracle.layout_bytes(layout)[2]
    hc = np.full((pages, ps * rb), 0x3C, np.uint8)
    dc = dev(hc)
    s = torch.zeros(1, dtype=torch.int32, device="cuda")
    if rope:
        pos = rng.integers(0, 65536, size=n).astype(np.int32)
        fr = W.rope_freqs(65536)
        _, st = oracle.store_rows_rope(hc, layout, ps, rows, pos, fr, loc)
        K.kvc_store_rows_rope(K.Cache(dc, layout, ps), dev(rows), dev(pos), dev(fr), dev(loc), s)
    else:
        st = oracle.store_rows(hc, layout, ps, rows, loc)
        K.kvc_store_rows(K.Cache(dc, layout, ps), dev(rows), dev(loc), s)
    torch.cuda.synchronize()
    assert st == 0 and int(s.item()) == 0
    assert np.array_equal(host(dc), hc)


def test_verify_longest_draft(K):
    """draft_len 64 (the largest), ring of 33 entries (rollback-safe)."""
    _say("verify draft 64")
    case = W.verify_case(440, 6, draft_len=64, ratio=2, page_size=16, max_pos=400,
                         ring_slots=33)
    r = run_compress(K, case, "V41", 2, oracle.VERIFY, page_table=case["page_table"],
                     draft_len=64, ring_slots=33)
    lat, slots = [], []
    for b in range(6):
        for j in range(64):
            q = int(case["pos"][b]) + j
            if q % 2 == 1:
                c = q // 2
                slots.append(int(case["page_table"][b, c // 16]) * 16 + c % 16)
                lat.append(b * 64 + j)
    check_compress(r, "V41", 16, slots, lat)


def test_dcp_decode_wide_group(K):
    """decode through the page table with 8 ranks in runs of 8: each rank
    stores only the rows it owns."""
    case = W.verify_case(450, 256, draft_len=1, ratio=2, page_size=64, max_pos=4096,
                         ring_slots=1)
    for rank in (0, 5, 7):
        _say("dcp decode rank", rank)
        r = run_compress(K, case, "V41_FP4", 2, oracle.DECODE, page_table=case["page_table"],
                         dcp_world=8, dcp_rank=rank, dcp_interleave=8)
        lat, slots = [], []
        for b in range(256):
            q = int(case["pos"][b])
            if q % 2 == 1:
                ow, u = oracle.dcp_owner(q // 2, 8, 8)
                slots.append(int(case["page_table"][b, u // 64]) * 64 + u % 64 if ow == rank else 0)
                lat.append(b)
        check_compress(r, "V41_FP4", 64, slots, lat)


def test_dcp_filter_widest_row(K):
    """rows of 65,536 ids (the largest k: 32 passes of 2048), 3 ranks in
    runs of 2 and a power-of-two group of 2 in runs of 8: slots and counts
    equal the oracle's on every rank."""
    c = W.dcp_ids_case(460, T=6, k=65536, n_req=3, max_rows=140000, world=3, page_size=64)
    c2 = W.dcp_ids_case(461, T=6, k=65536, n_req=3, max_rows=140000, world=2, page_size=64)
    for case, world, inter in ((c, 3, 2), (c2, 2, 8)):
        ids = case["ids"]
        for rank in range(world):
            _say("dcp filter widest row", world, inter, rank)
            bt = case["block_tables"][rank]
            want = oracle.dcp_filter_ids(ids, case["token_to_req"], bt, page_size=64,
                                         num_pages=case["num_pages"], world=world, rank=rank,
                                         interleave=inter, valid=case["valid"])
            T, k = ids.shape
            out = torch.full((T, k), 12345, dtype=torch.int32, device="cuda")
            lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
            s = torch.zeros(1, dtype=torch.int32, device="cuda")
            K.kvc_dcp_filter_ids(dev(ids), dev(case["token_to_req"]), dev(bt), out, lens,
                                 page_size=64, num_pages=case["num_pages"], world=world,
                                 rank=rank, interleave=inter, valid=dev(case["valid"]), status=s)
            torch.cuda.synchronize()
            assert np.array_equal(host(lens), want[1]) and np.array_equal(host(out), want[0])
            assert int(s.item()) == want[2]


@pytest.mark.parametrize("ratio", [1, 2])
def test_prefill_page_table_slice(K, ratio):
    """The page table passed as a column slice pt[:, :W] of a wider table
    whose spare columns hold valid pages: a row whose logical page is at or
    past W raises KVC_STATUS_PT_RANGE and is not stored (the width bounds the
    lookup; the row stride only addresses the rows), as the oracle does with
    the W-column table."""
    _say("prefill page-table slice", ratio)
    ps, Wd = 8, 3
    lengths, P = [70, 0, 33, 130], [0, 0, 5, 2]
    case = W.compress_case(470 + ratio, lengths, start_pos=P, ratio=ratio, page_size=ps,
                           fused=True)
    narrow = np.ascontiguousarray(case["page_table"][:, :Wd])
    r = run_compress(K, case, "V41", ratio, oracle.PREFILL, page_table=narrow, pt_spare_cols=4)
    assert r["st_o"] & oracle.ST_PT_RANGE
    lat, slots, L = [], [], 0
    for b in range(len(lengths)):
        n, p0 = lengths[b], P[b]
        qs = range(p0, p0 + n) if ratio == 1 else [q for q in range(p0, p0 + n) if q % 2 == 1]
        for q in qs:
            c = q if ratio == 1 else q // 2
            slots.append(int(narrow[b, c // ps]) * ps + c % ps if c // ps < Wd else 0)
            lat.append(L)
            L += 1
    assert 0 in slots and any(s != 0 for s in slots)
    check_compress(r, "V41", ps, slots, lat)


@pytest.mark.parametrize("ratio", [1, 2])
def test_prefill_token_rows_outside_buffer(K, ratio):
    """A slot whose extend rows run past the projection buffer, and one that
    starts before it, are skipped whole (no rows, no pending-state write)
    with KVC_STATUS_TOKEN_RANGE; the other slots are unaffected."""
    _say("prefill token rows outside the buffer", ratio)
    lengths, P = [40, 25, 31, 9], [0, 3, 1, 4]
    case = W.compress_case(480 + ratio, lengths, start_pos=P, ratio=ratio, page_size=16,
                           fused=True)
    T = case["kv"].shape[0]
    off = case["offsets"].copy()
    off[0, 1] = T - 10          # rows T-10 .. T+14
    off[0, 2] = -2              # rows -2 .. 28
    case = dict(case, offsets=off)
    r = run_compress(K, case, "V41_FP4", ratio, oracle.PREFILL)
    assert r["st_o"] == oracle.ST_TOKEN_RANGE
    lat, slots, L = [], [], 0
    for b in (0, 3):
        n, p0 = lengths[b], P[b]
        qs = range(p0, p0 + n) if ratio == 1 else [q for q in range(p0, p0 + n) if q % 2 == 1]
        for q in qs:
            c = q if ratio == 1 else q // 2
            slots.append(int(case["page_table"][b, c // 16]) * 16 + c % 16)
            lat.append(L)
            L += 1
    assert r["n_rows"] == L
    check_compress(r, "V41_FP4", 16, slots, lat)


def test_dcp_filter_block_table_slice(K):
    """The block table passed as a column slice bt[:, :W] of a wider table
    whose spare columns hold valid pages: ids whose page is at or past W are
    dropped with KVC_STATUS_PT_RANGE, as the oracle does with the W-column
    table."""
    _say("dcp filter block-table slice")
    c = W.dcp_ids_case(490, T=64, k=700, n_req=4, max_rows=6000, world=2, page_size=64)
    ids = c["ids"]
    for rank in range(2):
        bt = c["block_tables"][rank]
        Wd = 8                  # ids of requests past 1024 rows reach page 8
        narrow = np.ascontiguousarray(bt[:, :Wd])
        want = oracle.dcp_filter_ids(ids, c["token_to_req"], narrow, page_size=64,
                                     num_pages=c["num_pages"], world=2, rank=rank, interleave=4,
                                     valid=c["valid"])
        assert want[2] & oracle.ST_PT_RANGE
        wide = np.concatenate([narrow, np.random.default_rng(491).integers(
            0, c["num_pages"], size=(bt.shape[0], 5)).astype(np.int32)], axis=1)
        T, k = ids.shape
        out = torch.full((T, k), 12345, dtype=torch.int32, device="cuda")
        lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
        s = torch.zeros(1, dtype=torch.int32, device="cuda")
        K.kvc_dcp_filter_ids(dev(ids), dev(c["token_to_req"]), dev(wide)[:, :Wd], out, lens,
                             page_size=64, num_pages=c["num_pages"], world=2, rank=rank,
                             interleave=4, valid=dev(c["valid"]), status=s)
        torch.cuda.synchronize()
        assert np.array_equal(host(lens), want[1]) and np.array_equal(host(out), want[0])
        assert int(s.item()) == want[2]
