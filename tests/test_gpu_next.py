"""HIP path vs the oracle for the verify mode and pending-state ring, decode
context parallelism (owner predicate in the compressor, id filter), the
RoPE store and graph capture of the prefill compressor.

Bar: bit-exact for bytes and indices (RoPE store bytes, filtered slots and
counts, pending state, untouched cache bytes, the quantizer given the
kernel's own pre-quant rows); 2e-2 relative, codes within one step, for the
fused compressor's outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import spec
from tests.gpu_util import (assert_latent_close, assert_rows_close, check_compress, dev, host,
                            row_parts, run_compress, written_mask)

pytestmark = pytest.mark.gpu

LAYOUTS = ["V4", "V41", "V41_FP4"]


@pytest.fixture(scope="module")
def K():
    import fp8_fp4_quantized_amd as k
    return k


def _say(*a):
    print("[case]", *a, flush=True)


def _token_rows(case, ratio, world=1, rank=0, interleave=1):
    """(latent index, destination slot) of every token that emits a row in a
    decode / verify batch; slot 0 where nothing is stored."""
    S, D, ps = case["S"], case["draft_len"], case["page_size"]
    lat, slots = [], []
    for b in range(S):
        p0 = int(case["pos"][b])
        if p0 < 0:
            continue
        for j in range(D):
            q, t = p0 + j, b * D + j
            if ratio == 2 and q % 2 == 0:
                continue
            c = q // 2 if ratio == 2 else q
            if case["out_loc"] is not None:
                slot = int(case["out_loc"][t])
            else:
                r, u = oracle.dcp_owner(c, world, interleave)
                slot = int(case["page_table"][b, u // ps]) * ps + u % ps if r == rank else 0
            lat.append(t)
            slots.append(slot)
    return lat, slots


# ================================================================= verify
@pytest.mark.parametrize("explicit", [False, True])
@pytest.mark.parametrize("layout,ratio", [("V41", 2), ("V41_FP4", 2), ("V4", 2), ("V41", 1)])
def test_verify_batch(K, layout, ratio, explicit):
    """draft_len 4, ring of 3 entries, skipped slots, padded tokens."""
    _say("verify", layout, ratio, explicit)
    case = W.verify_case(200 + ratio, 96, draft_len=4, ratio=ratio, page_size=16, max_pos=512,
                         ring_slots=3, explicit_out_loc=explicit, skip_frac=0.1)
    r = run_compress(K, case, layout, ratio, oracle.VERIFY, out_loc=case["out_loc"],
                     page_table=case["page_table"], draft_len=4, ring_slots=3)
    lat, slots = _token_rows(case, ratio)
    assert r["n_rows"] == len(lat)
    check_compress(r, layout, 16, slots, lat)


def test_verify_bench_size(K):
    """the bench's verify batch: 1024 slots x 4 drafts, ring of 3, V41_FP4
    through page tables of 64-row pages (one wave per row)."""
    _say("verify bench size")
    case = W.verify_case(20261206, 1024, draft_len=4, ratio=2, page_size=64, max_pos=4096,
                         ring_slots=3)
    r = run_compress(K, case, "V41_FP4", 2, oracle.VERIFY, page_table=case["page_table"],
                     draft_len=4, ring_slots=3)
    lat, slots = _token_rows(case, 2)
    assert r["n_rows"] == len(lat)
    check_compress(r, "V41_FP4", 64, slots, lat)


@pytest.mark.parametrize("D,R", [(1, 1), (1, 3), (2, 2), (7, 4), (16, 1)])
def test_verify_draft_lengths_and_rings(K, D, R):
    """other draft lengths, a ring too small for rollback (still exact for
    one call: the last token sharing an entry wins) and plain decode, with
    one ring entry and with three (whose pending entry depends on the
    position)."""
    _say("verify D R", D, R)
    case = W.verify_case(210 + D, 40, draft_len=D, ratio=2, page_size=8, max_pos=300,
                         ring_slots=R)
    r = run_compress(K, case, "V41_FP4", 2, oracle.VERIFY, page_table=case["page_table"],
                     draft_len=D, ring_slots=R)
    lat, slots = _token_rows(case, 2)
    check_compress(r, "V41_FP4", 8, slots, lat)


def test_verify_rejection_steps(K):
    """Nine verify steps with random acceptance on device and in the oracle:
    every step's rows and the ring match; the ring restarts each step where
    the accepted drafts end."""
    _say("verify rejection steps")
    D, S, ps, layout = 4, 64, 8, "V41"
    base = W.verify_case(220, S, draft_len=D, page_size=ps, max_pos=64, ring_slots=3)
    rb = oracle.layout_bytes(layout)[2]
    hc = np.zeros((base["num_pages"], ps * rb), np.uint8)
    dc = dev(hc)
    st_h = np.zeros((S, 3, 2, 512), np.uint16)
    st_d = dev(st_h)
    pos = np.zeros(S, np.int32)
    rng = np.random.default_rng(221)
    written = set()
    for step in range(9):
        kv = W.normal_bf16(rng, (S * D, 1024))
        case = dict(base, kv=kv, pos=pos.copy())
        lat_o, pre_o, st_o, n = oracle.compress(
            ratio=2, mode=oracle.VERIFY, kv=kv, fused=True, start_pos=pos,
            page_table=base["page_table"], state=st_h, norm_w=base["norm_w"], eps=base["eps"],
            freqs=base["freqs"], cache=hc, layout=layout, page_size=ps, draft_len=D,
            ring_slots=3)
        lat = torch.zeros((S * D, 512), dtype=torch.int16, device="cuda")
        pre = torch.zeros_like(lat)
        s = torch.zeros(1, dtype=torch.int32, device="cuda")
        kvd = dev(kv)
        K.kvc_compress_store(ratio=2, mode=K.MODE_VERIFY, kv=kvd[:, :512], score=kvd[:, 512:],
                             start_pos=dev(pos), cache=K.Cache(dc, layout, ps),
                             norm_w=dev(base["norm_w"]), eps=base["eps"],
                             freqs=dev(base["freqs"]), latent_out=lat,
                             page_table=dev(base["page_table"]), state=st_d, prequant_out=pre,
                             status=s, draft_len=D, ring_slots=3)
        torch.cuda.synchronize()
        assert int(s.item()) == st_o == 0
        assert np.array_equal(host(st_d, np.uint16), st_h), step
        idx, slots = _token_rows(case, 2)
        lat_g, pre_g = host(lat, np.uint16), host(pre, np.uint16)
        assert_latent_close(lat_g[idx], lat_o[idx])
        cg = host(dc)
        gd = np.stack([row_parts(cg, layout, ps, q)[0] for q in slots])
        gs = np.stack([row_parts(cg, layout, ps, q)[1] for q in slots])
        od = np.stack([row_parts(hc, layout, ps, q)[0] for q in slots])
        os_ = np.stack([row_parts(hc, layout, ps, q)[1] for q in slots])
        qd, qs = oracle.store_row(layout, pre_g[idx])
        assert np.array_equal(qd, gd) and np.array_equal(qs, gs)
        assert_rows_close(layout, gd, gs, od, os_, spec.bf16_value(pre_o[idx]))
        written |= set(slots)
        pos = pos + rng.integers(0, D + 1, size=S).astype(np.int32)
    m = written_mask(hc.shape, layout, ps, written)
    assert np.array_equal(host(dc)[~m], hc[~m])


# ================================================================= DCP
@pytest.mark.parametrize("layout,slots", [("V41", 5), ("V41_FP4", 5), ("V41_FP4", 90),
                                          ("V41_FP4", 300)])
def test_dcp_prefill_owner_predicate(K, layout, slots):
    """prefill rows dealt over 3 ranks in runs of 2; each rank's call stores
    its own rows at its own page-table slots.  5 and 90 slots (lookup by
    ballots over one and two slots per lane) and 300 (the LDS tables and
    binary search of batches over 256 slots)."""
    world, K_, ps = 3, 2, 8
    if slots == 5:
        lengths, P = [37, 0, 120, 9, 64], [0, 0, 5, 2, 31]
    else:
        rng = np.random.default_rng(229)
        lengths = [int(x) for x in rng.integers(0, 70, size=slots)]
        P = [int(x) for x in rng.integers(0, 40, size=slots)]
    case = W.compress_case(230, lengths, start_pos=P, ratio=2, page_size=ps, fused=True, gap=2)
    tables, npg = W.per_rank_page_tables(231, world, len(lengths), case["page_table"].shape[1])
    for rank in range(world):
        _say("dcp prefill", layout, slots, rank)
        c = dict(case, page_table=tables[rank], num_pages=npg)
        r = run_compress(K, c, layout, 2, oracle.PREFILL, page_table=tables[rank],
                         dcp_world=world, dcp_rank=rank, dcp_interleave=K_)
        lat, slots, L = [], [], 0
        for b, (n, p0) in enumerate(zip(lengths, P)):
            for q in range(p0, p0 + n):
                if q % 2 == 1:
                    ow, u = oracle.dcp_owner(q // 2, world, K_)
                    slots.append(int(tables[rank][b, u // ps]) * ps + u % ps if ow == rank else 0)
                    lat.append(L)
                    L += 1
        assert r["n_rows"] == L
        check_compress(r, layout, ps, slots, lat)


def test_dcp_verify_owner_predicate(K):
    """verify through the page table under 2 ranks, runs of 4."""
    case = W.verify_case(232, 64, draft_len=4, ratio=2, page_size=16, max_pos=512, ring_slots=3)
    for rank in range(2):
        _say("dcp verify", rank)
        r = run_compress(K, case, "V41", 2, oracle.VERIFY, page_table=case["page_table"],
                         draft_len=4, ring_slots=3, dcp_world=2, dcp_rank=rank,
                         dcp_interleave=4)
        lat, slots = _token_rows(case, 2, world=2, rank=rank, interleave=4)
        check_compress(r, "V41", 16, slots, lat)


def _filter(K, c, world, rank, interleave, k=None, valid=True):
    ids = c["ids"] if k is None else c["ids"][:, :k]
    T, kk = ids.shape
    bt = c["block_tables"][rank]
    want = oracle.dcp_filter_ids(ids, c["token_to_req"], bt, page_size=c["page_size"],
                                 num_pages=c["num_pages"], world=world, rank=rank,
                                 interleave=interleave, valid=c["valid"] if valid else None)
    out = torch.full((T, kk), 12345, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    s = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvc_dcp_filter_ids(dev(ids), dev(c["token_to_req"]), dev(bt), out, lens,
                         page_size=c["page_size"], num_pages=c["num_pages"], world=world,
                         rank=rank, interleave=interleave,
                         valid=dev(c["valid"]) if valid else None, status=s)
    torch.cuda.synchronize()
    return want, (host(out), host(lens), int(s.item()))


@pytest.mark.parametrize("world,interleave,k", [(1, 1, 64), (2, 1, 100), (4, 4, 2048),
                                                 (3, 2, 7), (8, 16, 513), (4, 2, 4100),
                                                 (6, 4, 2100)])
def test_dcp_filter_ids(K, world, interleave, k):
    """every rank's slots and counts equal the oracle's; rows of one or more
    2048-id passes, full and partial, power-of-two groups and others."""
    _say("dcp filter", world, interleave, k)
    c = W.dcp_ids_case(240 + world, T=300, k=k, n_req=7, max_rows=max(3000, 2 * k),
                       world=world, page_size=64)
    total = 0
    for rank in range(world):
        (ws, wl, wst), (gs, gl, gst) = _filter(K, c, world, rank, interleave)
        assert np.array_equal(gl, wl) and np.array_equal(gs, ws) and gst == wst
        total += int(gl.sum())
    assert total == int(((c["ids"] >= 0) & (c["valid"][:, None] != 0)).sum())


def test_dcp_filter_bench_size(K):
    """the bench's filter: 4096 token rows x 2048 global ids, 32 requests,
    4 ranks in runs of 4, every rank (bit-exact; the ranks' counts
    partition the valid ids)."""
    _say("dcp filter bench size")
    c = W.dcp_ids_case(20261208, T=4096, k=2048, n_req=32, max_rows=65536, world=4,
                       page_size=64)
    total = 0
    for rank in range(4):
        (ws, wl, wst), (gs, gl, gst) = _filter(K, c, 4, rank, 4)
        assert np.array_equal(gl, wl) and np.array_equal(gs, ws) and gst == wst
        total += int(gl.sum())
    assert total == int(((c["ids"] >= 0) & (c["valid"][:, None] != 0)).sum())


def test_dcp_filter_edges(K):
    """no valid flags, an empty id row width, requests outside the table,
    pages outside the cache and past the table row."""
    _say("dcp filter edges")
    c = W.dcp_ids_case(250, T=70, k=130, n_req=4, max_rows=900, world=2, page_size=16)
    c["token_to_req"][::9] = 9                     # no such request
    c["block_tables"][1][1, 3] = c["num_pages"] + 5
    c["block_tables"][1][2, 0] = -3
    (ws, wl, wst), (gs, gl, gst) = _filter(K, c, 2, 1, 1, valid=False)
    assert np.array_equal(gl, wl) and np.array_equal(gs, ws) and gst == wst
    assert wst & oracle.ST_REQ_RANGE and wst & oracle.ST_PAGE_RANGE
    (ws, wl, wst), (gs, gl, gst) = _filter(K, c, 2, 0, 2, k=0)
    assert gs.shape[1] == 0 and np.all(gl == 0)
    # a block table two pages wide: ids past it are dropped with PT_RANGE
    c["block_tables"] = [np.ascontiguousarray(b[:, :2]) for b in c["block_tables"]]
    (ws, wl, wst), (gs, gl, gst) = _filter(K, c, 2, 1, 1, valid=False)
    assert np.array_equal(gl, wl) and np.array_equal(gs, ws) and gst == wst
    assert wst & oracle.ST_PT_RANGE


# ================================================================= RoPE store
@pytest.mark.parametrize("layout", LAYOUTS)
def test_rope_store_bit_exact(K, layout):
    """every byte equals the oracle's: rows of random lengths, positions
    across a 4096-entry table, padded rows and positions outside it."""
    _say("rope store", layout)
    c = W.rope_store_case(260, [700, 1, 129, 64], page_size=64, max_pos=4096, pad_frac=0.05,
                          bad_pos_frac=0.05)
    rb = oracle.layout_bytes(layout)[2]
    hc = np.full((c["num_pages"], 64 * rb), 0x5C, np.uint8)
    dc = dev(hc)
    _, st = oracle.store_rows_rope(hc, layout, 64, c["rows"], c["positions"], c["freqs"],
                                   c["out_loc"])
    s = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvc_store_rows_rope(K.Cache(dc, layout, 64), dev(c["rows"]), dev(c["positions"]),
                          dev(c["freqs"]), dev(c["out_loc"]), status=s)
    torch.cuda.synchronize()
    assert int(s.item()) == st == oracle.ST_POS_RANGE
    assert np.array_equal(host(dc), hc)


def test_rope_store_c2_size(K):
    """the ratio-1 store workload (8 requests, 512..4096 rows each) with a
    rotary position per row, V41_FP4: bit-exact."""
    _say("rope store C2 size")
    c2 = W.workload_c2()
    rng = np.random.default_rng(261)
    pos = rng.integers(0, 16384, size=c2["rows"].shape[0]).astype(np.int32)
    fr = W.rope_freqs(16384)
    rb = 288
    hc = np.zeros((c2["num_pages"], 64 * rb), np.uint8)
    dc = dev(hc)
    _, st = oracle.store_rows_rope(hc, "V41_FP4", 64, c2["rows"], pos, fr, c2["out_loc"])
    K.kvc_store_rows_rope(K.Cache(dc, "V41_FP4", 64), dev(c2["rows"]), dev(pos), dev(fr),
                          dev(c2["out_loc"]))
    torch.cuda.synchronize()
    assert st == 0 and np.array_equal(host(dc), hc)


def test_rope_store_every_magnitude(K):
    """V4 keeps the rotated rope dims as bf16, so its bytes show the fp64 ->
    bf16 rounding directly: rope dims drawn from every bf16 bit pattern
    (subnormals, the largest finite values, infinities, NaNs) meet subnormal
    and zero results, overflow to infinity and NaN; bytes equal the
    oracle's."""
    _say("rope store every magnitude")
    c = W.rope_store_case(262, [4096, 3000], page_size=64, max_pos=4096, pad_frac=0.0)
    rows = c["rows"].copy()
    rng = np.random.default_rng(263)
    n = rows.shape[0]
    pat = rng.integers(0, 1 << 16, size=(n, 64)).astype(np.uint16)
    # a third of the rows keep any pattern, a third get exponents 0..8 (bf16
    # subnormal and zero results), a third exponents 248..254 (overflow)
    mode = rng.integers(0, 3, size=(n, 1))
    expo = np.where(mode == 1, rng.integers(0, 9, size=(n, 64)), rng.integers(248, 255, size=(n, 64)))
    shaped = (pat & 0x807F) | (expo.astype(np.uint16) << 7)
    rows[:, 448:] = np.where(mode == 0, pat, shaped).astype(np.uint16)
    rb = oracle.layout_bytes("V4")[2]
    stride = -(-64 * rb // 16) * 16
    hc = np.zeros((c["num_pages"], stride), np.uint8)
    dc = dev(hc)
    _, st = oracle.store_rows_rope(hc, "V4", 64, rows, c["positions"], c["freqs"], c["out_loc"])
    K.kvc_store_rows_rope(K.Cache(dc, "V4", 64), dev(rows), dev(c["positions"]), dev(c["freqs"]),
                          dev(c["out_loc"]))
    torch.cuda.synchronize()
    got = host(dc)
    assert st == 0 and np.array_equal(got, hc)


# ================================================================= graph capture
def test_prefill_compress_graph_replay(K):
    """The prefill compressor captured once in a graph, its offsets, start
    positions, pending state and projection rows refreshed in place between
    replays: every replay equals an eager call on the same inputs
    (bit-exact) and the oracle (tolerance)."""
    layout, ps, S, T = "V41_FP4", 16, 8, 600
    cases = [W.compress_case(270 + i, W.ragged_lengths(np.random.default_rng(280 + i), T - 40, S),
                             start_pos=np.random.default_rng(290 + i).integers(0, 50, size=S),
                             ratio=2, page_size=ps, fused=True, pt_slack=3) for i in range(3)]
    rb = oracle.layout_bytes(layout)[2]
    npg = max(c["num_pages"] for c in cases)
    pts = max(c["page_table"].shape[1] for c in cases)
    max_rows = T // 2 + S

    proj = torch.zeros((T, 1024), dtype=torch.int16, device="cuda")
    offs = torch.zeros((2, S), dtype=torch.int32, device="cuda")
    start = torch.zeros(S, dtype=torch.int32, device="cuda")
    pt = torch.zeros((S, pts), dtype=torch.int32, device="cuda")
    state = torch.zeros((S, 2, 512), dtype=torch.int16, device="cuda")
    cache = torch.zeros((npg, ps * rb), dtype=torch.uint8, device="cuda")
    lat = torch.zeros((max_rows, 512), dtype=torch.int16, device="cuda")
    pre = torch.zeros_like(lat)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    w = dev(cases[0]["norm_w"])
    fr = dev(W.rope_freqs(T + 64))

    def load(c):
        proj.zero_()
        proj[:c["kv"].shape[0]].copy_(dev(c["kv"]))
        offs.copy_(dev(c["offsets"]))
        start.copy_(dev(c["start_pos"]))
        pt.zero_()
        pt[:, :c["page_table"].shape[1]].copy_(dev(c["page_table"]))
        state.copy_(dev(c["state"]))
        cache.zero_()
        lat.zero_()
        pre.zero_()

    def call():
        status.zero_()
        K.kvc_compress_store(ratio=2, mode=K.MODE_PREFILL, kv=proj[:, :512], score=proj[:, 512:],
                             start_pos=start, cache=K.Cache(cache, layout, ps), norm_w=w,
                             eps=1e-6, freqs=fr, latent_out=lat, offsets=offs, page_table=pt,
                             state=state, prequant_out=pre, status=status)

    def snap():
        return [host(t).copy() for t in (cache, lat, pre, state, status)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        load(cases[0])
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, c in enumerate(cases):
            _say("graph replay", rep, i)
            load(c)
            torch.cuda.synchronize()
            call()                                   # eager on the same inputs
            torch.cuda.synchronize()
            eager = snap()
            load(c)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            replay = snap()
            for a, b in zip(eager, replay):
                assert np.array_equal(a, b), (rep, i)
            if rep == 0:
                lat_o, _, st_o, n = oracle.compress(
                    ratio=2, mode=oracle.PREFILL, kv=c["kv"], fused=True, offsets=c["offsets"],
                    start_pos=c["start_pos"], page_table=c["page_table"],
                    state=c["state"].copy(), norm_w=cases[0]["norm_w"], eps=1e-6,
                    freqs=W.rope_freqs(T + 64), cache=np.zeros((c["num_pages"], ps * rb), np.uint8),
                    layout=layout, page_size=ps)
                assert st_o == 0 and int(replay[4][0]) == 0
                assert_latent_close(replay[1].view(np.uint16)[:n], lat_o)


def test_hot_path_graph_replay(K):
    """One step of the path captured in a graph: the prefill compressor, then
    a dequant-gather by physical slot that reads rows the compressor has just
    written (and some it has not, and -1 ids).  Inputs and ids are refreshed
    in place between replays, with eager work between them: every replay
    equals eager calls on the same inputs, bit for bit."""
    layout, ps, S, T, n_ids = "V41", 16, 6, 500, 700
    cases = [W.compress_case(600 + i, W.ragged_lengths(np.random.default_rng(610 + i), T - 30, S),
                             ratio=2, page_size=ps, fused=True, pt_slack=2) for i in range(3)]
    rb = oracle.layout_bytes(layout)[2]
    npg = max(c["num_pages"] for c in cases)
    pts = max(c["page_table"].shape[1] for c in cases)
    proj = torch.zeros((T, 1024), dtype=torch.int16, device="cuda")
    offs = torch.zeros((2, S), dtype=torch.int32, device="cuda")
    start = torch.zeros(S, dtype=torch.int32, device="cuda")
    pt = torch.zeros((S, pts), dtype=torch.int32, device="cuda")
    state = torch.zeros((S, 2, 512), dtype=torch.int16, device="cuda")
    cache = torch.zeros((npg, ps * rb), dtype=torch.uint8, device="cuda")
    lat = torch.zeros((T // 2 + S, 512), dtype=torch.int16, device="cuda")
    ids = torch.zeros(n_ids, dtype=torch.int32, device="cuda")
    out = torch.zeros((n_ids, 512), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    w = dev(cases[0]["norm_w"])
    fr = dev(W.rope_freqs(T + 64))

    def load(i, c):
        proj.zero_()
        proj[:c["kv"].shape[0]].copy_(dev(c["kv"]))
        offs.copy_(dev(c["offsets"]))
        start.copy_(dev(c["start_pos"]))
        pt.zero_()
        pt[:, :c["page_table"].shape[1]].copy_(dev(c["page_table"]))
        state.copy_(dev(c["state"]))
        cache.fill_(0x11)
        lat.zero_()
        out.fill_(7)
        # slots the compressor writes, other slots, and -1
        _, slots = _prefill_slots_of(c)
        rng = np.random.default_rng(620 + i)
        pick = np.concatenate([rng.choice(slots, size=n_ids // 2),
                               rng.integers(0, npg * ps, size=n_ids - n_ids // 2)])
        pick[rng.random(n_ids) < 0.05] = -1
        ids.copy_(torch.from_numpy(rng.permutation(pick).astype(np.int32)))

    def step():
        status.zero_()
        K.kvc_compress_store(ratio=2, mode=K.MODE_PREFILL, kv=proj[:, :512], score=proj[:, 512:],
                             start_pos=start, cache=K.Cache(cache, layout, ps), norm_w=w,
                             eps=1e-6, freqs=fr, latent_out=lat, offsets=offs, page_table=pt,
                             state=state, status=status)
        K.kvc_dequant_gather(K.Cache(cache, layout, ps), None, ids, out, status)

    def snap():
        return [host(t).copy() for t in (cache, lat, state, out, status)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        load(0, cases[0])
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, c in enumerate(cases):
            _say("hot path graph replay", rep, i)
            load(i, c)
            torch.cuda.synchronize()
            step()
            torch.cuda.synchronize()
            eager = snap()
            load(i, c)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            replay = snap()
            assert int(eager[4][0]) == 0
            for a, b in zip(eager, replay):
                assert np.array_equal(a, b), (rep, i)


def _prefill_slots_of(c):
    """(latent rows, cache slots) of a ratio-2 prefill case, in emission order."""
    lat, slots, L = [], [], 0
    ps = c["page_size"]
    for b in range(c["S"]):
        n, p0 = int(c["offsets"][1, b]), int(c["start_pos"][b])
        for q in range(p0, p0 + max(n, 0)):
            if q % 2 == 1:
                cc = q // 2
                slots.append(int(c["page_table"][b, cc // ps]) * ps + cc % ps)
                lat.append(L)
                L += 1
    return lat, slots


# ================================================================= quantizer, exhaustive
def _groups_to_rows(groups, gsize):
    """pack groups of gsize bf16 values into 512-dim rows (zero padded)."""
    per_row = 512 // gsize
    n = -(-len(groups) // per_row)
    rows = np.zeros((n * per_row, gsize), np.uint16)
    rows[:len(groups)] = groups
    return rows.reshape(n, 512)


def _all_finite_bf16_upto(a):
    """every finite bf16 pattern (both signs) with magnitude <= a."""
    b = spec.all_bf16()
    v = np.abs(spec.bf16_value(b))
    return b[v <= a]


def _store_and_compare(K, layout, rows):
    ps = 64
    n = rows.shape[0]
    npages = n // ps + 2
    rb = oracle.layout_bytes(layout)[2]
    loc = (np.arange(n) + ps).astype(np.int32)
    hc = np.zeros((npages, ps * rb), np.uint8)
    dc = dev(hc)
    assert oracle.store_rows(hc, layout, ps, rows, loc) == 0
    K.kvc_store_rows(K.Cache(dc, layout, ps), dev(rows), dev(loc))
    torch.cuda.synchronize()
    g = host(dc)
    bad = np.argwhere(g != hc)
    assert bad.size == 0, bad[:5]


def test_fp8_quantizer_every_value_every_exponent(K):
    """Every finite bf16 value under every ue8m0 exponent it can meet: group g
    holds the amax that gives exponent E and then every bf16 of magnitude up
    to it; the cache bytes equal the oracle's."""
    _say("fp8 quantizer exhaustive")
    top = float(spec.bf16_value(np.uint16(0x7F7F)))
    groups = []
    for E in range(114, 248):
        a = min(448.0 * 2.0 ** (E - 127), top)
        A = spec.bf16_nearest(np.array([a]))[0]
        if spec.bf16_value(A) > a:                     # largest bf16 not above a
            A = np.uint16(A - 1)
        assert oracle.ue8m0(np.array([spec.bf16_value(A)], np.float32))[0] == E
        xs = _all_finite_bf16_upto(float(spec.bf16_value(A)))
        pad = (-len(xs)) % 31
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        groups.append(np.concatenate([np.full((len(xs), 1), A, np.uint16), xs], axis=1))
    rows = _groups_to_rows(np.concatenate(groups), 32)
    _store_and_compare(K, "V41", rows)


def test_fp4_quantizer_every_value_every_scale(K):
    """Every finite bf16 value under every positive finite e4m3 scale it can
    meet (|x| <= 6 s, the group amax 6 s setting the scale s)."""
    _say("fp4 quantizer exhaustive")
    groups = []
    for c in range(1, 0x7F):
        s = float(oracle.e4m3_decode(np.array([c], np.uint8))[0])
        A = spec.bf16_nearest(np.array([6.0 * s]))[0]
        assert spec.bf16_value(A) == 6.0 * s
        assert oracle.fp4_scale(np.array([6.0 * s], np.float32))[0] == c
        xs = _all_finite_bf16_upto(6.0 * s)
        pad = (-len(xs)) % 15
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 15)
        groups.append(np.concatenate([np.full((len(xs), 1), A, np.uint16), xs], axis=1))
    rows = _groups_to_rows(np.concatenate(groups), 16)
    _store_and_compare(K, "V41_FP4", rows)


# ================================================================= launch shapes
@pytest.mark.parametrize("tile_rows", [1, 2, 4])
@pytest.mark.parametrize("layout,ratio,slots", [("V41_FP4", 2, 9), ("V41", 1, 9), ("V4", 2, 90),
                                               ("V41_FP4", 2, 200), ("V41", 1, 300)])
def test_prefill_every_tile_shape(K, tile_rows, layout, ratio, slots):
    """The prefill compressor under each work-item shape (rows per item 1, 2
    or 4) and each slot lookup (one, two or four slots per lane up to 256
    slots; LDS tables above): same rows as the oracle."""
    _say("tile shape", tile_rows, layout, ratio, slots)
    rng = np.random.default_rng(300 + slots + ratio)
    lengths = rng.integers(0, 90, size=slots)
    lengths[rng.random(slots) < 0.15] = 0
    P = rng.integers(0, 120, size=slots)
    case = W.compress_case(310 + tile_rows, lengths, start_pos=P, ratio=ratio, page_size=8,
                           fused=True, gap=2)
    r = run_compress(K, case, layout, ratio, oracle.PREFILL, tile_rows=tile_rows)
    lat, slots_ = [], []
    L = 0
    for b in range(len(lengths)):
        n, p0 = int(lengths[b]), int(P[b])
        qs = range(p0, p0 + n) if ratio == 1 else [q for q in range(p0, p0 + n) if q % 2 == 1]
        for q in qs:
            c = q if ratio == 1 else q // 2
            slots_.append(int(case["page_table"][b, c // 8]) * 8 + c % 8)
            lat.append(L)
            L += 1
    assert r["n_rows"] == L
    check_compress(r, layout, 8, slots_, lat)


@pytest.mark.parametrize("layout,gsize", [("V41_FP4", 16), ("V41", 32)])
def test_group_scale_every_amax(K, layout, gsize):
    """every positive finite bf16 as a group's amax (its sign alternating),
    the rest of the group random below it: scale bytes and codes equal the
    oracle's."""
    _say("scale every amax", layout)
    b = spec.all_bf16()
    b = b[(b & 0x8000) == 0]
    rng = np.random.default_rng(330 + gsize)
    amax = spec.bf16_value(b)
    frac = rng.random((b.size, gsize - 1))
    rest = spec.bf16_nearest(amax[:, None] * frac * np.where(rng.random(frac.shape) < 0.5, -1, 1))
    lead = np.where(np.arange(b.size) % 2 == 1, b | np.uint16(0x8000), b).astype(np.uint16)
    groups = np.concatenate([lead[:, None], rest], axis=1)
    rows = _groups_to_rows(groups, gsize)
    _store_and_compare(K, layout, rows)
