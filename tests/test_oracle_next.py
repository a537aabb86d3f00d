"""Pins of the oracle's verify mode, pending-state ring, decode context
parallelism and RoPE store.  No GPU.

Each test checks the oracle against something other than the function under
test: verify against a sequence of single-token decode calls, draft
rejection against a prefill of the accepted tokens, the DCP ownership rule
against a card-dealing simulation and against the pages' virtual-block
arithmetic, and the rotary store against a complex product rounded by a
nearest-value search.
"""
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


def _verify(case, layout, cache, state, *, mode=oracle.VERIFY, kv=None, start_pos=None,
            out_loc="case", draft_len=None, ring=None, max_out_rows=None, **kw):
    return oracle.compress(
        ratio=case["ratio"], mode=mode, kv=case["kv"] if kv is None else kv, fused=True,
        start_pos=case["pos"] if start_pos is None else start_pos,
        page_table=case["page_table"], out_loc=case["out_loc"] if isinstance(out_loc, str) else out_loc,
        state=state, norm_w=case["norm_w"], eps=case["eps"], freqs=case["freqs"], cache=cache,
        layout=layout, page_size=case["page_size"], max_out_rows=max_out_rows,
        draft_len=case["draft_len"] if draft_len is None else draft_len,
        ring_slots=case["ring_slots"] if ring is None else ring, **kw)


# ---------------------------------------------------------------- verify
@pytest.mark.parametrize("explicit", [False, True])
@pytest.mark.parametrize("ratio,layout", [(2, "V41"), (2, "V41_FP4"), (2, "V4"), (1, "V41")])
def test_verify_equals_sequence_of_decode_calls(ratio, layout, explicit):
    """A verify batch of D drafts per slot gives the same cache, pending ring
    and latent rows as D decode calls that feed the drafts one at a time
    (sglang PR #39652, Review: the decode-or-verify compressor, draft_len 4)."""
    case = W.verify_case(70 + ratio, 48, draft_len=4, ratio=ratio, page_size=16, max_pos=256,
                         ring_slots=3, explicit_out_loc=explicit, skip_frac=0.1)
    S, D = case["S"], case["draft_len"]
    rb = oracle.layout_bytes(layout)[2]
    cache_v = np.full((case["num_pages"], 16 * rb), 0x3C, np.uint8)
    cache_d = cache_v.copy()
    state_v, state_d = case["state"].copy(), case["state"].copy()
    lat_v, pre_v, st, n_rows = _verify(case, layout, cache_v, state_v)
    assert st == 0
    emitted = 0
    for j in range(D):
        rows = case["kv"][np.arange(S) * D + j]
        sp = np.where(case["pos"] < 0, -1, case["pos"] + j).astype(np.int32)
        ol = None if case["out_loc"] is None else case["out_loc"][np.arange(S) * D + j]
        lat_d, pre_d, st_d, n_d = _verify(case, layout, cache_d, state_d, mode=oracle.DECODE,
                                          kv=rows, start_pos=sp, out_loc=ol, draft_len=1)
        assert st_d == 0
        emitted += n_d
        assert np.array_equal(lat_v[np.arange(S) * D + j], lat_d)
        assert np.array_equal(pre_v[np.arange(S) * D + j], pre_d)
    assert emitted == n_rows
    assert np.array_equal(cache_v, cache_d)
    assert np.array_equal(state_v, state_d)
    assert (cache_v != 0x3C).any()


def test_verify_rejection_matches_prefill_of_accepted_tokens():
    """Steps of D = 4 drafts, each accepting a random prefix and restarting
    after it, leave every completed row of the cache and the pending token
    exactly as a prefill of the accepted tokens alone, when the ring has
    D / 2 + 1 entries.  One entry (the plain decode state) loses the pending
    token when a step at an odd position accepts nothing: the negative
    control."""
    D, S, steps, ps = 4, 12, 9, 8
    rng = np.random.default_rng(81)
    base = W.verify_case(82, S, draft_len=D, page_size=ps, max_pos=D * steps + 4, ring_slots=3)
    rb = oracle.layout_bytes("V41")[2]

    def run(ring):
        cache = np.zeros((base["num_pages"], ps * rb), np.uint8)
        state = np.zeros((S, ring, 2, 512), np.uint16)
        pos = np.zeros(S, np.int32)
        accepted = [[] for _ in range(S)]
        r2 = np.random.default_rng(83)
        for _ in range(steps):
            kv = W.normal_bf16(r2, (S * D, 1024))
            acc = r2.integers(0, D + 1, size=S)
            c = dict(base, kv=kv, pos=pos.copy())
            _verify(c, "V41", cache, state, ring=ring)
            for b in range(S):
                accepted[b] += [kv[b * D + j] for j in range(acc[b])]
            pos = pos + acc.astype(np.int32)
        return cache, state, pos, accepted

    cache, state, pos, accepted = run(3)
    # prefill of the accepted tokens from position 0, slot by slot
    lengths = [len(a) for a in accepted]
    proj = np.stack([t for a in accepted for t in a])
    offsets = np.stack([np.cumsum([0] + lengths[:-1]), lengths]).astype(np.int32)
    ref = np.zeros_like(cache)
    ref_state = np.zeros((S, 2, 512), np.uint16)
    oracle.compress(ratio=2, mode=oracle.PREFILL, kv=proj, fused=True, offsets=offsets,
                    start_pos=np.zeros(S, np.int32), page_table=base["page_table"],
                    state=ref_state, norm_w=base["norm_w"], eps=base["eps"],
                    freqs=base["freqs"], cache=ref, layout="V41", page_size=ps)
    db, sb = 512, 16
    for b in range(S):
        for c in range(lengths[b] // 2):
            p, r = base["page_table"][b, c // ps], c % ps
            assert np.array_equal(cache[p, r * db:(r + 1) * db], ref[p, r * db:(r + 1) * db])
            lo = ps * db + r * sb
            assert np.array_equal(cache[p, lo:lo + sb], ref[p, lo:lo + sb])
        if lengths[b] % 2 == 1:                      # a pending token is left
            k = (lengths[b] - 1) // 2
            assert np.array_equal(state[b, k % 3], ref_state[b])
    assert sum(lengths) > S * steps               # the run did accept drafts

    # negative control: one ring entry loses pending tokens on rejection
    cache1, _, _, acc1 = run(1)
    bad = 0
    for b in range(S):
        for c in range(len(acc1[b]) // 2):
            p, r = base["page_table"][b, c // ps], c % ps
            bad += not np.array_equal(cache1[p, r * db:(r + 1) * db], ref[p, r * db:(r + 1) * db])
    assert bad > 0


def test_prefill_uses_ring_entry_of_the_pair():
    """Prefill reads and writes the ring entry of the pending pair (k %
    ring_slots); with the same pending token the rows equal those of the
    one-entry state, and the other entries are left alone."""
    lengths, P = [7, 6, 9, 1], [3, 5, 10, 11]
    case = W.compress_case(84, lengths, start_pos=P, ratio=2, page_size=8, fused=True)
    R = 3
    rb = oracle.layout_bytes("V41_FP4")[2]
    args = dict(ratio=2, mode=oracle.PREFILL, kv=case["kv"], fused=True,
                offsets=case["offsets"], start_pos=case["start_pos"],
                page_table=case["page_table"], norm_w=case["norm_w"], eps=case["eps"],
                freqs=case["freqs"], layout="V41_FP4", page_size=8)
    c1 = np.zeros((case["num_pages"], 8 * rb), np.uint8)
    s1 = case["state"].copy()
    lat1, pre1, st1, _ = oracle.compress(cache=c1, state=s1, **args)
    ring = W.normal_bf16(np.random.default_rng(85), (len(lengths), R, 2, 512))
    for b, p in enumerate(P):
        ring[b, (p // 2) % R] = case["state"][b]       # the pair that starts before p
    ring0 = ring.copy()
    cR = np.zeros_like(c1)
    latR, preR, stR, _ = oracle.compress(cache=cR, state=ring, ring_slots=R, **args)
    assert st1 == stR == 0
    assert np.array_equal(lat1, latR) and np.array_equal(cR, c1)
    for b, (n, p) in enumerate(zip(lengths, P)):
        last = p + n - 1
        for e in range(R):
            if last % 2 == 0 and e == (last // 2) % R:
                assert np.array_equal(ring[b, e], s1[b])
            else:
                assert np.array_equal(ring[b, e], ring0[b, e])


# ---------------------------------------------------------------- DCP
def _deal(n, world, interleave):
    """Deal rows 0..n-1 to the ranks like cards: runs of `interleave`, round
    robin; each rank counts the rows it has received."""
    owner, local, seen = [], [], [0] * world
    rank = run = 0
    for _ in range(n):
        owner.append(rank)
        local.append(seen[rank])
        seen[rank] += 1
        run += 1
        if run == interleave:
            run, rank = 0, (rank + 1) % world
    return owner, local


@pytest.mark.parametrize("world", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("interleave", [1, 2, 8])
def test_dcp_owner_is_the_deal(world, interleave):
    owner, local = _deal(600, world, interleave)
    for c in range(600):
        assert oracle.dcp_owner(c, world, interleave) == (owner[c], local[c])


@pytest.mark.parametrize("world,interleave,bs", [(2, 1, 64), (2, 4, 64), (4, 8, 16), (3, 2, 8)])
def test_dcp_owner_matches_pages_virtual_blocks(world, interleave, bs):
    """flashinfer_sparse.py, DCP helpers: a virtual block of bs*W global states
    spans one page of every rank; the owner is the run of the offset in it
    modulo W and the row in the owner's page packs the owner's runs."""
    for c in range(5000):
        vblock, off = divmod(c, bs * world)
        own = (off // interleave) % world
        row = (off // (interleave * world)) * interleave + off % interleave
        r, loc = oracle.dcp_owner(c, world, interleave)
        assert (r, loc // bs, loc % bs) == (own, vblock, row)


@pytest.mark.parametrize("layout", ["V41", "V41_FP4"])
def test_dcp_compress_partitions_the_rows(layout):
    """With the rows dealt over W ranks, each rank stores exactly its own rows,
    at its own page-table slot, with the bytes the single-rank compressor
    stores; the latent rows are the same on every rank."""
    world, K, ps = 3, 2, 8
    lengths, P = [23, 0, 40, 9], [0, 0, 5, 2]
    case = W.compress_case(86, lengths, start_pos=P, ratio=2, page_size=ps, fused=True)
    db, sb, rb, _ = oracle.layout_bytes(layout)
    args = dict(ratio=2, mode=oracle.PREFILL, kv=case["kv"], fused=True,
                offsets=case["offsets"], start_pos=case["start_pos"], norm_w=case["norm_w"],
                eps=case["eps"], freqs=case["freqs"], layout=layout, page_size=ps)
    ref = np.zeros((case["num_pages"], ps * rb), np.uint8)
    lat1, _, st, n = oracle.compress(page_table=case["page_table"], cache=ref,
                                     state=case["state"].copy(), **args)
    assert st == 0
    tables, npg = W.per_rank_page_tables(87, world, len(lengths), case["page_table"].shape[1])
    caches = [np.full((npg, ps * rb), 0xEE, np.uint8) for _ in range(world)]
    for r in range(world):
        lat, _, st, _ = oracle.compress(page_table=tables[r], cache=caches[r],
                                        state=case["state"].copy(), dcp_world=world, dcp_rank=r,
                                        dcp_interleave=K, **args)
        assert st == 0 and np.array_equal(lat, lat1)
    owner, local = _deal(64, world, K)
    stored = [0] * world
    for b, (nn, p) in enumerate(zip(lengths, P)):
        for c in range(p // 2, (p + nn) // 2):     # pairs closed in the extend
            pr, rr = case["page_table"][b, c // ps], c % ps
            r, u = owner[c], local[c]
            pp, ru = tables[r][b, u // ps], u % ps
            assert np.array_equal(caches[r][pp, ru * db:(ru + 1) * db], ref[pr, rr * db:(rr + 1) * db])
            lo, lo2 = ps * db + ru * sb, ps * db + rr * sb
            assert np.array_equal(caches[r][pp, lo:lo + sb], ref[pr, lo2:lo2 + sb])
            stored[r] += 1
    for r in range(world):     # nothing else was written on any rank
        assert (caches[r] != 0xEE).sum() <= stored[r] * rb


@pytest.mark.parametrize("world,interleave", [(1, 1), (2, 1), (4, 4), (3, 2)])
def test_dcp_filter_against_brute_force(world, interleave):
    ps = 16
    c = W.dcp_ids_case(88 + world, T=40, k=96, n_req=5, max_rows=400, world=world,
                       page_size=ps)
    owner, local = _deal(400, world, interleave)
    total = 0
    for rank in range(world):
        bt = c["block_tables"][rank]
        slots, lens, st = oracle.dcp_filter_ids(
            c["ids"], c["token_to_req"], bt, page_size=ps, num_pages=c["num_pages"],
            world=world, rank=rank, interleave=interleave, valid=c["valid"])
        assert st == 0
        for t in range(c["ids"].shape[0]):
            want = []
            if c["valid"][t]:
                for i in c["ids"][t]:
                    if i >= 0 and owner[i] == rank:
                        u = local[i]
                        want.append(int(bt[c["token_to_req"][t], u // ps]) * ps + u % ps)
            assert lens[t] == len(want)
            assert list(slots[t, :len(want)]) == want
            assert np.all(slots[t, len(want):] == -1)
        total += int(lens.sum())
    # the ranks' shares partition the valid ids of the valid rows
    assert total == int(((c["ids"] >= 0) & (c["valid"][:, None] != 0)).sum())


def test_dcp_filter_status_and_single_rank():
    ps = 8
    ids = np.array([[5, -1, 17, 3], [40, 2, -1, -1], [1, 2, 3, 4]], np.int32)
    t2r = np.array([0, 1, 7], np.int32)                       # request 7 does not exist
    bt = np.array([[3, 4, 5], [6, -2, 9]], np.int32)          # -2: a bad page
    slots, lens, st = oracle.dcp_filter_ids(ids, t2r, bt, page_size=ps, num_pages=20, world=1,
                                            rank=0, interleave=1)
    # world 1: the block-table mapping with the -1 entries squeezed out
    assert list(slots[0]) == [3 * 8 + 5, 5 * 8 + 1, 3 * 8 + 3, -1] and lens[0] == 3
    # id 40 is past the 3-entry table row; id 2 maps through page 6
    assert list(slots[1]) == [6 * 8 + 2, -1, -1, -1] and lens[1] == 1
    assert lens[2] == 0 and np.all(slots[2] == -1)
    assert st == oracle.ST_PT_RANGE | oracle.ST_REQ_RANGE
    _, _, st = oracle.dcp_filter_ids(np.array([[9]], np.int32), np.array([1], np.int32), bt,
                                     page_size=ps, num_pages=20, world=1, rank=0, interleave=1)
    assert st == oracle.ST_PAGE_RANGE


# ---------------------------------------------------------------- RoPE store
def _table(cos, sin, n=4):
    f = np.empty((n, 64), np.float32)
    f[:, 0::2], f[:, 1::2] = cos, sin
    return f


def _store_args(c, layout):
    rb = oracle.layout_bytes(layout)[2]
    return np.zeros((c["num_pages"], c["page_size"] * rb), np.uint8)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_rope_store_identity_and_quarter_turn(layout):
    """cos = 1, sin = 0 is the plain store; cos = 0, sin = 1 maps each rope
    pair (a, b) to (-b, a) exactly."""
    c = W.rope_store_case(90, [70, 33], page_size=16, max_pos=4)
    rows, ol = c["rows"], c["out_loc"]
    pos = np.zeros(len(rows), np.int32)
    a, b = _store_args(c, layout), _store_args(c, layout)
    rot, st = oracle.store_rows_rope(a, layout, 16, rows, pos, _table(1.0, 0.0), ol)
    assert st == 0
    assert oracle.store_rows(b, layout, 16, rows, ol) == 0
    assert np.array_equal(a, b)
    kept = ol != 0
    assert np.array_equal(rot[kept], rows[kept]) and np.all(rot[~kept] == 0)
    a2, b2 = _store_args(c, layout), _store_args(c, layout)
    rot, st = oracle.store_rows_rope(a2, layout, 16, rows, pos, _table(0.0, 1.0), ol)
    swapped = rows.copy()
    swapped[:, 448::2] = rows[:, 449::2] ^ np.uint16(0x8000)
    swapped[:, 449::2] = rows[:, 448::2]
    assert np.array_equal(rot[kept], swapped[kept])
    oracle.store_rows(b2, layout, 16, swapped, ol)
    assert np.array_equal(a2, b2)


def test_rope_store_against_complex_product():
    """General angles: the rotated pair is the fp64 complex product (a + ib)(c
    + is) rounded to the nearest bf16 (search over every bf16 value)."""
    c = W.rope_store_case(91, [300], page_size=16, max_pos=2048, pad_frac=0.0)
    rows, pos, fr = c["rows"], c["positions"], c["freqs"]
    cache = _store_args(c, "V41")
    rot, st = oracle.store_rows_rope(cache, "V41", 16, rows, pos, fr, c["out_loc"])
    assert st == 0
    x = spec.bf16_value(rows[:, 448:])
    cs = fr[pos].astype(np.float64)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * (cs[:, 0::2] + 1j * cs[:, 1::2])
    want = np.empty_like(x)
    want[:, 0::2], want[:, 1::2] = z.real, z.imag
    assert np.array_equal(rot[:, 448:], spec.bf16_nearest(want))
    assert np.array_equal(rot[:, :448], rows[:, :448])


def test_rope_store_status_and_padding():
    c = W.rope_store_case(92, [64], page_size=16, max_pos=32, pad_frac=0.2, bad_pos_frac=0.3)
    cache = _store_args(c, "V41_FP4")
    rot, st = oracle.store_rows_rope(cache, "V41_FP4", 16, c["rows"], c["positions"],
                                     c["freqs"], c["out_loc"])
    bad = (c["positions"] < 0) | (c["positions"] >= 32)
    assert st == (oracle.ST_POS_RANGE if np.any(bad & (c["out_loc"] != 0)) else 0)
    stored = (~bad) & (c["out_loc"] != 0)
    assert np.all(rot[~stored] == 0) and np.all(np.any(rot[stored] != 0, axis=1))
    assert (cache != 0).sum() <= stored.sum() * 288
