"""Seeded synthetic inputs for the compressed-KV store and gather.

This module only draws inputs: random bf16 rows, page tables, gather ids,
ragged offsets, a RoPE frequency table and random cache bytes.  It holds none
of the method's arithmetic (no pooling, normalisation, rotation, quantisation
or address computation), so that the oracle under ``oracle/`` and the HIP
path can both consume the same inputs without sharing any of the method's code.

Every array is host memory (numpy).  bf16 tensors are carried as ``uint16``
bit patterns.  Each generator takes a ``seed``; the named workloads use
``20261202 + k`` for workload k (k = 1..5), so a run is reproducible.

Shapes and distributions follow the workloads of the DeepSeek-V4.1 low-ratio
compressed-KV path: 512-dim latent rows (448 "nope" + 64 "rope" dims),
``|kv|score|`` projection rows for ratio 2, int32 ``[2, slots]`` extend
offsets (sglang PR #46230, summary), page tables with physical page 0 kept
back as the padding page, and gather ids drawn without replacement.
"""
from __future__ import annotations

import numpy as np
import torch

D = 512            # latent width of one compressed KV row
ROPE_DIMS = 64     # the last 64 dims carry the rotary part
BASE_SEED = 20261202

__all__ = [
    "D", "ROPE_DIMS", "BASE_SEED", "bf16_bits", "bf16_to_f32", "normal_bf16",
    "norm_weight", "rope_freqs", "outlier_rows", "random_pages",
    "paged_cache_shape", "random_cache_bytes", "compress_case", "decode_case",
    "store_case", "gather_case", "ragged_lengths", "verify_case", "rope_store_case",
    "dcp_ids_case", "per_rank_page_tables", "workload_c4_id_sets",
    "workload_c4_disjoint_id_sets",
    "workload_c1", "workload_c2", "workload_c3", "workload_c4", "workload_c5",
]


# --------------------------------------------------------------------------
# element helpers (type plumbing only)
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 samples -> bf16 bit patterns (uint16), round to nearest even.

    Uses torch's CPU dtype conversion; it only prepares inputs."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def norm_weight(rng: np.random.Generator) -> np.ndarray:
    """RMSNorm weight, bf16 ``1 + 0.1 * N(0, 1)`` over the 512 dims."""
    return bf16_bits(1.0 + 0.1 * rng.standard_normal(D).astype(np.float32))


def rope_freqs(max_pos: int, theta: float = 10000.0) -> np.ndarray:
    """fp32 ``[max_pos, 64]`` rotary table: entry ``[p, 2j]`` is cos(p*t_j),
    ``[p, 2j+1]`` is sin(p*t_j), with ``t_j = theta ** (-2j / 64)``.

    Computed in fp64 and rounded once to fp32.  This is the model's
    precomputed position table, an input of the compressor, handed unchanged to
    both the oracle and the kernel."""
    j = np.arange(ROPE_DIMS // 2, dtype=np.float64)
    inv = theta ** (-2.0 * j / ROPE_DIMS)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    out = np.empty((max_pos, ROPE_DIMS), dtype=np.float32)
    out[:, 0::2] = np.cos(ang)
    out[:, 1::2] = np.sin(ang)
    return out


def outlier_rows(rng: np.random.Generator, n: int, n_out: int = 4,
                 factor: float = 50.0, zero_frac: float = 0.01) -> np.ndarray:
    """bf16 ``[n, 512]`` rows ~N(0,1) with ``n_out`` distinct random channels
    per row scaled by ``factor`` (in fp32, before the bf16 rounding) and each
    row zeroed with probability ``zero_frac``."""
    x = rng.standard_normal((n, D), dtype=np.float32)
    if n and n_out:
        ch = np.argsort(rng.random((n, D)), axis=1)[:, :n_out]
        np.put_along_axis(x, ch, np.take_along_axis(x, ch, axis=1) * factor, axis=1)
    if n and zero_frac > 0:
        x[rng.random(n) < zero_frac] = 0.0
    return bf16_bits(x)


def random_pages(rng: np.random.Generator, count: int, num_pages: int) -> np.ndarray:
    """``count`` distinct physical pages drawn from 1..num_pages-1 (page 0 is
    the padding page and is never handed out)."""
    assert count <= num_pages - 1
    return (rng.permutation(num_pages - 1)[:count] + 1).astype(np.int32)


def paged_cache_shape(num_pages: int, page_size: int, row_bytes: int) -> tuple[int, int]:
    """Byte shape ``[num_pages, page_stride]`` of a cache whose pages are
    packed back to back (page_stride = page_size * row_bytes)."""
    return num_pages, page_size * row_bytes


def random_cache_bytes(rng: np.random.Generator, nbytes: int) -> np.ndarray:
    """``nbytes`` random bytes with no fp8 e4m3fn NaN pattern (0x7F, 0xFF):
    a byte whose low seven bits are all set has its lowest bit cleared, so
    0x7E and 0xFE are drawn twice as often as the other values."""
    n8 = (nbytes + 7) // 8
    w = rng.bit_generator.random_raw(n8)
    t = w & np.uint64(0x7F7F7F7F7F7F7F7F)
    t += np.uint64(0x0101010101010101)
    t &= np.uint64(0x8080808080808080)
    t >>= np.uint64(7)
    w ^= t
    return w.view(np.uint8)[:nbytes]


def fill_scale_sections(cache: np.ndarray, page_size: int, data_bytes: int,
                        scale_bytes: int, values: np.ndarray) -> None:
    """Overwrite the scale section of every page (``cache`` is
    ``[num_pages, page_stride]`` bytes) with ``values`` (same length as the
    section).  Used to put chosen scale bytes in a randomly filled cache."""
    lo = page_size * data_bytes
    cache[:, lo:lo + page_size * scale_bytes] = values.reshape(cache.shape[0], -1)


# --------------------------------------------------------------------------
# ragged batches
# --------------------------------------------------------------------------
def ragged_lengths(rng: np.random.Generator, total: int, parts: int) -> np.ndarray:
    """``parts`` positive lengths summing to ``total``: differences of
    ``parts-1`` sorted distinct uniform cut points in [1, total-1]."""
    cuts = np.sort(rng.choice(np.arange(1, total), size=parts - 1, replace=False))
    edges = np.concatenate([[0], cuts, [total]])
    return np.diff(edges).astype(np.int32)


def compress_case(seed: int, lengths, start_pos=None, ratio: int = 2,
                  page_size: int = 64, fused: bool = True, gap: int = 0,
                  extra_slots: int = 0, pt_slack: int = 1,
                  state_random: bool = True, max_pos: int | None = None,
                  spare_pages: int = 4):
    """Prefill compress inputs for a ragged batch.

    lengths     extend length per request slot (0 = empty slot)
    start_pos   position of each slot's first extend token (default 0)
    fused       one ``|kv|score|`` buffer ``[T, 1024]`` (True) or separate
                ``kv``/``score`` buffers ``[T, 512]``
    gap         padding tokens inserted between consecutive requests (rows of
                the projection buffer that belong to no request)
    extra_slots trailing slots with no rows
    Page tables give every slot ``pt_slack`` more logical pages than its
    compressed rows need; pages are distinct and never page 0.
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    S = len(lengths) + extra_slots
    n = np.concatenate([lengths, np.zeros(extra_slots, np.int32)]).astype(np.int32)
    P = np.zeros(S, np.int32) if start_pos is None else np.concatenate(
        [np.asarray(start_pos, np.int32), np.zeros(extra_slots, np.int32)])
    first = np.zeros(S, np.int32)
    cur = 0
    for b in range(S):
        first[b] = cur
        cur += int(n[b]) + (gap if n[b] > 0 else 0)
    T = max(cur, 1)
    offsets = np.stack([first, n]).astype(np.int32)          # [2, S]
    # logical compressed pages per slot: enough for the last position touched
    last_pos = P + np.maximum(n, 1)
    pages_needed = (last_pos // ratio) // page_size + 1 + pt_slack
    pt_stride = int(pages_needed.max())
    num_pages = int(pages_needed.sum()) + 1 + spare_pages
    perm = random_pages(rng, int(pages_needed.sum()), num_pages)
    page_table = np.zeros((S, pt_stride), np.int32)
    k = 0
    for b in range(S):
        m = int(pages_needed[b])
        page_table[b, :m] = perm[k:k + m]
        k += m
    if fused:
        proj = normal_bf16(rng, (T, 2 * D))
        kv, score = proj, None
    else:
        kv = normal_bf16(rng, (T, D))
        score = normal_bf16(rng, (T, D)) if ratio == 2 else None
    state = normal_bf16(rng, (S, 2, D)) if state_random else np.zeros((S, 2, D), np.uint16)
    w = norm_weight(rng)
    if max_pos is None:
        max_pos = int(last_pos.max()) + 2
    return dict(ratio=ratio, fused=fused, kv=kv, score=score, offsets=offsets,
                start_pos=P, page_table=page_table, page_size=page_size,
                num_pages=num_pages, state=state, norm_w=w, eps=1e-6,
                freqs=rope_freqs(max_pos), T=T, S=S)


def decode_case(seed: int, batch: int, ratio: int = 2, page_size: int = 64,
                max_pos: int = 16384, explicit_out_loc: bool = True):
    """Decode compress inputs: one new token per slot.

    Positions are uniform in 1..max_pos-1.  With ``explicit_out_loc`` the
    destination slot of every row is drawn directly (distinct slots in pages
    1..); tokens that complete no row get 0.  Otherwise a per-slot page table
    covers the positions.  Odd-position slots (ratio 2) have a random pending
    token in ``state``."""
    rng = np.random.default_rng(seed)
    pos = rng.integers(1, max_pos, size=batch).astype(np.int32)
    proj = normal_bf16(rng, (batch, 2 * D))
    state = normal_bf16(rng, (batch, 2, D))
    w = norm_weight(rng)
    if ratio == 2:
        completes = (pos % 2) == 1
    else:
        completes = np.ones(batch, bool)
    num_pages = batch + 2
    out_loc = None
    page_table = None
    pt_stride = 0
    if explicit_out_loc:
        slots = rng.permutation((num_pages - 1) * page_size)[:batch] + page_size
        out_loc = np.where(completes, slots, 0).astype(np.int32)
    else:
        pt_stride = (max_pos // ratio) // page_size + 1
        pages = random_pages(rng, batch, num_pages)
        page_table = np.zeros((batch, pt_stride), np.int32)
        # each slot only needs the page that holds its current compressed row;
        # the other entries stay 0 (unallocated), as in a sparse block table
        cidx = pos // ratio
        page_table[np.arange(batch), cidx // page_size] = pages
    return dict(ratio=ratio, kv=proj, pos=pos, out_loc=out_loc,
                page_table=page_table, pt_stride=pt_stride, page_size=page_size,
                num_pages=num_pages, state=state, norm_w=w, eps=1e-6,
                freqs=rope_freqs(max_pos), S=batch)


def store_case(seed: int, lengths, page_size: int = 64, spare_pages: int = 2):
    """Plain store inputs: outlier rows and the destination slot of each row.

    Every request gets its own random pages and its rows fill the slots of
    those pages in order.  The slot list is the caller-provided ``out_loc``
    of a store, so it is an input here."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    N = int(lengths.sum())
    rows = outlier_rows(rng, N)
    npg = (lengths + page_size - 1) // page_size
    num_pages = int(npg.sum()) + 1 + spare_pages
    pages = random_pages(rng, int(npg.sum()), num_pages)
    out_loc = np.empty(N, np.int32)
    k = r = 0
    for b, L in enumerate(lengths):
        # the allocator hands request b the slots of its pages in order
        slots = np.concatenate([np.arange(p * page_size, (p + 1) * page_size)
                                for p in pages[k:k + npg[b]]])
        out_loc[r:r + L] = slots[:L]
        k += int(npg[b])
        r += int(L)
    return dict(rows=rows, out_loc=out_loc, num_pages=num_pages,
                page_size=page_size, lengths=lengths.astype(np.int32))


def gather_case(seed: int, logical_pages: int, page_size: int, n_ids: int,
                row_bytes: int, data_bytes: int, scale_bytes: int,
                scale_lo: int | None = 114, scale_hi: int | None = 140):
    """Gather inputs: a randomly filled paged cache, a random page table (a
    permutation of physical pages 1..logical_pages) and ``n_ids`` distinct
    logical row ids in random order.

    Data bytes are random valid fp8/fp4 codes; when ``scale_lo`` is given the
    scale section holds uniform bytes in [scale_lo, scale_hi] (ue8m0
    exponents), otherwise random bytes with no e4m3 NaN pattern."""
    rng = np.random.default_rng(seed)
    num_pages = logical_pages + 1
    stride = page_size * row_bytes
    cache = random_cache_bytes(rng, num_pages * stride).reshape(num_pages, stride)
    if scale_lo is not None:
        sc = rng.integers(scale_lo, scale_hi + 1, size=num_pages * page_size * scale_bytes,
                          dtype=np.uint8)
        fill_scale_sections(cache, page_size, data_bytes, scale_bytes, sc)
    page_table = (rng.permutation(logical_pages) + 1).astype(np.int32)
    ids = rng.choice(logical_pages * page_size, size=n_ids, replace=False).astype(np.int32)
    return dict(cache=cache, page_table=page_table, ids=ids, num_pages=num_pages,
                page_size=page_size, page_stride=stride)


def verify_case(seed: int, batch: int, draft_len: int = 4, ratio: int = 2,
                page_size: int = 16, max_pos: int = 512, ring_slots: int = 3,
                explicit_out_loc: bool = False, skip_frac: float = 0.0,
                pad_frac: float = 0.0625):
    """Speculative-decoding verify inputs: ``batch`` slots with ``draft_len``
    tokens each (token j of slot b is row ``b*draft_len + j`` of a fused
    ``|kv|score|`` buffer), start positions uniform in [0, max_pos -
    draft_len], a fraction ``skip_frac`` of slots with start position -1 and
    a random pending-state ring ``[batch, ring_slots, 2, 512]``.

    With ``explicit_out_loc`` every token gets its own destination slot
    (distinct, pages 1..), a fraction ``pad_frac`` of them 0 (padded).
    Otherwise each slot gets a page table of distinct random pages covering
    every position below ``max_pos``."""
    rng = np.random.default_rng(seed)
    n_tok = batch * draft_len
    pos = rng.integers(0, max_pos - draft_len + 1, size=batch).astype(np.int32)
    if skip_frac > 0:
        pos[rng.random(batch) < skip_frac] = -1
    proj = normal_bf16(rng, (n_tok, 2 * D))
    state = normal_bf16(rng, (batch, ring_slots, 2, D))
    w = norm_weight(rng)
    out_loc = page_table = None
    if explicit_out_loc:
        num_pages = n_tok // page_size + 3
        slots = rng.permutation((num_pages - 1) * page_size)[:n_tok] + page_size
        slots[rng.random(n_tok) < pad_frac] = 0
        out_loc = slots.astype(np.int32)
    else:
        lp = (max_pos // ratio) // page_size + 1
        num_pages = batch * lp + 1
        page_table = random_pages(rng, batch * lp, num_pages).reshape(batch, lp)
    return dict(ratio=ratio, kv=proj, pos=pos, out_loc=out_loc, page_table=page_table,
                page_size=page_size, num_pages=num_pages, state=state, norm_w=w, eps=1e-6,
                freqs=rope_freqs(max_pos), S=batch, draft_len=draft_len,
                ring_slots=ring_slots)


def rope_store_case(seed: int, lengths, page_size: int = 64, max_pos: int = 4096,
                    pad_frac: float = 0.03, bad_pos_frac: float = 0.0):
    """Store-with-RoPE inputs: ``store_case`` rows and slots plus a rotary
    position per row (uniform in [0, max_pos)), a fraction ``pad_frac`` of
    rows padded (out_loc 0) and a fraction ``bad_pos_frac`` given a position
    outside the table."""
    c = store_case(seed, lengths, page_size=page_size)
    rng = np.random.default_rng(seed + 1)
    n = c["rows"].shape[0]
    pos = rng.integers(0, max_pos, size=n).astype(np.int32)
    if bad_pos_frac > 0:
        bad = rng.random(n) < bad_pos_frac
        pos[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, max_pos + 7)
    out_loc = c["out_loc"].copy()
    out_loc[rng.random(n) < pad_frac] = 0
    c.update(positions=pos, out_loc=out_loc, freqs=rope_freqs(max_pos))
    return c


def per_rank_page_tables(seed: int, world: int, slots: int, entries: int):
    """One page table per rank of a context-parallel group: ``[world, slots,
    entries]`` distinct random pages of that rank's own cache (never page
    0); returns (tables, pages per rank cache)."""
    rng = np.random.default_rng(seed)
    num_pages = slots * entries + 1
    t = np.stack([random_pages(rng, slots * entries, num_pages).reshape(slots, entries)
                  for _ in range(world)])
    return t, num_pages


def dcp_ids_case(seed: int, T: int, k: int, n_req: int, max_rows: int, world: int,
                 page_size: int, neg_frac: float = 0.05, invalid_frac: float = 0.05):
    """Global compressed-row ids for a context-parallel gather: ``T`` token
    rows (request of each row sorted, uniform over ``n_req`` requests), each
    with ``k`` distinct ids below its request's row count (uniform in
    [1, max_rows]) in random order, a fraction ``neg_frac`` replaced by -1
    (and -1 wherever the request has fewer than k rows); per-rank block
    tables ``[world, n_req, entries]`` of distinct random pages with
    ``entries`` = max_rows // page_size + 1; a ``valid`` flag per row with
    a fraction ``invalid_frac`` of zeros (graph padding tokens)."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(1, max_rows + 1, size=n_req)
    t2r = np.sort(rng.integers(0, n_req, size=T)).astype(np.int32)
    ids = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = int(rows[t2r[t]])
        m = min(n, k)
        ids[t, :m] = rng.choice(n, size=m, replace=False)
        ids[t] = ids[t, rng.permutation(k)]
    ids[rng.random((T, k)) < neg_frac] = -1
    entries = max_rows // page_size + 1
    bt, num_pages = per_rank_page_tables(seed + 1, world, n_req, entries)
    valid = (rng.random(T) >= invalid_frac).astype(np.int32)
    return dict(ids=ids, token_to_req=t2r, block_tables=bt, num_pages=num_pages,
                valid=valid, rows=rows.astype(np.int32), page_size=page_size)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
def workload_c1():
    """Ratio-2 compress of one 64-token request (separate kv / score
    buffers, page 64, V41), then a gather of its 32 rows."""
    c = compress_case(BASE_SEED + 1, [64], ratio=2, page_size=64, fused=False,
                      pt_slack=0, state_random=False, spare_pages=0)
    return c


def workload_c2():
    """Ratio-1 store of 8 requests with extend lengths uniform in
    [512, 4096]: outlier rows, page 64."""
    rng = np.random.default_rng(BASE_SEED + 2)
    lengths = rng.integers(512, 4097, size=8)
    return store_case(BASE_SEED + 2, lengths, page_size=64)


def workload_c3(seed_offset: int = 0):
    """Ratio-2 ragged prefill: 16 requests totalling 32768 tokens, fused
    ``|kv|score|`` buffer, page 128.  The seed is advanced until at least two
    lengths are odd; the seed used is returned."""
    s = BASE_SEED + 3 + seed_offset
    while True:
        lengths = ragged_lengths(np.random.default_rng(s), 32768, 16)
        if int((lengths % 2).sum()) >= 2:
            break
        s += 1000
    c = compress_case(s, lengths, ratio=2, page_size=128, fused=True,
                      state_random=False)
    c["seed"] = s
    c["lengths"] = lengths
    return c


def workload_c4(n_ids: int = 262144, logical_pages: int = 16384, page_size: int = 64):
    """V41 cache of 16384 logical pages x 64 rows (1,048,576 rows), random
    page table, 262,144 distinct gather ids."""
    return gather_case(BASE_SEED + 4, logical_pages, page_size, n_ids,
                       row_bytes=528, data_bytes=512, scale_bytes=16)


def workload_c4_id_sets(count: int, n_ids: int = 262144, logical_pages: int = 16384,
                        page_size: int = 64):
    """``count`` id lists of the C4 gather: the workload's own list first,
    then lists of the same size drawn the same way from other seeds (so that
    consecutive gathers of a timing loop read different rows)."""
    sets = [workload_c4(n_ids, logical_pages, page_size)["ids"]]
    for j in range(1, count):
        rng = np.random.default_rng(BASE_SEED + 4 + 1000 * j)
        sets.append(rng.choice(logical_pages * page_size, size=n_ids,
                               replace=False).astype(np.int32))
    return sets


def workload_c4_disjoint_id_sets(count: int, n_ids: int = 262144, logical_pages: int = 16384,
                                 page_size: int = 64):
    """``count`` id lists of the C4 gather that share no row: the workload's
    own list first, then lists drawn without replacement from the rows it
    leaves (so a timing loop's consecutive gathers read different rows)."""
    first = workload_c4(n_ids, logical_pages, page_size)["ids"]
    total = logical_pages * page_size
    assert count * n_ids <= total
    rest = np.setdiff1d(np.arange(total, dtype=np.int32), first)
    rest = np.random.default_rng(BASE_SEED + 4 + 7000).permutation(rest)
    return [first] + [rest[j * n_ids:(j + 1) * n_ids].astype(np.int32).copy()
                      for j in range(count - 1)]


def workload_c5(batch: int = 1024):
    """Decode: 1024 slots x 1 new token at ratio 2, explicit out_loc (0 for
    tokens that complete no row), page 64, V4 layout."""
    return decode_case(BASE_SEED + 5, batch, ratio=2, page_size=64)
