"""The oracle model of the dequant-reuse head (sglang PR #45909, summary)
pinned to the page's rules, and the C ABI's reuse head compared with it
operation by operation (hit / miss is an exact, integer result)."""
import ctypes as C
import itertools

import numpy as np
import pytest

import oracle
from oracle.reuse_head import SparsePrefillKVBuffer
import workloads as W


def _counting():
    calls = []

    def dq(source, ids, n):
        calls.append((source, ids, n))
        return np.full((n, 2), len(calls), np.int64)     # rows stamped by run
    return dq, calls


def test_head_rules_from_the_page():
    """Matching (source, ids, row count) hits; each forget event named on
    the page -- a plain get, a reallocation, a new forward -- forces the next
    get_with_head to miss; a change of any key part misses."""
    dq, calls = _counting()
    buf = SparsePrefillKVBuffer(dq)
    rows, hit = buf.get_with_head("A", "ids0", 8)
    assert not hit and len(calls) == 1
    again, hit = buf.get_with_head("A", "ids0", 8)
    assert hit and len(calls) == 1 and again is rows        # no dequant ran
    for other in (("B", "ids0", 8), ("A", "ids1", 8), ("A", "ids0", 7)):
        buf.get_with_head("A", "ids0", 8)
        _, hit = buf.get_with_head(*other)
        assert not hit
    for forget in (lambda: buf.get("A", "ids0", 8), buf.reallocate, buf.begin_forward):
        buf.get_with_head("A", "ids0", 8)
        _, hit = buf.get_with_head("A", "ids0", 8)
        assert hit
        forget()
        n_before = len(calls)
        _, hit = buf.get_with_head("A", "ids0", 8)
        assert not hit and len(calls) == n_before + 1       # the miss ran the dequant


def test_plain_get_runs_the_dequant_and_keeps_no_head():
    dq, calls = _counting()
    buf = SparsePrefillKVBuffer(dq)
    buf.get("A", "i", 4)
    buf.get("A", "i", 4)
    assert len(calls) == 2 and buf.head is None


def test_reused_rows_equal_a_fresh_dequant():
    """With the oracle's gather as the dequant: every hit of a sequence of
    layers returns exactly the rows a fresh gather of the same ids gives
    (the page's verification), for several sources and id lists."""
    rng = np.random.default_rng(9100)
    caches = {}
    for s, layout in enumerate(("V41", "V41_FP4", "V4")):
        c = W.gather_case(9101 + s, logical_pages=6, page_size=16, n_ids=40,
                          **dict(zip(("row_bytes", "data_bytes", "scale_bytes"),
                                     {"V41": (528, 512, 16), "V41_FP4": (288, 256, 32),
                                      "V4": (584, 576, 8)}[layout])))
        caches[s] = (c, layout)
    id_lists = {j: rng.choice(96, size=40, replace=False).astype(np.int32) for j in range(3)}

    def fresh(source, ids, n):
        c, layout = caches[source]
        out, st = oracle.dequant_gather(c["cache"], layout, 16, c["page_table"], id_lists[ids][:n])
        assert st == 0
        return out

    buf = SparsePrefillKVBuffer(fresh)
    hits = 0
    for layer in range(60):
        if layer % 12 == 0:
            buf.begin_forward()
        src, ids, n = int(rng.integers(0, 3)), int(rng.integers(0, 3)), int(rng.integers(30, 41))
        if rng.random() < 0.6 and buf.head is not None:
            src, ids, n = buf.head                        # the next layer reads the same source
        rows, hit = buf.get_with_head(src, ids, n)
        hits += hit
        assert np.array_equal(rows, fresh(src, ids, n))
    assert hits > 10


FAKE = 0x7F0000000000     # never dereferenced: every gather below has n = 0 or is refused


def test_c_abi_head_follows_the_model():
    """A random sequence of gets with reuse, plain gets, reallocations (a new
    output buffer) and new forwards over three sources, three id lists and
    two row counts: kvc_dequant_gather_reuse's hit flags equal the model's at
    every step.  The C calls use n = 0 so that nothing is launched (the key
    logic is the same); each (id list, row count) of the model is its own id
    buffer there."""
    import fp8_fp4_quantized_amd as kvc
    L = kvc.lib()
    rng = np.random.default_rng(9200)
    sources = [kvc.kvc_cache(FAKE + (i << 24), 1, 64, 64 * 528, 16) for i in range(3)]
    page_tables = [FAKE + (7 << 28) + 4096 * i for i in range(3)]
    outs = itertools.count()
    out_ptr = [FAKE + (11 << 28)]

    def ids_ptr(ids, n_key):
        # one distinct id buffer per (id list, row count) of the model: the
        # C key then differs exactly where the model's does
        return FAKE + (9 << 28) + 65536 * (4 * ids + n_key)

    def c_get_with_head(src, ids, n_key):
        hit = C.c_int32(-1)
        rc = L.kvc_dequant_gather_reuse(kb, C.byref(sources[src]), page_tables[src], 16,
                                        ids_ptr(ids, n_key), 0, out_ptr[0], 512, None,
                                        C.byref(hit), None)
        assert rc == kvc.KVC_OK
        return bool(hit.value)

    kb = L.kvc_kvbuf_create()
    model = SparsePrefillKVBuffer(lambda s, i, n: None)
    for step in range(400):
        op = rng.choice(["reuse", "reuse", "reuse", "same", "get", "realloc", "forward"])
        if op == "same" and model.head is not None:
            src, ids, n = model.head
            op = "reuse"
        else:
            src, ids, n = int(rng.integers(0, 3)), int(rng.integers(0, 3)), int(rng.integers(1, 3))
        if op == "reuse":
            _, want = model.get_with_head(src, ids, n)
            assert c_get_with_head(src, ids, n) == want, step
        elif op == "get":
            model.get(src, ids, n)
            L.kvc_kvbuf_forget(kb)          # a plain get: the gather runs, the head is dropped
        elif op == "realloc":
            model.reallocate()
            out_ptr[0] = FAKE + (11 << 28) + 65536 * (next(outs) + 1)
        else:
            model.begin_forward()
            L.kvc_kvbuf_begin_forward(kb)
    L.kvc_kvbuf_destroy(kb)
