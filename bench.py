"""Benchmark of the DeepSeek-V4.1 low-ratio compressed-KV hot path on one
MI355X.

One step = one pass of both halves of the path over one batch:
  1. compress-store: ratio-2 ragged prefill of 16 requests totalling 32,768
     tokens (fused |kv|score| bf16 [32768, 1024], page 128, V41_FP4 cache);
  2. dequant-gather: 262,144 distinct ids from a V41 cache of 1,048,576 rows
     (16,384 pages x 64, random page table) into bf16 [262144, 512].
Inputs are seeded synthetic data, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is compressed KV rows per second over the
timed steps (rows compressed + rows gathered).  Each headline kernel is also
timed under three cache conditions, median and p90 (steady: 10 samples of 50
launches; the cold ones: --launches lone calls):
  steady      back to back, every call on other buffers than the calls
              before it (no reuse of what they left in the 256 MB Infinity
              Cache), as in a pipeline that keeps the device busy;
  cold        before each call a 512 MB scratch write and then a 512 MB
              scratch read, neither timed: the caches hold nothing of the
              call's data, and the write's dirty lines have reached HBM;
  cold_dirty  before each call the 512 MB scratch write alone (the flush as
              first specified): the call's interval then also carries the
              write-back of those dirty lines.
Beside each kernel, a streaming kernel that moves the same bytes with no
work (libkvc_ceiling.so) is timed the same way, and a 1 GiB device copy
gives the copy ceiling.  The roofline object is the gather's (the dominant
kernel), steady.  The CPU oracle is timed on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
FLUSH_BYTES = 512 << 20        # exceeds the 256 MB Infinity Cache plus the L2s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    runs (profiles/traffic.json), or None when the kernel's sources changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            e = json.load(fh).get(kernel)
        h = hashlib.sha256()
        for f in e["source_files"]:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
    except (OSError, ValueError, KeyError, TypeError, AttributeError):
        return None
    if h.hexdigest()[:16] != e.get("source_hash"):
        return None
    return e.get("bytes_per_launch")


TRAFFIC_SOURCE = ("profiles/traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE per dispatch, "
                  "scaled by the same counters on a 1 GiB copy; not measured in this run; "
                  "null once the kernel's sources differ from the counted build")


WARM_UP_S = 0.025


def warm_up_replays(g):
    """Replay a freshly captured graph untimed for about WARM_UP_S of device
    time (at least twice): the device idles while a graph is captured on the
    host, and the replays just after that ran up to 10% slower (the first 10
    ms or so).  Returns without waiting, so that the device is still busy
    with these replays while the caller queues its timed ones: after a long
    run of queued replays the host's next submissions can be slow, and a
    timed interval that starts on an idle device would hold that wait."""
    import torch
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    per = max(a.elapsed_time(b) / 1e3, 1e-6)
    for _ in range(min(200, max(2, int(WARM_UP_S / per) + 1))):
        g.replay()


class Timer:
    """Device time per launch of a kernel under three cache conditions, from
    HIP events on the launch stream (calls[k % len] is launch k):
      steady      a HIP graph of 50 back-to-back launches, replayed untimed
                  for about 25 ms, then 10 timed replays, each after an
                  untimed lead-in replay; one sample per timed replay (its
                  mean per launch).  No host launch cost falls inside an interval, and
                  the device's own gap before a replay's first kernel (about
                  10 us) is spread over 50 launches;
      cold        lone launches, each after a 512 MB scratch write and a
                  512 MB scratch read (neither timed), each bracketed by
                  events: the caches hold none of the call's data and no
                  dirty line; the interval carries the launch's dispatch and
                  completion (about 3 us at these sizes, the same for the
                  streaming yardstick timed beside it);
      cold_dirty  the same after the scratch write alone: the interval also
                  carries the write-back of the scratch's dirty lines."""

    PER_GRAPH = 50
    REPLAYS = 10

    def __init__(self, dev, launches: int):
        import torch
        self.torch = torch
        self.scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.launches = launches

    def write_flush(self):
        self.scratch.fill_(1)

    def read_flush(self):
        self.torch.amax(self.scratch.view(self.torch.int64))

    def steady(self, calls, replays: int = REPLAYS):
        torch = self.torch
        n = self.PER_GRAPH
        body = lambda: [calls[k % len(calls)]() for k in range(n)]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            body()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        warm_up_replays(g)
        stream = torch.cuda.current_stream()
        samples = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g.replay()                       # untimed lead-in: the device is busy
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b) * 1e3 / n)
        return samples

    def flushed(self, calls, dirty: bool):
        torch = self.torch
        stream = torch.cuda.current_stream()
        pairs = []
        for k in range(self.launches):
            self.write_flush()
            if not dirty:
                self.read_flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            calls[k % len(calls)]()
            b.record(stream)
            pairs.append((a, b))
            if len(pairs) % 25 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in pairs]

    def all(self, calls):
        return {"steady": self.steady(calls), "cold": self.flushed(calls, dirty=False),
                "cold_dirty": self.flushed(calls, dirty=True)}


def summarize(samples_us, nbytes, units, unit_name, ceiling_us=None, per_sample=Timer.PER_GRAPH):
    import numpy as np
    med = float(np.median(samples_us))
    r = {"us": med, "p90_us": float(np.percentile(samples_us, 90)),
         "min_us": float(np.min(samples_us)), "samples": len(samples_us),
         "launches_timed": len(samples_us) * per_sample,
         "gbps": nbytes / med / 1e3, "frac": nbytes / med / 1e3 / HBM_PEAK_GBS,
         unit_name: units / med * 1e6}
    if ceiling_us is not None:
        c = float(np.median(ceiling_us))
        r["same_shape_stream_us"] = c
        r["frac_of_same_shape_stream"] = c / med
    return r


def _time_events(fn, stream, reps: int, warmup: int = 3):
    """mean device time in seconds of one fn() call.  The calls are captured
    back to back in a HIP graph so that host-side launch cost does not pace
    them (small kernels run faster than Python can launch them); after the
    untimed warm-up replays, HIP events on the replay stream bracket three
    replays of the graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    warm_up_replays(g)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(3):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (3 * reps) / 1e3


def measure_next_rows(kvc, W, d, dev, stream, timer):
    """Throughput of the entry points beyond the two headline kernels, each on
    a workload of the path's own shapes, with its algorithmic HBM bytes.
    These are timed as graph replays of back-to-back calls on the same
    buffers (warm, as a decode step's freshly written inputs would be); each
    is also timed cold: lone calls after the flush, median and p90, the
    launch's dispatch and completion included."""
    import numpy as np
    import torch

    res = {}
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def entry(name, secs, nbytes, units, unit, cold_call=None):
        res[name] = {"us": secs * 1e6, "bytes": int(nbytes), "gbps": nbytes / secs / 1e9,
                     "frac": nbytes / secs / 1e9 / HBM_PEAK_GBS, unit: units / secs,
                     "condition": "warm (graph replay, same buffers)",
                     "traffic": measured_traffic(name)}
        if cold_call is not None:
            res[name]["cold"] = summarize(timer.flushed([cold_call], dirty=False), nbytes,
                                          units, unit, per_sample=1)

    # verify: 1024 slots x 4 drafts, ring of 3, V41_FP4 cache through page tables
    vc = W.verify_case(20261206, 1024, draft_len=4, ratio=2, page_size=64, max_pos=4096,
                       ring_slots=3)
    fp4 = kvc.kvc_layout_query("V41_FP4")
    S, D = vc["S"], vc["draft_len"]
    pos = vc["pos"].astype(np.int64)
    q = pos[:, None] + np.arange(D)[None, :]
    rows = int((q % 2 == 1).sum())
    pend = int((q % 2 == 0).sum())
    first_from_ring = int((pos % 2 == 1).sum())
    vbytes = S * D * 2048 + first_from_ring * 2048 + rows * (1024 + fp4.row_bytes) + pend * 2048
    vp = d(vc["kv"])
    vargs = dict(ratio=2, mode=kvc.MODE_VERIFY, kv=vp[:, :512], score=vp[:, 512:],
                 start_pos=d(vc["pos"]), page_table=d(vc["page_table"]), state=d(vc["state"]),
                 norm_w=d(vc["norm_w"]), eps=vc["eps"], freqs=d(vc["freqs"]),
                 latent_out=torch.empty((S * D, 512), dtype=torch.int16, device=dev),
                 cache=kvc.Cache(torch.zeros((vc["num_pages"], 64 * fp4.row_bytes),
                                             dtype=torch.uint8, device=dev), "V41_FP4", 64),
                 draft_len=D, ring_slots=3, status=status)
    v_call = lambda: kvc.kvc_compress_store(**vargs)
    secs = _time_events(v_call, stream, 50)
    entry("verify_1024x4_v41fp4", secs, vbytes, rows, "rows_per_s", v_call)

    # decode: 1024 slots x 1 token, ratio 2, explicit out_loc, V4 cache
    c5 = W.workload_c5()
    v4 = kvc.kvc_layout_query("V4")
    dp = d(c5["kv"])
    dpos = c5["pos"].astype(np.int64)
    drows = int((dpos % 2 == 1).sum())
    dbytes = 1024 * 2048 + drows * (2048 + 1024 + v4.row_bytes) + (1024 - drows) * 2048
    dargs = dict(ratio=2, mode=kvc.MODE_DECODE, kv=dp[:, :512], score=dp[:, 512:],
                 start_pos=d(c5["pos"]), out_loc=d(c5["out_loc"]), state=d(c5["state"]),
                 norm_w=d(c5["norm_w"]), eps=c5["eps"], freqs=d(c5["freqs"]),
                 latent_out=torch.empty((1024, 512), dtype=torch.int16, device=dev),
                 cache=kvc.Cache(torch.zeros((c5["num_pages"], 64 * v4.row_bytes),
                                             dtype=torch.uint8, device=dev), "V4", 64),
                 status=status)
    d_call = lambda: kvc.kvc_compress_store(**dargs)
    secs = _time_events(d_call, stream, 50)
    entry("decode_1024_v4", secs, dbytes, drows, "rows_per_s", d_call)

    # RoPE store: the ratio-1 store workload (8 requests, 512..4096 rows) with
    # a rotary position per row, into V41_FP4
    c2 = W.workload_c2()
    n2 = c2["rows"].shape[0]
    rng = np.random.default_rng(20261207)
    pos2 = d(rng.integers(0, 16384, size=n2).astype(np.int32))
    fr2 = d(W.rope_freqs(16384))
    rcache = kvc.Cache(torch.zeros((c2["num_pages"], 64 * fp4.row_bytes), dtype=torch.uint8,
                                   device=dev), "V41_FP4", 64)
    rrows, rloc = d(c2["rows"]), d(c2["out_loc"])
    st_fp4 = lambda: kvc.kvc_store_rows(rcache, rrows, rloc, status)
    secs = _time_events(st_fp4, stream, 50)
    entry("store_c2_v41fp4", secs, n2 * (1024 + fp4.row_bytes + 4), n2, "rows_per_s", st_fp4)
    # the dequant half of the same workload: every stored row back to bf16 by
    # its slot (no page table)
    dq_out = torch.empty((n2, 512), dtype=torch.int16, device=dev)
    dq_fp4 = lambda: kvc.kvc_dequant_gather(rcache, None, rloc, dq_out, status)
    secs = _time_events(dq_fp4, stream, 50)
    entry("dequant_c2_v41fp4", secs, n2 * (fp4.row_bytes + 1024 + 4), n2, "rows_per_s", dq_fp4)
    v41c = kvc.kvc_layout_query("V41")
    vcache = kvc.Cache(torch.zeros((c2["num_pages"], 64 * v41c.row_bytes), dtype=torch.uint8,
                                   device=dev), "V41", 64)
    st_v41 = lambda: kvc.kvc_store_rows(vcache, rrows, rloc, status)
    secs = _time_events(st_v41, stream, 50)
    entry("store_c2_v41", secs, n2 * (1024 + v41c.row_bytes + 4), n2, "rows_per_s", st_v41)
    dq_v41 = lambda: kvc.kvc_dequant_gather(vcache, None, rloc, dq_out, status)
    secs = _time_events(dq_v41, stream, 50)
    entry("dequant_c2_v41", secs, n2 * (v41c.row_bytes + 1024 + 4), n2, "rows_per_s", dq_v41)
    r_call = lambda: kvc.kvc_store_rows_rope(rcache, rrows, pos2, fr2, rloc, status)
    secs = _time_events(r_call, stream, 50)
    entry("rope_store_c2_v41fp4", secs, n2 * (1024 + fp4.row_bytes + 8), n2, "rows_per_s",
          r_call)

    # DCP filter: 4096 tokens x 2048 global ids, 4 ranks, runs of 4, rank 1
    dc = W.dcp_ids_case(20261208, T=4096, k=2048, n_req=32, max_rows=65536, world=4,
                        page_size=64)
    T, k = dc["ids"].shape
    f_ids, f_t2r, f_bt = d(dc["ids"]), d(dc["token_to_req"]), d(dc["block_tables"][1])
    f_valid = d(dc["valid"])
    f_out = torch.empty((T, k), dtype=torch.int32, device=dev)
    f_lens = torch.empty(T, dtype=torch.int32, device=dev)
    f_call = lambda: kvc.kvc_dcp_filter_ids(
        f_ids, f_t2r, f_bt, f_out, f_lens, page_size=64, num_pages=dc["num_pages"], world=4,
        rank=1, interleave=4, valid=f_valid, status=status)
    secs = _time_events(f_call, stream, 50)
    entry("dcp_filter_4096x2048_w4", secs, T * k * 8 + T * 12, T * k, "ids_per_s", f_call)

    # graph replay vs eager launch of the small prefill compress (one 64-token
    # request, ratio 2, V41): host wall time per call, back to back
    c1 = W.workload_c1()
    v41 = kvc.kvc_layout_query("V41")
    c1args = dict(ratio=2, mode=kvc.MODE_PREFILL, kv=d(c1["kv"]), score=d(c1["score"]),
                  start_pos=d(c1["start_pos"]), offsets=d(c1["offsets"]),
                  page_table=d(c1["page_table"]), state=d(c1["state"]), norm_w=d(c1["norm_w"]),
                  eps=c1["eps"], freqs=d(c1["freqs"]),
                  latent_out=torch.empty((32, 512), dtype=torch.int16, device=dev),
                  cache=kvc.Cache(torch.zeros((c1["num_pages"], 64 * v41.row_bytes),
                                              dtype=torch.uint8, device=dev), "V41", 64))
    n_calls = 2000
    for _ in range(10):
        kvc.kvc_compress_store(**c1args)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n_calls):
        kvc.kvc_compress_store(**c1args)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t) / n_calls
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kvc.kvc_compress_store(**c1args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(20):
            kvc.kvc_compress_store(**c1args)
    g.replay()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n_calls // 20):
        g.replay()
    torch.cuda.synchronize()
    replay = (time.perf_counter() - t) / n_calls
    res["graph_c1_compress"] = {"eager_us_per_call": eager * 1e6,
                                "graph_us_per_call": replay * 1e6,
                                "calls_per_graph": 20, "calls": n_calls}
    assert int(status.item()) == 0, f"device status {int(status.item())}"
    return res


def measure_reuse(kvc, cache, pt, idsets, outs, stream, layers: int, forwards: int = 20):
    """The C4 gather read by `layers` consumer layers of one forward pass:
    through the reuse head (one gather, then hits that launch nothing) and
    as fresh gathers.  Each forward uses the next id list, so its one gather
    is as cold as the bench's."""
    import torch
    buf = kvc.KVBuf()

    def fwd_reuse(f):
        buf.begin_forward()
        return sum(int(buf.kvc_dequant_gather_reuse(cache, pt, idsets[f % len(idsets)],
                                                    outs[f % len(outs)]))
                   for _ in range(layers))

    def fwd_fresh(f):
        for _ in range(layers):
            kvc.kvc_dequant_gather(cache, pt, idsets[f % len(idsets)], outs[f % len(outs)])
        return 0

    res = {"layers": layers, "forwards": forwards}
    for name, fn in (("fresh", fwd_fresh), ("reuse", fwd_reuse)):
        fn(0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hits = 0
        t = time.perf_counter()
        a.record(stream)
        for f in range(1, forwards + 1):
            hits += fn(f)
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t
        res[f"{name}_us_per_forward"] = a.elapsed_time(b) * 1e3 / forwards
        res[f"{name}_wall_us_per_forward"] = wall * 1e6 / forwards
        if name == "reuse":
            res["hits_per_forward"] = hits / forwards
    res["speedup"] = res["fresh_us_per_forward"] / res["reuse_us_per_forward"]
    return res


def measure_sweep(kvc, W, d, dev, stream):
    """Throughput against size: the prefill compress at 1, 2, 4 and 8 times
    the 32,768-token workload (16 requests per 32,768 ragged tokens, fused
    |kv|score| buffer, page 128, V41_FP4), and the gather from the 1,048,576-row
    V41 cache at 65,536 to 1,048,576 distinct ids (four id lists, disjoint
    where the cache's rows allow, and three outputs in turn).  Each size is timed as graph replays of back-to-back
    calls, like the next rows, with its inputs and outputs in turn."""
    import numpy as np
    import torch

    fp4 = kvc.kvc_layout_query("V41_FP4")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    out = []
    for mult in (1, 2, 4, 8):
        rng = np.random.default_rng(W.BASE_SEED + 100 + mult)
        S = 16 * mult
        lengths = W.ragged_lengths(rng, 32768 * mult, S)
        first = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int32)
        pages = (lengths // 2) // 128 + 2                # every compressed row's page, plus one
        num_pages = int(pages.sum()) + 5
        perm = W.random_pages(rng, int(pages.sum()), num_pages)
        pt = np.zeros((S, int(pages.max())), np.int32)
        k = 0
        for b in range(S):
            pt[b, :pages[b]] = perm[k:k + pages[b]]
            k += pages[b]
        T = int(lengths.sum())
        gen.manual_seed(W.BASE_SEED + mult)
        proj = torch.randn((T, 1024), device=dev, generator=gen).to(torch.bfloat16).view(torch.int16)
        rows, tails = int((lengths // 2).sum()), int((lengths % 2).sum())
        # copies of the input and of the outputs in turn, at least 512 MB of
        # input in all: no call reads or rewrites what an earlier one left in
        # the 256 MB Infinity Cache
        ncopy = max(3, -(-(1 << 29) // (T * 2048)))
        projs = [proj] + [proj.clone() for _ in range(ncopy - 1)]
        lats = [torch.empty((rows, 512), dtype=torch.int16, device=dev) for _ in range(ncopy)]
        caches = [kvc.Cache(torch.zeros((num_pages, 128 * fp4.row_bytes), dtype=torch.uint8,
                                        device=dev), "V41_FP4", 128) for _ in range(ncopy)]
        args = dict(ratio=2, mode=kvc.MODE_PREFILL, start_pos=d(np.zeros(S, np.int32)),
                    offsets=d(np.stack([first, lengths]).astype(np.int32)), page_table=d(pt),
                    state=torch.zeros((S, 2, 512), dtype=torch.int16, device=dev),
                    norm_w=d(W.norm_weight(rng)), eps=1e-6,
                    freqs=d(W.rope_freqs(int(lengths.max()) + 2)), status=status)
        turn = [0]

        def comp():
            k = turn[0]
            turn[0] += 1
            pj = projs[k % ncopy]
            kvc.kvc_compress_store(**args, kv=pj[:, :512], score=pj[:, 512:],
                                   latent_out=lats[k % ncopy], cache=caches[k % ncopy])
        secs = _time_events(comp, stream, 2 * ncopy)
        nbytes = rows * (4096 + 1024 + fp4.row_bytes) + tails * 4096
        out.append({"kernel": "compress_store", "tokens": T, "requests": S, "rows": rows,
                    "us": secs * 1e6, "bytes": nbytes, "gbps": nbytes / secs / 1e9,
                    "frac": nbytes / secs / 1e9 / HBM_PEAK_GBS})
        del proj, projs, lats, caches, args
        torch.cuda.empty_cache()
    c4 = W.workload_c4()
    cache, pt = kvc.Cache(d(c4["cache"]), "V41", 64), d(c4["page_table"])
    rows = 1048576
    for n in (65536, 262144, 524288, 1048576):
        # four lists cut in turn from one random order of the cache's rows:
        # disjoint up to 262,144 ids, each row in at most two lists at 524,288
        order = np.random.default_rng(W.BASE_SEED + 200 + n).permutation(rows).astype(np.int32)
        sets = [d(np.take(order, np.arange(j * n, (j + 1) * n) % rows)) for j in range(4)]
        outs = [torch.empty((n, 512), dtype=torch.int16, device=dev) for _ in range(3)]
        turn = [0]

        def call():
            k = turn[0]
            turn[0] += 1
            kvc.kvc_dequant_gather(cache, pt, sets[k % 4], outs[k % 3], status)
        secs = _time_events(call, stream, 12)
        nbytes = n * (528 + 1024 + 4)
        out.append({"kernel": "dequant_gather", "ids": n, "us": secs * 1e6, "bytes": nbytes,
                    "gbps": nbytes / secs / 1e9, "frac": nbytes / secs / 1e9 / HBM_PEAK_GBS})
        del sets, outs
        torch.cuda.empty_cache()
    assert int(status.item()) == 0, f"device status {int(status.item())}"
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(c3, c4, fp4_row_bytes):
    """The oracle as it stands, on the host's cores, on both halves of the
    step at their full size: the compress of the 32,768-token batch (16,379
    rows) and the gather of the 262,144 ids; each timed 5 times (about 2 s of
    CPU work on 16 cores), the median kept.  `value` is rows per second of
    the two run back to back."""
    import numpy as np
    import oracle
    lengths = c3["lengths"].astype(np.int64)
    rows_c = int((lengths // 2).sum())
    ids = c4["ids"]
    m = int(ids.size)
    comp_s, gath_s = [], []
    for _ in range(5):
        cache_h = np.zeros((c3["num_pages"], 128 * fp4_row_bytes), np.uint8)
        t = time.perf_counter()
        oracle.compress(ratio=2, mode=oracle.PREFILL, kv=c3["kv"], fused=True,
                        offsets=c3["offsets"].copy(), start_pos=c3["start_pos"],
                        page_table=c3["page_table"], state=c3["state"].copy(),
                        norm_w=c3["norm_w"], eps=c3["eps"], freqs=c3["freqs"], cache=cache_h,
                        layout="V41_FP4", page_size=128, want_prequant=False)
        comp_s.append(time.perf_counter() - t)
        t = time.perf_counter()
        oracle.dequant_gather(c4["cache"], "V41", 64, c4["page_table"], ids)
        gath_s.append(time.perf_counter() - t)
    tc, tg = float(np.median(comp_s)), float(np.median(gath_s))
    return {"value": (rows_c + m) / (tc + tg), "unit": "rows/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole step: compress of the 32,768-token batch ({rows_c} rows) and "
                      f"gather of the {m} ids, each timed 5 times, median",
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "halves": {"compress_store": {"rows": rows_c, "median_s": tc,
                                          "rows_per_s": rows_c / tc, "runs_s": comp_s},
                       "dequant_gather": {"rows": m, "median_s": tg, "rows_per_s": m / tg,
                                          "runs_s": gath_s}}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--launches", type=int, default=100,
                    help="timed lone launches per kernel in each cold condition (median, p90)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the verify / RoPE-store / DCP-filter / graph-replay / reuse measurements")
    ap.add_argument("--sweep", action="store_true",
                    help="only measure compress and gather throughput at several sizes, one "
                         "JSON line per size, and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy 5 times (the known-size "
                         "reference for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path runs on one GPU's share); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fp8_fp4_quantized_amd as kvc
    from fp8_fp4_quantized_amd import ceiling
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                          "launches": 5}), flush=True)
        return 0

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    if args.sweep:
        for rec in measure_sweep(kvc, W, d, dev, torch.cuda.current_stream()):
            print(json.dumps(rec), flush=True)
        return 0

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    c3 = W.workload_c3()
    c4 = W.workload_c4()
    log(f"inputs generated in {time.time() - t0:.1f}s")
    lengths = c3["lengths"].astype(np.int64)
    c3_rows = int((lengths // 2).sum())              # P = 0: one row per complete pair
    c3_tails = int((lengths % 2).sum())
    fp4 = kvc.kvc_layout_query("V41_FP4")
    v41 = kvc.kvc_layout_query("V41")
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    # eight copies of the projection buffer (512 MB) and four latent outputs
    # and caches, used in turn: a call reads and writes other lines than the
    # calls just before it, so nothing it touches is left in the 256 MB
    # Infinity Cache by them
    proj = d(c3["kv"])
    c3_projs = [proj] + [proj.clone() for _ in range(7)]
    c3_lats = [torch.empty((c3_rows, 512), dtype=torch.int16, device=dev) for _ in range(4)]
    c3_caches = [kvc.Cache(torch.zeros((c3["num_pages"], 128 * fp4.row_bytes), dtype=torch.uint8,
                                       device=dev), "V41_FP4", 128) for _ in range(4)]
    c3_common = dict(
        ratio=2, mode=kvc.MODE_PREFILL,
        start_pos=d(c3["start_pos"]), offsets=d(c3["offsets"]), page_table=d(c3["page_table"]),
        state=d(c3["state"]), norm_w=d(c3["norm_w"]), eps=c3["eps"], freqs=d(c3["freqs"]),
        status=status)
    compress_calls = [kvc.prepare_compress_store(
        **c3_common, kv=c3_projs[k % 8][:, :512], score=c3_projs[k % 8][:, 512:],
        latent_out=c3_lats[k % 4], cache=c3_caches[k % 4]) for k in range(8)]
    g_cache = kvc.Cache(d(c4["cache"]), "V41", 64)
    g_pt = d(c4["page_table"])
    n_ids = int(c4["ids"].size)
    # four id lists that share no row and four outputs, used in turn
    g_idsets = [d(ids) for ids in W.workload_c4_disjoint_id_sets(4)]
    g_outs = [torch.empty((n_ids, 512), dtype=torch.int16, device=dev) for _ in range(4)]
    gather_calls = [kvc.prepare_dequant_gather(g_cache, g_pt, g_idsets[k % 4], g_outs[k % 4],
                                               status) for k in range(4)]

    def step(k):
        compress_calls[k % 8]()
        gather_calls[k % 4]()

    # ---------------------------------------------------------------- timed steps
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, f"device status {int(status.item())}"
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps

    # ---------------------------------------------------------------- per kernel
    timer = Timer(dev, args.launches)
    comp_bytes = c3_rows * (4096 + 1024 + fp4.row_bytes) + c3_tails * 2 * 2048
    gath_bytes = n_ids * (v41.row_bytes + 1024 + 4)
    t_comp = timer.all(compress_calls)
    t_gath = timer.all(gather_calls)
    assert int(status.item()) == 0, f"device status {int(status.item())}"

    # the same bytes with no work: the compressor's shape (one item = two
    # rows) and the gather's shape (contiguous rows), eight inputs / four
    # outputs in turn like the kernels
    items = (c3_rows + 1) // 2
    cs_src = [torch.empty(items * 8192, dtype=torch.uint8, device=dev).fill_(k) for k in range(8)]
    cs_out = [[torch.empty(items * n, dtype=torch.uint8, device=dev) for n in (2048, 512, 64)]
              for _ in range(4)]
    cs_calls = [ceiling.compress_shape(cs_src[k % 8], *cs_out[k % 4], items) for k in range(8)]
    gs_src = [torch.empty(n_ids * 528, dtype=torch.uint8, device=dev).fill_(k) for k in range(4)]
    gs_out = [torch.empty(n_ids * 1024, dtype=torch.uint8, device=dev) for _ in range(4)]
    gs_calls = [ceiling.gather_shape(gs_src[k], gs_out[k], n_ids) for k in range(4)]
    c_comp = timer.all(cs_calls)
    c_gath = timer.all(gs_calls)
    cs_bytes = items * (8192 + 2048 + 512 + 64)
    gs_bytes = n_ids * (528 + 1024)
    # the copy ceiling: 1 GiB device-to-device copies, two pairs in turn
    cp = [(torch.ones(1 << 30, dtype=torch.uint8, device=dev),
           torch.empty(1 << 30, dtype=torch.uint8, device=dev)) for _ in range(2)]
    cp_calls = [lambda s=s_, t=t_: t.copy_(s) for s_, t_ in cp]
    saved, timer.launches = timer.launches, 10
    t_copy = {"steady": timer.steady(cp_calls, replays=2),
              "cold": timer.flushed(cp_calls, dirty=False)}
    timer.launches = saved
    copy_gbs = {c: (2 << 30) / float(np.median(v)) / 1e3 for c, v in t_copy.items()}
    # what a lone launch costs beyond its kernel under the cold flushes: a
    # one-element kernel timed the same way
    tiny = torch.zeros(1, dtype=torch.int32, device=dev)
    call_overhead = {"cold": float(np.median(timer.flushed([lambda: tiny.add_(1)], dirty=False))),
                     "cold_dirty": float(np.median(timer.flushed([lambda: tiny.add_(1)],
                                                                 dirty=True)))}
    del cs_src, cs_out, cs_calls, gs_src, gs_out, gs_calls, cp, cp_calls

    def kernel_entry(t, c, nbytes, ceil_bytes, rows, traffic_name):
        e = {"bytes": nbytes, "rows": rows,
             "timing": "steady: HIP events around 10 HIP-graph replays of 50 back-to-back "
                       "launches, one sample per replay; cold, cold_dirty: lone launches after "
                       "the flush, "
                       "each bracketed by events (dispatch and completion included)"}
        for cond in ("steady", "cold", "cold_dirty"):
            r = summarize(t[cond], nbytes, rows, "rows_per_s",
                          per_sample=Timer.PER_GRAPH if cond == "steady" else 1)
            cm = float(np.median(c[cond]))
            r["same_shape_stream_us"] = cm
            r["same_shape_stream_frac"] = ceil_bytes / cm / 1e3 / HBM_PEAK_GBS
            # the kernel's rate as a fraction of the stream's rate
            r["frac_of_same_shape_stream"] = (nbytes / r["us"]) / (ceil_bytes / cm)
            e[cond] = r
        # headline figures: steady
        for key in ("us", "p90_us", "gbps", "frac", "rows_per_s", "launches_timed"):
            e[key] = e["steady"][key]
        e["condition"] = "steady"
        e["copy_ceiling_frac"] = e["gbps"] / copy_gbs["steady"]
        e["traffic"] = measured_traffic(traffic_name)
        e["traffic_source"] = TRAFFIC_SOURCE
        return e

    k_comp = kernel_entry(t_comp, c_comp, comp_bytes, cs_bytes, c3_rows, "compress_store")
    k_gath = kernel_entry(t_gath, c_gath, gath_bytes, gs_bytes, n_ids, "dequant_gather")
    rows_step = c3_rows + n_ids
    value = rows_step / (ms_step / 1e3)
    for name, k in (("compress", k_comp), ("gather", k_gath)):
        log(f"{name}: steady {k['steady']['us']:.2f} us ({k['steady']['frac']:.3f}), cold "
            f"{k['cold']['us']:.2f} us ({k['cold']['frac']:.3f}), cold_dirty "
            f"{k['cold_dirty']['us']:.2f} us; same-shape stream "
            f"{k['steady']['same_shape_stream_us']:.2f} / {k['cold']['same_shape_stream_us']:.2f}"
            f" / {k['cold_dirty']['same_shape_stream_us']:.2f} us")
    log(f"copy ceiling: steady {copy_gbs['steady']:.0f} GB/s, cold {copy_gbs['cold']:.0f} GB/s; "
        f"step {ms_step * 1e3:.1f} us")

    out = {
        "metric": "compressed KV rows/sec + achieved HBM GB/s (compress-store, dequant-gather)",
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "prefill compress-store (ratio 2, 16 requests, 32768 tokens, fused "
                        "|kv|score| bf16 [32768,1024], page 128, V41_FP4) + sparse-prefill "
                        "dequant-gather (262144 ids from a 1048576-row V41 cache, page 64, "
                        "random page table -> bf16 [262144,512]; 4 disjoint id lists in turn)",
            "compress_rows": c3_rows, "gather_rows": n_ids,
            "seed_c3": int(c3["seed"]), "odd_lengths": c3_tails,
        },
        "hbm_gbps": (comp_bytes + gath_bytes) / (ms_step / 1e3) / 1e9,
        "kernels": {"compress_store": k_comp, "dequant_gather": k_gath},
        "lone_call_overhead_us": call_overhead,
        "copy_ceiling": {"bytes_per_copy": 2 << 30, "steady_gbps": copy_gbs["steady"],
                         "cold_gbps": copy_gbs["cold"],
                         "steady_frac": copy_gbs["steady"] / HBM_PEAK_GBS,
                         "cold_frac": copy_gbs["cold"] / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "achieved": k_gath["gbps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": k_gath["frac"], "traffic": k_gath["traffic"],
                     "traffic_source": TRAFFIC_SOURCE,
                     "copy_ceiling_frac": k_gath["copy_ceiling_frac"],
                     "condition": "steady", "kernel": "dequant_gather",
                     "algorithmic_bytes": gath_bytes},
        "cpu_baseline": None,
    }

    if not args.no_next_rows:
        out["next_rows"] = measure_next_rows(kvc, W, d, dev, torch.cuda.current_stream(), timer)
        out["next_rows"]["gather_reuse_c4_8_layers"] = measure_reuse(
            kvc, g_cache, g_pt, g_idsets, g_outs, torch.cuda.current_stream(), layers=8)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c3, c4, fp4.row_bytes)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
