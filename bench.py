"""Benchmark of the DeepSeek-V4.1 low-ratio compressed-KV hot path on one
MI355X.

One step = one pass of both halves of the path over one batch:
  1. compress-store: ratio-2 ragged prefill of 16 requests totalling 32,768
     tokens (fused |kv|score| bf16 [32768, 1024], page 128, V41_FP4 cache);
  2. dequant-gather: 262,144 distinct ids from a V41 cache of 1,048,576 rows
     (16,384 pages x 64, random page table) into bf16 [262144, 512].
Inputs are seeded synthetic data, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is compressed KV rows per second over the
step (rows compressed + rows gathered); the per-kernel HBM rates, the roofline
object of the dominant kernel (the gather) and the CPU-oracle baseline ride
along.
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


def _time_events(fn, stream, reps: int, warmup: int = 3):
    """mean device time in seconds of one fn() call.  The calls are captured
    back to back in a HIP graph so that host-side launch cost does not pace
    them (small kernels run faster than Python can launch them); HIP events
    on the replay stream bracket three replays of the graph."""
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
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(3):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (3 * reps) / 1e3


def measure_next_rows(kvc, W, d, dev, stream):
    """Throughput of the entry points beyond the two headline kernels, each on
    a workload of the path's own shapes, with its algorithmic HBM bytes."""
    import numpy as np
    import torch

    res = {}
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def entry(name, secs, nbytes, units, unit):
        res[name] = {"us": secs * 1e6, "bytes": int(nbytes), "gbps": nbytes / secs / 1e9,
                     "frac": nbytes / secs / 1e9 / HBM_PEAK_GBS, unit: units / secs,
                     "traffic": measured_traffic(name)}

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
    secs = _time_events(lambda: kvc.kvc_compress_store(**vargs), stream, 50)
    entry("verify_1024x4_v41fp4", secs, vbytes, rows, "rows_per_s")

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
    secs = _time_events(lambda: kvc.kvc_compress_store(**dargs), stream, 50)
    entry("decode_1024_v4", secs, dbytes, drows, "rows_per_s")

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
    secs = _time_events(lambda: kvc.kvc_store_rows(rcache, rrows, rloc, status), stream, 50)
    entry("store_c2_v41fp4", secs, n2 * (1024 + fp4.row_bytes + 4), n2, "rows_per_s")
    # the dequant half of the same workload: every stored row back to bf16 by
    # its slot (no page table)
    dq_out = torch.empty((n2, 512), dtype=torch.int16, device=dev)
    secs = _time_events(lambda: kvc.kvc_dequant_gather(rcache, None, rloc, dq_out, status),
                        stream, 50)
    entry("dequant_c2_v41fp4", secs, n2 * (fp4.row_bytes + 1024 + 4), n2, "rows_per_s")
    v41c = kvc.kvc_layout_query("V41")
    vcache = kvc.Cache(torch.zeros((c2["num_pages"], 64 * v41c.row_bytes), dtype=torch.uint8,
                                   device=dev), "V41", 64)
    secs = _time_events(lambda: kvc.kvc_store_rows(vcache, rrows, rloc, status), stream, 50)
    entry("store_c2_v41", secs, n2 * (1024 + v41c.row_bytes + 4), n2, "rows_per_s")
    secs = _time_events(lambda: kvc.kvc_dequant_gather(vcache, None, rloc, dq_out, status),
                        stream, 50)
    entry("dequant_c2_v41", secs, n2 * (v41c.row_bytes + 1024 + 4), n2, "rows_per_s")
    secs = _time_events(lambda: kvc.kvc_store_rows_rope(rcache, rrows, pos2, fr2, rloc, status),
                        stream, 50)
    entry("rope_store_c2_v41fp4", secs, n2 * (1024 + fp4.row_bytes + 8), n2, "rows_per_s")

    # DCP filter: 4096 tokens x 2048 global ids, 4 ranks, runs of 4, rank 1
    dc = W.dcp_ids_case(20261208, T=4096, k=2048, n_req=32, max_rows=65536, world=4,
                        page_size=64)
    T, k = dc["ids"].shape
    f_ids, f_t2r, f_bt = d(dc["ids"]), d(dc["token_to_req"]), d(dc["block_tables"][1])
    f_valid = d(dc["valid"])
    f_out = torch.empty((T, k), dtype=torch.int32, device=dev)
    f_lens = torch.empty(T, dtype=torch.int32, device=dev)
    secs = _time_events(lambda: kvc.kvc_dcp_filter_ids(
        f_ids, f_t2r, f_bt, f_out, f_lens, page_size=64, num_pages=dc["num_pages"], world=4,
        rank=1, interleave=4, valid=f_valid, status=status), stream, 50)
    entry("dcp_filter_4096x2048_w4", secs, T * k * 8 + T * 12, T * k, "ids_per_s")

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
        return sum(int(buf.kvc_dequant_gather_reuse(cache, pt, idsets[f % 4], outs[f % 3]))
                   for _ in range(layers))

    def fwd_fresh(f):
        for _ in range(layers):
            kvc.kvc_dequant_gather(cache, pt, idsets[f % 4], outs[f % 3])
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
    V41 cache at 65,536 to 1,048,576 distinct ids (four id lists and three
    outputs in turn).  Each size is timed as graph replays of back-to-back
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
    for n in (65536, 262144, 524288, 1048576):
        sets = [d(np.random.default_rng(W.BASE_SEED + 200 + j).choice(
            1048576, size=n, replace=False).astype(np.int32)) for j in range(4)]
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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
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
    if args.sweep:
        def d(a):
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        for rec in measure_sweep(kvc, W, d, dev, torch.cuda.current_stream()):
            print(json.dumps(rec), flush=True)
        return 0

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

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

    # four copies of the projection buffer (64 MB each) and three latent
    # outputs and caches used in turn, like the gather's id lists and outputs
    # below: back-to-back compresses read and write HBM, not lines the
    # previous call left in the 256 MB Infinity Cache
    proj = d(c3["kv"])
    c3_projs = [proj] + [proj.clone() for _ in range(3)]
    c3_lats = [torch.empty((c3_rows, 512), dtype=torch.int16, device=dev) for _ in range(3)]
    c3_caches = [kvc.Cache(torch.zeros((c3["num_pages"], 128 * fp4.row_bytes), dtype=torch.uint8,
                                       device=dev), "V41_FP4", 128) for _ in range(3)]
    c3_args = dict(
        ratio=2, mode=kvc.MODE_PREFILL,
        start_pos=d(c3["start_pos"]), offsets=d(c3["offsets"]), page_table=d(c3["page_table"]),
        state=d(c3["state"]), norm_w=d(c3["norm_w"]), eps=c3["eps"], freqs=d(c3["freqs"]))
    g_cache = kvc.Cache(d(c4["cache"]), "V41", 64)
    g_pt = d(c4["page_table"])
    n_ids = int(c4["ids"].size)
    # four id lists and three output buffers used in turn: a step neither
    # reads the rows nor rewrites the lines the previous steps left in the
    # 256 MB Infinity Cache, so the gather's reads and writes reach HBM as
    # they would in a forward pass (cold, not cache-served)
    g_idsets = [d(ids) for ids in W.workload_c4_id_sets(4)]
    g_outs = [torch.empty((n_ids, 512), dtype=torch.int16, device=dev) for _ in range(3)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    stream = torch.cuda.current_stream()

    def compress(k):
        pj = c3_projs[k % 4]
        kvc.kvc_compress_store(**c3_args, kv=pj[:, :512], score=pj[:, 512:],
                               latent_out=c3_lats[k % 3], cache=c3_caches[k % 3], status=status)

    def gather(k):
        kvc.kvc_dequant_gather(g_cache, g_pt, g_idsets[k % 4], g_outs[k % 3], status)

    def step(k):
        compress(k)
        gather(k)

    # ---------------------------------------------------------------- timing
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

    # per-kernel durations: HIP events on the launch stream around replays of
    # HIP graphs of 10 back-to-back launches of one kernel (each with its
    # inputs and outputs in turn).  An untimed compress replay comes
    # first, so the device is busy when the first event is reached and no
    # host launch latency falls inside an interval; the gathers follow the
    # compresses, as in a step.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        return g

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        compress(0)
        gather(0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g_comp = capture(lambda: [compress(k) for k in range(10)])
    g_gath = capture(lambda: [gather(k) for k in range(10)])
    torch.cuda.synchronize()
    runs = max(args.steps // 10, 2)
    comp_ms, gath_ms = [], []
    for r in range(runs):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        g_comp.replay()
        a.record(stream)
        g_comp.replay()
        b.record(stream)
        g_gath.replay()
        c.record(stream)
        torch.cuda.synchronize()
        comp_ms.append(a.elapsed_time(b) / 10)
        gath_ms.append(b.elapsed_time(c) / 10)
    assert int(status.item()) == 0, f"device status {int(status.item())}"

    comp_bytes = c3_rows * (4096 + 1024 + fp4.row_bytes) + c3_tails * 2 * 2048
    gath_bytes = n_ids * (v41.row_bytes + 1024 + 4)
    comp_s = float(np.mean(comp_ms)) / 1e3
    gath_s = float(np.mean(gath_ms)) / 1e3
    comp_gbs = comp_bytes / comp_s / 1e9
    gath_gbs = gath_bytes / gath_s / 1e9
    rows_step = c3_rows + n_ids
    value = rows_step / (ms_step / 1e3)
    log(f"compress: {np.mean(comp_ms)*1e3:.1f} us  {comp_gbs:.0f} GB/s  "
        f"gather: {np.mean(gath_ms)*1e3:.1f} us  {gath_gbs:.0f} GB/s  step {ms_step*1e3:.1f} us")

    traffic = measured_traffic("dequant_gather")
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
                        "random page table -> bf16 [262144,512]; 4 id lists used in turn)",
            "compress_rows": c3_rows, "gather_rows": n_ids,
            "seed_c3": int(c3["seed"]), "odd_lengths": c3_tails,
        },
        "hbm_gbps": (comp_bytes + gath_bytes) / (ms_step / 1e3) / 1e9,
        "kernels": {
            "compress_store": {"us": float(np.mean(comp_ms)) * 1e3, "p90_us": float(np.percentile(comp_ms, 90)) * 1e3,
                               "launches_timed": 10 * runs,
                               "bytes": comp_bytes, "gbps": comp_gbs, "frac": comp_gbs / HBM_PEAK_GBS,
                               "rows_per_s": c3_rows / comp_s,
                               "traffic": measured_traffic("compress_store")},
            "dequant_gather": {"us": float(np.mean(gath_ms)) * 1e3, "p90_us": float(np.percentile(gath_ms, 90)) * 1e3,
                               "launches_timed": 10 * runs,
                               "bytes": gath_bytes, "gbps": gath_gbs, "frac": gath_gbs / HBM_PEAK_GBS,
                               "rows_per_s": n_ids / gath_s},
        },
        "roofline": {"bound": "hbm", "achieved": gath_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gath_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "dequant_gather", "algorithmic_bytes": gath_bytes},
        "cpu_baseline": None,
    }

    if not args.no_next_rows:
        out["next_rows"] = measure_next_rows(kvc, W, d, dev, stream)
        out["next_rows"]["gather_reuse_c4_8_layers"] = measure_reuse(
            kvc, g_cache, g_pt, g_idsets, g_outs, stream, layers=8)

    # ---------------------------------------------------------------- oracle
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.num_threads()
        # bounded sample: the first 4 requests of the compress batch and the
        # first 65,536 gather ids, repeated until ~10 s of CPU work
        n4 = int(lengths[:4].sum())
        sub = dict(c3)
        sub_off = c3["offsets"][:, :4].copy()
        rows_sub = int((lengths[:4] // 2).sum())
        m = 65536
        ids_sub = c4["ids"][:m]
        reps, spent, done_rows = 0, 0.0, 0
        while spent < 10.0 and reps < 400:
            cache_h = np.zeros((c3["num_pages"], 128 * fp4.row_bytes), np.uint8)
            t = time.perf_counter()
            oracle.compress(ratio=2, mode=oracle.PREFILL, kv=c3["kv"][:n4], fused=True,
                            offsets=sub_off, start_pos=c3["start_pos"][:4],
                            page_table=c3["page_table"][:4], state=c3["state"][:4].copy(),
                            norm_w=c3["norm_w"], eps=c3["eps"], freqs=c3["freqs"], cache=cache_h,
                            layout="V41_FP4", page_size=128, want_prequant=False)
            oracle.dequant_gather(c4["cache"], "V41", 64, c4["page_table"], ids_sub)
            spent += time.perf_counter() - t
            done_rows += rows_sub + m
            reps += 1
        out["cpu_baseline"] = {"value": done_rows / spent, "unit": "rows/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{reps} x (compress of the first 4 requests = "
                                         f"{rows_sub} rows + gather of the first {m} ids), "
                                         f"{spent:.1f} s"}
        del sub
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
