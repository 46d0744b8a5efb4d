#!/usr/bin/env python
"""Benchmark of the decode-layer hot path on one MI355X.

Workload: the Llama-2-7B-shaped decode layer (batch 1, 32 query heads = 32
KV heads, d=128, S=16, 32768-token context = 2048 pages, top-K = 256 pages,
fp16 K/V with 4 outlier channels per head x8, fp16 query), built from the
seeded generators.  One step is one decode-layer call of the library:
append of the current token's K/V row and tail summary, page bounds of all
2048 pages, top-K per KV head, sparse attention over the 256 selected pages
with the split merge.  32 separate layer caches (as in a 32-layer model,
~17 GB) are visited in turn so that no call finds its bytes in the 256 MB
Infinity Cache; the 32 calls are captured once in a HIP graph and replayed.

The value is the achieved rate on the bytes the method must move per call
(summary scan + selected K/V + q/o + the append's row and summary record),
divided by the measured time per call.  Beside it: the same call on the
e4m3 summary copy, the call under a cold-cache protocol (a read of 1 GiB
before each of 200 event-timed calls, p50 and p95, under
`config.cold_flush`), and the NEXT-4 entry points.

    python bench.py [--steps K] [--warmup W] [--layers N] [--no-cpu-baseline]

`--workload chunk` measures the multi-query chunk path instead (64K
context, S=64, 512 queries with 64-page sets, 32/8 heads, fp8 K/V, groups
of 8 queries over page unions on fp8 MFMA): one line with µs per chunk call
and executed / useful MFMA TFLOP/s against the fp8 dense peak.
"""
import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("µs per decode-layer call + achieved HBM GB/s, 32K ctx, K=256 pages, "
          "32×128 heads")
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
CHUNK_METRIC = "µs per multi-query chunk call + fp8 MFMA TFLOP/s, 64K ctx, 512 queries, union-8"

# HBM traffic of one decode-layer call from two rocprofv3 --pmc passes of this
# bench (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, mean over the pass's
# dispatches of each kernel instance; `--workload decode --no-cpu-baseline
# --no-next-rows --no-cold-flush --steps 32 --warmup 4 --sub-steps 32
# --chunk-steps 8`), scaled by what the same counters read for a plain 1 GiB
# copy (`bench.py --copy-calibration`): FETCH_SIZE read 524300 KiB and
# WRITE_SIZE 1048576 KiB for 1048576 KiB moved, so fetch x2.0 and write x1.0.
# Valid only for the sources the decode-layer call is built from
# (DECODE_SOURCES); with other sources the line reports null.
DECODE_SOURCES = ("score.hip", "decode.hip", "decode_f32.hip", "decode_f16.hip",
                  "decode_bf16.hip", "decode_kernel.h", "attend_block.h", "topk_block.h",
                  "qas_device.h", "qas_internal.h", "qas_api.cpp")
PMC_TRAFFIC = {
    "sources_sha256": "5cf883cfe4fb445a17a33b65db9369b240935f5e2461ce6f8bdf94b2d1d27184",
    "fetch_kib": {"score_kernel": 16533.4, "decode_kernel": 34067.4},
    "write_kib": {"score_kernel": 597.1, "decode_kernel": 173.3},
    # the same passes, call on the e4m3 summary copy
    "fetch_kib_fp8": {"score8_kernel": 8492.9, "decode_kernel": 34067.4},
    "write_kib_fp8": {"score8_kernel": 304.3, "decode_kernel": 173.3},
    "fetch_factor": 2.0,
    "write_factor": 1.0,
}


# Counters of the union attention kernel (the chunk line), from the same
# passes plus one of SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE,
# SQ_INSTS_MFMA, SQ_INSTS_VALU, SQ_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_F8:
# medians over the dispatches with the chunk's own sets (the phase the chunk
# line times), the same scaling.  MFMA busy is a fraction of the SIMD cycles
# while the kernel runs: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x
# GRBM_GUI_ACTIVE / 8 XCDs, the counter's sum over the XCDs); executed fp8
# flops are MOPS_F8 x 512 (110.6 GFLOP: the union accounting's 98.30 GFLOP
# plus one row-sum MFMA per page, which that accounting leaves out).
# Valid only for CHUNK_SOURCES.
CHUNK_SOURCES = ("union.hip", "qas_device.h", "qas_internal.h", "qas_api.cpp")
CHUNK_PMC_TRAFFIC = {
    "sources_sha256": "f73f478306270a4102acb4715cc6b9938f952540c24e251c3af787d2d2a81d55",
    "fetch_kib": 83799.2,
    "write_kib": 4224.0,
    "mfma_busy_frac": 0.2516,
    "valu_insts_per_mfma": 24.49,
    "mfma_insts": 843732,
}


def sources_sha256(names):
    import hashlib
    d = os.path.join(ROOT, "query_aware_sparse_amd", "csrc")
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_sources_sha256():
    return sources_sha256(DECODE_SOURCES)


def chunk_counters():
    """HBM bytes per chunk call of the union kernel and its MFMA figures from
    the recorded counters, or None if its sources changed since."""
    t = CHUNK_PMC_TRAFFIC
    if t["sources_sha256"] != sources_sha256(CHUNK_SOURCES):
        return None
    kib = t["fetch_kib"] * PMC_TRAFFIC["fetch_factor"] + t["write_kib"] * PMC_TRAFFIC["write_factor"]
    return {"traffic": int(round(kib * 1024)), "mfma_busy_frac": t["mfma_busy_frac"],
            "valu_insts_per_mfma": t["valu_insts_per_mfma"], "mfma_insts": t["mfma_insts"]}


def chunk_traffic_bytes():
    c = chunk_counters()
    return None if c is None else c["traffic"]


def pmc_traffic_bytes(fp8=False):
    """HBM bytes per decode-layer call from the recorded counters (the call on
    the e4m3 summary copy if fp8), or None if the kernels changed since they
    were taken."""
    t = PMC_TRAFFIC
    if t["sources_sha256"] is None or t["sources_sha256"] != decode_sources_sha256():
        return None
    sfx = "_fp8" if fp8 else ""
    kib = (sum(t["fetch_kib" + sfx].values()) * t["fetch_factor"] +
           sum(t["write_kib" + sfx].values()) * t["write_factor"])
    return int(round(kib * 1024))


def copy_calibration():
    """A plain device copy of known size (1 GiB, four times) to scale the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 4}), flush=True)


def bench_micro(args):
    """Rates the decode path is measured against (libqas_micro.so): scattered
    whole-tile reads in the attention kernel's load pattern (16 rows of 1 KiB
    in flight per wave, 512 workgroups of 512 threads) against the same bytes
    read in order, per buffer size and tile size; an empty kernel inside a HIP
    graph; a chain of dependent global loads.  One JSON line."""
    import ctypes

    import torch

    from query_aware_sparse_amd.build import MICRO_LIB
    assert torch.cuda.is_available(), "bench.py --micro needs a GPU"
    torch.cuda.set_device(0)
    lib = ctypes.CDLL(MICRO_LIB)
    P = ctypes.c_void_p
    lib.qas_micro_read_tiles.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    lib.qas_micro_empty.argtypes = [P]
    lib.qas_micro_chase.argtypes = [P, ctypes.c_int, P, P]
    rng = np.random.default_rng(11)
    n_wg = 512
    sink = torch.zeros(n_wg, dtype=torch.int32, device="cuda")

    def graph_us(launches, reps=20):
        """Mean us per launch of a captured sequence, replayed `reps` times."""
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for fn in launches:
                    fn(s.cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(launches))

    read_bytes = 64 << 20          # bytes one launch reads (the attention's 64 MiB)
    launches = 8                   # launches in a graph, each on its own tiles where room

    def tiles(buf_bytes, tile, ordered):
        n = read_bytes // tile
        total = buf_bytes // tile
        sets = []
        for i in range(launches):
            if ordered:
                start = (i * n) % max(1, total - n + 1)
                ids = np.arange(start, start + n, dtype=np.uint32)
            elif total >= n * launches:
                ids = rng.choice(total, n * launches, replace=False).astype(np.uint32)[i * n:(i + 1) * n]
            else:
                ids = rng.permutation(total)[:n].astype(np.uint32)
            sets.append(torch.from_numpy(ids).cuda())
        return sets

    res = {"workload": "microbenchmarks (libqas_micro.so)", "read_bytes_per_launch": read_bytes,
           "workgroups": n_wg, "reads": []}
    cases = [(64 << 20, 4096), (512 << 20, 4096), (16 << 30, 4096), (16 << 30, 8192),
             (16 << 30, 16384)]
    bufs = {}
    for buf_bytes, tile in cases:
        if buf_bytes not in bufs:
            bufs[buf_bytes] = torch.ones(buf_bytes // 4, dtype=torch.int32, device="cuda")
        buf = bufs[buf_bytes]
        for ordered in (False, True):
            sets = tiles(buf_bytes, tile, ordered)
            per = len(sets[0]) // n_wg
            us = graph_us([lambda st, ids=ids: lib.qas_micro_read_tiles(
                buf.data_ptr(), ids.data_ptr(), n_wg, per, tile, sink.data_ptr(), st)
                for ids in sets])
            entry = {"buffer_bytes": buf_bytes, "tile_bytes": tile,
                     "order": "in order" if ordered else "scattered",
                     "us_per_launch": round(us, 2),
                     "TB/s": round(read_bytes / (us * 1e-6) / 1e12, 2)}
            res["reads"].append(entry)
            log(f"[micro] {buf_bytes >> 20} MiB buffer, {tile >> 10} KiB tiles, "
                f"{entry['order']}: {us:.2f} us per 64 MiB, {entry['TB/s']} TB/s")
    del bufs
    torch.cuda.empty_cache()
    # empty kernels back to back inside a graph
    us = graph_us([lambda st: lib.qas_micro_empty(st) for _ in range(64)], reps=50)
    res["empty_kernel_us_in_graph"] = round(us, 3)
    log(f"[micro] empty kernel in a graph: {us:.3f} us each")
    # dependent loads: one lane walks a random chain through 1 GiB (one slot per
    # 4 KiB), a fresh chain per trial after 1 GiB of other reads, eager launch
    slots = (1 << 30) // 4
    hops = 2048
    dev = torch.zeros(slots, dtype=torch.int32, device="cuda")
    flush = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    per_hop = []
    for trial in range(3):
        order = rng.permutation(slots // 1024)[:hops].astype(np.int64) * 1024
        order = order[order != 0][:hops - 1]
        chain = np.concatenate([[0], order])               # 0 -> order[0] -> ...
        nxt = torch.from_numpy(np.roll(chain, -1).astype(np.int32)).cuda()
        dev[torch.from_numpy(chain).cuda()] = nxt
        torch.cuda.synchronize()
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.qas_micro_chase(dev.data_ptr(), len(chain), out.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
        e1.record()
        torch.cuda.synchronize()
        per_hop.append(e0.elapsed_time(e1) * 1e6 / len(chain))
    res["dependent_load_ns"] = round(float(np.median(per_hop)), 1)
    log(f"[micro] dependent global load, cold chain over 1 GiB: {res['dependent_load_ns']} ns each")
    print(json.dumps(res), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


_CPU = {}       # arrays shared with forked oracle workers (set before the fork)


def _cpu_heads(heads):
    """Oracle of one decode-layer call restricted to KV heads `heads`: bounds
    of every page, the group score, top-K and attention per query head."""
    from oracle import quest
    c = _CPU
    g, S, K, L = c["g"], c["S"], c["K"], c["L"]
    for h in heads:
        qh = c["q"][h * g:(h + 1) * g]
        U = quest.kv_head_scores(quest.head_bounds(qh, c["m"][:, h:h + 1], c["M"][:, h:h + 1]),
                                 1)[0]
        sel = quest.top_k_pages(U, K)
        A = quest.support(sel, L, L - 1, S)
        for i in range(g):
            quest.attend(qh[i], c["keys"][:, h], c["values"][:, h], A, c["scale"])
    return len(heads)


def cpu_baseline(case, seconds, workers):
    """The oracle as it stands, timed on the host on the same call with the
    summaries prebuilt (the GPU keeps them current): bounds of every page,
    group scores, top-K and attention per head.  Two runs: one thread (BLAS
    held to one thread), then the KV heads spread over `workers` forked
    processes of one thread each (the oracle's (request, KV head) units are
    independent).  Runs before the GPU is touched."""
    import multiprocessing

    import threadpoolctl

    import oracle
    from oracle import quest
    from query_aware_sparse_amd import traffic

    L = int(case.seq_lens[0])
    keys, values = oracle.decoded_kv(case, 0)
    m, M = quest.page_summaries(keys, L, case.S)
    _CPU.update(keys=keys, values=values, m=m, M=M, q=oracle.decode(case.q[0][0], case.q_dtype),
                g=case.g, S=case.S, K=case.K, L=L, scale=case.sm_scale)
    nbytes = traffic.decode_layer_bytes(
        B=1, H_q=case.H_q, H_kv=case.H_kv, d=case.d, S=case.S, kv_bytes=2, q_bytes=2,
        pages_scanned=len(m), page_heads_selected=case.H_kv * case.K)["total"]
    heads = list(range(case.H_kv))

    def run(fn):
        calls, t0 = 0, time.perf_counter()
        while True:
            fn()
            calls += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return calls, el

    with threadpoolctl.threadpool_limits(1):
        n1, el1 = run(lambda: _cpu_heads(heads))
        ctx = multiprocessing.get_context("fork")
        with ctx.Pool(workers) as pool:
            chunks = [heads[w::workers] for w in range(workers) if heads[w::workers]]
            pool.map(_cpu_heads, chunks)                     # warm the workers
            nw, elw = run(lambda: pool.map(_cpu_heads, chunks))
    _CPU.clear()
    per1, perw = el1 / n1, elw / nw
    return {"value": round(nbytes / perw / 1e9, 4), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": (f"{nw} full decode-layer calls of the headline workload (layer 0, "
                       f"summaries prebuilt), {elw:.1f} s, float64 numpy, KV heads over "
                       f"{workers} single-threaded processes; {perw * 1e3:.1f} ms per call"),
            "cpu": cpu_model(),
            "single_thread": {"value": round(nbytes / per1 / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "calls": n1, "seconds": round(el1, 1),
                              "ms_per_call": round(per1 * 1e3, 2)}}


def chunk_accounting(case, ids=None):
    """Executed MFMA flops (every union page of every (group, KV head) tile:
    QK and PV of 32 rows x S tokens x d), useful flops (each query head over
    its own support), and K/V bytes (union-logical and distinct).  ``ids``
    ([H_kv][N]) is an execution order (groups of consecutive slots)."""
    import numpy as np
    P = -(-case.L // case.S)
    N, H, _ = case.sets.shape
    rows = 32
    executed = useful = 0
    union_pages = 0
    distinct = set()
    for h in range(H):
        order = range(N) if ids is None else [int(x) for x in ids[h]]
        for g0 in range(0, N, case.group):
            union = set()
            for n in (order[k] for k in range(g0, min(N, g0 + case.group))):
                s = {int(p) for p in case.sets[n, h] if 0 <= p < P}
                union |= s
                toks = sum(min(case.S, min(case.L, int(case.q_pos[n]) + 1) - p * case.S)
                           for p in s if p * case.S <= case.q_pos[n])
                useful += case.g * toks * case.d * 2 * 2
            union_pages += len(union)
            distinct |= {(h, p) for p in union}
    executed = union_pages * rows * case.S * case.d * 2 * 2
    page_bytes = 2 * case.S * case.d            # fp8 K + V of one page of one head
    return {"executed_flops": executed, "useful_flops": useful,
            "union_kv_bytes": union_pages * page_bytes,
            "distinct_kv_bytes": len(distinct) * page_bytes,
            "mean_union_pages": union_pages / (H * (-(-N // case.group)))}


def bench_chunk(args, NL=4, emit=True):
    """The multi-query chunk call; returns its result dict (and prints it as
    a line of its own if `emit`)."""
    import torch

    import query_aware_sparse_amd as qas
    from query_aware_sparse_amd.staging import ChunkBatch
    from workloads import multiquery_chunk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    NL = max(1, NL)
    case = multiquery_chunk()
    log(f"[bench] workload {case.name}: L={case.L} S={case.S} N={case.N} "
        f"kq={case.kq} heads={case.H_q}/{case.H_kv} copies={NL}")
    acct = chunk_accounting(case)
    base = ChunkBatch([case])
    copies = [base]
    for _ in range(1, NL):
        c = ChunkBatch.__new__(ChunkBatch)
        c.__dict__.update(base.__dict__)
        c.k_pool = base.k_pool.clone()
        c.v_pool = base.v_pool.clone()
        c.cache = qas.make_cache(c.k_pool.view(torch.float8_e4m3fn),
                                 c.v_pool.view(torch.float8_e4m3fn), None, base.k_scale,
                                 base.v_scale)
        copies.append(c)
    out = torch.empty((NL, case.N, case.H_q, case.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((NL, case.N, case.H_q), device="cuda")
    scale = 1.0 / math.sqrt(case.d)

    window = 64
    ids = [torch.empty((case.H_kv, case.N), dtype=torch.int32, device="cuda") for _ in range(NL)]

    def regroup(i):
        c = copies[i]
        qas.qas_regroup_queries(c.db.batch, c.q_indptr, c.sets, c.S, window, c.group, ids[i])

    def call(i, order=None):
        c = copies[i]
        qas.qas_chunk_attention(c.cache, c.db.batch, c.q_indptr, c.q_pos, c.q, c.sets,
                                c.group, scale, out[i], lse[i], ids=order)

    def timed(fn):
        """Graph of one pass over the copies, replayed; returns (wall ms per
        call, event-timed us per call, calls)."""
        steps = max(NL, args.chunk_steps)
        ms, us = graph_time(torch, [lambda i=i: fn(i) for i in range(NL)], steps,
                            max(NL, min(args.warmup, 8)), out)
        return ms, us, steps

    # original order (the line's value), then the windowed regroup
    ms, call_us, steps = timed(call)
    for i in range(NL):
        regroup(i)
    torch.cuda.synchronize()
    _, pre_us, _ = timed(lambda i: call(i, ids[i]))
    _, regroup_us, _ = timed(regroup)
    _, online_us, _ = timed(lambda i: (regroup(i), call(i, ids[i])))
    acct_rg = chunk_accounting(case, ids[0].cpu().numpy())
    moved = int((ids[0].cpu().numpy() != np.arange(case.N)[None, :]).sum())
    log(f"[bench] regroup W={window}: {moved} of {case.N * case.H_kv} slots moved, mean union "
        f"{acct_rg['mean_union_pages']:.1f} pages; precomputed {pre_us:.2f} us, regroup alone "
        f"{regroup_us:.2f} us, online {online_us:.2f} us")

    # the same chunk with the query sets shuffled (per KV head), so that
    # neighbouring queries no longer share pages: original order vs regroup
    rng = np.random.default_rng(4)
    shuf = torch.from_numpy(np.ascontiguousarray(np.stack(
        [case.sets[rng.permutation(case.N), h, :] for h in range(case.H_kv)], axis=1))).cuda()
    sets_nat = [c.sets for c in copies]
    for c in copies:
        c.sets = shuf
    _, shuf_us, _ = timed(call)
    for i in range(NL):
        regroup(i)
    torch.cuda.synchronize()
    _, shuf_pre_us, _ = timed(lambda i: call(i, ids[i]))
    _, shuf_online_us, _ = timed(lambda i: (regroup(i), call(i, ids[i])))
    case_shuf = type(case).__new__(type(case))
    case_shuf.__dict__.update(case.__dict__)
    case_shuf.sets = shuf.cpu().numpy()
    shuf_union = chunk_accounting(case_shuf)["mean_union_pages"]
    shuf_union_rg = chunk_accounting(case_shuf, ids[0].cpu().numpy())["mean_union_pages"]
    for c, st in zip(copies, sets_nat):
        c.sets = st
    log(f"[bench] shuffled sets: mean union {shuf_union:.1f} -> {shuf_union_rg:.1f} pages after "
        f"regroup; original {shuf_us:.2f} us, precomputed {shuf_pre_us:.2f} us, online "
        f"{shuf_online_us:.2f} us")
    exe = acct["executed_flops"] / (call_us * 1e-6) / 1e12
    use = acct["useful_flops"] / (call_us * 1e-6) / 1e12
    log(f"[bench] {steps} chunk calls: {ms * 1e3:.2f} us/call, executed {exe:.1f} TFLOP/s, "
        f"useful {use:.1f} TFLOP/s, mean union {acct['mean_union_pages']:.1f} pages")
    result = {
        "metric": CHUNK_METRIC, "value": round(call_us, 3), "unit": "us/call", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 (fp8 MFMA), bf16 q/out, fp32 softmax", "data": "synthetic",
        "config": {"workload": "multi-query chunk, 64K context", "context": case.L,
                   "page_size": case.S, "queries": case.N, "pages_per_set": case.kq,
                   "q_heads": case.H_q, "kv_heads": case.H_kv, "head_dim": case.d,
                   "group": case.group, "cache_copies": NL, "hip_graph": True, **acct,
                   "regroup": {"window": window, "slots_moved": moved,
                               "mean_union_pages": round(acct_rg["mean_union_pages"], 2),
                               "original_ids_us": round(call_us, 3),
                               "precomputed_pi_us": round(pre_us, 3),
                               "regroup_alone_us": round(regroup_us, 3),
                               "online_pi_us": round(online_us, 3),
                               "shuffled_sets": {
                                   "mean_union_pages": round(shuf_union, 2),
                                   "mean_union_pages_regrouped": round(shuf_union_rg, 2),
                                   "original_ids_us": round(shuf_us, 3),
                                   "precomputed_pi_us": round(shuf_pre_us, 3),
                                   "online_pi_us": round(shuf_online_us, 3)}}},
        "roofline": {"bound": "mfma", "achieved": round(exe, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(exe / FP8_PEAK_TFLOPS, 4),
                     "traffic": chunk_traffic_bytes(), "kernel": "union_attn_kernel",
                     "us_per_launch": round(call_us, 3),
                     "useful_tflops": round(use, 2),
                     "counters": chunk_counters()},
    }
    if emit:
        print(json.dumps(result), flush=True)
    del copies, base, out, lse, ids, shuf
    torch.cuda.empty_cache()
    return result


def graph_time(torch, calls, steps, warmup, check=None):
    """Time exactly `steps` calls cycling through `calls` (zero-argument
    callables, e.g. one per layer cache): `warmup` eager calls (at least one
    pass), then a HIP graph of one pass (and one of the first steps % n calls),
    each replayed once untimed, then replayed so that the timed region holds
    exactly `steps` calls, bracketed
    by a device synchronisation on both sides and by events on the stream the
    graphs replay on; a pass shorter than 32 calls is repeated inside the
    graph.  ``check`` (a tensor the calls write) must come out of
    a replay equal to the eager result.  Returns (wall ms per call,
    event-timed us per call)."""
    # short passes are repeated inside one graph (at least 32 calls), so that
    # a replay's host-side launch cost stays below its GPU time
    calls = list(calls) * max(1, -(-32 // len(calls)))
    n = len(calls)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for w in range(max(n, warmup)):
            calls[w % n]()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    eager = None if check is None else check.clone()
    full = torch.cuda.CUDAGraph()
    with torch.cuda.graph(full, stream=stream):
        for c in calls:
            c()
    part = None
    if steps % n:
        part = torch.cuda.CUDAGraph()
        with torch.cuda.graph(part, stream=stream):
            for c in calls[:steps % n]:
                c()
    torch.cuda.synchronize()
    full.replay()
    torch.cuda.synchronize()
    if eager is not None and not torch.equal(check, eager):
        raise RuntimeError("graph replay differs from the eager calls")
    # the first replay of a graph costs ~30 us more than later ones (a
    # one-time cost that would land in a short timed region), so the partial
    # graph is replayed once here too, untimed
    if part is not None:
        part.replay()
        torch.cuda.synchronize()
    rs = torch.cuda.current_stream()          # graph.replay() launches here
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(rs)
    for _ in range(steps // n):
        full.replay()
    if part is not None:
        part.replay()
    e1.record(rs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, e0.elapsed_time(e1) * 1e3 / steps


def event_percentiles(torch, fn, n=200, warm=20, busy_cycles=40000):
    """p50 / p95 (us) of single calls: before each call the stream is kept
    busy by a spin kernel, so that the start event is taken when the GPU
    reaches the call rather than when the host issued it."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for i in range(warm + n):
        torch.cuda._sleep(busy_cycles)
        if i >= warm:
            evs[i - warm][0].record()
        fn(i)
        if i >= warm:
            evs[i - warm][1].record()
    torch.cuda.synchronize()
    t = np.sort([a.elapsed_time(b) * 1e3 for a, b in evs])
    return float(np.percentile(t, 50)), float(np.percentile(t, 95))


def time_cold_flush(torch, call, warm=20, timed=200):
    """The cold-cache protocol: before every call a read of a 1 GiB buffer
    (a sum) evicts the 256 MB Infinity Cache and the L2s; each call is
    event-timed on its own (eager launches, layer 0); 20 warm-up calls, then
    200 timed.  The flush only reads: a read-and-write pass leaves 1 GiB of
    dirty lines whose write-back then lands inside the timed call.  Returns
    (p50, p95) in microseconds."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")    # 1 GiB
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(timed)]
    for i in range(warm + timed):
        sink.copy_(flush.sum().view(1))
        if i >= warm:
            evs[i - warm][0].record()
        call(0)
        if i >= warm:
            evs[i - warm][1].record()
    torch.cuda.synchronize()
    t = np.sort([a.elapsed_time(b) * 1e3 for a, b in evs])
    del flush, sink
    return float(np.percentile(t, 50)), float(np.percentile(t, 95))


def bench_next_rows(torch, qas, args, case, exact, db, qs, NL):
    """Timings of the NEXT-4 entry points on the same layer caches, replayed
    from a HIP graph like the decode-layer call: a 4-token speculative
    verification block (qas_decode_positions, the last 4 tokens taken as the
    drafts), the exact top-64 tokens by branch-and-bound (qas_exact_top_r),
    and the tail rescan of a rollback (qas_rollback to a cut 5 tokens back,
    run last since it rewrites the tail record)."""
    from query_aware_sparse_amd.staging import DeviceBatch, to_device
    from workloads.cases import cast
    gamma, R = 4, 64
    dev = qs.device
    rng = np.random.default_rng(4)
    qpos = to_device(cast(rng.standard_normal((NL, 1, gamma, case.H_q, case.d)), case.q_dtype),
                     case.q_dtype)
    out_pos = torch.empty((NL, 1, gamma, case.H_q, case.d), dtype=qpos.dtype, device=dev)
    ws_pos = torch.zeros(qas.qas_positions_workspace_bytes(exact[0], db.batch, case.H_q, gamma,
                                                           case.K), dtype=torch.uint8, device=dev)

    def call_pos(i):
        qas.qas_decode_positions(exact[i], db.batch, qpos[i], case.K, case.sm_scale, out_pos[i],
                                 None, ws_pos)

    tok = torch.empty((NL, 1, case.H_q, R), dtype=torch.int32, device=dev)
    lg = torch.empty((NL, 1, case.H_q, R), dtype=torch.float32, device=dev)
    pr = torch.zeros((NL, 1, case.H_q), dtype=torch.int32, device=dev)
    ws_topr = torch.zeros(qas.qas_exact_top_r_workspace_bytes(exact[0], db.batch, case.H_q, R),
                          dtype=torch.uint8, device=dev)

    def call_topr(i):
        qas.qas_exact_top_r(exact[i], db.batch, qs[i], R, tok[i], lg[i], ws_topr, pages_read=pr[i])

    L = int(case.seq_lens[0])
    cut = DeviceBatch(np.array([L - 5], np.int32), case.pages, case.S, device=dev)

    def call_rb(i):
        qas.qas_rollback(exact[i], cut.batch)

    res = {}
    for name, fn, o in (("speculative_positions_gamma4", call_pos, out_pos),
                        ("exact_top_r_64", call_topr, tok), ("rollback_rescan", call_rb, pr)):
        _, us = graph_time(torch, [lambda i=i, fn=fn: fn(i) for i in range(NL)], NL,
                           args.warmup, o)
        res[name] = {"us_per_call": round(us, 3)}
        log(f"[bench] {name}: {us:.2f} us/call")
    prh = pr.cpu().numpy()
    res["exact_top_r_64"]["pages_read_per_head"] = {
        "mean": round(float(prh.mean()), 1), "min": int(prh.min()), "max": int(prh.max()),
        "of": L // case.S}
    return res


def _free(torch):
    import gc
    gc.collect()
    torch.cuda.empty_cache()


def bench_decode_case(torch, qas, args, case, copies, steps_per_copy=1, corrupt=False):
    """A decode-layer workload other than the headline: `copies` device copies
    of its cache (visited in turn so that no call finds its bytes in the
    Infinity Cache), and for a case with append steps one call per step, each
    appending that step's token.  Returns a dict with us per call, the
    algorithmic bytes of the average call and the achieved rate.  With
    `corrupt`, also the attention alone on seeded corrupted lists (duplicates,
    invalid IDs, empty rows) through qas_sparse_decode."""
    from query_aware_sparse_amd import traffic
    from query_aware_sparse_amd.staging import DeviceBatch, PagedCache, prefill, to_device
    from workloads import corrupt_lists

    base = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype,
                      poison=False)
    prefill(base, case)
    caches = [base.cache]
    keep = [base]
    for _ in range(1, copies):
        pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype,
                        poison=False)
        pc.k_pool.copy_(base.k_pool)
        pc.v_pool.copy_(base.v_pool)
        pc.summary.copy_(base.summary)
        caches.append(pc.cache)
        keep.append(pc)
    n_steps = max(1, case.steps) if steps_per_copy else 1
    kvb = {"f32": 4, "f16": 2, "bf16": 2}[case.kv_dtype]
    plans, nbytes = [], []
    for s in range(n_steps):
        step = s if case.steps else -1
        L = case.lengths(step)
        db = DeviceBatch(L, case.pages, case.S)
        q = to_device(case.q[step + 1], case.q_dtype)
        kn = vn = None
        if case.steps:
            kn = to_device(np.stack([case.keys[r][L[r] - 1] for r in range(case.B)]),
                           case.kv_dtype)
            vn = to_device(np.stack([case.values[r][L[r] - 1] for r in range(case.B)]),
                           case.kv_dtype)
        P = [-(-int(x) // case.S) for x in L]
        plans.append((db, q, kn, vn))
        nbytes.append(traffic.decode_layer_bytes(
            B=case.B, H_q=case.H_q, H_kv=case.H_kv, d=case.d, S=case.S, kv_bytes=kvb,
            q_bytes=kvb, pages_scanned=sum(P),
            page_heads_selected=case.H_kv * sum(min(case.K, p) for p in P),
            append_tokens=case.B if case.steps else 0)["total"])
    max_pages = max(p[0].max_pages for p in plans)
    big = max(plans, key=lambda p: p[0].max_pages)[0]
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, caches[0], big.batch, case.H_q, case.K)
    out = torch.empty((copies, case.B, case.H_q, case.d), dtype=plans[0][1].dtype, device="cuda")
    lse = torch.empty((copies, case.B, case.H_q), device="cuda")
    calls = []
    for s, (db, q, kn, vn) in enumerate(plans):
        for c in range(copies):
            calls.append(lambda c=c, db=db, q=q, kn=kn, vn=vn: qas.qas_decode_layer(
                caches[c], db.batch, q, case.K, case.sm_scale, out[c], lse[c], ws,
                k_new=kn, v_new=vn))
    steps = max(len(calls), args.sub_steps - args.sub_steps % len(calls))
    ms, us = graph_time(torch, calls, steps, len(calls))
    avg = float(np.mean(nbytes))
    res = {"us_per_call": round(us, 3), "wall_us_per_call": round(ms * 1e3, 3),
           "calls_timed": steps, "bytes_per_call": int(round(avg)),
           "GB/s": round(avg / (us * 1e-6) / 1e9, 1),
           "frac_of_hbm_peak": round(avg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "cache_copies": copies, "kv_dtype": case.kv_dtype, "batch": case.B,
           "q_heads": case.H_q, "kv_heads": case.H_kv, "page_size": case.S,
           "top_k_pages": case.K, "max_pages": max_pages,
           "seq_lens": [int(x) for x in case.seq_lens]}
    if case.steps:
        res["steps"] = n_steps
        res["append_current_token"] = True
    if corrupt:
        db = plans[0][0]
        q = plans[0][1]
        sel = torch.empty((case.B, case.H_kv, case.K), dtype=torch.int32, device="cuda")
        qas.qas_decode_layer(caches[0], db.batch, q, case.K, case.sm_scale, out[0], lse[0], ws,
                             sel_out=sel)
        torch.cuda.synchronize()
        P = [-(-int(x) // case.S) for x in case.seq_lens]
        bad, cat = corrupt_lists(sel.cpu().numpy(), P, seed=5)
        bad_t = torch.from_numpy(bad).cuda()
        wsd = qas.make_workspace(qas.QAS_OP_SPARSE_DECODE, caches[0], db.batch, case.H_q, case.K)
        scalls = [lambda c=c: qas.qas_sparse_decode(caches[c], db.batch, q, bad_t, case.K,
                                                    case.sm_scale, out[c], lse[c], wsd)
                  for c in range(copies)]
        _, us_c = graph_time(torch, scalls, max(copies, args.sub_steps), copies)
        distinct = 0
        for r in range(case.B):
            for h in range(case.H_kv):
                distinct += len({int(x) for x in bad[r, h] if 0 <= x < P[r]})
        cb = traffic.decode_layer_bytes(B=case.B, H_q=case.H_q, H_kv=case.H_kv, d=case.d,
                                        S=case.S, kv_bytes=kvb, q_bytes=kvb, pages_scanned=0,
                                        page_heads_selected=distinct)["total"]
        res["corrupted_lists_attention"] = {
            "us_per_call": round(us_c, 3), "bytes_per_call": cb,
            "GB/s": round(cb / (us_c * 1e-6) / 1e9, 1),
            "empty_rows": int((cat == 4).sum()), "rows": int(cat.size),
            "entry_point": "qas_sparse_decode (dedupe, invalid IDs dropped)"}
    del keep, caches, plans, ws, out, lse, calls
    _free(torch)
    return res


SWEEP_LENGTHS = (2048, 4096, 8192, 16384, 32768, 65536)


def bench_length_sweep(torch, qas, args, lengths=SWEEP_LENGTHS):
    """Context-length scan of one decode layer of the headline shape (32
    query = 32 KV heads, d = 128, S = 16, budget K = 256 pages, f16): per
    length, full attention over every page (qas_sparse_decode on the whole
    page list) against the Quest call (qas_decode_layer) and its stages
    (qas_score_pages, qas_topk_pages, qas_sparse_decode on the selected
    pages), each replayed from a HIP graph over enough cache copies that the
    calls read at least 1 GiB of K/V between two visits of one copy.  K/V and
    queries are N(0, 1) fp16 from a seeded device generator, identity page
    table, summaries built by qas_append.  Below K * S tokens the budget
    covers every page.  Lengths run from 2K to twice the headline context
    (full attention through qas_sparse_decode takes rows of up to 4096
    pages)."""
    from query_aware_sparse_amd.staging import DeviceBatch, PagedCache
    H, d, S, K = 32, 128, 16, 256
    scale = 1.0 / math.sqrt(d)
    gen = torch.Generator(device="cuda")
    res = {"lengths": list(lengths), "quest_us": [], "dense_us": [], "score_us": [],
           "topk_us": [], "attention_us": [], "copies": []}
    for L in lengths:
        P = L // S
        kv_bytes = 2 * L * H * d * 2
        NL = int(min(16, max(2, -(-(1 << 30) // kv_bytes))))
        gen.manual_seed(1000 + L)
        pcs = [PagedCache(P, H, S, d, "f16", poison=False)]
        db = DeviceBatch([L], [np.arange(P, dtype=np.int32)], S)
        empty = DeviceBatch([0], [np.arange(P, dtype=np.int32)], S)
        before = qas.make_batch(empty.seq_lens, db.page_indptr, db.page_indices, db.total_pages,
                                db.max_pages)
        k = torch.randn((L, H, d), generator=gen, device="cuda").half()
        v = torch.randn((L, H, d), generator=gen, device="cuda").half()
        qas.qas_append(pcs[0].cache, before, torch.tensor([0, L], dtype=torch.int32,
                                                          device="cuda"), L, L, k, v)
        del k, v
        for _ in range(1, NL):
            pc = PagedCache(P, H, S, d, "f16", poison=False)
            pc.k_pool.copy_(pcs[0].k_pool)
            pc.v_pool.copy_(pcs[0].v_pool)
            pc.summary.copy_(pcs[0].summary)
            pcs.append(pc)
        q = torch.randn((NL, 1, H, d), generator=gen, device="cuda").half()
        out = torch.empty((NL, 1, H, d), dtype=torch.float16, device="cuda")
        lse = torch.empty((NL, 1, H), device="cuda")
        kk = min(K, P)
        wsl = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pcs[0].cache, db.batch, H, kk)
        wsd = qas.make_workspace(qas.QAS_OP_SPARSE_DECODE, pcs[0].cache, db.batch, H, P)
        full = torch.arange(P, dtype=torch.int32, device="cuda").repeat(1, H, 1).contiguous()
        scores = torch.empty((NL, P * H), device="cuda")
        sel = torch.empty((NL, 1, H, kk), dtype=torch.int32, device="cuda")
        quest = [lambda i=i: qas.qas_decode_layer(pcs[i].cache, db.batch, q[i], kk, scale,
                                                  out[i], lse[i], wsl) for i in range(NL)]
        dense = [lambda i=i: qas.qas_sparse_decode(pcs[i].cache, db.batch, q[i], full, P, scale,
                                                   out[i], lse[i], wsd) for i in range(NL)]
        score = [lambda i=i: qas.qas_score_pages(pcs[i].cache, db.batch, q[i], scores[i])
                 for i in range(NL)]
        topk = [lambda i=i: qas.qas_topk_pages(scores[i], db.batch, H, S, kk, sel[i])
                for i in range(NL)]
        attn = [lambda i=i: qas.qas_sparse_decode(pcs[i].cache, db.batch, q[i], sel[i], kk,
                                                  scale, out[i], lse[i], wsd)
                for i in range(NL)]
        steps = max(NL, 64)
        us = {}
        for name, calls, chk in (("quest", quest, out), ("dense", dense, out),
                                 ("score", score, scores), ("topk", topk, sel),
                                 ("attention", attn, out)):
            _, us[name] = graph_time(torch, calls, steps, NL, chk)
            res[name + "_us"].append(round(us[name], 3))
        res["copies"].append(NL)
        log(f"[bench] length {L}: quest {us['quest']:.2f} us (score {us['score']:.2f}, top-k "
            f"{us['topk']:.2f}, attention {us['attention']:.2f}), full attention "
            f"{us['dense']:.2f} us, {NL} copies")
        del pcs, db, empty, before, q, out, lse, wsl, wsd, full, scores, sel
        _free(torch)
    faster = [L for L, a, b in zip(lengths, res["quest_us"], res["dense_us"]) if a < b]
    res["quest_faster_from"] = faster[0] if faster else None
    res["note"] = ("per length: full attention = qas_sparse_decode over every page; quest = "
                   "qas_decode_layer (score + top-K + attention) with K = 256 pages (4096 "
                   "tokens; all pages below that); stages through their own entry points; "
                   "graph replays over cache copies, event-timed")
    return res


def bench_stages(torch, qas, args, case, exact, db, qs, NL):
    """Stages of the headline call timed through their own entry points over
    the same layer caches: page scores (qas_score_pages), top-K
    (qas_topk_pages; mean of a graph replay, and p50 / p95 of single calls)
    and attention with the split merge on those lists (qas_sparse_decode)."""
    from query_aware_sparse_amd import traffic
    L = int(case.seq_lens[0])
    P = L // case.S
    scores = torch.empty((NL, P * case.H_kv), device="cuda")
    sel = torch.empty((NL, 1, case.H_kv, case.K), dtype=torch.int32, device="cuda")
    out = torch.empty((NL, 1, case.H_q, case.d), dtype=torch.float16, device="cuda")
    lse = torch.empty((NL, 1, case.H_q), device="cuda")
    wsd = qas.make_workspace(qas.QAS_OP_SPARSE_DECODE, exact[0], db.batch, case.H_q, case.K)
    score = [lambda i=i: qas.qas_score_pages(exact[i], db.batch, qs[i], scores[i])
             for i in range(NL)]
    topk = [lambda i=i: qas.qas_topk_pages(scores[i], db.batch, case.H_kv, case.S, case.K, sel[i])
            for i in range(NL)]
    attn = [lambda i=i: qas.qas_sparse_decode(exact[i], db.batch, qs[i], sel[i], case.K,
                                              case.sm_scale, out[i], lse[i], wsd)
            for i in range(NL)]
    _, us_s = graph_time(torch, score, NL, NL, scores)
    _, us_t = graph_time(torch, topk, NL, NL, sel)
    _, us_a = graph_time(torch, attn, NL, NL, out)
    p50, p95 = event_percentiles(torch, lambda i: topk[i % NL]())
    parts = traffic.decode_layer_bytes(B=1, H_q=case.H_q, H_kv=case.H_kv, d=case.d, S=case.S,
                                       kv_bytes=2, q_bytes=2, pages_scanned=P,
                                       page_heads_selected=case.H_kv * case.K)
    sb = parts["summary"] + parts["q_out"] // 2
    ab = parts["selected_kv"] + parts["q_out"]
    log(f"[bench] stages: score {us_s:.2f} us, top-k {us_t:.2f} us (p50 {p50:.2f}, p95 {p95:.2f}),"
        f" attention+merge {us_a:.2f} us")
    res = {"score_us": round(us_s, 3), "score_GB/s": round(sb / (us_s * 1e-6) / 1e9, 1),
           "topk_us": round(us_t, 3), "topk_p50_us": round(p50, 3), "topk_p95_us": round(p95, 3),
           "attention_merge_us": round(us_a, 3),
           "attention_GB/s": round(ab / (us_a * 1e-6) / 1e9, 1),
           "note": ("each stage through its own entry point (qas_score_pages, qas_topk_pages, "
                    "qas_sparse_decode) over the same 32 layer caches; the fused call runs "
                    "the same stages with fewer kernel boundaries; top-K p50/p95 over 200 "
                    "single event-timed calls")}
    del scores, sel, out, lse, wsd
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640, help="timed decode-layer calls")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--layers", type=int, default=32, help="layer caches visited in turn")
    ap.add_argument("--sub-steps", type=int, default=256,
                    help="timed calls of each other workload (rounded to whole passes)")
    ap.add_argument("--chunk-steps", type=int, default=640, help="timed chunk calls per variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--workload", choices=("all", "decode", "chunk", "config1", "config3",
                                           "config5", "sweep"), default="all",
                    help="all: the headline line with every workload; the others time "
                         "one workload alone (profiling passes)")
    ap.add_argument("--micro", action="store_true",
                    help="only run the microbenchmarks of libqas_micro.so (read rates, "
                         "kernel boundary, dependent loads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy (counter calibration)")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the NEXT-4 timings")
    ap.add_argument("--no-cold-flush", action="store_true",
                    help="skip the cold-cache protocol")
    ap.add_argument("--no-length-sweep", action="store_true",
                    help="skip the context-length scan (its decode-layer calls share the "
                         "headline's kernels)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but the path runs on one GPU "
              "(no multi-GPU mode); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("bench.py: --steps must be >= 1")
    if args.copy_calibration:
        return copy_calibration()
    if args.micro:
        return bench_micro(args)
    if args.workload == "chunk":
        args.chunk_steps = args.steps
        return bench_chunk(args, NL=4 if args.layers == 32 else args.layers)

    from workloads import (batched_gqa_append, layer_queries, llama2_7b_layer,
                           stress_long_context, tiny_single_head)

    case = llama2_7b_layer()
    cpu = None
    if args.workload in ("all", "decode") and not args.no_cpu_baseline:
        # the oracle runs before the GPU is touched (its workers are forked)
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"[bench] timing the oracle on the host (1 thread, then {workers} processes) ...")
        cpu = cpu_baseline(case, args.cpu_seconds, workers)

    import torch

    import query_aware_sparse_amd as qas
    from query_aware_sparse_amd import traffic
    from query_aware_sparse_amd.staging import PagedCache, prefill, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    subs = {"config1": (lambda: tiny_single_head(), 1, "tiny single instance (d16, S4, 64 tokens)"),
            "config3": (lambda: batched_gqa_append(), 8,
                        "batched GQA decode with append (8 requests, 8K-64K, 32/8 heads, bf16)"),
            "config5": (lambda: stress_long_context(), 2,
                        "stress: 16 requests x 131072 tokens, 32/8 heads, S32, K41, fp16")}
    if args.workload == "sweep":
        res = bench_length_sweep(torch, qas, args)
        print(json.dumps({"workload": "sweep", **res}), flush=True)
        return
    if args.workload in subs:
        make, copies, what = subs[args.workload]
        res = bench_decode_case(torch, qas, args, make(), copies,
                                corrupt=args.workload == "config5")
        res["workload"] = what
        print(json.dumps({"workload": args.workload, **res}), flush=True)
        return

    NL = args.layers
    L = int(case.seq_lens[0])
    log(f"[bench] workload {case.name}: L={L} P={L // case.S} K={case.K} "
        f"H={case.H_q}x{case.d} layers={NL}")

    # layer 0 filled through the library's append (exact summaries and their
    # e4m3 copy); other layers are copies.  The line's value uses the exact
    # summaries; the e4m3-copy variant is reported beside it.
    base = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype,
                      fp8_summaries=True)
    db = prefill(base, case)
    layers = [base]
    for _ in range(1, NL):
        pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype,
                        poison=False, fp8_summaries=True)
        pc.k_pool.copy_(base.k_pool)
        pc.v_pool.copy_(base.v_pool)
        pc.summary.copy_(base.summary)
        pc.summary_fp8.copy_(base.summary_fp8)
        pc.summary_fp8_scale.copy_(base.summary_fp8_scale)
        layers.append(pc)
    exact = [qas.make_cache(pc.k_pool, pc.v_pool, pc.summary) for pc in layers]
    qs = to_device(layer_queries(case, NL), case.q_dtype)          # [NL][1][H][d]
    k_new = to_device(case.keys[0][L - 1:L], case.kv_dtype)      # current token
    v_new = to_device(case.values[0][L - 1:L], case.kv_dtype)
    out = torch.empty((NL, 1, case.H_q, case.d), dtype=torch.float16, device=dev)
    lse = torch.empty((NL, 1, case.H_q), dtype=torch.float32, device=dev)
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, base.cache, db.batch, case.H_q, case.K,
                            device=dev)
    torch.cuda.synchronize()

    def call(i):
        qas.qas_decode_layer(exact[i], db.batch, qs[i], case.K, case.sm_scale,
                             out[i], lse[i], ws, k_new=k_new, v_new=v_new)

    def call_fp8(i):
        qas.qas_decode_layer(layers[i].cache, db.batch, qs[i], case.K, case.sm_scale,
                             out[i], lse[i], ws, k_new=k_new, v_new=v_new)

    calls = [lambda i=i: call(i) for i in range(NL)]
    ms_per_step, call_us = graph_time(torch, calls, args.steps, args.warmup, out)
    sub_steps = max(NL, args.sub_steps - args.sub_steps % NL)
    ms_fp8, us_fp8 = graph_time(torch, [lambda i=i: call_fp8(i) for i in range(NL)], sub_steps,
                                NL, out)
    p50c, p95c = event_percentiles(torch, lambda i: call(i % NL))
    log(f"[bench] single calls: p50 {p50c:.2f} us, p95 {p95c:.2f} us")
    cold = None
    if not args.no_cold_flush:
        cold_p50, cold_p95 = time_cold_flush(torch, call)
        log(f"[bench] cold caches (1 GiB read before each call): p50 {cold_p50:.2f} us, "
            f"p95 {cold_p95:.2f} us")
        cold = {"protocol": "1 GiB read (sum) before each call, eager launch, "
                            "20 warm-up + 200 timed calls, event-timed each",
                "p50_us": round(cold_p50, 3), "p95_us": round(cold_p95, 3)}
    stages = bench_stages(torch, qas, args, case, exact, db, qs, NL)
    next_rows = None if args.no_next_rows else bench_next_rows(torch, qas, args, case, exact, db,
                                                               qs, NL)
    bytes_fp8 = traffic.decode_layer_bytes(
        B=1, H_q=case.H_q, H_kv=case.H_kv, d=case.d, S=case.S, kv_bytes=2, q_bytes=2,
        pages_scanned=L // case.S, page_heads_selected=case.H_kv * case.K,
        append_tokens=1, fp8_summaries=True)["total"]
    log(f"[bench] e4m3 summary copy: {us_fp8:.2f} us/call (events), "
        f"{bytes_fp8 / (us_fp8 * 1e-6) / 1e9:.1f} GB/s on {bytes_fp8} B")

    nbytes = traffic.decode_layer_bytes(
        B=1, H_q=case.H_q, H_kv=case.H_kv, d=case.d, S=case.S, kv_bytes=2, q_bytes=2,
        pages_scanned=L // case.S, page_heads_selected=case.H_kv * case.K,
        append_tokens=1)
    total = nbytes["total"]
    if cold:
        cold["GB/s_p50"] = round(total / (cold["p50_us"] * 1e-6) / 1e9, 1)
    value = total / (ms_per_step * 1e-3) / 1e9
    achieved = total / (call_us * 1e-6) / 1e9
    log(f"[bench] {args.steps} calls: {ms_per_step * 1e3:.2f} us/call (wall), "
        f"{call_us:.2f} us/call (events), {value:.1f} GB/s")
    del layers, exact, out, lse, ws, qs
    _free(torch)
    sweep = (bench_length_sweep(torch, qas, args)
             if args.workload == "all" and not args.no_length_sweep else None)

    # the other workloads, each with its own roofline fraction
    workloads = {}
    for key, (make, copies, what) in subs.items():
        log(f"[bench] {key}: {what} ...")
        res = bench_decode_case(torch, qas, args, make(), copies, corrupt=key == "config5")
        res["workload"] = what
        workloads[key] = res
        log(f"[bench] {key}: {res['us_per_call']:.2f} us/call, {res['GB/s']:.1f} GB/s")
    log("[bench] config4: multi-query chunk ...")
    chunk = bench_chunk(args, NL=4, emit=False)
    workloads["config4"] = {"workload": "multi-query chunk, 64K context, 512 queries, union-8, "
                                        "fp8 K/V",
                            "us_per_call": chunk["value"], **chunk["config"],
                            "roofline": chunk["roofline"]}
    workloads["config2"] = {"workload": "the headline line (this line's value)",
                            "us_per_call": round(call_us, 3),
                            "GB/s": round(achieved, 1),
                            "frac_of_hbm_peak": round(achieved / HBM_PEAK_GBS, 4)}

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "llama2-7b-shaped decode layer, 32K context",
                   "batch": 1, "q_heads": case.H_q, "kv_heads": case.H_kv,
                   "head_dim": case.d, "page_size": case.S, "context": L,
                   "pages": L // case.S, "top_k_pages": case.K, "kv_dtype": "f16",
                   "layer_caches": NL, "append_current_token": True,
                   "hip_graph": True, "us_per_call": round(ms_per_step * 1e3, 3),
                   "bytes_per_call": total, "bytes_parts": nbytes,
                   "single_call_p50_us": round(p50c, 3), "single_call_p95_us": round(p95c, 3),
                   "stages": stages,
                   "length_sweep": sweep,
                   "fp8_summary_copy": {
                       "us_per_call": round(us_fp8, 3), "bytes_per_call": bytes_fp8,
                       "GB/s": round(bytes_fp8 / (us_fp8 * 1e-6) / 1e9, 1),
                       "ms_per_step_wall": round(ms_fp8, 6),
                       "traffic": pmc_traffic_bytes(fp8=True)},
                   "cold_flush": cold,
                   "next_rows": next_rows,
                   "workloads": workloads},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": pmc_traffic_bytes(),
                     "kernel": "decode-layer call (score with fused append, top-k, attention with merge)",
                     "us_per_launch": round(call_us, 3)},
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
