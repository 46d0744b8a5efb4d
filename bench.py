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
# dispatches, `--no-next-rows --no-cold-flush`), scaled by what the same counters read for a
# plain 1 GiB copy (`bench.py --copy-calibration`): FETCH_SIZE read 524301.6
# KiB and WRITE_SIZE 1048576 KiB for 1048576 KiB moved, so fetch x2.0 and write
# x1.0.  Valid only for the sources the decode-layer call is built from
# (DECODE_SOURCES).
DECODE_SOURCES = ("score.hip", "decode.hip", "decode_f32.hip", "decode_f16.hip",
                  "decode_bf16.hip", "decode_kernel.h", "topk_block.h", "qas_device.h",
                  "qas_internal.h", "qas_api.cpp")
PMC_TRAFFIC = {
    "sources_sha256": "a352bbf5bba14f890b4944b10e75ba4e6f9b96c6701450d07f5ab02ab8f42989",
    "fetch_kib": {"score_kernel": 16562.1, "decode_kernel": 34061.7},
    "write_kib": {"score_kernel": 610.0, "decode_kernel": 173.2},
    # the same passes, call on the e4m3 summary copy
    "fetch_kib_fp8": {"score8_kernel": 8498.1, "decode_kernel": 34061.7},
    "write_kib_fp8": {"score8_kernel": 304.3, "decode_kernel": 173.2},
    "fetch_factor": 2.0,
    "write_factor": 1.0,
}


# Counters of the union attention kernel (the chunk line), from passes of
# `bench.py --workload chunk --no-cpu-baseline --steps 16 --warmup 4`: medians
# over the dispatches with the chunk's own sets (the phase the chunk line
# times), the same scaling; valid only for CHUNK_SOURCES.
CHUNK_SOURCES = ("union.hip", "qas_device.h", "qas_internal.h", "qas_api.cpp")
CHUNK_PMC_TRAFFIC = {
    "sources_sha256": "61dd3e0f23ea912b3fc18a060b7fa1717750c75b58f79554bcaf72631b6e795c",
    "fetch_kib": 145403.2,
    "write_kib": 4224.2,
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


def chunk_traffic_bytes():
    """HBM bytes per chunk call of the union kernel from the recorded
    counters, or None if its sources changed since they were taken."""
    t = CHUNK_PMC_TRAFFIC
    if t["sources_sha256"] != sources_sha256(CHUNK_SOURCES):
        return None
    kib = t["fetch_kib"] * PMC_TRAFFIC["fetch_factor"] + t["write_kib"] * PMC_TRAFFIC["write_factor"]
    return int(round(kib * 1024))


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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(case, seconds):
    """The oracle as it stands, timed on the host on the same call with the
    summaries prebuilt (the GPU keeps them current): bounds of every page,
    group scores, top-K and attention per head.  BLAS is held to one thread."""
    import threadpoolctl

    import oracle
    from oracle import quest
    from query_aware_sparse_amd import traffic

    L = int(case.seq_lens[0])
    keys, values = oracle.decoded_kv(case, 0)
    m, M = quest.page_summaries(keys, L, case.S)
    q = oracle.decode(case.q[0][0], case.q_dtype)
    calls = 0
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            U = quest.kv_head_scores(quest.head_bounds(q, m, M), case.H_kv)
            for h in range(case.H_kv):
                sel = quest.top_k_pages(U[h], case.K)
                for i in range(h * case.g, (h + 1) * case.g):
                    A = quest.support(sel, L, L - 1, case.S)
                    quest.attend(q[i], keys[:, h], values[:, h], A, case.sm_scale)
            calls += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    per_call = el / calls
    nbytes = traffic.decode_layer_bytes(
        B=1, H_q=case.H_q, H_kv=case.H_kv, d=case.d, S=case.S, kv_bytes=2, q_bytes=2,
        pages_scanned=len(m), page_heads_selected=case.H_kv * case.K)["total"]
    return {"value": round(nbytes / per_call / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{calls} full decode-layer calls of the same workload (layer 0, "
                       f"summaries prebuilt), {el:.1f} s, float64 numpy, 1 thread; "
                       f"{per_call * 1e3:.1f} ms per call"),
            "cpu": platform.processor() or platform.machine()}


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


def bench_chunk(args):
    import torch

    import query_aware_sparse_amd as qas
    from query_aware_sparse_amd.staging import ChunkBatch
    from workloads import multiquery_chunk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    NL = max(1, args.layers)
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
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for w in range(max(NL, args.warmup)):
                fn(w % NL)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(NL):
                fn(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, math.ceil(args.steps / NL))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        rs = torch.cuda.current_stream()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            e0.record(rs)
            graph.replay()
            e1.record(rs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        n = reps * NL
        return (wall * 1e3 / n, float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3 / NL,
                n)

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
                     "useful_tflops": round(use, 2)},
    }
    print(json.dumps(result), flush=True)


def time_decode_calls(torch, args, NL, call, out):
    """Eager warm-up, one pass over the layers captured in a HIP graph and
    replayed; the graph's outputs must equal the eager ones.  Returns (wall
    ms per call, event-timed us per call, calls timed)."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for w in range(max(NL, args.warmup)):
            call(w % NL)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    eager_out = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(NL):
            call(i)
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup // NL)):
        graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, eager_out):
        raise RuntimeError("graph replay differs from the eager calls")
    reps = max(1, math.ceil(args.steps / NL))
    steps = reps * NL
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    replay_stream = torch.cuda.current_stream()   # graph.replay() launches here
    for e0, e1 in evs:
        e0.record(replay_stream)
        graph.replay()
        e1.record(replay_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3 / NL
    return wall * 1e3 / steps, call_us, steps


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
        _, us, _ = time_decode_calls(torch, args, NL, fn, o)
        res[name] = {"us_per_call": round(us, 3)}
        log(f"[bench] {name}: {us:.2f} us/call")
    prh = pr.cpu().numpy()
    res["exact_top_r_64"]["pages_read_per_head"] = {
        "mean": round(float(prh.mean()), 1), "min": int(prh.min()), "max": int(prh.max()),
        "of": L // case.S}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640, help="timed decode-layer calls")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--layers", type=int, default=32, help="layer caches visited in turn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--workload", choices=("decode", "chunk"), default="decode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy (counter calibration)")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the NEXT-4 timings (counter passes of the decode-layer call)")
    ap.add_argument("--no-cold-flush", action="store_true",
                    help="skip the cold-cache protocol (counter passes of the decode-layer call)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but the path runs on one GPU "
              "(no multi-GPU mode); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        return copy_calibration()
    if args.workload == "chunk":
        if args.layers == 32:
            args.layers = 4
        return bench_chunk(args)

    import torch

    import query_aware_sparse_amd as qas
    from query_aware_sparse_amd import traffic
    from query_aware_sparse_amd.staging import PagedCache, prefill, to_device
    from workloads import llama2_7b_layer, layer_queries

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    NL = args.layers
    case = llama2_7b_layer()
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

    ms_per_step, call_us, steps = time_decode_calls(torch, args, NL, call, out)
    ms_fp8, us_fp8, _ = time_decode_calls(torch, args, NL, call_fp8, out)
    cold = None
    if not args.no_cold_flush:
        cold_p50, cold_p95 = time_cold_flush(torch, call)
        log(f"[bench] cold caches (1 GiB read before each call): p50 {cold_p50:.2f} us, "
            f"p95 {cold_p95:.2f} us")
        cold = {"protocol": "1 GiB read (sum) before each call, eager launch, "
                            "20 warm-up + 200 timed calls, event-timed each",
                "p50_us": round(cold_p50, 3), "p95_us": round(cold_p95, 3)}
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
    log(f"[bench] {steps} calls: {ms_per_step * 1e3:.2f} us/call (wall), "
        f"{call_us:.2f} us/call (events), {value:.1f} GB/s")

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "llama2-7b-shaped decode layer, 32K context",
                   "batch": 1, "q_heads": case.H_q, "kv_heads": case.H_kv,
                   "head_dim": case.d, "page_size": case.S, "context": L,
                   "pages": L // case.S, "top_k_pages": case.K, "kv_dtype": "f16",
                   "layer_caches": NL, "append_current_token": True,
                   "hip_graph": True, "us_per_call": round(ms_per_step * 1e3, 3),
                   "bytes_per_call": total, "bytes_parts": nbytes,
                   "fp8_summary_copy": {
                       "us_per_call": round(us_fp8, 3), "bytes_per_call": bytes_fp8,
                       "GB/s": round(bytes_fp8 / (us_fp8 * 1e-6) / 1e9, 1),
                       "ms_per_step_wall": round(ms_fp8, 6),
                       "traffic": pmc_traffic_bytes(fp8=True)},
                   "cold_flush": cold,
                   "next_rows": next_rows},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": pmc_traffic_bytes(),
                     "kernel": "decode-layer call (score with fused append, top-k, attention with merge)",
                     "us_per_launch": round(call_us, 3)},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
