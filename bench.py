"""Benchmark: single-query GQA decode attention on one MI355X.

One step = one pass of the whole decode path (partition kernel + merge kernel)
over one batch of synthetic inputs already resident in HBM.  The timed steps
are captured in a HIP graph; a bounded spin kernel keeps the stream busy while
the host submits the replay, and a HIP event pair on the launch stream around
the replay times the steps themselves (both sides bracketed by
synchronisations).  The output after the timed replay must equal an eager
step's bit for bit.  K/V are cycled over enough device copies (>= 1 GiB in
total, i.e. more than four times the 256 MB Infinity Cache) that no step can be
served from the cache a previous step filled; a pool under 16 MB (the
launch-bound tiny workload) is cycled over 64 copies only.

Prints ONE JSON line.  The headline workload is mixed_b256, the largest
configuration (256 sequences of log-normal lengths, both single-pass and split
sequences in one batch).  `value` is its K+V GB/s (algorithmic K+V bytes / time
per step); `roofline` gives the partition kernel's own HBM roofline fraction,
its mean launch duration timed with HIP events on the launch stream around the
timed steps' partition launches issued back to back, and its fraction of the
achievable read rate a streaming-read probe measures (`read_probe`, context
beside the published peak); `warm` repeats the steps on one K/V copy (no
rotation), labelled as such and never the headline; `cpu_baseline` times the
float64 oracle on a bounded sample of the same workload, in a pool of worker
processes; `also` carries the other full-size workloads and policies, each with
a roofline object of its own.

  python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload mixed_b256]
  python bench.py --summarize-rocprof DIR     # rocprofv3 csv -> short text
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "K/V HBM GB/s (and % of peak) + decode attention µs/step, 1 GPU"
PEAK_GBS = 8000.0                       # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30                  # K/V bytes cycled per step sequence
MAX_COPIES = 64                         # K/V copies at most (each is a device copy to make)
HEADLINE = "mixed_b256"            # the largest configuration (256 sequences, mixed lengths)
KERNEL_SRC = os.path.join(ROOT, "decode_attention_08_amd", "csrc", "gqa_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PROBE_LIB = os.path.join(ROOT, "decode_attention_08_amd", "libhbm_probe.so")
PROBE_BYTES = 4 << 30                   # streaming-read probe buffer
CPU_WORKERS_MAX = 16                    # oracle pool: at most the host's share for one GPU


def source_hash() -> str:
    """Hash of the kernel source's code: line comments and whitespace are
    dropped, so that a comment edit does not void recorded counters."""
    with open(KERNEL_SRC) as f:
        code = [line.split("//", 1)[0].split() for line in f]
    return hashlib.sha256(" ".join(t for line in code for t in line).encode()).hexdigest()[:16]


# ------------------------------------------------------------------ timing --

_SPIN_RATE = {}


def _spin_cycles(torch, stream, seconds: float) -> int:
    """Cycles of torch.cuda._sleep that keep the stream busy for about `seconds`
    (rate measured once with events)."""
    if "rate" not in _SPIN_RATE:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 1 << 20
        torch.cuda._sleep(n)                       # first launch: not timed
        a.record(stream)
        torch.cuda._sleep(n)
        b.record(stream)
        torch.cuda.synchronize()
        _SPIN_RATE["rate"] = n / max(1e-6, a.elapsed_time(b) * 1e-3)   # cycles per second
    return int(_SPIN_RATE["rate"] * seconds)


XSPLIT_SUFFIX = "_xsplit"
FUSED_ROWS = ("contig_b8", "paged_b64", "long_128k", "mixed_b256")   # also timed with the fused merge
VALU_ROWS = FUSED_ROWS        # also timed with the products on the vector ALU (dot2)
POLICIES = ("default", "pages", "fused", "valu")
BENCH_WORKLOADS = ["tiny_contig", "contig_b8", "paged_b64", "long_128k", "mixed_b256",
                   "contig_d256", "paged_b64_t4", "paged_b64_xsplit", "mixed_b256_xsplit"]


def bench_case(name: str):
    """A named workload; NAME_xsplit is the paged workload NAME with the same
    logical cache in the x-split pool layout."""
    import workloads as W
    if name.endswith(XSPLIT_SUFFIX):
        return W.xsplit_case(W.workload(name[:-len(XSPLIT_SUFFIX)]))
    return W.workload(name)


def bench_desc(name: str) -> str:
    import workloads as W
    if name.endswith(XSPLIT_SUFFIX):
        return W.WORKLOADS[name[:-len(XSPLIT_SUFFIX)]][1] + ", x-split pool layout"
    return W.WORKLOADS[name][1]


def time_workload(case, policy_name: str, steps: int, warmup: int):
    """Time `steps` decode steps of one workload; returns a dict of figures.

    Pass 1 (headline): the `steps` steps captured once in a HIP graph and
    replayed between two synchronisations, so host launch overhead is not part
    of the step time.  Pass 2 (kernel roofline): the steps' partition launches
    back to back between one HIP event pair on the launch stream, then their
    merge launches the same way (mean launch duration each).  Pass 3: eager
    steps with an event pair around each, for the spread of step times.
    """
    import torch
    import decode_attention_08_amd as gq
    from tests.parity import bits_to_device

    dev = torch.device("cuda:0")
    pol = {"default": gq.policy_default,
           "pages": gq.policy_pages,
           "fused": lambda: gq.policy_default(flags=gq.GQA_POLICY_FUSED_MERGE),
           "valu": lambda: gq.policy_default(flags=gq.GQA_POLICY_VALU_DOT2)}[policy_name]()
    q = bits_to_device(case.q, case.dtype, dev)
    k0 = bits_to_device(case.k, case.dtype, dev)
    v0 = bits_to_device(case.v, case.dtype, dev)
    pool_bytes = 2 * k0.numel() * k0.element_size()
    copies = max(2, min(MAX_COPIES, math.ceil(ROTATE_BYTES / max(1, pool_bytes))))
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        if case.layout in ("paged", "paged_xsplit"):
            bt = torch.from_numpy(case.block_table).to(dev)
            ctx = torch.from_numpy(case.ctx_lens).to(dev)
            call = gq.prepare(q, k0, v0, block_table=bt, ctx_lens=ctx, scale=case.scale,
                              policy=pol, stream=stream, xsplit=case.layout == "paged_xsplit")
        else:
            call = gq.prepare(q, k0, v0, scale=case.scale, policy=pol, stream=stream)
        max_ctx = case.max_blocks * case.block_size if case.block_table is not None else case.s_kv
        has_merge = max_ctx > pol.v1_max_ctx          # some sequence may split

        for i in range(warmup):
            call(ks[i % copies], vs[i % copies], phases=3)
        torch.cuda.synchronize()
        eager = call.out.clone()                     # every K/V copy holds the same values

        # ---- pass 1: graph replay of the timed steps.  A bounded spin kernel
        # first keeps the stream busy while the host submits the replay, so the
        # event pair around it times the steps alone, not the submission: the
        # per-step figure does not depend on how many steps are timed.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                call(ks[(warmup + i) % copies], vs[(warmup + i) % copies], phases=3)
        graph.replay()                               # first replay: not timed
        torch.cuda.synchronize()
        call.out.fill_(float("nan"))
        spin = _spin_cycles(torch, stream, seconds=2e-3)
        ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        torch.cuda._sleep(spin)
        ev_a.record(stream)
        graph.replay()
        ev_b.record(stream)
        torch.cuda.synchronize()
        wall_spin = time.perf_counter() - t0
        gpu_step = ev_a.elapsed_time(ev_b) * 1e-3 / steps
        # the timed steps computed what an eager step computes, bit for bit
        replay_matches = bool(torch.equal(call.out, eager))
        if not replay_matches:
            raise RuntimeError(f"{case.name}/{policy_name}: output after the timed replay "
                               "differs from the eager step's")
        # the same replay with no spin in front (wall clock, submission included)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        del graph

        # ---- pass 1b (warm, reported as such, never the headline): the same
        # number of steps, all on the first K/V copy, so the Infinity Cache
        # serves whatever part of the cache it holds
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                call(ks[0], vs[0], phases=3)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        warm = (time.perf_counter() - t0) / steps
        del graph

        # ---- pass 2 (kernel roofline): the `steps` partition launches of the
        # timed steps back to back (each on its own K/V copy), one event pair
        # around the batch; then the merge launches the same way.  A bounded
        # spin kernel first keeps the stream busy while the host enqueues the
        # batch, so the events time GPU work, not host launch latency.
        spin = _spin_cycles(torch, stream, seconds=max(2e-3, 400e-6 * steps))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        torch.cuda._sleep(spin)
        ev[0].record(stream)
        for i in range(steps):
            call(ks[(warmup + i) % copies], vs[(warmup + i) % copies], phases=1)
        ev[1].record(stream)
        torch.cuda.synchronize()
        mean_part = ev[0].elapsed_time(ev[1]) / steps              # ms
        mean_merge = 0.0
        if has_merge:
            torch.cuda._sleep(spin)
            ev[2].record(stream)
            for i in range(steps):
                call(phases=2)
            ev[3].record(stream)
            torch.cuda.synchronize()
            mean_merge = ev[2].elapsed_time(ev[3]) / steps

        # ---- pass 3 (step-time spread): eager steps with an event pair around
        # each; includes each launch's dispatch, so it reads above pass 1.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda._sleep(spin)
        for i in range(steps):
            kk, vv = ks[(warmup + i) % copies], vs[(warmup + i) % copies]
            evs[i][0].record(stream)
            call(kk, vv, phases=3)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
    step_ev = sorted(e[0].elapsed_time(e[1]) for e in evs)
    res = {"workload": case.name, "policy": policy_name,
           "partition_size": pol.partition_size, "v1_max_ctx": pol.v1_max_ctx,
           "kv_bytes": case.kv_bytes, "copies": copies,
           "ms_per_step": gpu_step * 1e3, "us_per_step": gpu_step * 1e6,
           "gbs": case.kv_bytes / gpu_step / 1e9,
           "wall_us_per_step": wall * 1e6,
           "wall_with_spin_s": wall_spin,
           "replay_matches_eager": replay_matches,
           "warm_us_per_step": warm * 1e6, "warm_gbs": case.kv_bytes / warm / 1e9,
           "partition_us_mean": mean_part * 1e3,
           "merge_us_mean": mean_merge * 1e3,
           "step_us_events_median": step_ev[len(step_ev) // 2] * 1e3,
           "step_us_events_p10": step_ev[len(step_ev) // 10] * 1e3,
           "step_us_events_p90": step_ev[(9 * len(step_ev)) // 10] * 1e3,
           "partition_gbs": case.kv_bytes / (mean_part * 1e-3) / 1e9}
    res["pct_of_peak"] = 100.0 * res["gbs"] / PEAK_GBS
    del ks, vs
    torch.cuda.empty_cache()
    return res


def _cpu_worker(name: str, w: int, n: int, budget_s: float) -> int:
    """One oracle worker process (bench.py --cpu-worker NAME W N BUDGET): builds
    the seeded workload, prints "ready" and waits for a line on stdin, then
    walks its share of the (sequence, KV head) slices (every n-th of a seeded
    order, repeated) for budget_s of wall time with one BLAS thread, and prints
    its counts as one JSON line."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import reference as R

    case = bench_case(name)
    G = case.h_q // case.h_kv
    pairs = [(s, j) for s in range(case.num_seqs) for j in range(case.h_kv)]
    order = np.random.default_rng(0).permutation(len(pairs))
    mine = [pairs[i] for i in order[w::n]] or [pairs[order[w % len(pairs)]]]
    done_bytes, done_pairs = 0, 0
    with threadpool_limits(limits=1):
        print("ready", flush=True)
        sys.stdin.readline()                      # the start signal, sent to all workers at once
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            s, j = mine[done_pairs % len(mine)]
            R.decode(case, heads=[(s, j * G + g) for g in range(G)])
            done_bytes += int(case.ctx_lens[s]) * case.d * 2 * 2
            done_pairs += 1
        elapsed = time.perf_counter() - t0
    print(json.dumps({"bytes": done_bytes, "pairs": done_pairs, "seconds": elapsed}), flush=True)
    return 0


def cpu_baseline(name: str, budget_s: float = 10.0):
    """The float64 oracle, as it stands, on the workload `name`: a pool of
    worker processes (one per available core, at most CPU_WORKERS_MAX), each
    with one BLAS thread, over whole (sequence, KV head) slices for about
    budget_s of wall time.  Rate = all workers' K/V bytes / the longest
    worker's time.  The workers are fresh Python processes (this script with
    --cpu-worker), started together once every one has built its inputs; each
    is waited for, or killed, before this returns, so no child process
    outlives the call."""
    import subprocess

    available = len(os.sched_getaffinity(0))
    n = max(1, min(CPU_WORKERS_MAX, available))
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-worker", name,
                               str(w), str(n), repr(budget_s)],
                              stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True, env=env)
             for w in range(n)]
    got = []
    try:
        for p in procs:
            if p.stdout.readline().strip() != "ready":
                raise RuntimeError("an oracle worker failed to start")
        for p in procs:                           # start them together
            p.stdin.write("go\n")
            p.stdin.flush()
        for p in procs:
            out, _ = p.communicate(timeout=budget_s + 600)
            got.append(json.loads(out.strip().splitlines()[-1]))
            if p.returncode != 0:
                raise RuntimeError(f"an oracle worker exited with {p.returncode}")
    finally:
        for p in procs:
            if p.poll() is None:
                p.kill()
            p.wait()
    done_bytes = sum(g["bytes"] for g in got)
    done_pairs = sum(g["pairs"] for g in got)
    t_used = max(g["seconds"] for g in got)
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": n, "kind": "oracle",
            "host_cores": os.cpu_count(), "available_cores": available,
            "sample": (f"{done_pairs} (sequence, KV head) slices of {name} over {n} worker "
                       f"processes (each every {n}-th slice of a seeded order, repeated), "
                       f"{done_bytes} K/V bytes in {t_used:.2f} s; float64 numpy oracle, one "
                       f"BLAS thread per worker; {available} cores available to the process, "
                       f"{os.cpu_count()} on the host"),
            "seconds": round(t_used, 3)}


def read_probe(reps: int = 10, sizes: dict | None = None):
    """Achievable HBM read rate: the streaming-read probe (libhbm_probe.so)
    reading a PROBE_BYTES buffer, `reps` launches back to back between HIP
    events on the launch stream; best over its access patterns (grid-stride;
    chunked with 8, 16 or 32 loads in flight per lane) and grid sizes.

    `sizes` ({name: bytes}) also times reads of exactly that many bytes, each
    launch at the next disjoint offset of the buffer (as a decode step reads a
    freshly rotated cache copy), chunked with 16 loads in flight and 1, 2, 4 or
    8 workgroups per CU (best reported): the rate a bare streaming read of a
    workload's K/V byte count reaches, fixed per-launch costs included."""
    import ctypes
    import torch

    lib = ctypes.CDLL(PROBE_LIB)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32,
                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hbm_read_probe.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    buf = torch.full((PROBE_BYTES,), 0x5A, dtype=torch.uint8, device=dev)   # folds to 0
    key = 0xFFFFFFFF                                                       # never matched
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.Stream(device=dev)
    sink = torch.zeros(cus * 8 * 256, dtype=torch.int32, device=dev)
    best = (0.0, 0, 0)
    sweep = {}
    names = ("stride8", "chunked8", "chunked16", "chunked32")
    for mode in range(4):
        for per_cu in ((2, 4, 8) if mode == 0 else (1, 2, 4, 8)):
            grid = cus * per_cu
            args = (buf.data_ptr(), PROBE_BYTES, key, sink.data_ptr(), grid, mode,
                    ctypes.c_void_p(stream.cuda_stream))
            torch.cuda.synchronize()
            for _ in range(2):
                assert lib.hbm_read_probe(*args) == 0
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                assert lib.hbm_read_probe(*args) == 0
            b.record(stream)
            torch.cuda.synchronize()
            gbs = PROBE_BYTES * reps / (a.elapsed_time(b) * 1e-3) / 1e9
            sweep[f"{names[mode]}/{per_cu}_per_cu"] = round(gbs, 1)
            if gbs > best[0]:
                best = (gbs, grid, mode)
    same = {}
    for name, nbytes in (sizes or {}).items():
        nbytes = nbytes // 4096 * 4096
        regions = PROBE_BYTES // nbytes
        if regions < 2:
            continue
        n_launch = min(reps * 2, regions)
        top = 0.0
        for per_cu in (1, 2, 4, 8):
            def launch(i):
                off = (i % regions) * nbytes
                return lib.hbm_read_probe(buf.data_ptr() + off, nbytes, key, sink.data_ptr(),
                                          cus * per_cu, 2, ctypes.c_void_p(stream.cuda_stream))
            torch.cuda.synchronize()
            assert launch(regions - 1) == 0
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(n_launch):
                assert launch(i) == 0
            b.record(stream)
            torch.cuda.synchronize()
            top = max(top, nbytes * n_launch / (a.elapsed_time(b) * 1e-3) / 1e9)
        same[name] = {"bytes": nbytes, "gbs": round(top, 1)}
    del buf, sink
    torch.cuda.empty_cache()
    return {"gbs": round(best[0], 1), "bytes": PROBE_BYTES, "grid": best[1],
            "pattern": names[best[2]],
            "pct_of_peak": round(100.0 * best[0] / PEAK_GBS, 2), "sweep": sweep,
            "same_size": same,
            "method": "16-byte non-temporal loads, 256-lane workgroups; "
                      "mean over back-to-back launches between HIP events"}


def _round(x, nd: int = 2):
    return None if x is None else round(x, nd)


def traffic_record(workload: str, policy: str) -> dict:
    """The rocprofv3 record of profiles/traffic.json for this workload and
    policy, if taken on the current kernel source, else {}."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    rec = t.get(f"{workload}/{policy}")
    if not rec or rec.get("source_sha") != source_hash():
        return {}
    return rec


def traffic_for(workload: str, policy: str):
    """(HBM bytes per partition-kernel launch, rocprofv3 mean kernel duration in
    us) recorded in profiles/, if taken on the current kernel source, else
    (None, None)."""
    rec = traffic_record(workload, policy)
    avg = rec.get("partition_avg_ns")
    return rec.get("bytes_per_launch"), (None if avg is None else round(avg * 1e-3, 3))


def roofline_of(res: dict, probe=None) -> dict:
    """Roofline object of one timed workload/policy: the partition kernel's
    algorithmic K+V bytes / its mean launch duration, against the 8 TB/s peak,
    with the rocprofv3 mean duration, calibrated HBM traffic and busy figures
    recorded in profiles/ for the same kernel source (null when none)."""
    rec = traffic_record(res["workload"], res["policy"])
    achieved = res["partition_gbs"]
    avg = rec.get("partition_avg_ns")
    out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / PEAK_GBS, 4), "traffic": rec.get("bytes_per_launch"),
           "kernel": "partition_kernel", "kernel_us_mean": round(res["partition_us_mean"], 3),
           "kernel_us_rocprof": None if avg is None else round(avg * 1e-3, 3),
           "valu_busy_pct": _round(rec.get("valu_busy_pct")),
           "mfma_util_pct": _round(rec.get("mfma_util_pct")),
           "merge_us_mean": round(res["merge_us_mean"], 3)}
    if probe:
        out["frac_of_read_probe"] = round(achieved / probe["gbs"], 4)
        same = probe["same_size"].get(res["workload"])
        out["frac_of_read_probe_same_size"] = round(achieved / same["gbs"], 4) if same else None
    return out


# ---------------------------------------------------------------- rocprof --

def _rocpd(path: str, pattern: str):
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(path, pattern, "*_results.db"), recursive=True))
    return [(db, sqlite3.connect(db)) for db in dbs]


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").split("(Params)")[0][:100]


def summarize_rocprof(path: str, probe_bytes: int = 1 << 30):
    """Condense the rocprofv3 databases of one profiled bench run.

    Expects `path`/trace (--kernel-trace --stats), `path`/fetch (--pmc
    FETCH_SIZE) and `path`/write (--pmc WRITE_SIZE), each made with
    --copy-probe 1024 for the counter runs, and optionally `path`/busy (--pmc
    VALUBusy MfmaUtil).  Counter values (KiB per dispatch)
    are scaled by what the same counter reads for the 1 GiB probe copy (the
    largest copy dispatch of the run).  Returns (text, traffic record).
    """
    lines, rec = [], {}
    for db, con in _rocpd(path, "trace"):
        lines.append(f"# kernel trace: {os.path.relpath(db, path)}")
        rows = con.execute(
            "select name, count(*), avg(duration), min(duration), max(duration), grid_x, "
            "workgroup_x, vgpr_count, accum_vgpr_count, lds_size from kernels group by name "
            "order by sum(duration) desc").fetchall()
        for n, c, avg, mn, mx, gx, wx, vg, ag, lds in rows:
            lines.append(f"{_short(n):100s} calls={c} avg_ns={avg:.0f} min_ns={mn} max_ns={mx} "
                         f"grid={gx} wg={wx} vgpr={vg} agpr={ag} lds={lds}")
            if "partition_" in n:
                rec["partition_avg_ns"] = avg
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        sub = "fetch" if counter == "FETCH_SIZE" else "write"
        for db, con in _rocpd(path, sub):
            lines.append(f"# counter {counter}: {os.path.relpath(db, path)}")
            rows = con.execute(
                "select kernel_name, dispatch_id, sum(value) from counters_collection "
                "where counter_name = ? group by dispatch_id", (counter,)).fetchall()
            per = {}
            for n, _, v in rows:
                per.setdefault(_short(n), []).append(v)
            probe = max((v for n, vs in per.items() if "copyBuffer" in n for v in vs), default=None)
            factor = probe_bytes / (probe * 1024.0) if probe else None
            for n, vs in sorted(per.items()):
                lines.append(f"{n:100s} {counter}_KiB avg={sum(vs) / len(vs):.1f} "
                             f"min={min(vs):.1f} max={max(vs):.1f} dispatches={len(vs)}")
            lines.append(f"calibration: 1 GiB probe copy reads {probe} KiB -> factor {factor}")
            part = [v for n, vs in per.items() if "partition_" in n for v in vs]
            if part and factor:
                rec[counter] = {"kib_avg": sum(part) / len(part), "factor": factor,
                                "bytes_per_launch": sum(part) / len(part) * 1024.0 * factor}
    for db, con in _rocpd(path, "busy"):
        lines.append(f"# counters VALUBusy, MfmaUtil (percent): {os.path.relpath(db, path)}")
        rows = con.execute(
            "select kernel_name, counter_name, avg(value), count(*) from counters_collection "
            "where counter_name in ('VALUBusy', 'MfmaUtil') group by kernel_name, counter_name "
            "order by kernel_name").fetchall()
        for n, cname, v, c in rows:
            lines.append(f"{_short(n):100s} {cname} avg={v:.2f}% dispatches={c}")
            if "partition_" in n:
                rec["valu_busy_pct" if cname == "VALUBusy" else "mfma_util_pct"] = v
    if "FETCH_SIZE" in rec and "WRITE_SIZE" in rec:
        rec["bytes_per_launch"] = rec["FETCH_SIZE"]["bytes_per_launch"] + rec["WRITE_SIZE"]["bytes_per_launch"]
    rec["source_sha"] = source_hash()
    return "\n".join(lines), rec


# ------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--policy", default="default", choices=list(POLICIES))
    ap.add_argument("--no-also", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run one torch copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    ap.add_argument("--cpu-worker", nargs=4, metavar=("WORKLOAD", "W", "N", "BUDGET"),
                    help=argparse.SUPPRESS)
    ap.add_argument("--record-traffic", metavar="WORKLOAD/POLICY",
                    help="with --summarize-rocprof: store the traffic record in profiles/traffic.json")
    args = ap.parse_args()

    if args.cpu_worker:
        wl, w, n, budget = args.cpu_worker
        return _cpu_worker(wl, int(w), int(n), float(budget))
    if args.summarize_rocprof:
        text, rec = summarize_rocprof(args.summarize_rocprof)
        print(text)
        print("# traffic record: " + json.dumps(rec))
        if args.record_traffic:
            try:
                with open(TRAFFIC_FILE) as f:
                    table = json.load(f)
            except (OSError, ValueError):
                table = {}
            table[args.record_traffic] = rec
            with open(TRAFFIC_FILE, "w") as f:
                json.dump(table, f, indent=1, sort_keys=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not built.", file=sys.stderr)
        return 2

    # the oracle pool first: its workers start before this process touches the GPU
    cpu = None if args.no_cpu else cpu_baseline(args.workload)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    case = bench_case(args.workload)
    head = time_workload(case, args.policy, args.steps, args.warmup)
    print(f"[bench] {case.name}/{args.policy}: {head['us_per_step']:.1f} us/step, "
          f"{head['gbs']:.0f} GB/s, partition {head['partition_us_mean']:.1f} us", file=sys.stderr,
          flush=True)

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    also = {}
    if not args.no_also:
        # the default and pages' policies first, then the comparison variants
        # (fused merge, packed FMA): those keep the vector ALU busy for longer,
        # and rows timed right after them read a few percent slow
        for group in (("default", "pages"), ("fused", "valu")):
            for name in BENCH_WORKLOADS:
                c = case if name == args.workload else bench_case(name)
                for pol in group:
                    if name == args.workload and pol == args.policy:
                        continue
                    if name.endswith(XSPLIT_SUFFIX) and pol != "default":
                        continue
                    if (pol == "fused" and name not in FUSED_ROWS) or (pol == "valu" and name not in VALU_ROWS):
                        continue
                    r = time_workload(c, pol, args.steps, args.warmup)
                    also[f"{name}/{pol}"] = r
                    print(f"[bench] {name}/{pol}: {r['us_per_step']:.1f} us/step, {r['gbs']:.0f} GB/s, "
                          f"partition {r['partition_us_mean']:.1f} us ({r['partition_gbs']:.0f} GB/s)",
                          file=sys.stderr, flush=True)

    sizes = {case.name: case.kv_bytes}
    for k, r in also.items():
        if k.endswith("/default") and not k.startswith("tiny_") and XSPLIT_SUFFIX not in k:
            sizes[k.split("/")[0]] = r["kv_bytes"]
    probe = None if args.no_also else read_probe(sizes=sizes)
    also_out = {}
    for key, r in also.items():
        rec = {k: (round(v, 3) if isinstance(v, float) else v)
               for k, v in r.items() if k not in ("workload", "policy")}
        rec["roofline"] = roofline_of(r, probe)
        also_out[key] = rec
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V; no dataset)",
        "config": {"workload": case.name, "desc": bench_desc(case.name),
                   "policy": args.policy, "partition_size": head["partition_size"],
                   "v1_max_ctx": head["v1_max_ctx"], "kv_bytes": case.kv_bytes,
                   "kv_copies_rotated": head["copies"]},
        "us_per_step": round(head["us_per_step"], 2),
        "pct_of_peak": round(100.0 * head["gbs"] / PEAK_GBS, 2),
        "timing": "graph replay of the timed steps between synchronisations; a bounded spin "
                  "kernel ahead of the replay, and HIP events on the launch stream around it "
                  "(wall_us_per_step: the same replay timed by the host clock with no spin); "
                  "kernel times: HIP events around the steps' partition (then merge) launches "
                  "issued back to back; step_us_events: events around each eager step, "
                  "dispatch included",
        "replay_matches_eager": head["replay_matches_eager"],
        "wall_us_per_step": round(head["wall_us_per_step"], 2),
        "warm": {"us_per_step": round(head["warm_us_per_step"], 2),
                 "gbs": round(head["warm_gbs"], 1),
                 "note": "unflushed: every step reads the same K/V copy, so the 256 MB "
                         "Infinity Cache serves what it holds; context only"},
        "step_us_events": {"median": round(head["step_us_events_median"], 2),
                           "p10": round(head["step_us_events_p10"], 2),
                           "p90": round(head["step_us_events_p90"], 2)},
        "roofline": roofline_of(head, probe),
        "read_probe": probe,
        "cpu_baseline": cpu,
        "also": also_out,
        "kernel_source_sha": source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
