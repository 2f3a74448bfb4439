"""Benchmark of paged-KV GQA decode attention on one MI355X.

A step is one pa_decode_run (partial kernel + merge kernel) over one batch of
synthetic decode inputs.  Default workload: Llama-3.2-1B-shaped decode,
batch 1, Hq 32 / Hkv 8, head_dim 64, fp16, 3060 tokens of context in a
shuffled 4096-page pool.

Timed region: W eager warm-up steps, then exactly K steps replayed from one
HIP graph, bracketed by synchronisations, timed with events on the launch
stream.  The K steps cycle over R replicas of the workload whose page pools
are independent random permutations of the same pages (every replica computes
the same result); R is large enough that a replica's KV is read again only
after four times the GPU's last-level cache capacity of other replicas' KV,
and a 1 GiB read flush runs before the timed replay (and before every
other measured phase), so each step reads its KV from HBM rather than
from cache at any K.  Inputs are resident in HBM before the timed region
starts.  cold_per_call_us: single calls timed one at a time, each after a
flush (p10 / median / p90 over --cold-calls calls).

value = algorithmic KV bytes per step / seconds per step (GB/s), where the
algorithmic bytes are the K and V bytes of the visible keys only.

roofline: the dominant kernel is the partial kernel; its average duration
comes from start/stop HIP events the library records around each of its
launches (pa_decode_profile_begin/end) in a second pass of K steps run
eagerly on the same stream.  achieved = algorithmic KV bytes per launch /
average partial-kernel duration; peak = 8 TB/s HBM.  traffic (HBM bytes per
launch measured with rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by the same
counters on a plain copy) is read from profiles/traffic.json and reported
only while the kernel sources hash to the value recorded there.

cpu_baseline: the float64 CPU oracle timed on this host on the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from paged_kv_decode_amd import binding  # noqa: E402
from paged_kv_decode_amd import workloads as W  # noqa: E402

METRIC = "decode-attention µs/step + achieved KV HBM GB/s (% of peak) at ctx 3k / 100k"
PEAK_GBPS = 8000.0
CACHE_BYTES = 288 << 20          # 256 MiB MALL + 8 x 4 MiB L2
FLUSH_BYTES = 1 << 30            # read and written before every timed phase
KERNEL_SOURCES = ["paged_kv_decode_amd/csrc/pa_decode_kernels.hip",
                  "paged_kv_decode_amd/csrc/partial_kernel.h",
                  "paged_kv_decode_amd/csrc/pa_decode_balanced.hip",
                  "paged_kv_decode_amd/csrc/planner.cpp"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Replicas:
    """R page-permuted copies of one problem, resident on the GPU."""

    def __init__(self, p: W.Problem, R: int, eng: binding.PagedDecode, partition_size: int,
                 table: str = "dense"):
        self.p = p
        dev = torch.device("cuda", 0)
        k0 = p.k_cache.to(dev)
        v0 = p.v_cache.to(dev)
        pt0 = p.page_table.to(dev)
        self.q = p.q.to(dev)
        self.lens = p.context_lens.to(dev)
        B, Hq, D = p.q.shape
        self.out = torch.empty((B, Hq, D), dtype=p.q.dtype, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        csr = W.to_csr(p) if table == "csr" else None
        if csr is not None:
            ws_bytes = binding.pa_decode_workspace_size_csr(eng.handle, B, csr.nnz_pages,
                                                            p.max_context_len, p.window,
                                                            partition_size)
            self.run = eng.run_csr_args
        else:
            ws_bytes = eng.workspace_size(B, p.max_context_len, p.window, partition_size)
            self.run = eng.run_args
        self.ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.caches = []
        self.args = []
        gen = torch.Generator(device="cpu")
        gen.manual_seed(1234)
        num_pages = k0.shape[0]
        for r in range(R):
            if r == 0:
                k, v, pt = k0, v0, pt0
                perm = None
            else:
                perm = torch.randperm(num_pages, generator=gen).to(dev)
                k = torch.empty_like(k0)
                v = torch.empty_like(v0)
                k[perm] = k0
                v[perm] = v0
                pt = perm.to(torch.int32)[pt0.long()]
            self.caches.append((k, v, pt))
            if csr is not None:
                idx = csr.indices.to(dev)
                if perm is not None and idx.numel():
                    idx = perm.to(torch.int32)[idx.long()]
                self.args.append(eng.make_csr_args(
                    self.q, k, v, csr.indptr.to(dev), idx.contiguous(), csr.last_page_len.to(dev),
                    csr.nnz_pages, p.scale, self.out, self.lse, max_context_len=p.max_context_len,
                    sliding_window=p.window, partition_size=partition_size, workspace=self.ws))
            else:
                self.args.append(eng.make_args(self.q, k, v, pt, self.lens, p.scale, self.out,
                                               self.lse, max_context_len=p.max_context_len,
                                               sliding_window=p.window,
                                               partition_size=partition_size, workspace=self.ws))


def run_oracle_baseline(p: W.Problem, budget_s: float):
    import oracle
    threads = oracle.max_threads()
    reps = 0
    t0 = time.perf_counter()
    out = lse = None
    while True:
        out, lse = oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens,
                                 p.scale, window=p.window, rotary=p.workload.rope)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return out, lse, reps, el, threads


def replica_count(kv_bytes, pool_bytes, layers=1, replicas=None):
    """Replicas in the cold-cache rotation: enough that a replica's K/V is
    read again only after 4 x CACHE_BYTES of other replicas' K/V (at most
    64 GiB of pools, at least two per layer), a whole number of steps of
    `layers` distinct caches; or the count asked for."""
    if replicas is None:
        R = max(2 * layers, math.ceil(4 * CACHE_BYTES / max(kv_bytes, 1)) + 1)
        R = min(R, max(2 * layers, int((64 << 30) // pool_bytes)))
    else:
        R = max(replicas, layers)
    return -(-R // layers) * layers


class Flusher:
    """Evicts the K/V a previous phase left in the GPU's caches: the library's
    read probe (the partial kernel's own 16-byte non-temporal load) reads
    FLUSH_BYTES, four times the 256 MB MALL and far past the 8 x 4 MB of L2.
    Measured on MI355X, a step timed right after this flush costs what it
    costs after 20 steps over another replica's K/V (the eviction a decode
    loop sees), while a flush with ordinary loads (torch's fill_ or sum over
    1 GiB) adds about 1 us per call more and slows the next ~20 ms of steps
    for reasons other than K/V residency.  Queued on the current stream
    outside every timed interval, right before its start event (no host
    synchronisation in between, so the GPU is busy with the flush while the
    timed work is being submitted)."""

    def __init__(self):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(binding.PA_DECODE_PROBE_WAVES, dtype=torch.int32, device="cuda")
        self.count = 0

    def __call__(self):
        binding.pa_decode_read_probe(self.buf.data_ptr(), 0, FLUSH_BYTES // 8192, 8192,
                                     self.sink.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        self.count += 1


def percentiles(xs):
    xs = sorted(xs)
    if not xs:
        return None
    q = lambda f: xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]  # noqa: E731
    return {"p10": round(q(0.10), 3), "median": round(q(0.5), 3), "p90": round(q(0.90), 3),
            "min": round(xs[0], 3), "max": round(xs[-1], 3), "n": len(xs)}


def bench_workload(name, steps, warmup, replicas, partition_size, mode, eng_cache,
                   table="dense", layers=1, phases="all", cold_calls=100, flusher=None):
    """One step = `layers` decode-attention calls on distinct KV caches
    (page-permuted copies of the workload's pool, one per layer), launched
    back to back.

    Cold caches at any step count: each replica's K/V is read again only
    after at least 4 x CACHE_BYTES of other replicas' K/V (R replicas in
    rotation), and a FLUSH_BYTES flush runs before every phase (warm-up,
    graph upload replay, timed replay, kernel-timing pass, each spread
    replay, the per-call figures), so no phase starts on data a previous
    phase left in a cache.  phases="cold" leaves out the warm-cache figure,
    the spread replays and the read probe (the profiler then sees only cold
    launches of the kernels)."""
    w = W.CONFIGS[name]
    S = w.partition_size if partition_size is None else partition_size
    t0 = time.perf_counter()
    p = W.generate(w)
    log("%s: generated in %.1fs" % (name, time.perf_counter() - t0))
    key = (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, w.rope)
    eng = eng_cache.get(key)
    if eng is None:
        eng = binding.PagedDecode(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype,
                                  max_batch=max(w.batch, 64), max_context_len=1 << 20,
                                  rope=w.rope)
        eng_cache[key] = eng
    flush = flusher if flusher is not None else Flusher()
    kv_bytes = p.kv_bytes()
    R = replica_count(kv_bytes, 2 * p.k_cache.numel() * p.k_cache.element_size(), layers,
                      replicas)
    reps = Replicas(p, R, eng, S, table)
    log("%s: %d replicas, %.1f MB KV per step" % (name, R, kv_bytes / 1e6))
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    # Every replica must produce the same bits (page-shuffle invariance).
    outs = []
    for r in (0, R - 1):
        reps.run(reps.args[r], sp)
        torch.cuda.synchronize()
        outs.append((reps.out.clone(), reps.lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), \
        "replicas disagree"
    plan = eng.last_plan().as_dict()

    L = layers
    flush()
    for i in range(warmup * L):
        reps.run(reps.args[i % R], sp)
    torch.cuda.synchronize()

    if mode == "graph":
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(steps * L):
                    reps.run(reps.args[i % R], cs)
        stream.wait_stream(cap)
        flush()
        g.replay()  # upload / first replay, untimed
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush()
    start.record(stream)
    if mode == "graph":
        g.replay()
    else:
        for i in range(steps * L):
            reps.run(reps.args[i % R], sp)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_per_step = ms_total / steps

    # Spread and warm-cache figures (after the timed region; not part of it):
    # the same graph replayed five more times, each after a flush (µs/step
    # of each replay), and, for graph mode, K steps on one replica only, so
    # that its K/V stays in the L2 and the 256 MB MALL where it fits.
    spread = None
    warm = None
    if mode == "graph" and phases == "all":
        per = []
        for _ in range(5):
            flush()
            start.record(stream)
            g.replay()
            stop.record(stream)
            torch.cuda.synchronize()
            per.append(1e3 * start.elapsed_time(stop) / steps)
        per.sort()
        spread = {"min": round(per[0], 3), "median": round(per[2], 3), "max": round(per[-1], 3),
                  "replays": 5}
        if layers == 1:
            gw = torch.cuda.CUDAGraph()
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                with torch.cuda.graph(gw, stream=cap):
                    cs = torch.cuda.current_stream().cuda_stream
                    for i in range(steps):
                        reps.run(reps.args[0], cs)
            stream.wait_stream(cap)
            gw.replay()
            torch.cuda.synchronize()
            start.record(stream)
            gw.replay()
            stop.record(stream)
            torch.cuda.synchronize()
            warm = round(1e3 * start.elapsed_time(stop) / steps, 3)
            del gw
    if mode == "graph":
        del g

    # Kernel durations: start/stop events recorded around each launch.
    nprof = min(steps, 2000)
    flush()
    binding.pa_decode_profile_begin(eng.handle, nprof)
    for i in range(nprof):
        reps.run(reps.args[i % R], sp)
    pm, pn, mm, mn = binding.pa_decode_profile_end(eng.handle)
    partial_us = 1e3 * pm / max(pn, 1)
    merge_us = 1e3 * mm / max(mn, 1) if mn else 0.0

    # One cold call at a time (layers == 1): a flush, then events around one
    # step (all of its kernels); the flush keeps the GPU busy while the step
    # is queued, so the interval holds the step's kernels and the gaps
    # between them, not the host's launch time.
    cold = None
    if layers == 1 and cold_calls > 0:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(cold_calls)]
        for i in range(cold_calls):
            flush()
            ev[i][0].record(stream)
            reps.run(reps.args[i % R], sp)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        cold = percentiles([1e3 * a.elapsed_time(b) for a, b in ev])

    ceiling = None
    if layers == 1 and phases == "all":
        flush()
        ceiling = same_pages_probe(reps, p, min(steps, 500), sp, flush)

    res = {
        "workload": name, "p": p, "plan": plan, "kv_bytes": kv_bytes * L, "replicas": R,
        "read_ceiling": ceiling, "spread": spread, "warm_us_per_step": warm,
        "cold_per_call_us": cold,
        "cold_guard": {"flush_bytes": FLUSH_BYTES, "flushes": flush.count,
                       "reread_after_bytes": int(kv_bytes * (R - 1)),
                       "cache_bytes": CACHE_BYTES,
                       "flushed_before": ["warm-up", "graph upload replay", "timed replay",
                                          "each spread replay", "kernel-timing pass",
                                          "each cold call", "read probe"]},
        "layers": L, "ms_per_step": ms_per_step, "us_per_step": 1e3 * ms_per_step,
        "us_per_layer": 1e3 * ms_per_step / L,
        "gbps": kv_bytes * L / (ms_per_step * 1e-3) / 1e9,
        "partial_us": partial_us, "merge_us": merge_us,
        "partial_gbps": kv_bytes / (partial_us * 1e-6) / 1e9, "kv_bytes_per_layer": kv_bytes,
        "gpu_out": outs[0][0].cpu(), "gpu_lse": outs[0][1].cpu(),
    }
    del reps
    torch.cuda.empty_cache()
    return res


def chunk_addresses(p: W.Problem, k: torch.Tensor, v: torch.Tensor, pt: torch.Tensor):
    """Device addresses of every KV chunk (one KV head's slice of one page) a
    decode step over `p` reads from caches k, v with page table pt: per
    (sequence, KV head), its visible pages in order, K then V per page."""
    eb = k.element_size()
    B = p.q.shape[0]
    Hkv = k.shape[1]
    lens = p.context_lens.tolist()
    rows = []
    for b in range(B):
        n = lens[b]
        lo = n - p.window if (p.window > 0 and n > p.window) else 0
        if n <= lo:
            continue
        ids = pt[b, lo // W.PAGE_SIZE:(n + W.PAGE_SIZE - 1) // W.PAGE_SIZE].long()
        for h in range(Hkv):
            off = (ids * k.stride(0) + h * k.stride(1)) * eb
            rows.append(torch.stack([k.data_ptr() + off, v.data_ptr() + off], 1).reshape(-1))
    if not rows:
        return torch.zeros(0, dtype=torch.int64, device=k.device)
    return torch.cat(rows).contiguous()


def same_pages_probe(reps, p: W.Problem, launches: int, stream_ptr: int, flush):
    """Read-rate ceiling next to the kernel: pa_decode_read_probe reading
    exactly the KV chunks a step reads (same replicas, same cold-cache
    rotation, graph-replayed like the steps), and a plain contiguous read of
    1 GiB.  Returns None when the chunk size is not one the probe takes."""
    D = p.q.shape[2]
    chunk = W.PAGE_SIZE * D * p.k_cache.element_size()
    if chunk not in (2048, 3072, 4096, 8192) or p.k_cache.stride(2) != D:
        return None   # a head's page slice must be one contiguous chunk
    lists = [chunk_addresses(p, k, v, pt) for k, v, pt in reps.caches]
    n = int(lists[0].numel())
    if n == 0:
        return None
    sink = torch.zeros(binding.PA_DECODE_PROBE_WAVES, dtype=torch.int32, device="cuda")
    R = len(lists)

    def probe(i, sp):
        binding.pa_decode_read_probe(0, lists[i % R].data_ptr(), n, chunk, sink.data_ptr(), sp)

    stream = torch.cuda.current_stream()
    for i in range(2 * R):
        probe(i, stream_ptr)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(launches):
                probe(i, cs)
    stream.wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush()
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / launches
    read_bytes = n * chunk

    # Contiguous 1 GiB, 8 KiB chunks.
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(3)
    nb = (1 << 30) // 8192
    for _ in range(3):
        binding.pa_decode_read_probe(big.data_ptr(), 0, nb, 8192, sink.data_ptr(), stream_ptr)
    a.record(stream)
    reps_c = 10
    for _ in range(reps_c):
        binding.pa_decode_read_probe(big.data_ptr(), 0, nb, 8192, sink.data_ptr(), stream_ptr)
    b.record(stream)
    torch.cuda.synchronize()
    contig = (1 << 30) * reps_c / (1e-3 * a.elapsed_time(b)) / 1e9
    del big
    return {"same_pages_us": round(us, 3), "same_pages_bytes": read_bytes,
            "same_pages_GBps": round(read_bytes / (us * 1e-6) / 1e9, 1),
            "contiguous_GBps": round(contig, 1)}


def parity_against(res, ref_out, ref_lse):
    """Errors of the GPU output against the oracle's, from outputs the
    cpu_baseline leg's oracle run already produced: rel-L2 against the
    oracle rounded to the output dtype, the worst (sequence, head) row (error
    beyond one output ulp per element, as a fraction of the row's norm; see
    tests/parity.py) and the largest lse error."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    p = res["p"]
    e = parity.out_errors(res["gpu_out"], ref_out, p.q.dtype)
    lerr, _ = parity.lse_error(res["gpu_lse"], ref_lse)
    b, h = divmod(e["row_worst"], p.q.shape[1])
    return {"out_rel_l2": e["rel_l2"], "row_excess_max": e["row_excess"],
            "worst_row": {"b": b, "h": h}, "row_rel_l2_max": e["row_rel_l2_max"],
            "out_max_abs_err": e["max_abs"], "lse_max_abs_err": lerr}


def traffic_for(name, plan):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    e = t.get("workloads", {}).get(name)
    if not e:
        return None
    return e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama1b_ctx3060_f16",
                    choices=W.CONFIG_ORDER + W.EXTRA_ORDER)
    ap.add_argument("--also", default="ctx100k_gqa6_f16,llama8b_b16_ragged_f16,d256_window4096_bf16,"
                    "llama8b_ctx32k_rope_f16,llama8b_b64_ctx1000_f16",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--also-steps", type=int, default=300)
    ap.add_argument("--replicas", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--layers", type=int, default=1,
                    help="decode-attention calls per step, each on its own KV cache (a "
                         "layer-stacked decode step); the extra workloads keep 1")
    ap.add_argument("--page-table", choices=["dense", "csr"], default="dense",
                    help="page-table form passed to the library (csr: pa_decode_run_csr)")
    ap.add_argument("--phases", choices=["all", "cold"], default="all",
                    help="cold: leave out the warm-cache figure, the spread replays and the "
                         "read probe (profiling runs, so that a kernel's trace holds cold "
                         "launches only)")
    ap.add_argument("--cold-calls", type=int, default=100,
                    help="single calls timed one at a time, each after a cache flush "
                         "(p10 / median / p90 reported)")
    ap.add_argument("--library", default=None,
                    help="load this build of the library instead of the package's (comparison "
                         "builds, e.g. python -m paged_kv_decode_amd.build --variant qk_valu)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--probe", choices=["copy", "read-sweep", "schedule-sweep"], default=None,
                    help="copy: time a plain device copy of --probe-bytes (the reference kernel "
                         "for the HBM traffic counters); read-sweep: the read probe's time "
                         "against size, contiguous and gathered, cold (the fixed cost and the "
                         "streaming rate of a kernel that only reads)")
    ap.add_argument("--probe-bytes", type=int, default=256 << 20)
    ap.add_argument("--profile-commands", metavar="DIR", default=None,
                    help="print the rocprofv3 commands whose output --summarize-profiles reads")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="write profiles/*.md and profiles/traffic.json from that output")
    ap.add_argument("--profile-set", choices=["main", "ab"], default="main",
                    help="which runs --profile-commands / --summarize-profiles cover (ab: q.k "
                         "on the matrix cores against the vector ALUs)")
    args = ap.parse_args()

    if args.profile_commands:
        print("\n".join("%s\t%s" % nc for nc in profile_commands(args.profile_commands,
                                                                  args.profile_set)))
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.profile_set)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this decode-attention path runs on a single "
              "MI355X and has no multi-GPU mode (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.probe == "copy":
        copy_probe(args.probe_bytes, args.steps, args.warmup)
        return
    if args.probe == "read-sweep":
        binding.load_library()
        read_sweep()
        return
    if args.probe == "schedule-sweep":
        binding.load_library()
        schedule_sweep()
        return
    if args.library:
        binding.use_library(os.path.join(ROOT, args.library))
    else:
        binding.load_library()

    engines = {}
    if args.layers < 1:
        ap.error("--layers must be >= 1")
    flusher = Flusher()
    main_res = bench_workload(args.workload, args.steps, args.warmup, args.replicas,
                              args.partition_size, args.mode, engines, args.page_table,
                              args.layers, args.phases, args.cold_calls, flusher)
    log("%s: %.2f us/step, %.0f GB/s; partial %.2f us (%.0f GB/s), merge %.2f us" % (
        args.workload, main_res["us_per_step"], main_res["gbps"], main_res["partial_us"],
        main_res["partial_gbps"], main_res["merge_us"]))
    also = {}
    for name in [s for s in args.also.split(",") if s and s != args.workload]:
        r = bench_workload(name, args.also_steps, 20, None, None, args.mode, engines,
                           args.page_table, 1, args.phases, args.cold_calls, flusher)
        also[name] = {
            "us_per_step": round(r["us_per_step"], 3), "GBps": round(r["gbps"], 1),
            "frac_of_peak": round(r["gbps"] / PEAK_GBPS, 4),
            "partial_us": round(r["partial_us"], 3), "merge_us": round(r["merge_us"], 3),
            "partial_GBps": round(r["partial_gbps"], 1),
            "partial_frac": round(r["partial_gbps"] / PEAK_GBPS, 4),
            "kv_bytes": r["kv_bytes"], "replicas": r["replicas"],
            "plan": {k: r["plan"][k] for k in ("partition_size", "num_partitions",
                                               "waves_per_group", "split")},
            "read_ceiling": r["read_ceiling"],
            "cold_per_call_us": r["cold_per_call_us"],
        }
        log("%s: %.2f us/step, %.0f GB/s; partial %.2f us (%.0f GB/s), merge %.2f us" % (
            name, r["us_per_step"], r["gbps"], r["partial_us"], r["partial_gbps"],
            r["merge_us"]))

    # cpu_baseline leg: the oracle timed on this host's cores over the main
    # workload; the outputs of that timed run also give the main workload's
    # parity figure.  Nothing else here runs the oracle (the tests hold the
    # parity checks of every workload).
    cpu = None
    par = None
    if args.cpu_budget > 0:
        p = main_res["p"]
        ref_out, ref_lse, reps, el, threads = run_oracle_baseline(p, args.cpu_budget)
        cpu = {"value": round(main_res["kv_bytes_per_layer"] * reps / el / 1e9, 4), "unit": "GB/s",
               "cores": threads, "kind": "oracle",
               "sample": "%d decode-attention calls (one layer each) of the %s workload (float64 C oracle, OpenMP), %.1f s"
                         % (reps, args.workload, el),
               "us_per_step": round(1e6 * el / reps, 1)}
        par = parity_against(main_res, ref_out, ref_lse)
    dtype_name = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
    w = W.CONFIGS[args.workload]
    traffic = traffic_for(args.workload, main_res["plan"])
    achieved = main_res["partial_gbps"]
    line = {
        "metric": METRIC,
        "value": round(main_res["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 6),
        "us_per_step": round(main_res["us_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name[w.dtype] + " in, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "context_lens": p_lens(main_res["p"]), "page_size": w.page_size,
                   "sliding_window": w.window, "kv_bytes_per_step": main_res["kv_bytes"],
                   "replicas": main_res["replicas"], "mode": args.mode,
                   "page_table": args.page_table, "layers": args.layers,
                   "us_per_layer": round(main_res["us_per_layer"], 3),
                   "us_per_step_replays": main_res["spread"],
                   "warm_us_per_step": main_res["warm_us_per_step"],
                   "cold_per_call_us": main_res["cold_per_call_us"],
                   "cold_guard": main_res["cold_guard"],
                   "plan": main_res["plan"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "partial_kernel", "kernel_us": round(main_res["partial_us"], 3),
                     "merge_us": round(main_res["merge_us"], 3),
                     "read_ceiling": main_res["read_ceiling"]},
        "cpu_baseline": cpu,
        "parity": par,
        "also": also,
    }
    print(json.dumps(line), flush=True)


def read_sweep(launches=50):
    """Time pa_decode_read_probe reading N bytes per launch, N from 4 MiB to
    1 GiB, as 8 KiB chunks that are contiguous or gathered at random from a
    pool, each launch on bytes no launch touched for >= 4 x CACHE_BYTES
    (rotation over a 6 GiB pool; a flush before each timed graph), graph-
    replayed; prints one JSON line per (layout, size) and a least-squares fit
    t = fixed + bytes / rate over the sizes from 64 MiB."""
    pool_bytes = 6 << 30
    pool = torch.ones(pool_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(binding.PA_DECODE_PROBE_WAVES, dtype=torch.int32, device="cuda")
    flush = Flusher()
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cpu")
    gen.manual_seed(77)
    chunk = 8192
    nchunks_pool = pool_bytes // chunk
    fits = {}
    for layout in ("contiguous", "gathered"):
        pts = []
        for mib in (4, 8, 16, 32, 64, 128, 256, 512, 1024):
            n = (mib << 20) // chunk
            # launches over disjoint ranges of the pool, in rotation, enough
            # of them that a range is read again only after 4 x CACHE_BYTES
            L = max(launches, -(-4 * CACHE_BYTES // (n * chunk)) + 1)
            per = max(1, min(L, nchunks_pool // n))
            if layout == "gathered":
                perm = torch.randperm(nchunks_pool, generator=gen)[: per * n]
                addrs = (pool.data_ptr() + perm.to(torch.int64) * chunk).to("cuda")
            else:
                addrs = (pool.data_ptr() + torch.arange(per * n, dtype=torch.int64) * chunk).to("cuda")
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    cs = torch.cuda.current_stream().cuda_stream
                    for i in range(L):
                        binding.pa_decode_read_probe(0, addrs[(i % per) * n:].data_ptr(), n, chunk,
                                                     sink.data_ptr(), cs)
            stream.wait_stream(cap)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            flush()
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / L
            cold = per * n * chunk - n * chunk >= 4 * CACHE_BYTES
            pts.append((n * chunk, us))
            print(json.dumps({"probe": "read-sweep", "layout": layout, "bytes": n * chunk,
                              "us_per_launch": round(us, 3),
                              "GBps": round(n * chunk / (us * 1e-6) / 1e9, 1),
                              "frac_of_8TBps": round(n * chunk / (us * 1e-6) / 1e9 / PEAK_GBPS, 4),
                              "rotation_launches": per, "cold": bool(cold)}), flush=True)
            del g
        big = [(x, y) for x, y in pts if x >= (64 << 20)]
        xs = np.array([x for x, _ in big], dtype=np.float64)
        ys = np.array([y for _, y in big], dtype=np.float64)
        A = np.stack([np.ones_like(xs), xs], 1)
        (c0, c1), *_ = np.linalg.lstsq(A, ys, rcond=None)
        fits[layout] = {"fixed_us": round(float(c0), 3), "rate_GBps": round(1e-3 / float(c1), 1)}
    print(json.dumps({"probe": "read-sweep-fit", "fit_from_bytes": 64 << 20, **fits}), flush=True)


def schedule_sweep(steps=200):
    """Fixed partitions (partition_size 0) against the length-balanced
    schedule (PA_DECODE_PARTITION_BALANCED) on Llama-3.1-8B-shaped batches
    (Hq 32 / Hkv 8, head_dim 128, f16; the first sequence 4096 tokens) of 4,
    8, 16 and 32 sequences with four length mixes (uniform in [1, 4096],
    uniform in [2048, 4096], mostly short (u^3 scaled), all 300), plus the
    batch-16 ragged workload's own lengths, without and with rotary: µs per
    graph-replayed step with cold caches (replica rotation, a flush before
    the timed replay), median of three replays; one JSON line per case with
    the mean / longest page ratio the CSR host rule looks at."""
    flush = Flusher()
    stream = torch.cuda.current_stream()
    c3 = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"]).context_lens.tolist()
    for rope in (None, (500000.0, 1.0)):
        eng = binding.PagedDecode(32, 8, 128, torch.float16, max_batch=64,
                                  max_context_len=1 << 20, rope=rope)
        gen = torch.Generator().manual_seed(11)
        cases = []
        for B in (4, 8, 16, 32):
            for kind in ("uniform", "upper_half", "mostly_short", "one_long"):
                if kind == "uniform":
                    lens = torch.randint(1, 4097, (B,), generator=gen).tolist()
                elif kind == "upper_half":
                    lens = torch.randint(2048, 4097, (B,), generator=gen).tolist()
                elif kind == "mostly_short":
                    lens = [int(x) for x in (torch.rand(B, generator=gen) ** 3 * 4095 + 1).tolist()]
                else:
                    lens = [300] * B
                lens[0] = 4096
                cases.append((B, kind, lens))
        cases.append((16, "batch16_ragged_workload", c3))
        for B, kind, lens in cases:
            w = W.custom(name="schedule_sweep", batch=B, num_q_heads=32, num_kv_heads=8,
                         head_dim=128, dtype=torch.float16, context_lens=lens,
                         seed=B * 7 + len(kind), rope=rope)
            p = W.generate(w)
            res = {}
            for label, S in (("fixed_us", 0), ("balanced_us", binding.PA_DECODE_PARTITION_BALANCED)):
                R = min(24, replica_count(p.kv_bytes(),
                                          2 * p.k_cache.numel() * p.k_cache.element_size()))
                reps = Replicas(p, R, eng, S)
                g = torch.cuda.CUDAGraph()
                cap = torch.cuda.Stream()
                cap.wait_stream(stream)
                with torch.cuda.stream(cap):
                    with torch.cuda.graph(g, stream=cap):
                        cs = torch.cuda.current_stream().cuda_stream
                        for i in range(steps):
                            reps.run(reps.args[i % R], cs)
                stream.wait_stream(cap)
                g.replay()
                torch.cuda.synchronize()
                ts = []
                for _ in range(3):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    flush()
                    a.record(stream)
                    g.replay()
                    b.record(stream)
                    torch.cuda.synchronize()
                    ts.append(1e3 * a.elapsed_time(b) / steps)
                res[label] = round(sorted(ts)[1], 3)
                del g, reps
                torch.cuda.empty_cache()
            nnz = sum(-(-n // 16) for n in lens)
            print(json.dumps({"probe": "schedule-sweep", "rotary": rope is not None, "batch": B,
                              "lengths": kind, "mean_over_longest_pages": round(nnz / (B * 256), 3),
                              "tokens": sum(lens), **res,
                              "balanced_gain": round(res["fixed_us"] / res["balanced_us"] - 1, 3)}),
                  flush=True)
        eng.close()


def copy_probe(nbytes, steps, warmup):
    """A plain copy of nbytes (read nbytes, write nbytes) repeated `steps` times."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"probe": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": steps + warmup, "us_per_copy": round(ms * 1e3, 2),
                      "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


# ---------------------------------------------------------------------------
# Profiling evidence: the rocprofv3 runs behind profiles/ and their summary.
# ---------------------------------------------------------------------------
PROFILED = ["llama1b_ctx3060_f16", "llama8b_b16_ragged_f16", "d256_window4096_bf16",
            "ctx100k_gqa6_f16", "llama8b_ctx32k_rope_f16", "ctx100k_gqa6_rope_f16",
            "llama8b_b64_ctx1000_f16"]
COPY_BYTES = 256 << 20
# Counter passes of every profiled workload (one rocprofv3 --pmc run each; at
# most 8 SQ and 4 TCC counters per run).
PMC_SETS = {
    "FETCH_SIZE": ["FETCH_SIZE"],
    "WRITE_SIZE": ["WRITE_SIZE"],
    "sqA": ["SQ_WAVES", "SQ_INSTS", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
            "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SMEM", "TCC_HIT", "TCC_MISS"],
    "sqB": ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY",
            "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_VALU",
            "SQ_LDS_IDX_ACTIVE"],
}
# q.k on the matrix cores (the library) against the vector ALUs (the
# comparison build python -m paged_kv_decode_amd.build --variant qk_valu).
AB_WORKLOADS = ["llama1b_ctx3060_f16", "ctx100k_gqa6_f16", "llama8b_b16_ragged_f16",
                "d256_window4096_bf16"]
AB_LIBS = {"mfma": None, "valu": "paged_kv_decode_amd/libpa_decode_qk_valu.so"}


def _run(w, steps, lib=None, eager=False, warmup=20):
    b = "/root/repo/bench.py"
    return ("python3 %s --workload %s --also '' --cpu-budget 0 --steps %d --warmup %d "
            "--phases cold --cold-calls 0%s%s" % (b, w, steps, warmup,
                                                  " --mode eager" if eager else "",
                                                  " --library %s" % lib if lib else ""))


def profile_commands(outdir, which="main"):
    """(name, command) of every run behind profiles/.  which="main": per
    workload a plain benchmark run (its stdout goes to <outdir>/<name>.log),
    a kernel trace and one counter run per PMC_SETS entry, then the copy
    calibration of FETCH_SIZE / WRITE_SIZE.  which="ab": per AB_WORKLOADS
    entry and library (AB_LIBS) a plain run and the two SQ counter passes.
    The rocprofv3 commands run from /tmp with TMPDIR=/tmp."""
    b = "/root/repo/bench.py"
    cmds = []
    if which == "ab":
        for w in AB_WORKLOADS:
            for lib_name, lib in AB_LIBS.items():
                steps = 2000 if w == "llama1b_ctx3060_f16" else 300
                cmds.append(("ab_bench_%s_%s" % (lib_name, w), _run(w, steps, lib)))
                for c in ("sqA", "sqB"):
                    cmds.append(("ab_pmc_%s_%s_%s" % (lib_name, w, c),
                                 "rocprofv3 --pmc %s --output-format csv -d %s/ab_pmc_%s_%s_%s -o %s -- %s"
                                 % (" ".join(PMC_SETS[c]), outdir, lib_name, w, c, w,
                                    _run(w, 20, lib, eager=True, warmup=2))))
        return cmds
    for w in PROFILED:
        steps = 2000 if w == "llama1b_ctx3060_f16" else 300
        run = _run(w, steps)
        cmds.append(("bench_%s" % w, run))
        cmds.append(("trace_%s" % w, "rocprofv3 --kernel-trace --stats --output-format csv -d %s/trace_%s "
                                     "-o %s -- %s" % (outdir, w, w, run)))
    for c, names in PMC_SETS.items():
        for w in PROFILED:
            cmds.append(("pmc_%s_%s" % (w, c),
                         "rocprofv3 --pmc %s --output-format csv -d %s/pmc_%s_%s -o %s -- %s"
                         % (" ".join(names), outdir, w, c, w, _run(w, 20, eager=True, warmup=2))))
        if c in ("FETCH_SIZE", "WRITE_SIZE"):
            cmds.append(("pmc_copy_%s" % c,
                         "rocprofv3 --pmc %s --output-format csv -d %s/pmc_copy_%s -o copy -- python3 %s "
                         "--probe copy --probe-bytes %d --steps 10 --warmup 2" % (c, outdir, c, b, COPY_BYTES)))
    return cmds


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name):
    """Kernel family of a trace or counter row (the three merge kernels count
    as the merge)."""
    if "partial_kernel" in name:
        return "partial_kernel"
    if "merge_kernel" in name or "merge_wave_kernel" in name or "merge_count_kernel" in name:
        return "merge_kernel"
    if "copyBuffer" in name:
        return "copyBuffer"
    return None


def _pmc_medians(path, names):
    """{(kernel family, counter): median per-dispatch value} of one counter
    run (rocprofv3 sums a counter over its instances in each dispatch)."""
    import statistics
    rows = _csv_rows(path)
    out = {}
    for k in ("partial_kernel", "merge_kernel"):
        for c in names:
            v = [float(r["Counter_Value"]) for r in rows
                 if _short(r["Kernel_Name"]) == k and r["Counter_Name"] == c]
            if v:
                out[(k, c)] = statistics.median(v)
    return out


def sq_summary(m, kernel="partial_kernel"):
    """Per-wave instruction mix and cycle figures of one kernel from the sqA /
    sqB medians (None when the counters are missing).  SQ_WAVE_CYCLES,
    SQ_WAIT_* and SQ_ACTIVE_INST_VALU count quad-cycles."""
    g = lambda c: m.get((kernel, c))  # noqa: E731
    waves = g("SQ_WAVES")
    if not waves:
        return None
    r = {"waves": int(waves)}
    for c, key in (("SQ_INSTS", "insts"), ("SQ_INSTS_VALU", "valu"), ("SQ_INSTS_MFMA", "mfma"),
                   ("SQ_INSTS_LDS", "lds"), ("SQ_INSTS_SALU", "salu"),
                   ("SQ_INSTS_VMEM_RD", "vmem_rd"), ("SQ_INSTS_SMEM", "smem")):
        if g(c) is not None:
            r[key + "_per_wave"] = round(g(c) / waves, 1)
    if g("TCC_HIT") is not None and g("TCC_MISS") is not None:
        tot = g("TCC_HIT") + g("TCC_MISS")
        r["l2_hit_rate"] = round(g("TCC_HIT") / tot, 4) if tot else None
    wc = g("SQ_WAVE_CYCLES")
    if wc:
        r["wave_cycles_per_wave"] = round(4 * wc / waves, 0)
        for c, key in (("SQ_WAIT_INST_ANY", "wait_inst_frac"), ("SQ_WAIT_ANY", "wait_any_frac"),
                       ("SQ_ACTIVE_INST_VALU", "valu_active_frac")):
            if g(c) is not None:
                r[key] = round(g(c) / wc, 4)
    if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
        r["mfma_busy_cycles"] = int(g("SQ_VALU_MFMA_BUSY_CYCLES"))
    if g("SQ_BUSY_CYCLES") is not None:
        r["busy_cycles"] = int(g("SQ_BUSY_CYCLES"))
    if g("SQ_LDS_IDX_ACTIVE"):
        r["lds_bank_conflict_frac"] = round((g("SQ_LDS_BANK_CONFLICT") or 0) / g("SQ_LDS_IDX_ACTIVE"), 4)
    return r


SQ_ROWS = [("waves", "waves"), ("insts_per_wave", "instructions / wave"),
           ("valu_per_wave", "VALU / wave"), ("mfma_per_wave", "MFMA / wave"),
           ("lds_per_wave", "LDS / wave"), ("salu_per_wave", "SALU / wave"),
           ("vmem_rd_per_wave", "vector memory reads / wave"), ("smem_per_wave", "scalar memory / wave"),
           ("l2_hit_rate", "L2 hit rate (TCC_HIT / (HIT + MISS))"),
           ("wave_cycles_per_wave", "cycles / wave (SQ_WAVE_CYCLES x 4 / waves)"),
           ("wait_any_frac", "waiting on anything / wave cycles"),
           ("wait_inst_frac", "waiting for issue / wave cycles"),
           ("valu_active_frac", "VALU active / wave cycles"),
           ("mfma_busy_cycles", "MFMA busy cycles (SQ_VALU_MFMA_BUSY_CYCLES)"),
           ("busy_cycles", "SQ busy cycles"),
           ("lds_bank_conflict_frac", "LDS bank-conflict cycles / LDS active cycles")]


def trace_phases(path, steps, warm=20):
    """Mean partial-kernel duration per phase of a --phases cold benchmark run
    from its rocprofv3 kernel trace: the two replica checks and the warm-up,
    the graph upload replay, the graph timed replay and the eager timing pass
    (in launch order); None when the trace does not have that shape."""
    import statistics
    if not os.path.exists(path):
        return None
    rows = [r for r in _csv_rows(path) if _short(r["Kernel_Name"]) == "partial_kernel"]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    pre = 2 + warm
    if len(d) != pre + 3 * steps:
        return None
    segs = [("checks and warm-up", d[:pre]), ("graph upload replay", d[pre:pre + steps]),
            ("graph timed replay", d[pre + steps:pre + 2 * steps]),
            ("eager timing pass", d[pre + 2 * steps:])]
    return {k: (len(v), statistics.mean(v)) for k, v in segs}


def _bench_line(path):
    line = None
    if os.path.exists(path):
        for ln in open(path):
            if ln.startswith("{"):
                line = json.loads(ln)
    return line


def summarize_profiles(indir, which="main"):
    """Writes profiles/<kernel>_<workload>.md and profiles/traffic.json from the
    output of profile_commands(indir) (which="ab": profiles/qk_mfma_vs_valu.md)."""
    import statistics
    prof = os.path.join(ROOT, "profiles")
    named = dict(profile_commands(indir, which))
    if which == "ab":
        return summarize_ab(indir, named)
    counters = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = _csv_rows(os.path.join(indir, "pmc_copy_%s" % c, "copy_counter_collection.csv"))
        vals = [float(r["Counter_Value"]) for r in rows if _short(r["Kernel_Name"]) == "copyBuffer"
                and r["Counter_Name"] == c]
        counters[c] = statistics.median(vals)
    fetch_scale = COPY_BYTES / 1024.0 / counters["FETCH_SIZE"]
    write_scale = COPY_BYTES / 1024.0 / counters["WRITE_SIZE"]
    traffic = {"kernel_hash": kernel_hash(), "kernel_sources": KERNEL_SOURCES,
               "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
               "calibration": "plain %d KiB device copy (__amd_rocclr_copyBuffer): FETCH_SIZE "
                              "%.1f KiB, WRITE_SIZE %.1f KiB per dispatch for %d KiB read and written"
                              % (COPY_BYTES >> 10, counters["FETCH_SIZE"], counters["WRITE_SIZE"],
                                 COPY_BYTES >> 10),
               "commands": [c for n, c in named.items() if n.startswith("pmc_")],
               "workloads": {}}
    for w in PROFILED:
        p = W.generate(W.CONFIGS[w])
        kv = p.kv_bytes()
        stats = {_short(r["Name"]): r for r in
                 _csv_rows(os.path.join(indir, "trace_%s" % w, "%s_kernel_stats.csv" % w))}
        line = _bench_line(os.path.join(indir, "bench_%s.log" % w))
        pmc = {}
        for c, names in PMC_SETS.items():
            path = os.path.join(indir, "pmc_%s_%s" % (w, c), "%s_counter_collection.csv" % w)
            if os.path.exists(path):
                pmc.update(_pmc_medians(path, names))
        fb = int(round(pmc[("partial_kernel", "FETCH_SIZE")] * 1024 * fetch_scale))
        wb = int(round(pmc[("partial_kernel", "WRITE_SIZE")] * 1024 * write_scale))
        sq = {k: sq_summary(pmc, k) for k in ("partial_kernel", "merge_kernel")}
        e = {"kernel": "partial_kernel", "fetch_bytes": fb, "write_bytes": wb,
             "bytes_per_launch": fb + wb, "algorithmic_kv_bytes": kv,
             "fetch_over_algorithmic": round(fb / kv, 4), "sq": sq}
        if ("merge_kernel", "FETCH_SIZE") in pmc:
            e["merge_kernel_fetch_bytes"] = int(round(pmc[("merge_kernel", "FETCH_SIZE")] * 1024 * fetch_scale))
            e["merge_kernel_write_bytes"] = int(round(pmc[("merge_kernel", "WRITE_SIZE")] * 1024 * write_scale))
        traffic["workloads"][w] = e

        part = stats["partial_kernel"]
        avg_us = float(part["AverageNs"]) / 1e3
        out = ["# %s -- partial and merge kernels on MI355X (gfx950)" % w, "",
               "Kernel trace (rocprofv3 --kernel-trace --stats), run from /tmp with TMPDIR=/tmp "
               "(cold launches only: --phases cold):",
               "  " + named["trace_%s" % w], "",
               "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k in ("partial_kernel", "merge_kernel"):
            if k in stats:
                r = stats[k]
                out.append("| %s | %s | %.3f | %.3f | %.3f |" % (
                    r["Name"].replace("void pa::(anonymous namespace)::", ""), r["Calls"],
                    float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
        out += ["", "Algorithmic KV bytes per launch: %d; at the trace's average partial-kernel "
                    "duration that is %.1f GB/s (%.1f%% of 8 TB/s)." % (kv, kv / avg_us / 1e3,
                                                                        kv / avg_us / 1e3 / PEAK_GBPS * 100)]
        phases = trace_phases(os.path.join(indir, "trace_%s" % w, "%s_kernel_trace.csv" % w),
                              2000 if w == "llama1b_ctx3060_f16" else 300)
        if phases:
            out += ["", "Partial-kernel dispatches of the traced run by phase (trace timestamps, "
                        "mean us): %s." % ", ".join("%s %d x %.3f" % (k, n, v) for k, (n, v) in phases.items())]
            if line:
                ev = line["roofline"]["kernel_us"]
                out += ["The benchmark's HIP events bracket the eager launches: %.3f us against the "
                        "trace's %.3f us for that phase (ratio %.3f); graph-replayed launches (the "
                        "timed region) run at %.3f us, so the event figure is %.1f%% conservative."
                        % (ev, phases["eager timing pass"][1], ev / phases["eager timing pass"][1],
                           phases["graph timed replay"][1],
                           100 * (ev / phases["graph timed replay"][1] - 1))]
        if line:
            ro = line["roofline"]
            out += ["", "The same benchmark without the profiler (HIP events around each launch):",
                    "  " + named["bench_%s" % w],
                    "gives partial %.3f us (%.1f GB/s, %.1f%% of peak), merge %.3f us, %.2f us per "
                    "graph-replayed step, %.1f GB/s per step." % (
                        ro["kernel_us"], ro["achieved"], 100 * ro["frac"], ro["merge_us"],
                        line["us_per_step"], line["value"])]
        out += ["", "HBM traffic per dispatch (rocprofv3 --pmc, one counter per run, median over "
                    "dispatches), C = FETCH_SIZE, then WRITE_SIZE:",
                "  " + named["pmc_%s_FETCH_SIZE" % w].replace("FETCH_SIZE", "{C}"),
                "calibration:",
                "  " + named["pmc_copy_FETCH_SIZE"].replace("FETCH_SIZE", "{C}"),
                "  copy of %d KiB: FETCH_SIZE reads %.1f KiB (scale %.4f), WRITE_SIZE reads %.1f KiB "
                "(scale %.4f)" % (COPY_BYTES >> 10, counters["FETCH_SIZE"], fetch_scale,
                                   counters["WRITE_SIZE"], write_scale), "",
                "| kernel | FETCH_SIZE KiB (raw) | fetched bytes (scaled) | WRITE_SIZE KiB | written bytes |",
                "|---|---|---|---|---|"]
        for k in ("partial_kernel", "merge_kernel"):
            if (k, "FETCH_SIZE") in pmc:
                out.append("| %s | %.1f | %d | %.1f | %d |" % (
                    k, pmc[(k, "FETCH_SIZE")], round(pmc[(k, "FETCH_SIZE")] * 1024 * fetch_scale),
                    pmc[(k, "WRITE_SIZE")], round(pmc[(k, "WRITE_SIZE")] * 1024 * write_scale)))
        out += ["", "partial kernel fetched / algorithmic KV bytes = %.4f" % (fb / kv)]
        if sq["partial_kernel"]:
            out += ["", "SQ / TCC counters (two --pmc runs, median per dispatch):",
                    "  " + named["pmc_%s_sqA" % w], "  " + named["pmc_%s_sqB" % w], "",
                    "| figure | partial kernel | merge kernel |", "|---|---|---|"]
            for key, label in SQ_ROWS:
                vals = [sq[k].get(key) if sq[k] else None for k in ("partial_kernel", "merge_kernel")]
                if vals[0] is not None:
                    out.append("| %s | %s | %s |" % (label, vals[0], "-" if vals[1] is None else vals[1]))
        out += ["", "kernel sources hash (bench.kernel_hash): %s" % kernel_hash(), ""]
        with open(os.path.join(prof, "partial_kernel_%s.md" % w), "w") as f:
            f.write("\n".join(out))
    with open(os.path.join(prof, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    print("wrote profiles/ for %s (kernel hash %s)" % (", ".join(PROFILED), kernel_hash()))


def summarize_ab(indir, named):
    """profiles/qk_mfma_vs_valu.md: per workload, step and partial-kernel time
    and the SQ figures of q.k on the matrix cores against the vector ALUs."""
    out = ["# q.k on the matrix cores against the vector ALUs (MI355X, gfx950)", "",
           "mfma: the library (the score MFMA, the K page tile as A and the GQA group's query "
           "rows as B).  valu: the comparison build `python -m paged_kv_decode_amd.build "
           "--variant qk_valu` (lane (token, chunk group) forms packed f16/bf16 dot products "
           "of its key row's chunks with every query row, the four chunk groups summed by lane "
           "swaps, the scores passed through a per-wave LDS buffer into the P.V operand "
           "layout).  Everything else is the same kernel; P.V is on the matrix cores in both.",
           "", "Commands (run from /tmp with TMPDIR=/tmp):"]
    out += ["  " + c for n, c in named.items()]
    rows = []
    res = {}
    for w in AB_WORKLOADS:
        for lib_name in AB_LIBS:
            line = _bench_line(os.path.join(indir, "ab_bench_%s_%s.log" % (lib_name, w)))
            pmc = {}
            for c in ("sqA", "sqB"):
                path = os.path.join(indir, "ab_pmc_%s_%s_%s" % (lib_name, w, c),
                                    "%s_counter_collection.csv" % w)
                if os.path.exists(path):
                    pmc.update(_pmc_medians(path, PMC_SETS[c]))
            res[(w, lib_name)] = (line, sq_summary(pmc))
    out += ["", "| workload | q.k on | us / step | partial us (events) | partial % of 8 TB/s | "
                "instructions / wave | VALU / wave | MFMA / wave | LDS / wave | cycles / wave | "
                "VALU active | waiting |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for w in AB_WORKLOADS:
        for lib_name in AB_LIBS:
            line, sq = res[(w, lib_name)]
            if not line:
                continue
            sq = sq or {}
            out.append("| %s | %s | %.2f | %.2f | %.1f | %s | %s | %s | %s | %s | %s | %s |" % (
                w, lib_name, line["us_per_step"], line["roofline"]["kernel_us"],
                100 * line["roofline"]["frac"], sq.get("insts_per_wave"), sq.get("valu_per_wave"),
                sq.get("mfma_per_wave"), sq.get("lds_per_wave"), sq.get("wave_cycles_per_wave"),
                sq.get("valu_active_frac"), sq.get("wait_any_frac")))
    out += ["", "kernel sources hash (bench.kernel_hash): %s" % kernel_hash(), ""]
    with open(os.path.join(ROOT, "profiles", "qk_mfma_vs_valu.md"), "w") as f:
        f.write("\n".join(out))
    print("wrote profiles/qk_mfma_vs_valu.md")


def p_lens(p):
    lens = p.context_lens.tolist()
    return lens if len(lens) <= 4 else {"n": len(lens), "sum": sum(lens), "max": max(lens)}


if __name__ == "__main__":
    main()
