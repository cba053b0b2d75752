"""Throughput of the sparse-MLA decode hot path on one MI355X.

One step = the whole path for one batch: stable top-k per row over the indexer scores (with length
clamping) -> canonical indices -> paged gather + MQA attention + split combine.  Workload: B=64
decode rows, H=64 heads, top-k 2048, d_qk 576 (512 latent + 64 rope), d_v 512, bf16 KV in pages of
64, context lengths uniform in [8192, 65536], random page tables.  Four independent (Q, scores) sets
rotate over one 2.7 GB KV pool so a step's gathered set (151 MB) is not already cache-resident.

Timing: one HIP graph holds K steps (--steps); after the graph of W warm-up steps (--warmup) it is
replayed, each replay bracketed by events on the stream the kernels run on, until at least
--min-timed-ms of replays are timed (and at least 5 replays); ms_per_step is the median replay time
divided by K.

Prints one JSON line.  `value` is rows/s of the whole step with every input resident in HBM;
`roofline` reports the attention call's gathered-KV bandwidth against the 8 TB/s HBM peak;
`cpu_baseline` times the CPU oracle on a bounded sample of the same rows, on every host core the
process may use (worker processes started before any GPU call) and on one core.

Also: `--summarize-trace DIR` and `--summarize-counters DIR...` turn rocprofv3 output (kernel-trace
statistics, counter collections) into the tables kept under profiles/; `--traffic-record` computes
the HBM bytes per call of the attention call from a FETCH_SIZE and a WRITE_SIZE pass.
"""

import argparse
import glob
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode rows/s + gathered-KV HBM GB/s (H=64, topk=2048, 1 GPU)"
METRIC_FP8 = "sparse-MLA decode rows/s + gathered-KV HBM GB/s (FP8 KV, B=128, H=64, topk=2048, 1 GPU)"
HBM_PEAK_GBPS = 8000.0
N_SETS = 4
WORKLOADS = ["decode_bf16", "decode_fp8", "topk_c1", "kv_write_fp8", "decode_window", "prefill_c4", "indexer"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="steps per timed graph replay (K)")
    ap.add_argument("--warmup", type=int, default=20, help="untimed warm-up steps before timing (W)")
    ap.add_argument("--min-timed-ms", type=float, default=200.0,
                    help="graph replays are timed until at least this much GPU time is covered")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="rows of the all-core CPU-oracle sample (0 = no CPU baseline)")
    ap.add_argument("--cpu-rows-1core", type=int, default=256, help="rows of the one-core CPU-oracle sample")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--workload", default="decode_bf16", choices=WORKLOADS,
                    help="decode_bf16: B=64, contexts U[8192, 65536], bf16 KV (the headline); "
                         "decode_fp8: B=128, contexts U[32768, 131072], FP8 KV; "
                         "topk_c1: top-k alone, 64 x 65536 fp32 rows of 256 distinct levels, k=2048, 32 rotating "
                         "copies (512 MiB, beyond the last-level cache); "
                         "kv_write_fp8: FP8 cache write of 65536 new tokens (and of 128, a decode step); "
                         "decode_window: the decode_bf16 rows plus 128 sliding-window + 5 draft positions "
                         "per row from a separate window cache in one softmax, window width 192 (and 256); "
                         "prefill_c4: one request, T=4096 query tokens at positions 126976..131071 of a "
                         "131072-token context, causal top-k 2048 + prefill attention; "
                         "indexer: indexer scores (paged MQA logits) of B=64 decode rows, 64 index heads of "
                         "width 128, contexts U[8192, 65536], score rows of 65536")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (calibrates rocprofv3 FETCH/WRITE_SIZE)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="print the library kernels of a rocprofv3 "
                    "--kernel-trace --stats output directory as a table, then exit")
    ap.add_argument("--summarize-counters", metavar="DIR", nargs="+", help="print per-kernel means of every "
                    "counter in rocprofv3 --pmc output directories, then exit")
    ap.add_argument("--traffic-record", metavar=("FETCH_DIR", "WRITE_DIR"), nargs=2,
                    help="print the HBM bytes per call of the attention call (copy-calibrated FETCH_SIZE and "
                         "WRITE_SIZE passes of this bench with --copy-probe) as a traffic-record line, then exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------------------------
# rocprofv3 output summaries (run on the GPU machine after the profiled command)
# ----------------------------------------------------------------------------------------------

def _short_kernel(name: str) -> str:
    n = name.replace("void ", "").replace("(anonymous namespace)::", "")
    if "smla::" in n:
        n = n[n.index("smla::"):]
        n = n.split("(")[0]
        return n
    if "copyBuffer" in n:
        return "__amd_rocclr_copyBuffer"
    return ""


def _counter_means(dirs):
    """{(kernel, counter): [values per dispatch]} over every counter_collection.csv under dirs."""
    import csv
    acc = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    k = _short_kernel(r["Kernel_Name"])
                    if k:
                        acc.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return acc


def summarize_counters(dirs):
    acc = _counter_means(dirs)
    print("| kernel | counter | dispatches | mean | min | max |")
    print("|---|---|---:|---:|---:|---:|")
    for (k, c), v in sorted(acc.items()):
        print(f"| `{k}` | {c} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")


def summarize_trace(d):
    import csv
    print("| kernel | calls | avg us | min us | max us |")
    print("|---|---:|---:|---:|---:|")
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = _short_kernel(r["Name"])
                if k.startswith("smla::"):
                    print(f"| `{k}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                          f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")


def traffic_record(fetch_dir, write_dir, workload):
    """Copy-calibrated HBM bytes per attention call (topk_c1: per top-k call): FETCH_SIZE and WRITE_SIZE are
    in KiB per dispatch;
    each is scaled by what the same counter reads for the 1 GiB copy of --copy-probe."""
    import hashlib
    f, w = _counter_means([fetch_dir]), _counter_means([write_dir])
    copy = "__amd_rocclr_copyBuffer"
    ff = 1048576.0 / max(f[(copy, "FETCH_SIZE")])
    fw = 1048576.0 / max(w[(copy, "WRITE_SIZE")])
    fp8 = workload == "decode_fp8"
    if workload == "topk_c1":   # the top-k call: every top-k kernel it dispatches
        ks = sorted({kk for (kk, c) in f if kk.startswith("smla::topk_")})
        src = "sparse_mla_attention_topk_amd/csrc/topk.hip"
    else:
        ks = [f"smla::sparse_mla_kernel<{'true' if fp8 else 'false'}>",
              f"smla::split_combine_kernel<{'true' if fp8 else 'false'}>"]
        src = "sparse_mla_attention_topk_amd/csrc/attention.hip"
    total = 0.0
    print(f"calibration: FETCH_SIZE x {ff:.5f}, WRITE_SIZE x {fw:.5f}")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB (scaled) | written MB (scaled) |")
    print("|---|---:|---:|---:|---:|")
    for k in ks + sorted({kk for (kk, c) in f if kk.startswith("smla::") and kk not in ks}):
        if (k, "FETCH_SIZE") not in f or (k, "WRITE_SIZE") not in w:
            continue
        fv = statistics.mean(f[(k, "FETCH_SIZE")])
        wv = statistics.mean(w[(k, "WRITE_SIZE")])
        print(f"| `{k}` | {fv:.1f} | {wv:.1f} | {fv * ff * 1024 / 1e6:.2f} | {wv * fw * 1024 / 1e6:.2f} |")
        if k in ks:
            total += (fv * ff + wv * fw) * 1024
    sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    print(f"\ntraffic-record: source={src} sha256={sha} bytes_per_call={int(round(total))}")


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_bf16_B64_H64_k2048_hbm_traffic.md")
INDEXER_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "indexer_B64_Hi64_L8K-64K_hbm_traffic.md")
FP8_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_fp8_B128_H64_k2048_hbm_traffic.md")
TOPK_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "topk_c1_R64_L65536_k2048_hbm_traffic.md")


def measured_traffic(record=TRAFFIC_RECORD):
    """HBM bytes per call from a committed counter record, or None when the kernel source has
    changed since the counters were taken."""
    import hashlib
    try:
        line = [l for l in open(record) if l.startswith("traffic-record:")][0]
    except (OSError, IndexError):
        return None
    fields = dict(kv.split("=", 1) for kv in line.split()[1:])
    src = os.path.join(ROOT, fields["source"])
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != fields["sha256"]:
        return None
    return int(fields["bytes_per_call"])


# ----------------------------------------------------------------------------------------------
# CPU oracle baseline: worker processes forked before any GPU call, the paged cache shared with them
# through one shared-memory block
# ----------------------------------------------------------------------------------------------

def _cpu_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _worker_init():
    # one BLAS thread per worker: set before numpy is first imported in this (forked) process
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[v] = "1"
    import numpy  # noqa: F401
    from threadpoolctl import threadpool_limits
    global _WORKER_LIMITS
    _WORKER_LIMITS = threadpool_limits(limits=1)


_WORKER_LIMITS = None


def _oracle_task(args):
    """One chunk of rows through the oracle's whole decode path; returns the rows done and the
    seconds it took in this worker."""
    import numpy as np
    from multiprocessing import shared_memory

    import oracle.reference as O
    kind = args["kind"]
    t0 = time.perf_counter()
    if kind == "decode":
        shm = shared_memory.SharedMemory(name=args["shm"])
        if args.get("worker", True):
            # the creating process owns (and unlinks) the block; attaching must not register it again
            from multiprocessing import resource_tracker
            resource_tracker.unregister(shm._name, "shared_memory")
        try:
            kv = np.ndarray(args["kv_shape"], dtype=np.uint8, buffer=shm.buf)
            O.decode_rows(args["q"], kv, args["kv_dtype"], args["bt"], args["row_req"], args["scores"],
                          args["lengths"], args["k"], args["scale"])
            del kv
        finally:
            shm.close()
    else:
        O.topk_rows(args["scores"], None, args["k"])
    return args["n"], time.perf_counter() - t0


class CpuBaseline:
    """The oracle timed on a bounded sample, on `workers` processes and on one core."""

    def __init__(self, enabled: bool):
        self.pool = None
        self.workers = _cpu_workers()
        if enabled and self.workers > 1:
            import multiprocessing
            self.pool = multiprocessing.get_context("fork").Pool(self.workers, initializer=_worker_init)

    def close(self):
        if self.pool is not None:
            self.pool.terminate()
            self.pool.join()

    def run(self, tasks, n_rows_1core, what):
        """tasks: list of task dicts cycling over the sample; returns the cpu_baseline object."""
        done1 = 0
        t1 = 0.0
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            for t in tasks:
                if done1 >= n_rows_1core:
                    break
                n, dt = _oracle_task(dict(t, worker=False))
                done1 += n
                t1 += dt
        one = done1 / t1 if t1 > 0 else None
        if self.pool is None:
            return {"value": one, "unit": "rows/s", "cores": 1, "kind": "oracle",
                    "sample": f"{done1} rows of {what} (numpy fp64, 1 process, 1 BLAS thread): {t1:.1f} s"}
        w0 = time.perf_counter()
        res = self.pool.map(_oracle_task, tasks, chunksize=1)
        wall = time.perf_counter() - w0
        rows = sum(r[0] for r in res)
        cpu_s = sum(r[1] for r in res)
        return {"value": rows / wall, "unit": "rows/s", "cores": self.workers, "kind": "oracle",
                "value_1core": one,
                "sample": f"{rows} rows of {what} (numpy fp64, {self.workers} worker processes of 1 BLAS thread "
                          f"each, {cpu_s:.1f} s of CPU time in {wall:.1f} s; one core: {done1} rows at "
                          f"{one:.1f} rows/s); host reports {os.cpu_count()} cores"}


def _decode_tasks(wl, kv_shape, shm_name, n_rows, chunk=16):
    """Chunks of rows of the rotating sets, in turn, until n_rows rows are listed."""
    import numpy as np
    import torch
    bt = wl.cache.block_table.cpu().numpy()
    host = []
    for rs in wl.sets:
        host.append((rs.q.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), rs.scores.cpu().numpy(),
                     rs.lengths.cpu().numpy(), rs.row_req.cpu().numpy()))
    tasks, done, i = [], 0, 0
    while done < n_rows:
        q, sc, ln, rq = host[i % len(host)]
        for r0 in range(0, q.shape[0], chunk):
            if done >= n_rows:
                break
            r1 = min(q.shape[0], r0 + chunk, r0 + n_rows - done)
            tasks.append({"kind": "decode", "shm": shm_name, "kv_shape": kv_shape, "kv_dtype": wl.cache.kv_dtype,
                          "bt": bt, "q": q[r0:r1], "scores": sc[r0:r1], "lengths": ln[r0:r1], "row_req": rq[r0:r1],
                          "k": wl.k, "scale": wl.scale, "n": r1 - r0})
            done += r1 - r0
        i += 1
    return tasks


# ----------------------------------------------------------------------------------------------
# GPU timing
# ----------------------------------------------------------------------------------------------

def _capture(torch, s, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    return g


def _replay_median(torch, s, run, min_ms, min_reps=5):
    """Replays `run` (a graph replay, or an eager loop) timing each with events on stream s, until
    at least min_ms of GPU time and min_reps replays are covered.  Returns (median ms, replays)."""
    times = []
    total = 0.0
    with torch.cuda.stream(s):
        while total < min_ms or len(times) < min_reps:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            run()
            e1.record(s)
            e1.synchronize()
            t = e0.elapsed_time(e1)
            times.append(t)
            total += t
            if len(times) > 100000:
                break
    return statistics.median(times), len(times)


def _timed_calls(torch, s, fn, n, warmup, min_ms, graph=True):
    """ms per call of fn(i): a graph of n calls (after a graph of warmup calls), replayed until min_ms
    are timed; the median replay over n.  Returns (ms per call, replays)."""
    s.wait_stream(torch.cuda.current_stream())
    if graph:
        with torch.cuda.stream(s):
            gw = _capture(torch, s, lambda: [fn(i) for i in range(warmup)])
            g = _capture(torch, s, lambda: [fn(i) for i in range(n)])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            gw.replay()
        torch.cuda.synchronize()
        ms, reps = _replay_median(torch, s, g.replay, min_ms)
    else:
        with torch.cuda.stream(s):
            for i in range(warmup):
                fn(i)
        torch.cuda.synchronize()
        ms, reps = _replay_median(torch, s, lambda: [fn(i) for i in range(n)], min_ms)
    return ms / n, reps


def _copy_probe(torch, dev):
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    torch.empty_like(a).copy_(a)
    torch.cuda.synchronize()


def _stream_copy_GBps(torch, dev, s, reps: int = 9) -> float:
    """Measured device-to-device copy rate of 1 GiB on the bench's stream: bytes read plus bytes written
    per second, the median of `reps` copies (the practical streaming peak the gather is compared with)."""
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(s):
        a.fill_(1.0)
        b.copy_(a)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            b.copy_(a)
            e1.record(s)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
    times.sort()
    del a, b
    return 2.0 * (1 << 30) / (times[len(times) // 2] * 1e-3) / 1e9


def _base_line(args, metric, value, unit, ms, reps, dtype, config):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config, "timed_replays": reps,
            "timing": f"median of {reps} timed replays of a graph of {args.steps} steps"}


# ----------------------------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------------------------

def bench_decode(args, cpu: CpuBaseline):
    import numpy as np
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8 = args.workload == "decode_fp8"
    wl = W.decode_fp8(dev, n_sets=N_SETS) if fp8 else W.decode_bf16(dev, n_sets=N_SETS)
    B, H, k = wl.sets[0].q.shape[0], wl.H, wl.k
    rec = W.FP8_RECORD_BYTES if fp8 else W.BF16_RECORD_BYTES
    gathered = B * k * rec                            # every row has >= k candidates
    flops = B * H * k * (576 + 512) * 2

    ws = smla.attention_workspace(B, H, k, dev, wl.cache.kv_dtype)
    tws = smla.topk_workspace(B, k, wl.sets[0].scores.shape[1], dev)
    idx = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(N_SETS)]
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    def topk(i):
        rs = wl.sets[i % N_SETS]
        smla.topk_per_row(rs.scores, k, lengths=rs.lengths, out=idx[i % N_SETS], workspace=tws)

    def attn(i):
        rs = wl.sets[i % N_SETS]
        smla.sparse_mla_decode(rs.q, wl.cache.kv, wl.cache.block_table, idx[i % N_SETS], wl.scale,
                               row_req=rs.row_req, kv_dtype=wl.cache.kv_dtype, out=out, lse=lse, workspace=ws)

    def step(i):
        topk(i)
        attn(i)

    for i in range(N_SETS):      # eager run first (also loads the kernels)
        step(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    g = not args.no_graph
    w0 = time.perf_counter()
    ms_step, reps = _timed_calls(torch, s, step, args.steps, args.warmup, args.min_timed_ms, g)
    attn_ms, _ = _timed_calls(torch, s, attn, args.steps, args.warmup, args.min_timed_ms, g)
    topk_ms, _ = _timed_calls(torch, s, topk, args.steps, args.warmup, args.min_timed_ms, g)
    wall = time.perf_counter() - w0
    rows_per_s = B / (ms_step * 1e-3)
    achieved = gathered / (attn_ms * 1e-3) / 1e9
    copy_GBps = _stream_copy_GBps(torch, dev, s)
    if args.copy_probe:
        _copy_probe(torch, dev)

    cpu_line = None
    if args.cpu_rows > 0:
        from multiprocessing import shared_memory
        kv_shape = tuple(wl.cache.kv.shape)
        shm = shared_memory.SharedMemory(create=True, size=int(np.prod(kv_shape)))
        try:
            host = np.ndarray(kv_shape, dtype=np.uint8, buffer=shm.buf)
            torch.from_numpy(host).copy_(wl.cache.kv)
            del host
            # FP8 rows cost the oracle about 4 times a bf16 row (record decoding)
            n = args.cpu_rows // 4 if fp8 else args.cpu_rows
            n1 = args.cpu_rows_1core // 4 if fp8 else args.cpu_rows_1core
            tasks = _decode_tasks(wl, kv_shape, shm.name, n)
            cpu_line = cpu.run(tasks, n1, "the same workload, the rotating sets in turn (top-k + gather + attention)")
        finally:
            shm.close()
            shm.unlink()

    line = _base_line(args, METRIC if not fp8 else METRIC_FP8, rows_per_s, "rows/s", ms_step, reps,
                      "fp8_e4m3/bf16" if fp8 else "bf16",
                      {"workload": wl.name, "rows": B, "heads": H, "topk": k, "d_qk": 576, "d_v": 512,
                       "page_block_size": 64, "kv": "fp8_e4m3_g128" if fp8 else "bf16",
                       "context": "uniform [32768, 131072]" if fp8 else "uniform [8192, 65536]",
                       "rotating_sets": N_SETS, "launch": "eager" if args.no_graph else "hip_graph_of_K_steps"})
    line.update({
        "gathered_kv_GBps": achieved,
        "step_gathered_kv_GBps": gathered / (ms_step * 1e-3) / 1e9,
        "stream_copy_GBps": copy_GBps, "frac_of_stream_copy": achieved / copy_GBps,
        "attention_ms": attn_ms, "topk_ms": topk_ms, "wall_s": wall,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(FP8_TRAFFIC_RECORD if fp8 else TRAFFIC_RECORD),
                     "kernel": "sparse_mla_decode call: attention kernel + split-combine kernel",
                     "algorithmic_bytes_per_launch": gathered,
                     "mfma_tflops": flops / (attn_ms * 1e-3) / 1e12},
        "cpu_baseline": cpu_line,
    })
    print(json.dumps(line), flush=True)


def bench_topk(args, cpu: CpuBaseline):
    """Top-k alone: 64 rows of 65536 fp32 scores with 256 distinct levels each (heavy ties), k = 2048,
    32 rotating copies (512 MiB, larger than the 256 MB last-level cache)."""
    import numpy as np
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R, L, k, copies = 64, 65536, 2048, 32
    sets = [W.topk_levels(dev, rows=R, L=L, seed=100 + c) for c in range(copies)]
    out = torch.empty((R, k), dtype=torch.int32, device=dev)
    tws = smla.topk_workspace(R, k, L, dev)

    def call(i):
        smla.topk_per_row(sets[i % copies], k, out=out, workspace=tws)
    for i in range(copies):
        call(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    n = max(args.steps, copies)
    ms, reps = _timed_calls(torch, s, call, n, args.warmup, args.min_timed_ms, not args.no_graph)
    alg = R * L * 4 + R * k * 4
    if args.copy_probe:
        _copy_probe(torch, dev)
    achieved = alg / (ms * 1e-3) / 1e9
    cpu_line = None
    if args.cpu_rows > 0:
        host = [sets[c].cpu().numpy() for c in range(4)]
        tasks = []
        done = 0
        while done < max(1, args.cpu_rows // 4):
            for h in host:
                for r0 in range(0, R, 8):
                    tasks.append({"kind": "topk", "scores": h[r0:r0 + 8], "k": k, "n": 8})
                    done += 8
        cpu_line = cpu.run(tasks, max(8, args.cpu_rows_1core // 4), "the same rows (top-k only)")
    line = _base_line(args, "stable top-k rows/s + scores-read HBM GB/s (64 x 65536 fp32, 256 levels, k=2048, 1 GPU)",
                      R / (ms * 1e-3), "rows/s", ms, reps, "fp32 keys / int32 indices",
                      {"workload": "topk_c1_R64_L65536_levels256_k2048", "rows": R, "candidates": L, "topk": k,
                       "levels": 256, "rotating_copies": copies, "launch": "hip_graph_of_K_calls"})
    line["steps"] = n
    line.update({
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(TOPK_TRAFFIC_RECORD),
                     "kernel": "topk_per_row call",
                     "algorithmic_bytes_per_launch": alg},
        "cpu_baseline": cpu_line,
    })
    print(json.dumps(line), flush=True)


def bench_kv_write(args):
    """FP8 cache write: T = 65536 new tokens (a 64K-token prefill) into a paged cache, four
    rotating token sets so the 75 MB of input per call is not cache-resident; plus T = 128 (one
    decode step of the FP8 decode workload's batch), and the inverse-RoPE form of both."""
    import numpy as np
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, pages, max_pos = 65536, 4200, 131072
    sets = [W.cache_write_tokens(dev, T=T, num_pages=pages, seed=20 + i) for i in range(N_SETS)]
    cache = torch.zeros((pages, 64, W.FP8_RECORD_BYTES), dtype=torch.uint8, device=dev)
    small = W.cache_write_tokens(dev, T=128, num_pages=pages, seed=30)
    cs = W.rope_cos_sin(max_pos, dev)
    pos = torch.randint(0, max_pos, (T,), generator=torch.Generator(device="cpu").manual_seed(31)).to(dev)
    for w in sets + [small]:
        smla.kv_cache_write(w.tokens, w.slots, cache)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    g = not args.no_graph
    big_ms, reps = _timed_calls(torch, s, lambda i: smla.kv_cache_write(sets[i % N_SETS].tokens, sets[i % N_SETS].slots,
                                                                       cache), args.steps, args.warmup,
                                args.min_timed_ms, g)
    small_ms, _ = _timed_calls(torch, s, lambda i: smla.kv_cache_write(small.tokens, small.slots, cache), args.steps,
                               args.warmup, args.min_timed_ms, g)
    rope_ms, _ = _timed_calls(torch, s, lambda i: smla.kv_cache_write(sets[i % N_SETS].tokens, sets[i % N_SETS].slots,
                                                                      cache, positions=pos, cos_sin=cs),
                              args.steps, args.warmup, args.min_timed_ms, g)
    per_tok = 2 * 576 + W.FP8_RECORD_BYTES + 8          # bf16 token in, record out, slot
    achieved = T * per_tok / (big_ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_rows > 0:
        import oracle.reference as O
        toks = sets[0].tokens[:args.cpu_rows * 2].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        for t in toks:
            O.encode_record(t, O.KV_FP8)
        dt = time.perf_counter() - t0
        cpu = {"value": len(toks) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{len(toks)} tokens of the same workload encoded by the oracle (numpy, 1 thread), "
                         f"{dt:.1f} s"}
    line = _base_line(args, "FP8 KV cache write tokens/s (e4m3, 128-entry fp32 scale groups, T=65536, 1 GPU)",
                      T / (big_ms * 1e-3), "tokens/s", big_ms, reps, "bf16->fp8_e4m3",
                      {"workload": "kv_write_fp8_T65536", "tokens": T, "record_bytes": W.FP8_RECORD_BYTES,
                       "rotating_sets": N_SETS, "launch": "hip_graph_of_K_calls"})
    line.update({
        "decode_step_T128_us": small_ms * 1e3,
        "inverse_rope_T65536_us": rope_ms * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "kernel": "kv_cache_write_kernel<true, false>",
                     "algorithmic_bytes_per_launch": T * per_tok},
        "cpu_baseline": cpu,
    })
    print(json.dumps(line), flush=True)


def bench_window(args):
    """Decode over compressed and sliding-window KV: the decode_bf16 rows (B = 64, H = 64, top-k 2048 of
    contexts U[8192, 65536]) plus, per row, its 128 window + 5 draft positions from a separate window
    cache, one softmax (smla_sparse_mla_decode_with_window), window width 192 and the same rows at 256.
    Four rotating (Q, scores) sets."""
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.decode_bf16(dev, n_sets=N_SETS)
    B, H, k = wl.sets[0].q.shape[0], wl.H, wl.k
    win = W.window_cache(wl.cache.ctx_lens, W.KV_BF16, dev, seed=61, max_pages=int(wl.cache.block_table.shape[1]))
    idxw256 = torch.full((B, 256), -1, dtype=torch.int32, device=dev)
    idxw256[:, :192] = win.idx
    idx = [smla.topk_per_row(rs.scores, k, lengths=rs.lengths) for rs in wl.sets]
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = smla.attention_workspace(B, H, k + 256, dev)
    tws = smla.topk_workspace(B, k, wl.sets[0].scores.shape[1], dev)

    def attn(iw):
        def f(i):
            rs = wl.sets[i % N_SETS]
            smla.sparse_mla_decode_with_window(rs.q, wl.cache.kv, wl.cache.block_table, idx[i % N_SETS], win.kv,
                                              win.block_table, iw, wl.scale, row_req=rs.row_req, out=out, lse=lse,
                                              workspace=ws)
        return f

    def step(i):
        rs = wl.sets[i % N_SETS]
        smla.topk_per_row(rs.scores, k, lengths=rs.lengths, out=idx[i % N_SETS], workspace=tws)
        attn(win.idx)(i)
    for i in range(N_SETS):
        step(i)
        attn(idxw256)(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    g = not args.no_graph
    step_ms, reps = _timed_calls(torch, s, step, args.steps, args.warmup, args.min_timed_ms, g)
    ms192, _ = _timed_calls(torch, s, attn(win.idx), args.steps, args.warmup, args.min_timed_ms, g)
    ms256, _ = _timed_calls(torch, s, attn(idxw256), args.steps, args.warmup, args.min_timed_ms, g)
    valid_w = int((win.idx >= 0).sum())
    gathered = (B * k + valid_w) * W.BF16_RECORD_BYTES
    achieved = gathered / (ms192 * 1e-3) / 1e9
    line = _base_line(args, "sparse-MLA decode rows/s over top-k 2048 + sliding-window 128 + draft 5 KV (width 192, "
                            "H=64, 1 GPU)", B / (step_ms * 1e-3), "rows/s", step_ms, reps, "bf16",
                      {"workload": "decode_window_B64_H64_k2048_w192", "rows": B, "heads": H, "topk": k,
                       "window_width": 192, "window_valid_per_row": 133, "rotating_sets": N_SETS,
                       "launch": "hip_graph_of_K_steps"})
    line.update({
        "attention_us_width192": ms192 * 1e3, "attention_us_width256": ms256 * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "sparse_mla_decode_with_window call: attention kernel + split-combine kernel",
                     "algorithmic_bytes_per_launch": gathered},
        "cpu_baseline": None,
    })
    print(json.dumps(line), flush=True)


def bench_prefill(args):
    """Prefill chunk: T = 4096 causal query rows of one 131072-token bf16 context (2 GiB of scores),
    top-k 2048 per row, then sparse_mla_prefill_chunk.  The context's 151 MB of KV is read 4096 x 2048
    times (9.66 GB algorithmic), so the attention is bound by MFMA and the L2/MALL, not HBM."""
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.prefill_chunk(dev)
    T, H, k = wl.q.shape[0], wl.H, wl.k
    lengths = smla.fill_causal_lengths(wl.first_pos, T, device=dev)
    bt = wl.cache.block_table[0].contiguous()
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = smla.attention_workspace(T, H, k, dev)
    tws = smla.topk_workspace(T, k, wl.scores.shape[1], dev)

    def topk(i):
        smla.topk_per_row(wl.scores, k, lengths=lengths, out=idx, workspace=tws)

    def attn(i):
        smla.sparse_mla_prefill_chunk(wl.q, wl.cache.kv, bt, idx, wl.scale, out=out, lse=lse, workspace=ws)

    def step(i):
        topk(i)
        attn(i)
    step(0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    n, w = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
    g = not args.no_graph
    step_ms, reps = _timed_calls(torch, s, step, n, w, args.min_timed_ms, g)
    attn_ms, _ = _timed_calls(torch, s, attn, n, w, args.min_timed_ms, g)
    topk_ms, _ = _timed_calls(torch, s, topk, n, w, args.min_timed_ms, g)
    flops = T * H * k * (576 + 512) * 2
    tflops = flops / (attn_ms * 1e-3) / 1e12
    gathered = T * k * W.BF16_RECORD_BYTES
    line = _base_line(args, "sparse-MLA prefill-chunk rows/s (T=4096 causal rows, 131072-token context, H=64, "
                            "topk=2048, 1 GPU)", T / (step_ms * 1e-3), "rows/s", step_ms, reps, "bf16",
                      {"workload": wl.name, "rows": T, "heads": H, "topk": k, "context": 131072,
                       "first_pos": wl.first_pos, "launch": "hip_graph_of_K_steps"})
    line.update({"steps": n, "warmup": w, "attention_ms": attn_ms, "topk_ms": topk_ms,
                 "attention_effective_GBps": gathered / (attn_ms * 1e-3) / 1e9,
                 "roofline": {"bound": "mfma", "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s",
                              "frac": tflops / 2500.0, "traffic": None,
                              "kernel": "sparse_mla_prefill_chunk call: attention kernel + split-combine kernel",
                              "algorithmic_flops_per_launch": flops},
                 "cpu_baseline": None})
    print(json.dumps(line), flush=True)


def bench_indexer(args):
    """Indexer scores (paged MQA logits) for B = 64 decode rows: 64 index heads of width 128, one bf16
    128-wide key per token (256 B) in pages of 64, contexts U[8192, 65536] (2.36 M keys, 604 MB per
    call, larger than the 256 MB last-level cache), every row written in full (65536 fp32 entries, -inf
    past its length).  Four rotating (Q, weights) sets."""
    import numpy as np
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.indexer_decode(dev, n_sets=N_SETS)
    B, Hi, S = wl.q[0].shape[0], wl.Hi, wl.stride
    out = torch.empty((B, S), dtype=torch.float32, device=dev)

    def call(i):
        smla.paged_mqa_logits(wl.q[i % N_SETS], wl.weights[i % N_SETS], wl.kidx, wl.block_table, lengths=wl.lengths,
                              row_req=wl.row_req, out=out)
    for i in range(N_SETS):
        call(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    ms, reps = _timed_calls(torch, s, call, args.steps, args.warmup, args.min_timed_ms, not args.no_graph)
    if args.copy_probe:
        _copy_probe(torch, dev)
    keys = int(wl.ctx_lens.sum())
    pages = int(sum((int(L) + 63) // 64 for L in wl.ctx_lens))
    key_bytes = keys * 256
    alg_bytes = key_bytes + B * S * 4 + B * Hi * 128 * 2 + B * Hi * 4 + pages * 4
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    flops = keys * Hi * 128 * 2
    cpu = None
    if args.cpu_rows > 0:
        from threadpoolctl import threadpool_limits

        import oracle.reference as O
        n = max(1, min(B, args.cpu_rows // 128))
        qb = wl.q[0][:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        kb = wl.kidx.view(torch.int16).cpu().numpy().view(np.uint16)
        wn, btn = wl.weights[0][:n].cpu().numpy(), wl.block_table.cpu().numpy()
        ln = wl.lengths.cpu().numpy()
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.indexer_scores(qb, wn, kb, btn, list(range(n)), ln[:n], S)
            dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} rows of the same workload ({int(ln[:n].sum())} keys) scored by the oracle "
                         f"(numpy fp64, 1 thread), {dt:.1f} s"}
    line = _base_line(args, "indexer scores (paged MQA logits) rows/s + key-stream HBM GB/s (B=64, Hi=64, d=128, 1 GPU)",
                      B / (ms * 1e-3), "rows/s", ms, reps, "bf16 (fp32 accumulate)",
                      {"workload": wl.name, "rows": B, "index_heads": Hi, "index_dim": 128, "page_block_size": 64,
                       "context": "uniform [8192, 65536]", "score_row": S, "keys_per_call": keys,
                       "rotating_sets": N_SETS, "launch": "hip_graph_of_K_calls"})
    line.update({
        "key_GBps": key_bytes / (ms * 1e-3) / 1e9,
        "mfma_tflops": flops / (ms * 1e-3) / 1e12,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(INDEXER_TRAFFIC_RECORD),
                     "kernel": "paged_mqa_logits_kernel<4, true, true>",
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
    })
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.traffic_record:
        return traffic_record(args.traffic_record[0], args.traffic_record[1], args.workload)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (rows shard across GPUs "
              f"without any exchange, so the per-GPU figure is the one to read)", file=sys.stderr)
        sys.exit(2)
    # The CPU-oracle workers are forked here, before anything touches the GPU.
    cpu = CpuBaseline(args.cpu_rows > 0 and args.workload in ("decode_bf16", "decode_fp8", "topk_c1"))
    try:
        if args.workload == "kv_write_fp8":
            return bench_kv_write(args)
        if args.workload == "decode_window":
            return bench_window(args)
        if args.workload == "prefill_c4":
            return bench_prefill(args)
        if args.workload == "indexer":
            return bench_indexer(args)
        if args.workload == "topk_c1":
            return bench_topk(args, cpu)
        return bench_decode(args, cpu)
    finally:
        cpu.close()


if __name__ == "__main__":
    main()
