"""Throughput of the sparse-MLA decode hot path on one MI355X.

One step = the whole path for one batch: stable top-k per row over the indexer scores (with length
clamping) -> canonical indices -> paged gather + MQA attention + split combine.  Workload: B=64
decode rows, H=64 heads, top-k 2048, d_qk 576 (512 latent + 64 rope), d_v 512, bf16 KV in pages of
64, context lengths uniform in [8192, 65536], random page tables.  Four independent (Q, scores) sets
rotate over one 2.7 GB KV pool so a step's gathered set (151 MB) is not already cache-resident.

Prints one JSON line.  `value` is rows/s of the whole step with every input resident in HBM;
`roofline` reports the attention kernel's gathered-KV bandwidth against the 8 TB/s HBM peak;
`cpu_baseline` times the CPU oracle on a bounded sample of the same rows.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode rows/s + gathered-KV HBM GB/s (H=64, topk=2048, 1 GPU)"
METRIC_FP8 = "sparse-MLA decode rows/s + gathered-KV HBM GB/s (FP8 KV, B=128, H=64, topk=2048, 1 GPU)"
HBM_PEAK_GBPS = 8000.0
N_SETS = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-rows", type=int, default=768, help="rows of the CPU-oracle sample (0 = skip)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--workload", default="decode_bf16", choices=["decode_bf16", "decode_fp8", "kv_write_fp8", "decode_swa192", "prefill_c4",
                                                              "indexer"],
                    help="decode_bf16: B=64, contexts U[8192, 65536], bf16 KV (the headline); "
                         "decode_fp8: B=128, contexts U[32768, 131072], FP8 KV; "
                         "kv_write_fp8: FP8 cache write of 65536 new tokens (and of 128, a decode step); "
                         "decode_swa192: B=64 draft rows over 128 sliding-window + 5 draft positions, index "
                         "width 192 (and the same rows at width 256); "
                         "prefill_c4: one request, T=4096 query tokens at positions 126976..131071 of a "
                         "131072-token context, causal top-k 2048 + prefill attention; "
                         "indexer: indexer scores (paged MQA logits) of B=64 decode rows, 64 index heads of "
                         "width 128, contexts U[8192, 65536], score rows of 65536")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (calibrates rocprofv3 FETCH/WRITE_SIZE)")
    return ap.parse_args()


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_bf16_B64_H64_k2048_hbm_traffic.md")
INDEXER_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "indexer_B64_Hi64_L8K-64K_hbm_traffic.md")
FP8_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_fp8_B128_H64_k2048_hbm_traffic.md")


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


def cpu_baseline(wl, n_rows):
    """The oracle, as it is, on n_rows rows taken from the rotating sets in order, cycling through them
    again when n_rows exceeds their rows (single BLAS thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle.reference as O

    kvh = wl.cache.kv.cpu().numpy()
    bt = wl.cache.block_table.cpu().numpy()
    done = 0
    t_total = 0.0
    with threadpool_limits(limits=1):
        for i in range(10 ** 6):
            if done >= n_rows:
                break
            rs = wl.sets[i % len(wl.sets)]
            take = min(n_rows - done, rs.q.shape[0])
            qb = rs.q[:take].contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
            sc = rs.scores[:take].cpu().numpy()
            ln = rs.lengths[:take].cpu().numpy()
            rq = rs.row_req[:take].cpu().numpy()
            t0 = time.perf_counter()
            O.decode_rows(qb, kvh, wl.cache.kv_dtype, bt, rq, sc, ln, wl.k, wl.scale)
            t_total += time.perf_counter() - t0
            done += take
    return {"value": done / t_total, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} rows of the same workload, the rotating sets in turn (top-k + gather + attention, "
                      f"numpy fp64, 1 thread): {t_total:.1f} s of CPU time on a host with {os.cpu_count()} cores"}


def _graph_time(torch, s, fn, n, warmup):
    """ms per call of fn over one HIP graph of n calls (after a graph of warmup calls), timed with
    events on the stream the kernels run on."""
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gw, g = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=s):
            for i in range(warmup):
                fn(i)
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        gw.replay()
        torch.cuda.synchronize()
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _eager_time(torch, s, fn, n, warmup):
    """ms per call of fn over n eager calls on stream s (after warmup calls), timed with events on s."""
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for i in range(n):
            fn(i)
        e1.record(s)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def bench_kv_write(args):
    """FP8 cache write: T = 65536 new tokens (a 64K-token prefill) into a paged cache, four
    rotating token sets so the 75 MB of input per call is not cache-resident; plus T = 128 (one
    decode step of the FP8 decode workload's batch)."""
    import numpy as np
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, pages = 65536, 4200
    sets = [W.cache_write_tokens(dev, T=T, num_pages=pages, seed=20 + i) for i in range(N_SETS)]
    cache = torch.zeros((pages, 64, W.FP8_RECORD_BYTES), dtype=torch.uint8, device=dev)
    small = W.cache_write_tokens(dev, T=128, num_pages=pages, seed=30)
    for w in sets + [small]:
        smla.kv_cache_write(w.tokens, w.slots, cache)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    big_ms = _graph_time(torch, s, lambda i: smla.kv_cache_write(sets[i % N_SETS].tokens, sets[i % N_SETS].slots,
                                                                 cache), args.steps, args.warmup)
    small_ms = _graph_time(torch, s, lambda i: smla.kv_cache_write(small.tokens, small.slots, cache), args.steps,
                           args.warmup)
    per_tok = 2 * 576 + W.FP8_RECORD_BYTES + 8          # bf16 token in, record out, slot
    achieved = T * per_tok / (big_ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_rows > 0:
        import oracle.reference as O
        toks = sets[0].tokens[:args.cpu_rows * 8].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        for t in toks:
            O.encode_record(t, O.KV_FP8)
        dt = time.perf_counter() - t0
        cpu = {"value": len(toks) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{len(toks)} tokens of the same workload encoded by the oracle (numpy, 1 thread), "
                         f"{dt:.1f} s"}
    line = {
        "metric": "FP8 KV cache write tokens/s (e4m3, 128-entry fp32 scale groups, T=65536, 1 GPU)",
        "value": T / (big_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": big_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->fp8_e4m3", "data": "synthetic",
        "config": {"workload": "kv_write_fp8_T65536", "tokens": T, "record_bytes": W.FP8_RECORD_BYTES,
                   "rotating_sets": N_SETS, "launch": "hip_graph_of_K_calls"},
        "decode_step_T128_us": small_ms * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "kernel": "kv_cache_write_kernel<true>",
                     "algorithmic_bytes_per_launch": T * per_tok},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_swa(args):
    """Attention over sliding-window + draft index rows: B = 64 rows, H = 64, each row 133 valid
    positions (128 window + 5 draft) padded with -1 to width 192, and the same rows padded to 256.
    Four rotating (Q, indices) sets over one bf16 KV pool of contexts U[8192, 65536]."""
    import torch

    import sparse_mla_attention_topk_amd as smla
    from sparse_mla_attention_topk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H = 64, 64
    wl = W.decode_bf16(dev, n_sets=N_SETS)
    ctx = wl.cache.ctx_lens.to(dev)
    idx192 = W.swa_draft_indices(ctx)
    idx256 = torch.full((B, 256), -1, dtype=torch.int32, device=dev)
    idx256[:, :192] = idx192
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream(dev)

    def call(idx):
        return lambda i: smla.sparse_mla_decode(wl.sets[i % N_SETS].q, wl.cache.kv, wl.cache.block_table, idx,
                                                wl.scale, row_req=wl.sets[i % N_SETS].row_req, out=out, lse=lse)
    for i in range(N_SETS):
        call(idx192)(i)
        call(idx256)(i)
    torch.cuda.synchronize()
    ms192 = _graph_time(torch, s, call(idx192), args.steps, args.warmup)
    ms256 = _graph_time(torch, s, call(idx256), args.steps, args.warmup)
    valid = int((idx192 >= 0).sum())
    gathered = valid * W.BF16_RECORD_BYTES
    achieved = gathered / (ms192 * 1e-3) / 1e9
    line = {
        "metric": "sparse-MLA decode rows/s, sliding-window + draft rows (128 + 5 valid, index width 192, H=64, 1 GPU)",
        "value": B / (ms192 * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms192, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_swa192_B64_H64", "rows": B, "heads": H, "index_width": 192,
                   "valid_per_row": 133, "rotating_sets": N_SETS, "launch": "hip_graph_of_K_calls"},
        "attention_us_width192": ms192 * 1e3, "attention_us_width256": ms256 * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "sparse_mla_decode call (one split: attention kernel only)",
                     "algorithmic_bytes_per_launch": gathered},
        "cpu_baseline": None,
    }
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
    step_ms = _graph_time(torch, s, step, n, w)
    attn_ms = _graph_time(torch, s, attn, n, w)
    topk_ms = _graph_time(torch, s, topk, n, w)
    flops = T * H * k * (576 + 512) * 2
    tflops = flops / (attn_ms * 1e-3) / 1e12
    gathered = T * k * W.BF16_RECORD_BYTES
    line = {
        "metric": "sparse-MLA prefill-chunk rows/s (T=4096 causal rows, 131072-token context, H=64, topk=2048, 1 GPU)",
        "value": T / (step_ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": n, "warmup": w,
        "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": T, "heads": H, "topk": k, "context": 131072,
                   "first_pos": wl.first_pos, "launch": "hip_graph_of_K_steps"},
        "attention_ms": attn_ms, "topk_ms": topk_ms,
        "attention_effective_GBps": gathered / (attn_ms * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s", "frac": tflops / 2500.0,
                     "traffic": None, "kernel": "sparse_mla_prefill_chunk call: attention kernel + split-combine kernel",
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
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
    if args.no_graph:
        ms = _eager_time(torch, s, call, args.steps, args.warmup)
    else:
        ms = _graph_time(torch, s, call, args.steps, args.warmup)
    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
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
        n = max(1, min(B, args.cpu_rows // 4))
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
    line = {
        "metric": "indexer scores (paged MQA logits) rows/s + key-stream HBM GB/s (B=64, Hi=64, d=128, 1 GPU)",
        "value": B / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": wl.name, "rows": B, "index_heads": Hi, "index_dim": 128, "page_block_size": 64,
                   "context": "uniform [8192, 65536]", "score_row": S, "keys_per_call": keys,
                   "rotating_sets": N_SETS, "launch": "hip_graph_of_K_calls"},
        "key_GBps": key_bytes / (ms * 1e-3) / 1e9,
        "mfma_tflops": flops / (ms * 1e-3) / 1e12,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(INDEXER_TRAFFIC_RECORD),
                     "kernel": "paged_mqa_logits_kernel<4, true, true>",
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (rows shard across GPUs "
              f"without any exchange, so the per-GPU figure is the one to read)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "kv_write_fp8":
        return bench_kv_write(args)
    if args.workload == "decode_swa192":
        return bench_swa(args)
    if args.workload == "prefill_c4":
        return bench_prefill(args)
    if args.workload == "indexer":
        return bench_indexer(args)
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
        rs = wl.sets[i]
        smla.topk_per_row(rs.scores, k, lengths=rs.lengths, out=idx[i], workspace=tws)

    def attn(i):
        rs = wl.sets[i]
        smla.sparse_mla_decode(rs.q, wl.cache.kv, wl.cache.block_table, idx[i], wl.scale, row_req=rs.row_req,
                               kv_dtype=wl.cache.kv_dtype, out=out, lse=lse, workspace=ws)

    def steps(n, what):
        for st in range(n):
            if what in ("step", "topk"):
                topk(st % N_SETS)
            if what in ("step", "attn"):
                attn(st % N_SETS)

    for i in range(N_SETS):      # eager run first (also loads the kernels)
        topk(i)
        attn(i)
    torch.cuda.synchronize()

    # Each timed region is one launch of K calls: a HIP graph holding them (or, with --no-graph, an
    # eager loop), bracketed by events on the stream the kernels run on.
    s = torch.cuda.Stream(dev)
    runs = {}
    if args.no_graph:
        for what in ("step", "attn", "topk"):
            runs[what] = (lambda what=what: steps(args.steps, what))
        warm = lambda: steps(args.warmup, "step")
    else:
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s):
            graphs = {}
            for what, n in (("warm", args.warmup), ("step", args.steps), ("attn", args.steps), ("topk", args.steps)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    steps(n, "step" if what == "warm" else what)
                graphs[what] = g
        torch.cuda.current_stream(dev).wait_stream(s)
        torch.cuda.synchronize()
        warm = graphs["warm"].replay
        for what in ("step", "attn", "topk"):
            runs[what] = graphs[what].replay

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1), time.perf_counter() - w0

    with torch.cuda.stream(s):
        warm()
    torch.cuda.synchronize()
    ms_total, wall = timed(runs["step"])
    attn_total, _ = timed(runs["attn"])
    topk_total, _ = timed(runs["topk"])
    ms_step = ms_total / args.steps
    attn_ms = attn_total / args.steps
    topk_ms = topk_total / args.steps
    rows_per_s = B / (ms_step * 1e-3)
    achieved = gathered / (attn_ms * 1e-3) / 1e9

    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if args.cpu_rows > 0:
        # FP8 rows cost the oracle about 4 times a bf16 row (record decoding): half the rows keeps the
        # sample near 20 s
        cpu = cpu_baseline(wl, args.cpu_rows // 2 if fp8 else args.cpu_rows)

    line = {
        "metric": METRIC if not fp8 else METRIC_FP8, "value": rows_per_s, "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3/bf16" if fp8 else "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "rows": B, "heads": H, "topk": k, "d_qk": 576, "d_v": 512,
                   "page_block_size": 64, "kv": "fp8_e4m3_g128" if fp8 else "bf16",
                   "context": "uniform [32768, 131072]" if fp8 else "uniform [8192, 65536]",
                   "rotating_sets": N_SETS, "launch": "eager" if args.no_graph else "hip_graph_of_K_steps"},
        "gathered_kv_GBps": achieved,
        "step_gathered_kv_GBps": gathered / (ms_step * 1e-3) / 1e9,
        "attention_ms": attn_ms, "topk_ms": topk_ms, "wall_s": wall,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(FP8_TRAFFIC_RECORD if fp8 else TRAFFIC_RECORD),
                     "kernel": "sparse_mla_decode call: attention kernel + split-combine kernel",
                     "algorithmic_bytes_per_launch": gathered,
                     "mfma_tflops": flops / (attn_ms * 1e-3) / 1e12},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
