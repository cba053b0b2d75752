"""HIP-graph replays of the calls the benchmark times in graphs: each replay, with eager calls and
synchronizations between replays, gives results bit-identical to the eager calls.  Outputs are
overwritten with garbage before every replay, so a replay that skips work shows."""

import pytest
import torch

import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def _capture(fn) -> torch.cuda.CUDAGraph:
    """Graph of fn, captured on a side stream after one warm-up call there."""
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8).clone()


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_decode_step_replays_equal_eager(fp8):
    """Top-k then attention (with the split combine) over two rotating sets, as the benchmark's
    step: bf16 cache with B = 64, FP8 cache with B = 128 (chunked top-k, two splits per workgroup)."""
    wl = W.decode_fp8(DEV, n_sets=2) if fp8 else W.decode_bf16(DEV, n_sets=2)
    B, H, k = wl.sets[0].q.shape[0], wl.H, wl.k
    log(f"[graph] decode {'fp8' if fp8 else 'bf16'} B={B} H={H} k={k}")
    ws = smla.attention_workspace(B, H, k, DEV, wl.cache.kv_dtype)
    tws = smla.topk_workspace(B, k, wl.sets[0].scores.shape[1], DEV)
    idx = [torch.empty((B, k), dtype=torch.int32, device=DEV) for _ in range(2)]
    out = [torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    lse = [torch.empty((B, H), dtype=torch.float32, device=DEV) for _ in range(2)]

    def step(i, o=None, l=None, ix=None):
        rs = wl.sets[i]
        ix = idx[i] if ix is None else ix
        smla.topk_per_row(rs.scores, k, lengths=rs.lengths, out=ix, workspace=tws)
        smla.sparse_mla_decode(rs.q, wl.cache.kv, wl.cache.block_table, ix, wl.scale, row_req=rs.row_req,
                               kv_dtype=wl.cache.kv_dtype, out=out[i] if o is None else o,
                               lse=lse[i] if l is None else l, workspace=ws)

    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    ref = [(_bits(idx[i]), _bits(out[i]), _bits(lse[i])) for i in range(2)]

    g = _capture(lambda: (step(0), step(1)))
    spare_o = torch.empty_like(out[0])
    spare_l = torch.empty_like(lse[0])
    spare_i = torch.empty_like(idx[0])
    for r in range(REPLAYS):
        for i in range(2):
            idx[i].fill_(-7)
            out[i].fill_(float("nan"))
            lse[i].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(_bits(idx[i]), ref[i][0]), f"replay {r} set {i}: indices"
            assert torch.equal(_bits(out[i]), ref[i][1]), f"replay {r} set {i}: output"
            assert torch.equal(_bits(lse[i]), ref[i][2]), f"replay {r} set {i}: LSE"
        j = r % 2   # eager work between replays, on the same workspaces
        step(j, o=spare_o, l=spare_l, ix=spare_i)
        torch.cuda.synchronize()
        assert torch.equal(_bits(spare_o), ref[j][1]) and torch.equal(_bits(spare_l), ref[j][2]), f"eager {r}"


def test_indexer_replays_equal_eager():
    """Paged MQA logits over two rotating (Q, weights) sets, B = 64, Hi = 64."""
    wl = W.indexer_decode(DEV, n_sets=2)
    B, S = wl.q[0].shape[0], wl.stride
    log(f"[graph] indexer B={B} stride={S}")
    out = [torch.empty((B, S), dtype=torch.float32, device=DEV) for _ in range(2)]

    def call(i, o=None):
        smla.paged_mqa_logits(wl.q[i], wl.weights[i], wl.kidx, wl.block_table, lengths=wl.lengths,
                              row_req=wl.row_req, out=out[i] if o is None else o)

    for i in range(2):
        call(i)
    torch.cuda.synchronize()
    ref = [_bits(out[i]) for i in range(2)]
    g = _capture(lambda: (call(0), call(1)))
    spare = torch.empty_like(out[0])
    for r in range(REPLAYS):
        for i in range(2):
            out[i].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(_bits(out[i]), ref[i]), f"replay {r} set {i}"
        call(r % 2, o=spare)
        torch.cuda.synchronize()
        assert torch.equal(_bits(spare), ref[r % 2]), f"eager {r}"


def test_kv_cache_write_replays_equal_eager():
    """FP8 cache write of 65536 tokens: each replay rewrites the same records into a cleared cache."""
    T, pages = 65536, 4200
    w = W.cache_write_tokens(DEV, T=T, num_pages=pages, seed=20)
    log(f"[graph] kv write T={T}")
    cache = torch.zeros((pages, 64, W.FP8_RECORD_BYTES), dtype=torch.uint8, device=DEV)
    smla.kv_cache_write(w.tokens, w.slots, cache)
    torch.cuda.synchronize()
    ref = cache.clone()
    g = _capture(lambda: smla.kv_cache_write(w.tokens, w.slots, cache))
    recs = cache.view(-1, W.FP8_RECORD_BYTES)
    ref_recs = ref.view(-1, W.FP8_RECORD_BYTES)
    hit = torch.zeros(recs.shape[0], dtype=torch.bool, device=DEV)
    hit[w.slots] = True
    for r in range(REPLAYS):
        cache.fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(recs[hit], ref_recs[hit]), f"replay {r}: written records"
        assert bool((recs[~hit] == 0xA5).all()), f"replay {r}: other records touched"
        cache2 = torch.zeros_like(cache)
        smla.kv_cache_write(w.tokens, w.slots, cache2)
        torch.cuda.synchronize()
        assert torch.equal(cache2, ref), f"eager {r}"


def test_swa_draft_decode_replays_equal_eager():
    """Decode over 192-wide sliding-window + draft indices (-1 padded; head split over workgroups)."""
    wl = W.decode_bf16(DEV, n_sets=1)
    rs = wl.sets[0]
    B, H = rs.q.shape[0], wl.H
    idx = W.swa_draft_indices(wl.cache.ctx_lens.to(DEV))
    log(f"[graph] swa192 B={B}")
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)

    def call(o, l):
        smla.sparse_mla_decode(rs.q, wl.cache.kv, wl.cache.block_table, idx, wl.scale, row_req=rs.row_req,
                               out=o, lse=l)

    call(out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = _bits(out), _bits(lse)
    g = _capture(lambda: call(out, lse))
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), ref_o) and torch.equal(_bits(lse), ref_l), f"replay {r}"
        o2, l2 = torch.empty_like(out), torch.empty_like(lse)
        call(o2, l2)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o2), ref_o) and torch.equal(_bits(l2), ref_l), f"eager {r}"


def test_prefill_step_replays_equal_eager():
    """Prefill chunk (causal lengths, top-k, prefill attention over several splits), T = 512 rows of
    a 32768-token context."""
    wl = W.prefill_chunk(DEV, T=512, ctx=32768)
    T, H, k = wl.q.shape[0], wl.H, wl.k
    log(f"[graph] prefill T={T} ctx=32768")
    lengths = smla.fill_causal_lengths(wl.first_pos, T, device=DEV)
    bt = wl.cache.block_table[0].contiguous()
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = smla.attention_workspace(T, H, k, DEV)
    tws = smla.topk_workspace(T, k, wl.scores.shape[1], DEV)

    def step():
        smla.fill_causal_lengths(wl.first_pos, T, out=lengths)
        smla.topk_per_row(wl.scores, k, lengths=lengths, out=idx, workspace=tws)
        smla.sparse_mla_prefill_chunk(wl.q, wl.cache.kv, bt, idx, wl.scale, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (_bits(idx), _bits(out), _bits(lse))
    g = _capture(step)
    for r in range(REPLAYS):
        lengths.fill_(-1)
        idx.fill_(-7)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(idx), ref[0]), f"replay {r}: indices"
        assert torch.equal(_bits(out), ref[1]) and torch.equal(_bits(lse), ref[2]), f"replay {r}: attention"
        step()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), ref[1]), f"eager {r}"
