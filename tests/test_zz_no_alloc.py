"""The workspace-free decode entry point (smla_sparse_mla_decode_noalloc, split partials in the
library's static per-GPU scratch array) against smla_sparse_mla_decode with a caller workspace: the
same kernels, so the outputs and LSEs must be identical bit for bit -- on two calls in a row, the
second with a smaller input, and on an FP8 cache."""

import ctypes

import pytest
import torch

import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import bits_equal, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(wl, rs, idx, rows, kv_dtype):
    q = rs.q[:rows].contiguous()
    rq = rs.row_req[:rows].contiguous()
    ix = idx[:rows].contiguous()
    H = q.shape[1]
    ref_out = torch.empty((rows, H, 512), dtype=torch.bfloat16, device=DEV)
    ref_lse = torch.empty((rows, H), dtype=torch.float32, device=DEV)
    smla.sparse_mla_decode(q, wl.cache.kv, wl.cache.block_table, ix, wl.scale, row_req=rq, kv_dtype=kv_dtype,
                           out=ref_out, lse=ref_lse)
    out = torch.full((rows, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((rows, H), float("nan"), dtype=torch.float32, device=DEV)
    smla.sparse_mla_decode_noalloc(q, wl.cache.kv, wl.cache.block_table, ix, wl.scale, out, lse=lse, row_req=rq,
                                   kv_dtype=kv_dtype)
    torch.cuda.synchronize()
    return ref_out, ref_lse, out, lse


def test_noalloc_decode_equals_workspace_decode_two_calls():
    log("[noalloc] B=64 H=64 k=2048 bf16, then 5 rows k=700")
    wl = W.decode_bf16(DEV)
    rs = wl.sets[0]
    idx = smla.topk_per_row(rs.scores, wl.k, lengths=rs.lengths)
    a, al, b, bl = _both(wl, rs, idx, 64, W.KV_BF16)
    assert bits_equal(a, b) and bits_equal(al, bl)
    # second call: a smaller input (fewer rows, another k, so another split count) on the same scratch
    idx2 = smla.topk_per_row(rs.scores, 700, lengths=rs.lengths)
    a, al, b, bl = _both(wl, rs, idx2, 5, W.KV_BF16)
    assert bits_equal(a, b) and bits_equal(al, bl)


def test_noalloc_decode_fp8_and_errors():
    log("[noalloc] FP8 B=8 k=2048")
    wl = W.decode_workload("noalloc_fp8", B=8, H=64, k=2048, ctx_lo=3000, ctx_hi=9000, kv_dtype=W.KV_FP8, seed=41,
                           device=DEV)
    rs = wl.sets[0]
    idx = smla.topk_per_row(rs.scores, wl.k, lengths=rs.lengths)
    a, al, b, bl = _both(wl, rs, idx, 8, W.KV_FP8)
    assert bits_equal(a, b) and bits_equal(al, bl)
    # argument errors are reported before anything is enqueued
    out = torch.empty((8, 64, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(smla.SmlaError):
        smla.sparse_mla_decode_noalloc(rs.q[:, :8].contiguous(), wl.cache.kv, wl.cache.block_table, idx, wl.scale,
                                       out, kv_dtype=W.KV_FP8)
