"""GPU parity of smla_sparse_mla_decode_with_window (decode over compressed and sliding-window KV in
one softmax) against the oracle, bit-identity of a row alone vs in a batch, empty window lists, and the
width check."""

import types

import numpy as np
import pytest
import torch

import oracle.reference as O
import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import assert_attention_close, bf16_bits_np, bits_equal, kv_np, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _call(wl, rs, idx, win, q=None, row_req=None, idx_win=None, sink=None):
    q = rs.q if q is None else q
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=DEV)
    out, _ = smla.sparse_mla_decode_with_window(q, wl.cache.kv, wl.cache.block_table, idx, win.kv, win.block_table,
                                                win.idx if idx_win is None else idx_win, wl.scale,
                                                row_req=rs.row_req if row_req is None else row_req,
                                                kv_dtype=wl.cache.kv_dtype, lse=lse, sink=sink)
    torch.cuda.synchronize()
    return out, lse


def _oracle(wl, rs, idx, win, rows, sink=None):
    return O.attention_rows_with_window(bf16_bits_np(rs.q), kv_np(wl.cache.kv), wl.cache.kv_dtype,
                                        wl.cache.block_table.cpu().numpy(), idx.cpu().numpy(), kv_np(win.kv),
                                        win.block_table.cpu().numpy(), win.idx.cpu().numpy(),
                                        rs.row_req.cpu().numpy(), wl.scale, rows=rows,
                                        sink=None if sink is None else sink.cpu().numpy().astype(np.float64))


@pytest.fixture(scope="module")
def big():
    log("[window] B=64 H=64 top-k 2048 + window 128 + draft 5 (width 192), bf16")
    wl = W.decode_bf16(DEV)
    win = W.window_cache(wl.cache.ctx_lens, W.KV_BF16, DEV, seed=61,
                         max_pages=int(wl.cache.block_table.shape[1]))
    rs = wl.sets[0]
    idx = smla.topk_per_row(rs.scores, wl.k, lengths=rs.lengths)
    return wl, win, rs, idx


def test_window_decode_all_rows(big):
    wl, win, rs, idx = big
    out, lse = _call(wl, rs, idx, win)
    O_ref, lse_ref = _oracle(wl, rs, idx, win, list(range(64)))
    st = assert_attention_close(out, lse, O_ref, lse_ref, "decode bf16 top-k 2048 + window 192 (all 64 rows)")
    log(f"[window] all rows {st}")


def test_window_decode_batch_invariance_and_empty_window(big):
    wl, win, rs, idx = big
    out, lse = _call(wl, rs, idx, win)
    for r in [0, 17, 63]:
        o1, l1 = _call(wl, rs, idx[r:r + 1].contiguous(), win, q=rs.q[r:r + 1].contiguous(),
                       row_req=rs.row_req[r:r + 1].contiguous(), idx_win=win.idx[r:r + 1].contiguous())
        assert bits_equal(o1[0], out[r]) and bits_equal(l1[0], lse[r]), r
    # empty window lists: the attention over the main selection alone (the units are still stretched
    # to the k + k_win slots, so the grouping differs from the plain decode's: compared with the oracle)
    none = torch.full_like(win.idx, -1)
    o2, l2 = _call(wl, rs, idx, win, idx_win=none)
    rows = [0, 1, 2, 3]
    O_ref, lse_ref = O.attention_rows(bf16_bits_np(rs.q), kv_np(wl.cache.kv), W.KV_BF16,
                                      wl.cache.block_table.cpu().numpy(), rs.row_req.cpu().numpy(), idx.cpu().numpy(),
                                      wl.scale, rows=rows)
    assert_attention_close(o2[rows], l2[rows], O_ref, lse_ref, "window decode with empty window lists")


@pytest.mark.parametrize("k,k_win,ctx_lo,ctx_hi", [(512, 64, 100, 700), (700, 192, 20, 3000), (2048, 256, 5000, 9000)])
def test_window_decode_shapes(k, k_win, ctx_lo, ctx_hi):
    """Short contexts (fewer than 133 window positions, empty top-k tails), k not a multiple of the
    tile, a window wider than the valid entries."""
    wl = W.decode_workload("win_shapes", B=6, H=32, k=k, ctx_lo=ctx_lo, ctx_hi=ctx_hi, kv_dtype=W.KV_BF16, seed=62,
                           device=DEV)
    win = W.window_cache(wl.cache.ctx_lens, W.KV_BF16, DEV, seed=63, width=k_win,
                         draft=5 if k_win >= 192 else 3, window=128 if k_win >= 192 else 40,
                         max_pages=int(wl.cache.block_table.shape[1]))
    rs = wl.sets[0]
    idx = smla.topk_per_row(rs.scores, k, lengths=rs.lengths)
    out, lse = _call(wl, rs, idx, win)
    O_ref, lse_ref = _oracle(wl, rs, idx, win, list(range(6)))
    st = assert_attention_close(out, lse, O_ref, lse_ref, f"window decode k={k} k_win={k_win}")
    log(f"[window] k={k} k_win={k_win} {st}")


def test_window_decode_fp8():
    wl = W.decode_workload("win_fp8", B=8, H=64, k=2048, ctx_lo=3000, ctx_hi=9000, kv_dtype=W.KV_FP8, seed=64,
                           device=DEV)
    win = W.window_cache(wl.cache.ctx_lens, W.KV_FP8, DEV, seed=65, max_pages=int(wl.cache.block_table.shape[1]))
    rs = wl.sets[0]
    idx = smla.topk_per_row(rs.scores, wl.k, lengths=rs.lengths)
    out, lse = _call(wl, rs, idx, win)
    O_ref, lse_ref = _oracle(wl, rs, idx, win, list(range(8)))
    st = assert_attention_close(out, lse, O_ref, lse_ref, "window decode fp8 k=2048 k_win=192", relative=True)
    log(f"[window] fp8 {st}")


@pytest.mark.parametrize("k,kv_dtype", [(700, W.KV_BF16), (2048, W.KV_BF16), (2048, W.KV_FP8)])
def test_window_decode_with_sink(k, kv_dtype):
    """Per-head sink logits (some -inf) with the window part: one split (k=700, width 192 in one unit per
    split) and several (k=2048), bf16 and FP8 caches; a row alone equals the row in the batch."""
    wl = W.decode_workload(f"win_sink_{k}_{kv_dtype}", B=6, H=64, k=k, ctx_lo=50, ctx_hi=3 * k, kv_dtype=kv_dtype,
                           seed=80 + k + kv_dtype, device=DEV)
    win = W.window_cache(wl.cache.ctx_lens, kv_dtype, DEV, seed=81 + k, max_pages=int(wl.cache.block_table.shape[1]))
    rs = wl.sets[0]
    g = torch.Generator(device="cpu").manual_seed(k + kv_dtype)
    sink = torch.randn(64, generator=g) * 3.0 + 2.0
    sink[2::7] = -float("inf")
    sink = sink.to(DEV)
    idx = smla.topk_per_row(rs.scores, wl.k, lengths=rs.lengths)
    out, lse = _call(wl, rs, idx, win, sink=sink)
    O_ref, lse_ref = _oracle(wl, rs, idx, win, list(range(6)), sink=sink)
    st = assert_attention_close(out, lse, O_ref, lse_ref, f"window decode + sink k={k} kv={kv_dtype}",
                                relative=kv_dtype == W.KV_FP8)
    one = types.SimpleNamespace(kv=win.kv, block_table=win.block_table, idx=win.idx[2:3].contiguous())
    o1, l1 = _call(wl, rs, idx[2:3].contiguous(), one, q=rs.q[2:3].contiguous(), row_req=rs.row_req[2:3].contiguous(),
                   sink=sink)
    assert bits_equal(o1[0], out[2]) and bits_equal(l1[0], lse[2])
    log(f"[window] sink k={k} kv={kv_dtype} {st}")


def test_window_decode_rejects_unpadded_width(big):
    wl, win, rs, idx = big
    with pytest.raises(smla.SmlaError):
        _call(wl, rs, idx, win, idx_win=win.idx[:, :133].contiguous())
