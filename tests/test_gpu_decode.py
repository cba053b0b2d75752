"""GPU parity of sparse_mla_decode (and the top-k feeding it) against the fp64 oracle, plus
bit-identity of a row alone vs in any batch."""

import numpy as np
import pytest
import torch

import oracle.reference as O
import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import assert_attention_close, bf16_bits_np, bits_equal, kv_np, log, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(wl, rs, idx=None, row_req=None, q=None):
    if idx is None:
        idx = smla.topk_per_row(rs.scores, wl.k, lengths=rs.lengths)
    q = rs.q if q is None else q
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=DEV)
    out, _ = smla.sparse_mla_decode(q, wl.cache.kv, wl.cache.block_table, idx, wl.scale,
                                    row_req=rs.row_req if row_req is None else row_req, lse=lse)
    torch.cuda.synchronize()
    return idx, out, lse


def _oracle_rows(wl, rs, rows, kv_host=None):
    kvh = kv_np(wl.cache.kv) if kv_host is None else kv_host
    return O.decode_rows(bf16_bits_np(rs.q), kvh, wl.cache.kv_dtype, wl.cache.block_table.cpu().numpy(),
                         rs.row_req.cpu().numpy(), rs.scores.cpu().numpy(), rs.lengths.cpu().numpy(), wl.k,
                         wl.scale, rows=rows)


@pytest.fixture(scope="module")
def tiny():
    return W.tiny_decode(DEV)


@pytest.fixture(scope="module")
def big():
    log("[decode] building B=64 H=64 k=2048 bf16 workload")
    wl = W.decode_bf16(DEV)
    return wl, kv_np(wl.cache.kv)


def test_tiny_decode_parity(tiny):
    rs = tiny.sets[0]
    idx, out, lse = _run(tiny, rs)
    ref_idx, O_ref, lse_ref = _oracle_rows(tiny, rs, [0, 1])
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    st = assert_attention_close(out, lse, O_ref, lse_ref, "tiny")
    log(f"[decode] tiny {st}")


def test_full_size_decode_all_rows(big):
    """Every row of the B=64, H=64, k=2048 batch against the oracle: indices bit-exact, attention within
    the stated bounds."""
    wl, kvh = big
    rs = wl.sets[0]
    idx, out, lse = _run(wl, rs)
    rows = list(range(64))
    ref_idx, O_ref, lse_ref = _oracle_rows(wl, rs, rows, kvh)
    assert np.array_equal(idx.cpu().numpy()[rows], ref_idx)
    st = assert_attention_close(out[rows], lse[rows], O_ref, lse_ref, "decode bf16 B64 H64 k2048 (all 64 rows)")
    log(f"[decode] full-size all rows {st}")


def test_full_size_batch_invariance(big):
    """Each row alone, the batch shuffled, and a repeat must reproduce the batch output bit for bit."""
    wl, _ = big
    rs = wl.sets[0]
    idx, out, lse = _run(wl, rs)
    for r in [0, 31, 63]:
        _, o1, l1 = _run(wl, rs, idx=idx[r:r + 1].contiguous(), row_req=rs.row_req[r:r + 1].contiguous(),
                         q=rs.q[r:r + 1].contiguous())
        assert bits_equal(o1[0], out[r]) and bits_equal(l1[0], lse[r]), r
    g = torch.Generator(device=DEV).manual_seed(3)
    perm = torch.randperm(64, generator=g, device=DEV)
    _, o2, l2 = _run(wl, rs, idx=idx[perm].contiguous(), row_req=rs.row_req[perm].contiguous(),
                     q=rs.q[perm].contiguous())
    assert bits_equal(o2, out[perm]) and bits_equal(l2, lse[perm])
    sub = perm[:7]
    _, o3, l3 = _run(wl, rs, idx=idx[sub].contiguous(), row_req=rs.row_req[sub].contiguous(),
                     q=rs.q[sub].contiguous())
    assert bits_equal(o3, out[sub]) and bits_equal(l3, lse[sub])
    for _ in range(3):
        _, o4, l4 = _run(wl, rs, idx=idx)
        assert bits_equal(o4, out) and bits_equal(l4, lse)


@pytest.mark.parametrize("H,k", [(16, 1), (16, 192), (32, 700), (48, 513), (64, 1024), (128, 2048), (64, 2500)])
def test_heads_and_widths(H, k):
    """Head counts 16..128 (two head blocks at 128) and widths that leave ragged tiles and splits."""
    wl = W.decode_workload(f"hk_{H}_{k}", B=5, H=H, k=k, ctx_lo=max(1, k // 2), ctx_hi=3 * k + 70,
                           kv_dtype=W.KV_BF16, seed=100 + H + k, device=DEV, score_kind="eighths")
    rs = wl.sets[0]
    idx, out, lse = _run(wl, rs)
    ref_idx, O_ref, lse_ref = _oracle_rows(wl, rs, list(range(5)))
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    st = assert_attention_close(out, lse, O_ref, lse_ref, f"H={H} k={k}")
    log(f"[decode] H={H} k={k} {st}")


def test_short_empty_and_invalid_slots():
    """Rows with fewer candidates than k (-1 tail), an empty row, -1 holes in the middle, positions
    past the block table, a bad request id: invalid slots contribute nothing; empty rows give 0/-inf."""
    wl = W.decode_workload("edge", B=6, H=64, k=1024, ctx_lo=100, ctx_hi=3000, kv_dtype=W.KV_BF16, seed=77,
                           device=DEV)
    rs = wl.sets[0]
    lens = rs.lengths.clone()
    lens[0] = 0            # empty row
    lens[1] = 37           # far fewer than k
    lens[2] = 1000         # just under k
    idx = smla.topk_per_row(rs.scores, wl.k, lengths=lens)
    idx_h = idx.cpu().numpy().copy()
    idx_h[3, 5:400:3] = -1                               # holes
    idx_h[4, 10] = 10 ** 7                               # past the block table -> skipped
    idx = torch.from_numpy(idx_h).to(DEV)
    row_req = rs.row_req.clone()
    row_req[5] = 999                                     # no such request -> empty row
    _, out, lse = _run(wl, rs, idx=idx, row_req=row_req)
    kvh = kv_np(wl.cache.kv)
    bt = wl.cache.block_table.cpu().numpy()
    idx_o = idx_h.copy()
    idx_o[4, 10] = -1
    idx_o[5, :] = -1
    req = row_req.cpu().numpy().copy()
    req[5] = 0
    O_ref, lse_ref = O.attention_rows(bf16_bits_np(rs.q), kvh, W.KV_BF16, bt, req, idx_o, wl.scale)
    st = assert_attention_close(out, lse, O_ref, lse_ref, "edge rows")
    assert (out[0].float() == 0).all() and torch.isneginf(lse[0]).all()
    assert (out[5].float() == 0).all() and torch.isneginf(lse[5]).all()
    log(f"[decode] edge {st}")


def test_poisoned_pages_never_read():
    """The cache's null page and the slots past each context are NaN; every output stays finite."""
    wl = W.decode_workload("poison", B=8, H=32, k=256, ctx_lo=65, ctx_hi=700, kv_dtype=W.KV_BF16, seed=5,
                           device=DEV)
    rs = wl.sets[0]
    _, out, lse = _run(wl, rs)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_head_split_invariance(big):
    """Launches with few (row, split) items split the heads over 2 or 4 workgroups; a head's result must
    not depend on that.  k = 256 (one split): 320 rows run 64 heads per workgroup, 128 rows 32, 64 rows
    and a single row 16 -- the shared rows must agree bit for bit."""
    wl, _ = big
    rs = wl.sets[0]
    k = 256
    idx = smla.topk_per_row(rs.scores, k, lengths=rs.lengths)
    rep = lambda t, n: t.repeat((n,) + (1,) * (t.dim() - 1))[: 64 * n].contiguous()
    outs = {}
    for n_rep in (5, 2, 1):
        _, o, l = _run(wl, rs, idx=rep(idx, n_rep), row_req=rep(rs.row_req, n_rep), q=rep(rs.q, n_rep))
        outs[n_rep] = (o[:64], l[:64])
    for n_rep in (2, 1):
        assert bits_equal(outs[n_rep][0], outs[5][0]) and bits_equal(outs[n_rep][1], outs[5][1]), n_rep
    _, o1, l1 = _run(wl, rs, idx=idx[9:10].contiguous(), row_req=rs.row_req[9:10].contiguous(),
                     q=rs.q[9:10].contiguous())
    assert bits_equal(o1[0], outs[5][0][9]) and bits_equal(l1[0], outs[5][1][9])


@pytest.mark.parametrize("k,with_sink", [(2048, True), (2048, False), (1024, True)])
def test_ragged_rows_in_multi_split_workgroups(k, with_sink):
    """320 rows x 64 heads is a launch large enough that each workgroup runs all 64 heads of several
    consecutive splits of its row; a batch of 7 rows runs one split of 16 heads per workgroup.  The
    shared rows -- an empty row, rows whose later splits have few or no valid slots (a split followed
    by one without tiles), a row with no valid slot at all -- must agree bit for bit, sink or not, and
    match the oracle."""
    B = 320
    wl = W.decode_workload(f"merge_{k}", B=B, H=64, k=k, ctx_lo=1, ctx_hi=2 * k + 100, kv_dtype=W.KV_BF16,
                           seed=500 + k, device=DEV)
    rs = wl.sets[0]
    lens = rs.lengths.clone()
    lens[5] = 0           # empty row
    lens[6] = 300         # splits 1.. empty
    lens[7] = min(513, int(rs.lengths[7]))
    idx = smla.topk_per_row(rs.scores, k, lengths=lens)
    idx[8] = -1           # no valid slot in any split
    if with_sink:
        g = torch.Generator(device="cpu").manual_seed(k)
        sink = torch.randn(64, generator=g) * 3.0 + 2.0
        sink[1::5] = -float("inf")
        sink = sink.to(DEV)
    else:
        sink = None

    def run(rows):
        lse = torch.empty((len(rows), 64), dtype=torch.float32, device=DEV)
        out, _ = smla.sparse_mla_decode(rs.q[rows].contiguous(), wl.cache.kv, wl.cache.block_table,
                                        idx[rows].contiguous(), wl.scale, row_req=rs.row_req[rows].contiguous(),
                                        lse=lse, sink=sink)
        torch.cuda.synchronize()
        return out, lse

    out, lse = run(list(range(B)))
    rows = [0, 5, 6, 7, 8, 100, 319]
    o1, l1 = run(rows)
    assert bits_equal(o1, out[rows]) and bits_equal(l1, lse[rows])
    O_ref, lse_ref = O.attention_rows(bf16_bits_np(rs.q[rows]), kv_np(wl.cache.kv), W.KV_BF16,
                                      wl.cache.block_table.cpu().numpy(), rs.row_req.cpu().numpy()[rows],
                                      idx.cpu().numpy()[rows], wl.scale,
                                      sink=None if sink is None else sink.cpu().numpy().astype(np.float64))
    st = assert_attention_close(out[rows], lse[rows], O_ref, lse_ref, f"ragged rows, multi-split workgroups k={k} sink={with_sink}")
    log(f"[decode] ragged rows in multi-split workgroups k={k} sink={with_sink} {st}")


def test_maximum_k_and_many_splits():
    """k = 16384, the largest supported width: 32 splits, combined in order by the split-combine kernel
    in several groups of loads."""
    k = 16384
    wl = W.decode_workload("maxk", B=3, H=16, k=k, ctx_lo=k, ctx_hi=k + 3000, kv_dtype=W.KV_BF16, seed=88,
                           device=DEV)
    rs = wl.sets[0]
    idx, out, lse = _run(wl, rs)
    ref_idx, O_ref, lse_ref = _oracle_rows(wl, rs, [0, 1, 2])
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    st = assert_attention_close(out, lse, O_ref, lse_ref, "k=16384")
    log(f"[decode] k=16384 {st}")


def test_workspace_smaller_than_the_batch():
    """A workspace that holds 2 rows: the call runs 4 launches of at most 2 rows; every row must equal
    its value from one launch with a workspace for all 7 rows."""
    wl = W.decode_workload("ws", B=7, H=64, k=1500, ctx_lo=1600, ctx_hi=5000, kv_dtype=W.KV_BF16, seed=99,
                           device=DEV)
    rs = wl.sets[0]
    idx, out, lse = _run(wl, rs)
    _, per_row = smla.workspace_size(smla.Capacity.make(1, 1500, 64, 1))
    small = torch.zeros(2 * per_row, dtype=torch.uint8, device=DEV)
    lse2 = torch.empty_like(lse)
    out2, _ = smla.sparse_mla_decode(rs.q, wl.cache.kv, wl.cache.block_table, idx, wl.scale, row_req=rs.row_req,
                                     lse=lse2, workspace=small)
    torch.cuda.synchronize()
    assert bits_equal(out, out2) and bits_equal(lse, lse2)
    ref_idx, O_ref, lse_ref = _oracle_rows(wl, rs, list(range(7)))
    assert_attention_close(out2, lse2, O_ref, lse_ref, "small workspace")
