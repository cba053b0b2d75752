"""GPU parity of smla_paged_mqa_logits (indexer scores) against the oracle.

Scores are compared element by element with the fp64 oracle within a bound derived from the
arithmetic: bf16 products are exact in fp32; the fp32 accumulation over 128 dims, the per-head
fused multiply-adds and the four-way sum each add at most about n * 2^-24 of the magnitudes
involved, so |gpu - oracle| <= 2^-14 * M with M = sum_h |w_h| sum_d |q_hd| |k_pd| (a margin of about
4x over that estimate).  Positions without a score must be -inf exactly.  A hand-worked case is
checked for exact values, a row is checked bit for bit alone and inside a batch, and the scores
feed the top-k selector."""

import json
import os

import numpy as np
import pytest
import torch

import oracle.reference as O
import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import bf16_bits_np, bits_equal, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2.0 ** -14


def _oracle(q, w, kidx, bt, row_req, lengths, stride, rows=None):
    qb, kb = bf16_bits_np(q), bf16_bits_np(kidx)
    wn = w.cpu().numpy()
    btn = bt.cpu().numpy()
    rr = None if row_req is None else row_req.cpu().numpy()
    ln = lengths.cpu().numpy()
    ref = O.indexer_scores(qb, wn, kb, btn, rr, ln, stride, rows=rows)
    mag = O.indexer_error_scale(qb, wn, kb, btn, rr, ln, stride, rows=rows)
    return ref, mag


def _assert_close(got, ref, mag, what):
    got = got.astype(np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf positions differ"
    fin = ~inf_ref
    assert np.all(np.isfinite(got[fin])), f"{what}: non-finite score where one is defined"
    err = np.abs(got[fin] - ref[fin])
    bound = TOL * mag[fin] + 1e-30
    ratio = float((err / bound).max()) if err.size else 0.0
    log(f"{what}: {int(fin.sum())} scores, max err {float(err.max()) if err.size else 0:.3e}, "
        f"max err / bound {ratio:.3e}")
    assert ratio <= 1.0, f"{what}: error above the bound ({ratio:.3f})"


def _workload(Hi, ctx, stride, seed):
    """Rows with the given context lengths (one request each) and an index-key cache for them."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    ctx_t = torch.tensor(ctx, dtype=torch.int64)
    bt, total = W.page_table(ctx_t, g, DEV)
    kidx = W.make_index_cache(bt, ctx_t, total + 1, g, DEV)
    q, w = W.indexer_queries(len(ctx), Hi, g, DEV)
    return q, w, kidx, bt.to(DEV), ctx_t.to(torch.int32).to(DEV)


@pytest.mark.parametrize("Hi", [64, 48, 32, 16])
def test_parity_ragged_rows(Hi):
    ctx = [1, 63, 64, 65, 1000, 4096 + 13, 3000]
    stride = 4096 + 77                      # not a multiple of 64 or of 256
    log(f"indexer parity Hi={Hi} ctx={ctx} stride={stride}")
    q, w, kidx, bt, lengths = _workload(Hi, ctx, stride, seed=10 + Hi)
    out = smla.paged_mqa_logits(q, w, kidx, bt, lengths=lengths, row_req=torch.arange(len(ctx), dtype=torch.int32,
                                                                                          device=DEV),
                                out_stride=stride)
    torch.cuda.synchronize()
    ref, mag = _oracle(q, w, kidx, bt, torch.arange(len(ctx), dtype=torch.int32), lengths, stride)
    _assert_close(out.cpu().numpy(), ref, mag, f"Hi={Hi}")


def test_hand_case_exact(golden_dir):
    """The hand-worked fixture, embedded in 16 heads x 128 dims with zero padding: the scores are
    small integers, so the kernel must give them exactly."""
    with open(os.path.join(golden_dir, "indexer_hand_case.json")) as f:
        case = json.load(f)
    log("indexer hand case on the GPU")
    q = torch.zeros((1, 16, 128), dtype=torch.float32)
    q[0, :2, :4] = torch.tensor(case["q"])
    w = torch.zeros((1, 16), dtype=torch.float32)
    w[0, :2] = torch.tensor(case["w"])
    kidx = torch.zeros((case["num_pages"], 64, 128), dtype=torch.float32)
    for e in case["keys"]:
        kidx[e["page"], e["slot"], :4] = torch.tensor(e["k"])
    q, w, kidx = q.to(torch.bfloat16).to(DEV), w.to(DEV), kidx.to(torch.bfloat16).to(DEV)
    for row in case["rows"]:
        bt = torch.tensor([row["block_table"]], dtype=torch.int32, device=DEV)
        lengths = torch.tensor([row["length"]], dtype=torch.int32, device=DEV)
        out = smla.paged_mqa_logits(q, w, kidx, bt, lengths=lengths, out_stride=row["stride"])
        got = out[0].cpu().numpy()
        for p, v in row["expected"].items():
            assert got[int(p)] == float(v), (row["name"], p, got[int(p)], v)
        L = min(max(row["length"], 0), row["stride"])
        for p in range(L):
            if str(p) not in row["expected"] and row["block_table"][p // 64] >= 0:
                assert got[p] == 0.0, (row["name"], p, got[p])


def test_edge_cases():
    """Lengths 0, negative and past the stride; an invalid request; unlisted and out-of-range
    pages; a stride of 1; NaN keys past a context end never leak into a score."""
    log("indexer edge cases")
    Hi, stride = 32, 700
    ctx = [700, 700, 700, 700, 700, 700]
    q, w, kidx, bt, _ = _workload(Hi, ctx, stride, seed=21)
    bt = bt.clone()
    bt[3, 2] = -1                        # unlisted page: positions 128..191 of row 3
    bt[4, 5] = kidx.shape[0] + 7         # page id past the cache: positions 320..383 of row 4
    lengths = torch.tensor([0, -5, 10 ** 6, 700, 650, 1], dtype=torch.int32, device=DEV)
    row_req = torch.tensor([0, 1, 2, 3, 4, 5], dtype=torch.int32, device=DEV)
    row_req_bad = row_req.clone()
    row_req_bad[5] = 99                  # request outside [0, num_reqs): nothing scored
    for rr in (row_req, row_req_bad):
        out = smla.paged_mqa_logits(q, w, kidx, bt, lengths=lengths, row_req=rr, out_stride=stride)
        torch.cuda.synchronize()
        rrc = rr.cpu().numpy().copy()
        rrc[rrc >= bt.shape[0]] = -1
        # an invalid request scores nothing; the other rows read their own request
        qb, kb = bf16_bits_np(q), bf16_bits_np(kidx)
        wn, btn, ln = w.cpu().numpy(), bt.cpu().numpy(), lengths.cpu().numpy()
        ref = np.full((len(ctx), stride), -np.inf)
        mag = np.zeros((len(ctx), stride))
        for r in range(len(ctx)):
            if rrc[r] < 0:
                continue
            ref[r] = O.indexer_scores(qb, wn, kb, btn, [int(rrc[r])] * len(ctx), ln, stride, rows=[r])[0]
            mag[r] = O.indexer_error_scale(qb, wn, kb, btn, [int(rrc[r])] * len(ctx), ln, stride, rows=[r])[0]
        _assert_close(out.cpu().numpy(), ref, mag, f"edge cases (row_req {rr.tolist()})")
    one = smla.paged_mqa_logits(q[:2], w[:2], kidx, bt, lengths=lengths[:2] * 0 + 1, out_stride=1)
    ref, mag = _oracle(q[:2], w[:2], kidx, bt, None, lengths[:2] * 0 + 1, 1)
    _assert_close(one.cpu().numpy(), ref, mag, "stride 1")
    empty = smla.paged_mqa_logits(q[:0], w[:0], kidx, bt, out_stride=10)
    assert empty.shape == (0, 10)


def test_row_alone_and_in_batch_bitwise():
    log("indexer batch invariance")
    wl = W.indexer_workload("inv", B=24, Hi=64, ctx_lo=500, ctx_hi=9000, seed=23, device=DEV, stride=9100)
    full = smla.paged_mqa_logits(wl.q[0], wl.weights[0], wl.kidx, wl.block_table, lengths=wl.lengths,
                                 row_req=wl.row_req, out_stride=wl.stride)
    for r in (0, 7, 23):
        alone = smla.paged_mqa_logits(wl.q[0][r:r + 1], wl.weights[0][r:r + 1], wl.kidx, wl.block_table,
                                      lengths=wl.lengths[r:r + 1], row_req=wl.row_req[r:r + 1], out_stride=wl.stride)
        assert bits_equal(alone[0], full[r]), r
    # the same rows in another order and with other neighbours
    perm = torch.tensor([5, 23, 0, 7, 7], device=DEV)
    mixed = smla.paged_mqa_logits(wl.q[0][perm], wl.weights[0][perm], wl.kidx, wl.block_table,
                                  lengths=wl.lengths[perm], row_req=wl.row_req[perm], out_stride=wl.stride)
    for i, r in enumerate(perm.tolist()):
        assert bits_equal(mixed[i], full[r]), (i, r)


def test_full_size_sampled_rows_and_tails():
    """The 64-row decode workload with contexts up to 65536 in the launch shape the benchmark times:
    every row's -inf tail and finite scores are checked, and 6 whole rows against the oracle."""
    log("indexer full size B=64 Hi=64 L<=65536")
    wl = W.indexer_decode(DEV)
    out = smla.paged_mqa_logits(wl.q[0], wl.weights[0], wl.kidx, wl.block_table, lengths=wl.lengths,
                                row_req=wl.row_req, out_stride=wl.stride)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    L = wl.ctx_lens.numpy()
    for r in range(got.shape[0]):
        assert np.all(np.isneginf(got[r, L[r]:])), r
        assert np.all(np.isfinite(got[r, :L[r]])), r
    rows = [int(np.argmax(L)), int(np.argmin(L)), 3, 17, 40, 63]
    # a compact copy of the cache holding only the pages these rows use (the indices are remapped;
    # the values are the workload's)
    bt = wl.block_table.cpu()
    used = sorted({int(p) for r in rows for p in bt[r, :(int(L[r]) + 63) // 64].tolist()})
    remap = {p: i for i, p in enumerate(used)}
    sub_k = wl.kidx[torch.tensor(used, device=DEV)]
    sub_bt = torch.zeros((len(rows), bt.shape[1]), dtype=torch.int32)
    for i, r in enumerate(rows):
        n = (int(L[r]) + 63) // 64
        sub_bt[i, :n] = torch.tensor([remap[int(p)] for p in bt[r, :n].tolist()], dtype=torch.int32)
    sel = torch.tensor(rows)
    ref, mag = _oracle(wl.q[0][sel.to(DEV)], wl.weights[0][sel.to(DEV)], sub_k, sub_bt,
                       torch.arange(len(rows), dtype=torch.int32), wl.lengths[sel.to(DEV)], wl.stride)
    _assert_close(got[rows], ref, mag, f"full-size rows {rows}")


def test_scores_feed_the_selector():
    """Indexer scores -> top-k on the GPU: the selection equals the oracle's top-k of the same
    scores bit for bit."""
    log("indexer -> top-k")
    wl = W.indexer_workload("chain", B=8, Hi=64, ctx_lo=3000, ctx_hi=20000, seed=24, device=DEV, stride=20480)
    scores = smla.paged_mqa_logits(wl.q[0], wl.weights[0], wl.kidx, wl.block_table, lengths=wl.lengths,
                                   row_req=wl.row_req, out_stride=wl.stride)
    idx = smla.topk_per_row(scores, 2048, lengths=wl.lengths)
    torch.cuda.synchronize()
    ref = O.topk_rows(scores.cpu().numpy(), wl.lengths.cpu().numpy(), 2048)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


def test_rows_sharing_a_request():
    """Several query rows of one request (MTP-style: each with its own causal length) read the same
    block-table row; each equals the oracle and the same row computed alone."""
    log("indexer rows sharing a request")
    Hi, stride = 64, 2048
    q, w, kidx, bt, _ = _workload(Hi, [2000, 1500], stride, seed=25)
    row_req = torch.tensor([0, 0, 0, 1, 1], dtype=torch.int32, device=DEV)
    lengths = torch.tensor([1997, 1998, 1999, 1400, 1500], dtype=torch.int32, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(26)
    q5, w5 = W.indexer_queries(5, Hi, g, DEV)
    out = smla.paged_mqa_logits(q5, w5, kidx, bt, lengths=lengths, row_req=row_req, out_stride=stride)
    torch.cuda.synchronize()
    ref, mag = _oracle(q5, w5, kidx, bt, row_req, lengths, stride)
    _assert_close(out.cpu().numpy(), ref, mag, "rows sharing a request")
    for r in range(5):
        alone = smla.paged_mqa_logits(q5[r:r + 1], w5[r:r + 1], kidx, bt, lengths=lengths[r:r + 1],
                                      row_req=row_req[r:r + 1], out_stride=stride)
        assert bits_equal(alone[0], out[r]), r
