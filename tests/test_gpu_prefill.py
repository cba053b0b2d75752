"""Prefill chunk (4096 query tokens at positions 126976..131071 of a 131072-token context, causal)
against the oracle on sampled rows, and bit-identity of those rows inside a mixed batch with 63
decode rows."""

import numpy as np
import pytest
import torch

import oracle.reference as O
import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import assert_attention_close, bf16_bits_np, bits_equal, kv_np, log, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def pf():
    log("[prefill] building T=4096 ctx=131072 workload")
    wl = W.prefill_chunk(DEV)
    T = wl.q.shape[0]
    lengths = smla.fill_causal_lengths(wl.first_pos, T, device=DEV)
    idx = smla.topk_per_row(wl.scores, wl.k, lengths=lengths)
    lse = torch.empty((T, wl.H), dtype=torch.float32, device=DEV)
    out, _ = smla.sparse_mla_prefill_chunk(wl.q, wl.cache.kv, wl.cache.block_table[0].contiguous(), idx, wl.scale,
                                           lse=lse)
    torch.cuda.synchronize()
    return wl, lengths, idx, out, lse


def test_causal_lengths(pf):
    wl, lengths, _, _, _ = pf
    assert np.array_equal(lengths.cpu().numpy(), O.causal_lengths(wl.first_pos, wl.q.shape[0]))


def test_prefill_sampled_rows_match_oracle(pf):
    """256 seeded rows of the 4096 (plus the first and the last) against the oracle."""
    wl, lengths, idx, out, lse = pf
    T = wl.q.shape[0]
    rows = sorted(set(sample_rows(T, 256, 4) + [0, T - 1]))
    scores_rows = wl.scores[rows].cpu().numpy()
    ref_idx = O.topk_rows(scores_rows, lengths.cpu().numpy()[rows], wl.k)
    assert np.array_equal(idx.cpu().numpy()[rows], ref_idx)
    kvh = kv_np(wl.cache.kv)
    O_ref, lse_ref = O.attention_rows(bf16_bits_np(wl.q[rows]), kvh, W.KV_BF16, wl.cache.block_table.cpu().numpy(),
                                      [0] * len(rows), ref_idx, wl.scale)
    st = assert_attention_close(out[rows], lse[rows], O_ref, lse_ref, f"prefill T=4096 ({len(rows)} seeded rows)")
    log(f"[prefill] {len(rows)} seeded rows {st}")


def test_mixed_batch_bit_identical(pf):
    """The prefill rows, rerun inside one batch with 63 decode rows at random positions (top-k and
    attention both), give the same bits as the prefill-only run; the decode rows give the same bits
    as a decode-only run."""
    wl, lengths, idx, out, lse = pf
    T = wl.q.shape[0]
    dec = wl.decode
    n_dec = dec.q.shape[0]
    stride = wl.scores.shape[1]
    # one score buffer holding the prefill rows followed by the decode rows
    buf = torch.full((T + n_dec, stride), float("inf"), dtype=torch.float32, device=DEV)
    buf[:T] = wl.scores
    buf[T:, :dec.scores.shape[1]] = dec.scores
    order = wl.mix_order.to(DEV)                        # mixed slot -> source row
    offs = order.to(torch.int64) * stride
    all_len = torch.cat([lengths, dec.lengths])
    mlen = all_len[order].contiguous()
    midx = smla.topk_per_row(buf, wl.k, lengths=mlen, row_offsets=offs, row_stride=stride)
    all_q = torch.cat([wl.q, dec.q])
    mq = all_q[order].contiguous()
    all_req = torch.cat([torch.zeros(T, dtype=torch.int32, device=DEV), dec.row_req])
    mreq = all_req[order].contiguous()
    mlse = torch.empty((T + n_dec, wl.H), dtype=torch.float32, device=DEV)
    mout, _ = smla.sparse_mla_decode(mq, wl.cache.kv, wl.cache.block_table, midx, wl.scale, row_req=mreq, lse=mlse)
    # decode-only reference run
    didx = smla.topk_per_row(dec.scores, wl.k, lengths=dec.lengths)
    dlse = torch.empty((n_dec, wl.H), dtype=torch.float32, device=DEV)
    dout, _ = smla.sparse_mla_decode(dec.q, wl.cache.kv, wl.cache.block_table, didx, wl.scale, row_req=dec.row_req,
                                     lse=dlse)
    torch.cuda.synchronize()
    is_pf = order < T
    src = order.clone()
    pf_slots = torch.nonzero(is_pf).flatten()
    dec_slots = torch.nonzero(~is_pf).flatten()
    assert torch.equal(midx[pf_slots], idx[src[pf_slots]])
    assert torch.equal(midx[dec_slots], didx[src[dec_slots] - T])
    assert bits_equal(mout[pf_slots], out[src[pf_slots]])
    assert bits_equal(mlse[pf_slots], lse[src[pf_slots]])
    assert bits_equal(mout[dec_slots], dout[src[dec_slots] - T])
    assert bits_equal(mlse[dec_slots], dlse[src[dec_slots] - T])
    log(f"[prefill] mixed batch of {T + n_dec} rows bit-identical")


def test_prefill_from_position_zero():
    """A chunk of 3072 query tokens at positions 0..3071 of a new sequence (causal: row t has t + 1
    candidates, so the rows below 2048 fill only their first splits and leave the rest without
    tiles): the large launch, whose workgroups run all heads of consecutive splits of a row, against
    the oracle on seeded rows, and bit for bit against the same rows in a launch of 10 rows."""
    T = 3072
    wl = W.prefill_chunk(DEV, seed=41, T=T, ctx=T, n_dec=1, dec_lo=64, dec_hi=64)
    lengths = smla.fill_causal_lengths(wl.first_pos, T, device=DEV)
    idx = smla.topk_per_row(wl.scores, wl.k, lengths=lengths)
    bt = wl.cache.block_table[0].contiguous()
    lse = torch.empty((T, wl.H), dtype=torch.float32, device=DEV)
    out, _ = smla.sparse_mla_prefill_chunk(wl.q, wl.cache.kv, bt, idx, wl.scale, lse=lse)
    rows = [0, 1, 63, 511, 512, 700, 1500, 2047, 2048, 3071]
    lse1 = torch.empty((len(rows), wl.H), dtype=torch.float32, device=DEV)
    o1, _ = smla.sparse_mla_prefill_chunk(wl.q[rows].contiguous(), wl.cache.kv, bt, idx[rows].contiguous(), wl.scale,
                                          lse=lse1)
    torch.cuda.synchronize()
    assert bits_equal(o1, out[rows]) and bits_equal(lse1, lse[rows])
    ref_idx = O.topk_rows(wl.scores[rows].cpu().numpy(), lengths.cpu().numpy()[rows], wl.k)
    assert np.array_equal(idx.cpu().numpy()[rows], ref_idx)
    O_ref, lse_ref = O.attention_rows(bf16_bits_np(wl.q[rows]), kv_np(wl.cache.kv), W.KV_BF16,
                                      wl.cache.block_table.cpu().numpy(), [0] * len(rows), ref_idx, wl.scale)
    st = assert_attention_close(out[rows], lse[rows], O_ref, lse_ref, f"prefill from position 0 ({len(rows)} rows)")
    log(f"[prefill] from position 0: {st}")


def test_prefill_fp8_cache_with_sink():
    """A prefill chunk over an FP8 cache with per-head sink logits (some -inf): 1024 rows at positions
    3072..4095 of a 4096-token context, k=2048 (several FP8 splits).  Seeded rows against the oracle, and
    every row bit-identical to the same rows run as a decode batch of the one request."""
    T, ctx, k, H = 1024, 4096, 2048, 64
    g = torch.Generator(device=DEV).manual_seed(91)
    cache = W.make_paged_cache(torch.tensor([ctx]), W.KV_FP8, g, DEV)
    q = torch.randn((T, H, 576), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    scores = torch.randn((T, ctx), generator=g, device=DEV, dtype=torch.float32)
    gs = torch.Generator(device="cpu").manual_seed(92)
    sink = torch.randn(H, generator=gs) * 3.0 + 2.0
    sink[3::6] = -float("inf")
    sink = sink.to(DEV)
    lengths = smla.fill_causal_lengths(ctx - T, T, device=DEV)
    idx = smla.topk_per_row(scores, k, lengths=lengths)
    bt = cache.block_table[0].contiguous()
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    out, _ = smla.sparse_mla_prefill_chunk(q, cache.kv, bt, idx, W.SOFTMAX_SCALE, kv_dtype=W.KV_FP8, lse=lse,
                                           sink=sink)
    lse2 = torch.empty_like(lse)
    out2, _ = smla.sparse_mla_decode(q, cache.kv, cache.block_table, idx, W.SOFTMAX_SCALE, kv_dtype=W.KV_FP8,
                                     lse=lse2, sink=sink)
    torch.cuda.synchronize()
    assert bits_equal(out, out2) and bits_equal(lse, lse2)
    rows = sorted(set(sample_rows(T, 24, 93) + [0, T - 1]))
    O_ref, lse_ref = O.attention_rows(bf16_bits_np(q[rows]), kv_np(cache.kv), W.KV_FP8, cache.block_table.cpu().numpy(),
                                      [0] * len(rows), idx.cpu().numpy()[rows], W.SOFTMAX_SCALE,
                                      sink=sink.cpu().numpy().astype(np.float64))
    st = assert_attention_close(out[rows], lse[rows], O_ref, lse_ref, f"prefill fp8 + sink ({len(rows)} rows)",
                                relative=True)
    log(f"[prefill] fp8 + sink: {st}")
