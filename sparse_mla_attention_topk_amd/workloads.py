"""Seeded synthetic inputs for the sparse-MLA decode / prefill path.

This module only draws random numbers and lays them out in the buffers the
library consumes.  It holds none of the method's arithmetic: no top-k, no
gather, no softmax.  Both the CPU oracle (under ``oracle/``) and the HIP path
consume the same bytes produced here.

Layouts (all row-major, contiguous):

* ``kv`` bf16 cache: ``uint16 [num_pages, 64, 576]`` (bf16 bit patterns); one
  token record is 576 bf16 = 1152 B: 512 latent values followed by 64 rope
  values.
* ``kv`` FP8 cache: ``uint8 [num_pages, 64, 656]``; one token record is
  ``[512 B e4m3 codes | 4 x fp32 group scales | 64 x bf16 rope]``.
* ``block_table`` ``int32 [num_requests, max_pages]``: logical page ``p`` of
  request ``r`` lives in physical page ``block_table[r, p]``.  Unused entries
  are 0, the null page.
* Physical page 0 is the null page and is filled with NaN.  Slots at or past a
  request's length inside its last page are NaN as well, so any read that is
  not asked for shows up as NaN in an output.
* ``scores`` ``float32 [rows, stride]``: entries at or past a row's candidate
  count are +inf, so a selector that looks past the length picks them.

Random draws are made with ``torch.Generator`` on the requested device, so the
same seed gives the same bytes on every run on that device kind.  Draw order
for a decode workload: context lengths, physical page permutation, scores, Q,
KV (latent/codes, then scales, then rope for FP8).
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

PAGE = 64
D_QK = 576
D_V = 512
D_ROPE = 64
BF16_RECORD_BYTES = D_QK * 2
FP8_RECORD_BYTES = 512 + 4 * 4 + D_ROPE * 2  # 656
KV_BF16 = 0
KV_FP8 = 1

BF16_NAN_BITS = 0x7FC0
FP8_NAN_CODE = 0x7F


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


@dataclasses.dataclass
class PagedCache:
    kv: torch.Tensor            # uint8 bytes [num_pages, 64, record_bytes]
    kv_dtype: int               # KV_BF16 or KV_FP8
    block_table: torch.Tensor   # int32 [num_requests, max_pages]
    ctx_lens: torch.Tensor      # int64 [num_requests]

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def record_bytes(self) -> int:
        return int(self.kv.shape[2])


@dataclasses.dataclass
class RowSet:
    """One batch of query rows against a paged cache."""
    q: torch.Tensor             # bf16 [rows, H, 576]
    scores: torch.Tensor        # fp32 [rows, stride]
    lengths: torch.Tensor       # int32 [rows]  candidate count per row
    row_req: torch.Tensor       # int32 [rows]  request each row reads


def uniform_int(lo: int, hi: int, n: int, g: torch.Generator, device) -> torch.Tensor:
    """n integers drawn uniformly from the inclusive range [lo, hi]."""
    return torch.randint(lo, hi + 1, (n,), generator=g, device=device, dtype=torch.int64)


def page_table(ctx_lens: torch.Tensor, g: torch.Generator, device):
    """Block table (CPU int32 [requests, max_pages]) that hands out physical pages 1..N through a
    seeded random permutation, and N.  Unused entries are 0 (the null page)."""
    npages = [int(math.ceil(int(L) / PAGE)) for L in ctx_lens]
    total = sum(npages)
    max_pages = max(1, max(npages) if npages else 1)
    perm = torch.randperm(total, generator=g, device=device).cpu() + 1
    bt = torch.zeros((len(npages), max_pages), dtype=torch.int32)
    off = 0
    for r, n in enumerate(npages):
        bt[r, :n] = perm[off:off + n].to(torch.int32)
        off += n
    return bt, total


def make_paged_cache(ctx_lens: torch.Tensor, kv_dtype: int, g: torch.Generator, device,
                     chunk_pages: int = 4096, fp8_scale_log2=(-4.0, 4.0)) -> PagedCache:
    """Allocate a paged cache holding one context per entry of ``ctx_lens``.

    Physical pages 1..N are handed out through a seeded random permutation;
    page 0 is the NaN null page.  Values: bf16 N(0,1) for the bf16 cache; for
    the FP8 cache, e4m3 codes of N(0,1) (round to nearest even), fp32 scales
    2**U(lo, hi) per (token, 128-group) with (lo, hi) = ``fp8_scale_log2``
    (default (-4, 4)) and bf16 N(0,1) rope.
    """
    ctx_lens = ctx_lens.to(torch.int64).cpu()
    bt, total = page_table(ctx_lens, g, device)
    rec = BF16_RECORD_BYTES if kv_dtype == KV_BF16 else FP8_RECORD_BYTES
    kv = torch.empty((total + 1, PAGE, rec), dtype=torch.uint8, device=device)
    # Fill physical pages in chunks so the fp32 intermediates stay small.
    for p0 in range(1, total + 1, chunk_pages):
        p1 = min(total + 1, p0 + chunk_pages)
        ntok = (p1 - p0) * PAGE
        if kv_dtype == KV_BF16:
            vals = torch.randn((ntok, D_QK), generator=g, device=device, dtype=torch.float32)
            kv[p0:p1] = vals.to(torch.bfloat16).view(torch.uint8).view(p1 - p0, PAGE, rec)
        else:
            lat = torch.randn((ntok, 512), generator=g, device=device, dtype=torch.float32)
            codes = lat.to(torch.float8_e4m3fn).view(torch.uint8)
            lo, hi = fp8_scale_log2
            expo = torch.rand((ntok, 4), generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo
            scales = torch.exp2(expo).contiguous().view(torch.uint8).view(ntok, 16)
            rope = torch.randn((ntok, D_ROPE), generator=g, device=device, dtype=torch.float32)
            rope_b = rope.to(torch.bfloat16).view(torch.uint8).view(ntok, 128)
            kv[p0:p1] = torch.cat([codes, scales, rope_b], dim=1).view(p1 - p0, PAGE, rec)
    poison_cache(kv, bt, ctx_lens, kv_dtype)
    return PagedCache(kv=kv, kv_dtype=kv_dtype, block_table=bt.to(device), ctx_lens=ctx_lens)


def _poison_record(kv_dtype: int, device) -> torch.Tensor:
    if kv_dtype == KV_BF16:
        return torch.full((D_QK,), BF16_NAN_BITS, dtype=torch.int16, device=device).view(torch.uint8)
    codes = torch.full((512,), FP8_NAN_CODE, dtype=torch.uint8, device=device)
    scales = torch.full((4,), float("nan"), dtype=torch.float32, device=device).view(torch.uint8)
    rope = torch.full((D_ROPE,), BF16_NAN_BITS, dtype=torch.int16, device=device).view(torch.uint8)
    return torch.cat([codes, scales, rope])


def poison_cache(kv: torch.Tensor, bt_cpu: torch.Tensor, ctx_lens, kv_dtype: int) -> None:
    """NaN-fill the null page and every slot past a context's end in its last page."""
    rec = _poison_record(kv_dtype, kv.device)
    kv[0] = rec
    for r, L in enumerate(ctx_lens):
        L = int(L)
        if L % PAGE:
            last = int(bt_cpu[r, L // PAGE])
            kv[last, L % PAGE:] = rec


def _scores_block(rows: int, stride: int, g, device, kind: str) -> torch.Tensor:
    if kind == "normal":
        return torch.randn((rows, stride), generator=g, device=device, dtype=torch.float32)
    if kind == "eighths":  # N(0,1) rounded to multiples of 1/8: forces ties and produces -0.0
        return torch.round(torch.randn((rows, stride), generator=g, device=device,
                                       dtype=torch.float32) * 8.0) / 8.0
    raise ValueError(kind)


def poison_score_tails(scores: torch.Tensor, lengths: torch.Tensor) -> None:
    """Set scores at or past each row's candidate count to +inf."""
    stride = scores.shape[1]
    pos = torch.arange(stride, device=scores.device).unsqueeze(0)
    mask = pos >= lengths.to(scores.device).to(torch.int64).clamp(min=0).unsqueeze(1)
    scores.masked_fill_(mask, float("inf"))


def make_rowset(cache: PagedCache, row_req: torch.Tensor, lengths: torch.Tensor, H: int, stride: int,
                g: torch.Generator, device, score_kind: str = "normal") -> RowSet:
    rows = int(row_req.numel())
    scores = _scores_block(rows, stride, g, device, score_kind)
    poison_score_tails(scores, lengths)
    q = torch.randn((rows, H, D_QK), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return RowSet(q=q, scores=scores, lengths=lengths.to(torch.int32).to(device),
                  row_req=row_req.to(torch.int32).to(device))


# --------------------------------------------------------------------------------------------
# Named workloads.  Sizes follow the decode / top-k / prefill shapes the method is run at.
# --------------------------------------------------------------------------------------------

SOFTMAX_SCALE = 1.0 / math.sqrt(D_QK)


@dataclasses.dataclass
class DecodeWorkload:
    name: str
    cache: PagedCache
    sets: List[RowSet]
    H: int
    k: int
    scale: float
    stride: int


def decode_workload(name: str, B: int, H: int, k: int, ctx_lo: int, ctx_hi: int, kv_dtype: int,
                    seed: int, device, n_sets: int = 1, score_kind: str = "normal",
                    stride: Optional[int] = None, fp8_scale_log2=(-4.0, 4.0)) -> DecodeWorkload:
    """B decode rows, one request each, context lengths uniform in [ctx_lo, ctx_hi].

    ``n_sets`` independent (Q, scores) sets share one cache; timing loops rotate
    through them so a step's gathered set is not already cache-resident.
    """
    g = _gen(seed, device)
    ctx = uniform_int(ctx_lo, ctx_hi, B, g, device).cpu()
    cache = make_paged_cache(ctx, kv_dtype, g, device, fp8_scale_log2=fp8_scale_log2)
    stride = int(stride if stride is not None else ctx_hi)
    row_req = torch.arange(B, dtype=torch.int32)
    sets = [make_rowset(cache, row_req, ctx.to(torch.int32), H, stride, g, device, score_kind)
            for _ in range(n_sets)]
    return DecodeWorkload(name=name, cache=cache, sets=sets, H=H, k=k, scale=SOFTMAX_SCALE, stride=stride)


def tiny_decode(device, seed: int = 0) -> DecodeWorkload:
    """B=2, H=16, 4096-token contexts (64 pages each), k=256, scores in steps of 1/8."""
    return decode_workload("tiny_decode_B2_H16_L4096_k256", B=2, H=16, k=256, ctx_lo=4096, ctx_hi=4096,
                           kv_dtype=KV_BF16, seed=seed, device=device, score_kind="eighths")


def decode_bf16(device, seed: int = 2, n_sets: int = 1) -> DecodeWorkload:
    """B=64, H=64, k=2048, contexts uniform in [8192, 65536], bf16 KV."""
    return decode_workload("decode_bf16_B64_H64_k2048_L8K-64K", B=64, H=64, k=2048, ctx_lo=8192, ctx_hi=65536,
                           kv_dtype=KV_BF16, seed=seed, device=device, n_sets=n_sets)


def decode_fp8(device, seed: int = 3, n_sets: int = 1) -> DecodeWorkload:
    """B=128, H=64, k=2048, contexts uniform in [32768, 131072], FP8 e4m3 latent with per-128 fp32 scales."""
    return decode_workload("decode_fp8_B128_H64_k2048_L32K-128K", B=128, H=64, k=2048, ctx_lo=32768,
                           ctx_hi=131072, kv_dtype=KV_FP8, seed=seed, device=device, n_sets=n_sets)


def topk_levels(device, rows: int = 64, L: int = 65536, levels: int = 256, seed: int = 1) -> torch.Tensor:
    """rows x L fp32 scores; each row uses ``levels`` distinct nonzero N(0,1) values (heavy ties)."""
    g = _gen(seed, device)
    out = torch.empty((rows, L), dtype=torch.float32, device=device)
    for r in range(rows):
        while True:
            lv = torch.randn((levels,), generator=g, device=device, dtype=torch.float32)
            if torch.unique(lv).numel() == levels and bool((lv != 0).all()):
                break
        pick = torch.randint(0, levels, (L,), generator=g, device=device)
        out[r] = lv[pick]
    return out


@dataclasses.dataclass
class PrefillWorkload:
    name: str
    cache: PagedCache           # request 0 is the prefill context; 1..63 the decode rows' contexts
    q: torch.Tensor             # bf16 [T, H, 576] prefill query rows
    scores: torch.Tensor        # fp32 [T, ctx] prefill scores (+inf past each row's causal length)
    first_pos: int              # position of query row 0
    decode: RowSet              # the decode rows mixed in later (row_req 1..63)
    mix_order: torch.Tensor     # int64 [T + n_dec]: mixed-batch slot -> source (< T prefill row, else decode row)
    H: int
    k: int
    scale: float


def prefill_chunk(device, seed: int = 4, T: int = 4096, ctx: int = 131072, H: int = 64, k: int = 2048,
                  n_dec: int = 63, dec_lo: int = 8192, dec_hi: int = 65536) -> PrefillWorkload:
    """One request: T query tokens at positions ctx-T .. ctx-1 of a ctx-token paged context (causal),
    plus n_dec decode rows (contexts uniform in [dec_lo, dec_hi]) to be mixed into one batch."""
    g = _gen(seed, device)
    dec_ctx = uniform_int(dec_lo, dec_hi, n_dec, g, device).cpu()
    all_ctx = torch.cat([torch.tensor([ctx], dtype=torch.int64), dec_ctx])
    cache = make_paged_cache(all_ctx, KV_BF16, g, device)
    first_pos = ctx - T
    causal = torch.arange(T, dtype=torch.int64) + first_pos + 1
    scores = _scores_block(T, ctx, g, device, "normal")
    poison_score_tails(scores, causal)
    q = torch.randn((T, H, D_QK), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    dec_req = torch.arange(1, n_dec + 1, dtype=torch.int32)
    dec = make_rowset(cache, dec_req, dec_ctx.to(torch.int32), H, dec_hi, g, device, "normal")
    mix_order = torch.randperm(T + n_dec, generator=g, device=device).cpu()
    return PrefillWorkload(name=f"prefill_T{T}_ctx{ctx}_H{H}_k{k}_mixed{n_dec}", cache=cache, q=q,
                           scores=scores, first_pos=first_pos, decode=dec, mix_order=mix_order, H=H, k=k,
                           scale=SOFTMAX_SCALE)


@dataclasses.dataclass
class CacheWriteWorkload:
    """New tokens to insert into a paged cache."""
    tokens: torch.Tensor        # bf16 [T, 576]: 512 latent, 64 rope
    slots: torch.Tensor         # int64 [T]: physical slot (page * 64 + offset) of each token
    num_pages: int


def cache_write_tokens(device, T: int, num_pages: int, seed: int = 5, spread: float = 8.0) -> CacheWriteWorkload:
    """T tokens of bf16 N(0,1) values, each 128-entry latent group (and the rope) multiplied by its own
    2**U(-spread, spread), rounded to bf16; the tokens go to T distinct slots of a cache of
    ``num_pages`` pages (page 0 excluded), drawn by a seeded permutation."""
    g = _gen(seed, device)
    vals = torch.randn((T, D_QK), generator=g, device=device, dtype=torch.float32)
    expo = torch.rand((T, 5), generator=g, device=device, dtype=torch.float32) * (2 * spread) - spread
    mult = torch.exp2(expo).repeat_interleave(torch.tensor([128, 128, 128, 128, 64], device=device), dim=1)
    tokens = (vals * mult).to(torch.bfloat16)
    nslots = (num_pages - 1) * PAGE
    if T > nslots:
        raise ValueError("more tokens than slots")
    slots = torch.randperm(nslots, generator=g, device=device)[:T] + PAGE
    return CacheWriteWorkload(tokens=tokens, slots=slots.to(torch.int64), num_pages=num_pages)


@dataclasses.dataclass
class WindowCache:
    """A sliding-window paged cache next to a main cache: each request keeps only the pages that hold
    its last window + draft positions; the block-table entries of its other logical pages are 0, the
    NaN null page (evicted)."""
    kv: torch.Tensor            # uint8 [num_pages, 64, record]
    block_table: torch.Tensor   # int32 [num_requests, max_pages]
    idx: torch.Tensor           # int32 [rows, width]: window + draft positions, ascending, -1 padded


def window_cache(ctx_lens: torch.Tensor, kv_dtype: int, device, seed: int, window: int = 128, draft: int = 5,
                 width: int = 192, max_pages: Optional[int] = None) -> WindowCache:
    """Window cache for requests with contexts ``ctx_lens``: request r (context c) holds positions
    max(0, c - draft - window) .. c - 1 in fresh pages handed out by a seeded permutation (records
    drawn like make_paged_cache's); its other logical pages map to the null page 0.  Slots of a held
    page outside that range, and the null page, hold NaN records.  ``idx`` row r lists those positions
    ascending, -1 padded to ``width`` (one row per request)."""
    g = _gen(seed, device)
    ctx = [int(c) for c in ctx_lens.tolist()]
    max_pages = max_pages or max(1, max((c + PAGE - 1) // PAGE for c in ctx))
    spans = []
    for c in ctx:
        lo = max(0, c - draft - window)
        spans.append((lo, c, lo // PAGE, (c - 1) // PAGE if c > 0 else lo // PAGE - 1))
    total = sum(max(0, p1 - p0 + 1) for _, _, p0, p1 in spans)
    rec = BF16_RECORD_BYTES if kv_dtype == KV_BF16 else FP8_RECORD_BYTES
    kv = torch.empty((total + 1, PAGE, rec), dtype=torch.uint8, device=device)
    perm = torch.randperm(total, generator=g, device=device).cpu() + 1
    bt = torch.zeros((len(ctx), max_pages), dtype=torch.int32)
    ntok = total * PAGE
    if kv_dtype == KV_BF16:
        vals = torch.randn((ntok, D_QK), generator=g, device=device, dtype=torch.float32)
        kv[1:] = vals.to(torch.bfloat16).view(torch.uint8).view(total, PAGE, rec)
    else:
        lat = torch.randn((ntok, 512), generator=g, device=device, dtype=torch.float32)
        codes = lat.to(torch.float8_e4m3fn).view(torch.uint8)
        expo = torch.rand((ntok, 4), generator=g, device=device, dtype=torch.float32) * 8.0 - 4.0
        scales = torch.exp2(expo).contiguous().view(torch.uint8).view(ntok, 16)
        rope = torch.randn((ntok, D_ROPE), generator=g, device=device, dtype=torch.float32)
        rope_b = rope.to(torch.bfloat16).view(torch.uint8).view(ntok, 128)
        kv[1:] = torch.cat([codes, scales, rope_b], dim=1).view(total, PAGE, rec)
    poison = _poison_record(kv_dtype, device)
    kv[0] = poison
    off = 0
    idx = torch.full((len(ctx), width), -1, dtype=torch.int32)
    for r, (lo, c, p0, p1) in enumerate(spans):
        for lp in range(p0, p1 + 1):
            pg = int(perm[off])
            off += 1
            bt[r, lp] = pg
            s0, s1 = max(lo, lp * PAGE), min(c, (lp + 1) * PAGE)        # held positions of this page
            if s0 > lp * PAGE:
                kv[pg, : s0 - lp * PAGE] = poison
            if s1 < (lp + 1) * PAGE:
                kv[pg, s1 - lp * PAGE:] = poison
        n = c - lo
        idx[r, :n] = torch.arange(lo, c, dtype=torch.int32)
    return WindowCache(kv=kv, block_table=bt.to(device), idx=idx.to(device))


def rope_cos_sin(max_pos: int, device, base: float = 10000.0) -> torch.Tensor:
    """A rotary table of the usual frequency schedule, fp32 [max_pos, 64]: row p holds cos(p f_i) for
    i < 32, then sin(p f_i), with f_i = base^(-i/32) (computed in float64, rounded to fp32)."""
    p = torch.arange(max_pos, dtype=torch.float64).view(-1, 1)
    f = base ** (-torch.arange(32, dtype=torch.float64) / 32.0)
    ang = p * f.view(1, -1)
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32).to(device)


def swa_draft_indices(ctx_lens: torch.Tensor, window: int = 128, draft: int = 5, width: int = 192) -> torch.Tensor:
    """Index rows of a draft batch over sliding-window KV: a request whose context holds c positions
    (the last ``draft`` of them draft tokens) attends to its last ``window`` committed positions and to
    all ``draft`` draft positions, i.e. positions max(0, c - draft - window) .. c - 1 in ascending order,
    padded with -1 to ``width`` (a multiple of the 64-entry tile: 192 for 128 + 5)."""
    rows = ctx_lens.numel()
    out = torch.full((rows, width), -1, dtype=torch.int32)
    for r, c in enumerate(ctx_lens.tolist()):
        lo = max(0, int(c) - draft - window)
        n = int(c) - lo
        out[r, :n] = torch.arange(lo, int(c), dtype=torch.int32)
    return out.to(ctx_lens.device)


# --------------------------------------------------------------------------------------------
# Indexer inputs: a paged index-key cache (one 128-wide bf16 key per token), index queries and
# per-row head weights.
# --------------------------------------------------------------------------------------------

D_INDEX = 128


def make_index_cache(block_table_cpu: torch.Tensor, ctx_lens, num_pages: int, g: torch.Generator, device,
                     chunk_pages: int = 8192) -> torch.Tensor:
    """bf16 [num_pages, 64, 128] index keys drawn N(0,1) for pages 1..num_pages-1; the null page 0
    and every slot past a context's end in its last page hold NaN."""
    kidx = torch.empty((num_pages, PAGE, D_INDEX), dtype=torch.bfloat16, device=device)
    for p0 in range(1, num_pages, chunk_pages):
        p1 = min(num_pages, p0 + chunk_pages)
        kidx[p0:p1] = torch.randn((p1 - p0, PAGE, D_INDEX), generator=g, device=device,
                                  dtype=torch.float32).to(torch.bfloat16)
    kidx[0] = float("nan")
    for r, L in enumerate(ctx_lens):
        L = int(L)
        if L % PAGE:
            kidx[int(block_table_cpu[r, L // PAGE]), L % PAGE:] = float("nan")
    return kidx


@dataclasses.dataclass
class IndexerWorkload:
    name: str
    kidx: torch.Tensor          # bf16 [num_pages, 64, 128]
    block_table: torch.Tensor   # int32 [num_requests, max_pages]
    ctx_lens: torch.Tensor      # int64 [num_requests] (CPU)
    q: List[torch.Tensor]       # per set: bf16 [rows, Hi, 128]
    weights: List[torch.Tensor] # per set: fp32 [rows, Hi]
    lengths: torch.Tensor       # int32 [rows]
    row_req: torch.Tensor       # int32 [rows]
    Hi: int
    stride: int


def indexer_queries(rows: int, Hi: int, g: torch.Generator, device):
    """Index queries bf16 N(0,1) [rows, Hi, 128] and head weights fp32 N(0, 1/Hi) [rows, Hi]."""
    q = torch.randn((rows, Hi, D_INDEX), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn((rows, Hi), generator=g, device=device, dtype=torch.float32) / math.sqrt(Hi)
    return q, w


def indexer_workload(name: str, B: int, Hi: int, ctx_lo: int, ctx_hi: int, seed: int, device, n_sets: int = 1,
                     stride: Optional[int] = None) -> IndexerWorkload:
    """B decode rows, one request each, context lengths uniform in [ctx_lo, ctx_hi]; each row
    scores its whole context.  Draw order: lengths, page permutation, keys, then (Q, weights) per set."""
    g = _gen(seed, device)
    ctx = uniform_int(ctx_lo, ctx_hi, B, g, device).cpu()
    bt, total = page_table(ctx, g, device)
    kidx = make_index_cache(bt, ctx, total + 1, g, device)
    qs, ws = [], []
    for _ in range(n_sets):
        q, w = indexer_queries(B, Hi, g, device)
        qs.append(q)
        ws.append(w)
    return IndexerWorkload(name=name, kidx=kidx, block_table=bt.to(device), ctx_lens=ctx, q=qs, weights=ws,
                           lengths=ctx.to(torch.int32).to(device),
                           row_req=torch.arange(B, dtype=torch.int32, device=device), Hi=Hi,
                           stride=int(stride if stride is not None else ctx_hi))


def indexer_decode(device, seed: int = 6, n_sets: int = 1) -> IndexerWorkload:
    """B=64 decode rows, 64 index heads of width 128, contexts uniform in [8192, 65536] (the decode
    rows the bf16 attention workload selects from), score rows of 65536 entries."""
    return indexer_workload("indexer_B64_Hi64_L8K-64K", B=64, Hi=64, ctx_lo=8192, ctx_hi=65536, seed=seed,
                            device=device, n_sets=n_sets)
