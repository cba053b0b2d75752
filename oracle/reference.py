"""CPU oracle for deterministic sparse MLA: stable top-k, canonical order, paged gather, MQA attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP path.

Everything here is written for a reader checking it by eye against the
definitions: plain numpy, float64 for all floating point, no blocking, no
fusion.  Library primitives used as single steps: ``np.lexsort`` (a sort),
``@`` (a matmul), ``np.exp`` / ``np.log``.

Sources (pages as titled; sections named):

* "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL"
  (vllm-project/vllm PR 54955), section "Deterministic sparse top-k": the
  selector ranks candidates by a composite score/index key with a stable
  tie-break, and the selected indices are put into one canonical order before
  attention so the reduction order is fixed.  Section "Sparse MLA and
  FlashMLA": decode gathers KV for the selected tokens and runs the same sparse
  attention as prefill; prefill chunks each request on its own.
* "[Bugfix] Make DSV4 sparse MLA work end-to-end for plain decode, MTP, and
  DSpark" (vllm-project/vllm PR 51538), section "Purpose", items "Negative
  indexer context lengths under MTP" and "Top-k kernels hardened against
  out-of-range lengths": lengths are clamped to [0, row stride] before any
  decision; rows with fewer candidates than k are padded with -1.  Item
  "Graph replay and draft KV": a token's cache slot is its physical block id
  times the block size plus its offset in the block.
* "Port DeepSeek-V4 optimization PR #174 to v0.26 ..." (MooreThreads/vllm-musa
  PR 178), table "Optimizations carried from PR #174": FP8 KV with fp32 scale
  groups kept contiguous, and an FP8 cache write that quantizes new tokens in
  128-element groups.  "[DeepSeek-V4][Preview] Batch-invariant kernels for
  0-diff RL", section on the fused group-quantization operator: 128-element
  groups with FP32 scales.

Readings where the pages are silent (each is listed with its reason in the
design notes):

* ties between equal scores go to the lower index; -0.0 equals +0.0 (IEEE
  comparison); +-inf are ordinary values; NaN ranks below -inf and NaNs tie
  among themselves by index;
* the selected indices are emitted in ascending index order, then -1 padding;
* indices are logical token positions in the row's request; the gather maps
  position p to physical slot block_table[req, p // 64] * 64 + p % 64;
* all heads share one 576-wide latent record K_j (512 latent + 64 rope) and
  the value vector is its first 512 entries;
* LSE is the natural-log log-sum-exp of the scaled scores; a row with no
  selected token has output 0 and LSE -inf;
* an attention sink is one logit per head (in the units of the scaled scores)
  that joins the softmax denominator and carries no value: p_j = e^{s_j} /
  (e^{sink} + sum_i e^{s_i}), LSE = log(e^{sink} + sum_i e^{s_i}); -inf means no
  sink ("[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL", section
  "MHC, CUDA graphs, and weight reload": the sink weights keep their -inf
  padding);
* the FP8 record is [512 e4m3 codes | 4 fp32 scales | 64 bf16 rope]; latent
  entry d is e4m3(code_d) * scale_{d // 128}; e4m3 is the OCP E4M3FN format;
* the cache write quantizes group g of a token's 512 latent values so that
  the group's largest magnitude amax maps to 448: the stored fp32 scale is
  s = amax / 448 and the codes are e4m3(x / s), the inverse of the
  dequantization, which multiplies a code by s (each division rounded to
  nearest-even in fp32; the code rounded to nearest-even and saturated at
  +-448); an all-zero group gets s = 0 and zero codes;
* the cache write's "inverse-RoPE" ("Port DeepSeek-V4 optimization PR #174
  ...", table "Optimizations carried from PR #174", row "Attention cache
  write") undoes the rotary embedding of the 64 rope values before they are
  stored: with the caller's tables cos[pos, i], sin[pos, i] (i < 32, fp32)
  and the pairs (x_2i, x_2i+1), the stored pair is
  (x_2i cos + x_2i+1 sin, -x_2i sin + x_2i+1 cos), evaluated exactly and
  rounded to bf16 once (nearest-even); without tables the rope values are
  stored unchanged; the rope inputs must be finite;
* indexer scores ("MQA logits" of the DSA indexer: the pages name the operation and its
  paged form -- "[SM120] Sync DS4 with upstream main + validated perf backports", sections
  "September 12 follow-up" and "2026-09-12 live validation and promotion update" -- but give
  no formula): the published lightning-indexer form of DeepSeek sparse attention, one shared
  128-wide bf16 index key per token (MQA) and index heads h with per-row weights w_h:
  score[p] = sum_h w_h * relu(<q_h, k_p>) with relu(x) = x if x > 0 else 0, for positions p
  below the clamped length whose page is listed; every other position of the row is -inf.
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

PAGE = 64
D_QK = 576
D_V = 512
KV_BF16 = 0
KV_FP8 = 1
BF16_RECORD_BYTES = 1152
FP8_RECORD_BYTES = 656


# ----------------------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64.  A bf16 value is the binary32 number whose upper 16 bits
    are the pattern and whose lower 16 bits are zero; the widening is exact."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes) -> np.ndarray:
    """OCP 8-bit floating point, E4M3 (FN) variant -> float64, from the format definition:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
    subnormals (m/8) * 2**-6; S.1111.111 is NaN; there are no infinities."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


def decode_record(rec: np.ndarray, kv_dtype: int) -> np.ndarray:
    """One token record (raw bytes, uint8) -> float64 [576] = [512 latent | 64 rope]."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    if kv_dtype == KV_BF16:
        assert rec.shape[-1] == BF16_RECORD_BYTES
        return bf16_to_f64(rec.view(np.uint16))
    assert rec.shape[-1] == FP8_RECORD_BYTES
    codes = rec[..., :512]
    scales = rec[..., 512:528].view(np.float32).astype(np.float64)       # [..., 4]
    rope = bf16_to_f64(rec[..., 528:656].view(np.uint16))                # [..., 64]
    lat = e4m3fn_to_f64(codes) * np.repeat(scales, 128, axis=-1)          # group g = d // 128
    return np.concatenate([lat, rope], axis=-1)


def _e4m3fn_finite_table() -> np.ndarray:
    """Values of the non-negative finite E4M3FN codes 0x00 .. 0x7E, in code order (ascending)."""
    return e4m3fn_to_f64(np.arange(0x7F))


def f32_to_e4m3fn(x) -> np.ndarray:
    """float32 values -> E4M3FN codes, rounding to the nearest representable value with ties to
    the code whose mantissa is even, and saturating magnitudes above 448 to +-448.  The sign of
    zero is kept.  NaN gives the NaN code 0x7F (sign kept)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    table = _e4m3fn_finite_table()
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0x00)
    hi = np.clip(np.searchsorted(table, np.minimum(a, table[-1]), side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(a - table[lo])
    d_hi = np.abs(table[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= table[-1], 0x7E, code)                       # saturate
    code = np.where(np.isnan(x), 0x7F, code)
    return (code | sign).astype(np.uint8)


def quantize_group(x_bits: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """One 128-entry scale group of bf16 latent values -> (e4m3 codes [128], fp32 scale).
    s = fp32(amax / 448), codes = e4m3(fp32(x / s)): the dequantization multiplies a code by s,
    so the quantization divides by it.  An all-zero group has s = 0, codes 0.  (For any nonzero
    bf16 amax, s is a nonzero fp32 number, so the quotient is always defined.)"""
    x = bf16_to_f64(x_bits).astype(np.float32)                        # exact widening
    amax = np.float32(np.max(np.abs(x)))
    if amax == 0:
        return np.zeros(len(x), dtype=np.uint8), np.float32(0.0)
    s = np.float32(amax / np.float32(448.0))                          # IEEE fp32 division
    y = (x / s).astype(np.float32)                                    # IEEE fp32 division
    return f32_to_e4m3fn(y), s


def exact_to_bf16_rne(v: Fraction) -> int:
    """An exact rational value -> the bf16 bit pattern of the nearest bf16 value, ties to the even
    pattern: the plain round-to-nearest-even of the exact value, with no intermediate rounding.
    Values that would round beyond the largest bf16 raise."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()      # 2^(e-1) < a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1                                                     # now 2^e <= a < 2^(e+1)
    e = max(e, -126)                                               # subnormals share the minimum exponent
    ulp = Fraction(2) ** (e - 7)                                   # 8 significant bits
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val >= Fraction(2) ** 128:
        raise OverflowError("bf16 overflow")
    bits = int(np.array(float(val), dtype=np.float32).view(np.uint32)) >> 16   # val is bf16-exact
    return sign | bits


def inverse_rope(rope_bits: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """The 64 rope values of one token (bf16 patterns) with the rotary embedding undone: pair i
    is (x_2i, x_2i+1); with c = cos[i], s = sin[i] (fp32 table entries of the token's position)
    the result is (x_2i c + x_2i+1 s, -x_2i s + x_2i+1 c), the rotation by minus the angle,
    evaluated exactly (rational arithmetic) and rounded once to bf16 (nearest-even)."""
    x = bf16_to_f64(rope_bits)
    c = np.asarray(cos, dtype=np.float32).astype(np.float64)
    s = np.asarray(sin, dtype=np.float32).astype(np.float64)
    out = np.empty(64, dtype=np.uint16)
    for i in range(32):
        a, b = Fraction(float(x[2 * i])), Fraction(float(x[2 * i + 1]))
        ci, si = Fraction(float(c[i])), Fraction(float(s[i]))
        out[2 * i] = exact_to_bf16_rne(a * ci + b * si)
        out[2 * i + 1] = exact_to_bf16_rne(-a * si + b * ci)
    return out


def encode_record(token_bits: np.ndarray, kv_dtype: int, cos: Optional[np.ndarray] = None,
                  sin: Optional[np.ndarray] = None) -> np.ndarray:
    """One token's 576 bf16 values (bit patterns: 512 latent, 64 rope) -> its cache record
    (uint8).  bf16 caches store the 1152 bytes as they are; FP8 caches store the 512 codes, the
    4 group scales and the 64 rope values.  With ``cos``/``sin`` (the 32 fp32 table entries of the
    token's position) the rope values are stored with the rotary embedding undone
    (``inverse_rope``)."""
    t = np.array(token_bits, dtype=np.uint16, copy=True)
    assert t.shape == (D_QK,)
    if cos is not None:
        t[512:] = inverse_rope(t[512:], cos, sin)
    if kv_dtype == KV_BF16:
        return t.view(np.uint8).copy()
    rec = np.zeros(FP8_RECORD_BYTES, dtype=np.uint8)
    scales = np.zeros(4, dtype=np.float32)
    for g in range(4):
        codes, s = quantize_group(t[128 * g:128 * (g + 1)])
        rec[128 * g:128 * (g + 1)] = codes
        scales[g] = s
    rec[512:528] = scales.view(np.uint8)
    rec[528:656] = t[512:576].view(np.uint8)
    return rec


def cache_write(cache: np.ndarray, kv_dtype: int, tokens_bits: np.ndarray,
                slot_mapping: Sequence[int], positions: Optional[Sequence[int]] = None,
                cos_table: Optional[np.ndarray] = None, sin_table: Optional[np.ndarray] = None) -> np.ndarray:
    """Writes token t's record to physical slot slot_mapping[t] (block id * 64 + offset) of the
    paged cache [num_pages, 64, record]; slots < 0 or past the cache are skipped.  With
    ``positions`` and the tables [max_pos, 32], token t's rope values are stored with the rotation
    of position positions[t] undone.  Returns the updated copy of the cache."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    flat = out.reshape(-1, out.shape[-1])
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if 0 <= slot < flat.shape[0]:
            if positions is None:
                flat[slot] = encode_record(tokens_bits[t], kv_dtype)
            else:
                p = int(positions[t])
                flat[slot] = encode_record(tokens_bits[t], kv_dtype, cos_table[p], sin_table[p])
    return out


# ----------------------------------------------------------------------------------------------
# A0: candidate counts
# ----------------------------------------------------------------------------------------------

def clamp_length(length: int, row_stride: int) -> int:
    """A row's candidate count is its length clamped to [0, row_stride]."""
    return int(min(max(int(length), 0), int(row_stride)))


def causal_lengths(first_pos: int, T: int) -> np.ndarray:
    """Query token t of a chunk sits at position first_pos + t and may attend to positions
    0..first_pos + t, so its candidate count is first_pos + t + 1, never below 0."""
    return np.array([max(0, first_pos + t + 1) for t in range(T)], dtype=np.int64)


# ----------------------------------------------------------------------------------------------
# A1-A3: stable top-k and canonical order
# ----------------------------------------------------------------------------------------------

def topk_row(scores_row: np.ndarray, length: int, k: int) -> np.ndarray:
    """Indices of the top n = min(k, L) candidates of one row, ascending, then -1 padding.

    Total order on candidates j in [0, L): a higher score comes first; equal scores (IEEE
    equality, so -0.0 == +0.0) come in increasing index order; NaN comes after every number
    and NaNs come in increasing index order.  The first n candidates in that order are the
    selection; the emitted list is the selection sorted by index.
    """
    L = clamp_length(length, len(scores_row))
    n = min(int(k), L)
    out = np.full(int(k), -1, dtype=np.int32)
    if n == 0:
        return out
    v = np.asarray(scores_row[:L], dtype=np.float64)
    is_nan = np.isnan(v)
    vv = np.where(is_nan, 0.0, v)
    # np.lexsort orders by the LAST key first: NaN flag (numbers first), then -score
    # (so higher scores first; -0.0 and +0.0 compare equal), then index.
    order = np.lexsort((np.arange(L), -vv, is_nan))
    out[:n] = np.sort(order[:n]).astype(np.int32)
    return out


def topk_rows(scores: np.ndarray, lengths: Optional[Sequence[int]], k: int,
              row_offsets: Optional[Sequence[int]] = None, row_stride: Optional[int] = None,
              rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """topk_row for each requested row.  ``scores`` is either a 2-D [R, stride] array or a flat
    array addressed through ``row_offsets`` (element offsets) with ``row_stride`` entries per row."""
    flat = scores.reshape(-1) if row_offsets is not None else None
    nrows = len(lengths) if lengths is not None else scores.shape[0]
    stride = int(row_stride if row_stride is not None else scores.shape[-1])
    idx = list(range(nrows)) if rows is None else list(rows)
    out = np.empty((len(idx), int(k)), dtype=np.int32)
    for o, r in enumerate(idx):
        if row_offsets is not None:
            base = int(row_offsets[r])
            row = flat[base:base + stride]
        else:
            row = scores[r]
        L = stride if lengths is None else int(lengths[r])
        out[o] = topk_row(row, L, k)
    return out


# ----------------------------------------------------------------------------------------------
# A4-A5: paged gather
# ----------------------------------------------------------------------------------------------

def physical_slot(block_table_row: np.ndarray, pos: int, page: int = PAGE) -> int:
    """Logical position -> physical cache slot: block id * block size + offset in the block."""
    return int(block_table_row[pos // page]) * page + pos % page


def gather_tokens(kv: np.ndarray, kv_dtype: int, block_table_row: np.ndarray,
                  positions: Sequence[int]) -> np.ndarray:
    """Records of the given logical positions (in the given order) as float64 [n, 576].
    ``kv`` holds the raw bytes [num_pages, 64, record_bytes]."""
    flat = kv.reshape(-1, kv.shape[-1])
    recs = [decode_record(flat[physical_slot(block_table_row, int(p))], kv_dtype) for p in positions]
    if not recs:
        return np.zeros((0, D_QK))
    return np.stack(recs)


# ----------------------------------------------------------------------------------------------
# A7-A9: MQA attention over the gathered latent tokens
# ----------------------------------------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, scale: float,
              sink: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of every head of ``q`` [H, 576] over the shared tokens ``K`` [n, 576].

    s[h, j] = scale * <q_h, K_j> over all 576 entries; the softmax denominator of head h is
    D_h = sum_j exp(s[h, j]) + exp(sink[h]) (no sink term when ``sink`` is None or -inf);
    O[h, :] = sum_j (exp(s[h, j]) / D_h) * K_j[:512]; LSE[h] = log D_h.
    With n = 0 the output is 0 and LSE is sink[h] (-inf without a sink).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    H = q.shape[0]
    sk = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64).reshape(H)
    if K.shape[0] == 0:
        return np.zeros((H, D_V)), sk.copy()
    s = scale * (q @ K.T)                       # [H, n]
    m = np.maximum(s.max(axis=1), sk)[:, None]  # [H, 1], finite: n >= 1
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True) + np.exp(sk[:, None] - m)
    p = e / l
    O = p @ K[:, :D_V]
    lse = (m + np.log(l))[:, 0]
    return O, lse


def split_combine(parts: Sequence[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine per-split (O_s, LSE_s) results of disjoint token subsets of one row, in the
    listed order: LSE = log sum_s exp(LSE_s); O = sum_s exp(LSE_s - LSE) * O_s.  Splits with
    LSE_s = -inf contribute nothing; if every split is empty the result is (0, -inf)."""
    lses = np.stack([p[1] for p in parts])      # [S, H]
    Os = np.stack([p[0] for p in parts])        # [S, H, D]
    m = lses.max(axis=0)                        # [H]
    H = lses.shape[1]
    O = np.zeros(Os.shape[1:])
    LSE = np.full(H, -np.inf)
    for h in range(H):
        if not np.isfinite(m[h]):
            continue
        w = np.exp(lses[:, h] - m[h])
        tot = w.sum()
        LSE[h] = m[h] + math.log(tot)
        for s in range(len(parts)):
            O[h] += (w[s] / tot) * Os[s, h]
    return O, LSE


# ----------------------------------------------------------------------------------------------
# Indexer scores (paged MQA logits): the producer of the scores the top-k consumes
# ----------------------------------------------------------------------------------------------

D_INDEX = 128
INDEX_RECORD_BYTES = 2 * D_INDEX


def indexer_scores_row(q: np.ndarray, w: np.ndarray, kidx: np.ndarray, block_table_row: np.ndarray,
                       length: int, stride: int, page: int = PAGE) -> np.ndarray:
    """Scores of one query row for positions 0 .. stride-1 (float64).

    ``q`` [Hi, d] and ``w`` [Hi] are the row's index queries and head weights (float64),
    ``kidx`` the index-key cache [num_pages, page, d] (float64).  With L the length clamped to
    [0, stride], position p < L whose page entry block_table_row[p // page] names a page of the
    cache has score sum_h w_h * relu(<q_h, k_p>), k_p = kidx[block_table_row[p // page], p % page];
    every other position has -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = np.full(int(stride), -np.inf)
    L = clamp_length(length, stride)
    num_pages = kidx.shape[0]
    for p in range(L):
        lp = p // page
        if lp >= len(block_table_row):
            continue
        pg = int(block_table_row[lp])
        if pg < 0 or pg >= num_pages:
            continue
        k = kidx[pg, p % page]
        dots = q @ k                                   # [Hi]: <q_h, k_p>
        relu = np.where(dots > 0, dots, 0.0)
        out[p] = float(np.sum(w * relu))
    return out


def indexer_scores(q_bits: np.ndarray, w: np.ndarray, kidx_bits: np.ndarray, block_table: np.ndarray,
                   row_req: Optional[Sequence[int]], lengths: Sequence[int], stride: int,
                   rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """indexer_scores_row for each requested row: ``q_bits`` bf16 patterns [R, Hi, d], ``w``
    fp32 [R, Hi], ``kidx_bits`` bf16 patterns [num_pages, 64, d]; row r reads the block table
    row of request row_req[r] (0 when row_req is None)."""
    sel = list(range(len(lengths))) if rows is None else list(rows)
    K = bf16_to_f64(kidx_bits)
    out = np.empty((len(sel), int(stride)))
    for o, r in enumerate(sel):
        req = 0 if row_req is None else int(row_req[r])
        out[o] = indexer_scores_row(bf16_to_f64(q_bits[r]), np.asarray(w[r], dtype=np.float64), K,
                                    block_table[req], int(lengths[r]), stride)
    return out


def indexer_error_scale(q_bits: np.ndarray, w: np.ndarray, kidx_bits: np.ndarray, block_table: np.ndarray,
                        row_req: Optional[Sequence[int]], lengths: Sequence[int], stride: int,
                        rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """M[r, p] = sum_h |w_h| * sum_d |q_hd| |k_pd| for the scored positions (0 elsewhere): the
    magnitude that bounds the rounding error of any fp32 evaluation of a score."""
    sel = list(range(len(lengths))) if rows is None else list(rows)
    K = np.abs(bf16_to_f64(kidx_bits))
    out = np.zeros((len(sel), int(stride)))
    for o, r in enumerate(sel):
        req = 0 if row_req is None else int(row_req[r])
        qa = np.abs(bf16_to_f64(q_bits[r]))
        wa = np.abs(np.asarray(w[r], dtype=np.float64))
        L = clamp_length(int(lengths[r]), stride)
        bt = block_table[req]
        for p in range(L):
            lp = p // PAGE
            if lp < len(bt) and 0 <= int(bt[lp]) < K.shape[0]:
                out[o, p] = float(wa @ (qa @ K[int(bt[lp]), p % PAGE]))
    return out


# ----------------------------------------------------------------------------------------------
# Whole rows: top-k -> canonical indices -> gather -> attention
# ----------------------------------------------------------------------------------------------

def attention_rows(q_bits: np.ndarray, kv: np.ndarray, kv_dtype: int, block_table: np.ndarray,
                   row_req: Optional[Sequence[int]], idx: np.ndarray, scale: float,
                   rows: Optional[Sequence[int]] = None,
                   sink: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for each requested row over the tokens listed in ``idx`` [R, k] (entries -1
    are skipped).  ``q_bits`` holds bf16 patterns [R, H, 576]; ``sink`` is the per-head sink
    logit [H] or None."""
    sel = list(range(idx.shape[0])) if rows is None else list(rows)
    H = q_bits.shape[1]
    O = np.zeros((len(sel), H, D_V))
    LSE = np.zeros((len(sel), H))
    for o, r in enumerate(sel):
        req = 0 if row_req is None else int(row_req[r])
        pos = [int(p) for p in idx[r] if p >= 0]
        K = gather_tokens(kv, kv_dtype, block_table[req], pos)
        O[o], LSE[o] = attention(bf16_to_f64(q_bits[r]), K, scale, sink)
    return O, LSE


def attention_rows_with_window(q_bits: np.ndarray, kv: np.ndarray, kv_dtype: int, block_table: np.ndarray,
                               idx: np.ndarray, kv_win: np.ndarray, block_table_win: np.ndarray,
                               idx_win: np.ndarray, row_req: Optional[Sequence[int]], scale: float,
                               rows: Optional[Sequence[int]] = None,
                               sink: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention over compressed and sliding-window KV in one softmax ("[DeepSeek-V4][Preview]
    Batch-invariant kernels for 0-diff RL", section "Sparse MLA and FlashMLA": decode gathers
    compressed and sliding-window KV; "[Bugfix] Make DSV4 sparse MLA work end-to-end ...", section
    "Purpose", item "SWA widths": the window + draft index width is padded to a multiple of the
    64-entry tile).  Row r attends to the tokens listed in ``idx[r]`` (logical positions in the
    paged cache ``kv`` of its request, through ``block_table``) together with the tokens listed in
    ``idx_win[r]`` (logical positions in the paged window cache ``kv_win``, through
    ``block_table_win``): one set of keys, one softmax, entries -1 skipped.  Same arithmetic as
    ``attention`` over that set."""
    sel = list(range(idx.shape[0])) if rows is None else list(rows)
    H = q_bits.shape[1]
    O = np.zeros((len(sel), H, D_V))
    LSE = np.zeros((len(sel), H))
    for o, r in enumerate(sel):
        req = 0 if row_req is None else int(row_req[r])
        K1 = gather_tokens(kv, kv_dtype, block_table[req], [int(p) for p in idx[r] if p >= 0])
        K2 = gather_tokens(kv_win, kv_dtype, block_table_win[req], [int(p) for p in idx_win[r] if p >= 0])
        O[o], LSE[o] = attention(bf16_to_f64(q_bits[r]), np.concatenate([K1, K2], axis=0), scale, sink)
    return O, LSE


def decode_rows(q_bits, kv, kv_dtype, block_table, row_req, scores, lengths, k, scale,
                rows=None, row_offsets=None, row_stride=None):
    """The whole decode path for the requested rows: (indices, O, LSE)."""
    sel = list(range(len(lengths))) if rows is None else list(rows)
    idx = topk_rows(scores, lengths, k, row_offsets=row_offsets, row_stride=row_stride, rows=sel)
    q_sel = np.asarray(q_bits)[sel]
    req_sel = None if row_req is None else [int(row_req[r]) for r in sel]
    O, LSE = attention_rows(q_sel, kv, kv_dtype, block_table, req_sel, idx, scale)
    return idx, O, LSE
