"""Pins for the CPU oracle: each test ties an oracle function to something other than itself
(brute force on tiny inputs, closed forms, library special cases, invariants, hand-derived
fixtures).  CPU only."""

import json
import math
import os
import random

import numpy as np
import pytest
import torch

import oracle.reference as O


def _num(x):
    if isinstance(x, str):
        return float(x)
    return float(x)


# ----------------------------------------------------------------------------------------------
# Top-k
# ----------------------------------------------------------------------------------------------

def _precedes(vi, i, vj, j):
    """Brute-force reading of the order, with Python float comparisons only."""
    ni, nj = math.isnan(vi), math.isnan(vj)
    if ni and nj:
        return i < j
    if ni != nj:
        return nj            # numbers before NaN
    if vi > vj:
        return True
    if vi == vj:
        return i < j
    return False


def brute_topk(scores, length, k):
    L = min(max(length, 0), len(scores))
    n = min(k, L)
    sel = []
    for j in range(L):
        ahead = sum(1 for i in range(L) if i != j and _precedes(scores[i], i, scores[j], j))
        if ahead < n:
            sel.append(j)
    assert len(sel) == n
    return sel + [-1] * (k - n)


VALUE_POOL = [0.0, -0.0, 1.0, -1.0, 0.5, 2.0, float("inf"), float("-inf"), float("nan"), 1e-30, -1e-30]


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_brute_force_on_tiny_rows(seed):
    rng = random.Random(seed)
    L = rng.randint(0, 24)
    pool = rng.sample(VALUE_POOL, rng.randint(1, len(VALUE_POOL)))
    row = [rng.choice(pool) for _ in range(L)] + [123.0] * rng.randint(0, 3)   # tail past the length
    for k in {1, 3, 16, max(1, L - 1), max(1, L), L + 5}:
        for length in {L, 0, -3, L + 7}:
            got = O.topk_row(np.array(row, dtype=np.float32), length, k).tolist()
            ref = brute_topk(row, length, k)
            assert got == ref, (row, length, k)


def test_topk_brute_force_random_float_rows():
    rng = np.random.default_rng(7)
    for _ in range(30):
        L = int(rng.integers(1, 60))
        row = rng.standard_normal(L).astype(np.float32)
        row[rng.integers(0, L, size=L // 3)] = row[0]            # planted ties
        k = int(rng.integers(1, L + 3))
        assert O.topk_row(row, L, k).tolist() == brute_topk(row.tolist(), L, k)


def test_topk_golden_hand_cases(golden_dir):
    data = json.load(open(os.path.join(golden_dir, "topk_hand_cases.json")))
    for c in data["cases"]:
        row = np.array([_num(x) for x in c["scores"]], dtype=np.float32)
        got = O.topk_row(row, c["length"], c["k"]).tolist()
        assert got == c["expected"], c["name"]


def test_topk_special_cases():
    rng = np.random.default_rng(3)
    row = rng.standard_normal(1000).astype(np.float32)
    # k >= L: every candidate, in order
    assert O.topk_row(row, 100, 100).tolist() == list(range(100))
    assert O.topk_row(row, 100, 130).tolist() == list(range(100)) + [-1] * 30
    # all equal: the k lowest indices
    assert O.topk_row(np.full(500, 3.5, np.float32), 500, 37).tolist() == list(range(37))
    # k = 1 is the first maximum (np.argmax returns the first occurrence)
    tied = np.round(row * 2) / 2
    assert O.topk_row(tied, 1000, 1).tolist() == [int(np.argmax(tied))]
    # strictly decreasing / increasing rows
    dec = np.arange(1000, 0, -1).astype(np.float32)
    assert O.topk_row(dec, 1000, 10).tolist() == list(range(10))
    assert O.topk_row(dec[::-1].copy(), 1000, 10).tolist() == list(range(990, 1000))
    # negative / zero lengths
    assert O.topk_row(row, -5, 4).tolist() == [-1] * 4
    assert O.topk_row(row, 0, 4).tolist() == [-1] * 4


def test_topk_selected_set_matches_partition_on_distinct_values():
    """With distinct values the selected set is the set np.argpartition picks."""
    rng = np.random.default_rng(11)
    for L, k in [(5000, 2048), (65536, 2048), (300, 299)]:
        row = rng.permutation(L).astype(np.float32) - L / 2
        part = np.argpartition(-row, k - 1)[:k]
        assert O.topk_row(row, L, k).tolist() == sorted(part.tolist())


def test_topk_heavy_ties_invariants():
    """256 distinct levels, 65536 candidates: selected count, ascending order, and that the
    cut respects both the score order and the lower-index rule."""
    rng = np.random.default_rng(5)
    levels = rng.standard_normal(256).astype(np.float32)
    row = levels[rng.integers(0, 256, 65536)]
    out = O.topk_row(row, 65536, 2048)
    assert (np.diff(out) > 0).all() and len(out) == 2048
    selv = row[out]
    mask = np.zeros(65536, bool)
    mask[out] = True
    t = selv.min()
    assert (row[~mask] <= t).all()                       # nothing better left out
    eq_idx = np.nonzero(row == t)[0]
    taken = eq_idx[mask[eq_idx]]
    assert (taken == eq_idx[:len(taken)]).all()          # ties at the cut: lowest indices


# Rows addressed through 64-bit element offsets into one flat buffer (unaligned and overlapping).
ROW_OFFSET_FLAT = [0.5, 3.0, -1.0, 2.0, 2.0, 7.0, 1.0, 1.0, 9.0, 0.0, -2.0, 4.0]
ROW_OFFSET_CASE = {"offsets": [3, 0, 6, 2], "stride": 5, "lengths": [5, 3, 5, 4], "k": 2,
                   # worked by hand:
                   #   row 0 = flat[3:8] = [2, 2, 7, 1, 1]: 7 (j=2), then the tie 2/2 -> j=0   -> [0, 2]
                   #   row 1 = flat[0:5], L=3 -> [0.5, 3, -1]: 3 (j=1), 0.5 (j=0)              -> [0, 1]
                   #   row 2 = flat[6:11] = [1, 1, 9, 0, -2]: 9 (j=2), tie 1/1 -> j=0          -> [0, 2]
                   #   row 3 = flat[2:7], L=4 -> [-1, 2, 2, 7]: 7 (j=3), tie 2/2 -> j=1        -> [1, 3]
                   "expected": [[0, 2], [0, 1], [0, 2], [1, 3]]}


def _row_offsets_case_holds(topk_rows_fn):
    c = ROW_OFFSET_CASE
    flat = np.array(ROW_OFFSET_FLAT, np.float32)
    got = topk_rows_fn(flat, c["lengths"], c["k"], row_offsets=np.array(c["offsets"], np.int64),
                       row_stride=c["stride"])
    if got.tolist() != c["expected"]:
        return False
    sub = topk_rows_fn(flat, c["lengths"], c["k"], row_offsets=np.array(c["offsets"], np.int64),
                       row_stride=c["stride"], rows=[3, 0])
    return sub.tolist() == [c["expected"][3], c["expected"][0]]


def test_topk_rows_row_offsets_hand_case():
    assert _row_offsets_case_holds(O.topk_rows)


def _ro_mutant_ignores_offsets(scores, lengths, k, row_offsets=None, row_stride=None, rows=None):
    flat = np.asarray(scores).reshape(-1)
    stride = int(row_stride)
    sel = list(range(len(lengths))) if rows is None else list(rows)
    return np.stack([O.topk_row(flat[r * stride:(r + 1) * stride], lengths[r], k) for r in sel])


def _ro_mutant_off_by_one(scores, lengths, k, row_offsets=None, row_stride=None, rows=None):
    return O.topk_rows(scores, lengths, k, row_offsets=np.asarray(row_offsets) + 1, row_stride=row_stride,
                       rows=rows)


@pytest.mark.parametrize("mutant", [_ro_mutant_ignores_offsets, _ro_mutant_off_by_one])
def test_pins_catch_row_offset_mutants(mutant):
    assert not _row_offsets_case_holds(mutant)


# Mutants: plausible mistakes, planted in copies of the oracle's top-k on the CPU, must fail a pin.

def _mutant_reverse_ties(row, length, k):
    L = O.clamp_length(length, len(row)); n = min(k, L)
    v = np.asarray(row[:L], np.float64); nan = np.isnan(v)
    order = np.lexsort((-np.arange(L), -np.where(nan, 0, v), nan))
    out = np.full(k, -1, np.int32); out[:n] = np.sort(order[:n]); return out


def _mutant_signed_zero(row, length, k):
    L = O.clamp_length(length, len(row)); n = min(k, L)
    v = np.asarray(row[:L], np.float64)
    key = np.where(np.isnan(v), -np.inf, v) + np.where(np.signbit(v) & (v == 0), -1e-300, 0.0)
    order = np.lexsort((np.arange(L), -key))
    out = np.full(k, -1, np.int32); out[:n] = np.sort(order[:n]); return out


def _mutant_no_clamp(row, length, k):
    L = len(row) if length < 0 else min(length, len(row))
    return O.topk_row(row, L, k)


@pytest.mark.parametrize("mutant", [_mutant_reverse_ties, _mutant_signed_zero, _mutant_no_clamp])
def test_pins_catch_topk_mutants(mutant, golden_dir):
    data = json.load(open(os.path.join(golden_dir, "topk_hand_cases.json")))
    caught = False
    for c in data["cases"]:
        row = np.array([_num(x) for x in c["scores"]], dtype=np.float32)
        if mutant(row, c["length"], c["k"]).tolist() != c["expected"]:
            caught = True
    assert caught


# ----------------------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------------------

def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint16)
    ours = O.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(ours[~np.isnan(ours)]), np.signbit(ref[~np.isnan(ref)]))


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3fn_spec_values(golden_dir):
    data = json.load(open(os.path.join(golden_dir, "fp8_e4m3fn_values.json")))
    for v in data["values"]:
        got = float(O.e4m3fn_to_f64(np.array([v["code"]], np.uint8))[0])
        exp = _num(v["value"])
        if math.isnan(exp):
            assert math.isnan(got)
        else:
            assert got == exp and math.copysign(1, got) == math.copysign(1, exp), v


def test_fp8_record_group_scales_and_rope():
    rec = np.zeros(656, np.uint8)
    rec[:512] = 0x38                                              # every code is 1.0
    rec[512:528] = np.array([1.0, 2.0, 0.25, -8.0], np.float32).view(np.uint8)
    rope = np.arange(64, dtype=np.float32) - 20.0                  # bf16-exact values
    rec[528:] = (rope.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8)
    out = O.decode_record(rec, O.KV_FP8)
    assert out.shape == (576,)
    np.testing.assert_array_equal(out[:512], np.repeat([1.0, 2.0, 0.25, -8.0], 128))
    np.testing.assert_array_equal(out[512:], rope)


# ----------------------------------------------------------------------------------------------
# FP8 cache write: e4m3 encoding and 128-entry group quantization
# ----------------------------------------------------------------------------------------------

def test_e4m3fn_encode_round_trips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3fn_to_f64(codes)
    fin = ~np.isnan(vals)
    np.testing.assert_array_equal(O.f32_to_e4m3fn(vals[fin].astype(np.float32)), codes[fin])


def test_e4m3fn_encode_matches_torch_inside_the_range():
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest-even; it is an independent
    # implementation for every magnitude up to 448 (it does not saturate, so nothing above).
    rng = np.random.default_rng(7)
    mags = np.concatenate([rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-12, 8.8, 20000)),
                           rng.uniform(0, 2 ** -6, 5000)])
    x = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.f32_to_e4m3fn(x), ref)


def test_e4m3fn_encode_ties_go_to_even_and_large_values_saturate():
    table = O.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mid = ((table[:-1] + table[1:]) / 2).astype(np.float32)          # exact in fp32
    got = O.f32_to_e4m3fn(mid)
    lo = np.arange(0x7E)
    np.testing.assert_array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    np.testing.assert_array_equal(O.f32_to_e4m3fn(-mid), np.where(lo % 2 == 0, lo, lo + 1) | 0x80)
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, 3e38], np.float32)
    np.testing.assert_array_equal(O.f32_to_e4m3fn(big), np.full(6, 0x7E))
    np.testing.assert_array_equal(O.f32_to_e4m3fn(-big), np.full(6, 0xFE))
    assert list(O.f32_to_e4m3fn(np.array([0.0, -0.0], np.float32))) == [0x00, 0x80]


def _bf16_bits(x):
    """float32 values that are bf16-exact -> bf16 bit patterns."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_rne_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_quantize_group_hand_case():
    # amax 896 gives s = 2; x / s: 3 -> 1.5 (0x3C), -896 -> -448 (0xFE), 1 -> 0.5 (0x30),
    # 0.25 -> 0.125 (0x20), 0.001953125 -> 2^-10, a tie between 0 and 2^-9 that goes to 0,
    # 448 -> 224 = 1.75 * 2^7 (exponent field 14, mantissa 6: 0x76).
    x = np.zeros(128, np.float32)
    x[:6] = [3.0, -896.0, 1.0, 0.25, 0.001953125, 448.0]
    codes, s = O.quantize_group(_bf16_bits(x))
    assert s == np.float32(2.0)
    assert list(codes[:6]) == [0x3C, 0xFE, 0x30, 0x20, 0x00, 0x76]
    assert (codes[6:] == 0).all()


def test_quantize_group_quotient_reading():
    # The codes are e4m3(x / s), the inverse of the dequantization (code * s).  amax = 416: s =
    # fp32(416/448) rounds down, and x = -312 gives the fp32 quotient -336 exactly, the midpoint of
    # -320 (0xFA, mantissa 2) and -352 (0xFB, mantissa 3); the tie goes to the even mantissa, 0xFA.
    # A multiplier form x * fp32(448/416) would land just beyond -336 and give 0xFB.
    s_exp = np.float32(np.float32(416.0) / np.float32(448.0))
    assert float(s_exp) < 416.0 / 448.0
    assert np.float32(np.float32(-312.0) / s_exp) == np.float32(-336.0)
    x = np.zeros(128, np.float32)
    x[0], x[1] = 416.0, -312.0
    codes, s = O.quantize_group(_bf16_bits(x))
    assert s == s_exp
    assert codes[0] == 0x7E and codes[1] == 0xFA


def test_quantize_group_tiny_amax():
    # The smallest bf16 magnitudes: amax = 2^-133 (the least bf16 subnormal) and 2^-126.  s stays
    # a nonzero fp32 number (2^-133 / 448 is about 2^-141.8, above the least fp32 subnormal 2^-149),
    # every code is finite (no NaN code 0x7F / 0xFF), the largest magnitude maps to +-448 (0x7E),
    # and zeros in the group stay zero codes.
    for amax in (2.0 ** -133, 2.0 ** -126, 3.0 * 2.0 ** -131):
        x = np.zeros(128, np.float32)
        x[0], x[1], x[2] = amax, -amax, amax / 2
        bits = _bf16_bits(x)
        assert O.bf16_to_f64(bits)[0] == amax
        codes, s = O.quantize_group(bits)
        assert s > 0 and s == np.float32(np.float32(amax) / np.float32(448.0))
        assert codes[0] == 0x7E and codes[1] == 0xFE
        assert (codes & 0x7F != 0x7F).all()
        assert (codes[3:] == 0).all()
        # the half-amax entry: 224 when s is a normal fp32 number (amax / s is then 448)
        if s >= np.float32(2.0 ** -126):
            assert codes[2] == 0x76


def test_quantize_group_scale_max_code_and_error_bound():
    rng = np.random.default_rng(11)
    for trial in range(200):
        mag = 2.0 ** rng.uniform(-20, 20)
        x = (rng.standard_normal(128) * mag).astype(np.float32)
        bits = _bf16_rne_bits(x)
        xv = O.bf16_to_f64(bits)
        codes, s = O.quantize_group(bits)
        amax = np.float32(np.abs(xv).max())
        assert s == np.float32(amax / np.float32(448.0))
        top = int(np.argmax(np.abs(xv)))
        assert codes[top] & 0x7F == 0x7E                             # the largest magnitude is +-448
        deq = O.e4m3fn_to_f64(codes) * float(s)
        y = np.abs(xv) / float(s)
        # half a unit in the last place: 2^-4 relative for normals, 2^-10 absolute (x s) below 2^-6,
        # plus the fp32 rounding of x / s and of s itself
        bound = np.where(y >= 2 ** -6, np.abs(xv) * 2 ** -4, float(s) * 2 ** -10) + np.abs(xv) * 2 ** -22 + 1e-300
        assert (np.abs(deq - xv) <= bound).all(), trial
        assert (np.signbit(deq[xv != 0]) == np.signbit(xv[xv != 0])).all()


def _quant_mutant_multiplier(x_bits):
    """The multiplier form e4m3(x * fp32(448 / amax)): must fail the quotient pin."""
    x = O.bf16_to_f64(x_bits).astype(np.float32)
    amax = np.float32(np.max(np.abs(x)))
    if amax == 0:
        return np.zeros(len(x), dtype=np.uint8), np.float32(0.0)
    s = np.float32(amax / np.float32(448.0))
    r = np.float32(np.float32(448.0) / amax)
    return O.f32_to_e4m3fn((x * r).astype(np.float32)), s


def test_pins_catch_quantizer_multiplier_mutant(monkeypatch):
    monkeypatch.setattr(O, "quantize_group", _quant_mutant_multiplier)
    with pytest.raises(AssertionError):
        test_quantize_group_quotient_reading()


def test_quantize_all_zero_group():
    codes, s = O.quantize_group(np.zeros(128, np.uint16))
    assert s == 0 and (codes == 0).all()
    codes, s = O.quantize_group(np.full(128, 0x8000, np.uint16))     # -0.0 everywhere
    assert s == 0 and (codes == 0).all()


def test_encode_record_layout_and_round_trip():
    rng = np.random.default_rng(3)
    tok = _bf16_rne_bits(rng.standard_normal(576).astype(np.float32) * np.repeat([1, 10, 0.01, 300, 1], [128] * 4 + [64]))
    rec = O.encode_record(tok, O.KV_FP8)
    assert rec.shape == (656,) and rec.dtype == np.uint8
    for g in range(4):
        codes, s = O.quantize_group(tok[128 * g:128 * (g + 1)])
        np.testing.assert_array_equal(rec[128 * g:128 * (g + 1)], codes)
        assert rec[512 + 4 * g:516 + 4 * g].view(np.float32)[0] == s
    np.testing.assert_array_equal(rec[528:].view(np.uint16), tok[512:])
    dec = O.decode_record(rec, O.KV_FP8)
    xv = O.bf16_to_f64(tok)
    np.testing.assert_array_equal(dec[512:], xv[512:])
    scales = np.repeat(rec[512:528].view(np.float32).astype(np.float64), 128)
    assert (np.abs(dec[:512] - xv[:512]) <= np.maximum(np.abs(xv[:512]) * 2 ** -4, scales * 2 ** -10) * 1.0001).all()
    np.testing.assert_array_equal(O.encode_record(tok, O.KV_BF16).view(np.uint16), tok)


def test_cache_write_slots():
    cache = np.full((3, 64, 656), 0xAB, np.uint8)
    rng = np.random.default_rng(5)
    toks = _bf16_rne_bits(rng.standard_normal((4, 576)).astype(np.float32))
    out = O.cache_write(cache, O.KV_FP8, toks, [5, -1, 64 * 3, 130])
    flat = out.reshape(-1, 656)
    np.testing.assert_array_equal(flat[5], O.encode_record(toks[0], O.KV_FP8))
    np.testing.assert_array_equal(flat[130], O.encode_record(toks[3], O.KV_FP8))
    untouched = np.ones(192, bool)
    untouched[[5, 130]] = False
    assert (flat[untouched] == 0xAB).all()
    assert (cache == 0xAB).all()                                       # input not modified


def _rope_tables(angles):
    a = np.asarray(angles, np.float64)
    return np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)


def test_inverse_rope_closed_forms():
    rng = np.random.default_rng(21)
    x = _bf16_rne_bits(rng.standard_normal(64).astype(np.float32))
    xv = O.bf16_to_f64(x)
    one, zero = np.ones(32, np.float32), np.zeros(32, np.float32)
    # angle 0: identity
    np.testing.assert_array_equal(O.inverse_rope(x, one, zero), x)
    # angle pi/2 (cos 0, sin 1 exactly): (a, b) -> (b, -a)
    y = O.bf16_to_f64(O.inverse_rope(x, zero, one))
    np.testing.assert_array_equal(y[0::2], xv[1::2])
    np.testing.assert_array_equal(y[1::2], -xv[0::2])
    # angle pi (cos -1, sin 0): negation
    np.testing.assert_array_equal(O.bf16_to_f64(O.inverse_rope(x, -one, zero)), -xv)
    # angle -pi/2 (cos 0, sin -1): (a, b) -> (-b, a), i.e. the inverse of the pi/2 case
    y = O.bf16_to_f64(O.inverse_rope(x, zero, -one))
    np.testing.assert_array_equal(y[0::2], -xv[1::2])
    np.testing.assert_array_equal(y[1::2], xv[0::2])
    # angle pi/3: cos 1/2 exact in fp32; a pair (1, 0) -> (1/2, -sin)
    c = np.full(32, 0.5, np.float32)
    sn = np.full(32, np.sqrt(3) / 2, np.float32)
    e = np.zeros(64, np.uint16)
    e[0::2] = _bf16_bits(np.ones(32, np.float32))
    y = O.bf16_to_f64(O.inverse_rope(e, c, sn))
    assert (y[0::2] == 0.5).all()
    assert (y[1::2] == O.bf16_to_f64(_bf16_rne_bits(-sn))).all()


def test_inverse_rope_undoes_a_forward_rotation():
    """Rotating by +angle (done here in float64, written out independently of the oracle) and then
    applying the oracle's inverse recovers the input to within the two bf16 roundings."""
    rng = np.random.default_rng(22)
    for trial in range(20):
        ang = rng.uniform(-np.pi, np.pi, 32) * (trial + 1)
        c, s = _rope_tables(ang)
        x = rng.standard_normal(64)
        a, b = x[0::2], x[1::2]
        fwd = np.empty(64)
        fwd[0::2] = a * c.astype(np.float64) - b * s.astype(np.float64)
        fwd[1::2] = a * s.astype(np.float64) + b * c.astype(np.float64)
        fb = _bf16_rne_bits(fwd.astype(np.float32))
        back = O.bf16_to_f64(O.inverse_rope(fb, c, s))
        scale = np.repeat(np.hypot(a, b), 2)
        assert (np.abs(back - x) <= scale * 2.0 ** -6).all(), trial


def test_inverse_rope_rounds_once_to_nearest_even():
    # Exact values on bf16 midpoints (bf16 has 8 significant bits: the spacing above 1 is 2^-7).
    # c = 1, s = 2^-8: the pair (1, 1) gives a*c + b*s = 1 + 2^-8, the midpoint of 1 (0x3F80, even)
    # and 1 + 2^-7 (0x3F81), so 0x3F80; the pair (1, 3) gives 1 + 3 * 2^-8, the midpoint of
    # 1 + 2^-7 (0x3F81) and 1 + 2^-6 (0x3F82, even), so 0x3F82.
    c = np.ones(32, np.float32)
    s = np.full(32, 2.0 ** -8, np.float32)
    x = np.zeros(64, np.float32)
    x[0::2] = 1.0
    x[1::2] = 1.0
    x[2], x[3] = 1.0, 3.0
    y = O.inverse_rope(_bf16_bits(x), c, s)
    assert y[0] == 0x3F80                        # 1 + 2^-8 -> 1.0 (tie, even)
    assert y[2] == 0x3F82                        # 1 + 3 * 2^-8 -> 1.015625 (tie, even)
    # the second entry of the first pair: -1 * 2^-8 + 1 = 0.99609375, exactly a bf16 value (0x3F7F)
    assert y[1] == 0x3F7F


def test_cache_write_with_inverse_rope():
    rng = np.random.default_rng(23)
    toks = _bf16_rne_bits(rng.standard_normal((3, 576)).astype(np.float32))
    ang = rng.uniform(0, 6, (8, 32))
    cos_t, sin_t = _rope_tables(ang)
    pos = [5, 0, 7]
    for kvd, rec in ((O.KV_FP8, 656), (O.KV_BF16, 1152)):
        cache = np.zeros((1, 64, rec), np.uint8)
        out = O.cache_write(cache, kvd, toks, [1, 2, 3], positions=pos, cos_table=cos_t, sin_table=sin_t)
        flat = out.reshape(-1, rec)
        for t in range(3):
            dec = O.decode_record(flat[1 + t], kvd)
            exp_rope = O.bf16_to_f64(O.inverse_rope(toks[t, 512:], cos_t[pos[t]], sin_t[pos[t]]))
            np.testing.assert_array_equal(dec[512:], exp_rope)
            plain = O.decode_record(O.encode_record(toks[t], kvd), kvd)
            np.testing.assert_array_equal(dec[:512], plain[:512])     # the latent part is not rotated


_INVERSE_ROPE = O.inverse_rope


def _rope_mutant_forward(rope_bits, cos, sin):            # rotates by +angle instead of undoing it
    return _INVERSE_ROPE(rope_bits, cos, -np.asarray(sin, np.float32))


def _rope_mutant_half_pairs(rope_bits, cos, sin):         # pairs (i, i + 32) instead of (2i, 2i + 1)
    x = np.asarray(rope_bits, np.uint16)
    inter = np.empty(64, np.uint16)
    inter[0::2], inter[1::2] = x[:32], x[32:]
    y = _INVERSE_ROPE(inter, cos, sin)
    return np.concatenate([y[0::2], y[1::2]])


@pytest.mark.parametrize("mutant", [_rope_mutant_forward, _rope_mutant_half_pairs])
def test_pins_catch_rope_mutants(mutant, monkeypatch):
    monkeypatch.setattr(O, "inverse_rope", mutant)
    caught = 0
    for t in (test_inverse_rope_closed_forms, test_inverse_rope_undoes_a_forward_rotation):
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught >= 1


def _enc_mutant_truncate(x):
    x = np.asarray(x, np.float32).astype(np.float64)
    table = O.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    code = np.clip(np.searchsorted(table, np.abs(x), side="right") - 1, 0, 0x7E)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _enc_mutant_ties_away(x):
    x = np.asarray(x, np.float32).astype(np.float64)
    table = O.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    code = np.where(np.abs(table[hi] - a) <= np.abs(a - table[lo]), hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("mutant", [_enc_mutant_truncate, _enc_mutant_ties_away])
def test_pins_catch_e4m3_encoder_mutants(mutant, monkeypatch):
    monkeypatch.setattr(O, "f32_to_e4m3fn", mutant)
    caught = 0
    for t in (test_e4m3fn_encode_matches_torch_inside_the_range,
              test_e4m3fn_encode_ties_go_to_even_and_large_values_saturate, test_quantize_group_hand_case):
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught >= 1


def test_bf16_record_layout():
    vals = (np.arange(576, dtype=np.float32) % 64 - 32.0) / 4.0  # at most 7 significant bits: bf16-exact
    rec = (vals.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8)
    np.testing.assert_array_equal(O.decode_record(rec, O.KV_BF16), vals)


# ----------------------------------------------------------------------------------------------
# Lengths and gather
# ----------------------------------------------------------------------------------------------

def test_causal_lengths_golden(golden_dir):
    data = json.load(open(os.path.join(golden_dir, "causal_lengths.json")))
    for c in data["cases"]:
        got = O.causal_lengths(c["first_pos"], c["T"])
        if "expected" in c:
            assert got.tolist() == c["expected"], c["name"]
        else:
            assert got[0] == c["expected_first"] and got[-1] == c["expected_last"]
            assert (np.diff(got) == 1).all()


def test_physical_slot_hand_example():
    bt = np.array([5, 2, 9])
    # position 130 is in logical block 2 (-> physical 9) at offset 2
    assert O.physical_slot(bt, 130) == 9 * 64 + 2
    assert O.physical_slot(bt, 0) == 5 * 64
    assert O.physical_slot(bt, 127) == 2 * 64 + 63


def test_gather_round_trips_a_dense_context():
    """Write a dense context into pages through a random block table, then gather it back."""
    rng = np.random.default_rng(2)
    L, npages = 300, 5
    dense = rng.standard_normal((L, 576)).astype(np.float32)
    dense_bits = (dense.view(np.uint32) >> 16).astype(np.uint16)
    perm = rng.permutation(np.arange(1, 9))[:npages]
    kv = np.full((9, 64, 576), 0x7FC0, np.uint16)                # NaN everywhere else
    for p in range(L):
        kv[perm[p // 64], p % 64] = dense_bits[p]
    pos = rng.permutation(L)[:50]
    got = O.gather_tokens(kv.view(np.uint8).reshape(9, 64, 1152), O.KV_BF16, perm, pos)
    np.testing.assert_array_equal(got, O.bf16_to_f64(dense_bits[pos]))


# ----------------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------------

def _bf16_round(x):
    return O.bf16_to_f64((np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16))


def test_attention_two_token_closed_form():
    """q is nonzero only in a rope entry, so the scores are (0, scale*c); the output mixes the
    two latent rows with weights 1/(1+e^x), e^x/(1+e^x); LSE = log(1 + e^x)."""
    rng = np.random.default_rng(0)
    H, c, scale = 3, 2.0, 1.0 / 24.0
    q = np.zeros((H, 576)); q[:, 512] = c * np.array([1.0, -1.0, 4.0])
    K = np.zeros((2, 576)); K[:, :512] = _bf16_round(rng.standard_normal((2, 512)))
    K[1, 512] = 1.0
    Oo, lse = O.attention(q, K, scale)
    for h, mult in enumerate([1.0, -1.0, 4.0]):
        x = scale * c * mult
        w1 = math.exp(x) / (1 + math.exp(x))
        np.testing.assert_allclose(Oo[h], (1 - w1) * K[0, :512] + w1 * K[1, :512], rtol=0, atol=1e-14)
        assert abs(lse[h] - math.log(1 + math.exp(x))) < 1e-14


def test_attention_q_zero_gives_mean_and_log_n():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((37, 576))
    Oo, lse = O.attention(np.zeros((4, 576)), K, 0.1)
    np.testing.assert_allclose(Oo, np.tile(K[:, :512].mean(0), (4, 1)), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(37), atol=1e-13)


def test_attention_weights_sum_to_one():
    """If every value row is the same vector v, the output is v: the weights sum to 1."""
    rng = np.random.default_rng(4)
    K = rng.standard_normal((50, 576)) * 3
    v = rng.standard_normal(512)
    K[:, :512] = v
    Oo, _ = O.attention(rng.standard_normal((8, 576)), K, 1 / 24)
    np.testing.assert_allclose(Oo, np.tile(v, (8, 1)), atol=1e-12)


def test_attention_matches_torch_sdpa_dense():
    """With every context token selected the method is textbook dense softmax attention."""
    rng = np.random.default_rng(6)
    H, n = 16, 200
    q = rng.standard_normal((H, 576)); K = rng.standard_normal((n, 576))
    Oo, lse = O.attention(q, K, 1 / 24)
    qt = torch.from_numpy(q)[None, :, None, :]                   # [1, H, 1, 576]
    kt = torch.from_numpy(K)[None, None].expand(1, H, n, 576)
    vt = torch.from_numpy(K[:, :512].copy())[None, None].expand(1, H, n, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1 / 24)[0, :, 0].numpy()
    np.testing.assert_allclose(Oo, ref, atol=1e-12)
    ref_lse = torch.logsumexp(torch.from_numpy(q @ K.T / 24), dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_attention_order_invariance_and_hull():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 576)); K = rng.standard_normal((64, 576))
    O1, l1 = O.attention(q, K, 1 / 24)
    perm = rng.permutation(64)
    O2, l2 = O.attention(q, K[perm], 1 / 24)
    np.testing.assert_allclose(O1, O2, atol=1e-13); np.testing.assert_allclose(l1, l2, atol=1e-13)
    lo, hi = K[:, :512].min(0), K[:, :512].max(0)
    assert ((O1 >= lo - 1e-12) & (O1 <= hi + 1e-12)).all()


def test_attention_single_token_and_empty():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 576)); K = rng.standard_normal((1, 576))
    Oo, lse = O.attention(q, K, 0.5)
    np.testing.assert_allclose(Oo, np.tile(K[0, :512], (2, 1)), atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (q @ K[0]), atol=1e-13)
    Oe, le = O.attention(q, np.zeros((0, 576)), 0.5)
    assert (Oe == 0).all() and np.isneginf(le).all()


def test_attention_sink_minus_inf_is_no_sink():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((16, 576))
    K = rng.standard_normal((40, 576))
    O0, l0 = O.attention(q, K, 1 / 24)
    O1, l1 = O.attention(q, K, 1 / 24, np.full(16, -np.inf))
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(l0, l1)


def test_attention_sink_is_a_valueless_extra_split():
    # The sink adds e^sink to the denominator and nothing to the numerator: the same as combining the
    # sink-free result with one more split whose output is 0 and whose LSE is the sink.
    rng = np.random.default_rng(22)
    q = rng.standard_normal((16, 576))
    K = rng.standard_normal((50, 576))
    sink = rng.standard_normal(16) * 3
    sink[3] = -np.inf
    O_s, l_s = O.attention(q, K, 1 / 24, sink)
    O_c, l_c = O.split_combine([O.attention(q, K, 1 / 24), (np.zeros((16, 512)), sink)])
    np.testing.assert_allclose(O_s, O_c, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_s, l_c, rtol=1e-13, atol=1e-13)


def test_attention_sink_closed_forms():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, 576))
    K = rng.standard_normal((1, 576))
    s = (q @ K.T)[0, 0] / 24
    sink = np.array([0.7])
    Ov, lv = O.attention(q, K, 1 / 24, sink)
    p = 1.0 / (1.0 + math.exp(sink[0] - s))                        # one token against the sink
    np.testing.assert_allclose(Ov[0], p * K[0, :512], rtol=1e-12)
    assert abs(lv[0] - math.log(math.exp(s) + math.exp(0.7))) < 1e-12
    Oe, le = O.attention(q, np.zeros((0, 576)), 1 / 24, sink)      # no tokens: O = 0, LSE = sink
    assert (Oe == 0).all() and le[0] == 0.7
    Ob, _ = O.attention(q, K, 1 / 24, np.array([500.0]))           # a dominant sink drives O to 0
    assert np.abs(Ob).max() < 1e-100


def test_split_combine_equals_single_pass():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((6, 576)); K = rng.standard_normal((90, 576)) * 2
    full = O.attention(q, K, 1 / 24)
    cuts = [0, 0, 17, 40, 40, 90]                                 # includes empty splits
    parts = [O.attention(q, K[a:b], 1 / 24) for a, b in zip(cuts[:-1], cuts[1:])]
    comb = O.split_combine(parts)
    np.testing.assert_allclose(comb[0], full[0], atol=1e-13)
    np.testing.assert_allclose(comb[1], full[1], atol=1e-13)
    empty = O.split_combine([O.attention(q, K[:0], 1 / 24)] * 3)
    assert (empty[0] == 0).all() and np.isneginf(empty[1]).all()


def test_decode_rows_composes_selection_gather_and_attention():
    """The composed path equals dense attention over exactly the brute-force-selected tokens."""
    rng = np.random.default_rng(12)
    L, H, k = 150, 2, 10
    npages = 3
    perm = np.array([3, 1, 2])
    dense = rng.standard_normal((L, 576)).astype(np.float32)
    bits = (dense.view(np.uint32) >> 16).astype(np.uint16)
    kv = np.full((4, 64, 576), 0x7FC0, np.uint16)
    for p in range(L):
        kv[perm[p // 64], p % 64] = bits[p]
    scores = np.round(rng.standard_normal((1, 160)) * 2) / 2
    q = (rng.standard_normal((1, H, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    idx, Oo, lse = O.decode_rows(q, kv.view(np.uint8).reshape(4, 64, 1152), O.KV_BF16, perm[None],
                                 [0], scores.astype(np.float32), [L], k, 1 / 24)
    sel = brute_topk(scores[0].astype(np.float32).tolist(), L, k)
    assert idx[0].tolist() == sel
    Kd = O.bf16_to_f64(bits[sel])
    qd = O.bf16_to_f64(q[0])
    s = qd @ Kd.T / 24
    p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(Oo[0], p @ Kd[:, :512], atol=1e-13)


# Attention over compressed + sliding-window KV (two paged caches, one softmax).

def _two_cache_case(seed=51, H=4):
    """A main cache and a window cache, one request, small index lists."""
    rng = np.random.default_rng(seed)
    def cache(pages):
        vals = rng.standard_normal((pages, 64, 576)).astype(np.float32)
        return _bf16_rne_bits(vals).view(np.uint8).reshape(pages, 64, 1152)
    kv, kvw = cache(4), cache(4)
    bt = np.array([[2, 0, 3, 1]], np.int32)
    btw = np.array([[0, 0, 2, 1]], np.int32)                 # logical pages 0, 1 evicted (null page 0)
    q = _bf16_rne_bits(rng.standard_normal((1, H, 576)).astype(np.float32))
    idx = np.array([[3, 70, 130, 200, -1, -1]], np.int32)
    idxw = np.array([[150, 151, 190, 250, -1, -1, -1, -1]], np.int32)
    return q, kv, bt, idx, kvw, btw, idxw


def test_window_attention_is_attention_over_the_union():
    q, kv, bt, idx, kvw, btw, idxw = _two_cache_case()
    Ow, L = O.attention_rows_with_window(q, kv, O.KV_BF16, bt, idx, kvw, btw, idxw, [0], 1 / 24)
    K1 = np.stack([O.bf16_to_f64(kv.reshape(-1, 1152)[bt[0][p // 64] * 64 + p % 64].view(np.uint16))
                   for p in idx[0] if p >= 0])
    K2 = np.stack([O.bf16_to_f64(kvw.reshape(-1, 1152)[btw[0][p // 64] * 64 + p % 64].view(np.uint16))
                   for p in idxw[0] if p >= 0])
    K = np.concatenate([K1, K2])
    # dense softmax attention written out with torch in float64
    qt = torch.from_numpy(O.bf16_to_f64(q[0]))
    Kt = torch.from_numpy(K)
    s = (qt @ Kt.T) / 24
    p = torch.softmax(s, dim=1)
    np.testing.assert_allclose(Ow[0], (p @ Kt[:, :512]).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L[0], torch.logsumexp(s, dim=1).numpy(), rtol=1e-12, atol=1e-12)


def test_window_attention_special_cases():
    q, kv, bt, idx, kvw, btw, idxw = _two_cache_case(52)
    # an empty window list is the plain sparse attention over the main cache
    none_w = np.full_like(idxw, -1)
    a = O.attention_rows_with_window(q, kv, O.KV_BF16, bt, idx, kvw, btw, none_w, [0], 1 / 24)
    b = O.attention_rows(q, kv, O.KV_BF16, bt, [0], idx, 1 / 24)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # an empty main list is attention over the window cache alone
    none = np.full_like(idx, -1)
    a = O.attention_rows_with_window(q, kv, O.KV_BF16, bt, none, kvw, btw, idxw, [0], 1 / 24)
    b = O.attention_rows(q, kvw, O.KV_BF16, btw, [0], idxw, 1 / 24)
    np.testing.assert_array_equal(a[0], b[0])
    # the union splits into two disjoint parts whose LSE-weighted combination is the whole
    w = O.attention_rows_with_window(q, kv, O.KV_BF16, bt, idx, kvw, btw, idxw, [0], 1 / 24)
    p1 = O.attention_rows(q, kv, O.KV_BF16, bt, [0], idx, 1 / 24)
    p2 = O.attention_rows(q, kvw, O.KV_BF16, btw, [0], idxw, 1 / 24)
    c = O.split_combine([(p1[0][0], p1[1][0]), (p2[0][0], p2[1][0])])
    np.testing.assert_allclose(w[0][0], c[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(w[1][0], c[1], rtol=1e-12, atol=1e-13)
    # a token moved from the window cache into the main cache (its index moved with it) changes nothing
    kv2 = kv.copy()
    src = btw[0][150 // 64] * 64 + 150 % 64
    kv2.reshape(-1, 1152)[bt[0][4 // 64] * 64 + 4 % 64] = kvw.reshape(-1, 1152)[src]
    idx2 = idx.copy(); idx2[0, 4] = 4
    idxw2 = idxw.copy(); idxw2[0, 0] = -1
    m = O.attention_rows_with_window(q, kv2, O.KV_BF16, bt, idx2, kvw, btw, idxw2, [0], 1 / 24)
    np.testing.assert_allclose(m[0], w[0], rtol=1e-12, atol=1e-13)


def _win_mutant_window_through_main_table(q, kv, kvd, bt, idx, kvw, btw, idxw, rq, scale):
    return O.attention_rows_with_window(q, kv, kvd, bt, idx, kvw, bt, idxw, rq, scale)


def _win_mutant_separate_softmax(q, kv, kvd, bt, idx, kvw, btw, idxw, rq, scale):
    a = O.attention_rows(q, kv, kvd, bt, rq, idx, scale)
    b = O.attention_rows(q, kvw, kvd, btw, rq, idxw, scale)
    return (a[0] + b[0]) / 2, np.logaddexp(a[1], b[1])


@pytest.mark.parametrize("mutant", [_win_mutant_window_through_main_table, _win_mutant_separate_softmax])
def test_pins_catch_window_mutants(mutant):
    q, kv, bt, idx, kvw, btw, idxw = _two_cache_case()
    good = O.attention_rows_with_window(q, kv, O.KV_BF16, bt, idx, kvw, btw, idxw, [0], 1 / 24)
    bad = mutant(q, kv, O.KV_BF16, bt, idx, kvw, btw, idxw, [0], 1 / 24)
    assert not np.allclose(bad[0], good[0], rtol=1e-6, atol=1e-9)


# Attention mutants, planted in copies of the oracle's attention on the CPU: each must fail a pin.

def _att_mutant_v_tail(q, K, scale):            # value taken from the last 512 entries
    s = scale * (q @ K.T); p = np.exp(s - s.max(1, keepdims=True)); l = p.sum(1, keepdims=True)
    return (p / l) @ K[:, -512:], (s.max(1, keepdims=True) + np.log(l))[:, 0]


def _att_mutant_no_scale(q, K, scale):
    return O.attention(q, K, 1.0)


def _att_mutant_log2(q, K, scale):
    Oo, lse = O.attention(q, K, scale)
    return Oo, lse / math.log(2)


def _att_mutant_rope_dropped(q, K, scale):      # scores over the latent part only
    K2 = K.copy(); K2[:, 512:] = 0
    Oo, lse = O.attention(q, K2, scale)
    return Oo, lse


@pytest.mark.parametrize("mutant", [_att_mutant_v_tail, _att_mutant_no_scale, _att_mutant_log2,
                                    _att_mutant_rope_dropped])
def test_pins_catch_attention_mutants(mutant):
    """The two-token closed form (rope-only query) and the SDPA comparison reject each mutant."""
    rng = np.random.default_rng(0)
    H, c, scale = 3, 2.0, 1.0 / 24.0
    q = np.zeros((H, 576)); q[:, 512] = c * np.array([1.0, -1.0, 4.0])
    K = np.zeros((2, 576)); K[:, :512] = _bf16_round(rng.standard_normal((2, 512)))
    K[1, 512] = 1.0
    Oo, lse = mutant(q, K, scale)
    ok_closed = True
    for h, mult in enumerate([1.0, -1.0, 4.0]):
        x = scale * c * mult
        w1 = math.exp(x) / (1 + math.exp(x))
        ok_closed &= bool(np.allclose(Oo[h], (1 - w1) * K[0, :512] + w1 * K[1, :512], atol=1e-12))
        ok_closed &= abs(lse[h] - math.log(1 + math.exp(x))) < 1e-12
    q2 = rng.standard_normal((4, 576)); K2 = rng.standard_normal((30, 576))
    Om, lm = mutant(q2, K2, 1 / 24)
    qt = torch.from_numpy(q2)[None, :, None, :]
    kt = torch.from_numpy(K2)[None, None].expand(1, 4, 30, 576)
    vt = torch.from_numpy(K2[:, :512].copy())[None, None].expand(1, 4, 30, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1 / 24)[0, :, 0].numpy()
    ok_sdpa = bool(np.allclose(Om, ref, atol=1e-10))
    assert not (ok_closed and ok_sdpa)


# ----------------------------------------------------------------------------------------------
# Indexer scores (paged MQA logits)
# ----------------------------------------------------------------------------------------------

def _indexer_hand_inputs(golden_dir):
    with open(os.path.join(golden_dir, "indexer_hand_case.json")) as f:
        case = json.load(f)
    q = np.array(case["q"]); w = np.array(case["w"])
    kidx = np.zeros((case["num_pages"], case["page"], q.shape[1]))
    for e in case["keys"]:
        kidx[e["page"], e["slot"]] = e["k"]
    return case, q, w, kidx


def _indexer_hand_case_holds(fn, golden_dir):
    """True when fn(q, w, kidx, block_table_row, length, stride) reproduces every hand-derived
    value of the fixture and scores 0 at the other positions below the clamped length."""
    case, q, w, kidx = _indexer_hand_inputs(golden_dir)
    for row in case["rows"]:
        got = fn(q, w, kidx, np.array(row["block_table"]), row["length"], row["stride"])
        for p, v in row["expected"].items():
            if not (got[int(p)] == _num(v)):
                return False
        L = min(max(row["length"], 0), row["stride"])
        listed = [p for p in range(L) if row["block_table"][p // 64] >= 0]
        special = {int(p) for p in row["expected"]}
        if any(got[p] != 0.0 for p in listed if p not in special):
            return False
    return True


def test_indexer_golden_hand_case(golden_dir):
    assert _indexer_hand_case_holds(O.indexer_scores_row, golden_dir)


def _brute_indexer(q, w, kidx, bt, length, stride):
    """Pure-Python loops over heads and dims (tiny inputs only)."""
    out = [-math.inf] * stride
    L = min(max(length, 0), stride)
    for p in range(L):
        pg = int(bt[p // 64]) if p // 64 < len(bt) else -1
        if pg < 0 or pg >= kidx.shape[0]:
            continue
        tot = 0.0
        for h in range(len(w)):
            dot = 0.0
            for d in range(q.shape[1]):
                dot += float(q[h, d]) * float(kidx[pg, p % 64, d])
            if dot > 0:
                tot += float(w[h]) * dot
        out[p] = tot
    return np.array(out)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_indexer_matches_brute_force_loops(seed):
    rng = np.random.default_rng(seed)
    Hi, d, npages = 3, 8, 4
    kidx = _bf16_round(rng.standard_normal((npages, 64, d)))
    q = _bf16_round(rng.standard_normal((Hi, d)))
    w = rng.standard_normal(Hi).astype(np.float32).astype(np.float64)
    bt = np.array([2, 0, -1, 3])
    for length, stride in [(150, 200), (64, 64), (255, 256), (0, 10), (300, 256)]:
        got = O.indexer_scores_row(q, w, kidx, bt, length, stride)
        ref = _brute_indexer(q, w, kidx, bt, length, stride)
        fin = np.isfinite(ref)
        np.testing.assert_array_equal(np.isfinite(got), fin)
        np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def _rand_bf16_bits(rng, shape):
    return _bf16_rne_bits(rng.standard_normal(shape).astype(np.float32))


def test_indexer_relu_odd_part_is_a_plain_product():
    """relu(x) - relu(-x) = x, so scores(q) - scores(-q) = sum_h w_h <q_h, k_p>: one matrix
    product over the dense context, gathered here by direct page arithmetic."""
    rng = np.random.default_rng(5)
    R, Hi, npages, L = 2, 16, 6, 300
    kbits = _rand_bf16_bits(rng, (npages, 64, 128))
    qbits = _rand_bf16_bits(rng, (R, Hi, 128))
    w = rng.standard_normal((R, Hi)).astype(np.float32)
    bt = np.array([[4, 1, 5, 0, 2], [3, 2, 1, 0, 4]])
    pos = O.indexer_scores(qbits, w, kbits, bt, [0, 1], [L, L], 320)
    neg = O.indexer_scores(qbits ^ np.uint16(0x8000), w, kbits, bt, [0, 1], [L, L], 320)
    K = O.bf16_to_f64(kbits)
    for r in range(R):
        dense = np.stack([K[bt[r][p >> 6], p & 63] for p in range(L)])            # [L, 128]
        lin = torch.from_numpy(dense) @ torch.from_numpy(O.bf16_to_f64(qbits[r])).T @ \
            torch.from_numpy(w[r].astype(np.float64))
        np.testing.assert_allclose(pos[r, :L] - neg[r, :L], lin.numpy(), rtol=1e-12, atol=1e-10)
        assert np.all(np.isneginf(pos[r, L:])) and np.all(np.isneginf(neg[r, L:]))


def test_indexer_weights_are_linear_and_one_hot_heads_isolate_relu():
    rng = np.random.default_rng(6)
    Hi, d = 4, 128
    kidx = _bf16_round(rng.standard_normal((3, 64, d)))
    q = _bf16_round(rng.standard_normal((Hi, d)))
    w = rng.standard_normal(Hi)
    bt = np.array([1, 2, 0])
    a = O.indexer_scores_row(q, w, kidx, bt, 170, 192)
    np.testing.assert_array_equal(O.indexer_scores_row(q, 2 * w, kidx, bt, 170, 192)[:170], 2 * a[:170])
    np.testing.assert_array_equal(O.indexer_scores_row(q, 0 * w, kidx, bt, 170, 192)[:170], np.zeros(170))
    # one head of weight 1 whose query is the unit vector e_7: the score is relu(k_p[7])
    e = np.zeros((1, d)); e[0, 7] = 1.0
    got = O.indexer_scores_row(e, np.ones(1), kidx, bt, 170, 192)
    k7 = np.array([kidx[bt[p // 64], p % 64, 7] for p in range(170)])
    np.testing.assert_array_equal(got[:170], np.maximum(k7, 0.0))


def test_indexer_page_permutation_invariance():
    """Moving the pages of the cache and rewriting the block table leaves every score as is."""
    rng = np.random.default_rng(7)
    kbits = _rand_bf16_bits(rng, (5, 64, 128))
    qbits = _rand_bf16_bits(rng, (1, 8, 128))
    w = rng.standard_normal((1, 8)).astype(np.float32)
    bt = np.array([[3, 0, 4]])
    perm = np.array([2, 4, 0, 1, 3])                 # new position of old page i
    moved = np.empty_like(kbits); moved[perm] = kbits
    a = O.indexer_scores(qbits, w, kbits, bt, None, [190], 192)
    b = O.indexer_scores(qbits, w, moved, perm[bt], None, [190], 192)
    np.testing.assert_array_equal(a, b)


# Indexer mutants, planted in copies of the oracle's row function on the CPU: each must fail a pin.

def _idx_mutant_relu_after_weight(q, w, kidx, bt, length, stride, page=64):
    out = O.indexer_scores_row(q, w, kidx, bt, length, stride)
    L = min(max(length, 0), stride)
    for p in range(L):
        if np.isfinite(out[p]):
            dots = q @ kidx[bt[p // 64], p % 64]
            out[p] = float(np.sum(np.maximum(w * dots, 0)))
    return out


def _idx_mutant_no_relu(q, w, kidx, bt, length, stride, page=64):
    out = O.indexer_scores_row(q, w, kidx, bt, length, stride)
    L = min(max(length, 0), stride)
    for p in range(L):
        if np.isfinite(out[p]):
            out[p] = float(w @ (q @ kidx[bt[p // 64], p % 64]))
    return out


def _idx_mutant_identity_pages(q, w, kidx, bt, length, stride, page=64):    # block table ignored
    return O.indexer_scores_row(q, w, kidx, np.where(np.asarray(bt) >= 0, np.arange(len(bt)), -1), length, stride)


def _idx_mutant_no_clamp(q, w, kidx, bt, length, stride, page=64):          # negative length wraps
    return O.indexer_scores_row(q, w, kidx, bt, length % stride if length < 0 else length, stride)


@pytest.mark.parametrize("mutant", [_idx_mutant_relu_after_weight, _idx_mutant_no_relu,
                                    _idx_mutant_identity_pages, _idx_mutant_no_clamp])
def test_pins_catch_indexer_mutants(mutant, golden_dir):
    assert not _indexer_hand_case_holds(mutant, golden_dir)


# indexer_error_scale: M[r, p] = sum_h |w_h| sum_d |q_hd| |k_pd|, the magnitude that bounds the GPU
# scores' rounding error.

def _scale_inputs():
    """One row, two index heads of width 128, one page; worked by hand below."""
    q = np.zeros((1, 2, 128), np.float32)
    q[0, 0, :2] = [1.0, -2.0]
    q[0, 1, 1:3] = [3.0, -1.0]
    w = np.array([[-0.5, 2.0]], np.float32)
    k = np.zeros((1, 64, 128), np.float32)
    k[0, 0, :3] = [-4.0, 1.0, 2.0]          # position 0
    k[0, 1, :3] = [1.0, 1.0, 1.0]           # position 1
    bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    return bits(q), w, bits(k), np.array([[0]], np.int32)


def _error_scale_case_holds(fn):
    qb, w, kb, bt = _scale_inputs()
    M = fn(qb, w, kb, bt, [0], [3], 4)
    # position 0: head 0: |1||-4| + |-2||1| = 6; head 1: |3||1| + |-1||2| = 5; M = 0.5*6 + 2*5 = 13
    # position 1: head 0: 1 + 2 = 3; head 1: 3 + 1 = 4; M = 0.5*3 + 2*4 = 9.5
    # position 2: the zero key -> 0; position 3: past the length -> 0
    return M.shape == (1, 4) and M[0].tolist() == [13.0, 9.5, 0.0, 0.0]


def test_indexer_error_scale_hand_case():
    assert _error_scale_case_holds(O.indexer_error_scale)


def test_indexer_error_scale_bounds_scores_and_is_tight_for_nonnegative_terms():
    rng = np.random.default_rng(31)
    Hi, pages = 4, 3
    q = _rand_bf16_bits(rng, (2, Hi, 128))
    k = _rand_bf16_bits(rng, (pages, 64, 128))
    w = rng.standard_normal((2, Hi)).astype(np.float32)
    bt = np.array([[2, 0, 1]], np.int32)
    args = (q, w, k, bt, [0, 0], [150, 190], 192)
    sc, M = O.indexer_scores(*args), O.indexer_error_scale(*args)
    fin = np.isfinite(sc)
    assert (np.abs(sc[fin]) <= M[fin] * (1 + 1e-12)).all()          # triangle inequality
    assert (M[~fin] == 0).all()
    # all-nonnegative inputs: relu is the identity and every term adds up, so score == M
    qa, ka = q & 0x7FFF, k & 0x7FFF
    wa = np.abs(w)
    args = (qa, wa, ka, bt, [0, 0], [150, 190], 192)
    sc, M = O.indexer_scores(*args), O.indexer_error_scale(*args)
    fin = np.isfinite(sc)
    np.testing.assert_allclose(sc[fin], M[fin], rtol=1e-12)


def _es_apply(q_bits, w, kidx_bits, block_table, lengths, stride, f, abs_w=True, abs_qk=True):
    """A planted variant of the error scale on the CPU: f(|w|, |q|, |k|) per scored position."""
    K = O.bf16_to_f64(kidx_bits)
    Q = O.bf16_to_f64(q_bits)
    out = np.zeros((len(lengths), stride))
    for r in range(len(lengths)):
        L = min(max(int(lengths[r]), 0), stride)
        qa = np.abs(Q[r]) if abs_qk else Q[r]
        wa = np.abs(w[r]) if abs_w else np.asarray(w[r], np.float64)
        for p in range(L):
            pg = int(block_table[0][p // 64])
            ka = np.abs(K[pg, p % 64]) if abs_qk else K[pg, p % 64]
            out[r, p] = f(wa, qa, ka)
    return out


def _es_mutant_signed_weights(q_bits, w, kidx_bits, block_table, row_req, lengths, stride, rows=None):
    return _es_apply(q_bits, w, kidx_bits, block_table, lengths, stride, lambda wa, qa, ka: wa @ (qa @ ka),
                     abs_w=False)


def _es_mutant_no_abs_qk(q_bits, w, kidx_bits, block_table, row_req, lengths, stride, rows=None):
    return _es_apply(q_bits, w, kidx_bits, block_table, lengths, stride, lambda wa, qa, ka: wa @ (qa @ ka),
                     abs_qk=False)


def _es_mutant_max_not_sum(q_bits, w, kidx_bits, block_table, row_req, lengths, stride, rows=None):
    return _es_apply(q_bits, w, kidx_bits, block_table, lengths, stride,
                     lambda wa, qa, ka: wa @ (qa * ka).max(axis=1))


def _es_mutant_heads_unweighted(q_bits, w, kidx_bits, block_table, row_req, lengths, stride, rows=None):
    return _es_apply(q_bits, w, kidx_bits, block_table, lengths, stride, lambda wa, qa, ka: (qa @ ka).sum())


@pytest.mark.parametrize("mutant", [_es_mutant_signed_weights, _es_mutant_no_abs_qk, _es_mutant_max_not_sum,
                                    _es_mutant_heads_unweighted])
def test_pins_catch_error_scale_mutants(mutant):
    assert not _error_scale_case_holds(mutant)
