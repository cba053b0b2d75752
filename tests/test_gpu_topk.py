"""GPU parity of topk_per_row against the oracle: bit-exact int32 indices (there is exactly one
correct result), at the workload shapes and on edge cases."""

import numpy as np
import pytest
import torch

import oracle.reference as O
import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import log, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle(scores_cpu: np.ndarray, lengths, k, rows=None):
    return O.topk_rows(scores_cpu, lengths, k, rows=rows)


def _check(scores: torch.Tensor, lengths, k: int, rows=None, what=""):
    log(f"[topk] {what}: {tuple(scores.shape)} k={k}")
    got = smla.topk_per_row(scores, k, lengths=lengths)
    torch.cuda.synchronize()
    s_np = scores.cpu().numpy()
    l_np = None if lengths is None else lengths.cpu().numpy()
    sel = list(range(scores.shape[0])) if rows is None else rows
    ref = _oracle(s_np, l_np, k, rows=sel)
    g = got.cpu().numpy()[sel]
    bad = np.nonzero((g != ref).any(axis=1))[0]
    assert bad.size == 0, f"{what}: rows {[sel[i] for i in bad[:5]]} differ"


def test_tiny_decode_scores_with_ties():
    wl = W.tiny_decode(DEV)
    rs = wl.sets[0]
    _check(rs.scores, rs.lengths, wl.k, what="tiny eighths")


def test_topk_alone_256_levels():
    s = W.topk_levels(DEV)
    _check(s, None, 2048, what="64x65536 levels=256")


def test_decode_shape_rows():
    g = torch.Generator(device=DEV).manual_seed(22)
    lens = W.uniform_int(8192, 65536, 64, g, DEV).to(torch.int32)
    s = torch.randn((64, 65536), generator=g, device=DEV)
    W.poison_score_tails(s, lens)
    _check(s, lens, 2048, what="64 rows L~U[8K,64K]")


def test_fp8_decode_shape_all_rows():
    g = torch.Generator(device=DEV).manual_seed(33)
    lens = W.uniform_int(32768, 131072, 128, g, DEV).to(torch.int32)
    s = torch.randn((128, 131072), generator=g, device=DEV)
    W.poison_score_tails(s, lens)
    _check(s, lens, 2048, what="128 rows L~U[32K,128K] (all rows)")


def test_clustered_candidates():
    """Rows whose best candidates crowd into a narrow band of positions (so far more of them than
    average fall to one 4096-position stretch of the row), rows with the band at the start, middle
    and end, with and without ties, at lengths that fill the registers-resident form; plus plain rows
    in the same batch.  Bit-exact against the oracle."""
    g = torch.Generator(device="cpu").manual_seed(21)
    rows, L = 12, 65536
    s = torch.randn((rows, L), generator=g, dtype=torch.float32)
    lengths = torch.full((rows,), L, dtype=torch.int32)
    for r, (start, width, tied) in enumerate([(0, 4096, False), (8192, 4096, False), (61440, 4096, False),
                                             (30000, 2500, False), (12288, 6000, True), (4000, 1000, True),
                                             (49152, 16384, False), (0, 3000, True)]):
        band = torch.randn((width,), generator=g, dtype=torch.float32).abs() + 4.0
        if tied:
            band = torch.round(band * 4) / 4          # few distinct values: heavy ties inside the band
        s[r, start:start + width] = band
    lengths[8] = 50000                                   # a band ending past the row's length
    s[8, 45000:52000] = 6.0
    lengths[9] = 20000
    s[9, 16000:20000] = torch.randn((4000,), generator=g).abs() + 5.0
    _check(s.to(DEV), lengths.to(DEV), 2048, what="clustered best candidates")


def test_long_rows_one_workgroup_clustered_and_spread():
    """Rows longer than the registers hold (131072 and 200003 candidates), one workgroup per row: spread
    candidates (one pass, every wave listing its own stretch of the row) and candidates crowded into one
    stretch (a wave's list overflows and the row is listed in two passes), with ties, bit-exact against
    the oracle and against the split path."""
    g = torch.Generator(device="cpu").manual_seed(23)
    k = 2048
    for stride in (131072, 200003):
        R = 8
        s = torch.randn((R, stride), generator=g, dtype=torch.float32)
        lens = torch.full((R,), stride, dtype=torch.int32)
        for r, (start, width, tied) in enumerate([(0, 6000, False), (70000, 3000, True), (stride - 5000, 5000, False),
                                                 (12000, 9000, True)]):
            band = torch.randn((width,), generator=g, dtype=torch.float32).abs() + 4.0
            if tied:
                band = torch.round(band * 4) / 4
            s[r, start:start + width] = band
        s[5] = torch.round(s[5] * 2) / 2                       # spread, heavy ties
        lens[6] = 100001                                        # a stretch that ends inside the row
        lens[7] = 70000
        s_d, lens_d = s.to(DEV), lens.to(DEV)
        log(f"[topk] long rows stride={stride}, one workgroup per row")
        whole = smla.topk_per_row(s_d, k, lengths=lens_d, split=False)
        split = smla.topk_per_row(s_d, k, lengths=lens_d)
        torch.cuda.synchronize()
        assert torch.equal(whole, split)
        ref = _oracle(s.numpy(), lens.numpy(), k)
        bad = np.nonzero((whole.cpu().numpy() != ref).any(axis=1))[0]
        assert bad.size == 0, f"stride {stride}: rows {bad[:5].tolist()} differ"


@pytest.mark.parametrize("k", [1, 2, 63, 192, 256, 2000, 2048, 4096, 16384])
def test_k_values_and_ragged_lengths(k):
    g = torch.Generator(device=DEV).manual_seed(1000 + k)
    R, stride = 24, 20000
    lens = torch.tensor([0, -5, 1, k - 1, k, k + 1, 2 * k + 3, stride, stride + 99, 2**31 - 1, 777, 12345,
                         19999, 5, 64, 65, 1023, 1024, 1025, 3000, 4097, 8191, 16385, 100], dtype=torch.int32)
    lens = lens[:R].to(DEV)
    s = torch.round(torch.randn((R, stride), generator=g, device=DEV) * 4) / 4     # ties
    _check(s, lens, k, what=f"ragged k={k}")


def test_special_values_rows():
    g = torch.Generator(device=DEV).manual_seed(7)
    R, L = 8, 5000
    s = torch.randn((R, L), generator=g, device=DEV)
    s[0] = 3.0                                                   # all equal
    s[1, ::3] = float("nan")                                     # NaNs rank last
    s[2, ::7] = float("inf"); s[2, 1::7] = float("-inf")         # infinities
    s[3] = 0.0; s[3, ::2] = -0.0                                 # -0 == +0
    s[4] = torch.arange(L, device=DEV, dtype=torch.float32)      # increasing
    s[5] = -torch.arange(L, device=DEV, dtype=torch.float32)     # decreasing
    s[6] = float("nan")                                          # all NaN
    s[7, :] = torch.round(s[7] * 2) / 2
    _check(s, None, 700, what="special values")


def test_row_offsets_unaligned_and_shared_buffer():
    """Rows addressed through arbitrary (unaligned) element offsets into one buffer, two rows
    sharing storage, and a row repeated: all rows must match the oracle on their own slice."""
    g = torch.Generator(device=DEV).manual_seed(9)
    buf = torch.randn(300001, generator=g, device=DEV)
    offs = torch.tensor([0, 1, 3, 12345, 12346, 250001, 3, 99999], dtype=torch.int64, device=DEV)
    stride = 50000
    lens = torch.tensor([50000, 49999, 300, 40000, 17, 50000, 300, 2049], dtype=torch.int32, device=DEV)
    got = smla.topk_per_row(buf, 2048, lengths=lens, row_offsets=offs, row_stride=stride)
    torch.cuda.synchronize()
    ref = O.topk_rows(buf.cpu().numpy(), lens.cpu().numpy(), 2048, row_offsets=offs.cpu().numpy(),
                      row_stride=stride)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_row_alone_equals_row_in_batch():
    g = torch.Generator(device=DEV).manual_seed(5)
    s = torch.round(torch.randn((16, 30000), generator=g, device=DEV) * 8) / 8
    lens = torch.randint(0, 30001, (16,), generator=g, device=DEV, dtype=torch.int32)
    full = smla.topk_per_row(s, 1024, lengths=lens)
    for r in [0, 7, 15]:
        alone = smla.topk_per_row(s[r:r + 1].contiguous(), 1024, lengths=lens[r:r + 1].contiguous())
        assert torch.equal(alone[0], full[r])
    perm = torch.randperm(16, generator=g, device=DEV)
    shuffled = smla.topk_per_row(s[perm].contiguous(), 1024, lengths=lens[perm].contiguous())
    assert torch.equal(shuffled, full[perm])


def test_causal_lengths_match_oracle():
    for first_pos, T in [(-2, 2), (98, 2), (126976, 4096), (0, 1), (-5000, 3000), (2**31 - 10, 20)]:
        got = smla.fill_causal_lengths(first_pos, T, device=DEV).cpu().numpy()
        ref = np.minimum(O.causal_lengths(first_pos, T), 2**31 - 1)
        assert np.array_equal(got, ref), (first_pos, T)


@pytest.mark.parametrize("stride", [114689, 131072, 200003, 262144, 524288])
def test_chunked_rows_equal_single_workgroup_rows(stride):
    """Few long rows are split into 32768-wide chunks and merged; the result must equal both the
    oracle and the one-workgroup-per-row path, including selections that straddle chunks, ties
    across chunk borders and rows shorter than k."""
    g = torch.Generator(device=DEV).manual_seed(stride)
    k = 2048
    lens = [0, 1, k - 1, k, k + 1, 16383, 16384, 16385, 16384 + k, stride - 1, stride, stride + 5,
            (stride * 3) // 4, 40000, 9000, 2**31 - 1, 32767, 32768, 32769, 32768 + k]
    R = len(lens)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    s = torch.round(torch.randn((R, stride), generator=g, device=DEV) * 2) / 2       # heavy ties
    s[0:4] = 1.0                                            # all equal: the first k indices win
    s[4, 32768 - 1000:] = 50.0                              # winners straddle the first chunk border
    s[17, 32768 - 300:32768 + 300] = 7.0                    # a tie straddling the first chunk border
    s[5, ::5] = float("nan")
    s[6, -k:] = float("inf")
    log(f"[topk] chunked stride={stride}")
    split = smla.topk_per_row(s, k, lengths=lens_t)
    whole = smla.topk_per_row(s, k, lengths=lens_t, split=False)
    torch.cuda.synchronize()
    assert torch.equal(split, whole)
    ref = _oracle(s.cpu().numpy(), lens_t.cpu().numpy(), k)
    g_np = split.cpu().numpy()
    bad = np.nonzero((g_np != ref).any(axis=1))[0]
    assert bad.size == 0, f"rows {bad[:5].tolist()} differ"


def test_chunked_path_with_row_offsets_and_small_workspace():
    """Rows given by offsets into one buffer; a workspace holding two rows runs several launches."""
    g = torch.Generator(device=DEV).manual_seed(5)
    stride, k, R = 131072, 512, 7
    buf = torch.randn(R * stride + 13, generator=g, device=DEV)
    offs = torch.tensor([13 + r * stride - (r % 3) for r in range(R)], dtype=torch.int64, device=DEV)
    lens = torch.tensor([stride, 100000, 513, 512, 16385, 131071, 20000], dtype=torch.int32, device=DEV)
    per_row = smla.topk_workspace(1, k, stride, DEV).numel()
    ws = torch.empty(2 * per_row + 100, dtype=torch.uint8, device=DEV)
    got = smla.topk_per_row(buf, k, lengths=lens, row_offsets=offs, row_stride=stride, rows=R, workspace=ws)
    whole = smla.topk_per_row(buf, k, lengths=lens, row_offsets=offs, row_stride=stride, rows=R, split=False)
    torch.cuda.synchronize()
    assert torch.equal(got, whole)
    b = buf.cpu().numpy()
    ref = O.topk_rows(b, lens.cpu().numpy(), k, row_offsets=offs.cpu().numpy(), row_stride=stride)
    assert np.array_equal(got.cpu().numpy(), ref)
