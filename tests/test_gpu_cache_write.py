"""GPU parity of smla_kv_cache_write against the oracle: FP8 records (e4m3 codes, fp32 group scales,
rope) and bf16 records must be byte-identical to the oracle's encoding; skipped slots and every other
record stay untouched; records written by the kernel decode back through sparse_mla_decode."""

import numpy as np
import pytest
import torch

import oracle.reference as O
import sparse_mla_attention_topk_amd as smla
from sparse_mla_attention_topk_amd import workloads as W
from tests.helpers import assert_attention_close, bf16_bits_np, kv_np, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FILL = 0xAB


def _cache(num_pages, kv_dtype):
    rec = 656 if kv_dtype == W.KV_FP8 else 1152
    return torch.full((num_pages, 64, rec), FILL, dtype=torch.uint8, device=DEV)


def _expected(cache_np, kv_dtype, tok_bits, slots):
    return O.cache_write(cache_np, kv_dtype, tok_bits, slots)


@pytest.mark.parametrize("kv_dtype", [W.KV_FP8, W.KV_BF16])
def test_records_match_oracle_bytes(kv_dtype):
    log(f"cache write parity kv_dtype={kv_dtype} T=1000")
    wl = W.cache_write_tokens(DEV, T=1000, num_pages=40, seed=5)
    slots = wl.slots.clone()
    slots[7] = -1                      # padding token
    slots[8] = 40 * 64                 # one past the cache: skipped
    slots[9] = -(1 << 40)
    cache = _cache(wl.num_pages, kv_dtype)
    before = kv_np(cache)
    smla.kv_cache_write(wl.tokens, slots, cache, kv_dtype=kv_dtype)
    torch.cuda.synchronize()
    exp = _expected(before, kv_dtype, bf16_bits_np(wl.tokens), slots.cpu().numpy())
    got = kv_np(cache)
    bad = np.argwhere((got != exp).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} records differ, first at {bad[:4].tolist()}"


def test_fp8_ties_subnormals_and_zero_groups():
    # Groups built so that x / s lands exactly on e4m3 midpoints (ties to even), in the subnormal
    # range, at +-448, and an all-zero group and a group of -0.0.
    table = O.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (table[:-1] + table[1:]) / 2                                # 126 midpoints, bf16-exact
    T = 8
    tok = np.zeros((T, 576), np.float32)
    for t in range(T):
        s = 2.0 ** (t - 4)                                             # power-of-two scale: x / s exact
        grp = np.concatenate([[448.0], mids, [-448.0]])[:128]
        tok[t, :128] = grp * s
        tok[t, 128:256] = -grp[::-1] * s
        tok[t, 256:384] = np.concatenate([[448.0], table[1:16], -table[1:16], np.zeros(97)]) * s   # subnormal codes
        tok[t, 384:512] = 0.0 if t % 2 == 0 else -0.0
        tok[t, 512:] = np.arange(64) - 31.5
    bits = (tok.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f64(bits), tok.astype(np.float64)), "inputs must be bf16-exact"
    tokens = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    slots = torch.arange(T, dtype=torch.int64, device=DEV) * 3 + 64
    cache = _cache(4, W.KV_FP8)
    before = kv_np(cache)
    smla.kv_cache_write(tokens, slots, cache, kv_dtype=W.KV_FP8)
    torch.cuda.synchronize()
    exp = _expected(before, W.KV_FP8, bits, slots.cpu().numpy())
    np.testing.assert_array_equal(kv_np(cache), exp)


def test_strided_input_and_token_independence():
    wl = W.cache_write_tokens(DEV, T=333, num_pages=10, seed=6)
    wide = torch.zeros((333, 640), dtype=torch.bfloat16, device=DEV)
    wide[:, :576] = wl.tokens
    view = wide[:, :576]
    a = _cache(10, W.KV_FP8)
    smla.kv_cache_write(view, wl.slots, a, kv_dtype=W.KV_FP8)
    b = _cache(10, W.KV_FP8)
    for lo, hi in [(0, 1), (1, 100), (100, 333)]:                      # the same tokens in three calls
        smla.kv_cache_write(wl.tokens[lo:hi], wl.slots[lo:hi], b, kv_dtype=W.KV_FP8)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    exp = _expected(np.full((10, 64, 656), FILL, np.uint8), W.KV_FP8, bf16_bits_np(wl.tokens), wl.slots.cpu().numpy())
    np.testing.assert_array_equal(kv_np(a), exp)


def test_zero_tokens_is_noop():
    cache = _cache(2, W.KV_FP8)
    smla.kv_cache_write(torch.zeros((0, 576), dtype=torch.bfloat16, device=DEV),
                        torch.zeros(0, dtype=torch.int64, device=DEV), cache)
    torch.cuda.synchronize()
    assert (cache == FILL).all()


def test_large_prefill_write_sampled():
    T, pages = 65536, 1100
    log(f"cache write sampled parity T={T}")
    wl = W.cache_write_tokens(DEV, T=T, num_pages=pages, seed=7)
    cache = torch.zeros((pages, 64, 656), dtype=torch.uint8, device=DEV)
    smla.kv_cache_write(wl.tokens, wl.slots, cache)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    pick = rng.choice(T, 256, replace=False)
    toks = bf16_bits_np(wl.tokens[torch.from_numpy(pick).to(DEV)])
    slots = wl.slots.cpu().numpy()[pick]
    flat = cache.view(-1, 656)
    got = flat[torch.from_numpy(slots).to(DEV)].cpu().numpy()
    for i in range(len(pick)):
        np.testing.assert_array_equal(got[i], O.encode_record(toks[i], O.KV_FP8), err_msg=f"token {pick[i]}")


def test_written_records_feed_the_fp8_decode():
    # A context written by the kernel, then attended over: compared with the oracle on the written bytes
    # and, through the oracle's exact dequantization, within the FP8 bound of the bf16 tokens themselves.
    ctx, H, k = 3000, 64, 1024
    npages = (ctx + 63) // 64 + 1
    wl = W.cache_write_tokens(DEV, T=ctx, num_pages=npages, seed=8, spread=2.0)
    slots = torch.arange(ctx, dtype=torch.int64, device=DEV) + 64      # pages 1.. in order
    cache = torch.zeros((npages, 64, 656), dtype=torch.uint8, device=DEV)
    smla.kv_cache_write(wl.tokens, slots, cache)
    bt = (torch.arange(npages - 1, dtype=torch.int32, device=DEV) + 1).view(1, -1)
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    rows = 4
    q = torch.randn((rows, H, 576), generator=g, device=DEV).to(torch.bfloat16)
    scores = torch.randn((rows, ctx), generator=g, device=DEV)
    idx = smla.topk_per_row(scores, k)
    lse = torch.empty((rows, H), dtype=torch.float32, device=DEV)
    out, _ = smla.sparse_mla_decode(q, cache, bt, idx, 1 / 24, lse=lse, kv_dtype=W.KV_FP8)
    torch.cuda.synchronize()
    O_ref, lse_ref = O.attention_rows(bf16_bits_np(q), kv_np(cache), O.KV_FP8, bt.cpu().numpy(), None,
                                      idx.cpu().numpy(), 1 / 24)
    assert_attention_close(out, lse, O_ref, lse_ref, "fp8 decode over written records", relative=True)


def test_fp8_tiny_amax_groups():
    # Groups whose largest magnitude is among the smallest bf16 values (down to the least subnormal
    # 2^-133): the quotient x / s stays defined (s is a nonzero fp32 number), every code is finite and
    # the bytes equal the oracle's.
    T = 6
    tok = np.zeros((T, 576), np.float32)
    amaxes = [2.0 ** -133, 2.0 ** -130, 3.0 * 2.0 ** -131, 2.0 ** -126, 2.0 ** -120, 2.0 ** -100]
    rng = np.random.default_rng(12)
    for t, a in enumerate(amaxes):
        for g in range(4):
            m = rng.integers(-8, 9, 128).astype(np.float64) / 8.0        # multiples of 1/8 in [-1, 1]
            m[0] = 1.0
            tok[t, 128 * g:128 * (g + 1)] = (m * a).astype(np.float32)
        tok[t, 512:] = rng.standard_normal(64).astype(np.float32)
    bits = (tok.view(np.uint32) >> 16).astype(np.uint16)
    tokens = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    slots = torch.arange(T, dtype=torch.int64, device=DEV) + 64
    cache = _cache(2, W.KV_FP8)
    before = kv_np(cache)
    smla.kv_cache_write(tokens, slots, cache, kv_dtype=W.KV_FP8)
    torch.cuda.synchronize()
    got = kv_np(cache)
    exp = _expected(before, W.KV_FP8, bits, slots.cpu().numpy())
    np.testing.assert_array_equal(got, exp)
    codes = got.reshape(-1, 656)[64:64 + T, :512]
    assert ((codes & 0x7F) != 0x7F).all()


def _bf16_order(bits):
    b = np.asarray(bits, np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


@pytest.mark.parametrize("kv_dtype,T", [(W.KV_FP8, 384), (W.KV_BF16, 384), (W.KV_FP8, 37), (W.KV_BF16, 37)])
def test_inverse_rope_cache_write(kv_dtype, T):
    """Inverse-RoPE write against the oracle; T = 37 leaves the last wave of two tokens half empty."""
    pages, max_pos = 12, 70000
    log(f"inverse-rope cache write kv_dtype={kv_dtype} T={T}")
    wl = W.cache_write_tokens(DEV, T=T, num_pages=pages, seed=15, spread=3.0)
    g = torch.Generator(device="cpu").manual_seed(16)
    pos = torch.randint(0, max_pos, (T,), generator=g, dtype=torch.int64)
    pos[5], pos[6] = -1, max_pos                          # outside the table: not written
    pos = pos.to(DEV)
    cs = W.rope_cos_sin(max_pos, DEV)
    cache = _cache(pages, kv_dtype)
    before = kv_np(cache)
    smla.kv_cache_write(wl.tokens, wl.slots, cache, kv_dtype=kv_dtype, positions=pos, cos_sin=cs)
    torch.cuda.synchronize()
    got = kv_np(cache).reshape(-1, cache.shape[-1])
    bits = bf16_bits_np(wl.tokens)
    csn = cs.cpu().numpy()
    slots = wl.slots.cpu().numpy()
    pn = pos.cpu().numpy()
    rope_off = 528 if kv_dtype == W.KV_FP8 else 1024
    exact = 0
    worst = 0
    for t in range(T):
        rec = got[slots[t]]
        if pn[t] < 0 or pn[t] >= max_pos:
            assert (rec == FILL).all(), t
            continue
        ref = O.encode_record(bits[t], kv_dtype, csn[pn[t], :32], csn[pn[t], 32:])
        np.testing.assert_array_equal(rec[:rope_off], ref[:rope_off], err_msg=f"token {t}: latent part")
        d = np.abs(_bf16_order(rec[rope_off:].view(np.uint16)) - _bf16_order(ref[rope_off:].view(np.uint16)))
        worst = max(worst, int(d.max()))
        exact += int((d == 0).sum())
    log(f"[cache write rope] kv_dtype={kv_dtype}: {exact} of {(T - 2) * 64} rope values bit-exact, "
        f"largest difference {worst} bf16 units")
    assert worst <= 1
    untouched = np.ones(got.shape[0], bool)
    untouched[slots] = False
    assert (got[untouched] == FILL).all()
