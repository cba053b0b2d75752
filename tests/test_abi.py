"""C-ABI boundary checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host (before any HIP call) with a message naming the
parameter."""

import ctypes
import os
import re

import pytest

import sparse_mla_attention_topk_amd as smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "smla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return smla.load_library()


def test_every_declared_function_is_exported(lib):
    declared = _header_functions()
    assert len(declared) >= 8
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(declared) == sorted(smla.exported_symbols)


def test_version_and_last_error(lib):
    assert smla.version().startswith("smla")
    assert isinstance(lib.smla_last_error(), bytes)


def _cap(**kw):
    base = dict(max_rows=64, max_k=2048, num_heads=64, max_candidates=65536)
    base.update(kw)
    return smla.Capacity.make(**base)


def test_supported_capacity():
    ok, msg = smla.is_supported(_cap())
    assert ok, msg


@pytest.mark.parametrize("field,value,needle", [
    ("num_heads", 8, "num_heads=8"),
    ("num_heads", 72, "num_heads=72"),
    ("num_heads", 256, "num_heads=256"),
    ("d_qk", 512, "d_qk=512"),
    ("d_v", 576, "d_v=576"),
    ("page_block_size", 16, "page_block_size=16"),
    ("max_k", 0, "max_k=0"),
    ("max_k", 20000, "max_k=20000"),
    ("max_candidates", 0, "max_candidates=0"),
    ("max_rows", 0, "max_rows=0"),
])
def test_unsupported_capacity_names_the_parameter(field, value, needle):
    cap = _cap()
    setattr(cap, field, value)
    ok, msg = smla.is_supported(cap)
    assert not ok
    assert needle in msg
    if field in ("num_heads", "d_qk", "d_v", "page_block_size", "max_k"):
        assert "supported" in msg


def test_workspace_size_derives_from_capacity_only():
    tk, at = smla.workspace_size(_cap(max_rows=64, max_k=2048, num_heads=64, max_candidates=131072))
    assert tk == 64 * (256 + 4 * 12288 * 8)    # rows x (chunk counts + 4 lists of 12288 pairs, 32768-candidate chunks)
    tk_short, _ = smla.workspace_size(_cap(max_rows=64, max_k=2048, num_heads=64, max_candidates=114688))
    assert tk_short == 0                         # rows of at most 114688 candidates are never split
    tk_long, _ = smla.workspace_size(_cap(max_rows=64, max_k=2048, num_heads=64, max_candidates=524289))
    assert tk_long == 0                          # more than 16 chunks: rows are never split
    tk_max, _ = smla.workspace_size(_cap(max_rows=2, max_k=2048, num_heads=64, max_candidates=524288))
    assert tk_max == 2 * (256 + 16 * 12288 * 8)   # 16 chunks, the most a split row has
    tk_many, _ = smla.workspace_size(_cap(max_rows=4096, max_k=512, num_heads=64, max_candidates=120000))
    assert tk_many == 255 * (256 + 4 * 12288 * 8)   # the split serves calls of fewer than 256 rows
    _, at = smla.workspace_size(_cap(max_rows=64, max_k=2048, num_heads=64, max_candidates=65536))
    assert at == 64 * 4 * 64 * (512 * 2 + 4)    # rows x splits x heads x (bf16 partial + fp32 LSE)
    _, at1 = smla.workspace_size(_cap(max_rows=1, max_k=512, num_heads=64))
    assert at1 == 0                              # a single split needs no partials
    _, at2 = smla.workspace_size(_cap(max_rows=3, max_k=513, num_heads=16))
    assert at2 == 3 * 2 * 16 * (512 * 2 + 4)
    _, at3 = smla.workspace_size(_cap(max_rows=2, max_k=2048, num_heads=64, kv_dtype=smla.KV_FP8))
    # FP8 caches: splits of 1024 slots, fp16 partials and fp32 LSEs, then 4 fp32 group factors per split
    assert at3 == 2 * (2 * 64 * (512 * 2 + 4) + 2 * 4 * 4)


P = ctypes.c_void_p


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_topk_validation(lib):
    f = lib.smla_topk_per_row
    st = f(_fake(0x1000), None, 100, None, 4, 0, _fake(0x2000), None, 0, None)
    assert st == 2 and b"k=0" in lib.smla_last_error()
    st = f(_fake(0x1000), None, 0, None, 4, 8, _fake(0x2000), None, 0, None)
    assert st == 5 and b"row_stride=0" in lib.smla_last_error()
    st = f(_fake(0x1000), None, 100, None, -1, 8, _fake(0x2000), None, 0, None)
    assert st == 1 and b"rows=-1" in lib.smla_last_error()
    st = f(None, None, 100, None, 4, 8, _fake(0x2000), None, 0, None)
    assert st == 1 and b"scores is NULL" in lib.smla_last_error()
    st = f(_fake(0x1002), None, 100, None, 4, 8, _fake(0x2000), None, 0, None)
    assert st == 4 and b"scores" in lib.smla_last_error()
    st = f(_fake(0x1000), _fake(0x3004), 100, None, 4, 8, _fake(0x2000), None, 0, None)
    assert st == 4 and b"row_offsets" in lib.smla_last_error()
    # zero rows is a valid no-op that touches nothing
    assert f(None, None, 100, None, 0, 8, None, None, 0, None) == 0


def _decode(lib, **kw):
    a = dict(q=0x10000, q_row_stride=64 * 576, kv=0x20000, kv_dtype=0, num_pages=10, bt=0x30000, bt_stride=4,
             num_reqs=1, row_req=None, idx=0x40000, rows=2, H=64, k=2048, scale=1 / 24, out=0x50000, lse=None,
             ws=0x60000, ws_bytes=1 << 30)
    a.update(kw)
    c = lambda v: None if v is None else _fake(v)
    return lib.smla_sparse_mla_decode(c(a["q"]), a["q_row_stride"], c(a["kv"]), a["kv_dtype"], a["num_pages"],
                                      c(a["bt"]), a["bt_stride"], a["num_reqs"], c(a["row_req"]), c(a["idx"]),
                                      a["rows"], a["H"], a["k"], a["scale"], c(a.get("sink")), c(a["out"]),
                                      c(a["lse"]), c(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(H=24), 2, b"num_heads=24"),
    (dict(k=0), 2, b"k=0"),
    (dict(kv_dtype=7), 2, b"kv_dtype=7"),
    (dict(rows=-3), 1, b"rows=-3"),
    (dict(num_pages=0), 1, b"num_pages=0"),
    (dict(num_pages=1 << 40), 5, b"num_pages="),
    (dict(scale=0.0), 1, b"softmax_scale"),
    (dict(scale=float("nan")), 1, b"softmax_scale"),
    (dict(q_row_stride=100), 1, b"q_row_stride=100"),
    (dict(q=None), 1, b"q is NULL"),
    (dict(idx=None), 1, b"idx is NULL"),
    (dict(q=0x10008), 4, b"q must be 16-byte aligned"),
    (dict(q_row_stride=64 * 576 + 4), 4, b"q_row_stride"),
    (dict(out=0x50004), 4, b"out must be 16-byte aligned"),
    (dict(ws=None), 3, b"ws is NULL"),
    (dict(ws_bytes=100), 3, b"ws_bytes=100"),
    (dict(ws=0x60010), 4, b"ws must be 256-byte aligned"),
    (dict(sink=0x70002), 4, b"sink must be 4-byte aligned"),
])
def test_decode_validation(lib, kw, status, needle):
    st = _decode(lib, **kw)
    assert st == status, lib.smla_last_error()
    assert needle in lib.smla_last_error()


def test_decode_zero_rows_is_noop(lib):
    assert _decode(lib, rows=0, q=None, idx=None, out=None) == 0


def test_single_split_needs_no_workspace(lib):
    # k <= 512 is one split: no workspace pointer needed; validation passes up to the launch, which is
    # not reached here because rows=0.
    assert _decode(lib, k=512, ws=None, ws_bytes=0, rows=0) == 0


def test_python_binding_requires_gpu_tensors():
    import torch
    with pytest.raises(ValueError):
        smla.topk_per_row(torch.zeros((2, 8)), 2)


def test_kv_cache_write_validation(lib):
    f = lib.smla_kv_cache_write
    P = _fake
    st = f(P(0x1000), 576, P(0x2000), 4, P(0x3000), 9, 10, None)
    assert st == 2 and b"kv_dtype=9" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2000), -1, P(0x3000), 1, 10, None)
    assert st == 1 and b"T=-1" in lib.smla_last_error()
    st = f(P(0x1000), 500, P(0x2000), 4, P(0x3000), 1, 10, None)
    assert st == 1 and b"in_row_stride=500" in lib.smla_last_error()
    st = f(P(0x1000), 580, P(0x2000), 4, P(0x3000), 1, 10, None)
    assert st == 4 and b"in_row_stride=580" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2000), 4, P(0x3000), 1, 0, None)
    assert st == 1 and b"num_pages=0" in lib.smla_last_error()
    st = f(P(0x1000), 576, None, 4, P(0x3000), 1, 10, None)
    assert st == 1 and b"slot_mapping is NULL" in lib.smla_last_error()
    st = f(P(0x1008), 576, P(0x2000), 4, P(0x3000), 1, 10, None)
    assert st == 4 and b"kv_in must be 16-byte aligned" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2004), 4, P(0x3000), 1, 10, None)
    assert st == 4 and b"slot_mapping" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2000), 4, P(0x3008), 1, 10, None)
    assert st == 4 and b"cache must be 16-byte aligned" in lib.smla_last_error()
    assert f(None, 576, None, 0, None, 1, 10, None) == 0        # T = 0: nothing to do


def test_kv_cache_write_rope_validation(lib):
    """The inverse-RoPE write checks its own arguments on the host before enqueueing anything (the
    cache-write checks it shares are covered above)."""
    f = lib.smla_kv_cache_write_rope
    P = _fake
    # kv_in, in_row_stride, slot_mapping, positions, cos_sin, max_pos, T, cache, kv_dtype, num_pages, stream
    st = f(P(0x1000), 576, P(0x2000), None, P(0x5000), 64, 4, P(0x3000), 1, 10, None)
    assert st == 1 and b"positions is NULL" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2000), P(0x4000), None, 64, 4, P(0x3000), 1, 10, None)
    assert st == 1 and b"cos_sin is NULL" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2000), P(0x4000), P(0x5000), 0, 4, P(0x3000), 1, 10, None)
    assert st == 1 and b"max_pos=0" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2000), P(0x4004), P(0x5000), 64, 4, P(0x3000), 1, 10, None)
    assert st == 4 and b"positions must be 8-byte aligned" in lib.smla_last_error()
    st = f(P(0x1000), 576, P(0x2000), P(0x4000), P(0x5002), 64, 4, P(0x3000), 1, 10, None)
    assert st == 4 and b"cos_sin must be 4-byte aligned" in lib.smla_last_error()
    st = f(P(0x1008), 576, P(0x2000), P(0x4000), P(0x5000), 64, 4, P(0x3000), 1, 10, None)
    assert st == 4 and b"kv_in must be 16-byte aligned" in lib.smla_last_error()
    assert f(None, 576, None, None, None, 64, 0, None, 1, 10, None) == 0   # T = 0: nothing to do


def test_paged_mqa_logits_validation(lib):
    f = lib.smla_paged_mqa_logits
    P = _fake

    def call(q=0x1000, qs=8192, w=0x2000, ws=64, k=0x3000, npages=10, bt=0x4000, bts=4, nreq=1, rreq=None,
             lens=None, rows=2, Hi=64, out=0x5000, ostride=256):
        return f(P(q) if q else None, qs, P(w) if w else None, ws, P(k) if k else None, npages,
                 P(bt) if bt else None, bts, nreq, P(rreq) if rreq else None, P(lens) if lens else None, rows, Hi,
                 P(out) if out else None, ostride, None)

    assert call(Hi=8) == 2 and b"Hi=8" in lib.smla_last_error()
    assert call(Hi=80) == 2 and b"Hi=80" in lib.smla_last_error()
    assert call(rows=-1) == 1 and b"rows=-1" in lib.smla_last_error()
    assert call(ostride=0) == 5 and b"out_stride=0" in lib.smla_last_error()
    assert call(npages=0) == 1 and b"num_pages=0" in lib.smla_last_error()
    assert call(bts=0) == 1 and b"bt_stride=0" in lib.smla_last_error()
    assert call(nreq=0) == 1 and b"num_reqs=0" in lib.smla_last_error()
    assert call(qs=100) == 1 and b"q_row_stride=100" in lib.smla_last_error()
    assert call(ws=32) == 1 and b"w_row_stride=32" in lib.smla_last_error()
    assert call(q=0) == 1 and b"q is NULL" in lib.smla_last_error()
    assert call(w=0) == 1 and b"weights is NULL" in lib.smla_last_error()
    assert call(k=0) == 1 and b"kidx is NULL" in lib.smla_last_error()
    assert call(out=0) == 1 and b"out is NULL" in lib.smla_last_error()
    assert call(q=0x1008) == 4 and b"q must be 16-byte aligned" in lib.smla_last_error()
    assert call(qs=8196) == 4 and b"q_row_stride=8196" in lib.smla_last_error()
    assert call(w=0x2004) == 4 and b"weights must be 16-byte aligned" in lib.smla_last_error()
    assert call(ws=66) == 4 and b"w_row_stride=66" in lib.smla_last_error()
    assert call(k=0x3008) == 4 and b"kidx must be 16-byte aligned" in lib.smla_last_error()
    assert call(lens=0x6002) == 4 and b"lengths" in lib.smla_last_error()
    assert call(out=0x5002) == 4 and b"out must be 4-byte aligned" in lib.smla_last_error()
    assert call(rows=0, q=0, w=0, k=0, bt=0, out=0) == 0          # rows = 0: nothing to do
