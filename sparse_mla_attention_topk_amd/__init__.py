"""Deterministic, batch-invariant sparse MLA for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/smla.h`` (``libsmla.so``, built in-tree by
``sparse_mla_attention_topk_amd.build``).  This module only marshals arguments: torch tensors
provide device memory and the current HIP stream; every step of the computation runs in the HIP
kernels of the library.  There is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "SmlaError", "KV_BF16", "KV_FP8", "Capacity", "library_path", "load_library", "exported_symbols",
    "version", "is_supported", "workspace_size", "fill_causal_lengths", "topk_per_row", "topk_workspace",
    "sparse_mla_decode", "sparse_mla_decode_noalloc", "sparse_mla_decode_with_window", "sparse_mla_prefill_chunk",
    "kv_cache_write",
    "paged_mqa_logits",
]

KV_BF16 = 0
KV_FP8 = 1

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None

exported_symbols = (
    "smla_last_error", "smla_version", "smla_is_supported", "smla_workspace_size",
    "smla_fill_causal_lengths", "smla_topk_per_row", "smla_sparse_mla_decode",
    "smla_sparse_mla_prefill_chunk", "smla_kv_cache_write", "smla_kv_cache_write_rope", "smla_paged_mqa_logits",
    "smla_sparse_mla_decode_noalloc", "smla_sparse_mla_decode_with_window",
)

_STATUS = {0: "SMLA_OK", 1: "SMLA_ERR_INVALID_ARG", 2: "SMLA_ERR_UNSUPPORTED", 3: "SMLA_ERR_WORKSPACE",
           4: "SMLA_ERR_ALIGNMENT", 5: "SMLA_ERR_CAPACITY", 6: "SMLA_ERR_HIP"}


class SmlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Capacity(ctypes.Structure):
    _fields_ = [("max_rows", ctypes.c_int32), ("max_k", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("page_block_size", ctypes.c_int32),
                ("max_candidates", ctypes.c_int64), ("kv_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    @classmethod
    def make(cls, max_rows: int, max_k: int, num_heads: int, max_candidates: int, kv_dtype: int = KV_BF16,
             d_qk: int = 576, d_v: int = 512, page_block_size: int = 64) -> "Capacity":
        return cls(max_rows, max_k, num_heads, d_qk, d_v, page_block_size, max_candidates, kv_dtype, 0)


def library_path() -> str:
    return os.path.join(_PKG_DIR, "libsmla.so")


def load_library() -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run `python -m sparse_mla_attention_topk_amd.build`)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "smla_last_error": ([], ctypes.c_char_p),
        "smla_version": ([], ctypes.c_char_p),
        "smla_is_supported": ([ctypes.POINTER(Capacity)], ctypes.c_int),
        "smla_workspace_size": ([ctypes.POINTER(Capacity), ctypes.POINTER(SZ), ctypes.POINTER(SZ)], ctypes.c_int),
        "smla_fill_causal_lengths": ([I64, I32, P, P], ctypes.c_int),
        "smla_topk_per_row": ([P, P, I64, P, I32, I32, P, P, SZ, P], ctypes.c_int),
        "smla_sparse_mla_decode": ([P, I64, P, I32, I64, P, I64, I32, P, P, I32, I32, I32, F32, P, P, P, P, SZ,
                                    P], ctypes.c_int),
        "smla_sparse_mla_prefill_chunk": ([P, I64, P, I32, I64, P, I64, P, I32, I32, I32, F32, P, P, P, P, SZ, P],
                                          ctypes.c_int),
        "smla_sparse_mla_decode_noalloc": ([P, I64, P, I32, I64, P, I64, I32, P, P, I32, I32, I32, F32, P, P, P, P],
                                           ctypes.c_int),
        "smla_sparse_mla_decode_with_window": ([P, I64, P, I32, I64, P, I64, P, I32, P, I64, P, I64, P, I32, I32, P,
                                                I32, I32, F32, P, P, P, P, SZ, P], ctypes.c_int),
        "smla_kv_cache_write": ([P, I64, P, I32, P, I32, I64, P], ctypes.c_int),
        "smla_kv_cache_write_rope": ([P, I64, P, P, P, I64, I32, P, I32, I64, P], ctypes.c_int),
        "smla_paged_mqa_logits": ([P, I64, P, I64, P, I64, P, I64, I32, P, P, I32, I32, P, I64, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().smla_last_error().decode()
        raise SmlaError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t: torch.Tensor, name: str, dtype, device=None, contiguous: bool = True) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def version() -> str:
    return load_library().smla_version().decode()


def is_supported(cap: Capacity) -> Tuple[bool, str]:
    lib = load_library()
    st = lib.smla_is_supported(ctypes.byref(cap))
    return st == 0, ("" if st == 0 else lib.smla_last_error().decode())


def workspace_size(cap: Capacity) -> Tuple[int, int]:
    lib = load_library()
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.smla_workspace_size(ctypes.byref(cap), ctypes.byref(a), ctypes.byref(b)))
    return int(a.value), int(b.value)


def fill_causal_lengths(first_pos: int, T: int, out: Optional[torch.Tensor] = None,
                        device=None) -> torch.Tensor:
    """lengths[t] = max(0, first_pos + t + 1) for a chunk of T query tokens starting at first_pos."""
    lib = load_library()
    if out is None:
        out = torch.empty(T, dtype=torch.int32, device=device or "cuda")
    _require(out, "out", torch.int32)
    if out.numel() < T:
        raise ValueError("out is shorter than T")
    _check(lib.smla_fill_causal_lengths(int(first_pos), int(T), _ptr(out), _stream(out.device)))
    return out


def topk_per_row(scores: torch.Tensor, k: int, lengths: Optional[torch.Tensor] = None,
                 row_offsets: Optional[torch.Tensor] = None, row_stride: Optional[int] = None,
                 rows: Optional[int] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, split: bool = True) -> torch.Tensor:
    """Stable top-k of each row, ascending indices, -1 padded: int32 [rows, k].

    ``workspace`` (uint8, 256-byte aligned) lets few long rows split over several workgroups; when
    None one is allocated if the split applies, unless ``split`` is False (then no workspace is
    passed and every row is one workgroup).  The result is the same either way.

    ``scores`` is fp32; either 2-D [rows, stride] (row r at r*stride) or any contiguous buffer
    addressed through ``row_offsets`` (int64 element offsets) with ``row_stride`` entries per row.
    """
    lib = load_library()
    _require(scores, "scores", torch.float32)
    if row_offsets is None:
        if scores.dim() != 2:
            raise ValueError("scores must be 2-D when row_offsets is not given")
        rows = scores.shape[0] if rows is None else rows
        row_stride = scores.shape[1] if row_stride is None else row_stride
    else:
        _require(row_offsets, "row_offsets", torch.int64, scores.device)
        rows = row_offsets.numel() if rows is None else rows
        if row_stride is None:
            raise ValueError("row_stride is required with row_offsets")
    if lengths is not None:
        _require(lengths, "lengths", torch.int32, scores.device)
        if lengths.numel() < rows:
            raise ValueError("lengths is shorter than rows")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    _require(out, "out", torch.int32, scores.device)
    if out.numel() < rows * k:
        raise ValueError("out is smaller than rows*k")
    if workspace is None and split:
        workspace = topk_workspace(rows, k, row_stride, scores.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.smla_topk_per_row(_ptr(scores), _ptr(row_offsets), int(row_stride), _ptr(lengths), int(rows), int(k),
                                 _ptr(out), _ptr(workspace), ws_bytes, _stream(scores.device)))
    return out


def _attn_outputs(rows: int, H: int, device, out, lse):
    if out is None:
        out = torch.empty((rows, H, 512), dtype=torch.bfloat16, device=device)
    _require(out, "out", torch.bfloat16, device)
    if out.numel() < rows * H * 512:
        raise ValueError("out is smaller than rows*H*512")
    if lse is not None:
        _require(lse, "lse", torch.float32, device)
        if lse.numel() < rows * H:
            raise ValueError("lse is smaller than rows*H")
    return out, lse


def _check_sink(sink: Optional[torch.Tensor], H: int, device) -> None:
    if sink is not None:
        _require(sink, "sink", torch.float32, device)
        if sink.numel() < H:
            raise ValueError("sink is shorter than H")


def _kv_dtype_of(kv: torch.Tensor, kv_dtype: Optional[int]) -> int:
    if kv_dtype is not None:
        return int(kv_dtype)
    return KV_BF16 if kv.shape[-1] == 1152 else KV_FP8


def topk_workspace(rows: int, k: int, row_stride: int, device) -> Optional[torch.Tensor]:
    """A top-k workspace that lets `rows` rows of `row_stride` candidates split over several
    workgroups (None when that split does not apply)."""
    tk, _ = workspace_size(Capacity.make(max(1, rows), k, 16, int(row_stride)))
    if tk == 0:
        return None
    return torch.empty(tk, dtype=torch.uint8, device=device)


def attention_workspace(rows: int, H: int, k: int, device, kv_dtype: int = KV_BF16) -> Optional[torch.Tensor]:
    """A workspace big enough for `rows` rows in one launch (None if k needs none).  Its contents
    on entry do not matter."""
    _, nbytes = workspace_size(Capacity.make(max(1, rows), k, H, 1, kv_dtype=kv_dtype))
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def sparse_mla_decode(q: torch.Tensor, kv: torch.Tensor, block_table: torch.Tensor, idx: torch.Tensor,
                      softmax_scale: float, row_req: Optional[torch.Tensor] = None,
                      kv_dtype: Optional[int] = None, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      sink: Optional[torch.Tensor] = None):
    """Sparse MLA attention of each row of ``q`` [rows, H, 576] (bf16) over the tokens in ``idx``
    [rows, k] (int32 logical positions, -1 skipped) of the paged cache ``kv`` (uint8 bytes
    [num_pages, 64, record]), with optional per-head sink logits ``sink`` (fp32 [H], -inf = none).
    Returns (out bf16 [rows, H, 512], lse fp32 [rows, H] or None)."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, contiguous=False)
    if q.dim() != 3 or q.shape[2] != 576 or q.stride(2) != 1 or q.stride(1) != 576:
        raise ValueError("q must be [rows, H, 576] with contiguous heads")
    dev = q.device
    _require(kv, "kv", torch.uint8, dev)
    _require(block_table, "block_table", torch.int32, dev)
    _require(idx, "idx", torch.int32, dev)
    rows, H = q.shape[0], q.shape[1]
    k = idx.shape[-1]
    if idx.numel() < rows * k:
        raise ValueError("idx is smaller than rows*k")
    if row_req is not None:
        _require(row_req, "row_req", torch.int32, dev)
    _check_sink(sink, H, dev)
    out, lse = _attn_outputs(rows, H, dev, out, lse)
    if workspace is None:
        workspace = attention_workspace(rows, H, k, dev, _kv_dtype_of(kv, kv_dtype))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    bt2 = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    _check(lib.smla_sparse_mla_decode(_ptr(q), q.stride(0), _ptr(kv), _kv_dtype_of(kv, kv_dtype), kv.shape[0],
                                      _ptr(bt2), bt2.shape[1], bt2.shape[0], _ptr(row_req), _ptr(idx), rows, H, k,
                                      float(softmax_scale), _ptr(sink), _ptr(out), _ptr(lse), _ptr(workspace),
                                      ws_bytes, _stream(dev)))
    return out, lse


def sparse_mla_decode_with_window(q: torch.Tensor, kv: torch.Tensor, block_table: torch.Tensor, idx: torch.Tensor,
                                  kv_win: torch.Tensor, block_table_win: torch.Tensor, idx_win: torch.Tensor,
                                  softmax_scale: float, row_req: Optional[torch.Tensor] = None,
                                  kv_dtype: Optional[int] = None, out: Optional[torch.Tensor] = None,
                                  lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                  sink: Optional[torch.Tensor] = None):
    """Sparse MLA attention of each row over the tokens ``idx`` [rows, k] of the main cache ``kv`` and
    the tokens ``idx_win`` [rows, k_win] (k_win a multiple of 64) of the window cache ``kv_win``, in one
    softmax.  ``block_table`` / ``block_table_win`` int32 [num_reqs, *]; ``row_req`` indexes both.
    Returns (out bf16 [rows, H, 512], lse fp32 [rows, H] or None)."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, contiguous=False)
    if q.dim() != 3 or q.shape[2] != 576 or q.stride(2) != 1 or q.stride(1) != 576:
        raise ValueError("q must be [rows, H, 576] with contiguous heads")
    dev = q.device
    for t, nm in ((kv, "kv"), (kv_win, "kv_win")):
        _require(t, nm, torch.uint8, dev)
    for t, nm in ((block_table, "block_table"), (block_table_win, "block_table_win"), (idx, "idx"),
                  (idx_win, "idx_win")):
        _require(t, nm, torch.int32, dev)
    rows, H = q.shape[0], q.shape[1]
    k, k_win = idx.shape[-1], idx_win.shape[-1]
    if idx.numel() < rows * k or idx_win.numel() < rows * k_win:
        raise ValueError("idx / idx_win are smaller than rows*k / rows*k_win")
    if block_table.dim() != 2 or block_table_win.dim() != 2 or block_table.shape[0] != block_table_win.shape[0]:
        raise ValueError("block_table and block_table_win must be 2-D with one row per request")
    if row_req is not None:
        _require(row_req, "row_req", torch.int32, dev)
    _check_sink(sink, H, dev)
    out, lse = _attn_outputs(rows, H, dev, out, lse)
    dt = _kv_dtype_of(kv, kv_dtype)
    if workspace is None:
        workspace = attention_workspace(rows, H, k + k_win, dev, dt)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.smla_sparse_mla_decode_with_window(
        _ptr(q), q.stride(0), _ptr(kv), dt, kv.shape[0], _ptr(block_table), block_table.shape[1], _ptr(idx), k,
        _ptr(kv_win), kv_win.shape[0], _ptr(block_table_win), block_table_win.shape[1], _ptr(idx_win), k_win,
        block_table.shape[0], _ptr(row_req), rows, H, float(softmax_scale), _ptr(sink), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse


def sparse_mla_decode_noalloc(q: torch.Tensor, kv: torch.Tensor, block_table: torch.Tensor, idx: torch.Tensor,
                              softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                              row_req: Optional[torch.Tensor] = None, kv_dtype: Optional[int] = None,
                              sink: Optional[torch.Tensor] = None):
    """sparse_mla_decode through the workspace-free entry point (the split partials live in the
    library's static per-GPU scratch array): the caller passes every output; nothing is allocated.
    Workspace-free calls on one GPU must be ordered on one stream."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, contiguous=False)
    if q.dim() != 3 or q.shape[2] != 576 or q.stride(2) != 1 or q.stride(1) != 576:
        raise ValueError("q must be [rows, H, 576] with contiguous heads")
    dev = q.device
    _require(kv, "kv", torch.uint8, dev)
    _require(block_table, "block_table", torch.int32, dev)
    _require(idx, "idx", torch.int32, dev)
    rows, H = q.shape[0], q.shape[1]
    k = idx.shape[-1]
    if idx.numel() < rows * k:
        raise ValueError("idx is smaller than rows*k")
    if row_req is not None:
        _require(row_req, "row_req", torch.int32, dev)
    _check_sink(sink, H, dev)
    _attn_outputs(rows, H, dev, out, lse)
    bt2 = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    _check(lib.smla_sparse_mla_decode_noalloc(_ptr(q), q.stride(0), _ptr(kv), _kv_dtype_of(kv, kv_dtype), kv.shape[0],
                                              _ptr(bt2), bt2.shape[1], bt2.shape[0], _ptr(row_req), _ptr(idx), rows,
                                              H, k, float(softmax_scale), _ptr(sink), _ptr(out), _ptr(lse),
                                              _stream(dev)))
    return out, lse


def sparse_mla_prefill_chunk(q: torch.Tensor, kv: torch.Tensor, block_table_row: torch.Tensor, idx: torch.Tensor,
                             softmax_scale: float, kv_dtype: Optional[int] = None,
                             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None):
    """Prefill chunk of one request: every row of ``q`` reads the request of ``block_table_row``."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, contiguous=False)
    if q.dim() != 3 or q.shape[2] != 576 or q.stride(2) != 1 or q.stride(1) != 576:
        raise ValueError("q must be [T, H, 576] with contiguous heads")
    dev = q.device
    _require(kv, "kv", torch.uint8, dev)
    _require(block_table_row, "block_table_row", torch.int32, dev)
    _require(idx, "idx", torch.int32, dev)
    T, H = q.shape[0], q.shape[1]
    k = idx.shape[-1]
    _check_sink(sink, H, dev)
    out, lse = _attn_outputs(T, H, dev, out, lse)
    if workspace is None:
        workspace = attention_workspace(T, H, k, dev, _kv_dtype_of(kv, kv_dtype))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.smla_sparse_mla_prefill_chunk(_ptr(q), q.stride(0), _ptr(kv), _kv_dtype_of(kv, kv_dtype), kv.shape[0],
                                             _ptr(block_table_row), block_table_row.numel(), _ptr(idx), T, H, k,
                                             float(softmax_scale), _ptr(sink), _ptr(out), _ptr(lse), _ptr(workspace),
                                             ws_bytes, _stream(dev)))
    return out, lse


def kv_cache_write(kv_in: torch.Tensor, slot_mapping: torch.Tensor, cache: torch.Tensor,
                   kv_dtype: Optional[int] = None, positions: Optional[torch.Tensor] = None,
                   cos_sin: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Writes the records of the tokens ``kv_in`` [T, 576] (bf16; rows may be strided) to the
    physical slots ``slot_mapping`` [T] (int64; < 0 skipped) of ``cache`` (uint8 [num_pages, 64,
    record]), quantizing to FP8 records for FP8 caches.  With ``positions`` (int64 [T]) and
    ``cos_sin`` (fp32 [max_pos, 64]: 32 cosines then 32 sines per position) the rope part is stored
    with the rotation of each token's position undone (smla_kv_cache_write_rope).  Returns ``cache``."""
    lib = load_library()
    _require(kv_in, "kv_in", torch.bfloat16, contiguous=False)
    if kv_in.dim() != 2 or kv_in.shape[1] != 576 or kv_in.stride(1) != 1:
        raise ValueError("kv_in must be [T, 576] with contiguous rows")
    dev = kv_in.device
    _require(slot_mapping, "slot_mapping", torch.int64, dev)
    _require(cache, "cache", torch.uint8, dev)
    T = kv_in.shape[0]
    if slot_mapping.numel() < T:
        raise ValueError("slot_mapping is shorter than T")
    dt = _kv_dtype_of(cache, kv_dtype)
    rec = 1152 if dt == KV_BF16 else 656
    if cache.dim() != 3 or cache.shape[1] != 64 or cache.shape[2] != rec:
        raise ValueError(f"cache must be [num_pages, 64, {rec}] for kv_dtype {dt}")
    if (positions is None) != (cos_sin is None):
        raise ValueError("positions and cos_sin go together")
    if positions is None:
        _check(lib.smla_kv_cache_write(_ptr(kv_in), kv_in.stride(0), _ptr(slot_mapping), T, _ptr(cache), dt,
                                       cache.shape[0], _stream(dev)))
        return cache
    _require(positions, "positions", torch.int64, dev)
    _require(cos_sin, "cos_sin", torch.float32, dev)
    if positions.numel() < T:
        raise ValueError("positions is shorter than T")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 64:
        raise ValueError("cos_sin must be [max_pos, 64] (32 cosines then 32 sines per position)")
    _check(lib.smla_kv_cache_write_rope(_ptr(kv_in), kv_in.stride(0), _ptr(slot_mapping), _ptr(positions),
                                        _ptr(cos_sin), cos_sin.shape[0], T, _ptr(cache), dt, cache.shape[0],
                                        _stream(dev)))
    return cache


def paged_mqa_logits(q: torch.Tensor, weights: torch.Tensor, kidx: torch.Tensor, block_table: torch.Tensor,
                     lengths: Optional[torch.Tensor] = None, row_req: Optional[torch.Tensor] = None,
                     out_stride: Optional[int] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer scores of each row of ``q`` [rows, Hi, 128] (bf16) with head weights ``weights``
    [rows, Hi] (fp32) over the paged index-key cache ``kidx`` (bf16 [num_pages, 64, 128]):
    out[r, p] = sum_h w[r, h] * relu(<q[r, h], key_p>) for p below the row's length (``lengths``
    int32 [rows], clamped to [0, out_stride]; None: out_stride) whose page is listed, -inf elsewhere.
    ``block_table`` int32 [num_reqs, max_pages]; ``row_req`` int32 [rows] (None: request 0).
    Returns ``out`` fp32 [rows, out_stride] (allocated when None)."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, contiguous=False)
    if q.dim() != 3 or q.shape[2] != 128 or q.stride(2) != 1 or q.stride(1) != 128:
        raise ValueError("q must be [rows, Hi, 128] with contiguous heads")
    dev = q.device
    rows, Hi = q.shape[0], q.shape[1]
    _require(weights, "weights", torch.float32, dev, contiguous=False)
    if weights.dim() != 2 or weights.shape[0] != rows or weights.shape[1] != Hi or weights.stride(1) != 1:
        raise ValueError("weights must be [rows, Hi] with contiguous rows")
    _require(kidx, "kidx", torch.bfloat16, dev)
    if kidx.dim() != 3 or kidx.shape[1] != 64 or kidx.shape[2] != 128:
        raise ValueError("kidx must be [num_pages, 64, 128]")
    _require(block_table, "block_table", torch.int32, dev)
    if lengths is not None:
        _require(lengths, "lengths", torch.int32, dev)
        if lengths.numel() < rows:
            raise ValueError("lengths is shorter than rows")
    if row_req is not None:
        _require(row_req, "row_req", torch.int32, dev)
        if row_req.numel() < rows:
            raise ValueError("row_req is shorter than rows")
    if out is None:
        if out_stride is None:
            raise ValueError("out_stride is required when out is not given")
        out = torch.empty(rows, int(out_stride), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", torch.float32, dev)
        if out.dim() != 2 or out.shape[0] != rows:
            raise ValueError("out must be a contiguous [rows, stride] tensor")
        if out_stride is not None and int(out_stride) != out.shape[1]:
            raise ValueError("out_stride does not match out")
    bt2 = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    _check(lib.smla_paged_mqa_logits(_ptr(q), q.stride(0), _ptr(weights), weights.stride(0), _ptr(kidx),
                                     kidx.shape[0], _ptr(bt2), bt2.shape[1], bt2.shape[0], _ptr(row_req),
                                     _ptr(lengths), rows, Hi, _ptr(out), out.shape[1],
                                     _stream(dev)))
    return out
