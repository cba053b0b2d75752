"""Shared test utilities: moving tensors to the oracle's numpy form and the parity checks."""

from __future__ import annotations

import sys

import numpy as np
import torch

# Attention tolerance against the fp64 oracle (bf16 inputs, fp32 accumulation, bf16 output).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# Stricter internal alarms.
REL_FRO = 1e-2
LSE_ABS = 1e-3


# Parity figures of this session (what, stats), printed at the end of the run by conftest.
PARITY_RECORDS = []


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def kv_np(kv: torch.Tensor) -> np.ndarray:
    return kv.detach().cpu().numpy()


def assert_attention_close(out_gpu: torch.Tensor, lse_gpu: torch.Tensor, O_ref: np.ndarray, lse_ref: np.ndarray,
                           what: str = "", relative: bool = False, out_scale: float = 1.0,
                           lse_tol=None) -> dict:
    """Bounds on |out - O_ref| (max and mean) and on the LSE.  With ``relative`` (the FP8-KV
    workloads, whose group scales of up to 2^4 give outputs far above unit scale, where bf16 output
    rounding alone exceeds the absolute bounds) every output error is divided by max(1, |reference|):
    elementwise for the max, by max(1, mean |O_ref|) for the mean.  The LSE bound is absolute in
    every case: the LSE is an fp32 result, never rounded to bf16.  ``out_scale`` (a power of two)
    multiplies both outputs before the comparison, which brings outputs of a known magnitude to unit
    scale without changing any rounding.  ``lse_tol`` replaces the LSE bound (a scalar, or one bound
    per (row, head)) where a test derives it from the magnitude of the scores."""
    o = out_gpu.detach().float().cpu().numpy().astype(np.float64) * out_scale
    O_ref = O_ref * out_scale
    assert o.shape == O_ref.shape, (o.shape, O_ref.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - O_ref)
    if relative:
        err = err / np.maximum(1.0, np.abs(O_ref))
    stats = {"max_abs": float(err.max()) if err.size else 0.0, "mean_abs": float(err.mean()) if err.size else 0.0}
    if relative and err.size:
        stats["mean_abs"] = float(np.abs(o - O_ref).mean() / max(1.0, float(np.abs(O_ref).mean())))
    ref_norm = float(np.linalg.norm(O_ref))
    stats["rel_fro"] = float(np.linalg.norm(o - O_ref) / ref_norm) if ref_norm > 0 else 0.0
    assert stats["max_abs"] <= MAX_ABS, (what, stats)
    assert stats["mean_abs"] <= MEAN_ABS, (what, stats)
    if ref_norm > 0:
        assert stats["rel_fro"] <= REL_FRO, (what, stats)
    if lse_gpu is not None:
        l = lse_gpu.detach().cpu().numpy().astype(np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isneginf(l), np.isneginf(lse_ref)), f"{what}: -inf lse mismatch"
        if fin.any():
            d = np.abs(l[fin] - lse_ref[fin])
            stats["lse_max_abs"] = float(d.max())
            tol = LSE_ABS if lse_tol is None else np.broadcast_to(np.asarray(lse_tol, np.float64), l.shape)[fin]
            assert (d <= tol).all(), (what, stats)
    stats["rows"] = int(O_ref.shape[0]) if O_ref.ndim >= 3 else 1
    PARITY_RECORDS.append((what, dict(stats)))
    return stats


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality of two tensors of the same dtype (NaN-safe)."""
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def sample_rows(n_rows: int, n: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(n_rows, size=min(n, n_rows), replace=False).tolist())
