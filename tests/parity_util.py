"""Helpers for GPU-vs-oracle parity tests: run libfa, run the oracle on the same bits, compare."""

from __future__ import annotations

import numpy as np
import torch

import io_aware_exact_23_amd as fa
from oracle import attention_fwd

# Tolerances against the fp64 oracle. bf16 inputs: O max-abs 2e-2 and mean-abs 2e-3, lse 1e-3.
# fp32 inputs: O max-abs and mean-abs 1e-5, lse 1e-3.
TOL = {"bf16": (2e-2, 2e-3, 1e-3), "fp32": (1e-5, 1e-5, 1e-3)}


def f32(scale: float) -> float:
    """The scale as the library receives it (fp32)."""
    return float(np.float32(scale))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a bf16 / fp32 tensor (device or host)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def run_lib(q, k, v, scale, causal=False, lens=None):
    o, lse = fa.attention(q, k, v, scale=scale, causal=causal, kv_seqlens=lens)
    torch.cuda.synchronize()
    return o, lse


def run_oracle(q, k, v, scale, causal=False, lens=None, rows=None, b_range=None, window=None):
    """Oracle on the exact input bits; optionally restricted to query rows and a batch range."""
    lens_l = None if lens is None else [int(x) for x in lens.to("cpu").tolist()]
    bs = range(q.shape[0]) if b_range is None else b_range
    outs, lses = [], []
    for b in bs:
        lb = None if lens_l is None else [lens_l[b]]
        qb = to_f64(q[b:b + 1])
        kb = to_f64(k[b:b + 1])
        vb = to_f64(v[b:b + 1])
        o, lse = attention_fwd(qb, kb, vb, f32(scale), causal=causal, kv_seqlens=lb, rows=rows,
                               window=window)
        outs.append(o)
        lses.append(lse)
    return np.concatenate(outs), np.concatenate(lses)


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
            dtype: str, row_mask: np.ndarray | None = None, what: str = ""):
    """Assert parity. row_mask (B, H, R) selects the compared rows (all when None)."""
    max_tol, mean_tol, lse_tol = TOL[dtype]
    if row_mask is None:
        row_mask = np.ones(lse_ref.shape, dtype=bool)
    og = o_gpu[row_mask]
    orf = o_ref[row_mask]
    lg = lse_gpu[row_mask]
    lr = lse_ref[row_mask]
    assert np.all(np.isfinite(og)), f"{what}: non-finite O"
    err = np.abs(og - orf)
    max_err = float(err.max()) if err.size else 0.0
    mean_err = float(err.mean()) if err.size else 0.0
    fin = np.isfinite(lr)
    assert np.array_equal(np.isfinite(lg), fin), f"{what}: lse finiteness differs"
    assert np.all(lg[~fin] == lr[~fin]), f"{what}: lse infinities differ"
    lse_err = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
    msg = f"{what}: O max {max_err:.3e} mean {mean_err:.3e}, lse max {lse_err:.3e}"
    print("parity", msg, flush=True)
    assert max_err <= max_tol and mean_err <= mean_tol and lse_err <= lse_tol, msg
    return max_err, mean_err, lse_err
