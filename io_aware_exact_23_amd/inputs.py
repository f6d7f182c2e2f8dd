"""Seeded synthetic inputs, shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws Q, K, V and the per-sequence key
lengths, so the same bits can be handed both to the HIP library and to the CPU oracle.

Recipe: Q, K and V are iid std * N(0, 1) in fp32 from ``torch.Generator(device).manual_seed``
with sub-seeds seed+0, +1, +2 for Q, K, V; bf16 tensors are rounded to nearest-even from
those fp32 draws. Key lengths are integers uniform on [lo, hi], both ends included, drawn on
the CPU with sub-seed seed+3. Cache slots at or past a sequence's length are set to zero
(``poison`` replaces them with a large finite value for the tests that check that masked
keys cannot leak into the result).
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from .configs import Workload

__all__ = ["normal", "lengths", "make", "fill_padding"]

_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def normal(shape, seed: int, device, dtype: str, std: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(_DT[dtype])


def lengths(batch: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int32)


def fill_padding(x: torch.Tensor, lens: torch.Tensor, value: float) -> None:
    """Set key slots j >= lens[b] of a (B, H, Nk, d) tensor to ``value`` in place."""
    nk = x.shape[2]
    for b, n in enumerate(lens.tolist()):
        if n < nk:
            x[b, :, n:, :] = value


def make(w: Workload, device="cpu", poison: Optional[float] = None
         ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Draw (q, k, v, kv_seqlens) for workload ``w`` on ``device``."""
    q = normal((w.B, w.H, w.Nq, w.d), w.seed + 0, device, w.dtype, w.input_std)
    k = normal((w.B, w.H, w.Nk, w.d), w.seed + 1, device, w.dtype, w.input_std)
    v = normal((w.B, w.H, w.Nk, w.d), w.seed + 2, device, w.dtype, w.input_std)
    lens = None
    if w.lengths is not None:
        lens = lengths(w.B, w.lengths[0], w.lengths[1], w.seed + 3)
        fill = 0.0 if poison is None else poison
        fill_padding(k, lens, fill)
        fill_padding(v, lens, -fill if fill else 0.0)
        lens = lens.to(device)
    return q, k, v, lens
