"""GPU parity on seeded random shapes: fa_fwd and fa_fwd_window against the fp64 oracle.

The hand-picked shapes elsewhere cover the edges each kernel was written for; these draw the
shape, mask, lengths, scale and value spread at random (seeded, so every run checks the same 40
cases) to reach combinations nobody picked: Nq from 1 (the decode path) to past 2048 (the
long-sequence kernel), Nq != Nk, lengths of 0 and past Nk (clamped), negative scales, and
sliding windows of every width. Each case compares every row with the oracle at the bars of its
dtype.
"""

import numpy as np
import pytest
import torch

import io_aware_exact_23_amd as fa
from io_aware_exact_23_amd import inputs

from parity_util import compare, run_lib, run_oracle, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()


def _draw(i):
    """Case i: (B, H, Nq, Nk, d, dtype, causal, lens, scale, std, window)."""
    r = np.random.default_rng(20260 + i)
    d = int(r.choice([64, 128]))
    dtype = "fp32" if r.random() < 0.2 else "bf16"
    kind = r.choice(["decode", "short", "short", "short", "long"])
    if kind == "decode":
        B, H, Nq, Nk = int(r.integers(1, 5)), int(r.integers(1, 4)), 1, int(r.integers(1, 1500))
    elif kind == "short":
        B, H = int(r.integers(1, 4)), int(r.integers(1, 4))
        Nq = int(r.integers(2, 700))
        Nk = Nq if r.random() < 0.5 else int(r.integers(1, 700))
    else:
        B, H = 1, 1
        Nq = int(r.integers(2048, 2600))
        Nk = Nq if r.random() < 0.6 else int(r.integers(1, 2600))
    if dtype == "fp32" and Nq > 1:
        Nq = min(Nq, 600)  # the fp32 kernel is the short one; keep the oracle quick
        Nk = Nq if Nk == Nq else min(Nk, 600)
    causal = Nq == Nk and Nq > 1 and r.random() < 0.6
    window = None
    if dtype == "bf16" and Nq > 1 and not causal and r.random() < 0.3:
        Nk = Nq  # a window with a bounded side is defined for Nq == Nk
        left = int(r.integers(-1, Nk + 2))
        right = int(r.integers(-1, Nk + 2)) if r.random() < 0.5 else 0
        window = (left, right)
    lens = None
    if r.random() < 0.5:
        lens = [int(x) for x in r.integers(0, Nk + 6, size=B)]
    scale = float(d ** -0.5 * r.choice([1.0, 0.5, 1.5, -1.0]))
    # The bf16 bars (O max-abs 2e-2) are absolute and set for unit-variance values: at |O| >= 4 a
    # bf16 ulp is 2^-5, so the bf16 cases keep std <= 1 and reach larger scores through the scale.
    std = float(r.choice([0.5, 1.0, 1.5] if dtype == "fp32" else [0.5, 1.0]))
    return B, H, Nq, Nk, d, dtype, causal, lens, scale, std, window


CASES = [_draw(i) for i in range(40)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_shape_against_oracle(case):
    B, H, Nq, Nk, d, dtype, causal, lens, scale, std, window = CASES[case]
    what = (f"random case {case}: {dtype} d={d} {B}x{H}x{Nq}x{Nk} causal={causal} lens={lens} "
            f"scale={scale:.4f} std={std} window={window}")
    print(what, flush=True)
    seed = 90000 + 17 * case
    q = inputs.normal((B, H, Nq, d), seed, DEV, dtype, std)
    k = inputs.normal((B, H, Nk, d), seed + 1, DEV, dtype, std)
    v = inputs.normal((B, H, Nk, d), seed + 2, DEV, dtype, std)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    if window is None:
        o, lse = run_lib(q, k, v, scale, causal, lt)
        o_ref, lse_ref = run_oracle(q, k, v, scale, causal, lt)
    else:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
        fa.fa_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, d, scale, window[0], window[1], lt, None)
        torch.cuda.synchronize()
        o_ref, lse_ref = run_oracle(q, k, v, scale, False, lt, window=window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, dtype, what=what)
