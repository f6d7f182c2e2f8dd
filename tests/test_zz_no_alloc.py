"""fa_fwd_noalloc (the entry point that allocates no device memory) against fa_fwd, through the
C ABI: the same kernels run, so outputs must be bit-identical. Two decode calls in a row, the
second smaller (the static scratch keeps the first call's contents), then a prefill call; the
larger decode is also held to the oracle's tolerance."""

import numpy as np
import pytest
import torch

import io_aware_exact_23_amd as fa
from io_aware_exact_23_amd import configs, inputs

from parity_util import compare, run_oracle, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()


def _both(q, k, v, lt, scale, causal):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    outs = []
    for fn in (fa.fa_fwd, fa.fa_fwd_noalloc):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
        fn(q, k, v, o, lse, B, H, Nq, Nk, d, scale, int(causal), lt, None)
        torch.cuda.synchronize()
        outs.append((o, lse))
    return outs


def _same(a, b, what):
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{what}: O differs"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"{what}: lse differs"


def test_noalloc_matches_fa_fwd_on_two_decode_calls_then_prefill():
    w = configs.DECODE_SPLIT_KV
    q, k, v, lt = inputs.make(w, DEV)
    print(f"noalloc decode {w.name}", flush=True)
    ref, got = _both(q, k, v, lt, w.scale, False)
    _same(ref, got, w.name)
    og, lg = to_f64(got[0]), to_f64(got[1])
    for b0 in (0, 56):
        o_ref, lse_ref = run_oracle(q, k, v, w.scale, False, lt, b_range=range(b0, b0 + 8))
        compare(og[b0:b0 + 8], lg[b0:b0 + 8], o_ref, lse_ref, "bf16", what=f"noalloc {w.name} b{b0}")

    # Second call, smaller: fewer partials than the first left in the scratch, d = 64.
    q2 = inputs.normal((3, 2, 1, 64), 11, DEV, "bf16")
    k2 = inputs.normal((3, 2, 700, 64), 12, DEV, "bf16")
    v2 = inputs.normal((3, 2, 700, 64), 13, DEV, "bf16")
    lt2 = torch.tensor([700, 129, 1], dtype=torch.int32, device=DEV)
    print("noalloc decode 3x2x700 d=64", flush=True)
    ref2, got2 = _both(q2, k2, v2, lt2, 0.125, False)
    _same(ref2, got2, "small decode")
    o_ref, lse_ref = run_oracle(q2, k2, v2, 0.125, False, lt2)
    compare(to_f64(got2[0]), to_f64(got2[1]), o_ref, lse_ref, "bf16", what="noalloc small decode")

    # Prefill needs no scratch: the same kernels as fa_fwd.
    q3, k3, v3 = (inputs.normal((2, 2, 300, 128), 20 + s, DEV, "bf16") for s in range(3))
    print("noalloc prefill 2x2x300 causal", flush=True)
    ref3, got3 = _both(q3, k3, v3, None, 128 ** -0.5, True)
    _same(ref3, got3, "prefill")
