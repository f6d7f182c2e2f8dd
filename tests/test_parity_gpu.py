"""GPU parity: libfa (through its C ABI) against the fp64 oracle on the same input bits.

Sizes span several tiles and ragged tails; the five named workloads run at full size (the
16K causal prefill compares two whole heads against the oracle and every row of every head
against bounds that hold at any size). Edge cases: single key, empty sequences, Nk == 0,
NaN / Inf / huge padding against the oracle, huge scores, negative and zero scale, bitwise
repeatability, decode (split-KV) against the tiled kernel, and the largest head the entry
points accept.
"""

import numpy as np
import pytest
import torch

import io_aware_exact_23_amd as fa
from io_aware_exact_23_amd import configs, inputs

from parity_util import compare, run_lib, run_oracle, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()  # raises if the HIP library is missing: no fallback exists


def _rand(shape, seed, dtype, std=1.0):
    return inputs.normal(shape, seed, DEV, dtype, std)


def _case(B, H, Nq, Nk, d, dtype, causal, lens, seed, std=1.0, scale=None):
    q = _rand((B, H, Nq, d), seed, dtype, std)
    k = _rand((B, H, Nk, d), seed + 1, dtype, std)
    v = _rand((B, H, Nk, d), seed + 2, dtype, std)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    if scale is None:
        scale = d ** -0.5
    return q, k, v, lt, scale


def _check(q, k, v, lt, scale, causal, dtype, what):
    """Run the library and the oracle on the same bits and compare; returns the three errors and
    the library's (O, lse)."""
    print(what, flush=True)
    o, lse = run_lib(q, k, v, scale, causal, lt)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal, lt)
    return compare(to_f64(o), to_f64(lse), o_ref, lse_ref, dtype, what=what) + (o, lse)


SMALL = [
    # B, H, Nq, Nk, causal, lens
    (1, 1, 17, 17, True, None),
    (2, 3, 100, 300, False, None),
    (1, 2, 129, 129, True, None),
    (2, 2, 256, 256, True, [256, 77]),
    (2, 1, 200, 333, False, [1, 333]),
    (1, 1, 64, 64, False, None),
    (3, 2, 300, 300, True, None),
    (2, 2, 2, 65, False, [65, 3]),
    # padded batch without a causal mask: equal lengths, an empty sequence, a ragged tail
    (5, 2, 150, 300, False, [130, 300, 17, 130, 0]),
    # causal, B*H*n_qtiles a multiple of 8*n_qtiles (the serpentine work order), ragged last tile
    (2, 4, 300, 300, True, None),
    (4, 4, 1000, 1000, True, [1000, 999, 512, 3]),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Nq,Nk,causal,lens", SMALL)
def test_small_shapes(dtype, d, B, H, Nq, Nk, causal, lens):
    q, k, v, lt, scale = _case(B, H, Nq, Nk, d, dtype, causal, lens, seed=Nq * 7 + Nk + d)
    _check(q, k, v, lt, scale, causal, dtype, f"small {dtype} d={d} {B}x{H}x{Nq}x{Nk} causal={causal} lens={lens}")


# Nq >= 2048 runs the 8-wave kernel (one wave's matrix work overlapped with its SIMD partner's
# softmax, 256-row tiles, separate unmasked and masked key loops); these shapes cover its masks,
# ragged tails, Nq != Nk, padding and empty sequences at both head dimensions.
LONG = [
    # B, H, Nq, Nk, d, causal, lens
    (1, 2, 2048, 2048, 128, True, None),
    (1, 1, 2113, 2113, 64, True, None),
    (2, 1, 2048, 2500, 128, False, [2500, 77]),
    (2, 2, 2300, 1000, 64, False, [1000, 0]),
    (1, 1, 2304, 2304, 64, False, [1000]),
    (1, 1, 4096, 4096, 128, True, None),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,lens", LONG)
def test_long_sequence_kernel(B, H, Nq, Nk, d, causal, lens):
    q, k, v, lt, scale = _case(B, H, Nq, Nk, d, "bf16", causal, lens, seed=Nq + Nk + d, std=0.7)
    _check(q, k, v, lt, scale, causal, "bf16", f"long d={d} {B}x{H}x{Nq}x{Nk} causal={causal} lens={lens}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Nk,lens", [(1, 1, 1, None), (2, 3, 700, [700, 1]), (3, 2, 513, [0, 256, 257]),
                                          (4, 2, 8192, [8192, 1024, 4097, 5]),
                                          # more partials per sequence than a wave has lanes, and a
                                          # count that is not a multiple of the combine's groups
                                          (2, 2, 21000, [21000, 8321])])
def test_decode_shapes(d, B, H, Nk, lens):
    q, k, v, lt, scale = _case(B, H, 1, Nk, d, "bf16", False, lens, seed=Nk + d)
    _check(q, k, v, lt, scale, False, "bf16", f"decode d={d} B={B} H={H} Nk={Nk} lens={lens}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_single_head_fp32_workload_and_dtypes(dtype):
    w = configs.SINGLE_HEAD_FP32
    q, k, v, _ = inputs.make(w, DEV)
    if dtype == "bf16":
        q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    _check(q, k, v, None, w.scale, w.causal, dtype, f"{w.name} as {dtype}")


def test_gpt2_small_causal_workload():
    w = configs.GPT2_SMALL_CAUSAL
    q, k, v, lt = inputs.make(w, DEV)
    _check(q, k, v, lt, w.scale, w.causal, "bf16", w.name)


def test_bert_large_padded_workload():
    w = configs.BERT_LARGE_PADDED
    q, k, v, lt = inputs.make(w, DEV)
    o, lse = run_lib(q, k, v, w.scale, w.causal, lt)
    o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal, lt)
    lens = lt.cpu().numpy()
    # Padded query rows (i >= L_b) are computed but not part of the result.
    rows = np.arange(w.Nq)[None, None, :] < lens[:, None, None]
    mask = np.broadcast_to(rows, lse_ref.shape)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", row_mask=mask, what=w.name)


def _row_bounds_every_row(q, k, v, o, lse, scale):
    """Properties of causal attention that hold at every row i of every head, checked on the
    device: lse_i is at least the scores of keys 0 and i (both allowed) and at most
    |scale| * |q_i| * max_{j<=i} |k_j| + ln(i+1) (Cauchy-Schwarz bounds every allowed score);
    O_i is a convex combination of v_0..v_i, so each coordinate lies between their running
    minimum and maximum. Slack: fp32 rounding of the scores; the bf16 rounding of P before P V
    (its weights sum to 1 within 2^-9) and of O."""
    n = q.shape[2]
    qf, kf, vf = q.float(), k.float(), v.float()
    s_diag = scale * (qf * kf).sum(-1)
    s_first = scale * (qf * kf[:, :, :1]).sum(-1)
    knorm_max = torch.cummax(kf.norm(dim=-1), dim=2).values
    upper = abs(scale) * qf.norm(dim=-1) * knorm_max + torch.log(
        torch.arange(1, n + 1, device=q.device, dtype=torch.float32))
    tol = 1e-3
    assert bool((lse >= torch.maximum(s_diag, s_first) - tol).all()), "lse below an allowed score"
    assert bool((lse <= upper + tol).all()), "lse above the Cauchy-Schwarz bound"
    vmax = torch.cummax(vf, dim=2).values
    vmin = -torch.cummax(-vf, dim=2).values
    of = o.float()
    slack = 2.0 ** -7 * torch.maximum(vmax.abs(), vmin.abs()) + 1e-6
    assert bool((of <= vmax + slack).all()) and bool((of >= vmin - slack).all()), \
        "O outside the range of the allowed V rows"


def test_long_causal_16k_workload_whole_heads():
    """The headline 16K causal shape (B 2, H 16, N 16384, d 128) in the launch configuration the
    benchmark times: two whole heads, (b 0, h 0) and (b 1, h 15), every one of their 16384 rows
    against the oracle (run in blocks of 2048 rows), and every row of all 32 heads against the
    bounds any causal attention satisfies."""
    w = configs.LONG_CAUSAL_16K
    q, k, v, lt = inputs.make(w, DEV)
    o, lse = run_lib(q, k, v, w.scale, w.causal, lt)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    _row_bounds_every_row(q, k, v, o, lse, w.scale)
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        qh, kh, vh = q[sl], k[sl], v[sl]
        og, lg = to_f64(o[sl]), to_f64(lse[sl])
        o_ref = np.zeros_like(og)
        lse_ref = np.zeros_like(lg)
        for r0 in range(0, w.Nq, 2048):
            rows = np.arange(r0, min(r0 + 2048, w.Nq))
            o_ref[:, :, rows], lse_ref[:, :, rows] = run_oracle(qh, kh, vh, w.scale, w.causal, None,
                                                                 rows=rows)
        compare(og, lg, o_ref, lse_ref, "bf16", what=f"{w.name} whole head b={b} h={h}")
        rel = np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)
        early = float(np.abs(og[:, :, :256] - o_ref[:, :, :256]).max())
        print(f"  relative Frobenius {rel:.3e}, rows < 256 max-abs {early:.3e}", flush=True)
        assert rel < 1e-2, f"relative Frobenius error {rel:.3e}"


def test_decode_split_kv_workload():
    w = configs.DECODE_SPLIT_KV
    q, k, v, lt = inputs.make(w, DEV)
    o, lse = run_lib(q, k, v, w.scale, w.causal, lt)
    og, lg = to_f64(o), to_f64(lse)
    for b0 in range(0, w.B, 8):
        o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal, lt, b_range=range(b0, b0 + 8))
        compare(og[b0:b0 + 8], lg[b0:b0 + 8], o_ref, lse_ref, "bf16", what=f"{w.name} b{b0}")


# Key / value paddings that any product touching them would turn into NaN or Inf.
POISONS = [(float("nan"), float("inf")), (float("-inf"), float("nan")), (1.0e4, -1.0e4)]


@pytest.mark.parametrize("Nq,d,dtype", [(1, 128, "bf16"), (1, 64, "bf16"), (200, 128, "bf16"),
                                        (200, 64, "bf16"), (200, 64, "fp32"), (2048, 128, "bf16"),
                                        (2048, 64, "bf16")])
def test_poisoned_padding_against_oracle(Nq, d, dtype):
    """Key slots at or past L_b hold NaN, Inf or huge values: the output must equal the oracle's
    (which never reads those slots) within the usual tolerance, and be bit-identical to the output
    with zero padding. Nq = 1 runs the split-KV decode, 200 the 4-wave kernel, 2048 the 8-wave one."""
    B, H, Nk = 3, 2, 300
    lens = [300, 45, 129]
    q, k, v, lt, scale = _case(B, H, Nq, Nk, d, dtype, False, lens, seed=31 + d + Nq)
    kc, vc = k.clone(), v.clone()
    inputs.fill_padding(kc, lt.cpu(), 0.0)
    inputs.fill_padding(vc, lt.cpu(), 0.0)
    o1, l1 = run_lib(q, kc, vc, scale, False, lt)
    for kfill, vfill in POISONS:
        kp, vp = k.clone(), v.clone()
        inputs.fill_padding(kp, lt.cpu(), kfill)
        inputs.fill_padding(vp, lt.cpu(), vfill)
        what = f"poisoned ({kfill}, {vfill}) Nq={Nq} d={d} {dtype}"
        o2, l2 = _check(q, kp, vp, lt, scale, False, dtype, what)[3:]
        bits = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(o1.view(bits), o2.view(bits)), what
        assert torch.equal(l1, l2), what


def test_poisoned_decode_workload_against_oracle():
    """The decode workload (B 64, H 32, Nk 8192, d 128, ragged lengths) with +Inf in the key slots
    past each length and -Inf in the value slots, every sequence against the oracle."""
    w = configs.DECODE_SPLIT_KV
    q, k, v, lt = inputs.make(w, DEV, poison=float("inf"))
    assert torch.isinf(k).any()
    o, lse = run_lib(q, k, v, w.scale, w.causal, lt)
    og, lg = to_f64(o), to_f64(lse)
    for b0 in range(0, w.B, 8):
        o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal, lt, b_range=range(b0, b0 + 8))
        compare(og[b0:b0 + 8], lg[b0:b0 + 8], o_ref, lse_ref, "bf16", what=f"poisoned {w.name} b{b0}")


@pytest.mark.parametrize("Nq", [1, 1024, 2048])
def test_bitwise_repeatable(Nq):
    Nk = max(Nq, 1024)  # causal (Nq > 1) needs Nq == Nk
    q, k, v, lt, scale = _case(2, 4, Nq, Nk, 128, "bf16", Nq > 1, None, seed=41)
    o1, l1 = run_lib(q, k, v, scale, Nq > 1, lt)
    o2, l2 = run_lib(q, k, v, scale, Nq > 1, lt)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_matches_tiled_kernel():
    # The same query twice (Nq = 2, non-causal) goes through the tiled kernel; Nq = 1 through the
    # split-KV kernels. Both must agree to fp32 rounding plus one bf16 rounding of O.
    B, H, Nk, d = 4, 3, 1500, 128
    q, k, v, lt, scale = _case(B, H, 1, Nk, d, "bf16", False, [1500, 700, 1, 1025], seed=51)
    o1, l1 = run_lib(q, k, v, scale, False, lt)
    o2, l2 = run_lib(q.expand(B, H, 2, d).contiguous(), k, v, scale, False, lt)
    assert torch.allclose(o1.float(), o2[:, :, :1].float(), atol=1.6e-2, rtol=0)
    assert torch.allclose(o2[:, :, 0].float(), o2[:, :, 1].float(), atol=0, rtol=0)
    assert torch.allclose(l1[:, :, 0], l2[:, :, 0], atol=1e-5, rtol=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_huge_scores_stay_finite(dtype):
    # Scores of magnitude ~1e2..1e3: naive exp in fp32 would overflow.
    # fp32 dot products of magnitude ~1e3 carry absolute errors ~1e-4, which the softmax passes
    # on to O; the 1e-5 fp32 bar does not apply to this stress case, the bf16 bar is used.
    # Only Q and K are scaled: V stays N(0, 1), as in every workload, so the absolute bar on O
    # keeps its meaning (P is rounded to bf16 before P V; that error scales with |V|).
    q, k, _, lt, _ = _case(2, 2, 150, 150, 64, dtype, True, None, seed=61, std=4.0)
    v = _rand((2, 2, 150, 64), 64, dtype)
    _check(q, k, v, lt, 2.0, True, "bf16", f"huge scores {dtype}")


def test_huge_scores_long_sequence_kernel():
    # The same stress on the 8-wave kernel: large, drifting scores keep moving the running max,
    # so its lazy rescaling of the output accumulator is exercised many times per row.
    q, k, _, lt, _ = _case(1, 2, 2048, 2048, 64, "bf16", True, None, seed=62, std=4.0)
    v = _rand((1, 2, 2048, 64), 65, "bf16")
    _check(q, k, v, lt, 2.0, True, "bf16", "huge scores, long sequence")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_rising_scores_move_the_offset_often(causal, d):
    # Scores that grow steadily with the key index (one coordinate of every query is 1 and the
    # same coordinate of key j is ~0.26*j), so the row maximum keeps rising: the exponent offset
    # of the kernels must move every few tiles, each time rescaling O and the row sum. Both
    # kernels (Nq = 130 and Nq = 2048) see the same kind of input.
    for Nq in (130, 2048):
        q, k, v, _, _ = _case(1, 2, Nq, Nq, d, "bf16", causal, None, seed=63, std=0.5)
        q[..., 0] = 1.0
        ramp = 0.26 * torch.arange(Nq, device=DEV, dtype=torch.float32)
        k[..., 0] = ramp.to(q.dtype)
        _check(q, k, v, None, 0.125, causal, "bf16", f"rising scores d={d} Nq={Nq} causal={causal}")


@pytest.mark.parametrize("scale", [-0.3, 0.0])
@pytest.mark.parametrize("Nq", [1, 90, 2050])
def test_negative_and_zero_scale(scale, Nq):
    q, k, v, lt, _ = _case(2, 2, Nq, 190, 64, "bf16", False, [190, 60], seed=71)
    _check(q, k, v, lt, scale, False, "bf16", f"scale={scale} Nq={Nq}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("Nq", [1, 40, 2048])
def test_empty_sequences_and_no_keys(dtype, Nq):
    if dtype == "fp32" and Nq == 1:
        Nq = 3
    q, k, v, lt, scale = _case(3, 2, Nq, 70, 128, dtype, False, [0, 1, 70], seed=81)
    _check(q, k, v, lt, scale, False, dtype, f"empty/one-key sequences {dtype} Nq={Nq}")
    # Nk == 0: every row has no allowed key.
    k0 = torch.empty((3, 2, 0, 128), dtype=q.dtype, device=DEV)
    o, lse = run_lib(q, k0, k0, scale, False, None)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_lengths_past_nk_are_clamped():
    q, k, v, _, scale = _case(2, 1, 33, 50, 64, "bf16", False, None, seed=91)
    big = torch.tensor([10_000, -5], dtype=torch.int32, device=DEV)
    o, lse = run_lib(q, k, v, scale, False, big)
    o_ref, lse_ref = run_oracle(q, k, v, scale, False, torch.tensor([50, 0], dtype=torch.int32))
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", what="clamped lengths")


def test_runs_on_a_side_stream():
    q, k, v, lt, scale = _case(2, 2, 300, 300, 128, "bf16", True, None, seed=101)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, scale=scale, causal=True)
    s.synchronize()
    o_ref, lse_ref = run_oracle(q, k, v, scale, True, None)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", what="side stream")


def test_largest_head_prefill_and_decode():
    """K and V at the largest head the entry points accept, 2^31 - 256 bytes (8388607 keys at
    d = 128): buffer offsets reach the top of their 32-bit range. One ragged length just below it,
    non-causal; the 8-wave kernel (2100 rows), the 4-wave kernel (300 rows) and the split-KV
    decode (1 row) on the same keys, each against the oracle on sampled rows."""
    d = 128
    nk = (1 << 31) // (2 * d) - 1
    q = _rand((1, 1, 2100, d), 401, "bf16")
    k = _rand((1, 1, nk, d), 402, "bf16")
    v = _rand((1, 1, nk, d), 403, "bf16")
    lt = torch.tensor([nk - 5], dtype=torch.int32, device=DEV)
    scale = d ** -0.5
    rows = np.array([0, 1, 299, 1023, 2047, 2048, 2099])
    o_ref, lse_ref = run_oracle(q, k, v, scale, False, lt, rows=rows)
    for nq in (2100, 300, 1):
        qs = q[:, :, :nq].contiguous()
        o, lse = run_lib(qs, k, v, scale, False, lt)
        sel = rows < nq
        rt = torch.as_tensor(rows[sel], device=DEV)
        og, lg = to_f64(o[:, :, rt]), to_f64(lse[:, :, rt])
        compare(og, lg, o_ref[:, :, sel], lse_ref[:, :, sel], "bf16", what=f"Nk={nk} Nq={nq}")
        rel = np.linalg.norm(og - o_ref[:, :, sel]) / np.linalg.norm(o_ref[:, :, sel])
        assert rel < 1e-2, f"Nq={nq}: relative Frobenius error {rel:.3e}"
    with pytest.raises(fa.FaError) as ei:
        fa.attention(q[:, :, :1].contiguous(), torch.cat([k, k[:, :, :1]], dim=2),
                     torch.cat([v, v[:, :, :1]], dim=2), scale=scale)
    assert ei.value.status == fa.FA_ERR_UNSUPPORTED


def test_bindings_reject_buffers_the_kernels_would_overrun():
    """Caller-supplied O, lse and length tensors are checked before any launch: a smaller, strided
    or mistyped buffer raises instead of being written past its end."""
    q, k, v, _, scale = _case(2, 2, 70, 70, 64, "bf16", False, None, seed=111)
    good_o, good_l = torch.empty_like(q), torch.empty((2, 2, 70), dtype=torch.float32, device=DEV)
    bad = [
        dict(out=torch.empty((2, 2, 69, 64), dtype=torch.bfloat16, device=DEV)),
        dict(out=torch.empty((2, 2, 64, 70), dtype=torch.bfloat16, device=DEV).transpose(2, 3)),
        dict(out=torch.empty_like(q, dtype=torch.float32)),
        dict(lse=torch.empty((2, 2, 70), dtype=torch.bfloat16, device=DEV)),
        dict(lse=torch.empty((2, 70), dtype=torch.float32, device=DEV)),
        dict(kv_seqlens=torch.tensor([70, 0, 70, 0], dtype=torch.int32, device=DEV)[::2]),
    ]
    for kw in bad:
        args = dict(out=good_o, lse=good_l, kv_seqlens=None)
        args.update(kw)
        with pytest.raises(ValueError):
            fa.attention(q, k, v, scale=scale, **args)
    o, lse = fa.attention(q, k, v, scale=scale, out=good_o, lse=good_l)
    assert o.data_ptr() == good_o.data_ptr() and lse.data_ptr() == good_l.data_ptr()
    with pytest.raises(ValueError):
        fa.attention_backward(q, k, v, o, lse[:, :1], torch.empty_like(q), scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = run_oracle(q, k, v, scale, False, None)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", what="caller buffers")


def test_decode_split_size_invariance(tmp_path):
    """The split size of the decode path is free: the logsumexp combine is exact for any chunk
    size. The decode workload (B 64, H 32, Nk 8192, d 128, ragged lengths) runs with 64-, 128- and
    256-key chunks, each in its own process (the library reads FA_DECODE_CHUNK once per process),
    one after the other. lse must agree across chunk sizes within 1e-6 relative; O, rounded to
    bf16 once from fp32 values that agree to about 2^-20 max|V|, within one bf16 unit in the last
    place plus that; and every run must match the oracle."""
    import os
    import subprocess
    import sys

    w = configs.DECODE_SPLIT_KV
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_chunk_child.py")
    runs = {}
    for chunk in (64, 128, 256):
        out = tmp_path / f"chunk{chunk}.npz"
        env = dict(os.environ, FA_DECODE_CHUNK=str(chunk))
        print(f"decode split size {chunk}", flush=True)
        r = subprocess.run([sys.executable, child, str(out)], env=env, timeout=300,
                           capture_output=True, text=True)
        assert r.returncode == 0, f"chunk {chunk}: child failed\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
        z = np.load(out)
        runs[chunk] = (z["o"].astype(np.float64), z["lse"].astype(np.float64))
    o_ref_all, lse_ref_all = [], []
    q, k, v, lt = inputs.make(w, DEV)
    for b0 in range(0, w.B, 8):
        o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal, lt, b_range=range(b0, b0 + 8))
        o_ref_all.append(o_ref)
        lse_ref_all.append(lse_ref)
    o_ref, lse_ref = np.concatenate(o_ref_all), np.concatenate(lse_ref_all)
    for chunk, (o, lse) in runs.items():
        compare(o, lse, o_ref, lse_ref, "bf16", what=f"{w.name} chunk {chunk}")
    # Before its rounding to bf16, O is a weighted mean of V rows accumulated in fp32, so two chunk
    # sizes agree to about 2^-20 max|V| absolute (O can be much smaller than the V entries it
    # averages); after rounding they differ by at most that plus one bf16 unit in the last place.
    vmax = v.float().abs().amax(dim=(2, 3)).cpu().numpy()[:, :, None, None]
    o0, l0 = runs[128]
    for chunk in (64, 256):
        o, lse = runs[chunk]
        dl = np.abs(lse - l0) / np.maximum(1.0, np.abs(l0))
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.maximum(np.abs(o), np.abs(o0)), 2.0 ** -126))) - 7)
        do = np.abs(o - o0)
        lim = ulp + 2.0 ** -20 * vmax
        frac = float(np.mean(do > 0))
        worst = np.unravel_index(np.argmax(do - lim), do.shape)
        print(f"chunk {chunk} vs 128: lse max rel {dl.max():.2e}, O max {do.max():.2e}, "
              f"{100 * frac:.3f}% of O elements differ; closest to the limit at {tuple(int(x) for x in worst)}: "
              f"|dO| {do[worst]:.3e} vs {lim[worst]:.3e} (O {o0[worst]:.4e})", flush=True)
        assert dl.max() <= 1e-6, f"chunk {chunk}: lse differs by {dl.max():.3e} relative"
        assert np.all(do <= lim), f"chunk {chunk}: O differs by more than one bf16 ulp + 2^-20 max|V|"


def test_prefill_in_a_replayed_hip_graph_matches_eager():
    """The benchmark times the short workloads from a replayed HIP graph of fa_fwd launches (the
    prefill path launches kernels only: no allocation, no memset). Three replays, with eager work
    and synchronisations between them, each bit-identical to the eager call."""
    w = configs.GPT2_SMALL_CAUSAL
    q, k, v, lt = inputs.make(w, DEV)
    o_e, l_e = run_lib(q, k, v, w.scale, w.causal, lt)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=DEV)

    def launch():
        fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lt, None)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), f"replay {rep}: O differs"
        assert torch.equal(lse, l_e), f"replay {rep}: lse differs"
        run_lib(q, k, v, w.scale, w.causal, lt)  # eager work between replays
