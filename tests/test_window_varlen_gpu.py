"""GPU parity of sliding-window masks (fa_fwd_window) and packed variable-length batches
(fa_fwd_varlen), through the C ABI, against the fp64 oracle on the same input bits.

Windows: causal sliding windows, symmetric local windows, left-only windows, the diagonal window
(0, 0), and the reductions (-1, 0) = causal and (-1, -1) = no mask, over ragged lengths, both head
sizes, Nq = 1 and huge scores. Packed batches: sequences of lengths 0, 1, ragged and long packed
head-major without padding, with and without windows, queries fewer than keys, and isolation
(poisoning one sequence's keys leaves the others bit-identical).
"""

import numpy as np
import pytest
import torch

import io_aware_exact_23_amd as fa
from io_aware_exact_23_amd import configs, inputs
from oracle import attention_fwd

from parity_util import compare, f32, run_oracle, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()


def _rand(shape, seed, std=1.0):
    return inputs.normal(shape, seed, DEV, "bf16", std)


WINDOWS = [
    # B, H, N, d, (left, right), lens
    (1, 2, 2048, 128, (255, 0), None),
    (2, 2, 2100, 64, (100, 100), [2100, 1500]),
    (1, 1, 3000, 128, (-1, 0), None),
    (2, 1, 700, 64, (0, 0), [700, 300]),
    (1, 2, 1000, 128, (64, -1), None),
    (1, 1, 513, 64, (-1, -1), None),
    (2, 2, 300, 128, (17, 3), [300, 129]),
    (1, 3, 4100, 64, (1023, 0), [4000]),
    # left-only windows: masked tiles at the front, then whole tiles (the boundary between the
    # masked prefix and the unmasked loop, where the second wave group lags one tile behind)
    (1, 1, 3000, 128, (700, -1), None),
    (1, 2, 2500, 64, (1, -1), [2500]),
]


@pytest.mark.parametrize("B,H,N,d,window,lens", WINDOWS)
def test_window(B, H, N, d, window, lens):
    q, k, v = (_rand((B, H, N, d), 7 * N + s + d) for s in range(3))
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = fa.attention(q, k, v, scale=d ** -0.5, kv_seqlens=lt, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = run_oracle(q, k, v, d ** -0.5, False, lt, window=window)
    print(f"window {window} {B}x{H}x{N} d={d} lens={lens}", flush=True)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", what=f"window {window} N={N}")


@pytest.mark.parametrize("window", [(255, 0), (100, 100), (-1, -1)])
def test_window_poisoned_padding_against_oracle(window):
    """NaN in the key slots and Inf in the value slots at or past L_b, under sliding windows: the
    output must match the oracle (which never reads those slots) and equal the zero-padded run bit
    for bit."""
    B, H, N, d = 2, 2, 2100, 128
    lens = [2100, 1333]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q, k, v = (_rand((B, H, N, d), 300 + s) for s in range(3))
    inputs.fill_padding(k, lt.cpu(), 0.0)
    inputs.fill_padding(v, lt.cpu(), 0.0)
    o1, l1 = fa.attention(q, k, v, scale=d ** -0.5, kv_seqlens=lt, window=window)
    kp, vp = k.clone(), v.clone()
    inputs.fill_padding(kp, lt.cpu(), float("nan"))
    inputs.fill_padding(vp, lt.cpu(), float("inf"))
    o2, l2 = fa.attention(q, kp, vp, scale=d ** -0.5, kv_seqlens=lt, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = run_oracle(q, kp, vp, d ** -0.5, False, lt, window=window)
    compare(to_f64(o2), to_f64(l2), o_ref, lse_ref, "bf16", what=f"poisoned window {window}")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_window_reductions_match_fa_fwd():
    # (-1, 0) is the causal mask and (-1, -1) no mask: the general kernel against fa_fwd's.
    q, k, v = (_rand((2, 2, 2048, 128), 90 + s) for s in range(3))
    for window, causal in (((-1, 0), True), ((-1, -1), False)):
        o1, l1 = fa.attention(q, k, v, window=window)
        o2, l2 = fa.attention(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert (o1.float() - o2.float()).abs().max().item() <= 2 ** -7
        assert (l1 - l2).abs().max().item() < 1e-5


def test_window_single_query_and_huge_scores():
    q, k, v = _rand((2, 2, 1, 128), 1), _rand((2, 2, 900, 128), 2), _rand((2, 2, 900, 128), 3)
    lt = torch.tensor([900, 77], dtype=torch.int32, device=DEV)
    o, lse = fa.attention(q, k, v, scale=128 ** -0.5, kv_seqlens=lt, window=(-1, -1))
    torch.cuda.synchronize()
    o_ref, lse_ref = run_oracle(q, k, v, 128 ** -0.5, False, lt)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", what="window Nq=1")
    q, k = _rand((1, 2, 2048, 64), 4, std=4.0), _rand((1, 2, 2048, 64), 5, std=4.0)
    v = _rand((1, 2, 2048, 64), 6)
    o, lse = fa.attention(q, k, v, scale=2.0, window=(300, 0))
    torch.cuda.synchronize()
    o_ref, lse_ref = run_oracle(q, k, v, 2.0, False, None, window=(300, 0))
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", what="window huge scores")


def _packed(lens_q, lens_k, H, d, seed, std=1.0):
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    q = _rand((H, tq, d), seed, std)
    k = _rand((H, tk, d), seed + 1, std)
    v = _rand((H, tk, d), seed + 2)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lens_q)]), dtype=torch.int32, device=DEV)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lens_k)]), dtype=torch.int32, device=DEV)
    return q, k, v, cq, ck


def _check_packed(q, k, v, cq, ck, scale, window, o, lse, what):
    cqn, ckn = cq.cpu().numpy(), ck.cpu().numpy()
    og, lg = to_f64(o), to_f64(lse)
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    for b in range(len(cqn) - 1):
        q0, q1, k0, k1 = cqn[b], cqn[b + 1], ckn[b], ckn[b + 1]
        if q1 == q0:
            continue
        o_ref, lse_ref = attention_fwd(qd[None, :, q0:q1], kd[None, :, k0:k1], vd[None, :, k0:k1],
                                       f32(scale), window=window)
        compare(og[None, :, q0:q1], lg[None, :, q0:q1], o_ref, lse_ref, "bf16", what=f"{what} seq {b}")


VARLEN = [
    # lengths (q == k), H, d, window
    ([0, 1, 130, 2049, 700, 64], 3, 128, (-1, 0)),
    ([513, 0, 77, 1024], 2, 64, (-1, -1)),
    ([3000, 5, 1500], 2, 128, (300, 0)),
    ([256, 257, 255], 1, 64, (40, 40)),
    ([2600, 900], 2, 128, (500, -1)),
]


@pytest.mark.parametrize("lens,H,d,window", VARLEN)
def test_varlen(lens, H, d, window):
    q, k, v, cq, ck = _packed(lens, lens, H, d, seed=sum(lens) + d)
    o, lse = fa.varlen_attention(q, k, v, cq, ck, max(lens), window=window)
    torch.cuda.synchronize()
    print(f"varlen {lens} H={H} d={d} window={window}", flush=True)
    _check_packed(q, k, v, cq, ck, d ** -0.5, window, o, lse, f"varlen {window}")


def test_varlen_fewer_queries_than_keys():
    # Query i of a sequence sits at key position i of the same sequence (the causal alignment).
    q, k, v, cq, ck = _packed([64, 300, 1], [200, 300, 900], 2, 128, seed=5)
    for window in ((-1, -1), (-1, 0), (20, 10)):
        o, lse = fa.varlen_attention(q, k, v, cq, ck, 300, window=window)
        torch.cuda.synchronize()
        _check_packed(q, k, v, cq, ck, 128 ** -0.5, window, o, lse, f"varlen q<k {window}")


def test_varlen_sequences_are_isolated():
    lens = [300, 2100, 90]
    q, k, v, cq, ck = _packed(lens, lens, 2, 64, seed=9)
    o1, l1 = fa.varlen_attention(q, k, v, cq, ck, max(lens), window=(-1, 0))
    k2, v2 = k.clone(), v.clone()
    k2[:, 300:2400] = 1.0e4
    v2[:, 300:2400] = float("nan")
    o2, l2 = fa.varlen_attention(q, k2, v2, cq, ck, max(lens), window=(-1, 0))
    torch.cuda.synchronize()
    for a, b in ((0, 300), (2400, 2490)):
        assert torch.equal(o1[:, a:b].view(torch.int16), o2[:, a:b].view(torch.int16))
        assert torch.equal(l1[:, a:b], l2[:, a:b])


def _sampled_rows(n, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(0, 8), np.arange(4088, 4104), g.integers(0, n, 32),
                                     np.arange(n - 8, n)]))


def test_sliding_window_16k_workload_sampled_rows():
    """The 4096-key causal sliding window on the 16K causal shape (B 2, H 16, N 16384, d 128), as
    timed by the benchmark; rows on both sides of the point where the window starts to slide."""
    w = configs.LONG_CAUSAL_16K
    q, k, v, _ = inputs.make(w, DEV)
    window = (4095, 0)
    o, lse = fa.attention(q, k, v, scale=w.scale, window=window)
    torch.cuda.synchronize()
    rows = _sampled_rows(w.Nq, 21)
    o_ref, lse_ref = run_oracle(q, k, v, w.scale, False, None, rows=rows, window=window)
    rt = torch.as_tensor(rows, device=DEV)
    compare(to_f64(o[:, :, rt]), to_f64(lse[:, :, rt]), o_ref, lse_ref, "bf16",
            what=f"{w.name} window {window} sampled rows")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_packed_16k_workload_sampled_rows():
    """The 16K causal shape's two sequences packed end to end, head-major ([H, 2*16384, d]), causal
    within each sequence, as timed by the benchmark."""
    w = configs.LONG_CAUSAL_16K
    q, k, v, _ = inputs.make(w, DEV)
    T = w.B * w.Nq
    qp, kp, vp = (t.permute(1, 0, 2, 3).reshape(w.H, T, w.d).contiguous() for t in (q, k, v))
    cu = torch.arange(0, T + 1, w.Nq, dtype=torch.int32, device=DEV)
    o, lse = fa.varlen_attention(qp, kp, vp, cu, cu, w.Nq, scale=w.scale, window=(-1, 0))
    torch.cuda.synchronize()
    rows = _sampled_rows(w.Nq, 22)
    o_ref, lse_ref = run_oracle(q, k, v, w.scale, True, None, rows=rows)
    rt = torch.as_tensor(rows, device=DEV)
    og = torch.stack([o[:, b * w.Nq + rt] for b in range(w.B)])
    lg = torch.stack([lse[:, b * w.Nq + rt] for b in range(w.B)])
    compare(to_f64(og), to_f64(lg), o_ref, lse_ref, "bf16", what=f"{w.name} packed sampled rows")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def _draw_varlen(i):
    """Seeded random packed batch i: per-sequence query and key lengths (queries <= keys, some
    empty, some past 2048), H, d and a window."""
    r = np.random.default_rng(47000 + i)
    n = int(r.integers(1, 7))
    lens_k = [int(x) for x in r.integers(0, 2600 if r.random() < 0.3 else 700, size=n)]
    same = r.random() < 0.6
    lens_q = list(lens_k) if same else [int(r.integers(0, lk + 1)) for lk in lens_k]
    H, d = int(r.integers(1, 4)), int(r.choice([64, 128]))
    kind = r.integers(0, 4)
    window = [(-1, -1), (-1, 0), (int(r.integers(0, 600)), 0),
              (int(r.integers(0, 300)), int(r.integers(0, 300)))][kind]
    return lens_q, lens_k, H, d, window


RANDOM_VARLEN = [_draw_varlen(i) for i in range(12)]


@pytest.mark.parametrize("case", range(len(RANDOM_VARLEN)))
def test_varlen_random_batches(case):
    """Seeded random packed batches against the oracle, sequence by sequence."""
    lens_q, lens_k, H, d, window = RANDOM_VARLEN[case]
    q, k, v, cq, ck = _packed(lens_q, lens_k, H, d, seed=700 + 11 * case)
    what = f"random varlen {case}: q {lens_q} k {lens_k} H={H} d={d} window={window}"
    print(what, flush=True)
    o, lse = fa.varlen_attention(q, k, v, cq, ck, max(max(lens_q), 1), window=window)
    torch.cuda.synchronize()
    _check_packed(q, k, v, cq, ck, d ** -0.5, window, o, lse, what)
