"""Checks that pin the CPU oracle to facts fixed by the definition and by mathematics.

Each ``pin_*`` takes an attention implementation with the oracle's signature
``impl(q, k, v, scale, causal=False, kv_seqlens=None, return_p=False)`` and raises
AssertionError when the implementation disagrees with:

* brute force at 50 significant digits (mpmath), P = e^S / sum e^S with no max shift;
* hand-worked cases (tests/golden/worked_examples.json);
* closed forms: Q = 0 gives the mean of the allowed V rows and lse = ln |A_i|; a single allowed
  key returns its V row and lse = its score; constant V returns that constant; causal row 0
  returns V_0;
* invariants: rows of P sum to 1, masked keys get exactly zero weight, permuting keys with
  their values changes nothing, shifting every key by t leaves O unchanged and moves lse by
  scale * q.t;
* stability: scores of magnitude ~1000 stay finite and exact;
* the padding contract: NaN, Inf or huge values in key slots at or past L_b leave every output
  bit-identical to zero padding (those slots never enter a product).

The same pins run against deliberately broken copies of the oracle (tests/test_oracle_mutants.py)
to show that a plausible mistake fails at least one of them.
"""

from __future__ import annotations

import json
import os

import mpmath
import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def brute_force_mp(q, k, v, scale, causal, lens, digits=50):
    """Definition evaluated in mpmath at ``digits`` significant digits, with no max shift."""
    mpmath.mp.dps = digits
    bsz, heads, nq, d = q.shape
    nk = k.shape[2]
    o = np.zeros((bsz, heads, nq, v.shape[3]))
    lse = np.zeros((bsz, heads, nq))
    for b in range(bsz):
        length = nk if lens is None else min(max(int(lens[b]), 0), nk)
        for h in range(heads):
            for i in range(nq):
                allowed = [j for j in range(nk) if j < length and (not causal or j <= i)]
                if not allowed:
                    o[b, h, i] = 0.0
                    lse[b, h, i] = -np.inf
                    continue
                sc = {}
                for j in allowed:
                    acc = mpmath.mpf(0)
                    for t in range(d):
                        acc += mpmath.mpf(float(q[b, h, i, t])) * mpmath.mpf(float(k[b, h, j, t]))
                    sc[j] = mpmath.mpf(float(scale)) * acc
                ex = {j: mpmath.exp(sc[j]) for j in allowed}
                z = mpmath.fsum(ex.values())
                for t in range(v.shape[3]):
                    o[b, h, i, t] = float(mpmath.fsum(ex[j] * mpmath.mpf(float(v[b, h, j, t]))
                                                      for j in allowed) / z)
                lse[b, h, i] = float(mpmath.log(z))
    return o, lse


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: infinities differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin])))
        assert err <= tol, f"{what}: error {err:.3e} > {tol:.1e}"


def pin_brute_force(impl):
    cases = [
        # (B, H, Nq, Nk, d, causal, lens, seed)
        (1, 1, 3, 5, 2, False, None, 1),
        (2, 1, 4, 7, 3, False, [7, 3], 2),
        (1, 2, 6, 6, 4, True, None, 3),
        (2, 2, 5, 5, 3, True, [5, 2], 4),
        (2, 1, 3, 8, 4, False, [0, 1], 5),
        (1, 1, 8, 8, 1, True, [6], 6),
    ]
    for bsz, heads, nq, nk, d, causal, lens, seed in cases:
        r = _rng(seed)
        q = r.standard_normal((bsz, heads, nq, d))
        k = r.standard_normal((bsz, heads, nk, d))
        v = r.standard_normal((bsz, heads, nk, d + 1))
        scale = 0.7
        o, lse = impl(q, k, v, scale, causal, lens)
        o_ref, lse_ref = brute_force_mp(q, k, v, scale, causal, lens)
        _close(o, o_ref, 1e-12, f"O brute force case seed={seed}")
        _close(lse, lse_ref, 1e-12, f"lse brute force case seed={seed}")


def pin_golden(impl):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        o_ref = np.array(c["o"], dtype=np.float64)
        lse_ref = np.array([[[float(x) for x in row] for row in hh] for hh in c["lse"]])
        o, lse = impl(q, k, v, c["scale"], c["causal"], c["kv_seqlens"])
        _close(o, o_ref, 1e-12, f"O golden {c['name']}")
        _close(lse, lse_ref, 1e-12, f"lse golden {c['name']}")


def pin_zero_query_is_mean(impl):
    r = _rng(11)
    for causal, lens in ((False, [9, 4, 1]), (True, None), (True, [9, 5, 2])):
        bsz, nq = 3, 9
        nk = nq
        q = np.zeros((bsz, 2, nq, 5))
        k = r.standard_normal((bsz, 2, nk, 5))
        v = r.standard_normal((bsz, 2, nk, 3))
        o, lse = impl(q, k, v, 0.9, causal, lens)
        for b in range(bsz):
            length = nk if lens is None else lens[b]
            for i in range(nq):
                allowed = [j for j in range(nk) if j < length and (not causal or j <= i)]
                if not allowed:
                    continue
                _close(o[b, :, i], v[b][:, allowed].mean(axis=1), 1e-14, "Q=0 mean")
                assert np.all(lse[b, :, i] == np.log(len(allowed))), "Q=0 lse = ln|A|"


def pin_single_key(impl):
    r = _rng(12)
    q = r.standard_normal((2, 2, 4, 6))
    k = r.standard_normal((2, 2, 5, 6))
    v = r.standard_normal((2, 2, 5, 6))
    o, lse = impl(q, k, v, 0.3, False, [1, 1])
    _close(o, np.broadcast_to(v[:, :, :1, :], o.shape), 1e-15, "single key O = V_0")
    s0 = 0.3 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0, :])
    _close(lse, s0, 1e-14, "single key lse = S_i0")
    # A single key without any length argument.
    o1, lse1 = impl(q, k[:, :, :1], v[:, :, :1], 0.3, False, None)
    _close(o1, np.broadcast_to(v[:, :, :1, :], o1.shape), 1e-15, "Nk=1 O = V_0")
    _close(lse1, s0, 1e-14, "Nk=1 lse")


def pin_constant_v(impl):
    r = _rng(13)
    q = r.standard_normal((1, 3, 7, 4))
    k = r.standard_normal((1, 3, 7, 4))
    v = np.full((1, 3, 7, 4), -2.75)
    for causal in (False, True):
        o, _ = impl(q, k, v, 1.3, causal, None)
        _close(o, np.full_like(o, -2.75), 1e-14, "constant V")


def pin_causal_first_row(impl):
    r = _rng(14)
    q = r.standard_normal((2, 2, 6, 3))
    k = r.standard_normal((2, 2, 6, 3))
    v = r.standard_normal((2, 2, 6, 3))
    o, lse = impl(q, k, v, 0.5, True, None)
    _close(o[:, :, 0], v[:, :, 0], 1e-15, "causal row 0 O = V_0")
    _close(lse[:, :, 0], 0.5 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-14, "causal lse_0")


def pin_probabilities(impl):
    r = _rng(15)
    q = r.standard_normal((2, 2, 6, 4))
    k = r.standard_normal((2, 2, 6, 4))
    v = r.standard_normal((2, 2, 6, 4))
    lens = [6, 3]
    for causal in (False, True):
        o, lse, p = impl(q, k, v, 0.8, causal, lens, return_p=True)
        for b in range(2):
            for i in range(6):
                allowed = np.array([j < lens[b] and (not causal or j <= i) for j in range(6)])
                assert np.all(p[b, :, i, ~allowed] == 0.0), "masked keys must have zero weight"
                assert np.all(p[b, :, i, allowed] > 0.0), "allowed keys have positive weight"
                _close(p[b, :, i].sum(axis=-1), np.ones(2), 1e-14, "rows of P sum to 1")
        _close(np.einsum("bhij,bhjd->bhid", p, v), o, 1e-14, "O = P V")


def pin_key_permutation(impl):
    r = _rng(16)
    q = r.standard_normal((2, 2, 5, 4))
    k = r.standard_normal((2, 2, 9, 4))
    v = r.standard_normal((2, 2, 9, 4))
    perm = r.permutation(9)
    o1, lse1 = impl(q, k, v, 0.6, False, None)
    o2, lse2 = impl(q, k[:, :, perm], v[:, :, perm], 0.6, False, None)
    _close(o2, o1, 1e-13, "key permutation O")
    _close(lse2, lse1, 1e-13, "key permutation lse")


def pin_key_shift(impl):
    r = _rng(17)
    q = r.standard_normal((1, 2, 6, 4))
    k = r.standard_normal((1, 2, 6, 4))
    v = r.standard_normal((1, 2, 6, 4))
    t = r.standard_normal(4)
    for causal, lens in ((False, [4]), (True, None)):
        o1, lse1 = impl(q, k, v, 0.7, causal, lens)
        o2, lse2 = impl(q, k + t, v, 0.7, causal, lens)
        _close(o2, o1, 1e-13, "key shift O")
        _close(lse2, lse1 + 0.7 * (q @ t), 1e-13, "key shift lse")


def pin_large_scores(impl):
    r = _rng(18)
    q = 20.0 * r.standard_normal((1, 1, 4, 3))
    k = 20.0 * r.standard_normal((1, 1, 6, 3))
    v = r.standard_normal((1, 1, 6, 3))
    o, lse = impl(q, k, v, 1.0, False, None)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "large scores stay finite"
    o_ref, lse_ref = brute_force_mp(q, k, v, 1.0, False, None)
    _close(o, o_ref, 1e-12, "large scores O")
    _close(lse, lse_ref, 1e-12, "large scores lse")


def poison_padding(x, lens, fill):
    """Copy of x (B, H, N, d) whose slots at or past each sequence's length hold ``fill``
    (a scalar or an array broadcast over those slots)."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[2]
    for b in range(y.shape[0]):
        length = n if lens is None else min(max(int(lens[b]), 0), n)
        y[b, :, length:] = fill
    return y


# Key and value paddings that a product touching them could not survive: NaN, both infinities,
# and huge finite values whose products overflow.
POISONS = ((np.nan, np.inf), (np.inf, np.nan), (-np.inf, -np.inf), (1e308, -1e308))


def pin_poisoned_padding(impl):
    """Key slots at or past L_b are outside every allowed set, so whatever they hold must leave
    O and lse bit-identical to zero padding: the slots must never enter a product."""
    cases = [
        # (B, H, Nq, Nk, d, causal, lens, seed)
        (4, 2, 4, 5, 3, False, [3, 5, 0, 1], 41),
        (2, 1, 6, 6, 2, True, [4, 6], 42),
        (1, 1, 3, 9, 4, False, [2], 43),
    ]
    for bsz, heads, nq, nk, d, causal, lens, seed in cases:
        r = _rng(seed)
        q = r.standard_normal((bsz, heads, nq, d))
        k = poison_padding(r.standard_normal((bsz, heads, nk, d)), lens, 0.0)
        v = poison_padding(r.standard_normal((bsz, heads, nk, d + 1)), lens, 0.0)
        o_ref, lse_ref = impl(q, k, v, 0.9, causal, lens)
        for kfill, vfill in POISONS:
            with np.errstate(all="ignore"):
                o, lse = impl(q, poison_padding(k, lens, kfill), poison_padding(v, lens, vfill),
                              0.9, causal, lens)
            assert np.all(np.isfinite(o)), f"poisoned padding ({kfill}, {vfill}) reached O"
            assert np.array_equal(o, o_ref), f"poisoned padding ({kfill}, {vfill}) changed O"
            assert np.array_equal(lse, lse_ref), f"poisoned padding ({kfill}, {vfill}) changed lse"


ALL_PINS = [pin_brute_force, pin_golden, pin_zero_query_is_mean, pin_single_key, pin_constant_v,
            pin_causal_first_row, pin_probabilities, pin_key_permutation, pin_key_shift,
            pin_large_scores, pin_poisoned_padding]


# ---- sliding windows: impl(q, k, v, scale, causal=False, kv_seqlens=None, return_p=False,
# window=None), window = (left, right) with -1 for an unlimited side; query i sits at key i.

def brute_force_window_mp(q, k, v, scale, lens, window, digits=50):
    """The windowed definition at ``digits`` digits, no max shift, from the allowed set written
    out key by key."""
    left, right = window
    mpmath.mp.dps = digits
    bsz, heads, nq, d = q.shape
    nk = k.shape[2]
    o = np.zeros((bsz, heads, nq, v.shape[3]))
    lse = np.zeros((bsz, heads, nq))
    for b in range(bsz):
        length = nk if lens is None else min(max(int(lens[b]), 0), nk)
        for h in range(heads):
            for i in range(nq):
                allowed = [j for j in range(nk)
                           if j < length and (left < 0 or i - j <= left) and (right < 0 or j - i <= right)]
                if not allowed:
                    o[b, h, i] = 0.0
                    lse[b, h, i] = -np.inf
                    continue
                ex = {}
                for j in allowed:
                    acc = mpmath.fsum(mpmath.mpf(float(q[b, h, i, t])) * mpmath.mpf(float(k[b, h, j, t]))
                                      for t in range(d))
                    ex[j] = mpmath.exp(mpmath.mpf(float(scale)) * acc)
                z = mpmath.fsum(ex.values())
                for t in range(v.shape[3]):
                    o[b, h, i, t] = float(mpmath.fsum(ex[j] * mpmath.mpf(float(v[b, h, j, t])) for j in allowed) / z)
                lse[b, h, i] = float(mpmath.log(z))
    return o, lse


def pin_window_brute_force(impl):
    cases = [
        # (B, H, Nq, Nk, d, lens, window, seed)
        (1, 1, 7, 7, 2, None, (2, 0), 21),
        (2, 1, 6, 6, 3, [6, 4], (1, 1), 22),
        (1, 2, 5, 9, 2, None, (0, 3), 23),
        (2, 1, 8, 8, 2, [8, 3], (3, -1), 24),
        (1, 1, 9, 5, 3, None, (-1, 2), 25),
    ]
    for bsz, heads, nq, nk, d, lens, window, seed in cases:
        r = _rng(seed)
        q = r.standard_normal((bsz, heads, nq, d))
        k = r.standard_normal((bsz, heads, nk, d))
        v = r.standard_normal((bsz, heads, nk, d + 1))
        o, lse = impl(q, k, v, 0.9, False, lens, window=window)
        o_ref, lse_ref = brute_force_window_mp(q, k, v, 0.9, lens, window)
        _close(o, o_ref, 1e-12, f"O window brute force seed={seed}")
        _close(lse, lse_ref, 1e-12, f"lse window brute force seed={seed}")


def pin_window_diagonal(impl):
    # Window (0, 0): each query sees only key i, so O_i = V_i and lse_i = scale * q_i . k_i
    # (rows i >= min(Nk, L_b) see nothing).
    r = _rng(26)
    q = r.standard_normal((2, 2, 6, 4))
    k = r.standard_normal((2, 2, 6, 4))
    v = r.standard_normal((2, 2, 6, 4))
    o, lse = impl(q, k, v, 0.4, False, [6, 4], window=(0, 0))
    diag = 0.4 * np.sum(q * k, axis=-1)
    for b, length in enumerate((6, 4)):
        _close(o[b, :, :length], v[b, :, :length], 1e-15, "window (0,0) O_i = V_i")
        _close(lse[b, :, :length], diag[b, :, :length], 1e-14, "window (0,0) lse_i = S_ii")
        assert np.all(o[b, :, length:] == 0.0) and np.all(np.isneginf(lse[b, :, length:]))


def pin_window_reductions(impl):
    # (-1, 0) is the causal mask; (-1, -1) and any window wider than the sequence are no mask.
    r = _rng(27)
    q = r.standard_normal((2, 2, 7, 3))
    k = r.standard_normal((2, 2, 7, 3))
    v = r.standard_normal((2, 2, 7, 3))
    for lens in (None, [7, 2]):
        oc, lc = impl(q, k, v, 0.6, True, lens)
        ow, lw = impl(q, k, v, 0.6, False, lens, window=(-1, 0))
        _close(ow, oc, 1e-15, "window (-1,0) = causal O")
        _close(lw, lc, 1e-15, "window (-1,0) = causal lse")
        on, ln_ = impl(q, k, v, 0.6, False, lens)
        for wnd in ((-1, -1), (6, 6), (100, -1)):
            ow, lw = impl(q, k, v, 0.6, False, lens, window=wnd)
            _close(ow, on, 1e-15, f"window {wnd} = no mask O")
            _close(lw, ln_, 1e-15, f"window {wnd} = no mask lse")


def pin_window_probabilities(impl):
    # Keys outside the window get exactly zero weight; inside, positive weights summing to 1.
    r = _rng(28)
    q = r.standard_normal((1, 2, 9, 3))
    k = r.standard_normal((1, 2, 9, 3))
    v = r.standard_normal((1, 2, 9, 3))
    for left, right in ((2, 0), (1, 3), (0, 2)):
        o, lse, p = impl(q, k, v, 0.5, False, None, return_p=True, window=(left, right))
        for i in range(9):
            allowed = np.array([i - left <= j <= i + right for j in range(9)])
            assert np.all(p[0, :, i, ~allowed] == 0.0), "keys outside the window have zero weight"
            assert np.all(p[0, :, i, allowed] > 0.0), "keys inside the window have positive weight"
            _close(p[0, :, i].sum(axis=-1), np.ones(2), 1e-14, "window rows of P sum to 1")


WINDOW_PINS = [pin_window_brute_force, pin_window_diagonal, pin_window_reductions,
               pin_window_probabilities]


# ---- backward pass: impl(q, k, v, do, scale, causal=False, kv_seqlens=None, window=None)
# returns (dq, dk, dv); checked against central differences of the (separately pinned) forward.

def _loss(fwd, q, k, v, do, scale, causal, lens, window):
    o, _ = fwd(q, k, v, scale, causal, lens, window=window)
    return float(np.sum(o * do))


def _fd_grad(fwd, x, which, args, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        g[idx] = (_loss(fwd, *args(which, xp)) - _loss(fwd, *args(which, xm))) / (2 * h)
    return g


def pin_bwd_finite_differences(impl, fwd):
    cases = [
        # (B, H, Nq, Nk, d, causal, lens, window, seed)
        (1, 1, 4, 4, 3, False, None, None, 31),
        (1, 2, 5, 5, 2, True, None, None, 32),
        (2, 1, 3, 6, 3, False, [6, 2], None, 33),
        (1, 1, 6, 6, 2, False, None, (1, 1), 34),
        (2, 1, 4, 4, 2, True, [4, 3], None, 35),
    ]
    for bsz, heads, nq, nk, d, causal, lens, window, seed in cases:
        r = _rng(seed)
        q = r.standard_normal((bsz, heads, nq, d))
        k = r.standard_normal((bsz, heads, nk, d))
        v = r.standard_normal((bsz, heads, nk, d + 1))
        do = r.standard_normal((bsz, heads, nq, d + 1))
        scale = 0.8
        dq, dk, dv = impl(q, k, v, do, scale, causal, lens, window=window)

        def args(which, x):
            qq, kk, vv = (x if which == 0 else q), (x if which == 1 else k), (x if which == 2 else v)
            return qq, kk, vv, do, scale, causal, lens, window
        for which, (g, x) in enumerate(((dq, q), (dk, k), (dv, v))):
            _close(g, _fd_grad(fwd, x, which, args), 1e-7, f"grad {'qkv'[which]} vs central differences seed={seed}")


def pin_bwd_single_key(impl, fwd):
    # One allowed key: the softmax is constant 1, so dQ = dK = 0 and dV_0 = sum_i dO_i.
    r = _rng(36)
    q = r.standard_normal((2, 2, 4, 3))
    k = r.standard_normal((2, 2, 5, 3))
    v = r.standard_normal((2, 2, 5, 3))
    do = r.standard_normal((2, 2, 4, 3))
    dq, dk, dv = impl(q, k, v, do, 0.7, False, [1, 1])
    assert np.all(dq == 0.0) and np.all(dk == 0.0), "single key: dQ = dK = 0"
    _close(dv[:, :, 0], do.sum(axis=2), 1e-14, "single key: dV_0 = sum dO")
    assert np.all(dv[:, :, 1:] == 0.0), "keys past the length get no gradient"


def pin_bwd_uniform(impl, fwd):
    # Q = 0: uniform weights over the allowed keys, so dV_j = sum_{i: j in A_i} dO_i / |A_i|.
    r = _rng(37)
    q = np.zeros((1, 2, 6, 3))
    k = r.standard_normal((1, 2, 6, 3))
    v = r.standard_normal((1, 2, 6, 2))
    do = r.standard_normal((1, 2, 6, 2))
    _, _, dv = impl(q, k, v, do, 0.9, True, None)
    ref = np.zeros_like(dv)
    for i in range(6):
        ref[:, :, : i + 1] += do[:, :, i : i + 1] / (i + 1)
    _close(dv, ref, 1e-14, "Q=0 causal dV")


def pin_bwd_key_shift_sums(impl, fwd):
    # O does not change when every key moves by the same vector t, so the derivative of the loss
    # along that move, sum_j dK_j . t, is 0 for every t: sum_j dK_j = 0 per (b, h).
    r = _rng(38)
    q = r.standard_normal((2, 2, 5, 4))
    k = r.standard_normal((2, 2, 5, 4))
    v = r.standard_normal((2, 2, 5, 3))
    do = r.standard_normal((2, 2, 5, 3))
    for causal, lens in ((False, [5, 3]), (True, None)):
        _, dk, _ = impl(q, k, v, do, 0.6, causal, lens)
        _close(dk.sum(axis=2), np.zeros((2, 2, 4)), 1e-13, "sum_j dK_j = 0")


def pin_bwd_poisoned_padding(impl, fwd):
    """Poisoned key slots past L_b leave dQ, dK and dV bit-identical to zero padding, and those
    slots get exactly zero gradient."""
    for bsz, heads, nq, nk, d, causal, lens, seed in ((3, 2, 4, 6, 3, False, [2, 6, 0], 44),
                                                      (2, 1, 5, 5, 2, True, [3, 5], 45)):
        r = _rng(seed)
        q = r.standard_normal((bsz, heads, nq, d))
        k = poison_padding(r.standard_normal((bsz, heads, nk, d)), lens, 0.0)
        v = poison_padding(r.standard_normal((bsz, heads, nk, d + 1)), lens, 0.0)
        do = r.standard_normal((bsz, heads, nq, d + 1))
        ref = impl(q, k, v, do, 0.8, causal, lens)
        for b, length in enumerate(lens):
            assert np.all(ref[1][b, :, length:] == 0.0) and np.all(ref[2][b, :, length:] == 0.0), \
                "slots past the length get zero key and value gradients"
        for kfill, vfill in POISONS:
            with np.errstate(all="ignore"):
                got = impl(q, poison_padding(k, lens, kfill), poison_padding(v, lens, vfill), do,
                           0.8, causal, lens)
            for name, g, g_ref in zip("qkv", got, ref):
                assert np.all(np.isfinite(g)), f"poisoned padding ({kfill}, {vfill}) reached d{name}"
                assert np.array_equal(g, g_ref), f"poisoned padding ({kfill}, {vfill}) changed d{name}"


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_single_key, pin_bwd_uniform, pin_bwd_key_shift_sums,
            pin_bwd_poisoned_padding]


# ---- FP8 (e4m3) path. Each pin takes a namespace ``f`` with the oracle's functions: decode,
# round, quantize, attention (attention_fwd_fp8) and bound (p_rounding_bound), and pins them to
# torch's own float8_e4m3fn conversion (a library routine of the same format), exact rational
# arithmetic, 50-digit brute force, and a simulation of the probability rounding.

def _torch_e4m3_codes(x):
    import torch
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values(codes):
    import torch
    t = torch.tensor(np.asarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _finite_positive_table():
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: +0 and every positive finite value
    return codes, _torch_e4m3_values(codes)


def pin_fp8_decode_table(f):
    codes = np.arange(256, dtype=np.uint8)
    got = np.asarray(f.decode(codes), dtype=np.float64)
    ref = _torch_e4m3_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN codes"
    assert np.array_equal(got[~nan], ref[~nan]), "decoded values differ from the library's"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "signs"
    # Landmarks of the format: largest finite, smallest normal, smallest subnormal, one.
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0xFE] == -448.0


def pin_fp8_round_library(f):
    rng = _rng(101)
    mags = np.exp2(rng.uniform(-13.0, np.log2(460.0), 4000))
    _, vals = _finite_positive_table()
    mids = (vals[:-1] + vals[1:]) / 2.0          # every tie between neighbours below 448
    x = np.concatenate([mags, vals, mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20), [0.0]])
    x = np.concatenate([x, -x]).astype(np.float32).astype(np.float64)
    got = np.asarray(f.round(x))
    ref = _torch_e4m3_codes(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"codes differ from the library's at x = {x[bad[:5]]}"


def pin_fp8_round_nearest(f):
    codes, vals = _finite_positive_table()
    rng = _rng(102)
    x = np.concatenate([np.exp2(rng.uniform(-12.0, 8.8, 3000)), (vals[1:] + vals[:-1]) / 2.0])
    x = x[x <= 448.0]
    got = np.asarray(f.round(x)).astype(np.int64)
    for xi, c in zip(x, got):
        dist = np.abs(vals - xi)
        best = np.nonzero(dist == dist.min())[0]
        assert c in codes[best], f"{xi}: code {c:#x} is not a nearest value"
        if best.size > 1:
            assert c % 2 == 0, f"{xi}: tie not resolved to the even mantissa"


def pin_fp8_round_trip_and_saturation(f):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = np.asarray(f.round(np.asarray(f.decode(codes), dtype=np.float64)))
    assert np.array_equal(back, codes), "encode(decode(c)) != c"
    sat = np.asarray(f.round(np.array([448.0, 470.0, 1.0e6, -500.0, np.inf])))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E], f"saturation: {sat}"
    assert int(np.asarray(f.round(np.array([np.nan])))[0]) & 0x7F == 0x7F


def _fp32_nearest(fr):
    """The fp32 value nearest to the Fraction fr (ties to even), found with exact arithmetic."""
    from fractions import Fraction
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        dist = abs(Fraction(float(cand)) - fr)
        key = (dist, int(np.frombuffer(np.float32(cand).tobytes(), dtype=np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def _bf16_grid(shape, seed, std=1.0):
    x = _rng(seed).normal(0.0, std, shape).astype(np.float32)
    b = (x.view(np.uint32) + np.uint32(0x8000)) & np.uint32(0xFFFF0000)  # round to bf16
    return b.view(np.float32).astype(np.float64)


def pin_fp8_quantize(f):
    from fractions import Fraction
    B, H, N, d = 2, 3, 70, 16
    x = _bf16_grid((B, H, N, d), 103, 2.0)
    x[1, 2] = 0.0                                   # an all-zero slice
    lens = [70, 33]
    poisoned = x.copy()
    poisoned[1, :, 33:] = 1.0e4
    codes, s = f.quantize(poisoned, kv_seqlens=lens)
    codes = np.asarray(codes)
    s = np.asarray(s, dtype=np.float32)
    codes0, s0 = f.quantize(x, kv_seqlens=lens)
    assert np.array_equal(codes, np.asarray(codes0)) and np.array_equal(s, np.asarray(s0)), \
        "rows past the length changed the result"
    assert np.all(codes[1, :, 33:] == 0), "rows past the length must be stored as zero"
    assert s[1, 2] == 1.0 and np.all(codes[1, 2] == 0), "all-zero slice"
    for b in range(B):
        L = lens[b]
        for h in range(H):
            rows = x[b, h, :L]
            amax = np.max(np.abs(rows))
            if amax == 0:
                continue
            # s is the fp32 value nearest to amax / 448 (exact rational arithmetic).
            assert s[b, h] == _fp32_nearest(Fraction(float(amax)) / 448), f"scale of ({b}, {h})"
            # Codes: e4m3 of the fp32 quotient x / s, the quotient rounded with exact arithmetic.
            sf = Fraction(float(s[b, h]))
            y = np.array([_fp32_nearest(Fraction(float(v)) / sf) for v in rows.ravel()],
                         dtype=np.float32)
            want = _torch_e4m3_codes(y).reshape(rows.shape)
            assert np.array_equal(codes[b, h, :L], want), f"codes of ({b}, {h})"
            # The largest magnitude maps to +-448; dequantised values are within half a unit.
            at = np.abs(rows) == amax
            assert np.all(np.isin(codes[b, h, :L][at], [0x7E, 0xFE]))
            deq = np.asarray(f.decode(codes[b, h, :L])) * float(s[b, h])
            assert np.all(np.abs(deq - rows) <= 2.0 ** -4 * np.abs(rows) + 2.0 ** -10 * float(s[b, h]) * 1.001)
    # Transposed layout: V^T per (b, h), columns padded with zeros to a multiple of 64.
    ct, st = f.quantize(poisoned, kv_seqlens=lens, transpose=True)
    ct = np.asarray(ct)
    assert ct.shape == (B, H, d, 128) and np.array_equal(np.asarray(st), s)
    assert np.array_equal(ct[:, :, :, :N], np.swapaxes(codes, 2, 3)) and np.all(ct[:, :, :, N:] == 0)


def pin_fp8_attention_brute_force(f):
    # Small codes with non-power-of-two scales against the 50-digit definition of the dequantised
    # values (V given transposed, as the path stores it).
    B, H, Nq, Nk, d = 1, 2, 5, 7, 4
    rng = _rng(104)
    q8 = rng.integers(0, 256, (B, H, Nq, d)).astype(np.uint8)
    k8 = rng.integers(0, 256, (B, H, Nk, d)).astype(np.uint8)
    v8 = rng.integers(0, 256, (B, H, Nk, d)).astype(np.uint8)
    for a in (q8, k8, v8):
        a[(a & 0x7F) == 0x7F] = 0x30  # no NaN codes
        a[(a & 0x7F) > 0x50] &= 0xC7  # keep magnitudes moderate
    dq = np.array([[0.37, 1.9]], dtype=np.float32)
    dk = np.array([[0.11, 0.6]], dtype=np.float32)
    dv = np.array([[3.3, 0.07]], dtype=np.float32)
    v8t = np.zeros((B, H, d, 64), dtype=np.uint8)
    v8t[:, :, :, :Nk] = np.swapaxes(v8, 2, 3)
    for causal, lens in ((False, None), (False, [4])):
        o, lse = f.attention(q8, k8, v8t, dq, dk, dv, 0.5, causal=causal, kv_seqlens=lens)
        qv = _torch_e4m3_values(q8) * dq[:, :, None, None].astype(np.float64)
        kv = _torch_e4m3_values(k8) * dk[:, :, None, None].astype(np.float64)
        vv = _torch_e4m3_values(v8) * dv[:, :, None, None].astype(np.float64)
        o_ref, lse_ref = brute_force_mp(qv, kv, vv, 0.5, causal, lens)
        _close(o, o_ref, 1e-12, "fp8 O vs brute force")
        _close(lse, lse_ref, 1e-12, "fp8 lse vs brute force")


def pin_fp8_bound_simulation(f):
    # Round 8 * 2^(t - m') to e4m3 for offsets m' at or below the row maximum (the GPU path's
    # lazy offset), normalise by the unrounded sum, and compare with the exact weights.
    rng = _rng(105)
    R, N = 256, 300
    t = rng.uniform(-24.0, 0.0, (R, N))
    t[rng.random((R, N)) < 0.1] = -np.inf                     # masked pairs
    t[:, 0] = 0.0                                              # row maximum 0
    p = np.exp2(t)
    p = p / p.sum(axis=1, keepdims=True)
    bound = np.asarray(f.bound(p))
    worst = 0.0
    for shift in (0.0, 0.7, 2.9):                              # m' = max - shift (p~ <= 2^shift)
        pt = np.exp2(t + shift)
        x = 8.0 * pt
        qv = _torch_e4m3_values(_torch_e4m3_codes(x))
        w = qv / (8.0 * pt.sum(axis=1, keepdims=True))
        err = np.abs(w - p)
        assert np.all(err <= bound * (1 + 1e-9) + 1e-300), "weight error above the bound"
        ok = bound > 0
        worst = max(worst, float(np.max(err[ok] / bound[ok])))
    assert np.all(bound[np.isinf(t)] == 0.0), "masked pairs must get a zero bound"
    assert worst > 0.5, f"bound far from tight ({worst:.3f}): it would hide real errors"


FP8_PINS = [pin_fp8_decode_table, pin_fp8_round_library, pin_fp8_round_nearest,
            pin_fp8_round_trip_and_saturation, pin_fp8_quantize, pin_fp8_attention_brute_force,
            pin_fp8_bound_simulation]
