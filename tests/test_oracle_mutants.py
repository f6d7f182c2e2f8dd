"""Planted mistakes in copies of the oracle (CPU only): each must fail at least one pin.

This shows the pins can tell a correct oracle from a plausible wrong one: a dropped scale, an
off-by-one causal or padding mask, a softmax over the wrong axis, a wrong sign in the max
shift, a missing max shift, a missing normalisation, a missing term in lse, a transposed
value product.
"""

import numpy as np
import pytest

from oracle_pins import ALL_PINS


def make_mutant(kind):
    def impl(q, k, v, scale, causal=False, kv_seqlens=None, return_p=False):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float)
        bsz, heads, nq, d = q.shape
        nk = k.shape[2]
        o = np.zeros((bsz, heads, nq, v.shape[3])); lse = np.zeros((bsz, heads, nq))
        pp = np.zeros((bsz, heads, nq, nk))
        for b in range(bsz):
            L = nk if kv_seqlens is None else min(max(int(kv_seqlens[b]), 0), nk)
            if kind == "padding_ignored":
                L = nk
            if kind == "padding_off_by_one":
                L = min(L + 1, nk)
            for h in range(heads):
                j = np.arange(nk)[None, :]
                i = np.arange(nq)[:, None]
                ok = np.broadcast_to(j < L, (nq, nk)).copy()
                if causal:
                    ok &= (j < i) if kind == "causal_strict" else (j <= i)
                sc = 1.0 if kind == "no_scale" else scale
                s = np.where(ok, sc * (q[b, h] @ k[b, h].T), -np.inf)
                has = ok.any(axis=1)
                m = np.where(has, s.max(axis=1), 0.0)
                if kind == "no_shift":
                    m = np.zeros_like(m)
                with np.errstate(over="ignore", invalid="ignore"):
                    if kind == "shift_sign":
                        e = np.where(ok, np.exp(s + m[:, None]), 0.0)
                    elif kind == "softmax_wrong_axis":
                        e = np.where(ok, np.exp(s - np.where(ok, s, -np.inf).max(axis=0, initial=-np.inf)[None, :]), 0.0)
                    else:
                        e = np.where(ok, np.exp(s - m[:, None]), 0.0)
                    if kind == "softmax_wrong_axis":
                        l = e.sum(axis=0)
                        p = np.where(ok, e / np.where(l > 0, l, 1.0)[None, :], 0.0)
                        l = e.sum(axis=1)
                    else:
                        l = e.sum(axis=1)
                        p = e if kind == "no_normalise" else np.where(has[:, None], e / np.where(l > 0, l, 1.0)[:, None], 0.0)
                if kind == "transposed_pv" and nq == nk:
                    out = p.T @ v[b, h]
                else:
                    out = p @ v[b, h]
                out[~has] = 0.0
                with np.errstate(divide="ignore"):
                    lv = np.log(l) if kind == "lse_no_max" else m + np.log(l)
                lv = np.where(has, lv, -np.inf)
                o[b, h], lse[b, h], pp[b, h] = out, lv, p
        if return_p:
            return o, lse, pp
        return o, lse
    return impl


MUTANTS = ["no_scale", "causal_strict", "padding_ignored", "padding_off_by_one", "no_shift",
           "shift_sign", "softmax_wrong_axis", "no_normalise", "lse_no_max", "transposed_pv"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_mutant_fails_some_pin(kind):
    impl = make_mutant(kind)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, FloatingPointError, ValueError, OverflowError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"


def test_unmutated_copy_passes_every_pin():
    impl = make_mutant("none")
    for pin in ALL_PINS:
        pin(impl)


# ---- planted mistakes in the sliding-window mask, each of which must fail a window pin
from oracle_pins import WINDOW_PINS  # noqa: E402


def make_window_mutant(kind):
    def impl(q, k, v, scale, causal=False, kv_seqlens=None, return_p=False, window=None):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float)
        bsz, heads, nq, d = q.shape
        nk = k.shape[2]
        o = np.zeros((bsz, heads, nq, v.shape[3])); lse = np.zeros((bsz, heads, nq))
        pp = np.zeros((bsz, heads, nq, nk))
        left, right = (-1, -1) if window is None else window
        if kind == "window_swapped":
            left, right = right, left
        for b in range(bsz):
            L = nk if kv_seqlens is None else min(max(int(kv_seqlens[b]), 0), nk)
            j = np.arange(nk)[None, :]
            i = np.arange(nq)[:, None] + (1 if kind == "window_shifted" else 0)
            ok = np.broadcast_to(j < L, (nq, nk)).copy()
            if causal:
                ok &= j <= np.arange(nq)[:, None]
            if left >= 0:
                ok &= (j > i - left) if kind == "window_left_strict" else (j >= i - left)
            if right >= 0 and kind != "window_right_ignored":
                ok &= j <= i + right
            for h in range(heads):
                s = np.where(ok, scale * (q[b, h] @ k[b, h].T), -np.inf)
                has = ok.any(axis=1)
                m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
                e = np.where(ok, np.exp(s - m[:, None]), 0.0)
                l = e.sum(axis=1)
                p = np.where(has[:, None], e / np.where(l > 0, l, 1.0)[:, None], 0.0)
                out = p @ v[b, h]
                with np.errstate(divide="ignore"):
                    lv = np.where(has, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
                o[b, h], lse[b, h], pp[b, h] = out, lv, p
        if return_p:
            return o, lse, pp
        return o, lse
    return impl


WINDOW_MUTANTS = ["window_left_strict", "window_right_ignored", "window_swapped", "window_shifted"]


@pytest.mark.parametrize("kind", WINDOW_MUTANTS)
def test_window_mutant_fails_some_pin(kind):
    impl = make_window_mutant(kind)
    failed = []
    for pin in WINDOW_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, FloatingPointError, ValueError, OverflowError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every window pin"


def test_unmutated_window_copy_passes_every_pin():
    impl = make_window_mutant("none")
    for pin in WINDOW_PINS:
        pin(impl)


# ---- planted mistakes in the backward pass, each of which must fail a backward pin
from oracle import attention_fwd  # noqa: E402
from oracle_pins import BWD_PINS  # noqa: E402


def _fwd(q, k, v, scale, causal=False, kv_seqlens=None, return_p=False, window=None):
    return attention_fwd(q, k, v, scale, causal=causal, kv_seqlens=kv_seqlens, return_p=return_p,
                         window=window)


def make_bwd_mutant(kind):
    def impl(q, k, v, do, scale, causal=False, kv_seqlens=None, window=None):
        bsz, heads, nq, _ = q.shape
        dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
        _, _, p_all = _fwd(q, k, v, scale, causal, kv_seqlens, return_p=True, window=window)
        for b in range(bsz):
            for h in range(heads):
                p = p_all[b, h]
                dv[b, h] = (p @ do[b, h][: p.shape[1]] if kind == "dv_not_transposed" and p.shape[0] == p.shape[1]
                            else p.T @ do[b, h])
                dp = do[b, h] @ v[b, h].T
                d_i = np.sum(p * dp, axis=1)
                ds = p * dp if kind == "no_row_term" else p * (dp - d_i[:, None])
                sq = 1.0 if kind == "dq_no_scale" else scale
                dq[b, h] = sq * (ds @ k[b, h])
                dk[b, h] = scale * (ds @ q[b, h] if kind == "dk_not_transposed" and ds.shape[0] == ds.shape[1]
                                    else ds.T @ q[b, h])
                if kind == "dk_sign":
                    dk[b, h] = -dk[b, h]
        return dq, dk, dv
    return impl


BWD_MUTANTS = ["dv_not_transposed", "no_row_term", "dq_no_scale", "dk_not_transposed", "dk_sign"]


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_backward_mutant_fails_some_pin(kind):
    impl = make_bwd_mutant(kind)
    failed = []
    for pin in BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl, _fwd)
        except (AssertionError, FloatingPointError, ValueError, OverflowError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every backward pin"


def test_unmutated_backward_copy_passes_every_pin():
    impl = make_bwd_mutant("none")
    for pin in BWD_PINS:
        pin(impl, _fwd)
