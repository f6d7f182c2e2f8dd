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
                # Only the slots below the length are read, unless the mutant multiplies its zero
                # weights through the padding.
                kk = k[b, h] if kind == "padding_multiplied" else k[b, h, :L]
                vv = v[b, h] if kind == "padding_multiplied" else v[b, h, :L]
                ok = ok[:, : kk.shape[0]]
                sc = 1.0 if kind == "no_scale" else scale
                with np.errstate(invalid="ignore", over="ignore"):
                    s = np.where(ok, sc * (q[b, h] @ kk.T), -np.inf)
                has = ok.any(axis=1)
                m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
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
                if kind == "transposed_pv" and nq == vv.shape[0]:
                    out = p.T @ vv
                else:
                    with np.errstate(invalid="ignore", over="ignore"):
                        out = p @ vv
                out[~has] = 0.0
                with np.errstate(divide="ignore"):
                    lv = np.log(l) if kind == "lse_no_max" else m + np.log(l)
                lv = np.where(has, lv, -np.inf)
                o[b, h], lse[b, h] = out, lv
                pp[b, h, :, : p.shape[1]] = p
        if return_p:
            return o, lse, pp
        return o, lse
    return impl


MUTANTS = ["no_scale", "causal_strict", "padding_ignored", "padding_off_by_one", "no_shift",
           "shift_sign", "softmax_wrong_axis", "no_normalise", "lse_no_max", "transposed_pv",
           "padding_multiplied"]


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
        nk = k.shape[2]
        for b in range(bsz):
            L = nk if kv_seqlens is None else min(max(int(kv_seqlens[b]), 0), nk)
            if kind == "padding_multiplied":
                L = nk  # zero weights multiplied through the padded slots
            for h in range(heads):
                p = p_all[b, h, :, :L]
                kk, vv = k[b, h, :L], v[b, h, :L]
                dv[b, h, :L] = (p @ do[b, h][: p.shape[1]] if kind == "dv_not_transposed" and p.shape[0] == p.shape[1]
                                else p.T @ do[b, h])
                with np.errstate(invalid="ignore", over="ignore"):
                    dp = do[b, h] @ vv.T
                    d_i = np.sum(p * dp, axis=1)
                    ds = p * dp if kind == "no_row_term" else p * (dp - d_i[:, None])
                    sq = 1.0 if kind == "dq_no_scale" else scale
                    dq[b, h] = sq * (ds @ kk)
                    dk[b, h, :L] = scale * (ds @ q[b, h] if kind == "dk_not_transposed" and ds.shape[0] == ds.shape[1]
                                            else ds.T @ q[b, h])
                if kind == "dk_sign":
                    dk[b, h] = -dk[b, h]
        return dq, dk, dv
    return impl


BWD_MUTANTS = ["dv_not_transposed", "no_row_term", "dq_no_scale", "dk_not_transposed", "dk_sign",
               "padding_multiplied"]


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


# ---- FP8 (e4m3) oracle: planted mistakes in the format, the quantiser, the attention of the
# quantised tensors and the rounding bound.

from oracle import fp8 as _fp8  # noqa: E402
from oracle_pins import FP8_PINS  # noqa: E402


def _round_variant(x, bias=7, mode="even", sub_limit=2.0 ** -6, overflow="saturate"):
    """A copy of the e4m3 rounding with switches for the planted mistakes."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    code = np.zeros(x.shape, dtype=np.int64)

    def rnd(v):
        if mode == "even":
            return np.rint(v)
        if mode == "half_up":
            return np.floor(v + 0.5)
        return np.floor(v)  # truncation

    sub = a < sub_limit
    code[sub] = rnd(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub & np.isfinite(a)
    f, e2 = np.frexp(a[nrm])
    e = e2 - 1
    m = rnd((2.0 * f - 1.0) * 8.0).astype(np.int64)
    e = np.where(m == 8, e + 1, e)
    m = np.where(m == 8, 0, m)
    big = (e > 15 - bias) | ((e == 15 - bias) & (m == 7))
    c = np.clip(e + bias, 0, 15) << 3 | m
    code[nrm] = np.where(big, 0x7F if overflow == "nan" else 0x7E, c)
    code[np.isinf(a)] = 0x7E
    code |= np.where(np.signbit(x), 0x80, 0)
    code[np.isnan(x)] = 0x7F
    return code.astype(np.uint8)


def _decode_bias8(codes):
    c = np.asarray(codes).astype(np.int64)
    v = _fp8.e4m3_decode(codes)
    normal = ((c >> 3) & 0xF) != 0
    return np.where(normal, v / 2.0, v)


def _quantize_variant(kind):
    def q(x, kv_seqlens=None, transpose=False):
        x = np.asarray(x, dtype=np.float64)
        bsz, heads, n, d = x.shape
        codes = np.zeros((bsz, heads, n, d), dtype=np.uint8)
        s_all = np.ones((bsz, heads), dtype=np.float32)
        for b in range(bsz):
            L = n if kv_seqlens is None else min(max(int(kv_seqlens[b]), 0), n)
            Lq = n if kind in ("amax_all_rows", "padding_kept") else L
            for h in range(heads):
                rows = x[b, h, :Lq].astype(np.float32)
                amax = np.float32(np.max(np.abs(x[b, h, :Lq if kind == "amax_all_rows" else L])))
                top = np.float32(240.0 if kind == "scale_240" else 448.0)
                s = np.float32(1.0) if amax == 0 else np.float32(amax / top)
                s_all[b, h] = s
                codes[b, h, :Lq] = _fp8.e4m3_round((rows / s).astype(np.float32).astype(np.float64))
        if not transpose:
            return codes, s_all
        cols = n if kind == "transpose_no_pad" else _fp8.vt_cols(n)
        out = np.zeros((bsz, heads, d, cols), dtype=np.uint8)
        out[:, :, :, :n] = np.swapaxes(codes, 2, 3) if kind != "transpose_swapped_dims" else \
            np.swapaxes(codes, 2, 3)[:, :, ::-1]
        return out, s_all
    return q


def _attention_variant(kind):
    def att(q8, k8, v8t, dq, dk, dv, scale, causal=False, kv_seqlens=None, rows=None, return_p=False):
        nk = np.asarray(k8).shape[2]
        q = _fp8.dequantize_e4m3(q8, dq)
        k = _fp8.dequantize_e4m3(k8, dk if kind != "k_uses_q_scale" else dq)
        v = _fp8.dequantize_e4m3(v8t, np.ones_like(dv) if kind == "no_dv" else dv, transposed=True, n=nk)
        if kind == "v_not_transposed":
            v = _fp8.dequantize_e4m3(np.asarray(v8t)[:, :, :nk, :], dv)
        from oracle import attention_fwd
        return attention_fwd(q, k, v, scale, causal=causal, kv_seqlens=kv_seqlens, rows=rows,
                             return_p=return_p)
    return att


def _bound_variant(kind):
    def bound(p):
        p = np.asarray(p, dtype=np.float64)
        inv_l = p.max(axis=-1, keepdims=True)
        rel = 2.0 ** -5 if kind == "bound_half" else 2.0 ** -4
        sub = 0.0 if kind == "bound_no_subnormal" else 2.0 ** -13
        b = np.where(p > 0, rel * p + sub * inv_l, 0.0)
        return 4.0 * b if kind == "bound_4x" else b
    return bound


def make_fp8_mutant(kind):
    import types
    ns = types.SimpleNamespace(decode=_fp8.e4m3_decode, round=_fp8.e4m3_round,
                               quantize=_fp8.quantize_e4m3, attention=_fp8.attention_fwd_fp8,
                               bound=_fp8.p_rounding_bound)
    if kind == "decode_bias8":
        ns.decode = _decode_bias8
    elif kind == "round_bias8":
        ns.round = lambda x: _round_variant(x, bias=8)
    elif kind in ("round_half_up", "round_truncate"):
        ns.round = lambda x: _round_variant(x, mode=kind[6:])
    elif kind == "round_subnormal_limit":
        ns.round = lambda x: _round_variant(x, sub_limit=2.0 ** -7)
    elif kind == "round_nan_on_overflow":
        ns.round = lambda x: _round_variant(x, overflow="nan")
    elif kind == "round_copy_ok":
        ns.round = lambda x: _round_variant(x)
    elif kind in ("scale_240", "amax_all_rows", "padding_kept", "transpose_no_pad",
                  "transpose_swapped_dims", "quantize_copy_ok"):
        ns.quantize = _quantize_variant(kind)
    elif kind in ("no_dv", "k_uses_q_scale", "v_not_transposed", "attention_copy_ok"):
        ns.attention = _attention_variant(kind)
    elif kind in ("bound_half", "bound_no_subnormal", "bound_4x", "bound_copy_ok"):
        ns.bound = _bound_variant(kind)
    return ns


FP8_MUTANTS = ["decode_bias8", "round_bias8", "round_half_up", "round_truncate",
               "round_subnormal_limit", "round_nan_on_overflow", "scale_240", "amax_all_rows",
               "padding_kept", "transpose_no_pad", "transpose_swapped_dims", "no_dv",
               "k_uses_q_scale", "v_not_transposed", "bound_half", "bound_no_subnormal", "bound_4x"]


@pytest.mark.parametrize("kind", FP8_MUTANTS)
def test_fp8_mutant_fails_some_pin(kind):
    ns = make_fp8_mutant(kind)
    failed = []
    for pin in FP8_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ns)
        except (AssertionError, FloatingPointError, ValueError, OverflowError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every fp8 pin"


@pytest.mark.parametrize("kind", ["round_copy_ok", "quantize_copy_ok", "attention_copy_ok", "bound_copy_ok"])
def test_unmutated_fp8_copies_pass_every_pin(kind):
    ns = make_fp8_mutant(kind)
    for pin in FP8_PINS:
        pin(ns)
