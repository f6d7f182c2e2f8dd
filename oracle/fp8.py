"""fp64 CPU oracle for the FP8 (e4m3) forward path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this module:
only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` use it. It shares no code with the HIP library.

What the pages say
------------------
[dataflow] = page "FlashAttention：把注意力从公式写成数据流".

Lower precision cuts the bytes moved and raises the peak rate, but changes how stable the
softmax is numerically ([dataflow] section "精度、掩码和边界情况"). FP8 in particular saves HBM
bytes but may need transposes, scaling and error compensation, its conversions can eat the
bandwidth it saves, and its error has to be reported next to its speed ([dataflow] section
"用实验验证而不是背诵结论"). FA3 combines low-precision matrix units with overlapped data
movement ([dataflow] section "FA2 与 FA3"). The pages fix neither a format nor a scaling rule,
so this module takes the plainest reading:

* format: OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities; S.1111.111 is NaN, the largest finite magnitude is 448 = 1.75 * 2^8, the smallest
  normal 2^-6 and the smallest subnormal 2^-9). Rounding to nearest, ties to the even mantissa;
  magnitudes that would round past 448 saturate to 448 (the quantiser below never produces
  such a value);
* scaling: one scale per (batch, head) slice, s = amax / 448 in fp32, where amax is the largest
  magnitude over the slice's valid rows (rows at or past the sequence's key length L_b are
  excluded and stored as zero), and s = 1 for an all-zero slice. The stored code is
  e4m3(x / s) with x / s rounded to fp32 first (a correctly rounded fp32 division), so that the
  integer decision is taken in the precision of the GPU quantiser. Dequantised value: s * e4m3;
* transposition: V may be stored transposed, as V^T with layout [d][cols] per (batch, head),
  cols = Nk rounded up to a multiple of 64, the padding columns zero;
* attention of the quantised tensors: exact attention (``attention_fwd``) of the dequantised
  Q, K and V, in fp64.

One step of the GPU path lies outside this definition: it rounds the probabilities to e4m3
(scaled by 8 first) before the P V product, while its normaliser l sums the unrounded values.
That rounding moves a normalised weight P_ij by at most
    2^-4 P_ij + 2^-13 / l_i,      l_i = sum_j exp(S_ij - max_j S_ij):
a normal e4m3 value is off by at most half a unit, 2^-4 of its size; a subnormal one by at most
2^-10 absolute, which the scaled normaliser 8 * l (at least 8 * l_i, since the GPU path's
exponent offset never exceeds the row maximum) turns into 2^-13 / l_i. ``p_rounding_bound``
returns this per-pair bound; the parity tests build their tolerance from it.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_fwd

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_round", "quantize_e4m3", "dequantize_e4m3",
           "vt_cols", "attention_fwd_fp8", "p_rounding_bound"]

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUB_STEP = 2.0 ** -9


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as fp64; NaN for the two NaN codes."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = (c & 7).astype(np.float64)
    mag = np.where(ef == 0, mf * _SUB_STEP, np.ldexp(1.0 + mf / 8.0, (ef - 7).astype(np.int64)))
    out = sign * mag
    out[(c & 0x7F) == 0x7F] = np.nan
    return out


def e4m3_round(x) -> np.ndarray:
    """E4M3 code (uint8) nearest to each value, ties to even; saturating at 448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    code = np.zeros(x.shape, dtype=np.int64)
    sub = a < _MIN_NORMAL
    # Subnormal range: multiples of 2^-9 (rint rounds half to even); 8 * 2^-9 is the code of 2^-6.
    code[sub] = np.rint(a[sub] / _SUB_STEP).astype(np.int64)
    nrm = ~sub & np.isfinite(a)
    if np.any(nrm):
        f, e2 = np.frexp(a[nrm])          # a = f * 2^e2, f in [0.5, 1)
        e = e2 - 1                        # a = (2f) * 2^e, 2f in [1, 2)
        m = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)  # exact scaling, then half to even
        carry = m == 8
        e = np.where(carry, e + 1, e)
        m = np.where(carry, 0, m)
        big = (e > 8) | ((e == 8) & (m == 7))
        c = ((e + 7) << 3) | m
        c = np.where(big, 0x7E, c)
        code[nrm] = c
    code[np.isinf(a)] = 0x7E
    code = code | np.where(np.signbit(x), 0x80, 0)
    code[np.isnan(x)] = 0x7F
    return code.astype(np.uint8)


def vt_cols(nk: int) -> int:
    """Columns of a transposed e4m3 V: Nk rounded up to a multiple of 64."""
    return (int(nk) + 63) // 64 * 64


def _length(kv_seqlens, b: int, n: int) -> int:
    if kv_seqlens is None:
        return n
    return int(min(max(int(kv_seqlens[b]), 0), n))


def quantize_e4m3(x, kv_seqlens=None, transpose: bool = False):
    """Per-(batch, head) E4M3 quantisation of x (B, H, N, d), values exactly representable in fp32.

    Returns (codes, descale): codes uint8 of shape (B, H, N, d), or (B, H, d, vt_cols(N)) when
    ``transpose``; descale float32 (B, H), the scale s of each slice.
    """
    x = np.asarray(x, dtype=np.float64)
    bsz, heads, n, d = x.shape
    codes = np.zeros((bsz, heads, n, d), dtype=np.uint8)
    descale = np.ones((bsz, heads), dtype=np.float32)
    for b in range(bsz):
        length = _length(kv_seqlens, b, n)
        for h in range(heads):
            rows = x[b, h, :length].astype(np.float32)
            amax = np.float32(np.max(np.abs(rows))) if length > 0 else np.float32(0.0)
            s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))
            descale[b, h] = s
            y = (rows / s).astype(np.float32)  # fp32 division, correctly rounded
            codes[b, h, :length] = e4m3_round(y.astype(np.float64))
    if not transpose:
        return codes, descale
    out = np.zeros((bsz, heads, d, vt_cols(n)), dtype=np.uint8)
    out[:, :, :, :n] = np.swapaxes(codes, 2, 3)
    return out, descale


def dequantize_e4m3(codes, descale, transposed: bool = False, n: int | None = None) -> np.ndarray:
    """fp64 values s * e4m3(code) in the (B, H, N, d) layout (``n`` keys when ``transposed``)."""
    v = e4m3_decode(codes) * np.asarray(descale, dtype=np.float64)[:, :, None, None]
    if transposed:
        v = np.swapaxes(v, 2, 3)[:, :, : int(n)]
    return v


def attention_fwd_fp8(q8, k8, v8t, dq, dk, dv, scale: float, causal: bool = False,
                      kv_seqlens=None, rows=None, return_p: bool = False):
    """Exact attention (fp64) of the dequantised e4m3 tensors.

    q8 (B, H, Nq, d) and k8 (B, H, Nk, d) codes; v8t (B, H, d, vt_cols(Nk)) codes of V^T;
    dq, dk, dv (B, H) scales. Returns what attention_fwd returns for those values.
    """
    nk = np.asarray(k8).shape[2]
    q = dequantize_e4m3(q8, dq)
    k = dequantize_e4m3(k8, dk)
    v = dequantize_e4m3(v8t, dv, transposed=True, n=nk)
    return attention_fwd(q, k, v, scale, causal=causal, kv_seqlens=kv_seqlens, rows=rows,
                         return_p=return_p)


def p_rounding_bound(p) -> np.ndarray:
    """Per-pair bound on |weight error| from rounding the probabilities to e4m3 (see above).

    p: (..., R, Nk) exact probabilities; 0 on masked pairs. Since P_ij = exp(S_ij - M_i) / l_i,
    the row's largest weight is 1 / l_i. Masked pairs and empty rows get 0.
    """
    p = np.asarray(p, dtype=np.float64)
    pmax = p.max(axis=-1, keepdims=True)
    inv_l = np.where(pmax > 0, pmax, 0.0)  # 1 / l_i
    return np.where(p > 0, 2.0 ** -4 * p + 2.0 ** -13 * inv_l, 0.0)
