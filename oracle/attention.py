"""fp64 CPU oracle for exact softmax attention, forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` use it. It shares no code with the HIP library.

What it computes
----------------
Citations name the page by its title and then the section:
  [card]     page "FlashAttention 与边缘设备上的注意力内存瓶颈" (a reading card)
  [dataflow] page "FlashAttention：把注意力从公式写成数据流" (an engineering essay)

The pages say the method reaches exactly the result of standard attention, only in another
order of execution ([card] section "3.2 Online Softmax"; [dataflow] section "分块与在线
softmax"). So this oracle is the plain definition, computed the naive way the pages describe
standard attention ([card] section "2 标准 attention 的问题"; [dataflow] opening paragraph):
scores S = QK^T, a softmax, then a product with V, with the full score matrix S and the
probability matrix P materialised for one (batch, head) at a time.

For batch b, head h and query row i:

* allowed keys   A_i = { j : j < L_b  and  (not causal  or  j <= i)
                         and (left < 0 or j >= i - left)  and  (right < 0 or j <= i + right) }
                 (L_b = kv_seqlens[b] clamped to [0, Nk], or Nk when no lengths are given;
                 (left, right) is an optional sliding window around key position i, -1 on a
                 side meaning no limit there; invalid positions must not enter the
                 normalisation, and sliding windows are one of the mask kinds named next to
                 causal masks and variable-length batches: [dataflow] section
                 "精度、掩码和边界情况")
* scores         S_ij = scale * sum_k q_ik k_jk            for j in A_i
* softmax        m_i = max_{j in A_i} S_ij,  e_ij = exp(S_ij - m_i),  l_i = sum_j e_ij,
                 P_ij = e_ij / l_i  (P_ij = 0 for j not in A_i)
* output         O_i = sum_j P_ij v_j
* logsumexp      lse_i = m_i + ln(l_i)   (natural log)
* empty row      A_i empty  ->  O_i = 0,  lse_i = -inf

Readings taken where the pages are silent: the scale is an argument (the workloads use
1/sqrt(d)); lse is the natural-log logsumexp of the scaled, masked scores; causal masking is
defined only for Nq == Nk; padded query rows are computed like any other row; a window places
query i at key position i (the same alignment as the causal mask), for any Nq and Nk. The max shift
m_i changes nothing in exact arithmetic; it keeps exp finite for large scores.

Every quantity is fp64. Inputs arrive as fp64 arrays that hold bf16 or fp32 values exactly
(``bf16_bits_to_f64`` converts raw bf16 bit patterns without rounding).

Backward pass (``attention_bwd``). Training needs the gradients of this forward pass, and a tiled
implementation gets them by recomputing S and P from Q, K and the saved logsumexp rather than
storing P ([dataflow] section "用实验验证而不是背诵结论" on training needing recomputation;
[vocus] page "[2205.14135] FlashAttention ...", section "三、FLOPs（計算能力）並非 Speedup 的主因素"
on the extra recomputation FLOPs). The pages give no formulas, so the oracle is the plain chain
rule of the definition above, for an upstream gradient dO, materialising P:
  dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij  (= dO_i . O_i),
  dS_ij = P_ij (dP_ij - D_i),   dQ = scale * dS K,   dK = scale * dS^T Q;
masked pairs have P_ij = 0 and so contribute nothing; rows with no allowed key get dQ_i = 0.

Key slots at or past L_b are outside every allowed set; the oracle slices them off before any
product (forward and backward), so whatever they hold -- NaN and Inf included -- cannot reach a
result, and their key and value gradients are zero. Invalid positions must stay out of the
computation altogether ([dataflow] section "精度、掩码和边界情况").
"""

from __future__ import annotations

import numpy as np

__all__ = ["bf16_bits_to_f64", "allowed_mask", "attention_fwd", "attention_rows", "attention_bwd"]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact conversion of bf16 bit patterns (uint16 / int16 arrays) to float64.

    A bf16 value is the upper half of an IEEE binary32 value, so shifting the 16 bits into
    the high half of a 32-bit word gives that binary32 exactly; binary32 -> binary64 is exact.
    """
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _length(kv_seqlens, b: int, nk: int) -> int:
    if kv_seqlens is None:
        return nk
    return int(min(max(int(kv_seqlens[b]), 0), nk))


def allowed_mask(rows: np.ndarray, nk: int, length: int, causal: bool, window=None) -> np.ndarray:
    """Boolean matrix M[r, j] = (key j is in A_{rows[r]})."""
    j = np.arange(nk)[None, :]
    i = np.asarray(rows)[:, None]
    ok = j < length
    if causal:
        ok = ok & (j <= i)
    if window is not None:
        left, right = int(window[0]), int(window[1])
        if left >= 0:
            ok = ok & (j >= i - left)
        if right >= 0:
            ok = ok & (j <= i + right)
    return np.broadcast_to(ok, (len(rows), nk)).copy()


def attention_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                   scale: float, causal: bool, length: int, return_p: bool = False, window=None):
    """The definition for one (batch, head) and a set of query rows.

    q_rows: (R, d) fp64, the query vectors of the rows listed in ``rows`` (their indices i).
    k, v:   (Nk, d) fp64; only rows below ``length`` are read.
    Returns O (R, d), lse (R,) and, when asked, P (R, Nk) (zero at and past ``length``).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    nk = np.shape(k)[0]
    # Key slots at or past the length are outside every allowed set and are never read: they
    # may hold anything (NaN, Inf), so they are cut off before any arithmetic touches them.
    length = int(min(max(int(length), 0), nk))
    k = np.asarray(k, dtype=np.float64)[:length]
    v = np.asarray(v, dtype=np.float64)[:length]
    ok = allowed_mask(rows, length, length, causal, window)

    # S = scale * Q K^T, with masked entries at -inf (they never enter the normalisation).
    s = np.full((len(rows), length), -np.inf)
    dots = q_rows @ k.T
    s[ok] = float(scale) * dots[ok]

    # Row-wise softmax over the allowed set, shifted by the row maximum.
    has_key = ok.any(axis=1)
    m = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(ok, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[has_key] = e[has_key] / l[has_key, None]

    o = p @ v
    lse = np.full(len(rows), -np.inf)
    lse[has_key] = m[has_key] + np.log(l[has_key])
    o[~has_key] = 0.0
    if return_p:
        p_full = np.zeros((len(rows), nk))
        p_full[:, :length] = p
        return o, lse, p_full
    return o, lse


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                  causal: bool = False, kv_seqlens=None, rows=None, return_p: bool = False,
                  window=None):
    """Exact attention for a whole batch.

    q: (B, H, Nq, d); k, v: (B, H, Nk, d); all fp64 (or anything numpy turns into fp64 exactly).
    kv_seqlens: None or a length-B integer sequence (valid key count per sequence).
    rows: None for every query row, else a 1-D array of query indices evaluated for every
          (b, h) -- each row of the definition depends only on its own query vector.
    window: None, or (left, right) with -1 for an unlimited side (see A_i above).
    Returns O (B, H, R, d) and lse (B, H, R) with R = Nq or len(rows); also P (B, H, R, Nk)
    when ``return_p``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, heads, nq, d = q.shape
    nk = k.shape[2]
    if causal and nq != nk:
        raise ValueError("causal masking is defined here only for Nq == Nk")
    idx = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((bsz, heads, len(idx), v.shape[3]))
    lse = np.zeros((bsz, heads, len(idx)))
    p_all = np.zeros((bsz, heads, len(idx), nk)) if return_p else None
    for b in range(bsz):
        length = _length(kv_seqlens, b, nk)
        for h in range(heads):
            res = attention_rows(q[b, h, idx], k[b, h], v[b, h], idx, scale, causal, length,
                                 return_p=return_p, window=window)
            o[b, h], lse[b, h] = res[0], res[1]
            if return_p:
                p_all[b, h] = res[2]
    if return_p:
        return o, lse, p_all
    return o, lse


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                  causal: bool = False, kv_seqlens=None, window=None):
    """Gradients (dQ, dK, dV) of O = attention(Q, K, V) for the upstream gradient dO.

    Shapes as in attention_fwd; do has O's shape (B, H, Nq, d_v). All fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    bsz, heads, nq, _ = q.shape
    nk = k.shape[2]
    if causal and nq != nk:
        raise ValueError("causal masking is defined here only for Nq == Nk")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(nq)
    for b in range(bsz):
        length = _length(kv_seqlens, b, nk)
        for h in range(heads):
            # Only the key slots below the length enter any product; the gradients of the
            # slots past it stay zero.
            kb, vb = k[b, h, :length], v[b, h, :length]
            _, _, p = attention_rows(q[b, h], kb, vb, rows, scale, causal, length,
                                     return_p=True, window=window)
            dv[b, h, :length] = p.T @ do[b, h]
            dp = do[b, h] @ vb.T
            d_i = np.sum(p * dp, axis=1)
            ds = p * (dp - d_i[:, None])
            dq[b, h] = float(scale) * (ds @ kb)
            dk[b, h, :length] = float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv
