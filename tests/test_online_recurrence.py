"""The exactness claim of tiling with online softmax, checked in fp64 on the CPU.

The pages state that processing K/V tile by tile while keeping a running maximum, a running
normaliser and a rescaled output accumulator gives exactly the standard-attention result, only
in another order (page 'FlashAttention 与边缘设备上的注意力内存瓶颈', section '3.2 Online
Softmax'; page 'FlashAttention：把注意力从公式写成数据流', section '分块与在线 softmax').
This test-only recurrence, with random tile sizes, must equal the oracle to fp64 rounding.
It pins the recurrence the GPU kernels implement without sharing any code with them.
"""

import numpy as np
import pytest

from oracle import attention_fwd


def online_softmax_attention(q, k, v, scale, causal, lens, rng):
    bsz, heads, nq, d = q.shape
    nk = k.shape[2]
    o = np.zeros((bsz, heads, nq, v.shape[3]))
    lse = np.zeros((bsz, heads, nq))
    for b in range(bsz):
        L = nk if lens is None else lens[b]
        for h in range(heads):
            q0 = 0
            while q0 < nq:
                bm = int(rng.integers(1, 9))
                rows = np.arange(q0, min(q0 + bm, nq))
                m = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), v.shape[3]))
                k0 = 0
                while k0 < nk:
                    bn = int(rng.integers(1, 9))
                    cols = np.arange(k0, min(k0 + bn, nk))
                    ok = (cols[None, :] < L) & (~causal | (cols[None, :] <= rows[:, None]))
                    s = np.where(ok, scale * (q[b, h, rows] @ k[b, h, cols].T), -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    live = np.isfinite(m_new)
                    alpha = np.where(live, np.exp(np.where(live, m - np.where(live, m_new, 0), 0)), 1.0)
                    p = np.where(ok & live[:, None], np.exp(s - np.where(live, m_new, 0)[:, None]), 0.0)
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, cols]
                    m = m_new
                    k0 += bn
                live = l > 0
                o[b, h, rows] = np.where(live[:, None], acc / np.where(live, l, 1)[:, None], 0.0)
                lse[b, h, rows] = np.where(live, m + np.log(np.where(live, l, 1)), -np.inf)
                q0 += bm
    return o, lse


@pytest.mark.parametrize("causal,lens,seed", [(False, None, 1), (True, None, 2),
                                              (False, [19, 0, 3], 3), (True, [25, 10, 1], 4)])
def test_online_equals_definition(causal, lens, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((3, 2, 25, 6))
    k = rng.standard_normal((3, 2, 25, 6))
    v = rng.standard_normal((3, 2, 25, 5))
    o, lse = online_softmax_attention(q, k, v, 0.45, causal, lens, rng)
    o_ref, lse_ref = attention_fwd(q, k, v, 0.45, causal, lens)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - lse_ref[fin])) <= 1e-12


def lazy_offset_attention(q, k, v, scale, causal, lens, rng, cap):
    """The recurrence with a lazy exponent offset, in base-2 units t = log2(e) * scale * q.k: p is
    taken against an offset m that moves to the row maximum only on the row's first tile with an
    allowed key or when the tile's sum of p exceeds `cap`; O and l carry the factor 2^-m, so any
    offset gives the same result. This is the update the bf16 kernels run, written independently."""
    c = scale / np.log(2.0)
    bsz, heads, nq, d = q.shape
    nk = k.shape[2]
    o = np.zeros((bsz, heads, nq, v.shape[3]))
    lse = np.zeros((bsz, heads, nq))
    for b in range(bsz):
        L = nk if lens is None else lens[b]
        for h in range(heads):
            for i in range(nq):
                m, l, acc = -np.inf, 0.0, np.zeros(v.shape[3])
                k0 = 0
                while k0 < nk:
                    cols = np.arange(k0, min(k0 + int(rng.integers(1, 9)), nk))
                    ok = (cols < L) & (~causal | (cols <= i))
                    t = np.where(ok, c * (k[b, h, cols] @ q[b, h, i]), -np.inf)
                    off = 0.0 if m == -np.inf else m
                    p = np.exp2(t - off)
                    if (m == -np.inf and ok.any()) or p.sum() > cap:
                        m_new = max(m, t.max())
                        alpha = 1.0 if m == -np.inf else np.exp2(m - m_new)
                        l, acc, m = alpha * l, alpha * acc, m_new
                        p = np.exp2(t - m)
                    l += p.sum()
                    acc += p @ v[b, h, cols]
                    k0 = cols[-1] + 1
                o[b, h, i] = acc / l if l > 0 else 0.0
                lse[b, h, i] = (m + np.log2(l)) * np.log(2.0) if l > 0 else -np.inf
    return o, lse


@pytest.mark.parametrize("cap", [1.5, 4.0, 4096.0])
@pytest.mark.parametrize("causal,lens,seed", [(False, None, 11), (True, None, 12), (True, [30, 7, 0], 13)])
def test_lazy_offset_equals_definition(cap, causal, lens, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((3, 1, 30, 5))
    k = rng.standard_normal((3, 1, 30, 5))
    # Scores that rise along the keys make the sum pass the cap and the offset move often.
    k += np.linspace(0.0, 6.0, 30)[None, None, :, None] * np.sign(q.mean(axis=2, keepdims=True))
    v = rng.standard_normal((3, 1, 30, 4))
    o, lse = lazy_offset_attention(q, k, v, 0.7, causal, lens, rng, cap)
    o_ref, lse_ref = attention_fwd(q, k, v, 0.7, causal, lens)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - lse_ref[fin])) <= 1e-12
