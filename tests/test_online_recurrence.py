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
