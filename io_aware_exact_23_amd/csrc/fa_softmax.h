// fa_softmax.h -- the online-softmax update of one K/V tile for one query row.
//
// The method keeps, per query row, a running maximum, a running normaliser and an output
// accumulator, and rescales the latter two whenever the maximum grows (page "FlashAttention 与
// 边缘设备上的注意力内存瓶颈", section "3.2 Online Softmax"; page "FlashAttention：把注意力从公式
// 写成数据流", section "分块与在线 softmax"). Here scores are kept in base-2 units: a raw dot
// product s becomes t = c*s with c = scale*log2(e), and p = 2^(t - m) on v_exp_f32.
//
// Lazy rescaling. The offset m used for p need not be the exact running maximum: any offset
// gives the same O = sum p v / sum p and lse = m + log2(sum p). The offset is raised only when a
// tile's maximum exceeds it by more than kTau (so p <= 2^kTau stays far from fp32 overflow),
// which skips the rescale of the output accumulator on almost every tile.
#pragma once

#include "fa_device.h"

namespace fa {

constexpr float kTau = 8.0f;

// Reductions over a lane's scores written as balanced trees (three-input max/min steps, pairwise
// sums), so a wave running them alone is not held up by one long chain of dependent instructions.
template <int N>
__device__ __forceinline__ float tree_max(const float (&x)[N]) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    constexpr int M = (N + 2) / 3;
    float y[M];
#pragma unroll
    for (int k = 0; k < M; ++k) {
      const int a = 3 * k;
      y[k] = a + 2 < N ? fmaxf(fmaxf(x[a], x[a + 1]), x[a + 2]) : (a + 1 < N ? fmaxf(x[a], x[a + 1]) : x[a]);
    }
    return tree_max<M>(y);
  }
}
template <int N>
__device__ __forceinline__ float tree_min(const float (&x)[N]) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    constexpr int M = (N + 2) / 3;
    float y[M];
#pragma unroll
    for (int k = 0; k < M; ++k) {
      const int a = 3 * k;
      y[k] = a + 2 < N ? fminf(fminf(x[a], x[a + 1]), x[a + 2]) : (a + 1 < N ? fminf(x[a], x[a + 1]) : x[a]);
    }
    return tree_min<M>(y);
  }
}
template <int N>
__device__ __forceinline__ float tree_sum(const float (&x)[N]) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    constexpr int M = (N + 1) / 2;
    float y[M];
#pragma unroll
    for (int k = 0; k < M; ++k) y[k] = 2 * k + 1 < N ? x[2 * k] + x[2 * k + 1] : x[2 * k];
    return tree_sum<M>(y);
  }
}

// One query row is shared by the lane pair (l, l ^ 32); each lane holds NV scores of it.
// On entry s[] holds raw dot products q.k; valid(i) tells whether score i's key is allowed
// (only consulted when kMask). On return s[] holds p (0 for masked keys), lsum includes
// them, and the return value is the factor by which the caller must multiply its output
// accumulator (1 when nothing changed); `rescaled` is wave-uniform.
template <int NV, bool kMask, typename ValidFn>
__device__ __forceinline__ float softmax_tile(float (&s)[NV], ValidFn valid,
                                              float c, bool neg, float& m_used, float& lsum,
                                              bool& rescaled) {
  // The row extreme of t = c*s is max(s)*c for c >= 0 and min(s)*c for c < 0; masked entries
  // get the sentinel that can never be the extreme.
  const float sentinel = neg ? kInf : -kInf;
  if constexpr (kMask) {
#pragma unroll
    for (int i = 0; i < NV; ++i) s[i] = valid(i) ? s[i] : sentinel;
  }
  float ext;
  if (!neg) ext = pair32_max(tree_max(s));
  else ext = pair32_min(tree_min(s));
  const float mt = (ext == sentinel) ? -kInf : ext * c;

  float alpha = 1.0f;
  rescaled = wave_any(mt > m_used + kTau);
  if (rescaled) {
    const float mn = fmaxf(m_used, mt);
    alpha = (mn == -kInf) ? 1.0f : fast_exp2(m_used - mn);
    m_used = mn;
    lsum *= alpha;
  }
  const float moff = (m_used == -kInf) ? 0.0f : m_used;
  // All exponent arguments first, then the exponentials: no exp waits on the product before it.
  float t[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) t[i] = fmaf(s[i], c, -moff);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float p = fast_exp2(t[i]);
    // Allowed scores are finite, so the sentinel marks exactly the masked keys (this also covers
    // c == 0, where the sentinel times c would give NaN).
    if constexpr (kMask) p = (s[i] == sentinel) ? 0.0f : p;
    s[i] = p;
  }
  lsum += tree_sum(s);
  return alpha;
}

// The same update with a lazier offset, for c > 0 (a caller with a negative scale negates its
// copy of Q and passes |c|). On a row's first tile with an allowed key the offset goes to the row
// maximum as above. After that the exponentials are taken against the offset as it stands, and
// the offset moves to the row maximum only when a lane's sum of its NV values of p exceeds
// kSumCap: with the offset held every p <= kSumCap, so nothing overflows, and most tiles need
// neither the row maximum nor its cross-lane exchange (one FMA, one exponential and one addition
// per score). In that rare case the raw scores, already overwritten, are produced again by
// recompute(s). Arguments and result as in softmax_tile.
constexpr float kSumCap = 4096.0f;
template <int NV, bool kMask, typename ValidFn, typename RecomputeFn>
__device__ __forceinline__ float softmax_tile_lazy(float (&s)[NV], ValidFn valid, float c,
                                                   float& m_used, float& lsum, bool& rescaled,
                                                   RecomputeFn recompute) {
  // Exponent arguments c*s - off in place; masked keys get -inf, so their p is exactly 0.
  auto args = [&](float off) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float t = fmaf(s[i], c, -off);
      if constexpr (kMask) s[i] = valid(i) ? t : -kInf;
      else s[i] = t;
    }
  };
  // Offset to the row maximum (and the factor for what was accumulated under the old offset),
  // given the arguments in s taken against moff; then p.
  auto to_row_max = [&](float moff) __attribute__((always_inline)) {
    const float mt = pair32_max(tree_max(s)) + moff;  // row maximum of c*s; -inf if all masked
    const float mn = fmaxf(m_used, mt);
    const float alpha = (m_used == -kInf) ? 1.0f : fast_exp2(m_used - mn);
    const float shift = ((mn == -kInf) ? 0.0f : mn) - moff;
#pragma unroll
    for (int i = 0; i < NV; ++i) s[i] = fast_exp2(s[i] - shift);
    lsum *= alpha;
    m_used = mn;
    return alpha;
  };
  float alpha = 1.0f;
  if (wave_any(m_used == -kInf)) {
    args(0.0f);
    alpha = to_row_max(0.0f);
    rescaled = true;
  } else {
    const float moff = m_used;
    args(moff);
#pragma unroll
    for (int i = 0; i < NV; ++i) s[i] = fast_exp2(s[i]);
    rescaled = wave_any(tree_sum(s) > kSumCap);
    if (rescaled) {
      recompute(s);
      args(moff);
      alpha = to_row_max(moff);
    }
  }
  lsum += tree_sum(s);
  return alpha;
}

}  // namespace fa
