// fa_prefill_f32.hip -- tiled attention forward for fp32 Q/K/V on gfx950 (MI355X).
//
// Same decomposition as the bf16 kernel (one workgroup of 4 waves per 128 query rows of one
// (b, h); K/V tiles streamed through LDS; online softmax in registers; page "FlashAttention：把
// 注意力从公式写成数据流", section "分块与在线 softmax"), on the fp32 matrix instruction
// v_mfma_f32_32x32x2_f32. Each wave again computes S^T = K Q^T so that a lane holds 16 scores of
// one query, and accumulates O^T += V^T P^T. Operands of this instruction are single elements,
// so K and V stay in their natural [key][d] layout in LDS and no key permutation is needed.
// One LDS stage (fetch, barrier, store, barrier, compute): this path serves fp32 inputs, whose
// workloads are small.
#include "fa_device.h"
#include "fa_params.h"
#include "fa_softmax.h"

namespace fa {

template <int D>
struct PrefillF32Cfg {
  static constexpr int kThreads = 256;
  static constexpr int kBM = 128;             // 4 waves x 32 query rows
  static constexpr int kBN = 32;              // keys per K/V tile
  static constexpr int kKStride = D + 1;      // floats per K row in LDS (breaks bank aliasing)
  static constexpr int kVStride = D + 4;
  static constexpr int kLdsBytes = (kBN * kKStride + kBN * kVStride) * 4;
  static constexpr int kChunks = kBN * D / 4 / kThreads;  // 16-byte pieces per thread, K and V each
  static_assert(kChunks * kThreads * 4 == kBN * D, "tile must split evenly");
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void prefill_f32_kernel(PrefillParams p) {
  using C = PrefillF32Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) float smemf[];
  float* Ks = smemf;
  float* Vs = smemf + C::kBN * C::kKStride;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, p.n_tiles);
  const int bh = tile / p.n_qtiles;
  int qt = tile - bh * p.n_qtiles;
  if (p.causal) qt = p.n_qtiles - 1 - qt;
  const int b = bh / p.H;
  const int q0 = qt * C::kBM;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  int kend = L;
  if (p.causal) kend = min(kend, min(q0 + C::kBM, p.Nq));
  const int ntiles = kend > 0 ? (kend + C::kBN - 1) / C::kBN : 0;

  const float* Qg = static_cast<const float*>(p.q) + (size_t)bh * p.Nq * D;
  const float* Kg = static_cast<const float*>(p.k) + (size_t)bh * p.Nk * D;
  const float* Vg = static_cast<const float*>(p.v) + (size_t)bh * p.Nk * D;

  const int qw0 = q0 + w * 32;
  const int qi = qw0 + r32;
  const int qw_last = min(qw0 + 32, p.Nq) - 1;
  const float c = p.c;
  const bool neg = c < 0.0f;

  // Q row qi, elements 2*ks + g: the B operand of S^T = K Q^T.
  float qreg[D / 2];
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks) qreg[ks] = qi < p.Nq ? Qg[(size_t)qi * D + 2 * ks + g] : 0.0f;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
  float m_used = -kInf, lsum = 0.0f;

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * C::kBN;
    f32x4 kx[C::kChunks], vx[C::kChunks];
#pragma unroll
    for (int it = 0; it < C::kChunks; ++it) {
      const int idx = tid + it * C::kThreads;
      const int row = idx / (D / 4);
      const int ch = idx % (D / 4);
      const int key = k0 + row;
      f32x4 zk = {0.f, 0.f, 0.f, 0.f}, zv = {0.f, 0.f, 0.f, 0.f};
      if (key < L) {
        zk = *reinterpret_cast<const f32x4*>(Kg + (size_t)key * D + ch * 4);
        zv = *reinterpret_cast<const f32x4*>(Vg + (size_t)key * D + ch * 4);
      }
      kx[it] = zk;
      vx[it] = zv;
    }
    __syncthreads();  // everyone is done reading the previous tile
#pragma unroll
    for (int it = 0; it < C::kChunks; ++it) {
      const int idx = tid + it * C::kThreads;
      const int row = idx / (D / 4);
      const int ch = idx % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[row * C::kKStride + ch * 4 + e] = kx[it][e];
      *reinterpret_cast<f32x4*>(Vs + row * C::kVStride + ch * 4) = vx[it];
    }
    __syncthreads();

    const bool active = (qw_last >= qw0) && (!p.causal || k0 <= qw_last);
    if (!active) continue;

    // S^T[key][query], keys k0 .. k0+31: accumulator entry i of lane (r32, g) is key
    // k0 + 8*(i/4) + 4*g + i%4 and query qi.
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[r32 * C::kKStride + 2 * ks + g], qreg[ks], sacc, 0, 0, 0);

    const bool need_mask = (k0 + C::kBN > L) || (p.causal && k0 + C::kBN - 1 > qw0);
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = sacc[i];
    // Score i belongs to key k0 + 4*g + 8*(i/4) + i%4; rem counts this lane's allowed keys from
    // k0 + 4*g on (keys < L, and keys <= qi when causal).
    const int rem = (p.causal ? min(L, qi + 1) : L) - (k0 + 4 * g);
    auto valid = [&](int i) { return 8 * (i >> 2) + (i & 3) < rem; };
    bool rescaled;
    const float alpha = need_mask ? softmax_tile<16, true>(s, valid, c, neg, m_used, lsum, rescaled)
                                  : softmax_tile<16, false>(s, valid, c, neg, m_used, lsum, rescaled);
    if (rescaled) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }

    // O^T[d][query] += V^T[d][key] P^T[key][query]: step i takes key 8*(i/4) + 4*g + i%4
    // from lane half g, the key whose probability this lane holds in s[i].
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = 8 * (i >> 2) + 4 * g + (i & 3);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[kr * C::kVStride + db * 32 + r32], s[i], oacc[db], 0, 0, 0);
    }
  }

  float* Og = static_cast<float*>(p.o) + (size_t)bh * p.Nq * D;
  float* lseg = p.lse + (size_t)bh * p.Nq;
  const float lt = pair32_sum(lsum);
  if (qi < p.Nq) {
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (g == 0) lseg[qi] = lt > 0.0f ? (m_used + fast_log2(lt)) * kLn2 : -kInf;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        f32x4 x = {oacc[db][4 * jq] * inv, oacc[db][4 * jq + 1] * inv, oacc[db][4 * jq + 2] * inv,
                   oacc[db][4 * jq + 3] * inv};
        *reinterpret_cast<f32x4*>(Og + (size_t)qi * D + db * 32 + 8 * jq + 4 * g) = x;
      }
  }
}

template <int D>
static hipError_t launch_f32(PrefillParams p, hipStream_t stream) {
  using C = PrefillF32Cfg<D>;
  p.n_qtiles = (p.Nq + C::kBM - 1) / C::kBM;
  p.n_tiles = p.B * p.H * p.n_qtiles;
  if (p.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3(p.n_tiles), dim3(C::kThreads), C::kLdsBytes, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream) {
  if (d == 64) return launch_f32<64>(p, stream);
  return launch_f32<128>(p, stream);
}

}  // namespace fa
