// fa_prefill_bf16.hip -- tiled attention forward for bf16 Q/K/V on gfx950 (MI355X).
//
// One workgroup of 4 waves owns BM = 4 * 32 * NQB query rows of one (b, h) and streams the K/V
// tiles of that head through LDS (page "FlashAttention：把注意力从公式写成数据流", sections
// "分块与在线 softmax" and "SRAM 预算与 tile 选择"; page "FlashAttention 与边缘设备上的注意力内存
// 瓶颈", section "3.1 Tiling"). The score and probability tiles live only in registers; the
// output accumulator stays in registers for the whole key loop and is written once.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulation). Each wave computes the
// TRANSPOSED score tile S^T = K * Q^T (32 keys x 32 queries per instruction), so that in the
// accumulator every lane holds scores of ONE query (lane % 32) for 16 keys; the two lanes l and
// l ^ 32 share a query. Then:
//   * the softmax row reductions are in-lane plus one cross-half exchange;
//   * the probabilities are already in the B-operand layout of O^T += V^T * P^T, and the output
//     accumulator O^T again has one query per lane, so the per-row rescale needs no shuffle.
// The K rows fed to the A operand are permuted within each 32-key block (bits 2 and 3 of the row
// index swapped) so that each lane's 16 scores are two runs of 8 consecutive keys; a run of 8
// consecutive keys is exactly one 16-byte read of V^T from LDS.
//
// LDS per stage: K tile [BN][D + 8] (16-byte row padding) and V^T tile [D][BN] built by an
// in-register 4x8 transpose at store time, its 16-byte units XOR-swizzled by row. Two stages:
// tile j + 1 is fetched from HBM into registers while tile j is consumed from LDS.
#include "fa_device.h"
#include "fa_params.h"
#include "fa_softmax.h"

namespace fa {

template <int D, int NQB>
struct PrefillBf16Cfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kQW = 32 * NQB;          // query rows per wave
  static constexpr int kBM = kWaves * kQW;      // query rows per workgroup
  static constexpr int kBN = 64;                // keys per K/V tile
  static constexpr int kKStride = D + 8;        // bf16 per K row in LDS
  static constexpr int kKElems = kBN * kKStride;
  static constexpr int kVtElems = D * kBN;
  static constexpr int kStageElems = kKElems + kVtElems;
  static constexpr int kLdsBytes = 2 * kStageElems * 2;
  static constexpr int kKChunks = kBN * D / 8 / kThreads;  // 16-byte K pieces per thread
  static constexpr int kVJobs = (kBN / 4) * (D / 8);       // 4-key x 8-d V blocks per tile
  static_assert(kKChunks * kThreads * 8 == kBN * D, "K tile must split evenly");
  static_assert(kVJobs <= kThreads, "one V block per thread at most");
};

// Row of the K tile in LDS that holds key `r` (an involution: swap bits 2 and 3).
__device__ __forceinline__ int k_perm(int r) {
  return (r & ~0xC) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 2);
}
// XOR swizzle of the 16-byte units (8 keys) of V^T row d.
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D, int NQB>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillParams p) {
  using C = PrefillBf16Cfg<D, NQB>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // Work decomposition: workgroup -> (b, h, query tile); causal tiles heaviest first.
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

  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Nq * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.Nk * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.Nk * D;

  const int qw0 = q0 + w * C::kQW;
  const int qw_last = min(qw0 + C::kQW, p.Nq) - 1;  // < qw0 when the wave has no rows
  const float c = p.c;
  const bool neg = c < 0.0f;

  // Q tile -> registers, already in the B-operand layout of S^T = K Q^T.
  bf16x8 qreg[NQB][D / 16];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = qw0 + qb * 32 + r32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < p.Nq) x = *reinterpret_cast<const u32x4*>(Qg + (size_t)row * D + ks * 16 + g * 8);
      qreg[qb][ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[NQB][D / 32];
  float m_used[NQB], lsum[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_used[qb] = -kInf;
    lsum[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.0f;
  }

  // K/V tile fetch (HBM -> registers) and store (registers -> LDS stage).
  u32x4 kpre[C::kKChunks];
  u32x4 vpre[4];
  const int vc = tid % (D / 8);  // this thread's 8-wide d chunk of V
  const int vkq = tid / (D / 8); // and its group of 4 keys

  auto fetch = [&](int j) {
    const int k0 = j * C::kBN;
#pragma unroll
    for (int it = 0; it < C::kKChunks; ++it) {
      const int idx = tid + it * C::kThreads;
      const int row = idx / (D / 8);
      const int ch = idx % (D / 8);
      const int key = k0 + row;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < L) x = *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + ch * 8);
      kpre[it] = x;
    }
    if (tid < C::kVJobs) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + vkq * 4 + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < L) x = *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + vc * 8);
        vpre[r] = x;
      }
    }
  };

  auto store = [&](int stage) {
    uint16_t* Ks = smem + stage * C::kStageElems;
    uint16_t* Vt = Ks + C::kKElems;
#pragma unroll
    for (int it = 0; it < C::kKChunks; ++it) {
      const int idx = tid + it * C::kThreads;
      const int row = idx / (D / 8);
      const int ch = idx % (D / 8);
      *reinterpret_cast<u32x4*>(Ks + k_perm(row) * C::kKStride + ch * 8) = kpre[it];
    }
    if (tid < C::kVJobs) {
      const int unit = vkq >> 1;   // 8-key unit of the V^T row
      const int half = vkq & 1;    // which 4 keys of the unit
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = vc * 8 + e;
        const int wd = e >> 1;
        uint32_t w01, w23;
        if ((e & 1) == 0) {
          w01 = (vpre[0][wd] & 0xffffu) | (vpre[1][wd] << 16);
          w23 = (vpre[2][wd] & 0xffffu) | (vpre[3][wd] << 16);
        } else {
          w01 = (vpre[0][wd] >> 16) | (vpre[1][wd] & 0xffff0000u);
          w23 = (vpre[2][wd] >> 16) | (vpre[3][wd] & 0xffff0000u);
        }
        u32x2 pr = {w01, w23};
        *reinterpret_cast<u32x2*>(Vt + d * C::kBN + ((unit ^ vt_swz(d)) << 3) + half * 4) = pr;
      }
    }
  };

  if (ntiles > 0) {
    fetch(0);
    store(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int st = j & 1;
    if (j + 1 < ntiles) fetch(j + 1);

    const int k0 = j * C::kBN;
    const bool active = (qw_last >= qw0) && (!p.causal || k0 <= qw_last);
    if (active) {
      const uint16_t* Ks = smem + st * C::kStageElems;
      const uint16_t* Vt = Ks + C::kKElems;

      // Scores: S^T[key][query] for the two 32-key blocks of the tile.
      f32x16 sacc[NQB][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[qb][kb][i] = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* krow = Ks + (kb * 32 + r32) * C::kKStride + g * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ks * 16);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], sacc[qb][kb], 0, 0, 0);
        }
      }

      // Masks are needed only on the tail tile and on tiles that cross this wave's diagonal.
      const bool need_mask = (k0 + C::kBN > L) || (p.causal && k0 + C::kBN - 1 > qw0);

      bf16x8 pk[NQB][2][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw0 + qb * 32 + r32;
        float s[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb * 16 + i] = sacc[qb][kb][i];
        // Score s[kb*16 + i] belongs to key k0 + kb*32 + 16*(i/8) + 8*g + i%8.
        auto valid = [&](int x) {
          const int kb = x >> 4, i = x & 15;
          const int key = k0 + kb * 32 + ((i >> 3) << 4) + (g << 3) + (i & 7);
          return key < L && (!p.causal || key <= qi);
        };
        bool rescaled;
        const float alpha = softmax_tile<32>(s, need_mask, valid, c, neg, m_used[qb], lsum[qb], rescaled);
        if (rescaled) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            u32x4 x;
#pragma unroll
            for (int t = 0; t < 4; ++t)
              x[t] = pack_bf16(s[kb * 16 + hh * 8 + 2 * t], s[kb * 16 + hh * 8 + 2 * t + 1]);
            pk[qb][kb][hh] = __builtin_bit_cast(bf16x8, x);
          }
      }

      // O^T[d][query] += V^T[d][keys] * P^T[keys][query], 16 keys per instruction.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int unit = kb * 4 + hh * 2 + g;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int d = db * 32 + r32;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vt + d * C::kBN + ((unit ^ vt_swz(d)) << 3));
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[qb][kb][hh], oacc[qb][db], 0, 0, 0);
          }
        }
    }

    if (j + 1 < ntiles) store(st ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, lse = ln 2 * (m + log2 l); a row with no allowed key gets 0 and -inf.
  uint16_t* Og = static_cast<uint16_t*>(p.o) + (size_t)bh * p.Nq * D;
  float* lseg = p.lse + (size_t)bh * p.Nq;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = pair32_sum(lsum[qb]);
    const int qi = qw0 + qb * 32 + r32;
    if (qi < p.Nq) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      if (g == 0) lseg[qi] = lt > 0.0f ? (m_used[qb] + fast_log2(lt)) * kLn2 : -kInf;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          // Accumulator entries 4*jq .. 4*jq+3 are d = db*32 + 8*jq + 4*g + 0..3 of row qi.
          u32x2 x = {pack_bf16(oacc[qb][db][4 * jq + 0] * inv, oacc[qb][db][4 * jq + 1] * inv),
                     pack_bf16(oacc[qb][db][4 * jq + 2] * inv, oacc[qb][db][4 * jq + 3] * inv)};
          *reinterpret_cast<u32x2*>(Og + (size_t)qi * D + db * 32 + 8 * jq + 4 * g) = x;
        }
    }
  }
}

template <int D, int NQB>
static hipError_t launch_bf16(PrefillParams p, hipStream_t stream) {
  using C = PrefillBf16Cfg<D, NQB>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_bf16_kernel<D, NQB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  p.n_qtiles = (p.Nq + C::kBM - 1) / C::kBM;
  p.n_tiles = p.B * p.H * p.n_qtiles;
  if (p.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NQB>), dim3(p.n_tiles), dim3(C::kThreads),
                     C::kLdsBytes, stream, p);
  return hipGetLastError();
}

// Rows per workgroup used for a given head dimension (the host checks grid limits with it).
int prefill_bf16_rows_per_wg(int d) { return d == 64 ? PrefillBf16Cfg<64, 1>::kBM : PrefillBf16Cfg<128, 1>::kBM; }

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream) {
  if (d == 64) return launch_bf16<64, 1>(p, stream);
  return launch_bf16<128, 1>(p, stream);
}

}  // namespace fa
