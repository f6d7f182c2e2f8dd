// fa_backward.hip -- backward pass of the attention forward for bf16 Q/K/V on gfx950 (MI355X).
//
// Training needs the gradients of the forward pass, and the tiled method gets them by
// recomputing S and P tile by tile from Q, K and the logsumexp the forward pass saved, instead of
// storing P (page "FlashAttention：把注意力从公式写成数据流", section "用实验验证而不是背诵结论";
// page "[2205.14135] FlashAttention ...", section "三、FLOPs（計算能力）並非 Speedup 的主因素").
// With D_i = dO_i . O_i the chain rule of the forward definition gives, per allowed pair (i, j):
//   P_ij = exp(scale q_i.k_j - lse_i),  dV_j += P_ij dO_i,  dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),  dQ_i += scale dS_ij k_j,  dK_j += scale dS_ij q_i.
// Three kernels:
//   bwd_delta_kernel  D_i = dO_i . O_i for every query row (fp32), several rows per wave;
//   bwd_dq_kernel     one workgroup of 8 waves per 128 query rows, K/V tiles through LDS; per
//                     SIMD one wave computes S^T = K Q^T and P^T, its partner dP^T = V dO^T,
//                     then both dS^T and half each of dQ^T += K^T dS^T;
//   bwd_dkdv_kernel   one workgroup of 8 waves per 128 keys, Q/dO tiles through LDS; per SIMD
//                     one wave computes S = Q K^T, P and dV^T += dO^T P, its partner dP = dO V^T,
//                     then (taking P through LDS) dS and dK^T += Q^T dS.
// Splitting dQ from dK/dV recomputes S and dP once more (7 matrix products per tile pair instead
// of 5) but needs no atomics and gives run-to-run identical gradients. All products are bf16 on
// the matrix cores with fp32 accumulation; P and dS are rounded to bf16 before their products,
// gradients to bf16 once at the end.
//
// Operand layouts (v_mfma_f32_32x32x16_bf16, 64 lanes; lane l = 32 g + r32):
//   A operand: lane holds A[m = r32][k = 8g .. 8g+7] (+16 per k step); B operand: lane holds
//   B[k = 8g .. 8g+7][n = r32]; accumulator entry e of lane l is C[8(e/4) + 4g + e%4][r32].
// Row-read operands whose rows become the accumulator's rows are read in the order of
// bwd_perm (bits 2 and 3 of the row index swapped), so that a lane's 16 accumulator entries are
// two runs of 8 consecutive rows: exactly a B operand of the next product, with no shuffle.
#include "fa_device.h"
#include "fa_params.h"

#include <type_traits>

namespace fa {

// Row of a 32-row block read by accumulator row r: key_row_perm (bits 2 and 3 swapped).
__device__ __forceinline__ int bwd_perm(int r) { return key_row_perm(r); }

// ---- D_i = dO_i . O_i (fp32). D/8 lanes share a row, 16 bytes of O and of dO each, so one wave
// load covers 64/(D/8) whole rows; each lane takes kRowSteps rows, all loads issued before the
// arithmetic. Per row: an in-lane sum of 8 products, then a sum over the row's lanes.
template <int D>
struct BwdDeltaCfg {
  static constexpr int kLanesPerRow = D / 8;
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kRowSteps = 4;
  static constexpr int kRowsPerWave = kRowsPerLoad * kRowSteps;
  static constexpr int kRowsPerWg = 4 * kRowsPerWave;  // 4 waves
};

template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BackwardParams p) {
  using C = BwdDeltaCfg<D>;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int part = lane % C::kLanesPerRow;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  const int64_t row0 = (int64_t)blockIdx.x * C::kRowsPerWg + w * C::kRowsPerWave + lane / C::kLanesPerRow;
  u32x4 a[C::kRowSteps], bb[C::kRowSteps];
#pragma unroll
  for (int r = 0; r < C::kRowSteps; ++r) {
    const int64_t row = row0 + r * C::kRowsPerLoad;
    const u32x4 z = {0u, 0u, 0u, 0u};
    a[r] = row < rows ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.o) + row * D + part * 8) : z;
    bb[r] = row < rows ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.dout) + row * D + part * 8) : z;
  }
#pragma unroll
  for (int r = 0; r < C::kRowSteps; ++r) {
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) acc += bf16_lo(a[r][t]) * bf16_lo(bb[r][t]) + bf16_hi(a[r][t]) * bf16_hi(bb[r][t]);
#pragma unroll
    for (int m = 1; m < C::kLanesPerRow; m <<= 1) acc += __shfl_xor(acc, m, 64);
    const int64_t row = row0 + r * C::kRowsPerLoad;
    if (part == 0 && row < rows) p.delta[row] = acc;
  }
}

template <int D>
struct BwdCfg {
  static constexpr int kNch = D / 8;  // 16-byte pieces per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = 64 * kRowBytes;  // one 64-row tile of K, V, Q or dO
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kKiBPerWave = kTileBytes / 1024 / 4;
};

// 16-byte piece swizzle of LDS row r, for tiles the backward kernels read both as rows and
// transposed. The LDS serves 256 bytes a pass: 16 lanes of a 16-byte row read (ds_read_b128), 32
// lanes of an 8-byte transposed read (ds_read_b64_tr_b16). Row reads take one piece of 16 rows of
// an aligned block of 16 (in bwd_perm order or not), so the swizzle must be a bijection on each
// such block. Transposed reads take, in each pass, two 16-lane groups: 4 consecutive rows (r % 4
// varying) times 4 pieces (two adjacent pieces per group, the groups' pieces 2 apart).
// With x = r % 16 (bits x3 x2 x1 x0):
// d = 128 (16 pieces per row, one row per 256-byte bank line): (x1, x0, x3, x2). Bits 3 and 2 of
// the swizzle are a bijection of r % 4, which separates the 4 rows of a transposed pass while
// the pieces (bits 1 and 0) separate the lanes within a row. An earlier form, (x3, x1, x0, x2^x3),
// let rows r and r + 1 collide in those passes: one conflict cycle per three active ones.
// d = 64 (8 pieces; two rows share a 256-byte line): (x0 ^ x1 ^ x3, x0 ^ x2, x1).
template <int D>
__device__ __forceinline__ int bwd_swz(int r) {
  const int x0 = r & 1, x1 = (r >> 1) & 1, x2 = (r >> 2) & 1, x3 = (r >> 3) & 1;
  if (D == 128) return (x1 << 3) | (x0 << 2) | (x3 << 1) | x2;
  return ((x0 ^ x1 ^ x3) << 2) | ((x0 ^ x2) << 1) | x1;
}

// Per-lane byte offsets of the direct HBM -> LDS copies of a 64-row tile (lane i of a KiB block
// fills LDS row rb + i / kNch, slot i % kNch). Permuted rows (the dQ kernel's K): LDS row r holds
// tile row bwd_perm(r); plain rows: LDS row r holds tile row r; piece slot ^ bwd_swz(r) in both.
template <int D>
__device__ __forceinline__ uint32_t bwd_off_row(int w, int it, int lane) {
  using C = BwdCfg<D>;
  const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
  const int slot = lane % C::kNch;
  return (uint32_t)(bwd_perm(row) * C::kRowBytes + ((slot ^ bwd_swz<D>(row)) << 4));
}
template <int D>
__device__ __forceinline__ uint32_t bwd_off_tr(int w, int it, int lane) {
  using C = BwdCfg<D>;
  const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
  const int slot = lane % C::kNch;
  return (uint32_t)(row * C::kRowBytes + ((slot ^ bwd_swz<D>(row)) << 4));
}

// ---- dQ, two waves per SIMD. A workgroup of 8 waves owns 128 query rows; waves w and w + 4 (one
// SIMD) share the 32-row block qb = w & 3, with one query per lane in both. Per 64-key tile (K with
// rows in bwd_perm order and V, both in stages of LDS):
//   phase A   S wave (w < 4):   S^T = K Q^T, P^T = 2^(c s - lse2) (masked) -> LDS as bf16;
//             dP wave (w >= 4): dP^T = V dO^T, (dP^T - D) -> LDS as bf16;
//   barrier
//   phase B   each wave one 32-key block (S wave keys 0..31, dP wave 32..63): dS^T = P^T (dP^T - D)
//             of that block from its own value and the partner's, then dQ^T += K^T dS^T over
//             the whole head dimension into its own accumulator;
//   barrier (after this wave's copies of the next tile have landed).
// 24 MFMAs per wave and tile, none recomputed, and the S wave's exponentials overlap the dP wave's
// matrix work on the same SIMD. Splitting phase B by keys rather than by head dimension means
// each wave forms and exchanges only the half of dS it uses; the two partial dQ sums are added
// once, at the end.
template <int D>
struct BwdQCfg {
  static constexpr int kWaves = 8;
  static constexpr int kNch = D / 8;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = 64 * kRowBytes;            // a 64-key tile of K or V
  static constexpr int kStageBytes = 2 * kTileBytes;           // K tile, V tile
  static constexpr int kXBase = 2 * kStageBytes;
  static constexpr int kXBytes = 4 * 2 * 4 * 64 * 16;          // 4 pairs x 2 values x 4 slots x 64 lanes x 16 B
  static constexpr int kLdsBytes = kXBase + kXBytes;
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kKiBPerWave = kTileBytes / 1024 / kWaves;  // per tensor per tile
  static constexpr int kHalf = D / 64;                         // 32-d blocks of dQ per wave
  static_assert(kKiBPerWave * kWaves * 1024 == kTileBytes, "tile must split over the waves");
  static_assert(kXBase <= 65536, "stages must sit within the LDS immediate-offset range");
  static_assert(8 * kHalf * 4096 <= kXBase, "the closing exchange of dQ halves fits in the stage area");
};

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BackwardParams p) {
  using C = BwdQCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qb = w & 3;
  const bool swave = w < 4;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  // Workgroups in order of decreasing work: under causal masking the last query tiles of every
  // head first (the head index runs fastest), so the heaviest tiles never start last.
  const int nqt = (p.Nq + 127) / 128;
  const int nbh = p.B * p.H;
  const int qr_ = blockIdx.x / nbh;
  const int bh = blockIdx.x - qr_ * nbh;
  const int qt = p.causal ? nqt - 1 - qr_ : qr_;
  const int b = bh / p.H;
  const int q0 = qt * 128;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  int kend = L;
  if (p.causal) kend = min(kend, min(q0 + 128, p.Nq));
  const int ntiles = kend > 0 ? (kend + 63) / 64 : 0;

  const uint16_t* QDg = static_cast<const uint16_t*>(swave ? p.q : p.dout) + (size_t)bh * p.Nq * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.Nk * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t qdrs = make_rsrc(QDg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, (uint32_t)kend * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vg, (uint32_t)kend * C::kRowBytes);

  // B operands: lane (r32, g) holds Q (S wave) or dO (dP wave) of query qi, [16 ks + 8 g .. +8].
  const int qi = q0 + qb * 32 + r32;
  bf16x8 qd[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qd[ks] = __builtin_bit_cast(bf16x8, buf_load16(qdrs, ((uint32_t)qi * D + ks * 16 + g * 8) * 2));
  // The S wave needs this query's base-2 logsumexp (+inf for rows past Nq or without keys: P = 0),
  // the dP wave its D.
  float lsd = swave ? kInf : 0.0f;
  if (qi < p.Nq) {
    const size_t qrow = (size_t)bh * p.Nq + qi;
    if (swave) {
      const float l = p.lse[qrow];
      lsd = l == -kInf ? kInf : l * kLog2e;
    } else {
      lsd = p.delta[qrow];
    }
  }
  // Wait for the register loads once and hide their origin, so the loop carries no vector-memory
  // waits for them (such waits would also drain the tile copies in flight).
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(qd[ks]));
  asm volatile("" : "+v"(lsd));
  const float c = p.scale * kLog2e;

  // Tile copies: K rows permuted (LDS row r holds key bwd_perm(r)), V rows plain, pieces slot ^
  // bwd_swz(r); wave w moves KiB blocks w*kKiBPerWave .. of each tensor.
  uint32_t koff[C::kKiBPerWave], voff[C::kKiBPerWave];
#pragma unroll
  for (int it = 0; it < C::kKiBPerWave; ++it) {
    const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
    const int slot = lane % C::kNch;
    koff[it] = (uint32_t)(bwd_perm(row) * C::kRowBytes + ((slot ^ bwd_swz<D>(row)) << 4));
    voff[it] = (uint32_t)(row * C::kRowBytes + ((slot ^ bwd_swz<D>(row)) << 4));
  }
  auto issue = [&](int tile, int stage) {
    char* dst = smem + stage * C::kStageBytes;
    const uint32_t base = (uint32_t)tile * C::kTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKiBPerWave; ++it) {
      char* blk = dst + (w * C::kKiBPerWave + it) * 1024;
      buf_load16_lds(krs, blk, base + koff[it]);
      buf_load16_lds(vrs, blk + C::kTileBytes, base + voff[it]);
    }
  };

  // Per-lane LDS offsets. Row operands: K (S wave) LDS row kb*32 + r32, V (dP wave) LDS row
  // kb*32 + bwd_perm(r32) (its keys in the S wave's order), piece (2 ks + g) ^ bwd_swz(row).
  // K^T operands (both): in 16-lane group G (gp = G % 2), lane 4a+b addresses key
  // 16u + 8g + 4rd + a, which sits in LDS row 16u + 8rd + 4g + a, and d = db*32 + 16gp + 4b for
  // this wave's half of the blocks db. Exchange: own and partner slots of pair qb.
  const int li = lane & 15;
  const int ta = li >> 2, tb = li & 3;
  const int gp = (lane >> 4) & 1;
  const int rrow = swave ? r32 : bwd_perm(r32);
  uint32_t rofs[D / 16], kt[2][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    rofs[ks] = (uint32_t)((swave ? 0 : C::kTileBytes) + rrow * C::kRowBytes + (((2 * ks + g) ^ bwd_swz<D>(rrow)) << 4));
    asm volatile("" : "+v"(rofs[ks]));
  }
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int r = 8 * rd + 4 * g + ta;
      const int piece = db * 4 + 2 * gp + (tb >> 1);
      kt[rd][db] = (uint32_t)(r * C::kRowBytes + ((piece ^ bwd_swz<D>(r)) << 4) + 8 * (tb & 1));
      asm volatile("" : "+v"(kt[rd][db]));
    }
  uint32_t xown = (uint32_t)(C::kXBase + qb * 8192 + (swave ? 0 : 4096) + lane * 16);
  uint32_t xoth = (uint32_t)(C::kXBase + qb * 8192 + (swave ? 4096 : 0) + lane * 16);
  asm volatile("" : "+v"(xown), "+v"(xoth));

  f32x16 acc[D / 32];  // this wave's keys' share of dQ^T: entry e of block db is dQ[qi][db*32 + 8(e/4) + 4g + e%4]
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
  f32x16 xs[2];  // P^T (S wave) or dP^T - D (dP wave) of the tile's two 32-key blocks

  constexpr int kNR = 2 * (D / 16);    // phase A: key block kb = m & 1, step ks = m >> 1
  constexpr int kNT = 2 * (D / 32);   // phase B: 16-key step u2 = m / (D/32) of the wave's block, d block m % (D/32)
  constexpr int kAhead = 3;

  auto phase_a = [&](auto stage_tag, int k0) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    auto fetch = [&](int m) -> bf16x8 __attribute__((always_inline)) {
      const int kb = m & 1, ks = m >> 1;
      return *reinterpret_cast<const bf16x8*>(smem + (S * C::kStageBytes + kb * 32 * C::kRowBytes + (int)rofs[ks]));
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) xs[kb][e] = 0.0f;
    bf16x8 op[kNR];
#pragma unroll
    for (int m = 0; m < kAhead; ++m) op[m] = fetch(m);
#pragma unroll
    for (int m = 0; m < kNR; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + kAhead < kNR) op[m + kAhead] = fetch(m + kAhead);
      xs[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], qd[m >> 1], xs[m & 1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Entry e of block kb is key k0 + kb*32 + 16(e/8) + 8g + e%8 of this lane's query qi. The
    // mask (keys past L, keys after the query when causal) matters only on tiles reaching past L
    // or past the workgroup's first row: elsewhere one FMA and one exponential per score.
    const int rem = (p.causal ? min(L, qi + 1) : L) - (k0 + 8 * g);
    const bool masked = k0 + 64 > L || (p.causal && k0 + 63 > q0);
    // One code path per role and mask case (a role test inside the loop would be if-converted,
    // making every wave compute both roles' values).
    auto values = [&](auto role_tag, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool kS = decltype(role_tag)::value;
      constexpr bool kMask = decltype(mask_tag)::value;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 xo;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            float v2[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int e = hh * 8 + 2 * t2 + u;
              if constexpr (kS) {
                const float e2 = fast_exp2(fmaf(xs[kb][e], c, -lsd));
                if constexpr (kMask) v2[u] = (kb * 32 + 16 * hh + 2 * t2 + u < rem) ? e2 : 0.0f;
                else v2[u] = e2;
              } else {
                v2[u] = xs[kb][e] - lsd;
              }
              xs[kb][e] = v2[u];
            }
            xo[t2] = pack_bf16(v2[0], v2[1]);
          }
          // Only the partner's key block crosses over (the S wave's block is 0, the dP wave's 1).
          if (kb == (kS ? 1 : 0)) *reinterpret_cast<u32x4*>(smem + ((kb * 2 + hh) * 1024 + (int)xown)) = xo;
        }
    };
    if (swave) {
      if (masked) values(std::true_type{}, std::true_type{});
      else values(std::true_type{}, std::false_type{});
    } else {
      values(std::false_type{}, std::false_type{});
    }
  };

  auto phase_b = [&](auto stage_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    // One code path per role: the wave's key block kbo must be known at compile time so that xs
    // is indexed statically.
    auto run = [&](auto role_tag) __attribute__((always_inline)) {
      constexpr int kbo = decltype(role_tag)::value ? 0 : 1;
      auto fetch = [&](int m) -> bf16x8 __attribute__((always_inline)) {
        const int u = 2 * kbo + m / (D / 32), db = m % (D / 32);
        const int o = S * C::kStageBytes + u * 16 * C::kRowBytes;
        const s16x4 a8[2] = {lds_read_tr16(smem + (o + (int)kt[0][db])), lds_read_tr16(smem + (o + (int)kt[1][db]))};
        return __builtin_bit_cast(bf16x8, a8);
      };
      bf16x8 op[kNT];
#pragma unroll
      for (int m = 0; m < kAhead; ++m) op[m] = fetch(m);
      // dS^T of this wave's key block = own value times the partner's (P^T times dP^T - D), as
      // bf16 B operands.
      bf16x8 dsk[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 oth = *reinterpret_cast<const u32x4*>(smem + ((kbo * 2 + hh) * 1024 + (int)xoth));
        u32x4 xo;
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2)
          xo[t2] = pack_bf16(xs[kbo][hh * 8 + 2 * t2] * bf16_lo(oth[t2]), xs[kbo][hh * 8 + 2 * t2 + 1] * bf16_hi(oth[t2]));
        dsk[hh] = __builtin_bit_cast(bf16x8, xo);
      }
#pragma unroll
      for (int m = 0; m < kNT; ++m) {
        __builtin_amdgcn_sched_barrier(0);
        if (m + kAhead < kNT) op[m + kAhead] = fetch(m + kAhead);
        const int db = m % (D / 32);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], dsk[m / (D / 32)], acc[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    if (swave) run(std::true_type{});
    else run(std::false_type{});
  };

  auto interval = [&](auto stage_tag, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    const bool more = t + 1 < ntiles;
    if (more) issue(t + 1, 1 - S);
    if (swave) __builtin_amdgcn_s_setprio(1);
    phase_a(stage_tag, t * 64);
    __builtin_amdgcn_s_setprio(0);
    wg_barrier_lds();
    phase_b(stage_tag);
    if (more) wait_vmcnt<0>();
    wg_barrier_lds();
  };

  if (ntiles > 0) {
    issue(0, 0);
    wait_vmcnt<0>();
  }
  wg_barrier_lds();
  for (int t = 0; t < ntiles; t += 2) {
    interval(std::integral_constant<int, 0>{}, t);
    if (t + 1 >= ntiles) break;
    interval(std::integral_constant<int, 1>{}, t + 1);
  }
  wait_vmcnt<0>();

  // The two waves of a pair hold the sums over their own keys for the whole head dimension. Each
  // writes the half the partner stores into the stage area (no longer read: the loop's last
  // barrier has passed), then adds the partner's share of its own half and stores it. Block j of
  // half h for pair qb sits at ((qb * 2 + h) * kHalf + j) * 4 KiB, 16 bytes per lane and quarter.
  // One code path per role, so that every accumulator index is a compile-time constant (a
  // run-time index would move the accumulators to scratch memory).
  auto finish = [&](auto role_tag) __attribute__((always_inline)) {
    constexpr bool kS = decltype(role_tag)::value;
    constexpr int kOwn = kS ? 0 : C::kHalf, kOth = kS ? C::kHalf : 0;  // first d block of each half
    constexpr int hOwn = kS ? 0 : 1, hOth = kS ? 1 : 0;
#pragma unroll
    for (int j = 0; j < C::kHalf; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 x = {acc[kOth + j][4 * e4], acc[kOth + j][4 * e4 + 1], acc[kOth + j][4 * e4 + 2], acc[kOth + j][4 * e4 + 3]};
        *reinterpret_cast<f32x4*>(smem + (((qb * 2 + hOth) * C::kHalf + j) * 4 + e4) * 1024 + lane * 16) = x;
      }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < C::kHalf; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(smem + (((qb * 2 + hOwn) * C::kHalf + j) * 4 + e4) * 1024 + lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kOwn + j][4 * e4 + i] += x[i];
      }
    if (qi < p.Nq) {
      uint16_t* dQg = static_cast<uint16_t*>(p.dq) + (size_t)bh * p.Nq * D + (size_t)qi * D;
#pragma unroll
      for (int j = 0; j < C::kHalf; ++j)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const u32x2 x = {pack_bf16(acc[kOwn + j][4 * jq] * p.scale, acc[kOwn + j][4 * jq + 1] * p.scale),
                           pack_bf16(acc[kOwn + j][4 * jq + 2] * p.scale, acc[kOwn + j][4 * jq + 3] * p.scale)};
          *reinterpret_cast<u32x2*>(dQg + (kOwn + j) * 32 + 8 * jq + 4 * g) = x;
        }
    }
  };
  if (swave) finish(std::true_type{});
  else finish(std::false_type{});
}

// ---- dK, dV, two waves per SIMD. A workgroup of 8 waves owns 128 keys; waves w and w + 4 (one
// SIMD) share the 32-key block kb = w & 3 and split the four products of each 64-query tile:
//   phase A   P wave (w < 4):   S = Q K^T, P = 2^(c s - lse2) (masked), P -> LDS as bf16;
//             dS wave (w >= 4): dP = dO V^T, kept in registers;
//   barrier
//   phase B   P wave:           dV^T += dO^T P (P still in its registers);
//             dS wave:          P <- LDS, dS = P (dP - D), dK^T += Q^T dS;
//   barrier (after this wave's copies of the next tile have landed).
// Neither wave recomputes S; in each phase both issue 16 MFMAs per 32 keys, and the P wave's
// exponentials (phase A) and the dS wave's dS (phase B) overlap the partner's matrix work on the
// same SIMD. Rows are read in bwd_perm order, so the S accumulator of the P wave and the dP
// accumulator of the dS wave hold the same (query, key) pairs entry by entry: P crosses over lane
// for lane. Two stages (tile t, and tile t + 1 in flight) sit in the low 64 KiB of LDS so that every
// stage address is a per-lane register plus an immediate; P and the lse/D rows lie above.
template <int D>
struct BwdKvCfg {
  static constexpr int kWaves = 8;
  static constexpr int kNch = D / 8;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = 64 * kRowBytes;            // a 64-row tile of Q or dO
  static constexpr int kStageBytes = 2 * kTileBytes;           // Q tile, dO tile
  static constexpr int kPBase = 2 * kStageBytes;
  static constexpr int kPBytes = 4 * 4 * 64 * 16;              // 4 key blocks x 4 slots x 64 lanes x 16 B
  static constexpr int kLsBase = kPBase + kPBytes;             // per stage: lse2[64], D[64]
  static constexpr int kLdsBytes = kLsBase + 2 * 512;
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kKiBPerWave = kTileBytes / 1024 / kWaves;  // per tensor per tile
  static_assert(kKiBPerWave * kWaves * 1024 == kTileBytes, "tile must split over the waves");
  static_assert(kPBase <= 65536, "stages must sit within the LDS immediate-offset range");
};

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BackwardParams p) {
  using C = BwdKvCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = w & 3;
  const bool pwave = w < 4;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  // Workgroups in order of decreasing work: under causal masking the first key tiles of every head
  // first (the head index runs fastest), so the heaviest tiles never start last.
  const int nkt = (p.Nk + 127) / 128;
  const int nbh = p.B * p.H;
  const int kt = blockIdx.x / nbh;
  const int bh = blockIdx.x - kt * nbh;
  const int b = bh / p.H;
  const int k0 = kt * 128;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  const int kj = k0 + kb * 32 + r32;  // this lane's key
  // Query tiles that can see a key of this workgroup: from the first row at or after k0 when
  // causal, none when every key is past L.
  const int t0 = (p.causal && k0 < L) ? k0 / 64 : 0;
  const int tn = k0 < L ? (p.Nq + 63) / 64 : 0;

  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Nq * D;
  const uint16_t* dOg = static_cast<const uint16_t*>(p.dout) + (size_t)bh * p.Nq * D;
  const uint16_t* KVg = static_cast<const uint16_t*>(pwave ? p.k : p.v) + (size_t)bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dOg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t kvrs = make_rsrc(KVg, (uint32_t)L * C::kRowBytes);
  const float* lse_bh = p.lse + (size_t)bh * p.Nq;
  const float* dl_bh = p.delta + (size_t)bh * p.Nq;

  // B operands: lane (r32, g) holds K (P wave) or V (dS wave) of key kj, [16 ks + 8 g .. +8];
  // keys past L read as zeros.
  bf16x8 kv[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    kv[ks] = __builtin_bit_cast(bf16x8, buf_load16(kvrs, ((uint32_t)kj * D + ks * 16 + g * 8) * 2));
  // Wait for these loads once, then hide their origin: otherwise the loop's matrix instructions
  // carry conservative vector-memory waits that also drain the next tile's copies issued just
  // before them, serialising the prefetch.
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(kv[ks]));
  const float c = p.scale * kLog2e;

  // Copies of a query tile into a stage: LDS row r holds tile row r, 16-byte piece slot ^
  // bwd_swz(r); wave w moves KiB blocks w*kKiBPerWave .. of each tensor.
  uint32_t toff[C::kKiBPerWave];
#pragma unroll
  for (int it = 0; it < C::kKiBPerWave; ++it) {
    const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
    const int slot = lane % C::kNch;
    toff[it] = (uint32_t)(row * C::kRowBytes + ((slot ^ bwd_swz<D>(row)) << 4));
  }
  float st_l = -kInf, st_d = 0.0f;  // wave 0: lse and D of the tile in flight, one row per lane
  auto issue = [&](int tile, int stage) {
    char* dst = smem + stage * C::kStageBytes;
    const uint32_t base = (uint32_t)tile * C::kTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKiBPerWave; ++it) {
      char* blk = dst + (w * C::kKiBPerWave + it) * 1024;
      buf_load16_lds(qrs, blk, base + toff[it]);
      buf_load16_lds(drs, blk + C::kTileBytes, base + toff[it]);
    }
    if (w == 0) {
      // Raw values only: converting them here would wait for the loads (and, counters draining
      // in order, for the tile copies) at the start of the interval.
      const int qrow = tile * 64 + lane;
      st_l = -kInf;
      st_d = 0.0f;
      if (qrow < p.Nq) {
        st_l = lse_bh[qrow];
        st_d = dl_bh[qrow];
      }
    }
  };
  auto publish = [&](int stage) {
    if (w == 0) {
      float* ls = reinterpret_cast<float*>(smem + C::kLsBase + stage * 512);
      ls[lane] = st_l == -kInf ? kInf : st_l * kLog2e;  // +inf: rows past Nq or without keys
      ls[64 + lane] = st_d;
    }
  };

  // Per-lane LDS offsets, computed once (the empty asm keeps them from being re-derived per use).
  // Row operands (Q for the P wave, dO for the dS wave) in bwd_perm order: row qb*32 + bwd_perm(r32),
  // piece (2 ks + g) ^ bwd_swz(row). Transposed operands (dO^T for the P wave, Q^T for the dS
  // wave): in 16-lane group G (gp = G % 2), lane 4a+b addresses query 16u + 8g + 4rd + a,
  // d = db*32 + 16gp + 4b. P crossing: key block kb, slot (qb, hh), lane. lse/D: query 8g + ...
  const int qr = bwd_perm(r32);
  const int li = lane & 15;
  const int ta = li >> 2, tb = li & 3;
  const int gp = (lane >> 4) & 1;
  const int rt = pwave ? 0 : C::kTileBytes;  // tensor of the row operands within a stage
  const int tt = pwave ? C::kTileBytes : 0;  // tensor of the transposed operands
  uint32_t rofs[D / 16], tofs[2][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    rofs[ks] = (uint32_t)(rt + qr * C::kRowBytes + (((2 * ks + g) ^ bwd_swz<D>(qr)) << 4));
    asm volatile("" : "+v"(rofs[ks]));
  }
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int piece = db * 4 + 2 * gp + (tb >> 1);
      const int row = 8 * g + 4 * rd + ta;
      tofs[rd][db] = (uint32_t)(tt + row * C::kRowBytes + ((piece ^ bwd_swz<D>(row)) << 4) + 8 * (tb & 1));
      asm volatile("" : "+v"(tofs[rd][db]));
    }
  uint32_t pofs = (uint32_t)(C::kPBase + kb * 4 * 64 * 16 + lane * 16);
  uint32_t lofs = (uint32_t)(C::kLsBase + 8 * g * 4);
  asm volatile("" : "+v"(pofs), "+v"(lofs));

  f32x16 acc[D / 32];  // dV^T (P wave) or dK^T (dS wave): entry e of block db is row kj, column
#pragma unroll         // db*32 + 8(e/4) + 4g + e%4
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
  f32x16 xs[2];     // S (P wave) or dP (dS wave) of the tile's two 32-query blocks
  bf16x8 pbv[2][2]; // the P wave's P operands of the tile
  f32x4 lq[2][2][2];  // lse2 (P wave) or D (dS wave) of this lane's 8 queries per (qb, hh)

  constexpr int kNR = 2 * (D / 16);  // phase A products: block qb = m / (D/16), step ks = m % (D/16)
  constexpr int kNT = 4 * (D / 32);  // phase B products: slot u = m / (D/32) (qb = u/2, hh = u%2), db
  constexpr int kAhead = 3;

  // Phase A on stage S (tile `tile`): the row products, then (P wave) P and its copy to LDS.
  auto phase_a = [&](auto stage_tag, int tile) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    auto fetch = [&](int m) -> bf16x8 __attribute__((always_inline)) {
      const int qb = m / (D / 16), ks = m % (D / 16);
      return *reinterpret_cast<const bf16x8*>(smem + (S * C::kStageBytes + qb * 32 * C::kRowBytes + (int)rofs[ks]));
    };
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) xs[qb][e] = 0.0f;
    bf16x8 op[kNR];
#pragma unroll
    for (int m = 0; m < kAhead; ++m) op[m] = fetch(m);
    // This lane's lse2 (P wave, for P) or D (dS wave, for dS in phase B), read ahead of the matrix
    // work so that their latency is hidden behind it.
    {
      const float* lsr = reinterpret_cast<const float*>(smem + (S * 512 + (int)lofs)) + (pwave ? 0 : 64);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          lq[qb][hh][0] = *reinterpret_cast<const f32x4*>(lsr + qb * 32 + 16 * hh);
          lq[qb][hh][1] = *reinterpret_cast<const f32x4*>(lsr + qb * 32 + 16 * hh + 4);
        }
    }
#pragma unroll
    for (int m = 0; m < kNR; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + kAhead < kNR) op[m + kAhead] = fetch(m + kAhead);
      const int qb = m / (D / 16), ks = m % (D / 16);
      xs[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], kv[ks], xs[qb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!pwave) return;
    // Entry e of block qb is query tile*64 + qb*32 + 16(e/8) + 8g + e%8 against key kj. The mask
    // (keys past L, keys after the query when causal) matters only on the workgroup's diagonal
    // tiles and in a ragged last key block: elsewhere one FMA and one exponential per score.
    const bool masked = k0 + 128 > L || (p.causal && tile * 64 < k0 + 128);
    auto p_values = [&](auto mask_tag) __attribute__((always_inline)) {
      constexpr bool kMask = decltype(mask_tag)::value;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int qo = qb * 32 + 16 * hh;  // + 8g (in lofs)
          const f32x4 l0 = lq[qb][hh][0];
          const f32x4 l1 = lq[qb][hh][1];
          u32x4 xo;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            float pv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int j = 2 * t2 + u;
              const float lq = j < 4 ? l0[j] : l1[j - 4];
              const float e2 = fast_exp2(fmaf(xs[qb][hh * 8 + j], c, -lq));
              if constexpr (kMask) {
                const int qq = tile * 64 + qo + 8 * g + j;
                const bool ok = kj < L && (!p.causal || kj <= qq);
                pv[u] = ok ? e2 : 0.0f;
              } else {
                pv[u] = e2;
              }
            }
            xo[t2] = pack_bf16(pv[0], pv[1]);
          }
          pbv[qb][hh] = __builtin_bit_cast(bf16x8, xo);
          *reinterpret_cast<u32x4*>(smem + ((qb * 2 + hh) * 64 * 16 + (int)pofs)) = xo;
        }
    };
    if (masked) p_values(std::true_type{});
    else p_values(std::false_type{});
  };

  // Phase B on stage S: (dS wave) P from LDS and dS; then the transposed products into acc.
  auto phase_b = [&](auto stage_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    auto fetch = [&](int m) -> bf16x8 __attribute__((always_inline)) {
      const int u = m / (D / 32), db = m % (D / 32);
      const int o = S * C::kStageBytes + u * 16 * C::kRowBytes;
      const s16x4 a8[2] = {lds_read_tr16(smem + (o + (int)tofs[0][db])), lds_read_tr16(smem + (o + (int)tofs[1][db]))};
      return __builtin_bit_cast(bf16x8, a8);
    };
    bf16x8 op[kNT];
#pragma unroll
    for (int m = 0; m < kAhead; ++m) op[m] = fetch(m);
    bf16x8 bop[2][2];
    if (pwave) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) bop[qb][hh] = pbv[qb][hh];
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x4 d0 = lq[qb][hh][0];
          const f32x4 d1 = lq[qb][hh][1];
          const u32x4 pin = *reinterpret_cast<const u32x4*>(smem + ((qb * 2 + hh) * 64 * 16 + (int)pofs));
          u32x4 xo;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            const int j0 = 2 * t2, j1 = 2 * t2 + 1;
            const float dq0 = j0 < 4 ? d0[j0] : d1[j0 - 4];
            const float dq1 = j1 < 4 ? d0[j1] : d1[j1 - 4];
            xo[t2] = pack_bf16(bf16_lo(pin[t2]) * (xs[qb][hh * 8 + j0] - dq0),
                               bf16_hi(pin[t2]) * (xs[qb][hh * 8 + j1] - dq1));
          }
          bop[qb][hh] = __builtin_bit_cast(bf16x8, xo);
        }
    }
#pragma unroll
    for (int m = 0; m < kNT; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + kAhead < kNT) op[m + kAhead] = fetch(m + kAhead);
      const int u = m / (D / 32), db = m % (D / 32);
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], bop[u >> 1][u & 1], acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Interval for tile t on stage S: copy tile t + 1 into the other stage, phase A, barrier,
  // phase B, this wave's copies landed, barrier.
  auto interval = [&](auto stage_tag, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    const bool more = t + 1 < tn;
    if (more) issue(t + 1, 1 - S);
    // The P wave runs phase A at raised priority, so its matrix work issues first and its
    // exponentials then overlap the partner's matrix work.
    if (pwave) __builtin_amdgcn_s_setprio(1);
    phase_a(stage_tag, t);
    __builtin_amdgcn_s_setprio(0);
    wg_barrier_lds();
    phase_b(stage_tag);
    if (more) {
      wait_vmcnt<0>();
      publish(1 - S);
    }
    wg_barrier_lds();
  };

  if (t0 < tn) {
    issue(t0, 0);
    wait_vmcnt<0>();
    publish(0);
  }
  __syncthreads();
  for (int t = t0; t < tn; t += 2) {
    interval(std::integral_constant<int, 0>{}, t);
    if (t + 1 >= tn) break;
    interval(std::integral_constant<int, 1>{}, t + 1);
  }
  wait_vmcnt<0>();

  if (kj < p.Nk) {
    uint16_t* outg = static_cast<uint16_t*>(pwave ? p.dv : p.dk) + (size_t)bh * p.Nk * D + (size_t)kj * D;
    const float f = pwave ? 1.0f : p.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const u32x2 x = {pack_bf16(acc[db][4 * jq] * f, acc[db][4 * jq + 1] * f),
                         pack_bf16(acc[db][4 * jq + 2] * f, acc[db][4 * jq + 3] * f)};
        *reinterpret_cast<u32x2*>(outg + db * 32 + 8 * jq + 4 * g) = x;
      }
  }
}

hipError_t launch_backward(const BackwardParams& p, int d, hipStream_t stream) {
  const int64_t bh = (int64_t)p.B * p.H;
  if (bh == 0) return hipSuccess;
  const int64_t rows = bh * p.Nq;
  if (rows > 0) {
    const int per_wg = d == 64 ? BwdDeltaCfg<64>::kRowsPerWg : BwdDeltaCfg<128>::kRowsPerWg;
    const dim3 g0((unsigned)((rows + per_wg - 1) / per_wg));
    if (d == 64) hipLaunchKernelGGL(bwd_delta_kernel<64>, g0, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(bwd_delta_kernel<128>, g0, dim3(256), 0, stream, p);
    const dim3 g1((unsigned)(bh * ((p.Nq + 127) / 128)));
    if (d == 64) hipLaunchKernelGGL(bwd_dq_kernel<64>, g1, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL(bwd_dq_kernel<128>, g1, dim3(512), 0, stream, p);
  }
  if (p.Nk > 0) {
    const dim3 g2((unsigned)(bh * ((p.Nk + 127) / 128)));
    if (d == 64) hipLaunchKernelGGL(bwd_dkdv_kernel<64>, g2, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL(bwd_dkdv_kernel<128>, g2, dim3(512), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
