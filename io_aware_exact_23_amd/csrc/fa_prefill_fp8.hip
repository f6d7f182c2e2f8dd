// fa_prefill_fp8.hip -- tiled attention forward on e4m3 (OCP FP8) Q, K and V^T for gfx950 (MI355X).
//
// Lower precision halves the bytes moved and doubles the matrix-core rate; it needs a scale per
// tensor slice, and FP8 matrix operands want V transposed (page "FlashAttention：把注意力从公式
// 写成数据流", sections "用实验验证而不是背诵结论" and "精度、掩码和边界情况"; FA3's use of
// low-precision units, section "FA2 与 FA3"). The method is the same tiled forward with an online
// softmax as the bf16 path (same page, section "分块与在线 softmax"), on inputs quantised by
// fa_quantize_fp8: Q and K as [B][H][N][D] e4m3 codes, V as V^T [B][H][D][ldv] (ldv = Nk rounded
// up to 64), with one fp32 scale per (b, h) slice of each.
//
// Structure: the 8-wave workgroup of the bf16 long-sequence kernel (two groups of four waves, one
// group in its matrix phase while the other runs its softmax, one barrier per 64-key tile, four
// LDS slots fed by direct HBM -> LDS copies), with v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x fp8,
// unit scales, fp32 accumulation) for both products:
//   S^T = K Q^T  per 32-key block: D/64 instructions, A = K rows from LDS, B = Q in registers;
//   O^T += V^T P^T per 32-d block: one instruction over the tile's 64 keys, A = V^T rows from
//   LDS (no transposing reads: V arrives transposed), B = P^T from the score accumulators.
// Operand layout: lane (r32, g) holds 32 bytes, byte j standing for reduction index 32g + j of
// the instruction (A rows / B columns r32). The S^T accumulator entry e of lane (r32, g) in key
// block kb is the score of query r32 against LDS K row 32kb + 8(e/4) + 4g + e%4; that row holds
// key 32g + 16kb + e of the tile, so the lane's 32 scores are exactly the keys 32g .. 32g+31 its
// P^T operand must hold, in byte order, and the V^T operand reads keys 32g .. 32g+31 of a row.
//
// Probabilities in e4m3. p = 2^(t - m) scaled by 8 is rounded to e4m3 for the P V product; the
// normaliser l sums the unrounded values. The lazy offset m of the bf16 kernel is kept with a cap
// that fits the format: m moves when a lane's sum of its 32 scaled values exceeds 448 (so every
// value is <= 448, the largest e4m3 magnitude), and on the row's first tile with an allowed key;
// with m at the row maximum the scaled values are <= 8 and sum to <= 256, so the cap never fires
// without a new maximum. The scale 8 keeps values down to 2^-9 of the maximum in e4m3's normal
// range.
#include "fa_device.h"
#include "fa_params.h"

#include <type_traits>

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int D>
struct PrefillFp8Cfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kQW = 32;                   // query rows per wave
  static constexpr int kBM = kWaves * kQW;         // query rows per workgroup
  static constexpr int kBN = 64;                   // keys per tile
  static constexpr int kTileBytes = kBN * D;       // K tile [64][D], V^T tile [D][64]
  static constexpr int kUnitBytes = 2 * kTileBytes;
  static constexpr int kKiB = kUnitBytes / 1024;   // KiB blocks per unit
  static constexpr int kLoadsPerUnit = kKiB / kWaves;
  static constexpr int kKSteps = D / 64;           // S instructions per 32-key block
  static constexpr int kDB = D / 32;               // PV instructions per tile
  static_assert(kLoadsPerUnit * kWaves == kKiB, "unit must split over the waves");
};

// 16-byte piece swizzles, chosen so that 8 consecutive rows (a 128-byte bank window) and 16
// consecutive rows (256 bytes) read by ds_read_b128 at the same logical piece hit distinct banks.
// 128-byte rows (K at D = 128): piece ^ f8(r); 64-byte rows (V^T, K at D = 64): piece ^ f4(r).
__device__ __forceinline__ int fp8_f8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int fp8_f4(int r) { return ((((r >> 1) ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1); }
template <int D>
__device__ __forceinline__ int fp8_kswz(int r) { return D == 128 ? fp8_f8(r) : fp8_f4(r); }

// Key of the tile held by LDS K row rho = 32 kb + 8 a + 4 g + b: 32 g + 16 kb + 4 a + b.
__device__ __forceinline__ int fp8_k_key(int rho) {
  const int kb = rho >> 5, a = (rho >> 3) & 3, g = (rho >> 2) & 1, b = rho & 3;
  return 32 * g + 16 * kb + 4 * a + b;
}


__device__ __forceinline__ float fp8_vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Maximum of a lane's 32 values, then across the lane pair (l, l ^ 32) that holds the row's other keys.
__device__ __forceinline__ float fp8_row_max32(const float (&s)[32]) {
  float a[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) a[i] = fp8_vmax3(s[3 * i], s[3 * i + 1], s[3 * i + 2]);
  const float c0 = fp8_vmax3(a[0], a[1], a[2]), c1 = fp8_vmax3(a[3], a[4], a[5]);
  const float c2 = fp8_vmax3(a[6], a[7], a[8]), c3 = fp8_vmax3(a[9], s[30], s[31]);
  const float x = fp8_vmax3(c0, c1, fp8_vmax3(c2, c3, c3));
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fp8_vmax3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fp8_tree_sum32(const float (&x)[32]) {
  float a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  return a[0];
}

__device__ __forceinline__ f32x16 fp8_mfma(i32x8 a, i32x8 b, f32x16 c) {
  // Formats 0/0: e4m3 x e4m3; scale exponents 127: both operand scales are 1.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void prefill_fp8_kernel(PrefillFp8Params p) {
  using C = PrefillFp8Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char slot0[C::kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char slot1[C::kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char slot2[C::kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char slot3[C::kUnitBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;                    // waves w and w + 4 share a SIMD
  const int rblk = 2 * (w & 3) + grp;        // the wave's 32-row block
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, p.n_tiles);
  const int bh = tile / p.n_qtiles;
  int qt = tile - bh * p.n_qtiles;
  if (p.causal) qt = p.n_qtiles - 1 - qt;    // heaviest causal tiles first
  const int b = bh / p.H;
  const int q0 = qt * C::kBM;
  const int Nq = p.Nq;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  int kend = L;
  if (p.causal) kend = min(kend, min(q0 + C::kBM, Nq));
  const int n = kend > 0 ? (kend + C::kBN - 1) / C::kBN : 0;

  const uint8_t* Qg = p.q + (size_t)bh * Nq * D;
  const uint8_t* Kg = p.k + (size_t)bh * p.Nk * D;
  const uint8_t* Vg = p.vt + (size_t)bh * D * p.ldv;
  uint16_t* Og = static_cast<uint16_t*>(p.o) + (size_t)bh * Nq * D;
  float* lseg = p.lse + (size_t)bh * Nq;
  // Rows >= Nq of Q and keys >= kend of K read as zeros. V^T is read within its slice only; the
  // columns a tile reads past kend are the slice's own (finite) codes or zero padding, weighted 0.
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, (uint32_t)Nq * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, (uint32_t)kend * D);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vg, (uint32_t)D * p.ldv);

  // Scores in base-2 units t = c * (q8 . k8) with c = scale * log2(e) * s_q * s_k; for c < 0 the
  // kernel flips the sign bits of its copy of Q and uses -c.
  const float sq = p.dq ? p.dq[bh] : 1.0f, sk = p.dk ? p.dk[bh] : 1.0f, sv = p.dv ? p.dv[bh] : 1.0f;
  float c_all = p.c * sq * sk;
  if (c_all == 0.0f) c_all = 1e-30f;
  const bool neg = c_all < 0.0f;
  const float c = neg ? -c_all : c_all;

  const int qw0 = q0 + rblk * C::kQW;
  // Q -> B operands of S^T: lane (r32, g) holds Q[row][64 ks + 32 g .. +31].
  i32x8 qreg[C::kKSteps];
  {
    const uint32_t row = (uint32_t)(qw0 + r32);
    const uint32_t flip = neg ? 0x80808080u : 0u;
#pragma unroll
    for (int ks = 0; ks < C::kKSteps; ++ks) {
      const u32x4 lo = buf_load16(qrs, row * D + ks * 64 + g * 32);
      const u32x4 hi = buf_load16(qrs, row * D + ks * 64 + g * 32 + 16);
      qreg[ks] = i32x8{(int)(lo[0] ^ flip), (int)(lo[1] ^ flip), (int)(lo[2] ^ flip), (int)(lo[3] ^ flip),
                       (int)(hi[0] ^ flip), (int)(hi[1] ^ flip), (int)(hi[2] ^ flip), (int)(hi[3] ^ flip)};
    }
  }

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
  float m_used = -kInf, lsum = 0.0f;

  // ---- HBM -> LDS. Unit u = (K tile u, V^T tile u - 1) fills one slot: K rows [64][D] then V^T
  // rows [D][64]. The unit's KiB blocks are spread over the waves: wave w moves blocks w + 8 j.
  // A K block holds 1024 / D rows, a V^T block 16 rows; lane i fills 16-byte piece i of its block.
  uint32_t goff[C::kLoadsPerUnit];
  bool isk[C::kLoadsPerUnit];
#pragma unroll
  for (int j = 0; j < C::kLoadsPerUnit; ++j) {
    const int blk = w + 8 * j;
    const int kblocks = C::kTileBytes / 1024;
    isk[j] = blk < kblocks;
    if (isk[j]) {
      const int rho = blk * (1024 / D) + lane / (D / 16);
      const int sl = lane % (D / 16);
      goff[j] = (uint32_t)(fp8_k_key(rho) * D + ((sl ^ fp8_kswz<D>(rho)) << 4));
    } else {
      const int d = (blk - kblocks) * 16 + lane / 4;
      const int sl = lane % 4;
      goff[j] = (uint32_t)(d * p.ldv + ((sl ^ fp8_f4(d)) << 4));
    }
  }
  auto issue_unit = [&](int u, char* dst) __attribute__((always_inline)) {
    const uint32_t kbase = (uint32_t)u * C::kTileBytes;
    // V^T tile u - 1 starts 64 (u - 1) bytes into each row; tile -1 is placed out of range.
    const uint32_t vbase = u > 0 ? (uint32_t)(u - 1) * C::kBN : 0x80000000u;
#pragma unroll
    for (int j = 0; j < C::kLoadsPerUnit; ++j) {
      char* blkp = dst + (w + 8 * j) * 1024;
      if (isk[j]) buf_load16_lds(krs, blkp, kbase + goff[j]);
      else buf_load16_lds(vrs, blkp, vbase + goff[j]);
    }
  };

  // ---- LDS -> operands: per-lane byte offsets, computed once (the empty asm keeps them in
  // registers so a matrix phase issues only LDS reads and MFMAs).
  uint32_t kofs[C::kKSteps][2], vofs[2];
#pragma unroll
  for (int ks = 0; ks < C::kKSteps; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kofs[ks][h] = (uint32_t)(r32 * D + (((4 * ks + 2 * g + h) ^ fp8_kswz<D>(r32)) << 4));
      asm volatile("" : "+v"(kofs[ks][h]));
    }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    vofs[h] = (uint32_t)(C::kTileBytes + r32 * 64 + (((2 * g + h) ^ fp8_f4(r32)) << 4));
    asm volatile("" : "+v"(vofs[h]));
  }

  f32x16 sacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[kb][e] = -kInf;
  i32x8 pk = i32x8{0, 0, 0, 0, 0, 0, 0, 0};  // P^T of the previous tile (zero before tile 0)
  constexpr float kCap = 448.0f;              // bound on a lane's sum of its 32 scaled values
  constexpr float kLogSigma = 3.0f;           // probabilities enter e4m3 scaled by 2^3

  constexpr int kNS = 2 * C::kKSteps;         // S instructions: block kb = m % 2, step ks = m / 2
  constexpr int kNM = kNS + C::kDB;           // then one PV instruction per 32-d block
  constexpr int kAhead = kNM > 4 ? 3 : 2;

  // Exponent arguments t = c*s - moff of the tile in sacc, in place; masked keys get -inf.
  // Lane (r32, g) holds keys k0 + 32 g + 16 kb + e.
  auto exponent_args = [&](auto mask_tag, int k0, float moff) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    int rem = 32;
    if constexpr (kMask) {
      const int qi = qw0 + r32;
      rem = (p.causal ? min(L, qi + 1) : L) - (k0 + 32 * g);
      if (qi >= Nq) rem = 0;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float t = fmaf(sacc[kb][e], c, -moff);
        if constexpr (kMask) sacc[kb][e] = (16 * kb + e < rem) ? t : -kInf;
        else sacc[kb][e] = t;
      }
    return rem > 0;
  };

  auto fetch = [&](const char* unit, int m) -> i32x8 __attribute__((always_inline)) {
    const char* a;
    const char* bq;
    if (m < kNS) {
      const int kb = m & 1, ks = m >> 1;
      a = unit + (kb * 32 * D + (int)kofs[ks][0]);
      bq = unit + (kb * 32 * D + (int)kofs[ks][1]);
    } else {
      const int db = m - kNS;
      a = unit + (db * 32 * 64 + (int)vofs[0]);
      bq = unit + (db * 32 * 64 + (int)vofs[1]);
    }
    const u32x4 lo = *reinterpret_cast<const u32x4*>(a);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(bq);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  // Matrix phase: S_i = K_i Q^T (both key blocks), then O^T += V_{i-1}^T P_{i-1}^T, each LDS
  // operand read kAhead instructions before its MFMA. Edges are handled by data: unit 0 carries
  // V^T tile -1 (out of range, zeros) and P before tile 0 is zero; K tile n reads as zeros.
  auto matrix_phase = [&](const char* unit) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
    i32x8 op[kNM];
#pragma unroll
    for (int m = 0; m < kAhead; ++m) op[m] = fetch(unit, m);
#pragma unroll
    for (int m = 0; m < kNM; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + kAhead < kNM) op[m + kAhead] = fetch(unit, m + kAhead);
      if (m < kNS) sacc[m & 1] = fp8_mfma(op[m], qreg[m >> 1], sacc[m & 1]);
      else oacc[m - kNS] = fp8_mfma(op[m], pk, oacc[m - kNS]);
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(sacc[0]), "+v"(sacc[1]));
  };

  auto pin_softmax = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(pk), "+v"(lsum), "+v"(m_used));
  };
  // Softmax phase of the tile in sacc (keys from k0): scaled probabilities 2^(t - m + 3), the
  // lazy offset update with the rescale of O and l, P^T -> e4m3 operand, l += sum.
  auto softmax_phase = [&](auto mask_tag, int k0) __attribute__((always_inline)) {
    const float moff = (m_used == -kInf) ? 0.0f : m_used;
    const bool any_key = exponent_args(mask_tag, k0, moff - kLogSigma);
    float pr[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) pr[kb * 16 + e] = fast_exp2(sacc[kb][e]);
    float ps = fp8_tree_sum32(pr);
    if (wave_any(ps > kCap || (m_used == -kInf && any_key))) {
      float t[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) t[kb * 16 + e] = sacc[kb][e];
      const float mt = fp8_row_max32(t) + (moff - kLogSigma);  // row maximum of c*s
      const float mn = fmaxf(m_used, mt);
      const float alpha = (m_used == -kInf) ? 1.0f : fast_exp2(m_used - mn);
      const float shift = ((mn == -kInf) ? 0.0f : mn) - moff;
#pragma unroll
      for (int x = 0; x < 32; ++x) pr[x] = fast_exp2(t[x] - shift);
      ps = fp8_tree_sum32(pr);
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      lsum *= alpha;
      m_used = mn;
    }
    // Byte j = 16 kb + e of the operand is key 32 g + j: dword i holds values 4i .. 4i+3.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // The low half first; the old dword only fills the high half the next convert overwrites.
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(pr[4 * i], pr[4 * i + 1], pk[i], false);
      pk[i] = __builtin_amdgcn_cvt_pk_fp8_f32(pr[4 * i + 2], pr[4 * i + 3], x, true);
    }
    lsum += ps;
    pin_softmax();
  };

  auto set_prio = [&](int pr) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if (pr) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Interval i: issue U_{i+3} into the slot freed at the last barrier; group 0 runs matrix phase
  // i then the softmax of tile i, group 1 the softmax of tile i-1 then matrix phase i; U_{i+1}
  // must have landed before the barrier.
  auto interval = [&](auto order_tag, auto mask_tag, int i, const char* unit, char* ahead)
      __attribute__((always_inline)) {
    constexpr bool kMatrixFirst = decltype(order_tag)::value;
    if constexpr (kMatrixFirst) {
      matrix_phase(unit);
      issue_unit(i + 3, ahead);
      set_prio(1);
      softmax_phase(mask_tag, i * C::kBN);
      set_prio(0);
    } else {
      issue_unit(i + 3, ahead);
      set_prio(1);
      softmax_phase(mask_tag, (i - 1) * C::kBN);
      set_prio(0);
      matrix_phase(unit);
    }
    wait_vmcnt<2 * C::kLoadsPerUnit>();
    wg_barrier();
  };
  // Tiles below i_u1 need no mask for any row of the workgroup (whole, and below q0 when causal);
  // interval n only completes tile n - 1 (its own tile is fully masked).
  int i_u1 = min(n, L / C::kBN);
  if (p.causal) i_u1 = min(i_u1, q0 / C::kBN);
  auto run = [&](auto order_tag) __attribute__((always_inline)) {
    int i = 0;
    for (; i + 4 <= i_u1; i += 4) {
      interval(order_tag, std::false_type{}, i, slot0, slot3);
      interval(order_tag, std::false_type{}, i + 1, slot1, slot0);
      interval(order_tag, std::false_type{}, i + 2, slot2, slot1);
      interval(order_tag, std::false_type{}, i + 3, slot3, slot2);
    }
    for (; i <= n; i += 4) {
      interval(order_tag, std::true_type{}, i, slot0, slot3);
      if (i + 1 <= n) {
        interval(order_tag, std::true_type{}, i + 1, slot1, slot0);
        if (i + 2 <= n) {
          interval(order_tag, std::true_type{}, i + 2, slot2, slot1);
          if (i + 3 <= n) interval(order_tag, std::true_type{}, i + 3, slot3, slot2);
        }
      }
    }
  };

  issue_unit(0, slot0);
  issue_unit(1, slot1);
  issue_unit(2, slot2);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  wg_barrier();
  if (grp == 0) run(std::true_type{});
  else run(std::false_type{});
  wait_vmcnt<0>();

  // O = s_v * O^T / l, lse = ln 2 * (m + log2(l) - 3); a row with no allowed key gets 0 and -inf.
  const float lt = pair32_sum(lsum);
  const int qi = qw0 + r32;
  if (qi < Nq) {
    const float inv = lt > 0.0f ? sv / lt : 0.0f;
    if (g == 0) lseg[qi] = lt > 0.0f ? (m_used + fast_log2(lt) - kLogSigma) * kLn2 : -kInf;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        u32x2 x = {pack_bf16(oacc[db][4 * jq + 0] * inv, oacc[db][4 * jq + 1] * inv),
                   pack_bf16(oacc[db][4 * jq + 2] * inv, oacc[db][4 * jq + 3] * inv)};
        *reinterpret_cast<u32x2*>(Og + (size_t)qi * D + db * 32 + 8 * jq + 4 * g) = x;
      }
  }
}

int prefill_fp8_rows_per_wg() { return PrefillFp8Cfg<128>::kBM; }

template <int D>
static hipError_t launch_fp8(PrefillFp8Params p, hipStream_t stream) {
  using C = PrefillFp8Cfg<D>;
  p.n_qtiles = (p.Nq + C::kBM - 1) / C::kBM;
  p.n_tiles = p.B * p.H * p.n_qtiles;
  if (p.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_fp8_kernel<D>, dim3(p.n_tiles), dim3(C::kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill_fp8(const PrefillFp8Params& p, int d, hipStream_t stream) {
  if (d == 64) return launch_fp8<64>(p, stream);
  return launch_fp8<128>(p, stream);
}

}  // namespace fa
