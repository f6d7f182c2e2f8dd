// fa_prefill_pp.hip -- tiled attention forward for bf16 Q/K/V on gfx950 (MI355X), with the
// matrix work of one wave overlapped against the softmax of its partner wave.
//
// What is computed is the tiled forward pass with an online softmax (page "FlashAttention：把注意
// 力从公式写成数据流", sections "分块与在线 softmax" and "SRAM 预算与 tile 选择"; page
// "FlashAttention 与边缘设备上的注意力内存瓶颈", sections "3.1 Tiling" and "3.2 Online Softmax"):
// each query row keeps a running maximum, a running normaliser and an output accumulator in
// registers while the K/V tiles of its head stream through LDS.
//
// Why two wave groups. On gfx950 a wave that interleaves v_exp_f32 with matrix instructions gets
// no overlap between them, while the exponentials of one wave and the matrix instructions of
// another wave on the same SIMD do overlap. So a workgroup holds 8 waves (2 per SIMD) in two
// groups of 4, and the groups alternate between two kinds of phase, separated by workgroup
// barriers:
//   matrix phase i:  S_i = K_i Q^T (scores of key tile i) and O^T += V_{i-1}^T P_{i-1}^T
//   softmax phase i: P_i = 2^(t - m) as bf16, normaliser update, and (rarely) a new offset m
// Group 1 runs one phase behind group 0, so in every phase each SIMD has one wave on the matrix
// cores and one on the vector ALUs. (This is the scheduling idea the pages credit to FA3 for
// Hopper, page "FlashAttention：把注意力从公式写成数据流", section "FA2 与 FA3", rebuilt with
// workgroup barriers and per-SIMD wave pairs instead of warp specialisation.)
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulation). Each wave owns 32 query rows
// and computes the TRANSPOSED score tile S^T = K Q^T, so every lane holds scores of ONE query
// (lane % 32): the softmax row reductions are in-lane plus one cross-half exchange, the
// probabilities are already the B operand of O^T += V^T P^T, and O^T again has one query per lane.
// K rows are permuted inside each 32-key block (bits 2 and 3 swapped) so that a lane's 16 scores
// of a block are two runs of 8 consecutive keys, the key order the V^T operand wants.
//
// Data movement. A pipeline unit U_i = (K tile i, V tile i-1) is consumed in the two phases
// 2i, 2i+1 of the workgroup timeline. Four LDS slots hold U_i .. U_{i+3}; every wave copies its
// 1/8 share of each unit from HBM straight into LDS (buffer_load_dwordx4 ... lds, no registers,
// range-checked so keys past the workgroup's range read as zeros) about three phases before it
// is needed. V^T operands come from transposing LDS reads (ds_read_b64_tr_b16). Every LDS
// operand address is a per-lane register computed once plus an immediate, so a matrix phase
// issues nothing but LDS reads and MFMAs: a vector instruction in that stream would wait behind
// the partner wave's softmax work and stall the matrix cores.
//
// Lazy offset. The exponent offset m of a row is not the running maximum: it only moves when a
// tile would make the probabilities too large (this lane's half-row sum of p above 2^12) and on
// the first tile with an allowed key. With the offset held, p = 2^(t - m) <= 2^12 never
// overflows, and the usual softmax algebra (O and l both carry the factor 2^-m) is unchanged;
// the row maximum is computed only on the tiles that move m, so most softmax phases are just
// one FMA, one exponential and one addition per score plus the bf16 packing.
#include "fa_device.h"
#include "fa_params.h"
#include "fa_softmax.h"

#include <type_traits>

namespace fa {

// Maximum of the 32 scores a lane holds for its query row, then across the lane pair (l, l^32)
// that holds the row's other keys: 16 three-input maxima and one exchange. Written as asm so the
// compiler adds no NaN-quieting copies of the matrix results in front of each maximum.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float row_max32(const float (&s)[32]) {
  float a[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) a[i] = vmax3(s[3 * i], s[3 * i + 1], s[3 * i + 2]);
  const float c0 = vmax3(a[0], a[1], a[2]), c1 = vmax3(a[3], a[4], a[5]), c2 = vmax3(a[6], a[7], a[8]);
  const float c3 = vmax3(a[9], s[30], s[31]);
  const float x = vmax3(c0, c1, vmax3(c2, c3, c3));
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

template <int D>
struct PrefillPPCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kQW = 32;                  // query rows per wave
  static constexpr int kBM = kWaves * kQW;        // query rows per workgroup
  static constexpr int kBN = 64;                  // keys per K/V tile
  static constexpr int kNch = D / 8;              // 16-byte pieces per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kBN * kRowBytes;
  static constexpr int kUnitBytes = 2 * kTileBytes;  // K tile, then V tile
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kKiBPerWave = kTileBytes / 1024 / kWaves;  // per tensor per tile
  static constexpr int kLoadsPerUnit = 2 * kKiBPerWave;           // per wave
  static_assert(kKiBPerWave * kWaves * 1024 == kTileBytes, "tile must split over the waves");
};


// kGen = false: the fa_fwd masks (causal, key lengths) on [B][H][N][D] tensors. kGen = true:
// sliding windows (left, right) and, with cu_q / cu_k, packed sequences; the loop structure gains
// a masked prefix (tiles that reach below the window of the workgroup's last row) and the
// K/V stream starts at the first tile any row of the workgroup may see.
template <int D, bool kGen>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_pp_kernel(PrefillParams p) {
  using C = PrefillPPCfg<D>;
  __shared__ __attribute__((aligned(1024))) char slot0[C::kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char slot1[C::kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char slot2[C::kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char slot3[C::kUnitBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int grp = w >> 2;                                  // waves w and w + 4 share a SIMD
  // The wave's 32-row block: SIMD s holds blocks s and 7 - s, so on the causal diagonal, where
  // the fully masked 32-key blocks of each wave are skipped, every SIMD keeps the same matrix work
  // (blocks r and 7 - r need r + 1 and 8 - r of the diagonal's eight key blocks).
  const int rblk = grp ? 7 - (w & 3) : (w & 3);
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // Work decomposition: workgroup -> (b, h, query tile); causal tiles heaviest first.
  const int tile = xcd_remap(blockIdx.x, p.n_tiles);
  const int bh = tile / p.n_qtiles;
  int qt = tile - bh * p.n_qtiles;
  const bool right_bounded = kGen ? p.win_right >= 0 : p.causal != 0;
  if (right_bounded) qt = p.n_qtiles - 1 - qt;
  const int b = bh / p.H;
  const int q0 = qt * C::kBM;

  // Sequence geometry: this (b, h)'s query rows [0, Nq) and valid keys [0, L), their base rows.
  int Nq = p.Nq, L;
  const uint16_t *Qg, *Kg, *Vg;
  uint16_t* Og;
  float* lseg;
  if (kGen && p.cu_q) {
    const int h = bh - b * p.H;
    const int qr0 = clampi(p.cu_q[b], 0, p.Tq), qr1 = clampi(p.cu_q[b + 1], qr0, p.Tq);
    const int kr0 = clampi(p.cu_k[b], 0, p.Tk), kr1 = clampi(p.cu_k[b + 1], kr0, p.Tk);
    Nq = qr1 - qr0;
    L = kr1 - kr0;
    const size_t qrow = (size_t)h * p.Tq + qr0, krow = (size_t)h * p.Tk + kr0;
    Qg = static_cast<const uint16_t*>(p.q) + qrow * D;
    Og = static_cast<uint16_t*>(p.o) + qrow * D;
    lseg = p.lse + qrow;
    Kg = static_cast<const uint16_t*>(p.k) + krow * D;
    Vg = static_cast<const uint16_t*>(p.v) + krow * D;
  } else {
    L = seq_len(p.kv_seqlens, b, p.Nk);
    Qg = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Nq * D;
    Og = static_cast<uint16_t*>(p.o) + (size_t)bh * p.Nq * D;
    lseg = p.lse + (size_t)bh * p.Nq;
    Kg = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.Nk * D;
    Vg = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.Nk * D;
  }
  if (kGen && q0 >= Nq) return;  // a query tile past this packed sequence (uniform per workgroup)

  // Key range of the workgroup: tiles i_lo .. n-1 (n exclusive); kend is one past its last key.
  // Without a window i_lo = 0. With one, the stream starts at the first tile any of its rows may
  // see, and the buffer views below start there too, so keys before it are never read.
  int i_lo = 0, kend = L;
  if constexpr (kGen) {
    const int q_last = min(q0 + C::kBM, Nq) - 1;
    if (p.win_left >= 0) i_lo = max(0, q0 - p.win_left) / C::kBN;
    if (p.win_right >= 0) kend = min(kend, q_last + p.win_right + 1);
    kend = max(kend, i_lo * C::kBN);
  } else {
    if (p.causal) kend = min(kend, min(q0 + C::kBM, Nq));
  }
  const int n = kend > 0 ? (kend + C::kBN - 1) / C::kBN : 0;  // key tiles end (exclusive)
  const int kfirst = i_lo * C::kBN;

  // Range-checked views: rows >= Nq of Q and keys outside [kfirst, kend) of K and V read as
  // zeros, so the loads need no branches, masked keys can never bring NaN or Inf into the
  // products, and tiles past this workgroup's last one cost no memory traffic.
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, (uint32_t)Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg + (size_t)kfirst * D, (uint32_t)(kend - kfirst) * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vg + (size_t)kfirst * D, (uint32_t)(kend - kfirst) * C::kRowBytes);

  const int qw0 = q0 + rblk * C::kQW;
  // Scores are handled in base-2 units t = c * (q.k). For c < 0 the kernel negates its copy of Q
  // (a sign flip, exact in bf16 and in every product and sum) and uses -c, so below c > 0 always
  // and the running extreme is always a maximum.
  const bool neg = p.c < 0.0f;
  const float c = neg ? -p.c : p.c;

  // Q rows -> registers, already in the B-operand layout of S^T = K Q^T.
  bf16x8 qreg[D / 16];
  {
    const uint32_t row = (uint32_t)(qw0 + r32);
    const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = buf_load16(qrs, (row * D + ks * 16 + g * 8) * 2);
      x ^= flip;
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
  float m_used = -kInf, lsum = 0.0f;

  // ---- HBM -> LDS. Wave w moves KiB blocks w*kKiBPerWave .. of each tile; in a block, lane i
  // fills LDS row rb + i/kNch, 16-byte slot i%kNch. A K row r holds key key_row_perm(r) with piece
  // (slot ^ kswz(r)); a V row r holds key r with piece (slot ^ vswz(r)). At d = 128 a row fills
  // the 256-byte bank line: kswz(r) = r % 16, vswz(r) = 4 * (r % 4). At d = 64 two rows share a
  // line, and rows of one parity must differ in their pieces: kswz(r) = (r / 2) % 8 for the
  // 16-byte K reads of 16 consecutive rows, vswz(r) = 4 * ((r ^ r / 2) % 2) for the transposed V
  // reads of 4 consecutive rows (the d = 128 forms would put rows r and r + 8, and r and r + 2,
  // on the same banks).
  auto kswz = [](int r) { return (C::kRowBytes >= 256 ? r : r >> 1) % C::kNch; };
  auto vswz = [](int r) { return C::kRowBytes >= 256 ? 4 * (r % (C::kNch / 4)) : 4 * ((r ^ (r >> 1)) & 1); };
  uint32_t koff[C::kKiBPerWave], voff[C::kKiBPerWave];
#pragma unroll
  for (int it = 0; it < C::kKiBPerWave; ++it) {
    const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
    const int slot = lane % C::kNch;
    koff[it] = (uint32_t)(key_row_perm(row) * C::kRowBytes + ((slot ^ kswz(row)) << 4));
    voff[it] = (uint32_t)(row * C::kRowBytes + ((slot ^ vswz(row)) << 4));
  }
  // Unit u = (K tile i_lo + u, V tile i_lo + u - 1), offsets relative to the views' start. V tile
  // i_lo - 1 and K tile n lie outside the buffer range and read as zeros (the unsigned offset of
  // tile -1 wraps far past any valid range).
  auto issue_unit = [&](int u, char* dst) __attribute__((always_inline)) {
    const uint32_t kbase = (uint32_t)u * C::kTileBytes;
    const uint32_t vbase = (uint32_t)(u - 1) * C::kTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKiBPerWave; ++it) {
      char* blk = dst + (w * C::kKiBPerWave + it) * 1024;
      buf_load16_lds(krs, blk, kbase + koff[it]);
      buf_load16_lds(vrs, blk + C::kTileBytes, vbase + voff[it]);
    }
  };

  // ---- LDS -> operands (loop-invariant per-lane byte offsets).
  // K A-operand: lane (r32, g) reads row kb*32 + r32, piece 2*ks + g.
  const int krow_off = r32 * C::kRowBytes;
  const int kx = kswz(r32);
  // V^T A-operand via transposed reads: in 16-lane group grp16 = lane/16 (gp = grp16%2,
  // g = grp16/2), lane 4a+b addresses key (kb*32 + hh*16 + 8*g + 4*t + a), d = db*32 + 16*gp + 4*b.
  const int li = lane & 15;
  const int ta = li >> 2, tb = li & 3;
  const int gp = (lane >> 4) & 1;
  int vt_off[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int piece = db * 4 + 2 * gp + (tb >> 1);
    const int sw = vswz(ta);  // rows 8g + ta (+4): bits 0 and 1 are ta's
    vt_off[db] = (8 * g + ta) * C::kRowBytes + ((piece ^ sw) << 4) + 8 * (tb & 1);
  }
  // Per-lane LDS byte offsets of every operand read, computed once. The immediate offset field of
  // an LDS read holds 16 bits, so for slots 2 and 3 (64 KiB and up when d = 128) each offset has
  // a copy 64 KiB higher that the immediate subtracts again; the empty asm keeps the compiler
  // from folding the copies back, so the matrix phase issues no address arithmetic.
  constexpr int kHi = 4 * C::kUnitBytes > 65536 ? 65536 : 0;
  uint32_t kofs[2][D / 16], vofs[2][D / 32];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kofs[h][ks] = (uint32_t)(h * kHi + krow_off + (((2 * ks + g) ^ kx) << 4));
      asm volatile("" : "+v"(kofs[h][ks]));
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      vofs[h][db] = (uint32_t)(h * kHi + vt_off[db]);
      asm volatile("" : "+v"(vofs[h][db]));
    }
  }

  f32x16 sacc[2];   // S^T of key tile i (two 32-key blocks), then t = c*s - m in place, then p
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[kb][e] = -kInf;
  bf16x8 pk[2][2];  // P^T of the previous key tile as bf16 B operands (zero before tile 0)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) pk[kb][hh] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  constexpr float kSumCap = 4096.0f;  // bound on a lane's half-row sum of p before m moves

  constexpr int kAhead = 4;
  constexpr int kNS = 2 * (D / 16);  // S MFMAs: key block kb = m % 2, d step ks = m / 2
  constexpr int kNP = 4 * (D / 32);  // PV MFMAs: d block db = m % (D/32), key step u = m / (D/32)
  constexpr int kNM = kNS + kNP;

  // Exponent arguments t = c*s - moff of the tile in sacc, written back into sacc. With kMask,
  // keys this lane may not see (key k0 + 8*g + off with off = kb*32 + 16*(e/8) + e%8 allowed iff
  // off < rem; rem counts the allowed keys from k0 + 8*g on: keys < L, keys <= qi when causal,
  // none for rows past Nq) get t = -inf, so their p is exactly 0. Returns whether this lane has
  // an allowed key in the tile.
  auto exponent_args = [&](auto mask_tag, int k0, float moff) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    int rem = 64, lo = 0;  // allowed offsets: lo <= off < rem
    if constexpr (kMask) {
      const int qi = qw0 + r32;
      const int kl = k0 + 8 * g;
      if constexpr (kGen) {
        // Window of row qi: keys max(0, qi - left) .. min(L, qi + right + 1) - 1.
        int hi = L;
        if (p.win_right >= 0) hi = min(hi, qi + p.win_right + 1);
        rem = hi - kl;
        if (p.win_left >= 0) lo = qi - p.win_left - kl;
      } else {
        rem = (p.causal ? min(L, qi + 1) : L) - kl;
      }
      if (qi >= Nq) rem = 0;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float t = fmaf(sacc[kb][e], c, -moff);
        const int off = kb * 32 + ((e >> 3) << 4) + (e & 7);
        if constexpr (kMask && kGen) sacc[kb][e] = (off < rem && off >= lo) ? t : -kInf;
        else if constexpr (kMask) sacc[kb][e] = (off < rem) ? t : -kInf;
        else sacc[kb][e] = t;
      }
    // Whether [lo, rem) meets this lane's offsets 0..55; an over-estimate only costs a rescale.
    return rem > 0 && rem > lo && lo < 56;
  };

  // ---- Matrix phase i: one software-pipelined sequence of kNM MFMAs, S_i = K_i Q^T and then
  // O^T += V_{i-1}^T P_{i-1}^T, whose LDS operand m is read kAhead instructions before the MFMA
  // that consumes it; the V reads start while the last S MFMAs run, so the phase pays the LDS
  // latency once. Nothing else runs in this phase: a wave issues vector instructions slowly on
  // its own, and each one it slots between its MFMAs delays the next MFMA.
  // Every interval runs this same code; the edges are handled by data instead of branches (a
  // branch would make the compiler copy the accumulators at every join): unit 0 carries V tile
  // -1 and unit n carries K tile n, both outside the buffer range and read as zeros; P before
  // tile 0 is zero; and a tile with no allowed key for this wave (tile n, tiles past the wave's
  // causal diagonal, rows past Nq) is fully masked, so its P is exactly zero.
  // With kSkip (the masked intervals of fa_fwd), sb and pb are how many leading 32-key blocks of
  // tile i (S) and of tile i-1 (PV) hold a key allowed for any row of this wave: the products of
  // the blocks past them are left out (their scores are masked, their P is zero), so causal
  // diagonal tiles and the closing interval cost only the matrix work they need. The count is
  // uniform over the wave, so the branches do not diverge.
  auto matrix_phase = [&](auto skip_tag, const char* unit, int hs, int sb, int pb) __attribute__((always_inline)) {
    constexpr bool kSkip = decltype(skip_tag)::value;
    const int h = kHi > 0 ? hs : 0;
    const char* Vs = unit + C::kTileBytes;
    auto fetch = [&](int m) -> bf16x8 __attribute__((always_inline)) {
      if (m < kNS) {
        const int kb = m & 1, ks = m >> 1;
        return *reinterpret_cast<const bf16x8*>(unit + ((kb * 32 * C::kRowBytes - h * kHi) + (int)kofs[h][ks]));
      }
      const int mp = m - kNS;
      const int db = mp % (D / 32), u = mp / (D / 32);
      const char* vrow = Vs + ((u * 16 * C::kRowBytes - h * kHi) + (int)vofs[h][db]);
      const s16x4 a8[2] = {lds_read_tr16(vrow), lds_read_tr16(vrow + 4 * C::kRowBytes)};
      return __builtin_bit_cast(bf16x8, a8);
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
    bf16x8 op[kNM];
#pragma unroll
    for (int m = 0; m < kAhead; ++m) op[m] = fetch(m);
#pragma unroll
    for (int m = 0; m < kNM; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + kAhead < kNM) op[m + kAhead] = fetch(m + kAhead);
      if (m < kNS) {
        if (!kSkip || (m & 1) < sb)
          sacc[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], qreg[m >> 1], sacc[m & 1], 0, 0, 0);
      } else {
        const int mp = m - kNS;
        const int db = mp % (D / 32), u = mp / (D / 32);
        if (!kSkip || (u >> 1) < pb)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], pk[u >> 1][u & 1], oacc[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Keep the softmax work of the other phase from being scheduled into this one.
    asm volatile("" : "+v"(sacc[0]), "+v"(sacc[1]));
  };

  // Keep the exponentials next to the rest of the softmax work (without this the compiler sinks
  // them to their use in the next PV matrix instructions, where this chip serialises them with the
  // wave's MFMAs).
  auto pin_softmax = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(pk[0][0]), "+v"(pk[0][1]), "+v"(pk[1][0]), "+v"(pk[1][1]), "+v"(lsum),
                 "+v"(m_used));
  };
  // ---- Softmax phase for the tile whose scores sit in sacc (key k0 onwards): exponent
  // arguments, p = 2^t, the row sums, the lazy offset update with its rescale of O (after the PV
  // of the previous tile, before the PV of this one), P -> bf16 B operands. Runs at raised wave
  // priority: on a SIMD whose other wave issues matrix instructions, the exponentials otherwise
  // lose most issue cycles to it, and the softmax is the longer of the two phases.
  auto softmax_phase = [&](auto mask_tag, int k0) __attribute__((always_inline)) {
    const float moff = (m_used == -kInf) ? 0.0f : m_used;
    const bool any_key = exponent_args(mask_tag, k0, moff);
    float pr[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) pr[kb * 16 + e] = fast_exp2(sacc[kb][e]);
    float ps = tree_sum(pr);
    // Lazy offset: keep m while this lane's half-row sum of p stays <= kSumCap (then every
    // p <= kSumCap, so nothing overflows); otherwise, and on the row's first tile with an allowed
    // key, move m to the row maximum, redo the exponentials against it and rescale O and l by
    // 2^(m_old - m_new). The decision is wave-wide, so both lanes of a row take the same path.
    if (wave_any(ps > kSumCap || (m_used == -kInf && any_key))) {
      float t[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) t[kb * 16 + e] = sacc[kb][e];
      const float mt = row_max32(t) + moff;  // row maximum of c*s; -inf when the row is masked
      const float mn = fmaxf(m_used, mt);
      const float alpha = (m_used == -kInf) ? 1.0f : fast_exp2(m_used - mn);
      const float shift = ((mn == -kInf) ? 0.0f : mn) - moff;
#pragma unroll
      for (int x = 0; x < 32; ++x) pr[x] = fast_exp2(t[x] - shift);
      ps = tree_sum(pr);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      lsum *= alpha;
      m_used = mn;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 x;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          x[q] = pack_bf16(pr[kb * 16 + hh * 8 + 2 * q], pr[kb * 16 + hh * 8 + 2 * q + 1]);
        pk[kb][hh] = __builtin_bit_cast(bf16x8, x);
      }
    lsum += ps;
    pin_softmax();
  };

  // One barrier interval i per key tile. Every wave issues its share of U_{i+3} into `ahead`, the
  // slot that held U_{i-1} (consumed by both groups before the last barrier), outside its matrix
  // phase. Group 0 runs matrix phase i (S_i, PV_{i-1}) and then the softmax of tile i; group 1
  // runs the softmax of tile i-1 and then matrix phase i. So while a wave of one group works on
  // the vector ALUs, the wave of the other group on its SIMD issues matrix instructions; the
  // softmax runs at wave priority 1, the matrix phase at 0. Before the barrier, this wave's share
  // of U_{i+1} must have landed; U_{i+2} and U_{i+3} may still be in flight (loads get three
  // intervals). hs selects the slot's LDS offset copy; kMask selects the masked softmax (group 1
  // applies it to tile i-1).
  auto set_prio = [&](int pr) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if (pr) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // One past the last key any row of this wave may see (causal diagonal, length, kend), for the
  // block counts of the masked fa_fwd intervals; rows past Nq see none.
  const int wave_kend = qw0 >= Nq ? 0 : min(kend, p.causal ? min(qw0 + C::kQW, Nq) : kend);
  auto blocks_needed = [&](int k0) __attribute__((always_inline)) {
    return clampi((wave_kend - k0 + 31) >> 5, 0, 2);
  };
  auto interval = [&](auto order_tag, auto mask_tag, int t, const char* unit, int hs, char* ahead)
      __attribute__((always_inline)) {
    constexpr bool kMatrixFirst = decltype(order_tag)::value;
    constexpr bool kSkip = !kGen && decltype(mask_tag)::value;
    const int i = i_lo + t;  // key tile of this interval (t counts from the first one)
    const int sb = kSkip ? blocks_needed(i * C::kBN) : 2;
    const int pb = kSkip ? blocks_needed((i - 1) * C::kBN) : 2;
    if constexpr (kMatrixFirst) {
      matrix_phase(std::integral_constant<bool, kSkip>{}, unit, hs, sb, pb);
      issue_unit(t + 3, ahead);
      // Tile n (the closing interval's own) is fully masked: its softmax would add nothing.
      if (!kSkip || i < n) {
        set_prio(1);
        softmax_phase(mask_tag, i * C::kBN);
        set_prio(0);
      }
    } else {
      issue_unit(t + 3, ahead);
      set_prio(1);
      softmax_phase(mask_tag, (i - 1) * C::kBN);
      set_prio(0);
      matrix_phase(std::integral_constant<bool, kSkip>{}, unit, hs, sb, pb);
    }
    wait_vmcnt<2 * C::kLoadsPerUnit>();
    wg_barrier();
  };
  // Loops with a single code path each (a branch per tile would make the compiler copy the
  // accumulators at every join), over t = i - i_lo = 0 .. n - i_lo (interval n - i_lo only
  // completes the last tile; its own tile is fully masked). Tiles i_u0 .. i_u1 - 1 need no mask
  // for any row of the workgroup; the others take the masked variant, a no-op mask on tiles that
  // happen to be whole. Needing a mask: the ragged tail (key k0 + 63 >= L); tiles reaching past
  // the workgroup's first row when causal (k0 + 63 > q0), or past q0 + right with a window; and,
  // with a window's left limit, tiles starting below q_last - left. The loops are unrolled by the
  // slot count (slot = t % 4) so every LDS access names its slot array; the guards of the last
  // loop are nested so that the compiler's wait-count tracking sees only the paths that happen.
  const int t_end = n - i_lo;
  int t_u0 = 0, t_u1;
  if constexpr (kGen) {
    const int q_last = min(q0 + C::kBM, Nq) - 1;
    int hi_min = L;  // every row of the workgroup may see keys below hi_min ...
    if (p.win_right >= 0) hi_min = min(hi_min, q0 + p.win_right + 1);
    int lo_max = 0;  // ... and at or above lo_max
    if (p.win_left >= 0) lo_max = max(0, q_last - p.win_left);
    t_u0 = max(0, (lo_max + C::kBN - 1) / C::kBN - i_lo);
    t_u1 = min(t_end, hi_min / C::kBN - i_lo);
  } else {
    t_u1 = min(n, L / C::kBN);
    if (p.causal) t_u1 = min(t_u1, q0 / C::kBN);
  }
  // Interval t runs group 0's softmax of tile t but group 1's of tile t - 1, so an unmasked
  // interval needs both tiles unmasked: the masked prefix covers t <= t_u0 whenever t_u0 > 0.
  const int t_pre = t_u0 > 0 ? t_u0 + 1 : 0;
  auto run = [&](auto order_tag) __attribute__((always_inline)) {
    int t = 0;
    if constexpr (kGen) {
      for (; t < t_pre && t + 3 <= t_end; t += 4) {
        interval(order_tag, std::true_type{}, t, slot0, 0, slot3);
        interval(order_tag, std::true_type{}, t + 1, slot1, 0, slot0);
        interval(order_tag, std::true_type{}, t + 2, slot2, 1, slot1);
        interval(order_tag, std::true_type{}, t + 3, slot3, 1, slot2);
      }
    }
    for (; t + 4 <= t_u1; t += 4) {
      interval(order_tag, std::false_type{}, t, slot0, 0, slot3);
      interval(order_tag, std::false_type{}, t + 1, slot1, 0, slot0);
      interval(order_tag, std::false_type{}, t + 2, slot2, 1, slot1);
      interval(order_tag, std::false_type{}, t + 3, slot3, 1, slot2);
    }
    for (; t <= t_end; t += 4) {
      interval(order_tag, std::true_type{}, t, slot0, 0, slot3);
      if (t + 1 <= t_end) {
        interval(order_tag, std::true_type{}, t + 1, slot1, 0, slot0);
        if (t + 2 <= t_end) {
          interval(order_tag, std::true_type{}, t + 2, slot2, 1, slot1);
          if (t + 3 <= t_end) interval(order_tag, std::true_type{}, t + 3, slot3, 1, slot2);
        }
      }
    }
  };

  // Prologue: Q and units 0, 1, 2 complete before anyone starts. Units past n (issued by the
  // last intervals) fall outside the buffer range and only write zeros into free slots.
  issue_unit(0, slot0);
  issue_unit(1, slot1);
  issue_unit(2, slot2);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  wg_barrier();
  // Group 1's first exponential phase (of "tile -1") sees t = -inf everywhere: p = 0, no effect.
  // After the last interval group 1 leaves tile n's exponentials undone; that tile is fully
  // masked, so they would add nothing.
  if (grp == 0) run(std::true_type{});
  else run(std::false_type{});
  wait_vmcnt<0>();  // nothing may still write into LDS when the workgroup ends

  // Epilogue: O = O^T / l, lse = ln 2 * (m + log2 l); a row with no allowed key gets 0 and -inf.
  const float lt = pair32_sum(lsum);
  const int qi = qw0 + r32;
  if (qi < Nq) {
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (g == 0) lseg[qi] = lt > 0.0f ? (m_used + fast_log2(lt)) * kLn2 : -kInf;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        // Accumulator entries 4*jq .. 4*jq+3 are d = db*32 + 8*jq + 4*g + 0..3 of row qi.
        u32x2 x = {pack_bf16(oacc[db][4 * jq + 0] * inv, oacc[db][4 * jq + 1] * inv),
                   pack_bf16(oacc[db][4 * jq + 2] * inv, oacc[db][4 * jq + 3] * inv)};
        *reinterpret_cast<u32x2*>(Og + (size_t)qi * D + db * 32 + 8 * jq + 4 * g) = x;
      }
  }
}

template <int D, bool kGen>
static hipError_t launch_pp(PrefillParams p, int max_nq, hipStream_t stream) {
  using C = PrefillPPCfg<D>;
  p.n_qtiles = (max_nq + C::kBM - 1) / C::kBM;
  p.n_tiles = p.B * p.H * p.n_qtiles;
  if (p.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_bf16_pp_kernel<D, kGen>), dim3(p.n_tiles), dim3(C::kThreads), 0, stream, p);
  return hipGetLastError();
}

int prefill_bf16_pp_rows_per_wg() { return PrefillPPCfg<128>::kBM; }

hipError_t launch_prefill_bf16_pp(const PrefillParams& p, int d, hipStream_t stream) {
  if (d == 64) return launch_pp<64, false>(p, p.Nq, stream);
  return launch_pp<128, false>(p, p.Nq, stream);
}

// Sliding windows and packed sequences: max_nq bounds every sequence's query count.
hipError_t launch_prefill_bf16_general(const PrefillParams& p, int d, int max_nq, hipStream_t stream) {
  if (d == 64) return launch_pp<64, true>(p, max_nq, stream);
  return launch_pp<128, true>(p, max_nq, stream);
}

}  // namespace fa
