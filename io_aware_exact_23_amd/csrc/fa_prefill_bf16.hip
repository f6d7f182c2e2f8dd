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
// index swapped) so that each lane's 16 scores are two runs of 8 consecutive keys, which is
// exactly the key order the V^T operand wants.
//
// Data movement. K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds), with
// no registers and no ALU work on the way; the buffer's range check turns keys past the
// sequence length into zeros. Both tiles keep their natural row layout, with the 16-byte pieces
// of each row XOR-swizzled against LDS bank conflicts; the V^T operand is read back transposed
// with ds_read_b64_tr_b16. Two LDS stages, one per static array, so the compiler can see that the
// loads into one stage never alias the reads of the other: tile j + 1 streams in while tile j is
// consumed.
#include "fa_device.h"
#include "fa_params.h"
#include "fa_softmax.h"

#include <type_traits>

namespace fa {

template <int D, int NQB>
struct PrefillBf16Cfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kQW = 32 * NQB;            // query rows per wave
  static constexpr int kBM = kWaves * kQW;        // query rows per workgroup
  static constexpr int kBN = 64;                  // keys per K/V tile
  static constexpr int kNch = D / 8;              // 16-byte pieces per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kBN * kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;  // K tile, then V tile
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kKiBPerWave = kTileBytes / 1024 / kWaves;  // per tensor per tile
  static_assert(kKiBPerWave * kWaves * 1024 == kTileBytes, "tile must split over the waves");
};


// WPE waves per SIMD, i.e. WPE workgroups per CU. At d = 64 a wave needs about 150 VGPRs and a
// workgroup 32 KB of LDS, so three fit: with one wave per workgroup on each SIMD, the matrix work
// of one wave can then run under the softmax of the others, which the kernel itself does not
// arrange (13-16% faster than two on the GPT-2- and BERT-shaped workloads). d = 128 needs about
// 250 VGPRs and keeps two.
template <int D, int NQB, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WPE, WPE)))
void prefill_bf16_kernel(PrefillParams p) {
  using C = PrefillBf16Cfg<D, NQB>;
  __shared__ __attribute__((aligned(1024))) char stage_a[C::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char stage_b[C::kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // Work decomposition: workgroup -> (b, h, query tile). Causal: tiles of similar total weight
  // share a CU (serpentine order), or else heaviest first within a head. Key lengths without a
  // causal mask: longest sequences first, so the workgroups that run after the first resident
  // wave of them are the lightest. Otherwise tiles that share K/V share an XCD.
  int bh, qt;
  const bool placed = p.causal
      ? causal_serpentine(blockIdx.x, p.n_tiles, p.n_qtiles, p.cus_per_xcd, bh, qt)
      : longest_first(blockIdx.x, p.kv_seqlens, p.B, p.H, p.n_qtiles, p.Nk, bh, qt);
  if (!placed) {
    const int tile = xcd_remap(blockIdx.x, p.n_tiles);
    bh = tile / p.n_qtiles;
    qt = tile - bh * p.n_qtiles;
    if (p.causal) qt = p.n_qtiles - 1 - qt;
  }
  const int b = bh / p.H;
  const int q0 = qt * C::kBM;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  int kend = L;
  if (p.causal) kend = min(kend, min(q0 + C::kBM, p.Nq));
  const int ntiles = kend > 0 ? (kend + C::kBN - 1) / C::kBN : 0;

  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Nq * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.Nk * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.Nk * D;
  // Range-checked views: rows >= Nq of Q and keys >= L of K and V read as zeros, so the loads
  // need no branches and masked keys can never bring NaN or Inf into the products.
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, (uint32_t)L * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vg, (uint32_t)L * C::kRowBytes);

  const int qw0 = q0 + w * C::kQW;
  const int qw_last = min(qw0 + C::kQW, p.Nq) - 1;  // < qw0 when the wave has no rows
  // Scores are handled in base-2 units t = c * (q.k). For c < 0 the kernel negates its copy of Q
  // (a sign flip, exact in bf16 and in every product and sum) and uses -c, so below c > 0.
  const bool neg = p.c < 0.0f;
  const float c = neg ? -p.c : p.c;

  // Q tile -> registers, already in the B-operand layout of S^T = K Q^T.
  bf16x8 qreg[NQB][D / 16];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const uint32_t row = (uint32_t)(qw0 + qb * 32 + r32);
    const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = buf_load16(qrs, (row * D + ks * 16 + g * 8) * 2);
      x ^= flip;
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

  // ---- HBM -> LDS. Wave w moves KiB blocks w*kKiBPerWave .. of each tile; in a block, lane i
  // fills LDS row rb + i/kNch, 16-byte slot i%kNch. A K row r holds key key_row_perm(r) with piece
  // (slot ^ kswz(r)); a V row r holds key r with piece (slot ^ vswz(r)). Both spread what one pass
  // of a read serves over all 64 banks. At d = 128 a row fills the 256-byte bank line: kswz(r) =
  // r % 16, vswz(r) = 4 * (r % 4). At d = 64 two rows share a line, so rows of one parity must
  // differ in their pieces: kswz(r) = (r / 2) % 8 (16-byte K reads of 16 consecutive rows), and
  // vswz(r) = 4 * ((r ^ r / 2) % 2) (transposed V reads of 4 consecutive rows, two adjacent pieces
  // each). The plain r % 8 and 4 * (r % 2) put rows r and r + 8 (K) and r and r + 2 (V) on the
  // same banks, which the conflict counter showed as one conflict cycle per LDS cycle.
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
  auto issue = [&](int j, char* stage) {
    const uint32_t base = (uint32_t)j * C::kTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKiBPerWave; ++it) {
      char* blk = stage + (w * C::kKiBPerWave + it) * 1024;
      buf_load16_lds(krs, blk, base + koff[it]);
      buf_load16_lds(vrs, blk + C::kTileBytes, base + voff[it]);
    }
  };

  // ---- LDS -> operands (loop-invariant per-lane byte offsets).
  // K A-operand: lane (r32, g) reads row kb*32 + r32, piece 2*ks + g.
  const int krow_off = r32 * C::kRowBytes;
  const int kx = kswz(r32);
  // V^T A-operand via transposed reads: in 16-lane group grp = lane/16 (gp = grp%2, g = grp/2),
  // lane 4a+b addresses key (kb*32 + hh*16 + 8*g + 4*t + a), d = db*32 + 16*gp + 4*b.
  const int li = lane & 15;
  const int ta = li >> 2, tb = li & 3;
  const int gp = (lane >> 4) & 1;
  int vt_off[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int piece = db * 4 + 2 * gp + (tb >> 1);
    const int sw = vswz(ta);  // row 8g + ta, and 4 rows on: bits 0 and 1 of the row are ta's
    vt_off[db] = (8 * g + ta) * C::kRowBytes + ((piece ^ sw) << 4) + 8 * (tb & 1);
  }

  // One K/V tile for this wave: scores, online softmax, output update. kMask selects the
  // variant with per-element masks (tail tile, tiles crossing the wave's diagonal).
  auto tile_step = [&](auto mask_tag, const char* stage, int k0) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const char* Ks = stage;
    const char* Vs = stage + C::kTileBytes;

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
      const char* krow = Ks + kb * 32 * C::kRowBytes + krow_off;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((2 * ks + g) ^ kx) << 4));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], sacc[qb][kb], 0, 0, 0);
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pk[NQB][2][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qi = qw0 + qb * 32 + r32;
      float s[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb * 16 + i] = sacc[qb][kb][i];
      // Score s[kb*16 + i] belongs to key k0 + 8*g + off(x) with the compile-time offset
      // off(x) = kb*32 + 16*(i/8) + i%8; it is allowed iff off(x) < rem, where rem is this lane's
      // count of allowed keys from k0 + 8*g on (keys < L, and keys <= qi when causal).
      const int rem = (p.causal ? min(L, qi + 1) : L) - (k0 + 8 * g);
      auto valid = [&](int x) {
        const int kb = x >> 4, i = x & 15;
        return kb * 32 + ((i >> 3) << 4) + (i & 7) < rem;
      };
      // The raw scores of block qb again, from the K tile still in this stage (the softmax
      // needs them only when it moves the offset after the row's first tile, which is rare).
      auto recompute = [&](float (&x)[32]) __attribute__((always_inline)) {
        f32x16 r[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) r[kb][i] = 0.0f;
          const char* krow = Ks + kb * 32 * C::kRowBytes + krow_off;
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((2 * ks + g) ^ kx) << 4));
            r[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], r[kb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) x[kb * 16 + i] = r[kb][i];
      };
      bool rescaled;
      const float alpha = softmax_tile_lazy<32, kMask>(s, valid, c, m_used[qb], lsum[qb], rescaled, recompute);
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

    __builtin_amdgcn_sched_barrier(0);
    // O^T[d][query] += V^T[d][keys] * P^T[keys][query], 16 keys per instruction; the 8 keys of
    // a lane's operand come from two transposed reads of 4 keys each.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* vrow = Vs + (kb * 32 + hh * 16) * C::kRowBytes;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const s16x4 lo = lds_read_tr16(vrow + vt_off[db]);
          const s16x4 hi = lds_read_tr16(vrow + 4 * C::kRowBytes + vt_off[db]);
          const s16x4 a8[2] = {lo, hi};
          const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[qb][kb][hh], oacc[qb][db], 0, 0, 0);
        }
      }
  };

  // One iteration: start the next tile's loads into the other stage (free since the barrier
  // that ended the previous iteration), consume this stage, then wait for the loads and meet.
  auto iteration = [&](int j, const char* cur, char* nxt) {
    if (j + 1 < ntiles) issue(j + 1, nxt);
    const int k0 = j * C::kBN;
    const bool active = (qw_last >= qw0) && (!p.causal || k0 <= qw_last);
    if (active) {
      // Masks are needed only on the tail tile and on tiles that cross this wave's diagonal.
      const bool need_mask = (k0 + C::kBN > L) || (p.causal && k0 + C::kBN - 1 > qw0);
      if (need_mask) tile_step(std::true_type{}, cur, k0);
      else tile_step(std::false_type{}, cur, k0);
    }
    wait_vmcnt<0>();  // this wave's loads have landed in LDS
    __syncthreads();
  };

  // The Q loads must complete before the loop: the vector-memory counter is in order, so a Q load
  // still pending inside the loop would make every wait for it also wait for the next tile's
  // loads. The first tile's loads go out right behind them and one wait covers both, so a
  // workgroup pays one memory latency before its first tile, not two. The scheduling barriers
  // keep the compiler from moving the loads across the wait.
  __builtin_amdgcn_sched_barrier(0);
  if (ntiles > 0) issue(0, stage_a);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();  // Q and tile 0
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    iteration(j, stage_a, stage_b);
    if (j + 1 < ntiles) iteration(j + 1, stage_b, stage_a);
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

template <int D, int NQB, int WPE>
static hipError_t launch_bf16(PrefillParams p, hipStream_t stream) {
  using C = PrefillBf16Cfg<D, NQB>;
  p.n_qtiles = (p.Nq + C::kBM - 1) / C::kBM;
  p.n_tiles = p.B * p.H * p.n_qtiles;
  if (p.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NQB, WPE>), dim3(p.n_tiles), dim3(C::kThreads), 0, stream, p);
  return hipGetLastError();
}

// Rows per workgroup used for a given head dimension (the host checks grid limits with it).
int prefill_bf16_rows_per_wg(int d) { return d == 64 ? PrefillBf16Cfg<64, 1>::kBM : PrefillBf16Cfg<128, 1>::kBM; }

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream) {
  if (d == 64) return launch_bf16<64, 1, 3>(p, stream);
  return launch_bf16<128, 1, 2>(p, stream);
}

}  // namespace fa
