// fa_standard.hip -- standard (materialising) attention for bf16 Q/K/V on gfx950 (MI355X): the
// baseline that the tiled kernels are measured against.
//
// The pages describe the naive algorithm as three passes over device memory: S = Q K^T is
// written out in full, read back for the softmax, and P is written and read again for P V (page
// "FlashAttention：把注意力从公式写成数据流", opening paragraph and section "用 IO 复杂度重写直觉";
// page "FlashAttention 与边缘设备上的注意力内存瓶颈", section "2 标准 attention 的问题"). The speedup
// of the tiled method over it is the pages' headline measurement (page "[2205.14135]
// FlashAttention ...", section "一、HBM 記憶體頻寬：速度差異的主要來源"). These kernels are that
// algorithm, each pass written for this chip:
//   std_scores_kernel   S = scale * Q K^T over the full Nq x Nk grid, fp32, on MFMA, 256 x 256
//                       blocks with the K block shared through LDS (d is only 64 or 128, so each
//                       S element costs 4 bytes written against 2d FLOPs: the pass is write-bound);
//   std_softmax_kernel  rows held in registers (one wave per row up to 2048 keys, four up to
//                       16384, a two-read kernel beyond): masked max and sum, then
//                       P = exp(S - m) / l as bf16 over the whole row (zeros where masked), and
//                       lse = m + ln l;
//   std_pv_kernel       O = P V over all Nk keys, P rows straight from memory as the A operand,
//                       V tiles through LDS and read back transposed as the B operand.
// S is kept in fp32 so that the baseline's results meet the same tolerances as the tiled
// kernels (bf16 scores would add a rounding of up to 2^-9 * |s| to every logit); P is bf16,
// as the tiled kernels round it before P V. Masking is applied in the softmax, as in the naive
// algorithm, but key rows at or past the sequence length are never read: the loads are
// range-checked and return zeros there.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {

// ---- Pass 1: S = scale * Q K^T. One workgroup of 4 waves per 256 x 256 block of S. The block's
// 256 K rows are copied once into LDS (straight from memory, 16-byte pieces XOR-swizzled by row
// against bank conflicts); wave w computes query rows 64w .. 64w+63 (two 32-row blocks) against
// all 256 keys, 32 keys at a time, and writes each of its rows 1 KB back to back. K is thus read
// from L2 once per 256 query rows (D*2 / (256*4) bytes per byte of S written), and the pass is
// left with what the algorithm asks of it: writing S.
constexpr int kStdRows = 256, kStdKeys = 256;
template <int D>
__global__ __launch_bounds__(256) void std_scores_kernel(StandardParams p) {
  constexpr int kNch = D / 8;  // 16-byte pieces per K row
  constexpr int kRowBytes = D * 2;
  constexpr int kLoads = kStdKeys * kRowBytes / 1024 / 4;  // 1 KiB blocks per wave
  __shared__ __attribute__((aligned(1024))) char ks_lds[kStdKeys * kRowBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int nkt = (p.Nk + kStdKeys - 1) / kStdKeys;
  const int nqt = (p.Nq + kStdRows - 1) / kStdRows;
  int t = blockIdx.x;
  const int kt = t % nkt;
  t /= nkt;
  const int qt = t % nqt;
  const int bh = t / nqt;
  const int b = bh / p.H;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);

  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Nq * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.Nk * D + (size_t)kt * kStdKeys * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, (uint32_t)p.Nq * D * 2);
  const int kvalid = max(0, min(kStdKeys, L - kt * kStdKeys));  // keys of this block below L
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, (uint32_t)kvalid * kRowBytes);

  // K block -> LDS: lane i of 1 KiB block bl fills row bl*(1024/kRowBytes) + i/kNch, slot i%kNch,
  // which holds piece slot ^ kswz(row) of that key row. kswz keeps the 16 rows of one 16-byte read
  // pass on distinct banks: r % 16 when a row fills the 256-byte bank line (d = 128), (r / 2) % 8
  // when two rows share it (d = 64; r % 8 there puts rows r and r + 8 on the same banks).
  auto kswz = [](int r) { return (kRowBytes >= 256 ? r : r >> 1) % kNch; };
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int bl = w * kLoads + it;
    const int row = bl * (1024 / kRowBytes) + lane / kNch;
    const int slot = lane % kNch;
    buf_load16_lds(krs, ks_lds + bl * 1024, (uint32_t)(row * kRowBytes + ((slot ^ kswz(row)) << 4)));
  }

  // A operands (Q rows): lane (r32, g) holds Q[row 64w + 32 rb + r32][16 ks + 8 g .. +8].
  bf16x8 qa[2][D / 16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint32_t qrow = (uint32_t)(qt * kStdRows + w * 64 + rb * 32 + r32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qa[rb][ks] = __builtin_bit_cast(bf16x8, buf_load16(qrs, (qrow * D + ks * 16 + g * 8) * 2));
  }
  wait_vmcnt<0>();  // this wave's K pieces have landed
  __syncthreads();

  float* Sg = p.s + (size_t)bh * p.Nq * p.ld;
  const int i0 = qt * kStdRows + w * 64;
  const int kx = kswz(r32);
  for (int nb = 0; nb < kStdKeys / 32; ++nb) {
    // B operand (K^T): lane (r32, g) holds K[key 32 nb + r32][16 ks + 8 g .. +8].
    const char* krow = ks_lds + (nb * 32 + r32) * kRowBytes;
    f32x16 acc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(krow + (((2 * ks + g) ^ kx) << 4));
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][ks], kb, acc[rb], 0, 0, 0);
    }
    // Accumulator entry e of lane (r32, g) is S[row 8(e/4) + 4g + e%4][key r32] of the block.
    const int j = kt * kStdKeys + nb * 32 + r32;
    if (j < p.Nk) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = i0 + rb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
          if (i < p.Nq) __builtin_nontemporal_store(acc[rb][e] * p.scale, Sg + (size_t)i * p.ld + j);
        }
    }
  }
}

// ---- Pass 2: row softmax. Allowed keys of row i: j < L and, when causal, j <= i.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Rows of up to 4*64*WPR*CH entries, held in registers: WPR waves per row (4/WPR rows per
// workgroup), each lane holding CH chunks of 4 consecutive scores (chunk c of lane t of the row
// covers entries 4(t + 64 WPR c) .. +3). One read of S, one write of P.
template <int WPR, int CH>
__global__ __launch_bounds__(256) void std_softmax_kernel(StandardParams p) {
  __shared__ float red[2][4];
  const int w = threadIdx.x >> 6;
  const int tl = threadIdx.x & (64 * WPR - 1);  // thread index within its row group
  const int wr = w % WPR;                        // wave index within its row group
  const int row = blockIdx.x * (4 / WPR) + w / WPR;  // bh * Nq + i
  const int nrows = p.B * p.H * p.Nq;
  const bool live = row < nrows;
  const int rr = live ? row : 0;
  const int bh = rr / p.Nq;
  const int i = rr - bh * p.Nq;
  const int L = seq_len(p.kv_seqlens, bh / p.H, p.Nk);
  const int jmax = live ? (p.causal ? min(L, i + 1) : L) : 0;  // allowed keys 0 .. jmax-1
  const float* Sr = p.s + (size_t)rr * p.ld;
  uint16_t* Pr = p.pm + (size_t)rr * p.ld;

  // Scores in base-2 units x = s * log2(e); masked entries -inf.
  float x[CH][4];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j0 = 4 * (tl + 64 * WPR * c);
    f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
    if (j0 < jmax) s4 = *reinterpret_cast<const f32x4*>(Sr + j0);
#pragma unroll
    for (int u = 0; u < 4; ++u) x[c][u] = (j0 + u < jmax) ? s4[u] * kLog2e : -kInf;
  }
  float m = -kInf;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u) m = fmaxf(m, x[c][u]);
  m = wave_max(m);
  if constexpr (WPR > 1) {
    if ((threadIdx.x & 63) == 0) red[0][w] = m;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < WPR; ++k) m = fmaxf(m, red[0][(w / WPR) * WPR + k]);
  }
  // m == -inf only for a row without allowed keys; then every p is 0 below.
  const float mo = m == -kInf ? 0.0f : m;
  float l = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[c][u] = fast_exp2(x[c][u] - mo);
      l += x[c][u];
    }
  l = wave_sum(l);
  if constexpr (WPR > 1) {
    if ((threadIdx.x & 63) == 0) red[1][w] = l;
    __syncthreads();
    l = 0.0f;
#pragma unroll
    for (int k = 0; k < WPR; ++k) l += red[1][(w / WPR) * WPR + k];
  }
  (void)wr;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (!live) return;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j0 = 4 * (tl + 64 * WPR * c);
    if (j0 < p.ld) {
      const u32x2 pk = {pack_bf16(x[c][0] * inv, x[c][1] * inv), pack_bf16(x[c][2] * inv, x[c][3] * inv)};
      *reinterpret_cast<u32x2*>(Pr + j0) = pk;
    }
  }
  if (tl == 0) p.lse[row] = l > 0.0f ? (m + fast_log2(l)) * kLn2 : -kInf;
}

// Rows longer than 16384 entries: one workgroup per row, two reads of S (max and sum, then P).
__global__ __launch_bounds__(256) void std_softmax_long_kernel(StandardParams p) {
  __shared__ float red_m[4], red_l[4];
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int row = blockIdx.x;  // bh * Nq + i
  const int bh = row / p.Nq;
  const int i = row - bh * p.Nq;
  const int b = bh / p.H;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  const int jmax = p.causal ? min(L, i + 1) : L;  // allowed keys are 0 .. jmax-1
  const float* Sr = p.s + (size_t)row * p.ld;
  uint16_t* Pr = p.pm + (size_t)row * p.ld;

  // Per-thread running max and sum of 2^(x - m), x = s * log2(e).
  float m = -kInf, l = 0.0f;
  for (int j0 = 4 * tid; j0 < jmax; j0 += 1024) {
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(Sr + j0);
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = (j0 + u < jmax) ? s4[u] * kLog2e : -kInf;
    const float mc = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float mn = fmaxf(m, mc);
    float add = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) add += fast_exp2(x[u] - mn);
    l = (m == -kInf ? 0.0f : l * fast_exp2(m - mn)) + add;
    m = mn;
  }
  // Combine over the workgroup: m_row = max m, l_row = sum l * 2^(m - m_row).
  const float mw = wave_max(m);
  const float lw = wave_sum(m == -kInf ? 0.0f : l * fast_exp2(m - mw));
  if ((tid & 63) == 0) {
    red_m[w] = mw;
    red_l[w] = lw;
  }
  __syncthreads();
  float mr = -kInf;
#pragma unroll
  for (int k = 0; k < 4; ++k) mr = fmaxf(mr, red_m[k]);
  float lr = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) lr += red_m[k] == -kInf ? 0.0f : red_l[k] * fast_exp2(red_m[k] - mr);

  // P over the whole row (ld entries): 2^(x - m_row) / l_row where allowed, 0 elsewhere.
  const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
  for (int j0 = 4 * tid; j0 < p.ld; j0 += 1024) {
    float pv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (j0 < jmax) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(Sr + j0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pv[u] = (j0 + u < jmax) ? fast_exp2(s4[u] * kLog2e - mr) * inv : 0.0f;
    }
    const u32x2 pk = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
    *reinterpret_cast<u32x2*>(Pr + j0) = pk;
  }
  if (tid == 0) p.lse[row] = lr > 0.0f ? (mr + fast_log2(lr)) * kLn2 : -kInf;
}

template <int WPR, int CH>
static void launch_softmax_reg(const StandardParams& p, int64_t rows, hipStream_t stream) {
  const int per = 4 / WPR;
  hipLaunchKernelGGL((std_softmax_kernel<WPR, CH>), dim3((unsigned)((rows + per - 1) / per)), dim3(256), 0,
                     stream, p);
}

// Smallest register-resident variant whose rows hold ld entries; the two-read kernel beyond.
static void launch_softmax(const StandardParams& p, int64_t rows, hipStream_t stream) {
  const int ld = p.ld;
  if (ld <= 256) launch_softmax_reg<1, 1>(p, rows, stream);
  else if (ld <= 512) launch_softmax_reg<1, 2>(p, rows, stream);
  else if (ld <= 1024) launch_softmax_reg<1, 4>(p, rows, stream);
  else if (ld <= 2048) launch_softmax_reg<1, 8>(p, rows, stream);
  else if (ld <= 4096) launch_softmax_reg<4, 4>(p, rows, stream);
  else if (ld <= 8192) launch_softmax_reg<4, 8>(p, rows, stream);
  else if (ld <= 16384) launch_softmax_reg<4, 16>(p, rows, stream);
  else hipLaunchKernelGGL(std_softmax_long_kernel, dim3((unsigned)rows), dim3(256), 0, stream, p);
}

// ---- Pass 3: O = P V. One workgroup of 4 waves per 128 query rows; wave w owns rows
// 32w .. 32w+31 and keeps its 32 x D block of O in registers over all Nk keys. Per 64-key tile,
// the V tile goes HBM -> LDS (two stages) and is read back transposed as the B operand; the P
// rows come straight from memory as the A operand (each P element is used once), one tile ahead.
// (128-key tiles, or 8 waves over 256 rows, measured slower: more registers, fewer tiles in
// flight per CU.)
template <int D>
struct StdPvCfg {
  static constexpr int kWaves = 4;
  static constexpr int kRows = 32 * kWaves;
  static constexpr int kKeys = 64;    // keys per tile
  static constexpr int kSteps = kKeys / 16;
  static constexpr int kNch = D / 8;  // 16-byte pieces per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kKeys * kRowBytes;
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kKiBPerWave = kTileBytes / 1024 / kWaves;
  static_assert(kKiBPerWave * kWaves * 1024 == kTileBytes, "tile must split over the waves");
};


template <int D>
__global__ __launch_bounds__(256) void std_pv_kernel(StandardParams p) {
  using C = StdPvCfg<D>;
  __shared__ __attribute__((aligned(1024))) char stage_a[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char stage_b[C::kTileBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int nqt = (p.Nq + C::kRows - 1) / C::kRows;
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int b = bh / p.H;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  const int ntiles = (p.Nk + C::kKeys - 1) / C::kKeys;

  const uint16_t* Pg = p.pm + (size_t)bh * p.Nq * p.ld;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(Pg, (uint32_t)p.Nq * p.ld * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vg, (uint32_t)L * C::kRowBytes);

  // V tile -> LDS: wave w moves KiB blocks w*kKiBPerWave ..; lane i fills row rb + i/kNch,
  // 16-byte slot i%kNch, which holds piece slot ^ vswz(row) of key row `row`. vswz keeps the 4
  // rows of one transposed read pass on distinct banks: 4 * (r % 4) when a row fills the 256-byte
  // bank line (d = 128), 4 * ((r ^ r / 2) % 2) when two rows share it (d = 64).
  auto vswz = [](int r) { return C::kRowBytes >= 256 ? 4 * (r % (C::kNch / 4)) : 4 * ((r ^ (r >> 1)) & 1); };
  uint32_t voff[C::kKiBPerWave];
#pragma unroll
  for (int it = 0; it < C::kKiBPerWave; ++it) {
    const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
    const int slot = lane % C::kNch;
    voff[it] = (uint32_t)(row * C::kRowBytes + ((slot ^ vswz(row)) << 4));
  }
  auto issue_v = [&](int tile, char* stage) {
    const uint32_t base = (uint32_t)tile * C::kTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKiBPerWave; ++it)
      buf_load16_lds(vrs, stage + (w * C::kKiBPerWave + it) * 1024, base + voff[it]);
  };
  // A operand (P rows): lane (r32, g) holds P[row r32][16u + 8g .. +8] of the tile.
  const uint32_t prow = (uint32_t)(qt * C::kRows + w * 32 + r32);
  auto load_p = [&](int tile, bf16x8 (&dst)[C::kSteps]) {
#pragma unroll
    for (int u = 0; u < C::kSteps; ++u)
      dst[u] = __builtin_bit_cast(
          bf16x8, buf_load16(prs, (prow * (uint32_t)p.ld + (uint32_t)(tile * C::kKeys + 16 * u + 8 * g)) * 2));
  };
  // B operand (V, keys x d) via transposed reads: in 16-lane group G = lane/16 (gp = G%2,
  // kg = G/2), lane 4a+b addresses key 16u + 8kg + a (+4 for the second read) and
  // d = db*32 + 16gp + 4b, so that lane (r32, g) receives V[16u + 8g .. +8][db*32 + r32].
  const int li = lane & 15;
  const int ta = li >> 2, tb = li & 3;
  const int gp = (lane >> 4) & 1;
  int vt_off[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int piece = db * 4 + 2 * gp + (tb >> 1);
    const int sw = vswz(ta);  // rows 16u + 8kg + ta (+4): bits 0 and 1 are ta's
    vt_off[db] = (8 * g + ta) * C::kRowBytes + ((piece ^ sw) << 4) + 8 * (tb & 1);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;

  auto step = [&](const char* stage, const bf16x8 (&pa)[C::kSteps]) {
#pragma unroll
    for (int u = 0; u < C::kSteps; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const char* vrow = stage + u * 16 * C::kRowBytes + vt_off[db];
        const s16x4 b8[2] = {lds_read_tr16(vrow), lds_read_tr16(vrow + 4 * C::kRowBytes)};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[u], __builtin_bit_cast(bf16x8, b8), acc[db], 0, 0, 0);
      }
  };

  // Double buffer: tile t+1 (V into the other stage, P into registers) is in flight while
  // tile t is consumed. Loads complete in order, so "all but the newest batch" is a vmcnt.
  bf16x8 pa[2][C::kSteps];
  if (ntiles > 0) {
    issue_v(0, stage_a);
    load_p(0, pa[0]);
  }
  for (int t = 0; t < ntiles; t += 2) {
    const bool more = t + 1 < ntiles;
    if (more) {
      issue_v(t + 1, stage_b);
      load_p(t + 1, pa[1]);
      wait_vmcnt<C::kKiBPerWave + C::kSteps>();  // tile t landed
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    step(stage_a, pa[0]);
    __syncthreads();  // stage_a is free again
    if (!more) break;
    const bool more2 = t + 2 < ntiles;
    if (more2) {
      issue_v(t + 2, stage_a);
      load_p(t + 2, pa[0]);
      wait_vmcnt<C::kKiBPerWave + C::kSteps>();  // tile t+1 landed
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    step(stage_b, pa[1]);
    __syncthreads();
  }

  // Accumulator entry e of lane (r32, g) in block db is O[row 8(e/4) + 4g + e%4][db*32 + r32].
  uint16_t* Og = static_cast<uint16_t*>(p.o) + (size_t)bh * p.Nq * D;
  const int i0 = qt * C::kRows + w * 32;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = i0 + 8 * (e >> 2) + 4 * g + (e & 3);
      if (i < p.Nq) Og[(size_t)i * D + db * 32 + r32] = (uint16_t)(pack_bf16(acc[db][e], 0.0f) & 0xffffu);
    }
}

hipError_t launch_standard(const StandardParams& p, int d, hipStream_t stream) {
  const int64_t bh = (int64_t)p.B * p.H;
  if (bh == 0 || p.Nq == 0) return hipSuccess;
  if (p.Nk > 0) {
    const dim3 g1((unsigned)(bh * ((p.Nq + kStdRows - 1) / kStdRows) * ((p.Nk + kStdKeys - 1) / kStdKeys)));
    if (d == 64) hipLaunchKernelGGL(std_scores_kernel<64>, g1, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(std_scores_kernel<128>, g1, dim3(256), 0, stream, p);
  }
  launch_softmax(p, bh * p.Nq, stream);
  const dim3 g3((unsigned)(bh * ((p.Nq + 127) / 128)));
  if (d == 64) hipLaunchKernelGGL(std_pv_kernel<64>, g3, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(std_pv_kernel<128>, g3, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
