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
//   bwd_delta_kernel  D_i = dO_i . O_i for every query row (fp32);
//   bwd_dq_kernel     one workgroup of 4 waves per 128 query rows, K/V tiles through LDS as in
//                     the forward kernel: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T;
//   bwd_dkdv_kernel   one workgroup of 4 waves per 128 keys, Q/dO tiles through LDS: S = Q K^T,
//                     dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS.
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

namespace fa {

// Row of a 32-row block read by accumulator row r (an involution: swap bits 2 and 3).
__device__ __forceinline__ int bwd_perm(int r) {
  return (r & ~0xC) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 2);
}

template <int N>
__device__ __forceinline__ void bwd_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// ---- D_i = dO_i . O_i (fp32), one wave per row, 8 bf16 per lane and step.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BackwardParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  if (row >= rows) return;
  const uint16_t* o = static_cast<const uint16_t*>(p.o) + row * D;
  const uint16_t* d = static_cast<const uint16_t*>(p.dout) + row * D;
  float acc = 0.0f;
  for (int c = lane * 8; c < D; c += 512) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + c);
    const u32x4 bb = *reinterpret_cast<const u32x4*>(d + c);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc += bf16_lo(a[t]) * bf16_lo(bb[t]) + bf16_hi(a[t]) * bf16_hi(bb[t]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) p.delta[row] = acc;
}

template <int D>
struct BwdCfg {
  static constexpr int kNch = D / 8;  // 16-byte pieces per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = 64 * kRowBytes;  // one 64-row tile of K, V, Q or dO
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kKiBPerWave = kTileBytes / 1024 / 4;
};

// Per-lane byte offsets of the direct HBM -> LDS copies of a 64-row tile. "Row" layout (the
// forward's K): LDS row r holds tile row bwd_perm(r), piece slot ^ (r % kNch). "Transposable"
// layout (the forward's V): LDS row r holds tile row r, piece slot ^ 4 (r % (kNch / 4)).
template <int D>
__device__ __forceinline__ uint32_t bwd_off_row(int w, int it, int lane) {
  using C = BwdCfg<D>;
  const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
  const int slot = lane % C::kNch;
  return (uint32_t)(bwd_perm(row) * C::kRowBytes + ((slot ^ (row % C::kNch)) << 4));
}
template <int D>
__device__ __forceinline__ uint32_t bwd_off_tr(int w, int it, int lane) {
  using C = BwdCfg<D>;
  const int row = (w * C::kKiBPerWave + it) * C::kRowsPerKiB + lane / C::kNch;
  const int slot = lane % C::kNch;
  return (uint32_t)(row * C::kRowBytes + ((slot ^ (4 * (row % (C::kNch / 4)))) << 4));
}

// ---- dQ. Wave w owns query rows q0 + 32w .. +31; per 64-key tile (K in the row layout, V in the
// transposable layout): S^T = K Q^T and dP^T = V dO^T (keys x queries, one query per lane),
// P^T = 2^(c s - lse2), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BackwardParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char stage_a[2 * C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char stage_b[2 * C::kTileBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int nqt = (p.Nq + 127) / 128;
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int b = bh / p.H;
  const int q0 = qt * 128;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  int kend = L;
  if (p.causal) kend = min(kend, min(q0 + 128, p.Nq));
  const int ntiles = kend > 0 ? (kend + 63) / 64 : 0;

  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Nq * D;
  const uint16_t* dOg = static_cast<const uint16_t*>(p.dout) + (size_t)bh * p.Nq * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.Nk * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dOg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, (uint32_t)kend * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vg, (uint32_t)kend * C::kRowBytes);

  // B operands: lane (r32, g) holds Q[row r32][16 ks + 8 g .. +8] and the same of dO.
  const int qw0 = q0 + w * 32;
  const int qi = qw0 + r32;
  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t off = ((uint32_t)qi * D + ks * 16 + g * 8) * 2;
    qreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(qrs, off));
    doreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(drs, off));
  }
  // This lane's query: base-2 logsumexp (+inf for rows past Nq or without keys: P = 0) and D.
  const size_t qrow = (size_t)bh * p.Nq + qi;
  float lse2 = kInf, dlt = 0.0f;
  if (qi < p.Nq) {
    const float l = p.lse[qrow];
    lse2 = l == -kInf ? kInf : l * kLog2e;
    dlt = p.delta[qrow];
  }
  const float c = p.scale * kLog2e;

  uint32_t koff[C::kKiBPerWave], voff[C::kKiBPerWave];
#pragma unroll
  for (int it = 0; it < C::kKiBPerWave; ++it) {
    koff[it] = bwd_off_row<D>(w, it, lane);
    voff[it] = bwd_off_tr<D>(w, it, lane);
  }
  auto issue = [&](int tile, char* stage) {
    const uint32_t base = (uint32_t)tile * C::kTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKiBPerWave; ++it) {
      char* blk = stage + (w * C::kKiBPerWave + it) * 1024;
      buf_load16_lds(krs, blk, base + koff[it]);
      buf_load16_lds(vrs, blk + C::kTileBytes, base + voff[it]);
    }
  };

  // A operand K rows (row layout): lane reads LDS row kb*32 + r32, piece 2 ks + g.
  const int kx = r32 % C::kNch;
  // A operand V rows in bwd_perm order from the transposable layout: LDS row kb*32 + vr.
  const int vr = bwd_perm(r32);
  const int vsw = 4 * (vr % (C::kNch / 4));
  // A operand K^T (d x keys) by transposed reads of the row layout: in 16-lane group G
  // (gp = G%2), lane 4a+b addresses key 16u + 8g + 4rd + a, which sits in LDS row
  // 16u + 8rd + 4g + a, and d = db*32 + 16gp + 4b.
  const int li = lane & 15;
  const int ta = li >> 2, tb = li & 3;
  const int gp = (lane >> 4) & 1;
  int kt_off[2][D / 32];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int r = 8 * rd + 4 * g + ta;
      const int piece = db * 4 + 2 * gp + (tb >> 1);
      kt_off[rd][db] = r * C::kRowBytes + ((piece ^ (r % C::kNch)) << 4) + 8 * (tb & 1);
    }

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.0f;

  auto step = [&](const char* stage, int k0) {
    const char* Ks = stage;
    const char* Vs = stage + C::kTileBytes;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = dp[kb][e] = 0.0f;
      const char* krow = Ks + (kb * 32 + r32) * C::kRowBytes;
      const char* vrow = Vs + (kb * 32 + vr) * C::kRowBytes;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + (((2 * ks + g) ^ kx) << 4));
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vrow + (((2 * ks + g) ^ vsw) << 4));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, doreg[ks], dp[kb], 0, 0, 0);
      }
    }
    // Entry e of block kb is key k0 + kb*32 + 16(e/8) + 8g + e%8 of this lane's query qi.
    const int rem = (p.causal ? min(L, qi + 1) : L) - (k0 + 8 * g);
    bf16x8 dsk[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 x;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float ds2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = hh * 8 + 2 * t + u;
            const bool ok = kb * 32 + 16 * hh + 2 * t + u < rem;
            const float pr = ok ? fast_exp2(fmaf(s[kb][e], c, -lse2)) : 0.0f;
            ds2[u] = pr * (dp[kb][e] - dlt);
          }
          x[t] = pack_bf16(ds2[0], ds2[1]);
        }
        dsk[kb][hh] = __builtin_bit_cast(bf16x8, x);
      }
    // dQ^T += K^T dS^T over the tile's four 16-key steps.
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const char* base = Ks + u * 16 * C::kRowBytes;
        const s16x4 a8[2] = {lds_read_tr16(base + kt_off[0][db]), lds_read_tr16(base + kt_off[1][db])};
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), dsk[u >> 1][u & 1],
                                                        dq[db], 0, 0, 0);
      }
  };

  if (ntiles > 0) issue(0, stage_a);
  for (int t = 0; t < ntiles; t += 2) {
    const bool more = t + 1 < ntiles;
    if (more) {
      issue(t + 1, stage_b);
      bwd_wait_vmcnt<2 * C::kKiBPerWave>();
    } else {
      bwd_wait_vmcnt<0>();
    }
    __syncthreads();
    step(stage_a, t * 64);
    __syncthreads();
    if (!more) break;
    if (t + 2 < ntiles) {
      issue(t + 2, stage_a);
      bwd_wait_vmcnt<2 * C::kKiBPerWave>();
    } else {
      bwd_wait_vmcnt<0>();
    }
    __syncthreads();
    step(stage_b, (t + 1) * 64);
    __syncthreads();
  }
  bwd_wait_vmcnt<0>();

  // dQ^T entry e of block db (lane r32, g) is dQ[qi][db*32 + 8(e/4) + 4g + e%4].
  if (qi < p.Nq) {
    uint16_t* dQg = static_cast<uint16_t*>(p.dq) + (size_t)bh * p.Nq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const u32x2 x = {pack_bf16(dq[db][4 * jq] * p.scale, dq[db][4 * jq + 1] * p.scale),
                         pack_bf16(dq[db][4 * jq + 2] * p.scale, dq[db][4 * jq + 3] * p.scale)};
        *reinterpret_cast<u32x2*>(dQg + db * 32 + 8 * jq + 4 * g) = x;
      }
  }
}

// ---- dK, dV. Wave w owns keys k0 + 32w .. +31; per 64-query tile (Q and dO in the transposable
// layout, their lse2 and D in LDS): S = Q K^T and dP = dO V^T (queries x keys, one key per lane,
// rows read in bwd_perm order), P = 2^(c s - lse2), dS = P (dP - D), dV^T += dO^T P,
// dK^T += Q^T dS.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BackwardParams p) {
  using C = BwdCfg<D>;
  constexpr int kStage = 2 * C::kTileBytes + 2 * 64 * 4;  // Q tile, dO tile, lse2[64], D[64]
  __shared__ __attribute__((aligned(1024))) char stage_a[kStage];
  __shared__ __attribute__((aligned(1024))) char stage_b[kStage];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int nkt = (p.Nk + 127) / 128;
  const int bh = blockIdx.x / nkt;
  const int kt = blockIdx.x - bh * nkt;
  const int b = bh / p.H;
  const int k0 = kt * 128;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  const int kj = k0 + w * 32 + r32;  // this lane's key
  // Query tiles that can see a key of this workgroup: from the first row at or after k0 when
  // causal, none when every key is past L.
  const int t0 = (p.causal && k0 < L) ? k0 / 64 : 0;
  const int tn = k0 < L ? (p.Nq + 63) / 64 : 0;

  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Nq * D;
  const uint16_t* dOg = static_cast<const uint16_t*>(p.dout) + (size_t)bh * p.Nq * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.Nk * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.Nk * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dOg, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, (uint32_t)L * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vg, (uint32_t)L * C::kRowBytes);
  const float* lse_bh = p.lse + (size_t)bh * p.Nq;
  const float* dl_bh = p.delta + (size_t)bh * p.Nq;

  // B operands: lane (r32, g) holds K[key kj][16 ks + 8 g .. +8] and the same of V (keys past L
  // read as zeros).
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t off = ((uint32_t)kj * D + ks * 16 + g * 8) * 2;
    kreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(krs, off));
    vreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(vrs, off));
  }
  const float c = p.scale * kLog2e;

  uint32_t toff[C::kKiBPerWave];
#pragma unroll
  for (int it = 0; it < C::kKiBPerWave; ++it) toff[it] = bwd_off_tr<D>(w, it, lane);
  // Tile t: Q and dO rows by direct copies; lse2 and D of its 64 rows by wave 0 (registers, then
  // LDS once they have landed).
  float st_l = kInf, st_d = 0.0f;
  auto issue = [&](int tile, char* stage) {
    const uint32_t base = (uint32_t)tile * C::kTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKiBPerWave; ++it) {
      char* blk = stage + (w * C::kKiBPerWave + it) * 1024;
      buf_load16_lds(qrs, blk, base + toff[it]);
      buf_load16_lds(drs, blk + C::kTileBytes, base + toff[it]);
    }
    if (w == 0) {
      const int qrow = tile * 64 + lane;
      st_l = kInf;
      st_d = 0.0f;
      if (qrow < p.Nq) {
        const float l = lse_bh[qrow];
        st_l = l == -kInf ? kInf : l * kLog2e;
        st_d = dl_bh[qrow];
      }
    }
  };
  auto publish = [&](char* stage) {
    if (w == 0) {
      float* ls = reinterpret_cast<float*>(stage + 2 * C::kTileBytes);
      ls[lane] = st_l;
      ls[64 + lane] = st_d;
    }
  };

  // A operands Q and dO rows in bwd_perm order from the transposable layout.
  const int qr = bwd_perm(r32);
  const int qsw = 4 * (qr % (C::kNch / 4));
  // A operands Q^T and dO^T (d x queries) by transposed reads: lane 4a+b of 16-lane group G
  // addresses query 16u + 8g + 4rd + a, d = db*32 + 16gp + 4b (the forward's V^T reads).
  const int li = lane & 15;
  const int ta = li >> 2, tb = li & 3;
  const int gp = (lane >> 4) & 1;
  int tr_off[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int piece = db * 4 + 2 * gp + (tb >> 1);
    const int sw = 4 * (ta % (C::kNch / 4));
    tr_off[db] = (8 * g + ta) * C::kRowBytes + ((piece ^ sw) << 4) + 8 * (tb & 1);
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[db][e] = dv[db][e] = 0.0f;

  // One 32-query block at a time: S and dP of the block, then its P and dS, then its two 16-query
  // steps of dV^T and dK^T (keeps the live accumulators to those of one block).
  auto step = [&](const char* stage, int qt0) {
    const char* Qs = stage;
    const char* dOs = stage + C::kTileBytes;
    const float* ls = reinterpret_cast<const float*>(stage + 2 * C::kTileBytes);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.0f;
      const char* qrow = Qs + (qb * 32 + qr) * C::kRowBytes;
      const char* drow = dOs + (qb * 32 + qr) * C::kRowBytes;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int pc = ((2 * ks + g) ^ qsw) << 4;
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qrow + pc);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(drow + pc);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vreg[ks], dp, 0, 0, 0);
      }
      // Entry e is query qt0 + qb*32 + 16(e/8) + 8g + e%8 against this lane's key kj.
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ql = qb * 32 + 16 * hh + 8 * g;  // tile-local query of entry hh*8
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(ls + ql);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(ls + ql + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(ls + 64 + ql);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(ls + 64 + ql + 4);
        u32x4 xp, xs;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float pv[2], dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int j = 2 * t + u;  // 0..7
            const int e = hh * 8 + j;
            const int qq = qt0 + ql + j;
            const float lq = j < 4 ? l0[j] : l1[j - 4];
            const float dq = j < 4 ? d0[j] : d1[j - 4];
            const bool ok = kj < L && (!p.causal || kj <= qq);
            pv[u] = ok ? fast_exp2(fmaf(s[e], c, -lq)) : 0.0f;
            dsv[u] = pv[u] * (dp[e] - dq);
          }
          xp[t] = pack_bf16(pv[0], pv[1]);
          xs[t] = pack_bf16(dsv[0], dsv[1]);
        }
        pb[hh] = __builtin_bit_cast(bf16x8, xp);
        dsb[hh] = __builtin_bit_cast(bf16x8, xs);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the block's two 16-query steps.
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int o = (qb * 2 + hh) * 16 * C::kRowBytes + tr_off[db];
          const s16x4 da8[2] = {lds_read_tr16(dOs + o), lds_read_tr16(dOs + o + 4 * C::kRowBytes)};
          const s16x4 qa8[2] = {lds_read_tr16(Qs + o), lds_read_tr16(Qs + o + 4 * C::kRowBytes)};
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, da8), pb[hh], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa8), dsb[hh], dk[db], 0, 0, 0);
        }
    }
  };

  if (t0 < tn) {
    issue(t0, stage_a);
    bwd_wait_vmcnt<0>();
    publish(stage_a);
  }
  for (int t = t0; t < tn; t += 2) {
    const bool more = t + 1 < tn;
    if (more) issue(t + 1, stage_b);
    __syncthreads();  // stage_a (tile t) complete and visible
    step(stage_a, t * 64);
    if (more) {
      bwd_wait_vmcnt<0>();
      publish(stage_b);
    }
    __syncthreads();  // stage_a free, stage_b (tile t+1) complete
    if (!more) break;
    const bool more2 = t + 2 < tn;
    if (more2) issue(t + 2, stage_a);
    step(stage_b, (t + 1) * 64);
    if (more2) {
      bwd_wait_vmcnt<0>();
      publish(stage_a);
    }
    __syncthreads();
  }
  bwd_wait_vmcnt<0>();

  // dK^T / dV^T entry e of block db (lane r32, g) is row kj, column db*32 + 8(e/4) + 4g + e%4.
  if (kj < p.Nk) {
    uint16_t* dKg = static_cast<uint16_t*>(p.dk) + (size_t)bh * p.Nk * D + (size_t)kj * D;
    uint16_t* dVg = static_cast<uint16_t*>(p.dv) + (size_t)bh * p.Nk * D + (size_t)kj * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const u32x2 xk = {pack_bf16(dk[db][4 * jq] * p.scale, dk[db][4 * jq + 1] * p.scale),
                          pack_bf16(dk[db][4 * jq + 2] * p.scale, dk[db][4 * jq + 3] * p.scale)};
        const u32x2 xv = {pack_bf16(dv[db][4 * jq], dv[db][4 * jq + 1]),
                          pack_bf16(dv[db][4 * jq + 2], dv[db][4 * jq + 3])};
        *reinterpret_cast<u32x2*>(dKg + db * 32 + 8 * jq + 4 * g) = xk;
        *reinterpret_cast<u32x2*>(dVg + db * 32 + 8 * jq + 4 * g) = xv;
      }
  }
}

hipError_t launch_backward(const BackwardParams& p, int d, hipStream_t stream) {
  const int64_t bh = (int64_t)p.B * p.H;
  if (bh == 0) return hipSuccess;
  const int64_t rows = bh * p.Nq;
  if (rows > 0) {
    const dim3 g0((unsigned)((rows + 3) / 4));
    if (d == 64) hipLaunchKernelGGL(bwd_delta_kernel<64>, g0, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(bwd_delta_kernel<128>, g0, dim3(256), 0, stream, p);
    const dim3 g1((unsigned)(bh * ((p.Nq + 127) / 128)));
    if (d == 64) hipLaunchKernelGGL(bwd_dq_kernel<64>, g1, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(bwd_dq_kernel<128>, g1, dim3(256), 0, stream, p);
  }
  if (p.Nk > 0) {
    const dim3 g2((unsigned)(bh * ((p.Nk + 127) / 128)));
    if (d == 64) hipLaunchKernelGGL(bwd_dkdv_kernel<64>, g2, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(bwd_dkdv_kernel<128>, g2, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
