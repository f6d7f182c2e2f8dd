// fa_quant_fp8.hip -- e4m3 (OCP FP8) quantisation of bf16 tensors for the FP8 forward pass, on
// gfx950 (MI355X).
//
// FP8 operands halve the bytes moved and double the matrix-core rate, at the price of a
// conversion with a scale and, for V, a transpose (page "FlashAttention：把注意力从公式写成数据流",
// sections "用实验验证而不是背诵结论" and "精度、掩码和边界情况"). One scale per (batch, head)
// slice: s = amax / 448 in fp32 over the slice's valid rows (rows at or past the sequence's
// length are excluded and stored as zero), s = 1 for an all-zero slice; each element becomes
// e4m3(x / s), the quotient a correctly rounded fp32 division, the conversion round-to-nearest-even
// (v_cvt_pk_fp8_f32). Two passes, both bound by HBM bandwidth:
//   quant_amax_kernel      one workgroup per (chunk of rows, slice): the chunk's amax, read as the
//                          largest bf16 magnitude bit pattern (exact, no float compare);
//   quant_rows_kernel      [N][D] output, 16 elements per thread and step;
//   quant_transpose_kernel [D][cols] output (V^T, cols = N rounded up to 64), one 64-key tile
//                          per workgroup, transposed in registers.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {

// Largest |x| of the chunk's valid rows as the bf16 magnitude pattern (bits 0..14): for finite
// values the integer order of these patterns is the order of the magnitudes.
__global__ __launch_bounds__(256) void quant_amax_kernel(QuantParams p) {
  const int bh = blockIdx.x, c = blockIdx.y;
  const int L = seq_len(p.lens, bh / p.H, p.N);
  const int r0 = c * p.rows_per_chunk;
  const int r1 = min(r0 + p.rows_per_chunk, L);
  uint32_t m = 0;
  if (r1 > r0) {
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + ((size_t)bh * p.N + r0) * p.D);
    const int n = (r1 - r0) * p.D / 8;
    for (int i = threadIdx.x; i < n; i += 256) {
      const u32x4 w = __builtin_nontemporal_load(src + i);
#pragma unroll
      for (int t = 0; t < 4; ++t) m = max(m, max(w[t] & 0x7fffu, (w[t] >> 16) & 0x7fffu));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t a = max(max(red[0], red[1]), max(red[2], red[3]));
    p.partial[(size_t)bh * p.n_chunks + c] = __uint_as_float(a << 16);
  }
}

// The slice's scale from its chunk maxima (every wave computes it; n_chunks <= 64).
__device__ __forceinline__ float slice_scale(const QuantParams& p, int bh) {
  const int lane = threadIdx.x & 63;
  float a = lane < p.n_chunks ? p.partial[(size_t)bh * p.n_chunks + lane] : 0.0f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  return a > 0.0f ? a / 448.0f : 1.0f;
}

// Four bf16 values (two words) -> four e4m3 bytes of x / s.
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, float s) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w0) / s, bf16_hi(w0) / s, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w1) / s, bf16_hi(w1) / s, r, true);
  return (uint32_t)r;
}

__global__ __launch_bounds__(256) void quant_rows_kernel(QuantParams p) {
  const int bh = blockIdx.x;
  const float s = slice_scale(p, bh);
  if (blockIdx.y == 0 && threadIdx.x == 0) p.descale[bh] = s;
  const int L = seq_len(p.lens, bh / p.H, p.N);
  const int64_t n = (int64_t)p.N * p.D / 16;        // 16-element pieces of the slice
  const int64_t nvalid = (int64_t)L * p.D / 16;     // pieces of rows < L (D is a multiple of 16)
  const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (size_t)bh * p.N * p.D);
  u32x4* dst = reinterpret_cast<u32x4*>(p.y + (size_t)bh * p.N * p.D);
  for (int64_t i = (int64_t)blockIdx.y * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.y * 256) {
    u32x4 out = {0u, 0u, 0u, 0u};
    if (i < nvalid) {
      const u32x4 a = __builtin_nontemporal_load(src + 2 * i);
      const u32x4 b = __builtin_nontemporal_load(src + 2 * i + 1);
      out[0] = quant4(a[0], a[1], s);
      out[1] = quant4(a[2], a[3], s);
      out[2] = quant4(b[0], b[1], s);
      out[3] = quant4(b[2], b[3], s);
    }
    dst[i] = out;
  }
}

// V^T: tile of keys k0 .. k0+63 of one slice; LDS tile t[d][64] bytes.
template <int D>
__global__ __launch_bounds__(256) void quant_transpose_kernel(QuantParams p) {
  // One 64-key tile per workgroup, transposed in registers: thread (c8, kq) takes keys
  // 4kq .. 4kq+3 of 8-element piece c8 (kq = 0..15 within a wave, so a wave's loads cover 64-byte
  // runs of 16 rows), quantises them, and gathers byte j of the four keys into one word per
  // dimension, which goes to V^T[8 c8 + j][k0 + 4 kq]: each store instruction writes 64-byte runs.
  // No LDS: an earlier version staged the tile through LDS with byte writes that put 16 lanes
  // on one bank.
  constexpr int kThreadsPerRowPiece = 16;          // kq
  constexpr int kPieces = D / 8;                   // c8: 8 (d = 64) or 16 (d = 128)
  constexpr int kPasses = kPieces * kThreadsPerRowPiece / 256;  // 1 for d = 128; d = 64 uses half
  const int bh = blockIdx.x;
  const float s = slice_scale(p, bh);
  if (blockIdx.y == 0 && threadIdx.x == 0) p.descale[bh] = s;
  const int k0 = blockIdx.y * 64;
  if (k0 >= p.cols) return;
  const int L = seq_len(p.lens, bh / p.H, p.N);
  const uint16_t* src = p.x + (size_t)bh * p.N * D;
  uint8_t* dst = p.y + (size_t)bh * D * p.cols + k0;
  const int kq = threadIdx.x % kThreadsPerRowPiece;
  const int c8 = threadIdx.x / kThreadsPerRowPiece;
  if (kPasses == 0 && c8 >= kPieces) return;  // d = 64: 128 threads cover the tile
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = k0 + 4 * kq + i;
    lo[i] = 0u;
    hi[i] = 0u;
    if (key < L) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)key * D) + c8);
      lo[i] = quant4(w[0], w[1], s);  // dimensions 8 c8 + 0..3
      hi[i] = quant4(w[2], w[3], s);  // dimensions 8 c8 + 4..7
    }
  }
  auto gather = [](const uint32_t (&x)[4], int j) {
    const int sh = 8 * j;
    return ((x[0] >> sh) & 0xffu) | (((x[1] >> sh) & 0xffu) << 8) | (((x[2] >> sh) & 0xffu) << 16) |
           (((x[3] >> sh) & 0xffu) << 24);
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<uint32_t*>(dst + (size_t)(8 * c8 + j) * p.cols + 4 * kq) = gather(lo, j);
    *reinterpret_cast<uint32_t*>(dst + (size_t)(8 * c8 + 4 + j) * p.cols + 4 * kq) = gather(hi, j);
  }
}

hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t stream) {
  const int64_t bh = (int64_t)p.B * p.H;
  if (bh == 0) return hipSuccess;
  // Slices along x, chunks / tiles along y (at most 65535: the caller bounds cols / 64).
  hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)bh, p.n_chunks), dim3(256), 0, stream, p);
  if (p.transpose) {
    const dim3 grid((unsigned)bh, (unsigned)(p.cols >= 64 ? p.cols / 64 : 1));
    if (p.D == 64) hipLaunchKernelGGL(quant_transpose_kernel<64>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(quant_transpose_kernel<128>, grid, dim3(256), 0, stream, p);
  } else {
    const int64_t pieces = (int64_t)p.N * p.D / 16;
    int64_t blocks = (pieces + 1023) / 1024;
    blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)bh, (unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
