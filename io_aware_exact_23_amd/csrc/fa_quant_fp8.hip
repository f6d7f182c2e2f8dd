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
//                          per workgroup, transposed through LDS.
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
  __shared__ __attribute__((aligned(16))) uint8_t t[D * 64];
  const int bh = blockIdx.x;
  const float s = slice_scale(p, bh);
  if (blockIdx.y == 0 && threadIdx.x == 0) p.descale[bh] = s;
  const int k0 = blockIdx.y * 64;
  if (k0 >= p.cols) return;
  const int L = seq_len(p.lens, bh / p.H, p.N);
  const uint16_t* src = p.x + (size_t)bh * p.N * D;
  constexpr int kPieces = 64 * D / 8;  // 8 bf16 per piece
#pragma unroll
  for (int it = 0; it < kPieces / 256; ++it) {
    const int pc = it * 256 + threadIdx.x;
    const int r = pc / (D / 8), c8 = pc % (D / 8);
    const int key = k0 + r;
    uint32_t lo = 0u, hi = 0u;
    if (key < L) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)key * D) + c8);
      lo = quant4(w[0], w[1], s);
      hi = quant4(w[2], w[3], s);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[(8 * c8 + j) * 64 + r] = (uint8_t)(lo >> (8 * j));
      t[(8 * c8 + 4 + j) * 64 + r] = (uint8_t)(hi >> (8 * j));
    }
  }
  __syncthreads();
  uint8_t* dst = p.y + (size_t)bh * D * p.cols + k0;
#pragma unroll
  for (int it = 0; it < D * 4 / 256; ++it) {
    const int pc = it * 256 + threadIdx.x;
    const int d = pc >> 2, part = pc & 3;
    *reinterpret_cast<u32x4*>(dst + (size_t)d * p.cols + 16 * part) =
        *reinterpret_cast<const u32x4*>(t + d * 64 + 16 * part);
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
