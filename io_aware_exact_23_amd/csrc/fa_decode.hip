// fa_decode.hip -- split-KV attention for one query per (b, h) (decode), bf16, gfx950.
//
// Decode is a separate phase that the pages ask to be measured apart from prefill (page
// "FlashAttention：把注意力从公式写成数据流", section "评估清单"), and the vocus page names
// FlashDecoding as its IO-aware form (section "結論"). With one query there is no reuse of K/V,
// so the pass is bound by HBM bandwidth: every valid key is read exactly once.
//
// Kernel 1 (split): one workgroup per (chunk of CHUNK keys, h, b). Each wave streams
// kDecodeKeysPerWave keys with 16-byte non-temporal loads (the keys are read once: keeping them in the caches only
// evicts what other workgroups still need; +5.5% on the decode workload), kLanesPerKey lanes
// per key row (whole rows per load instruction: perfectly coalesced), forms the dot products on
// the vector ALUs, and keeps a local max, sum and unnormalised output. The waves merge through
// LDS into one partial (o_c, lse_c) per chunk: o_c normalised, lse_c = log2 sum_j 2^(t_j) in
// base-2 units.
// Kernel 2 (combine): per (b, h), lse* = max_c lse_c, w_c = 2^(lse_c - lse*),
// O = sum w_c o_c / sum w_c, lse = ln 2 * (lse* + log2 sum w_c). Exact in exact arithmetic,
// for any chunk size.
#include <mutex>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {

// Scratch of the allocation-free entry point (fa_fwd_noalloc): the decode path's partial outputs
// and logsumexps live here instead of in a stream-ordered allocation. 72 MiB holds the
// 64 x 32 x ceil(8192 / 128) partials of a cache of 64 sequences x 32 heads x 8192 keys at
// d = 128 (64.5 MiB). Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, per device (decode_scratch below).
constexpr size_t kNoAllocScratchBytes = size_t(72) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

size_t decode_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of the current device's copy of `scratch`, looked up once per device (with that
// device current) and kept.
hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Keys per chunk and per wave. Measured on the decode workload (64 x 32 heads, up to 8192 keys),
// whole call: 128-key chunks of 4 waves x 32 keys 5.94 TB/s; of 2 waves x 64 keys 5.89 (with 8 x 16
// the same); 256-key chunks 5.7, 512-key chunks 4.4; 96-key chunks 5.77, 64-key chunks 5.4-5.5,
// where the partial outputs and their combine cost more than the finer balance gains. 128 is the
// default; 64 and 256 are built too, since the split size is free (the combine is exact for any
// chunk size) and the results must agree across it to fp32 rounding.
constexpr int kDecodeKeysPerWave = 32;

// Sum over aligned groups of N lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int D, int CHUNK>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * CHUNK / kDecodeKeysPerWave, 64 * CHUNK / kDecodeKeysPerWave)))
void decode_split_kernel(DecodeParams p) {
  constexpr int kWaves = CHUNK / kDecodeKeysPerWave;
  constexpr int kLanesPerKey = D / 8;          // 16 bytes (8 bf16) per lane
  constexpr int kKeysPerLoad = 64 / kLanesPerKey;
  constexpr int kKeysPerWave = kDecodeKeysPerWave;
  constexpr int kRounds = kKeysPerWave / kKeysPerLoad;
  static_assert(kRounds * kKeysPerLoad == kKeysPerWave, "chunk must split evenly");
  static_assert(kWaves * 64 >= D, "the merge gives one thread per output element");

  __shared__ float sm_m[kWaves], sm_l[kWaves];
  __shared__ float sm_o[kWaves][D];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  const int key0 = split * CHUNK;
  if (key0 >= L) return;  // the whole workgroup leaves together: no barrier is skipped

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int slot = lane / kLanesPerKey;  // which key of a load round
  const int part = lane % kLanesPerKey;  // which 8-wide piece of d
  const size_t bh = (size_t)b * p.H + h;

  const u32x4 qx = *reinterpret_cast<const u32x4*>(p.q + bh * D + part * 8);
  float qf[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    qf[2 * t] = bf16_lo(qx[t]);
    qf[2 * t + 1] = bf16_hi(qx[t]);
  }

  const uint16_t* Kb = p.k + bh * (size_t)p.Nk * D + part * 8;
  const uint16_t* Vb = p.v + bh * (size_t)p.Nk * D + part * 8;
  const int kw0 = key0 + w * kKeysPerWave + slot;

  u32x4 kr[kRounds], vr[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int key = kw0 + r * kKeysPerLoad;
    u32x4 z = {0u, 0u, 0u, 0u};
    kr[r] = key < L ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kb + (size_t)key * D)) : z;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int key = kw0 + r * kKeysPerLoad;
    u32x4 z = {0u, 0u, 0u, 0u};
    vr[r] = key < L ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vb + (size_t)key * D)) : z;
  }

  // Scores in base-2 units, t = c * q.k; keys past L get -inf.
  float t[kRounds];
  float mx = -kInf;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot = fmaf(qf[2 * e], bf16_lo(kr[r][e]), dot);
      dot = fmaf(qf[2 * e + 1], bf16_hi(kr[r][e]), dot);
    }
    dot = group_sum<kLanesPerKey>(dot);
    const int key = kw0 + r * kKeysPerLoad;
    t[r] = key < L ? dot * p.c : -kInf;
    mx = fmaxf(mx, t[r]);
  }
#pragma unroll
  for (int m = kLanesPerKey; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));

  float lw = 0.0f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.0f;
  if (mx != -kInf) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const float pr = fast_exp2(t[r] - mx);  // 0 for masked keys
      lw += pr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = fmaf(pr, bf16_lo(vr[r][e]), o[2 * e]);
        o[2 * e + 1] = fmaf(pr, bf16_hi(vr[r][e]), o[2 * e + 1]);
      }
    }
  }
#pragma unroll
  for (int m = kLanesPerKey; m < 64; m <<= 1) {
    lw += __shfl_xor(lw, m, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], m, 64);
  }
  if (slot == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[w][part * 8 + e] = o[e];
    if (part == 0) {
      sm_m[w] = mx;
      sm_l[w] = lw;
    }
  }
  __syncthreads();

  if (tid < D) {
    float M = sm_m[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sm_m[i]);
    // M is finite: key0 < L, so wave 0 saw at least one valid key.
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const float f = sm_m[i] == -kInf ? 0.0f : fast_exp2(sm_m[i] - M);
      lt = fmaf(sm_l[i], f, lt);
      ot = fmaf(sm_o[i][tid], f, ot);
    }
    const size_t ws = bh * p.n_splits + split;
    p.ws_o[ws * D + tid] = ot / lt;
    if (tid == 0) p.ws_lse[ws] = M + fast_log2(lt);
  }
}

template <int D, int CHUNK>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void decode_combine_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int lane = threadIdx.x;
  const int L = seq_len(p.kv_seqlens, b, p.Nk);
  const int n = (L + CHUNK - 1) / CHUNK;
  const float* lse_s = p.ws_lse + (size_t)bh * p.n_splits;
  const float* o_s = p.ws_o + (size_t)bh * p.n_splits * D;

  // lse* = max over the partials: lanes take partials lane, lane + 64, ..., then a wave maximum.
  float M = -kInf;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, lse_s[s]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  // Weighted sum over the partials in order, lanes over d. Partials go in groups of 8 whose loads
  // are all issued before their arithmetic, so the loop waits for memory once per group rather
  // than once per partial.
  constexpr int kG = 8;
  float W = 0.0f;
  float acc[D / 64];
#pragma unroll
  for (int t = 0; t < D / 64; ++t) acc[t] = 0.0f;
  int s = 0;
  for (; s + kG <= n; s += kG) {
    float lg[kG], og[kG][D / 64];
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      lg[u] = lse_s[s + u];
#pragma unroll
      for (int t = 0; t < D / 64; ++t) og[u][t] = o_s[(size_t)(s + u) * D + lane + 64 * t];
    }
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const float wgt = fast_exp2(lg[u] - M);
      W += wgt;
#pragma unroll
      for (int t = 0; t < D / 64; ++t) acc[t] = fmaf(wgt, og[u][t], acc[t]);
    }
  }
  for (; s < n; ++s) {
    const float wgt = fast_exp2(lse_s[s] - M);
    W += wgt;
#pragma unroll
    for (int t = 0; t < D / 64; ++t) acc[t] = fmaf(wgt, o_s[(size_t)s * D + lane + 64 * t], acc[t]);
  }
  const float inv = n > 0 ? 1.0f / W : 0.0f;
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    const float x = acc[t] * inv;
    p.o[(size_t)bh * D + lane + 64 * t] = (uint16_t)(pack_bf16(x, 0.0f) & 0xffffu);
  }
  if (lane == 0) p.lse[bh] = n > 0 ? (M + fast_log2(W)) * kLn2 : -kInf;
}

template <int D, int CHUNK>
void launch_decode(const DecodeParams& p, hipStream_t stream) {
  constexpr int kThreads = 64 * CHUNK / kDecodeKeysPerWave;
  if (p.n_splits > 0)
    hipLaunchKernelGGL((decode_split_kernel<D, CHUNK>), dim3(p.n_splits, p.H, p.B), dim3(kThreads), 0,
                       stream, p);
  hipLaunchKernelGGL((decode_combine_kernel<D, CHUNK>), dim3(p.B * p.H), dim3(64), 0, stream, p);
}

// chunk: keys per split, 64, 128 or 256 (p.n_splits = ceil(Nk / chunk)); the caller checks it.
hipError_t launch_decode_bf16(const DecodeParams& p, int d, int chunk, hipStream_t stream) {
  if (d == 64) {
    if (chunk == 64) launch_decode<64, 64>(p, stream);
    else if (chunk == 256) launch_decode<64, 256>(p, stream);
    else launch_decode<64, 128>(p, stream);
  } else {
    if (chunk == 64) launch_decode<128, 64>(p, stream);
    else if (chunk == 256) launch_decode<128, 256>(p, stream);
    else launch_decode<128, 128>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace fa
