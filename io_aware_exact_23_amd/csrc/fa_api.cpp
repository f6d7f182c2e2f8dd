// fa_api.cpp -- the C ABI of libfa: argument checks, dispatch and launches (host side).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "fa.h"
#include "fa_params.h"

namespace fa {
hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream);
hipError_t launch_prefill_bf16_pp(const PrefillParams& p, int d, hipStream_t stream);
hipError_t launch_prefill_bf16_general(const PrefillParams& p, int d, int max_nq, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, int d, int chunk, hipStream_t stream);
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);
hipError_t launch_standard(const StandardParams& p, int d, hipStream_t stream);
hipError_t launch_backward(const BackwardParams& p, int d, hipStream_t stream);
hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t stream);
hipError_t launch_prefill_fp8(const PrefillFp8Params& p, int d, hipStream_t stream);
int prefill_fp8_rows_per_wg();
int prefill_bf16_rows_per_wg(int d);
int prefill_bf16_pp_rows_per_wg();
constexpr int kPrefillLongNq = 2048;  // query rows from which the 8-wave prefill kernel is used
}  // namespace fa

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* msg) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return status;
}

int fail_hip(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return FA_ERR_HIP;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Checks shared by the entry points. Returns FA_OK, an error, or 1 for "valid no-op".
// elem_bytes is the size of one element of q, k and v. The kernels address one head's rows
// through buffer views with 32-bit sizes and byte offsets, so a head's Q, K or V must stay below
// 2^31 bytes.
int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 const int32_t* kv_seqlens, int elem_bytes) {
  g_last_error[0] = '\0';
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "B, H, Nq, Nk must be >= 0");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d must be 64 or 128");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (causal && Nq != Nk) return fail(FA_ERR_UNSUPPORTED, "causal masking needs Nq == Nk");
  const int64_t bh = (int64_t)B * H;
  if (bh > std::numeric_limits<int32_t>::max())
    return fail(FA_ERR_UNSUPPORTED, "B*H exceeds int32");
  if ((int64_t)std::max(Nq, Nk) * d * elem_bytes >= ((int64_t)1 << 31))
    return fail(FA_ERR_UNSUPPORTED, "one head's q, k or v must stay below 2^31 bytes");
  if (bh == 0 || Nq == 0) return 1;
  if (!q || !o || !lse) return fail(FA_ERR_INVALID_ARGUMENT, "q, o and lse must be non-null");
  if (Nk > 0 && (!k || !v)) return fail(FA_ERR_INVALID_ARGUMENT, "k and v must be non-null");
  if (!aligned(q, 16) || !aligned(o, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)))
    return fail(FA_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4) || (kv_seqlens && !aligned(kv_seqlens, 4)))
    return fail(FA_ERR_INVALID_ARGUMENT, "lse and kv_seqlens must be 4-byte aligned");
  return FA_OK;
}

// Keys per split of the decode path: 128, unless the environment variable FA_DECODE_CHUNK, read
// once per process, names 64 or 256 (the split size is free: the combine is exact for any size,
// so this exists to check that results agree across it). Any other value makes every decode call
// fail rather than silently run another size.
int decode_chunk_keys() {
  static const int chunk = [] {
    const char* s = std::getenv("FA_DECODE_CHUNK");
    if (s == nullptr || *s == '\0') return 128;
    if (std::strcmp(s, "64") == 0) return 64;
    if (std::strcmp(s, "128") == 0) return 128;
    if (std::strcmp(s, "256") == 0) return 256;
    return -1;
  }();
  return chunk;
}

// Compute units per XCD of the current device (the MI355X has 8 XCDs), 0 when the count is not a
// multiple of 8 or cannot be read. Cached per device; the query has no side effects, so threads
// that race to fill an entry store the same value.
int cus_per_xcd() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return c > 0 ? c : 0;
  }
  int n = 0;
  const bool ok = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  const int per = (ok && n > 0 && n % 8 == 0) ? n / 8 : -1;
  if (dev < kMaxDev) cache[dev].store(per, std::memory_order_relaxed);
  return per > 0 ? per : 0;
}

fa::PrefillParams prefill_params(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int H, int Nq, int Nk, float scale, int causal,
                                 const int32_t* kv_seqlens) {
  fa::PrefillParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.kv_seqlens = kv_seqlens;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.c = (float)((double)scale * 1.4426950408889634);  // scores in base-2 units
  // A zero scale makes every allowed score 0. The kernels rely on c != 0 (a masked key's
  // sentinel score times c must be -inf), so use a scale so small that every 2^(c*s) still rounds
  // to exactly 1 and c*s is far below the resolution of the logsumexp: the results are those of c = 0.
  if (p.c == 0.0f) p.c = 1e-30f;
  p.causal = causal;
  p.cus_per_xcd = cus_per_xcd();
  return p;
}

}  // namespace

namespace {

// The bf16 forward behind fa_fwd and fa_fwd_noalloc. Decode (Nq == 1) needs a workspace for its
// partial results: with noalloc it is the library's static scratch (sizes beyond it are
// rejected), else a stream-ordered allocation freed after the kernels.
int fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
             int Nk, int d, float scale, int causal, const int32_t* kv_seqlens, void* stream,
             bool noalloc) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, 2);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (Nq == 1) {
    if (B > 65535 || H > 65535) return fail(FA_ERR_UNSUPPORTED, "decode needs B, H <= 65535");
    fa::DecodeParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.kv_seqlens = kv_seqlens;
    p.B = B;
    p.H = H;
    p.Nk = Nk;
    p.c = (float)((double)scale * 1.4426950408889634);
    const int chunk = decode_chunk_keys();
    if (chunk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "FA_DECODE_CHUNK must be 64, 128 or 256");
    p.n_splits = (Nk + chunk - 1) / chunk;
    const size_t n_part = (size_t)B * H * (size_t)p.n_splits;
    const size_t ws_bytes = n_part * (size_t)(d + 1) * sizeof(float);
    void* ws = nullptr;
    if (n_part > 0) {
      if (noalloc) {
        if (ws_bytes > fa::decode_scratch_bytes())
          return fail(FA_ERR_UNSUPPORTED,
                      "decode partials (4*(d+1)*B*H*ceil(Nk/chunk) bytes) exceed the 72 MiB scratch "
                      "of fa_fwd_noalloc");
        hipError_t e = fa::decode_scratch(&ws);
        if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
      } else {
        hipError_t e = hipMallocAsync(&ws, ws_bytes, s);
        if (e != hipSuccess) return fail_hip(e, "hipMallocAsync(decode workspace)");
      }
      p.ws_o = static_cast<float*>(ws);
      p.ws_lse = p.ws_o + n_part * d;
    }
    hipError_t e = fa::launch_decode_bf16(p, d, chunk, s);
    if (ws && !noalloc) {
      hipError_t ef = hipFreeAsync(ws, s);
      if (e == hipSuccess) e = ef;
    }
    if (e != hipSuccess) return fail_hip(e, "decode launch");
    return FA_OK;
  }

  const int bm = fa::prefill_bf16_rows_per_wg(d);
  const int64_t n_wg = (int64_t)B * H * ((Nq + bm - 1) / bm);
  if (n_wg > std::numeric_limits<int32_t>::max()) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  fa::PrefillParams p = prefill_params(q, k, v, o, lse, B, H, Nq, Nk, scale, causal, kv_seqlens);
  // Long query sequences go to the 8-wave kernel that overlaps one wave's matrix work with its
  // SIMD partner's softmax; its deeper pipeline and 256-row tiles pay off over many key tiles.
  // Short sequences (few key tiles per workgroup, fewer workgroups) run faster on the 4-wave
  // kernel with 128-row tiles.
  hipError_t e = Nq >= fa::kPrefillLongNq ? fa::launch_prefill_bf16_pp(p, d, s)
                                          : fa::launch_prefill_bf16(p, d, s);
  if (e != hipSuccess) return fail_hip(e, "prefill launch");
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      const int32_t* kv_seqlens, void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, stream, false);
}

extern "C" int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Nq, int Nk, int d, float scale, int causal,
                              const int32_t* kv_seqlens, void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, stream, true);
}

extern "C" int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int Nq, int Nk, int d, float scale, int causal,
                          const int32_t* kv_seqlens, void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, 4);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  const int64_t n_wg = (int64_t)B * H * ((Nq + 127) / 128);
  if (n_wg > std::numeric_limits<int32_t>::max()) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  fa::PrefillParams p = prefill_params(q, k, v, o, lse, B, H, Nq, Nk, scale, causal, kv_seqlens);
  hipError_t e = fa::launch_prefill_f32(p, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "prefill launch");
  return FA_OK;
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                      int d, float scale, int causal, const int32_t* kv_seqlens, void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, 2);
  if (st == 1) {
    // No query rows: dK and dV are still defined, zero, when there are keys (the dK/dV kernel
    // writes them without visiting any query tile; the other kernels have no rows to run on).
    if ((int64_t)B * H > 0 && Nk > 0 && Nq == 0) {
      // The kernel still reads K and V (it loads its keys before finding no query tile).
      if (!k || !v || !dk || !dv) return fail(FA_ERR_INVALID_ARGUMENT, "k, v, dk and dv must be non-null");
      if (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return fail(FA_ERR_INVALID_ARGUMENT, "k, v, dk and dv must be 16-byte aligned");
      if (kv_seqlens && !aligned(kv_seqlens, 4))
        return fail(FA_ERR_INVALID_ARGUMENT, "lse and kv_seqlens must be 4-byte aligned");
      fa::BackwardParams p{};
      p.dk = dk;
      p.dv = dv;
      p.k = k;
      p.v = v;
      p.kv_seqlens = kv_seqlens;
      p.B = B;
      p.H = H;
      p.Nk = Nk;
      p.scale = scale;
      hipError_t e = fa::launch_backward(p, d, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return fail_hip(e, "backward launch");
    }
    return FA_OK;
  }
  if (st != FA_OK) return st;
  if (!dout || !dq || (Nk > 0 && (!dk || !dv)))
    return fail(FA_ERR_INVALID_ARGUMENT, "dout, dq, dk and dv must be non-null");
  if (!aligned(dout, 16) || !aligned(dq, 16) || (dk && !aligned(dk, 16)) || (dv && !aligned(dv, 16)))
    return fail(FA_ERR_INVALID_ARGUMENT, "dout, dq, dk and dv must be 16-byte aligned");
  const int64_t bh = (int64_t)B * H;
  if (bh * ((Nq + 127) / 128) > std::numeric_limits<int32_t>::max() ||
      bh * ((Nk + 127) / 128) > std::numeric_limits<int32_t>::max() ||
      (bh * Nq + 3) / 4 > std::numeric_limits<int32_t>::max())
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  fa::BackwardParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.kv_seqlens = kv_seqlens;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.causal = causal;
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, (size_t)bh * Nq * sizeof(float), s);
  if (e != hipSuccess) return fail_hip(e, "hipMallocAsync(backward workspace)");
  p.delta = static_cast<float*>(ws);
  e = fa::launch_backward(p, d, s);
  hipError_t ef = hipFreeAsync(ws, s);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return fail_hip(e, "backward launch");
  return FA_OK;
}

namespace {
int check_window(int left, int right) {
  if (left < -1 || right < -1)
    return fail(FA_ERR_INVALID_ARGUMENT, "window_left and window_right must be >= -1");
  return FA_OK;
}
}  // namespace

extern "C" int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int d, float scale, int window_left,
                             int window_right, const int32_t* kv_seqlens, void* stream) {
  const bool bounded = window_left >= 0 || window_right >= 0;
  int st = check_window(window_left, window_right);
  if (st != FA_OK) return st;
  st = check_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, 0, kv_seqlens, 2);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if (bounded && Nq != Nk) return fail(FA_ERR_UNSUPPORTED, "a bounded window needs Nq == Nk");
  const int bm = fa::prefill_bf16_pp_rows_per_wg();
  if ((int64_t)B * H * ((Nq + bm - 1) / bm) > std::numeric_limits<int32_t>::max())
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  fa::PrefillParams p = prefill_params(q, k, v, o, lse, B, H, Nq, Nk, scale, 0, kv_seqlens);
  p.win_left = window_left;
  p.win_right = window_right;
  hipError_t e = fa::launch_prefill_bf16_general(p, d, Nq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "prefill launch");
  return FA_OK;
}

extern "C" int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int total_q, int total_k, int max_seqlen_q, int d,
                             float scale, int window_left, int window_right,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* stream) {
  g_last_error[0] = '\0';
  int st = check_window(window_left, window_right);
  if (st != FA_OK) return st;
  if (B < 0 || H < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "B, H, total_q, total_k, max_seqlen_q must be >= 0");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d must be 64 or 128");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
  const int64_t bh = (int64_t)B * H;
  if (bh == 0 || total_q == 0 || max_seqlen_q == 0) return FA_OK;
  if (!q || !o || !lse || !cu_seqlens_q || !cu_seqlens_k)
    return fail(FA_ERR_INVALID_ARGUMENT, "q, o, lse and the cu_seqlens arrays must be non-null");
  if (total_k > 0 && (!k || !v)) return fail(FA_ERR_INVALID_ARGUMENT, "k and v must be non-null");
  if (!aligned(q, 16) || !aligned(o, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)))
    return fail(FA_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(FA_ERR_INVALID_ARGUMENT, "lse and the cu_seqlens arrays must be 4-byte aligned");
  if ((int64_t)total_q * d * 2 > std::numeric_limits<int32_t>::max() ||
      (int64_t)total_k * d * 2 > std::numeric_limits<int32_t>::max())
    return fail(FA_ERR_UNSUPPORTED, "one head's packed rows must stay below 2^31 bytes");
  const int bm = fa::prefill_bf16_pp_rows_per_wg();
  if (bh * (((int64_t)max_seqlen_q + bm - 1) / bm) > std::numeric_limits<int32_t>::max())
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  fa::PrefillParams p = prefill_params(q, k, v, o, lse, B, H, 0, 0, scale, 0, nullptr);
  p.win_left = window_left;
  p.win_right = window_right;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.Tq = total_q;
  p.Tk = total_k;
  hipError_t e = fa::launch_prefill_bf16_general(p, d, max_seqlen_q, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "prefill launch");
  return FA_OK;
}

namespace {
// Row stride (elements) of the standard path's S and P buffers: Nk rounded up to a whole 128-key
// tile, so that every tile the kernels touch lies inside its row.
int64_t std_ld(int Nk) { return ((int64_t)Nk + 127) / 128 * 128; }
}  // namespace

extern "C" size_t fa_std_workspace_bytes(int B, int H, int Nq, int Nk) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0) return 0;
  const double bytes = (double)B * H * Nq * (double)std_ld(Nk) * 6.0;
  if (bytes > 9.0e18) return 0;
  return (size_t)B * H * (size_t)Nq * (size_t)std_ld(Nk) * 6u;
}

extern "C" int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Nq, int Nk, int d, float scale, int causal,
                          const int32_t* kv_seqlens, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, 2);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  const int64_t ld = std_ld(Nk);
  if ((int64_t)Nq * ld * 4 > std::numeric_limits<int32_t>::max())
    return fail(FA_ERR_UNSUPPORTED, "Nq * Nk too large for one head's score matrix");
  const int64_t bh = (int64_t)B * H;
  if (bh * Nq > std::numeric_limits<int32_t>::max() ||
      bh * ((Nq + 127) / 128) * ((Nk + 127) / 128) > std::numeric_limits<int32_t>::max())
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = fa_std_workspace_bytes(B, H, Nq, Nk);
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_INVALID_ARGUMENT, "workspace must be non-null");
    if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID_ARGUMENT, "workspace smaller than fa_std_workspace_bytes()");
  }
  fa::StandardParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.kv_seqlens = kv_seqlens;
  p.s = static_cast<float*>(workspace);
  p.pm = need > 0 ? reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + (size_t)bh * Nq * ld * 4)
                  : nullptr;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.ld = (int)ld;
  p.scale = scale;
  p.causal = causal;
  hipError_t e = fa::launch_standard(p, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "standard attention launch");
  return FA_OK;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT: an argument is out of range";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid but not supported by this library";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown fa status";
  }
}

extern "C" const char* fa_last_error(void) { return g_last_error; }

#define FA_STR2(x) #x
#define FA_STR(x) FA_STR2(x)
extern "C" const char* fa_build_info(void) {
  return "compiler: clang " __clang_version__ "; HIP headers " FA_STR(HIP_VERSION_MAJOR) "." FA_STR(
      HIP_VERSION_MINOR) "." FA_STR(HIP_VERSION_PATCH) "; device code: gfx950, packed fp32 VALU ops disabled";
}

extern "C" int fa_fp8_vt_cols(int Nk) { return Nk <= 0 ? 0 : (int)(((int64_t)Nk + 63) / 64 * 64); }

extern "C" int fa_quantize_fp8(const void* x, void* y, float* descale, int B, int H, int N, int d,
                               const int32_t* lens, int transpose, void* stream) {
  g_last_error[0] = '\0';
  if (B < 0 || H < 0 || N < 0) return fail(FA_ERR_INVALID_ARGUMENT, "B, H, N must be >= 0");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d must be 64 or 128");
  if (transpose != 0 && transpose != 1) return fail(FA_ERR_INVALID_ARGUMENT, "transpose must be 0 or 1");
  if ((int64_t)N * d >= ((int64_t)1 << 31)) return fail(FA_ERR_UNSUPPORTED, "one slice must hold fewer than 2^31 elements");
  const int64_t bh = (int64_t)B * H;
  if (bh > std::numeric_limits<int32_t>::max()) return fail(FA_ERR_UNSUPPORTED, "B*H exceeds int32");
  if (bh == 0) return FA_OK;
  if (!descale || (N > 0 && (!x || !y))) return fail(FA_ERR_INVALID_ARGUMENT, "x, y and descale must be non-null");
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)))
    return fail(FA_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned");
  if (!aligned(descale, 4) || (lens && !aligned(lens, 4)))
    return fail(FA_ERR_INVALID_ARGUMENT, "descale and lens must be 4-byte aligned");
  fa::QuantParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.y = static_cast<uint8_t*>(y);
  p.descale = descale;
  p.lens = lens;
  p.B = B;
  p.H = H;
  p.N = N;
  p.D = d;
  p.transpose = transpose;
  p.cols = transpose ? fa_fp8_vt_cols(N) : 0;
  if (transpose && p.cols / 64 > 65535)
    return fail(FA_ERR_UNSUPPORTED, "N too large for the transposed layout (at most 4194240 rows)");
  // Chunks of about 64 KiB of input for the amax pass, at most 64 per slice.
  const int64_t bytes = (int64_t)N * d * 2;
  p.n_chunks = (int)std::min<int64_t>(64, std::max<int64_t>(1, bytes / 65536));
  p.rows_per_chunk = std::max(1, (N + p.n_chunks - 1) / p.n_chunks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, (size_t)bh * p.n_chunks * sizeof(float), s);
  if (e != hipSuccess) return fail_hip(e, "hipMallocAsync(quantiser workspace)");
  p.partial = static_cast<float*>(ws);
  e = fa::launch_quantize_fp8(p, s);
  hipError_t ef = hipFreeAsync(ws, s);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return fail_hip(e, "quantiser launch");
  return FA_OK;
}

extern "C" int fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* descale_q,
                          const float* descale_k, const float* descale_v, void* o, float* lse,
                          int B, int H, int Nq, int Nk, int d, float scale, int causal,
                          const int32_t* kv_seqlens, void* stream) {
  int st = check_common(q8, k8, vt8, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, 1);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if ((descale_q && !aligned(descale_q, 4)) || (descale_k && !aligned(descale_k, 4)) ||
      (descale_v && !aligned(descale_v, 4)))
    return fail(FA_ERR_INVALID_ARGUMENT, "descale arrays must be 4-byte aligned");
  // The transposed V is padded to whole 64-key tiles: its head must also stay below 2^31 bytes.
  if ((int64_t)fa_fp8_vt_cols(Nk) * d >= ((int64_t)1 << 31))
    return fail(FA_ERR_UNSUPPORTED, "one head's q, k or v must stay below 2^31 bytes");
  const int bm = fa::prefill_fp8_rows_per_wg();
  const int64_t n_wg = (int64_t)B * H * ((Nq + bm - 1) / bm);
  if (n_wg > std::numeric_limits<int32_t>::max()) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  fa::PrefillFp8Params p{};
  p.q = static_cast<const uint8_t*>(q8);
  p.k = static_cast<const uint8_t*>(k8);
  p.vt = static_cast<const uint8_t*>(vt8);
  p.dq = descale_q;
  p.dk = descale_k;
  p.dv = descale_v;
  p.o = o;
  p.lse = lse;
  p.kv_seqlens = kv_seqlens;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.ldv = fa_fp8_vt_cols(Nk);
  p.c = (float)((double)scale * 1.4426950408889634);
  if (p.c == 0.0f) p.c = 1e-30f;  // as in the bf16 path: the results of c = 0
  p.causal = causal;
  hipError_t e = fa::launch_prefill_fp8(p, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "fp8 prefill launch");
  return FA_OK;
}
