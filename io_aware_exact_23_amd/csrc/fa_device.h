// fa_device.h -- small device helpers shared by the libfa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kInf = __builtin_inff();

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Valid key count of sequence b: kv_seqlens[b] clamped to [0, Nk], or Nk without lengths.
__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int nk) {
  return lens ? clampi(lens[b], 0, nk) : nk;
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Cross-half combines over lanes l and l ^ 32 of the wave, on v_permlane32_swap (a VALU
// exchange of the two 32-lane halves). The swap of (x, x) returns, in every lane, the pair
// {own value, partner value} in some order, so a symmetric combine of the two results is
// the combine over the lane pair.
__device__ __forceinline__ float pair32_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_min(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Wave-uniform "any lane true".
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// bf16 <-> fp32. A bf16 value is the upper half of a binary32 value.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32). `a` lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// Raw buffer resource over `bytes` bytes from `base`. Loads through it are range-checked by the
// hardware: any 16-byte piece that does not lie inside [0, bytes) reads as zero, with no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane i's bytes
// land at lds_base + 16*i, and pieces outside the buffer's range are written as zeros.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, (int)byte_off, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane 4a+b receives,
// as its element j (j = 0..3), element b of the 4 consecutive 16-bit values addressed by lane
// 4j+a of the group.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// s_waitcnt immediates in the gfx9 encoding that gfx950 uses: vmcnt in bits 3:0 and 15:14, expcnt
// in bits 6:4, lgkmcnt (LDS, scalar memory) in bits 11:8. A field at its maximum (63, 7, 15) does
// not wait on that counter.
constexpr int waitcnt_imm(int vmcnt, int expcnt, int lgkmcnt) {
  return (vmcnt & 15) | ((vmcnt >> 4) << 14) | ((expcnt & 7) << 4) | ((lgkmcnt & 15) << 8);
}
constexpr int kWaitLdsOnly = waitcnt_imm(63, 7, 0);  // this wave's LDS accesses, nothing else

// Wait until at most N of this wave's vector-memory operations are outstanding (loads complete in
// order, so the older ones have landed), leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 7, 15));
}

// Workgroup barrier with no memory wait of its own; the scheduling barriers keep the compiler from
// moving instructions across it.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that waits only for this wave's LDS accesses (lgkmcnt 0, vmcnt untouched):
// __syncthreads() would also drain every vector-memory load in flight, including the next tile's
// copies, and so serialise the prefetch. A wave waits for its own tile copies explicitly before
// the barrier that publishes them. The empty asm keeps the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void wg_barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Row permutation of a 32-key block held in LDS (an involution: bits 2 and 3 swapped). With K rows
// stored in this order, the 16 scores a lane holds in the accumulator of a 32x32 S^T = K Q^T block
// are two runs of 8 consecutive keys, so each run is one 16-byte read of the transposed V tile.
__device__ __forceinline__ int key_row_perm(int r) {
  return (r & ~0xC) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 2);
}

// Workgroups of one launch are handed out round-robin over the 8 XCDs of the MI355X, and each
// XCD has its own L2. Map hardware workgroup id -> logical tile so that every XCD receives one
// contiguous range of logical tiles (tiles that share K/V then share an L2).
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  constexpr int kXcd = 8;
  const int xcd = wg % kXcd;
  const int slot = wg / kXcd;
  const int per = n / kXcd;
  const int rem = n % kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// Causal launches whose workgroups stay resident together. Within an XCD the hardware places the
// workgroups it is handed breadth-first: local slots s, s + P, s + 2P, ... (P = CUs per XCD) share
// a CU. Ordering each XCD's tiles heaviest first within a head (the plain causal order) then gives
// one CU the same query-tile position of several heads, e.g. three of the heaviest tiles next to
// a CU with three of the lightest. Instead, rank the XCD's tiles by weight (query tile descending,
// heads cycling) and hand them out in serpentine order: ranks 0..P-1 to the CUs in order, the
// next P in reverse, and so on, so that each CU's resident tiles sum to about the same work. The
// XCD keeps the same contiguous range of tiles as xcd_remap gives it (same heads, same L2).
// Applies when every XCD's range holds whole heads; otherwise returns false.
__device__ __forceinline__ bool causal_serpentine(int wg, int n, int nq, int P, int& bh, int& qt) {
  constexpr int kXcd = 8;
  if (P <= 0 || n % (kXcd * nq) != 0) return false;
  const int cnt = n / kXcd;        // tiles per XCD: whole heads
  const int k = cnt / nq;          // heads per XCD
  const int xcd = wg % kXcd;
  const int s = wg / kXcd;         // local slot, in the order this XCD receives its workgroups
  const int r = s / P, c = s - r * P;
  const int j = ((r & 1) == 0 || (r + 1) * P > cnt) ? s : r * P + (P - 1 - c);  // weight rank
  qt = nq - 1 - j / k;
  bh = xcd * k + j % k;
  return true;
}

// Padded batches without a causal mask: whole sequences longest first (the longest-processing-time
// order), so that the workgroups a launch runs after its first wave of resident ones are the
// lightest. Workgroup wg -> (rank, query tile, head) with rank outermost; the sequence of a rank is
// found by every lane b < B counting the sequences ordered before sequence b (length descending,
// then index). Consecutive workgroups are consecutive heads, so with H a multiple of 8 all query
// tiles of a head land on one XCD (workgroups are dealt to the XCDs round-robin). Needs
// B <= 64 (one lane per sequence); returns false otherwise.
__device__ __forceinline__ bool longest_first(int wg, const int32_t* lens, int B, int H, int nq, int nk,
                                              int& bh, int& qt) {
  if (lens == nullptr || B > 64) return false;
  const int lane = threadIdx.x & 63;
  const int per_rank = H * nq;
  const int rank = wg / per_rank;
  const int rest = wg - rank * per_rank;
  qt = rest / H;
  const int h = rest - qt * H;
  const int mylen = lane < B ? seq_len(lens, lane, nk) : -1;
  int ahead = 0;
  for (int o = 0; o < B; ++o) {
    const int lo = __shfl(mylen, o, 64);
    ahead += (lo > mylen || (lo == mylen && o < lane)) ? 1 : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && ahead == rank);
  const int b = __builtin_amdgcn_readfirstlane(hit ? (int)__builtin_ctzll(hit) : 0);
  bh = b * H + h;
  return true;
}

}  // namespace fa
