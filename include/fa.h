/*
 * fa.h -- C ABI of libfa, an exact-attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * What is computed. For every batch b, head h and query row i:
 *   allowed keys  A_i = { j : j < L_b and (causal == 0 or j <= i) }
 *   S_ij = scale * q_i . k_j  (j in A_i),  P_i = softmax over A_i of S_i,  O_i = sum_j P_ij v_j,
 *   lse_i = ln sum_{j in A_i} exp(S_ij)   (natural log);  A_i empty -> O_i = 0, lse_i = -inf.
 * This is standard softmax attention (page "FlashAttention：把注意力从公式写成数据流", opening
 * paragraph; page "FlashAttention 与边缘设备上的注意力内存瓶颈", section "2 标准 attention 的问题"),
 * computed tile by tile with an online softmax so that S and P never reach device memory
 * (same pages: sections "分块与在线 softmax" and "3.1 Tiling" / "3.2 Online Softmax"). Masked
 * and padded keys never enter the normalisation (page "FlashAttention：把注意力从公式写成数据流",
 * section "精度、掩码和边界情况"). The logsumexp output is part of this library's contract.
 *
 * Layout (all row-major, d fastest, no strides):
 *   q, o : [B][H][Nq][d]      k, v : [B][H][Nk][d]      lse : [B][H][Nq] fp32
 *   kv_seqlens : int32 [B] valid key count per sequence, clamped to [0, Nk] on the device;
 *                NULL means every sequence has Nk valid keys.
 * q, k, v and o must be 16-byte aligned; lse and kv_seqlens 4-byte aligned.
 * One head's q, k or v (max(Nq, Nk) * d * element size) must stay below 2^31 bytes, else
 * FA_ERR_UNSUPPORTED: the kernels address a head through 32-bit buffer offsets.
 *
 * Ownership. Every pointer is device memory owned by the caller. The library reads q, k, v and
 * kv_seqlens, writes only o and lse (and, for Nq == 1, a workspace it allocates and frees
 * stream-ordered on `stream`), and keeps no pointer after the call. Key slots at or past L_b are
 * never read, so they may hold anything.
 *
 * Streams and errors. `stream` is a hipStream_t (NULL = the default stream). All work is enqueued
 * on it; the call never synchronises. Arguments are checked before anything is enqueued: on any
 * error nothing is launched and a negative fa_status_t comes back. Faults that happen inside a
 * kernel surface at the caller's next synchronisation, as for any stream-ordered API.
 * Calls on different streams are independent (no shared mutable state).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = -1, /* null pointer, negative size, misalignment, non-finite scale */
  FA_ERR_UNSUPPORTED = -2,      /* d not in {64, 128}; causal with Nq != Nk; sizes too large     */
  FA_ERR_HIP = -3               /* the HIP runtime refused a launch or an allocation           */
} fa_status_t;

/*
 * fa_fwd -- bf16 attention forward: q, k, v, o hold bf16 values (raw 16-bit patterns);
 * lse is fp32. Arithmetic: bf16 products on the matrix cores with fp32 accumulation, softmax in
 * fp32, O rounded to bf16 (nearest even) once at the end.
 *   B, H >= 0; Nq, Nk >= 0; d in {64, 128}; scale finite (any sign); causal in {0, 1} and,
 *   if set, Nq == Nk. B*H*Nq == 0 is a valid no-op; Nk == 0 gives O = 0 and lse = -inf.
 *   Nq == 1 runs the split-KV decode kernels (one query per (b, h)); any other Nq runs the
 *   tiled prefill kernel.
 *   Decode splits each sequence's keys into chunks of 128 and combines the chunks' partial
 *   (o, lse) by their logsumexp; the combine is exact for any chunk size, so results agree across
 *   it to fp32 rounding. The environment variable FA_DECODE_CHUNK (64, 128 or 256), read once per
 *   process, overrides the chunk size; any other value makes every Nq == 1 call return
 *   FA_ERR_INVALID_ARGUMENT.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           const int32_t* kv_seqlens, void* stream);

/*
 * fa_fwd_noalloc -- fa_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): it allocates nothing. The
 * decode path (Nq == 1) keeps its partial results in a static 72 MiB device array of the library
 * (each GPU it runs on holds its own copy until the process ends) instead of a stream-ordered
 * allocation; every other Nq runs exactly what fa_fwd runs, which needs no workspace.
 *   Same arguments, layouts, arithmetic and results as fa_fwd (bit for bit). Decode calls whose
 *   partials need more than 72 MiB, 4*(d+1)*B*H*ceil(Nk/128) bytes (a cache of 64 x 32
 *   sequences x 8192 keys at d = 128 needs 64.5 MiB), return FA_ERR_UNSUPPORTED before anything
 *   is launched. Every call on one GPU shares that GPU's array: decode calls that overlap on one
 *   GPU (different streams, or host threads) race and must be ordered by the caller. Nothing in
 *   the array needs to start at zero.
 */
int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   const int32_t* kv_seqlens, void* stream);

/*
 * fa_fwd_f32 -- the same operation with fp32 q, k, v and o (fp32 products and accumulation on
 * the matrix cores, fp32 softmax). Same argument rules as fa_fwd; every Nq runs the tiled kernel.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               const int32_t* kv_seqlens, void* stream);

/*
 * fa_fwd_window -- fa_fwd with a sliding-window mask instead of the causal flag: key j is
 * allowed for query i iff j < L_b, j >= i - window_left (if window_left >= 0) and
 * j <= i + window_right (if window_right >= 0); -1 means no limit on that side. Query i sits at
 * key position i, the alignment of the causal mask, so (-1, 0) is the causal mask, (W-1, 0) a
 * causal window of the W most recent keys, (-1, -1) no mask. Sliding windows are among the
 * masks the pages name beside causal masks and variable-length batches as making tile edges
 * irregular (page "FlashAttention：把注意力从公式写成数据流", section "精度、掩码和边界情况").
 * Tiles outside every row's window are neither read nor computed.
 *   Same arguments and layouts as fa_fwd, with window_left, window_right >= -1 and, when either
 *   is >= 0, Nq == Nk (else FA_ERR_UNSUPPORTED). Every Nq (also 1) runs the tiled kernel.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale, int window_left,
                  int window_right, const int32_t* kv_seqlens, void* stream);

/*
 * fa_fwd_varlen -- packed variable-length batch: B sequences of different lengths stored back
 * to back, without padding (the "变长 batch" of the same section). Sequence b holds query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.
 * Within a sequence the mask is that of fa_fwd_window (query i at key position i of its own
 * sequence; use window (-1, 0) for causal, (-1, -1) for none).
 *   Layout (head-major, rows of d contiguous):
 *     q, o : [H][total_q][d]   k, v : [H][total_k][d]   lse : [H][total_q] fp32
 *   cu_seqlens_q, cu_seqlens_k : device int32 [B+1], non-decreasing, starting at 0 and ending at
 *     total_q / total_k. Offsets are clamped to [0, total] on the device, so no access leaves the
 *     tensors even for malformed offsets.
 *   max_seqlen_q >= the longest query sequence (sets the grid; rows past it are not computed).
 *   B, H, total_q, total_k, max_seqlen_q >= 0; d in {64, 128}; one head's rows of q, o, k or v
 *   below 2^31 bytes. B*H*total_q == 0 or max_seqlen_q == 0 is a valid no-op.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int total_q, int total_k, int max_seqlen_q, int d, float scale,
                  int window_left, int window_right, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, void* stream);

/*
 * fa_bwd -- backward pass of fa_fwd: the gradients dq, dk, dv of O for an upstream gradient
 * dout, recomputing S and P tile by tile from q, k and the forward's lse instead of storing P
 * (training needs this recomputation: page "FlashAttention：把注意力从公式写成数据流", section
 * "用实验验证而不是背诵结论"; page "[2205.14135] FlashAttention ...", section "三、FLOPs"). With
 * D_i = dout_i . o_i, per allowed pair (i, j): P_ij = exp(scale q_i.k_j - lse_i),
 * dv_j += P_ij dout_i, dS_ij = P_ij (dout_i . v_j - D_i), dq_i += scale dS_ij k_j,
 * dk_j += scale dS_ij q_i. Keys at or past L_b get dk = dv = 0; rows without keys get dq = 0.
 *   q, k, v, o, dout, dq, dk, dv: bf16 in the fa_fwd layouts ([B][H][Nq or Nk][d]); lse: the fp32
 *   [B][H][Nq] fa_fwd wrote for the same inputs, scale, mask and lengths. Arguments as for fa_fwd
 *   (any Nq). bf16 products on the matrix cores with fp32 accumulation; P and dS rounded to bf16
 *   before their products; gradients rounded to bf16 once. Deterministic (no atomics). A
 *   workspace of 4*B*H*Nq bytes is allocated and freed stream-ordered on `stream`. With Nq == 0
 *   and B*H*Nk > 0, dk and dv are written as zeros, and k, v, dk and dv must then be valid
 *   (non-null, 16-byte aligned).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d,
           float scale, int causal, const int32_t* kv_seqlens, void* stream);

/*
 * fa_std_fwd -- the same bf16 operation computed by the standard, materialising algorithm, the
 * baseline the tiled path is measured against (page "FlashAttention：把注意力从公式写成数据流",
 * opening paragraph: S = Q K^T is written to device memory, read back for the softmax, and P is
 * written and read again for P V). Three kernels: S = scale * Q K^T over the full Nq x Nk grid in
 * fp32; a row softmax that applies the mask, writes P as bf16 (0 where masked) and lse; O = P V
 * over all Nk keys with fp32 accumulation, O rounded to bf16 once.
 *   Same arguments and rules as fa_fwd (any Nq, including 1, runs these kernels), plus:
 *   workspace        device memory owned by the caller, 256-byte aligned, at least
 *                    fa_std_workspace_bytes(B, H, Nq, Nk) bytes (may be NULL when that is 0).
 *                    It receives S ([B][H][Nq][ld] fp32) followed by P ([B][H][Nq][ld] bf16),
 *                    ld = Nk rounded up to a multiple of 128; on return it holds S and P.
 *   workspace_bytes  its size; smaller than required -> FA_ERR_INVALID_ARGUMENT.
 *   One head's S must stay below 2^31 bytes (Nq * ld * 4), else FA_ERR_UNSUPPORTED.
 * As with fa_fwd, key rows at or past L_b are never read.
 */
int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               const int32_t* kv_seqlens, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_std_fwd needs: 6 * B * H * Nq * ld (0 if any size is <= 0). */
size_t fa_std_workspace_bytes(int B, int H, int Nq, int Nk);

/*
 * fa_quantize_fp8 -- e4m3 (OCP FP8: 4 exponent bits with bias 7, 3 mantissa bits, largest finite
 * 448) quantisation of a bf16 tensor for fa_fwd_fp8. FP8 halves the bytes the forward pass moves
 * and doubles the matrix-core rate, at the cost of a scaled conversion and, for V, a transpose
 * (page "FlashAttention：把注意力从公式写成数据流", sections "用实验验证而不是背诵结论" and
 * "精度、掩码和边界情况"). One scale per (b, h) slice: s = amax / 448 in fp32 over the slice's
 * valid rows (rows at or past lens[b], clamped to [0, N], are excluded and stored as zero), s = 1
 * for an all-zero slice; element x becomes e4m3(x / s), the quotient a correctly rounded fp32
 * division and the conversion round-to-nearest-even. The values must be finite.
 *   x        bf16 [B][H][N][d], 16-byte aligned.
 *   y        e4m3 codes, 16-byte aligned: [B][H][N][d] when transpose == 0; the transpose
 *            [B][H][d][fa_fp8_vt_cols(N)] when transpose == 1 (padding columns zero).
 *   descale  fp32 [B*H], receives s per slice (dequantised value = s * e4m3 value).
 *   lens     int32 [B] or NULL (all N rows valid). d in {64, 128}; N * d < 2^31; transposed
 *            N <= 4194240.
 * A workspace of 4 * B * H * min(64, max(1, N*d/32768)) bytes is allocated and freed
 * stream-ordered on `stream`. Errors as for fa_fwd.
 */
int fa_quantize_fp8(const void* x, void* y, float* descale, int B, int H, int N, int d,
                    const int32_t* lens, int transpose, void* stream);

/* Columns of a transposed e4m3 V: Nk rounded up to a multiple of 64 (0 if Nk <= 0). */
int fa_fp8_vt_cols(int Nk);

/*
 * fa_fwd_fp8 -- the attention forward of fa_fwd on e4m3 inputs (from fa_quantize_fp8): the
 * result is that of fa_fwd's definition on the dequantised values s_q * q8, s_k * k8, s_v * v8,
 * except that the probabilities are rounded to e4m3 (after scaling by 8) for the P V product, a
 * weight error of at most 2^-4 P_ij + 2^-13 / l_i per pair (l_i = sum_j exp(S_ij - max_j S_ij)).
 * Arithmetic: e4m3 x e4m3 products on the matrix cores with fp32 accumulation, softmax and the
 * normaliser in fp32 (from the unrounded probabilities), O rounded to bf16 once.
 *   q8       e4m3 [B][H][Nq][d]     k8  e4m3 [B][H][Nk][d]
 *   vt8      e4m3 V^T [B][H][d][fa_fp8_vt_cols(Nk)]; it must hold no NaN code (0x7F, 0xFF) in
 *            any column, padding included (fa_quantize_fp8 writes zeros there).
 *   descale_q, descale_k, descale_v  fp32 [B*H] slice scales, or NULL for 1.
 *   o        bf16 [B][H][Nq][d];    lse fp32 [B][H][Nq] (natural log, of the dequantised scores).
 *   Other arguments and rules as for fa_fwd; q8, k8, vt8, o 16-byte aligned; one head's q8, k8
 *   and vt8 below 2^31 bytes. Key rows of k8 at or past L_b are never read.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* descale_q,
               const float* descale_k, const float* descale_v, void* o, float* lse,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               const int32_t* kv_seqlens, void* stream);

/* Static description of a status code (never NULL). */
const char* fa_status_string(int status);

/* Detail of the last failed call on this host thread ("" if none). */
const char* fa_last_error(void);

/* Static text naming the compiler and HIP headers the library was built with and its device
 * target, so a measurement can record what produced the code it timed (never NULL; no GPU call). */
const char* fa_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
