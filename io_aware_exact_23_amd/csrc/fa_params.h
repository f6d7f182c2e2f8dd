// fa_params.h -- plain argument blocks passed by value to the libfa kernels (host and device).
#pragma once

#include <stdint.h>

namespace fa {

// Tiled forward (prefill) kernels, bf16 and fp32. Element pointers are typed by the kernel.
struct PrefillParams {
  const void* q;  // [B][H][Nq][D]
  const void* k;  // [B][H][Nk][D]
  const void* v;  // [B][H][Nk][D]
  void* o;        // [B][H][Nq][D]
  float* lse;     // [B][H][Nq]
  const int32_t* kv_seqlens;  // [B] or nullptr
  int B, H, Nq, Nk;
  float c;        // scale * log2(e): scores are handled in base-2 units
  int causal;
  int n_qtiles;   // ceil(Nq / BM)
  int n_tiles;    // B * H * n_qtiles (the grid size)
  int cus_per_xcd;  // compute units per XCD of the device (0 if unknown)
  // Generalised masks and layouts (the window / packed-sequence entry points only).
  int win_left, win_right;    // key j allowed for query i iff i-left <= j <= i+right; -1: no limit
  const int32_t* cu_q;        // packed sequences: [B+1] row offsets of each sequence, or nullptr
  const int32_t* cu_k;        //   (then q, o are [H][Tq][D], k, v [H][Tk][D], lse [H][Tq])
  int Tq, Tk;                 // packed sequences: rows per head
};

// Split-KV decode (Nq == 1): one workgroup per (split, h, b), then a combine pass.
struct DecodeParams {
  const uint16_t* q;  // [B][H][1][D] bf16
  const uint16_t* k;  // [B][H][Nk][D] bf16
  const uint16_t* v;  // [B][H][Nk][D] bf16
  uint16_t* o;        // [B][H][1][D] bf16
  float* lse;         // [B][H]
  const int32_t* kv_seqlens;
  float* ws_o;        // [B][H][n_splits][D]  normalised partial outputs, fp32
  float* ws_lse;      // [B][H][n_splits]     partial logsumexp in base-2 units
  int B, H, Nk;
  int n_splits;       // ceil(Nk / CHUNK)
  float c;            // scale * log2(e)
};

// Backward pass: gradients of the forward for an upstream gradient dO (all bf16 but lse).
struct BackwardParams {
  const void* q;     // [B][H][Nq][D]
  const void* k;     // [B][H][Nk][D]
  const void* v;     // [B][H][Nk][D]
  const void* o;     // [B][H][Nq][D] forward output
  const void* dout;  // [B][H][Nq][D] upstream gradient
  const float* lse;  // [B][H][Nq] forward logsumexp (natural log)
  void* dq;          // [B][H][Nq][D]
  void* dk;          // [B][H][Nk][D]
  void* dv;          // [B][H][Nk][D]
  const int32_t* kv_seqlens;
  float* delta;      // [B][H][Nq] workspace: D_i = dO_i . O_i
  int B, H, Nq, Nk;
  float scale;
  int causal;
};

// Standard (materialising) attention: S = scale * Q K^T and P = softmax(S) both go to device
// memory, then O = P V. Rows of S and P are ld elements apart (ld = Nk rounded up to 64).
struct StandardParams {
  const void* q;  // [B][H][Nq][D] bf16
  const void* k;  // [B][H][Nk][D] bf16
  const void* v;  // [B][H][Nk][D] bf16
  void* o;        // [B][H][Nq][D] bf16
  float* lse;     // [B][H][Nq]
  const int32_t* kv_seqlens;  // [B] or nullptr
  float* s;       // [B][H][Nq][ld] fp32 scores
  uint16_t* pm;   // [B][H][Nq][ld] bf16 probabilities
  int B, H, Nq, Nk, ld;
  float scale;
  int causal;
};

// e4m3 quantisation of a bf16 tensor with one scale per (b, h) slice (rows of the slice past
// its sequence's length are excluded from the scale and stored as zero).
struct QuantParams {
  const uint16_t* x;      // [B][H][N][D] bf16
  uint8_t* y;             // [B][H][N][D] e4m3, or [B][H][D][cols] when transpose
  float* descale;         // [B*H] the scale s of each slice
  float* partial;         // [B*H][n_chunks] workspace: amax of each chunk of rows
  const int32_t* lens;    // [B] valid rows per sequence, or nullptr
  int B, H, N, D;
  int cols;               // transposed row length: N rounded up to 64
  int n_chunks;           // row chunks per slice for the amax pass (1..64)
  int rows_per_chunk;
  int transpose;
};

// FP8 (e4m3) forward: Q, K as [B][H][N][D] codes, V as V^T [B][H][D][ldv] codes, one scale per
// (b, h) slice of each; output and lse as in the bf16 forward.
struct PrefillFp8Params {
  const uint8_t* q;       // [B][H][Nq][D]
  const uint8_t* k;       // [B][H][Nk][D]
  const uint8_t* vt;      // [B][H][D][ldv]
  const float* dq;        // [B*H] scales (nullptr: 1)
  const float* dk;
  const float* dv;
  void* o;                // [B][H][Nq][D] bf16
  float* lse;             // [B][H][Nq]
  const int32_t* kv_seqlens;
  int B, H, Nq, Nk, ldv;
  float c;                // scale * log2(e)
  int causal;
  int n_qtiles, n_tiles;
};

}  // namespace fa
