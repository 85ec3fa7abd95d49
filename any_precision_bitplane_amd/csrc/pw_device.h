// Device-side building blocks shared by the libpagedweight kernels (gfx950).
//
// Storage format of a block (N rows, K columns, W = K/32 words per row):
// plane-major uint32 [8][N][W]; bit j of word [p][n][c] is plane p (plane 0 =
// most significant) of weight (n, 32c + j).  The code of a weight at bitwidth
// q is the value of its first q planes; its weight is the row's fp16 table
// entry for that code ("Technical summary: PagedWeight", Core components 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__host__ __device__ constexpr int lut_offset(int N, int b) { return N * ((1 << b) - 8); }

// ---------------------------------------------------------------------------
// Bit-plane -> code fields.
//
// The q plane words of one row hold 32 weights.  We transpose the q x 32 bit
// matrix inside each byte lane with three block-swap levels (4, 2, 1), the
// classic recursive 8x8 bit transpose run on four byte lanes at once.  Input
// register R[r] supplies field bit r; after the transpose, byte b of R[c] is
// the field of weight 8b + c.
//
// For q <= 7 plane p goes to field bit q - p, so the field is 2*code: the byte
// offset of the entry in an fp16 table.  For q = 8 the field is the code itself
// (2*code needs 9 bits) and the caller doubles it.
// ---------------------------------------------------------------------------
template <int S>
__device__ __forceinline__ void swap_level(uint32_t (&R)[8], uint32_t hi) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if ((r & S) == 0) {
      const uint32_t a = R[r], b = R[r + S];
      R[r] = (a & ~hi) | ((b << S) & hi);
      R[r + S] = (b & hi) | ((a >> S) & ~hi);
    }
  }
}

template <int Q>
__device__ __forceinline__ void planes_to_fields(const uint32_t (&P)[Q], uint32_t (&R)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) R[r] = 0u;
#pragma unroll
  for (int p = 0; p < Q; ++p) {
    if constexpr (Q == 8) R[7 - p] = P[p];
    else R[Q - p] = P[p];
  }
  swap_level<4>(R, 0xF0F0F0F0u);
  swap_level<2>(R, 0xCCCCCCCCu);
  swap_level<1>(R, 0xAAAAAAAAu);
}

// Byte offset into an fp16 table of the weight at position j (0..31) of the
// word group, given the transposed fields.
template <int Q>
__device__ __forceinline__ uint32_t field_offset(const uint32_t (&R)[8], int j) {
  const uint32_t f = (R[j & 7] >> (8 * (j >> 3))) & 0xFFu;
  if constexpr (Q == 8) return f << 1;
  else return f;
}

__device__ __forceinline__ uint32_t lds_u16(const uint8_t* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint16_t*>(base + byte_off);
}

// Weights j, j+1 (j even) of the 32-weight group, looked up in the row table
// and packed as (w_j, w_j+1) fp16 pair.
template <int Q>
__device__ __forceinline__ half2_t lookup_pair(const uint32_t (&R)[8], const uint8_t* tab, int j) {
  const uint32_t lo = lds_u16(tab, field_offset<Q>(R, j));
  const uint32_t hi = lds_u16(tab, field_offset<Q>(R, j + 1));
  return __builtin_bit_cast(half2_t, lo | (hi << 16));
}

// Buffer resource over [base, base + bytes): loads past the end return 0, which
// is how out-of-range rows and columns read as zero without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset that reads as zero

// ---------------------------------------------------------------------------
// Wave-wide sum (all lanes get the result).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Workspace status word: set bits, never cleared by kernels of the forward.
__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bits) {
  atomicOr(status, bits);
}

}  // namespace pw
