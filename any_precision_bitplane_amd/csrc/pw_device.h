// Device-side building blocks shared by the libpagedweight kernels (gfx950).
//
// Bit planes of a block (N rows, K columns, W = K/32 words per row): bit j of
// word (p, n, c) is plane p (plane 0 = most significant) of weight
// (n, 32c + j).  The code of a weight at bitwidth q is the value of its first
// q planes; its weight is the row's fp16 table entry for that code
// ("Technical summary: PagedWeight", Core components 1).  The kernels read the
// device layout described below (written by pw_pack_planes).
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
// Device plane layout.
//
// Planes stay outermost, so a block at bitwidth q is the prefix of its first
// q planes, and a plane holds exactly N W words.  Inside a plane the words
// sit in tiles of 16 device rows by 16 words, tile-row-major; inside a tile
// the 16 rows follow each other, each holding the tile's words (16, or
// W mod 16 in the last column tile):
//   word (d, c) -> (d >> 4) 16 W + (c >> 4) 256 + (d & 15) wct(c) + (c & 15),
//   wct(c) = min(16, W - (c & ~15)).
// So 16 rows x 16 words (512 weights per row) are one contiguous 1 KB piece,
// and the 16 words of one row are 64 contiguous bytes.  In a gate_up block
// (N = 2I) the device rows interleave gate and up: tile t holds gate rows
// 8t .. 8t+7 and then the matching up rows I + 8t .. I + 8t + 7, so every
// tile carries both halves SwiGLU needs.  Down blocks keep their row order.
// Requires N % 16 == 0 and, for gate_up, I % 8 == 0.
// ---------------------------------------------------------------------------
__host__ __device__ inline int dev_row_of_gate(int i) { return ((i >> 3) << 4) + (i & 7); }
__host__ __device__ inline int dev_row_of_up(int i) { return ((i >> 3) << 4) + 8 + (i & 7); }

// canonical row n of a block -> device row (gu: gate_up block with I = N / 2)
__host__ __device__ inline int dev_row(int n, int I, bool gu) {
  return !gu ? n : (n < I ? dev_row_of_gate(n) : dev_row_of_up(n - I));
}

// device row d -> canonical row
__host__ __device__ inline int canon_row(int d, int I, bool gu) {
  if (!gu) return d;
  const int t = d >> 4, r = d & 15;
  return r < 8 ? 8 * t + r : I + 8 * t + (r - 8);
}

// words per row in the column tile of word c
__host__ __device__ inline uint32_t tile_width(int c, int W) {
  const int rest = W - (c & ~15);
  return (uint32_t)(rest < 16 ? rest : 16);
}

// word offset of (device row d, word c) inside one plane
__host__ __device__ inline uint32_t dev_word(int d, int c, int W) {
  return (uint32_t)(d >> 4) * 16u * (uint32_t)W + (uint32_t)(c >> 4) * 256u + (uint32_t)(d & 15) * tile_width(c, W) +
         (uint32_t)(c & 15);
}

// ---------------------------------------------------------------------------
// Bit-plane -> code fields.
//
// The q plane words of one row hold 32 weights.  We transpose the q x 32 bit
// matrix inside each byte lane with three block-swap levels (the recursive 8x8
// bit transpose, run on four byte lanes at once; the levels commute, so each
// bitwidth uses the order that needs the fewest instructions given which input
// registers are zero).  Input register R[r] supplies field bit r; after the
// transpose, byte b of R[c] is the field of weight 8b + c.
//
// For q <= 7 plane p goes to field bit q - p, so the field is 2*code: the byte
// offset of the entry in an fp16 table.  For q = 8 the field is the code itself
// (2*code needs 9 bits) and the address step doubles it.
// ---------------------------------------------------------------------------

// v_bfi_b32: (a & m) | (b & ~m).  Written out because the compiler tends to
// expand it into and/and/or.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "s"(m), "v"(a), "v"(b));
  return d;
}

template <int S>
__device__ __forceinline__ constexpr uint32_t level_mask() {
  return S == 4 ? 0xF0F0F0F0u : S == 2 ? 0xCCCCCCCCu : 0xAAAAAAAAu;
}

// One swap level on rows r and r+S (r & S == 0), with compile-time knowledge of
// which rows are still all-zero (bit r of Z).  Returns the new zero set.
template <int S, unsigned Z>
__host__ __device__ constexpr unsigned level_zero_after() {
  unsigned z = Z;
  for (int r = 0; r < 8; ++r)
    if ((r & S) == 0) {
      const bool both = ((Z >> r) & 1u) && ((Z >> (r + S)) & 1u);
      z = both ? (z | (1u << r) | (1u << (r + S))) : (z & ~(1u << r) & ~(1u << (r + S)));
    }
  return z;
}

template <int S, unsigned Z>
__device__ __forceinline__ void swap_level(uint32_t (&R)[8]) {
  constexpr uint32_t H = level_mask<S>();
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if ((r & S) != 0) continue;
    const bool za = (Z >> r) & 1u, zb = (Z >> (r + S)) & 1u;
    const uint32_t a = R[r], b = R[r + S];
    if (za && zb) continue;
    if (za) {
      R[r] = (b << S) & H;
      R[r + S] = b & H;
    } else if (zb) {
      R[r] = a & ~H;
      R[r + S] = (a >> S) & ~H;
    } else {
      R[r] = bfi(H, b << S, a);
      R[r + S] = bfi(H, b, a >> S);
    }
  }
}

// planes_to_fields in its parts: the inputs placed (fields_init), then swap
// level LV = 0, 1, 2 (fields_level), so a caller can spread the levels over
// other work.  Same instructions, same result.
template <int Q>
struct FieldsPlan {
  static constexpr unsigned Z0 = Q == 8 ? 0u : (0xFFu & ~(((1u << Q) - 1u) << 1));
  // level orders with the fewest instructions for each zero pattern
  static constexpr int L0 = (Q == 3) ? 2 : (Q == 5) ? 1 : (Q == 4) ? 2 : 4;
  static constexpr int L1 = (Q == 3) ? 1 : (Q == 5) ? 4 : (Q == 4) ? 1 : 2;
  static constexpr int L2 = (Q == 3) ? 4 : (Q == 5) ? 2 : (Q == 4) ? 4 : 1;
  static constexpr unsigned Z1 = level_zero_after<L0, Z0>();
  static constexpr unsigned Z2 = level_zero_after<L1, Z1>();
};

template <int Q>
__device__ __forceinline__ void fields_init(const uint32_t (&P)[Q], uint32_t (&R)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) R[r] = 0u;
#pragma unroll
  for (int p = 0; p < Q; ++p) {
    if constexpr (Q == 8) R[7 - p] = P[p];
    else R[Q - p] = P[p];
  }
}

template <int Q, int LV>
__device__ __forceinline__ void fields_level(uint32_t (&R)[8]) {
  using F = FieldsPlan<Q>;
  if constexpr (LV == 0) swap_level<F::L0, F::Z0>(R);
  else if constexpr (LV == 1) swap_level<F::L1, F::Z1>(R);
  else swap_level<F::L2, F::Z2>(R);
}

template <int Q>
__device__ __forceinline__ void planes_to_fields(const uint32_t (&P)[Q], uint32_t (&R)[8]) {
  fields_init<Q>(P, R);
  fields_level<Q, 0>(R);
  fields_level<Q, 1>(R);
  fields_level<Q, 2>(R);
}

// Byte B of r added to base (one SDWA instruction).
template <int B>
__device__ __forceinline__ uint32_t add_byte(uint32_t base, uint32_t r) {
  uint32_t d;
  if constexpr (B == 0)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(d) : "v"(base), "v"(r));
  else if constexpr (B == 1)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(d) : "v"(base), "v"(r));
  else if constexpr (B == 2)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(d) : "v"(base), "v"(r));
  else
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(d) : "v"(base), "v"(r));
  return d;
}

// 2 * byte B of r (one SDWA instruction).
template <int B>
__device__ __forceinline__ uint32_t twice_byte(uint32_t r) {
  uint32_t d;
  if constexpr (B == 0)
    asm("v_add_u32_sdwa %0, %1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:BYTE_0"
        : "=v"(d) : "v"(r));
  else if constexpr (B == 1)
    asm("v_add_u32_sdwa %0, %1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:BYTE_1"
        : "=v"(d) : "v"(r));
  else if constexpr (B == 2)
    asm("v_add_u32_sdwa %0, %1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:BYTE_2"
        : "=v"(d) : "v"(r));
  else
    asm("v_add_u32_sdwa %0, %1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:BYTE_3"
        : "=v"(d) : "v"(r));
  return d;
}

// LDS byte address of weight J's table entry: base + 2*code.
template <int Q, int J>
__device__ __forceinline__ uint32_t entry_addr(const uint32_t (&R)[8], uint32_t base) {
  if constexpr (Q == 8) return base + twice_byte<(J >> 3)>(R[J & 7]);
  else return add_byte<(J >> 3)>(base, R[J & 7]);
}

typedef const __attribute__((address_space(3))) uint16_t* lds_u16_ptr;
typedef __attribute__((address_space(3))) uint8_t* lds_u8_ptr;

__device__ __forceinline__ uint32_t lds_u16_at(uint32_t addr) { return *(lds_u16_ptr)(size_t)addr; }

// 32-bit LDS address of a location inside a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(lds_u8_ptr)(const_cast<void*>(p));
}

// Weights J, J+1 (J even) of the group, looked up in the row table whose LDS
// address is `base`, packed as an fp16 pair.
template <int Q, int J>
__device__ __forceinline__ half2_t lookup_pair(const uint32_t (&R)[8], uint32_t base) {
  const uint32_t lo = lds_u16_at(entry_addr<Q, J>(R, base));
  const uint32_t hi = lds_u16_at(entry_addr<Q, J + 1>(R, base));
  return __builtin_bit_cast(half2_t, lo | (hi << 16));
}

// Row tables kept at a 256-byte LDS stride (512 for q = 8): for q <= 7 the
// field byte is 2 * code, so an entry's address is the table base with its
// low byte replaced by the field (one v_perm_b32); for q = 8 the field is the
// code and the address is base + 2 * code.
template <int Q>
constexpr int kTabStride = Q == 8 ? 512 : 256;

template <int Q>
__device__ __forceinline__ uint32_t tab_entry(const uint32_t (&R)[8], uint32_t base, int j) {
  const uint32_t f = R[j & 7];
  const int b = j >> 3;
  if constexpr (Q == 8) return base + (((f >> (8 * b)) & 0xFFu) << 1);
  else return __builtin_amdgcn_perm(base, f, 0x07060500u | (uint32_t)b);
}

// The 32 weights of one group (fields R, row table at `base`, kTabStride
// aligned) as 16 packed fp16 pairs: pair p = weights (2p, 2p + 1).  The
// lookups go out in batches of eight (one sub-step's weights 8b .. 8b + 7)
// ahead of the packing, so the wave waits on LDS about once per batch.
template <int Q>
__device__ __forceinline__ void decode_group(const uint32_t (&R)[8], uint32_t base, uint32_t (&packed)[16]) {
  uint32_t v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = lds_u16_at(tab_entry<Q>(R, base, j));
#pragma unroll
  for (int p = 0; p < 16; ++p) packed[p] = v[2 * p] | (v[2 * p + 1] << 16);
  constexpr int kValu = 0x002, kDsRead = 0x100;
  constexpr int kAddrOps = Q == 8 ? 2 : 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(kValu, 8 * kAddrOps, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 8, 0);
  }
}

// Decode of one row's 32-weight group into 16 fp16 pairs.
template <int Q, int J>
struct GroupDecode {
  __device__ static __forceinline__ void run(const uint32_t (&R)[8], uint32_t base, uint32_t (&out)[16]) {
    out[J >> 1] = __builtin_bit_cast(uint32_t, lookup_pair<Q, J>(R, base));
    GroupDecode<Q, J + 2>::run(R, base, out);
  }
};
template <int Q>
struct GroupDecode<Q, 32> {
  __device__ static __forceinline__ void run(const uint32_t (&)[8], uint32_t, uint32_t (&)[16]) {}
};

// Buffer resource over [base, base + bytes): loads past the end return 0, which
// is how out-of-range rows and columns read as zero without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset that reads as zero

// z * sigmoid(z) with the hardware reciprocal (1 ulp) in place of a division.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Weighted top-k combine of token t at hidden positions n .. n+3:
// sum over j < k, ascending, of w[t][j] * o[t k + j][n ..] (each o row the sum
// of its K parts), fp32 fused multiply-adds; dropped slots (inv < 0) add
// nothing.  Every loaded value of a group of eight slots is requested before
// any is used.  The one definition every kernel that combines uses, so their
// results agree bit for bit.
__device__ __forceinline__ floatx4 combine4(const float* __restrict__ o, const float* __restrict__ w,
                                            const int32_t* __restrict__ inv, int t, int k, int H, int kparts,
                                            size_t part_stride, int n) {
  constexpr int G = 8;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j0 = 0; j0 < k; j0 += G) {
    bool ok[G];
    float wj[G];
    floatx4 v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int j = j0 + i;
      ok[i] = false;
      wj[i] = 0.f;
      v[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (j < k) {
        const size_t slot = (size_t)t * k + j;
        ok[i] = inv[slot] >= 0;
        wj[i] = w[slot];
        v[i] = *reinterpret_cast<const floatx4*>(o + slot * H + n);
        for (int kp = 1; kp < kparts; ++kp)
          v[i] += *reinterpret_cast<const floatx4*>(o + kp * part_stride + slot * H + n);
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (!ok[i]) continue;
      a0 = __builtin_fmaf(wj[i], v[i][0], a0);
      a1 = __builtin_fmaf(wj[i], v[i][1], a1);
      a2 = __builtin_fmaf(wj[i], v[i][2], a2);
      a3 = __builtin_fmaf(wj[i], v[i][3], a3);
    }
  }
  return floatx4{a0, a1, a2, a3};
}

// Four fp32 values rounded to fp16 (nearest even), packed little-endian.
__device__ __forceinline__ uint2 pack_half4(floatx4 a) {
  const _Float16 h0 = (_Float16)a[0], h1 = (_Float16)a[1], h2 = (_Float16)a[2], h3 = (_Float16)a[3];
  uint2 p;
  p.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  p.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
  return p;
}

// Values the kernels load from memory at a wave-uniform address are the same
// in every lane, but the compiler cannot always prove it (it must use a vector
// load when the memory may be written during the kernel).  These helpers say
// so, which keeps descriptors in scalar registers and branches uniform.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Workspace status word: set bits, never cleared by kernels of the forward.
__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bits) {
  atomicOr(status, bits);
}

}  // namespace pw
