// Dequant-to-LDS MFMA kernels for experts with many tokens (prefill).
// "Technical summary: PagedWeight", Core components 3 (fused mixed-precision
// kernel): each block is read at its own committed bitwidth q from the device
// page table; here the decoded weights feed the matrix cores instead of a
// GEMV, because with hundreds of tokens per expert the product is a dense
// contraction.
//
// Tile: 512 tokens x 128 device rows (eight 16-row tiles of the device
// layout) per workgroup of four waves, one per SIMD; each wave multiplies
// 128 tokens by all 128 rows (a 128 x 128 fp32 accumulator, 256 registers,
// v_mfma_f32_16x16x32_f16), so every weight decoded into LDS feeds 512
// tokens and every LDS byte of it feeds 128 tokens of one wave.
//   * Weights: every thread decodes one 32-weight plane word per K step (its
//     q plane words transposed into code fields, looked up in the row's table
//     in LDS) into a double-buffered fp16 B tile in LDS; the decode of step
//     k + 1 runs while the matrix cores work on step k.
//   * Activations: a wave's token rows are read only by that wave, so they
//     go straight from memory into the A operand registers, one 32-wide
//     sub-step ahead; no LDS, and LDS bandwidth is left to the decode and the
//     B operand.
// K order.  A K step is two plane words per row; which K positions a step
// holds is free as long as the A and B operands agree.  Thread (row r, half
// h) loads plane words 8 Q + 4 h .. +4 of its row for a quad Q of four steps
// (one 16-byte load per plane: the device layout keeps a row's 16-word run
// contiguous) and decodes word 8 Q + 4 h + j at step j of the quad into slot
// h of the B tile; sub-step h of the step multiplies slot h with the
// activations of the same word.
// gate_up tiles hold 8 gate rows and their 8 up rows per 16-row tile (the
// device layout's interleave), so SwiGLU pairs MFMA columns n and n + 8.
//
// Work items are (token tile, row tile) pairs; token tiles come from the route
// kernel's list.  The items are dealt evenly over the 8 XCDs, a run of
// consecutive items each, which sweeps the row tiles of one token tile, so its
// activation rows stay in that XCD's L2.
#include <type_traits>

#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfTM = kMfmaTileM;        // tokens per tile
constexpr int kPfWM = kPfTM / kPfWaves;  // tokens per wave
static_assert(kPfWM == 128, "eight 16-token groups per wave");
constexpr int kPfTN = 128;               // device rows per tile
constexpr int kPfTileGroup = 2;          // token tiles whose items of one row tile run together
constexpr int kPfTG = kPfWM / 16;        // token groups per wave
constexpr int kPfRG = kPfTN / 16;        // row groups
constexpr int kPfBStride = 2 * 64 + 16;  // bytes per B-tile row: 64 fp16 of one step + pad (conflict-free reads)
constexpr int kPfBBytes = kPfTN * kPfBStride;
constexpr int kPfTabBytes = kPfTN * 512; // row tables: 256-byte slots (q <= 7) or 512 (q = 8)
constexpr int kPfLds = kPfTabBytes + 2 * kPfBBytes;
constexpr int kXcds = 8;

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(3))) u32x4v* lds_u4c;
typedef __attribute__((address_space(3))) u32x4v* lds_u4;
typedef const __attribute__((address_space(3))) _Float16* lds_f16c;

__device__ __forceinline__ _Float16 lds_f16_at(uint32_t addr) { return *(lds_f16c)(size_t)addr; }

// True, but the compiler cannot see it: code under `if (always_true())` is a
// basic block of its own, and the compiler schedules within basic blocks.
__device__ __forceinline__ bool always_true() {
  int v = 1;
  asm volatile("" : "+s"(v));
  return v != 0;
}

struct MfmaArgs {
  int H, I, E, k, T;
  const pw_block_desc* blocks;
  const uint8_t* q;
  Route rt;
  const uint16_t* act;   // gate_up: x [T][H]; down: h [slots][I]
  uint16_t* hout;        // gate_up output
  float* oout;           // down output
  int ntiles;            // row tiles per block
  int kparts;            // parts of the K range (down product), each its own items and o slice
  size_t part_stride;    // floats between the o slices of two parts
  uint32_t act_bytes;    // activation bytes (< 2^31): out-of-range offsets read zero
};

template <int Q, bool GU>
__device__ __forceinline__ void pf_tile(const MfmaArgs& A, int e, int n_e, int off_e, int m0, int nt, int part,
                                        uint8_t* lds) {
  constexpr int TAB = (1 << Q) * 2;
  constexpr int TSTRIDE = kTabStride<Q>;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int H = A.H, I = A.I;
  const int N = GU ? 2 * I : H;
  const int K = GU ? H : I;
  const int W = K >> 5;
  // K part `part` of A.kparts: quads [q0, q0 + nq) of the row's eight-word
  // quads, words [w0, w1)
  const int nqa = (W + 7) >> 3;
  const int nqp = (nqa + A.kparts - 1) / A.kparts;
  const int q0 = part * nqp;
  const int nq = nqa - q0 < nqp ? (nqa - q0 > 0 ? nqa - q0 : 0) : nqp;
  const int w0 = 8 * q0;
  const int w1 = w0 + 8 * nq < W ? w0 + 8 * nq : W;
  const int nsteps = 4 * nq;
  const int nm = n_e - m0 < kPfTM ? n_e - m0 : kPfTM;

  uint8_t* tabs = lds;
  uint8_t* btile = lds + kPfTabBytes;

  const pw_block_desc d = A.blocks[2 * e + (GU ? 0 : 1)];
  const uint32_t pstride = (uint32_t)N * (uint32_t)W * 4u;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(uniform_ptr(d.planes), pstride * (uint32_t)Q);
  const uint16_t* __restrict__ lut = uniform_ptr(d.lut_all) + lut_offset(N, Q);

  // Row tables -> LDS: tile row r in a TSTRIDE slot; a table smaller than its
  // slot sits at byte offset skew(r) = TAB * r mod 256 of it, applied as an
  // XOR (entry c at byte 2c ^ skew(r)), which spreads the 16 rows of a
  // half-wave's lookups over the LDS banks.  Direct buffer-to-LDS loads.
  auto skew_of = [&](int r) -> uint32_t { return TAB < 256 ? (uint32_t)((TAB * r) & 255) : 0u; };
  {
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lut, (uint32_t)N * (uint32_t)TAB);
    constexpr int NI = kPfTN * TSTRIDE / 1024;
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += kPfWaves) {
      const int i = i0 + wave;
      const int pos = 1024 * i + 16 * lane;
      const int r = pos / TSTRIDE;
      const int chunk = (pos % TSTRIDE) / 16 ^ (int)(skew_of(r) >> 4);
      const int crow = canon_row(kPfTN * nt + r, I, GU);
      const uint32_t voff =
          (16 * chunk < TAB && crow < N) ? (uint32_t)crow * (uint32_t)TAB + 16u * (uint32_t)chunk : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)(tabs + 1024 * i), 16,
                                               voff, 0, 0, 0);
    }
  }

  // Decode job: tile row r, half h.
  const int r = tid >> 1, h = tid & 1;
  const int drow = kPfTN * nt + r;
  const uint32_t tbase = lds_addr(tabs) + (uint32_t)(r * TSTRIDE);
  const uint32_t skew4 = skew_of(r) * 0x01010101u;
  const bool vec = (W & 3) == 0;
  auto load_quad = [&](uint32_t (&P)[Q][4], int qd) {
    const int wd = w0 + 8 * qd + 4 * h;
    const bool live = qd < nq && wd < w1 && drow < N;
    const uint32_t voff = live ? dev_word(drow, wd, W) * 4u : kOutOfRange;
    if (vec) {
#pragma unroll
      for (int p = 0; p < Q; ++p) {
        const uint4 v = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(prs, (int)voff, (int)((uint32_t)p * pstride), 0));
        P[p][0] = v.x; P[p][1] = v.y; P[p][2] = v.z; P[p][3] = v.w;
      }
    } else {
#pragma unroll
      for (int p = 0; p < Q; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          P[p][i] = buf_load_u32(prs, (live && wd + i < w1) ? dev_word(drow, wd + i, W) * 4u : kOutOfRange,
                                 (uint32_t)p * pstride);
    }
  };
  // Decode of one plane word into B-tile buffer `buf`, slot h, in parts that
  // the steps spread over their pieces: the fields (inputs placed, three
  // swap levels, the bank skew); the LDS addresses of the eight lookups of
  // byte b of every field (weights 8 b .. 8 b + 7); those lookups; packing
  // them into fp16 pairs 4 b .. 4 b + 3; the stores.
  uint32_t R[8];
  uint32_t la[8];
  uint32_t lv[4][8];
  uint32_t pk[16];
  auto fields_in = [&](const uint32_t (&P)[Q][4], auto Jc) {
    constexpr int J = decltype(Jc)::value;
    uint32_t W8[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) W8[p] = P[p][J];
    fields_init<Q>(W8, R);
    fields_level<Q, 0>(R);
  };
  auto fields_out = [&]() {
    fields_level<Q, 2>(R);
    if constexpr (TAB < 256) {
#pragma unroll
      for (int c = 0; c < 8; ++c) R[c] ^= skew4;
    }
  };
  auto lookup_addrs = [&](int bb) {
#pragma unroll
    for (int c = 0; c < 8; ++c) la[c] = tab_entry<Q>(R, tbase, 8 * bb + c);
  };
  auto lookups = [&](int bb) {
#pragma unroll
    for (int c = 0; c < 8; ++c) lv[bb][c] = lds_u16_at(la[c]);
  };
  auto pack = [&](int bb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[4 * bb + i] = lv[bb][2 * i] | (lv[bb][2 * i + 1] << 16);
  };
  auto store_b = [&](int buf) {
    const uint32_t dst = lds_addr(btile + buf * kPfBBytes + r * kPfBStride + h * 64);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      *(lds_u4)(size_t)(dst + 16u * v) = u32x4v{pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]};
  };
  auto decode_all = [&](const uint32_t (&P)[Q][4], auto Jc, int buf) {
    fields_in(P, Jc);
    fields_level<Q, 1>(R);
    fields_out();
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      lookup_addrs(bb);
      lookups(bb);
      pack(bb);
    }
    store_b(buf);
  };

  // A operand: lane (m = lane & 15, g = lane >> 4) holds token 16 tg + m of
  // the wave's 128, K slots 8 g .. +8 of the sub-step's word.  Tokens past
  // the tile's end read row 0 (their accumulator rows are never stored);
  // words past the row's end read through an empty buffer (zeros).  The
  // word's offset is a scalar, so an activation load costs no vector
  // instruction.
  const int m = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A.act, A.act_bytes);
  const __amdgpu_buffer_rsrc_t ars0 = make_rsrc(A.act, 0u);
  uint32_t arow[kPfTG];
#pragma unroll
  for (int tg = 0; tg < kPfTG; ++tg) {
    const int mt = kPfWM * wave + 16 * tg + m;
    uint32_t row = 0;
    if (mt < nm) {
      const int pos = off_e + m0 + mt;
      row = GU ? (uint32_t)(A.rt.perm[pos] / A.k) * (uint32_t)A.H * 2u : (uint32_t)pos * (uint32_t)A.I * 2u;
    }
    arow[tg] = row + 16u * (uint32_t)g;
  }
  // sub-step s = 2 k + hh of step k: word 8 (k >> 2) + 4 hh + (k & 3)
  auto load_a = [&](u32x4v (&Ar)[kPfTG], int s) {
    const int k = s >> 1, hh = s & 1;
    const int wd = w0 + 8 * (k >> 2) + 4 * hh + (k & 3);
    const bool in = wd < w1;
    const __amdgpu_buffer_rsrc_t rs = in ? ars : ars0;
    const int woff = in ? 64 * wd : 0;
#pragma unroll
    for (int tg = 0; tg < kPfTG; ++tg)
      Ar[tg] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)arow[tg], woff, 0));
  };

  float4v acc[kPfTG][kPfRG];
#pragma unroll
  for (int i = 0; i < kPfTG; ++i)
#pragma unroll
    for (int j = 0; j < kPfRG; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  // B fragment of row group rg, sub-step hh, from buffer `buf`: lane (m, g)
  // holds row 16 rg + m, K slots 8 g .. +8.
  const uint32_t bbase = lds_addr(btile) + (uint32_t)(m * kPfBStride + 16 * g);
  auto read_b = [&](int buf, int hh, int rg) -> u32x4v {
    return *(lds_u4c)(size_t)(bbase + (uint32_t)(buf * kPfBBytes + 16 * rg * kPfBStride + hh * 64));
  };
  auto mma = [&](const u32x4v (&Ar)[kPfTG], const u32x4v& b, int rg) {
#pragma unroll
    for (int tg = 0; tg < kPfTG; ++tg)
      acc[tg][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8v, Ar[tg]),
                                                           __builtin_bit_cast(half8v, b), acc[tg][rg], 0, 0, 0);
  };
  constexpr int kMfma = 0x008, kValu = 0x002;

  // Prologue: planes of quads 0 and 1, activations of sub-step 0; tables in;
  // decode step 0 into buffer 0; the fields of step 1.
  uint32_t P0[Q][4], P1[Q][4];
  u32x4v A0[kPfTG], A1[kPfTG];
  load_quad(P0, 0);
  load_quad(P1, 1);
  load_a(A0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the tables and the first planes have landed
  __syncthreads();
  decode_all(P0, std::integral_constant<int, 0>{}, 0);
  fields_in(P0, std::integral_constant<int, 1>{});
  fields_level<Q, 1>(R);
  fields_out();
  __syncthreads();

  // Step k: products of sub-step 0 (A0) and sub-step 1 (A1) from buffer
  // k & 1; the decode of step k + 1 into the other buffer from the fields
  // computed in step k - 1; the fields of step k + 2 (after the last steps
  // this decodes zero planes into buffers nobody reads; plane and activation
  // loads past the end read zero).  Sixteen pieces, one per row group and
  // sub-step.  A piece first issues its memory operations (the next piece's
  // B fragment, the lookups of one byte, the B-tile stores, the activation
  // and plane loads), then, in a block of its own, its eight products
  // interleaved with a part of the decode's vector work (fields, lookup
  // addresses, packing), which so runs in the shadow of the matrix cores.
  // The block is a branch on an always-true value the compiler cannot see
  // through: the compiler keeps the pieces' order and their short register
  // lifetimes, and since no memory operation sits inside a block, both ways
  // around it leave the same loads in flight and the memory-counter waits
  // stay exact.
  // Word of step s: quad s >> 2, word s & 3 of it; quads alternate between
  // P0 (even) and P1 (odd).  A quad's registers take the quad two ahead once
  // the fields of its last word are done.  Unrolled over two quads so every
  // plane-register index is static.
  auto step = [&](auto Jf, uint32_t (&Pf)[Q][4], auto Ld, int k) {
    constexpr int JF = decltype(Jf)::value;   // word of step k + 2 inside its quad (held in Pf)
    constexpr bool LD = decltype(Ld)::value;  // JF == 3: Pf takes the quad two ahead afterwards
    const int cur = k & 1;
    u32x4v b = read_b(cur, 0, 0);
    auto piece = [&](auto Ic) {
      constexpr int I = decltype(Ic)::value;   // 0 .. 15: sub-step I / 8, row group I % 8
      constexpr int HH = I / 8, RG = I % 8;
      u32x4v bn = b;
      if constexpr (I < 15) bn = read_b(cur, (I + 1) / 8, (I + 1) % 8);
      if constexpr (I == 0) load_a(A1, 2 * k + 1);
      if constexpr (I >= 1 && I <= 4) lookups(I - 1);
      if constexpr (I == 6) store_b(cur ^ 1);
      if constexpr (I == 8) load_a(A0, 2 * k + 2);
      if constexpr (I == 11 && LD) load_quad(Pf, ((k + 2) >> 2) + 2);
      if (always_true()) {
        mma(HH == 0 ? A0 : A1, b, RG);
        if constexpr (I <= 3) lookup_addrs(I);
        if constexpr (I >= 2 && I <= 5) pack(I - 2);
        if constexpr (I == 8) fields_in(Pf, Jf);
        if constexpr (I == 9) fields_level<Q, 1>(R);
        if constexpr (I == 10) fields_out();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kValu, 3, 0);
        }
      }
      b = bn;
    };
    piece(std::integral_constant<int, 0>{});
    piece(std::integral_constant<int, 1>{});
    piece(std::integral_constant<int, 2>{});
    piece(std::integral_constant<int, 3>{});
    piece(std::integral_constant<int, 4>{});
    piece(std::integral_constant<int, 5>{});
    piece(std::integral_constant<int, 6>{});
    piece(std::integral_constant<int, 7>{});
    piece(std::integral_constant<int, 8>{});
    piece(std::integral_constant<int, 9>{});
    piece(std::integral_constant<int, 10>{});
    piece(std::integral_constant<int, 11>{});
    piece(std::integral_constant<int, 12>{});
    piece(std::integral_constant<int, 13>{});
    piece(std::integral_constant<int, 14>{});
    piece(std::integral_constant<int, 15>{});
    __syncthreads();
  };
  using std::integral_constant;
  using F = integral_constant<bool, false>;
  using T = integral_constant<bool, true>;
  for (int k0 = 0; k0 < nsteps; k0 += 8) {
    step(integral_constant<int, 2>{}, P0, F{}, k0);
    step(integral_constant<int, 3>{}, P0, T{}, k0 + 1);
    step(integral_constant<int, 0>{}, P1, F{}, k0 + 2);
    step(integral_constant<int, 1>{}, P1, F{}, k0 + 3);
    if (k0 + 4 >= nsteps) break;
    step(integral_constant<int, 2>{}, P1, F{}, k0 + 4);
    step(integral_constant<int, 3>{}, P1, T{}, k0 + 5);
    step(integral_constant<int, 0>{}, P0, F{}, k0 + 6);
    step(integral_constant<int, 1>{}, P0, F{}, k0 + 7);
  }

  // Epilogue.  acc[tg][rg] element v: token 128 wave + 16 tg + 4 g + v,
  // MFMA column m = device row 128 nt + 16 rg + m.
  if constexpr (GU) {
    // Column m < 8 holds gate row 8 dt + m, column m + 8 the matching up row.
    // Per pair of elements (v, v + 1) the lanes of a column pair swap one
    // value (DPP rotate by 8 within each row of 16 lanes): lane m < 8 then
    // holds gate and up of token v, lane m + 8 those of token v + 1, and
    // each computes one SwiGLU output.
    const bool lo = m < 8;
    const int col = m & 7;
#pragma unroll
    for (int tg = 0; tg < kPfTG; ++tg) {
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const int mt = kPfWM * wave + 16 * tg + 4 * g + v + (lo ? 0 : 1);
        const bool ok = mt < nm;
        const size_t pos = (size_t)(off_e + m0 + mt);
#pragma unroll
        for (int rg = 0; rg < kPfRG; ++rg) {
          const int dt = 8 * nt + rg;   // device tile
          const float a0 = acc[tg][rg][v], a1 = acc[tg][rg][v + 1];
          const float recv = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, lo ? a1 : a0), 0x128, 0xF, 0xF, false));
          const float gate = lo ? a0 : recv;
          const float up = lo ? recv : a1;
          if (ok && 8 * dt + col < I) {
            const _Float16 hh = (_Float16)(silu_f32(gate) * up);
            A.hout[pos * I + 8 * dt + col] = __builtin_bit_cast(uint16_t, hh);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int tg = 0; tg < kPfTG; ++tg) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int mt = kPfWM * wave + 16 * tg + 4 * g + v;
        if (mt >= nm) continue;
        const size_t orow = (size_t)part * A.part_stride + (size_t)A.rt.perm[off_e + m0 + mt] * H;
#pragma unroll
        for (int rg = 0; rg < kPfRG; ++rg) {
          const int dt = 8 * nt + rg;   // device tile
          if (16 * dt + m < H) A.oout[orow + 16 * dt + m] = acc[tg][rg][v];
        }
      }
    }
  }
}

template <bool GU>
__device__ __forceinline__ void pf_zero_tile(const MfmaArgs& A, int n_e, int off_e, int m0, int nt, int part) {
  const int nm = n_e - m0 < kPfTM ? n_e - m0 : kPfTM;
  for (int i = threadIdx.x; i < nm * kPfTN; i += kPfThreads) {
    const int mt = i / kPfTN, r = i % kPfTN;
    const int dr = kPfTN * nt + r;
    const size_t pos = (size_t)(off_e + m0 + mt);
    if constexpr (GU) {
      if ((dr & 15) < 8 && dr < 2 * A.I) A.hout[pos * A.I + 8 * (dr >> 4) + (dr & 7)] = 0;
    } else {
      if (dr < A.H) A.oout[(size_t)part * A.part_stride + (size_t)A.rt.perm[pos] * A.H + dr] = 0.0f;
    }
  }
  if (threadIdx.x == 0 && nt == 0 && m0 == 0 && part == 0) raise_status(A.rt.status, PW_DEV_BAD_BITWIDTH);
}

template <bool GU>
__global__ __launch_bounds__(kPfThreads, 1) void mfma_kernel(MfmaArgs A) {
  __shared__ __align__(1024) uint8_t lds[kPfLds];
  // Workgroups go to the eight XCDs round-robin (workgroup i to XCD i mod 8)
  // and the grid is sized for the most token tiles routing can produce.  The
  // items that exist (token tiles x K parts x row tiles, counted on the
  // device) are dealt evenly, a run of consecutive items per XCD, so the XCDs
  // finish together and one XCD sweeps the row tiles of a few token tiles,
  // whose activation rows then stay near it.  Items run in groups of
  // kPfTileGroup consecutive token tiles (an expert's tiles are adjacent in
  // the list): inside a group the tiles of one (K part, row tile) are
  // adjacent, so they read that row tile's planes at about the same time and
  // the second read finds them in L2 (Mixtral prefill, two tiles per expert:
  // gate_up 2.31 -> 2.25 ms, down 1.21 -> 1.17 ms against tile-major items).
  const int ntl = uniform(*A.rt.num_mtiles);
  const int nitems = ntl * A.kparts * A.ntiles;
  const int per_xcd = (nitems + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + slot;
  if (slot >= per_xcd || item >= nitems) return;
  const int per_group = kPfTileGroup * A.kparts * A.ntiles;
  const int full = ntl / kPfTileGroup;   // whole groups; the last one may hold fewer tiles
  const bool whole = item < full * per_group;
  const int g0 = whole ? item / per_group * kPfTileGroup : full * kPfTileGroup;
  const int gn = whole ? kPfTileGroup : ntl - full * kPfTileGroup;
  const int r = whole ? item % per_group : item - full * per_group;
  const int mi = g0 + r % gn;
  const int part = r / (gn * A.ntiles);
  const int nt = (r / gn) % A.ntiles;
  const int e = uniform(A.rt.mtiles[2 * mi]);
  const int m0 = uniform(A.rt.mtiles[2 * mi + 1]);
  const int n_e = uniform(A.rt.counts[e]);
  const int off_e = uniform(A.rt.offsets[e]);
  const int qv = uniform(A.q[2 * e + (GU ? 0 : 1)]);
  switch (qv) {
    case 3: pf_tile<3, GU>(A, e, n_e, off_e, m0, nt, part, lds); break;
    case 4: pf_tile<4, GU>(A, e, n_e, off_e, m0, nt, part, lds); break;
    case 5: pf_tile<5, GU>(A, e, n_e, off_e, m0, nt, part, lds); break;
    case 6: pf_tile<6, GU>(A, e, n_e, off_e, m0, nt, part, lds); break;
    case 7: pf_tile<7, GU>(A, e, n_e, off_e, m0, nt, part, lds); break;
    case 8: pf_tile<8, GU>(A, e, n_e, off_e, m0, nt, part, lds); break;
    default: pf_zero_tile<GU>(A, n_e, off_e, m0, nt, part); break;
  }
}

template <bool GU>
static hipError_t launch_mfma(const ExpertArgs& a, const uint16_t* act, uint16_t* h, float* o, hipStream_t s,
                              const KernelEvents& ev) {
  MfmaArgs A{};
  A.H = a.H; A.I = a.I; A.E = a.E; A.k = a.k; A.T = a.T;
  A.blocks = a.blocks; A.q = a.q; A.rt = a.rt;
  A.act = act; A.hout = h; A.oout = o;
  A.ntiles = ((GU ? 2 * a.I : a.H) + kPfTN - 1) / kPfTN;
  A.kparts = GU ? 1 : (a.kparts > 0 ? a.kparts : 1);
  A.part_stride = (size_t)a.T * a.k * a.H;
  const long long act_bytes = 2LL * (GU ? (long long)a.T * a.H : (long long)a.T * a.k * a.I);
  if (act_bytes >= 0x80000000LL) return hipErrorInvalidValue;   // the A operand is addressed with 32-bit offsets
  A.act_bytes = (uint32_t)act_bytes;
  const long long items = (long long)mtile_bound(a.E, a.T, a.k) * A.kparts * A.ntiles;
  const long long grid = (items + kXcds - 1) / kXcds * kXcds;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  return launch_kernel(mfma_kernel<GU>, dim3((unsigned)grid), dim3(kPfThreads), s, ev, A);
}

hipError_t launch_mfma_gate_up(const ExpertArgs& a, const uint16_t* x, uint16_t* h, hipStream_t s,
                               const KernelEvents& ev) {
  return launch_mfma<true>(a, x, h, nullptr, s, ev);
}

hipError_t launch_mfma_down(const ExpertArgs& a, const uint16_t* h, float* o, hipStream_t s, const KernelEvents& ev) {
  return launch_mfma<false>(a, h, nullptr, o, s, ev);
}

}  // namespace pw
