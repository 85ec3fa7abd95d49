// Matrix-core GEMV kernels for experts with a moderate number of tokens (a
// few to a few hundred; any count is handled, 32 tokens per pass over K).
// "Technical summary: PagedWeight", Core components 3 (fused mixed-precision
// kernel): every block is read at its own committed bitwidth q from the
// device page table.
//
// A workgroup is one wave and owns 32 device rows of one routed block (two
// 16-row device tiles; gate_up: 16 gate rows and their 16 up rows) for the
// whole K range and a tile of up to 32 tokens.  Each weight is decoded once,
// in registers, straight into the B operand of v_mfma_f32_32x32x16_f16, whose
// 32 x 32 output covers all 32 rows and all 32 tokens: one activation
// fragment feeds 32 weight rows.  Lane l supplies B column l & 31 (the weight
// row) and K slots 8 (l >> 5) .. +8, and A row l & 31 (the token) at the same
// K slots.  The K order inside one instruction is free as long as A and B
// agree, so lane half h = l >> 5 takes plane word w_h of its row (32
// weights), transposes its q plane words into code fields, looks the 32
// weights up in the row's table in LDS, and feeds byte b of the word
// (weights 8b .. 8b + 7) to product b; the activations of product b are
// x[token][32 w_h + 8b .. +8], one 16-byte load.  In a 256-wide super-chunk
// C, half h reads words 8 C + 4 h .. +4 with one load per plane and
// sub-chunk i uses word 8 C + 4 h + i.  Plane words are requested two
// super-chunks ahead and activations two sub-chunks ahead (each of the two
// activation buffers is refilled right after its products are issued; one
// sub-chunk ahead left the loop waiting on the L2: Mixtral-shaped T = 8
// gate_up 192 -> 178 us, T = 64 254 -> 247 us).  gate_up pairs
// gate and up rows in columns c and c + 8, so SwiGLU is one lane swap on the
// accumulators.
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kMgRows = 32;
constexpr long long kMgMaxGrid = 32768;   // workgroups per launch (several per SIMD)
static_assert(kMgTileM == 32, "a tile fills the 32 MFMA rows");

typedef _Float16 mg_half8 __attribute__((ext_vector_type(8)));
typedef float mg_float16 __attribute__((ext_vector_type(16)));

struct MgArgs {
  int H, I, E, k, T;
  const pw_block_desc* blocks;
  const uint8_t* q;
  Route rt;
  const uint16_t* act;   // gate_up: x [T][H]; down: h [slots][I] by sorted position
  uint16_t* hout;
  float* oout;           // o [slots][H] by slot (one K part)
  int chunks;            // 32-row chunks per block
  int kparts;            // parts of the K range (down product), each its own items and o slice
  size_t part_stride;    // floats between the o slices of two parts
  uint32_t act_bytes;    // < 2^31: out-of-range offsets read zero
};

template <int Q, bool GU>
__device__ __forceinline__ void mg_chunk(const MgArgs& A, int e, int n_e, int off_e, int ch, int part,
                                         uint8_t* tabs) {
  constexpr int TAB = (1 << Q) * 2;
  const int lane = threadIdx.x;
  const int c = lane & 31, hf = lane >> 5;
  const int H = A.H, I = A.I;
  const int N = GU ? 2 * I : H;
  const int K = GU ? H : I;
  const int W = K >> 5;

  const pw_block_desc d = A.blocks[2 * e + (GU ? 0 : 1)];
  const uint32_t pstride = (uint32_t)N * (uint32_t)W * 4u;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(uniform_ptr(d.planes), pstride * (uint32_t)Q);
  const uint16_t* __restrict__ lut = uniform_ptr(d.lut_all) + lut_offset(N, Q);

  // the lane's row: device row 32 ch + c
  const int drow = kMgRows * ch + c;
  const bool row_ok = drow < N;

  // K is walked in 256-wide super-chunks C: half h reads plane words
  // 8 C + 4 h .. +4 of its row (the device layout keeps a row's 16-word run
  // contiguous), and word 8 C + 4 h + i feeds sub-chunk i.  With W % 4 == 0
  // a lane's four words are one aligned 16-byte load; otherwise four 4-byte
  // loads.  Words past the row's end are not read and count as zero.
  // K part `part` of A.kparts: super-chunks [C0, C0 + nsc)
  const int nsa = (W + 7) >> 3;
  const int nsp = (nsa + A.kparts - 1) / A.kparts;
  const int C0 = part * nsp;
  const int nsc = nsa - C0 < nsp ? (nsa - C0 > 0 ? nsa - C0 : 0) : nsp;
  const bool vec = (W & 3) == 0;
  auto load_planes = [&](uint32_t (&P)[Q][4], int C) {
    const int wd = 8 * (C0 + C) + 4 * hf;
    const bool live = row_ok && C < nsc && wd < W;
    const uint32_t voff = live ? dev_word(drow, wd, W) * 4u : kOutOfRange;
    if (vec) {
#pragma unroll
      for (int p = 0; p < Q; ++p) {
        const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      prs, (int)voff, (int)((uint32_t)p * pstride), 0));
        P[p][0] = v.x; P[p][1] = v.y; P[p][2] = v.z; P[p][3] = v.w;
      }
    } else {
#pragma unroll
      for (int p = 0; p < Q; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          P[p][i] = buf_load_u32(prs, (live && wd + i < W) ? dev_word(drow, wd + i, W) * 4u : kOutOfRange,
                                 (uint32_t)p * pstride);
    }
  };
  uint32_t P0[Q][4], P1[Q][4];
  load_planes(P0, 0);
  load_planes(P1, 1);

  // the 32 row tables -> LDS, row c at c * TAB (rows outside the block read as zero)
  for (int i = lane; i < kMgRows * TAB / 16; i += kWave) {
    const int r = i / (TAB / 16), cc = i % (TAB / 16);
    const int dr = kMgRows * ch + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (dr < N) v = *reinterpret_cast<const uint4*>(lut + (size_t)canon_row(dr, I, GU) * (1 << Q) + cc * 8);
    *reinterpret_cast<uint4*>(tabs + i * 16) = v;
  }
  __syncthreads();
  const uint32_t base = lds_addr(tabs) + (uint32_t)(c * TAB);

  // activation row of the lane's token (A row = lane & 31); tokens past the
  // tile read zero and their output rows are not stored
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A.act, A.act_bytes);
  uint32_t aoff = kOutOfRange;
  if (c < n_e) {
    const int pos = off_e + c;
    aoff = GU ? (uint32_t)(A.rt.perm[pos] / A.k) * (uint32_t)H * 2u : (uint32_t)pos * (uint32_t)I * 2u;
  }

  mg_float16 acc = {};

  // Software-pipelined sub-chunks (sub-chunk s = word 8 (s >> 2) + 4 h + (s & 3)):
  // each step issues its lookups, then requests the next sub-chunk's
  // activations and transposes its plane words while the lookups are in
  // flight, and only then multiplies.  Unrolled over two super-chunks so every
  // register index is static.
  auto load_a = [&](uint4 (&ar)[4], int s) {
    const int wd = 8 * (C0 + (s >> 2)) + 4 * hf + (s & 3);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t voff = wd < W ? aoff + (uint32_t)(wd * 32 + 8 * b) * 2u : kOutOfRange;
      ar[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)voff, 0, 0));
    }
  };
  auto fields = [&](const uint32_t (&P)[Q][4], int i, uint32_t (&R)[8]) {
    uint32_t W8[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) W8[p] = P[p][i];
    planes_to_fields<Q>(W8, R);
  };
  auto multiply = [&](const uint4 (&ar)[4], const uint32_t (&packed)[16]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const mg_half8 bop = __builtin_bit_cast(
          mg_half8, make_uint4(packed[4 * b], packed[4 * b + 1], packed[4 * b + 2], packed[4 * b + 3]));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(mg_half8, ar[b]), bop, acc, 0, 0, 0);
    }
  };

  const int S = 4 * nsc;   // sub-chunks (past the last word they read zero activations)
  uint4 A0[4], A1[4];
  uint32_t R[8];
  load_a(A0, 0);
  load_a(A1, 1);
  fields(P0, 0, R);
  // one step: lookups of s (fields in R), fields of s + 1 from (Pn, in) into
  // R, the products of s with Ac, then the activations of s + 2 into Ac
#define PW_MG_STEP(Ac, An, Pn, in, s_)                         \
  {                                                            \
    uint32_t packed[16];                                       \
    GroupDecode<Q, 0>::run(R, base, packed);                   \
    if ((s_) + 1 < S) fields(Pn, in, R);                       \
    multiply(Ac, packed);                                      \
    if ((s_) + 2 < S) load_a(Ac, (s_) + 2);                    \
  }
  for (int s0 = 0; s0 < S; s0 += 8) {
    const int C = s0 >> 2;
    PW_MG_STEP(A0, A1, P0, 1, s0);
    PW_MG_STEP(A1, A0, P0, 2, s0 + 1);
    PW_MG_STEP(A0, A1, P0, 3, s0 + 2);
    PW_MG_STEP(A1, A0, P1, 0, s0 + 3);
    load_planes(P0, C + 2);   // super-chunk C is transposed; its buffer takes C + 2
    if (s0 + 4 >= S) break;
    PW_MG_STEP(A0, A1, P1, 1, s0 + 4);
    PW_MG_STEP(A1, A0, P1, 2, s0 + 5);
    PW_MG_STEP(A0, A1, P1, 3, s0 + 6);
    PW_MG_STEP(A1, A0, P0, 0, s0 + 7);
    load_planes(P1, C + 3);
  }
#undef PW_MG_STEP

  // acc element i: token 8 (i / 4) + 4 h + i % 4, column c = device row 32 ch + c
  if constexpr (GU) {
    // Column c (c & 8 == 0) holds gate row 8 t + (c & 7) of device tile
    // t = 2 ch + (c >> 4), column c + 8 the matching up row.  Per pair of
    // elements (i, i + 1) the lanes of a column pair swap one value (DPP
    // rotate by 8 within each row of 16 lanes): the gate lane then holds gate
    // and up of token 8 (i / 4) + 4 h + i % 4, the up lane those of the next
    // token, and each computes one SwiGLU output.
    const bool lo = (c & 8) == 0;
    const int col = 8 * (2 * ch + (c >> 4)) + (c & 7);
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float a0 = acc[i], a1 = acc[i + 1];
      const float recv = __builtin_bit_cast(
          float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, lo ? a1 : a0), 0x128, 0xF, 0xF, false));
      const float gate = lo ? a0 : recv;
      const float up = lo ? recv : a1;
      const int m = 8 * (i >> 2) + 4 * hf + (i & 3) + (lo ? 0 : 1);
      if (m < n_e && col < I) {
        const _Float16 hh = (_Float16)(silu_f32(gate) * up);
        A.hout[(size_t)(off_e + m) * I + col] = __builtin_bit_cast(uint16_t, hh);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 8 * (i >> 2) + 4 * hf + (i & 3);
      if (row_ok && m < n_e) A.oout[(size_t)part * A.part_stride + (size_t)A.rt.perm[off_e + m] * H + drow] = acc[i];
    }
  }
}

template <bool GU>
__device__ __forceinline__ void mg_zero(const MgArgs& A, int n_e, int off_e, int ch, int part, bool first_tile) {
  const int N = GU ? 2 * A.I : A.H;
  for (int i = threadIdx.x; i < n_e * kMgRows; i += kWave) {
    const int m = i / kMgRows, r = i % kMgRows;
    const int dr = kMgRows * ch + r;
    if (dr >= N) continue;
    if constexpr (GU) {
      if ((dr & 15) < 8) A.hout[(size_t)(off_e + m) * A.I + 8 * (dr >> 4) + (dr & 7)] = 0;
    } else {
      A.oout[(size_t)part * A.part_stride + (size_t)A.rt.perm[off_e + m] * A.H + dr] = 0.0f;
    }
  }
  if (threadIdx.x == 0 && ch == 0 && part == 0 && first_tile) raise_status(A.rt.status, PW_DEV_BAD_BITWIDTH);
}

// Work items are (32-token tile, row chunk) pairs; the route kernel lists the
// tiles of the experts in this family's band, so an expert with many tokens
// gets more items rather than longer ones.  The grid is capped and each
// workgroup walks items grid-strided, so a launch whose band holds no expert
// costs a few microseconds whatever the bound on the tile count.
template <bool GU>
__global__ __launch_bounds__(kWave) void mgemv_kernel(MgArgs A) {
  __shared__ __align__(16) uint8_t tabs[kMgRows * (1 << kMaxBits) * 2];
  const int items = uniform(*A.rt.num_mgtiles) * A.kparts * A.chunks;
  for (int item = (int)blockIdx.x; item < items; item += (int)gridDim.x) {
    if (item != (int)blockIdx.x) __syncthreads();   // the previous item's lookups are done before new tables land
    const int t = item / (A.kparts * A.chunks);
    const int part = item / A.chunks % A.kparts;
    const int ch = item % A.chunks;
    const int e = uniform(A.rt.mgtiles[2 * t]);
    const int m0 = uniform(A.rt.mgtiles[2 * t + 1]);
    const int n_e = uniform(A.rt.counts[e]);
    const int nm = n_e - m0 < kMgTileM ? n_e - m0 : kMgTileM;
    const int off_e = uniform(A.rt.offsets[e]) + m0;
    const int qv = uniform(A.q[2 * e + (GU ? 0 : 1)]);
    switch (qv) {
      case 3: mg_chunk<3, GU>(A, e, nm, off_e, ch, part, tabs); break;
      case 4: mg_chunk<4, GU>(A, e, nm, off_e, ch, part, tabs); break;
      case 5: mg_chunk<5, GU>(A, e, nm, off_e, ch, part, tabs); break;
      case 6: mg_chunk<6, GU>(A, e, nm, off_e, ch, part, tabs); break;
      case 7: mg_chunk<7, GU>(A, e, nm, off_e, ch, part, tabs); break;
      case 8: mg_chunk<8, GU>(A, e, nm, off_e, ch, part, tabs); break;
      default: mg_zero<GU>(A, nm, off_e, ch, part, m0 == 0); break;
    }
  }
}

template <bool GU>
static hipError_t launch_mg(const ExpertArgs& a, const uint16_t* act, uint16_t* h, float* o, hipStream_t s,
                            const KernelEvents& ev) {
  MgArgs A{};
  A.H = a.H; A.I = a.I; A.E = a.E; A.k = a.k; A.T = a.T;
  A.blocks = a.blocks; A.q = a.q; A.rt = a.rt;
  A.act = act; A.hout = h; A.oout = o;
  A.chunks = ((GU ? 2 * a.I : a.H) + kMgRows - 1) / kMgRows;
  A.kparts = GU ? 1 : (a.kparts > 0 ? a.kparts : 1);
  A.part_stride = (size_t)a.T * a.k * a.H;
  const long long act_bytes = 2LL * (GU ? (long long)a.T * a.H : (long long)a.T * a.k * a.I);
  if (act_bytes >= 0x80000000LL) return hipErrorInvalidValue;
  A.act_bytes = (uint32_t)act_bytes;
  long long grid = (long long)mgtile_bound(a.E, a.T, a.k) * A.kparts * A.chunks;
  if (grid > 0x7FFFFFFFLL - kMgMaxGrid) return hipErrorInvalidValue;   // the kernel counts items in int
  const bool timed = ev.start || ev.stop;
  if ((grid == 0 || a.min_tokens >= a.max_tokens) && !timed) return hipSuccess;
  // with events attached an empty band still launches (one workgroup, no items)
  if (grid == 0) grid = 1;
  if (grid > kMgMaxGrid) grid = kMgMaxGrid;
  return launch_kernel(mgemv_kernel<GU>, dim3((unsigned)grid), dim3(kWave), s, ev, A);
}

hipError_t launch_mgemv_gate_up(const ExpertArgs& a, const uint16_t* x, uint16_t* h, hipStream_t s,
                                const KernelEvents& ev) {
  return launch_mg<true>(a, x, h, nullptr, s, ev);
}

hipError_t launch_mgemv_down(const ExpertArgs& a, const uint16_t* h, float* o, hipStream_t s,
                             const KernelEvents& ev) {
  return launch_mg<false>(a, h, nullptr, o, s, ev);
}

}  // namespace pw
