// Matrix-core GEMV kernels for experts with a moderate number of tokens (a
// few to a few hundred; any count is handled, 32 tokens per pass over K).
// "Technical summary: PagedWeight", Core components 3 (fused mixed-precision
// kernel): every block is read at its own committed bitwidth q from the
// device page table.
//
// A workgroup is one wave and owns 16 weight rows of one routed block for the
// whole K range (gate_up: 8 gate rows and the matching 8 up rows; down: 16
// rows).  Each weight is decoded exactly once, in registers, straight into the
// matrix cores' B operand, and multiplies up to 32 tokens (two 16-token
// groups) with v_mfma_f32_16x16x32_f16 -- no weight tile in LDS, no barrier in
// the K loop.  For v_mfma_f32_16x16x32_f16 lane l supplies B column l & 15
// (the weight row) and K slots 8 (l >> 4) .. +8, and A row l & 15 (the token)
// at the same K slots.  The K order inside one instruction is free as long as
// A and B agree, so lane group g = l >> 4 takes plane word w of its row (32
// weights), transposes its q plane words into code fields once, looks the 32
// weights up in the row's table in LDS, and feeds byte b of the word (weights
// 8b .. 8b + 7) to sub-step b; the activations of sub-step b are
// x[token][32 w + 8b .. +8], one 16-byte load.  In a 512-wide super-chunk C,
// group g reads words 16 C + 4 g .. +4 with one load per plane (the four
// groups cover a row's 64-byte line) and sub-chunk i uses word 16 C + 4 g + i.
// Plane words are requested two super-chunks ahead and activations one
// sub-chunk ahead.  gate_up pairs gate and up rows in columns n and n + 8, so
// SwiGLU is one lane swap on the accumulators.
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kMgRows = 16;
constexpr long long kMgMaxGrid = 32768;   // workgroups per launch (several per SIMD)
constexpr int kMgGroups = 2;                 // 16-token groups per wave
static_assert(16 * kMgGroups == kMgTileM, "a tile fills the token groups");

typedef _Float16 mg_half8 __attribute__((ext_vector_type(8)));
typedef float mg_float4 __attribute__((ext_vector_type(4)));

struct MgArgs {
  int H, I, E, k, T;
  const pw_block_desc* blocks;
  const uint8_t* q;
  Route rt;
  const uint16_t* act;   // gate_up: x [T][H]; down: h [slots][I] by sorted position
  uint16_t* hout;
  float* oout;           // o [slots][H] by slot (one K part)
  int chunks;            // row chunks per block
  uint32_t act_bytes;    // < 2^31: out-of-range offsets read zero
};

// Tile-local row r (0..15) of chunk ch -> block row, and whether it exists.
template <bool GU>
__device__ __forceinline__ int mg_row(int ch, int r, int I, int H, bool& ok) {
  if constexpr (GU) {
    const int x = 8 * ch + (r & 7);
    ok = x < I;
    return (r < 8 ? 0 : I) + x;
  } else {
    const int x = 16 * ch + r;
    ok = x < H;
    return x;
  }
}

template <int Q, bool GU>
__device__ __forceinline__ void mg_chunk(const MgArgs& A, int e, int n_e, int off_e, int ch, uint8_t* tabs) {
  constexpr int TAB = (1 << Q) * 2;
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int H = A.H, I = A.I;
  const int N = GU ? 2 * I : H;
  const int K = GU ? H : I;
  const int W = K >> 5;

  const pw_block_desc d = A.blocks[2 * e + (GU ? 0 : 1)];
  const uint32_t pstride = (uint32_t)N * (uint32_t)W * 4u;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(uniform_ptr(d.planes), pstride * (uint32_t)Q);
  const uint16_t* __restrict__ lut = uniform_ptr(d.lut_all) + lut_offset(N, Q);

  bool row_ok;
  const int row = mg_row<GU>(ch, n, I, H, row_ok);

  // K is walked in 512-wide super-chunks C: lane group g reads plane words
  // 16 C + 4 g .. +4 of its row, and word 16 C + 4 g + i feeds sub-chunk i.
  // The item's 16 rows are device tile ch (gate_up: 8 gate rows and their 8
  // up rows), so the wave's load of one plane is the tile's contiguous 1 KB
  // piece (less in a narrower last column tile).  With W % 4 == 0 a lane's
  // four words are one aligned 16-byte load; otherwise four 4-byte loads.
  // Words past the row's end are not read and count as zero.
  const int ns = (W + 15) >> 4;
  const bool vec = (W & 3) == 0;
  const int drow = 16 * ch + n;
  auto load_planes = [&](uint32_t (&P)[Q][4], int C) {
    const int wd = 16 * C + 4 * g;
    const bool live = row_ok && C < ns && wd < W;
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

  // the 16 row tables -> LDS, row r at r * TAB (rows outside the block read as zero)
  for (int c = lane; c < kMgRows * TAB / 16; c += kWave) {
    const int r = c / (TAB / 16), cc = c % (TAB / 16);
    bool ok;
    const int rr = mg_row<GU>(ch, r, I, H, ok);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (ok) v = *reinterpret_cast<const uint4*>(lut + (size_t)rr * (1 << Q) + cc * 8);
    *reinterpret_cast<uint4*>(tabs + c * 16) = v;
  }
  __syncthreads();
  const uint32_t base = lds_addr(tabs) + (uint32_t)(n * TAB);

  // activation rows of the lane's token in each group (A row = lane & 15)
  const int ntg = (n_e + 15) >> 4;
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A.act, A.act_bytes);
  uint32_t aoff[kMgGroups];
#pragma unroll
  for (int tg = 0; tg < kMgGroups; ++tg) {
    const int m = 16 * tg + n;
    aoff[tg] = kOutOfRange;
    if (m < n_e) {
      const int pos = off_e + m;
      aoff[tg] = GU ? (uint32_t)(A.rt.perm[pos] / A.k) * (uint32_t)H * 2u : (uint32_t)pos * (uint32_t)I * 2u;
    }
  }

  mg_float4 acc[kMgGroups];
#pragma unroll
  for (int tg = 0; tg < kMgGroups; ++tg) acc[tg] = mg_float4{0.f, 0.f, 0.f, 0.f};

  // sub-chunk: plane word wd (its four plane bytes b = sub-steps)
  // Software-pipelined sub-chunks (sub-chunk s = word 16 (s >> 2) + 4 g + (s & 3)):
  // each step issues its lookups, then requests the next sub-chunk's
  // activations and transposes its plane words while the lookups are in
  // flight, and only then multiplies.  Unrolled over two super-chunks so every
  // register index is static.
  auto load_a = [&](uint4 (&ar)[kMgGroups][4], int s) {
    const int wd = 16 * (s >> 2) + 4 * g + (s & 3);
#pragma unroll
    for (int tg = 0; tg < kMgGroups; ++tg) {
      if (tg >= ntg) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t voff = wd < W ? aoff[tg] + (uint32_t)(wd * 32 + 8 * b) * 2u : kOutOfRange;
        ar[tg][b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)voff, 0, 0));
      }
    }
  };
  auto fields = [&](const uint32_t (&P)[Q][4], int i, uint32_t (&R)[8]) {
    uint32_t W8[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) W8[p] = P[p][i];
    planes_to_fields<Q>(W8, R);
  };
  auto multiply = [&](const uint4 (&ar)[kMgGroups][4], const uint32_t (&packed)[16]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const mg_half8 bop = __builtin_bit_cast(
          mg_half8, make_uint4(packed[4 * b], packed[4 * b + 1], packed[4 * b + 2], packed[4 * b + 3]));
#pragma unroll
      for (int tg = 0; tg < kMgGroups; ++tg) {
        if (tg >= ntg) continue;
        acc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mg_half8, ar[tg][b]), bop, acc[tg], 0,
                                                         0, 0);
      }
    }
  };

  const int S = 4 * ns;   // sub-chunks (past the last word they read zero activations)
  uint4 A0[kMgGroups][4], A1[kMgGroups][4];
  uint32_t R[8];
  load_a(A0, 0);
  fields(P0, 0, R);
  // one step: lookups of s (fields in R), next activations into An, fields of s + 1
  // from (Pn, in) into R, then the products of s with Ac
#define PW_MG_STEP(Ac, An, Pn, in, s_)                         \
  {                                                            \
    uint32_t packed[16];                                       \
    GroupDecode<Q, 0>::run(R, base, packed);                   \
    if ((s_) + 1 < S) {                                        \
      load_a(An, (s_) + 1);                                    \
      fields(Pn, in, R);                                       \
    }                                                          \
    multiply(Ac, packed);                                      \
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

  // acc[tg] element v: token 16 tg + 4 g + v, tile column n
#pragma unroll
  for (int tg = 0; tg < kMgGroups; ++tg) {
    if (tg >= ntg) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * tg + 4 * g + v;
      if constexpr (GU) {
        const float gate = acc[tg][v];
        const float up = __shfl_xor(gate, 8, kWave);   // column n + 8 holds the matching up row
        if (n < 8 && row_ok && m < n_e) {
          const _Float16 hh = (_Float16)(silu_f32(gate) * up);
          A.hout[(size_t)(off_e + m) * I + 8 * ch + n] = __builtin_bit_cast(uint16_t, hh);
        }
      } else {
        if (row_ok && m < n_e) {
          const size_t slot = (size_t)A.rt.perm[off_e + m];
          A.oout[slot * H + row] = acc[tg][v];
        }
      }
    }
  }
}

template <bool GU>
__device__ __forceinline__ void mg_zero(const MgArgs& A, int n_e, int off_e, int ch, bool first_tile) {
  for (int i = threadIdx.x; i < n_e * kMgRows; i += kWave) {
    const int m = i / kMgRows, r = i % kMgRows;
    bool ok;
    const int row = mg_row<GU>(ch, r, A.I, A.H, ok);
    if (!ok) continue;
    if constexpr (GU) {
      if (r < 8) A.hout[(size_t)(off_e + m) * A.I + 8 * ch + r] = 0;
    } else {
      A.oout[(size_t)A.rt.perm[off_e + m] * A.H + row] = 0.0f;
    }
  }
  if (threadIdx.x == 0 && ch == 0 && first_tile) raise_status(A.rt.status, PW_DEV_BAD_BITWIDTH);
}

// Work items are (32-token tile, row chunk) pairs; the route kernel lists the
// tiles of the experts in this family's band, so an expert with many tokens
// gets more items rather than longer ones.  The grid is capped and each
// workgroup walks items grid-strided, so a launch whose band holds no expert
// costs a few microseconds whatever the bound on the tile count.
template <bool GU>
__global__ __launch_bounds__(kWave) void mgemv_kernel(MgArgs A) {
  __shared__ __align__(16) uint8_t tabs[kMgRows * (1 << kMaxBits) * 2];
  const int items = uniform(*A.rt.num_mgtiles) * A.chunks;
  for (int item = (int)blockIdx.x; item < items; item += (int)gridDim.x) {
    if (item != (int)blockIdx.x) __syncthreads();   // the previous item's lookups are done before new tables land
    const int t = item / A.chunks;
    const int ch = item - t * A.chunks;
    const int e = uniform(A.rt.mgtiles[2 * t]);
    const int m0 = uniform(A.rt.mgtiles[2 * t + 1]);
    const int n_e = uniform(A.rt.counts[e]);
    const int nm = n_e - m0 < kMgTileM ? n_e - m0 : kMgTileM;
    const int off_e = uniform(A.rt.offsets[e]) + m0;
    const int qv = uniform(A.q[2 * e + (GU ? 0 : 1)]);
    switch (qv) {
      case 3: mg_chunk<3, GU>(A, e, nm, off_e, ch, tabs); break;
      case 4: mg_chunk<4, GU>(A, e, nm, off_e, ch, tabs); break;
      case 5: mg_chunk<5, GU>(A, e, nm, off_e, ch, tabs); break;
      case 6: mg_chunk<6, GU>(A, e, nm, off_e, ch, tabs); break;
      case 7: mg_chunk<7, GU>(A, e, nm, off_e, ch, tabs); break;
      case 8: mg_chunk<8, GU>(A, e, nm, off_e, ch, tabs); break;
      default: mg_zero<GU>(A, nm, off_e, ch, m0 == 0); break;
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
  A.chunks = GU ? (a.I + 7) / 8 : (a.H + kMgRows - 1) / kMgRows;
  const long long act_bytes = 2LL * (GU ? (long long)a.T * a.H : (long long)a.T * a.k * a.I);
  if (act_bytes >= 0x80000000LL) return hipErrorInvalidValue;
  A.act_bytes = (uint32_t)act_bytes;
  long long grid = (long long)mgtile_bound(a.E, a.T, a.k) * A.chunks;
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
