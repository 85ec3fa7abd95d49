// Dequant-to-LDS MFMA kernels for experts with many tokens (prefill).
// "Technical summary: PagedWeight", Core components 3 (fused mixed-precision
// kernel): each block is read at its own committed bitwidth q from the device
// page table; here the decoded weights feed the matrix cores instead of a
// GEMV, because with hundreds of tokens per expert the product is a dense
// contraction.
//
// Tile: 256 tokens x 128 weight rows per 8-wave workgroup, K step 64.
//   * every wave decodes: a pair of threads turns one 32-weight group (the
//     first q plane words of one row) into fp16 through the row's table in
//     LDS, each thread half of it with its lookups issued together, and
//     writes it to a double-buffered weight tile;
//   * all waves stage the gathered activation tile (half a token row each);
//   * every wave multiplies a 64 x 64 sub-tile with v_mfma_f32_16x16x32_f16
//     (fp32 accumulation).
// Plane words are prefetched into registers two K steps ahead and
// activations one step ahead, and the decode of step k+1 is issued while the
// matrix cores work on step k.  gate_up tiles take 64 gate rows and the
// matching 64 up rows; each wave holds matching gate and up columns, so SwiGLU
// runs on the accumulators and h leaves as fp16.  Token tiles less than half
// full take a variant that feeds the matrix cores' activation operand from
// registers loaded straight from memory (no LDS activation tile).
//
// Work items are (token tile, row tile) pairs; token tiles come from the route
// kernel's list.  Consecutive items on one XCD (workgroups are dealt to the 8
// XCDs round-robin) sweep the row tiles of one token tile, so the activation
// rows stay in that XCD's L2.
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kMfmaThreads = 512;
constexpr int kTM = kMfmaTileM;        // 256 tokens
constexpr int kTN = 128;               // weight rows
constexpr int kTK = 64;                // reduction step
constexpr int kTileStride = kTK + 8;   // fp16 elements per LDS tile row (padding against bank conflicts)
constexpr int kXcds = 8;

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

struct MfmaArgs {
  int H, I, E, k, T;
  const pw_block_desc* blocks;
  const uint8_t* q;
  Route rt;
  const uint16_t* act;   // gate_up: x [T][H]; down: h [slots][I]
  uint16_t* hout;        // gate_up output
  float* oout;           // down output
  int ntiles;            // row tiles per block
  int grid;              // launched workgroups (multiple of 8)
  int direct_ok;         // activations addressable with 32-bit offsets (variant for partial tiles)
};

// Row of the block held at tile-local row r (0..127).
template <bool GU>
__device__ __forceinline__ int mrow(int nt, int r, int I) {
  if constexpr (GU) return (r < 64 ? 0 : I) + nt * 64 + (r & 63);
  else return nt * kTN + r;
}

template <bool GU>
__device__ __forceinline__ bool mrow_ok(int nt, int r, int I, int H) {
  if constexpr (GU) return nt * 64 + (r & 63) < I;
  else return nt * kTN + r < H;
}

constexpr int kLdsTabs = kTN * (1 << kMaxBits) * 2;              // 64 KB
constexpr int kLdsW = kTN * kTileStride * 2;                     // one weight tile
constexpr int kLdsX = kTM * kTileStride * 2;                     // activation tile
constexpr int kMfmaLds = kLdsTabs + 2 * kLdsW + kLdsX;

// Sixteen weights of a group: fields of weights j (0..15) in byte j >> 3 of
// F[j & 7]; all sixteen lookups are issued before any is packed.
template <int Q>
struct HalfGroupDecode {
  __device__ static __forceinline__ void run(const uint32_t (&F)[8], uint32_t base, uint32_t (&out)[8]) {
    uint32_t v[16];
    lookups<0>(F, base, v);
#pragma unroll
    for (int p = 0; p < 8; ++p) out[p] = v[2 * p] | (v[2 * p + 1] << 16);
  }
  template <int J>
  __device__ static __forceinline__ void lookups(const uint32_t (&F)[8], uint32_t base, uint32_t (&v)[16]) {
    if constexpr (J < 16) {
      v[J] = lds_u16_at(entry_addr<Q, J>(F, base));
      lookups<J + 1>(F, base, v);
    }
  }
};

template <int Q, bool GU>
__device__ __forceinline__ void mfma_tile(const MfmaArgs& A, int e, int n_e, int off_e, int m0, int nt, uint8_t* lds) {
  constexpr int TAB = (1 << Q) * 2;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int H = A.H, I = A.I;
  const int N = GU ? 2 * I : H;
  const int K = GU ? H : I;
  const int W = K >> 5;
  const int nk = (K + kTK - 1) / kTK;

  uint8_t* tabs = lds;
  _Float16* wt0 = reinterpret_cast<_Float16*>(lds + kLdsTabs);
  _Float16* wt1 = wt0 + kTN * kTileStride;
  _Float16* xt = wt1 + kTN * kTileStride;

  const pw_block_desc d = A.blocks[2 * e + (GU ? 0 : 1)];
  const uint32_t pstride = (uint32_t)N * (uint32_t)W * 4u;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(uniform_ptr(d.planes), pstride * (uint32_t)Q);
  const uint16_t* __restrict__ lut = uniform_ptr(d.lut_all) + lut_offset(N, Q);

  // Row tables -> LDS (uint4 chunks; rows outside the block read as zero).
  for (int c = tid; c < kTN * TAB / 16; c += kMfmaThreads) {
    const int r = c / (TAB / 16), cc = c % (TAB / 16);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (mrow_ok<GU>(nt, r, I, H))
      v = *reinterpret_cast<const uint4*>(lut + (size_t)mrow<GU>(nt, r, I) * (1 << Q) + cc * 8);
    *reinterpret_cast<uint4*>(tabs + c * 16) = v;
  }

  // Decode job: row dr, word dw of each K step, weights [16 dh, 16 dh + 16)
  // of that word (the two threads of a pair load the same plane words).
  const int dr = tid >> 2, dw = (tid >> 1) & 1, dh = tid & 1;
  const bool dr_ok = mrow_ok<GU>(nt, dr, I, H);
  const int ddev = dev_row(mrow<GU>(nt, dr, I), I, GU);   // device-layout row
  const uint32_t tab_base = lds_addr(tabs) + (uint32_t)(dr * TAB);
  // Activation job (all waves): token row xr, columns [32 xh, +32) of each K step.
  const int xr = tid >> 1, xh = tid & 1;
  const uint16_t* xsrc = nullptr;
  if (xr < n_e - m0) {
    const int pos = off_e + m0 + xr;
    xsrc = GU ? A.act + (size_t)(A.rt.perm[pos] / A.k) * H : A.act + (size_t)pos * I;
  }

  uint32_t Pa[Q], Pb[Q];
  uint4 X[4];

  // plane words of a K step, two steps ahead
  auto prefetch_planes = [&](uint32_t (&P)[Q], int step) {
    if (step >= nk) return;
    const int wc = ((step * kTK) >> 5) + dw;
    const uint32_t voff = (dr_ok && wc < W) ? dev_word(ddev, wc, W) * 4u : kOutOfRange;
#pragma unroll
    for (int p = 0; p < Q; ++p) P[p] = buf_load_u32(prs, voff, (uint32_t)p * pstride);
  };
  // activations of a K step (everyone), one step ahead (they hit L2)
  auto prefetch_x = [&](int step) {
    if (step >= nk) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = step * kTK + 32 * xh + 8 * v;
      X[v] = make_uint4(0u, 0u, 0u, 0u);
      if (xsrc != nullptr && c < K) X[v] = *reinterpret_cast<const uint4*>(xsrc + c);
    }
  };
  auto decode = [&](uint32_t (&P)[Q], _Float16* wt) {
    uint32_t R[8];
    planes_to_fields<Q>(P, R);
    // this thread's half: fields of weights 16 dh + j sit in bytes 2 dh, 2 dh + 1 of R[j & 7]
    uint32_t F[8];
    const uint32_t sel = dh ? 0x0c0c0302u : 0x0c0c0100u;
#pragma unroll
    for (int i = 0; i < 8; ++i) F[i] = __builtin_amdgcn_perm(0u, R[i], sel);
    uint32_t packed[8];
    HalfGroupDecode<Q>::run(F, tab_base, packed);
    uint4* dst = reinterpret_cast<uint4*>(wt + dr * kTileStride + dw * 32 + dh * 16);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  };
  auto stage_x = [&]() {
    uint4* dst = reinterpret_cast<uint4*>(xt + xr * kTileStride + 32 * xh);
#pragma unroll
    for (int v = 0; v < 4; ++v) dst[v] = X[v];
  };

  // Wave sub-tile: tokens [64 wm, +64); rows: gate_up -> gate [32 wn, +32) and
  // up [64 + 32 wn, +32); down -> [64 wn, +64).
  const int wm = wave & 3, wn = wave >> 2;
  int ncol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ncol[j] = GU ? ((j < 2 ? 0 : 64) + 32 * wn + 16 * (j & 1)) : (64 * wn + 16 * j);

  float4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  auto mma = [&](const _Float16* wt) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      __builtin_amdgcn_sched_barrier(0);   // keep the two K halves' fragments from being live together
      half8v af[4], bf[4];
      const int kk = kh * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const half8v*>(xt + (64 * wm + 16 * i + (lane & 15)) * kTileStride + kk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const half8v*>(wt + (ncol[j] + (lane & 15)) * kTileStride + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Prologue: planes of steps 0 and 1 and activations of step 0 in flight;
  // stage step 0; activations of step 1 in flight.
  prefetch_planes(Pa, 0);
  prefetch_planes(Pb, 1);
  prefetch_x(0);
  __syncthreads();                        // tables in LDS
  decode(Pa, wt0);
  stage_x();
  prefetch_planes(Pa, 2);
  prefetch_x(1);
  __syncthreads();

  // Step k: matrix cores on (xt, wt[k&1]); meanwhile decode step k+1 into the
  // other weight buffer; then stage the activations of step k+1.
  for (int k = 0; k < nk; k += 2) {
    // even step k: weights in wt0; planes of step k+1 in Pb
    mma(wt0);
    if (k + 1 < nk) {
      decode(Pb, wt1);
      prefetch_planes(Pb, k + 3);
    }
    __syncthreads();
    if (k + 1 < nk) {
      stage_x();
      prefetch_x(k + 2);
    }
    __syncthreads();
    if (k + 1 >= nk) break;
    // odd step k+1: weights in wt1; planes of step k+2 in Pa
    mma(wt1);
    if (k + 2 < nk) {
      decode(Pa, wt0);
      prefetch_planes(Pa, k + 4);
    }
    __syncthreads();
    if (k + 2 < nk) {
      stage_x();
      prefetch_x(k + 3);
    }
    __syncthreads();
  }

  // Epilogue.  acc[i][j] element v: token 64 wm + 16 i + 4 (lane >> 4) + v,
  // tile column ncol[j] + (lane & 15).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 64 * wm + 16 * i + 4 * (lane >> 4) + v;
      if (m >= n_e - m0) continue;
      const size_t pos = (size_t)(off_e + m0 + m);
      if constexpr (GU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = ncol[j] + (lane & 15);          // gate row (tile-local < 64)
          if (!mrow_ok<GU>(nt, r, I, H)) continue;
          const float g = acc[i][j][v], u = acc[i][j + 2][v];
          const _Float16 hh = (_Float16)(silu_f32(g) * u);
          A.hout[pos * I + nt * 64 + r] = __builtin_bit_cast(uint16_t, hh);
        }
      } else {
        const size_t slot = (size_t)A.rt.perm[pos];   // o rows are indexed by slot
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = ncol[j] + (lane & 15);
          if (!mrow_ok<GU>(nt, r, I, H)) continue;
          A.oout[slot * H + nt * kTN + r] = acc[i][j][v];
        }
      }
    }
  }
}

// Variant for token tiles less than half full (moderate batches): the
// matrix-core A operand is loaded straight from the activation rows into
// registers, one K step ahead, instead of being staged in LDS, so a step needs
// one barrier instead of two and absent tokens cost no loads; waves whose
// tokens are all absent skip the matrix-core work.  With full tiles the
// LDS-staged kernel above hides the activation latency better (measured on
// the Mixtral-shaped prefill layer: 9.1 ms staged, 10.2 ms direct); with 16
// tokens per expert (Mixtral-shaped layer, T = 64) the call takes 1.43 ms
// instead of 1.98, the batched Qwen-shaped call 0.68 ms instead of 0.81.  The
// switch point (fewer than 128 tokens) was the fastest of 64/128/192/256 on
// the prefill layer; the other two calls did not depend on it.
constexpr int kDirectBelow = 128;
template <int Q, bool GU>
__device__ __forceinline__ void mfma_tile_direct(const MfmaArgs& A, int e, int n_e, int off_e, int m0, int nt, uint8_t* lds) {
  constexpr int TAB = (1 << Q) * 2;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int H = A.H, I = A.I;
  const int N = GU ? 2 * I : H;
  const int K = GU ? H : I;
  const int W = K >> 5;
  const int nk = (K + kTK - 1) / kTK;

  uint8_t* tabs = lds;
  _Float16* wt0 = reinterpret_cast<_Float16*>(lds + kLdsTabs);
  _Float16* wt1 = wt0 + kTN * kTileStride;   // (the activation tile's LDS is unused here)

  const pw_block_desc d = A.blocks[2 * e + (GU ? 0 : 1)];
  const uint32_t pstride = (uint32_t)N * (uint32_t)W * 4u;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(uniform_ptr(d.planes), pstride * (uint32_t)Q);
  const uint16_t* __restrict__ lut = uniform_ptr(d.lut_all) + lut_offset(N, Q);

  // Row tables -> LDS (uint4 chunks; rows outside the block read as zero).
  for (int c = tid; c < kTN * TAB / 16; c += kMfmaThreads) {
    const int r = c / (TAB / 16), cc = c % (TAB / 16);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (mrow_ok<GU>(nt, r, I, H))
      v = *reinterpret_cast<const uint4*>(lut + (size_t)mrow<GU>(nt, r, I) * (1 << Q) + cc * 8);
    *reinterpret_cast<uint4*>(tabs + c * 16) = v;
  }

  // Decode job: row dr, word dw of each K step, weights [16 dh, 16 dh + 16)
  // of that word (the two threads of a pair load the same plane words).
  const int dr = tid >> 2, dw = (tid >> 1) & 1, dh = tid & 1;
  const bool dr_ok = mrow_ok<GU>(nt, dr, I, H);
  const int ddev = dev_row(mrow<GU>(nt, dr, I), I, GU);   // device-layout row
  const uint32_t tab_base = lds_addr(tabs) + (uint32_t)(dr * TAB);
  uint32_t Pa[Q], Pb[Q];

  // plane words of a K step, two steps ahead
  auto prefetch_planes = [&](uint32_t (&P)[Q], int step) {
    if (step >= nk) return;
    const int wc = ((step * kTK) >> 5) + dw;
    const uint32_t voff = (dr_ok && wc < W) ? dev_word(ddev, wc, W) * 4u : kOutOfRange;
#pragma unroll
    for (int p = 0; p < Q; ++p) P[p] = buf_load_u32(prs, voff, (uint32_t)p * pstride);
  };
  auto decode = [&](uint32_t (&P)[Q], _Float16* wt) {
    uint32_t R[8];
    planes_to_fields<Q>(P, R);
    // this thread's half: fields of weights 16 dh + j sit in bytes 2 dh, 2 dh + 1 of R[j & 7]
    uint32_t F[8];
    const uint32_t sel = dh ? 0x0c0c0302u : 0x0c0c0100u;
#pragma unroll
    for (int i = 0; i < 8; ++i) F[i] = __builtin_amdgcn_perm(0u, R[i], sel);
    uint32_t packed[8];
    HalfGroupDecode<Q>::run(F, tab_base, packed);
    uint4* dst = reinterpret_cast<uint4*>(wt + dr * kTileStride + dw * 32 + dh * 16);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  };
  // Wave sub-tile: tokens [64 wm, +64); rows: gate_up -> gate [32 wn, +32) and
  // up [64 + 32 wn, +32); down -> [64 wn, +64).
  const int wm = wave & 3, wn = wave >> 2;
  // Matrix-core A operand straight from the activation rows (no LDS stage):
  // for token block i the lane holds token 64 wm + 16 i + (lane & 15),
  // columns 8 (lane >> 4) .. +8 of each 32-column half of a K step.
  const uint32_t abytes = (uint32_t)((GU ? (size_t)A.T * H : (size_t)A.T * A.k * I) * 2u);
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A.act, abytes);
  uint32_t aoff[4];   // byte offset of the lane's token row (out of range: reads zero)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 64 * wm + 16 * i + (lane & 15);
    aoff[i] = kOutOfRange;
    if (m < n_e - m0) {
      const int pos = off_e + m0 + m;
      aoff[i] = GU ? (uint32_t)(A.rt.perm[pos] / A.k) * (uint32_t)H * 2u : (uint32_t)pos * (uint32_t)I * 2u;
    }
  }
  int ncol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ncol[j] = GU ? ((j < 2 ? 0 : 64) + 32 * wn + 16 * (j & 1)) : (64 * wn + 16 * j);

  float4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  uint4 Ar[2][4];
  auto load_a = [&](uint4 (&Ar)[2][4], int step) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int c = step * kTK + kh * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t voff = c < K ? aoff[i] + 2u * (uint32_t)c : kOutOfRange;
        Ar[kh][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)voff, 0, 0));
      }
    }
  };
  // a wave whose 64 tokens all lie past the expert's last one has nothing to multiply
  const bool wave_live = 64 * wm < n_e - m0;
  auto mma = [&](const _Float16* wt, const uint4 (&Ar)[2][4]) {
    if (!wave_live) return;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      __builtin_amdgcn_sched_barrier(0);   // keep the two K halves' fragments from being live together
      half8v af[4], bf[4];
      const int kk = kh * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = __builtin_bit_cast(half8v, Ar[kh][i]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const half8v*>(wt + (ncol[j] + (lane & 15)) * kTileStride + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Prologue: planes of steps 0 and 1 and activations of step 0 in flight;
  // decode step 0.
  load_a(Ar, 0);
  prefetch_planes(Pa, 0);
  prefetch_planes(Pb, 1);
  __syncthreads();                        // tables in LDS
  decode(Pa, wt0);
  prefetch_planes(Pa, 2);
  __syncthreads();

  // Step k: matrix cores on wt[k&1] with the activations in registers; then
  // request the activations of step k+1 and decode step k+1 into the other
  // weight buffer.  One barrier per step: after it the decoded tile is
  // complete and nobody reads the buffer the next decode overwrites.
  for (int k = 0; k < nk; k += 2) {
    mma(wt0, Ar);
    if (k + 1 < nk) {
      load_a(Ar, k + 1);
      decode(Pb, wt1);
      prefetch_planes(Pb, k + 3);
    }
    __syncthreads();
    if (k + 1 >= nk) break;
    mma(wt1, Ar);
    if (k + 2 < nk) {
      load_a(Ar, k + 2);
      decode(Pa, wt0);
      prefetch_planes(Pa, k + 4);
    }
    __syncthreads();
  }

  // Epilogue.  acc[i][j] element v: token 64 wm + 16 i + 4 (lane >> 4) + v,
  // tile column ncol[j] + (lane & 15).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 64 * wm + 16 * i + 4 * (lane >> 4) + v;
      if (m >= n_e - m0) continue;
      const size_t pos = (size_t)(off_e + m0 + m);
      if constexpr (GU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = ncol[j] + (lane & 15);          // gate row (tile-local < 64)
          if (!mrow_ok<GU>(nt, r, I, H)) continue;
          const float g = acc[i][j][v], u = acc[i][j + 2][v];
          const _Float16 hh = (_Float16)(silu_f32(g) * u);
          A.hout[pos * I + nt * 64 + r] = __builtin_bit_cast(uint16_t, hh);
        }
      } else {
        const size_t slot = (size_t)A.rt.perm[pos];   // o rows are indexed by slot
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = ncol[j] + (lane & 15);
          if (!mrow_ok<GU>(nt, r, I, H)) continue;
          A.oout[slot * H + nt * kTN + r] = acc[i][j][v];
        }
      }
    }
  }
}

template <bool GU>
__device__ __forceinline__ void mfma_zero_tile(const MfmaArgs& A, int n_e, int off_e, int m0, int nt) {
  for (int i = threadIdx.x; i < kTM * kTN; i += kMfmaThreads) {
    const int m = i / kTN, r = i % kTN;
    if (m >= n_e - m0) continue;
    const size_t pos = (size_t)(off_e + m0 + m);
    if constexpr (GU) {
      if (r < 64 && mrow_ok<GU>(nt, r, A.I, A.H)) A.hout[pos * A.I + nt * 64 + r] = 0;
    } else {
      if (mrow_ok<GU>(nt, r, A.I, A.H)) A.oout[(size_t)A.rt.perm[pos] * A.H + nt * kTN + r] = 0.0f;
    }
  }
  if (threadIdx.x == 0 && nt == 0 && m0 == 0) raise_status(A.rt.status, PW_DEV_BAD_BITWIDTH);
}

template <bool GU>
__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(MfmaArgs A) {
  __shared__ __align__(16) uint8_t lds[kMfmaLds];
  // deal items so that one XCD works through consecutive items
  const int per_xcd = A.grid / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int mi = item / A.ntiles;
  const int nt = item % A.ntiles;
  if (mi >= uniform(*A.rt.num_mtiles)) return;
  const int e = uniform(A.rt.mtiles[2 * mi]);
  const int m0 = uniform(A.rt.mtiles[2 * mi + 1]);
  const int n_e = uniform(A.rt.counts[e]);
  const int off_e = uniform(A.rt.offsets[e]);
  const int qv = uniform(A.q[2 * e + (GU ? 0 : 1)]);
  if (qv < kMinBits || qv > kMaxBits) {
    mfma_zero_tile<GU>(A, n_e, off_e, m0, nt);
  } else if (n_e - m0 >= kDirectBelow || !A.direct_ok) {
    switch (qv) {
      case 3: mfma_tile<3, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 4: mfma_tile<4, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 5: mfma_tile<5, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 6: mfma_tile<6, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 7: mfma_tile<7, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      default: mfma_tile<8, GU>(A, e, n_e, off_e, m0, nt, lds); break;
    }
  } else {
    switch (qv) {
      case 3: mfma_tile_direct<3, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 4: mfma_tile_direct<4, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 5: mfma_tile_direct<5, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 6: mfma_tile_direct<6, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      case 7: mfma_tile_direct<7, GU>(A, e, n_e, off_e, m0, nt, lds); break;
      default: mfma_tile_direct<8, GU>(A, e, n_e, off_e, m0, nt, lds); break;
    }
  }
}

template <bool GU>
static hipError_t launch_mfma(const ExpertArgs& a, const uint16_t* act, uint16_t* h, float* o, hipStream_t s,
                              const KernelEvents& ev) {
  MfmaArgs A{};
  A.H = a.H; A.I = a.I; A.E = a.E; A.k = a.k; A.T = a.T;
  A.blocks = a.blocks; A.q = a.q; A.rt = a.rt;
  A.act = act; A.hout = h; A.oout = o;
  A.ntiles = GU ? (a.I + 63) / 64 : (a.H + kTN - 1) / kTN;
  const long long act_bytes = 2LL * (GU ? (long long)a.T * a.H : (long long)a.T * a.k * a.I);
  A.direct_ok = act_bytes < 0x80000000LL ? 1 : 0;
  const long long items = (long long)mtile_bound(a.E, a.T, a.k) * A.ntiles;
  const long long grid = (items + kXcds - 1) / kXcds * kXcds;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  A.grid = (int)grid;
  return launch_kernel(mfma_kernel<GU>, dim3((unsigned)grid), dim3(kMfmaThreads), s, ev, A);
}

hipError_t launch_mfma_gate_up(const ExpertArgs& a, const uint16_t* x, uint16_t* h, hipStream_t s,
                               const KernelEvents& ev) {
  return launch_mfma<true>(a, x, h, nullptr, s, ev);
}

hipError_t launch_mfma_down(const ExpertArgs& a, const uint16_t* h, float* o, hipStream_t s, const KernelEvents& ev) {
  return launch_mfma<false>(a, h, nullptr, o, s, ev);
}

}  // namespace pw
