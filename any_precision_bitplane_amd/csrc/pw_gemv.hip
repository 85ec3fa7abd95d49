// Bit-plane / lookup-table GEMV kernels for the expert products when an
// expert has few tokens (decode).  "Technical summary: PagedWeight", Core
// components 3 (fused mixed-precision kernel): the kernel reads the planes and
// the tables directly and runs every block at its own committed bitwidth q,
// which it reads from the device page table, so a commit never changes a launch
// argument.
//
// Work decomposition.  A workgroup is one wave and owns 8 rows of one routed
// expert's block.  Its 64 lanes split a row's K/32 plane words (lane = word
// column, slices of 64 words), so
//   * each plane load of a row is one 256-byte coalesced wave access, and only
//     planes 0..q-1 are read (buffer loads, plane offset in a scalar register);
//   * a lane's 32 activations per token stay in registers for all 8 rows;
//   * all lanes look up the same row's table, which keeps the LDS gather free
//     of bank conflicts up to 64 table entries, and the row's table address is
//     an instruction immediate.
// The gate_up workgroup takes 4 matching gate and up rows (i and I + i), so
// SwiGLU runs in the epilogue and h = SiLU(gate) * up leaves as fp16.
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kRows = 8;                                   // rows per workgroup (= wave)
constexpr int kMaxTabBytes = (1 << kMaxBits) * 2;          // 512 B per row table

struct GemvParams {
  ExpertArgs a;
  const uint16_t* act;   // gate_up: x [T][H];  down: h [slots][I] (sorted positions)
  void* out;             // gate_up: h fp16 [slots][I];  down: o fp32 [slots][H]
  int tiles;             // row tiles per expert
};

// Row r (0..7) of tile `tile`; gate_up tiles hold gate rows i..i+3 then the
// matching up rows I+i..I+i+3.
template <bool GU>
__device__ __forceinline__ int tile_row(int tile, int r, int I) {
  if constexpr (GU) return (r < 4 ? 0 : I) + tile * 4 + (r & 3);
  else return tile * kRows + r;
}

template <bool GU>
__device__ __forceinline__ bool row_valid(int tile, int r, int I, int H) {
  if constexpr (GU) return tile * 4 + (r & 3) < I;
  else return tile * kRows + r < H;
}

template <int Q, int NT, bool GU>
__device__ __forceinline__ void gemv_body(const GemvParams& p, int e, int n_e, int tile, uint8_t* lds) {
  const int lane = threadIdx.x;
  const int H = p.a.H, I = p.a.I, k = p.a.k;
  const int N = GU ? 2 * I : H;
  const int K = GU ? H : I;
  const int W = K >> 5;
  const pw_block_desc d = p.a.blocks[2 * e + (GU ? 0 : 1)];
  const uint32_t pstride = (uint32_t)N * (uint32_t)W * 4u;          // bytes per plane
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(d.planes, pstride * Q);
  const uint16_t* __restrict__ lut = d.lut_all + lut_offset(N, Q);
  const int off_e = p.a.rt.offsets[e];
  const int* __restrict__ perm = p.a.rt.perm;

  // Stage the 8 row tables (2^Q fp16 each) into LDS.
  constexpr int TAB = (1 << Q) * 2;
  constexpr int CH = TAB / 16;            // 16-byte chunks per table
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const bool rv = row_valid<GU>(tile, r, I, H);
    for (int c = lane; c < CH; c += kWave) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (rv) v = *reinterpret_cast<const uint4*>(lut + (size_t)tile_row<GU>(tile, r, I) * (1 << Q) + c * 8);
      *reinterpret_cast<uint4*>(lds + r * TAB + c * 16) = v;
    }
  }
  __syncthreads();

  for (int t0 = 0; t0 < n_e; t0 += NT) {
    const int nt = min(NT, n_e - t0);
    float acc[kRows][NT];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = 0.0f;

    for (int s0 = 0; s0 < W; s0 += kWave) {
      const int wc = s0 + lane;
      const bool cv = wc < W;

      // First Q plane words of the 8 rows (zero outside the block).
      uint32_t P[kRows][Q];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const bool ok = cv && row_valid<GU>(tile, r, I, H);
        const uint32_t voff = ok ? ((uint32_t)tile_row<GU>(tile, r, I) * (uint32_t)W + (uint32_t)wc) * 4u
                                 : kOutOfRange;
#pragma unroll
        for (int pp = 0; pp < Q; ++pp) P[r][pp] = buf_load_u32(prs, voff, pp * pstride);
      }

      // Activations of this word column (32 values per token).
      half2_t xr[NT][16];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint16_t* src = nullptr;
        if (t < nt && cv) {
          const int pos = off_e + t0 + t;
          src = GU ? p.act + (size_t)(perm[pos] / k) * H : p.act + (size_t)pos * I;
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint4 u = make_uint4(0u, 0u, 0u, 0u);
          if (src) u = *reinterpret_cast<const uint4*>(src + wc * 32 + v * 8);
          xr[t][4 * v + 0] = __builtin_bit_cast(half2_t, u.x);
          xr[t][4 * v + 1] = __builtin_bit_cast(half2_t, u.y);
          xr[t][4 * v + 2] = __builtin_bit_cast(half2_t, u.z);
          xr[t][4 * v + 3] = __builtin_bit_cast(half2_t, u.w);
        }
      }

#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        uint32_t R[8];
        planes_to_fields<Q>(P[r], R);
        const uint8_t* tab = lds + r * TAB;
#pragma unroll
        for (int j = 0; j < 32; j += 2) {
          const half2_t w2 = lookup_pair<Q>(R, tab, j);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[r][t] = __builtin_amdgcn_fdot2(w2, xr[t][j >> 1], acc[r][t], false);
        }
      }
    }

#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = wave_sum(acc[r][t]);

    if constexpr (GU) {
      uint16_t* hout = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (lane == r * NT + t && t < nt && row_valid<GU>(tile, r, I, H)) {
            const float h = silu_f32(acc[r][t]) * acc[r + 4][t];
            const _Float16 hh = (_Float16)h;
            hout[(size_t)(off_e + t0 + t) * I + tile_row<GU>(tile, r, I)] = __builtin_bit_cast(uint16_t, hh);
          }
    } else {
      float* oout = reinterpret_cast<float*>(p.out);
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (lane == r * NT + t && t < nt && row_valid<GU>(tile, r, I, H))
            oout[(size_t)(off_e + t0 + t) * H + tile_row<GU>(tile, r, I)] = acc[r][t];
    }
  }
}

// Rows of a block whose committed bitwidth is invalid read as zero.
template <bool GU>
__device__ void gemv_zero_rows(const GemvParams& p, int e, int n_e, int tile) {
  const int lane = threadIdx.x;
  const int H = p.a.H, I = p.a.I;
  const int off_e = p.a.rt.offsets[e];
  for (int t = lane; t < n_e; t += kWave) {
#pragma unroll
    for (int r = 0; r < (GU ? 4 : kRows); ++r) {
      if (!row_valid<GU>(tile, r, I, H)) continue;
      const int row = tile_row<GU>(tile, r, I);
      if constexpr (GU) reinterpret_cast<uint16_t*>(p.out)[(size_t)(off_e + t) * I + row] = 0;
      else reinterpret_cast<float*>(p.out)[(size_t)(off_e + t) * H + row] = 0.0f;
    }
  }
  if (lane == 0 && tile == 0) raise_status(p.a.rt.status, PW_DEV_BAD_BITWIDTH);
}

template <int Q, bool GU>
__device__ __forceinline__ void gemv_by_tokens(const GemvParams& p, int e, int n_e, int tile, uint8_t* lds) {
  if (n_e == 1) gemv_body<Q, 1, GU>(p, e, n_e, tile, lds);
  else gemv_body<Q, 2, GU>(p, e, n_e, tile, lds);
}

template <bool GU>
__global__ __launch_bounds__(kWave) void gemv_kernel(GemvParams p) {
  __shared__ __align__(16) uint8_t lds[kRows * kMaxTabBytes];
  const int a = blockIdx.x / p.tiles;
  const int tile = blockIdx.x % p.tiles;
  if (a >= *p.a.rt.num_active) return;
  const int e = p.a.rt.active[a];
  const int n_e = p.a.rt.counts[e];
  if (n_e < p.a.min_tokens || n_e >= p.a.max_tokens) return;
  switch (p.a.q[2 * e + (GU ? 0 : 1)]) {
    case 3: gemv_by_tokens<3, GU>(p, e, n_e, tile, lds); break;
    case 4: gemv_by_tokens<4, GU>(p, e, n_e, tile, lds); break;
    case 5: gemv_by_tokens<5, GU>(p, e, n_e, tile, lds); break;
    case 6: gemv_by_tokens<6, GU>(p, e, n_e, tile, lds); break;
    case 7: gemv_by_tokens<7, GU>(p, e, n_e, tile, lds); break;
    case 8: gemv_by_tokens<8, GU>(p, e, n_e, tile, lds); break;
    default: gemv_zero_rows<GU>(p, e, n_e, tile); break;
  }
}

static int active_bound(const ExpertArgs& a) { return a.E < a.T * a.k ? a.E : a.T * a.k; }

hipError_t launch_gemv_gate_up(const ExpertArgs& a, const uint16_t* x, uint16_t* h, hipStream_t s) {
  GemvParams p{a, x, h, (a.I + 3) / 4};
  const int grid = active_bound(a) * p.tiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(gemv_kernel<true>, dim3(grid), dim3(kWave), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const ExpertArgs& a, const uint16_t* h, float* o, hipStream_t s) {
  GemvParams p{a, h, o, (a.H + kRows - 1) / kRows};
  const int grid = active_bound(a) * p.tiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(gemv_kernel<false>, dim3(grid), dim3(kWave), 0, s, p);
  return hipGetLastError();
}

}  // namespace pw
