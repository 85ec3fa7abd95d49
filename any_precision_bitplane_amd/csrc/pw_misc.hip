// Weighted top-k combine and the block dequantization export.
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

// y[t][n] = fp16( sum_{j < k, ascending} w[t][j] * o[t*k + j][n] ), where o
// is indexed by slot and is the sum of its K parts (the down product may split
// K across waves).  The router weights are used as given; a slot the routing
// dropped (expert id out of range) has inv = -1 and adds nothing (its o row is
// never written).  Fixed j order and no atomics, so the result is
// deterministic (combine4 in pw_device.h).
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ o,
                                                                  const float* __restrict__ w,
                                                                  const int32_t* __restrict__ inv, int k, int H,
                                                                  int kparts, size_t part_stride,
                                                                  uint16_t* __restrict__ y) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * kCombineThreads + threadIdx.x) * 4;
  if (n >= H) return;
  const floatx4 a = combine4(o, w, inv, t, k, H, kparts, part_stride, n);
  *reinterpret_cast<uint2*>(y + (size_t)t * H + n) = pack_half4(a);
}

hipError_t launch_combine(const float* o, const float* w, const int32_t* inv, int T, int k, int H, int kparts,
                          uint16_t* y, hipStream_t s) {
  const int per_block = kCombineThreads * 4;
  dim3 grid((H + per_block - 1) / per_block, T);
  const size_t part_stride = (size_t)T * k * H;
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombineThreads), 0, s, o, w, inv, k, H, kparts, part_stride, y);
  return hipGetLastError();
}

// Canonical planes [nplanes][N][W] -> device layout (see pw_device.h).  One
// thread per destination word, in destination order, so the stores are
// contiguous; the loads gather along rows.  A pure permutation of words.
__global__ __launch_bounds__(256) void pack_kernel(const uint32_t* __restrict__ src, int N, int W, size_t total,
                                                   int I_gu, uint32_t* __restrict__ dst) {
  const size_t plane = (size_t)N * W;
  const uint32_t tile_row = 16u * (uint32_t)W;
  const int nfull = W >> 4;                 // full 16-word column tiles
  const int wlast = W - 16 * nfull;         // width of the last, partial one (0: none)
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t p = i / plane;
    const uint32_t off = (uint32_t)(i - p * plane);
    const uint32_t rt = off / tile_row;
    const uint32_t rem = off - rt * tile_row;
    int r, c;
    if (rem < 256u * (uint32_t)nfull) {
      const uint32_t ct = rem >> 8, within = rem & 255u;
      r = (int)(within >> 4);
      c = (int)(16u * ct + (within & 15u));
    } else {
      const uint32_t within = rem - 256u * (uint32_t)nfull;
      r = (int)(within / (uint32_t)wlast);
      c = 16 * nfull + (int)(within - (uint32_t)r * (uint32_t)wlast);
    }
    const int d = (int)(16u * rt) + r;
    const int n = I_gu > 0 ? canon_row(d, I_gu, true) : d;
    dst[i] = src[p * plane + (size_t)n * W + c];
  }
}

hipError_t launch_pack(const uint32_t* canon, int N, int K, int nplanes, int module, uint32_t* out, hipStream_t s) {
  const int W = K >> 5;
  const size_t total = (size_t)nplanes * N * W;
  size_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, canon, N, W, total,
                     module == 0 ? N / 2 : 0, out);
  return hipGetLastError();
}

// Dequantize one block at bitwidth Q: out[n][c] = table_Q[n][code_Q(n, c)]
// ("Technical summary: PagedWeight", Core components 1), rows in canonical
// order, planes read from the device layout.  Same decode as the GEMV
// kernels: a wave owns 8 rows, lanes own plane-word columns, the row tables
// sit in LDS.
constexpr int kDqThreads = 256;
constexpr int kDqRowsPerWave = 8;

template <int Q>
__global__ __launch_bounds__(kDqThreads) void dequant_kernel(const uint32_t* __restrict__ planes,
                                                            const uint16_t* __restrict__ lut_all, int N, int K,
                                                            int I_gu, uint16_t* __restrict__ out) {
  constexpr int TAB = (1 << Q) * 2;
  constexpr int CH = TAB / 16;
  __shared__ __align__(16) uint8_t lds[(kDqThreads / kWave) * kDqRowsPerWave * TAB];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int W = K >> 5;
  const size_t pstride = (size_t)N * W;
  const uint16_t* lut = lut_all + lut_offset(N, Q);
  const int row0 = (blockIdx.x * (kDqThreads / kWave) + wave) * kDqRowsPerWave;
  uint8_t* tabs = lds + wave * kDqRowsPerWave * TAB;

#pragma unroll
  for (int r = 0; r < kDqRowsPerWave; ++r) {
    const int row = row0 + r;
    for (int c = lane; c < CH; c += kWave) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < N) v = *reinterpret_cast<const uint4*>(lut + (size_t)row * (1 << Q) + c * 8);
      *reinterpret_cast<uint4*>(tabs + r * TAB + c * 16) = v;
    }
  }
  __syncthreads();

  for (int s0 = 0; s0 < W; s0 += kWave) {
    const int wc = s0 + lane;
    if (wc >= W) continue;
#pragma unroll
    for (int r = 0; r < kDqRowsPerWave; ++r) {
      const int row = row0 + r;
      if (row >= N) continue;
      const size_t src = dev_word(I_gu > 0 ? dev_row(row, I_gu, true) : row, wc, W);
      uint32_t P[Q];
#pragma unroll
      for (int pp = 0; pp < Q; ++pp) P[pp] = planes[pp * pstride + src];
      uint32_t R[8];
      planes_to_fields<Q>(P, R);
      uint32_t packed[16];
      GroupDecode<Q, 0>::run(R, lds_addr(tabs + r * TAB), packed);
      uint4* dst = reinterpret_cast<uint4*>(out + (size_t)row * K + (size_t)wc * 32);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        dst[v] = make_uint4(packed[4 * v], packed[4 * v + 1], packed[4 * v + 2], packed[4 * v + 3]);
    }
  }
}

hipError_t launch_dequant(const uint32_t* planes, const uint16_t* lut_all, int N, int K, int q, int module,
                          uint16_t* out, hipStream_t s) {
  const int rows_per_block = (kDqThreads / kWave) * kDqRowsPerWave;
  dim3 grid((N + rows_per_block - 1) / rows_per_block);
  const int I_gu = module == 0 ? N / 2 : 0;
  switch (q) {
    case 3: hipLaunchKernelGGL(dequant_kernel<3>, grid, dim3(kDqThreads), 0, s, planes, lut_all, N, K, I_gu, out); break;
    case 4: hipLaunchKernelGGL(dequant_kernel<4>, grid, dim3(kDqThreads), 0, s, planes, lut_all, N, K, I_gu, out); break;
    case 5: hipLaunchKernelGGL(dequant_kernel<5>, grid, dim3(kDqThreads), 0, s, planes, lut_all, N, K, I_gu, out); break;
    case 6: hipLaunchKernelGGL(dequant_kernel<6>, grid, dim3(kDqThreads), 0, s, planes, lut_all, N, K, I_gu, out); break;
    case 7: hipLaunchKernelGGL(dequant_kernel<7>, grid, dim3(kDqThreads), 0, s, planes, lut_all, N, K, I_gu, out); break;
    case 8: hipLaunchKernelGGL(dequant_kernel<8>, grid, dim3(kDqThreads), 0, s, planes, lut_all, N, K, I_gu, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pw

namespace pw {

// Zero [p, p + bytes): 16-byte stores for the aligned body, byte stores for the tail.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* p, size_t n16, size_t bytes) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0u, 0u, 0u, 0u);
  const size_t tail = n16 * 16;
  for (size_t i = tail + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes; i += stride) p[i] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint8_t*>(p), n16,
                     bytes);
  return hipGetLastError();
}

}  // namespace pw
