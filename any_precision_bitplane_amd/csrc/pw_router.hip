// Router and online routing statistics.
//
// "Technical summary: PagedWeight", Core components 2, second bullet (online
// routing statistics): the system tracks each expert's routing mass, how often
// it is selected and with what weight.  The router itself is the plain top-k
// softmax router of the synthetic layers: logits = x Wr^T, the k largest
// logits in descending order (lower expert id first on equal logits), weights
// = softmax over the selected logits.
//
// Two launches (a single-workgroup variant for decode batches, logits in LDS,
// took 17.6 us instead of 9.2 on the Qwen-shaped decode layer: its 32 serial
// wave sums cost more than the second launch):
//   logits_kernel  one wave per (expert, tile of 4 tokens): lanes stride over H
//                  in 8-element chunks, fp16 pairs multiplied into fp32 with
//                  v_dot2, one butterfly sum per token; logits fp32 [T][E].
//   topk_kernel    one wave per token: k rounds of a wave-wide (value desc,
//                  id asc) butterfly arg-max; lane j keeps slot j; softmax
//                  with the device exp; lane j writes slot j and adds it to
//                  the routing statistics (count exact, mass an fp32 atomic
//                  sum whose order varies between runs).
#include <limits.h>

#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kRouterTokens = 4;     // tokens per wave in the logits kernel
constexpr int kRouterWaves = 4;      // waves per workgroup (both kernels)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__global__ __launch_bounds__(kRouterWaves * kWave) void logits_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ wr, int T, int H,
                                                                       int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.y * kRouterWaves + (int)(threadIdx.x / kWave);
  const int t0 = blockIdx.x * kRouterTokens;
  if (e >= E) return;
  const int nt = T - t0 < kRouterTokens ? T - t0 : kRouterTokens;
  float acc[kRouterTokens];
#pragma unroll
  for (int t = 0; t < kRouterTokens; ++t) acc[t] = 0.f;
  const uint16_t* wrow = wr + (size_t)e * H;
  for (int h = lane * 8; h < H; h += kWave * 8) {
    const half8_t wv = *reinterpret_cast<const half8_t*>(wrow + h);
#pragma unroll
    for (int t = 0; t < kRouterTokens; ++t) {
      if (t >= nt) continue;
      const half8_t xv = *reinterpret_cast<const half8_t*>(x + (size_t)(t0 + t) * H + h);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[t] = __builtin_amdgcn_fdot2(half2_t{wv[2 * i], wv[2 * i + 1]}, half2_t{xv[2 * i], xv[2 * i + 1]}, acc[t],
                                        false);
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterTokens; ++t) {
    if (t >= nt) continue;
    const float s = wave_sum(acc[t]);
    if (lane == 0) logits[(size_t)(t0 + t) * E + e] = s;
  }
}

// Selection and softmax of token t from its logits l[e] (e < E; lane owns
// e = lane + 64 i, E <= 256): k rounds of a (value desc, id asc) butterfly
// arg-max, slot j kept in lane j; lane j writes slot j and its statistics.
__device__ __forceinline__ void select_topk(const float* l, int E, int k, int t, int32_t* ids, float* w,
                                            uint32_t* count, float* mass) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[4];
  bool live[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    live[i] = e < E;
    v[i] = live[i] ? l[e] : 0.f;
  }
  float my_l = 0.f;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + kWave * i;
      if (live[i] && (bi == INT_MAX || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (oi != INT_MAX && (bi == INT_MAX || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == j) {
      my_l = bv;
      my_e = bi;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + kWave * i == bi) live[i] = false;
  }
  const float top = __shfl(my_l, 0, kWave);
  const float z = lane < k ? __expf(my_l - top) : 0.f;
  const float s = wave_sum(z);
  if (lane < k) {
    const float wj = z / s;
    const size_t slot = (size_t)t * k + lane;
    ids[slot] = my_e;
    w[slot] = wj;
    if (count) atomicAdd(count + my_e, 1u);
    if (mass) atomicAdd(mass + my_e, wj);
  }
}

// One wave per token over logits fp32 [T][E] in global memory.
__global__ __launch_bounds__(kRouterWaves * kWave) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                                     int k, int32_t* __restrict__ ids,
                                                                     float* __restrict__ w,
                                                                     uint32_t* __restrict__ count,
                                                                     float* __restrict__ mass) {
  const int t = blockIdx.x * kRouterWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  select_topk(logits + (size_t)t * E, E, k, t, ids, w, count, mass);
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k, float* logits,
                         int32_t* ids, float* w, uint32_t* count, float* mass, hipStream_t s) {
  dim3 g1((T + kRouterTokens - 1) / kRouterTokens, (E + kRouterWaves - 1) / kRouterWaves);
  hipLaunchKernelGGL(logits_kernel, g1, dim3(kRouterWaves * kWave), 0, s, x, wr, T, H, E, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((T + kRouterWaves - 1) / kRouterWaves);
  hipLaunchKernelGGL(topk_kernel, g2, dim3(kRouterWaves * kWave), 0, s, logits, T, E, k, ids, w, count, mass);
  return hipGetLastError();
}

}  // namespace pw
