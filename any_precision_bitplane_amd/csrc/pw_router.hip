// Router and online routing statistics.
//
// "Technical summary: PagedWeight", Core components 2, second bullet (online
// routing statistics): the system tracks each expert's routing mass, how often
// it is selected and with what weight.  The router itself is the plain top-k
// softmax router of the synthetic layers: logits = x Wr^T, the k largest
// logits in descending order (lower expert id first on equal logits), weights
// = softmax over the selected logits.
//
// One launch: a workgroup of sixteen waves takes TT tokens (1 for batches of
// up to 256 tokens, 4 above, so larger batches share each router row read),
// the waves split the experts, each wave's lanes stride over H in 8-element
// chunks (fp16 pairs multiplied into fp32 with v_dot2, one wave-wide DPP sum
// per token and expert), and the logits meet in LDS; then wave t selects the
// top-k of token t: k rounds of a wave-wide DPP max and a ballot for the
// lowest id holding it, lane j keeping slot j, softmax with the device exp,
// lane j writing slot j and its statistics (count exact, mass an fp32 atomic
// sum whose order varies between runs).  An earlier form used two launches (logits, then top-k through global
// memory); on the Qwen-shaped decode layer the second launch and its gap cost
// about as much as the work.
#include <limits.h>

#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kRouterTokens = 4;     // tokens per workgroup for batches above 256 tokens
constexpr int kRouterWaves = 16;     // waves per workgroup

// Wave-wide sum and max in DPP: inside each 16-lane row, partners lane ^ 1,
// lane ^ 2, then the mirror inside 8 lanes and inside 16 lanes (each pairing
// is symmetric, so every lane of a row ends with the same bits); then the four
// rows' values read out of lanes 0, 16, 32, 48 and combined the same way in
// every lane.  All 64 lanes must be active.  A shuffle-based butterfly (one
// LDS permute per step) made the router's top-k rounds a chain of permutes.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kHalfRowMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row_lane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_row<kQuadXor1>(v);
  v += dpp_row<kQuadXor2>(v);
  v += dpp_row<kHalfRowMirror>(v);
  v += dpp_row<kRowMirror>(v);
  return (row_lane(v, 0) + row_lane(v, 16)) + (row_lane(v, 32) + row_lane(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_row<kQuadXor1>(v));
  v = fmaxf(v, dpp_row<kQuadXor2>(v));
  v = fmaxf(v, dpp_row<kHalfRowMirror>(v));
  v = fmaxf(v, dpp_row<kRowMirror>(v));
  return fmaxf(fmaxf(row_lane(v, 0), row_lane(v, 16)), fmaxf(row_lane(v, 32), row_lane(v, 48)));
}

// Selection and softmax of token t from its logits l[e] (e < E; lane owns
// e = lane + 64 i, E <= 256): k rounds of a wave-wide max over the live
// logits, the lowest expert id holding it found by ballot (so equal logits
// go to the lower id), slot j kept in lane j; lane j writes slot j and its
// statistics.  NaN logits count as -inf.
__device__ __forceinline__ void select_topk(const float* l, int E, int k, int t, int32_t* ids, float* w,
                                            uint32_t* count, float* mass) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[4];
  bool live[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    live[i] = e < E;
    const float x = live[i] ? l[e] : -INFINITY;
    v[i] = x == x ? x : -INFINITY;
  }
  float my_l = 0.f, top = 0.f;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (live[i]) lm = fmaxf(lm, v[i]);
    const float m = wave_max(lm);
    int bi = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned long long b = __ballot(live[i] && v[i] == m);
      if (bi < 0 && b) bi = kWave * i + __ffsll((long long)b) - 1;
    }
    if (j == 0) top = m;
    if (lane == j) {
      my_l = m;
      my_e = bi;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + kWave * i == bi) live[i] = false;
  }
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

// Logits of the tile's tokens from x rows (global memory, or LDS), into lg.
// Wave w takes experts w, w + 16, w + 32, ... in groups of four whose router
// rows are read together, lanes striding over H in 8-element chunks; the
// four experts' (and TT tokens') butterfly sums run as independent chains.
constexpr int kRtGroup = 4;
template <int TT>
__device__ __forceinline__ void router_logits(const uint16_t* x, size_t x_stride, const uint16_t* __restrict__ wr,
                                              int nt, int H, int E, float (&lg)[TT][kMaxExperts]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int e0 = wave; e0 < E; e0 += kRouterWaves * kRtGroup) {
    float acc[kRtGroup][TT];
#pragma unroll
    for (int g = 0; g < kRtGroup; ++g)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[g][t] = 0.f;
    // U 512-element chunks per pass, every load of a pass issued before any
    // arithmetic (one memory round trip per pass instead of one per chunk)
    constexpr int U = 4 / TT;
    for (int hb = 0; hb < H; hb += U * kWave * 8) {
      half8_t xv[U][TT], wv[U][kRtGroup];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int h = hb + u * kWave * 8 + lane * 8;
        if (h >= H) continue;
#pragma unroll
        for (int t = 0; t < TT; ++t)
          if (t < nt) xv[u][t] = *reinterpret_cast<const half8_t*>(x + (size_t)t * x_stride + h);
#pragma unroll
        for (int g = 0; g < kRtGroup; ++g) {
          const int e = e0 + g * kRouterWaves;
          if (e < E) wv[u][g] = *reinterpret_cast<const half8_t*>(wr + (size_t)e * H + h);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int h = hb + u * kWave * 8 + lane * 8;
        if (h >= H) continue;
#pragma unroll
        for (int g = 0; g < kRtGroup; ++g) {
          if (e0 + g * kRouterWaves >= E) continue;
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            if (t >= nt) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[g][t] = __builtin_amdgcn_fdot2(half2_t{wv[u][g][2 * i], wv[u][g][2 * i + 1]},
                                                 half2_t{xv[u][t][2 * i], xv[u][t][2 * i + 1]}, acc[g][t], false);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kRtGroup; ++g)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[g][t] = wave_sum(acc[g][t]);
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < kRtGroup; ++g) {
        const int e = e0 + g * kRouterWaves;
#pragma unroll
        for (int t = 0; t < TT; ++t)
          if (e < E && t < nt) lg[t][e] = acc[g][t];
      }
    }
  }
}

template <int TT>
__global__ __launch_bounds__(kRouterWaves * kWave) void router_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ wr, int T, int H,
                                                                       int E, int k, int32_t* __restrict__ ids,
                                                                       float* __restrict__ w,
                                                                       uint32_t* __restrict__ count,
                                                                       float* __restrict__ mass) {
  __shared__ float lg[TT][kMaxExperts];
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * TT;
  const int nt = T - t0 < TT ? T - t0 : TT;
  router_logits<TT>(x + (size_t)t0 * H, (size_t)H, wr, nt, H, E, lg);
  __syncthreads();
  if (wave < nt) select_topk(lg[wave], E, k, t0 + wave, ids, w, count, mass);
}

// Layer boundary of a multi-layer call: token t's weighted combine of the
// previous layer (the combine kernel's arithmetic, combine4) is written to
// x_out and kept in LDS, then routed for the next layer.  w may alias w_prev:
// every read of w_prev precedes the barrier, every write of w follows it.
__global__ __launch_bounds__(kRouterWaves * kWave) void combine_router_kernel(
    const float* __restrict__ o, const float* w_prev, const int32_t* __restrict__ inv, int kparts, size_t part_stride,
    uint16_t* __restrict__ x_out, const uint16_t* __restrict__ wr, int H, int E, int k, int32_t* __restrict__ ids,
    float* w, uint32_t* __restrict__ count, float* __restrict__ mass) {
  __shared__ float lg[1][kMaxExperts];
  __shared__ __align__(16) uint16_t xs[kMaxRouterHidden];
  const int t = blockIdx.x;
  for (int n = 4 * (int)threadIdx.x; n < H; n += 4 * kRouterWaves * kWave) {
    const uint2 p = pack_half4(combine4(o, w_prev, inv, t, k, H, kparts, part_stride, n));
    *reinterpret_cast<uint2*>(x_out + (size_t)t * H + n) = p;
    *reinterpret_cast<uint2*>(xs + n) = p;
  }
  __syncthreads();
  router_logits<1>(xs, (size_t)H, wr, 1, H, E, lg);
  __syncthreads();
  if (threadIdx.x < kWave) select_topk(lg[0], E, k, t, ids, w, count, mass);
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k, int32_t* ids, float* w,
                         uint32_t* count, float* mass, hipStream_t s) {
  if (T <= 256) {
    hipLaunchKernelGGL(router_kernel<1>, dim3(T), dim3(kRouterWaves * kWave), 0, s, x, wr, T, H, E, k, ids, w, count,
                       mass);
  } else {
    static_assert(kRouterTokens <= kRouterWaves, "one selecting wave per token of the tile");
    hipLaunchKernelGGL(router_kernel<kRouterTokens>, dim3((T + kRouterTokens - 1) / kRouterTokens),
                       dim3(kRouterWaves * kWave), 0, s, x, wr, T, H, E, k, ids, w, count, mass);
  }
  return hipGetLastError();
}

hipError_t launch_combine_router(const float* o, const float* w_prev, const int32_t* inv, int kparts,
                                 uint16_t* x_out, const uint16_t* wr, int T, int H, int E, int k, int32_t* ids,
                                 float* w, uint32_t* count, float* mass, hipStream_t s) {
  if (H > kMaxRouterHidden) return hipErrorInvalidValue;
  const size_t part_stride = (size_t)T * k * H;
  hipLaunchKernelGGL(combine_router_kernel, dim3(T), dim3(kRouterWaves * kWave), 0, s, o, w_prev, inv, kparts,
                     part_stride, x_out, wr, H, E, k, ids, w, count, mass);
  return hipGetLastError();
}

}  // namespace pw
