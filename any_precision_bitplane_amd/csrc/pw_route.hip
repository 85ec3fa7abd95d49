// Token -> expert permutation: per-expert slot counts, exclusive offsets, the
// list of routed ("active") experts and a stable scatter of every (t, j) slot
// to an expert-sorted position.  The router's ids and weights are inputs of the
// layer ("Technical summary: PagedWeight", Core components 2 speaks of the
// routing mass as selection frequency and weight; the layer consumes both).
//
// One workgroup of 1024 threads handles any number of slots: counts with LDS
// integer atomics (order-free, so deterministic), one wave's scan over <= 256
// experts (which also lists the token tiles of the MFMA and matrix-core GEMV
// families), then the slots in chunks of 1024 in slot order.  Inside a chunk each
// wave ranks its lanes per expert with one ballot per expert-id bit, and the
// per-wave counts are scanned per expert, so a slot's position is
//   offsets[e] + #{earlier slots routed to e}
// exactly (a stable counting sort).
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ ids, int T, int k,
                                                              int E, int mfma_min_tokens, int mg_min_tokens,
                                                              int mg_max_tokens, int mfma_tail, Route rt) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kRouteWaves][kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int S = T * k;

  for (int e = tid; e < E; e += kRouteThreads) {
    cnt[e] = 0;
    base[e] = 0;
  }
  __syncthreads();

  bool bad = false;
  for (int s = tid; s < S; s += kRouteThreads) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else bad = true;
  }
  if (bad) raise_status(rt.status, PW_DEV_BAD_EXPERT_ID);
  __syncthreads();

  if (wave == 0) {
    // Lane l owns experts 4l .. 4l+3 (E <= 256).  Four exclusive scans over the
    // wave give each expert its offset, its index in the active list and the
    // first entries of its MFMA (512-token) and matrix-core GEMV (32-token)
    // tiles, so every list is written in parallel, in expert order.  An MFMA
    // expert whose tokens past its last whole 512-token tile number at most
    // mfma_tail hands them to the matrix-core GEMV (tiles from token g0 on):
    // a nearly empty MFMA tile costs as much as a full one.
    int c[4], na[4], nm[4], ng[4], g0[4];
    int sc = 0, sa = 0, sm = 0, sg = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? cnt[e] : 0;
      na[i] = c[i] > 0 ? 1 : 0;
      const bool mf = c[i] > 0 && c[i] >= mfma_min_tokens;
      const int rem = c[i] % kMfmaTileM;
      const bool tail = mf && rem > 0 && rem <= mfma_tail;
      nm[i] = mf ? (tail ? c[i] / kMfmaTileM : (c[i] + kMfmaTileM - 1) / kMfmaTileM) : 0;
      g0[i] = tail ? c[i] - rem : 0;
      ng[i] = tail ? (rem + kMgTileM - 1) / kMgTileM
                   : ((c[i] > 0 && c[i] >= mg_min_tokens && c[i] < mg_max_tokens) ? (c[i] + kMgTileM - 1) / kMgTileM
                                                                                  : 0);
      sc += c[i]; sa += na[i]; sm += nm[i]; sg += ng[i];
    }
    int xc = sc, xa = sa, xm = sm, xg = sg;   // inclusive scans
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int yc = __shfl_up(xc, d, kWave), ya = __shfl_up(xa, d, kWave);
      const int ym = __shfl_up(xm, d, kWave), yg = __shfl_up(xg, d, kWave);
      if (lane >= d) { xc += yc; xa += ya; xm += ym; xg += yg; }
    }
    int pc = xc - sc, pa = xa - sa, pm = xm - sm, pg = xg - sg;   // exclusive
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        off[e] = pc;
        if (na[i]) rt.active[pa] = e;
        for (int t = 0; t < nm[i]; ++t) {
          rt.mtiles[2 * (pm + t)] = e;
          rt.mtiles[2 * (pm + t) + 1] = t * kMfmaTileM;
        }
        for (int t = 0; t < ng[i]; ++t) {
          rt.mgtiles[2 * (pg + t)] = e;
          rt.mgtiles[2 * (pg + t) + 1] = g0[i] + t * kMgTileM;
        }
      }
      pc += c[i]; pa += na[i]; pm += nm[i]; pg += ng[i];
    }
    if (lane == kWave - 1) {
      off[E] = xc;
      rt.offsets[E] = xc;
      *rt.num_active = xa;
      *rt.num_mtiles = xm;
      *rt.num_mgtiles = xg;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    rt.counts[e] = cnt[e];
    rt.offsets[e] = off[e];
  }

  for (int c0 = 0; c0 < S; c0 += kRouteThreads) {
    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();

    const int s = c0 + tid;
    int e = -1;
    if (s < S) {
      e = ids[s];
      if (e < 0 || e >= E) e = -1;
    }
    // lanes routed to the same expert: one ballot per bit of the expert id
    // (at most 8 for E <= 256) instead of one round per distinct expert
    unsigned long long same = __ballot(e >= 0);
    for (int bit = 0; (1 << bit) < E; ++bit) {
      const unsigned long long ones = __ballot(e >= 0 && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? ones : ~ones;
    }
    int rank = 0;
    if (e >= 0) {
      rank = __popcll(same & ((1ull << lane) - 1ull));
      if (rank == 0) wcnt[wave][e] = __popcll(same);   // the expert's first lane in the wave
    }
    __syncthreads();

    for (int x = tid; x < E; x += kRouteThreads) {
      int run = base[x];
      for (int w = 0; w < kRouteWaves; ++w) {
        const int c = wcnt[w][x];
        wcnt[w][x] = run;
        run += c;
      }
      base[x] = run;
    }
    __syncthreads();

    if (s < S) {
      if (e >= 0) {
        const int pos = off[e] + wcnt[wave][e] + rank;
        rt.perm[pos] = s;
        rt.inv[s] = pos;
      } else {
        rt.inv[s] = -1;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_route(const int32_t* ids, int T, int k, int E, int mfma_min_tokens, int mg_min_tokens,
                        int mg_max_tokens, int mfma_tail, const Route& rt, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, s, ids, T, k, E, mfma_min_tokens, mg_min_tokens,
                     mg_max_tokens, mfma_tail, rt);
  return hipGetLastError();
}

__global__ void status_clear_kernel(uint32_t* status) { *status = 0u; }

hipError_t launch_status_clear(uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(1), 0, s, status);
  return hipGetLastError();
}

}  // namespace pw
