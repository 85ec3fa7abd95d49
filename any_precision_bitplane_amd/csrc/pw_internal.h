// Internal interfaces between the C-ABI host layer and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pagedweight.h"

namespace pw {

constexpr int kMaxExperts = 256;
constexpr int kMinBits = 3;   // committed bitwidths with a table: 3..8
constexpr int kMaxBits = 8;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kMfmaTileM = 512;   // tokens per MFMA tile
constexpr int kMaxRouterTopK = 64; // the router's top-k kernel keeps slot j in lane j
constexpr int kMaxRouterHidden = 16384;   // a multi-layer call's router keeps one token's x in LDS

inline int mtile_bound(int E, int T, int k) {
  const int slots = T * k;
  return (E < slots ? E : slots) + (slots + kMfmaTileM - 1) / kMfmaTileM;
}

constexpr int kMgTileM = 32;      // tokens per matrix-core GEMV pass

// Prefill: the tokens of an MFMA expert past its last whole 512-token tile
// go to the matrix-core GEMV when there are at most this many.  An MFMA tile
// costs the same whatever its token count (the weight decode and the products
// of all its 512 token rows); a 32-token matrix-core GEMV tile of the same
// expert costs about a quarter of it, so up to three such tiles win.
constexpr int kMfmaTailTokens = 96;

inline int mgtile_bound(int E, int T, int k) {
  const int slots = T * k;
  return (E < slots ? E : slots) + (slots + kMgTileM - 1) / kMgTileM;
}

// Parts of the down product's K range given to separate waves when a small
// batch would otherwise leave most of the chip idle.
inline int down_kparts(int H, int I, int E, int k, int T) {
  const int slots = T * k;
  if (slots > 64 || slots <= 0) return 1;
  const int bound = E < slots ? E : slots;
  const int waves = bound * (H / 16);
  const int nsl = (I / 32 + 63) / 64;
  int kp = (2048 + waves - 1) / waves;
  if (kp > nsl) kp = nsl;
  return kp < 1 ? 1 : kp;
}

// Parts of the down product's K range for the MFMA kernels when they run
// alone (prefill): the down product has few row tiles (H / 128), so with
// few token tiles its workgroups would fill the CUs only once or twice and
// the last round would run mostly empty.  Parts double until there are
// enough (token tile, row tile, part) items for two rounds, each part keeping
// at least sixteen quads of eight plane words.  Every part writes its own o
// slice, which the combine reads back: on the Mixtral-shaped prefill (512
// items) one part takes the call 3.48 -> 3.45 ms against the two that a
// four-round target gave (down kernel 1.164 -> 1.155 ms).
constexpr int kNumCUs = 256;
inline int mfma_down_kparts(int H, int I, int E, int k, int T) {
  (void)E;
  const long long slots = (long long)T * k;
  if (slots <= 0) return 1;
  const long long items = (slots + kMfmaTileM - 1) / kMfmaTileM * ((H + 127) / 128);
  const int quads = (I / 32 + 7) / 8;
  int kp = 1;
  while (kp < 4 && items * kp < 2LL * kNumCUs && quads >= 16 * 2 * kp) kp *= 2;
  return kp;
}

// Parts of the down product's K range for the matrix-core GEMV when it runs
// alone: a 32-row chunk of the down block walks all of I, and with few token
// tiles (decode batches: about one per routed expert) there are too few
// (tile, chunk) items to keep the CUs busy.  Parts double until there are
// about 2048 items, each part keeping at least eight super-chunks of eight
// plane words; every part stages the chunk's row tables again and writes its
// own o slice, so more parts cost more than they spread (Mixtral-shaped down
// product at T = 64, 1024 (tile, chunk) items: 177 / 136 / 141 / 156 us with
// 1 / 2 / 4 / 8 parts).
inline int mgemv_down_kparts(int H, int I, int E, int k, int T) {
  const long long slots = (long long)T * k;
  if (slots <= 0) return 1;
  const long long tiles = (E < slots ? E : slots) > (slots + kMgTileM - 1) / kMgTileM
                              ? (E < slots ? E : slots)
                              : (slots + kMgTileM - 1) / kMgTileM;
  const long long items = tiles * ((H + 31) / 32);
  const int supers = (I / 32 + 7) / 8;
  int kp = 1;
  while (kp < 8 && items * kp < 2048 && supers >= 8 * 2 * kp) kp *= 2;
  return kp;
}

// Workspace layout (byte offsets from the workspace base).  The first 256
// bytes are the header: status word, active-expert count.
struct WsLayout {
  size_t status = 0;        // uint32 status bits
  size_t num_active = 4;    // int32 number of experts with at least one slot
  size_t num_mtiles = 8;    // int32 number of MFMA token tiles
  size_t num_mgtiles = 12;  // int32 number of matrix-core GEMV token tiles
  size_t counts = 0;        // int32 [E]    slots per expert
  size_t offsets = 0;       // int32 [E+1]  first sorted position per expert
  size_t active = 0;        // int32 [E]    active expert ids, ascending
  size_t perm = 0;          // int32 [T*k]  sorted position -> slot (t*k + j)
  size_t inv = 0;           // int32 [T*k]  slot -> sorted position, -1 if dropped
  size_t mtiles = 0;        // int32 [2 * mtile_bound] MFMA token tiles
  size_t mgtiles = 0;       // int32 [2 * mgtile_bound] matrix-core GEMV token tiles
  size_t h = 0;             // fp16  [T*k][I] activations between the products
  size_t o = 0;             // fp32  [kparts][T*k][H] expert outputs by slot (t*k + j), before the combine
  size_t xl = 0;            // fp16  [2][T][H] layer inputs of a multi-layer call (ping-pong)
  size_t rids = 0;          // int32 [T*k]    router expert ids (routed forward)
  size_t rw = 0;            // fp32  [T*k]    router weights (routed forward)
  size_t adesc = 0;         // ActiveDesc [E] down-product work descriptors (calls routed inside gate_up)
  size_t total = 0;
};

inline WsLayout ws_layout(int H, int I, int E, int k, int T) {
  WsLayout L;
  size_t off = kAlign;
  const size_t slots = (size_t)T * (size_t)k;
  const int kpg = down_kparts(H, I, E, k, T), kpm = mfma_down_kparts(H, I, E, k, T);
  const int kpv = mgemv_down_kparts(H, I, E, k, T);
  const int kpx = kpg > kpm ? kpg : kpm;
  const size_t kp = (size_t)(kpx > kpv ? kpx : kpv);
  L.counts = off;  off = align_up(off + sizeof(int32_t) * E, kAlign);
  L.offsets = off; off = align_up(off + sizeof(int32_t) * (E + 1), kAlign);
  L.active = off;  off = align_up(off + sizeof(int32_t) * E, kAlign);
  L.perm = off;    off = align_up(off + sizeof(int32_t) * slots, kAlign);
  L.inv = off;     off = align_up(off + sizeof(int32_t) * slots, kAlign);
  L.mtiles = off;  off = align_up(off + sizeof(int32_t) * 2 * mtile_bound(E, T, k), kAlign);
  L.mgtiles = off; off = align_up(off + sizeof(int32_t) * 2 * mgtile_bound(E, T, k), kAlign);
  L.h = off;       off = align_up(off + sizeof(uint16_t) * slots * I, kAlign);
  L.o = off;       off = align_up(off + sizeof(float) * kp * slots * H, kAlign);
  L.xl = off;      off = align_up(off + sizeof(uint16_t) * 2 * (size_t)T * H, kAlign);
  L.rids = off;    off = align_up(off + sizeof(int32_t) * slots, kAlign);
  L.rw = off;      off = align_up(off + sizeof(float) * slots, kAlign);
  L.adesc = off;   off = align_up(off + 32 * (size_t)E, kAlign);
  L.total = off;
  return L;
}

// Pointers into one workspace for one call.
// What a down-product wave needs about the a-th routed expert, in one
// 32-byte record: written by the gate_up kernel that routes a small batch, so
// the down kernel reaches its planes after one dependent load.
struct ActiveDesc {
  int32_t e, n_e, off_e, q;
  const uint32_t* planes;
  const uint16_t* lut_all;
};
static_assert(sizeof(ActiveDesc) == 32, "one record per 32 bytes");

struct Route {
  uint32_t* status;
  int32_t* num_active;
  int32_t* counts;
  int32_t* offsets;
  int32_t* active;
  int32_t* perm;
  int32_t* inv;
  int32_t* mtiles;        // (expert, first sorted position) per MFMA token tile
  int32_t* num_mtiles;
  int32_t* mgtiles;       // (expert, first token) per matrix-core GEMV token tile
  int32_t* num_mgtiles;
  ActiveDesc* adesc;      // [E] down work descriptors by active index (inline routing only)
};


struct ExpertArgs {
  int H, I, E, k, T;
  const pw_block_desc* blocks;
  const uint8_t* q;
  Route rt;
  int min_tokens;   // process experts with min_tokens <= n_e < max_tokens
  int max_tokens;
  int kparts;       // parts of the down product's K range (MFMA kernels running alone)
};

// Everything the GEMV kernels need for one call.
struct GemvLaunch {
  int H, I, E, k, T;
  const pw_block_desc* blocks;
  const uint8_t* q;
  const int32_t* ids;
  Route rt;
  int inline_route;          // T*k <= 64: no route kernel, gate_up waves route by themselves
  int min_tokens, max_tokens;
  const uint16_t* x;
  uint16_t* h;
  float* o;
  int kparts;
};

// Optional start / stop events of one kernel: the library hands them to the
// launch itself, so they carry the timestamps of that kernel's execution
// rather than of the stream around it.  Null members are not recorded.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename F, typename... Args>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t s, const KernelEvents& ev,
                                Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

// Launchers (return hipSuccess or the launch error).
// mfma_tail: an MFMA expert's tokens past its last whole 512-token tile, when
// at most this many (0: never), are listed as matrix-core GEMV tiles instead
hipError_t launch_route(const int32_t* ids, int T, int k, int E, int mfma_min_tokens, int mg_min_tokens,
                        int mg_max_tokens, int mfma_tail, const Route& rt, hipStream_t s);
hipError_t launch_gemv_gate_up(const GemvLaunch& g, hipStream_t s, const KernelEvents& ev);
hipError_t launch_gemv_down(const GemvLaunch& g, hipStream_t s, const KernelEvents& ev);
hipError_t launch_mfma_gate_up(const ExpertArgs& a, const uint16_t* x, uint16_t* h, hipStream_t s,
                               const KernelEvents& ev);
hipError_t launch_mfma_down(const ExpertArgs& a, const uint16_t* h, float* o, hipStream_t s, const KernelEvents& ev);
hipError_t launch_mgemv_gate_up(const ExpertArgs& a, const uint16_t* x, uint16_t* h, hipStream_t s,
                                const KernelEvents& ev);
hipError_t launch_mgemv_down(const ExpertArgs& a, const uint16_t* h, float* o, hipStream_t s,
                             const KernelEvents& ev);
hipError_t launch_combine(const float* o, const float* w, const int32_t* inv, int T, int k, int H, int kparts,
                          uint16_t* y, hipStream_t s);
hipError_t launch_dequant(const uint32_t* planes, const uint16_t* lut_all, int N, int K, int q, int module,
                          uint16_t* out, hipStream_t s);
hipError_t launch_pack(const uint32_t* canon, int N, int K, int nplanes, int module, uint32_t* out, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k, int32_t* ids, float* w,
                         uint32_t* count, float* mass, hipStream_t s);
// The previous layer's weighted combine (o, w_prev, inv, kparts as the
// combine kernel takes them) written to x_out, then the router on it.
hipError_t launch_combine_router(const float* o, const float* w_prev, const int32_t* inv, int kparts,
                                 uint16_t* x_out, const uint16_t* wr, int T, int H, int E, int k, int32_t* ids,
                                 float* w, uint32_t* count, float* mass, hipStream_t s);
hipError_t launch_status_clear(uint32_t* status, hipStream_t s);

// The fused layer on a caller-provided scratch area (the workspace, or the
// allocation-free entry point's static array).  `status`, if non-null,
// replaces the status word of the scratch header as the place device errors
// are raised.  Arguments are checked by the caller.
pw_status forward_on(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const int32_t* ids, const float* w,
                     const pw_block_desc* blocks, const uint8_t* q, uint16_t* y, uint8_t* scratch,
                     uint32_t* status, const pw_moe_options* opts, hipStream_t s, bool combine = true);

// Host checks shared by the forward entry points (everything but the scratch).
pw_status check_forward_args(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const int32_t* ids,
                             const float* w, const pw_block_desc* blocks, const uint8_t* q, uint16_t* y,
                             const pw_moe_options* opts);

}  // namespace pw
