// C-ABI host layer of libpagedweight: argument checks, workspace carving and
// the launch sequence of the fused mixed-precision MoE layer
// ("Technical summary: PagedWeight", Core components 3, fused kernel).
//
// A forward is at most five launches on the caller's stream and never
// synchronizes: route, gate_up (GEMV and/or MFMA family), down (same), combine.
// The committed bitwidths are read on the device, so the launch sequence does
// not depend on them.
#include <limits.h>
#include <string.h>

#include "pw_internal.h"

using namespace pw;

namespace {

// AUTO picks one kernel family per call from the mean number of routed slots
// per routed expert (measured on the Qwen- and Mixtral-shaped layers: the
// families run one after another, so a call that mixes them pays each one's
// fill and drain): GEMV below a mean of 1.6, the matrix-core GEMV up to 64, the
// MFMA form (with its short tails on the matrix-core GEMV) above.  The upper
// edge depends on how evenly the tokens spread: with evenly routed tokens the
// matrix-core GEMV stays 10-17% faster up to a mean of about 100 (Qwen shape;
// Mixtral ties to 104), but with Zipf-routed tokens the hot experts fill MFMA
// tiles and the MFMA form wins from about 48 (Qwen shape at 68 / 85 / 96: 0.384
// / 0.479 / 0.472 ms against 0.479 / 0.563 / 0.619 with the edge at 96).
// Against the GEMV the matrix-core GEMV wins from a mean of about 1.6 with even
// routing: the GEMV is 5% faster at 1.33 on the Qwen shape and 7% at 1.5 on
// the Mixtral shape, within 2% at 1.6, and 11% (Qwen, 1.87) and 18% (Mixtral,
// 1.75) slower above; with Zipf routing the matrix-core GEMV wins throughout.
// The GEMV takes calls with m < kGemvBelowNum / kGemvBelowDen.
constexpr int kGemvBelowNum = 8, kGemvBelowDen = 5;
constexpr int kMgemvUpToMean = 64;
// With explicit thresholds in the options (either one > 0) AUTO splits the
// experts into token-count bands instead; these fill the one not given.
constexpr int kDefaultMgemvMinTokens = 1;
constexpr int kDefaultMfmaMinTokens = 256;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

pw_status check_shape(const pw_moe_shape* s, int32_t T) {
  if (!s || T < 0) return PW_ERR_INVALID_ARG;
  if (s->hidden <= 0 || s->inter <= 0 || s->num_experts <= 0 || s->top_k <= 0) return PW_ERR_INVALID_ARG;
  if (s->hidden % 32 || s->inter % 32) return PW_ERR_UNSUPPORTED_SHAPE;
  if (s->num_experts > kMaxExperts || s->top_k > s->num_experts) return PW_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)T * s->top_k > INT_MAX / 4) return PW_ERR_UNSUPPORTED_SHAPE;
  // the kernels address a block's planes (2I x H weights, 8 planes) with
  // 32-bit byte offsets, out-of-range offsets at 2^31 and up
  if ((int64_t)2 * s->inter * s->hidden > INT_MAX) return PW_ERR_UNSUPPORTED_SHAPE;
  return PW_OK;
}

pw_status hip_status(hipError_t e) { return e == hipSuccess ? PW_OK : PW_ERR_HIP; }

// Which kernel families a call runs and how the experts split between them:
// token-count bands per expert, GEMV [0, b1), matrix-core GEMV [b1, b2), MFMA
// [b2, inf).  A band whose lower end no expert can reach (an expert gets at
// most T tokens unless a token lists it twice) is not launched and the band
// below it takes its experts.
struct Plan {
  bool gemv, mgemv, mfma;
  int b1, b2;          // b2 == INT_MAX: no MFMA launch
  bool inline_route;   // <= 64 slots on the GEMV alone: the gate_up kernel routes
  int kparts;          // parts of the GEMV down product's K range
  int tail;            // MFMA experts' last <= tail tokens past whole tiles take the
                       // matrix-core GEMV (0: none); only the AUTO rule's prefill sets it
};

pw_status make_plan(const pw_moe_shape* shape, int32_t T, const pw_moe_options* opts, Plan& pl) {
  const int path = opts ? opts->path : PW_PATH_AUTO;
  if (path != PW_PATH_AUTO && path != PW_PATH_GEMV && path != PW_PATH_MFMA && path != PW_PATH_MGEMV)
    return PW_ERR_INVALID_ARG;
  const int H = shape->hidden, I = shape->inter, E = shape->num_experts, k = shape->top_k;
  const int max_slots = T * k;
  const int routed_bound = E < max_slots ? E : max_slots;   // routed experts, at most
  // the matrix-core GEMV addresses activations with 32-bit offsets
  const bool mg_ok = 2LL * (long long)T * (H > k * I ? H : k * I) < 0x80000000LL;
  if (path == PW_PATH_MGEMV && !mg_ok) return PW_ERR_UNSUPPORTED_SHAPE;
  const bool explicit_bands = opts && (opts->mfma_min_tokens > 0 || opts->mgemv_min_tokens > 0);
  int b1, b2;
  if (path == PW_PATH_GEMV) b1 = b2 = INT_MAX;
  else if (path == PW_PATH_MFMA) b1 = b2 = 0;
  else if (path == PW_PATH_MGEMV) { b1 = 0; b2 = INT_MAX; }
  else if (explicit_bands) {
    b2 = opts->mfma_min_tokens > 0 ? opts->mfma_min_tokens : kDefaultMfmaMinTokens;
    b1 = opts->mgemv_min_tokens > 0 ? opts->mgemv_min_tokens : kDefaultMgemvMinTokens;
    if (b1 > b2) b1 = b2;
  } else if ((long long)kGemvBelowDen * max_slots < (long long)kGemvBelowNum * routed_bound) {
    b1 = b2 = INT_MAX;                        // decode: GEMV alone
  } else if ((long long)max_slots <= (long long)kMgemvUpToMean * routed_bound && mg_ok) {
    b1 = 0; b2 = INT_MAX;                     // moderate batches: matrix-core GEMV alone
  } else {
    b1 = b2 = 0;                              // prefill: MFMA alone
  }
  pl.mfma = b2 <= T;
  if (!pl.mfma) b2 = INT_MAX;
  // with explicit bands, calls averaging fewer than 1.6 slots per
  // routed expert still stay on the GEMV kernels alone
  const bool mg_worth =
      !explicit_bands || (long long)kGemvBelowDen * max_slots >= (long long)kGemvBelowNum * routed_bound;
  pl.mgemv = b1 < b2 && b1 <= T && mg_ok && (path == PW_PATH_MGEMV || mg_worth);
  if (!pl.mgemv) b1 = b2;
  pl.gemv = b1 > 1;     // a routed expert has at least one token
  pl.b1 = b1;
  pl.b2 = b2;
  pl.inline_route = max_slots <= 64 && !pl.mfma && !pl.mgemv;
  pl.tail = (path == PW_PATH_AUTO && !explicit_bands && pl.mfma && !pl.mgemv && !pl.gemv && mg_ok) ? kMfmaTailTokens : 0;
  // the families write one K part of o each, except one family running alone
  // (MFMA with its tails counts as one: the matrix-core GEMV then splits the
  // K range as the MFMA kernels do), which then splits the down product's K range
  const int nfam = (int)pl.mfma + (int)pl.mgemv + (int)pl.gemv;
  if (nfam != 1) pl.kparts = 1;
  else if (pl.mfma) pl.kparts = mfma_down_kparts(H, I, E, k, T);
  else if (pl.mgemv) pl.kparts = mgemv_down_kparts(H, I, E, k, T);
  else pl.kparts = down_kparts(H, I, E, k, T);
  return PW_OK;
}

}  // namespace

namespace pw {

pw_status check_forward_args(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const int32_t* ids,
                             const float* w, const pw_block_desc* blocks, const uint8_t* q, uint16_t* y,
                             const pw_moe_options* opts) {
  pw_status st = check_shape(shape, T);
  if (st != PW_OK) return st;
  if (T == 0) return PW_OK;
  if (!x || !ids || !w || !blocks || !q || !y) return PW_ERR_INVALID_ARG;
  const int path = opts ? opts->path : PW_PATH_AUTO;
  if (path != PW_PATH_AUTO && path != PW_PATH_GEMV && path != PW_PATH_MFMA && path != PW_PATH_MGEMV)
    return PW_ERR_INVALID_ARG;
  if (opts && opts->event_mode != PW_EVENTS_STAGES && opts->event_mode != PW_EVENTS_KERNELS)
    return PW_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ids, 4) || !aligned(w, 4) || !aligned(blocks, 8))
    return PW_ERR_ALIGNMENT;
  Plan pl;
  return make_plan(shape, T, opts, pl);
}

pw_status forward_on(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const int32_t* ids, const float* w,
                     const pw_block_desc* blocks, const uint8_t* q, uint16_t* y, uint8_t* ws, uint32_t* status,
                     const pw_moe_options* opts, hipStream_t s, bool combine) {
  const int H = shape->hidden, I = shape->inter, E = shape->num_experts, k = shape->top_k;
  const WsLayout L = ws_layout(H, I, E, k, T);
  Plan pl;
  pw_status st = make_plan(shape, T, opts, pl);
  if (st != PW_OK) return st;
  const bool use_gemv = pl.gemv, use_mfma = pl.mfma;
  const bool use_mg = pl.mgemv || pl.tail > 0;   // its band, or only the MFMA experts' tails
  const int b1 = pl.b1, b2 = pl.b2, thresh = pl.b2;

  Route rt;
  rt.status = status ? status : reinterpret_cast<uint32_t*>(ws + L.status);
  rt.num_active = reinterpret_cast<int32_t*>(ws + L.num_active);
  rt.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  rt.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  rt.active = reinterpret_cast<int32_t*>(ws + L.active);
  rt.perm = reinterpret_cast<int32_t*>(ws + L.perm);
  rt.inv = reinterpret_cast<int32_t*>(ws + L.inv);
  rt.mtiles = reinterpret_cast<int32_t*>(ws + L.mtiles);
  rt.num_mtiles = reinterpret_cast<int32_t*>(ws + L.num_mtiles);
  rt.mgtiles = reinterpret_cast<int32_t*>(ws + L.mgtiles);
  rt.num_mgtiles = reinterpret_cast<int32_t*>(ws + L.num_mgtiles);
  rt.adesc = reinterpret_cast<ActiveDesc*>(ws + L.adesc);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  float* o = reinterpret_cast<float*>(ws + L.o);

  const bool inline_route = pl.inline_route;
  ExpertArgs mfma{H, I, E, k, T, blocks, q, rt, thresh == 0 ? 1 : thresh, INT_MAX, pl.mfma ? pl.kparts : 1};
  ExpertArgs mg{H, I, E, k, T, blocks, q, rt, pl.mgemv ? (b1 == 0 ? 1 : b1) : 1, pl.mgemv ? b2 : INT_MAX,
                use_mg ? pl.kparts : 1};
  GemvLaunch g{};
  g.H = H; g.I = I; g.E = E; g.k = k; g.T = T;
  g.blocks = blocks; g.q = q; g.ids = ids; g.rt = rt;
  g.inline_route = inline_route ? 1 : 0;
  g.min_tokens = 0;
  g.max_tokens = b1;
  g.x = x; g.h = h; g.o = o;
  // the other families write one K part of o; the GEMV splits K only when it runs alone
  g.kparts = pl.kparts;

  // Events: at stage boundaries on the stream, or carried by the product
  // kernels themselves (start on the first kernel of a product, stop on its last).
  void* const* ev = (opts && opts->stage_events[0]) ? opts->stage_events : nullptr;
  const bool kernel_ev = ev && opts->event_mode == PW_EVENTS_KERNELS;
  auto mark = [&](int i) -> hipError_t {
    return (ev && !kernel_ev) ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess;
  };
  // kernel events of one product: `first`/`last` say whether this launch opens / closes the product
  auto kev = [&](int product, bool first, bool last) {
    KernelEvents r;
    if (kernel_ev) {
      if (first) r.start = (hipEvent_t)ev[2 * product];
      if (last) r.stop = (hipEvent_t)ev[2 * product + 1];
    }
    return r;
  };
  const int nfam = (int)use_gemv + (int)use_mg + (int)use_mfma;

  hipError_t e = mark(PW_STAGE_ROUTE);
  if (e == hipSuccess && !inline_route)
    e = launch_route(ids, T, k, E, use_mfma ? (thresh == 0 ? 1 : thresh) : INT_MAX,
                     pl.mgemv ? (b1 == 0 ? 1 : b1) : INT_MAX, pl.mgemv ? b2 : INT_MAX, pl.tail, rt, s);
  for (int product = 0; product < 2 && e == hipSuccess; ++product) {
    e = mark(product == 0 ? PW_STAGE_GATE_UP : PW_STAGE_DOWN);
    int done = 0;
    if (e == hipSuccess && use_gemv) {
      const KernelEvents kv = kev(product, done == 0, done + 1 == nfam);
      e = product == 0 ? launch_gemv_gate_up(g, s, kv) : launch_gemv_down(g, s, kv);
      ++done;
    }
    if (e == hipSuccess && use_mg) {
      const KernelEvents kv = kev(product, done == 0, done + 1 == nfam);
      e = product == 0 ? launch_mgemv_gate_up(mg, x, h, s, kv) : launch_mgemv_down(mg, h, o, s, kv);
      ++done;
    }
    if (e == hipSuccess && use_mfma) {
      const KernelEvents kv = kev(product, done == 0, done + 1 == nfam);
      e = product == 0 ? launch_mfma_gate_up(mfma, x, h, s, kv) : launch_mfma_down(mfma, h, o, s, kv);
      ++done;
    }
  }
  if (e == hipSuccess) e = mark(PW_STAGE_COMBINE);
  if (e == hipSuccess && combine) e = launch_combine(o, w, rt.inv, T, k, H, g.kparts, y, s);
  if (e == hipSuccess) e = mark(PW_NUM_STAGES);
  if (e == hipErrorNotSupported) return PW_ERR_UNSUPPORTED;
  return hip_status(e);
}

}  // namespace pw

extern "C" {

int32_t pw_abi_version(void) { return PW_ABI_VERSION; }

const char* pw_status_str(pw_status s) {
  switch (s) {
    case PW_OK: return "ok";
    case PW_ERR_INVALID_ARG: return "invalid argument";
    case PW_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case PW_ERR_BITWIDTH: return "bitwidth outside 3..8";
    case PW_ERR_WORKSPACE: return "workspace too small";
    case PW_ERR_ALIGNMENT: return "misaligned pointer";
    case PW_ERR_HIP: return "HIP runtime error";
    case PW_ERR_UNSUPPORTED: return "unsupported option";
    case PW_ERR_OUT_OF_MEMORY: return "arena has no free range large enough";
    default: return "unknown status";
  }
}

size_t pw_plane_words(int32_t N, int32_t K) {
  if (N <= 0 || K <= 0 || K % 32) return 0;
  return (size_t)8 * (size_t)N * (size_t)(K / 32);
}

size_t pw_lut_elems(int32_t N) { return N > 0 ? (size_t)504 * (size_t)N : 0; }

size_t pw_lut_offset(int32_t N, int32_t b) {
  if (N <= 0 || b < kMinBits || b > kMaxBits) return 0;
  return (size_t)N * (size_t)((1 << b) - 8);
}

pw_status pw_check_shape(const pw_moe_shape* shape, int32_t T) { return check_shape(shape, T); }

size_t pw_workspace_bytes(const pw_moe_shape* s, int32_t T_max) {
  if (check_shape(s, T_max) != PW_OK) return 0;
  return ws_layout(s->hidden, s->inter, s->num_experts, s->top_k, T_max).total;
}

pw_status pw_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < kAlign) return PW_ERR_INVALID_ARG;
  if (!aligned(workspace, kAlign)) return PW_ERR_ALIGNMENT;
  return hip_status(launch_fill_zero(workspace, workspace_bytes, (hipStream_t)stream));
}

pw_status pw_moe_forward(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const int32_t* ids,
                         const float* w, const pw_block_desc* blocks, const uint8_t* q, uint16_t* y,
                         void* workspace, size_t workspace_bytes, const pw_moe_options* opts, void* stream) {
  pw_status st = check_forward_args(shape, T, x, ids, w, blocks, q, y, opts);
  if (st != PW_OK || T == 0) return st;
  if (!workspace) return PW_ERR_INVALID_ARG;
  if (!aligned(workspace, kAlign)) return PW_ERR_ALIGNMENT;
  const WsLayout L = ws_layout(shape->hidden, shape->inter, shape->num_experts, shape->top_k, T);
  if (workspace_bytes < L.total) return PW_ERR_WORKSPACE;
  return forward_on(shape, T, x, ids, w, blocks, q, y, reinterpret_cast<uint8_t*>(workspace), nullptr, opts,
                    (hipStream_t)stream);
}

pw_status pw_router_topk(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const uint16_t* router_w,
                         int32_t* ids, float* w, uint32_t* stat_count, float* stat_mass, void* workspace,
                         size_t workspace_bytes, void* stream) {
  pw_status st = check_shape(shape, T);
  if (st != PW_OK) return st;
  if (shape->top_k > kMaxRouterTopK) return PW_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return PW_OK;
  if (!x || !router_w || !ids || !w || !workspace) return PW_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(ids, 4) || !aligned(w, 4) ||
      !aligned(stat_count, 4) || !aligned(stat_mass, 4) || !aligned(workspace, kAlign))
    return PW_ERR_ALIGNMENT;
  const WsLayout L = ws_layout(shape->hidden, shape->inter, shape->num_experts, shape->top_k, T);
  if (workspace_bytes < L.total) return PW_ERR_WORKSPACE;
  return hip_status(launch_router(x, router_w, T, shape->hidden, shape->num_experts, shape->top_k, ids, w,
                                  stat_count, stat_mass, (hipStream_t)stream));
}

pw_status pw_moe_path_info(const pw_moe_shape* shape, int32_t T, const pw_moe_options* opts, pw_path_info* info) {
  if (!info) return PW_ERR_INVALID_ARG;
  pw_status st = check_shape(shape, T);
  if (st != PW_OK) return st;
  memset(info, 0, sizeof(*info));
  if (T == 0) return PW_OK;
  Plan pl;
  st = make_plan(shape, T, opts, pl);
  if (st != PW_OK) return st;
  info->gemv = pl.gemv ? 1 : 0;
  info->mgemv = (pl.mgemv || pl.tail > 0) ? 1 : 0;
  info->mfma = pl.mfma ? 1 : 0;
  info->mgemv_from = pl.mgemv ? (pl.b1 == 0 ? 1 : pl.b1) : 0;
  info->mfma_from = pl.mfma ? (pl.b2 == 0 ? 1 : pl.b2) : 0;
  info->inline_route = pl.inline_route ? 1 : 0;
  info->down_kparts = pl.kparts;
  info->mfma_tail = pl.tail;
  const int families = (int)pl.gemv + (int)(pl.mgemv || pl.tail > 0) + (int)pl.mfma;
  info->launches = (pl.inline_route ? 0 : 1) + 2 * families + 1;
  return PW_OK;
}

pw_status pw_moe_forward_routed(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const uint16_t* router_w,
                                const pw_block_desc* blocks, const uint8_t* q, uint16_t* y, uint32_t* stat_count,
                                float* stat_mass, void* workspace, size_t workspace_bytes, const pw_moe_options* opts,
                                void* stream) {
  pw_status st = check_shape(shape, T);
  if (st != PW_OK) return st;
  if (T == 0) return PW_OK;
  if (!workspace) return PW_ERR_INVALID_ARG;
  if (!aligned(workspace, kAlign)) return PW_ERR_ALIGNMENT;
  const WsLayout L = ws_layout(shape->hidden, shape->inter, shape->num_experts, shape->top_k, T);
  if (workspace_bytes < L.total) return PW_ERR_WORKSPACE;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.rids);
  float* w = reinterpret_cast<float*>(ws + L.rw);
  // argument checks of the forward before anything is enqueued
  if (!blocks || !q || !y) return PW_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(blocks, 8)) return PW_ERR_ALIGNMENT;
  Plan pl;   // a path the forward would refuse is refused before the router runs
  st = make_plan(shape, T, opts, pl);
  if (st != PW_OK) return st;
  st = pw_router_topk(shape, T, x, router_w, ids, w, stat_count, stat_mass, workspace, workspace_bytes, stream);
  if (st != PW_OK) return st;
  return pw_moe_forward(shape, T, x, ids, w, blocks, q, y, workspace, workspace_bytes, opts, stream);
}

size_t pw_planes_bytes(int32_t N, int32_t K, int32_t nplanes) {
  if (N <= 0 || K <= 0 || K % 32 || N % 16 || nplanes < 1 || nplanes > kMaxBits) return 0;
  return (size_t)nplanes * (size_t)N * (size_t)(K / 32) * 4u;
}

pw_status pw_pack_planes(const uint32_t* canon, int32_t N, int32_t K, int32_t nplanes, int32_t module,
                         uint32_t* dev_layout, void* stream) {
  if (!canon || !dev_layout || N <= 0 || K <= 0 || nplanes < 1 || nplanes > kMaxBits) return PW_ERR_INVALID_ARG;
  if (module != 0 && module != 1) return PW_ERR_INVALID_ARG;
  if (K % 32 || N % 16) return PW_ERR_UNSUPPORTED_SHAPE;
  if ((size_t)N * (size_t)(K / 32) * (size_t)nplanes > 0xFFFFFFFFull) return PW_ERR_UNSUPPORTED_SHAPE;
  if (!aligned(canon, 4) || !aligned(dev_layout, 16)) return PW_ERR_ALIGNMENT;
  if ((const void*)canon == (const void*)dev_layout) return PW_ERR_INVALID_ARG;   // not in place
  return hip_status(launch_pack(canon, N, K, nplanes, module, dev_layout, (hipStream_t)stream));
}

pw_status pw_moe_forward_layers(const pw_moe_shape* shape, int32_t L, int32_t T, const uint16_t* x,
                                const uint16_t* const* router_w, const pw_block_desc* const* blocks,
                                const uint8_t* const* q, uint16_t* y, uint32_t* stat_count, float* stat_mass,
                                void* workspace, size_t workspace_bytes, const pw_moe_options* opts, void* stream) {
  pw_status st = check_shape(shape, T);
  if (st != PW_OK) return st;
  if (L < 1 || !router_w || !blocks || !q) return PW_ERR_INVALID_ARG;
  if (shape->top_k > kMaxRouterTopK || shape->hidden > kMaxRouterHidden) return PW_ERR_UNSUPPORTED_SHAPE;
  if (opts && opts->stage_events[0]) return PW_ERR_UNSUPPORTED;   // events time one layer
  for (int l = 0; l < L; ++l) {
    if (!router_w[l] || !blocks[l] || !q[l]) return PW_ERR_INVALID_ARG;
    if (!aligned(router_w[l], 16) || !aligned(blocks[l], 8)) return PW_ERR_ALIGNMENT;
  }
  if (!aligned(stat_count, 4) || !aligned(stat_mass, 4)) return PW_ERR_ALIGNMENT;
  // the forward's checks, with stand-ins for the ids / weights the routers write
  st = check_forward_args(shape, T, x, reinterpret_cast<const int32_t*>(workspace),
                          reinterpret_cast<const float*>(workspace), blocks[0], q[0], y, opts);
  if (st != PW_OK || T == 0) return st;
  if (!workspace) return PW_ERR_INVALID_ARG;
  if (!aligned(workspace, kAlign)) return PW_ERR_ALIGNMENT;
  const int H = shape->hidden, I = shape->inter, E = shape->num_experts, k = shape->top_k;
  const WsLayout W = ws_layout(H, I, E, k, T);
  if (workspace_bytes < W.total) return PW_ERR_WORKSPACE;
  Plan pl;
  st = make_plan(shape, T, opts, pl);
  if (st != PW_OK) return st;

  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + W.rids);
  float* w = reinterpret_cast<float*>(ws + W.rw);
  const float* o = reinterpret_cast<const float*>(ws + W.o);
  const int32_t* inv = reinterpret_cast<const int32_t*>(ws + W.inv);
  uint16_t* xl[2] = {reinterpret_cast<uint16_t*>(ws + W.xl), reinterpret_cast<uint16_t*>(ws + W.xl) + (size_t)T * H};
  hipStream_t s = (hipStream_t)stream;
  auto cnt = [&](int l) { return stat_count ? stat_count + (size_t)l * E : nullptr; };
  auto mss = [&](int l) { return stat_mass ? stat_mass + (size_t)l * E : nullptr; };

  hipError_t e = launch_router(x, router_w[0], T, H, E, k, ids, w, cnt(0), mss(0), s);
  if (e != hipSuccess) return PW_ERR_HIP;
  st = forward_on(shape, T, x, ids, w, blocks[0], q[0], y, ws, nullptr, opts, s, L == 1);
  for (int l = 1; l < L && st == PW_OK; ++l) {
    uint16_t* xin = xl[(l - 1) & 1];
    e = launch_combine_router(o, w, inv, pl.kparts, xin, router_w[l], T, H, E, k, ids, w, cnt(l), mss(l), s);
    if (e != hipSuccess) return PW_ERR_HIP;
    st = forward_on(shape, T, xin, ids, w, blocks[l], q[l], y, ws, nullptr, opts, s, l == L - 1);
  }
  return st;
}

pw_status pw_dequant_block(const uint32_t* planes, const uint16_t* lut_all, int32_t N, int32_t K, int32_t q,
                           int32_t module, uint16_t* w_out, void* stream) {
  if (!planes || !lut_all || !w_out || N <= 0 || K <= 0) return PW_ERR_INVALID_ARG;
  if (module != 0 && module != 1) return PW_ERR_INVALID_ARG;
  if (K % 32 || N % 16) return PW_ERR_UNSUPPORTED_SHAPE;
  if (q < kMinBits || q > kMaxBits) return PW_ERR_BITWIDTH;
  if (!aligned(planes, 4) || !aligned(lut_all, 16) || !aligned(w_out, 16)) return PW_ERR_ALIGNMENT;
  return hip_status(launch_dequant(planes, lut_all, N, K, q, module, w_out, (hipStream_t)stream));
}

pw_status pw_get_device_status(void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return PW_ERR_INVALID_ARG;
  if (!aligned(workspace, kAlign)) return PW_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  uint32_t v = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return PW_ERR_HIP;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return PW_ERR_HIP;
  if (launch_status_clear(reinterpret_cast<uint32_t*>(workspace), s) != hipSuccess) return PW_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PW_ERR_HIP;
  *flags = v;
  return PW_OK;
}

}  // extern "C"
