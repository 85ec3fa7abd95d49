// Bit-plane / lookup-table GEMV kernels for the expert products when an
// expert has few tokens (decode).  "Technical summary: PagedWeight", Core
// components 3 (fused mixed-precision kernel): the kernel reads the planes and
// the tables directly and runs every block at its own committed bitwidth q,
// read from the device page table, so a commit never changes a launch argument.
//
// Work decomposition.  A workgroup is one wave.  The grid is about as many
// waves as stay resident together; once a wave knows how many experts are
// routed, the grid splits evenly over the (expert, K part) segments and each
// wave takes an even share of its segment's rows, at most one chunk (8 gate_up
// row pairs with their up rows, or 16 down rows), so the waves carry about the
// same work however many experts are routed.  The down product of a small
// batch also splits K.  A wave's 64 lanes split a row's K/32 plane words
// (lane = word column, slices of 64 words), so
//   * each plane load is one 256-byte coalesced wave access and only planes
//     0..q-1 are read (buffer loads; the plane offset is a scalar operand);
//   * a lane's 32 activations per token stay in registers for a whole slice;
//   * all lanes look up the same row's table, which keeps the LDS gather free
//     of bank conflicts up to 64 entries; the row tables sit at 256-byte
//     strides, so an entry's address is one byte permute of the table base
//     and the code field, and the lookups go out in batches;
//   * row groups are double-buffered: the planes of the next group are in
//     flight while the current one is decoded;
//   * at q = 3 the 8-entry tables are expanded in LDS into 64-entry pair
//     tables (same 256 bytes), so one lookup gives two packed weights.
// gate_up chunks hold 8 gate rows and the matching 8 up rows (i and I + i), so
// SwiGLU runs in the epilogue and h = SiLU(gate) * up leaves as fp16.
//
// Batches of at most 64 routed slots skip the separate route step: every
// gate_up wave finds its expert and token slots with ballots over the slot
// ids, the first wave publishes the routing (counts, offsets, active list,
// slot order) for the down and combine kernels that follow on the stream, and
// the last wave one work descriptor per routed expert for the down kernel.
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

constexpr int kChunkRows = 16;
constexpr int kWaitVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0); expcnt and lgkmcnt not waited on
constexpr int kMaxTabBytes = (1 << kMaxBits) * 2;          // 512 B per row table

struct GemvArgs {
  int H, I, E, k, T;
  const pw_block_desc* blocks;
  const uint8_t* q;
  const int32_t* ids;       // router ids [T*k]          (inline routing)
  Route rt;                 // route-kernel results      (routed mode)
  int inline_route;         // 1: T*k <= 64 and every wave routes by itself
  int min_tokens, max_tokens;
  const uint16_t* act;      // gate_up: x [T][H];  down: h [slots][I]
  uint16_t* hout;           // gate_up: h [slots][I]
  float* oout;              // down: o [kparts][slots][H], rows by slot t*k + j
  int kparts;               // parts of the K range (down)
  int desc_mode;            // down after inline routing: work descriptors, fixed split
};

// ---------------------------------------------------------------------------
// Lane helpers
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside 8-lane halves
constexpr int kDppRor8 = 0x128;         // lane i <- (i+8) mod 16 inside 16-lane rows

// a in the lower 32 lanes, b in the upper: returns a + a' (lower) / b + b'
// (upper), where ' is the partner lane l ^ 32.  v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; the
// instruction is written out because the compiler builtin returns the second
// operand's new value incorrectly.  The compiler's hazard tracking does not
// look inside inline assembly, so the pads are written out: a dot-product
// result read by another VALU op needs three wait states (the accumulators
// arrive here straight from v_dot2), an ordinary VALU result two; s_nop 3
// gives four.  The trailing pad covers the permlane result feeding a VALU op.
__device__ __forceinline__ float swap32_add(float a, float b) {
  asm("s_nop 3\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}
// Same across 16-lane rows (odd rows of the first operand <-> even rows of the
// second): lanes with bit 4 clear keep a's pair sum, set keep b's.
__device__ __forceinline__ float swap16_add(float a, float b) {
  asm("s_nop 3\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}

// Split step inside 16-lane rows: lanes with (lane & bit) clear keep value
// a's pair sum, the others b's; the partner lane comes from a DPP pattern that
// pairs each lane with one lane of the opposite half.
template <int CTRL>
__device__ __forceinline__ float split_add(float a, float b, bool upper) {
  const float mine = upper ? b : a;
  const float give = upper ? a : b;
  return mine + dpp_f<CTRL>(give);
}

// Reduce M per-lane values (M = 1..16, power of two) over the wave.  Afterwards
// the total of value i sits in every lane l with l >> (6 - log2 M) == i.
template <int M>
__device__ __forceinline__ float multi_reduce(float (&v)[M]) {
  const int lane = threadIdx.x;
  float a[M > 1 ? M / 2 : 1];
  if constexpr (M >= 2) {
#pragma unroll
    for (int i = 0; i < M / 2; ++i) a[i] = swap32_add(v[i], v[i + M / 2]);
  } else {
    a[0] = swap32_add(v[0], v[0]);
  }
  constexpr int M1 = M > 1 ? M / 2 : 1;
  float b[M1 > 1 ? M1 / 2 : 1];
  if constexpr (M1 >= 2) {
#pragma unroll
    for (int i = 0; i < M1 / 2; ++i) b[i] = swap16_add(a[i], a[i + M1 / 2]);
  } else {
    b[0] = swap16_add(a[0], a[0]);
  }
  constexpr int M2 = M1 > 1 ? M1 / 2 : 1;
  float c[M2 > 1 ? M2 / 2 : 1];
  if constexpr (M2 >= 2) {
#pragma unroll
    for (int i = 0; i < M2 / 2; ++i) c[i] = split_add<kDppRor8>(b[i], b[i + M2 / 2], (lane & 8) != 0);
  } else {
    c[0] = b[0] + dpp_f<kDppRor8>(b[0]);
  }
  constexpr int M3 = M2 > 1 ? M2 / 2 : 1;
  float d;
  if constexpr (M3 >= 2) {
    static_assert(M3 == 2, "at most 16 values");
    d = split_add<kDppHalfMirror>(c[0], c[1], (lane & 4) != 0);
  } else {
    d = c[0] + dpp_f<kDppHalfMirror>(c[0]);
  }
  d += dpp_f<kDppXor2>(d);
  d += dpp_f<kDppXor1>(d);
  return d;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Exclusive prefix sum over the wave with DPP: shifts inside 16-lane rows,
// then the row totals carried by row_bcast:15 / row_bcast:31.
__device__ __forceinline__ int wave_excl_scan(int v) {
  int s = v;
  s += dpp_i<0x111, 0xF>(s);   // row_shr:1
  s += dpp_i<0x112, 0xF>(s);   // row_shr:2
  s += dpp_i<0x114, 0xF>(s);   // row_shr:4
  s += dpp_i<0x118, 0xF>(s);   // row_shr:8
  s += dpp_i<0x142, 0xA>(s);   // row_bcast:15 into rows 1 and 3
  s += dpp_i<0x143, 0xC>(s);   // row_bcast:31 into rows 2 and 3
  return s - v;
}

// ---------------------------------------------------------------------------
// Table lookups of one row
//
// The GEMV kernels keep each row table at a 256-byte (q <= 7) or 512-byte
// (q = 8) stride in LDS.  For q <= 7 the field byte is 2*code, so an entry's
// address is the table base with its low byte replaced by the field: one
// v_perm_b32.  For q = 8 the field is the code and the address is
// base + 2*code.
// ---------------------------------------------------------------------------
template <int Q>
__device__ __forceinline__ uint32_t row_entry(const uint32_t (&R)[8], uint32_t base, int j) {
  return tab_entry<Q>(R, base, j);
}

// acc[t] += sum_j W[j] * x[t][j] over the row's 32 weights.  The 32 lookups
// go out in batches of eight, two batches ahead of the arithmetic that
// consumes them, so the wave waits on LDS about once per batch.
template <int Q, int NT>
__device__ __forceinline__ void row_dot(const uint32_t (&R)[8], uint32_t base, const half2_t (&xr)[NT][16],
                                        float* acc) {
  constexpr int kBatch = 8;
  constexpr int kAddrOps = Q == 8 ? 2 : 1;
  constexpr int kUseOps = (kBatch / 2) * (1 + NT);
  uint32_t v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = lds_u16_at(row_entry<Q>(R, base, j));
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const half2_t w2 = __builtin_bit_cast(half2_t, v[2 * p] | (v[2 * p + 1] << 16));
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_fdot2(w2, xr[t][p], acc[t], false);
  }
  constexpr int kValu = 0x002, kDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kValu, kBatch * kAddrOps, 0);
  __builtin_amdgcn_sched_group_barrier(kDsRead, kBatch, 0);
  __builtin_amdgcn_sched_group_barrier(kValu, kBatch * kAddrOps, 0);
  __builtin_amdgcn_sched_group_barrier(kDsRead, kBatch, 0);
#pragma unroll
  for (int i = 2; i < 32 / kBatch; ++i) {
    __builtin_amdgcn_sched_group_barrier(kValu, kUseOps, 0);
    __builtin_amdgcn_sched_group_barrier(kValu, kBatch * kAddrOps, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, kBatch, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kValu, 2 * kUseOps, 0);
}

// ---------------------------------------------------------------------------
// 3-bit blocks: pair tables
//
// At q = 3 a row's table has 8 entries, so a table of all 64 entry pairs
// (fp16 LUT[a] in the low half, LUT[b] in the high half) takes the same 256
// bytes of LDS; one lookup then yields two weights already packed for v_dot2,
// which halves the address, lookup and packing work per weight.  The bit
// transpose below produces, for the pair of weights (8k + c, 8k + c + 4), the
// byte (code_a << 5) | (code_b << 2) = 4 * pair index in byte k of R[c]
// (c, k = 0..3): the planes enter the 8 x 8 transpose of each byte lane as
// rows 7, 6, 5 (weights 0..3 of the lane, code bits from the most significant
// plane down) and, shifted down by four, rows 4, 3, 2 (weights 4..7); only the
// output rows 0..3 are formed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void planes_to_pairs3(const uint32_t (&P)[3], uint32_t (&R)[4]) {
  constexpr uint32_t H4 = 0xF0F0F0F0u, H2 = 0xCCCCCCCCu, H1 = 0xAAAAAAAAu;
  // level 4, output rows 0..3 only (input rows 0, 1 are zero)
  R[0] = P[0] & H4;
  R[1] = (P[2] << 4) & H4;
  R[2] = bfi(H4, P[1] << 4, P[2] >> 4);
  R[3] = bfi(H4, P[0] << 4, P[1] >> 4);
  // levels 2 and 1 inside rows 0..3
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint32_t a = R[r], b = R[r + 2];
    R[r] = bfi(H2, b << 2, a);
    R[r + 2] = bfi(H2, b, a >> 2);
  }
#pragma unroll
  for (int r = 0; r < 4; r += 2) {
    const uint32_t a = R[r], b = R[r + 1];
    R[r] = bfi(H1, b << 1, a);
    R[r + 1] = bfi(H1, b, a >> 1);
  }
}

typedef const __attribute__((address_space(3))) uint32_t* lds_u32_cptr;
typedef __attribute__((address_space(3))) uint32_t* lds_u32_ptr;

// acc[t] += sum over the 16 pairs of the row's 32 weights; pair (c, k) meets the
// activation pair xr[t][4c + k] = (x[8k + c], x[8k + c + 4]).
template <int NT>
__device__ __forceinline__ void row_dot_pairs3(const uint32_t (&R)[4], uint32_t base, const half2_t (&xr)[NT][16],
                                               float* acc) {
  uint32_t v[16];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[4 * c + k] = *(lds_u32_cptr)(size_t)__builtin_amdgcn_perm(base, R[c], 0x07060500u | (uint32_t)k);
#pragma unroll
  for (int p = 0; p < 16; ++p)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v[p]), xr[t][p], acc[t], false);
}

// In place: every 8-entry row table of the chunk (at the start of its 256-byte
// slot) becomes its 64-entry pair table.
__device__ __forceinline__ void build_pair_tables3(uint32_t tab_base) {
  const int lane = threadIdx.x;
  const uint32_t ia = 2u * (uint32_t)(lane >> 3), ib = 2u * (uint32_t)(lane & 7);
  uint32_t pr[kChunkRows];
#pragma unroll
  for (int r = 0; r < kChunkRows; ++r) {
    const uint32_t row = tab_base + 256u * (uint32_t)r;
    pr[r] = lds_u16_at(row + ia) | (lds_u16_at(row + ib) << 16);
  }
#pragma unroll
  for (int r = 0; r < kChunkRows; ++r) *(lds_u32_ptr)(size_t)(tab_base + 256u * (uint32_t)r + 4u * (uint32_t)lane) = pr[r];
}

// ---------------------------------------------------------------------------
// Which expert and which token slots a wave works on
// ---------------------------------------------------------------------------
struct Slots {
  int e, n_e, off_e, num_active;
  int qd;                    // bitwidth of the block when `pre` (down: from the work descriptor)
  bool pre;                  // qd and d already hold the block's page-table entry
  unsigned long long mask;   // inline routing: slots routed to e (bit = slot)
  pw_block_desc d;           // page-table entry of this product's block of e
};

struct RouteLds {
  int cnt[kMaxExperts];
  int off[kMaxExperts];
  int e_sel;
};

// Write the routing one wave computed in LDS to the workspace, in the same
// form the route kernel produces (stable expert-sorted slot order).
__device__ __forceinline__ void publish_route(const GemvArgs& A, RouteLds& L, int id, bool valid, const int (&c)[4], int nzr,
                              int run) {
  const int lane = threadIdx.x;
  const int S = A.T * A.k;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = 4 * lane + i;
    if (ex < A.E) {
      A.rt.counts[ex] = c[i];
      A.rt.offsets[ex] = run;
      if (c[i] > 0) A.rt.active[nzr++] = ex;
    }
    run += c[i];
  }
  if (lane == kWave - 1) {
    A.rt.offsets[A.E] = run;
    *A.rt.num_active = nzr;
  }
  int rank = 0;
  unsigned long long todo = __ballot(valid);
  while (todo) {
    const int leader = __ffsll(todo) - 1;
    const int le = __shfl(id, leader, kWave);
    const unsigned long long m = __ballot(valid && id == le);
    if (valid && id == le) rank = __popcll(m & ((1ull << lane) - 1ull));
    todo &= ~m;
  }
  if (lane < S) {
    const int pos = valid ? L.off[id] + rank : -1;
    A.rt.inv[lane] = pos;
    if (valid) A.rt.perm[pos] = lane;
  }
}

// The down kernel's work descriptors, one per routed expert in active order.
// Written by the grid's last wave, which seldom has an expert of its own, so
// the page-table loads here do not lengthen a wave that does.
__device__ __forceinline__ void publish_desc(const GemvArgs& A, const int (&c)[4], int nzr, int run) {
  const int lane = threadIdx.x;
  int qd[4];
  pw_block_desc bd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // every entry requested before any record is stored
    const int ex = 4 * lane + i;
    qd[i] = 0;
    bd[i].planes = nullptr;
    bd[i].lut_all = nullptr;
    if (ex < A.E && c[i] > 0) {
      qd[i] = A.q[2 * ex + 1];
      bd[i] = A.blocks[2 * ex + 1];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = 4 * lane + i;
    if (ex < A.E && c[i] > 0) {
      ActiveDesc dsc;
      dsc.e = ex;
      dsc.n_e = c[i];
      dsc.off_e = run;
      dsc.q = qd[i];
      dsc.planes = bd[i].planes;
      dsc.lut_all = bd[i].lut_all;
      A.rt.adesc[nzr++] = dsc;
    }
    run += c[i];
  }
}

// The grid splits evenly over the (routed expert, K part) segments; a wave's
// segment index (>= n_act * kparts: no work).
// Waves per segment: an even split of the grid, but no more than keeps a
// wave's share at kTargetPairs gate_up pairs / kTargetRows down rows (a wave's
// fixed costs, the routing and the table staging, need some rows to spread over).
constexpr int kTargetPairs = 8;
constexpr int kTargetRows = 8;
template <bool GU>
__device__ __forceinline__ int waves_per_segment(const GemvArgs& A, int n_act) {
  const int rows = GU ? A.I : A.H;
  const int target = GU ? kTargetPairs : kTargetRows;
  return max(1, min((int)gridDim.x / (n_act * A.kparts), (rows + target - 1) / target));
}

template <bool GU>
__device__ __forceinline__ int wave_segment(const GemvArgs& A, int n_act) {
  return (int)blockIdx.x / waves_per_segment<GU>(A, n_act);
}

// Inline routing over S = T*k <= 64 slots, one slot per lane.  Returns false
// when fewer than a+1 experts are routed.
__device__ __forceinline__ bool find_expert_inline(const GemvArgs& A, int& a, Slots& sl, RouteLds& L) {
  const int lane = threadIdx.x;
  const int S = A.T * A.k;
  // With at most 64 experts, lane i requests expert i's gate_up page-table
  // entry together with the ids, so the routed expert's entry is a readlane
  // away instead of a load that waits for the routing.
  const bool pre = A.E <= kWave;
  int pq = 0;
  uint64_t pp = 0, pt = 0;
  if (pre && lane < A.E) {
    pq = A.q[2 * lane];
    const pw_block_desc bd = A.blocks[2 * lane];
    pp = reinterpret_cast<uint64_t>(bd.planes);
    pt = reinterpret_cast<uint64_t>(bd.lut_all);
  }
  const int id = lane < S ? A.ids[lane] : -1;
  const bool valid = id >= 0 && id < A.E;
  if (blockIdx.x == 0 && __ballot(lane < S && !valid) != 0ull && lane == 0)
    raise_status(A.rt.status, PW_DEV_BAD_EXPERT_ID);
  for (int i = lane; i < A.E; i += kWave) L.cnt[i] = 0;
  if (lane == 0) L.e_sel = -1;
  __syncthreads();
  if (valid) atomicAdd(&L.cnt[id], 1);
  __syncthreads();
  int c[4], tot = 0, nz = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = 4 * lane + i;
    c[i] = ex < A.E ? L.cnt[ex] : 0;
    tot += c[i];
    nz += c[i] > 0 ? 1 : 0;
  }
  int run = wave_excl_scan(tot);
  int nzr = wave_excl_scan(nz);
  const int run_base = run, nzr_base = nzr;
  const int n_act = uniform(__shfl(nzr + nz, kWave - 1, kWave));
  a = n_act > 0 ? wave_segment<true>(A, n_act) / A.kparts : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = 4 * lane + i;
    if (ex < A.E) L.off[ex] = run;
    run += c[i];
    if (c[i] > 0) {
      if (nzr == a) L.e_sel = ex;
      ++nzr;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) publish_route(A, L, id, valid, c, nzr_base, run_base);
  if (blockIdx.x == gridDim.x - 1) publish_desc(A, c, nzr_base, run_base);
  // Values read back from LDS are the same in every lane; saying so keeps the
  // block's buffer descriptor in scalar registers.
  sl.num_active = __builtin_amdgcn_readfirstlane(n_act);
  if (a >= sl.num_active) return false;
  const int e = __builtin_amdgcn_readfirstlane(L.e_sel);
  sl.e = e;
  sl.n_e = __builtin_amdgcn_readfirstlane(L.cnt[e]);
  sl.off_e = __builtin_amdgcn_readfirstlane(L.off[e]);
  sl.mask = __ballot(id == e);
  sl.pre = pre;
  if (pre) {
    auto pick = [e](uint64_t v) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, e);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), e);
      return ((uint64_t)hi << 32) | lo;
    };
    sl.qd = __builtin_amdgcn_readlane(pq, e);
    sl.d.planes = reinterpret_cast<const uint32_t*>(pick(pp));
    sl.d.lut_all = reinterpret_cast<const uint16_t*>(pick(pt));
  }
  return true;
}

template <bool GU>
__device__ __forceinline__ bool find_expert_routed(const GemvArgs& A, int& a, Slots& sl) {
  const int n_act = uniform(*A.rt.num_active);
  sl.num_active = n_act;
  sl.pre = false;
  a = n_act > 0 ? wave_segment<GU>(A, n_act) / A.kparts : 0;
  if (a >= n_act) return false;
  const int e = uniform(A.rt.active[a]);
  sl.e = e;
  sl.n_e = uniform(A.rt.counts[e]);
  sl.off_e = uniform(A.rt.offsets[e]);
  sl.mask = 0ull;
  return true;
}

// Down product after inline routing: once the active count is known, one
// load of the wave's 32-byte work descriptor gives the expert, its token
// range and the page-table entry of its down block (instead of three dependent
// loads: expert id, count and offset, page-table entry).
__device__ __forceinline__ bool find_expert_desc(const GemvArgs& A, int& a, Slots& sl, int& per) {
  const int n_act = uniform(*A.rt.num_active);
  sl.num_active = n_act;
  sl.mask = 0ull;
  sl.pre = false;
  if (n_act <= 0) return false;
  per = waves_per_segment<false>(A, n_act);
  a = ((int)blockIdx.x / per) / A.kparts;
  if (a >= n_act) return false;
  const ActiveDesc dsc = A.rt.adesc[a];
  sl.e = uniform(dsc.e);
  sl.n_e = uniform(dsc.n_e);
  sl.off_e = uniform(dsc.off_e);
  sl.qd = uniform(dsc.q);
  sl.d.planes = uniform_ptr(dsc.planes);
  sl.d.lut_all = uniform_ptr(dsc.lut_all);
  return true;
}

// Slot (t*k + j) of the r-th token of the expert, in slot order.
__device__ __forceinline__ int slot_of(const GemvArgs& A, const Slots& sl, int r) {
  if (A.inline_route) {
    unsigned long long m = sl.mask;
    for (int i = 0; i < r; ++i) m &= m - 1ull;
    return __ffsll(m) - 1;
  }
  return uniform(A.rt.perm[sl.off_e + r]);
}

// ---------------------------------------------------------------------------
// One chunk of 16 rows at bitwidth Q for up to NT tokens at a time
// ---------------------------------------------------------------------------
// A chunk: gate_up pairs [first, first + n) (n <= 8; chunk row r < 8 is gate
// row first + r, chunk row 8 + r the matching up row), or down rows
// [first, first + n) (n <= 16) of K part kpart.  Chunk rows past n are masked.
// Rows of one row group are consecutive rows of the block; in the device
// layout a row's 16-word runs of consecutive rows sit next to each other, so
// the four loads of a group touch the same 256-byte spans.
struct Chunk {
  int first, n, kpart;
};

template <bool GU>
__device__ __forceinline__ int chunk_row(const Chunk& ch, int r, int I) {
  if constexpr (GU) return (r < 8 ? 0 : I) + ch.first + (r & 7);
  else return ch.first + r;
}

template <bool GU>
__device__ __forceinline__ bool chunk_row_valid(const Chunk& ch, int r) {
  return GU ? (r & 7) < ch.n : r < ch.n;
}

// Device-layout row of chunk row r (gate_up rows are interleaved per tile).
template <bool GU>
__device__ __forceinline__ int chunk_dev_row(const Chunk& ch, int r) {
  if constexpr (GU) return r < 8 ? dev_row_of_gate(ch.first + r) : dev_row_of_up(ch.first + (r & 7));
  else return ch.first + r;
}

template <int Q, int NT, bool GU>
__device__ __forceinline__ void chunk_body(const GemvArgs& A, const Slots& sl, const Chunk& ch, uint8_t* tabs) {
  constexpr int G = 4;                         // rows per pipeline group
  constexpr int NGR = kChunkRows / G;          // groups per slice
  constexpr int TAB = (1 << Q) * 2;            // bytes per row table
  constexpr int TSTRIDE = kTabStride<Q>;       // LDS bytes between row tables
  constexpr int M = G * NT;                    // values reduced per group
  constexpr int MSH = 6 - (M == 1 ? 0 : M == 2 ? 1 : M == 4 ? 2 : M == 8 ? 3 : 4);
  const int lane = threadIdx.x;
  const int H = A.H, I = A.I;
  const int N = GU ? 2 * I : H;
  const int K = GU ? H : I;
  const int W = K >> 5;
  const pw_block_desc d = sl.d;
  const uint32_t pstride = (uint32_t)N * (uint32_t)W * 4u;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(uniform_ptr(d.planes), pstride * (uint32_t)Q);
  const uint16_t* __restrict__ lut = uniform_ptr(d.lut_all) + lut_offset(N, Q);

  // Row tables of the chunk -> LDS with direct buffer-to-LDS loads (no
  // registers, no LDS store instructions): load i fills LDS bytes
  // [1024 i, 1024 i + 1024), lane l the 16 bytes at 1024 i + 16 l, taken from
  // the table row and piece those bytes belong to (row tables sit TSTRIDE apart;
  // the bytes past a row's table and the rows past the chunk read as zero).
  // They land asynchronously; the wait before the first lookup covers them.
  {
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lut, (uint32_t)N * (uint32_t)TAB);
    constexpr int NI = kChunkRows * TSTRIDE / 1024;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int dst = 1024 * i + 16 * lane;
      const int pos = dst / TSTRIDE, col = dst % TSTRIDE;
      const uint32_t voff = (col < TAB && chunk_row_valid<GU>(ch, pos))
                                ? (uint32_t)chunk_row<GU>(ch, pos, I) * (uint32_t)TAB + (uint32_t)col
                                : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)(tabs + 1024 * i), 16,
                                               voff, 0, 0, 0);
    }
  }

  const uint32_t tab_base = lds_addr(tabs);
  const int nsl = (W + kWave - 1) / kWave;
  const int spp = (nsl + A.kparts - 1) / A.kparts;
  const int s_begin = ch.kpart * spp;
  const int s_end = min(nsl, s_begin + spp);
  const int nsteps = max(0, s_end - s_begin) * NGR;
  const int slots = A.T * A.k;
  // a row group with no row inside the chunk is neither loaded nor computed
  auto group_live = [&](int g) { return chunk_row_valid<GU>(ch, g * G); };   // its first row

  for (int t0 = 0; t0 < sl.n_e; t0 += NT) {
    const int nt = min(NT, sl.n_e - t0);
    const uint16_t* xsrc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      xsrc[t] = nullptr;
      if (t < nt) {
        if constexpr (GU) xsrc[t] = A.act + (size_t)(slot_of(A, sl, t0 + t) / A.k) * H;
        else xsrc[t] = A.act + (size_t)(sl.off_e + t0 + t) * I;
      }
    }

    float tot = 0.0f;                // lane (t * 16 + r): total of chunk row r, token t
    // down: o rows are indexed by slot (t*k + j), so the combine needs no
    // indirection; the lane's slot is requested here and used at the end
    int oslot = 0;
    if constexpr (!GU) {
      const int tl = lane >> 4;
      if (lane < 32 && t0 + tl < sl.n_e) oslot = A.rt.perm[sl.off_e + t0 + tl];
    }
    uint32_t Pa[G][Q], Pb[G][Q];
    half2_t xr[NT][16];
    int xslice = -1;

    auto load_group = [&](uint32_t (&P)[G][Q], int st) {
      const int slice = s_begin + st / NGR;
      const int g = st % NGR;
      if (!group_live(g)) return;
      const int wc = slice * kWave + lane;
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const uint32_t voff = (wc < W && chunk_row_valid<GU>(ch, g * G + r))
                                  ? dev_word(chunk_dev_row<GU>(ch, g * G + r), wc, W) * 4u
                                  : kOutOfRange;
#pragma unroll
        for (int p = 0; p < Q; ++p) P[r][p] = buf_load_u32(prs, voff, (uint32_t)p * pstride);
      }
    };

    auto load_x = [&](int slice) {
      xslice = slice;
      const int wc = slice * kWave + lane;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint4 u[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          u[v] = make_uint4(0u, 0u, 0u, 0u);
          if (xsrc[t] != nullptr && wc < W) u[v] = *reinterpret_cast<const uint4*>(xsrc[t] + wc * 32 + v * 8);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if constexpr (Q == 3) {
            // pairs (x[8v + c], x[8v + c + 4]) at 4c + v
            xr[t][0 + v] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(u[v].z, u[v].x, 0x05040100u));
            xr[t][4 + v] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(u[v].z, u[v].x, 0x07060302u));
            xr[t][8 + v] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(u[v].w, u[v].y, 0x05040100u));
            xr[t][12 + v] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(u[v].w, u[v].y, 0x07060302u));
          } else {
            xr[t][4 * v + 0] = __builtin_bit_cast(half2_t, u[v].x);
            xr[t][4 * v + 1] = __builtin_bit_cast(half2_t, u[v].y);
            xr[t][4 * v + 2] = __builtin_bit_cast(half2_t, u[v].z);
            xr[t][4 * v + 3] = __builtin_bit_cast(half2_t, u[v].w);
          }
        }
      }
    };

    auto compute_group = [&](uint32_t (&P)[G][Q], int st) {
      const int slice = s_begin + st / NGR;
      const int g = st % NGR;
      if (!group_live(g)) return;
      if (slice != xslice) load_x(slice);
      float acc[M];
#pragma unroll
      for (int i = 0; i < M; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int r = 0; r < G; ++r) {
        // one row at a time: keeps the scheduler from interleaving the decode
        // of several rows, which would cost registers and occupancy
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (Q == 3) {
          uint32_t R[4];
          planes_to_pairs3(P[r], R);
          row_dot_pairs3<NT>(R, tab_base + (uint32_t)((g * G + r) * TSTRIDE), xr, &acc[r * NT]);
        } else {
          uint32_t R[8];
          planes_to_fields<Q>(P[r], R);
          row_dot<Q, NT>(R, tab_base + (uint32_t)((g * G + r) * TSTRIDE), xr, &acc[r * NT]);
        }
      }
      const float red = multi_reduce<M>(acc);
      // lane L = t * 16 + row takes value (row - g*G) * NT + t from lane vi << MSH
      const int t_l = lane >> 4;
      const int r_l = (lane & 15) - g * G;
      const int vi = (r_l >= 0 && r_l < G) ? r_l * NT + t_l : 0;
      const float v = __shfl(red, vi << MSH, kWave);
      if (t_l < NT && r_l >= 0 && r_l < G) tot += v;
    };

    // the activations of the first slice, then the first two row groups
    if (nsteps > 0) load_x(s_begin);
    if (nsteps > 0) load_group(Pa, 0);
    if (nsteps > 1) load_group(Pb, 1);
    // everything issued so far, the staged row tables included, has landed
    // (the builtin, unlike inline assembly, is seen by the compiler's wait
    // tracking, which then does not wait for the table loads again in the
    // row loop); 3-bit tables then become pair tables
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if constexpr (Q == 3) {
      if (t0 == 0) build_pair_tables3(tab_base);
    }
    for (int st = 0; st < nsteps; st += 2) {
      compute_group(Pa, st);
      if (st + 2 < nsteps) load_group(Pa, st + 2);
      if (st + 1 < nsteps) compute_group(Pb, st + 1);
      if (st + 3 < nsteps) load_group(Pb, st + 3);
    }

    const int t_l = lane >> 4;
    const int r_l = lane & 15;
    if constexpr (GU) {
      // up row r + 8 sits 8 lanes above gate row r inside the same 16-lane row
      const float u = dpp_f<kDppRor8>(tot);
      const int pair = r_l;
      if (lane < 32 && r_l < 8 && pair < ch.n && t_l < nt) {
        const float h = silu_f32(tot) * u;
        const _Float16 hh = (_Float16)h;
        A.hout[(size_t)(sl.off_e + t0 + t_l) * I + ch.first + pair] = __builtin_bit_cast(uint16_t, hh);
      }
    } else {
      if (lane < 32 && t_l < nt && r_l < ch.n)
        A.oout[((size_t)ch.kpart * slots + oslot) * H + ch.first + r_l] = tot;
    }
  }
}

// Rows of a block whose committed bitwidth is invalid read as zero.
template <bool GU>
__device__ __forceinline__ void chunk_zero(const GemvArgs& A, const Slots& sl, const Chunk& ch) {
  const int lane = threadIdx.x;
  const int slots = A.T * A.k;
  for (int i = lane; i < sl.n_e * ch.n; i += kWave) {
    const int t = i / ch.n, r = i % ch.n;
    if constexpr (GU) A.hout[(size_t)(sl.off_e + t) * A.I + ch.first + r] = 0;
    else A.oout[((size_t)ch.kpart * slots + A.rt.perm[sl.off_e + t]) * A.H + ch.first + r] = 0.0f;
  }
  if (lane == 0 && ch.first == 0 && ch.kpart == 0) raise_status(A.rt.status, PW_DEV_BAD_BITWIDTH);
}

template <int Q, bool GU>
__device__ __forceinline__ void chunk_by_tokens(const GemvArgs& A, const Slots& sl, const Chunk& ch, uint8_t* tabs) {
  if (sl.n_e == 1) chunk_body<Q, 1, GU>(A, sl, ch, tabs);
  else chunk_body<Q, 2, GU>(A, sl, ch, tabs);
}

// The grid is at least as many one-wave workgroups as stay resident together,
// and enough that every wave's share fits one chunk.  Once the number of
// routed experts n is known, each (expert, K part) segment gets
// floor(grid / (n * kparts)) consecutive waves, and each of them an even share
// of the segment's rows (gate_up row pairs, down rows): at most 8 pairs / 16
// rows, so all waves carry about the same work whatever n is.
template <bool GU>
__global__ __launch_bounds__(kWave) void gemv_kernel(GemvArgs A) {
  __shared__ __align__(512) uint8_t tabs[kChunkRows * kMaxTabBytes];   // row tables at kTabStride<Q>
  __shared__ RouteLds L;
  Slots sl;
  int a = 0, per = 1;
  bool have;
  if (!GU && A.desc_mode) {
    have = find_expert_desc(A, a, sl, per);
  } else {
    have = A.inline_route ? find_expert_inline(A, a, sl, L) : find_expert_routed<GU>(A, a, sl);
    if (have) per = waves_per_segment<GU>(A, sl.num_active);
  }
  if (!have) return;
  if (sl.n_e < A.min_tokens || sl.n_e >= A.max_tokens) return;

  const int rows = GU ? A.I : A.H;
  const int seg = (int)blockIdx.x / per;
  const int c = (int)blockIdx.x - seg * per;
  Chunk ch;
  ch.kpart = seg - a * A.kparts;
  ch.first = (int)(((long long)c * rows) / per);
  ch.n = (int)(((long long)(c + 1) * rows) / per) - ch.first;
  if (ch.n <= 0) return;
  // bitwidth and page-table entry of the block, requested together
  int qv;
  if ((!GU && A.desc_mode) || sl.pre) {
    qv = sl.qd;   // the work descriptor, or the routing step, carried the entry
  } else {
    qv = uniform(A.q[2 * sl.e + (GU ? 0 : 1)]);
    sl.d = A.blocks[2 * sl.e + (GU ? 0 : 1)];
  }
  switch (qv) {
    case 3: chunk_by_tokens<3, GU>(A, sl, ch, tabs); break;
    case 4: chunk_by_tokens<4, GU>(A, sl, ch, tabs); break;
    case 5: chunk_by_tokens<5, GU>(A, sl, ch, tabs); break;
    case 6: chunk_by_tokens<6, GU>(A, sl, ch, tabs); break;
    case 7: chunk_by_tokens<7, GU>(A, sl, ch, tabs); break;
    case 8: chunk_by_tokens<8, GU>(A, sl, ch, tabs); break;
    default: chunk_zero<GU>(A, sl, ch); break;
  }
}

// Resident one-wave workgroups of a kernel (cached per device).
template <bool GU>
static int resident_waves() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  if (cache[dev] == 0) {
    int ncu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemv_kernel<GU>, kWave, 0) != hipSuccess || per_cu <= 0)
      per_cu = 4;
    cache[dev] = ncu * per_cu;
  }
  return cache[dev];
}

static GemvArgs make_args(const GemvLaunch& g) {
  GemvArgs A{};
  A.H = g.H; A.I = g.I; A.E = g.E; A.k = g.k; A.T = g.T;
  A.blocks = g.blocks; A.q = g.q; A.ids = g.ids; A.rt = g.rt;
  A.min_tokens = g.min_tokens; A.max_tokens = g.max_tokens;
  return A;
}

// Waves for a launch: the resident count, but at least enough that with every
// expert routed each wave's share is one chunk (8 pairs / 16 rows), and no more
// than the split can use (shares of kTargetPairs / kTargetRows).
template <bool GU>
static int gemv_grid(const GemvArgs& A) {
  const long long bound = (long long)(A.E < A.T * A.k ? A.E : A.T * A.k) * A.kparts;
  const int rows = GU ? A.I : A.H;
  const int chunk = GU ? 8 : kChunkRows;
  const int target = GU ? kTargetPairs : kTargetRows;
  const long long need = bound * ((rows + chunk - 1) / chunk);
  const long long cap = bound * ((rows + target - 1) / target);
  long long g = resident_waves<GU>();
  if (g < need) g = need;
  if (g > cap) g = cap;
  return (int)g;
}

hipError_t launch_gemv_gate_up(const GemvLaunch& g, hipStream_t s, const KernelEvents& ev) {
  GemvArgs A = make_args(g);
  A.inline_route = g.inline_route;
  A.act = g.x; A.hout = g.h; A.oout = nullptr;
  A.kparts = 1;
  return launch_kernel(gemv_kernel<true>, dim3(gemv_grid<true>(A)), dim3(kWave), s, ev, A);
}

hipError_t launch_gemv_down(const GemvLaunch& g, hipStream_t s, const KernelEvents& ev) {
  GemvArgs A = make_args(g);
  A.inline_route = 0;    // the gate_up kernel or the route kernel published the routing
  A.act = g.h; A.hout = nullptr; A.oout = g.o;
  A.kparts = g.kparts;
  A.desc_mode = g.inline_route;   // the gate_up kernel published the work descriptors
  return launch_kernel(gemv_kernel<false>, dim3(gemv_grid<false>(A)), dim3(kWave), s, ev, A);
}

}  // namespace pw
