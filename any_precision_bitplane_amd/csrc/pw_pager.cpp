// Weight pager: the Weight Page Table's bookkeeping, asynchronous page
// movement and safe-boundary commits.
//
// "Technical summary: PagedWeight" (gist.science, paper 2607.16184):
//   - Core components 1, third bullet: the page table keeps per block a desired
//     bitwidth d_i and a committed bitwidth q_i; a page is GPU-resident,
//     CPU-resident or in transfer.
//   - Core components 3, first bullet: pages are offloaded to CPU memory and
//     reloaded asynchronously to hide the latency; committed bitwidths change
//     only at safe boundaries, so inference is never interrupted.
//
// Here a page is one bit plane of one block.  The host keeps all eight planes
// of every block (pinned memory, caller-owned), so offloading a plane is
// dropping it from the GPU and reloading it is one host-to-device copy.  On the
// GPU a block's resident planes 0..r-1 form one extent of the caller's arena
// (plane-major storage makes them a contiguous prefix).  Raising d beyond r
// grows the extent in place when the following range is free, otherwise moves
// the block to a new extent (device-to-device copy of the resident planes);
// the missing planes come from the host.  All copies run on the caller's copy
// stream and are fenced by one event per execute call.  A commit is one small
// kernel on the compute stream that rewrites the page-table entries (plane
// pointer, table pointer) and the q bytes of every changed block together, so
// forwards enqueued before it see the old bitwidths and storage and forwards
// after it the new ones.  Arena ranges a commit leaves unused (a lowered
// block's plane suffix, a moved block's old extent) go back to the allocator
// only once the compute stream has passed the commit.
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "pw_arena.h"
#include "pw_internal.h"

namespace pw {

struct CommitRec {
  const uint32_t* planes;
  const uint16_t* lut;
  int32_t index;
  int32_t q;
};
constexpr int kCommitBatch = 128;   // 24-byte records: the batch stays within 4 KB of kernel arguments
struct CommitBatch {
  pw_block_desc* blocks;
  uint8_t* q;
  int32_t n;
  CommitRec rec[kCommitBatch];
};

__global__ __launch_bounds__(kCommitBatch) void commit_kernel(CommitBatch b) {
  const int i = threadIdx.x;
  if (i >= b.n) return;
  const CommitRec r = b.rec[i];
  b.blocks[r.index].planes = r.planes;
  b.blocks[r.index].lut_all = r.lut;
  b.q[r.index] = (uint8_t)r.q;
}

}  // namespace pw

using namespace pw;

namespace {

constexpr size_t kNoExtent = ExtentArena::kNone;

struct Block {
  int32_t N = 0, K = 0;
  size_t plane_bytes = 0;
  const uint32_t* host = nullptr;    // pinned host planes [8][N][K/32]
  const uint16_t* lut = nullptr;     // device tables [504 N]
  int32_t desired = 0;               // d_i (0: never requested)
  int32_t committed = 0;             // q_i as the page table holds it (0: not committed yet)
  int32_t resident = 0;              // planes of the committed extent on the GPU
  size_t off = kNoExtent;            // committed extent
  // staged by execute, applied by commit
  bool pending = false;
  int32_t target = 0;
  size_t new_off = kNoExtent;
  int32_t event = -1;                // index into Pager::events of the copies it waits for, -1 if none
};

struct Retired {
  hipEvent_t ev;                                   // recorded on the compute stream after the commit
  std::vector<std::pair<size_t, size_t>> ranges;   // (offset, bytes) unused from then on
  std::vector<hipEvent_t> fences;                  // copy fences the commit waited for
};

}  // namespace

struct pw_pager {
  std::vector<Block> blocks;
  uint8_t* arena = nullptr;
  ExtentArena alloc;
  pw_block_desc* table = nullptr;
  uint8_t* qtab = nullptr;
  std::vector<hipEvent_t> events;        // copy fences of the plan being staged
  std::vector<Retired> retired;
};

namespace {

size_t ext_bytes(const Block& b, int planes) { return b.plane_bytes * (size_t)planes; }

hipError_t new_event(hipEvent_t* ev) { return hipEventCreateWithFlags(ev, hipEventDisableTiming); }

// Release the ranges of retirements whose commit the compute stream has passed.
pw_status reclaim(pw_pager* p) {
  size_t keep = 0;
  for (size_t i = 0; i < p->retired.size(); ++i) {
    Retired& r = p->retired[i];
    const hipError_t q = hipEventQuery(r.ev);
    if (q == hipErrorNotReady) {
      p->retired[keep++] = std::move(r);
      continue;
    }
    if (q != hipSuccess) return PW_ERR_HIP;
    for (const auto& rg : r.ranges) p->alloc.release(rg.first, rg.second);
    for (hipEvent_t f : r.fences) hipEventDestroy(f);
    hipEventDestroy(r.ev);
  }
  p->retired.resize(keep);
  return PW_OK;
}

bool valid_pager(const pw_pager* p) { return p != nullptr; }

}  // namespace

extern "C" {

pw_status pw_pager_create(int32_t num_blocks, const int32_t* rows, const int32_t* cols, void* arena,
                          size_t arena_bytes, pw_block_desc* blocks, uint8_t* q, pw_pager** out) {
  if (!out) return PW_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0 || !rows || !cols || !arena || !blocks || !q) return PW_ERR_INVALID_ARG;
  if ((uintptr_t)arena % kAlign || (uintptr_t)blocks % 8) return PW_ERR_ALIGNMENT;
  for (int32_t b = 0; b < num_blocks; ++b) {
    if (rows[b] <= 0 || cols[b] <= 0) return PW_ERR_INVALID_ARG;
    if (cols[b] % 32) return PW_ERR_UNSUPPORTED_SHAPE;
    // the kernels address planes with 32-bit byte offsets
    if ((int64_t)rows[b] * cols[b] > INT32_MAX) return PW_ERR_UNSUPPORTED_SHAPE;
  }
  pw_pager* p = new (std::nothrow) pw_pager();
  if (!p) return PW_ERR_INVALID_ARG;
  p->blocks.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) {
    p->blocks[b].N = rows[b];
    p->blocks[b].K = cols[b];
    p->blocks[b].plane_bytes = (size_t)rows[b] * (size_t)(cols[b] / 8);
  }
  p->arena = reinterpret_cast<uint8_t*>(arena);
  p->alloc.reset(arena_bytes, kAlign);
  p->table = blocks;
  p->qtab = q;
  *out = p;
  return PW_OK;
}

pw_status pw_pager_destroy(pw_pager* p) {
  if (!p) return PW_OK;
  pw_status st = PW_OK;
  for (hipEvent_t ev : p->events) {
    if (hipEventSynchronize(ev) != hipSuccess) st = PW_ERR_HIP;
    hipEventDestroy(ev);
  }
  for (Retired& r : p->retired) {
    if (hipEventSynchronize(r.ev) != hipSuccess) st = PW_ERR_HIP;
    for (hipEvent_t f : r.fences) hipEventDestroy(f);
    hipEventDestroy(r.ev);
  }
  delete p;
  return st;
}

pw_status pw_pager_set_block(pw_pager* p, int32_t b, const uint32_t* host_planes, const uint16_t* lut_all) {
  if (!valid_pager(p) || b < 0 || b >= (int32_t)p->blocks.size() || !host_planes || !lut_all)
    return PW_ERR_INVALID_ARG;
  if ((uintptr_t)lut_all % 16 || (uintptr_t)host_planes % 4) return PW_ERR_ALIGNMENT;
  Block& k = p->blocks[b];
  if (k.committed != 0 || k.pending) return PW_ERR_INVALID_ARG;   // only before the block's first commit
  k.host = host_planes;
  k.lut = lut_all;
  return PW_OK;
}

pw_status pw_pager_request(pw_pager* p, int32_t b, int32_t desired) {
  if (!valid_pager(p) || b < 0 || b >= (int32_t)p->blocks.size()) return PW_ERR_INVALID_ARG;
  if (desired < kMinBits || desired > kMaxBits) return PW_ERR_BITWIDTH;
  Block& k = p->blocks[b];
  if (!k.host || !k.lut) return PW_ERR_INVALID_ARG;
  k.desired = desired;
  return PW_OK;
}

pw_status pw_pager_execute(pw_pager* p, void* copy_stream) {
  if (!valid_pager(p)) return PW_ERR_INVALID_ARG;
  pw_status st = reclaim(p);
  if (st != PW_OK) return st;
  hipStream_t s = (hipStream_t)copy_stream;
  bool copied = false;
  const int32_t ev_index = (int32_t)p->events.size();
  for (Block& k : p->blocks) {
    if (k.pending || k.desired == 0 || k.desired == k.committed) continue;
    const int32_t d = k.desired;
    if (d <= k.resident) {   // planes already on the GPU: nothing moves
      k.pending = true;
      k.target = d;
      k.new_off = k.off;
      k.event = -1;
      continue;
    }
    size_t dst;
    bool moved = false;
    if (k.off != kNoExtent && p->alloc.grow(k.off, ext_bytes(k, k.resident), ext_bytes(k, d))) {
      dst = k.off;
    } else {
      dst = p->alloc.alloc(ext_bytes(k, d));
      if (dst == kNoExtent) {
        st = PW_ERR_OUT_OF_MEMORY;   // this block and the ones after it stay as they are
        break;
      }
      moved = k.off != kNoExtent;
    }
    hipError_t e = hipSuccess;
    if (moved)
      e = hipMemcpyAsync(p->arena + dst, p->arena + k.off, ext_bytes(k, k.resident), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(p->arena + dst + ext_bytes(k, k.resident),
                         reinterpret_cast<const uint8_t*>(k.host) + ext_bytes(k, k.resident),
                         ext_bytes(k, d - k.resident), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      // not staged: the range goes back (any copy that did enqueue runs on this
      // stream before whatever reuses it) and the block keeps its committed state
      if (dst == k.off)
        p->alloc.release(k.off + p->alloc.round(ext_bytes(k, k.resident)),
                         p->alloc.round(ext_bytes(k, d)) - p->alloc.round(ext_bytes(k, k.resident)));
      else
        p->alloc.release(dst, ext_bytes(k, d));
      copied = copied || moved;
      st = PW_ERR_HIP;
      break;
    }
    copied = true;
    k.pending = true;
    k.target = d;
    k.new_off = dst;
    k.event = ev_index;
  }
  if (copied) {
    // one fence for every copy this call enqueued (also when it stopped early)
    hipEvent_t ev;
    if (new_event(&ev) != hipSuccess) return PW_ERR_HIP;
    if (hipEventRecord(ev, s) != hipSuccess) {
      hipEventDestroy(ev);
      return PW_ERR_HIP;
    }
    p->events.push_back(ev);
  }
  return st;
}

pw_status pw_pager_commit(pw_pager* p, void* stream, int32_t wait, int32_t* committed) {
  if (!valid_pager(p)) return PW_ERR_INVALID_ARG;
  if (committed) *committed = 0;
  pw_status st = reclaim(p);
  if (st != PW_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> todo;
  for (int32_t b = 0; b < (int32_t)p->blocks.size(); ++b)
    if (p->blocks[b].pending) todo.push_back(b);
  if (todo.empty()) return PW_OK;

  // The plan is committed as a whole, once every copy it started has landed.
  for (hipEvent_t ev : p->events) {
    const hipError_t q = hipEventQuery(ev);
    if (q == hipSuccess) continue;
    if (q != hipErrorNotReady) return PW_ERR_HIP;
    if (!wait) return PW_OK;
    if (hipStreamWaitEvent(s, ev, 0) != hipSuccess) return PW_ERR_HIP;
  }

  for (size_t i0 = 0; i0 < todo.size(); i0 += kCommitBatch) {
    CommitBatch batch;
    batch.blocks = p->table;
    batch.q = p->qtab;
    batch.n = 0;
    for (size_t i = i0; i < todo.size() && batch.n < kCommitBatch; ++i) {
      const Block& k = p->blocks[todo[i]];
      CommitRec& r = batch.rec[batch.n++];
      r.planes = reinterpret_cast<const uint32_t*>(p->arena + k.new_off);
      r.lut = k.lut;
      r.index = todo[i];
      r.q = k.target;
    }
    hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(kCommitBatch), 0, s, batch);
    if (hipGetLastError() != hipSuccess) return PW_ERR_HIP;
  }

  Retired r;
  if (new_event(&r.ev) != hipSuccess) return PW_ERR_HIP;
  if (hipEventRecord(r.ev, s) != hipSuccess) {
    hipEventDestroy(r.ev);
    return PW_ERR_HIP;
  }
  for (int32_t b : todo) {
    Block& k = p->blocks[b];
    if (k.new_off != k.off) {
      if (k.off != kNoExtent) r.ranges.emplace_back(k.off, p->alloc.round(ext_bytes(k, k.resident)));
    } else if (k.target < k.resident) {
      const size_t keep = p->alloc.round(ext_bytes(k, k.target));
      const size_t had = p->alloc.round(ext_bytes(k, k.resident));
      if (had > keep) r.ranges.emplace_back(k.off + keep, had - keep);
    }
    k.off = k.new_off;
    k.committed = k.target;
    k.resident = k.target;
    k.pending = false;
    k.new_off = kNoExtent;
    k.event = -1;
  }
  // the fences stay alive until the compute stream has passed the commit
  r.fences.swap(p->events);
  p->retired.push_back(std::move(r));
  if (committed) *committed = (int32_t)todo.size();
  return PW_OK;
}

pw_status pw_pager_info(const pw_pager* p, int32_t b, pw_page_info* info) {
  if (!valid_pager(p) || !info || b < 0 || b >= (int32_t)p->blocks.size()) return PW_ERR_INVALID_ARG;
  const Block& k = p->blocks[b];
  info->desired = k.desired;
  info->committed = k.committed;
  info->resident = k.resident;
  info->pending = k.pending ? k.target : 0;
  if (k.pending && k.event >= 0 && k.event < (int32_t)p->events.size() &&
      hipEventQuery(p->events[k.event]) == hipErrorNotReady)
    info->state = PW_PAGE_IN_TRANSFER;
  else if (k.resident == 0 && !k.pending)
    info->state = PW_PAGE_CPU;
  else
    info->state = PW_PAGE_GPU;
  info->arena_offset = k.off == kNoExtent ? UINT64_MAX : (uint64_t)k.off;
  return PW_OK;
}

size_t pw_pager_arena_used(const pw_pager* p) { return p ? p->alloc.used() : 0; }

}  // extern "C"
