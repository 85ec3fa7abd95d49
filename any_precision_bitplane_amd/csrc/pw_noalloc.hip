// Allocation-free variant of the fused layer's forward, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The routing lists, h and o that pw_moe_forward keeps in the caller's
// workspace live here in one static device array per GPU, `scratch`
// (PW_NOALLOC_SCRATCH_BYTES, held until the process ends).  Host code never
// passes the array's name to a kernel: the name is a host-side stand-in, not a
// device address.  The first call on a device, with that device current, asks
// the runtime for the array's device address once and keeps it per device;
// every kernel argument uses that address.
//
// What must start at zero: nothing.  Every scratch byte the forward reads was
// written earlier in the same call (routing lists, h, o, work descriptors), so
// the contents left by the previous call do no harm.  Device errors are raised
// in the caller's status word when one is passed, else in a word of the scratch
// header that nobody reads.  All calls on one GPU share its array: calls that
// overlap in time on one GPU (different streams, different host threads) race.
#include <mutex>

#include "pw_internal.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[PW_NOALLOC_SCRATCH_BYTES];

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

// Device address of this GPU's copy of `scratch` (the current device's).
pw_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PW_ERR_HIP;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d]() {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    d.ptr = d.err == hipSuccess ? p : nullptr;
  });
  if (d.err != hipSuccess || d.ptr == nullptr) return PW_ERR_HIP;
  *out = d.ptr;
  return PW_OK;
}

}  // namespace

extern "C" pw_status pw_moe_forward_noalloc(const pw_moe_shape* shape, int32_t T, const uint16_t* x,
                                            const int32_t* ids, const float* w, const pw_block_desc* blocks,
                                            const uint8_t* q, uint16_t* y, uint32_t* status,
                                            const pw_moe_options* opts, void* stream) {
  pw_status st = pw::check_forward_args(shape, T, x, ids, w, blocks, q, y, opts);
  if (st != PW_OK || T == 0) return st;
  if (status && (uintptr_t)status % 4) return PW_ERR_ALIGNMENT;
  const pw::WsLayout L = pw::ws_layout(shape->hidden, shape->inter, shape->num_experts, shape->top_k, T);
  if (L.total > (size_t)PW_NOALLOC_SCRATCH_BYTES) return PW_ERR_WORKSPACE;
  void* base = nullptr;
  st = scratch_address(&base);
  if (st != PW_OK) return st;
  return pw::forward_on(shape, T, x, ids, w, blocks, q, y, reinterpret_cast<uint8_t*>(base), status, opts,
                        (hipStream_t)stream);
}
