// moe_forward_persistent for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the workspace and
// the ring live in a file-scope device array instead of caller buffers.
//
// The array is kNoAllocBytes per GPU, held by every GPU the library runs on until the
// process ends: the first kNoAllocWsBytes are the workspace (control words, layout and task
// tables), the rest is the ring.  Host code never uses the array's name as an address: the
// device address is looked up once per device with hipGetSymbolAddress and kept.  Every call
// on one GPU shares that GPU's array; the persistent path clears what must start at zero
// (the preparation kernel zeroes the control block, the layout kernels write every table
// they later read), so a call never sees an earlier call's contents, but calls that overlap
// on one GPU (different streams, no ordering between them) race on the array.
#include "common.hpp"

namespace moe {

constexpr size_t kNoAllocBytes = size_t(128) << 20;
constexpr size_t kNoAllocWsBytes = size_t(8) << 20;
static_assert(kNoAllocBytes == size_t(MOE_NOALLOC_SCRATCH_BYTES), "scratch size and header disagree");
static_assert(kNoAllocWsBytes == size_t(MOE_NOALLOC_WORKSPACE_BYTES), "workspace size and header disagree");

static __device__ __align__(256) char scratch[kNoAllocBytes];

__global__ void noalloc_status_kernel(const int32_t* src, int32_t* dst) { *dst = *src; }

namespace {
// per-device address of `scratch`, looked up once per device (with that device current)
char* scratch_ptr(int* rc) {
  static std::atomic<char*> ptrs[64];          // zero-initialised (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *rc = MOE_EHIP;
    return nullptr;
  }
  char* p = ptrs[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
      *rc = MOE_EHIP;
      return nullptr;
    }
    p = static_cast<char*>(q);
    ptrs[dev].store(p, std::memory_order_release);   // a repeated lookup in a race is harmless
  }
  *rc = MOE_OK;
  return p;
}
}  // namespace

}  // namespace moe

using namespace moe;

extern "C" int moe_forward_persistent_noalloc(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                                              const float* const* logits, const void* const* x, const void* w1,
                                              const void* w3, const void* w2, void* const* recv, void* const* y,
                                              int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                              int32_t* pull_src, int32_t* slot_of, int32_t* status, void* stream) {
  if (ex && ex->trace != 0) return MOE_EINVAL;            // the trace needs a caller workspace
  const size_t need = moe_persistent_workspace_bytes(s, p, ex);
  if (need == 0) return MOE_EINVAL;                       // bad shape or placement
  if (need > kNoAllocWsBytes) return MOE_ENOSPC;          // shape beyond the array's workspace part
  if (status && (reinterpret_cast<uintptr_t>(status) & 3)) return MOE_EALIGN;
  if (s->dtype != MOE_BF16) return MOE_EUNSUP;               // the MXFP8 ring needs the weights' scales
  int rc = MOE_OK;
  char* base = scratch_ptr(&rc);
  if (!base) return rc;
  rc = moe_forward_persistent(s, p, ex, logits, x, w1, w3, w2, nullptr, base + kNoAllocWsBytes, kNoAllocBytes - kNoAllocWsBytes,
                              recv, y, topk_idx, topk_w, counts, offsets, pull_src, slot_of, base, kNoAllocWsBytes,
                              stream);
  if (rc || !status) return rc;
  hipLaunchKernelGGL(noalloc_status_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<const int32_t*>(base) + kCtrlStatus, status);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
