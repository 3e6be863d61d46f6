// Ceilings of one MI355X that the kernels' rooflines are read against: the MFMA issue rate
// with no memory traffic, and the bandwidth of the direct global->LDS fills the grouped
// GEMM tiles use, with and without L2 hits.  A measurement utility beside the signal
// probe; no part of the layer's path.
//
//   kind 0: v_mfma_f32_32x32x16_bf16, 8 independent accumulators per wave, operands in
//           registers; 4 waves (one per SIMD) per workgroup, one workgroup per CU.
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit scales), the same shape.
//   kind 2: 512-thread workgroups (one per CU) each stream a contiguous share of `src`
//           through two 64 KiB LDS stages with global_load_lds_dwordx4, one barrier per
//           64 KiB round -- the tiles' fill pattern without their MFMAs.  Rows miss the L2.
//   kind 3: the same, every workgroup re-reading one 64 KiB window of the first 1 MiB of
//           `src` (16 windows, workgroup w takes window w mod 16): the fills hit the L2.
// Each thread writes one word of its result to scratch, so that the work is observable:
// MFMA kinds the value of its first accumulator element (16 * reps for bf16 ones, 64 *
// reps for unit E4M3 codes); fill kinds the LDS word at its index in the last stage
// filled, i.e. a word of `src` the caller can predict.
#include <algorithm>

#include "common.hpp"

namespace moe {

constexpr int kCeilMfmaThreads = 256, kCeilFillThreads = 512;
constexpr int kCeilRound = 65536;           // bytes per fill round (one LDS stage)

typedef __attribute__((address_space(3))) void* ceil_lds_ptr;
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kCeilMfmaThreads) void ceil_mfma_bf16_kernel(int reps, uint32_t abits, float* out) {
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
  const bf16x8 a = __builtin_bit_cast(bf16x8, i32x4{int(abits), int(abits), int(abits), int(abits)});
  for (int r = 0; r < reps; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[i], 0, 0, 0);
  }
  float s = acc[0][0];
#pragma unroll
  for (int i = 1; i < 8; ++i) s += acc[i][0] * 0.0f;     // keep every chain live
  out[blockIdx.x * kCeilMfmaThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kCeilMfmaThreads) void ceil_mfma_mx_kernel(int reps, uint32_t abits, float* out) {
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
  const int w = int(abits);
  const i32x8_t a = {w, w, w, w, w, w, w, w};
  for (int r = 0; r < reps; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[i], 0, 0, 0, 127, 0, 127);
  }
  float s = acc[0][0];
#pragma unroll
  for (int i = 1; i < 8; ++i) s += acc[i][0] * 0.0f;
  out[blockIdx.x * kCeilMfmaThreads + threadIdx.x] = s;
}

// Round j of workgroup b reads src + base(b) + (j mod period) * 64 KiB; wave w, load i of a
// round fetches the round's 1 KiB block i * 8 + w into the same place of the stage.
__global__ __launch_bounds__(kCeilFillThreads) void ceil_fill_kernel(const char* __restrict__ src, int64_t share,
                                                                     int rounds, int resident, int32_t* out) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const char* base = resident ? src + int64_t(blockIdx.x & 15) * kCeilRound : src + int64_t(blockIdx.x) * share;
  const int period = resident ? 1 : int(share / kCeilRound);
  for (int j = 0; j < rounds; ++j) {
    const char* rb = base + int64_t(j % period) * kCeilRound;
    char* st = smem + (j & 1) * kCeilRound;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int blk = i * 8 + wave;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(rb + blk * 1024 + lane * 16),
                                       (ceil_lds_ptr)(st + blk * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const char* last = smem + ((rounds - 1) & 1) * kCeilRound;
  out[blockIdx.x * kCeilFillThreads + tid] = reinterpret_cast<const int32_t*>(last)[tid];
}

}  // namespace moe

using namespace moe;

namespace {
int ceil_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}
}  // namespace

extern "C" size_t moe_ceiling_probe_bytes(void) {
  const int cus = ceil_cus();
  return cus > 0 ? size_t(cus) * kCeilFillThreads * 4 : 0;
}

extern "C" int moe_ceiling_probe(int32_t kind, int32_t reps, const void* src, size_t src_bytes, void* scratch,
                                 size_t scratch_bytes, double* work, float* ms, void* stream) {
  if (kind < 0 || kind > 3 || reps < 1 || reps > 1000000 || !scratch || !work || !ms) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(scratch) & 255) return MOE_EALIGN;
  const int cus = ceil_cus();
  if (cus <= 0) return MOE_EHIP;
  if (scratch_bytes < size_t(cus) * kCeilFillThreads * 4) return MOE_ENOSPC;
  int64_t share = 0;
  if (kind >= 2) {
    if (!src) return MOE_EINVAL;
    if (reinterpret_cast<uintptr_t>(src) & 15) return MOE_EALIGN;
    share = int64_t(src_bytes / size_t(cus)) / kCeilRound * kCeilRound;
    if (kind == 2 && share < kCeilRound) return MOE_ENOSPC;
    if (kind == 3 && src_bytes < size_t(16) * kCeilRound) return MOE_ENOSPC;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* fo = static_cast<float*>(scratch);
  int32_t* io = static_cast<int32_t*>(scratch);
  const char* s = static_cast<const char*>(src);
  // kind 2 streams every workgroup's share `reps` times over; kind 3 re-reads its window
  // 16 times per rep, so that both move enough bytes to time
  const int rounds = kind == 2 ? int(std::min<int64_t>(int64_t(reps) * (share / kCeilRound), 1 << 30))
                               : (kind == 3 ? reps * 16 : 0);
  auto launch = [&]() {
    if (kind == 0)
      hipLaunchKernelGGL(ceil_mfma_bf16_kernel, dim3(cus), dim3(kCeilMfmaThreads), 0, st, reps, 0x3F803F80u, fo);
    else if (kind == 1)
      hipLaunchKernelGGL(ceil_mfma_mx_kernel, dim3(cus), dim3(kCeilMfmaThreads), 0, st, reps, 0x38383838u, fo);
    else
      hipLaunchKernelGGL(ceil_fill_kernel, dim3(cus), dim3(kCeilFillThreads), 2 * kCeilRound, st, s, share, rounds,
                         kind == 3 ? 1 : 0, io);
    return hipGetLastError();
  };
  if (kind >= 2 && hipFuncSetAttribute(reinterpret_cast<const void*>(ceil_fill_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kCeilRound) != hipSuccess)
    return MOE_EHIP;
  hipError_t e = launch();                  // warm-up (clocks, code load)
  hipEvent_t e0, e1;
  if (e != hipSuccess || hipEventCreate(&e0) != hipSuccess) return MOE_EHIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return MOE_EHIP;
  }
  e = hipEventRecord(e0, st);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float t = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return MOE_EHIP;
  const double waves = double(cus) * (kCeilMfmaThreads / 64);
  if (kind == 0) *work = waves * reps * 8 * (32.0 * 32 * 16 * 2);
  else if (kind == 1) *work = waves * reps * 8 * (32.0 * 32 * 64 * 2);
  else *work = double(cus) * double(rounds) * kCeilRound;
  *ms = t;
  return MOE_OK;
}
