// Inter-partition signal latency on one GPU.
//
// The pages compare how long the receiving side of a transfer waits for the signal that its
// data is complete: after a push the destination collects completion signals from every
// peer, after a pull it only observes its own reads (MoK article, kucoin.com/es "Cursor's MoK
// logra un aumento del 2.37x ...", section 02, the push/pull comparison and its multi-node
// signalling microbenchmark).  On one MI355X the analogue is the hand-off between two
// workgroups through device memory: a producer writes a payload, makes it visible and bumps a
// flag; the consumer observes the flag, reads the payload and acknowledges.  The round trip
// depends on where the two workgroups run (one XCD shares an L2; different XCDs do not) and
// on the visibility protocol:
//   scope 0 (L2-local): producer stores, waits for them (vmcnt 0), relaxed flag store; the
//     consumer polls the flag and invalidates its CU's L1 (buffer_inv sc1; the workgroup-scope
//     buffer_inv sc0 leaves L1 lines of earlier rounds in place, which a payload smaller than
//     the L1 exposes) before reading.  Sufficient when both sides share one L2; across XCDs the
//     payload may be stale.
//   scope 1 (agent): release store of the flag / acquire load, which on gfx950 write back and
//     invalidate the XCD's L2 (buffer_wbl2 sc1 / buffer_inv sc1).  Correct anywhere.
//   scope 2: as scope 0 with a workgroup-scope invalidate (buffer_inv sc0) instead -- kept to
//     show that it is not enough: it leaves the consumer CU's L1 lines in place, so a payload
//     that fits the L1 reads stale from the second round on.
//   scope 3: as scope 0 without any invalidate, the payload read with device-coherent sc1
//     loads (no L1 hit) -- the form the persistent kernel's same-XCD hand-offs use.
// Every pair runs `rounds` hand-offs; the consumer counts payload words that do not hold the
// round's values.  Every wait is bounded by a wall-clock budget.
#include "common.hpp"

namespace moe {

constexpr int kProbeWGs = 256;      // 128 producer/consumer pairs
constexpr int kProbeThreads = 256;

struct ProbeArgs {
  int* data;         // [pairs][payload_words]
  int* flag;         // [pairs]
  int* ack;          // [pairs]
  int* xcc_of;       // [kProbeWGs]
  int* counters;     // [0] stale words, [1] timeouts
  int payload, rounds, cross;
  long long budget;  // wall-clock ticks per wait
};

template <int SCOPE>
__global__ __launch_bounds__(kProbeThreads) void signal_probe_kernel(ProbeArgs A) {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  const int w = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) A.xcc_of[w] = int(x & 7);
  // workgroup w runs on XCD w mod 8: partner w ^ 8 shares the XCD, w ^ 1 does not.  The
  // lower of the two produces; pairs are numbered 0..127 by their producer.
  const int partner = A.cross ? (w ^ 1) : (w ^ 8);
  const bool producer = w < partner;
  const int pw = producer ? w : partner;
  const int cpair = A.cross ? (pw >> 1) : ((pw & 7) | ((pw >> 4) << 3));
  int* buf = A.data + size_t(cpair) * A.payload;
  __shared__ int bad, stop;
  if (tid == 0) {
    bad = 0;
    stop = 0;
  }
  __syncthreads();
  for (int r = 1; r <= A.rounds; ++r) {
    int* wait_on = producer ? &A.ack[cpair] : &A.flag[cpair];
    const int target = producer ? r - 1 : r;
    if (tid == 0) {
      const long long t0 = wall_clock64();
      while (__hip_atomic_load(wait_on, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > A.budget) {
          stop = 1;
          atomicAdd(&A.counters[1], 1);
          break;
        }
      }
      if (SCOPE == 1) __hip_atomic_load(wait_on, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (stop) break;
    if (producer) {
      for (int i = tid; i < A.payload; i += kProbeThreads) buf[i] = r * 1000003 + i;
    } else {
      if (SCOPE == 0) asm volatile("buffer_inv sc1" ::: "memory");
      if (SCOPE == 2) asm volatile("buffer_inv sc0" ::: "memory");
      int e = 0;
      if (SCOPE == 3) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(buf, (short)0, A.payload * 4, 0x00020000);
        for (int i = tid; i < A.payload; i += kProbeThreads)
          e += __builtin_amdgcn_raw_buffer_load_b32(rs, i * 4, 0, 16) != uint32_t(r * 1000003 + i);
      } else {
        for (int i = tid; i < A.payload; i += kProbeThreads) e += buf[i] != r * 1000003 + i;
      }
      if (e) atomicAdd(&bad, e);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      int* sig = producer ? &A.flag[cpair] : &A.ack[cpair];
      if (SCOPE != 1) __hip_atomic_store(sig, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else __hip_atomic_store(sig, r, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (tid == 0 && bad) atomicAdd(&A.counters[0], bad);
}

__global__ void probe_clear_kernel(int* p, size_t words) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < words; i += size_t(gridDim.x) * blockDim.x)
    p[i] = 0;
}

size_t probe_layout(int payload, size_t* data, size_t* flag, size_t* ack, size_t* xcc, size_t* counters) {
  size_t o = 0;
  *data = o;     o = align256(o + size_t(kProbeWGs / 2) * payload * 4);
  *flag = o;     o = align256(o + size_t(kProbeWGs / 2) * 4);
  *ack = o;      o = align256(o + size_t(kProbeWGs / 2) * 4);
  *xcc = o;      o = align256(o + size_t(kProbeWGs) * 4);
  *counters = o; o = align256(o + 64);
  return o;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_signal_probe_bytes(int32_t payload_words) {
  if (payload_words < 0 || payload_words > (1 << 20)) return 0;
  size_t a, b, c, d, e;
  return probe_layout(payload_words, &a, &b, &c, &d, &e);
}

extern "C" int moe_signal_probe(int32_t cross_xcd, int32_t scope, int32_t payload_words, int32_t rounds,
                                void* scratch, size_t scratch_bytes, float* us_per_round, int32_t* stale_words,
                                int32_t* timeouts, int32_t* pairs_same_xcd, void* stream) {
  if ((cross_xcd != 0 && cross_xcd != 1) || scope < 0 || scope > 3) return MOE_EINVAL;
  if (payload_words < 0 || payload_words > (1 << 20) || rounds < 1 || rounds > 100000) return MOE_EINVAL;
  if (!scratch || !us_per_round || !stale_words || !timeouts || !pairs_same_xcd) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(scratch) & 255) return MOE_EALIGN;
  size_t o_data, o_flag, o_ack, o_xcc, o_cnt;
  const size_t need = probe_layout(payload_words, &o_data, &o_flag, &o_ack, &o_xcc, &o_cnt);
  if (scratch_bytes < need) return MOE_ENOSPC;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* s = static_cast<char*>(scratch);
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    khz = 100000;
  ProbeArgs A{};
  A.data = reinterpret_cast<int*>(s + o_data);
  A.flag = reinterpret_cast<int*>(s + o_flag);
  A.ack = reinterpret_cast<int*>(s + o_ack);
  A.xcc_of = reinterpret_cast<int*>(s + o_xcc);
  A.counters = reinterpret_cast<int*>(s + o_cnt);
  A.payload = payload_words;
  A.rounds = rounds;
  A.cross = cross_xcd;
  A.budget = static_cast<long long>(khz) * 2000;     // 2 s per wait
  hipLaunchKernelGGL(probe_clear_kernel, dim3(256), dim3(256), 0, st, reinterpret_cast<int*>(s), need / 4);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return MOE_EHIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return MOE_EHIP;
  }
  hipError_t e = hipEventRecord(e0, st);
  if (e == hipSuccess) {
    if (scope == 0)
      hipLaunchKernelGGL(signal_probe_kernel<0>, dim3(kProbeWGs), dim3(kProbeThreads), 0, st, A);
    else if (scope == 1)
      hipLaunchKernelGGL(signal_probe_kernel<1>, dim3(kProbeWGs), dim3(kProbeThreads), 0, st, A);
    else if (scope == 2)
      hipLaunchKernelGGL(signal_probe_kernel<2>, dim3(kProbeWGs), dim3(kProbeThreads), 0, st, A);
    else
      hipLaunchKernelGGL(signal_probe_kernel<3>, dim3(kProbeWGs), dim3(kProbeThreads), 0, st, A);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  int host[2] = {0, 0}, xcc[kProbeWGs];
  if (e == hipSuccess) e = hipMemcpy(host, A.counters, sizeof(host), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(xcc, A.xcc_of, sizeof(xcc), hipMemcpyDeviceToHost);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return MOE_EHIP;
  int same = 0;
  for (int w = 0; w < kProbeWGs; ++w) {
    const int p = cross_xcd ? (w ^ 1) : (w ^ 8);
    if (w < p && xcc[w] == xcc[p]) ++same;
  }
  *us_per_round = ms * 1000.0f / float(rounds);
  *stale_words = host[0];
  *timeouts = host[1];
  *pairs_same_xcd = same;
  return host[1] ? MOE_ETIMEOUT : MOE_OK;
}
