// Persistent forward for gfx950: pull dispatch, grouped SwiGLU FFN and push combine in
// one kernel, with the CUs split into a data-movement partition and a compute partition
// that signal each other through device-resident counters and a fixed ring of slots.
//
// Operation (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 02: one megakernel whose SMs are split between communication and expert
// compute, GPU-local counters in both directions, tokens released a minibatch at a time,
// and a fixed-size ring token buffer reused right after combine so the combine of one
// macrobatch overlaps the dispatch of the next; qubstore.ru "Смесь котят ...", ring buffer
// and megakernel paragraphs: no CPU in the loop, a buffer of a few hundred MB instead of
// worst-case staging).
//
// MI355X design:
// * Pipelines per XCD.  The eight XCDs' L2 caches are not coherent with one another, and
//   an agent-scope release/acquire on gfx950 writes back / invalidates the whole L2
//   (buffer_wbl2 / buffer_inv sc1).  The row tiles are therefore split into P contiguous
//   ranges, one pipeline per XCD (workgroup w runs on XCD w mod 8; the kernel reads the
//   XCC id from the hardware), each with its own ring partition and counters.  Every
//   producer -> consumer hand-off then stays inside one L2: the producer waits for its
//   stores (vmcnt 0) and bumps a counter atomically; the consumer polls the counter and
//   invalidates its CU's L1 (buffer_inv sc0).  When the ring is too small for eight
//   partitions, pipelines span XCDs and every hand-off uses agent-scope release/acquire.
// * Roles.  The first comm_per_part workgroups of a pipeline move data: they claim, in
//   order, the next chunk whose ring slot is free (gather its rows from the source
//   buffers) or the next row tile whose down GEMM is complete (push its rows to recv and
//   free its slots), never blocking while holding a claim.  The others take GEMM tasks
//   from the pipeline's ticket: for each 256-row tile, its gate/up tiles, then its down
//   tiles.  A gate/up tile waits for its chunks; a down tile waits for all gate/up tiles of
//   its row tile and writes its output in place over the ring rows it no longer needs.
// * Ring.  A slot holds one chunk (1 << blk_log2 rows) of token rows (later the expert
//   output) plus its h rows.  Chunk q of a pipeline uses slot q mod S_p; it may be
//   gathered once the chunk S_p before it has been pushed.  S_p >= chunks per row tile
//   makes progress certain: the chunks a task waits for never wait on that task.
// * Watchdog.  Every wait is bounded by a wall-clock budget; on expiry the workgroup sets
//   the status word (MOE_ETIMEOUT) and an abort flag that every loop checks, so all
//   workgroups exit.
#include "gemm_tile.hpp"

namespace moe {

// control block (int32 words, zeroed by persist_init_kernel before every launch)
enum PersistCtrl {
  kPcAbort = 0,
  kPcPipe = 16,          // 8 words per pipeline: join, gather_next, combine_next, task_next
  kPcPipeStride = 8,
  kPcArrays = 128,       // then: filled[chunks], g1_done[mtiles], g2_done[mtiles], slot_epoch[slots]
};

struct PersistArgs {
  RankPtrs<const char*> x;
  RankPtrs<char*> recv;
  const int32_t* pull_src;
  const int32_t* slot_of;
  const int32_t* offsets;
  const int32_t* mtile_base;
  const int32_t* ctrl;          // layout control words (row tiles)
  const uint16_t* w1;
  const uint16_t* w3;
  const uint16_t* w2;
  char* ring;
  int32_t* pc;                  // persistent control block
  int32_t* ws_status;           // the workspace status word: a watchdog expiry writes MOE_ETIMEOUT
  long long slot_bytes;
  long long budget;             // wall-clock ticks per wait
  int T, k, d, F, El;
  int blk_log2, cpm;            // chunk rows (log2) and chunks per 256-row tile
  int n_part, light;            // pipelines; 1 = every pipeline on one XCD
  int comm_per_part;
  int slots_per_part;
  int max_mtiles;
  int lookahead;                // 1: gate/up tiles of row tile i+1 go before the down tiles of i
};

__device__ __forceinline__ int ld_relaxed(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Producer side: every thread's stores have reached the L2 before thread 0 bumps `ctr`.
__device__ __forceinline__ void release_add(int32_t* ctr, int v, bool light) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (light) __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Consumer side, after thread 0 observed the counter: make the producer's data visible.
__device__ __forceinline__ void acquire_after_poll(bool light) {
  if (light) {
    asm volatile("buffer_inv sc0" ::: "memory");      // this CU's L1; the L2 is shared
  } else {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
}

// Thread 0 waits until *p >= target (or abort / watchdog); returns false on abort.
// Block-uniform result via LDS.
__device__ bool wait_ge(const int32_t* p, int target, const PersistArgs& A, int* sh_flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (ld_relaxed(p) < target) {
      const long long t0 = wall_clock64();
      while (ld_relaxed(p) < target) {
        if (ld_relaxed(A.pc + kPcAbort)) { ok = 0; break; }
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > A.budget) {
          __hip_atomic_store(A.ws_status, MOE_ETIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(A.pc + kPcAbort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
      }
    }
    *sh_flag = ok;
  }
  __syncthreads();
  const bool ok = *sh_flag;
  __syncthreads();
  return ok;
}

// 16-byte row copy by one wave
__device__ __forceinline__ void wave_copy_row(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int n16,
                                              int lane) {
  for (int base = 0; base < n16; base += 64 * 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 64 + lane;
      if (i < n16) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 64 + lane;
      if (i < n16) dst[i] = v[u];
    }
  }
}

__global__ void persist_init_kernel(int32_t* pc, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) pc[i] = 0;
}

__global__ __launch_bounds__(kGemmThreads, 1) void moe_persistent_kernel(PersistArgs A) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int sh[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const int p = int(xcc & 7) * A.n_part / 8;
  const bool light = A.light;
  int32_t* pipe = A.pc + kPcPipe + p * kPcPipeStride;
  int32_t* filled = A.pc + kPcArrays;
  int32_t* g1_done = filled + A.max_mtiles * 4;
  int32_t* g2_done = g1_done + A.max_mtiles;
  int32_t* slot_epoch = g2_done + A.max_mtiles;

  if (tid == 0) sh[0] = __hip_atomic_fetch_add(pipe + 0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int rank = sh[0];
  __syncthreads();

  // this pipeline's row tiles [m_lo, m_hi)
  const int n_mt = A.ctrl[kCtrlMTiles];
  const int per = (n_mt + A.n_part - 1) / A.n_part;
  const int m_lo = min(n_mt, p * per), m_hi = min(n_mt, m_lo + per);
  const int n_m = m_hi - m_lo;
  const int n_chunks = n_m * A.cpm;
  const int S = A.slots_per_part;
  const int NT1 = (A.F + kGemmBN / 2 - 1) / (kGemmBN / 2);
  const int NT2 = (A.d + kGemmBN - 1) / kGemmBN;
  const int chunk_rows = 1 << A.blk_log2;
  const int row_bytes = A.d * 2;
  const int n16 = row_bytes >> 4;
  const long long xpart = (long long)chunk_rows * A.d * 2;   // token/output rows of a slot

  auto slot_ptr = [&](int q) -> char* {                       // pipeline-local chunk q
    return A.ring + (long long)(p * S + q % S) * A.slot_bytes;
  };
  auto tile_rows = [&](int m, int* row0, int* l) -> int {     // global row tile m
    *l = find_expert(A.mtile_base, A.El, m);
    *row0 = A.offsets[*l] + (m - A.mtile_base[*l]) * kGemmBM;
    return min(kGemmBM, A.offsets[*l + 1] - *row0);
  };

  if (rank < A.comm_per_part) {
    // ------------------------------------------------------------ data movement
    long long idle_since = wall_clock64();
    while (true) {
      if (tid == 0) {
        int act = 0, arg = 0;      // 1 = combine row tile arg, 2 = gather chunk arg, 3 = done, 4 = abort
        if (ld_relaxed(A.pc + kPcAbort)) act = 4;
        const int ci = ld_relaxed(pipe + 2);
        if (!act && ci < n_m && ld_relaxed(g2_done + m_lo + ci) == NT2) {
          if (atomicCAS(pipe + 2, ci, ci + 1) == ci) { act = 1; arg = ci; }
        }
        const int qi = ld_relaxed(pipe + 1);
        if (!act && qi < n_chunks && ld_relaxed(slot_epoch + p * S + qi % S) >= qi / S) {
          if (atomicCAS(pipe + 1, qi, qi + 1) == qi) { act = 2; arg = qi; }
        }
        if (!act && ci >= n_m && qi >= n_chunks) act = 3;
        if (!act) {
          __builtin_amdgcn_s_sleep(1);
          if (wall_clock64() - idle_since > A.budget) {
            __hip_atomic_store(A.ws_status, MOE_ETIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(A.pc + kPcAbort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            act = 4;
          }
        } else {
          idle_since = wall_clock64();
        }
        sh[1] = act;
        sh[2] = arg;
      }
      __syncthreads();
      const int act = sh[1], arg = sh[2];
      __syncthreads();
      if (act >= 3) break;
      if (act == 0) continue;          // nothing claimable this round
      if (act == 1) {
        // push combine of row tile m_lo + arg: output rows (in place in the ring) -> recv
        acquire_after_poll(light);
        int row0, l;
        const int m = m_lo + arg;
        const int rows = tile_rows(m, &row0, &l);
        for (int r = wave; r < rows; r += kGemmThreads / 64) {
          const int s = row0 + r;
          const int rk = A.pull_src[2 * (long long)s];
          const int t = A.pull_src[2 * (long long)s + 1];
          const int32_t* so = A.slot_of + ((long long)rk * A.T + t) * A.k;
          int j = 0;
          for (int jj = 0; jj < A.k; ++jj)
            if (so[jj] == s) j = jj;
          const char* src = slot_ptr(arg * A.cpm + (r >> A.blk_log2)) + (long long)(r & (chunk_rows - 1)) * row_bytes;
          wave_copy_row(reinterpret_cast<const u32x4*>(src),
                        reinterpret_cast<u32x4*>(A.recv.p[rk] + ((long long)t * A.k + j) * row_bytes), n16, lane);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
          for (int h = 0; h < A.cpm; ++h) {
            const int q = arg * A.cpm + h;
            if (light) __hip_atomic_fetch_add(slot_epoch + p * S + q % S, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else __hip_atomic_fetch_add(slot_epoch + p * S + q % S, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
          }
      } else {  // act == 2
        // gather chunk arg: its rows of the row tile, pulled from the source buffers
        if (!light) acquire_after_poll(light);
        int row0, l;
        const int m = m_lo + arg / A.cpm, h = arg % A.cpm;
        const int rows = tile_rows(m, &row0, &l);
        const int c_lo = h * chunk_rows, c_n = min(chunk_rows, rows - c_lo);
        char* dst = slot_ptr(arg);
        for (int r = wave; r < c_n; r += kGemmThreads / 64) {
          const int s = row0 + c_lo + r;
          const int rk = A.pull_src[2 * (long long)s];
          const int t = A.pull_src[2 * (long long)s + 1];
          wave_copy_row(reinterpret_cast<const u32x4*>(A.x.p[rk] + (long long)t * row_bytes),
                        reinterpret_cast<u32x4*>(dst + (long long)r * row_bytes), n16, lane);
        }
        release_add(filled + m * A.cpm + h, 1, light);
      }
    }
  } else {
    // ------------------------------------------------------------ expert compute
    const int n_tasks = n_m * (NT1 + NT2);
    while (true) {
      if (tid == 0) sh[3] = __hip_atomic_fetch_add(pipe + 3, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int task = sh[3];
      __syncthreads();
      if (task >= n_tasks) break;
      // task -> (row tile i, j < NT1: gate/up tile j, else down tile j - NT1)
      int i, j;
      if (!A.lookahead) {
        i = task / (NT1 + NT2);
        j = task % (NT1 + NT2);
      } else if (task < NT1) {
        i = 0;
        j = task;
      } else {
        const int u = task - NT1, b = u / (NT1 + NT2), r = u % (NT1 + NT2);
        if (b < n_m - 1 && r < NT1) { i = b + 1; j = r; }      // gate/up of the next row tile
        else if (b < n_m - 1) { i = b; j = r; }                 // down of this row tile (r >= NT1)
        else { i = b; j = NT1 + r; }                            // last block: down tiles only
      }
      const int m = m_lo + i;
      int row0, l;
      const int rows = tile_rows(m, &row0, &l);
      bool ok = true;
      if (j < NT1) {
        for (int h = 0; h < A.cpm && ok; ++h) ok = wait_ge(filled + m * A.cpm + h, 1, A, sh);
      } else {
        ok = wait_ge(g1_done + m, NT1, A, sh);
      }
      if (!ok) break;
      acquire_after_poll(light);
      char* s0 = slot_ptr(i * A.cpm + 0);
      char* s1 = slot_ptr(i * A.cpm + min(1, A.cpm - 1));
      char* s2 = slot_ptr(i * A.cpm + min(2, A.cpm - 1));
      char* s3 = slot_ptr(i * A.cpm + min(3, A.cpm - 1));
      TileIO io;
      io.blk_log2 = A.blk_log2;
      io.rows = rows;
      io.row_dst = nullptr;
      io.row_src = nullptr;
      if (j < NT1) {
        io.a0 = reinterpret_cast<const uint16_t*>(s0);
        io.a1 = reinterpret_cast<const uint16_t*>(s1);
        io.a2 = reinterpret_cast<const uint16_t*>(s2);
        io.a3 = reinterpret_cast<const uint16_t*>(s3);
        io.o0 = reinterpret_cast<uint16_t*>(s0 + xpart);
        io.o1 = reinterpret_cast<uint16_t*>(s1 + xpart);
        io.o2 = reinterpret_cast<uint16_t*>(s2 + xpart);
        io.o3 = reinterpret_cast<uint16_t*>(s3 + xpart);
        io.a_ld = A.d;
        io.o_ld = A.F;
        const uint16_t* b0 = A.w1 + size_t(l) * A.F * A.d;
        const uint16_t* b1 = A.w3 + size_t(l) * A.F * A.d;
        gemm_tile<0>(io, b0, b1, j * (kGemmBN / 2), A.F, A.d, smem, A.d);
        release_add(g1_done + m, 1, light);
      } else {
        io.a0 = reinterpret_cast<const uint16_t*>(s0 + xpart);
        io.a1 = reinterpret_cast<const uint16_t*>(s1 + xpart);
        io.a2 = reinterpret_cast<const uint16_t*>(s2 + xpart);
        io.a3 = reinterpret_cast<const uint16_t*>(s3 + xpart);
        io.o0 = reinterpret_cast<uint16_t*>(s0);
        io.o1 = reinterpret_cast<uint16_t*>(s1);
        io.o2 = reinterpret_cast<uint16_t*>(s2);
        io.o3 = reinterpret_cast<uint16_t*>(s3);
        io.a_ld = A.F;
        io.o_ld = A.d;
        const uint16_t* b0 = A.w2 + size_t(l) * A.d * A.F;
        gemm_tile<1>(io, b0, b0, (j - NT1) * kGemmBN, A.d, A.F, smem, A.F);
        release_add(g2_done + m, 1, light);
      }
    }
  }
}

// ---------------------------------------------------------------------------- host side
int persist_ctrl_words(int max_mtiles, int slots) { return kPcArrays + max_mtiles * 6 + slots; }
int persist_ctrl_bytes(int max_mtiles) { return persist_ctrl_words(max_mtiles, kMaxRingSlots) * 4; }

hipError_t launch_persistent(const moe_shape_t& s, int El, const void* const* x, const void* w1, const void* w3,
                             const void* w2, const int32_t* pull_src, const int32_t* slot_of,
                             const int32_t* offsets, char* ring, long long slot_bytes, int slots, int blk_log2,
                             int comm_cus, int n_part, int cus, long long budget, void* const* recv, char* ws,
                             const WsLayout& L, hipStream_t st) {
  int32_t* pc = reinterpret_cast<int32_t*>(ws + L.pctrl);
  PersistArgs A{};
  for (int r = 0; r < s.R; ++r) {
    A.x.p[r] = static_cast<const char*>(x[r]);
    A.recv.p[r] = static_cast<char*>(recv[r]);
  }
  A.pull_src = pull_src;
  A.slot_of = slot_of;
  A.offsets = offsets;
  A.mtile_base = reinterpret_cast<const int32_t*>(ws + L.mtile_base);
  A.ctrl = reinterpret_cast<const int32_t*>(ws + L.ctrl);
  A.ws_status = reinterpret_cast<int32_t*>(ws + L.ctrl) + kCtrlStatus;
  A.w1 = static_cast<const uint16_t*>(w1);
  A.w3 = static_cast<const uint16_t*>(w3);
  A.w2 = static_cast<const uint16_t*>(w2);
  A.ring = ring;
  A.pc = pc;
  A.slot_bytes = slot_bytes;
  A.budget = budget;
  A.T = s.T;
  A.k = s.k;
  A.d = s.d;
  A.F = s.F;
  A.El = El;
  A.blk_log2 = blk_log2;
  A.cpm = kGemmBM >> blk_log2;
  A.n_part = n_part;
  A.light = (n_part == 8) ? 1 : 0;
  A.comm_per_part = comm_cus / n_part;
  A.slots_per_part = slots / n_part;
  A.max_mtiles = L.max_mtiles;
  A.lookahead = (A.slots_per_part >= 2 * A.cpm) ? 1 : 0;

  static std::atomic<uint64_t> attr_set{0};
  const hipError_t ea = once_per_device(attr_set, [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(moe_persistent_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
  });
  if (ea != hipSuccess) return ea;
  const int words = persist_ctrl_words(L.max_mtiles, slots);
  hipLaunchKernelGGL(persist_init_kernel, dim3((words + 255) / 256), dim3(256), 0, st, pc, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void* args[] = {&A};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(moe_persistent_kernel), dim3(cus),
                                    dim3(kGemmThreads), args, kGemmLds, st);
}

}  // namespace moe
