// Persistent forward for gfx950: pull dispatch into a fixed ring, the grouped SwiGLU FFN and
// the push combine in one kernel, with the CUs split into a data-movement partition and a
// compute partition that signal each other through device-resident counters.
//
// Operation (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 02: one megakernel whose SMs are split between communication and expert
// compute, GPU-local counters in both directions, tokens released a minibatch at a time,
// and a fixed-size ring token buffer reused right after combine, so the combine of one
// batch overlaps the dispatch of the next; qubstore.ru "Смесь котят ...", ring buffer and
// megakernel paragraphs: no CPU in the loop, a buffer of a few hundred MB instead of
// worst-case staging).  The scheduling rules (pipelines, groups, ticket order, slot reuse,
// mover claims) are persist_sched.hpp, shared with a host-threaded model of this kernel.
//
// MI355X design:
// * Launch.  An ordinary launch of one 512-thread workgroup per CU with 128 KiB of LDS,
//   132 KiB with MXFP8 weights (the launch shape of the grouped GEMM kernels).  No
//   grid-wide barrier is used, so nothing needs a cooperative launch.  Roles go by
//   arrival order inside a pipeline, so the first workgroups to run are the movers;
//   compute workgroups take tickets in order and a task waits only for movers or smaller
//   tickets, so progress does not depend on every workgroup being resident at once.  A
//   compute workgroup whose pipeline has no ticket left joins the movers, so the last
//   pushes (after the last GEMM) are spread over more CUs.
// * Pipelines per XCD.  The eight XCDs' L2 caches are not coherent with one another, and an
//   agent-scope release/acquire writes back / invalidates a whole L2.  With a ring large
//   enough, the row tiles are split into eight pipelines, one per XCD (the kernel reads the
//   XCC id from the hardware), each with its own ring partition and counters: every
//   producer -> consumer hand-off stays inside one L2 (stores waited for, then a relaxed
//   counter bump, no L2 write-back; the consumer reads the data with device-coherent sc1
//   loads, which bypass its CU's L1).  Otherwise pipelines span XCDs and hand-offs use
//   agent-scope release/acquire (the producer also writes back its XCD's L2, the consumer
//   drops stale lines of its own).
// * Ring slot.  One minibatch (chunk) of token rows, overwritten in place by the expert
//   outputs of those rows, followed by the rows' h.  In MXFP8 the slot holds the rows'
//   E4M3 codes and scale words (quantised by the gather, as the standalone quantising
//   gather does), then h's codes and scale words (quantised by the gate/up GEMM's
//   epilogue); the down GEMM stores each bf16 output row straight to recv.
// * Reverse ring (qubstore.ru, ring buffer paragraph: the forward walks the ring in reverse
//   so that at its end the ring holds the activations the gradients need).  Each pipeline
//   takes its row tiles from last to first: the rules below run on the pipeline's own order
//   (tile index m in [lo, hi)) and only the data addressing maps m to the layout's row tile
//   lo + hi - 1 - m.  The down GEMM then stores each output row straight to its recv slot,
//   so a slot keeps its chunk's token rows and h rows until it is reused, and a push only
//   frees the slot.  The last S chunks of a pipeline's order -- its first chunks in layout
//   order -- are never overwritten; the check kernel records which slot holds each of them.
// * Watchdog.  Every wait is bounded by a wall-clock budget; on expiry the workgroup sets
//   the status word (MOE_ETIMEOUT) and an abort word that every loop checks, so all
//   workgroups exit.  A check kernel afterwards reports MOE_EINCOMPLETE if any pipeline's
//   work was left undone (e.g. a pipeline that received no workgroup).
#include "gemm_mx_tile.hpp"
#include "persist_sched.hpp"

namespace moe {

using sched::CtrlLayout;

struct PersistArgs {
  RankPtrs<const char*> x;
  RankPtrs<char*> recv;
  const int32_t* pull_src;
  const int32_t* slot_of;
  const int32_t* offsets;
  const int32_t* mtile_base;
  const int32_t* ctrl;          // layout control words (row tile count)
  const uint16_t* w1;
  const uint16_t* w3;
  const uint16_t* w2;
  char* ring;
  int32_t* pc;                  // persistent control block
  int32_t* status;              // the workspace status word
  moe_trace_event_t* trace;     // null: no trace
  int32_t* trace_count;
  int trace_cap;
  long long slot_bytes;
  long long budget;             // wall-clock ticks per wait
  int T, k, d, F, El;
  int blk_log2, cpm;            // chunk rows (log2) and chunks per 256-row tile
  int n_part, light, comm_pp, S, G, lookahead;
  int reverse;                  // 1: reverse ring (pipelines walk their row tiles backwards)
  int steal;                    // 1: compute workgroups out of tickets take other pipelines' last down tiles
  int max_mtiles;               // entries of the resident record: 4 per row tile
  const uint64_t* row_dst;      // reverse ring and MXFP8: per local pair, the address of its recv row
  // MXFP8: weight codes and scales (the MXFP8 scale layout over each weight matrix's
  // E_local * rows), and the slot layout: token codes at 0 (row stride d), their scale words
  // at tok_s_off (K-tile planes 4 * chunk rows apart), h codes at h_off (row stride F), h's
  // scale words at h_s_off
  int mx;
  const uint8_t* w1q;
  const uint8_t* w3q;
  const uint8_t* w2q;
  const uint8_t* w1s;
  const uint8_t* w3s;
  const uint8_t* w2s;
  long long tok_s_off, h_off, h_s_off;
  CtrlLayout cl;
};

// Layout row tile of pipeline tile m (the pipeline owns [lo, lo + n_m)).
__device__ __forceinline__ int layout_tile(int reverse, int lo, int n_m, int m) {
  return reverse ? 2 * lo + n_m - 1 - m : m;
}

struct DevOps {
  int32_t* pc;
  __device__ int ld(int w) const { return __hip_atomic_load(pc + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
  __device__ bool cas(int w, int expected, int desired) const {
    return atomicCAS(pc + w, expected, desired) == expected;
  }
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

// A gate/up tile of a row tile another XCD may take down tiles of (work stealing): the light
// hand-off as above, and the tile that completes the row tile (the counter reaches `target`)
// then writes back its XCD's L2 -- every gate/up tile of the row tile ran on this XCD, so
// that one write-back publishes all their h rows -- and adds 1 more, the mark a down tile
// on another XCD waits for (target + 1).
__device__ __forceinline__ void release_add_publish(int32_t* ctr, int target) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == target - 1) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Consumer side, after the workgroup observed the counter: make the producer's data visible.
// Light (same XCD, one L2): nothing to invalidate, because every read of data another CU
// wrote during the kernel (ring rows in the GEMMs' A loads and in the push) is a device-
// coherent sc1 load, which does not hit this CU's L1.  The L1 must be kept out of it: a
// CU that touched a slot's lines earlier (it gathered into the slot, or read its previous
// contents) still holds them, and a workgroup-scope invalidate (buffer_inv sc0) leaves them
// in place (measured on MI355X: a push then copied stale input lines instead of the expert
// output).  Across XCDs: an agent-scope acquire (buffer_inv sc1) also drops the stale lines
// of this XCD's L2.
__device__ __forceinline__ void acquire_after_poll(bool light) {
  if (light) asm volatile("" ::: "memory");
  else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ void set_abort(const PersistArgs& A, int code) {
  __hip_atomic_store(A.status, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(A.pc + A.cl.abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 waits until *p >= target (or abort / watchdog); the result is block-uniform
// (broadcast through LDS).  Every thread of the workgroup calls it.
__device__ bool wait_ge(const int32_t* p, int target, const PersistArgs& A, int* sh_flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (ld_relaxed(p) < target) {
      const long long t0 = wall_clock64();
      while (ld_relaxed(p) < target) {
        if (ld_relaxed(A.pc + A.cl.abort_word)) { ok = 0; break; }
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > A.budget) {
          set_abort(A, MOE_ETIMEOUT);
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

__device__ __forceinline__ void trace_event(const PersistArgs& A, int kind, int idx, int pipe, long long t_begin,
                                            long long t_end, long long t_wait) {
  if (!A.trace || threadIdx.x != 0) return;
  const int i = atomicAdd(A.trace_count, 1);
  if (i >= A.trace_cap) return;
  moe_trace_event_t ev;
  ev.t_begin = t_begin;
  ev.t_end = t_end;
  ev.t_wait = static_cast<int32_t>(t_wait > 0x7fffffffLL ? 0x7fffffffLL : t_wait);
  ev.index = idx;
  ev.workgroup = static_cast<int32_t>(blockIdx.x);
  ev.kind = static_cast<int16_t>(kind);
  ev.pipeline = static_cast<int16_t>(pipe);
  A.trace[i] = ev;
}

typedef __attribute__((address_space(1))) const u32x4* gsrc_t;
typedef __attribute__((address_space(1))) u32x4* gdst_t;

// 16 bytes at vector c of the row at `row` (c < n16).  SC1: a device-coherent load (sc1, no
// L1 hit) through a buffer resource spanning the row.
template <bool SC1>
__device__ __forceinline__ u32x4 row_load(uint64_t row, int c, int n16) {
  if constexpr (SC1) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(row), (short)0, n16 * 16, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, 16);
  } else {
    return reinterpret_cast<gsrc_t>(row)[c];
  }
}

// Copy nrows rows of n16 16-byte vectors from src[r] to dst[r] (row addresses staged in
// LDS) with the whole workgroup.  Each wave moves two rows at a time (r and r + 8), 16
// vectors per lane of each: 32 outstanding 16-byte loads per lane (224 KiB per workgroup
// for 14 KiB rows).  The loads are unconditional (columns past the row end are clamped to
// its last vector; a lone last row reads itself twice) so the compiler issues them back to
// back; only the stores are predicated.  SC1_SRC: sources written by other CUs during the
// kernel (ring rows) are read with device-coherent loads.
template <bool SC1_SRC>
__device__ void wg_copy_rows(const uint64_t* src, const uint64_t* dst, int nrows, int n16) {
  constexpr int U = 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kGemmThreads / 64;
  for (int r = wave; r < nrows; r += 2 * kWaves) {
    const int r2 = r + kWaves;
    const bool two = r2 < nrows;
    const uint64_t s0 = src[r], s1 = src[two ? r2 : r];
    const gdst_t t0 = reinterpret_cast<gdst_t>(dst[r]);
    const gdst_t t1 = reinterpret_cast<gdst_t>(dst[two ? r2 : r]);
    for (int c0 = 0; c0 < n16; c0 += 64 * U) {
      u32x4 a[U], b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(c0 + u * 64 + lane, n16 - 1);
        a[u] = row_load<SC1_SRC>(s0, c, n16);
        b[u] = row_load<SC1_SRC>(s1, c, n16);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < n16) {
          t0[c] = a[u];
          if (two) t1[c] = b[u];
        }
      }
    }
  }
}

// Zero the control block and build every pipeline's group and phase tables (one block; the
// per-expert row-tile prefix is staged in LDS first, so the group walk reads no global memory).
// The local expert of every row tile is looked up by all threads at once (when the tiles
// fit in LDS), so the per-pipeline threads that build the groups read it with one LDS load
// instead of each running a binary search per tile.
constexpr int kPrepLdsTiles = 8192;

__global__ __launch_bounds__(1024) void persist_prep_kernel(PersistArgs A, int zero_words) {
  __shared__ int32_t mtb[1025];                 // E_local <= E <= 1024
  __shared__ int16_t s_exp[kPrepLdsTiles];      // local expert of row tile m (E_local <= 1024)
  for (int i = threadIdx.x; i < zero_words; i += blockDim.x) A.pc[i] = 0;
  for (int i = threadIdx.x; i <= A.El; i += blockDim.x) mtb[i] = A.mtile_base[i];
  if (A.trace && threadIdx.x == 0) *A.trace_count = 0;
  const int n_mt = A.ctrl[kCtrlMTiles];
  const bool in_lds = n_mt <= kPrepLdsTiles;
  __syncthreads();
  if (in_lds)
    for (int m = threadIdx.x; m < n_mt; m += blockDim.x) s_exp[m] = int16_t(find_expert(mtb, A.El, m));
  __syncthreads();
  const int p = threadIdx.x;
  if (p >= A.n_part) return;
  int lo, hi;
  sched::pipe_range(n_mt, A.n_part, p, &lo, &hi);
  int32_t* gf = A.pc + A.cl.grp_first + lo;
  int32_t* gl = A.pc + A.cl.grp_len + lo;
  const int El = A.El;
  const int rev = A.reverse, n_m = hi - lo;
  const int n = sched::build_groups(
      lo, hi, A.G,
      [&](int m) {
        const int ml = layout_tile(rev, lo, n_m, m);
        return in_lds ? int(s_exp[ml]) : find_expert(mtb, El, ml);
      },
      gf, gl);
  const int NT1 = (A.F + kGemmBN / 2 - 1) / (kGemmBN / 2);
  const int NT2 = (A.d + kGemmBN - 1) / kGemmBN;
  const int tickets = n ? sched::build_phases(n, gl, NT1, NT2, A.lookahead != 0, A.pc + A.cl.phase_start + 2 * lo + p)
                        : 0;
  int32_t* pw = A.pc + A.cl.pipe0 + p * sched::kPipeWords;
  pw[sched::kNGroups] = n;
  pw[sched::kNTickets] = tickets;
  pw[sched::kLo] = lo;
  pw[sched::kHi] = hi;
}

// After the persistent kernel: every pipeline must have claimed all its gathers, pushes and
// tickets; otherwise (and unless a watchdog already reported) MOE_EINCOMPLETE.  Then the
// record of the chunks the ring still holds (reverse ring only, and only after a clean run:
// pipeline p's last S chunks in its order, each in slot q mod S, never overwritten).  One
// block of 1024 threads; the first wave holds one thread per pipeline.
__global__ __launch_bounds__(1024) void persist_check_kernel(PersistArgs A) {
  const int p = threadIdx.x;
  bool bad = false;
  if (p < A.n_part) {
    const int32_t* pw = A.pc + A.cl.pipe0 + p * sched::kPipeWords;
    const int n_m = pw[sched::kHi] - pw[sched::kLo];
    bad = pw[sched::kGatherNext] < n_m * A.cpm || pw[sched::kPushNext] < n_m * A.cpm ||
          pw[sched::kTicketNext] < pw[sched::kNTickets];
  }
  const bool any_bad = __any(bad);              // pipelines <= 8: all in wave 0
  if (any_bad && threadIdx.x == 0 && *A.status == MOE_OK) *A.status = MOE_EINCOMPLETE;
  int32_t* res = A.pc + A.cl.resident;
  for (int i = threadIdx.x; i < A.max_mtiles * 4; i += blockDim.x) res[i] = 0;
  __syncthreads();
  if (!A.reverse || any_bad || *A.status != MOE_OK || p >= A.n_part) return;
  const int32_t* pw = A.pc + A.cl.pipe0 + p * sched::kPipeWords;
  const int lo = pw[sched::kLo], n_m = pw[sched::kHi] - lo;
  const int n_chunks = n_m * A.cpm;
  for (int q = max(0, n_chunks - A.S); q < n_chunks; ++q) {
    const int m = layout_tile(1, lo, n_m, lo + q / A.cpm);
    res[m * 4 + q % A.cpm] = 1 + p * A.S + sched::chunk_slot(q, A.S);
  }
}

// One workgroup's view of its pipeline.
struct PipeCtx {
  int p, lo, n_m, S, cpm, chunk_rows, row_bytes, n16, NT2;
  bool light, reverse;
};

__device__ __forceinline__ char* slot_ptr(const PersistArgs& A, const PipeCtx& c, int q) {   // pipeline-local chunk q
  return A.ring + (long long)(c.p * c.S + sched::chunk_slot(q, c.S)) * A.slot_bytes;
}

__device__ __forceinline__ int tile_rows(const PersistArgs& A, int m, int* row0, int* l) {    // global row tile m
  *l = find_expert(A.mtile_base, A.El, m);
  *row0 = A.offsets[*l] + (m - A.mtile_base[*l]) * kGemmBM;
  return min(kGemmBM, A.offsets[*l + 1] - *row0);
}

// Gather pipeline-local chunk q (rows of row tile lo + q / cpm) from the source buffers into
// its slot, then signal it (whole workgroup; the row tables live in LDS).
__device__ void do_gather(const PersistArgs& A, const PipeCtx& c, int q, char* smem) {
  uint64_t* src_tab = reinterpret_cast<uint64_t*>(smem);
  uint64_t* dst_tab = src_tab + kGemmBM;
  int row0, l;
  const int m = c.lo + q / c.cpm, h = q % c.cpm;
  const int rows = tile_rows(A, layout_tile(c.reverse, c.lo, c.n_m, m), &row0, &l);
  const int c_lo = h * c.chunk_rows, c_n = min(c.chunk_rows, rows - c_lo);
  char* dst = slot_ptr(A, c, q);
  for (int r = threadIdx.x; r < c_n; r += kGemmThreads) {
    const int s = row0 + c_lo + r;
    const int rk = A.pull_src[2 * (long long)s];
    const int t = A.pull_src[2 * (long long)s + 1];
    src_tab[r] = reinterpret_cast<uint64_t>(A.x.p[rk] + (long long)t * c.row_bytes);
    dst_tab[r] = reinterpret_cast<uint64_t>(dst + (long long)r * c.row_bytes);
  }
  __syncthreads();
  if (c_n > 0) wg_copy_rows<false>(src_tab, dst_tab, c_n, c.n16);   // the sources never change
  release_add(A.pc + A.cl.filled + m * 4 + h, 1, c.light);
  __syncthreads();                                              // the row tables are reused
}

// MXFP8: gather chunk q's rows quantised on the way (E4M3 codes at row stride d; the scale
// word of row r in K-tile plane p at tok_s_off + p * 4 * chunk_rows + 4 * r), then signal it.
// One wave per row, 8 of the row's 16-byte vectors per lane at a time; every lane of the wave
// takes part in the quantiser's shuffles (lanes past the row end carry zeros).
__device__ void do_gather_mx(const PersistArgs& A, const PipeCtx& c, int q, char* smem) {
  uint64_t* src_tab = reinterpret_cast<uint64_t*>(smem);
  int row0, l;
  const int m = c.lo + q / c.cpm, h = q % c.cpm;
  const int rows = tile_rows(A, layout_tile(c.reverse, c.lo, c.n_m, m), &row0, &l);
  const int c_lo = h * c.chunk_rows, c_n = min(c.chunk_rows, rows - c_lo);
  char* dst = slot_ptr(A, c, q);
  for (int r = threadIdx.x; r < c_n; r += kGemmThreads) {
    const int s = row0 + c_lo + r;
    const int rk = A.pull_src[2 * (long long)s];
    const int t = A.pull_src[2 * (long long)s + 1];
    src_tab[r] = reinterpret_cast<uint64_t>(A.x.p[rk] + (long long)t * A.d * 2);
  }
  __syncthreads();
  constexpr int U = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = A.d >> 3;                        // d % 128 == 0: whole 16-lane groups
  const long long splane = 4LL * c.chunk_rows;
  for (int r = wave; r < c_n; r += kGemmThreads / 64) {
    const u32x4* src = reinterpret_cast<const u32x4*>(src_tab[r]);    // the sources never change
    uint2* code = reinterpret_cast<uint2*>(dst + (long long)r * A.d);
    char* sw0 = dst + A.tok_s_off + 4LL * r;
    for (int base = 0; base < n16; base += 64 * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * 64 + lane;
        v[u] = u32x4{0, 0, 0, 0};
        if (i < n16) v[u] = src[i];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * 64 + lane;
        uint32_t sc;
        const uint2 qv = mx_quant8_bf16(v[u], &sc);     // all lanes: quad shuffles inside
        const uint32_t sw = mx_scale_word(sc);            // all lanes: row shifts inside
        if (i < n16) {
          code[i] = qv;
          if ((i & 15) == 0) *reinterpret_cast<uint32_t*>(sw0 + (i >> 4) * splane) = sw;
        }
      }
    }
  }
  release_add(A.pc + A.cl.filled + m * 4 + h, 1, c.light);
  __syncthreads();                                              // the row table is reused
}

template <bool MX>
__device__ __forceinline__ void gather_chunk(const PersistArgs& A, const PipeCtx& c, int q, char* smem) {
  if constexpr (MX) do_gather_mx(A, c, q, smem);
  else do_gather(A, c, q, smem);
}

// Push pipeline-local chunk q: its output rows (in place in the ring) to recv[rank][token][j];
// then free its slot (whole workgroup).
__device__ void do_push(const PersistArgs& A, const PipeCtx& c, int q, char* smem) {
  if (A.row_dst) {      // the down GEMM already stored the rows to recv: only free the slot
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(A.pc + sched::slot_epoch_word(A.cl, c.p, c.S, q), 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  uint64_t* src_tab = reinterpret_cast<uint64_t*>(smem);
  uint64_t* dst_tab = src_tab + kGemmBM;
  int row0, l;
  const int m = c.lo + q / c.cpm, h = q % c.cpm;
  const int rows = tile_rows(A, layout_tile(c.reverse, c.lo, c.n_m, m), &row0, &l);
  const int c_lo = h * c.chunk_rows, c_n = min(c.chunk_rows, rows - c_lo);
  const char* src = slot_ptr(A, c, q);
  for (int r = threadIdx.x; r < c_n; r += kGemmThreads) {
    const int s = row0 + c_lo + r;
    const int rk = A.pull_src[2 * (long long)s];
    const int t = A.pull_src[2 * (long long)s + 1];
    const int32_t* so = A.slot_of + ((long long)rk * A.T + t) * A.k;
    int j = 0;
    for (int jj = 0; jj < A.k; ++jj)
      if (so[jj] == s) j = jj;
    src_tab[r] = reinterpret_cast<uint64_t>(src + (long long)r * c.row_bytes);
    dst_tab[r] = reinterpret_cast<uint64_t>(A.recv.p[rk] + ((long long)t * A.k + j) * c.row_bytes);
  }
  __syncthreads();
  if (c_n > 0) wg_copy_rows<true>(src_tab, dst_tab, c_n, c.n16);    // output rows other CUs wrote
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");             // the slot's reads are done
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(A.pc + sched::slot_epoch_word(A.cl, c.p, c.S, q), 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// A compute workgroup waits until every chunk of row tile m is in its slot; meanwhile it
// gathers claimable chunks of its pipeline itself (a gather never waits, so this cannot
// deadlock).  Returns false on abort or watchdog expiry.
// Work stealing at the end of a launch (outputs stored straight to recv; persist_sched.hpp
// states the rule).  Thread 0 only: polls the other pipelines (those some
// workgroup joined) for a ticket in their last phase.  0: *tp / *t hold the ticket; 1: every
// other pipeline has handed out all its tickets; 2: abort or watchdog.
__device__ int steal_next(const PersistArgs& A, int p, int* tp, int* t) {
  const DevOps ops{A.pc};
  const long long t0 = wall_clock64();
  while (true) {
    if (ld_relaxed(A.pc + A.cl.abort_word)) return 2;
    bool pending = false;
    for (int k = 1; k < A.n_part; ++k) {
      const int v = p + k < A.n_part ? p + k : p + k - A.n_part;
      const int32_t* vw = A.pc + A.cl.pipe0 + v * sched::kPipeWords;
      if (ld_relaxed(vw + sched::kJoin) == 0) continue;
      const int ng = vw[sched::kNGroups], nt = vw[sched::kNTickets];    // written by the preparation kernel
      if (ng == 0) continue;
      const int last = A.pc[A.cl.phase_start + 2 * vw[sched::kLo] + v + 2 * ng - 1];
      const int r = sched::steal_claim(ops, A.cl, v, last, nt);
      if (r >= 0) {
        *tp = v;
        *t = r;
        return 0;
      }
      if (r == sched::kStealWait) pending = true;
    }
    if (!pending) return 1;
    __builtin_amdgcn_s_sleep(2);
    if (wall_clock64() - t0 > A.budget) {
      set_abort(A, MOE_ETIMEOUT);
      return 2;
    }
  }
}

template <bool MX>
__device__ bool wait_chunks(const PersistArgs& A, const PipeCtx& c, int m, char* smem, int* sh) {
  const DevOps ops{A.pc};
  long long t0 = wall_clock64();
  while (true) {
    if (threadIdx.x == 0) {
      int st = 0, arg = 0;            // 0 wait, 1 ready, 2 abort, 3 gather chunk arg
      bool ready = true;
      for (int h = 0; h < c.cpm; ++h)
        if (ld_relaxed(A.pc + A.cl.filled + m * 4 + h) < 1) ready = false;
      if (ready) {
        st = 1;
      } else if (ld_relaxed(A.pc + A.cl.abort_word)) {
        st = 2;
      } else if (sched::mover_claim(ops, A.cl, c.p, c.lo, c.n_m, c.cpm, c.S, c.NT2, &arg, true) == sched::kGather) {
        st = 3;
      } else {
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > A.budget) {
          set_abort(A, MOE_ETIMEOUT);
          st = 2;
        }
      }
      sh[1] = st;
      sh[2] = arg;
    }
    __syncthreads();
    const int st = sh[1], arg = sh[2];
    __syncthreads();
    if (st == 1) return true;
    if (st == 2) return false;
    if (st == 3) {
      const long long tb = wall_clock64();
      gather_chunk<MX>(A, c, arg, smem);
      trace_event(A, 1, arg, c.p, tb, wall_clock64(), tb - t0);
      t0 = wall_clock64();
    }
  }
}

template <bool MX>
__global__ __launch_bounds__(kGemmThreads, 1) void moe_persistent_kernel(PersistArgs A) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int sh[4];
  const int tid = threadIdx.x;
  const long long t_start = wall_clock64();

  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  PipeCtx c;
  c.p = int(xcc & 7) * A.n_part / 8;
  const int p = c.p;
  c.light = A.light;
  c.reverse = A.reverse != 0;
  const int pbase = A.cl.pipe0 + p * sched::kPipeWords;
  int32_t* pw = A.pc + pbase;
  int32_t* g1_done = A.pc + A.cl.g1_done;
  int32_t* g2_done = A.pc + A.cl.g2_done;

  if (tid == 0) sh[0] = __hip_atomic_fetch_add(pw + sched::kJoin, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int rank = sh[0];
  __syncthreads();
  const bool mover = rank < A.comm_pp;
  trace_event(A, 0, mover ? 0 : 1, p, t_start, t_start, 0);

  // this pipeline's row tiles [lo, hi) and tables (written by the preparation kernel)
  c.lo = pw[sched::kLo];
  c.n_m = pw[sched::kHi] - c.lo;
  const int lo = c.lo;
  const int n_groups = pw[sched::kNGroups], n_tickets = pw[sched::kNTickets];
  c.S = A.S;
  c.cpm = A.cpm;
  c.chunk_rows = 1 << A.blk_log2;
  c.row_bytes = A.d * 2;
  c.n16 = c.row_bytes >> 4;
  c.NT2 = (A.d + kGemmBN - 1) / kGemmBN;
  const int cpm = c.cpm;
  const bool light = c.light;
  const int NT1 = (A.F + kGemmBN / 2 - 1) / (kGemmBN / 2);
  const long long xpart = (long long)c.chunk_rows * c.row_bytes;   // token / output rows of a slot

  // Compute workgroups take tickets until none is left, then join the data movement for the
  // tail (the last pushes); data-movement workgroups move data from the start.
  bool aborted = false;
  if (!mover && n_tickets > 0) {
    // ------------------------------------------------------------ expert compute
    const int32_t* phase_start = A.pc + A.cl.phase_start + 2 * lo + p;
    const int32_t* grp_first = A.pc + A.cl.grp_first + lo;
    const int32_t* grp_len = A.pc + A.cl.grp_len + lo;
    // with stealing on, the gate/up tiles of this pipeline's last group release at agent
    // scope: another XCD may run the down tiles that read their h rows
    const int last_first = n_groups > 0 ? grp_first[n_groups - 1] : lo;
    bool own_left = true;                                  // thread 0's view
    while (true) {
      if (tid == 0) {
        int st = 0, tp = p, t = -1;                        // st: 0 task, 1 none left, 2 abort
        if (own_left) {
          t = __hip_atomic_fetch_add(pw + sched::kTicketNext, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (t >= n_tickets) own_left = false;
        }
        if (!own_left) {
          st = 1;
          if (A.steal) st = steal_next(A, p, &tp, &t);
        }
        sh[1] = st;
        sh[2] = tp;
        sh[3] = t;
      }
      __syncthreads();
      const int st = sh[1], tp = sh[2], ticket = sh[3];
      __syncthreads();
      if (st == 2) {
        aborted = true;
        break;
      }
      if (st == 1) break;
      // the ticket's pipeline: another one for a stolen ticket (a down tile of its last group)
      PipeCtx cv = c;
      const int32_t* t_ps = phase_start;
      const int32_t* t_gf = grp_first;
      const int32_t* t_gl = grp_len;
      int t_ng = n_groups;
      bool remote = false;
      {
        if (tp != p) {
          const int32_t* vw = A.pc + A.cl.pipe0 + tp * sched::kPipeWords;
          cv.p = tp;
          cv.lo = vw[sched::kLo];
          cv.n_m = vw[sched::kHi] - cv.lo;
          t_ng = vw[sched::kNGroups];
          t_ps = A.pc + A.cl.phase_start + 2 * cv.lo + tp;
          t_gf = A.pc + A.cl.grp_first + cv.lo;
          t_gl = A.pc + A.cl.grp_len + cv.lo;
          remote = true;
        }
      }
      const sched::Task tk = sched::task_of_ticket(ticket, t_ng, t_ps, t_gf, t_gl, A.lookahead != 0);
      const int m = tk.m;                                   // pipeline order
      const int ml = layout_tile(A.reverse, cv.lo, cv.n_m, m);   // layout row tile
      int row0, l;
      const int rows = tile_rows(A, ml, &row0, &l);
      const long long t_w = wall_clock64();
      // (a stolen down tile waits for the publishing mark of its row tile's gate/up tiles when
      // they handed off L2-locally)
      const bool ok = !tk.down ? wait_chunks<MX>(A, cv, m, smem, sh)
                               : wait_ge(g1_done + m, NT1 + ((remote && light) ? 1 : 0), A, sh);
      if (!ok) {
        aborted = true;
        break;
      }
      const long long t_b = wall_clock64();
      acquire_after_poll(light && !remote);                // a stolen tile's h came through another L2
      const int q0 = (m - cv.lo) * cpm;
      char* s0 = slot_ptr(A, cv, q0);
      char* s1 = slot_ptr(A, cv, q0 + min(1, cpm - 1));
      char* s2 = slot_ptr(A, cv, q0 + min(2, cpm - 1));
      char* s3 = slot_ptr(A, cv, q0 + min(3, cpm - 1));
      if constexpr (MX) {
        // the tile's rows are the chunks' slots: token codes / scale words for the gate/up
        // GEMM, h codes / scale words for the down GEMM, whose outputs go straight to recv
        char* sl[4] = {s0, s1, s2, s3};
        TileMX io{};
        io.blk_log2 = A.blk_log2;
        io.rows = rows;
        io.as_plane = 4LL * c.chunk_rows;
        io.os_plane = 4LL * c.chunk_rows;
        if (!tk.down) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            io.ablk[i] = reinterpret_cast<const uint8_t*>(sl[i]);
            io.asblk[i] = reinterpret_cast<const uint8_t*>(sl[i] + A.tok_s_off);
            io.oblk[i] = reinterpret_cast<uint8_t*>(sl[i] + A.h_off);
            io.osblk[i] = reinterpret_cast<uint8_t*>(sl[i] + A.h_s_off);
          }
          const uint8_t* b0 = A.w1q + size_t(l) * A.F * A.d;
          const uint8_t* b1 = A.w3q + size_t(l) * A.F * A.d;
          gemm_mx_tile<0, 16, true>(io, b0, b1, A.w1s + 4 * size_t(l) * A.F, A.w3s + 4 * size_t(l) * A.F,
                                    4LL * A.El * A.F, tk.j * (kGemmBN / 2), A.F, A.d, smem);
          if (A.steal && m >= last_first && light) release_add_publish(g1_done + m, NT1);
          else release_add(g1_done + m, 1, light);
          trace_event(A, 3, ml * 256 + tk.j, p, t_b, wall_clock64(), t_b - t_w);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            io.ablk[i] = reinterpret_cast<const uint8_t*>(sl[i] + A.h_off);
            io.asblk[i] = reinterpret_cast<const uint8_t*>(sl[i] + A.h_s_off);
          }
          io.row_dst = A.row_dst + row0;
          const uint8_t* b0 = A.w2q + size_t(l) * A.d * A.F;
          const uint8_t* bs0 = A.w2s + 4 * size_t(l) * A.d;
          gemm_mx_tile<1, 16, true>(io, b0, b0, bs0, bs0, 4LL * A.El * A.d, tk.j * kGemmBN, A.d, A.F, smem);
          release_add(g2_done + m, 1, light && !remote);
          trace_event(A, 4, ml * 256 + tk.j, tp, t_b, wall_clock64(), t_b - t_w);
        }
      } else {
        TileIO io;
        io.blk_log2 = A.blk_log2;
        io.rows = rows;
        io.row_dst = nullptr;
        io.row_src = nullptr;
        io.dh = nullptr;
        io.dab = nullptr;
        if (!tk.down) {
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
          gemm_tile<0, 16>(io, b0, b1, tk.j * (kGemmBN / 2), A.F, A.d, smem, A.d);   // x rows: sc1 loads
          if (A.steal && m >= last_first && light) release_add_publish(g1_done + m, NT1);
          else release_add(g1_done + m, 1, light);
          trace_event(A, 3, ml * 256 + tk.j, p, t_b, wall_clock64(), t_b - t_w);
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
          if (A.row_dst) io.row_dst = A.row_dst + row0;       // outputs straight to recv
          const uint16_t* b0 = A.w2 + size_t(l) * A.d * A.F;
          gemm_tile<1, 16>(io, b0, b0, tk.j * kGemmBN, A.d, A.F, smem, A.F);         // h rows: sc1 loads
          release_add(g2_done + m, 1, light && !remote);
          trace_event(A, 4, ml * 256 + tk.j, tp, t_b, wall_clock64(), t_b - t_w);
        }
      }
    }
  }
  if (!aborted) {
    // ------------------------------------------------------------ data movement
    const DevOps ops{A.pc};
    long long idle_since = wall_clock64();
    while (true) {
      if (tid == 0) {
        int act = sched::kIdle, arg = 0;
        if (ld_relaxed(A.pc + A.cl.abort_word)) {
          act = sched::kDone;
        } else {
          act = sched::mover_claim(ops, A.cl, p, lo, c.n_m, cpm, c.S, c.NT2, &arg);
          if (act == sched::kIdle) {
            __builtin_amdgcn_s_sleep(1);
            if (wall_clock64() - idle_since > A.budget) {
              set_abort(A, MOE_ETIMEOUT);
              act = sched::kDone;
            }
          }
        }
        sh[1] = act;
        sh[2] = arg;
      }
      __syncthreads();
      const int act = sh[1], arg = sh[2];
      __syncthreads();
      if (act == sched::kDone) break;
      if (act == sched::kIdle) continue;
      const long long t_b = wall_clock64();
      acquire_after_poll(light);
      if (act == sched::kPush) {
        do_push(A, c, arg, smem);
        trace_event(A, 2, arg, p, t_b, wall_clock64(), t_b - idle_since);
      } else {
        gather_chunk<MX>(A, c, arg, smem);
        trace_event(A, 1, arg, p, t_b, wall_clock64(), t_b - idle_since);
      }
      idle_since = wall_clock64();
    }
  }
  trace_event(A, 5, mover ? 0 : 1, p, wall_clock64(), wall_clock64(), 0);
}

// ---------------------------------------------------------------------------- host side
int persist_ctrl_words(int max_mtiles) { return sched::ctrl_layout(max_mtiles, kMaxRingSlots).words; }

// MXFP8 ring slot of cr rows: the token rows' codes, their scale words (d / 128 K-tile planes
// of cr words), h's codes, h's scale words; each part 256-byte aligned.  Returns the slot size.
long long persist_mx_slot_layout(int d, int F, int cr, long long* tok_s_off, long long* h_off, long long* h_s_off) {
  long long o = static_cast<long long>(cr) * d;
  *tok_s_off = static_cast<long long>(align256(size_t(o)));
  o = *tok_s_off + 4LL * cr * (d / 128);
  *h_off = static_cast<long long>(align256(size_t(o)));
  o = *h_off + static_cast<long long>(cr) * F;
  *h_s_off = static_cast<long long>(align256(size_t(o)));
  o = *h_s_off + 4LL * cr * (F / 128);
  return static_cast<long long>(align256(size_t(o)));
}

hipError_t persistent_occupancy(int* blocks_per_cu, bool mx) {
  static std::atomic<uint64_t> attr_set{0};
  const hipError_t ea = once_per_device(attr_set, [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_persistent_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_persistent_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
    return e;
  });
  if (ea != hipSuccess) return ea;
  return mx ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                  blocks_per_cu, reinterpret_cast<const void*>(moe_persistent_kernel<true>), kGemmThreads, kMxLds)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                  blocks_per_cu, reinterpret_cast<const void*>(moe_persistent_kernel<false>), kGemmThreads, kGemmLds);
}

hipError_t launch_persistent(const moe_shape_t& s, int El, const void* const* x, const void* w1, const void* w3,
                             const void* w2, const int32_t* pull_src, const int32_t* slot_of,
                             const int32_t* offsets, char* ring, long long slot_bytes, int blk_log2,
                             const sched::Plan& plan, int grid, long long budget, void* const* recv, char* ws,
                             const WsLayout& L, moe_trace_event_t* trace, int32_t* trace_count, int trace_cap,
                             const uint64_t* row_dst, bool reverse, const moe_mx_scales_t* w_scales,
                             hipStream_t st) {
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
  A.status = reinterpret_cast<int32_t*>(ws + L.ctrl) + kCtrlStatus;
  A.w1 = static_cast<const uint16_t*>(w1);
  A.w3 = static_cast<const uint16_t*>(w3);
  A.w2 = static_cast<const uint16_t*>(w2);
  A.ring = ring;
  A.pc = reinterpret_cast<int32_t*>(ws + L.pctrl);
  A.trace = trace;
  A.trace_count = trace_count;
  A.trace_cap = trace_cap;
  A.slot_bytes = slot_bytes;
  A.budget = budget;
  A.T = s.T;
  A.k = s.k;
  A.d = s.d;
  A.F = s.F;
  A.El = El;
  A.blk_log2 = blk_log2;
  A.cpm = kGemmBM >> blk_log2;
  A.n_part = plan.n_part;
  A.light = plan.light;
  A.comm_pp = plan.comm_pp;
  A.S = plan.S;
  A.G = plan.G;
  A.lookahead = plan.lookahead;
  A.reverse = reverse ? 1 : 0;
  A.max_mtiles = L.max_mtiles;
  A.row_dst = row_dst;
  A.cl = sched::ctrl_layout(L.max_mtiles, kMaxRingSlots);
  A.mx = w_scales ? 1 : 0;
  if (A.mx) {
    A.w1q = static_cast<const uint8_t*>(w1);
    A.w3q = static_cast<const uint8_t*>(w3);
    A.w2q = static_cast<const uint8_t*>(w2);
    A.w1s = w_scales->w1;
    A.w3s = w_scales->w3;
    A.w2s = w_scales->w2;
    persist_mx_slot_layout(s.d, s.F, 1 << blk_log2, &A.tok_s_off, &A.h_off, &A.h_s_off);
  }
  // work stealing at the end of the launch: outputs stored straight to recv, and more than
  // one pipeline
  A.steal = (row_dst && plan.n_part > 1) ? 1 : 0;

  int occ = 0;
  hipError_t e = persistent_occupancy(&occ, A.mx != 0);
  if (e != hipSuccess) return e;
  const int zero_words = A.cl.slot_epoch + plan.n_part * plan.S;
  hipLaunchKernelGGL(persist_prep_kernel, dim3(1), dim3(1024), 0, st, A, zero_words);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (A.mx)
    hipLaunchKernelGGL(moe_persistent_kernel<true>, dim3(grid), dim3(kGemmThreads), kMxLds, st, A);
  else
    hipLaunchKernelGGL(moe_persistent_kernel<false>, dim3(grid), dim3(kGemmThreads), kGemmLds, st, A);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(persist_check_kernel, dim3(1), dim3(1024), 0, st, A);
  return hipGetLastError();
}

}  // namespace moe
