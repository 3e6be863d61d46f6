// Shared device/host definitions of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/moe.h"
#include "persist_sched.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// fixed tile geometry
// ---------------------------------------------------------------------------
constexpr int kTokPerLayoutBlock = 64;   // tokens per histogram block of the layout
constexpr int kGemmBM = 256;             // rows of one grouped-GEMM tile (bf16 path)
constexpr int kGemmBN = 256;             // output columns of one tile
constexpr int kGemmBK = 64;              // K step staged in LDS
constexpr int kF32BM = 64;               // fp32 MFMA path tile (rows x columns)
constexpr int kF32BN = 64;

// ---------------------------------------------------------------------------
// host: a kernel-attribute grant (hipFuncSetAttribute acts on the current device), done
// once per device; safe from several host threads (a grant repeated in a race is harmless)
// ---------------------------------------------------------------------------
template <typename F>
inline hipError_t once_per_device(std::atomic<uint64_t>& done, F grant) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = grant();
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// ---------------------------------------------------------------------------
// workspace layout (computed on the host from the shape; every region 256-byte aligned)
// ---------------------------------------------------------------------------
enum CtrlSlot {
  kCtrlStatus = 0,   // device status word (MOE_OK / MOE_EINVAL / MOE_ETIMEOUT)
  kCtrlN = 1,        // local pairs N
  kCtrlMTiles = 2,   // grouped-GEMM row tiles over all local experts
  kCtrlChunks = 3,   // minibatch chunks over all local experts
  kCtrlWords = 64
};

constexpr int kMaxRingSlots = 65536;

struct WsLayout {
  size_t ctrl, l2g, mtile_base, chunk_base, blockhist, blockbase, pctrl, hbuf, push_dst, pull_addr, total;
  int32_t nb;        // layout blocks
  int64_t max_pairs;
  int32_t max_mtiles;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline WsLayout ws_layout(const moe_shape_t& s, int32_t E_local) {
  WsLayout w{};
  const int64_t tokens = int64_t(s.R) * s.T;
  w.nb = int32_t((tokens + kTokPerLayoutBlock - 1) / kTokPerLayoutBlock);
  w.max_pairs = tokens * (s.k < E_local ? s.k : E_local);
  const int bm = (s.dtype == MOE_F32) ? kF32BM : kGemmBM;
  w.max_mtiles = int32_t((w.max_pairs + bm - 1) / bm + E_local);
  const size_t esz = (s.dtype == MOE_F32) ? 4 : 2;
  size_t o = 0;
  w.ctrl = o;        o = align256(o + kCtrlWords * 4);
  w.l2g = o;         o = align256(o + size_t(E_local) * 4);
  w.mtile_base = o;  o = align256(o + size_t(E_local + 1) * 4);
  w.chunk_base = o;  o = align256(o + size_t(E_local + 1) * 4);
  w.blockhist = o;   o = align256(o + size_t(w.nb) * s.E * 4);
  w.blockbase = o;   o = align256(o + size_t(w.nb) * E_local * 4);
  // persistent-path control block (counters, task tables, one epoch word per ring slot)
  w.pctrl = o;       o = align256(o + size_t(sched::ctrl_layout(w.max_mtiles, kMaxRingSlots).words) * 4);
  // h staging: fp32/bf16 rows, or MXFP8 codes followed (256-aligned) by their block scales
  const size_t hbytes = (s.dtype == MOE_MXFP8)
                            ? align256(size_t(w.max_pairs) * s.F) + size_t(w.max_pairs) * (s.F / 32)
                            : size_t(w.max_pairs) * s.F * esz;
  w.hbuf = o;        o = align256(o + hbytes);
  // per local pair: the address of its recv row (the push fused into the down GEMM)
  w.push_dst = o;    o = align256(o + size_t(w.max_pairs) * 8);
  // per local pair: the address of its source token row (the pull fused into the gate/up GEMM)
  w.pull_addr = o;   o = align256(o + size_t(w.max_pairs) * 8);
  w.total = o;
  return w;
}

// Backward workspace: the per-row gradients handed from one backward stage to the next,
// and the per-pair gate gradients of the push.  MXFP8 adds the MX codes and block scales
// of dO (along d) and of [da | db] (along F) for the data-gradient GEMMs, and bf16 copies
// of the dispatched token rows for the weight gradients.
struct BwdLayout {
  size_t dO, dg, dh, h, dab, dX, dgp;
  size_t rows, blks, held;            // moe_backward_ring: token row addresses (per row, per 64-row block),
                                      // and whether each block is read in the ring
  size_t dOq, dOs, dabq, dabs, xeb;   // MXFP8 only (0 otherwise)
  size_t total;
};

inline BwdLayout bwd_layout(const moe_shape_t& s, int32_t E_local) {
  BwdLayout b{};
  const int64_t mp = int64_t(s.R) * s.T * (s.k < E_local ? s.k : E_local);
  const size_t d = size_t(s.d), F = size_t(s.F), n = size_t(mp);
  size_t o = 0;
  b.dO = o;   o = align256(o + n * d * 2);
  b.dg = o;   o = align256(o + n * 4);
  b.dh = o;   o = align256(o + n * F * 2);
  b.h = o;    o = align256(o + n * F * 2);
  b.dab = o;  o = align256(o + n * F * 4);
  b.dX = o;   o = align256(o + n * d * 2);
  b.dgp = o;  o = align256(o + size_t(s.R) * s.T * s.k * 4);
  const size_t mtiles = size_t((mp + kGemmBM - 1) / kGemmBM + E_local);
  b.rows = o; o = align256(o + n * 8);
  b.blks = o; o = align256(o + mtiles * 4 * 8);
  b.held = o; o = align256(o + mtiles * 4 * 4);
  if (s.dtype == MOE_MXFP8) {
    b.dOq = o;  o = align256(o + n * d);
    b.dOs = o;  o = align256(o + n * (d / 32));
    b.dabq = o; o = align256(o + n * 2 * F);
    b.dabs = o; o = align256(o + n * (2 * F / 32));
    b.xeb = o;  o = align256(o + n * d * 2);
  }
  b.total = o;
  return b;
}

// which local expert owns global row tile mt (binary search on the tile prefix)
__device__ __forceinline__ int find_expert(const int32_t* __restrict__ mtile_base, int El, int mt) {
  int lo = 0, hi = El - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mtile_base[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// per-rank pointer table passed by value to kernels
template <typename T>
struct RankPtrs {
  T p[MOE_MAX_RANKS];
};

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// round-to-nearest-even fp32 -> bf16 (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two fp32 values rounded to nearest even into one bf16 pair (lo in the low half): gfx950's
// packed conversion, one instruction.  For finite inputs it equals f32_to_bf16 on each half
// (checked on the device over 16.7 M random pairs with denormals, values near the top of the
// range and every tie pattern of the low 16 bits).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace moe
