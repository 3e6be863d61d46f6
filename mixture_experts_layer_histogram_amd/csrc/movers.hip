// Row movers for gfx950: pull dispatch, push combine and the ordered weighted merge.
//
// Operations (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// sections 01-03): the expert side pulls each token row it needs from its source
// buffer (dispatch); results are pushed back to the token's own position (combine);
// the final weighted merge sums a token's expert outputs with its gate weights.
//
// These are HBM-bound copies, so every lane moves 16-byte vectors and keeps several
// of them in flight; there is no reuse for LDS staging to exploit.  A wave owns one
// row at a time; the grid strides over rows, and the row count N is read from the
// layout's control block on the device (no host round trip).
#include "common.hpp"

namespace moe {

// UNROLL = 16-byte vectors in flight per lane (16: a 16 KiB row in one round trip).
// Measured on MI355X at the DeepSeek-V3 share: the gather (random source rows, sequential
// destination) is fastest with 16 in flight and 4 resident blocks per CU; the push
// (sequential source, scattered destination) with 8 in flight and 8 blocks per CU.
template <int UNROLL>
__device__ __forceinline__ void copy_row(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int n16,
                                         int lane) {
  for (int base = 0; base < n16; base += 64 * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int i = base + u * 64 + lane;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int i = base + u * 64 + lane;
      if (i < n16) dst[i] = v[u];
    }
  }
}

// xe[s] = x[pull_src[s].rank][pull_src[s].token]
__global__ __launch_bounds__(256) void dispatch_pull_kernel(RankPtrs<const char*> x,
                                                            const int32_t* __restrict__ pull_src,
                                                            const int32_t* __restrict__ ctrl,
                                                            char* __restrict__ xe, int row_bytes) {
  const int N = ctrl[kCtrlN];
  const int lane = threadIdx.x & 63;
  const int n16 = row_bytes >> 4;
  const int nw = gridDim.x * 4;
  for (int s = blockIdx.x * 4 + (threadIdx.x >> 6); s < N; s += nw) {
    const int r = pull_src[2 * int64_t(s)];
    const int t = pull_src[2 * int64_t(s) + 1];
    copy_row<16>(reinterpret_cast<const u32x4*>(x.p[r] + int64_t(t) * row_bytes),
             reinterpret_cast<u32x4*>(xe + int64_t(s) * row_bytes), n16, lane);
  }
}

// The backward after a reverse-ring persistent forward: where each expert-side token row is.
// Block b of row tile m is its rows row0 + 64 b .. (at most 64).  If the ring slot that still
// holds its chunk is recorded (resident[m * 4 + h] = 1 + slot, slot < n_slots), the block is
// read in place there; else its rows are pulled again from the source buffers into xe at
// their rows.  ring_blocks_kernel writes blk_src[m * 4 + b] (the block's first row) and a
// held flag per block, one thread per block; ring_rows_kernel then gives every row s its
// address row_src[s] and pulls the rows of blocks not held, one wave per row as the gather.
__global__ __launch_bounds__(256) void ring_blocks_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ mtile_base,
                                                          const int32_t* __restrict__ ctrl,
                                                          const int32_t* __restrict__ resident, const char* ring,
                                                          long long slot_bytes, int n_slots, int chunk_log2,
                                                          char* xe, int El, int max_mtiles, int row_bytes,
                                                          uint64_t* __restrict__ blk_src, int32_t* __restrict__ blk_held) {
  const int n_mt = min(ctrl[kCtrlMTiles], max_mtiles);
  for (int bid = blockIdx.x * 256 + threadIdx.x; bid < n_mt * 4; bid += gridDim.x * 256) {
    const int m = bid >> 2, b = bid & 3;
    const int l = find_expert(mtile_base, El, m);
    const int row0 = offsets[l] + (m - mtile_base[l]) * kGemmBM;
    const int r_lo = b * 64;
    const int h = r_lo >> chunk_log2;
    int rs = ring ? resident[m * 4 + h] : 0;
    if (rs < 1 || rs > n_slots) rs = 0;
    const char* base = rs ? ring + (long long)(rs - 1) * slot_bytes + (long long)(r_lo - (h << chunk_log2)) * row_bytes
                          : xe + (long long)(row0 + r_lo) * row_bytes;
    blk_src[bid] = reinterpret_cast<uint64_t>(base);
    blk_held[bid] = rs ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void ring_rows_kernel(RankPtrs<const char*> x, const int32_t* __restrict__ pull_src,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ mtile_base,
                                                        const int32_t* __restrict__ ctrl,
                                                        const uint64_t* __restrict__ blk_src,
                                                        const int32_t* __restrict__ blk_held, char* xe, int El,
                                                        int row_bytes, uint64_t* __restrict__ row_src) {
  __shared__ int32_t s_off[1025], s_mtb[1025];           // E_local <= E <= 1024
  for (int i = threadIdx.x; i <= El; i += blockDim.x) {
    s_off[i] = offsets[i];
    s_mtb[i] = mtile_base[i];
  }
  __syncthreads();
  const int N = ctrl[kCtrlN];
  const int lane = threadIdx.x & 63;
  const int n16 = row_bytes >> 4;
  const int nw = gridDim.x * 4;
  for (int s = blockIdx.x * 4 + (threadIdx.x >> 6); s < N; s += nw) {
    int lo = 0, hi = El - 1;                              // the expert whose rows hold s
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= s) lo = mid; else hi = mid - 1;
    }
    const int i = s - s_off[lo];
    const int bid = (s_mtb[lo] + (i >> 8)) * 4 + ((i & 255) >> 6);
    if (lane == 0) row_src[s] = blk_src[bid] + uint64_t(i & 63) * uint64_t(row_bytes);
    if (!blk_held[bid]) {
      const int rk = pull_src[2 * int64_t(s)];
      const int t = pull_src[2 * int64_t(s) + 1];
      copy_row<16>(reinterpret_cast<const u32x4*>(x.p[rk] + int64_t(t) * row_bytes),
                   reinterpret_cast<u32x4*>(xe + int64_t(s) * row_bytes), n16, lane);
    }
  }
}

// recv[r][t][j] = ye[s] for the pair (r, t, j) whose row is s.  In the backward (push
// reverse-dispatch) ye holds dX and the row's gate gradient dg[s] travels with it into
// dgp[r][t][j] (dg == nullptr in the forward).
__global__ __launch_bounds__(256) void combine_push_kernel(const char* __restrict__ ye,
                                                           const int32_t* __restrict__ pull_src,
                                                           const int32_t* __restrict__ slot_of,
                                                           const int32_t* __restrict__ ctrl,
                                                           RankPtrs<char*> recv, int T, int k,
                                                           int row_bytes, const float* __restrict__ dg,
                                                           float* __restrict__ dgp) {
  const int N = ctrl[kCtrlN];
  const int lane = threadIdx.x & 63;
  const int n16 = row_bytes >> 4;
  const int nw = gridDim.x * 4;
  for (int s = blockIdx.x * 4 + (threadIdx.x >> 6); s < N; s += nw) {
    const int r = pull_src[2 * int64_t(s)];
    const int t = pull_src[2 * int64_t(s) + 1];
    // the pair's j: lanes 0..k-1 compare their slot_of entry at once (k <= 16)
    const int32_t* so = slot_of + (int64_t(r) * T + t) * k;
    const unsigned long long hit = __ballot(lane < k && so[lane < k ? lane : 0] == s);
    const int j = hit ? __builtin_ctzll(hit) : 0;
    if (dg && lane == 0) dgp[(int64_t(r) * T + t) * k + j] = dg[s];
    copy_row<8>(reinterpret_cast<const u32x4*>(ye + int64_t(s) * row_bytes),
             reinterpret_cast<u32x4*>(recv.p[r] + (int64_t(t) * k + j) * row_bytes), n16, lane);
  }
}

// Per-pair address tables for the fused FFN: push_dst[s] = address of recv[r][t][j] (the
// push fused into the down GEMM), and, when pull_addr is not null, pull_addr[s] = address of
// x_r[t] (the pull fused into the gate/up GEMM), with (r, t) = pull_src[s] and
// slot_of[r][t][j] = s; in the backward, dgp[r][t][j] = dg[s] as well (the push of the gate
// gradients, whose dX rows the dX GEMM pushes itself).
__global__ __launch_bounds__(256) void pair_addr_kernel(const int32_t* __restrict__ pull_src,
                                                        const int32_t* __restrict__ slot_of,
                                                        const int32_t* __restrict__ ctrl, RankPtrs<char*> recv,
                                                        RankPtrs<const char*> x, int T, int k, int row_bytes,
                                                        uint64_t* __restrict__ push_dst,
                                                        uint64_t* __restrict__ pull_addr,
                                                        const float* __restrict__ dg, float* __restrict__ dgp) {
  const int N = ctrl[kCtrlN];
  for (int s = blockIdx.x * 256 + threadIdx.x; s < N; s += gridDim.x * 256) {
    const int r = pull_src[2 * int64_t(s)];
    const int t = pull_src[2 * int64_t(s) + 1];
    const int32_t* so = slot_of + (int64_t(r) * T + t) * k;
    int j = 0;
    for (int jj = 0; jj < k; ++jj)
      if (so[jj] == s) j = jj;
    push_dst[s] = reinterpret_cast<uint64_t>(recv.p[r] + (int64_t(t) * k + j) * row_bytes);
    if (pull_addr) pull_addr[s] = reinterpret_cast<uint64_t>(x.p[r] + int64_t(t) * row_bytes);
    if (dgp) dgp[(int64_t(r) * T + t) * k + j] = dg[s];     // backward: the pair's gate gradient
  }
}

// y[r][t] = sum over ascending j with a local expert of g[r][t][j] * recv[r][t][j]
// (g = 1 when topk_w is null: the backward's ordered sum of the pushed dX rows)
// A wave task is one column segment (64 * VPL 16-byte vectors) of one token row.  The
// token's local j are compacted into a mask; for each local j all VPL loads of the
// segment are issued before any is used, so a task costs one memory round trip per j.
// Measured on MI355X at the DeepSeek-V3 share: short segments (VPL 4) and a grid of 16
// blocks per CU keep the most rows in flight (180 us against 199 us for VPL 8 with 4
// blocks per CU); prefetching the next task's metadata changed less than 1 %.  A row whose
// vector count is a multiple of 64 * 7 (d = 7168 in bf16: 896 vectors) takes VPL 7, which
// splits it into two full segments instead of three and a half.
template <bool BF16, int VPL>
__global__ __launch_bounds__(256) void weighted_merge_kernel(RankPtrs<const char*> recv,
                                                             RankPtrs<char*> y,
                                                             const int32_t* __restrict__ slot_of,
                                                             const float* __restrict__ topk_w, int R,
                                                             int T, int k, int d) {
  constexpr int EPV = BF16 ? 8 : 4;      // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int row_bytes = d * (BF16 ? 2 : 4);
  const int n16 = row_bytes >> 4;
  const int nseg = (n16 + 64 * VPL - 1) / (64 * VPL);
  const int64_t tasks = int64_t(R) * T * nseg;
  const int64_t nw = int64_t(gridDim.x) * 4;
  for (int64_t task = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); task < tasks; task += nw) {
    const int64_t g = task / nseg;
    const int cb = int(task - g * nseg) * 64 * VPL;
    const int r = int(g / T);
    const int t = int(g - int64_t(r) * T);
    const int32_t* so = slot_of + g * k;
    const float* gw = topk_w ? topk_w + g * k : nullptr;
    // the token's local j (ascending) as a bit mask: lanes 0..k-1 test their entry at once
    const unsigned long long lm = __ballot(lane < k && so[lane < k ? lane : 0] >= 0);
    uint32_t local = uint32_t(lm);
    const char* rrow = recv.p[r] + int64_t(t) * k * row_bytes;
    u32x4* yrow = reinterpret_cast<u32x4*>(y.p[r] + int64_t(t) * row_bytes);
    float acc[VPL][EPV];
#pragma unroll
    for (int u = 0; u < VPL; ++u)
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[u][e] = 0.0f;
    for (uint32_t m = local; m; m &= m - 1) {
      const int j = __builtin_ctz(m);
      const float gj = gw ? gw[j] : 1.0f;
      const u32x4* src = reinterpret_cast<const u32x4*>(rrow + int64_t(j) * row_bytes);
      u32x4 v[VPL];
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int i = cb + u * 64 + lane;
        if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
      }
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int i = cb + u * 64 + lane;
        if (i < n16) {
          if (BF16) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              acc[u][2 * w] = fmaf(gj, __uint_as_float(v[u][w] << 16), acc[u][2 * w]);
              acc[u][2 * w + 1] = fmaf(gj, __uint_as_float(v[u][w] & 0xFFFF0000u), acc[u][2 * w + 1]);
            }
          } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[u][w] = fmaf(gj, __uint_as_float(v[u][w]), acc[u][w]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int i = cb + u * 64 + lane;
      if (i < n16) {
        u32x4 o;
        if (BF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(acc[u][2 * w], acc[u][2 * w + 1]);
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(acc[u][w]);
        }
        __builtin_nontemporal_store(o, yrow + i);
      }
    }
  }
}

constexpr int kGatherBlocksPerCU = 4, kPushBlocksPerCU = 8, kMergeBlocksPerCU = 16;

hipError_t launch_dispatch(const moe_shape_t& s, const void* const* x, const int32_t* pull_src, char* xe,
                           const int32_t* ctrl, int cus, hipStream_t st) {
  RankPtrs<const char*> xp{};
  for (int r = 0; r < s.R; ++r) xp.p[r] = static_cast<const char*>(x[r]);
  const int row_bytes = s.d * (s.dtype == MOE_F32 ? 4 : 2);
  hipLaunchKernelGGL(dispatch_pull_kernel, dim3(cus * kGatherBlocksPerCU), dim3(256), 0, st, xp, pull_src, ctrl, xe,
                     row_bytes);
  return hipGetLastError();
}

// blk_held: n_mt * 4 int32 of scratch
hipError_t launch_ring_rows(const moe_shape_t& s, int El, int max_mtiles, const void* const* x, const int32_t* pull_src,
                            const int32_t* offsets, const int32_t* mtile_base, const int32_t* ctrl,
                            const int32_t* resident, const void* ring, long long slot_bytes, int n_slots,
                            int chunk_log2, void* xe, uint64_t* blk_src, int32_t* blk_held, uint64_t* row_src, int cus,
                            hipStream_t st) {
  RankPtrs<const char*> xp{};
  for (int r = 0; r < s.R; ++r) xp.p[r] = static_cast<const char*>(x[r]);
  const int row_bytes = s.d * 2;
  hipLaunchKernelGGL(ring_blocks_kernel, dim3((max_mtiles * 4 + 255) / 256), dim3(256), 0, st, offsets, mtile_base,
                     ctrl, resident, static_cast<const char*>(ring), slot_bytes, n_slots, chunk_log2,
                     static_cast<char*>(xe), El, max_mtiles, row_bytes, blk_src, blk_held);
  hipLaunchKernelGGL(ring_rows_kernel, dim3(cus * kGatherBlocksPerCU), dim3(256), 0, st, xp, pull_src, offsets,
                     mtile_base, ctrl, blk_src, blk_held, static_cast<char*>(xe), El, row_bytes, row_src);
  return hipGetLastError();
}

hipError_t launch_push(const moe_shape_t& s, const char* ye, const int32_t* pull_src, const int32_t* slot_of,
                       void* const* recv, const int32_t* ctrl, int cus, hipStream_t st) {
  RankPtrs<char*> rp{};
  for (int r = 0; r < s.R; ++r) rp.p[r] = static_cast<char*>(recv[r]);
  const int row_bytes = s.d * (s.dtype == MOE_F32 ? 4 : 2);
  hipLaunchKernelGGL(combine_push_kernel, dim3(cus * kPushBlocksPerCU), dim3(256), 0, st, ye, pull_src, slot_of, ctrl, rp,
                     s.T, s.k, row_bytes, nullptr, nullptr);
  return hipGetLastError();
}

// push reverse-dispatch: dX rows to recv[r][t][j], their dg to dgp[r][t][j]
hipError_t launch_push_grad(const moe_shape_t& s, const char* dX, const float* dg, const int32_t* pull_src,
                            const int32_t* slot_of, void* const* recv, float* dgp, const int32_t* ctrl, int cus,
                            hipStream_t st) {
  RankPtrs<char*> rp{};
  for (int r = 0; r < s.R; ++r) rp.p[r] = static_cast<char*>(recv[r]);
  hipLaunchKernelGGL(combine_push_kernel, dim3(cus * kPushBlocksPerCU), dim3(256), 0, st, dX, pull_src, slot_of, ctrl, rp,
                     s.T, s.k, s.d * 2, dg, dgp);
  return hipGetLastError();
}

// x: null (no pull table), or the R source buffers
hipError_t launch_pair_addr(const moe_shape_t& s, const int32_t* pull_src, const int32_t* slot_of,
                            void* const* recv, const void* const* x, const int32_t* ctrl, uint64_t* push_dst,
                            uint64_t* pull_addr, int cus, hipStream_t st, const float* dg, float* dgp) {
  RankPtrs<char*> rp{};
  RankPtrs<const char*> xp{};
  for (int r = 0; r < s.R; ++r) {
    rp.p[r] = static_cast<char*>(recv[r]);
    if (x) xp.p[r] = static_cast<const char*>(x[r]);
  }
  const int row_bytes = s.d * (s.dtype == MOE_F32 ? 4 : 2);
  hipLaunchKernelGGL(pair_addr_kernel, dim3(cus * 2), dim3(256), 0, st, pull_src, slot_of, ctrl, rp, xp, s.T, s.k,
                     row_bytes, push_dst, x ? pull_addr : nullptr, dg, dgp);
  return hipGetLastError();
}

hipError_t launch_merge(const moe_shape_t& s, const int32_t* slot_of, const float* topk_w, void* const* recv,
                        void* const* y, int cus, hipStream_t st) {
  RankPtrs<const char*> rcp{};
  RankPtrs<char*> yp{};
  for (int r = 0; r < s.R; ++r) {
    rcp.p[r] = static_cast<const char*>(recv[r]);
    yp.p[r] = static_cast<char*>(y[r]);
  }
  const int n16 = s.d * (s.dtype == MOE_F32 ? 4 : 2) / 16;
  const dim3 grid(cus * kMergeBlocksPerCU);
  if (s.dtype != MOE_F32) {
    if (n16 % (64 * 7) == 0)
      hipLaunchKernelGGL((weighted_merge_kernel<true, 7>), grid, dim3(256), 0, st, rcp, yp, slot_of, topk_w, s.R, s.T,
                         s.k, s.d);
    else
      hipLaunchKernelGGL((weighted_merge_kernel<true, 4>), grid, dim3(256), 0, st, rcp, yp, slot_of, topk_w, s.R, s.T,
                         s.k, s.d);
  } else {
    hipLaunchKernelGGL((weighted_merge_kernel<false, 4>), grid, dim3(256), 0, st, rcp, yp, slot_of, topk_w, s.R, s.T,
                       s.k, s.d);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const moe_shape_t& s, const char* ye, const int32_t* pull_src,
                          const int32_t* slot_of, const float* topk_w, void* const* recv, void* const* y,
                          const int32_t* ctrl, int cus, hipStream_t st) {
  const hipError_t e = launch_push(s, ye, pull_src, slot_of, recv, ctrl, cus, st);
  if (e != hipSuccess) return e;
  return launch_merge(s, slot_of, topk_w, recv, y, cus, st);
}

}  // namespace moe
