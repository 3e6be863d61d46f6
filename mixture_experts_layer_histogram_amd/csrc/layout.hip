// Routing and sort-free layout generation for gfx950.
//
// Operation (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 01; qubstore.ru "Смесь котят ...", pull paragraph): every token keeps its
// k best experts; the expert side counts pairs per expert, takes an exclusive
// prefix over its local experts and gives each pair a destination row so that one
// expert's rows are contiguous, recording only (source rank, source token) -- a
// two-column pull schedule built without sorting.
//
// Three launches:
//   1. topk_hist   : one 16-lane group per token (4 tokens per wave, a block's 64
//                    tokens at once for E <= 256); k rounds of a 16-lane max over
//                    packed (logit, ~id) keys; gate = softmax over the kept logits;
//                    per-block expert histogram in LDS.
//   2. layout_scan : block 0 validates the placement, scans the local experts'
//                    block histograms (flattened exclusive scan = offsets and
//                    per-block bases at once) and the GEMM-tile / chunk tables;
//                    blocks 1.. reduce the global per-expert counts.
//   3. slot_assign : one wave per histogram block walks its pairs in (r, t, j)
//                    order; equal-expert lanes are found with ballots over the id
//                    bits, ranked with a popcount, offset by an LDS running count.
#include "common.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// packed ordering key: larger key = larger logit, ties -> lower expert id
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long make_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0u) u = 0u;                           // -0.0 orders like +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);       // monotone float -> uint
  return (static_cast<unsigned long long>(u) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_value(unsigned long long key) {
  uint32_t u = static_cast<uint32_t>(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_expert(unsigned long long key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// VPL = logits held per lane (E <= 16 * VPL); NT threads per block, so NT / 16 tokens in
// flight per pass over the block's kTokPerLayoutBlock tokens.  With up to 256 experts the
// block has 1024 threads (every token of the block in one pass) and the ordering keys are
// built once per token; wider rows keep 256 threads and rebuild the keys every round.
template <int VPL, int NT>
__global__ __launch_bounds__(NT) void topk_hist_kernel(RankPtrs<const float*> logits, int R, int T,
                                                       int E, int k, int32_t* __restrict__ topk_idx,
                                                       float* __restrict__ topk_w,
                                                       int32_t* __restrict__ blockhist) {
  constexpr bool kKeys = VPL <= 16;        // keys kept in registers
  constexpr int kGroups = NT / 16;         // tokens in flight per pass
  __shared__ int hist[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += NT) hist[e] = 0;
  __syncthreads();

  const int grp = tid >> 4, sl = tid & 15;
  const int64_t RT = int64_t(R) * T;
  const int64_t tok0 = int64_t(blockIdx.x) * kTokPerLayoutBlock;

#pragma unroll 1
  for (int pass = 0; pass < kTokPerLayoutBlock / kGroups; ++pass) {
    const int64_t g = tok0 + pass * kGroups + grp;
    const bool valid = g < RT;
    float v[VPL];
    if (valid) {
      const int r = int(g / T);
      const int t = int(g - int64_t(r) * T);
      const float* row = logits.p[r] + size_t(t) * E;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = sl + 16 * i;
        v[i] = (e < E) ? row[e] : 0.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPL; ++i) v[i] = 0.0f;
    }
    unsigned long long keys[kKeys ? VPL : 1];
    if constexpr (kKeys) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = sl + 16 * i;
        keys[i] = (e < E) ? make_key(v[i], e) : 0ull;       // 0 is below every real key
      }
    }

    unsigned long long taken = 0ull;
    int my_idx = 0;
    float my_val = 0.0f;
    for (int j = 0; j < k; ++j) {
      unsigned long long best = 0ull;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = sl + 16 * i;
        const unsigned long long key = kKeys ? keys[i] : make_key(v[i], e);
        const bool ok = (e < E) && !((taken >> i) & 1ull);
        best = (ok && key > best) ? key : best;
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off, 16);
        best = o > best ? o : best;
      }
      const int ew = key_expert(best);
      if ((ew & 15) == sl) taken |= 1ull << (ew >> 4);
      if (sl == j) {
        my_idx = ew;
        my_val = key_value(best);
      }
    }
    // gate: softmax over the kept logits, max = the first kept logit
    const float m = __shfl(my_val, 0, 16);
    const float z = (sl < k) ? expf(my_val - m) : 0.0f;
    float zs = z;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) zs += __shfl_xor(zs, off, 16);
    if (valid && sl < k) {
      topk_idx[g * k + sl] = my_idx;
      topk_w[g * k + sl] = z / zs;
      atomicAdd(&hist[my_idx], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) blockhist[size_t(blockIdx.x) * E + e] = hist[e];
}

// exclusive scan over a 1024-thread block; returns the thread's exclusive prefix
__device__ int block_excl_scan_1024(int v, int* tmp16, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp16[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = (lane < 16) ? tmp16[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(s, off, 64);
      if (lane >= off) s += y;
    }
    if (lane < 16) tmp16[lane] = s;
  }
  __syncthreads();
  const int excl = (w > 0 ? tmp16[w - 1] : 0) + x - v;
  *total = tmp16[15];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(1024) void layout_scan_kernel(
    const int32_t* __restrict__ e2l, int E, int El, int nb, int bm, int mb,
    const int32_t* __restrict__ blockhist, int32_t* __restrict__ blockbase,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ l2g,
    int32_t* __restrict__ mtile_base, int32_t* __restrict__ chunk_base, int32_t* __restrict__ ctrl) {
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    // global per-expert counts: 16 threads per expert
    const int e = (blockIdx.x - 1) * 64 + (tid >> 4), q = tid & 15;
    int sum = 0;
    if (e < E) {
#pragma unroll 8
      for (int b = q; b < nb; b += 16) sum += blockhist[size_t(b) * E + e];
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 16);
    if (e < E && q == 0) counts[e] = sum;
    return;
  }

  __shared__ int seen[1024];
  __shared__ int l2g_s[1024];
  __shared__ int col_off[1025];
  __shared__ int tmp16[16];
  __shared__ int bad;
  for (int l = tid; l < El; l += 1024) seen[l] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    const int l = e2l[e];
    if (l < -1 || l >= El) {
      atomicOr(&bad, 1);
    } else if (l >= 0) {
      atomicAdd(&seen[l], 1);
      l2g_s[l] = e;
    }
  }
  __syncthreads();
  for (int l = tid; l < El; l += 1024)
    if (seen[l] != 1) atomicOr(&bad, 1);
  __syncthreads();
  if (bad) {
    for (int l = tid; l <= El; l += 1024) {
      offsets[l] = 0;
      mtile_base[l] = 0;
      chunk_base[l] = 0;
    }
    if (tid == 0) {
      ctrl[kCtrlStatus] = MOE_EINVAL;
      ctrl[kCtrlN] = 0;
      ctrl[kCtrlMTiles] = 0;
      ctrl[kCtrlChunks] = 0;
    }
    return;
  }
  for (int l = tid; l < El; l += 1024) l2g[l] = l2g_s[l];

  // flattened (column, segment) exclusive scan: column c = local expert, segment q
  // = a run of histogram blocks.  Its value at (c, q) is offsets[c] plus all earlier
  // segments of column c, i.e. the base row of the segment's first block.
  int p2 = 1;
  while (p2 < El) p2 <<= 1;
  const int tpc = 1024 / p2;                 // threads per column (>= 1; El <= 1024)
  const int c = tid / tpc, q = tid - c * tpc;
  const int seg = (nb + tpc - 1) / tpc;
  const int b0 = q * seg, b1 = min(nb, b0 + seg);
  // a thread's segment of at most kSegRegs blocks is loaded once, all loads in flight
  // together, and kept in registers for the second pass
  constexpr int kSegRegs = 16;
  int hv[kSegRegs];
  int mysum = 0;
  const int col = (c < El) ? l2g_s[c] : 0;
  if (c < El) {
    if (seg <= kSegRegs) {
#pragma unroll
      for (int i = 0; i < kSegRegs; ++i) {
        const int b = b0 + i;
        hv[i] = (b < b1) ? blockhist[size_t(b) * E + col] : 0;
      }
#pragma unroll
      for (int i = 0; i < kSegRegs; ++i) mysum += hv[i];
    } else {
      for (int b = b0; b < b1; ++b) mysum += blockhist[size_t(b) * E + col];
    }
  }
  int N = 0;
  const int ex = block_excl_scan_1024(mysum, tmp16, &N);
  if (c < El) {
    int run = ex;
    if (seg <= kSegRegs) {
#pragma unroll
      for (int i = 0; i < kSegRegs; ++i) {
        const int b = b0 + i;
        if (b < b1) blockbase[size_t(b) * El + c] = run;
        run += hv[i];
      }
    } else {
      for (int b = b0; b < b1; ++b) {
        blockbase[size_t(b) * El + c] = run;
        run += blockhist[size_t(b) * E + col];
      }
    }
    if (q == 0) col_off[c] = ex;
  }
  if (tid == 0) col_off[El] = N;
  __syncthreads();
  for (int l = tid; l <= El; l += 1024) offsets[l] = col_off[l];

  // per-expert GEMM row tiles (bm rows) and minibatch chunks (mb rows)
  int cnt = (tid < El) ? col_off[tid + 1] - col_off[tid] : 0;
  int nt_total = 0, nc_total = 0;
  const int mt_ex = block_excl_scan_1024((cnt + bm - 1) / bm, tmp16, &nt_total);
  const int ch_ex = block_excl_scan_1024((cnt + mb - 1) / mb, tmp16, &nc_total);
  if (tid < El) {
    mtile_base[tid] = mt_ex;
    chunk_base[tid] = ch_ex;
  }
  if (tid == 0) {
    mtile_base[El] = nt_total;
    chunk_base[El] = nc_total;
    ctrl[kCtrlN] = N;
    ctrl[kCtrlMTiles] = nt_total;
    ctrl[kCtrlChunks] = nc_total;
    ctrl[kCtrlStatus] = MOE_OK;
  }
}

__global__ __launch_bounds__(64) void slot_assign_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ e2l, int R, int T, int E, int k,
    int El, const int32_t* __restrict__ blockbase, const int32_t* __restrict__ ctrl,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ pull_src) {
  __shared__ int cnt[1024];
  __shared__ int map[1024];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) map[e] = e2l[e];
  for (int l = lane; l < El; l += 64) cnt[l] = 0;
  __syncthreads();
  const bool ok = ctrl[kCtrlStatus] == MOE_OK;
  const int64_t RT = int64_t(R) * T;
  const int64_t g0 = int64_t(blockIdx.x) * kTokPerLayoutBlock;
  const int64_t g1 = min(g0 + kTokPerLayoutBlock, RT);
  const int64_t p0 = g0 * k, p1 = g1 * k;
  const int nbits = 32 - __clz(El);          // bits of (l + 1) in [0, El]
  const int32_t* base = blockbase + size_t(blockIdx.x) * El;
  const unsigned long long below = (1ull << lane) - 1ull;

  for (int64_t pb = p0; pb < p1; pb += 64) {
    const int64_t p = pb + lane;
    const bool inr = p < p1;
    int l = -1;
    if (inr && ok) l = map[topk_idx[p]];
    const int key = l + 1;
    unsigned long long m = __ballot(l >= 0);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const unsigned long long bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    if (inr) {
      if (l >= 0) {
        const int slot = base[l] + cnt[l] + __popcll(m & below);
        slot_of[p] = slot;
        const int64_t g = p / k;
        const int r = int(g / T);
        pull_src[2 * int64_t(slot)] = r;
        pull_src[2 * int64_t(slot) + 1] = int(g - int64_t(r) * T);
      } else {
        slot_of[p] = -1;
      }
    }
    __syncthreads();
    if (l >= 0 && (m >> lane) == 1ull) cnt[l] += __popcll(m);
    __syncthreads();
  }
}

template <int VPL>
static void launch_topk(dim3 grid, hipStream_t st, const RankPtrs<const float*>& lp, const moe_shape_t& s,
                        int32_t* topk_idx, float* topk_w, int32_t* blockhist) {
  constexpr int NT = VPL <= 16 ? 1024 : 256;
  hipLaunchKernelGGL((topk_hist_kernel<VPL, NT>), grid, dim3(NT), 0, st, lp, s.R, s.T, s.E, s.k, topk_idx,
                     topk_w, blockhist);
}

hipError_t launch_layout(const moe_shape_t& s, const int32_t* e2l, int El, int mb,
                         const float* const* logits, int32_t* topk_idx, float* topk_w, int32_t* counts,
                         int32_t* offsets, int32_t* pull_src, int32_t* slot_of, char* ws,
                         const WsLayout& L, hipStream_t st) {
  RankPtrs<const float*> lp{};
  for (int r = 0; r < s.R; ++r) lp.p[r] = logits[r];
  int32_t* blockhist = reinterpret_cast<int32_t*>(ws + L.blockhist);
  int32_t* blockbase = reinterpret_cast<int32_t*>(ws + L.blockbase);
  int32_t* ctrl = reinterpret_cast<int32_t*>(ws + L.ctrl);
  const dim3 grid(L.nb);
  const int vpl_need = (s.E + 15) / 16;
  if (vpl_need <= 1) launch_topk<1>(grid, st, lp, s, topk_idx, topk_w, blockhist);
  else if (vpl_need <= 2) launch_topk<2>(grid, st, lp, s, topk_idx, topk_w, blockhist);
  else if (vpl_need <= 4) launch_topk<4>(grid, st, lp, s, topk_idx, topk_w, blockhist);
  else if (vpl_need <= 8) launch_topk<8>(grid, st, lp, s, topk_idx, topk_w, blockhist);
  else if (vpl_need <= 16) launch_topk<16>(grid, st, lp, s, topk_idx, topk_w, blockhist);
  else if (vpl_need <= 32) launch_topk<32>(grid, st, lp, s, topk_idx, topk_w, blockhist);
  else launch_topk<64>(grid, st, lp, s, topk_idx, topk_w, blockhist);

  const int bm = (s.dtype == MOE_F32) ? kF32BM : kGemmBM;
  hipLaunchKernelGGL(layout_scan_kernel, dim3(1 + (s.E + 63) / 64), dim3(1024), 0, st, e2l, s.E, El,
                     L.nb, bm, mb, blockhist, blockbase, counts, offsets,
                     reinterpret_cast<int32_t*>(ws + L.l2g), reinterpret_cast<int32_t*>(ws + L.mtile_base),
                     reinterpret_cast<int32_t*>(ws + L.chunk_base), ctrl);
  hipLaunchKernelGGL(slot_assign_kernel, grid, dim3(64), 0, st, topk_idx, e2l, s.R, s.T, s.E, s.k, El,
                     blockbase, ctrl, slot_of, pull_src);
  return hipGetLastError();
}

}  // namespace moe
