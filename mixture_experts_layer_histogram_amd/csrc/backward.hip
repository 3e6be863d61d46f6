// Backward of one GPU's share of the MoE layer on gfx950 (bf16): the kernels around the
// grouped GEMMs.
//
// Operations (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 01: training adds two communication rounds in the opposite direction; section
// 02: the backward's pull reverse-combine and push reverse-dispatch).  With the loss's
// incoming gradient dY of every token output y:
//   pull reverse-combine: expert row s of pair (r, t, j) pulls dO_s = g_j dY[r][t] by the
//     forward's pull schedule; its gate gradient is dg_s = <dY[r][t], o_s>  (o_s = ye[s]);
//   push reverse-dispatch: dX_s goes back to recv[r][t][j] (and dg_s beside it), then an
//     ordered sum over ascending j gives dx[r][t];
//   gate gradient: for the k kept experts of a token dl_j = g_j (dg_j - sum_i g_i dg_i),
//     the other logits get 0; a pair whose expert is not local has dg = 0 here.
// The weight-gradient GEMMs contract over an expert's rows, so their operands are the
// expert rows transposed, one contiguous [cols][K_l] block per expert with K_l its row
// count rounded up to 64 (one K step) and the padding zero; transpose_kernel builds them
// (and the transposed weights the backward's row GEMMs read).  Everything here is
// HBM-bound: 16-byte vectors per lane.
#include "common.hpp"

namespace moe {

// dO[s] = g dY[r][t] (bf16) and dg[s] = <dY[r][t], ye[s]> (fp32), one wave per row
__global__ __launch_bounds__(256) void pull_reverse_kernel(RankPtrs<const char*> dy, const uint16_t* __restrict__ ye,
                                                           const int32_t* __restrict__ pull_src,
                                                           const int32_t* __restrict__ slot_of,
                                                           const float* __restrict__ topk_w,
                                                           const int32_t* __restrict__ ctrl, uint16_t* __restrict__ dO,
                                                           float* __restrict__ dg, int T, int k, int d) {
  constexpr int UNROLL = 8;
  const int N = ctrl[kCtrlN];
  const int lane = threadIdx.x & 63;
  const int n16 = d >> 3;
  const int nw = gridDim.x * 4;
  for (int s = blockIdx.x * 4 + (threadIdx.x >> 6); s < N; s += nw) {
    const int r = pull_src[2 * int64_t(s)];
    const int t = pull_src[2 * int64_t(s) + 1];
    const int64_t pair0 = (int64_t(r) * T + t) * k;
    const unsigned long long hit = __ballot(lane < k && slot_of[pair0 + (lane < k ? lane : 0)] == s);
    const int j = hit ? __builtin_ctzll(hit) : 0;
    const float g = topk_w[pair0 + j];
    const u32x4* src = reinterpret_cast<const u32x4*>(dy.p[r] + int64_t(t) * d * 2);
    const u32x4* yr = reinterpret_cast<const u32x4*>(ye + int64_t(s) * d);
    u32x4* out = reinterpret_cast<u32x4*>(dO + int64_t(s) * d);
    float acc = 0.0f;
    for (int base = 0; base < n16; base += 64 * UNROLL) {
      u32x4 a[UNROLL], b[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = base + u * 64 + lane;
        if (i < n16) {
          a[u] = __builtin_nontemporal_load(src + i);
          b[u] = __builtin_nontemporal_load(yr + i);
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = base + u * 64 + lane;
        if (i < n16) {
          u32x4 o;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float lo = __uint_as_float(a[u][w] << 16), hi = __uint_as_float(a[u][w] & 0xFFFF0000u);
            acc = fmaf(lo, __uint_as_float(b[u][w] << 16), acc);
            acc = fmaf(hi, __uint_as_float(b[u][w] & 0xFFFF0000u), acc);
            o[w] = pack_bf16x2(g * lo, g * hi);
          }
          out[i] = o;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) dg[s] = acc;
  }
}

// poff[l] = sum over l' < l of round_up(offsets[l'+1] - offsets[l'], 64); poff[El] = Np.
// One wave, 64 experts per step.
__global__ __launch_bounds__(64) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int El,
                                                         int32_t* __restrict__ poff) {
  const int lane = threadIdx.x;
  int run = 0;
  for (int base = 0; base < El; base += 64) {
    const int l = base + lane;
    const int v = l < El ? ((offsets[l + 1] - offsets[l] + 63) & ~63) : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (l < El) poff[l] = run + incl - v;
    run += __shfl(incl, 63);
  }
  if (lane == 0) poff[El] = run;
}

// Transposes in 64 x 64 tiles through LDS.
//   poff != nullptr (expert rows): p runs over [0, poff[El]); for p in expert l's padded
//     range, q = p - poff[l] < K_l = poff[l+1] - poff[l], the expert's block [C][K_l] at
//     dst + C * poff[l] gets dst_l[c][q] = src[offsets[l] + q][c], or 0 past its last row.
//     One expert's block is contiguous, so the weight-gradient GEMM reads rows K_l apart.
//   poff == nullptr (weights): `batches` matrices of P rows each (P % 64 == 0),
//     dst[c][p] = src[p][c] with row stride ldt.
// C % 64 == 0; rows of src and dst are 16-byte aligned.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                        int64_t src_bstride, uint16_t* __restrict__ dst, int64_t ldt,
                                                        int64_t dst_bstride, int C, int P, int batches,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ poff, int El) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];   // 144-byte rows: 16-byte aligned
  const int ncb = C >> 6;
  const int npb = poff ? (poff[El] >> 6) : (P >> 6);
  const int64_t tasks = int64_t(poff ? 1 : batches) * npb * ncb;
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const int bt = int(task / (int64_t(npb) * ncb));
    const int rem = int(task - int64_t(bt) * npb * ncb);
    const int pb = rem / ncb, cb = rem - pb * ncb;
    const int p0 = pb * 64, c0 = cb * 64;
    int s0 = p0, s_end = P;
    int64_t dbase = int64_t(bt) * dst_bstride + p0, dld = ldt;
    if (poff) {
      // the expert owning columns [p0, p0 + 64): the last l with poff[l] <= p0
      int lo = 0, hi = El - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
      }
      s0 = offsets[lo] + (p0 - poff[lo]);
      s_end = offsets[lo + 1];
      dld = poff[lo + 1] - poff[lo];
      dbase = int64_t(C) * poff[lo] + (p0 - poff[lo]);
    }
    const uint16_t* sb = src + int64_t(bt) * src_bstride;
    uint16_t* db = dst + dbase;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = threadIdx.x + 256 * i;        // 64 rows x 8 vectors
      const int pr = v >> 3, cv = v & 7;
      const int s = s0 + pr;
      u32x4 val = u32x4{0, 0, 0, 0};
      if (s < s_end) val = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sb + int64_t(s) * ld_src + c0) + cv);
      *reinterpret_cast<u32x4*>(&tile[pr][cv * 8]) = val;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = threadIdx.x + 256 * i;        // 64 output rows x 8 vectors of 8 p
      const int c = v >> 3, pv = v & 7;
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        o[w] = uint32_t(tile[pv * 8 + 2 * w][c]) | (uint32_t(tile[pv * 8 + 2 * w + 1][c]) << 16);
      *reinterpret_cast<u32x4*>(db + int64_t(c0 + c) * dld + pv * 8) = o;
    }
    __syncthreads();
  }
}

// dlogits[r][t][:] = 0 except dl_j at the k kept experts; one wave per token
__global__ __launch_bounds__(256) void gate_grad_kernel(const float* __restrict__ topk_w,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const int32_t* __restrict__ slot_of,
                                                        const float* __restrict__ dgp, RankPtrs<float*> dlog, int R,
                                                        int T, int k, int E) {
  const int lane = threadIdx.x & 63;
  const int64_t tokens = int64_t(R) * T;
  const int64_t nw = int64_t(gridDim.x) * 4;
  for (int64_t g = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); g < tokens; g += nw) {
    const int r = int(g / T), t = int(g - int64_t(r) * T);
    const bool in = lane < k;
    const float gw = in ? topk_w[g * k + lane] : 0.0f;
    const int so = in ? slot_of[g * k + lane] : -1;
    const float dgv = so >= 0 ? dgp[g * k + lane] : 0.0f;
    const int idx = in ? topk_idx[g * k + lane] : -1;
    float S = 0.0f;                                  // sum_j g_j dg_j in ascending j
    for (int j = 0; j < k; ++j) S = fmaf(__shfl(gw, j), __shfl(dgv, j), S);
    const float dl = gw * (dgv - S);
    int ij[16];
    float dj[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      ij[j] = __shfl(idx, j);
      dj[j] = __shfl(dl, j);
    }
    float* row = dlog.p[r] + int64_t(t) * E;
    for (int e = lane; e < E; e += 64) {
      float v = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < k && ij[j] == e) v = dj[j];
      row[e] = v;
    }
  }
}

constexpr int kPullRevBlocksPerCU = 4, kTransposeBlocksPerCU = 8, kGateBlocksPerCU = 4;

hipError_t launch_pull_reverse(const moe_shape_t& s, const void* const* dy, const uint16_t* ye,
                               const int32_t* pull_src, const int32_t* slot_of, const float* topk_w,
                               const int32_t* ctrl, uint16_t* dO, float* dg, int cus, hipStream_t st) {
  RankPtrs<const char*> dp{};
  for (int r = 0; r < s.R; ++r) dp.p[r] = static_cast<const char*>(dy[r]);
  hipLaunchKernelGGL(pull_reverse_kernel, dim3(cus * kPullRevBlocksPerCU), dim3(256), 0, st, dp, ye, pull_src, slot_of,
                     topk_w, ctrl, dO, dg, s.T, s.k, s.d);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int El, int32_t* poff, hipStream_t st) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(64), 0, st, offsets, El, poff);
  return hipGetLastError();
}

hipError_t launch_transpose_rows(const uint16_t* src, int64_t ld_src, uint16_t* dst, int C, const int32_t* offsets,
                                 const int32_t* poff, int El, int cus, hipStream_t st) {
  hipLaunchKernelGGL(transpose_kernel, dim3(cus * kTransposeBlocksPerCU), dim3(256), 0, st, src, ld_src, int64_t(0), dst,
                     int64_t(0), int64_t(0), C, 0, 1, offsets, poff, El);
  return hipGetLastError();
}

hipError_t launch_transpose_batched(const uint16_t* src, int64_t src_bstride, uint16_t* dst, int64_t ldt,
                                    int64_t dst_bstride, int P, int C, int batches, int cus, hipStream_t st) {
  hipLaunchKernelGGL(transpose_kernel, dim3(cus * kTransposeBlocksPerCU), dim3(256), 0, st, src, int64_t(C),
                     src_bstride, dst, ldt, dst_bstride, C, P, batches, nullptr, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_gate_grad(const moe_shape_t& s, const float* topk_w, const int32_t* topk_idx, const int32_t* slot_of,
                            const float* dgp, float* const* dlogits, int cus, hipStream_t st) {
  RankPtrs<float*> lp{};
  for (int r = 0; r < s.R; ++r) lp.p[r] = dlogits[r];
  hipLaunchKernelGGL(gate_grad_kernel, dim3(cus * kGateBlocksPerCU), dim3(256), 0, st, topk_w, topk_idx, slot_of, dgp, lp,
                     s.R, s.T, s.k, s.E);
  return hipGetLastError();
}

}  // namespace moe
