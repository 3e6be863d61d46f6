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
// The grouped GEMMs of the backward are in gemm_bwd.hip (and GEMM1's backward epilogue in
// gemm_tile.hpp).  Everything here is HBM-bound: 16-byte vectors per lane.
#include "mx.hpp"

namespace moe {

// dO[s] = g dY[r][t] (bf16) and dg[s] = <dY[r][t], o_s> (fp32), one wave per row; o_s is
// ye[s], or with FROM_RECV the pair's recv row recv[r][t][j], where the forward pushed it.
template <bool FROM_RECV>
__global__ __launch_bounds__(256) void pull_reverse_kernel(RankPtrs<const char*> dy, const uint16_t* __restrict__ ye,
                                                           RankPtrs<const char*> recv,
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
    const u32x4* yr = FROM_RECV ? reinterpret_cast<const u32x4*>(recv.p[r] + (int64_t(t) * k + j) * d * 2)
                                : reinterpret_cast<const u32x4*>(ye + int64_t(s) * d);
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

// The MXFP8 variant: dO[s] = g dY[r][t] as bf16 (for the weight gradients) and as MX codes
// of the fp32 products in blocks of 32 along d (for dh = dO W2; scales in the MXFP8 scale
// layout of nmax rows), and dg[s] = <dY[r][t], ye[s]>.  One wave per row, every lane in the
// quad shuffles of the quantiser (lanes past the row end carry zeros).  The dO and code
// stores are non-temporal: measured at the DeepSeek-V3 share the kernel takes 327 us with
// them and 437 us with plain stores (the code stores account for almost all of the
// difference); the bf16 kernel above and the forward's quantising gather are slower with
// non-temporal stores, so they keep plain ones.
__global__ __launch_bounds__(256) void pull_reverse_mx_kernel(RankPtrs<const char*> dy, const uint16_t* __restrict__ ye,
                                                              const int32_t* __restrict__ pull_src,
                                                              const int32_t* __restrict__ slot_of,
                                                              const float* __restrict__ topk_w,
                                                              const int32_t* __restrict__ ctrl,
                                                              uint16_t* __restrict__ dO, uint8_t* __restrict__ dOq,
                                                              uint8_t* __restrict__ dOs, float* __restrict__ dg, int T,
                                                              int k, int d, int64_t nmax) {
  constexpr int UNROLL = 8;
  const int N = ctrl[kCtrlN];
  const int lane = threadIdx.x & 63;
  const int n16 = d >> 3;                 // 16-byte vectors of 8 bf16 (d % 128 == 0: whole 16-lane groups)
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
    uint2* qout = reinterpret_cast<uint2*>(dOq + int64_t(s) * d);
    float acc = 0.0f;
    for (int base = 0; base < n16; base += 64 * UNROLL) {
      u32x4 a[UNROLL], b[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = base + u * 64 + lane;
        a[u] = u32x4{0, 0, 0, 0};
        b[u] = u32x4{0, 0, 0, 0};
        if (i < n16) {
          a[u] = __builtin_nontemporal_load(src + i);
          b[u] = __builtin_nontemporal_load(yr + i);
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = base + u * 64 + lane;
        f32x4 p0, p1;
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = __uint_as_float(a[u][w] << 16), hi = __uint_as_float(a[u][w] & 0xFFFF0000u);
          acc = fmaf(lo, __uint_as_float(b[u][w] << 16), acc);
          acc = fmaf(hi, __uint_as_float(b[u][w] & 0xFFFF0000u), acc);
          const float glo = g * lo, ghi = g * hi;
          if (w < 2) { p0[2 * w] = glo; p0[2 * w + 1] = ghi; } else { p1[2 * w - 4] = glo; p1[2 * w - 3] = ghi; }
          o[w] = pack_bf16x2(glo, ghi);
        }
        uint32_t sc;
        const uint2 q = mx_quant8_f32(p0, p1, &sc);          // all lanes: quad shuffles inside
        const uint32_t sw = mx_scale_word(sc);                // all lanes: row shifts inside
        if (i < n16) {
          __builtin_nontemporal_store(o, out + i);
          __builtin_nontemporal_store(q.x, reinterpret_cast<uint32_t*>(qout + i));
          __builtin_nontemporal_store(q.y, reinterpret_cast<uint32_t*>(qout + i) + 1);
          if ((i & 15) == 0) *reinterpret_cast<uint32_t*>(dOs + mx_scale_index(nmax, s, i >> 2)) = sw;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) dg[s] = acc;
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

constexpr int kPullRevBlocksPerCU = 4, kPullRevMxBlocksPerCU = 8, kGateBlocksPerCU = 4;

// o rows from ye, or (recv != null) from the forward's recv rows
hipError_t launch_pull_reverse(const moe_shape_t& s, const void* const* dy, const uint16_t* ye,
                               const int32_t* pull_src, const int32_t* slot_of, const float* topk_w,
                               const int32_t* ctrl, uint16_t* dO, float* dg, int cus, hipStream_t st,
                               void* const* recv) {
  RankPtrs<const char*> dp{}, rp{};
  for (int r = 0; r < s.R; ++r) {
    dp.p[r] = static_cast<const char*>(dy[r]);
    if (recv) rp.p[r] = static_cast<const char*>(recv[r]);
  }
  if (recv)
    hipLaunchKernelGGL(pull_reverse_kernel<true>, dim3(cus * kPullRevBlocksPerCU), dim3(256), 0, st, dp, ye, rp,
                       pull_src, slot_of, topk_w, ctrl, dO, dg, s.T, s.k, s.d);
  else
    hipLaunchKernelGGL(pull_reverse_kernel<false>, dim3(cus * kPullRevBlocksPerCU), dim3(256), 0, st, dp, ye, rp,
                       pull_src, slot_of, topk_w, ctrl, dO, dg, s.T, s.k, s.d);
  return hipGetLastError();
}

hipError_t launch_pull_reverse_mx(const moe_shape_t& s, const void* const* dy, const uint16_t* ye,
                                  const int32_t* pull_src, const int32_t* slot_of, const float* topk_w,
                                  const int32_t* ctrl, uint16_t* dO, uint8_t* dOq, uint8_t* dOs, float* dg, int64_t nmax,
                                  int cus, hipStream_t st) {
  RankPtrs<const char*> dp{};
  for (int r = 0; r < s.R; ++r) dp.p[r] = static_cast<const char*>(dy[r]);
  hipLaunchKernelGGL(pull_reverse_mx_kernel, dim3(cus * kPullRevMxBlocksPerCU), dim3(256), 0, st, dp, ye, pull_src,
                     slot_of, topk_w, ctrl, dO, dOq, dOs, dg, s.T, s.k, s.d, nmax);
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
