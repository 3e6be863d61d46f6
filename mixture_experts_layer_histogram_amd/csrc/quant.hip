// MXFP8 quantisers on gfx950: the standalone row quantiser (expert weights, offline) and
// the pull dispatch that quantises each gathered token row on its way into the expert
// rows (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 02: quantisation fused into the dispatch data path; section 02 also gives the
// pull: the expert side reads each row it needs from its source buffer).
//
// A lane holds one 16-byte vector of 8 bf16 values; an aligned lane quad holds one
// 32-value block, so the block maximum is two quad shuffles.  Both kernels are HBM-bound:
// per element they read 2 (bf16) or 4 (fp32) bytes and write 1 + 1/32.
#include "mx.hpp"

namespace moe {

// codes[i] for the n8 groups of 8 consecutive values of src ([rows][K]); the scale of each
// 32-value block goes to its place in the K-tile-major scale layout
template <bool BF16>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const void* __restrict__ src, int64_t n8, int64_t rows,
                                                          int K, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int g8 = K >> 3;             // groups of 8 per row
  // n8 is a multiple of 4, so every lane quad is either wholly inside or wholly outside
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < n8; t += stride) {
    uint32_t sc;
    uint2 q;
    if (BF16) {
      const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(src) + t);
      q = mx_quant8_bf16(v, &sc);
    } else {
      const f32x4* p = static_cast<const f32x4*>(src) + 2 * t;
      q = mx_quant8_f32(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1), &sc);
    }
    reinterpret_cast<uint2*>(codes)[t] = q;
    if ((t & 3) == 0) {
      const int64_t r = t / g8;
      scales[mx_scale_index(rows, r, int(t - r * g8) >> 2)] = uint8_t(sc);
    }
  }
}

// xe[s] / xe_scales[s] = MX(x[pull_src[s].rank][pull_src[s].token]); one wave per row,
// the whole bf16 row (up to 16 KiB) in flight at once.
__global__ __launch_bounds__(256) void dispatch_pull_mx_kernel(RankPtrs<const char*> x,
                                                               const int32_t* __restrict__ pull_src,
                                                               const int32_t* __restrict__ ctrl,
                                                               uint8_t* __restrict__ xe,
                                                               uint8_t* __restrict__ xes, int d, int64_t nmax) {
  constexpr int UNROLL = 16;
  const int N = ctrl[kCtrlN];
  const int lane = threadIdx.x & 63;
  const int n16 = d >> 3;            // 16-byte source vectors per row (d % 32 == 0: whole quads)
  const int nw = gridDim.x * 4;
  for (int s = blockIdx.x * 4 + (threadIdx.x >> 6); s < N; s += nw) {
    const int r = pull_src[2 * int64_t(s)];
    const int t = pull_src[2 * int64_t(s) + 1];
    const u32x4* src = reinterpret_cast<const u32x4*>(x.p[r] + int64_t(t) * d * 2);
    uint2* dst = reinterpret_cast<uint2*>(xe + int64_t(s) * d);
    for (int base = 0; base < n16; base += 64 * UNROLL) {
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = base + u * 64 + lane;
        v[u] = u32x4{0, 0, 0, 0};
        if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = base + u * 64 + lane;
        uint32_t sc;
        const uint2 q = mx_quant8_bf16(v[u], &sc);     // all lanes: quad shuffles inside
        if (i < n16) {
          dst[i] = q;
          if ((i & 3) == 0) xes[mx_scale_index(nmax, s, i >> 2)] = uint8_t(sc);
        }
      }
    }
  }
}

constexpr int kQuantBlocksPerCU = 8, kGatherMxBlocksPerCU = 4;

hipError_t launch_mx_quantize(const void* src, int src_dtype, int64_t rows, int K, uint8_t* codes,
                              uint8_t* scales, int cus, hipStream_t st) {
  const int64_t n8 = rows * (K / 8);
  if (n8 == 0) return hipSuccess;
  const int64_t need = (n8 + 255) / 256;
  const int grid = int(need < int64_t(cus) * kQuantBlocksPerCU ? need : int64_t(cus) * kQuantBlocksPerCU);
  if (src_dtype == MOE_BF16)
    hipLaunchKernelGGL(mx_quantize_kernel<true>, dim3(grid), dim3(256), 0, st, src, n8, rows, K, codes, scales);
  else
    hipLaunchKernelGGL(mx_quantize_kernel<false>, dim3(grid), dim3(256), 0, st, src, n8, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_dispatch_mx(const moe_shape_t& s, const void* const* x, const int32_t* pull_src, uint8_t* xe,
                              uint8_t* xe_scales, int64_t nmax, const int32_t* ctrl, int cus, hipStream_t st) {
  RankPtrs<const char*> xp{};
  for (int r = 0; r < s.R; ++r) xp.p[r] = static_cast<const char*>(x[r]);
  hipLaunchKernelGGL(dispatch_pull_mx_kernel, dim3(cus * kGatherMxBlocksPerCU), dim3(256), 0, st, xp, pull_src, ctrl,
                     xe, xe_scales, s.d, nmax);
  return hipGetLastError();
}

}  // namespace moe
