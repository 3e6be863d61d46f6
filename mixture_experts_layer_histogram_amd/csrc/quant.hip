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
// the whole bf16 row (up to 16 KiB) in flight at once.  A workgroup takes `cr` consecutive
// rows at a time and keeps their scale words in LDS (row stride nq + 1 words, so the
// column-wise reads below hit distinct banks); once all its waves are done it writes each
// K-tile plane's cr words as one contiguous run.  Written row by row, every 4-byte scale
// word was a partial write to its own line (56 lines per row at d = 7168).  Measured at the
// DeepSeek-V3 share: 133 us that way, 126 us this way, 116 us with no scale stores at all.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void dispatch_pull_mx_kernel(RankPtrs<const char*> x,
                                                               const int32_t* __restrict__ pull_src,
                                                               const int32_t* __restrict__ ctrl,
                                                               uint8_t* __restrict__ xe,
                                                               uint8_t* __restrict__ xes, int d, int64_t nmax,
                                                               int cr) {
  constexpr int UNROLL = 16;
  extern __shared__ uint32_t s_sc[];           // [cr][nq + 1]
  const int N = ctrl[kCtrlN];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = d >> 3;            // 16-byte source vectors per row (d % 128 == 0: whole 16-lane groups)
  const int nq = d >> 7;             // scale words (K-tile planes) per row
  const int nchunks = (N + cr - 1) / cr;
  uint32_t* xw = reinterpret_cast<uint32_t*>(xes);
  for (int c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int s0 = c * cr, rows = min(cr, N - s0);
    for (int rr = wave; rr < rows; rr += 4) {
      const int s = s0 + rr;
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
          const uint32_t sw = mx_scale_word(sc);          // all lanes: row shifts inside
          if (i < n16) {
            dst[i] = q;
            if ((i & 15) == 0) s_sc[rr * (nq + 1) + (i >> 4)] = sw;
          }
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nq * cr; e += 256) {
      const int q = e / cr, rr = e - q * cr;
      if (rr < rows) xw[nmax * q + s0 + rr] = s_sc[rr * (nq + 1) + q];
    }
    __syncthreads();                 // the next chunk's waves overwrite s_sc
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
  const int cr = mx_chunk_rows(s.d);
  hipLaunchKernelGGL(dispatch_pull_mx_kernel, dim3(cus * kGatherMxBlocksPerCU), dim3(256),
                     size_t(cr) * ((s.d >> 7) + 1) * 4, st, xp, pull_src, ctrl, xe, xe_scales, s.d, nmax, cr);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// MX codes of the transposes of `batches` bf16 matrices [P][C]: for c < C and p < P the
// value src[bt][p][c] becomes element k = k0 + p of row bt * C + c of the code matrix (row
// stride ldk), quantised in blocks of 32 along p; the block scale goes to the MXFP8 scale
// layout of a matrix of `rows_total` rows.  Used for the weights of the backward's
// data-gradient GEMMs, whose K runs along the other axis (W2 along d, W1 and W3 along F).
// 64 (p) x 128 (c) tiles through LDS, filled with 16-byte loads; each of the 256 threads
// then quantises one 32-value column block.  P % 64 == 0, C % 128 == 0.
__global__ __launch_bounds__(256) void mx_quantize_t_kernel(const uint16_t* __restrict__ src, int P, int C, int batches,
                                                            uint8_t* __restrict__ codes, int64_t ldk, int k0,
                                                            uint8_t* __restrict__ scales, int64_t rows_total) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][136];   // 272-byte rows: 16-byte aligned
  const int npb = P >> 6, ncb = C >> 7;
  const int64_t tasks = int64_t(batches) * npb * ncb;
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const int bt = int(task / (int64_t(npb) * ncb));
    const int rem = int(task - int64_t(bt) * npb * ncb);
    const int pb = rem / ncb, cb = rem - pb * ncb;
    const uint16_t* s0 = src + (int64_t(bt) * P + pb * 64) * C + cb * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = threadIdx.x + 256 * i;           // 64 rows x 16 vectors of 8 values
      const int r = v >> 4, cv = v & 15;
      *reinterpret_cast<u32x4*>(&tile[r][cv * 8]) =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s0 + int64_t(r) * C) + cv);
    }
    __syncthreads();
    const int c = threadIdx.x & 127, half = threadIdx.x >> 7;   // column c, p block half
    float v[32];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t b = tile[half * 32 + i][c];
      v[i] = bf16_to_f32(uint16_t(b));
      mx = max(mx, (b << 16) & 0x7FFFFFFFu);
    }
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t sc = 0;
    if (mx != 0) {
      const int e = mx_block_exp(mx);
      const float inv = mx_inv_scale(e);
      sc = uint32_t(e + 127);
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = mx_pack4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], inv);
    }
    const int64_t row = int64_t(bt) * C + cb * 128 + c;
    const int k = k0 + pb * 64 + half * 32;
    u32x4* dst = reinterpret_cast<u32x4*>(codes + row * ldk + k);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    scales[mx_scale_index(rows_total, row, k >> 5)] = uint8_t(sc);
    __syncthreads();
  }
}

hipError_t launch_mx_quantize_t(const uint16_t* src, int P, int C, int batches, uint8_t* codes, int64_t ldk, int k0,
                                uint8_t* scales, int64_t rows_total, int cus, hipStream_t st) {
  hipLaunchKernelGGL(mx_quantize_t_kernel, dim3(cus * 8), dim3(256), 0, st, src, P, C, batches, codes, ldk, k0, scales,
                     rows_total);
  return hipGetLastError();
}

}  // namespace moe
