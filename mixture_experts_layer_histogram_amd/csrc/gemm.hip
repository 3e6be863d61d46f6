// Grouped SwiGLU expert FFN for gfx950.
//
// Operation (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 01: a grouped GEMM fed with expert-contiguous rows; section 02: SwiGLU in
// the expert path).  For local expert l and its rows [offsets[l], offsets[l+1]):
//   GEMM1: h = silu(X W1^T) * (X W3^T)       X [rows][d], W1/W3 [F][d]
//   GEMM2: y = h W2^T                        W2 [d][F]
// Every operand is K-contiguous (row-major X and h, weights stored [out][in]), so
// each MFMA lane's 8 consecutive K values are one 16-byte LDS read.
//
// bf16 path: 256x256 output tiles, 8 waves (two per SIMD) of 64x128, each a 2x4 grid of
// v_mfma_f32_32x32x16_bf16 tiles; K staged 64 at a time through two LDS buffers
// (2 x 64 KiB) filled by direct global->LDS loads, with an XOR swizzle of the 16-byte
// chunks that keeps the MFMA fragment reads free of bank conflicts.  GEMM1 interleaves 32-row blocks of W1 and W3 in the B tile so
// a lane holds the gate and the up value of the same (row, f) and applies SwiGLU in
// registers.  A persistent grid (one workgroup per CU) walks the tile list; the
// list is split into 8 contiguous ranges, one per XCD (workgroup w runs on XCD
// w mod 8), and ordered expert-major with the row tiles of one expert innermost, so
// the workgroups sharing an XCD's L2 work on one expert's weights at a time.
// Tile -> (expert, row tile) comes from the layout's per-expert tile prefix on the
// device, so the host never reads N.
#include "common.hpp"

namespace moe {

// which local expert owns global row tile mt (binary search on the tile prefix)
__device__ __forceinline__ int find_expert(const int32_t* __restrict__ mtile_base, int El, int mt) {
  int lo = 0, hi = El - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mtile_base[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kStageBytes = (kGemmBM + kGemmBN) * kGemmBK * 2;   // 64 KiB
constexpr int kGemmLds = 2 * kStageBytes;                          // 128 KiB
constexpr int kGemmThreads = 512;                                  // 8 waves, 2 per SIMD

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// LDS byte offset of 16-byte chunk `chunk` of tile row `row` (128-byte rows).  The chunk
// index is XORed with bits 1..3 of the row so that the 16 lanes one ds_read_b128 serves
// per cycle (rows r..r+15 of one chunk column) hit 16 distinct bank groups of the 64-bank
// LDS (row parity picks the half, (row >> 1) & 7 the chunk).
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * (kGemmBK * 2) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// MODE 0: A = xe [*][d], B0 = W1, B1 = W3 -> C = h [*][F]   (tile = 256 rows x 128 f)
// MODE 1: A = h [*][F],  B0 = W2          -> C = ye [*][d]  (tile = 256 rows x 256 cols)
// 8 waves as 4 (rows) x 2 (cols); each wave owns a 64 x 128 block = 2 x 4 MFMA tiles.
// Operands move global -> LDS with global_load_lds_dwordx4 (no VGPR staging): one wave
// instruction fills 8 tile rows (1 KiB); the lane's source chunk is pre-swizzled so the
// linear LDS fill lands in the layout swz_off() reads.
template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, const int32_t* __restrict__ mtile_base,
    const int32_t* __restrict__ ctrl, int El, int K, int Nout) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hi = lane >> 5;
  // LDS fill geometry: lane -> row lrow of an 8-row group, LDS chunk position lpos, which
  // holds logical chunk lpos ^ (((g & 1) * 4 + (lrow >> 1)) & 7) for group g
  const int lrow = lane >> 3, lpos = lane & 7;
  const int lch_even = lpos ^ (lrow >> 1);
  const int lch_odd = lpos ^ (4 + (lrow >> 1));

  const int cols_per_tile = (MODE == 0) ? kGemmBN / 2 : kGemmBN;
  const int NT = (Nout + cols_per_tile - 1) / cols_per_tile;
  const int total = ctrl[kCtrlMTiles] * NT;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int wg_per_xcd = gridDim.x >> 3;
  const int nk = K / kGemmBK;

  for (int tt = blockIdx.x >> 3; tt < per_xcd; tt += wg_per_xcd) {
    const int tau = xcd * per_xcd + tt;
    if (tau >= total) break;
    const int mtg = tau / NT;
    const int l = find_expert(mtile_base, El, mtg);
    const int mt0 = mtile_base[l];
    const int mtl = mtile_base[l + 1] - mt0;
    const int i_in = tau - mt0 * NT;
    const int nt = i_in / mtl, mt = i_in - nt * mtl;
    const int row0 = offsets[l] + mt * kGemmBM;
    const int rows = min(kGemmBM, offsets[l + 1] - row0);
    const int c0 = nt * cols_per_tile;

    // this wave fills row groups g = wave*4 + i (rows g*8 + lrow) of the A and B tiles;
    // rows past the tile's end re-read its last row, B rows past Nout re-read the last one
    const uint16_t* abase = A + size_t(row0) * K;
    const uint16_t* b0base = B0 + size_t(l) * Nout * K;
    const uint16_t* b1base = (MODE == 0) ? B1 + size_t(l) * Nout * K : b0base;
    uint32_t ao[4], bo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (wave * 4 + i) * 8 + lrow;
      const int lch = (i & 1) ? lch_odd : lch_even;
      ao[i] = uint32_t(min(row, rows - 1)) * uint32_t(K) + lch * 8;
      // GEMM1 B tile: 32-row blocks alternate W1 / W3 rows of the same 32 f values
      const int n = (MODE == 0) ? min(c0 + (row >> 6) * 32 + (row & 31), Nout - 1) : min(c0 + row, Nout - 1);
      bo[i] = uint32_t(n) * uint32_t(K) + lch * 8;
    }
    auto bsrc = [&](int i) -> const uint16_t* {
      const int row = (wave * 4 + i) * 8 + lrow;
      return (MODE == 0 && ((row >> 5) & 1)) ? b1base : b0base;
    };
    auto issue = [&](int ks) {
      char* sa = smem + (ks & 1) * kStageBytes;
      char* sb = sa + kGemmBM * kGemmBK * 2;
      const int koff = ks * kGemmBK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = wave * 4 + i;
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(abase + ao[i] + koff),
                                         (lds_void_ptr)(sa + g * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(bsrc(i) + bo[i] + koff),
                                         (lds_void_ptr)(sb + g * 1024), 16, 0, 0);
      }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    issue(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 1 < nk) issue(ks + 1);     // other stage: everyone finished reading it
      const char* sa = smem + (ks & 1) * kStageBytes;
      const char* sb = sa + kGemmBM * kGemmBK * 2;
      bf16x8 fa[2][2], fb[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m) fa[0][m] = *reinterpret_cast<const bf16x8*>(sa + swz_off(wm * 64 + m * 32 + r32, hi));
#pragma unroll
      for (int n = 0; n < 4; ++n) fb[0][n] = *reinterpret_cast<const bf16x8*>(sb + swz_off(wn * 128 + n * 32 + r32, hi));
#pragma unroll
      for (int sub = 0; sub < kGemmBK / 16; ++sub) {
        const int cur = sub & 1;
        if (sub + 1 < kGemmBK / 16) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
            fa[cur ^ 1][m] = *reinterpret_cast<const bf16x8*>(sa + swz_off(wm * 64 + m * 32 + r32, (sub + 1) * 2 + hi));
#pragma unroll
          for (int n = 0; n < 4; ++n)
            fb[cur ^ 1][n] = *reinterpret_cast<const bf16x8*>(sb + swz_off(wn * 128 + n * 32 + r32, (sub + 1) * 2 + hi));
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][m], fb[cur][n], acc[m][n], 0, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);      // this wave's fills of the next stage landed
      __syncthreads();                    // ... and everyone's
    }

    // epilogue: lane holds column r32 and rows 8*(e/4) + 4*hi + e%4 of each 32x32 block
    if (MODE == 0) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int f = c0 + (wn * 2 + q) * 32 + r32;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = wm * 64 + m * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
            if (row < rows && f < Nout) {
              const float h = silu_f32(acc[m][2 * q][e]) * acc[m][2 * q + 1][e];
              C[size_t(row0 + row) * Nout + f] = f32_to_bf16(h);
            }
          }
        }
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int col = c0 + wn * 128 + n * 32 + r32;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = wm * 64 + m * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
            if (row < rows && col < Nout) C[size_t(row0 + row) * Nout + col] = f32_to_bf16(acc[m][n][e]);
          }
        }
    }
  }
}

// fp32 path (small shapes): 64 rows x 64 output columns per tile, 16 rows per thread
template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    float* __restrict__ C, const int32_t* __restrict__ offsets, const int32_t* __restrict__ mtile_base,
    const int32_t* __restrict__ ctrl, int El, int K, int Nout) {
  const int NT = (Nout + kSimtBN - 1) / kSimtBN;
  const int total = ctrl[kCtrlMTiles] * NT;
  const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
  for (int tau = blockIdx.x; tau < total; tau += gridDim.x) {
    const int mtg = tau / NT;
    const int nt = tau - mtg * NT;
    const int l = find_expert(mtile_base, El, mtg);
    const int row0 = offsets[l] + (mtg - mtile_base[l]) * kSimtBM;
    const int rows = min(kSimtBM, offsets[l + 1] - row0);
    const int col = nt * kSimtBN + cl;
    if (col >= Nout) continue;
    float a[16], b[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = b[r] = 0.0f;
    const float* w0 = B0 + (size_t(l) * Nout + col) * K;
    const float* w1 = (MODE == 0) ? B1 + (size_t(l) * Nout + col) * K : nullptr;
    for (int kk = 0; kk < K; ++kk) {
      const float u0 = w0[kk];
      const float u1 = (MODE == 0) ? w1[kk] : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = min(rg * 16 + r, rows - 1);
        const float xv = A[size_t(row0 + row) * K + kk];
        a[r] = fmaf(xv, u0, a[r]);
        if (MODE == 0) b[r] = fmaf(xv, u1, b[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rg * 16 + r;
      if (row < rows) C[size_t(row0 + row) * Nout + col] = (MODE == 0) ? silu_f32(a[r]) * b[r] : a[r];
    }
  }
}

hipError_t launch_ffn(const moe_shape_t& s, int El, const void* xe, const int32_t* offsets, const void* w1,
                      const void* w3, const void* w2, void* ye, char* ws, const WsLayout& L, int cus,
                      hipStream_t st) {
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(ws + L.ctrl);
  const int32_t* mtb = reinterpret_cast<const int32_t*>(ws + L.mtile_base);
  if (s.dtype == MOE_F32) {
    float* h = reinterpret_cast<float*>(ws + L.hbuf);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<0>, dim3(cus * 4), dim3(256), 0, st,
                       static_cast<const float*>(xe), static_cast<const float*>(w1),
                       static_cast<const float*>(w3), h, offsets, mtb, ctrl, El, s.d, s.F);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<1>, dim3(cus * 4), dim3(256), 0, st,
                       static_cast<const float*>(h), static_cast<const float*>(w2), nullptr,
                       static_cast<float*>(ye), offsets, mtb, ctrl, El, s.F, s.d);
    return hipGetLastError();
  }
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<0>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<1>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.hbuf);
  const int grid = (cus / 8) * 8;
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<0>, dim3(grid), dim3(kGemmThreads), kGemmLds, st,
                     static_cast<const uint16_t*>(xe), static_cast<const uint16_t*>(w1),
                     static_cast<const uint16_t*>(w3), h, offsets, mtb, ctrl, El, s.d, s.F);
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<1>, dim3(grid), dim3(kGemmThreads), kGemmLds, st,
                     static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w2), nullptr,
                     static_cast<uint16_t*>(ye), offsets, mtb, ctrl, El, s.F, s.d);
  return hipGetLastError();
}

}  // namespace moe
