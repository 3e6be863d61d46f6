// Grouped SwiGLU expert FFN for gfx950.
//
// Operation (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 01: a grouped GEMM fed with expert-contiguous rows; section 02: SwiGLU in
// the expert path).  For local expert l and its rows [offsets[l], offsets[l+1]):
//   GEMM1: h = silu(X W1^T) * (X W3^T)       X [rows][d], W1/W3 [F][d]
//   GEMM2: y = h W2^T                        W2 [d][F]
// The tile itself (MFMA layout, LDS staging, SwiGLU epilogue) is gemm_tile() in
// gemm_tile.hpp.  Here a persistent grid (one workgroup per CU) walks the tile list; the
// list is split into 8 contiguous ranges, one per XCD (workgroup w runs on XCD w mod 8),
// and ordered expert-major with the row tiles of one expert innermost, so the
// workgroups sharing an XCD's L2 work on one expert's weights at a time.  Tile ->
// (expert, row tile) comes from the layout's per-expert tile prefix on the device, so
// the host never reads N.  The fp32 path (small shapes) runs a smaller fp32-MFMA tile.
#include "gemm_tile.hpp"

namespace moe {

// MODE 0: A = xe [*][d], B0 = W1, B1 = W3 -> C = h [*][F]   (tile = 256 rows x 128 f)
// MODE 1: A = h [*][F],  B0 = W2          -> C = ye [*][d]  (tile = 256 rows x 256 cols), or
//         with RowDst each row s to the address RowDst[s] instead (the push fused in)
// RowSrc (any MODE): A row s read from the address RowSrc[s] instead (the pull fused in)
// MODE 2: as MODE 0, with the backward epilogue: DH in, C = h, DAB = [da | db] out
// ROWSRC: A rows by address (RowSrc, the pull fused in) instead of from A
template <int MODE, bool ROWSRC>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, const int32_t* __restrict__ mtile_base,
    const int32_t* __restrict__ ctrl, int El, int K, int Nout, const uint16_t* __restrict__ DH,
    uint16_t* __restrict__ DAB, const uint64_t* __restrict__ RowDst, const uint64_t* __restrict__ RowSrc) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int cols_per_tile = (MODE != 1) ? kGemmBN / 2 : kGemmBN;
  const int NT = (Nout + cols_per_tile - 1) / cols_per_tile;
  const int total = ctrl[kCtrlMTiles] * NT;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int wg_per_xcd = gridDim.x >> 3;

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
    TileIO io;
    io.a0 = A ? A + size_t(row0) * K : nullptr;        // null A: rows come from RowSrc
    io.a1 = A ? io.a0 + size_t(128) * K : nullptr;
    io.a2 = io.a3 = io.a1;
    io.o0 = C ? C + size_t(row0) * Nout : nullptr;     // null C: MODE 1 with RowDst
    io.o1 = C ? io.o0 + size_t(128) * Nout : nullptr;
    io.o2 = io.o3 = io.o1;
    io.a_ld = K;
    io.o_ld = Nout;
    io.blk_log2 = 7;
    io.rows = min(kGemmBM, offsets[l + 1] - row0);
    io.dh = (MODE == 2) ? DH + size_t(row0) * Nout : nullptr;
    io.dab = (MODE == 2) ? DAB + size_t(row0) * 2 * Nout : nullptr;
    io.row_dst = (MODE == 1 && RowDst) ? RowDst + row0 : nullptr;
    io.row_src = ROWSRC ? RowSrc + row0 : nullptr;
    const uint16_t* b0 = B0 + size_t(l) * Nout * K;
    const uint16_t* b1 = (MODE != 1) ? B1 + size_t(l) * Nout * K : b0;
    gemm_tile<MODE, 0, ROWSRC>(io, b0, b1, nt * cols_per_tile, Nout, K, smem, K);
  }
}

// fp32 path (small shapes) on the fp32 MFMA (v_mfma_f32_32x32x2_f32): a 64-row x 64-column
// output tile per 256-thread workgroup, wave w owning the 32 x 32 block (w >> 1, w & 1); in
// MODE 0 each wave keeps a gate and an up accumulator for the same (row, f), so SwiGLU runs
// in registers.  K steps of 32 staged in LDS (rows padded to 36 floats: a 16-lane
// ds_read_b128 then touches 16 disjoint 4-bank groups); K past the end and rows past the
// tile's end are filled with zeros / the last row.  Within a K step lane l of a wave feeds
// k = 8 c + s (l < 32) or 8 c + 4 + s (l >= 32) to MFMA step s of 8-wide chunk c, so one
// 16-byte LDS read per operand serves four MFMAs.
constexpr int kF32BK = 32, kF32Pitch = kF32BK + 4;

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    float* __restrict__ C, const int32_t* __restrict__ offsets, const int32_t* __restrict__ mtile_base,
    const int32_t* __restrict__ ctrl, int El, int K, int Nout, const uint64_t* __restrict__ RowDst,
    const uint64_t* __restrict__ RowSrc) {
  constexpr int kBRows = (MODE == 0) ? 2 * kF32BN : kF32BN;     // W1 rows then W3 rows
  __shared__ __attribute__((aligned(16))) float sa[kF32BM * kF32Pitch];
  __shared__ __attribute__((aligned(16))) float sb[kBRows * kF32Pitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, r32 = lane & 31, hi = lane >> 5;
  const int NT = (Nout + kF32BN - 1) / kF32BN;
  const int total = ctrl[kCtrlMTiles] * NT;
  for (int tau = blockIdx.x; tau < total; tau += gridDim.x) {
    const int mtg = tau / NT;
    const int nt = tau - mtg * NT;
    const int l = find_expert(mtile_base, El, mtg);
    const int row0 = offsets[l] + (mtg - mtile_base[l]) * kF32BM;
    const int rows = min(kF32BM, offsets[l + 1] - row0);
    const int c0 = nt * kF32BN;
    const float* w0 = B0 + size_t(l) * Nout * K;
    const float* w1 = (MODE == 0) ? B1 + size_t(l) * Nout * K : nullptr;
    f32x16 acc0, acc1;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc0[e] = acc1[e] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += kF32BK) {
      // fills: consecutive threads take consecutive k of one row (128-byte row segments)
      for (int i = tid; i < kF32BM * kF32BK; i += 256) {
        const int r = i / kF32BK, k = i - r * kF32BK;
        const int row = min(r, rows - 1);
        const float* src = RowSrc ? reinterpret_cast<const float*>(RowSrc[row0 + row]) : A + size_t(row0 + row) * K;
        sa[r * kF32Pitch + k] = (k0 + k < K) ? src[k0 + k] : 0.0f;
      }
      for (int i = tid; i < kBRows * kF32BK; i += 256) {
        const int r = i / kF32BK, k = i - r * kF32BK;
        const int n = min(c0 + (r % kF32BN), Nout - 1);
        const float* src = (MODE == 0 && r >= kF32BN) ? w1 : w0;
        sb[r * kF32Pitch + k] = (k0 + k < K) ? src[size_t(n) * K + k0 + k] : 0.0f;
      }
      __syncthreads();
      const float* pa = sa + (wm * 32 + r32) * kF32Pitch + hi * 4;
      const float* pb0 = sb + (wn * 32 + r32) * kF32Pitch + hi * 4;
      const float* pb1 = pb0 + kF32BN * kF32Pitch;
#pragma unroll
      for (int c = 0; c < kF32BK / 8; ++c) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(pa + c * 8);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(pb0 + c * 8);
        f32x4 b1 = b0;
        if (MODE == 0) b1 = *reinterpret_cast<const f32x4*>(pb1 + c * 8);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[st], b0[st], acc0, 0, 0, 0);
          if (MODE == 0) acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[st], b1[st], acc1, 0, 0, 0);
        }
      }
      __syncthreads();                         // the next fills overwrite the tiles
    }
    // lane l holds column wn * 32 + (l & 31), rows wm * 32 + 8 (e >> 2) + 4 (l >> 5) + (e & 3)
    const int col = c0 + wn * 32 + r32;
    if (col < Nout) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (row < rows) {
          float* dst = (MODE == 1 && RowDst) ? reinterpret_cast<float*>(RowDst[row0 + row])
                                              : C + size_t(row0 + row) * Nout;
          dst[col] = (MODE == 0) ? silu_f32(acc0[e]) * acc1[e] : acc0[e];
        }
      }
    }
  }
}

// the tile's 128 KiB of dynamic LDS, granted once per kernel
hipError_t set_gemm_lds_attrs() {
  static std::atomic<uint64_t> done{0};
  return once_per_device(done, [] {
    const void* ks[] = {reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<0, false>),
                        reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<0, true>),
                        reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<1, false>),
                        reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<2, false>),
                        reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<2, true>)};
    for (const void* k : ks) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
}

// row_dst: null (GEMM2 writes ye), or per local pair the address of its output row;
// row_src: null (GEMM1 reads xe), or per local pair the address of its source token row
hipError_t launch_ffn(const moe_shape_t& s, int El, const void* xe, const int32_t* offsets, const void* w1,
                      const void* w3, const void* w2, void* ye, char* ws, const WsLayout& L, int cus,
                      hipStream_t st, const uint64_t* row_dst, const uint64_t* row_src) {
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(ws + L.ctrl);
  const int32_t* mtb = reinterpret_cast<const int32_t*>(ws + L.mtile_base);
  if (s.dtype == MOE_F32) {
    float* h = reinterpret_cast<float*>(ws + L.hbuf);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<0>, dim3(cus * 4), dim3(256), 0, st,
                       static_cast<const float*>(xe), static_cast<const float*>(w1),
                       static_cast<const float*>(w3), h, offsets, mtb, ctrl, El, s.d, s.F, nullptr, row_src);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<1>, dim3(cus * 4), dim3(256), 0, st,
                       static_cast<const float*>(h), static_cast<const float*>(w2), nullptr,
                       static_cast<float*>(ye), offsets, mtb, ctrl, El, s.F, s.d, row_dst, nullptr);
    return hipGetLastError();
  }
  hipError_t e = set_gemm_lds_attrs();
  if (e != hipSuccess) return e;
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.hbuf);
  const int grid = (cus / 8) * 8;
  if (row_src)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<0, true>), dim3(grid), dim3(kGemmThreads), kGemmLds, st, nullptr,
                       static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3), h, offsets, mtb, ctrl, El,
                       s.d, s.F, nullptr, nullptr, nullptr, row_src);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<0, false>), dim3(grid), dim3(kGemmThreads), kGemmLds, st,
                       static_cast<const uint16_t*>(xe), static_cast<const uint16_t*>(w1),
                       static_cast<const uint16_t*>(w3), h, offsets, mtb, ctrl, El, s.d, s.F, nullptr, nullptr, nullptr,
                       nullptr);
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<1, false>), dim3(grid), dim3(kGemmThreads), kGemmLds, st,
                     static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w2), nullptr,
                     static_cast<uint16_t*>(ye), offsets, mtb, ctrl, El, s.F, s.d, nullptr, nullptr, row_dst, nullptr);
  return hipGetLastError();
}

// ---- backward (bf16) ----
// GEMM1 again with the backward epilogue: h and [da | db] from xe, W1, W3 and dh
// row_src: null (token rows from xe), or per local pair the address of its token row
hipError_t launch_gemm1_bwd(const uint16_t* xe, const uint16_t* w1, const uint16_t* w3, const uint16_t* dh,
                            uint16_t* h, uint16_t* dab, int d, int F, const int32_t* offsets, const int32_t* mtb,
                            const int32_t* ctrl, int El, int cus, hipStream_t st, const uint64_t* row_src) {
  hipError_t e = set_gemm_lds_attrs();
  if (e != hipSuccess) return e;
  if (row_src)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<2, true>), dim3((cus / 8) * 8), dim3(kGemmThreads), kGemmLds, st,
                       nullptr, w1, w3, h, offsets, mtb, ctrl, El, d, F, dh, dab, nullptr, row_src);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<2, false>), dim3((cus / 8) * 8), dim3(kGemmThreads), kGemmLds, st,
                       xe, w1, w3, h, offsets, mtb, ctrl, El, d, F, dh, dab, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe
