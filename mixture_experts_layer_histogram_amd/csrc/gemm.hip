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
// the host never reads N.  The fp32 path (small shapes) is a plain SIMT kernel.
#include "gemm_tile.hpp"

namespace moe {

// MODE 0: A = xe [*][d], B0 = W1, B1 = W3 -> C = h [*][F]   (tile = 256 rows x 128 f)
// MODE 1: A = h [*][F],  B0 = W2          -> C = ye [*][d]  (tile = 256 rows x 256 cols), or
//         with RowDst each row s to the address RowDst[s] instead (the push fused in)
// RowSrc (any MODE): A row s read from the address RowSrc[s] instead (the pull fused in)
// MODE 2: as MODE 0, with the backward epilogue: DH in, C = h, DAB = [da | db] out
template <int MODE>
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
    io.row_src = RowSrc ? RowSrc + row0 : nullptr;
    const uint16_t* b0 = B0 + size_t(l) * Nout * K;
    const uint16_t* b1 = (MODE != 1) ? B1 + size_t(l) * Nout * K : b0;
    gemm_tile<MODE>(io, b0, b1, nt * cols_per_tile, Nout, K, smem, K);
  }
}

// fp32 path (small shapes): 64 rows x 64 output columns per tile, 16 rows per thread
template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    float* __restrict__ C, const int32_t* __restrict__ offsets, const int32_t* __restrict__ mtile_base,
    const int32_t* __restrict__ ctrl, int El, int K, int Nout, const uint64_t* __restrict__ RowDst,
    const uint64_t* __restrict__ RowSrc) {
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
        const float xv = RowSrc ? reinterpret_cast<const float*>(RowSrc[row0 + row])[kk] : A[size_t(row0 + row) * K + kk];
        a[r] = fmaf(xv, u0, a[r]);
        if (MODE == 0) b[r] = fmaf(xv, u1, b[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rg * 16 + r;
      if (row < rows) {
        float* dst = (MODE == 1 && RowDst) ? reinterpret_cast<float*>(RowDst[row0 + row]) : C + size_t(row0 + row) * Nout;
        dst[col] = (MODE == 0) ? silu_f32(a[r]) * b[r] : a[r];
      }
    }
  }
}

// the tile's 128 KiB of dynamic LDS, granted once per kernel
hipError_t set_gemm_lds_attrs() {
  static std::atomic<uint64_t> done{0};
  return once_per_device(done, [] {
    const void* ks[] = {reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<0>),
                        reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<1>),
                        reinterpret_cast<const void*>(grouped_gemm_bf16_kernel<2>)};
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
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<0>, dim3(grid), dim3(kGemmThreads), kGemmLds, st,
                     static_cast<const uint16_t*>(xe), static_cast<const uint16_t*>(w1),
                     static_cast<const uint16_t*>(w3), h, offsets, mtb, ctrl, El, s.d, s.F, nullptr, nullptr, nullptr, row_src);
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<1>, dim3(grid), dim3(kGemmThreads), kGemmLds, st,
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
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<2>, dim3((cus / 8) * 8), dim3(kGemmThreads), kGemmLds, st,
                     row_src ? nullptr : xe, w1, w3, h, offsets, mtb, ctrl, El, d, F, dh, dab, nullptr, row_src);
  return hipGetLastError();
}

}  // namespace moe
