// Grouped SwiGLU expert FFN in MXFP8 on gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Operation (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// section 01: grouped GEMM over expert-contiguous rows; section 02: SwiGLU, and MXFP8
// quantisation fused into the grouped-GEMM and SwiGLU data paths):
//   GEMM1: h = MX(silu(X W1^T) * (X W3^T))   X, W1, W3 in MXFP8 (blocks of 32 along d)
//   GEMM2: y = h W2^T (bf16 out)              h, W2 in MXFP8 (blocks of 32 along F)
// h is quantised in GEMM1's epilogue, so it reaches HBM once, at one byte per value.
//
// The tile mirrors the bf16 one (256 x 256, 8 waves as 4 x 2, direct global->LDS fills,
// the same XOR swizzle of 16-byte chunks in 128-byte LDS rows) with 128 K values per
// stage, plus one 32-bit word of four E8M0 scales per tile row and stage, fetched into LDS
// by one more direct load per wave.  Scale arrays are K-tile-major (one plane of 32-bit
// words per 128-value K tile, rows consecutive inside a plane), so that load reads 256
// contiguous bytes; with row-major scales the same load touched 64 lines and cost a quarter
// of GEMM1's time.  Lane layout of the scaled MFMA (checked on the
// device): lane (row r32, half hi) supplies K chunks hi and 2 + hi (16 values each) of
// the 64-value step, and the scale of block hi of that step; so a lane shifts its row's
// scale word right by 8 * hi and selects byte 0 or 2 with op_sel for the two steps.
#include "gemm_mx_tile.hpp"

namespace moe {

// MODE 0: A = xe codes [*][d], B0/B1 = W1/W3 -> h codes [*][F] + scales   (256 rows x 128 f)
// MODE 1: A = codes [*][K],    B0 = codes [Nout][K] per expert -> bf16 [*][Nout]   (256 x 256)
//         (GEMM2 y = h W2^T; in the backward dh = dO W2 and dX = [da | db] [W1; W3], with
//         the weights quantised along the backward's K)
// MODE 2: as MODE 0 with the backward epilogue: DH in; HB, DAB (bf16) and DABQ/DABS out
// Tile enumeration as in the bf16 grouped GEMM: a persistent grid walks 8 contiguous
// per-XCD ranges of the expert-major tile list.
template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B0,
    const uint8_t* __restrict__ B1, const uint8_t* __restrict__ Bs0, const uint8_t* __restrict__ Bs1,
    void* __restrict__ C, uint8_t* __restrict__ Cs, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ mtile_base, const int32_t* __restrict__ ctrl, int El, int K, int Nout,
    int64_t nmax, const uint16_t* __restrict__ DH, uint16_t* __restrict__ DAB, uint8_t* __restrict__ DABQ,
    uint8_t* __restrict__ DABS, const uint64_t* __restrict__ RowDst) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int cols_per_tile = (MODE != 1) ? kGemmBN / 2 : kGemmBN;
  const int NT = (Nout + cols_per_tile - 1) / cols_per_tile;
  const int total = ctrl[kCtrlMTiles] * NT;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int wg_per_xcd = gridDim.x >> 3;
  const int64_t bs_plane = 4 * int64_t(El) * Nout;    // weight scale planes hold every expert's rows

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
    TileMX io;
    io.a = A + size_t(row0) * K;
    io.as = As + 4 * size_t(row0);
    io.as_plane = 4 * nmax;
    if (MODE == 0) {
      io.o = static_cast<uint8_t*>(C) + size_t(row0) * Nout;
      io.os = Cs + 4 * size_t(row0);
      io.os_plane = 4 * nmax;
    } else {
      io.o = C ? static_cast<uint16_t*>(C) + size_t(row0) * Nout : nullptr;   // null C: MODE 1 with RowDst
      io.os = nullptr;
      io.os_plane = 0;
    }
    io.rows = min(kGemmBM, offsets[l + 1] - row0);
    io.dh = (MODE == 2) ? DH + size_t(row0) * Nout : nullptr;
    io.hb = (MODE == 2) ? static_cast<uint16_t*>(C) + size_t(row0) * Nout : nullptr;
    io.dab = (MODE == 2) ? DAB + size_t(row0) * 2 * Nout : nullptr;
    io.dabq = (MODE == 2) ? DABQ + size_t(row0) * 2 * Nout : nullptr;
    io.dabs = DABS;
    io.row0 = row0;
    io.nmax = nmax;
    io.row_dst = (MODE == 1 && RowDst) ? RowDst + row0 : nullptr;
    const uint8_t* b0 = B0 + size_t(l) * Nout * K;
    const uint8_t* b1 = (MODE != 1) ? B1 + size_t(l) * Nout * K : b0;
    const uint8_t* bs0 = Bs0 + 4 * size_t(l) * Nout;
    const uint8_t* bs1 = (MODE != 1) ? Bs1 + 4 * size_t(l) * Nout : bs0;
    gemm_mx_tile<MODE>(io, b0, b1, bs0, bs1, bs_plane, nt * cols_per_tile, Nout, K, smem);
  }
}

// h codes at hbuf, h scales after them (both within the workspace's h staging region)
size_t mx_h_scales_offset(const WsLayout& L, const moe_shape_t& s) {
  return L.hbuf + align256(size_t(L.max_pairs) * s.F);
}

hipError_t launch_ffn_mx(const moe_shape_t& s, int El, const uint8_t* xe, const uint8_t* xe_scales,
                         const int32_t* offsets, const uint8_t* w1, const uint8_t* w3, const uint8_t* w2,
                         const uint8_t* w1s, const uint8_t* w3s, const uint8_t* w2s, void* ye, char* ws,
                         const WsLayout& L, int cus, hipStream_t st, const uint64_t* row_dst) {
  static std::atomic<uint64_t> attr_set{0};
  const hipError_t ea = once_per_device(attr_set, [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(grouped_gemm_mx_kernel<0>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(grouped_gemm_mx_kernel<1>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
    return e;
  });
  if (ea != hipSuccess) return ea;
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(ws + L.ctrl);
  const int32_t* mtb = reinterpret_cast<const int32_t*>(ws + L.mtile_base);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hbuf);
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + mx_h_scales_offset(L, s));
  const int grid = (cus / 8) * 8;
  hipLaunchKernelGGL(grouped_gemm_mx_kernel<0>, dim3(grid), dim3(kGemmThreads), kMxLds, st, xe, xe_scales, w1, w3,
                     w1s, w3s, static_cast<void*>(hq), hs, offsets, mtb, ctrl, El, s.d, s.F, int64_t(L.max_pairs),
                     nullptr, nullptr, nullptr, nullptr, nullptr);
  hipLaunchKernelGGL(grouped_gemm_mx_kernel<1>, dim3(grid), dim3(kGemmThreads), kMxLds, st, hq, hs, w2, nullptr,
                     w2s, nullptr, ye, nullptr, offsets, mtb, ctrl, El, s.F, s.d, int64_t(L.max_pairs), nullptr, nullptr,
                     nullptr, nullptr, row_dst);
  return hipGetLastError();
}

hipError_t set_mx_bwd_lds_attrs() {
  static std::atomic<uint64_t> done{0};
  return once_per_device(done, [] {
    const void* ks[] = {reinterpret_cast<const void*>(grouped_gemm_mx_kernel<1>),
                        reinterpret_cast<const void*>(grouped_gemm_mx_kernel<2>)};
    for (const void* k : ks) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
}

// C[s] = A[s] B_l^T in MXFP8 for the rows of every local expert: A codes [*][K] with scales
// of nmax rows, B codes [E_local][Nout][K] with scales of E_local * Nout rows; bf16 out.
hipError_t launch_rows_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, uint16_t* C, int K,
                          int Nout, int64_t nmax, const int32_t* offsets, const int32_t* mtb, const int32_t* ctrl,
                          int El, int cus, hipStream_t st, const uint64_t* row_dst) {
  hipError_t e = set_mx_bwd_lds_attrs();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(grouped_gemm_mx_kernel<1>, dim3((cus / 8) * 8), dim3(kGemmThreads), kMxLds, st, A, As, B, nullptr,
                     Bs, nullptr, static_cast<void*>(C), nullptr, offsets, mtb, ctrl, El, K, Nout, nmax, nullptr,
                     nullptr, nullptr, nullptr, row_dst);
  return hipGetLastError();
}

// GEMM1 again in MXFP8 with the backward epilogue: h, [da | db] (bf16) and [da | db] codes
hipError_t launch_gemm1_bwd_mx(const uint8_t* xe, const uint8_t* xes, const uint8_t* w1, const uint8_t* w3,
                               const uint8_t* w1s, const uint8_t* w3s, const uint16_t* dh, uint16_t* h, uint16_t* dab,
                               uint8_t* dabq, uint8_t* dabs, int d, int F, int64_t nmax, const int32_t* offsets,
                               const int32_t* mtb, const int32_t* ctrl, int El, int cus, hipStream_t st) {
  hipError_t e = set_mx_bwd_lds_attrs();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(grouped_gemm_mx_kernel<2>, dim3((cus / 8) * 8), dim3(kGemmThreads), kMxLds, st, xe, xes, w1, w3,
                     w1s, w3s, static_cast<void*>(h), nullptr, offsets, mtb, ctrl, El, d, F, nmax, dh, dab, dabq, dabs,
                     nullptr);
  return hipGetLastError();
}

}  // namespace moe
