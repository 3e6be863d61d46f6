// The backward's grouped GEMMs on gfx950 (bf16 MFMA), reading every operand as stored.
//
// The backward (MoK article, kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
// sections 01-03: training adds a backward pass, sped up like the forward) multiplies by
// the expert weights in the other orientation (dh = dO W2, dX = da W1 + db W3) and
// contracts over an expert's rows for the weight gradients (dW1 = da^T x, dW3 = db^T x,
// dW2 = dO^T h).  Those operands are stored with M or N contiguous ("MN-major") rather than
// K contiguous.  gfx950's transposing LDS read ds_read_b64_tr_b16 turns an MN-major LDS
// tile into the K-contiguous fragments v_mfma_f32_32x32x16_bf16 wants, so nothing is
// transposed in HBM: the tile is staged row-major in K, and each lane's 8 consecutive K
// values of one column come from two transposing reads.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, lane 16g + 4a + b receives, as its
// 4 halfwords c = 0..3, halfword b of the 8 bytes addressed by lane 16g + a + 4c (lane
// layout measured on MI355X).  So a lane addressing row kb + 8*(lane/32) + (lane%16)/4,
// column c0 + 16*((lane/16)%2) + 4*(lane%4) makes lane (i = lane%32, hi = lane/32) receive
// rows kb + 8hi + 0..3 of column c0 + i; a second read 4 rows down completes the fragment.
//
// Tile geometry is the forward's (gemm_tile.hpp): 256 x 256 outputs, 8 waves as 4 x 2,
// K staged 64 at a time through two 64 KiB LDS stages filled by global_load_lds_dwordx4.
// An MN-major stage holds [64 k][256 columns] (512-byte rows); 16-byte chunk ch of row k
// sits at chunk position ch ^ (4 * (k % 4)), which spreads one transposing read's eight
// rows over all sixteen 16-byte bank groups (two passes, the minimum for 512 bytes).
#include "gemm_tile.hpp"

namespace moe {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

// One GEMM operand of a 256-wide tile.
//   K-major: p0 = the tile's first row (of K contiguous values), ld = row stride,
//            rows = valid tile rows (loads past them re-read the last one).
//   MN-major: element (k, c) of the tile is at p0 + k * ld + c for k < ksplit and at
//            p1 + (k - ksplit) * ld + c after; rows = valid tile columns (a multiple of 8);
//            K rows from kvalid on re-read row kvalid - 1 (and are zeroed when masked).
//            With kblk (the B operand of a tile instantiated with B_BLK): K rows come in
//            blocks of 64, block i starting at kblk[i], and element (k, c) is at
//            kblk[k / 64] + (k % 64) * ld + coff + c.
struct Operand {
  const uint16_t* p0;
  const uint16_t* p1;
  int ld;
  int rows;
  int ksplit;
  int kvalid;
  const uint64_t* kblk = nullptr;
  int coff = 0;
};

__device__ __forceinline__ int mn_off(int row, int col) {
  return row * (kGemmBM * 2) + ((((col >> 3) ^ (4 * (row & 3))) & 31) << 4) + (col & 7) * 2;
}

// The K-contiguous fragment (k = kb + 8hi + 0..7 of column c0 + lane%32) from an MN-major
// stage; values with stage-relative k >= klim are zero.
__device__ __forceinline__ bf16x8 ld_frag_mn(const char* tile, int kb, int c0, int lane, int klim) {
  const int row = kb + 8 * (lane >> 5) + ((lane >> 2) & 3);
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(tile + mn_off(row, col)));
  const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(tile + mn_off(row + 4, col)));
  v8i16 v = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
  if (klim < kGemmBK) {
    const int k0 = kb + 8 * (lane >> 5);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k0 + e >= klim) v[e] = 0;
  }
  return __builtin_bit_cast(bf16x8, v);
}

// out[r][c] = sum_k A[r][k] B[c][k] for r < orows, c < ocols of one 256 x 256 tile, in the
// orientation each operand is stored.  K % 64 == 0.  MASK_K zeroes A's values at k >= A.kvalid.
// ROW_DST: row_dst[r] is the address output row r goes to (then `out` is unused and col0 is
// the tile's first output column); the tile is staged in LDS and stored row by row in 16-byte
// vectors (ocols % 8 == 0).  A compile-time switch, so the other instantiations keep their code.
template <bool A_MN, bool B_MN, bool MASK_K, bool ROW_DST = false, bool B_BLK = false>
__device__ __forceinline__ void gemm_tile_t(const Operand& A, const Operand& B, uint16_t* __restrict__ out, int o_ld,
                                            int orows, int ocols, int K, char* smem,
                                            const uint64_t* __restrict__ row_dst = nullptr, int col0 = 0) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hi = lane >> 5;
  const int lrow = lane >> 3, lpos = lane & 7;
  const int lch_even = lpos ^ (lrow >> 1);
  const int lch_odd = lpos ^ (4 + (lrow >> 1));
  const int nk = K / kGemmBK;

  // Fills take the scalar-base form: a wave-uniform 64-bit base per operand and K step plus
  // a 32-bit byte offset per lane.  K-major: the base is the tile's first row, the offset
  // that of the lane's row and 16-byte chunk, plus the K step's.  MN-major: the base is the
  // K step's first K row (from p0 or p1: ksplit is a multiple of 64, so one K step never
  // straddles it; or the K step's 64-row block), the offset that of the lane's K row within
  // the step, clamped to kvalid - 1, and of its column.
  uint32_t akoff[4], bkoff[4];
  int acol[4], bcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int krow = (wave * 4 + i) * 8 + lrow;            // K-major: tile row of this lane
    const int lch = (i & 1) ? lch_odd : lch_even;
    const int mrow = 8 * wave + 2 * i + hi;                 // MN-major: K row of this lane
    const int mcol = (r32 ^ (4 * (mrow & 3))) * 8;
    if (!A_MN) akoff[i] = (uint32_t(min(krow, A.rows - 1)) * uint32_t(A.ld) + uint32_t(lch * 8)) * 2u;
    else acol[i] = min(mcol, A.rows - 8);
    if (!B_MN) bkoff[i] = (uint32_t(min(krow, B.rows - 1)) * uint32_t(B.ld) + uint32_t(lch * 8)) * 2u;
    else bcol[i] = min(mcol, B.rows - 8);
  }
  const char* akbase = A_MN ? nullptr : reinterpret_cast<const char*>(wave_uniform(A.p0));
  const char* bkbase = B_MN ? nullptr : reinterpret_cast<const char*>(wave_uniform(B.p0));
  auto mn_base = [&](const Operand& X, int koff) -> const char* {
    return reinterpret_cast<const char*>(wave_uniform(koff < X.ksplit ? X.p0 + size_t(koff) * X.ld
                                                                     : X.p1 + size_t(koff - X.ksplit) * X.ld));
  };
  auto mn_lane_off = [&](const Operand& X, int koff, int i, int col) -> uint32_t {
    const int kr = min(8 * wave + 2 * i + hi, X.kvalid - 1 - koff);
    return (uint32_t(kr) * uint32_t(X.ld) + uint32_t(col)) * 2u;
  };
  // B_BLK: the base of B's 64-row block of the K step being issued (bblk), and of the next
  // one, loaded a K step ahead
  const uint16_t* bblk = nullptr;
  uint64_t bnext = 0;
  // LDS destination of this wave's fills (the M0 operand), as a scalar
  const uint32_t lds_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(smem + wave * 4 * 1024));
  auto issue = [&](int ks) {
    const uint32_t da = lds_dst0 + uint32_t((ks & 1) * kStageBytes);
    const uint32_t db = da + uint32_t(kGemmBM * kGemmBK * 2);
    const int koff = ks * kGemmBK;
    const char* abase = A_MN ? mn_base(A, koff) : akbase;
    const char* bbase;
    if constexpr (B_BLK) bbase = reinterpret_cast<const char*>(wave_uniform(bblk + B.coff));
    else bbase = B_MN ? mn_base(B, koff) : bkbase;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const lds_void_ptr la = (lds_void_ptr)(uintptr_t)(da + uint32_t(i * 1024));
      const lds_void_ptr lb = (lds_void_ptr)(uintptr_t)(db + uint32_t(i * 1024));
      const uint32_t ao = A_MN ? mn_lane_off(A, koff, i, acol[i]) : akoff[i] + uint32_t(koff * 2);
      const uint32_t bo = B_MN ? mn_lane_off(B, koff, i, bcol[i]) : bkoff[i] + uint32_t(koff * 2);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(abase + ao), la, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bbase + bo), lb, 16, 0, 0);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  if constexpr (B_BLK) {
    bblk = reinterpret_cast<const uint16_t*>(B.kblk[0]);
    if (nk > 1) bnext = B.kblk[1];
  }
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) {
      if constexpr (B_BLK) {
        bblk = reinterpret_cast<const uint16_t*>(bnext);
        if (ks + 2 < nk) bnext = B.kblk[ks + 2];
      }
      issue(ks + 1);
    }
    const char* sa = smem + (ks & 1) * kStageBytes;
    const char* sb = sa + kGemmBM * kGemmBK * 2;
    const int klim = MASK_K ? A.kvalid - ks * kGemmBK : kGemmBK;
    auto lda = [&](int sub, int m) -> bf16x8 {
      if (A_MN) return ld_frag_mn(sa, sub * 16, wm * 64 + m * 32, lane, klim);
      return *reinterpret_cast<const bf16x8*>(sa + swz_off(wm * 64 + m * 32 + r32, sub * 2 + hi));
    };
    auto ldb = [&](int sub, int n) -> bf16x8 {
      if (B_MN) return ld_frag_mn(sb, sub * 16, wn * 128 + n * 32, lane, kGemmBK);
      return *reinterpret_cast<const bf16x8*>(sb + swz_off(wn * 128 + n * 32 + r32, sub * 2 + hi));
    };
    bf16x8 fa[2][2], fb[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m) fa[0][m] = lda(0, m);
#pragma unroll
    for (int n = 0; n < 4; ++n) fb[0][n] = ldb(0, n);
#pragma unroll
    for (int sub = 0; sub < kGemmBK / 16; ++sub) {
      const int cur = sub & 1;
      if (sub + 1 < kGemmBK / 16) {
#pragma unroll
        for (int m = 0; m < 2; ++m) fa[cur ^ 1][m] = lda(sub + 1, m);
#pragma unroll
        for (int n = 0; n < 4; ++n) fb[cur ^ 1][n] = ldb(sub + 1, n);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][m], fb[cur][n], acc[m][n], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // lane holds column r32 and rows 8*(e/4) + 4*hi + e%4 of each 32 x 32 block
  if constexpr (ROW_DST) {
    // [256 rows][256 cols] bf16 in LDS, 16-byte chunks XOR-swizzled by row; the K loop ended
    // on a barrier, so the stages are free
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int col = wn * 128 + n * 32 + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * 64 + m * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
          *reinterpret_cast<uint16_t*>(smem + row * 512 + (((col >> 3) ^ (row & 31)) << 4) + (col & 7) * 2) =
              f32_to_bf16(acc[m][n][e]);
        }
      }
    __syncthreads();
    for (int v = tid; v < kGemmBM * (kGemmBN / 8); v += kGemmThreads) {
      const int row = v >> 5, cv = v & 31;
      if (row < orows && cv * 8 < ocols)
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(row_dst[row]) + col0 + cv * 8) =
            *reinterpret_cast<const u32x4*>(smem + row * 512 + ((cv ^ (row & 31)) << 4));
    }
    __syncthreads();                      // the next tile's fills reuse the stages
    return;
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int col = wn * 128 + n * 32 + r32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * 64 + m * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (row < orows && col < ocols) out[size_t(row) * o_ld + col] = f32_to_bf16(acc[m][n][e]);
      }
    }
}

// C[s] = A[s] B_l for the rows s of every local expert, B_l stored [K][Nout] (K rows of
// Nout contiguous values; rows ksplit.. of K come from B1):
//   dh = dO W2    (B0 = W2 [E_local][d][F], K = d, Nout = F);
//   dX = [da|db] [W1; W3]   (B0 = W1, B1 = W3 [E_local][F][d], K = 2F, ksplit = F, Nout = d).
// Tiles walk as the forward's grouped GEMM: 8 contiguous ranges, one per XCD, expert-major.
template <bool ROW_DST>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_rows_bmn_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int ksplit,
    uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, const int32_t* __restrict__ mtile_base,
    const int32_t* __restrict__ ctrl, int El, int K, int Nout, const uint64_t* __restrict__ RowDst) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int NT = (Nout + kGemmBN - 1) / kGemmBN;
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
    const int rows = min(kGemmBM, offsets[l + 1] - row0);
    const int c0 = nt * kGemmBN;
    const Operand a{A + size_t(row0) * K, nullptr, K, rows, 0, 0};
    const Operand b{B0 + size_t(l) * ksplit * Nout + c0,
                    B1 ? B1 + size_t(l) * (K - ksplit) * Nout + c0 : nullptr, Nout, Nout - c0, ksplit, K};
    gemm_tile_t<false, true, false, ROW_DST>(a, b, ROW_DST ? nullptr : C + size_t(row0) * Nout + c0, Nout, rows,
                                             Nout - c0, K, smem, ROW_DST ? RowDst + row0 : nullptr, c0);
  }
}

// Weight gradients of every local expert, C_l [M][Nc] = sum over the expert's rows s of
// A[s][m] B[s][c] (A, B row-major with strides lda, ldb; the expert's rows are
// [offsets[l], offsets[l+1]), summed in ascending order within each K step of 64):
//   dW1 = da^T xe, dW3 = db^T xe (A = columns of [da|db], M = F; B = xe, Nc = d);
//   dW2 = dO^T h (A = dO, M = d; B = h, Nc = F).
// K runs over the expert's rows rounded up to 64; A's values past the last row are zeroed.
// An expert with no rows gets zeros.
// B_BLK: B's rows are read by 64-row blocks, block b of row tile m starting at
// BBlk[m * 4 + b] (mtile_base gives each expert's first row tile), instead of from Bm.
template <bool B_BLK>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_wgrad_bf16_kernel(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ Bm, int ldb,
    const int32_t* __restrict__ offsets, uint16_t* __restrict__ C, int El, int M, int Nc,
    const uint64_t* __restrict__ BBlk, const int32_t* __restrict__ mtile_base) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int MT = (M + kGemmBM - 1) / kGemmBM, NT = (Nc + kGemmBN - 1) / kGemmBN;
  const int total = El * MT * NT;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int wg_per_xcd = gridDim.x >> 3;
  for (int tt = blockIdx.x >> 3; tt < per_xcd; tt += wg_per_xcd) {
    const int tau = xcd * per_xcd + tt;
    if (tau >= total) break;
    const int l = tau / (MT * NT);
    const int rem = tau - l * MT * NT;
    const int nt = rem / MT, mt = rem - nt * MT;      // row tiles innermost: shared B panel
    const int m0 = mt * kGemmBM, c0 = nt * kGemmBN;
    const int rows = min(kGemmBM, M - m0), cols = min(kGemmBN, Nc - c0);
    uint16_t* out = C + (size_t(l) * M + m0) * Nc + c0;
    const int r0 = offsets[l];
    const int n = offsets[l + 1] - r0;
    if (n == 0) {
      for (int v = threadIdx.x; v < kGemmBM * (kGemmBN / 8); v += kGemmThreads) {
        const int row = v >> 5, cv = v & 31;
        if (row < rows && cv * 8 < cols)
          *reinterpret_cast<u32x4*>(out + size_t(row) * Nc + cv * 8) = u32x4{0, 0, 0, 0};
      }
      continue;
    }
    const Operand a{A + size_t(r0) * lda + m0, nullptr, lda, M - m0, 1 << 30, n};
    Operand b{B_BLK ? nullptr : Bm + size_t(r0) * ldb + c0, nullptr, ldb, Nc - c0, 1 << 30, n};
    if constexpr (B_BLK) {
      b.kblk = BBlk + size_t(mtile_base[l]) * 4;
      b.coff = c0;
    }
    gemm_tile_t<true, true, true, false, B_BLK>(a, b, out, Nc, rows, cols, (n + kGemmBK - 1) & ~(kGemmBK - 1), smem);
  }
}

hipError_t set_bwd_gemm_lds_attrs() {
  static std::atomic<uint64_t> done{0};
  return once_per_device(done, [] {
    const void* ks[] = {reinterpret_cast<const void*>(grouped_rows_bmn_kernel<false>),
                        reinterpret_cast<const void*>(grouped_rows_bmn_kernel<true>),
                        reinterpret_cast<const void*>(grouped_wgrad_bf16_kernel<false>),
                        reinterpret_cast<const void*>(grouped_wgrad_bf16_kernel<true>)};
    for (const void* k : ks) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
}

// row_dst: null (rows to C), or per pair the address its output row goes to
hipError_t launch_rows_bmn(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, int ksplit, uint16_t* C, int K,
                           int Nout, const int32_t* offsets, const int32_t* mtb, const int32_t* ctrl, int El, int cus,
                           hipStream_t st, const uint64_t* row_dst) {
  hipError_t e = set_bwd_gemm_lds_attrs();
  if (e != hipSuccess) return e;
  if (row_dst)
    hipLaunchKernelGGL(grouped_rows_bmn_kernel<true>, dim3((cus / 8) * 8), dim3(kGemmThreads), kGemmLds, st, A, B0, B1,
                       ksplit, C, offsets, mtb, ctrl, El, K, Nout, row_dst);
  else
    hipLaunchKernelGGL(grouped_rows_bmn_kernel<false>, dim3((cus / 8) * 8), dim3(kGemmThreads), kGemmLds, st, A, B0,
                       B1, ksplit, C, offsets, mtb, ctrl, El, K, Nout, row_dst);
  return hipGetLastError();
}

// b_blk: null (B rows from B), or the 64-row block table of B's rows (with mtile_base)
hipError_t launch_wgrad(const uint16_t* A, int lda, const uint16_t* B, int ldb, const int32_t* offsets, uint16_t* C,
                        int El, int M, int Nc, int cus, hipStream_t st, const uint64_t* b_blk,
                        const int32_t* mtile_base) {
  hipError_t e = set_bwd_gemm_lds_attrs();
  if (e != hipSuccess) return e;
  if (b_blk)
    hipLaunchKernelGGL(grouped_wgrad_bf16_kernel<true>, dim3((cus / 8) * 8), dim3(kGemmThreads), kGemmLds, st, A, lda,
                       nullptr, ldb, offsets, C, El, M, Nc, b_blk, mtile_base);
  else
    hipLaunchKernelGGL(grouped_wgrad_bf16_kernel<false>, dim3((cus / 8) * 8), dim3(kGemmThreads), kGemmLds, st, A,
                       lda, B, ldb, offsets, C, El, M, Nc, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe
