// One 256-row x 256-column tile of the grouped SwiGLU FFN on gfx950 (bf16 MFMA).
// Shared by the standalone grouped GEMM kernels and the persistent forward kernel.
//
// GEMM1 (MODE 0): h = silu(X W1^T) * (X W3^T); GEMM2 (MODE 1): y = h W2^T.  MODE 2 is
// GEMM1 of the backward: the same products a = X W1^T, b = X W3^T, then from the incoming
// dh of each (row, f) the epilogue writes h, da = dh * b * silu'(a) and db = dh * silu(a),
// silu'(a) = sigma(a) (1 + a (1 - sigma(a))) (needs F % 8 == 0).  Every operand is
// K-contiguous (row-major X and h, weights stored [out][in]), so each MFMA lane's 8
// consecutive K values are one 16-byte LDS read.
//
// 8 waves (two per SIMD) as 4 (rows) x 2 (cols); each wave owns a 64 x 128 block = 2 x 4
// tiles of v_mfma_f32_32x32x16_bf16.  K is staged 64 at a time through two LDS buffers
// (2 x 64 KiB) filled by direct global->LDS loads (global_load_lds_dwordx4, no VGPR
// staging).  GEMM1's B tile interleaves 32-row blocks of W1 and W3 for the same f values,
// so a lane holds the gate and the up accumulator of one (row, f) and applies SwiGLU in
// registers.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {

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

// Where the tile's rows live: up to 4 blocks of (1 << blk_log2) consecutive rows each
// (one block = one ring slot in the persistent kernel; blocks of 128 rows back to back in
// the standalone GEMM).  Rows >= rows are not stored; their loads re-read row rows-1.
struct TileIO {
  const uint16_t* a0;
  const uint16_t* a1;
  const uint16_t* a2;
  const uint16_t* a3;
  uint16_t* o0;
  uint16_t* o1;
  uint16_t* o2;
  uint16_t* o3;
  int a_ld, o_ld;      // row strides in elements
  int blk_log2;        // 6, 7 or 8
  int rows;            // valid rows, 1..256
  const uint16_t* dh;  // MODE 2: incoming dh of the tile's first row ([rows][Nout] contiguous)
  uint16_t* dab;       // MODE 2: [da | db] rows of 2 * Nout from the tile's first row
  const uint64_t* row_dst;  // MODE 1: null, or per tile row the address its output row goes to
  const uint64_t* row_src;  // null, or per tile row the address of its A row (replaces a0..a3)
};

// A pointer the caller knows to be the same in every lane of the wave, moved to scalar
// registers (the compiler cannot prove that values derived from the wave index are uniform).
template <typename T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<T*>((uint64_t(hi) << 32) | lo);
}

template <typename P>
__device__ __forceinline__ P pick4(int i, P p0, P p1, P p2, P p3) {
  return i == 0 ? p0 : (i == 1 ? p1 : (i == 2 ? p2 : p3));
}

// MFMA operand fragments of one sub-step (16 K values): two A blocks, four B blocks
struct Frags {
  i32x4 a0, a1, b0, b1, b2, b3;
};

__device__ __forceinline__ uint32_t lds_addr(const char* q) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)q));
}

// ACC[m][n] += A_m B_n for one sub-step (fragments C), with the 6 fragments of the next
// sub-step read into N from LDS (A blocks at AA, AA + 4096; B blocks at BA + n * 4096)
// between the MFMAs (reads spread over the block keep the eight waves' LDS requests from
// arriving in one burst), then one lgkmcnt(0).  A macro, so that ACC stays a register
// array of the caller.
#define MOE_MFMA_SUBSTEP_READ(ACC, C, N, AA, BA)                                                          \
  asm volatile(                                                                                           \
      "v_mfma_f32_32x32x16_bf16 %0, %14, %16, %0\n\t"                                                     \
      "ds_read_b128 %8, %20\n\t"                                                                          \
      "v_mfma_f32_32x32x16_bf16 %1, %14, %17, %1\n\t"                                                     \
      "ds_read_b128 %9, %20 offset:4096\n\t"                                                              \
      "v_mfma_f32_32x32x16_bf16 %2, %14, %18, %2\n\t"                                                     \
      "ds_read_b128 %10, %21\n\t"                                                                         \
      "v_mfma_f32_32x32x16_bf16 %3, %14, %19, %3\n\t"                                                     \
      "ds_read_b128 %11, %21 offset:4096\n\t"                                                             \
      "v_mfma_f32_32x32x16_bf16 %4, %15, %16, %4\n\t"                                                     \
      "ds_read_b128 %12, %21 offset:8192\n\t"                                                             \
      "v_mfma_f32_32x32x16_bf16 %5, %15, %17, %5\n\t"                                                     \
      "ds_read_b128 %13, %21 offset:12288\n\t"                                                            \
      "v_mfma_f32_32x32x16_bf16 %6, %15, %18, %6\n\t"                                                     \
      "v_mfma_f32_32x32x16_bf16 %7, %15, %19, %7\n\t"                                                     \
      "s_waitcnt lgkmcnt(0)"                                                                              \
      : "+v"(ACC[0][0]), "+v"(ACC[0][1]), "+v"(ACC[0][2]), "+v"(ACC[0][3]), "+v"(ACC[1][0]),              \
        "+v"(ACC[1][1]), "+v"(ACC[1][2]), "+v"(ACC[1][3]), "=&v"(N.a0), "=&v"(N.a1), "=&v"(N.b0),          \
        "=&v"(N.b1), "=&v"(N.b2), "=&v"(N.b3)                                                             \
      : "v"(C.a0), "v"(C.a1), "v"(C.b0), "v"(C.b1), "v"(C.b2), "v"(C.b3), "v"(AA), "v"(BA))

// The same sub-step for a wave whose second 32-row block lies wholly past the tile's valid
// rows: only the m = 0 MFMAs, and no read of the second A block.
#define MOE_MFMA_SUBSTEP_READ_M1(ACC, C, N, AA, BA)                                                       \
  asm volatile(                                                                                           \
      "v_mfma_f32_32x32x16_bf16 %0, %9, %10, %0\n\t"                                                      \
      "ds_read_b128 %4, %14\n\t"                                                                          \
      "v_mfma_f32_32x32x16_bf16 %1, %9, %11, %1\n\t"                                                      \
      "ds_read_b128 %5, %15\n\t"                                                                          \
      "ds_read_b128 %6, %15 offset:4096\n\t"                                                              \
      "v_mfma_f32_32x32x16_bf16 %2, %9, %12, %2\n\t"                                                      \
      "ds_read_b128 %7, %15 offset:8192\n\t"                                                              \
      "ds_read_b128 %8, %15 offset:12288\n\t"                                                             \
      "v_mfma_f32_32x32x16_bf16 %3, %9, %13, %3\n\t"                                                      \
      "s_waitcnt lgkmcnt(0)"                                                                              \
      : "+v"(ACC[0][0]), "+v"(ACC[0][1]), "+v"(ACC[0][2]), "+v"(ACC[0][3]), "=&v"(N.a0), "=&v"(N.b0),     \
        "=&v"(N.b1), "=&v"(N.b2), "=&v"(N.b3)                                                             \
      : "v"(C.a0), "v"(C.b0), "v"(C.b1), "v"(C.b2), "v"(C.b3), "v"(AA), "v"(BA))

// The same two sub-steps with the MFMA operands swapped (B block first): each accumulator
// then holds the transposed 32 x 32 block, so a lane owns one output row and 4
// consecutive columns per group of 4 values (the forward epilogues store 8 bytes at a
// time; the backward's GEMM1, MODE 2, keeps the original orientation).  Every output
// element is the same dot product over the same K values.
#define MOE_MFMA_SUBSTEP_READ_T(ACC, C, N, AA, BA)                                                          \
  asm volatile(                                                                                           \
      "v_mfma_f32_32x32x16_bf16 %0, %16, %14, %0\n\t"                                                     \
      "ds_read_b128 %8, %20\n\t"                                                                          \
      "v_mfma_f32_32x32x16_bf16 %1, %17, %14, %1\n\t"                                                     \
      "ds_read_b128 %9, %20 offset:4096\n\t"                                                              \
      "v_mfma_f32_32x32x16_bf16 %2, %18, %14, %2\n\t"                                                     \
      "ds_read_b128 %10, %21\n\t"                                                                         \
      "v_mfma_f32_32x32x16_bf16 %3, %19, %14, %3\n\t"                                                     \
      "ds_read_b128 %11, %21 offset:4096\n\t"                                                             \
      "v_mfma_f32_32x32x16_bf16 %4, %16, %15, %4\n\t"                                                     \
      "ds_read_b128 %12, %21 offset:8192\n\t"                                                             \
      "v_mfma_f32_32x32x16_bf16 %5, %17, %15, %5\n\t"                                                     \
      "ds_read_b128 %13, %21 offset:12288\n\t"                                                            \
      "v_mfma_f32_32x32x16_bf16 %6, %18, %15, %6\n\t"                                                     \
      "v_mfma_f32_32x32x16_bf16 %7, %19, %15, %7\n\t"                                                     \
      "s_waitcnt lgkmcnt(0)"                                                                              \
      : "+v"(ACC[0][0]), "+v"(ACC[0][1]), "+v"(ACC[0][2]), "+v"(ACC[0][3]), "+v"(ACC[1][0]),              \
        "+v"(ACC[1][1]), "+v"(ACC[1][2]), "+v"(ACC[1][3]), "=&v"(N.a0), "=&v"(N.a1), "=&v"(N.b0),          \
        "=&v"(N.b1), "=&v"(N.b2), "=&v"(N.b3)                                                             \
      : "v"(C.a0), "v"(C.a1), "v"(C.b0), "v"(C.b1), "v"(C.b2), "v"(C.b3), "v"(AA), "v"(BA))

#define MOE_MFMA_SUBSTEP_READ_M1_T(ACC, C, N, AA, BA)                                                       \
  asm volatile(                                                                                           \
      "v_mfma_f32_32x32x16_bf16 %0, %10, %9, %0\n\t"                                                      \
      "ds_read_b128 %4, %14\n\t"                                                                          \
      "v_mfma_f32_32x32x16_bf16 %1, %11, %9, %1\n\t"                                                      \
      "ds_read_b128 %5, %15\n\t"                                                                          \
      "ds_read_b128 %6, %15 offset:4096\n\t"                                                              \
      "v_mfma_f32_32x32x16_bf16 %2, %12, %9, %2\n\t"                                                      \
      "ds_read_b128 %7, %15 offset:8192\n\t"                                                              \
      "ds_read_b128 %8, %15 offset:12288\n\t"                                                             \
      "v_mfma_f32_32x32x16_bf16 %3, %13, %9, %3\n\t"                                                      \
      "s_waitcnt lgkmcnt(0)"                                                                              \
      : "+v"(ACC[0][0]), "+v"(ACC[0][1]), "+v"(ACC[0][2]), "+v"(ACC[0][3]), "=&v"(N.a0), "=&v"(N.b0),     \
        "=&v"(N.b1), "=&v"(N.b2), "=&v"(N.b3)                                                             \
      : "v"(C.a0), "v"(C.b0), "v"(C.b1), "v"(C.b2), "v"(C.b3), "v"(AA), "v"(BA))

// b0/b1: this expert's weight matrices ([Nout][K], row stride b_ld); c0: first output
// column of the tile.  A_CPOL: cache policy of the A-row loads (0 = default; 16 = sc1, a
// device-coherent load that does not hit this CU's L1, for rows another CU just wrote).
template <int MODE, int A_CPOL = 0, bool A_BY_ADDR = false>
__device__ __forceinline__ void gemm_tile(const TileIO& io, const uint16_t* __restrict__ b0,
                                          const uint16_t* __restrict__ b1, int c0, int Nout, int K,
                                          char* smem, int b_ld) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hi = lane >> 5;
  // LDS fill geometry: lane -> row lrow of an 8-row group, LDS chunk position lpos, which
  // holds logical chunk lpos ^ (((g & 1) * 4 + (lrow >> 1)) & 7) for group g
  const int lrow = lane >> 3, lpos = lane & 7;
  const int lch_even = lpos ^ (lrow >> 1);
  const int lch_odd = lpos ^ (4 + (lrow >> 1));
  const int nk = K / kGemmBK;
  const int rows = io.rows;
  const int bmask = (1 << io.blk_log2) - 1;

  // this wave fills row groups g = wave*4 + i (rows g*8 + lrow) of the A and B tiles.  A
  // rows come from one block (the wave's 32 rows, or the clamped last row, lie in one block of
  // 1 << blk_log2 rows) unless A_BY_ADDR, where each row has its own address (row_src).  The B
  // rows of one wave are all W1 rows or all W3 rows (32-row blocks alternate, and wave w fills
  // rows 32 w .. 32 w + 31).  So A (from blocks) and B are scalar bases plus 32-bit byte
  // offsets, the fills' scalar-base form.
  const uint16_t* ap[4];
  uint32_t aoff[4];
  const char* abase = nullptr;
  if constexpr (!A_BY_ADDR)
    abase = reinterpret_cast<const char*>(
        wave_uniform(pick4(min(wave * 32, rows - 1) >> io.blk_log2, io.a0, io.a1, io.a2, io.a3)));
  const char* bbase = reinterpret_cast<const char*>(wave_uniform((MODE != 1 && (wave & 1)) ? b1 : b0));
  uint32_t boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 8 + lrow;
    const int lch = (i & 1) ? lch_odd : lch_even;
    const int rr = min(row, rows - 1);
    if constexpr (A_BY_ADDR) ap[i] = reinterpret_cast<const uint16_t*>(io.row_src[rr]) + lch * 8;
    else aoff[i] = (uint32_t(rr & bmask) * uint32_t(io.a_ld) + uint32_t(lch * 8)) * 2u;
    // (MODE 0/2: 32-row blocks alternate W1 / W3 rows of the same 32 f values)
    const int n = (MODE != 1) ? min(c0 + (row >> 6) * 32 + (row & 31), Nout - 1) : min(c0 + row, Nout - 1);
    boff[i] = (uint32_t(n) * uint32_t(b_ld) + uint32_t(lch * 8)) * 2u;
  }
  // LDS destination of this wave's fills (the M0 operand): the wave's first A row group in
  // stage 0, as a scalar; stage 1 and the B tile are constant offsets from it
  const uint32_t lds_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(smem + wave * 4 * 1024));
  auto issue = [&](int ks) {
    const uint32_t da = lds_dst0 + uint32_t((ks & 1) * kStageBytes);
    const uint32_t db = da + uint32_t(kGemmBM * kGemmBK * 2);
    const int koff = ks * kGemmBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const lds_void_ptr la = (lds_void_ptr)(uintptr_t)(da + uint32_t(i * 1024));
      const lds_void_ptr lb = (lds_void_ptr)(uintptr_t)(db + uint32_t(i * 1024));
      if constexpr (A_BY_ADDR)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(ap[i] + koff), la, 16, 0, A_CPOL);
      else
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(abase + (aoff[i] + uint32_t(koff * 2))), la, 16, 0,
                                         A_CPOL);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bbase + (boff[i] + uint32_t(koff * 2))), lb, 16, 0, 0);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // Software pipeline over K.  Each sub-step is one block: its 8 MFMAs with the next
  // sub-step's 6 fragment reads between them, then one lgkmcnt(0); the next fragments are
  // early-clobber outputs, so they sit in registers of their own.  The barrier of a K step
  // comes after sub-step 2, whose block already read sub-step 3's fragments: by then every
  // wave is done with this stage, so the fill two steps ahead goes into it right away and
  // sub-step 3's MFMAs cover the reads of the next stage's first fragments.  A fill is
  // issued four sub-steps before the barrier that waits for it.  Per accumulator the MFMAs
  // run in K order, so the result does not depend on this schedule.
  auto a_at = [&](const char* st, int sub) -> uint32_t {
    return lds_addr(st + swz_off(wm * 64 + r32, sub * 2 + hi));
  };
  auto b_at = [&](const char* st, int sub) -> uint32_t {
    return lds_addr(st + kGemmBM * kGemmBK * 2 + swz_off(wn * 128 + r32, sub * 2 + hi));
  };
  Frags cur;

  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nk > 1) issue(1);
  cur.a0 = *reinterpret_cast<const i32x4*>(smem + swz_off(wm * 64 + r32, hi));
  cur.a1 = *reinterpret_cast<const i32x4*>(smem + swz_off(wm * 64 + 32 + r32, hi));
  cur.b0 = *reinterpret_cast<const i32x4*>(smem + kGemmBM * kGemmBK * 2 + swz_off(wn * 128 + r32, hi));
  cur.b1 = *reinterpret_cast<const i32x4*>(smem + kGemmBM * kGemmBK * 2 + swz_off(wn * 128 + 32 + r32, hi));
  cur.b2 = *reinterpret_cast<const i32x4*>(smem + kGemmBM * kGemmBK * 2 + swz_off(wn * 128 + 64 + r32, hi));
  cur.b3 = *reinterpret_cast<const i32x4*>(smem + kGemmBM * kGemmBK * 2 + swz_off(wn * 128 + 96 + r32, hi));

  // Row padding: the last row tile of an expert is usually partial.  A wave whose 32-row
  // blocks lie wholly past the valid rows skips their MFMAs (and fragment reads); it still
  // fills and meets every barrier.  Waves w and w + 4 share a SIMD and own rows 64(w/2) and
  // 64(w/2) + 128, so a tile of at most 128 valid rows keeps each SIMD at most half busy.
  // Skipped MFMAs only ever accumulate into rows that are never stored.
  const int mv = __builtin_amdgcn_readfirstlane(min(2, max(0, (rows - wm * 64 + 31) >> 5)));
  auto substep = [&](auto mvc, uint32_t aa, uint32_t ba) {
    constexpr int MV = decltype(mvc)::value;
    if constexpr (MV == 2) {
      Frags nxt;
      if constexpr (MODE <= 1) MOE_MFMA_SUBSTEP_READ_T(acc, cur, nxt, aa, ba);
      else MOE_MFMA_SUBSTEP_READ(acc, cur, nxt, aa, ba);
      cur = nxt;
    } else if constexpr (MV == 1) {
      Frags nxt;
      if constexpr (MODE <= 1) MOE_MFMA_SUBSTEP_READ_M1_T(acc, cur, nxt, aa, ba);
      else MOE_MFMA_SUBSTEP_READ_M1(acc, cur, nxt, aa, ba);
      cur.a0 = nxt.a0;
      cur.b0 = nxt.b0;
      cur.b1 = nxt.b1;
      cur.b2 = nxt.b2;
      cur.b3 = nxt.b3;
    }
  };
  auto kloop = [&](auto mvc) {
    for (int ks = 0; ks < nk; ++ks) {
      const char* st = smem + (ks & 1) * kStageBytes;
#pragma unroll
      for (int sub = 0; sub < kGemmBK / 16 - 1; ++sub) substep(mvc, a_at(st, sub + 1), b_at(st, sub + 1));
      __builtin_amdgcn_s_waitcnt(0);      // this wave's fills of the next stage landed
      __syncthreads();                    // ... and everyone's; every wave is done with this stage
      if (ks + 2 < nk) issue(ks + 2);     // into this stage
      // the next stage's first fragments (after the last K step these reads land in the
      // other stage, inside the LDS allocation, and are not used)
      const char* sn = smem + ((ks + 1) & 1) * kStageBytes;
      substep(mvc, a_at(sn, 0), b_at(sn, 0));
    }
  };
  if (mv == 2) kloop(std::integral_constant<int, 2>{});
  else if (mv == 1) kloop(std::integral_constant<int, 1>{});
  else kloop(std::integral_constant<int, 0>{});

  // The MFMAs above are inline assembly, which the compiler's hazard recognizer does not
  // see: a read of an accumulator right after the MFMA that writes it would see the old
  // value (MFMA results are not interlocked for dependent reads).  24 wait states cover the
  // longest MFMA->read distance; taking every accumulator as an operand keeps all reads
  // of them after this point.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]), "+v"(acc[1][0]),
                 "+v"(acc[1][1]), "+v"(acc[1][2]), "+v"(acc[1][3]));

  // The epilogue's lane indices are re-derived through an opaque copy, so the compiler
  // cannot hoist its per-row store offsets above the main loop, where they would hold
  // registers the loop needs for double-buffered fragments.
  int lane_o = lane;
  asm volatile("" : "+v"(lane_o));
  const int r32o = lane_o & 31, hio = lane_o >> 5;

  if (MODE == 1) {
    // The tile is staged as bf16 in LDS ([256 rows][256 cols], 16-byte chunks XOR-swizzled
    // by row), then written back row by row in 16-byte vectors, so every output row receives
    // whole 128-byte lines: rows of ye, or with row_dst (the fused push) each row at its own
    // destination (a recv row).  The main loop ended on a barrier, so the stages are free.
    char* stg = smem;
    // (transposed blocks: lane owns row r32 and columns 8 j + 4 hi + 0..3 of each 32 x 32 block)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int row = wm * 64 + m * 32 + r32o;
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = wn * 128 + n * 32 + 8 * j + 4 * hio;
          uint2 v;
          v.x = pack_bf16x2(acc[m][n][4 * j], acc[m][n][4 * j + 1]);
          v.y = pack_bf16x2(acc[m][n][4 * j + 2], acc[m][n][4 * j + 3]);
          *reinterpret_cast<uint2*>(stg + row * 512 + (((col >> 3) ^ (row & 31)) << 4) + (col & 7) * 2) = v;
        }
    }
    __syncthreads();
    const int ncols = min(kGemmBN, Nout - c0);
    for (int v = tid; v < kGemmBM * (kGemmBN / 8); v += kGemmThreads) {
      const int row = v >> 5, cv = v & 31;                  // 32 vectors of 8 bf16 per row
      if (row < rows && cv * 8 < ncols) {
        uint16_t* orow = io.row_dst ? reinterpret_cast<uint16_t*>(io.row_dst[row])
                                    : pick4(row >> io.blk_log2, io.o0, io.o1, io.o2, io.o3) + size_t(row & bmask) * io.o_ld;
        *reinterpret_cast<u32x4*>(orow + c0 + cv * 8) = *reinterpret_cast<const u32x4*>(stg + row * 512 + ((cv ^ (row & 31)) << 4));
      }
    }
    __syncthreads();                                        // the next tile's fills reuse the stages
    return;
  }

  if (MODE == 2) {
    // Backward epilogue, in two passes of 128 tile rows (m = 0, 1): every wave stages its
    // (a, b) pairs as fp32 in LDS ([128 rows][128 f] float2 = the whole 128 KiB), then each
    // thread finishes 8 consecutive f of one row -- one 16-byte load of dh, 16-byte stores
    // of h, da and db.  The main loop ended on a barrier, so the stages are free.
    float2* stg = reinterpret_cast<float2*>(smem);
#pragma unroll   // acc[m] must stay in registers: a run-time m would move acc to scratch
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int lr = wm * 32 + 8 * (e >> 2) + 4 * hio + (e & 3);
          stg[lr * 128 + (wn * 2 + q) * 32 + r32o] = make_float2(acc[m][2 * q][e], acc[m][2 * q + 1][e]);
        }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = tid + i * kGemmThreads;             // 128 rows x 16 vectors of 8 f
        const int lr = u >> 4, f8 = (u & 15) * 8;
        const int trow = (lr >> 5) * 64 + m * 32 + (lr & 31);
        const int f = c0 + f8;
        if (trow < rows && f < Nout) {
          const u32x4 dv = *reinterpret_cast<const u32x4*>(io.dh + size_t(trow) * Nout + f);
          const f32x4* sp = reinterpret_cast<const f32x4*>(stg + lr * 128 + f8);
          u32x4 hv, dav, dbv;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x4 ab = sp[w];                       // a, b of f8 + 2w and f8 + 2w + 1
            float hh[2], ga[2], gb[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const float a = ab[2 * z], b = ab[2 * z + 1];
              const float dh = __uint_as_float(z ? (dv[w] & 0xFFFF0000u) : (dv[w] << 16));
              const float sg = 1.0f / (1.0f + __expf(-a));
              const float sa = a * sg;
              hh[z] = sa * b;
              ga[z] = dh * b * (sg * (1.0f + a * (1.0f - sg)));
              gb[z] = dh * sa;
            }
            hv[w] = pack_bf16x2(hh[0], hh[1]);
            dav[w] = pack_bf16x2(ga[0], ga[1]);
            dbv[w] = pack_bf16x2(gb[0], gb[1]);
          }
          uint16_t* orow = pick4(trow >> io.blk_log2, io.o0, io.o1, io.o2, io.o3) + size_t(trow & bmask) * io.o_ld;
          *reinterpret_cast<u32x4*>(orow + f) = hv;
          uint16_t* drow = io.dab + size_t(trow) * (2 * Nout);
          *reinterpret_cast<u32x4*>(drow + f) = dav;
          *reinterpret_cast<u32x4*>(drow + Nout + f) = dbv;
        }
      }
      __syncthreads();
    }
    return;
  }

  // SwiGLU epilogue (MODE 0; MODE 1 and 2 returned above)
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int rb = wm * 64 + m * 32;                     // 32-row block, inside one row block
    uint16_t* orow = pick4(rb >> io.blk_log2, io.o0, io.o1, io.o2, io.o3) + size_t(rb & bmask) * io.o_ld;
    if (MODE == 0) {
      // transposed blocks: lane owns row r32 and f = 8 j + 4 hi + 0..3 of each 32-f block
      if (rb + r32o < rows) {
        uint16_t* prow = orow + size_t(r32o) * io.o_ld;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int f = c0 + (wn * 2 + q) * 32 + 8 * j + 4 * hio;
            if (f < Nout) {
              float h[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) h[i] = silu_f32(acc[m][2 * q][4 * j + i]) * acc[m][2 * q + 1][4 * j + i];
              uint2 v;
              v.x = pack_bf16x2(h[0], h[1]);
              v.y = pack_bf16x2(h[2], h[3]);
              *reinterpret_cast<uint2*>(prow + f) = v;
            }
          }
      }
    }
  }
}

}  // namespace moe
