// One 256-row x 256-column tile of the grouped SwiGLU FFN in MXFP8 on gfx950
// (v_mfma_scale_f32_32x32x64_f8f6f4).  Shared by the standalone grouped MXFP8 GEMM kernels
// and the persistent forward kernel; the operation and the tile's design are described at
// the top of gemm_mx.hip.
#pragma once

#include "gemm_tile.hpp"
#include "mx.hpp"

namespace moe {

constexpr int kMxBK = 128;                                              // K values (bytes) per stage
constexpr int kMxDataBytes = (kGemmBM + kGemmBN) * kMxBK;               // 64 KiB
constexpr int kMxStageBytes = kMxDataBytes + (kGemmBM + kGemmBN) * 4;   // + a scale word per row
constexpr int kMxLds = 2 * kMxStageBytes;                               // 132 KiB

struct TileMX {
  const uint8_t* a;     // the tile's first A row; row stride K
  const uint8_t* as;    // the scale word of its first row in K-tile plane 0
  int64_t as_plane;     // bytes between K-tile planes of the A scales (4 * total A rows)
  void* o;              // MODE 0: h codes, MODE 1: bf16 rows; row stride Nout elements
  uint8_t* os;          // MODE 0: the h scale word of the tile's first row in plane 0
  int64_t os_plane;     // MODE 0: bytes between planes of the h scales
  int rows;             // valid rows, 1..256; rows beyond re-read row rows-1 and are not stored
  // MODE 2 (backward GEMM1): dh in, h and [da | db] out as bf16, [da | db] as MX codes
  const uint16_t* dh;   // [rows][Nout] from the tile's first row
  uint16_t* hb;         // [rows][Nout]
  uint16_t* dab;        // [rows][2 Nout]
  uint8_t* dabq;        // [rows][2 Nout] codes
  uint8_t* dabs;        // scales of the whole [nmax][2 Nout] code matrix (MXFP8 scale layout)
  int64_t row0, nmax;   // global index of the tile's first row; rows of the scale layout
  const uint64_t* row_dst;  // MODE 1: null, or per tile row the address its output row goes to
  // Block mode (the BLK template argument; blk_log2 = 6, 7 or 8): the tile's rows live in 256 >> blk_log2 blocks
  // of 1 << blk_log2 consecutive rows each (the persistent kernel's ring slots), block b's
  // codes at ablk[b] (row stride K) and its scale word of plane 0 at asblk[b] + 4 * row
  // (planes as_plane apart); MODE 0 writes h codes to oblk[b] (row stride Nout) and their scale
  // words to osblk[b] (planes os_plane apart).  Rows past `rows` read whatever their block holds
  // (never stored; a block is a whole slot, so the reads stay inside it).
  int blk_log2;
  const uint8_t* ablk[4];
  const uint8_t* asblk[4];
  uint8_t* oblk[4];
  uint8_t* osblk[4];
};

__device__ __forceinline__ i32x8 ld_frag(const char* s, int row, int c0) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(s + swz_off(row, c0));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(s + swz_off(row, c0 + 2));
  return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

// b0/b1: this expert's weight codes ([Nout][K]); bs0/bs1: the scale word of its row 0 in
// plane 0; bs_plane: bytes between the weights' K-tile planes.  A_CPOL: cache policy of the
// A code and A scale loads (0 = default; 16 = sc1, a device-coherent load that does not hit
// this CU's L1, for rows another CU just wrote).
template <int MODE, int A_CPOL = 0, bool BLK = false>
__device__ __forceinline__ void gemm_mx_tile(const TileMX& io, const uint8_t* __restrict__ b0,
                                             const uint8_t* __restrict__ b1, const uint8_t* __restrict__ bs0,
                                             const uint8_t* __restrict__ bs1, int64_t bs_plane, int c0, int Nout,
                                             int K, char* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hi = lane >> 5;
  const int lrow = lane >> 3, lpos = lane & 7;
  const int lch_even = lpos ^ (lrow >> 1);
  const int lch_odd = lpos ^ (4 + (lrow >> 1));
  const int nk = K / kMxBK;
  const int rows = io.rows;

  // fills: this wave's row groups g = wave*4 + i (rows g*8 + lrow) of the A and B tiles
  // (32-bit offsets from a base shared by the wave: B rows of one wave are all W1 rows or all
  // W3 rows, since rows 32 w .. 32 w + 31 are filled by wave w)
  // (block mode, BLK: a wave's 32 rows lie in one block, whose base is the wave's A base)
  constexpr bool bmode = BLK;
  const int bmask = bmode ? (1 << io.blk_log2) - 1 : 0;
  // (both bases are the same for the whole wave; read through readfirstlane they stay in
  // scalar registers, so every fill takes the scalar-base + 32-bit-offset form instead of a
  // 64-bit vector address add per fill)
  const uint8_t* abase = wave_uniform(
      bmode ? pick4((wave * 32) >> io.blk_log2, io.ablk[0], io.ablk[1], io.ablk[2], io.ablk[3]) : io.a);
  const uint8_t* bbase = wave_uniform((MODE != 1 && (wave & 1)) ? b1 : b0);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 8 + lrow;
    const int lch = (i & 1) ? lch_odd : lch_even;
    aoff[i] = uint32_t(bmode ? (row & bmask) : min(row, rows - 1)) * uint32_t(K) + lch * 16;
    const int n = (MODE != 1) ? min(c0 + (row >> 6) * 32 + (row & 31), Nout - 1) : min(c0 + row, Nout - 1);
    boff[i] = uint32_t(n) * uint32_t(K) + lch * 16;
  }
  // scale words: waves 0-3 fetch A rows 64*wave + lane, waves 4-7 B rows 64*(wave-4) + lane
  const uint8_t* sp;
  int64_t splane;
  {
    const int row = (wave & 3) * 64 + lane;
    if (wave < 4) {
      sp = bmode ? pick4(row >> io.blk_log2, io.asblk[0], io.asblk[1], io.asblk[2], io.asblk[3]) + 4 * size_t(row & bmask)
                 : io.as + 4 * size_t(min(row, rows - 1));
      splane = io.as_plane;
    } else if (MODE != 1) {
      const int n = min(c0 + (row >> 6) * 32 + (row & 31), Nout - 1);
      sp = (((row >> 5) & 1) ? bs1 : bs0) + 4 * size_t(n);
      splane = bs_plane;
    } else {
      sp = bs0 + 4 * size_t(min(c0 + row, Nout - 1));
      splane = bs_plane;
    }
  }
  // LDS destinations of this wave's fills (the M0 operand) as scalars: the wave's first A
  // row group and its scale words in stage 0; stage 1 and the B tile are constant offsets
  const uint32_t lds_dst0 = __builtin_amdgcn_readfirstlane(lds_addr(smem + wave * 4 * 1024));
  const uint32_t lds_sc0 = __builtin_amdgcn_readfirstlane(lds_addr(smem + kMxDataBytes + wave * 256));
  auto issue = [&](int ks) {
    const uint32_t stage = uint32_t((ks & 1) * kMxStageBytes);
    const uint32_t da = lds_dst0 + stage, db = da + uint32_t(kGemmBM * kMxBK);
    const lds_void_ptr ls = (lds_void_ptr)(uintptr_t)(lds_sc0 + stage);
    const int koff = ks * kMxBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(abase + (aoff[i] + koff)),
                                       (lds_void_ptr)(uintptr_t)(da + uint32_t(i * 1024)), 16, 0, A_CPOL);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bbase + (boff[i] + koff)),
                                       (lds_void_ptr)(uintptr_t)(db + uint32_t(i * 1024)), 16, 0, 0);
    }
    if (A_CPOL != 0 && wave < 4)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(sp + ks * splane), ls, 4, 0, A_CPOL);
    else
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(sp + ks * splane), ls, 4, 0, 0);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // Software pipeline over K (two sub-steps of 64 per 128-value stage).  A fragment or scale
  // register is reloaded as soon as the last MFMA that reads it has issued, so the reads of
  // the next sub-step overlap the MFMAs of this one; each MFMA waits only for its own
  // operands.  A stage's barrier sits between its two sub-steps: by then every wave has read
  // the stage's second-sub-step fragments, so the fill two stages ahead goes into it, and the
  // second sub-step's MFMAs cover the reads of the next stage's first fragments and of its
  // scales.  A fill has one stage of MFMA work to land.  Per accumulator the MFMAs run in K
  // order, so the result does not depend on this schedule.  Scales: lane (row r32, half hi)
  // takes byte 2 st + hi of its row's word (block hi of sub-step st), read as one byte.
  // Per-lane LDS byte offsets inside a stage: the two 16-byte chunks of a fragment of
  // sub-step st (rows 32 apart share the XOR pattern, so a row block adds 4096), and the
  // scale word of the lane's row (a row block adds 128).  They are passed
  // through an opaque copy every K step, so the compiler keeps these ten values instead of
  // hoisting every address of both stages out of the loop.
  int offA[2][2], offB[2][2], offSA, offSB;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      offA[st][h] = swz_off(wm * 64 + r32, 4 * st + hi + 2 * h);
      offB[st][h] = kGemmBM * kMxBK + swz_off(wn * 128 + r32, 4 * st + hi + 2 * h);
    }
  offSA = kMxDataBytes + 4 * (wm * 64 + r32);
  offSB = kMxDataBytes + 4 * (kGemmBM + wn * 128 + r32);
  auto ld2 = [&](const char* stg, int o0, int o1, int imm) -> i32x8 {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(stg + o0 + imm);
    const u32x4 up = *reinterpret_cast<const u32x4*>(stg + o1 + imm);
    return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(up[0]), int(up[1]), int(up[2]), int(up[3])};
  };
  auto frag_a = [&](const char* stg, int st, int m) { return ld2(stg, offA[st][0], offA[st][1], m * 4096); };
  auto frag_b = [&](const char* stg, int st, int n) { return ld2(stg, offB[st][0], offB[st][1], n * 4096); };
  // the scale word of a row (its four blocks), shifted so that byte 0 / byte 2 is block
  // hi / 2 + hi: the MFMA's op_sel picks the sub-step's byte
  auto scl_a = [&](const char* stg, int m) -> int {
    return int(*reinterpret_cast<const uint32_t*>(stg + offSA + 128 * m) >> (8 * hi));
  };
  auto scl_b = [&](const char* stg, int n) -> int {
    return int(*reinterpret_cast<const uint32_t*>(stg + offSB + 128 * n) >> (8 * hi));
  };
  auto mfma = [&](int st, int m, int n, const i32x8& a, const i32x8& b, int sa, int sb) {
    if (st == 0) acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[m][n], 0, 0, 0, sa, 0, sb);
    else acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[m][n], 0, 0, 2, sa, 2, sb);
  };

  issue(0);
  if (nk > 1) issue(1);
  if (nk > 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");   // stage 0 landed (9 fills a stage)
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Row padding: a wave whose 32-row blocks lie wholly past the tile's valid rows skips
  // their fragment reads and MFMAs (they only feed rows that are never stored); it still
  // fills and meets every barrier.
  const int mv = __builtin_amdgcn_readfirstlane(min(2, max(0, (rows - wm * 64 + 31) >> 5)));
  auto kloop = [&](auto mvc) {
    constexpr int MV = decltype(mvc)::value;
    i32x8 fa[2], fb[4];
    int sa[2], sb[4];                 // the stage's scale words; the next stage's are loaded in
                                      // place after their last MFMA
    if constexpr (MV > 0) {
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        fa[m] = frag_a(smem, 0, m);
        sa[m] = scl_a(smem, m);
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        fb[n] = frag_b(smem, 0, n);
        sb[n] = scl_b(smem, n);
      }
    }
    for (int ks = 0; ks < nk; ++ks) {
      const char* cs = smem + (ks & 1) * kMxStageBytes;
      const char* ns = smem + ((ks + 1) & 1) * kMxStageBytes;   // after the last stage: stale, unused
      asm volatile("" : "+v"(offA[0][0]), "+v"(offA[0][1]), "+v"(offA[1][0]), "+v"(offA[1][1]), "+v"(offB[0][0]),
                   "+v"(offB[0][1]), "+v"(offB[1][0]), "+v"(offB[1][1]), "+v"(offSA), "+v"(offSB));
      // sub-step 0 of stage ks; reload sub-step 1's fragments of stage ks
      if constexpr (MV == 2) {
        mfma(0, 0, 0, fa[0], fb[0], sa[0], sb[0]);
        mfma(0, 0, 1, fa[0], fb[1], sa[0], sb[1]);
        mfma(0, 0, 2, fa[0], fb[2], sa[0], sb[2]);
        mfma(0, 0, 3, fa[0], fb[3], sa[0], sb[3]);
        fa[0] = frag_a(cs, 1, 0);
        mfma(0, 1, 0, fa[1], fb[0], sa[1], sb[0]);
        fb[0] = frag_b(cs, 1, 0);
        mfma(0, 1, 1, fa[1], fb[1], sa[1], sb[1]);
        fb[1] = frag_b(cs, 1, 1);
        mfma(0, 1, 2, fa[1], fb[2], sa[1], sb[2]);
        fb[2] = frag_b(cs, 1, 2);
        mfma(0, 1, 3, fa[1], fb[3], sa[1], sb[3]);
        fb[3] = frag_b(cs, 1, 3);
        fa[1] = frag_a(cs, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      } else if constexpr (MV == 1) {
        mfma(0, 0, 0, fa[0], fb[0], sa[0], sb[0]);
        fb[0] = frag_b(cs, 1, 0);
        mfma(0, 0, 1, fa[0], fb[1], sa[0], sb[1]);
        fb[1] = frag_b(cs, 1, 1);
        mfma(0, 0, 2, fa[0], fb[2], sa[0], sb[2]);
        fb[2] = frag_b(cs, 1, 2);
        mfma(0, 0, 3, fa[0], fb[3], sa[0], sb[3]);
        fb[3] = frag_b(cs, 1, 3);
        fa[0] = frag_a(cs, 1, 0);
      }
      // this wave's fills of stage ks + 1 and its reads of stage ks are done; then everyone's.
      // The accumulators pass through the statement, so no MFMA moves across the barrier.
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier"
                   : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]), "+v"(acc[1][0]),
                     "+v"(acc[1][1]), "+v"(acc[1][2]), "+v"(acc[1][3])
                   :
                   : "memory");
      if (ks + 2 < nk) issue(ks + 2);     // into stage ks, which nobody reads any more
      // sub-step 1 of stage ks; reload the next stage's sub-step-0 fragments and scale words
      if constexpr (MV == 2) {
        mfma(1, 0, 0, fa[0], fb[0], sa[0], sb[0]);
        mfma(1, 0, 1, fa[0], fb[1], sa[0], sb[1]);
        mfma(1, 0, 2, fa[0], fb[2], sa[0], sb[2]);
        mfma(1, 0, 3, fa[0], fb[3], sa[0], sb[3]);
        fa[0] = frag_a(ns, 0, 0);
        sa[0] = scl_a(ns, 0);
        mfma(1, 1, 0, fa[1], fb[0], sa[1], sb[0]);
        fb[0] = frag_b(ns, 0, 0);
        sb[0] = scl_b(ns, 0);
        mfma(1, 1, 1, fa[1], fb[1], sa[1], sb[1]);
        fb[1] = frag_b(ns, 0, 1);
        sb[1] = scl_b(ns, 1);
        mfma(1, 1, 2, fa[1], fb[2], sa[1], sb[2]);
        fb[2] = frag_b(ns, 0, 2);
        sb[2] = scl_b(ns, 2);
        mfma(1, 1, 3, fa[1], fb[3], sa[1], sb[3]);
        fb[3] = frag_b(ns, 0, 3);
        sb[3] = scl_b(ns, 3);
        fa[1] = frag_a(ns, 0, 1);
        sa[1] = scl_a(ns, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
      } else if constexpr (MV == 1) {
        mfma(1, 0, 0, fa[0], fb[0], sa[0], sb[0]);
        fb[0] = frag_b(ns, 0, 0);
        sb[0] = scl_b(ns, 0);
        mfma(1, 0, 1, fa[0], fb[1], sa[0], sb[1]);
        fb[1] = frag_b(ns, 0, 1);
        sb[1] = scl_b(ns, 1);
        mfma(1, 0, 2, fa[0], fb[2], sa[0], sb[2]);
        fb[2] = frag_b(ns, 0, 2);
        sb[2] = scl_b(ns, 2);
        mfma(1, 0, 3, fa[0], fb[3], sa[0], sb[3]);
        fb[3] = frag_b(ns, 0, 3);
        sb[3] = scl_b(ns, 3);
        fa[0] = frag_a(ns, 0, 0);
        sa[0] = scl_a(ns, 0);
      }
    }
  };
  if (mv == 2) kloop(std::integral_constant<int, 2>{});
  else if (mv == 1) kloop(std::integral_constant<int, 1>{});
  else kloop(std::integral_constant<int, 0>{});
  __syncthreads();                        // the epilogues reuse the stages

  if (MODE == 2) {
    // Backward epilogue, two passes of 128 tile rows: stage (a, b) as fp32 pairs in LDS
    // ([128][128] float2 = 128 KiB), then each thread takes one 32-value f block of one
    // row: h = silu(a) b, da = dh b silu'(a), db = dh silu(a) as bf16, and da, db quantised
    // along F (MX blocks of 32; the block maximum is taken over a first pass, the codes
    // over a second that recomputes the values).
    float2* stg = reinterpret_cast<float2*>(smem);
    const int F2 = 2 * Nout;
#pragma unroll   // acc[m] must stay in registers
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int lr = wm * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
          stg[lr * 128 + (wn * 2 + q) * 32 + r32] = make_float2(acc[m][2 * q][e], acc[m][2 * q + 1][e]);
        }
      __syncthreads();
      const int lr = tid >> 2, q32 = tid & 3;                    // 128 rows x 4 blocks = 512 threads
      const int trow = (lr >> 5) * 64 + m * 32 + (lr & 31);
      const int f0 = c0 + q32 * 32;
      if (trow < rows && f0 < Nout) {
        const float2* sp = stg + lr * 128 + q32 * 32;
        u32x4 dv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) dv[c] = reinterpret_cast<const u32x4*>(io.dh + size_t(trow) * Nout + f0)[c];
        auto grad = [&](int i, float* hh, float* ga, float* gb) {
          const float2 ab = sp[i];
          const uint32_t w = dv[i >> 3][(i & 7) >> 1];
          const float dhv = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
          const float sg = 1.0f / (1.0f + __expf(-ab.x));
          const float sa = ab.x * sg;
          *hh = sa * ab.y;
          *ga = dhv * ab.y * (sg * (1.0f + ab.x * (1.0f - sg)));
          *gb = dhv * sa;
        };
        uint32_t mda = 0, mdb = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 hv, dav, dbv;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float hh[2], ga[2], gb[2];
            grad(c * 8 + 2 * w, &hh[0], &ga[0], &gb[0]);
            grad(c * 8 + 2 * w + 1, &hh[1], &ga[1], &gb[1]);
            mda = max(mda, max(__float_as_uint(ga[0]) & 0x7FFFFFFFu, __float_as_uint(ga[1]) & 0x7FFFFFFFu));
            mdb = max(mdb, max(__float_as_uint(gb[0]) & 0x7FFFFFFFu, __float_as_uint(gb[1]) & 0x7FFFFFFFu));
            hv[w] = pack_bf16x2(hh[0], hh[1]);
            dav[w] = pack_bf16x2(ga[0], ga[1]);
            dbv[w] = pack_bf16x2(gb[0], gb[1]);
          }
          reinterpret_cast<u32x4*>(io.hb + size_t(trow) * Nout + f0)[c] = hv;
          reinterpret_cast<u32x4*>(io.dab + size_t(trow) * F2 + f0)[c] = dav;
          reinterpret_cast<u32x4*>(io.dab + size_t(trow) * F2 + Nout + f0)[c] = dbv;
        }
        const int ea = mda ? mx_block_exp(mda) : 0, eb = mdb ? mx_block_exp(mdb) : 0;
        const float ia = mx_inv_scale(ea), ib = mx_inv_scale(eb);
        uint32_t qa[8], qb[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float hh[4], ga[4], gb[4];
#pragma unroll
          for (int z = 0; z < 4; ++z) grad(c * 4 + z, &hh[z], &ga[z], &gb[z]);
          qa[c] = mda ? mx_pack4(ga[0], ga[1], ga[2], ga[3], ia) : 0u;
          qb[c] = mdb ? mx_pack4(gb[0], gb[1], gb[2], gb[3], ib) : 0u;
        }
        u32x4* qd = reinterpret_cast<u32x4*>(io.dabq + size_t(trow) * F2 + f0);
        qd[0] = u32x4{qa[0], qa[1], qa[2], qa[3]};
        qd[1] = u32x4{qa[4], qa[5], qa[6], qa[7]};
        u32x4* qe = reinterpret_cast<u32x4*>(io.dabq + size_t(trow) * F2 + Nout + f0);
        qe[0] = u32x4{qb[0], qb[1], qb[2], qb[3]};
        qe[1] = u32x4{qb[4], qb[5], qb[6], qb[7]};
        const int64_t grow = io.row0 + trow;
        io.dabs[mx_scale_index(io.nmax, grow, f0 >> 5)] = uint8_t(mda ? ea + 127 : 0);
        io.dabs[mx_scale_index(io.nmax, grow, (Nout + f0) >> 5)] = uint8_t(mdb ? eb + 127 : 0);
      }
      __syncthreads();
    }
    return;
  }

  // Epilogue through LDS (the stages are free after the last barrier).  Each wave writes
  // its results into a row-major tile whose rows are padded by 16 bytes; the lane layout of
  // the accumulators is column r32, rows 8*(e/4) + 4*hi + e%4 of each 32x32 block.
  //  MODE 0: the fp32 h tile [256][128]; then every thread quantises whole 32-value blocks
  //          of it on its own and writes 32 code bytes as two 16-byte vectors plus the scale.
  //  MODE 1: the bf16 output tile [256][256]; then 16-byte row segments go to global memory.
  constexpr int kPitch = 528;                                   // 512 bytes of data + 16
  static_assert(kGemmBM * kPitch <= kMxLds, "staged tile exceeds the LDS stages");
  char* ot = smem;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int rb = wm * 64 + m * 32;
    if (MODE == 0) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int fc = (wn * 2 + q) * 32 + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rb + 8 * (e >> 2) + 4 * hi + (e & 3);
          *reinterpret_cast<float*>(ot + row * kPitch + fc * 4) = silu_f32(acc[m][2 * q][e]) * acc[m][2 * q + 1][e];
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int cc = wn * 128 + n * 32 + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rb + 8 * (e >> 2) + 4 * hi + (e & 3);
          *reinterpret_cast<uint16_t*>(ot + row * kPitch + cc * 2) = f32_to_bf16(acc[m][n][e]);
        }
      }
    }
  }
  __syncthreads();
  if (MODE == 0) {
    uint8_t* hq = static_cast<uint8_t*>(io.o);
    for (int b = tid; b < kGemmBM * 4; b += kGemmThreads) {    // 4 blocks of 32 f per row
      const int row = b >> 2, blk = b & 3;
      if (row >= rows) continue;
      const f32x4* src = reinterpret_cast<const f32x4*>(ot + row * kPitch + blk * 128);
      f32x4 v[8];
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = src[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) mx = max(mx, __float_as_uint(v[i][w]) & 0x7FFFFFFFu);
      }
      u32x4 c0v = {0, 0, 0, 0}, c1v = {0, 0, 0, 0};
      uint32_t sc = 0;
      if (mx != 0) {
        const int ex = mx_block_exp(mx);
        const float inv = mx_inv_scale(ex);
        sc = uint32_t(ex + 127);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          c0v[w] = mx_pack4(v[w][0], v[w][1], v[w][2], v[w][3], inv);
          c1v[w] = mx_pack4(v[4 + w][0], v[4 + w][1], v[4 + w][2], v[4 + w][3], inv);
        }
      }
      uint8_t* hrow = bmode ? pick4(row >> io.blk_log2, io.oblk[0], io.oblk[1], io.oblk[2], io.oblk[3]) + size_t(row & bmask) * Nout
                           : hq + size_t(row) * Nout;
      uint8_t* srow = bmode ? pick4(row >> io.blk_log2, io.osblk[0], io.osblk[1], io.osblk[2], io.osblk[3]) + 4 * size_t(row & bmask)
                           : io.os + 4 * size_t(row);
      u32x4* dst = reinterpret_cast<u32x4*>(hrow + c0 + blk * 32);
      dst[0] = c0v;
      dst[1] = c1v;
      srow[(c0 >> 7) * io.os_plane + blk] = uint8_t(sc);
    }
  } else {
    uint16_t* orow0 = static_cast<uint16_t*>(io.o);
    const int ncols = min(kGemmBN, Nout - c0);
    for (int v = tid; v < kGemmBM * (kGemmBN / 8); v += kGemmThreads) {
      const int row = v >> 5, cv = v & 31;                   // 32 vectors of 8 bf16 per row
      if (row < rows && cv * 8 < ncols) {
        uint16_t* orow = io.row_dst ? reinterpret_cast<uint16_t*>(io.row_dst[row]) : orow0 + size_t(row) * Nout;
        *reinterpret_cast<u32x4*>(orow + c0 + cv * 8) = *reinterpret_cast<const u32x4*>(ot + row * kPitch + cv * 16);
      }
    }
  }
  __syncthreads();     // the next tile's fills reuse the stages
}

}  // namespace moe
