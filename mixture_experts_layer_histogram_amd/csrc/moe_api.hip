// extern "C" entry points of libmoe: argument checks, workspace sizing, launches.
// Every check runs before the first HIP call, so argument errors need no GPU.
#include <string.h>

#include "common.hpp"

namespace moe {
hipError_t launch_layout(const moe_shape_t& s, const int32_t* e2l, int El, int mb, const float* const* logits,
                         int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                         int32_t* pull_src, int32_t* slot_of, char* ws, const WsLayout& L, hipStream_t st);
hipError_t launch_dispatch(const moe_shape_t& s, const void* const* x, const int32_t* pull_src, char* xe,
                           const int32_t* ctrl, int cus, hipStream_t st);
hipError_t launch_ffn(const moe_shape_t& s, int El, const void* xe, const int32_t* offsets, const void* w1,
                      const void* w3, const void* w2, void* ye, char* ws, const WsLayout& L, int cus,
                      hipStream_t st, const uint64_t* row_dst, const uint64_t* row_src);
hipError_t launch_pair_addr(const moe_shape_t& s, const int32_t* pull_src, const int32_t* slot_of,
                            void* const* recv, const void* const* x, const int32_t* ctrl, uint64_t* push_dst,
                            uint64_t* pull_addr, int cus, hipStream_t st, const float* dg, float* dgp);
hipError_t launch_combine(const moe_shape_t& s, const char* ye, const int32_t* pull_src,
                          const int32_t* slot_of, const float* topk_w, void* const* recv, void* const* y,
                          const int32_t* ctrl, int cus, hipStream_t st);
hipError_t launch_mx_quantize(const void* src, int src_dtype, int64_t rows, int K, uint8_t* codes,
                              uint8_t* scales, int cus, hipStream_t st);
hipError_t launch_dispatch_mx(const moe_shape_t& s, const void* const* x, const int32_t* pull_src, uint8_t* xe,
                              uint8_t* xe_scales, int64_t nmax, const int32_t* ctrl, int cus, hipStream_t st);
hipError_t launch_ffn_mx(const moe_shape_t& s, int El, const uint8_t* xe, const uint8_t* xe_scales,
                         const int32_t* offsets, const uint8_t* w1, const uint8_t* w3, const uint8_t* w2,
                         const uint8_t* w1s, const uint8_t* w3s, const uint8_t* w2s, void* ye, char* ws,
                         const WsLayout& L, int cus, hipStream_t st, const uint64_t* row_dst);
hipError_t launch_merge(const moe_shape_t& s, const int32_t* slot_of, const float* topk_w, void* const* recv,
                        void* const* y, int cus, hipStream_t st);
hipError_t launch_persistent(const moe_shape_t& s, int El, const void* const* x, const void* w1, const void* w3,
                             const void* w2, const int32_t* pull_src, const int32_t* slot_of,
                             const int32_t* offsets, char* ring, long long slot_bytes, int blk_log2,
                             const sched::Plan& plan, int grid, long long budget, void* const* recv, char* ws,
                             const WsLayout& L, moe_trace_event_t* trace, int32_t* trace_count, int trace_cap,
                             const uint64_t* row_dst, bool reverse, const moe_mx_scales_t* w_scales,
                             hipStream_t st);
hipError_t persistent_occupancy(int* blocks_per_cu, bool mx);
long long persist_mx_slot_layout(int d, int F, int cr, long long* tok_s_off, long long* h_off, long long* h_s_off);
hipError_t launch_rows_bmn(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, int ksplit, uint16_t* C, int K,
                           int Nout, const int32_t* offsets, const int32_t* mtb, const int32_t* ctrl, int El, int cus,
                           hipStream_t st, const uint64_t* row_dst);
hipError_t launch_gemm1_bwd(const uint16_t* xe, const uint16_t* w1, const uint16_t* w3, const uint16_t* dh,
                            uint16_t* h, uint16_t* dab, int d, int F, const int32_t* offsets, const int32_t* mtb,
                            const int32_t* ctrl, int El, int cus, hipStream_t st, const uint64_t* row_src = nullptr);
hipError_t launch_wgrad(const uint16_t* A, int lda, const uint16_t* B, int ldb, const int32_t* offsets, uint16_t* C,
                        int El, int M, int Nc, int cus, hipStream_t st, const uint64_t* b_blk = nullptr,
                        const int32_t* mtile_base = nullptr);
hipError_t launch_pull_reverse(const moe_shape_t& s, const void* const* dy, const uint16_t* ye,
                               const int32_t* pull_src, const int32_t* slot_of, const float* topk_w,
                               const int32_t* ctrl, uint16_t* dO, float* dg, int cus, hipStream_t st,
                               void* const* recv = nullptr);
hipError_t launch_ring_rows(const moe_shape_t& s, int El, int max_mtiles, const void* const* x, const int32_t* pull_src,
                            const int32_t* offsets, const int32_t* mtile_base, const int32_t* ctrl,
                            const int32_t* resident, const void* ring, long long slot_bytes, int n_slots,
                            int chunk_log2, void* xe, uint64_t* blk_src, int32_t* blk_held, uint64_t* row_src, int cus,
                            hipStream_t st);
hipError_t launch_gate_grad(const moe_shape_t& s, const float* topk_w, const int32_t* topk_idx, const int32_t* slot_of,
                            const float* dgp, float* const* dlogits, int cus, hipStream_t st);
hipError_t launch_push_grad(const moe_shape_t& s, const char* dX, const float* dg, const int32_t* pull_src,
                            const int32_t* slot_of, void* const* recv, float* dgp, const int32_t* ctrl, int cus,
                            hipStream_t st);
hipError_t launch_mx_quantize_t(const uint16_t* src, int P, int C, int batches, uint8_t* codes, int64_t ldk, int k0,
                                uint8_t* scales, int64_t rows_total, int cus, hipStream_t st);
hipError_t launch_pull_reverse_mx(const moe_shape_t& s, const void* const* dy, const uint16_t* ye,
                                  const int32_t* pull_src, const int32_t* slot_of, const float* topk_w,
                                  const int32_t* ctrl, uint16_t* dO, uint8_t* dOq, uint8_t* dOs, float* dg, int64_t nmax,
                                  int cus, hipStream_t st);
hipError_t launch_rows_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, uint16_t* C, int K,
                          int Nout, int64_t nmax, const int32_t* offsets, const int32_t* mtb, const int32_t* ctrl,
                          int El, int cus, hipStream_t st, const uint64_t* row_dst);
hipError_t launch_gemm1_bwd_mx(const uint8_t* xe, const uint8_t* xes, const uint8_t* w1, const uint8_t* w3,
                               const uint8_t* w1s, const uint8_t* w3s, const uint16_t* dh, uint16_t* h, uint16_t* dab,
                               uint8_t* dabq, uint8_t* dabs, int d, int F, int64_t nmax, const int32_t* offsets,
                               const int32_t* mtb, const int32_t* ctrl, int El, int cus, hipStream_t st);
}  // namespace moe

using namespace moe;

namespace {

int check_shape(const moe_shape_t* s, const moe_placement_t* p) {
  if (!s || !p) return MOE_EINVAL;
  if (s->R < 1 || s->R > MOE_MAX_RANKS || s->T < 1 || s->d < 1 || s->F < 1) return MOE_EINVAL;
  if (s->E < 1 || s->E > 1024 || s->k < 1 || s->k > 16 || s->k > s->E) return MOE_EINVAL;
  if (p->E_local < 1 || p->E_local > s->E) return MOE_EINVAL;
  if (int64_t(s->R) * s->T * s->k >= (int64_t(1) << 31)) return MOE_EINVAL;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16 && s->dtype != MOE_MXFP8) return MOE_EINVAL;
  const int esz = s->dtype == MOE_F32 ? 4 : 2;
  if ((int64_t(s->d) * esz) % 16 || (int64_t(s->F) * esz) % 16) return MOE_EALIGN;
  if (s->dtype == MOE_BF16 && (s->d % kGemmBK || s->F % kGemmBK)) return MOE_EALIGN;
  if (s->dtype == MOE_MXFP8 && (s->d % 128 || s->F % 128)) return MOE_EALIGN;   // one 128-value GEMM stage
  return MOE_OK;
}

int check_ws(const moe_shape_t* s, const moe_placement_t* p, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return MOE_EALIGN;
  if (ws_bytes < ws_layout(*s, p->E_local).total) return MOE_ENOSPC;
  return MOE_OK;
}

template <typename T>
int check_ptr_table(const T* const* tab, int R) {
  if (!tab) return MOE_EINVAL;
  for (int r = 0; r < R; ++r)
    if (!tab[r] || (reinterpret_cast<uintptr_t>(tab[r]) & 15)) return tab[r] ? MOE_EALIGN : MOE_EINVAL;
  return MOE_OK;
}

int aligned16(const void* q) { return q && !(reinterpret_cast<uintptr_t>(q) & 15); }

// non-null and 4-byte aligned (scale arrays, read as 32-bit words)
int check_scales(const void* q) {
  if (!q) return MOE_EINVAL;
  return (reinterpret_cast<uintptr_t>(q) & 3) ? MOE_EALIGN : MOE_OK;
}

int check_w_scales(const moe_mx_scales_t* w) {
  if (!w) return MOE_EINVAL;
  int rc;
  if ((rc = check_scales(w->w1)) || (rc = check_scales(w->w3)) || (rc = check_scales(w->w2))) return rc;
  return MOE_OK;
}

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::atomic<int> cached[64];       // zero-initialised (static storage)
  const bool slot = dev >= 0 && dev < 64;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (n < 8) n = 8;
  if (slot) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int minibatch_of(const moe_exec_t* ex) { return (ex && ex->minibatch_rows > 0) ? ex->minibatch_rows : 128; }

// persistent path: chunk rows must divide the 256-row GEMM tile (64, 128 or 256)
int chunk_log2_of(const moe_exec_t* ex) {
  const int mb = minibatch_of(ex);
  return mb == 64 ? 6 : mb == 128 ? 7 : mb == 256 ? 8 : -1;
}

size_t ring_slot_bytes(const moe_shape_t& s, int blk_log2) {
  if (s.dtype == MOE_MXFP8) {     // codes and scale words of the token rows and of h
    long long a, b, c;
    return size_t(persist_mx_slot_layout(s.d, s.F, 1 << blk_log2, &a, &b, &c));
  }
  return (size_t(1) << blk_log2) * (size_t(s.d) + size_t(s.F)) * 2;
}

long long wall_ticks_per_us() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    khz = 100000;
  return khz / 1000 > 0 ? khz / 1000 : 1;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// execution knobs of the multi-kernel entry points: the trace is the persistent path's only
int check_ex(const moe_exec_t* ex) {
  if (ex && (ex->trace != 0 || ex->reverse_ring != 0 || ex->minibatch_rows < 0)) return MOE_EINVAL;
  return MOE_OK;
}

// backward calls: a shape of the given dtype, the forward's workspace, and the backward workspace
int check_bwd(const moe_shape_t* s, const moe_placement_t* p, const void* ws, size_t ws_bytes, const void* bws,
              size_t bws_bytes, int dtype = MOE_BF16) {
  int rc = check_shape(s, p);
  if (rc) return rc;
  if (s->dtype != dtype) return MOE_EUNSUP;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  if (!bws) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(bws) & 255) return MOE_EALIGN;
  if (bws_bytes < bwd_layout(*s, p->E_local).total) return MOE_ENOSPC;
  return MOE_OK;
}

}  // namespace

extern "C" {

int64_t moe_max_pairs(const moe_shape_t* s, const moe_placement_t* p) {
  if (!s || !p || s->R < 1 || s->T < 1 || s->k < 1 || p->E_local < 1) return -1;
  return int64_t(s->R) * s->T * (s->k < p->E_local ? s->k : p->E_local);
}

size_t moe_workspace_bytes(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex) {
  (void)ex;
  if (check_shape(s, p) != MOE_OK) return 0;
  return ws_layout(*s, p->E_local).total;
}

int moe_mx_quantize(const void* src, int32_t src_dtype, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                    void* stream) {
  if (src_dtype != MOE_BF16 && src_dtype != MOE_F32) return MOE_EINVAL;
  if (rows < 0 || K < 1 || rows > (int64_t(1) << 40) / K) return MOE_EINVAL;
  if (K % 128) return MOE_EALIGN;                // whole 32-bit scale words per row
  if (!src || !codes || !scales) return MOE_EINVAL;
  if (!aligned16(src) || !aligned16(codes)) return MOE_EALIGN;
  return hip_rc(launch_mx_quantize(src, src_dtype, rows, K, codes, scales, cu_count(),
                                   static_cast<hipStream_t>(stream)));
}

int moe_layout(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
               const float* const* logits, int32_t* topk_idx, float* topk_w, int32_t* counts,
               int32_t* offsets, int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes,
               void* stream) {
  int rc = check_shape(s, p);
  if (rc || (rc = check_ex(ex))) return rc;
  if (!p->expert_to_local || !topk_idx || !topk_w || !counts || !offsets || !pull_src || !slot_of)
    return MOE_EINVAL;
  if (ex && ex->minibatch_rows < 0) return MOE_EINVAL;
  if ((rc = check_ptr_table(logits, s->R))) return rc;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  const WsLayout L = ws_layout(*s, p->E_local);
  return hip_rc(launch_layout(*s, p->expert_to_local, p->E_local, minibatch_of(ex), logits, topk_idx, topk_w,
                              counts, offsets, pull_src, slot_of, static_cast<char*>(ws), L,
                              static_cast<hipStream_t>(stream)));
}

int moe_dispatch_pull(const moe_shape_t* s, const moe_placement_t* p, const void* const* x,
                      const int32_t* pull_src, const int32_t* offsets, void* xe, uint8_t* xe_scales, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_shape(s, p);
  if (rc) return rc;
  if (!pull_src || !offsets) return MOE_EINVAL;
  if (!aligned16(xe)) return xe ? MOE_EALIGN : MOE_EINVAL;
  if (s->dtype == MOE_MXFP8 && (rc = check_scales(xe_scales))) return rc;
  if ((rc = check_ptr_table(x, s->R))) return rc;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  const WsLayout L = ws_layout(*s, p->E_local);
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + L.ctrl);
  if (s->dtype == MOE_MXFP8)
    return hip_rc(launch_dispatch_mx(*s, x, pull_src, static_cast<uint8_t*>(xe), xe_scales, L.max_pairs, ctrl,
                                     cu_count(), static_cast<hipStream_t>(stream)));
  return hip_rc(launch_dispatch(*s, x, pull_src, static_cast<char*>(xe), ctrl, cu_count(),
                                static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex, const void* xe,
                   const uint8_t* xe_scales, const int32_t* offsets, const void* w1, const void* w3, const void* w2,
                   const moe_mx_scales_t* w_scales, void* ye, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(s, p);
  if (rc || (rc = check_ex(ex))) return rc;
  if (!offsets) return MOE_EINVAL;
  const void* bufs[] = {xe, w1, w3, w2, ye};
  for (const void* b : bufs)
    if (!aligned16(b)) return b ? MOE_EALIGN : MOE_EINVAL;
  if (s->dtype == MOE_MXFP8 && ((rc = check_scales(xe_scales)) || (rc = check_w_scales(w_scales)))) return rc;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  const WsLayout L = ws_layout(*s, p->E_local);
  if (s->dtype == MOE_MXFP8)
    return hip_rc(launch_ffn_mx(*s, p->E_local, static_cast<const uint8_t*>(xe), xe_scales, offsets,
                                static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w3),
                                static_cast<const uint8_t*>(w2), w_scales->w1, w_scales->w3, w_scales->w2, ye,
                                static_cast<char*>(ws), L, cu_count(), static_cast<hipStream_t>(stream), nullptr));
  return hip_rc(launch_ffn(*s, p->E_local, xe, offsets, w1, w3, w2, ye, static_cast<char*>(ws), L, cu_count(),
                           static_cast<hipStream_t>(stream), nullptr, nullptr));
}

int moe_expert_ffn_push(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                        const void* const* x, const void* xe, const uint8_t* xe_scales, const int32_t* offsets,
                        const void* w1, const void* w3, const void* w2, const moe_mx_scales_t* w_scales,
                        const int32_t* pull_src, const int32_t* slot_of, void* const* recv, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc = check_shape(s, p);
  if (rc || (rc = check_ex(ex))) return rc;
  if (!offsets || !pull_src || !slot_of) return MOE_EINVAL;
  if (x && s->dtype == MOE_MXFP8) return MOE_EUNSUP;      // MXFP8 rows are quantised by the gather
  const void* bufs[] = {x ? w1 : xe, w1, w3, w2};
  for (const void* b : bufs)
    if (!aligned16(b)) return b ? MOE_EALIGN : MOE_EINVAL;
  if (x && (rc = check_ptr_table(x, s->R))) return rc;
  if (s->dtype == MOE_MXFP8 && ((rc = check_scales(xe_scales)) || (rc = check_w_scales(w_scales)))) return rc;
  if ((rc = check_ptr_table(recv, s->R))) return rc;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  const WsLayout L = ws_layout(*s, p->E_local);
  char* w = static_cast<char*>(ws);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint64_t* dst = reinterpret_cast<uint64_t*>(w + L.push_dst);
  uint64_t* src = x ? reinterpret_cast<uint64_t*>(w + L.pull_addr) : nullptr;
  const hipError_t e = launch_pair_addr(*s, pull_src, slot_of, recv, x, reinterpret_cast<const int32_t*>(w + L.ctrl),
                                        dst, src, cu_count(), st, nullptr, nullptr);
  if (e != hipSuccess) return MOE_EHIP;
  if (s->dtype == MOE_MXFP8)
    return hip_rc(launch_ffn_mx(*s, p->E_local, static_cast<const uint8_t*>(xe), xe_scales, offsets,
                                static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w3),
                                static_cast<const uint8_t*>(w2), w_scales->w1, w_scales->w3, w_scales->w2, nullptr,
                                w, L, cu_count(), st, dst));
  return hip_rc(launch_ffn(*s, p->E_local, x ? nullptr : xe, offsets, w1, w3, w2, nullptr, w, L, cu_count(), st, dst,
                           src));
}

int moe_weighted_merge(const moe_shape_t* s, const moe_placement_t* p, const int32_t* slot_of, const float* topk_w,
                       void* const* recv, void* const* y, void* stream) {
  int rc = check_shape(s, p);
  if (rc) return rc;
  if (!slot_of || !topk_w) return MOE_EINVAL;
  if ((rc = check_ptr_table(recv, s->R)) || (rc = check_ptr_table(y, s->R))) return rc;
  return hip_rc(launch_merge(*s, slot_of, topk_w, recv, y, cu_count(), static_cast<hipStream_t>(stream)));
}

int moe_combine_push(const moe_shape_t* s, const moe_placement_t* p, const void* ye, const int32_t* pull_src,
                     const int32_t* slot_of, const float* topk_w, const int32_t* offsets, void* const* recv,
                     void* const* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(s, p);
  if (rc) return rc;
  if (!pull_src || !slot_of || !topk_w || !offsets) return MOE_EINVAL;
  if (!aligned16(ye)) return ye ? MOE_EALIGN : MOE_EINVAL;
  if ((rc = check_ptr_table(recv, s->R))) return rc;
  if ((rc = check_ptr_table(y, s->R))) return rc;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  const WsLayout L = ws_layout(*s, p->E_local);
  return hip_rc(launch_combine(*s, static_cast<const char*>(ye), pull_src, slot_of, topk_w, recv, y,
                               reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + L.ctrl), cu_count(),
                               static_cast<hipStream_t>(stream)));
}

int moe_forward(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex, const float* const* logits,
                const void* const* x, const void* w1, const void* w3, const void* w2, const moe_mx_scales_t* w_scales,
                void* xe, uint8_t* xe_scales, void* ye, void* const* recv, void* const* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                int32_t* offsets, int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes,
                void* stream) {
  int rc = check_shape(s, p);
  if (rc || (rc = check_ex(ex))) return rc;
  // validate every stage's arguments before launching any of them
  if (!p->expert_to_local || !topk_idx || !topk_w || !counts || !offsets || !pull_src || !slot_of)
    return MOE_EINVAL;
  const void* bufs[] = {xe, ye, w1, w3, w2};
  for (const void* b : bufs)
    if (!aligned16(b)) return b ? MOE_EALIGN : MOE_EINVAL;
  if (s->dtype == MOE_MXFP8 && ((rc = check_scales(xe_scales)) || (rc = check_w_scales(w_scales)))) return rc;
  if ((rc = check_ptr_table(logits, s->R)) || (rc = check_ptr_table(x, s->R)) ||
      (rc = check_ptr_table(recv, s->R)) || (rc = check_ptr_table(y, s->R)))
    return rc;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  if ((rc = moe_layout(s, p, ex, logits, topk_idx, topk_w, counts, offsets, pull_src, slot_of, ws, ws_bytes,
                       stream)))
    return rc;
  if ((rc = moe_dispatch_pull(s, p, x, pull_src, offsets, xe, xe_scales, ws, ws_bytes, stream))) return rc;
  if ((rc = moe_expert_ffn(s, p, ex, xe, xe_scales, offsets, w1, w3, w2, w_scales, ye, ws, ws_bytes, stream)))
    return rc;
  return moe_combine_push(s, p, ye, pull_src, slot_of, topk_w, offsets, recv, y, ws, ws_bytes, stream);
}

int moe_forward_fused(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                      const float* const* logits, const void* const* x, const void* w1, const void* w3,
                      const void* w2, const moe_mx_scales_t* w_scales, void* xe, uint8_t* xe_scales,
                      void* const* recv, void* const* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                      int32_t* offsets, int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_shape(s, p);
  if (rc || (rc = check_ex(ex))) return rc;
  // validate every stage's arguments before launching any of them
  if (!p->expert_to_local || !topk_idx || !topk_w || !counts || !offsets || !pull_src || !slot_of)
    return MOE_EINVAL;
  const bool mx = s->dtype == MOE_MXFP8;      // only MXFP8 stages its rows (the gather quantises them)
  const void* bufs[] = {mx ? xe : w1, w1, w3, w2};
  for (const void* b : bufs)
    if (!aligned16(b)) return b ? MOE_EALIGN : MOE_EINVAL;
  if (mx && ((rc = check_scales(xe_scales)) || (rc = check_w_scales(w_scales)))) return rc;
  if ((rc = check_ptr_table(logits, s->R)) || (rc = check_ptr_table(x, s->R)) ||
      (rc = check_ptr_table(recv, s->R)) || (rc = check_ptr_table(y, s->R)))
    return rc;
  if ((rc = check_ws(s, p, ws, ws_bytes))) return rc;
  if ((rc = moe_layout(s, p, ex, logits, topk_idx, topk_w, counts, offsets, pull_src, slot_of, ws, ws_bytes,
                       stream)))
    return rc;
  if (mx && (rc = moe_dispatch_pull(s, p, x, pull_src, offsets, xe, xe_scales, ws, ws_bytes, stream))) return rc;
  if ((rc = moe_expert_ffn_push(s, p, ex, mx ? nullptr : x, xe, xe_scales, offsets, w1, w3, w2, w_scales, pull_src,
                                slot_of, recv, ws, ws_bytes, stream)))
    return rc;
  return moe_weighted_merge(s, p, slot_of, topk_w, recv, y, stream);
}

size_t moe_ring_slot_bytes(const moe_shape_t* s, const moe_exec_t* ex) {
  if (!s || (s->dtype != MOE_BF16 && s->dtype != MOE_MXFP8) || s->d < 1 || s->F < 1) return 0;
  if (s->dtype == MOE_MXFP8 && (s->d % 128 || s->F % 128)) return 0;
  const int b = chunk_log2_of(ex);
  return b < 0 ? 0 : ring_slot_bytes(*s, b);
}

namespace {
// trace region of the persistent workspace: an int32 count, then events from +256
int trace_capacity(const moe_shape_t& s, const WsLayout& L, const moe_exec_t* ex) {
  const int b = chunk_log2_of(ex);
  const int cpm = b < 0 ? 1 : (kGemmBM >> b);
  const int NT1 = (s.F + kGemmBN / 2 - 1) / (kGemmBN / 2), NT2 = (s.d + kGemmBN - 1) / kGemmBN;
  const int64_t cap = int64_t(L.max_mtiles) * (cpm + 1 + NT1 + NT2) + 2 * 4096;
  return cap > (int64_t(1) << 30) ? (1 << 30) : int(cap);
}
size_t trace_bytes(const moe_shape_t& s, const WsLayout& L, const moe_exec_t* ex) {
  return align256(256 + size_t(trace_capacity(s, L, ex)) * sizeof(moe_trace_event_t));
}
// reverse ring and MXFP8: the per-pair recv address table of the down GEMM's stores, at L.hbuf
size_t reverse_table_bytes(const moe_shape_t& s, const WsLayout& L, const moe_exec_t* ex) {
  return ((ex && ex->reverse_ring == 1) || s.dtype == MOE_MXFP8) ? align256(size_t(L.max_pairs) * 8) : 0;
}
}  // namespace

size_t moe_persistent_workspace_bytes(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex) {
  if (check_shape(s, p) != MOE_OK) return 0;
  const WsLayout L = ws_layout(*s, p->E_local);
  return L.hbuf + reverse_table_bytes(*s, L, ex) + ((ex && ex->trace) ? trace_bytes(*s, L, ex) : 0);   // no h staging
}

int moe_persistent_trace_info(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex, size_t* offset,
                              int32_t* capacity, int32_t* ticks_per_us) {
  if (check_shape(s, p) != MOE_OK || !ex || ex->trace != 1 || !offset || !capacity || !ticks_per_us)
    return MOE_EINVAL;
  const WsLayout L = ws_layout(*s, p->E_local);
  *offset = L.hbuf + reverse_table_bytes(*s, L, ex);
  *capacity = trace_capacity(*s, L, ex);
  *ticks_per_us = static_cast<int32_t>(wall_ticks_per_us());
  return MOE_OK;
}

int moe_persistent_resident_info(const moe_shape_t* s, const moe_placement_t* p, size_t* offset, int32_t* entries) {
  if (check_shape(s, p) != MOE_OK || !offset || !entries) return MOE_EINVAL;
  const WsLayout L = ws_layout(*s, p->E_local);
  *offset = L.pctrl + size_t(sched::ctrl_layout(L.max_mtiles, kMaxRingSlots).resident) * 4;
  *entries = L.max_mtiles * 4;
  return MOE_OK;
}

namespace {
// Checks shared by the persistent entry points and the launch plan they derive; every
// check runs before the first HIP call.
struct PersistSetup {
  WsLayout L;
  sched::Plan plan;
  long long slot_bytes, budget;
  int blk_log2, cus;
  bool tracing, reverse;
  size_t rev_bytes;      // reverse ring and MXFP8: the recv address table at L.hbuf
  const moe_mx_scales_t* w_scales;   // MXFP8: the weights' scales; null in bf16
};

int persist_setup(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex, const void* const* x,
                  const void* w1, const void* w3, const void* w2, const moe_mx_scales_t* w_scales,
                  const void* ring, size_t ring_bytes, void* const* recv, const void* ws, size_t ws_bytes,
                  PersistSetup* out) {
  int rc = check_shape(s, p);
  if (rc) return rc;
  if (s->dtype != MOE_BF16 && s->dtype != MOE_MXFP8) return MOE_EUNSUP;
  if (s->dtype == MOE_MXFP8 && (rc = check_w_scales(w_scales))) return rc;
  out->w_scales = s->dtype == MOE_MXFP8 ? w_scales : nullptr;
  const void* bufs[] = {w1, w3, w2};
  for (const void* b : bufs)
    if (!aligned16(b)) return b ? MOE_EALIGN : MOE_EINVAL;
  if (!ring) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(ring) & 255) return MOE_EALIGN;
  if ((rc = check_ptr_table(x, s->R)) || (rc = check_ptr_table(recv, s->R))) return rc;
  if (ex && (ex->minibatch_rows < 0 || ex->comm_cus < 0 || ex->ring_slots < 0 || ex->trace < 0 || ex->trace > 1 ||
             ex->reverse_ring < 0 || ex->reverse_ring > 1))
    return MOE_EINVAL;
  out->blk_log2 = chunk_log2_of(ex);
  if (out->blk_log2 < 0) return MOE_EUNSUP;
  out->L = ws_layout(*s, p->E_local);
  if (!ws) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return MOE_EALIGN;
  out->tracing = ex && ex->trace == 1;
  out->reverse = ex && ex->reverse_ring == 1;
  out->rev_bytes = reverse_table_bytes(*s, out->L, ex);
  if (ws_bytes < out->L.hbuf + out->rev_bytes + (out->tracing ? trace_bytes(*s, out->L, ex) : 0)) return MOE_ENOSPC;
  const int cpm = kGemmBM >> out->blk_log2;
  out->slot_bytes = static_cast<long long>(ring_slot_bytes(*s, out->blk_log2));
  long long slots = static_cast<long long>(ring_bytes / size_t(out->slot_bytes));
  if (ex && ex->ring_slots > 0 && ex->ring_slots < slots) slots = ex->ring_slots;
  if (slots > kMaxRingSlots) slots = kMaxRingSlots;
  if (slots < cpm) return MOE_ENOSPC;                     // one row tile must fit
  out->cus = cu_count();
  const int comm_req = (ex && ex->comm_cus > 0) ? ex->comm_cus : 16;
  // eight pipelines (one per XCD) only on the whole chip: 256 CUs in eight XCDs, workgroup w
  // on XCD w mod 8
  out->plan = sched::plan_persistent(out->cus, out->cus == 256, slots, cpm, comm_req);
  if (!out->plan.ok) return MOE_EINVAL;                   // no CU left for the expert GEMMs
  const long long us = (ex && ex->watchdog_us > 0) ? static_cast<long long>(ex->watchdog_us) : 2000000LL;
  out->budget = us * wall_ticks_per_us();
  return MOE_OK;
}

int persist_launch(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex, const PersistSetup& P,
                   const void* const* x, const void* w1, const void* w3, const void* w2, void* ring,
                   const int32_t* pull_src, const int32_t* slot_of, const int32_t* offsets, void* const* recv,
                   void* ws, hipStream_t st) {
  char* wsc = static_cast<char*>(ws);
  const size_t toff = P.L.hbuf + P.rev_bytes;
  moe_trace_event_t* trace = P.tracing ? reinterpret_cast<moe_trace_event_t*>(wsc + toff + 256) : nullptr;
  int32_t* trace_count = P.tracing ? reinterpret_cast<int32_t*>(wsc + toff) : nullptr;
  uint64_t* row_dst = nullptr;
  if (P.reverse || P.w_scales) {      // the recv address of every local pair, for the down GEMM's stores
    row_dst = reinterpret_cast<uint64_t*>(wsc + P.L.hbuf);
    const hipError_t e = launch_pair_addr(*s, pull_src, slot_of, recv, nullptr,
                                          reinterpret_cast<const int32_t*>(wsc + P.L.ctrl), row_dst, nullptr,
                                          P.cus, st, nullptr, nullptr);
    if (e != hipSuccess) return MOE_EHIP;
  }
  return hip_rc(launch_persistent(*s, p->E_local, x, w1, w3, w2, pull_src, slot_of, offsets, static_cast<char*>(ring),
                                  P.slot_bytes, P.blk_log2, P.plan, P.cus, P.budget, recv, wsc, P.L, trace,
                                  trace_count, P.tracing ? trace_capacity(*s, P.L, ex) : 0, row_dst, P.reverse,
                                  P.w_scales, st));
}

int persist_occupancy_ok(bool mx) {
  int occ = 0;
  if (persistent_occupancy(&occ, mx) != hipSuccess) return MOE_EHIP;
  return occ < 1 ? MOE_EUNSUP : MOE_OK;                   // one workgroup per CU must fit
}
}  // namespace

int moe_persistent_dispatch_ffn_combine(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                                        const void* const* x, const void* w1, const void* w3, const void* w2,
                                        const moe_mx_scales_t* w_scales, void* ring, size_t ring_bytes,
                                        const int32_t* pull_src, const int32_t* slot_of, const int32_t* offsets,
                                        void* const* recv, void* ws, size_t ws_bytes, void* stream) {
  PersistSetup P;
  int rc = persist_setup(s, p, ex, x, w1, w3, w2, w_scales, ring, ring_bytes, recv, ws, ws_bytes, &P);
  if (rc) return rc;
  if (!pull_src || !slot_of || !offsets) return MOE_EINVAL;
  if ((rc = persist_occupancy_ok(P.w_scales != nullptr))) return rc;
  return persist_launch(s, p, ex, P, x, w1, w3, w2, ring, pull_src, slot_of, offsets, recv, ws,
                        static_cast<hipStream_t>(stream));
}

int moe_forward_persistent(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                           const float* const* logits, const void* const* x, const void* w1, const void* w3,
                           const void* w2, const moe_mx_scales_t* w_scales, void* ring, size_t ring_bytes,
                           void* const* recv, void* const* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes,
                           void* stream) {
  PersistSetup P;
  int rc = persist_setup(s, p, ex, x, w1, w3, w2, w_scales, ring, ring_bytes, recv, ws, ws_bytes, &P);
  if (rc) return rc;
  if (!p->expert_to_local || !topk_idx || !topk_w || !counts || !offsets || !pull_src || !slot_of)
    return MOE_EINVAL;
  if ((rc = check_ptr_table(logits, s->R)) || (rc = check_ptr_table(y, s->R))) return rc;
  if ((rc = persist_occupancy_ok(P.w_scales != nullptr))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_layout(*s, p->expert_to_local, p->E_local, minibatch_of(ex), logits, topk_idx, topk_w, counts,
                               offsets, pull_src, slot_of, static_cast<char*>(ws), P.L, st);
  if (e != hipSuccess) return MOE_EHIP;
  if ((rc = persist_launch(s, p, ex, P, x, w1, w3, w2, ring, pull_src, slot_of, offsets, recv, ws, st))) return rc;
  return hip_rc(launch_merge(*s, slot_of, topk_w, recv, y, cu_count(), st));
}

size_t moe_backward_workspace_bytes(const moe_shape_t* s, const moe_placement_t* p) {
  if (check_shape(s, p) != MOE_OK || (s->dtype != MOE_BF16 && s->dtype != MOE_MXFP8)) return 0;
  return bwd_layout(*s, p->E_local).total;
}

int moe_backward_prepare_mx(const moe_shape_t* s, const moe_placement_t* p, const void* w1, const void* w3,
                            const void* w2, uint8_t* w2t, uint8_t* w2t_scales, uint8_t* w13t, uint8_t* w13t_scales,
                            void* stream) {
  int rc = check_shape(s, p);
  if (rc) return rc;
  if (s->dtype != MOE_MXFP8) return MOE_EUNSUP;
  const void* bufs[] = {w1, w3, w2, w2t, w13t};
  for (const void* q : bufs)
    if (!aligned16(q)) return q ? MOE_EALIGN : MOE_EINVAL;
  if ((rc = check_scales(w2t_scales)) || (rc = check_scales(w13t_scales))) return rc;
  const int El = p->E_local, d = s->d, F = s->F, cus = cu_count();
  hipStream_t st = static_cast<hipStream_t>(stream);
  // W2 along d -> [E_local][F][d] codes; W1 and W3 along F -> [E_local][d][2F] codes
  hipError_t e = launch_mx_quantize_t(static_cast<const uint16_t*>(w2), d, F, El, w2t, d, 0, w2t_scales,
                                      int64_t(El) * F, cus, st);
  if (e == hipSuccess)
    e = launch_mx_quantize_t(static_cast<const uint16_t*>(w1), F, d, El, w13t, 2 * F, 0, w13t_scales, int64_t(El) * d,
                             cus, st);
  if (e == hipSuccess)
    e = launch_mx_quantize_t(static_cast<const uint16_t*>(w3), F, d, El, w13t, 2 * F, F, w13t_scales, int64_t(El) * d,
                             cus, st);
  return hip_rc(e);
}

int moe_backward_mx(const moe_shape_t* s, const moe_placement_t* p, const void* const* dy, const void* const* x,
                    const uint8_t* xe, const uint8_t* xe_scales, const void* ye, const uint8_t* w1q, const uint8_t* w3q,
                    const moe_mx_scales_t* w_scales, const uint8_t* w2t, const uint8_t* w2t_scales, const uint8_t* w13t,
                    const uint8_t* w13t_scales, const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                    const int32_t* pull_src, const int32_t* slot_of, const void* ws, size_t ws_bytes,
                    void* const* recv, void* const* dx, float* const* dlogits, void* dw1, void* dw3, void* dw2,
                    void* bws, size_t bws_bytes, void* stream) {
  int rc = check_bwd(s, p, ws, ws_bytes, bws, bws_bytes, MOE_MXFP8);
  if (rc) return rc;
  if (!topk_idx || !topk_w || !offsets || !pull_src || !slot_of) return MOE_EINVAL;
  const void* bufs[] = {xe, ye, w1q, w3q, w2t, w13t, dw1, dw3, dw2};
  for (const void* q : bufs)
    if (!aligned16(q)) return q ? MOE_EALIGN : MOE_EINVAL;
  if ((rc = check_scales(xe_scales)) || (rc = check_w_scales(w_scales)) || (rc = check_scales(w2t_scales)) ||
      (rc = check_scales(w13t_scales)))
    return rc;
  if ((rc = check_ptr_table(dy, s->R)) || (rc = check_ptr_table(x, s->R)) || (rc = check_ptr_table(recv, s->R)) ||
      (rc = check_ptr_table(dx, s->R)))
    return rc;
  if (!dlogits) return MOE_EINVAL;
  for (int r = 0; r < s->R; ++r)
    if (!dlogits[r]) return MOE_EINVAL;

  const WsLayout L = ws_layout(*s, p->E_local);
  const BwdLayout B = bwd_layout(*s, p->E_local);
  const char* w = static_cast<const char*>(ws);
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(w + L.ctrl);
  const int32_t* mtb = reinterpret_cast<const int32_t*>(w + L.mtile_base);
  char* b = static_cast<char*>(bws);
  uint16_t* dO = reinterpret_cast<uint16_t*>(b + B.dO);
  float* dg = reinterpret_cast<float*>(b + B.dg);
  uint16_t* dh = reinterpret_cast<uint16_t*>(b + B.dh);
  uint16_t* h = reinterpret_cast<uint16_t*>(b + B.h);
  uint16_t* dab = reinterpret_cast<uint16_t*>(b + B.dab);
  uint16_t* dX = reinterpret_cast<uint16_t*>(b + B.dX);
  float* dgp = reinterpret_cast<float*>(b + B.dgp);
  uint8_t* dOq = reinterpret_cast<uint8_t*>(b + B.dOq);
  uint8_t* dOs = reinterpret_cast<uint8_t*>(b + B.dOs);
  uint8_t* dabq = reinterpret_cast<uint8_t*>(b + B.dabq);
  uint8_t* dabs = reinterpret_cast<uint8_t*>(b + B.dabs);
  uint16_t* xeb = reinterpret_cast<uint16_t*>(b + B.xeb);
  const int El = p->E_local, d = s->d, F = s->F, cus = cu_count();
  const int64_t nmax = L.max_pairs;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // pull reverse-combine (dO bf16 and MX codes along d, dg)
  hipError_t e = launch_pull_reverse_mx(*s, dy, static_cast<const uint16_t*>(ye), pull_src, slot_of, topk_w, ctrl, dO,
                                        dOq, dOs, dg, nmax, cus, st);
  // MX data-gradient GEMMs: dh = dO W2; GEMM1 again with the backward epilogue; dX = [da|db] [W1; W3]
  if (e == hipSuccess)
    e = launch_rows_mx(dOq, dOs, w2t, w2t_scales, dh, d, F, nmax, offsets, mtb, ctrl, El, cus, st, nullptr);
  if (e == hipSuccess)
    e = launch_gemm1_bwd_mx(xe, xe_scales, w1q, w3q, w_scales->w1, w_scales->w3, dh, h, dab, dabq, dabs, d, F, nmax,
                            offsets, mtb, ctrl, El, cus, st);
  // the push of dX fused into its GEMM: each dX row goes straight to recv[r][t][j] (the per-pair
  // address table lives in the dX staging region, which the fused GEMM leaves unused), and the
  // table kernel pushes the gate gradients dg to dgp
  uint64_t* dx_dst = reinterpret_cast<uint64_t*>(dX);
  if (e == hipSuccess)
    e = launch_pair_addr(*s, pull_src, slot_of, recv, nullptr, ctrl, dx_dst, nullptr, cus, st, dg, dgp);
  if (e == hipSuccess)
    e = launch_rows_mx(dabq, dabs, w13t, w13t_scales, nullptr, 2 * F, d, nmax, offsets, mtb, ctrl, El, cus, st, dx_dst);
  // bf16 weight gradients over each expert's rows (the token rows gathered again in bf16)
  if (e == hipSuccess) e = launch_dispatch(*s, x, pull_src, reinterpret_cast<char*>(xeb), ctrl, cus, st);
  if (e == hipSuccess) e = launch_wgrad(dab, 2 * F, xeb, d, offsets, static_cast<uint16_t*>(dw1), El, F, d, cus, st);
  if (e == hipSuccess)
    e = launch_wgrad(dab + F, 2 * F, xeb, d, offsets, static_cast<uint16_t*>(dw3), El, F, d, cus, st);
  if (e == hipSuccess) e = launch_wgrad(dO, d, h, F, offsets, static_cast<uint16_t*>(dw2), El, d, F, cus, st);
  // ordered sum of the pushed dX rows, gate gradients
  if (e == hipSuccess) e = launch_merge(*s, slot_of, nullptr, recv, dx, cus, st);
  if (e == hipSuccess) e = launch_gate_grad(*s, topk_w, topk_idx, slot_of, dgp, dlogits, cus, st);
  return hip_rc(e);
}

int moe_combine_pull_reverse(const moe_shape_t* s, const moe_placement_t* p, const void* const* dy, const void* ye,
                             const int32_t* pull_src, const int32_t* slot_of, const float* topk_w, const void* ws,
                             size_t ws_bytes, void* bws, size_t bws_bytes, void* stream) {
  int rc = check_bwd(s, p, ws, ws_bytes, bws, bws_bytes);
  if (rc) return rc;
  if (!pull_src || !slot_of || !topk_w) return MOE_EINVAL;
  if (!aligned16(ye)) return ye ? MOE_EALIGN : MOE_EINVAL;
  if ((rc = check_ptr_table(dy, s->R))) return rc;
  const WsLayout L = ws_layout(*s, p->E_local);
  const BwdLayout B = bwd_layout(*s, p->E_local);
  char* b = static_cast<char*>(bws);
  return hip_rc(launch_pull_reverse(*s, dy, static_cast<const uint16_t*>(ye), pull_src, slot_of, topk_w,
                                    reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + L.ctrl),
                                    reinterpret_cast<uint16_t*>(b + B.dO), reinterpret_cast<float*>(b + B.dg),
                                    cu_count(), static_cast<hipStream_t>(stream)));
}

// recv == null: dX rows to the backward workspace (the staged API); else the push of dX fused
// into its GEMM (rows straight to recv, the gate gradients pushed to dgp by the table kernel)
// row_src / blk_src (both or neither): the token rows by address (per row, and per 64-row
// block of each row tile) instead of from xe
static int ffn_backward_impl(const moe_shape_t* s, const moe_placement_t* p, const void* xe, const int32_t* offsets,
                             const void* w1, const void* w3, const void* w2, const void* ws, void* dw1, void* dw3,
                             void* dw2, void* bws, const int32_t* pull_src, const int32_t* slot_of, void* const* recv,
                             void* stream, const uint64_t* row_src = nullptr, const uint64_t* blk_src = nullptr) {
  const WsLayout L = ws_layout(*s, p->E_local);
  const BwdLayout B = bwd_layout(*s, p->E_local);
  const char* w = static_cast<const char*>(ws);
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(w + L.ctrl);
  const int32_t* mtb = reinterpret_cast<const int32_t*>(w + L.mtile_base);
  char* b = static_cast<char*>(bws);
  uint16_t* dO = reinterpret_cast<uint16_t*>(b + B.dO);
  uint16_t* dh = reinterpret_cast<uint16_t*>(b + B.dh);
  uint16_t* h = reinterpret_cast<uint16_t*>(b + B.h);
  uint16_t* dab = reinterpret_cast<uint16_t*>(b + B.dab);
  uint16_t* dX = reinterpret_cast<uint16_t*>(b + B.dX);
  const uint16_t* xeb = static_cast<const uint16_t*>(xe);
  const uint16_t* w1b = static_cast<const uint16_t*>(w1);
  const uint16_t* w3b = static_cast<const uint16_t*>(w3);
  const uint16_t* w2b = static_cast<const uint16_t*>(w2);
  const int El = p->E_local, d = s->d, F = s->F, cus = cu_count();
  hipStream_t st = static_cast<hipStream_t>(stream);
  // dh = dO W2; then h, da, db in GEMM1's backward epilogue; dX = [da|db] [W1; W3]
  hipError_t e = launch_rows_bmn(dO, w2b, nullptr, d, dh, d, F, offsets, mtb, ctrl, El, cus, st, nullptr);
  if (e == hipSuccess) e = launch_gemm1_bwd(xeb, w1b, w3b, dh, h, dab, d, F, offsets, mtb, ctrl, El, cus, st, row_src);
  uint64_t* dx_dst = nullptr;
  if (recv) {             // the address table lives in the dX staging region, unused when fused
    dx_dst = reinterpret_cast<uint64_t*>(dX);
    if (e == hipSuccess)
      e = launch_pair_addr(*s, pull_src, slot_of, recv, nullptr, ctrl, dx_dst, nullptr, cus, st,
                           reinterpret_cast<const float*>(b + B.dg), reinterpret_cast<float*>(b + B.dgp));
  }
  if (e == hipSuccess)
    e = launch_rows_bmn(dab, w1b, w3b, F, recv ? nullptr : dX, 2 * F, d, offsets, mtb, ctrl, El, cus, st, dx_dst);
  // weight gradients over each expert's rows: dW1 = da^T x, dW3 = db^T x, dW2 = dO^T h
  if (e == hipSuccess)
    e = launch_wgrad(dab, 2 * F, xeb, d, offsets, static_cast<uint16_t*>(dw1), El, F, d, cus, st, blk_src, mtb);
  if (e == hipSuccess)
    e = launch_wgrad(dab + F, 2 * F, xeb, d, offsets, static_cast<uint16_t*>(dw3), El, F, d, cus, st, blk_src, mtb);
  if (e == hipSuccess) e = launch_wgrad(dO, d, h, F, offsets, static_cast<uint16_t*>(dw2), El, d, F, cus, st);
  return hip_rc(e);
}

int moe_expert_ffn_backward(const moe_shape_t* s, const moe_placement_t* p, const void* xe, const int32_t* offsets,
                            const void* w1, const void* w3, const void* w2, const void* ws, size_t ws_bytes, void* dw1,
                            void* dw3, void* dw2, void* bws, size_t bws_bytes, void* stream) {
  int rc = check_bwd(s, p, ws, ws_bytes, bws, bws_bytes);
  if (rc) return rc;
  if (!offsets) return MOE_EINVAL;
  const void* bufs[] = {xe, w1, w3, w2, dw1, dw3, dw2};
  for (const void* q : bufs)
    if (!aligned16(q)) return q ? MOE_EALIGN : MOE_EINVAL;
  return ffn_backward_impl(s, p, xe, offsets, w1, w3, w2, ws, dw1, dw3, dw2, bws, nullptr, nullptr, nullptr, stream);
}

int moe_dispatch_push_reverse(const moe_shape_t* s, const moe_placement_t* p, const int32_t* pull_src,
                              const int32_t* slot_of, const int32_t* topk_idx, const float* topk_w, const void* ws,
                              size_t ws_bytes, void* const* recv, void* const* dx, float* const* dlogits, void* bws,
                              size_t bws_bytes, void* stream) {
  int rc = check_bwd(s, p, ws, ws_bytes, bws, bws_bytes);
  if (rc) return rc;
  if (!pull_src || !slot_of || !topk_idx || !topk_w) return MOE_EINVAL;
  if ((rc = check_ptr_table(recv, s->R)) || (rc = check_ptr_table(dx, s->R))) return rc;
  if (!dlogits) return MOE_EINVAL;
  for (int r = 0; r < s->R; ++r)
    if (!dlogits[r]) return MOE_EINVAL;
  const WsLayout L = ws_layout(*s, p->E_local);
  const BwdLayout B = bwd_layout(*s, p->E_local);
  char* b = static_cast<char*>(bws);
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + L.ctrl);
  float* dgp = reinterpret_cast<float*>(b + B.dgp);
  const int cus = cu_count();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_push_grad(*s, b + B.dX, reinterpret_cast<const float*>(b + B.dg), pull_src, slot_of, recv,
                                  dgp, ctrl, cus, st);
  if (e == hipSuccess) e = launch_merge(*s, slot_of, nullptr, recv, dx, cus, st);
  if (e == hipSuccess) e = launch_gate_grad(*s, topk_w, topk_idx, slot_of, dgp, dlogits, cus, st);
  return hip_rc(e);
}

int moe_backward(const moe_shape_t* s, const moe_placement_t* p, const void* const* dy, const void* xe, const void* ye,
                 const void* w1, const void* w3, const void* w2, const int32_t* topk_idx,
                 const float* topk_w, const int32_t* offsets, const int32_t* pull_src, const int32_t* slot_of,
                 const void* ws, size_t ws_bytes, void* const* recv, void* const* dx, float* const* dlogits, void* dw1,
                 void* dw3, void* dw2, void* bws, size_t bws_bytes, void* stream) {
  int rc = check_bwd(s, p, ws, ws_bytes, bws, bws_bytes);
  if (rc) return rc;
  // validate every stage's arguments before launching any of them
  if (!topk_idx || !topk_w || !offsets || !pull_src || !slot_of) return MOE_EINVAL;
  const void* bufs[] = {xe, ye, w1, w3, w2, dw1, dw3, dw2};
  for (const void* q : bufs)
    if (!aligned16(q)) return q ? MOE_EALIGN : MOE_EINVAL;
  if ((rc = check_ptr_table(dy, s->R)) || (rc = check_ptr_table(recv, s->R)) || (rc = check_ptr_table(dx, s->R)))
    return rc;
  if (!dlogits) return MOE_EINVAL;
  for (int r = 0; r < s->R; ++r)
    if (!dlogits[r]) return MOE_EINVAL;
  if ((rc = moe_combine_pull_reverse(s, p, dy, ye, pull_src, slot_of, topk_w, ws, ws_bytes, bws, bws_bytes, stream)))
    return rc;
  // the expert backward with the push of dX fused into its GEMM, then the ordered sum and the
  // gate gradients (moe_dispatch_push_reverse without its push)
  if ((rc = ffn_backward_impl(s, p, xe, offsets, w1, w3, w2, ws, dw1, dw3, dw2, bws, pull_src, slot_of, recv, stream)))
    return rc;
  const BwdLayout B = bwd_layout(*s, p->E_local);
  float* dgp = reinterpret_cast<float*>(static_cast<char*>(bws) + B.dgp);
  const int cus = cu_count();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_merge(*s, slot_of, nullptr, recv, dx, cus, st);
  if (e == hipSuccess) e = launch_gate_grad(*s, topk_w, topk_idx, slot_of, dgp, dlogits, cus, st);
  return hip_rc(e);
}

int moe_backward_ring(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                      const void* const* dy, const void* const* x, const void* ring, size_t ring_bytes,
                      const void* pws, size_t pws_bytes, const void* w1, const void* w3, const void* w2,
                      const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                      const int32_t* pull_src, const int32_t* slot_of, void* const* recv, void* const* dx,
                      float* const* dlogits, void* dw1, void* dw3, void* dw2, void* xe, void* bws,
                      size_t bws_bytes, void* stream) {
  int rc = check_shape(s, p);
  if (rc) return rc;
  if (s->dtype != MOE_BF16) return MOE_EUNSUP;
  // the forward's workspace: its layout tables and control block (moe_persistent_workspace_bytes)
  const WsLayout L = ws_layout(*s, p->E_local);
  if (!pws) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(pws) & 255) return MOE_EALIGN;
  if (pws_bytes < L.hbuf) return MOE_ENOSPC;
  if (!bws) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(bws) & 255) return MOE_EALIGN;
  const BwdLayout B = bwd_layout(*s, p->E_local);
  if (bws_bytes < B.total) return MOE_ENOSPC;
  if (ex && (ex->minibatch_rows < 0 || ex->reverse_ring < 0 || ex->reverse_ring > 1)) return MOE_EINVAL;
  const int blk_log2 = chunk_log2_of(ex);
  if (blk_log2 < 0) return MOE_EUNSUP;
  if (!topk_idx || !topk_w || !offsets || !pull_src || !slot_of) return MOE_EINVAL;
  const void* bufs[] = {xe, w1, w3, w2, dw1, dw3, dw2};
  for (const void* q : bufs)
    if (!aligned16(q)) return q ? MOE_EALIGN : MOE_EINVAL;
  if (ring && (reinterpret_cast<uintptr_t>(ring) & 255)) return MOE_EALIGN;
  if ((rc = check_ptr_table(dy, s->R)) || (rc = check_ptr_table(x, s->R)) || (rc = check_ptr_table(recv, s->R)) ||
      (rc = check_ptr_table(dx, s->R)))
    return rc;
  if (!dlogits) return MOE_EINVAL;
  for (int r = 0; r < s->R; ++r)
    if (!dlogits[r]) return MOE_EINVAL;
  // ring slots the recorded chunks may name (a slot past the ring counts as not held)
  const long long slot_bytes = static_cast<long long>(ring_slot_bytes(*s, blk_log2));
  long long n_slots = ring ? static_cast<long long>(ring_bytes / size_t(slot_bytes)) : 0;
  if (n_slots > kMaxRingSlots) n_slots = kMaxRingSlots;

  const char* w = static_cast<const char*>(pws);
  const int32_t* ctrl = reinterpret_cast<const int32_t*>(w + L.ctrl);
  const int32_t* mtb = reinterpret_cast<const int32_t*>(w + L.mtile_base);
  const sched::CtrlLayout cl = sched::ctrl_layout(L.max_mtiles, kMaxRingSlots);
  const int32_t* resident = reinterpret_cast<const int32_t*>(w + L.pctrl) + cl.resident;
  char* b = static_cast<char*>(bws);
  uint64_t* row_src = reinterpret_cast<uint64_t*>(b + B.rows);
  uint64_t* blk_src = reinterpret_cast<uint64_t*>(b + B.blks);
  const int cus = cu_count();
  hipStream_t st = static_cast<hipStream_t>(stream);
  // pull reverse-combine with the expert outputs read from recv, then where every token row is
  hipError_t e = launch_pull_reverse(*s, dy, nullptr, pull_src, slot_of, topk_w, ctrl,
                                     reinterpret_cast<uint16_t*>(b + B.dO), reinterpret_cast<float*>(b + B.dg), cus, st,
                                     recv);
  if (e == hipSuccess)
    e = launch_ring_rows(*s, p->E_local, L.max_mtiles, x, pull_src, offsets, mtb, ctrl, resident, ring, slot_bytes,
                         int(n_slots), blk_log2, xe, blk_src, reinterpret_cast<int32_t*>(b + B.held), row_src, cus, st);
  if (e != hipSuccess) return MOE_EHIP;
  if ((rc = ffn_backward_impl(s, p, nullptr, offsets, w1, w3, w2, pws, dw1, dw3, dw2, bws, pull_src, slot_of, recv,
                              stream, row_src, blk_src)))
    return rc;
  float* dgp = reinterpret_cast<float*>(b + B.dgp);
  e = launch_merge(*s, slot_of, nullptr, recv, dx, cus, st);
  if (e == hipSuccess) e = launch_gate_grad(*s, topk_w, topk_idx, slot_of, dgp, dlogits, cus, st);
  return hip_rc(e);
}

int moe_read_status(const void* ws, void* stream) {
  if (!ws) return MOE_EINVAL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_EHIP;
  int32_t st = 0;
  if (hipMemcpy(&st, static_cast<const char*>(ws) + kCtrlStatus * 4, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_EHIP;
  return st;
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (shape, k, dtype, placement or null pointer)";
    case MOE_EALIGN: return "misaligned buffer or unsupported d/F multiple";
    case MOE_ENOSPC: return "workspace or ring too small";
    case MOE_EHIP: return "HIP launch failed";
    case MOE_ETIMEOUT: return "device wait exceeded its watchdog budget";
    case MOE_EUNSUP: return "combination not supported by this build";
    case MOE_EINCOMPLETE: return "persistent kernel ended with work left undone (a pipeline got no workgroup)";
    default: return "unknown error";
  }
}

const char* moe_version(void) { return "libmoe 0.3 gfx950"; }

}  // extern "C"
