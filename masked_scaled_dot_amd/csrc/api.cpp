// C ABI of the library: host-side argument checks, then dispatch to the gfx950 kernels.
// Every check here runs before any HIP call, so bad arguments return a status without
// touching the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/sa.h"
#include "kernels.h"
#include "plan_layout.h"

namespace {

enum Op { kOpSddmm, kOpSoftmax, kOpSpmm, kOpFused, kOpPlan, kOpValidate };

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int check_problem(const sa_problem* p, Op op) {
  if (!p) return SA_ERR_NULL;
  if (p->reserved != 0) return SA_ERR_UNSUPPORTED;
  if (p->flags & ~SA_FLAG_VALIDATE) return SA_ERR_UNSUPPORTED;
  if (p->dtype != SA_F32 && p->dtype != SA_BF16) return SA_ERR_DTYPE;
  if (p->B < 0 || p->H < 0 || p->n < 0 || p->d <= 0) return SA_ERR_SHAPE;
  if (p->d != 32 && p->d != 64 && p->d != 128) return SA_ERR_UNSUPPORTED;
  if (p->block != 1 && p->block != 64) return SA_ERR_UNSUPPORTED;
  if (!std::isfinite(p->scale)) return SA_ERR_SHAPE;
  const bool dense = p->row_ptr == nullptr;
  const bool element_csr = !dense && p->block == 1;
  switch (op) {
    case kOpSddmm:
    case kOpSoftmax:
    case kOpSpmm:
    case kOpPlan:
      if (!element_csr) return SA_ERR_UNSUPPORTED;
      break;
    case kOpValidate:
      if (dense) return SA_ERR_NULL;
      break;
    case kOpFused:
      break;
  }
  if (!dense) {
    if (p->nnz < 0 || p->nnz > INT32_MAX) return SA_ERR_SHAPE;
    if (p->nnz > 0 && !p->col_idx) return SA_ERR_NULL;
    if (p->block == 64 && p->n > 0) {
      const long long nb = (p->n + 63) / 64;
      if (p->nnz > nb * nb) return SA_ERR_SHAPE;
    } else if ((long long)p->nnz > (long long)p->n * (long long)p->n) {
      return SA_ERR_SHAPE;
    }
  }
  if (p->key_mask && p->key_mask_heads != 1 && p->key_mask_heads != p->H) return SA_ERR_SHAPE;
  if (p->plan && !aligned16(p->plan)) return SA_ERR_ALIGN;  // its records are read 16 bytes at a time
  // Buffer element counts must fit in 64-bit byte offsets used by the kernels.
  const long long bh = (long long)p->B * p->H;
  if (bh > INT32_MAX) return SA_ERR_SHAPE;
  if (bh * p->n > INT32_MAX) return SA_ERR_SHAPE;  // (head, row) units are indexed in 32 bits
  if (bh * (long long)p->n * p->d > (1ll << 40)) return SA_ERR_SHAPE;
  if (!dense && bh * (long long)p->nnz > (1ll << 40)) return SA_ERR_SHAPE;
  if (p->bias && (long long)p->H * p->n * (long long)p->n > (1ll << 40)) return SA_ERR_SHAPE;
  return SA_OK;
}

bool empty_problem(const sa_problem* p) { return p->B == 0 || p->H == 0 || p->n == 0; }

thread_local hipError_t g_last_hip_error = hipSuccess;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SA_OK;
  g_last_hip_error = e;
  return SA_ERR_HIP;
}

// An error left pending by unrelated HIP calls in this thread would otherwise be reported
// as a failure of the next launch; take it off before launching.
void clear_stale_error() { (void)hipGetLastError(); }

// Device validation of the pattern; synchronises the stream.
int validate_now(const sa_problem* p, hipStream_t s) {
  if (empty_problem(p) && p->n == 0) return SA_OK;
  int* flag = nullptr;
  clear_stale_error();
  if (hipMalloc(&flag, sizeof(int)) != hipSuccess) return SA_ERR_HIP;
  int host = 0;
  int st = SA_OK;
  if (hipMemsetAsync(flag, 0, sizeof(int), s) != hipSuccess ||
      sa::launch_validate(*p, flag, s) != hipSuccess ||
      hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    st = SA_ERR_HIP;
  } else if (host != 0) {
    st = SA_ERR_CSR;
  }
  (void)hipFree(flag);
  return st;
}

// With SA_FLAG_VALIDATE and a caller plan, check that the plan was built for this pattern.
int check_plan_now(const sa_problem* p, hipStream_t s) {
  int hdr[sa::kPlanHeaderWords];
  if (hipMemcpyAsync(hdr, p->plan, sizeof(hdr), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return SA_ERR_HIP;
  const long long nnz = (long long)(uint32_t)hdr[sa::kHNnzLo] | ((long long)hdr[sa::kHNnzHi] << 32);
  if (hdr[sa::kHMagic] != sa::kPlanMagic || hdr[sa::kHN] != p->n || nnz != p->nnz ||
      hdr[sa::kHValid] != 1)
    return SA_ERR_WORKSPACE;
  // the scratch of split rows is sized for (B*H, d)
  if ((long long)p->B * p->H > hdr[sa::kHBH] || p->d > hdr[sa::kHD]) return SA_ERR_WORKSPACE;
  return SA_OK;
}

int pre_launch(const sa_problem* p, hipStream_t s) {
  clear_stale_error();
  if (p->flags & SA_FLAG_VALIDATE) {
    if (p->row_ptr) {
      const int st = validate_now(p, s);
      if (st != SA_OK) return st;
    }
    if (p->plan) {
      const int st = check_plan_now(p, s);
      if (st != SA_OK) return st;
    }
  }
  return SA_OK;
}

}  // namespace

extern "C" {

size_t sa_plan_bytes_segments(const sa_problem* p, int64_t max_segments) {
  if (check_problem(p, kOpPlan) != SA_OK || max_segments < 0) return 0;
  const long long BH = (long long)p->B * p->H;
  // a long row has more than kLongRow entries, so at least this many segments
  const long long min_segs = (sa::kLongRow + 1 + sa::kSeg - 1) / sa::kSeg;
  const long long n = p->n, nnz = p->nnz;
  long long S = nnz / sa::kSeg + nnz / (sa::kLongRow + 1);  // segments cannot exceed this
  S = S < max_segments ? S : max_segments;
  long long L = nnz / (sa::kLongRow + 1);
  L = L < n ? L : n;
  L = L < S / min_segs ? L : S / min_segs;
  return sa::plan_bytes_for(n, L, S, BH, p->d);
}

size_t sa_plan_bytes(const sa_problem* p) { return sa_plan_bytes_segments(p, sa::kPlanMaxSegs); }

int sa_plan_build(const sa_problem* p, void* plan, size_t plan_bytes, hipStream_t stream) {
  int st = check_problem(p, kOpPlan);
  if (st != SA_OK) return st;
  if (!plan) return SA_ERR_NULL;
  if (!aligned16(plan)) return SA_ERR_ALIGN;
  if (plan_bytes < sa::plan_bytes_for(p->n, 0, 0, 0, p->d)) return SA_ERR_WORKSPACE;  // header, rows, tiles
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_plan(*p, plan, plan_bytes, stream));
}

int sa_sddmm(const sa_problem* p, const void* q, const void* k, float* scores, hipStream_t stream) {
  int st = check_problem(p, kOpSddmm);
  if (st != SA_OK) return st;
  if (empty_problem(p) || p->nnz == 0) return SA_OK;
  if (!q || !k || !scores) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(scores)) return SA_ERR_ALIGN;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_sddmm(*p, q, k, scores, stream));
}

int sa_sparse_softmax(const sa_problem* p, const float* scores, float* weights, hipStream_t stream) {
  int st = check_problem(p, kOpSoftmax);
  if (st != SA_OK) return st;
  if (empty_problem(p) || p->nnz == 0) return SA_OK;
  if (!scores || !weights) return SA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(weights)) return SA_ERR_ALIGN;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_softmax(*p, scores, weights, stream));
}

int sa_spmm(const sa_problem* p, const float* weights, const void* v, float* out, hipStream_t stream) {
  int st = check_problem(p, kOpSpmm);
  if (st != SA_OK) return st;
  if (empty_problem(p)) return SA_OK;
  if (!v || !out || (p->nnz > 0 && !weights)) return SA_ERR_NULL;
  if (!aligned16(v) || !aligned16(out) || (weights && !aligned16(weights))) return SA_ERR_ALIGN;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_spmm(*p, weights, v, out, stream));
}

int sa_fused_forward(const sa_problem* p, const void* q, const void* k, const void* v, float* out,
                     float* lse, hipStream_t stream) {
  int st = check_problem(p, kOpFused);
  if (st != SA_OK) return st;
  if (empty_problem(p)) return SA_OK;
  if (!q || !k || !v || !out) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SA_ERR_ALIGN;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  if (sa::fused_resident_supported(*p))
    return hip_status(sa::launch_fused_resident(*p, q, k, v, out, lse, stream));
  if (sa::fused_tile_supported(*p)) return hip_status(sa::launch_fused_tile(*p, q, k, v, out, lse, stream));
  return hip_status(sa::launch_fused_valu(*p, q, k, v, out, lse, stream));
}

int sa_fused_backward(const sa_problem* p, const void* q, const void* k, const void* v,
                      const float* out, const float* lse, const void* dout, const int32_t* t_row_ptr,
                      const int32_t* t_col_idx, float* dq, float* dk, float* dv, float* dscores,
                      float* workspace, hipStream_t stream) {
  int st = check_problem(p, kOpFused);
  if (st != SA_OK) return st;
  if (p->row_ptr && p->block != 64) return SA_ERR_UNSUPPORTED;  // dense or block CSR
  if (p->row_ptr && p->nnz > 0 && (!t_row_ptr || !t_col_idx)) return SA_ERR_NULL;
  if (p->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (dscores && (long long)p->B * p->H * (long long)p->n * p->n > (1ll << 40)) return SA_ERR_SHAPE;
  if (empty_problem(p)) return SA_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(out))
    return SA_ERR_ALIGN;
  if ((long long)p->n * p->d * 2 > 0x7ffffff0ll) return SA_ERR_SHAPE;  // raw buffer range of a head
  // the tiles address a bias head [n, n] through one raw buffer with 32-bit offsets
  if (p->bias && (long long)p->n * p->n * 4 > 0x7ffffff0ll) return SA_ERR_UNSUPPORTED;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_fused_backward(*p, q, k, v, out, lse, dout, dq, dk, dv, dscores,
                                              workspace, t_row_ptr, t_col_idx, stream));
}

int sa_fused_backward_noalloc(const sa_problem* p, const void* q, const void* k, const void* v,
                              const float* out, const float* lse, const void* dout,
                              const int32_t* t_row_ptr, const int32_t* t_col_idx, float* dq, float* dk,
                              float* dv, float* dscores, hipStream_t stream) {
  int st = check_problem(p, kOpFused);
  if (st != SA_OK) return st;
  // device validation allocates a result flag: not available here
  if (p->flags & SA_FLAG_VALIDATE) return SA_ERR_UNSUPPORTED;
  if ((long long)p->B * p->H * (long long)p->n * 4 > (long long)sa::kNoAllocScratchBytes)
    return SA_ERR_WORKSPACE;
  if (empty_problem(p)) return SA_OK;
  void* ws = nullptr;
  clear_stale_error();
  const hipError_t e = sa::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e);
  return sa_fused_backward(p, q, k, v, out, lse, dout, t_row_ptr, t_col_idx, dq, dk, dv, dscores,
                           static_cast<float*>(ws), stream);
}

size_t sa_transpose_workspace_bytes(const sa_problem* p) {
  if (check_problem(p, kOpSoftmax) != SA_OK) return 0;
  return sa::transpose_workspace_bytes(p->n, p->nnz);
}

int sa_csr_transpose(const sa_problem* p, int32_t* row_ptr_t, int32_t* col_idx_t, int32_t* perm,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_problem(p, kOpSoftmax);  // element CSR
  if (st != SA_OK) return st;
  if (!row_ptr_t || (p->nnz > 0 && (!col_idx_t || !perm || !workspace))) return SA_ERR_NULL;
  if (p->n == 0) return SA_OK;
  if (p->nnz > 0 && workspace_bytes < sa::transpose_workspace_bytes(p->n, p->nnz)) return SA_ERR_WORKSPACE;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_csr_transpose(*p, row_ptr_t, col_idx_t, perm, workspace, workspace_bytes, stream));
}

int sa_gather_entries(const sa_problem* p, const int32_t* perm, const float* src, float* dst,
                      hipStream_t stream) {
  int st = check_problem(p, kOpSoftmax);
  if (st != SA_OK) return st;
  if (empty_problem(p) || p->nnz == 0) return SA_OK;
  if (!perm || !src || !dst) return SA_ERR_NULL;
  if (src == dst) return SA_ERR_SHAPE;  // a permutation cannot be applied in place here
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_gather_entries(*p, perm, src, dst, stream));
}

int sa_gather_order_build(const sa_problem* p, const int32_t* perm, int32_t* order, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  int st = check_problem(p, kOpSoftmax);
  if (st != SA_OK) return st;
  if (p->nnz == 0) return SA_OK;
  if (!perm || !order || !workspace) return SA_ERR_NULL;
  if (workspace_bytes < sa::transpose_workspace_bytes(p->n, p->nnz)) return SA_ERR_WORKSPACE;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_gather_order_build(*p, perm, order, workspace, workspace_bytes, stream));
}

int sa_gather_entries_ordered(const sa_problem* p, const int32_t* order, const float* src_a,
                              float* dst_a, const float* src_b, float* dst_b, hipStream_t stream) {
  int st = check_problem(p, kOpSoftmax);
  if (st != SA_OK) return st;
  if (empty_problem(p) || p->nnz == 0) return SA_OK;
  if (!order || !src_a || !dst_a || (src_b == nullptr) != (dst_b == nullptr)) return SA_ERR_NULL;
  // no destination may alias a source or the other destination
  if (src_a == dst_a || (src_b && (src_b == dst_b || src_a == dst_b || src_b == dst_a || dst_a == dst_b)))
    return SA_ERR_SHAPE;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_gather_ordered(*p, order, src_a, dst_a, src_b, dst_b, stream));
}

int sa_bias_grad(const sa_problem* p, const float* dscores, float factor, float* dbias,
                 hipStream_t stream) {
  if (!p) return SA_ERR_NULL;
  int st = check_problem(p, p->row_ptr ? kOpSoftmax : kOpFused);  // element CSR or dense
  if (st != SA_OK) return st;
  if (!p->row_ptr && p->block != 1) return SA_ERR_UNSUPPORTED;
  if (!std::isfinite(factor)) return SA_ERR_SHAPE;
  if ((long long)p->H * p->n * (long long)p->n > (1ll << 40)) return SA_ERR_SHAPE;
  if (empty_problem(p) || (p->row_ptr && p->nnz == 0)) return SA_OK;
  if (!dscores || !dbias) return SA_ERR_NULL;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_bias_grad(*p, dscores, factor, dbias, stream));
}

int sa_sparse_softmax_backward(const sa_problem* p, const float* weights, const float* dweights,
                               float out_scale, float* dscores, hipStream_t stream) {
  int st = check_problem(p, kOpSoftmax);
  if (st != SA_OK) return st;
  if (!std::isfinite(out_scale)) return SA_ERR_SHAPE;
  if (empty_problem(p) || p->nnz == 0) return SA_OK;
  if (!weights || !dweights || !dscores) return SA_ERR_NULL;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_softmax_backward(*p, weights, dweights, out_scale, dscores, stream));
}

size_t sa_mask_workspace_bytes(int32_t n, int64_t nnz) {
  if (n < 0 || nnz < 0 || nnz > INT32_MAX - 1) return 0;
  return sa::mask_workspace_bytes(n, nnz);
}

int sa_coo_to_csr(int32_t n, int64_t nnz, const int32_t* rows, const int32_t* cols, int32_t* row_ptr,
                  int32_t* col_idx, int32_t* counts, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  if (n < 0 || nnz < 0 || nnz > INT32_MAX - 1) return SA_ERR_SHAPE;
  if (!row_ptr || !counts || (nnz > 0 && (!rows || !cols || !col_idx || !workspace))) return SA_ERR_NULL;
  if (nnz > 0 && workspace_bytes < sa::mask_workspace_bytes(n, nnz)) return SA_ERR_WORKSPACE;
  clear_stale_error();
  return hip_status(sa::launch_coo_to_csr(n, nnz, rows, cols, row_ptr, col_idx, counts, workspace,
                                          workspace_bytes, stream));
}

int sa_key_mask_from_lengths(int32_t B, int32_t n, const int32_t* seqlen_k, float* key_mask,
                             hipStream_t stream) {
  if (B < 0 || n < 0 || (long long)B * n > INT32_MAX) return SA_ERR_SHAPE;
  if ((long long)B * n == 0) return SA_OK;
  if (!seqlen_k || !key_mask) return SA_ERR_NULL;
  clear_stale_error();
  return hip_status(sa::launch_key_mask_from_lengths(B, n, seqlen_k, key_mask, stream));
}

namespace {
// Largest pattern a packed batch can give: every token attends at most min(total, 2w + 1) keys.
int check_varlen(int32_t B, int32_t total, int32_t window) {
  if (B < 0 || total < 0) return SA_ERR_SHAPE;
  const long long per_row = window >= 0 && 2ll * window + 1 < total ? 2ll * window + 1 : total;
  if ((long long)total * per_row > INT32_MAX) return SA_ERR_SHAPE;
  return SA_OK;
}
}  // namespace

int sa_varlen_row_ptr(int32_t B, int32_t total, const int32_t* cu_seqlens, int32_t window,
                      int32_t* row_ptr, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_varlen(B, total, window);
  if (st != SA_OK) return st;
  if (!row_ptr || (total > 0 && (!cu_seqlens || !workspace))) return SA_ERR_NULL;
  if (total > 0 && workspace_bytes < sa::mask_workspace_bytes(total, 0)) return SA_ERR_WORKSPACE;
  if (total > 0 && B == 0) return SA_ERR_SHAPE;  // tokens but no sequence
  clear_stale_error();
  return hip_status(sa::launch_varlen_row_ptr(B, total, cu_seqlens, window, row_ptr, workspace,
                                              workspace_bytes, stream));
}

int sa_varlen_col_idx(int32_t B, int32_t total, const int32_t* cu_seqlens, int32_t window,
                      const int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                      hipStream_t stream) {
  const int st = check_varlen(B, total, window);
  if (st != SA_OK) return st;
  if (col_capacity < 0) return SA_ERR_SHAPE;
  if (total == 0 || col_capacity == 0) return SA_OK;
  if (!cu_seqlens || !row_ptr || !col_idx) return SA_ERR_NULL;
  if (B == 0) return SA_ERR_SHAPE;
  clear_stale_error();
  return hip_status(sa::launch_varlen_col_idx(B, total, cu_seqlens, window, row_ptr, col_idx,
                                              col_capacity, stream));
}

int sa_topk_mask(int32_t n, int32_t k, const float* scores, int32_t* row_ptr, int32_t* col_idx,
                 hipStream_t stream) {
  if (n < 0 || k < 0) return SA_ERR_SHAPE;
  const int32_t kk = k < n ? k : n;
  if ((long long)n * kk > INT32_MAX) return SA_ERR_SHAPE;
  if (!row_ptr || (n > 0 && (!scores || (kk > 0 && !col_idx)))) return SA_ERR_NULL;
  clear_stale_error();
  return hip_status(sa::launch_topk_mask(n, kk, scores, row_ptr, col_idx, stream));
}

namespace {
constexpr int32_t kCoverMaxN = 1 << 22;  // block-row bitmap of ceil(n/64) bits in LDS

int check_cover_problem(const sa_problem* p) {
  const int st = check_problem(p, kOpSoftmax);  // element CSR
  if (st != SA_OK) return st;
  if (p->n > kCoverMaxN) return SA_ERR_SHAPE;
  return SA_OK;
}

int check_cover(const sa_problem* p, const sa_block_cover* c) {
  if (!c) return SA_ERR_NULL;
  const long long nb = (p->n + 63) / 64;
  if (c->nnz < 0 || c->nnz > nb * nb) return SA_ERR_SHAPE;
  if (p->n > 0 && (!c->row_ptr || !c->t_row_ptr)) return SA_ERR_NULL;
  if (c->nnz > 0 && (!c->col_idx || !c->t_col_idx || !c->bits || !c->bits_t)) return SA_ERR_NULL;
  return SA_OK;
}
}  // namespace

int sa_block_cover_row_ptr(const sa_problem* p, int32_t* cover_row_ptr, hipStream_t stream) {
  int st = check_cover_problem(p);
  if (st != SA_OK) return st;
  if (!cover_row_ptr || (p->n > 0 && !p->row_ptr)) return SA_ERR_NULL;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_block_cover_rows(p->n, p->nnz, p->row_ptr, p->col_idx, cover_row_ptr, stream));
}

int sa_block_cover_col_idx(const sa_problem* p, const int32_t* cover_row_ptr, int64_t cover_nnz,
                           int32_t* cover_col_idx, hipStream_t stream) {
  int st = check_cover_problem(p);
  if (st != SA_OK) return st;
  const long long nb = (p->n + 63) / 64;
  if (cover_nnz < 0 || cover_nnz > nb * nb) return SA_ERR_SHAPE;
  if (!cover_row_ptr || (cover_nnz > 0 && !cover_col_idx)) return SA_ERR_NULL;
  if (p->n == 0 || cover_nnz == 0) return SA_OK;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_block_cover_cols(p->n, p->nnz, p->row_ptr, p->col_idx, cover_row_ptr,
                                                cover_nnz, cover_col_idx, stream));
}

int sa_block_cover_bits(const sa_problem* p, const sa_block_cover* c, hipStream_t stream) {
  int st = check_cover_problem(p);
  if (st != SA_OK) return st;
  if ((st = check_cover(p, c)) != SA_OK) return st;
  if (p->n == 0 || c->nnz == 0) return SA_OK;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_block_cover_bits(p->n, p->nnz, p->row_ptr, p->col_idx, c->row_ptr,
                                                c->col_idx, c->t_row_ptr, c->t_col_idx, c->nnz,
                                                c->bits, c->bits_t, stream));
}

int sa_fused_backward_cover(const sa_problem* p, const sa_block_cover* c, const void* q, const void* k,
                            const void* v, const float* out, const float* lse, const void* dout,
                            float* dq, float* dk, float* dv, float* dscores, float* workspace,
                            hipStream_t stream) {
  int st = check_problem(p, kOpFused);
  if (st != SA_OK) return st;
  if (!p->row_ptr || p->block != 1) return SA_ERR_UNSUPPORTED;  // element CSR
  if ((st = check_cover(p, c)) != SA_OK) return st;
  if (p->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (dscores && (long long)p->B * p->H * (long long)p->n * p->n > (1ll << 40)) return SA_ERR_SHAPE;
  if (empty_problem(p)) return SA_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(out))
    return SA_ERR_ALIGN;
  if ((long long)p->n * p->d * 2 > 0x7ffffff0ll) return SA_ERR_SHAPE;
  if (p->bias && (long long)p->n * p->n * 4 > 0x7ffffff0ll) return SA_ERR_UNSUPPORTED;
  if ((st = pre_launch(p, stream)) != SA_OK) return st;
  return hip_status(sa::launch_fused_backward_cover(*p, c->row_ptr, c->col_idx, c->t_row_ptr,
                                                    c->t_col_idx, c->nnz, c->bits, c->bits_t, q, k, v,
                                                    out, lse, dout, dq, dk, dv, dscores, workspace,
                                                    stream));
}

int sa_validate_csr(const sa_problem* p, hipStream_t stream) {
  const int st = check_problem(p, kOpValidate);
  if (st != SA_OK) return st;
  return validate_now(p, stream);
}

const char* sa_last_hip_error_string(void) {
  return g_last_hip_error == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip_error);
}

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL: a required pointer is NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE: inconsistent shape, size or broadcast dimension";
    case SA_ERR_CSR: return "SA_ERR_CSR: malformed CSR pattern";
    case SA_ERR_DTYPE: return "SA_ERR_DTYPE: unsupported element type";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: head size, block size, flag or pattern kind not supported by this call";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN: buffer not 16-byte aligned";
    case SA_ERR_HIP: return "SA_ERR_HIP: HIP runtime or launch failure";
    case SA_ERR_WORKSPACE:
      return "SA_ERR_WORKSPACE: plan or workspace too small (or the library's fixed scratch, for the "
             "entry points that allocate nothing), or a plan built for another pattern";
  }
  return "unknown sa status";
}

}  // extern "C"
