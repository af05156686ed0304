// Internal launchers of the gfx950 kernels. The host-side ABI (api.cpp) validates the
// arguments and then calls these; each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include "../../include/sa.h"

namespace sa {

hipError_t launch_sddmm(const sa_problem& p, const void* q, const void* k, float* scores,
                        hipStream_t s);
hipError_t launch_softmax(const sa_problem& p, const float* scores, float* weights, hipStream_t s);
hipError_t launch_spmm(const sa_problem& p, const float* weights, const void* v, float* out,
                       hipStream_t s);
hipError_t launch_fused_valu(const sa_problem& p, const void* q, const void* k, const void* v,
                             float* out, float* lse, hipStream_t s);
hipError_t launch_fused_tile(const sa_problem& p, const void* q, const void* k, const void* v,
                             float* out, float* lse, hipStream_t s);
bool fused_tile_supported(const sa_problem& p);
// Dense pattern with the head's K and V resident in LDS (bf16, small n).
hipError_t launch_fused_resident(const sa_problem& p, const void* q, const void* k, const void* v,
                                 float* out, float* lse, hipStream_t s);
bool fused_resident_supported(const sa_problem& p);

// Backward pass pieces: pattern transpose, per-entry gather, softmax gradient.
size_t transpose_workspace_bytes(long long n, long long nnz);
hipError_t launch_csr_transpose(const sa_problem& p, int* row_ptr_t, int* col_idx_t, int* perm,
                                void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_gather_entries(const sa_problem& p, const int* perm, const float* src, float* dst,
                                 hipStream_t s);
hipError_t launch_gather_order_build(const sa_problem& p, const int* perm, int* order, void* ws,
                                     size_t ws_bytes, hipStream_t s);
hipError_t launch_gather_ordered(const sa_problem& p, const int* order, const float* src_a,
                                 float* dst_a, const float* src_b, float* dst_b, hipStream_t s);
hipError_t launch_bias_grad(const sa_problem& p, const float* ds, float factor, float* dbias,
                            hipStream_t s);
hipError_t launch_softmax_backward(const sa_problem& p, const float* w, const float* dw,
                                   float out_scale, float* ds, hipStream_t s);

// Backward of the fused forward (dense, or block CSR with its transposed block pattern) from
// the saved lse (delta: [B*H*n] workspace).
hipError_t launch_fused_backward(const sa_problem& p, const void* q, const void* k, const void* v,
                                 const float* out, const float* lse, const void* dout, float* dq,
                                 float* dk, float* dv, float* dscores, float* delta,
                                 const int* t_row_ptr, const int* t_col_idx, hipStream_t s);
hipError_t launch_fused_backward_cover(const sa_problem& p, const int* c_row_ptr, const int* c_col_idx,
                                       const int* t_row_ptr, const int* t_col_idx, long long cover_nnz,
                                       const uint64_t* bits, const uint64_t* bits_t, const void* q,
                                       const void* k, const void* v, const float* out, const float* lse,
                                       const void* dout, float* dq, float* dk, float* dv, float* dscores,
                                       float* delta, hipStream_t s);
hipError_t launch_block_cover_rows(int n, long long nnz, const int* row_ptr, const int* col_idx,
                                   int* cover_row_ptr, hipStream_t s);
hipError_t launch_block_cover_cols(int n, long long nnz, const int* row_ptr, const int* col_idx,
                                   const int* cover_row_ptr, long long cover_nnz, int* cover_col_idx,
                                   hipStream_t s);
hipError_t launch_block_cover_bits(int n, long long nnz, const int* row_ptr, const int* col_idx,
                                   const int* c_row_ptr, const int* c_col_idx, const int* t_row_ptr,
                                   const int* t_col_idx, long long cover_nnz, uint64_t* bits,
                                   uint64_t* bits_t, hipStream_t s);

// Mask construction: COO -> CSR, key mask from key lengths, packed variable-length batches.
size_t mask_workspace_bytes(long long n, long long nnz);
hipError_t launch_coo_to_csr(int n, long long nnz, const int* rows, const int* cols, int* row_ptr,
                             int* col_idx, int* counts, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_key_mask_from_lengths(int B, int n, const int* seqlen_k, float* key_mask,
                                        hipStream_t s);
hipError_t launch_varlen_row_ptr(int B, int total, const int* cu, int window, int* row_ptr,
                                 void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_varlen_col_idx(int B, int total, const int* cu, int window, const int* row_ptr,
                                 int* col_idx, long long cap, hipStream_t s);
hipError_t launch_topk_mask(int n, int k, const float* scores, int* row_ptr, int* col_idx,
                            hipStream_t s);

// The library's fixed device scratch (16 MiB per GPU) for the entry points that allocate
// nothing: its device address on the current device (looked up on the first call there).
constexpr size_t kNoAllocScratchBytes = 16u << 20;
hipError_t noalloc_scratch(void** ptr);

// CSR row plan and validation.
size_t plan_bytes_for(long long n, long long long_rows, long long segs, long long BH, long long d);
hipError_t launch_plan(const sa_problem& p, void* plan, size_t bytes, hipStream_t s);
hipError_t launch_validate(const sa_problem& p, int* flag_dev, hipStream_t s);

}  // namespace sa
