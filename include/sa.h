/*
 * sa.h -- masked scaled dot-product attention over a CSR attention mask,
 *         for AMD Instinct MI355X (gfx950 / CDNA4).
 *
 * What is computed (for every head t = b*H + h and query row i):
 *
 *   S[t,i,j] = scale * (q[t,i,:] . k[t,j,:]) + bias[h,i,j] + key_mask[b,hm,j]   for (i,j) in P
 *   W[t,i,j] = exp(S[t,i,j] - m) / sum_{j' in P_i} exp(S[t,i,j'] - m),  m = max_{j in P_i} S[t,i,j]
 *   O[t,i,:] = sum_{j in P_i} W[t,i,j] * v[t,j,:]
 *   lse[t,i] = m + log sum_{j in P_i} exp(S[t,i,j] - m)
 *
 * P is the attention pattern: query i attends key j iff the user's (n, n) mask
 * holds a nonzero at (i, j) (gluon-nlp issue "[Proposal] Unified
 * Interface/Implementation for Sparse Attention", opening post: the mask is a
 * CSR/COO matrix of shape (n, n)). The three steps of that post are exported
 * as sa_sddmm (scores at the nonzeros, same pattern as the mask), sa_sparse_softmax
 * (softmax over each sparse row, same pattern) and sa_spmm (CSR weights times
 * dense V). sa_fused_forward computes O in one pass with a running maximum and
 * a running sum that rescale earlier partial results, dividing once at the end
 * (the streaming-dataflow SDPA review on nubint.ai, "proposed method" list:
 * reordering the divide by the distributive law, and running max / running
 * sum with delta rescaling). The additive bias and key mask follow the shapes
 * of the flash-attention pull request "support attentions in AlphaFold2"
 * (the mask [total_size, 1 or head, 1, seq_k] and bias [1, head, seq_q, seq_k]
 * shape lists).
 *
 * Conventions (readings where the pages are silent):
 *   - The scale multiplies q.k only; bias and key_mask are added unscaled.
 *   - A row with no stored entry, or whose every score is -inf, has W = 0 at
 *     its stored entries, O = 0 and lse = -inf.
 *   - Every output is fp32. Inputs q/k/v are fp32 or bf16 (SA_F32 / SA_BF16).
 *
 * Memory: every pointer argument and every pointer inside sa_problem is a
 * DEVICE pointer (hipMalloc / torch CUDA tensor on the current device),
 * row-major and contiguous, owned by the caller. The library keeps no pointer
 * after a call returns. Calls are asynchronous on the given stream (0 = the
 * null stream); outputs are valid after the stream is synchronised. The library
 * keeps no state between calls; buffers the caller passes (a row plan among them, see
 * below) are the caller's to order between streams.
 *
 * Errors: every call returns SA_OK (0) or a negative sa_status, and checks its
 * arguments on the host before touching the device. Host checks cover pointers,
 * shapes, dtypes, alignment and the descriptor; the CSR content (monotone
 * row_ptr, nnz == row_ptr[n], columns sorted, unique and in range) is checked on
 * the device only when flags has SA_FLAG_VALIDATE (that call then synchronises
 * the stream) or by sa_validate_csr. Without it, kernels clamp every index they
 * read into range, so a malformed CSR gives wrong numbers but no invalid access.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_NULL = -1,        /* a required pointer is NULL                                  */
  SA_ERR_SHAPE = -2,       /* B, H, n, d, nnz or a broadcast dimension is inconsistent   */
  SA_ERR_CSR = -3,         /* device validation found a malformed CSR                     */
  SA_ERR_DTYPE = -4,       /* dtype is not SA_F32 / SA_BF16                               */
  SA_ERR_UNSUPPORTED = -5, /* d not in {32,64,128}, block not in {1,64}, or pattern kind
                              not accepted by this call                                   */
  SA_ERR_ALIGN = -6,       /* q/k/v/out (or plan) base pointer not 16-byte aligned        */
  SA_ERR_HIP = -7,         /* a HIP runtime call or kernel launch failed                  */
  SA_ERR_WORKSPACE = -8    /* plan or workspace too small (or the fixed scratch of the
                              no-allocation entry point), or a plan for another problem    */
} sa_status;

typedef enum sa_dtype { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

#define SA_FLAG_VALIDATE 1 /* validate the CSR on the device first (synchronises the stream) */

/* Problem descriptor. Field order and sizes are part of the ABI.
 *
 * q, k, v are [B*H, n, d] with head t = b*H + h (the q/k/v shape
 * [total_size * head, seq, head_dim] of the AlphaFold2 pull request).
 *
 * Pattern kinds:
 *   block == 1,  row_ptr != NULL : element CSR. row_ptr [n+1], col_idx [nnz], nnz == row_ptr[n].
 *   block == 64, row_ptr != NULL : block CSR of 64x64 tiles. row_ptr [ceil(n/64)+1] over
 *                                  block-rows, col_idx [nnz] block-columns, nnz == stored blocks.
 *                                  A ragged last tile covers only the rows/columns < n.
 *   row_ptr == NULL              : dense pattern (every (i, j)); nnz and col_idx ignored.
 * Columns of a row must be sorted ascending and unique. One pattern serves every head.
 *
 * bias     : NULL or fp32 [H, n, n] (the [1, H, seq_q, seq_k] bias), added to S.
 * key_mask : NULL or fp32 [B, key_mask_heads, n] (the [B, 1 or H, 1, seq_k] additive
 *            key mask, usually 0 / -inf); key_mask_heads is 1 or H.
 * plan     : NULL, or a buffer filled by sa_plan_build for this same pattern (16-byte aligned,
 *            SA_ERR_ALIGN otherwise); calls that schedule rows read it instead of building
 *            their own.
 * seqlen_k : NULL or int32 [B] on the device: keys j >= seqlen_k[b] (clamped to [0, n]) are
 *            masked for every head and query of batch b, as if the key mask held -inf there
 *            (the one-int-per-batch key padding of the AlphaFold2 pull request, key-padding
 *            discussion). Read by sa_sddmm and sa_fused_forward (the dense and block-CSR
 *            tiles skip the key blocks past the length; the element-CSR plan tiles mask
 *            the keys past it); it may be combined with key_mask. */
typedef struct sa_problem {
  int32_t B, H, n, d;
  int32_t dtype;           /* sa_dtype of q, k, v                                     */
  int32_t block;           /* 1 or 64                                                 */
  const int32_t *row_ptr;  /* see pattern kinds                                       */
  const int32_t *col_idx;
  int64_t nnz;             /* stored entries of col_idx                               */
  float scale;             /* multiplies q.k                                          */
  int32_t key_mask_heads;  /* 1 or H; ignored when key_mask is NULL                   */
  const float *bias;
  const float *key_mask;
  const void *plan;
  const int32_t *seqlen_k; /* NULL or [B] valid keys per batch                        */
  int32_t flags;           /* SA_FLAG_*                                               */
  int32_t reserved;        /* must be 0                                               */
} sa_problem;

/* --- CSR row plan (load-balancing schedule) ------------------------------------------
 * The plan cuts every row of an element CSR into segments of at most a fixed
 * number of entries, so that rows of very different length (variable per-token
 * windows and global tokens, gluon-nlp issue replies; global tokens in the
 * "Sparse Attention" notes) become work units of similar size, and classifies each
 * 64-row tile (matrix-core tile, banded, gathered far columns, vector rows). Its
 * schedule depends on the pattern only (row_ptr, col_idx, n, nnz); it also holds the
 * merge counters and partial rows of split rows for B*H heads of d dimensions, which
 * sa_spmm and sa_fused_forward write during a call. Hence a plan serves one call at a
 * time: calls that may overlap (on other streams) need plans of their own, built from the
 * same pattern; stream-ordered calls may share one, for any B*H and d up to those it was
 * sized for (SA_ERR_WORKSPACE under SA_FLAG_VALIDATE otherwise).
 *
 * sa_plan_bytes: size in bytes of the plan buffer for problem p, from n, nnz, B*H and d
 *   alone (host-only, no device access; 0 on a bad descriptor). Requires block == 1 and
 *   row_ptr != NULL. It holds up to 1024 long-row segments; a pattern needing more gets a
 *   plan without segments, and its long rows are then computed whole (slower, same results).
 * sa_plan_bytes_segments: the same for up to max_segments segments. A row of len > 1024
 *   entries takes ceil(len / 256) segments; the sum over the pattern's rows is the count
 *   that keeps every long row split.
 * sa_plan_build: fills plan (16-byte aligned device buffer of at least the size of a plan
 *   without segments, caller-owned) on stream. The plan stays valid while the pattern's content is
 *   unchanged.
 * A plan pays off where 64-row tiles are dense enough for the matrix cores (windows, blocks,
 * dense rows). A pattern that is sparse everywhere (e.g. a few hundred random columns per row
 * out of thousands) runs about 10-25% faster with plan = NULL, whose row kernels need no LDS
 * and keep more waves per compute unit; rows longer than 1024 entries are then not split. */
size_t sa_plan_bytes(const sa_problem *p);
size_t sa_plan_bytes_segments(const sa_problem *p, int64_t max_segments);
int sa_plan_build(const sa_problem *p, void *plan, size_t plan_bytes, hipStream_t stream);

/* --- SDDMM: scores at the mask's nonzeros ----------------------------------------------
 * gluon-nlp issue, opening post, first bullet: a dot product between query i and key j
 * for each nonzero coordinate of the mask; the scores keep the mask's CSR format.
 * scores[t * nnz + e] = scale * q[t,i,:].k[t,col_idx[e],:] (+ bias[h,i,col]) (+ key_mask[b,hm,col])
 * for the row i that holds entry e. scores: fp32 [B*H, nnz], written entirely.
 * Pattern: element CSR only (else SA_ERR_UNSUPPORTED). */
int sa_sddmm(const sa_problem *p, const void *q, const void *k, float *scores, hipStream_t stream);

/* --- Sparse row softmax ------------------------------------------------------------------
 * gluon-nlp issue, opening post, second bullet: a softmax over each sparse row; the weights
 * keep the scores' pattern. weights[t*nnz + e] over the entries of each row; rows whose
 * scores are all -inf (or empty rows) get 0. scores and weights: fp32 [B*H, nnz]; they may
 * be the same buffer (in place). bias/key_mask/q/k are not used.
 * Pattern: element CSR only. */
int sa_sparse_softmax(const sa_problem *p, const float *scores, float *weights, hipStream_t stream);

/* --- SpMM: CSR weights times dense V ------------------------------------------------------
 * gluon-nlp issue, opening post, third bullet: the product of the sparse weights with the
 * dense value tensor gives the context. out[t,i,:] = sum_{e in row i} weights[t*nnz+e] *
 * v[t,col_idx[e],:]. out: fp32 [B*H, n, d], written entirely (0 for empty rows).
 * v has dtype p->dtype. Pattern: element CSR only. */
int sa_spmm(const sa_problem *p, const float *weights, const void *v, float *out, hipStream_t stream);

/* --- Fused forward --------------------------------------------------------------------------
 * One pass per row with a running maximum and running sum whose earlier partial sums are
 * rescaled when the maximum grows, and one division at the end (streaming-dataflow SDPA
 * review, "proposed method"); never writes S or W. Accepts every pattern kind, bias and
 * key_mask. out: fp32 [B*H, n, d]. lse: NULL or fp32 [B*H, n].
 * Element CSR with a plan runs the plan's dense-enough 64-row tiles on bf16 matrix cores
 * (dtype == SA_BF16) and the other rows on the vector ALUs (without a plan: all rows on the
 * vector ALUs); block CSR (block == 64) and the dense pattern run 64-query tiles on bf16
 * matrix cores when dtype == SA_BF16, as each stored tile is a dense product (block-sparse
 * replies of the gluon-nlp issue; the AlphaFold2 pull request for the dense pattern with
 * bias and key mask). */
int sa_fused_forward(const sa_problem *p, const void *q, const void *k, const void *v,
                     float *out, float *lse, hipStream_t stream);

/* --- Backward pass of the CSR pipeline -----------------------------------------------------
 * With dO the gradient of a loss with respect to the context, the chain rule through the
 * three steps of the gluon-nlp proposal (opening post), taken in reverse, is, per head and
 * stored entry (i, j):  dW = dO[i].v[j] (sa_sddmm of dO and V at scale 1, no bias/mask),
 * dS = W (dW - sum_row W dW) (sa_sparse_softmax_backward), dQ = scale * dS K (sa_spmm),
 * dK = scale * dS^T Q and dV = W^T dO (sa_spmm over the transposed pattern, with dS and W
 * gathered into its order by sa_gather_entries or sa_gather_entries_ordered). dS is also the gradient of the additive
 * bias and key mask at the stored entries. Element CSR only.
 *
 * sa_transpose_workspace_bytes: device workspace bytes sa_csr_transpose needs (host-only;
 *   0 on a bad descriptor).
 * sa_csr_transpose: the transposed pattern, built on the device on stream: row_ptr_t
 *   int32 [n+1], col_idx_t int32 [nnz] (each column's rows, ascending) and perm int32 [nnz]
 *   (perm[k] = index in the original CSR of transposed entry k). Depends on the pattern
 *   only: build it once per mask. All buffers are caller-owned; workspace is scratch for the
 *   duration of the call (SA_ERR_WORKSPACE if smaller than the size above).
 * sa_gather_entries: dst[t*nnz + k] = src[t*nnz + perm[k]] for every head t; src and dst
 *   are fp32 [B*H, nnz] and must not alias.
 * sa_gather_order_build: from perm, the read order of sa_gather_entries_ordered: order is
 *   int32 [2*nnz], caller-owned; within each block of 4096 consecutive positions k, the
 *   sources perm[k] ascending (first half) and the position each goes to (second half).
 *   Depends on the pattern only; workspace as for sa_csr_transpose (same size).
 * sa_gather_entries_ordered: the same result as sa_gather_entries with the perm that order
 *   was built from, for one array (src_b = dst_b = NULL) or two at once (e.g. dS and W);
 *   reads the sources in ascending runs, which is faster when the pattern is banded. No
 *   destination may alias a source or the other destination (SA_ERR_SHAPE).
 * sa_bias_grad: the gradient of the shared bias [H, n, n] (the flash-attention pull request's
 *   bias-gradient question): dbias[h, i, j] = factor * sum over b of dscores[(b*H + h)*nnz + e]
 *   for each stored entry e = (i, j); entries outside the pattern are not written (the caller
 *   zeroes dbias). With dscores from sa_sparse_softmax_backward at out_scale = scale, pass
 *   factor = 1 / scale (or out_scale = 1 and factor = 1). dbias fp32 [H, n, n]. With
 *   row_ptr = NULL (the dense pattern) dscores is [B*H, n, n], as sa_fused_backward writes
 *   it, and every (i, j) is written.
 * sa_sparse_softmax_backward: dscores[t*nnz + e] = out_scale * W[e] * (dW[e] - D_row),
 *   D_row = sum over the row's entries of W * dW; weights, dweights and dscores are fp32
 *   [B*H, nnz] (dscores may alias dweights). out_scale = scale gives the operand of dQ
 *   and dK; out_scale = 1 gives the gradient of the scores. */
/* --- Backward of the fused forward ---------------------------------------------------------
 * sa_fused_backward: the gradients of the fused forward over the dense pattern (additive
 *   bias, key mask and key lengths as in sa_fused_forward; the AlphaFold2 pull request's
 *   training and bias-gradient questions) or over block CSR of 64x64 tiles, from its
 *   outputs: out fp32 [B*H, n, d] and lse
 *   fp32 [B*H, n]. dout is the gradient of out, in the dtype of q/k/v (bf16 only). The
 *   weights are recomputed from lse (P = exp(S - lse)), never stored: dQ = scale dS K,
 *   dK = scale dS^T Q, dV = P^T dO with dS = P (dO V^T - rowsum(dO * O)). dq, dk, dv fp32
 *   [B*H, n, d]. dscores (optional, fp32 [B*H, n, n]) receives dS, the gradient of the
 *   scores and so of the bias and key mask at each pair of the pattern (pairs outside a
 *   block pattern are not written; sa_bias_grad with row_ptr = NULL sums it over the
 *   batches). workspace: fp32 [B*H*n], caller-owned scratch.
 *   Block CSR also needs the transposed block pattern, t_row_ptr [ceil(n/64)+1] and
 *   t_col_idx [nnz] (the block-rows holding each block-column, e.g. sa_csr_transpose of a
 *   descriptor whose n is the number of block-rows); they are ignored for the dense pattern.
 *   Pattern: dense or block CSR (element CSR: SA_ERR_UNSUPPORTED); dtype bf16 only; with a
 *   bias, n <= 23170 (a bias head addressed with 32-bit offsets; else SA_ERR_UNSUPPORTED). */
int sa_fused_backward(const sa_problem *p, const void *q, const void *k, const void *v,
                      const float *out, const float *lse, const void *dout,
                      const int32_t *t_row_ptr, const int32_t *t_col_idx, float *dq, float *dk,
                      float *dv, float *dscores, float *workspace, hipStream_t stream);

/* --- Fused backward without a workspace argument ---------------------------------------------
 * For callers that cannot allocate device memory (code under HIP stream capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, arguments and outputs as
 * sa_fused_backward without `workspace`; the row sums it needs live in a fixed device array of
 * the library, 16 MiB on each GPU it runs on (held until the process ends), so B*H*n <= 4 Mi
 * (else SA_ERR_WORKSPACE). Allocates nothing and calls no allocating routine; SA_FLAG_VALIDATE
 * is refused (SA_ERR_UNSUPPORTED), since device validation allocates. Every call on one GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams, other threads)
 * race and give wrong gradients; serialise them. */
int sa_fused_backward_noalloc(const sa_problem *p, const void *q, const void *k, const void *v,
                              const float *out, const float *lse, const void *dout,
                              const int32_t *t_row_ptr, const int32_t *t_col_idx, float *dq, float *dk,
                              float *dv, float *dscores, hipStream_t stream);

/* --- Block cover of an element pattern; fused backward over element CSR -----------------
 * The block-sparse replies of the gluon-nlp issue compute whole 64x64 blocks on fast
 * kernels; the cover carries an element CSR pattern onto them. It is the set of 64x64 blocks
 * of the (n, n) grid holding at least one entry, as block CSR over nb = ceil(n/64)
 * block-rows, with two arrays of 64-bit words: bits [nnz * 64], word r of cover block
 * (R, C) having bit c set when (64R + r, 64C + c) is an entry; bits_t [nnz * 64], word c of
 * the block at position j of the transposed cover (block-column C, block-row R) having bit
 * r set for the same entries. Built once per mask, on the device, in this order:
 *   sa_block_cover_row_ptr: cover row_ptr int32 [nb+1]; its last value is the cover's nnz
 *     (read it back to size the arrays below).
 *   sa_block_cover_col_idx: cover col_idx int32 [cover_nnz], each block-row's block-columns
 *     ascending.
 *   sa_csr_transpose of an element-CSR descriptor over the cover (n = nb, nnz = cover_nnz):
 *     t_row_ptr [nb+1], t_col_idx [cover_nnz] (the block-rows holding each block-column).
 *   sa_block_cover_bits: fills c->bits and c->bits_t from the pattern and the four arrays.
 * p: the element CSR pattern (block 1, columns ascending and unique), n <= 2^22 (SA_ERR_SHAPE).
 * Entries with a column outside [0, n) are skipped. The caller owns every array.
 *
 * sa_fused_backward_cover: the gradients of sa_fused_forward over an element CSR pattern
 *   (same inputs and outputs as sa_fused_backward) computed on its block cover: each cover
 *   block is computed whole and the words give pairs outside the pattern no weight. dscores
 *   (optional, fp32 [B*H, n, n]) is written at every pair of the cover's blocks (0 outside
 *   the pattern). bf16 only; bias, key_mask and seqlen_k as in sa_fused_backward. */
typedef struct sa_block_cover {
  const int32_t *row_ptr;    /* [nb+1]                                             */
  const int32_t *col_idx;    /* [nnz] block-columns                                */
  const int32_t *t_row_ptr;  /* [nb+1] transposed cover                            */
  const int32_t *t_col_idx;  /* [nnz] block-rows                                   */
  uint64_t *bits;            /* [nnz * 64] per block row                           */
  uint64_t *bits_t;          /* [nnz * 64] per transposed block column             */
  int64_t nnz;               /* stored blocks                                      */
} sa_block_cover;

int sa_block_cover_row_ptr(const sa_problem *p, int32_t *cover_row_ptr, hipStream_t stream);
int sa_block_cover_col_idx(const sa_problem *p, const int32_t *cover_row_ptr, int64_t cover_nnz,
                           int32_t *cover_col_idx, hipStream_t stream);
int sa_block_cover_bits(const sa_problem *p, const sa_block_cover *c, hipStream_t stream);
int sa_fused_backward_cover(const sa_problem *p, const sa_block_cover *c, const void *q,
                            const void *k, const void *v, const float *out, const float *lse,
                            const void *dout, float *dq, float *dk, float *dv, float *dscores,
                            float *workspace, hipStream_t stream);

size_t sa_transpose_workspace_bytes(const sa_problem *p);
int sa_csr_transpose(const sa_problem *p, int32_t *row_ptr_t, int32_t *col_idx_t, int32_t *perm,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);
int sa_gather_entries(const sa_problem *p, const int32_t *perm, const float *src, float *dst,
                      hipStream_t stream);
int sa_gather_order_build(const sa_problem *p, const int32_t *perm, int32_t *order,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);
int sa_gather_entries_ordered(const sa_problem *p, const int32_t *order, const float *src_a,
                              float *dst_a, const float *src_b, float *dst_b, hipStream_t stream);
int sa_sparse_softmax_backward(const sa_problem *p, const float *weights, const float *dweights,
                               float out_scale, float *dscores, hipStream_t stream);
int sa_bias_grad(const sa_problem *p, const float *dscores, float factor, float *dbias,
                 hipStream_t stream);

/* --- Mask construction ---------------------------------------------------------------------
 * The gluon-nlp proposal (opening post) takes the mask as a sparse (n, n) matrix in CSR or
 * COO form, possibly generated at run time; the flash-attention pull request "support
 * attentions in AlphaFold2" (key-padding discussion) proposes one int per batch, the number
 * of valid keys, when the masked keys are a suffix, and packs variable-length sequences by a
 * prefix of their starts (cu_seqlens). These calls turn those forms into the inputs the
 * kernels above read. All run on stream, take device pointers and allocate nothing.
 *
 * sa_mask_workspace_bytes: device workspace bytes for sa_coo_to_csr with n and nnz pairs,
 *   and for sa_varlen_row_ptr with total = n (host-only; 0 on bad sizes).
 * sa_coo_to_csr: rows, cols int32 [nnz] (any order) -> row_ptr int32 [n+1] and col_idx
 *   int32 (capacity nnz): the CSR of the set of pairs with 0 <= row, col < n, each row's
 *   columns ascending and unique. Pairs outside [0, n) are dropped and repeated pairs are
 *   merged; counts int32 [3] receives {stored entries (= row_ptr[n]), pairs dropped, pairs
 *   merged}. nnz < 2^31 - 1 (SA_ERR_SHAPE), SA_ERR_WORKSPACE if the workspace is short.
 * sa_key_mask_from_lengths: key_mask fp32 [B, n] (the layout of sa_problem.key_mask with
 *   key_mask_heads = 1): 0 for keys j < seqlen_k[b] (clamped to [0, n]), -inf after.
 * sa_varlen_row_ptr / sa_varlen_col_idx: the pattern of a packed batch of B sequences,
 *   sequence b holding tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of total (cu_seqlens int32
 *   [B+1], ascending, cu_seqlens[0] = 0): token i attends the keys of its own sequence, and
 *   only those with |i - j| <= window when window >= 0. Tokens outside every sequence get
 *   empty rows. The first call writes row_ptr int32 [total+1] (read row_ptr[total] for the
 *   entry count); the second writes col_idx (writing nothing at or past col_capacity). Used
 *   with B = 1 and n = total in sa_problem, q/k/v laid out [H, total, d]. SA_ERR_SHAPE if
 *   the pattern could exceed 2^31 - 1 entries (total * min(total, 2 window + 1)).
 * sa_topk_mask: a mask generated from scores at run time: every query keeps the k keys of
 *   largest score, a constant number per query (the SPARSEK abstract's selection; the
 *   scoring network is the caller's). scores fp32 [n, n] row-major; row_ptr int32 [n+1]
 *   gets i * min(k, n) and col_idx int32 [n * min(k, n)] each row's chosen columns in
 *   ascending order. Equal scores are taken lowest column first; NaN counts as -inf and -0
 *   as +0. SA_ERR_SHAPE if n * min(k, n) >= 2^31. */
size_t sa_mask_workspace_bytes(int32_t n, int64_t nnz);
int sa_coo_to_csr(int32_t n, int64_t nnz, const int32_t *rows, const int32_t *cols,
                  int32_t *row_ptr, int32_t *col_idx, int32_t *counts, void *workspace,
                  size_t workspace_bytes, hipStream_t stream);
int sa_key_mask_from_lengths(int32_t B, int32_t n, const int32_t *seqlen_k, float *key_mask,
                             hipStream_t stream);
int sa_varlen_row_ptr(int32_t B, int32_t total, const int32_t *cu_seqlens, int32_t window,
                      int32_t *row_ptr, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);
int sa_varlen_col_idx(int32_t B, int32_t total, const int32_t *cu_seqlens, int32_t window,
                      const int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                      hipStream_t stream);
int sa_topk_mask(int32_t n, int32_t k, const float *scores, int32_t *row_ptr, int32_t *col_idx,
                 hipStream_t stream);

/* --- Validation and status ----------------------------------------------------------------
 * sa_validate_csr: checks the pattern on the device (monotone row_ptr starting at 0,
 *   row_ptr[last] == nnz, columns in range, strictly ascending within each row) and
 *   synchronises the stream. Returns SA_OK, SA_ERR_CSR, or an argument error.
 * sa_status_string: a static, human-readable name for a status code.
 * sa_last_hip_error_string: the HIP runtime's description of the most recent HIP failure
 *   behind an SA_ERR_HIP returned to the calling thread ("no HIP error" if none). */
int sa_validate_csr(const sa_problem *p, hipStream_t stream);
const char *sa_status_string(int status);
const char *sa_last_hip_error_string(void);

#ifdef __cplusplus
}
#endif
#endif /* SA_H */
