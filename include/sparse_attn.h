/*
 * sparse_attn.h -- C ABI of the block-sparse attention forward library for
 * AMD MI355X (gfx950): token reorder, block-mask prediction, sparse
 * FlashAttention-style forward, inverse reorder.
 *
 * What is computed (sources cited by page title and section):
 *   - Attention restricted to a kept key set is the softmax over the kept keys
 *     only ("AIGC 基本功|视频稀疏注意力的误差与布局-SparseAttn", section 3.1);
 *     reordering Q, K, V and both mask axes together and undoing the reorder on
 *     the output leaves the operator unchanged (same article, section 3.4).
 *   - Block-mask prediction from mean-pooled block representatives, a
 *     self-similarity guard theta, a compressed softmax and TopCdf selection
 *     at cumulative mass tau ("SpargeAttention: 中文精读笔记", section 2.2),
 *     with first-frame / text sink blocks, a [t,h,w]-window or Hilbert token
 *     reorder and a sparsity keep floor (MindIE-SD "稀疏" page: rf_v2 and the
 *     sparse_attention interface; SpargeAttn notes, section 2.5), and a causal
 *     sliding window ("44. Local Sliding and Sparse Attention", Step 2).
 *   - Online-softmax attention over the kept (query block, key block) pairs,
 *     skipping QK^T and PV for dropped blocks, and optionally skipping PV for a
 *     group of query rows when the running-max gap is below lambda
 *     (SpargeAttn notes, sections 2.1 and 2.3).
 *
 * Conventions shared by every entry point:
 *   - Tensors are contiguous BNSD: [batch, heads, tokens, head_dim], row-major,
 *     with 16-byte aligned base pointers.  bf16 tensors are passed as uint16_t
 *     bit patterns.
 *   - Device pointers are owned by the caller.  The library never allocates,
 *     frees or keeps device memory, never synchronizes, and enqueues work only
 *     on the caller's stream (`stream` is a hipStream_t; NULL = the default
 *     stream).  There is no global mutable state: calls are reentrant.
 *   - Inputs are read-only; outputs are fully overwritten.
 *   - Return value: SA_OK, or a negative SA_ERR_* code.  Argument checks are
 *     done synchronously on the host before anything is enqueued, and never
 *     touch the HIP runtime, so they also work on a machine without a GPU.
 *     Conditions only visible on the device are written to the caller's
 *     `dev_status` word (device memory, int32), which the call resets to
 *     SA_OK first; read it after synchronizing.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define SA_OK                    0
#define SA_ERR_INVALID_ARGUMENT (-1) /* bad shape, pointer or parameter */
#define SA_ERR_UNSUPPORTED      (-2) /* head dim or block-size pair not compiled */
#define SA_ERR_CAPACITY         (-3) /* col_idx too small (device status) */
#define SA_ERR_EMPTY_ROW        (-4) /* a query block keeps no key block (device status) */
#define SA_ERR_HIP              (-5) /* a HIP launch failed */

/* ---- element types accepted by sa_permute ---------------------------- */
#define SA_BF16 0
#define SA_F32  1

/* ---- token orders for sa_plan_permutation ---------------------------- */
#define SA_ORDER_IDENTITY 0
#define SA_ORDER_WINDOW   1
#define SA_ORDER_HILBERT  2

/* Query rows that share one PV-skip decision: the rows of one wavefront. */
#define SA_PV_GROUP_ROWS 32

/* Largest number of key blocks per query block the mask predictor handles. */
#define SA_MAX_KEY_BLOCKS 2048

/* Token layout of one sequence (MindIE-SD "稀疏" page, sparse_attention
 * arguments txt_len and latent_shape [t,h,w]).  In the original order the
 * txt_len text tokens come first, then the t*h*w video tokens frame by frame
 * in raster order. */
typedef struct sa_layout {
    int64_t n_tokens;         /* N; must equal txt_len + t*h*w unless order is IDENTITY */
    int32_t order;            /* SA_ORDER_* */
    int32_t t, h, w;          /* latent grid of the video tokens */
    int32_t win_t, win_h, win_w; /* reorder window, SA_ORDER_WINDOW only */
    int32_t txt_len;          /* text tokens (prepended in the original order) */
    int32_t first_frame_sink; /* 1: frame 0 stays first, in raster order */
} sa_layout;

/* Block-mask prediction parameters (SpargeAttn notes, sections 2.1-2.2;
 * MindIE-SD sparse_attention arguments). */
typedef struct sa_mask_params {
    int32_t B, Hq, Hkv;       /* batch, query heads, key/value heads (Hq % Hkv == 0) */
    int32_t D;                /* head dim: 64 or 128 */
    int64_t N;                /* tokens per sequence */
    int32_t block_q, block_k; /* b_q, b_k (tokens per query / key block), 1..256 */
    int32_t causal;           /* 0 or 1 */
    int32_t sink_rows;        /* query blocks touching tokens [0, sink_rows) keep their whole
                                 valid row (MindIE-SD first-frame sink, read as full rows);
                                 0 = off, at most N */
    int64_t window;           /* causal sliding window W in tokens (0 = off; needs causal) */
    int64_t sink_front;       /* key blocks touching tokens [0, sink_front) are always kept */
    int64_t sink_back;        /* key blocks touching tokens [N-sink_back, N) are always kept */
    double tau;               /* TopCdf mass in (0, 1]; negative = unset */
    double theta;             /* self-similarity guard; <= 0 = off */
    double sparsity;          /* keep floor: ceil((1-s)*|valid|) blocks per row, s in [0,1); negative = unset */
    float scale;              /* score scale; 0 = 1/sqrt(D) */
    int32_t n_keys;           /* keys per sequence when they differ from the N queries
                                 (MindIE-SD latent_shape_k != latent_shape_q); 0 = N;
                                 not with causal; k is then [B,Hkv,n_keys,D] and the key
                                 blocks, back sink and key similarity cover n_keys tokens */
} sa_mask_params;

/* Sparse attention parameters (SpargeAttn notes, section 2.1 table). */
typedef struct sa_attn_params {
    int32_t B, Hq, Hkv;
    int32_t D, Dv;            /* D == Dv, 64 or 128 */
    int32_t block_q, block_k; /* compiled pairs: (16,16), (128,64), (128,128) */
    int32_t causal;
    int64_t N;
    float lambda;             /* PV-skip threshold (< 0); -INFINITY = off */
    float scale;              /* 0 = 1/sqrt(D) */
    int64_t col_cap;          /* entries col_idx holds; CSR entries at or past it are not read */
    int64_t n_keys;           /* keys per sequence, k and v [B,Hkv,n_keys,D]; 0 = N; not with causal */
} sa_attn_params;

/* Static text for a status code.  Never NULL. */
const char* sa_status_string(int code);

/* Host only.  Token reorder (MindIE-SD "稀疏" page, rf_v2 window reorder and
 * first-frame sink; SpargeAttn notes, section 2.5, Hilbert order).
 *   perm_host[i] = original index of the token placed at position i.
 * IDENTITY: perm = 0..N-1.  Otherwise frame 0 comes first in raster order when
 * first_frame_sink is set; the remaining frames follow in window order
 * (window t, h, w, then t, h, w inside a window, all raster) or Hilbert order
 * (J. Skilling's transform on the enclosing 2^k cube, axis 0 = t most
 * significant); the text tokens come last, in their original order.
 * n must equal L->n_tokens.  Returns SA_OK or SA_ERR_INVALID_ARGUMENT. */
int sa_plan_permutation(const sa_layout* L, int32_t* perm_host, int64_t n);

/* Host only.  3-D tile windows as a forced block pattern (the sliding-tile
 * idea the SparseAttn article discusses under Sliding Tile Attention: one
 * query tile shares one set of key tiles).  A video token at latent (t,h,w)
 * that takes part in the reorder lies in tile ((t-t0)/tile_t, h/tile_h,
 * w/tile_w), t0 = 1 with first_frame_sink, else 0; text tokens and the sink
 * frame are untiled.  In the order sa_plan_permutation gives for L (any
 * order; N must equal txt_len + t*h*w), query block i (block_q tokens) and key
 * block j (block_k tokens) are paired, pattern_host[i*n_kb + j] = 1, when some
 * token of i and some token of j lie in tiles that differ by at most
 * radius_t, radius_h, radius_w along t, h, w; else 0.  n_qb and n_kb must be
 * ceil(N/block_q) and ceil(N/block_k).  The pattern is an input of
 * sa_predict_mask_ex.  Returns SA_OK or SA_ERR_INVALID_ARGUMENT. */
int sa_plan_tile_window(const sa_layout* L, int32_t tile_t, int32_t tile_h, int32_t tile_w,
                        int32_t radius_t, int32_t radius_h, int32_t radius_w, int32_t block_q,
                        int32_t block_k, uint8_t* pattern_host, int64_t n_qb, int64_t n_kb);

/* Row gather with conversion to bf16 (SparseAttn article, section 3.4):
 *   y[b,h,i,:] = bf16_round_nearest_even(x[b,h,perm[i],:])
 * x: device [B,H,N,D] of x_dtype (SA_BF16 or SA_F32); y: device bf16 [B,H,N,D];
 * perm_dev: device int32 [N], a permutation of 0..N-1 (not checked; a row
 * whose entry lies outside 0..N-1 reads nothing and is written as zeros).
 * D must be a multiple of 8 and N * D/8 must fit in int32 (else
 * SA_ERR_UNSUPPORTED).  With the identity permutation this is the
 * documented way to hand fp32 inputs to the bf16 kernels.  x and y must not
 * overlap. */
int sa_permute(const void* x, int x_dtype, uint16_t* y, const int32_t* perm_dev,
               int32_t B, int32_t H, int64_t N, int32_t D, void* stream);

/* Inverse row scatter (SparseAttn article, section 3.4):
 *   x[b,h,perm[i],:] = y[b,h,i,:]
 * y, x: device fp32 [B,H,N,Dv] (no overlap); perm_dev: device int32 [N], a
 * permutation of 0..N-1 (not checked; an entry outside 0..N-1 stores nothing).
 * Dv must be a multiple of 4 and N * Dv/4 must fit in int32 (else
 * SA_ERR_UNSUPPORTED). */
int sa_unpermute(const float* y, float* x, const int32_t* perm_dev,
                 int32_t B, int32_t H, int64_t N, int32_t Dv, void* stream);

/* Bytes of device workspace sa_predict_mask needs for these parameters
 * (block means and similarities, the dense block mask, row counts), or 0 when
 * the parameters are invalid. */
size_t sa_predict_workspace_bytes(const sa_mask_params* p);

/* Byte offsets inside the workspace, for inspection after a call:
 * off[0] query-block means fp32 [B,Hq,n_qb,D]; off[1] key-block means fp32
 * [B,Hkv,n_kb,D]; off[2] query-block similarity fp32 [B,Hq,n_qb];
 * off[3] key-block similarity fp32 [B,Hkv,n_kb]; off[4] block mask uint8
 * [B,Hq,n_qb,n_kb]; off[5] kept blocks per row int32 [B*Hq*n_qb],
 * followed by the kept blocks of each group of g consecutive query blocks of
 * one head, int32 [G], G = B*Hq*ceil(n_qb/g), g in 8..16 chosen from B*Hq
 * and n_qb, and by the kept blocks of each run of 256 consecutive groups,
 * int32 [ceil(G/256)] (sa_predict_workspace_bytes accounts for both).
 * Returns SA_OK or SA_ERR_INVALID_ARGUMENT. */
int sa_predict_workspace_offsets(const sa_mask_params* p, int64_t off[6]);

/* Block-mask prediction on the PERMUTED q (device bf16 [B,Hq,N,D]) and k
 * (device bf16 [B,Hkv,N_k,D], N_k = n_keys or N) (SpargeAttn notes, section 2.2;
 * MindIE-SD rf_v2).  Per (batch b, query head h, query block i), with
 * n_qb = ceil(N/b_q), n_kb = ceil(N_k/b_k), KV head h / (Hq/Hkv):
 *   1. block means and similarity ||mean_t x_t/||x_t||||^2 over the block's real tokens;
 *   2. valid key blocks: all, or (causal) those whose first token is not after
 *      the query block's last token;
 *   3. forced key blocks (within the valid set): key similarity < theta; sink
 *      blocks; causal: window blocks (last key >= first query - W + 1) and the
 *      blocks overlapping the query block;
 *   4. query similarity < theta, or a query block touching the first
 *      sink_rows tokens: the whole valid row is kept;
 *   5. otherwise the other valid blocks are candidates: scores
 *      qbar.kbar*scale, softmax over the candidates, sorted by probability
 *      descending then block index ascending; TopCdf keeps the blocks whose
 *      preceding mass is still < tau (tau unset: none); the keep floor adds
 *      blocks up to ceil((1-s)*|valid|) kept in total (s unset: none);
 *   6. row = forced + kept.
 * Outputs: row_ptr device int32 [B*Hq*n_qb + 1] and col_idx device int32
 * [col_cap], the CSR of kept key blocks per row, rows in (b, h, i) order, each
 * row ascending.  When the total exceeds col_cap, col_idx keeps the first
 * col_cap entries and dev_status is set to SA_ERR_CAPACITY (row_ptr is still
 * the full count).  Optional (NULL = not written): mask_out device uint8
 * [B,Hq,n_qb,n_kb] (1 = kept), sim_q device fp32 [B,Hq,n_qb], sim_k device fp32
 * [B,Hkv,n_kb].  ws: device workspace of ws_bytes >= sa_predict_workspace_bytes(p),
 * 256-byte aligned.  n_kb must not exceed SA_MAX_KEY_BLOCKS and B*Hq*n_qb + 1
 * must fit in int32 (else SA_ERR_UNSUPPORTED). */
int sa_predict_mask(const uint16_t* q, const uint16_t* k, const sa_mask_params* p,
                    void* ws, size_t ws_bytes, int32_t* row_ptr, int32_t* col_idx,
                    int64_t col_cap, uint8_t* mask_out, float* sim_q, float* sim_k,
                    int32_t* dev_status, void* stream);

/* Sparse attention forward over the CSR of kept key blocks (SpargeAttn notes,
 * section 2.1: online softmax m, l, O; section 2.3: PV skip).
 * q device bf16 [B,Hq,N,D], k and v device bf16 [B,Hkv,N,D] (permuted order),
 * o device fp32 [B,Hq,N,Dv].  row_ptr/col_idx as written by sa_predict_mask
 * (any CSR with ascending in-range columns is accepted).  For each query row:
 * the keys of its kept blocks (causal: only keys at or before it), softmax
 * with scores q.k*scale, output sum p v.  Key blocks are visited in ascending
 * order; with lambda set, for each group of SA_PV_GROUP_ROWS rows of a query
 * block, if max over the group of (block row max - new running max) < lambda,
 * the block's PV product is skipped for the group (the running sum still
 * counts it).  A row that keeps no key gets NaN and dev_status is set to
 * SA_ERR_EMPTY_ROW.  CSR entries at positions >= p->col_cap are ignored and
 * set SA_ERR_CAPACITY; a column outside [0, n_kb) is ignored and sets
 * SA_ERR_INVALID_ARGUMENT, and so does a negative row_ptr entry (its row then
 * reads no entry).  With several conditions the last one written stays.
 * Optional (NULL = not written): pv_skip device uint8 [nnz * ceil(block_q/32)]
 * (G = ceil(block_q/32) flags per CSR entry, col_cap entries)
 * with pv_skip[e*G + g] = 1 when group g skipped the PV of CSR entry e;
 * counters device int64 [3] = {QK block products, PV group-blocks executed,
 * PV group-blocks skipped}, reset by the call.
 * max(N, n_keys) * D * 2 must be below 2^31 (one head of q, k or v under
 * 2 GiB) and B*Hq*ceil(N/block_q) + 1 must fit in int32, else
 * SA_ERR_UNSUPPORTED. */
int sa_sparse_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o,
                       const sa_attn_params* p, const int32_t* row_ptr, const int32_t* col_idx,
                       uint8_t* pv_skip, int64_t* counters, int32_t* dev_status, void* stream);

/* The reorder folded into the two calls above, as an index map instead of a
 * copy (reordering is a relabelling of the tokens: "AIGC 基本功|视频稀疏注意力的
 * 误差与布局-SparseAttn", section 3.4).  q, k and v are in the ORIGINAL token
 * order; perm_dev (device int32 [N], as written by sa_plan_permutation) gives
 * position i of the reordered sequence as token perm_dev[i].
 *   sa_predict_mask_gather(q, k, perm, ...) == sa_predict_mask on
 *     q'[b,h,i,:] = q[b,h,perm[i],:], k' likewise (bf16 inputs only): the same
 *     CSR, mask and similarities, indexed by reordered blocks, bit for bit.
 *   sa_sparse_attn_fwd_gather(q, k, v, perm, o, ...) == sa_sparse_attn_fwd on
 *     q', k', v' followed by sa_unpermute: o is written in the original order,
 *     o[b,h,perm[i],:] = o'[b,h,i,:], bit for bit.
 * perm_dev must be a permutation of 0..N-1.  This is not checked; an entry
 * outside 0..N-1 never makes a kernel access memory outside q, k, v and o,
 * but the results are then unspecified.
 * One permutation serves queries and keys, so n_keys must be 0 or N (keys of
 * another length: SA_ERR_UNSUPPORTED; reorder them with sa_permute instead).
 * Other arguments, errors and outputs as in the non-gather calls; perm_dev must
 * not be NULL. */
int sa_predict_mask_gather(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                           const sa_mask_params* p, void* ws, size_t ws_bytes, int32_t* row_ptr,
                           int32_t* col_idx, int64_t col_cap, uint8_t* mask_out, float* sim_q,
                           float* sim_k, int32_t* dev_status, void* stream);
int sa_sparse_attn_fwd_gather(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* perm_dev, float* o, const sa_attn_params* p,
                              const int32_t* row_ptr, const int32_t* col_idx, uint8_t* pv_skip,
                              int64_t* counters, int32_t* dev_status, void* stream);

/* sa_predict_mask with both options in one call: perm_dev as in
 * sa_predict_mask_gather (NULL: q and k are already in the reordered order;
 * non-NULL only with n_keys 0 or N, else SA_ERR_UNSUPPORTED),
 * and forced_dev, a device uint8 [n_qb*n_kb] block pattern shared by every
 * (batch, head) (NULL: none), e.g. the tile windows of sa_plan_tile_window:
 * a nonzero entry (i, j) adds key block j to the forced blocks of query
 * block i (step 3 of sa_predict_mask; valid blocks only), so it is always
 * kept and counts toward the keep floor.  Other arguments, errors and outputs
 * as in sa_predict_mask. */
int sa_predict_mask_ex(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                       const uint8_t* forced_dev, const sa_mask_params* p, void* ws, size_t ws_bytes,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, uint8_t* mask_out,
                       float* sim_q, float* sim_k, int32_t* dev_status, void* stream);

/* Rows per K quantization block of sa_sparse_attn_fwd_qk8 (the 64-key tile). */
#define SA_FP8_KEY_ROWS 64

/* Per-block 8-bit quantization of a QK operand (SpargeAttn notes, section
 * 2.4: the sparse kernel's QK path takes Q and K quantized block by block,
 * each block with one dequantization scale).  The format is OCP FP8 E4M3
 * (bias 7, 3 mantissa bits, largest finite 448, subnormals, no infinities).
 * x: device bf16 [B,H,N,D] in the ORIGINAL token order; perm_dev: device
 * int32 [N] as for the gather calls, or NULL (identity).  Block j of each
 * (b, h) is the rows perm[j*block .. j*block+block-1] (the last block may be
 * short).  With amax = max |x| over the block (float32):
 *   scales[b,h,j] = amax / 448          (1 when amax = 0)
 *   codes[b,h,r,:] = E4M3 code nearest to clamp(x[b,h,r,:] * (448 / amax),
 *                    -448, 448), ties to even, sign kept, for every row r of
 *                    block j, written at the row's own (original) position
 * amax, both divisions and the product are IEEE float32 operations.
 * codes: device uint8 [B,H,N,D] (8-byte aligned), scales: device fp32
 * [B,H,ceil(N/block)].  D is 64 or 128 (else SA_ERR_UNSUPPORTED); block is
 * 1..128.  Q takes block = block_q, K takes block = SA_FP8_KEY_ROWS.  An
 * entry of perm_dev outside 0..N-1 makes its row take no part (nothing is
 * read or written for it). */
int sa_quantize_fp8(const uint16_t* x, const int32_t* perm_dev, int32_t B, int32_t H, int64_t N,
                    int32_t D, int32_t block, uint8_t* codes, float* scales, void* stream);

/* sa_predict_mask_ex (no forced pattern, no optional outputs) that also writes,
 * in the same pass over Q and K, what sa_quantize_fp8 writes for them with the
 * same perm_dev: q8 device uint8 [B,Hq,N,D] and q_scale device fp32
 * [B,Hq,ceil(N/block_q)] (blocks of block_q rows), k8 device uint8 [B,Hkv,N_k,D]
 * and k_scale device fp32 [B,Hkv,ceil(N_k/SA_FP8_KEY_ROWS)], bit for bit (for a
 * perm_dev that is a permutation).  The inputs of sa_sparse_attn_fwd_qk8 thus
 * come out of the mask prediction (SpargeAttn notes, sections 2.2 and 2.4: the
 * prediction and the quantized QK path read the same Q and K blocks).  Needs
 * block_q <= 128 and block_k = 64 or 128 (else SA_ERR_UNSUPPORTED); q8 and k8
 * 8-byte aligned.  Other arguments, errors and outputs as in sa_predict_mask_ex. */
int sa_predict_mask_qk8(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                        const sa_mask_params* p, void* ws, size_t ws_bytes, int32_t* row_ptr,
                        int32_t* col_idx, int64_t col_cap, uint8_t* q8, float* q_scale, uint8_t* k8,
                        float* k_scale, int32_t* dev_status, void* stream);

/* sa_sparse_attn_fwd (perm_dev NULL) or sa_sparse_attn_fwd_gather (perm_dev
 * non-NULL) with the QK products taken on FP8 operands (SpargeAttn notes,
 * section 2.4; the SageAttention idea on the gfx950 FP8 matrix cores): the
 * score of query row i and key j is
 *   (q8[i] . k8[j]) * q_scale[block of i] * k_scale[tile of j] * scale,
 * the dot product of the E4M3 values taken exactly and summed in fp32; the
 * softmax, the PV-skip rule and the P V products (v in bf16) are those of
 * sa_sparse_attn_fwd.  q8: device uint8 [B,Hq,N,D] with q_scale device fp32
 * [B,Hq,ceil(N/block_q)]; k8: device uint8 [B,Hkv,N_k,D] with k_scale device
 * fp32 [B,Hkv,ceil(N_k/SA_FP8_KEY_ROWS)], both as written by sa_quantize_fp8
 * (with the same perm_dev).  Needs D = 128, block_q = 128, block_k = 64 or
 * 128 and ceil(N_k/64) below 4096 (else SA_ERR_UNSUPPORTED).  q8 and k8 16-byte aligned.  Other arguments, errors
 * and outputs as in sa_sparse_attn_fwd / sa_sparse_attn_fwd_gather. */
int sa_sparse_attn_fwd_qk8(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                           const float* k_scale, const uint16_t* v, const int32_t* perm_dev, float* o,
                           const sa_attn_params* p, const int32_t* row_ptr, const int32_t* col_idx,
                           uint8_t* pv_skip, int64_t* counters, int32_t* dev_status, void* stream);

/* Bytes of the fixed device workspace of sa_predict_mask_gather_noalloc
 * (64 MiB, one copy per GPU for the life of the process). */
#define SA_NOALLOC_SCRATCH_BYTES (64ll << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sa_predict_mask_gather without the ws/ws_bytes arguments.  The workspace is
 * a fixed SA_NOALLOC_SCRATCH_BYTES device array inside this library (one per
 * GPU, kept until the process ends); the call allocates nothing.  Parameters
 * whose sa_predict_workspace_bytes exceeds SA_NOALLOC_SCRATCH_BYTES are refused
 * with SA_ERR_CAPACITY before anything is enqueued.  All calls on one GPU share
 * that GPU's array: calls that may run at the same time on one GPU (different
 * streams without ordering) race and must not be issued; calls ordered on one
 * stream are safe.  The first call on a device looks the array's address up
 * (a HIP runtime query, no allocation); a failure there returns SA_ERR_HIP.
 * Outputs, errors and the other arguments as in sa_predict_mask_gather. */
int sa_predict_mask_gather_noalloc(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                                   const sa_mask_params* p, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_cap, uint8_t* mask_out, float* sim_q, float* sim_k,
                                   int32_t* dev_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
