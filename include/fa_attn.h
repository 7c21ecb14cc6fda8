/*
 * fa_attn.h -- C ABI of the exact-attention library (libfa_attn.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * The library computes exact scaled dot-product attention
 *
 *     O = softmax(scale * Q K^T) V,     LSE_i = ln sum_j exp(scale * q_i . k_j)
 *
 * over visible keys j, without ever writing the N x N score or probability
 * matrix to device memory: query blocks stay resident on chip while key/value
 * tiles stream past, and each query row carries a running maximum, denominator
 * and unnormalised numerator that are rescaled whenever a later tile raises
 * the maximum ("Flash Attention: IO-Aware Exact Attention", sections "Online
 * softmax makes tiling exact" and "Loop order changes which data is
 * reloaded"; Road to Intelligence "FlashAttention", section "The trick that
 * makes tiling possible").
 *
 * Layout.  Every tensor argument is a dense, contiguous [B][H][N][d] array of
 * the element type ``dtype`` (d innermost; d_v = d), 16-byte aligned, resident
 * in device memory of the current HIP device, except in the *_strided calls,
 * which take element strides for the batch, head and row axes.  ``lse`` is
 * always a dense [B][H][N] float array.
 *
 * Ownership.  All pointers belong to the caller; the library never allocates,
 * frees or retains them.  Its only mutable global state is the fixed scratch
 * array of attn_bwd_noalloc (one copy per GPU) and the table of its device
 * addresses.  ``o`` must not overlap q, k or v.
 *
 * Streams and errors.  Work is enqueued on ``stream`` (a hipStream_t; NULL is
 * the default stream) and the call returns without waiting.  Every argument
 * check happens before anything is enqueued and returns a status code; no call
 * throws or prints.  A fault while the kernel runs is reported by the HIP
 * runtime at the caller's next synchronisation.  FA_ERR_HIP means a launch was
 * rejected by the runtime (hipGetLastError).
 */
#ifndef FA_ATTN_H
#define FA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, o (and of dout, dq, dk, dv in the backward). */
enum fa_dtype { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 };

/* FA_MASK_CAUSAL: key j is visible to query i iff j <= i (lower-triangular
 * mask filled with -inf before the softmax, as in nanoGPT's manual attention
 * on "FlashAttention -- the same attention, made memory-aware", section 00). */
enum fa_mask { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1 };

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  FA_ERR_SHAPE = 2,       /* B, H or N < 1, an element count overflows, or one head spans >= 2 GiB */
  FA_ERR_DTYPE = 3,       /* dtype is not one of enum fa_dtype                  */
  FA_ERR_MASK = 4,        /* mask is not one of enum fa_mask                    */
  FA_ERR_SCALE = 5,       /* scale is NaN or infinite                           */
  FA_ERR_UNSUPPORTED = 6, /* head dimension or variant not built (see each call) */
  FA_ERR_WORKSPACE = 7,   /* backward workspace missing or too small            */
  FA_ERR_HIP = 8,         /* the HIP runtime rejected a launch                  */
  FA_ERR_ALIGN = 9,       /* a tensor pointer is not 16-byte aligned            */
  FA_ERR_WINDOW = 10,     /* sliding window < 1                                 */
  FA_ERR_STRIDE = 11,     /* a stride is unusable (see attn_fwd_strided)        */
  FA_ERR_SCRATCH = 12     /* the problem exceeds attn_bwd_noalloc's fixed scratch */
};

/*
 * attn_fwd -- forward pass.
 *
 *   q, k, v  [B][H][N][d] inputs of type dtype.
 *   o        [B][H][N][d] output of type dtype: O = P V with P the row softmax of
 *            scale * Q K^T (masked), accumulated in fp32 and rounded to nearest
 *            even once at the end.
 *   lse      [B][H][N] fp32 output, the natural-log log-sum-exp of each row's
 *            scaled, masked scores (the normalisation statistic the backward
 *            pass recomputes probabilities from: "Flash Attention: IO-Aware
 *            Exact Attention", section "Storage, arithmetic and IO are
 *            separate quantities").  May be NULL, in which case it is not
 *            written.
 *   B, H, N  batch, heads, sequence length (queries and keys), each >= 1.
 *   d        head dimension of q, k and v: 64, 96, 128 or 256.  d = 256
 *            takes FA_F16 or FA_BF16 (FA_ERR_UNSUPPORTED for FA_F32) and
 *            runs a kernel of its own: one workgroup per CU that keeps the
 *            256-wide accumulators of 128 queries in registers.  The
 *            key/value-outer call returns FA_ERR_UNSUPPORTED for d = 256;
 *            attn_bwd, attn_bwd_strided, the sliding-window, the
 *            block-sparse and the d_v != d calls take it.
 *   mask     enum fa_mask.
 *   scale    finite multiplier of the raw dot products (any sign; usually
 *            1/sqrt(d)).
 *   dtype    enum fa_dtype.
 *   stream   hipStream_t to enqueue on, or NULL.
 *
 * The result is deterministic: the same inputs give bitwise the same outputs.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d,
             int mask, float scale, int dtype, void* stream);

/*
 * attn_fwd_window -- forward pass with a causal sliding window.
 *
 * As attn_fwd with mask = FA_MASK_CAUSAL, except that key j is visible to
 * query i iff i - window < j <= i: each query sees the `window` most recent
 * keys, its own position included.  Key tiles wholly outside every window of
 * a query block are skipped, the way causal attention skips the tiles above
 * the diagonal ("Flash Attention: IO-Aware Exact Attention", section
 * "Storage, arithmetic and IO are separate quantities": blocks that are
 * skipped change which pairs are computed).
 *
 *   window   >= 1; window >= N is plain causal attention.  FA_ERR_WINDOW
 *            if window < 1.
 *   other arguments as for attn_fwd; lse is the log-sum-exp over the window.
 */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t H, int64_t N, int64_t d, int64_t window,
                    float scale, int dtype, void* stream);

/*
 * attn_bwd -- backward pass by recomputation.
 *
 * Gradients of L = sum(O * dout) with respect to q, k and v for the forward
 * pass above.  No N x N matrix is stored or read: score and probability tiles
 * are recomputed from q, k and the forward's lse ("Flash Attention: IO-Aware
 * Exact Attention", section "Storage, arithmetic and IO are separate
 * quantities"; Road to Intelligence "FlashAttention", section "The trick that
 * makes tiling possible").  With P = exp(scale q k^T - lse):
 *     dv = P^T dout,  dP = dout v^T,  dS = P * (dP - rowsum(P * dP)),
 *     dq = scale dS k,  dk = scale dS^T q.
 *
 *   q, k, v, dout     [B][H][N][d] inputs of type dtype.
 *   o                 [B][H][N][d] forward output of type dtype.  The row
 *                     term D_i = sum_j P_ij dP_ij (= dout_i . o_i in exact
 *                     arithmetic) is formed from the recomputed P and dP in
 *                     fp32, which keeps o's rounding out of dS.  For
 *                     d = d_v <= 128 under plain and window masks the dq
 *                     kernel also reads o: it accumulates dq with the
 *                     estimate dout_i . o_i and corrects it with the exact D
 *                     at the end, so o moves only the rounding of dq, not its
 *                     value in exact arithmetic.  The other paths check o but
 *                     do not read it.
 *   lse               [B][H][N] fp32 natural-log log-sum-exp returned by
 *                     attn_fwd for the same q, k, v, mask and scale.
 *   dq, dk, dv        [B][H][N][d] outputs of type dtype (must not overlap the
 *                     inputs or each other).
 *   workspace         device memory of at least attn_bwd_workspace_bytes()
 *                     bytes, 16-byte aligned, owned by the caller; its
 *                     contents are scratch on return.
 *   mask, scale, B, H, N, d, stream: as for attn_fwd (d = 256 runs the
 *                     two-pass kernels at one workgroup per CU).
 *   dtype             FA_F16 or FA_BF16 (FA_F32 returns FA_ERR_UNSUPPORTED).
 *
 * Deterministic: no atomics are used.  FA_ERR_WORKSPACE if workspace is NULL
 * or too small.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int64_t B, int64_t H, int64_t N, int64_t d,
             int mask, float scale, int dtype, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * attn_bwd_window -- backward pass of attn_fwd_window.
 *
 * As attn_bwd with mask = FA_MASK_CAUSAL and the sliding window of
 * attn_fwd_window; lse must come from attn_fwd_window with the same window.
 * FA_ERR_WINDOW if window < 1.
 */
int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv,
                    int64_t B, int64_t H, int64_t N, int64_t d, int64_t window,
                    float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.
 *
 * Same arguments, results and errors as attn_bwd (all mask, scale, dtype and
 * head-dimension rules included; the gradients are bitwise those of attn_bwd),
 * except that the scratch attn_bwd takes from `workspace` lives in a fixed
 * array of 8 MiB inside the library, so B * H * N may not exceed
 * attn_bwd_noalloc_max_rows() = 1,048,576 query rows (FA_ERR_SCRATCH
 * otherwise).  The call allocates nothing.  Each GPU holds its own copy of
 * the array from the first call on it until the process ends, and every call
 * on that GPU uses it: calls that overlap in time on one GPU (other streams,
 * other threads) race on it and must be serialised by the caller.  Nothing in
 * it needs to start at zero: every scratch value the kernels read is written
 * earlier in the same call.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int64_t B, int64_t H, int64_t N, int64_t d,
                     int mask, float scale, int dtype, void* stream);

/* Largest B * H * N that attn_bwd_noalloc accepts. */
size_t attn_bwd_noalloc_max_rows(void);

/* Bytes of workspace attn_bwd needs for these sizes (8 * B * H * N today);
 * 0 if the sizes, d or dtype are invalid. */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

/*
 * attn_fwd_strided -- attn_fwd on strided views.
 *
 * q, k and v, and o, are [B][H][N][d] views whose d elements are contiguous,
 * with element strides {batch, head, row} given by q_strides (q), kv_strides
 * (k and v) and o_strides (o): host arrays of three int64_t, read during the
 * call.  A dense [B][H][N][d] tensor has {H*N*d, N*d, d}; a [B][N][H][d] one
 * {N*H*d, d, H*d}; q, k and v sliced out of one packed [B][N][3][H][d] tensor
 * share {N*3*H*d, d, 3*H*d}.  A head stride of 0 in kv_strides shares one k
 * and one v head among all query heads (multi-query attention).  The pages'
 * interface takes (B, nh, T, hs) tensors ("FlashAttention -- the same
 * attention, made memory-aware", section 00); these strides describe such
 * tensors, transposed or packed, without a copy.
 *
 *   strides    every stride >= 0 and a multiple of 16 bytes; the row stride
 *              >= d; one head's rows span < 2 GiB.  Output rows must not
 *              overlap (ordered by stride, each dimension of extent > 1 steps
 *              past what the smaller ones cover).  FA_ERR_STRIDE otherwise,
 *              FA_ERR_NULL if an array is NULL.
 *   lse        dense [B][H][N] fp32, may be NULL.
 *   other arguments and errors as for attn_fwd.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d,
                     const int64_t* q_strides, const int64_t* kv_strides, const int64_t* o_strides,
                     int mask, float scale, int dtype, void* stream);

/*
 * attn_bwd_strided -- attn_bwd on strided views: q, k, v, o and dout share
 * in_strides, dq, dk and dv share grad_strides (strides as for
 * attn_fwd_strided; the gradient layout must not overlap, so k and v cannot
 * be broadcast here).  lse is the dense [B][H][N] array of the forward; the
 * workspace is as for attn_bwd.
 */
int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int64_t B, int64_t H, int64_t N, int64_t d,
                     const int64_t* in_strides, const int64_t* grad_strides,
                     int mask, float scale, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * attn_fwd_dv -- forward pass with values of another width than the keys.
 *
 * As attn_fwd, except that v and o are dense [B][H][N][dv] arrays while q and
 * k are [B][H][N][d]: the pages define V as N x d_v ("Flash Attention:
 * IO-Aware Exact Attention", section "Why intermediate matrices cost memory
 * traffic"), and the scores only need q and k to share d.  Supported
 * (d, dv): d and dv in {64, 96, 128, 256} (dv == d runs the attn_fwd
 * kernels; a pair with a 256-wide side runs the d = 256 kernel and takes
 * FA_F16 or FA_BF16 only); FA_ERR_UNSUPPORTED for other pairs, FA_ERR_SHAPE
 * for dv < 1.
 */
int attn_fwd_dv(const void* q, const void* k, const void* v, void* o, float* lse,
                int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
                int mask, float scale, int dtype, void* stream);

/*
 * attn_bwd_dv -- backward pass of attn_fwd_dv.
 *
 * As attn_bwd, except that v, o, dout and dv are dense [B][H][N][d_v] arrays
 * while q, k, dq and dk are [B][H][N][d].  In the gradients of attn_bwd,
 * dP = dout v^T and dv = P^T dout contract or produce d_v columns, while the
 * recomputed S = q k^T, dq = scale dS k and dk = scale dS^T q stay over d
 * (V is N x d_v in "Flash Attention: IO-Aware Exact Attention", section "Why
 * intermediate matrices cost memory traffic").  Supported
 * (d, d_v): d and d_v in {64, 96, 128, 256} (d_v == d runs the attn_bwd
 * kernels);
 * FA_ERR_UNSUPPORTED for other pairs and for FA_F32, FA_ERR_SHAPE for
 * d_v < 1.  The workspace is as for attn_bwd (attn_bwd_workspace_bytes).
 */
int attn_bwd_dv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv,
                int64_t B, int64_t H, int64_t N, int64_t d, int64_t d_v,
                int mask, float scale, int dtype, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * attn_fwd_block_sparse -- forward pass with a block-sparse mask.
 *
 * As attn_fwd, except that key j is visible to query i only if the mask
 * block of (query block i / 64, key block j / 64) is nonzero (and, with
 * FA_MASK_CAUSAL, also j <= i).  Key tiles that no query of a block of 256
 * rows may see are not read or computed at all, the way causal attention
 * skips the tiles above the diagonal ("Flash Attention: IO-Aware Exact
 * Attention", section "Storage, arithmetic and IO are separate quantities":
 * blocks that are skipped change which pairs are computed).  A row that
 * sees no key at all gets O = 0 and LSE = -inf.
 *
 *   block_mask    device uint8 array [mask_batches][mask_heads][nb][nb],
 *                 nb = ceil(N / 64), dense; nonzero = visible.
 *   mask_batches  1 (one pattern for all batches) or B; FA_ERR_SHAPE else.
 *   mask_heads    1 (one pattern for all heads) or H; FA_ERR_SHAPE else.
 *   N             at most 2048 * 64 = 131072 (FA_ERR_UNSUPPORTED above).
 *   other arguments and errors as for attn_fwd; FA_ERR_NULL if block_mask
 *   is NULL.
 */
int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          const uint8_t* block_mask, int64_t mask_batches, int64_t mask_heads,
                          int mask, float scale, int dtype, void* stream);

/*
 * attn_bwd_block_sparse -- backward pass of attn_fwd_block_sparse: as attn_bwd
 * with the block mask of the forward (same block_mask, mask_batches,
 * mask_heads and mask).  Tiles hidden from every block of a workgroup are
 * skipped; rows that saw no key get dq = 0, keys no query saw get
 * dk = dv = 0.
 *
 * The workspace must hold attn_bwd_block_sparse_workspace_bytes() bytes
 * (FA_ERR_WORKSPACE otherwise): besides attn_bwd's per-query terms, a counter
 * per 128 keys and fp32 partial dK and dV of up to four chunks per key.  A
 * key block that many query tiles see (a global block) has its tiles split
 * over up to four workgroups of at least 32 tiles each; the last of them to
 * finish adds the partials in chunk order, so the result is still the same
 * bits on every call.  Calls that share a workspace must not overlap.
 */
size_t attn_bwd_block_sparse_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

int attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          const uint8_t* block_mask, int64_t mask_batches, int64_t mask_heads,
                          int mask, float scale, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * attn_fwd_kv_outer -- the same forward pass in the original key/value-outer
 * loop order, for comparing the two orders' memory traffic.
 *
 * "Flash Attention: IO-Aware Exact Attention", section "Loop order changes
 * which data is reloaded": the original algorithm keeps one key/value block
 * on chip and visits every query block under it, reloading Q and the row
 * state and writing the updated state back for each key/value block.  The
 * update is the normalised one of "FlashAttention -- the same attention, made
 * memory-aware", sections 03 and 04.  One workgroup per (batch, head) walks
 * the key/value tiles; its row state (O, running maximum, denominator) lives
 * in fp32 in the workspace between tiles.  Results equal attn_fwd's up to
 * rounding; attn_fwd is the fast path.
 *
 *   arguments     as for attn_fwd; dtype FA_F16 or FA_BF16
 *                 (FA_ERR_UNSUPPORTED for FA_F32).
 *   workspace     device memory of at least
 *                 attn_fwd_kv_outer_workspace_bytes() bytes, 16-byte aligned,
 *                 owned by the caller (FA_ERR_WORKSPACE if NULL or smaller).
 *                 Overwritten; calls that share one workspace must be
 *                 ordered on one stream.
 */
int attn_fwd_kv_outer(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t N, int64_t d,
                      int mask, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace attn_fwd_kv_outer needs: (4 * d + 8) * B * H * N; 0 if
 * the sizes, d or dtype are invalid or dtype is FA_F32. */
size_t attn_fwd_kv_outer_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_str(int status);

/* Version of this ABI; bumped on any incompatible change. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_ATTN_H */
