/*
 * seer.h -- C ABI of libseer, the MI355X (gfx950) decode-time hot path of
 * SeerAttention-R block-sparse attention.
 *
 * Pages cited:
 *   [CP] chapterpal.com summary page "SeerAttention-R: Sparse Attention
 *        Adaptation for Long Reasoning" (its numbered "Knowl" sections);
 *   [PN] papernotes.org ICLR 2026 notes page "Sparse Attention Adaptation
 *        for Long Reasoning" (its "key design" paragraphs).
 *
 * One decode step of one attention layer is
 *   seer_kcomp_update  -> seer_gate_scores -> seer_select_blocks
 *   -> seer_sparse_decode            (seer_dense_decode is the full baseline)
 * or the same four stages fused into two launches by seer_decode_step
 * (seer_decode_step_noalloc: the same without a workspace argument, for
 * callers that cannot allocate).  The training side has one call:
 * seer_prefill_attention, the causal prefill forward with the gate's ground
 * truth.
 *
 * Conventions shared by every call
 *   - "bf16" buffers hold raw bfloat16 bit patterns (uint16_t).
 *   - Every pointer argument is a DEVICE pointer unless marked (host); the
 *     `dims` struct is always a host pointer.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and returns as soon as its kernels are
 *     queued.  No call synchronises the host with the device.
 *   - The caller owns every buffer.  The library allocates nothing and keeps
 *     no pointer after a call returns (seer_decode_step_noalloc uses a
 *     static array of the library instead of a caller's workspace).
 *     Outputs are fully overwritten (including padding), so callers never
 *     pre-initialise them; the only exception is the decode workspace of
 *     seer_sparse_decode / seer_dense_decode (and their paged forms), which
 *     holds counters that must be zero before it is first used (every call
 *     leaves them zero again).  The fused step's workspace needs no
 *     particular contents.
 *   - Host-detectable errors return before anything is launched; nothing is
 *     written.  A kernel launch failure returns SEER_ERR_HIP.  Device-side
 *     data problems cannot be reported synchronously: out-of-range lengths
 *     are clamped to [0, max_seq_len], block indices outside
 *     [0, ceil(L/b)) are skipped, and stale cache counters are clamped.
 *   - seer_last_error_message() gives a human-readable reason for the most
 *     recent non-OK return on the calling thread.
 *
 * Tensor layouts (row-major, innermost last)
 *   q, q_nope  [B, H_q, d]            bf16, contiguous.  Query head
 *                                     hq = h*g + i belongs to KV head h
 *                                     (g = H_q / H_kv).
 *   K, V, K_nope [B, H_kv, Lmax, d]   bf16; element strides kv_stride_b,
 *                                     kv_stride_h, kv_stride_t, d contiguous.
 *                                     Token t of sequence b sits at
 *                                     b*sb + h*sh + t*st.  K is post-RoPE (the
 *                                     model's), K_nope pre-RoPE.
 *   w_q        [H_kv, d_gate, g*d]    bf16, contiguous (one W_q per KV head,
 *                                     [PN key design 1]).
 *   w_k        [H_kv, d_gate, 3*d]    bf16, contiguous; column blocks are
 *                                     [max | min | avg] ([CP Knowl 1]).
 *   kcomp      [B, H_kv, NBmax, d_gate] bf16, contiguous;
 *                                     NBmax = ceil(Lmax / b).
 *   seq_lens, kcomp_lens  [B]         int32.  seq_lens counts the current
 *                                     token.
 *   logits     [B, H_kv, NBmax]       float32, un-softmaxed block scores.
 *   block_idx  [B, H_kv, max_selected] int32, ascending, -1 padded.
 *   num_selected [B, H_kv]            int32.
 *   out        [B, H_q, d]            bf16.
 *   lse        [B, H_q]               float32 natural-log sum of exp.
 */
#ifndef SEER_H_
#define SEER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SEER_OK = 0,
  SEER_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or value   */
  SEER_ERR_UNSUPPORTED = 2, /* valid but not built: d, d_gate, b, g, NBmax  */
  SEER_ERR_WORKSPACE = 3,   /* workspace missing or too small               */
  SEER_ERR_HIP = 4          /* HIP runtime error (launch, device query)     */
};

enum { SEER_SELECT_TOPK = 1, SEER_SELECT_THRESHOLD = 2, SEER_SELECT_TOPP = 3 };
/* num_split of the decode calls: the balanced division (see seer_sparse_decode). */
enum { SEER_SPLIT_BALANCED = -1 };

typedef struct seer_dims {
  int32_t batch;        /* B >= 1                                           */
  int32_t num_q_heads;  /* H_q, a multiple of H_kv                          */
  int32_t num_kv_heads; /* H_kv >= 1; g = H_q / H_kv must be in [1, 16]      */
  int32_t head_dim;     /* d: 64 or 128                                     */
  int32_t d_gate;       /* gate width per KV head: 64 or 128                */
  int32_t block_size;   /* b: 64 or 128                                     */
  int32_t max_seq_len;  /* Lmax: KV capacity per sequence (tokens)          */
  int32_t reserved;     /* must be 0                                        */
  int64_t kv_stride_b;  /* element strides of K, V and K_nope, multiples of */
  int64_t kv_stride_h;  /* 8 (16-byte rows); kv_stride_t >= d               */
  int64_t kv_stride_t;
} seer_dims;

/*
 * seer_kcomp_update -- append K Compression Cache entries for blocks that
 * have become complete.
 *
 * [CP Knowl 5]: the cache holds K_gate per block and is updated once every b
 * new tokens by pooling the latest b keys and applying the linear layer.
 * [CP Knowl 2]: K_gate = RoPE(W_k concat[P_max, P_min, P_avg](K_nope)) with
 * kernel = stride = b pooling; [CP Knowl 1]: the RoPE position of a
 * compressed block is its first token.
 *
 * For every sequence b and KV head h, with L = seq_lens[b], nb = floor(L/b)
 * and c = kcomp_lens[b], entries j = c .. min(nb, c + max_new_blocks) - 1 are
 * computed as bf16(RoPE(W_k[h] . [max, min, mean of K_nope rows j*b ..
 * j*b+b-1], j*b)) (round to nearest even), and kcomp_lens[b] is then raised
 * to min(nb, c + max_new_blocks).  Entries already present are not touched.
 * Bulk build of a prompt: kcomp_lens = 0, max_new_blocks = NBmax.
 * Decode: max_new_blocks = 1, once per step, before seer_gate_scores.
 *
 *   k_nope      pre-RoPE keys (layout above); may alias k_cache.
 *   w_k         [H_kv, d_gate, 3d] bf16.
 *   seq_lens    [B] int32 (read).   kcomp_lens [B] int32 (read, then raised).
 *   kcomp       [B, H_kv, NBmax, d_gate] bf16 (entries written).
 *   max_new_blocks >= 1; rope_theta > 0 (RoPE base, e.g. 10000).
 * Launches two kernels; the second raises kcomp_lens after all entries are
 * written.  An out-of-range kcomp_lens[b] is clamped to [0, NBmax].
 */
int seer_kcomp_update(const seer_dims* dims, const uint16_t* k_nope,
                      const uint16_t* w_k, const int32_t* seq_lens,
                      int32_t* kcomp_lens, uint16_t* kcomp,
                      int32_t max_new_blocks, double rope_theta, void* stream);

/*
 * seer_gate_scores -- block scores of the current token against the cache.
 *
 * [CP Knowl 2]: Q_gate = RoPE(W_q reshape(Q_nope, [.., g*d])) and the scores
 * are Q_gate K_gate^T / sqrt(d_gate) (softmax not applied: [CP Knowl 5] top-k
 * runs on the un-softmaxed logits).  The query position is L-1.
 *
 * Writes logits[b, h, j] = Q_gate[b,h] . kcomp[b,h,j] / sqrt(d_gate) for
 * j < n_c = min(kcomp_lens[b], floor(L/b)), and -inf for n_c <= j < NBmax.
 * Q_gate itself ([B, H_kv, d_gate] float32) is left at the start of the
 * workspace.
 *
 *   q_nope     [B, H_q, d] bf16.   w_q [H_kv, d_gate, g*d] bf16.
 *   workspace  >= seer_gate_workspace_bytes(dims) bytes, 16-byte aligned,
 *              no initialisation needed.
 *   logits     [B, H_kv, NBmax] float32.
 */
size_t seer_gate_workspace_bytes(const seer_dims* dims);
int seer_gate_scores(const seer_dims* dims, const uint16_t* q_nope,
                     const uint16_t* w_q, const uint16_t* kcomp,
                     const int32_t* kcomp_lens, const int32_t* seq_lens,
                     double rope_theta, void* workspace, size_t workspace_bytes,
                     float* logits, void* stream);

/*
 * seer_select_blocks -- binarise block scores into active-block indices.
 *
 * [CP Knowl 5]: (1) token budget: top-k block indices by un-softmaxed logit,
 * k = ceil(budget / b) (the caller passes k); (2) threshold: blocks whose
 * softmax score exceeds tau.  The incomplete last block is selected
 * unconditionally.  [CP Knowl 6]: the index tensor is
 * [batch, heads_kv, max_selected_blocks].
 *
 * With n_c = min(kcomp_lens[b], floor(L/b)) scored blocks and
 * N = ceil(L/b) blocks in all:
 *   TOPK:      the min(k, n_c) largest logits; equal logits go to the lower
 *              index.
 *   THRESHOLD: the j < n_c with logits[j] > ln(tau) + logsumexp(logits[0..n_c))
 *              (softmax_j > tau, strict), evaluated in float32.
 *   TOPP:      the shortest run of the blocks in descending logit order
 *              (equal logits: lower index first) whose softmax mass reaches
 *              p ([CP Knowl 14] names top-p as the adaptive-sparsity
 *              direction).  Each block's mass is rounded to a multiple of
 *              2^-30 (float32 softmax); the run ends at the first block where
 *              the running mass reaches ceil(p * 2^30) units.  p = 0 selects
 *              no scored block; a p the total does not reach selects all.
 * plus every block in [n_c, N) (normally only the partial block).  Indices
 * are written ascending, -1 after the last; num_selected gets the count.
 * The blocks of [n_c, N) come first when the row is short (possible only in
 * TOPK, when the cache lags so that more than one block is unscored): the
 * last min(N - n_c, max_selected) of them are kept -- the partial block is
 * always among them -- and k shrinks to the room left in the row.
 *
 *   mode            SEER_SELECT_TOPK (uses topk_blocks >= 0),
 *                   SEER_SELECT_THRESHOLD (uses 0 <= threshold <= 1) or
 *                   SEER_SELECT_TOPP (threshold is the mass p, 0..1).
 *   max_selected    capacity per (b, h): TOPK needs
 *                   >= min(topk_blocks + 1, NBmax), THRESHOLD and TOPP need
 *                   >= NBmax.
 *   NBmax <= 8192 (SEER_ERR_UNSUPPORTED otherwise).
 */
int seer_select_blocks(const seer_dims* dims, const float* logits,
                       const int32_t* kcomp_lens, const int32_t* seq_lens,
                       int32_t mode, int32_t topk_blocks, float threshold,
                       int32_t max_selected, int32_t* block_idx,
                       int32_t* num_selected, void* stream);

/*
 * Decode workspace: one completion counter per (b, h) followed by the
 * per-split partial results (lse and output of each split of each (b, h));
 * 0 bytes when the call uses one split.  `max_blocks` is max_selected
 * (sparse) or NBmax (dense); `num_split` 0 means "choose automatically"
 * and SEER_SPLIT_BALANCED the balanced division of seer_sparse_decode (both
 * query the current device; the balanced size includes the stream-K
 * partials where that division applies).
 * The counters must be ZERO before the first call that uses a workspace;
 * every call leaves them zero again, so one zero-fill at allocation is
 * enough while the workspace serves calls of at most as many (b, h) pairs
 * as the first (the counters are the first B * H_kv words; a call with
 * more pairs finds partial results there: zero it again first).  One
 * workspace must not be used by two calls that can run at the same time.
 */
size_t seer_decode_workspace_bytes(const seer_dims* dims, int32_t max_blocks,
                                   int32_t num_split);
/* The same size under the name of the boundary's outline: bytes of the
 * workspace of seer_sparse_decode / seer_dense_decode for max_blocks and
 * num_split, exactly seer_decode_workspace_bytes(dims, max_blocks,
 * num_split). */
size_t seer_workspace_bytes(const seer_dims* dims, int32_t max_blocks, int32_t num_split);

/* The split count a decode call will use (resolves num_split = 0 and
 * SEER_SPLIT_BALANCED to the automatic count). */
int seer_decode_num_split(const seer_dims* dims, int32_t max_blocks,
                          int32_t num_split, int32_t* num_split_out /* host */);

/*
 * seer_sparse_decode -- block-sparse flash decoding over the active blocks.
 *
 * [CP Knowl 6]: grid (batch, heads_kv, num_split); the work of each
 * (b, h) is split along num_split from its list of active blocks, the kernel
 * loops only over active indices and skips invalid entries; [PN key design
 * 4] same.  With more than one split, the last split of each (b, h) to
 * finish merges the splits by log-sum-exp in the same launch.
 *
 * For each query head hq = h*g + i of sequence b: over the tokens
 * T = union over the first num_selected[b,h] entries j of block_idx[b,h] with
 * 0 <= j < ceil(L/b) of [j*b, min(j*b+b, L)),
 *   out[b,hq] = sum_t softmax_T(scale * q.K_t) V_t   (bf16, round to nearest)
 *   lse[b,hq] = ln sum_T exp(scale * q.K_t)          (float32; may be NULL)
 * An empty T gives out = 0 and lse = -inf.
 *
 *   q          [B, H_q, d] post-RoPE bf16.   k_cache, v_cache: layout above.
 *   block_idx  [B, H_kv, max_selected], num_selected [B, H_kv] (as written
 *              by seer_select_blocks; indices must not repeat).
 *   scale      usually 1/sqrt(d).   num_split 0 = automatic, 1 .. 128 as
 *              given, or SEER_SPLIT_BALANCED: the division the fused step
 *              gives threshold and top-p selections, whose pairs keep
 *              different numbers of blocks -- with fewer (b, h) pairs than
 *              compute units, all pairs' chunks divided evenly over the grid
 *              (stream-K; the same bits as the fused step), otherwise the
 *              automatic split count.  The paged and dense calls take it as
 *              0.
 *   workspace  >= seer_decode_workspace_bytes(dims, max_selected, num_split)
 *              bytes, 256-byte aligned, counters zero (see above); may be
 *              NULL when that size is 0.  A balanced call given only the
 *              fixed-split size runs fixed splits.
 */
int seer_sparse_decode(const seer_dims* dims, const uint16_t* q,
                       const uint16_t* k_cache, const uint16_t* v_cache,
                       const int32_t* seq_lens, const int32_t* block_idx,
                       const int32_t* num_selected, int32_t max_selected,
                       float scale, int32_t num_split, void* workspace,
                       size_t workspace_bytes, uint16_t* out, float* lse,
                       void* stream);

/*
 * seer_dense_decode -- the full-attention decode baseline: the same kernel
 * over every block 0 .. ceil(L/b)-1 (the role FlashAttention-3 plays in
 * [CP Knowl 9]).  Arguments as seer_sparse_decode; the workspace is sized
 * with max_blocks = NBmax.
 */
int seer_dense_decode(const seer_dims* dims, const uint16_t* q,
                      const uint16_t* k_cache, const uint16_t* v_cache,
                      const int32_t* seq_lens, float scale, int32_t num_split,
                      void* workspace, size_t workspace_bytes, uint16_t* out,
                      float* lse, void* stream);

/*
 * seer_sparse_decode_paged / seer_dense_decode_paged -- the decodes above on
 * a paged KV cache.
 *
 * [CP Knowl 14] names PagedAttention support as needed for serving.  The
 * cache is a pool of pages of b tokens (one block per page); logical block j
 * of sequence b lives in page block_table[b * table_stride + j].  Only where
 * a block's rows are read changes; results are bit-identical to the
 * contiguous call on the same rows.
 *
 *   k_pages, v_pages  page pools, bf16: row t (0 <= t < b) of head h in page
 *                     p starts at element p*page_stride + h*page_head_stride
 *                     + t*dims.kv_stride_t and holds d contiguous values
 *                     (e.g. [num_pages, H_kv, b, d]: page_head_stride = b*d,
 *                     page_stride = H_kv*b*d, kv_stride_t = d).
 *                     dims.kv_stride_b and kv_stride_h are not used.
 *   num_pages         pages in the pool; a block whose page is outside
 *                     [0, num_pages) is skipped like an invalid index entry.
 *   block_table       [B, table_stride] int32 (device); entries of blocks
 *                     0 .. ceil(L/b)-1 are read (a block >= table_stride is
 *                     skipped).
 * Strides are in elements, multiples of 8.  Everything else as
 * seer_sparse_decode / seer_dense_decode.
 */
int seer_sparse_decode_paged(const seer_dims* dims, const uint16_t* q, const uint16_t* k_pages,
                             const uint16_t* v_pages, int64_t page_stride,
                             int64_t page_head_stride, int32_t num_pages,
                             const int32_t* block_table, int32_t table_stride,
                             const int32_t* seq_lens, const int32_t* block_idx,
                             const int32_t* num_selected, int32_t max_selected, float scale,
                             int32_t num_split, void* workspace, size_t workspace_bytes,
                             uint16_t* out, float* lse, void* stream);
int seer_dense_decode_paged(const seer_dims* dims, const uint16_t* q, const uint16_t* k_pages,
                            const uint16_t* v_pages, int64_t page_stride, int64_t page_head_stride,
                            int32_t num_pages, const int32_t* block_table, int32_t table_stride,
                            const int32_t* seq_lens, float scale, int32_t num_split,
                            void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                            void* stream);

/*
 * seer_decode_step -- one whole decode step of one layer in two launches,
 * with the same results as seer_kcomp_update (with max_new_blocks), then
 * seer_gate_scores, seer_select_blocks and seer_sparse_decode, in that order
 * ([CP Knowl 5]: cache update, gating and binarisation; [CP Knowl 6]: the
 * block-sparse decode).
 *
 * Launch 1 runs one workgroup per (b, h): the cache entries of blocks
 * completed since the last update (up to 4; with max_new_blocks > 4 a
 * staged cache update runs before it), the gate query, the block scores and
 * the selection.  Launch 2 is the sparse decode with its split merge, whose
 * first workgroup also raises kcomp_lens -- so kcomp_lens keeps its old
 * value until then and nothing else may read it in between.
 *
 * Under SEER_SELECT_THRESHOLD and SEER_SELECT_TOPP the pairs keep different
 * numbers of blocks.  With num_split = 0 (or SEER_SPLIT_BALANCED), fewer
 * (b, h) pairs than compute units, and a workspace of at least
 * seer_decode_step_workspace_bytes(dims, max_selected, 0), launch 2 then
 * divides all pairs' selected chunks evenly over its grid (stream-K)
 * instead of splitting each pair num_split ways -- the division
 * seer_sparse_decode gives with SEER_SPLIT_BALANCED, with the same bits.
 * The result equals the split decode up to summation order (the same
 * tolerance to the exact attention), and is the same from run to run.
 *
 *   q_nope, q        [B, H_q, d] pre-/post-RoPE queries (may alias).
 *   k_nope, k_cache, v_cache  caches (layout above; k_nope may alias k_cache).
 *   w_q, w_k         gate weights.   seq_lens [B] includes the current token.
 *   kcomp_lens, kcomp  the cache (updated in place).  max_new_blocks >= 0
 *                    (0: no update, e.g. when the caller keeps it current).
 *   mode, topk_blocks, threshold, max_selected  as seer_select_blocks.
 *   block_idx, num_selected  the selection (outputs).
 *   logits           [B, H_kv, NBmax] float32 block scores, or NULL to skip
 *                    writing them.
 *   scale, num_split as seer_sparse_decode.
 *   workspace        >= seer_decode_step_workspace_bytes(dims, max_selected,
 *                    num_split) bytes, 256-byte aligned, no initial contents
 *                    needed: the gate queries (rounded up to 256 bytes), then
 *                    the decode workspace, whose split counters launch 1
 *                    zeroes.  One workspace may serve calls of any sizes.
 *                    With num_split = 0 or SEER_SPLIT_BALANCED the size
 *                    includes the stream-K decode's per-workgroup
 *                    partials; a workspace sized for
 *                    the split decode alone is still accepted (no stream-K).
 *   out, lse         as seer_sparse_decode.
 */
size_t seer_decode_step_workspace_bytes(const seer_dims* dims, int32_t max_selected,
                                        int32_t num_split);
int seer_decode_step(const seer_dims* dims, const uint16_t* q_nope, const uint16_t* q,
                     const uint16_t* k_nope, const uint16_t* k_cache,
                     const uint16_t* v_cache, const uint16_t* w_q, const uint16_t* w_k,
                     const int32_t* seq_lens, int32_t* kcomp_lens, uint16_t* kcomp,
                     int32_t max_new_blocks, double rope_theta, int32_t mode,
                     int32_t topk_blocks, float threshold, int32_t max_selected,
                     int32_t* block_idx, int32_t* num_selected, float* logits,
                     float scale, int32_t num_split, void* workspace,
                     size_t workspace_bytes, uint16_t* out, float* lse, void* stream);

/*
 * seer_decode_step_noalloc -- seer_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and results, without
 * the workspace.  The library keeps the workspace in a static device array
 * of 16 MiB (SEER_NOALLOC_SCRATCH_BYTES), one per GPU, held until the
 * process ends; the call itself allocates nothing.
 *
 *   The step's workspace is seer_decode_step_workspace_bytes(dims,
 *   max_selected, num_split) bytes, exactly what a caller of
 *   seer_decode_step would size, so both calls take the same path and give
 *   bit-identical results.  A step that needs more than the array holds
 *   returns SEER_ERR_WORKSPACE before any launch.
 *
 *   The first call on a device takes the array's device address (a host
 *   query, no launch).  The array needs no particular contents: as in
 *   seer_decode_step, the gate launch zeroes the decode's split counters.
 *
 *   Every call on one GPU uses that GPU's one array, which keeps the last
 *   call's contents: calls that overlap on one GPU (other streams, other
 *   threads, graphs replayed concurrently) race on it and must be ordered
 *   by the caller.
 */
#define SEER_NOALLOC_SCRATCH_BYTES (16u << 20)
int seer_decode_step_noalloc(const seer_dims* dims, const uint16_t* q_nope, const uint16_t* q,
                             const uint16_t* k_nope, const uint16_t* k_cache,
                             const uint16_t* v_cache, const uint16_t* w_q, const uint16_t* w_k,
                             const int32_t* seq_lens, int32_t* kcomp_lens, uint16_t* kcomp,
                             int32_t max_new_blocks, double rope_theta, int32_t mode,
                             int32_t topk_blocks, float threshold, int32_t max_selected,
                             int32_t* block_idx, int32_t* num_selected, float* logits,
                             float scale, int32_t num_split, uint16_t* out, float* lse,
                             void* stream);

/*
 * seer_prefill_attention -- causal prefill attention of whole sequences (a
 * FlashAttention-2 forward) and, optionally, the block-level ground truth
 * that the AttnGate is distilled towards ([CP Knowl 3]): the attention map
 * max-pooled over keys in blocks of b, max-pooled over the g query heads of
 * each KV head, normalised to sum to 1 per query.  The ground truth is
 * formed from each key tile's row maximum of the scores, stored during the
 * forward and rescaled by the row's final max and normaliser afterwards
 * ([CP Knowl 4]); the O(L^2) map is never built.
 *
 * The queries of sequence b are its tokens 0 .. L-1 (L = seq_lens[b],
 * clamped to [0, Lmax]); query t attends keys 0 .. t.
 *   q        [B, H_q, Lmax, d] bf16, contiguous.
 *   k, v     [B, H_kv, Lmax, d] bf16 with the dims strides (as K, V above).
 *   scale    softmax scale (1/sqrt(d)), finite and > 0.
 *   workspace >= seer_prefill_workspace_bytes(dims) bytes, 256-byte aligned,
 *            no initial contents needed: V transposed, then the stored row
 *            maxima ([B, H_q, NBmax, Lmax rounded up to 64] float32).
 *   out      [B, H_q, Lmax, d] bf16: attention output of rows t < L.
 *   lse      [B, H_q, Lmax] float32: natural-log normaliser of rows t < L
 *            (required).
 *   gt       [B, H_kv, Lmax, NBmax] float32 ground truth of rows t < L
 *            (blocks after the row's own are 0), or NULL for attention only.
 * Rows t >= L of out, lse and gt are left untouched.  d, b and g as above.
 */
size_t seer_prefill_workspace_bytes(const seer_dims* dims);
int seer_prefill_attention(const seer_dims* dims, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* seq_lens, float scale,
                           void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                           float* gt, void* stream);

/* Host-only helpers. */
const char* seer_status_string(int status);
const char* seer_last_error_message(void);
const char* seer_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEER_H_ */
