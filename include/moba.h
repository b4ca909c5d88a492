/*
 * moba.h - C ABI of libmoba.so: MoBA (Mixture of Block Attention) on MI355X (gfx950),
 * the prefill forward with its backward, packed sequences, dense and decode paths.
 *
 * MoBA (Mixture of Block Attention): the keys of a sequence are cut into blocks of
 * `block` tokens, each block is mean-pooled into a centroid, every query is scored
 * against the centroids of its causal past by inner product and routed to its top-k
 * blocks, its own current block always among them, and causal softmax attention runs
 * over the selected blocks only ("MoBA: Mixture of Block Attention for Long-Context
 * LLMs", paper summary page on atlas.scime.ai, section "Approach"; MoBA README,
 * intro bullets "Trainable Block Sparse Attention" and "Parameter-less Gating
 * Mechanism").  The library splits that attention into the history blocks and the
 * causal current block; the current-block kernel merges the two by log-sum-exp as it
 * writes the output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers named q, k, v, out, centroids, idx, list_offsets, entries, workspace are
 * DEVICE pointers (hipMalloc'd or torch CUDA tensors); `stream` is a hipStream_t
 * (NULL = the default stream).  All device work is enqueued on `stream` and the call
 * returns without synchronising.  The caller owns every buffer; the library allocates
 * no device memory and keeps no state between calls, so calls on different streams
 * with separate buffers may run concurrently.  Calls that share a workspace must be
 * ordered on one stream.  No entry point calls a HIP memset, copy, allocation or
 * synchronisation, and every workspace word a kernel reads is written earlier in the
 * same call, so a call may be captured into a HIP graph (hipStreamBeginCapture on
 * `stream`) and replayed; the _profile and _timed forms record events and the
 * _profile form synchronises, so only the plain forms are meant for capture.
 *
 * Layouts (contiguous, row-major; b = batch, T = seqlen, d = head_dim,
 * nb = ceil(T / block), G = hq / hkv, query head h reads kv-head h / G):
 *   q, out       [b, T, hq, d]   bfloat16
 *   k, v         [b, T, hkv, d]  bfloat16
 *   lse          [b, hq, T]      float32, natural log of the softmax denominator
 *   idx          [b, hq, T, topk] int32: the selected blocks of each query in
 *                ascending order (so the current block is the last valid one), then
 *                -1 padding when fewer than topk blocks are causal
 *   centroids    [b, hkv, nb, d] float32
 *
 * Supported shapes: head_dim 64 or 128; hq % hkv == 0; block >= 16 and a multiple of
 * 16; scale finite and > 0; batch * seqlen * hq < 2^31; topk >= 1 (topk counts the
 * current block).  seqlen need not be a multiple of block: the last block is then
 * partial.  It is only ever a current block (no later token routes to it), so routing
 * is unchanged; its centroid is the mean of the keys present.
 *   topk >= nb: every row selects every causal block, so the layer is dense causal
 *     attention (README bullet "Seamlessly Transition between Full and Sparse
 *     Attention"); any such topk is accepted, idx lists blocks 0 .. c then -1, and the
 *     library runs the dense kernel without gate, index or workspace.
 *   topk < nb: at most 64 history slots (topk <= 65), at most 8192 blocks, and
 *     seqlen * G < 2^27 (2^26 with more than 32 history slots).
 * Anything else returns MOBA_ERR_UNSUPPORTED or MOBA_ERR_INVALID_ARG before any device
 * work.
 *
 * Errors: every check runs on the host before the first launch, so a call that
 * returns an error has written nothing.  MOBA_ERR_HIP means a launch failed; the
 * outputs are then undefined.  No entry point aborts or throws.
 */
#ifndef MOBA_H
#define MOBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOBA_OK = 0,
  MOBA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, hq % hkv != 0 ... */
  MOBA_ERR_UNSUPPORTED = -2, /* valid MoBA shape this library does not run */
  MOBA_ERR_WORKSPACE = -3,   /* workspace smaller than the minimum */
  MOBA_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} moba_status;

/* Validates a problem shape on the host (touches no device): the block partition, the
 * top-k routing with the current block counted, and the grouped query heads that
 * moba_forward computes ("MoBA: Mixture of Block Attention for Long-Context LLMs",
 * paper summary page, "Approach"), against the limits listed above.  Returns MOBA_OK,
 * MOBA_ERR_INVALID_ARG or MOBA_ERR_UNSUPPORTED. */
int moba_check_args(int batch, int seqlen, int hq, int hkv, int head_dim, int block,
                    int topk, float scale);

/* Bytes of device workspace moba_forward uses: the centroids, the inverted index of
 * the gathered query tiles and their partial results (FlashMoBA story, paragraph on
 * Gather-and-Densify: the queries that chose a block are gathered and run as one dense
 * tile).  Returns the size that processes all kv-heads in one pass, and stores in
 * *min_bytes (if not NULL) the size that processes one kv-head per pass.  Any size in
 * between also works: moba_forward then loops over groups of kv-heads.  With
 * topk >= nb (dense causal attention) no workspace is used and both sizes are 256.
 * Returns 0 if the shape is not supported. */
size_t moba_workspace_bytes(int batch, int seqlen, int hq, int hkv, int head_dim,
                            int block, int topk, size_t* min_bytes);

/* The whole prefill forward pass (paper summary page, "Approach"):
 * centroids -> gate and top-k -> inverted index -> history attention ->
 * current-block causal attention fused with the log-sum-exp merge.
 * Writes out, lse and idx.  `workspace` must hold at least the minimum of
 * moba_workspace_bytes and be 256-byte aligned. */
int moba_forward(const void* q, const void* k, const void* v, int batch, int seqlen,
                 int hq, int hkv, int head_dim, int block, int topk, float scale,
                 void* out, float* lse, int32_t* idx, void* workspace,
                 size_t workspace_bytes, void* stream);

/* moba_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace
 * argument and calls no allocating routine; its workspace is a fixed 128 MiB device
 * array inside the library, one per GPU, kept from the first call on that GPU until the
 * process ends.  The array of the CURRENT device (hipGetDevice) is used, so `stream`
 * must belong to that device.  Inputs, outputs, layouts and results are those of
 * moba_forward (the same kernels; kv-heads run in groups sized to the 128 MiB).
 * Returns MOBA_ERR_WORKSPACE, before any device work, when one kv-head's workspace
 * (the min_bytes of moba_workspace_bytes) exceeds 128 MiB.  Every call on a GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  No word of the array needs to start
 * at zero: every word a call reads it writes first.  This entry point, unlike the
 * others, keeps state: the array and its per-device address. */
int moba_forward_noalloc(const void* q, const void* k, const void* v, int batch, int seqlen,
                         int hq, int hkv, int head_dim, int block, int topk, float scale,
                         void* out, float* lse, int32_t* idx, void* stream);

/* moba_forward, then a wait for `stream`, and the GPU time of each step measured with
 * HIP events recorded on `stream` between the steps, in milliseconds, summed over
 * kv-head groups:
 *   stage_ms[0] centroid pool   [1] gate + top-k   [2] inverted index
 *   stage_ms[3] history attention   [4] current-block attention + merge
 * stage_ms is a HOST array of MOBA_NUM_STAGES floats.  Meant for measurement: it
 * synchronises, unlike moba_forward. */
#define MOBA_NUM_STAGES 5
int moba_forward_profile(const void* q, const void* k, const void* v, int batch,
                         int seqlen, int hq, int hkv, int head_dim, int block, int topk,
                         float scale, void* out, float* lse, int32_t* idx,
                         void* workspace, size_t workspace_bytes, void* stream,
                         float* stage_ms);

/* Dense causal attention, for the layers that stay on full attention (README bullet
 * "Seamlessly Transition between Full and Sparse Attention": with every block
 * selected, the layer is full attention).  The same result as moba_forward with
 * topk >= seqlen / block, without gating or index: out[b,t,h] = softmax over keys
 * u <= t of scale * q.k_u, times V; lse as for moba_forward.  Layouts, dtypes and
 * stream semantics as for moba_forward; needs no workspace.  Any seqlen >= 1; the
 * other shape limits are moba_forward's. */
int moba_dense_forward(const void* q, const void* k, const void* v, int batch, int seqlen,
                       int hq, int hkv, int head_dim, float scale, void* out, float* lse,
                       void* stream);

/* moba_forward that also records HIP events at the step boundaries, on `stream`,
 * without synchronising: stage_events is a HOST array of MOBA_NUM_STAGES + 1 hipEvent_t
 * handles created by the caller (timing enabled); stage_events[0] is recorded before
 * the first step and stage_events[i + 1] after step i (numbered as for
 * moba_forward_profile).  When the workspace makes the call loop over several kv-head
 * groups, the events mark the boundaries of the last group.  The caller reads the
 * times with hipEventElapsedTime once the stream has passed them.  Returns
 * MOBA_ERR_INVALID_ARG when stage_events or one of its handles is NULL. */
int moba_forward_timed(const void* q, const void* k, const void* v, int batch, int seqlen,
                       int hq, int hkv, int head_dim, int block, int topk, float scale,
                       void* out, float* lse, int32_t* idx, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* stage_events);

/* ---------------------------------------------------------------------------
 * Backward pass, for training with MoBA attention (MoBA README, bullet "Trainable
 * Block Sparse Attention"; paper summary page on atlas.scime.ai, which reports
 * continual pre-training and SFT with MoBA layers).  The block selection of the
 * forward (idx) is held fixed: it is a top-k over inner products with parameter-less
 * mean-pooled keys (README bullet "Parameter-less Gating Mechanism"), piecewise
 * constant, so no gradient flows through it.  For each query row, with N its
 * attended keys (its selected history blocks whole, its current block up to itself)
 * and p_u = exp(scale q.k_u - lse), D = dO.out:
 *   dq      = scale * sum_u p_u (dO.v_u - D) k_u
 *   dk_u   += scale * p_u (dO.v_u - D) q          (summed over the rows attending u
 *   dv_u   += p_u dO                                and the G query heads of a kv-head)
 * ------------------------------------------------------------------------- */

/* Workspace bytes moba_backward uses: the size that processes all kv-heads in one
 * pass is returned, the one-kv-head-per-pass size stored in *min_bytes (if not
 * NULL); sizes in between loop over groups of kv-heads, as for moba_forward.  Returns
 * 0 if the shape is not supported by the backward (see moba_backward). */
size_t moba_backward_workspace_bytes(int batch, int seqlen, int hq, int hkv,
                                     int head_dim, int block, int topk,
                                     size_t* min_bytes);

/* Gradients of moba_forward with respect to q, k and v.
 *   q, k, v, out, lse, idx   the inputs and the outputs of moba_forward for this
 *                            problem (device pointers, layouts as above); idx must be
 *                            a valid selection in moba_forward's format
 *   dout                     [b, T, hq, d] bf16, the gradient of out
 *   dq                       [b, T, hq, d] bf16, written
 *   dk, dv                   [b, T, hkv, d] bf16, written (every element)
 * Accumulation is float32; dq sums fp32 per-history-block parts in slot order and dk,
 * dv are each summed by one workgroup in a fixed row order: deterministic.  Shape
 * limits are moba_forward's (a partial last block included; any G = hq / hkv).
 * `workspace` must hold at least the minimum of
 * moba_backward_workspace_bytes and be 256-byte aligned (MOBA_ERR_WORKSPACE,
 * MOBA_ERR_INVALID_ARG).  Enqueued on `stream` without synchronising. */
int moba_backward(const void* q, const void* k, const void* v, const void* out,
                  const float* lse, const int32_t* idx, const void* dout, int batch,
                  int seqlen, int hq, int hkv, int head_dim, int block, int topk,
                  float scale, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Full-attention decode, the hand-off after a MoBA prefill: generation switches to
 * full attention (paper summary page on atlas.scime.ai, "Limitations"; README bullet
 * "Seamlessly Transition between Full and Sparse Attention").  The n_new query tokens
 * are the last n_new positions of a cache of kv_len keys: new token i (0-based) sits at
 * position kv_len - n_new + i and attends keys 0 .. kv_len - n_new + i.
 *   q          [b, n_new, hq, d] bf16
 *   k, v       [b, kv_len, hkv, d] bf16 (the cache, the new tokens' keys included)
 *   out        [b, n_new, hq, d] bf16, written
 *   lse        [b, hq, n_new] float32, natural log, written
 * The keys are split over many wavefronts that write fp32 partials to the workspace,
 * merged by log-sum-exp in a second kernel.  The (hq / hkv) * n_new query rows of a
 * kv-head go in tiles of 32, each tile reading the cache once (one tile for decode).
 * Limits: head_dim 64 or 128, (hq / hkv) * n_new <= 1024, 1 <= n_new <= kv_len
 * (MOBA_ERR_UNSUPPORTED or
 * MOBA_ERR_INVALID_ARG otherwise).  `workspace` must hold moba_decode_workspace_bytes
 * and be 256-byte aligned (MOBA_ERR_WORKSPACE, MOBA_ERR_INVALID_ARG).  Enqueued on
 * `stream` without synchronising; capturable like moba_forward. */
size_t moba_decode_workspace_bytes(int batch, int n_new, int kv_len, int hq, int hkv,
                                   int head_dim);
int moba_decode(const void* q, const void* k, const void* v, int batch, int n_new,
                int kv_len, int hq, int hkv, int head_dim, float scale, void* out,
                float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of moba_forward_varlen (packed sequences, each with its own block grid):
 * the same gradients as moba_backward run on each sequence alone.  q, k, v, out, dout,
 * dq, dk, dv in the packed [total, heads, d] layout; lse [hq, total]; idx
 * [hq, total, topk]; cu_seqlens as for moba_forward_varlen (DEVICE, unchecked
 * contents).  Limits as moba_forward_varlen's. */
size_t moba_backward_varlen_workspace_bytes(int nseq, int total, int max_seqlen, int hq,
                                            int hkv, int head_dim, int block, int topk,
                                            size_t* min_bytes);
int moba_backward_varlen(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const int32_t* idx, const void* dout,
                         const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                         int hq, int hkv, int head_dim, int block, int topk, float scale,
                         void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Packed variable-length prefill: several sequences of different lengths in one call,
 * each with its own block grid (block j of sequence i is its tokens jB .. jB+B-1,
 * the last one possibly partial), routed and attended only within the sequence, as if
 * each were a batch-1 moba_forward (paper summary page, "Approach", applied per
 * sequence).
 *   cu_seqlens  DEVICE int32 [nseq + 1]: cu_seqlens[0] = 0, non-decreasing,
 *               cu_seqlens[nseq] = total, every length <= max_seqlen.  The library
 *               cannot check device values: other contents are undefined behaviour.
 *   q, out      [total, hq, d] bf16;  k, v  [total, hkv, d] bf16
 *   lse         [hq, total] float32;  idx  [hq, total, topk] int32 (moba_forward's rows,
 *               block ids counted within each sequence)
 * Shape limits are moba_forward's with batch = nseq and seqlen = max_seqlen, plus
 * total * hq < 2^31.  Returns as moba_forward.
 * ------------------------------------------------------------------------- */

/* Workspace for moba_forward_varlen (all kv-heads at once; *min_bytes: one per pass).
 * The index part is sized for every token using every history slot, since the lengths
 * are only known on the device.  0 if unsupported. */
size_t moba_varlen_workspace_bytes(int nseq, int total, int max_seqlen, int hq, int hkv,
                                   int head_dim, int block, int topk, size_t* min_bytes);

int moba_forward_varlen(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                        int hq, int hkv, int head_dim, int block, int topk, float scale,
                        void* out, float* lse, int32_t* idx, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Short convolution of the keys within blocks (FlashMoBA story on hyper.ai, paragraph
 * on short convolutions: a short convolution inside each block clusters the block's
 * relevant information and strengthens the routing signal).  Depthwise and causal
 * along tokens, per kv-head channel, and no tap crosses a block boundary:
 *   out[t, g, c] = sum over i < width with t - i in t's block of
 *                  weight[g, c, i] * k[t - i, g, c]
 * accumulated in float32, rounded to bf16 (nearest even).  The result is meant to be
 * passed as the keys of moba_forward / moba_forward_varlen.
 *   k, out      [batch, seqlen, hkv, d] bf16, or with cu_seqlens (DEVICE int32
 *               [batch + 1], as for moba_forward_varlen; seqlen = the longest
 *               sequence) packed [total, hkv, d].  out must not overlap k.
 *   weight      DEVICE float32 [hkv, d, width]
 *   width       1 .. 8 (MOBA_ERR_UNSUPPORTED above, MOBA_ERR_INVALID_ARG below)
 * Shape limits as moba_forward's (with hq = hkv); total is ignored without cu_seqlens.
 * Enqueued on `stream` without synchronising; needs no workspace.
 * ------------------------------------------------------------------------- */
int moba_key_short_conv(const void* k, const float* weight, const int32_t* cu_seqlens,
                        int batch, int seqlen, int total, int hkv, int head_dim, int block,
                        int width, void* out, void* stream);

/* A static, human-readable message for a status code returned by any entry point of
 * this library (the error reporting of the calls above; it computes nothing of the
 * method itself).  Never NULL; unknown codes give "unknown status". */
const char* moba_strerror(int status);

/* ---------------------------------------------------------------------------
 * Stage entry points.  Each runs one step of moba_forward on its own, with the
 * same kernels, so that every step can be checked separately.
 * ------------------------------------------------------------------------- */

/* Workspace bytes the stage entry points below need for this shape (the largest of
 * them); 0 if unsupported. */
size_t moba_stage_workspace_bytes(int batch, int seqlen, int hq, int hkv,
                                  int head_dim, int block, int topk);

/* Centroid mean-pool (paper summary page, "Approach": each block is represented by
 * its mean-pooled key): centroids[b][g][j][:] = mean of k[b, jB .. jB+B-1, g, :],
 * summed in float32 in a fixed order (deterministic). */
int moba_pool_centroids(const void* k, int batch, int seqlen, int hkv, int head_dim,
                        int block, float* centroids, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Gate and top-k (paper summary page, "Approach"; README bullet "Parameter-less
 * Gating Mechanism"; FlashMoBA story on hyper.ai, paragraph on FlashTopK: the score
 * matrix is never materialised).  For query (t, h) with c = t / block the score of
 * block j < c is <q[t,h], centroids[h/G][j]>; the topk-1 best history blocks
 * (score descending, lower index first on ties) and block c are written to idx.
 * Rows with c + 1 <= topk take every block 0..c. */
int moba_gate_topk(const void* q, const float* centroids, int batch, int seqlen,
                   int hq, int hkv, int head_dim, int block, int topk, int32_t* idx,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Number of inverted-index entries for kv-heads [kv_begin, kv_begin + kv_count):
 * every (query row, history slot) pair of their query heads. */
int64_t moba_index_entries(int batch, int seqlen, int hq, int hkv, int block, int topk,
                           int kv_count);

/* Inverted index (FlashMoBA story, paragraph on Gather-and-Densify: the queries that
 * chose a block are gathered together).  For each list (b, g, j), g in
 * [kv_begin, kv_begin + kv_count), the entries of every query row (t, h) with
 * h / G == g whose history set holds block j < t / block.
 *   list_offsets  int32 [batch * kv_count * nb + 1]: list L = (b * kv_count +
 *                 (g - kv_begin)) * nb + j holds entries[list_offsets[L] ..
 *                 list_offsets[L + 1]).
 *   entries       uint32 [moba_index_entries(...)]: ((t * G + h % G) << sb) | slot,
 *                 slot = the position of j in the row of idx, sb = 5 bits for up to
 *                 32 history slots (topk <= 33) and 6 beyond.  A block id that a row
 *                 repeats is listed at its first slot only.  topk <= 65. 
 * Lists are ordered by (chunk of 256 rows, slot, row), rows being r = t * G + h % G:
 * a deterministic order, identical on every run. */
int moba_build_index(const int32_t* idx, int batch, int seqlen, int hq, int hkv,
                     int block, int topk, int kv_begin, int kv_count,
                     int32_t* list_offsets, uint32_t* entries, void* workspace,
                     size_t workspace_bytes, void* stream);

/* History attention (FlashMoBA story on hyper.ai, paragraph on Gather-and-Densify:
 * the queries that chose a KV block are gathered into a dense tile and run against
 * that block; paper summary page, "Approach": each query attends the keys of its
 * selected blocks).  For every entry of the inverted index of kv-heads [kv_begin,
 * kv_begin + kv_count) (list_offsets and entries exactly as moba_build_index writes
 * them for the same range), softmax attention of the entry's query row (t, h) over
 * all keys of its block j, written as a part:
 *   part_o    bf16 [batch][kv_count * G][T][topk - 1][head_dim]: the part's output
 *             (normalised, rounded to nearest even) at the row's slot of block j, its
 *             head_dim values in the order the kernel's lanes hold them: position
 *             p = dt * 32 + j * 16 + hf * 8 + u * 4 + r holds dimension
 *             dt * 32 + (2 * j + u) * 8 + hf * 4 + r (dt < head_dim/32, j, hf, u < 2,
 *             r < 4), so that the two lanes that own a row read and write 32
 *             contiguous bytes of it at a time;
 *   part_lse  fp32 [topk - 1][batch][kv_count * G][T]: ln sum_u exp(scale q.k_u).
 * Heads h = kv_begin * G .. are numbered from 0 within the range.  Slots a row does
 * not have (t / block <= slot) are not written.  Splitting a row's keys into such
 * parts and merging them by log-sum-exp (moba_current_merge) gives the one-softmax
 * result.  tile_order_seed 0 runs the tiles in list order; any other value runs them
 * in a seeded permuted order, which must give bit-identical parts: each part is
 * written by exactly one tile, so the launch order does not matter (a check for
 * races between tiles).  Needs topk >= 2 (MOBA_ERR_UNSUPPORTED otherwise) and the
 * index limits of moba_build_index; workspace: moba_stage_workspace_bytes.  Enqueued
 * on `stream` without synchronising. */
int moba_history_partials(const void* q, const void* k, const void* v, int batch,
                          int seqlen, int hq, int hkv, int head_dim, int block, int topk,
                          float scale, int kv_begin, int kv_count,
                          const int32_t* list_offsets, const uint32_t* entries,
                          uint32_t tile_order_seed, void* part_o, float* part_lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Current block and merge (paper summary page, "Approach": each query also attends its
 * own current block, causally).  For every query head of kv-heads [kv_begin, kv_begin +
 * kv_count): causal attention of (t, h) over keys c*block .. t of its block c,
 * merged by log-sum-exp with the row's min(c, topk - 1) history parts from
 * moba_history_partials (same layout and kv range): L = ln(e^lse_c + sum_s e^lse_s),
 * out = e^(lse_c - L) o_c + sum_s e^(lse_s - L) o_s, lse = L, written into out
 * [batch, seqlen, hq, head_dim] bf16 and lse [batch, hq, seqlen] fp32 at those heads.
 * part_o and part_lse may be NULL when topk == 1.  pool -> gate -> build_index ->
 * history_partials -> current_merge over all kv-heads is moba_forward, bit for bit,
 * when topk * block < seqlen.  Needs no workspace; enqueued on `stream`. */
int moba_current_merge(const void* q, const void* k, const void* v, int batch, int seqlen,
                       int hq, int hkv, int head_dim, int block, int topk, float scale,
                       int kv_begin, int kv_count, const void* part_o,
                       const float* part_lse, void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H */
