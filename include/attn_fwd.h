/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) FlashAttention forward library.
 *
 * The library computes O = softmax(scale * Q K^T) V per (sequence, query head)
 * without materialising the score matrix, for dense batched inputs and for
 * variable-length packed inputs, plus the row gather/scatter that moves packed
 * rows between the padded and the compact layouts, attention over a paged KV
 * cache, and the gradients of the attention (backward by recomputation).
 *
 * Sources of the operations (web pages, cited by title and section):
 *  - "Intro to FlashAttention on Ascend CANN" (ai6s.net): the standard
 *    definition (section on where the traditional implementation is slow), the
 *    blockwise computation with an online softmax that keeps a running row max
 *    m and row sum d (sections "tiled computation" and "the first pitfall"),
 *    and the fused causal mask that skips masked positions (paragraph on the
 *    ops-transformer source).
 *  - "Lesson 5: IAW model FA2 vs FA3 measured": the packed path of section 1
 *    (padded (B, total_len, H, D) -> unpad gather by indices -> varlen
 *    attention on (total_valid, H, D) -> pad scatter by indices) and the
 *    kernels of section 2 and section 6 that perform those moves.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates nothing, frees nothing and never synchronises the stream; the
 *    only scratch memory it uses is a workspace the caller passes (_ws calls,
 *    attn_fwd_paged), except attn_fwd_paged_noalloc, which uses a fixed array
 *    of the library's own in device memory (declared with it below).
 *  - bfloat16 tensors are passed as raw 16-bit storage (const void*).
 *  - `stream` is a hipStream_t cast to void*; NULL means the default stream.
 *    Work is enqueued asynchronously on it.
 *  - All argument checks run on the host before anything is enqueued.  On any
 *    error nothing is launched and the status says why.  Device-side faults (for
 *    example cu_seqlens that do not match the tensors) surface at the caller's
 *    next synchronisation; the preconditions below say what must hold.
 *  - Tuning and test overrides (environment variables read at each call; unset
 *    means the library's own choice, which is what the results are measured
 *    with): ATTN_FWD_TILE=<policy> forces a compiled forward tile policy
 *    (sweeps; an uncompiled one returns ATTN_ERR_UNSUPPORTED),
 *    ATTN_FWD_SPLIT_TILES=<n> forces key-range parts of at most n tiles on the
 *    split-capable policies when a workspace is given, ATTN_FWD_ORDER=<1..4>
 *    forces the workgroup order (head-remapped block-major, sequence-major,
 *    unit-major, compact), ATTN_FP8_TILE=128|256 forces the fp8 query block,
 *    ATTN_PAGED_VARIANT=<0..3>, ATTN_PAGED_ORDER=0|1 and
 *    ATTN_PAGED_CHUNK_TILES=<n> force the paged kernel's layout, grid order
 *    and key-range parts, and ATTN_BWD_SPLIT=1 runs the backward's dV and dK
 *    as two passes.  Every forced choice computes the same attention; the
 *    GPU tests compare them with the oracle and, where the arithmetic is the
 *    same, bit for bit with the default.
 *  - Debug mode: with the environment variable ATTN_FWD_DEBUG set (to anything
 *    but "0"), every call that takes device-resident metadata first checks it
 *    on the device (cu_seqlens start at 0, never decrease, end at the total,
 *    lengths within max_seqlen; indices strictly increasing and, where
 *    required, in range; seqlens_k within max_seqlen_k), synchronises the
 *    stream, and returns ATTN_ERR_SHAPE without launching the work if a check
 *    fails.
 *  - Zero work (no sequences, no rows, zero-length tensors) returns ATTN_OK
 *    without launching.
 *  - No exception crosses the ABI.  The library keeps no per-call state; calls
 *    on different streams from different host threads are safe.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is negative or sizes disagree */
  ATTN_ERR_UNSUPPORTED = 3, /* head_dim not in {32,64,128,256}, scale not finite, ... */
  ATTN_ERR_ALIGN = 4,       /* a pointer or row size is not 16-byte aligned */
  ATTN_ERR_HIP = 5,         /* the HIP runtime rejected the launch */
  ATTN_ERR_SCRATCH = 6      /* the call needs more than the library's static scratch */
} attn_status_t;

/*
 * attn_fwd_varlen -- attention over variable-length sequences packed back to back.
 *
 * Passage: page "Lesson 5: IAW model FA2 vs FA3 measured", section 1 (the
 * varlen attention on the compact tensor); the computation is the one of page
 * "Intro to FlashAttention on Ascend CANN" named in the file header.
 *
 * q    (total_q, num_heads_q, head_dim) bf16, row-major, contiguous.
 * k, v (total_k, num_heads_k, head_dim) bf16, row-major, contiguous.
 * cu_seqlens_q, cu_seqlens_k: device int32 arrays of num_seqs+1 offsets;
 *      sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) and key
 *      rows [cu_seqlens_k[s], cu_seqlens_k[s+1]).  Preconditions: element 0 is
 *      0, offsets never decrease, the last equals total_q (resp. total_k), and
 *      no query length exceeds max_seqlen.  Zero-length sequences are allowed.
 * max_seqlen: an upper bound on every query length (host value; sizes the grid).
 * scale: multiplies the raw scores q.k (use 1/sqrt(head_dim)); any finite value.
 *      A negative scale weights the smallest q.k highest; zero gives every
 *      visible key the same weight (out = mean of the visible value rows,
 *      lse = ln(number of visible keys)).
 * causal: nonzero => key j is visible to query i when j <= i + (Lk - Lq)
 *      (bottom-right alignment; with Lq == Lk this is j <= i).
 * out  (total_q, num_heads_q, head_dim) fp32, written once per element.
 * lse  (num_heads_q, total_q) fp32 natural-log log-sum-exp of the scaled
 *      visible scores, or NULL to skip it.  A query that sees no key gets out
 *      = 0 and lse = -inf.
 * Grouped-query attention: num_heads_q must be a multiple of num_heads_k;
 * query head h reads key/value head h / (num_heads_q / num_heads_k).
 * head_dim must be 32, 64, 128 or 256.  Every pointer must be 16-byte aligned.
 * Size limit: q and k must each span less than 4 GiB (tile loads use 32-bit
 * byte offsets); larger inputs return ATTN_ERR_SHAPE.
 */
attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t num_seqs, int32_t total_q, int32_t total_k,
                              int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                              int32_t max_seqlen, float scale, int32_t causal,
                              float* out, float* lse, void* stream);

/*
 * attn_fwd_dense -- attention over a dense batch of equal-length sequences.
 *
 * Passage: page "Intro to FlashAttention on Ascend CANN", section "how to use
 * it" (dense q, k, v with an is_causal flag) and the definition named in the
 * file header; page "Lesson 5: IAW model FA2 vs FA3 measured", section 7 (the
 * dense ViT attention).
 *
 * q   (batch, seqlen_q, num_heads_q, head_dim) bf16
 * k,v (batch, seqlen_k, num_heads_k, head_dim) bf16
 * out (batch, seqlen_q, num_heads_q, head_dim) fp32
 * strides: NULL for contiguous tensors in the layouts above, else a host array
 *      of 12 element strides {q_b, q_s, q_h, k_b, k_s, k_h, v_b, v_s, v_h,
 *      o_b, o_s, o_h}; the head_dim stride is always 1, every stride must be a
 *      multiple of 8 elements (16 bytes of bf16) and of 4 for out.
 * lse (batch, num_heads_q, seqlen_q) fp32 contiguous, or NULL.
 * scale, causal, head_dim, grouped-query heads and the fully-masked-row rule
 * are as for attn_fwd_varlen.  Size limit: one sequence of q, k or v must span
 * less than 4 GiB (seqlen * seq stride * 2 bytes); else ATTN_ERR_SHAPE.
 */
attn_status_t attn_fwd_dense(const void* q, const void* k, const void* v,
                             int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                             int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                             const int64_t* strides, float scale, int32_t causal,
                             float* out, float* lse, void* stream);

/*
 * attn_fwd_varlen_ws, attn_fwd_dense_ws -- the two calls above with a caller-
 * owned workspace that lets the library split long key ranges.
 *
 * Passage: the same as attn_fwd_varlen / attn_fwd_dense.  The split relies on
 * the rule of page "Intro to FlashAttention on Ascend CANN", section "the first
 * pitfall": softmax partials over disjoint key ranges combine exactly once each
 * carries its running maximum and sum.  Here a part stores O_r normalised by
 * its own sum and L_r = log2 of that sum in base-2 exponent units, and a merge
 * launch forms O = sum_r 2^(L_r - L) O_r, L = log2 sum_r 2^(L_r).
 *
 * When a launch has few query blocks and their key loops are long (a causal
 * sequence with few heads), the longest block bounds the run time while most
 * CUs idle.  With a workspace the key loop of such blocks is cut into parts of
 * about the per-CU share of all key tiles, each run by its own workgroup.
 *
 * workspace: device memory of at least workspace_bytes bytes, 16-byte aligned,
 *      owned by the caller; contents need no initialisation and are scratch
 *      after the call.  NULL, or fewer bytes than attn_fwd_workspace_bytes
 *      reports for the shape, runs the call without splitting (same results up
 *      to rounding order).  Two calls that share one workspace must not overlap
 *      in time (same stream, or synchronised).
 * workspace_bytes: size of workspace; negative returns ATTN_ERR_SHAPE.
 * All other arguments, results and errors are those of the call without _ws.
 * Results differ from the unsplit call only in floating-point rounding order.
 */
attn_status_t attn_fwd_varlen_ws(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t num_seqs, int32_t total_q, int32_t total_k,
                                 int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                                 int32_t max_seqlen, float scale, int32_t causal,
                                 float* out, float* lse, void* workspace,
                                 int64_t workspace_bytes, void* stream);

attn_status_t attn_fwd_dense_ws(const void* q, const void* k, const void* v,
                                int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                                int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                                const int64_t* strides, float scale, int32_t causal,
                                float* out, float* lse, void* workspace,
                                int64_t workspace_bytes, void* stream);

/*
 * attn_fwd_workspace_bytes -- workspace size that enables splitting for a shape.
 *
 * num_seqs (batch for dense), max_seqlen (seqlen_q for dense), num_heads_q,
 * head_dim and causal as in the calls above.  Returns the byte count the _ws
 * calls need to split key ranges for this shape, or 0 when the library would
 * not split it (or the arguments are invalid).  Pure host computation.
 */
int64_t attn_fwd_workspace_bytes(int32_t num_seqs, int32_t max_seqlen, int32_t num_heads_q,
                                 int32_t head_dim, int32_t causal);

/*
 * attn_fwd_launch_plan -- how the library would launch a forward call.
 *
 * Passage: page "FlashAttention tuning: block_size and head_dim" (the block
 * size is chosen per shape, from measurements; its checklist records the best
 * configuration per sequence length).  This reports the choice for one shape
 * so that sweeps and tests can see it.
 *
 * varlen: nonzero for attn_fwd_varlen (then total_q is the packed query count),
 *      zero for attn_fwd_dense (num_seqs = batch, max_seqlen = seqlen_q).
 * workspace_bytes: the workspace the _ws call would get (0: none).
 * plan: host array of 4 int32 receiving {tile policy id, workgroup order, key-
 *      range parts per query block (1 = no split), queries per block}.  Orders:
 *      0 block-major, 1 block-major with (sequence, head) rows spread over the
 *      XCDs, 2 sequence-major, 3 (sequence, head) units dealt to the XCDs, 4
 *      compact (one workgroup slot per real query block of a varlen pack).
 * The environment overrides ATTN_FWD_TILE (policy), ATTN_FWD_ORDER (order) and
 * ATTN_FWD_SPLIT_TILES apply as they do to the calls.  Returns ATTN_ERR_SHAPE
 * for non-positive sizes, ATTN_ERR_UNSUPPORTED for a head_dim, policy or
 * order the library cannot use, ATTN_ERR_NULL when plan is NULL.  Pure host
 * computation.
 */
attn_status_t attn_fwd_launch_plan(int32_t varlen, int32_t num_seqs, int32_t total_q,
                                   int32_t max_seqlen, int32_t num_heads_q, int32_t head_dim,
                                   int32_t causal, int64_t workspace_bytes, int32_t* plan);

/*
 * attn_fwd_tile_policy_compiled -- 1 if tile policy `policy` is compiled for
 * head_dim (so ATTN_FWD_TILE=<policy> can force it), else 0.  Passage as for
 * attn_fwd_launch_plan.  Pure host computation.
 */
int32_t attn_fwd_tile_policy_compiled(int32_t policy, int32_t head_dim);

/*
 * attn_unpad_gather -- copy the rows named by `indices` into a compact tensor.
 *
 * Passage: page "Lesson 5: IAW model FA2 vs FA3 measured", section 1 (unpad:
 * gather rows by indices into (total_valid, H, D)) and section 2 (the gather
 * kernels that perform it).
 *
 * For each of the n_tensors (1..3) pairs: dst[t] row r = src[t] row indices[r],
 * for r < n_valid.  A row is row_bytes bytes (H * D * element size); src[t]
 * holds n_rows_src rows, dst[t] holds n_valid rows.  `src` and `dst` are HOST
 * arrays of n_tensors device pointers; every tensor shares `indices` (device
 * int32, n_valid entries).  All q, k and v of one packed batch move in one
 * launch.  row_bytes must be a positive multiple of 16; pointers 16-byte
 * aligned.  An index outside [0, n_rows_src) yields a zero row (never an
 * out-of-bounds read).  The copy is bit-exact.
 */
attn_status_t attn_unpad_gather(const void* const* src, void* const* dst, int32_t n_tensors,
                                const int32_t* indices, int32_t n_valid, int32_t n_rows_src,
                                int64_t row_bytes, void* stream);

/*
 * attn_mask_to_varlen -- the unpad inputs from a padding mask, on the device.
 *
 * Passage: page "Lesson 5: IAW model FA2 vs FA3 measured", section 1 (unpad
 * gathers the non-padding rows named by indices; the varlen attention takes
 * the packing offsets).
 *
 * mask (batch, seqlen) bytes, device: the padded tensor's rows as `batch`
 *      slots of `seqlen` rows; nonzero = valid row.  Slot b's valid rows (in
 *      row order) form sequence b; an all-padding slot is an empty sequence.
 * indices (device int32, capacity batch * seqlen): the valid rows b * seqlen +
 *      i in increasing order; only the first n_valid entries are written.
 * cu_seqlens (device int32, batch + 1): cu_seqlens[b] = valid rows in slots
 *      0..b-1.
 * stats (device int32, 2): {n_valid, max_seqlen}.  Read them back (one small
 *      copy) when the host needs the sizes; seqlen is always a valid
 *      max_seqlen bound for the attention calls.
 * Three launches on `stream`; nothing is allocated.  batch * seqlen < 2^31.
 * The results equal those of the oracle's definition exactly (integer work).
 * For attn_fwd_padded each slot's valid rows must be consecutive (a run at
 * any position in the slot); a mask with holes inside a slot gives indices
 * that the unpad/varlen/pad calls accept but the fused padded call does not.
 */
attn_status_t attn_mask_to_varlen(const void* mask, int32_t batch, int32_t seqlen,
                                  int32_t* indices, int32_t* cu_seqlens, int32_t* stats,
                                  void* stream);

/*
 * attn_pad_scatter -- put compact rows back into the padded layout.
 *
 * Passage: page "Lesson 5: IAW model FA2 vs FA3 measured", section 1 (pad:
 * scatter rows back to (B, total_len, H, D) by indices) and section 6 (the
 * fill and index kernels of the pad step).
 *
 * dst row indices[r] = src row r for r < n_valid; every other dst row (of
 * n_rows_total) is written with +0.0 bytes.  One pass writes each dst byte
 * exactly once, so no separate fill is needed.  Precondition: `indices`
 * (device int32, n_valid entries) is strictly increasing; entries outside
 * [0, n_rows_total) are ignored.  row_bytes must be a positive multiple of
 * 16; pointers 16-byte aligned.  The copy is bit-exact.
 */
attn_status_t attn_pad_scatter(const void* src, void* dst, const int32_t* indices,
                               int32_t n_valid, int32_t n_rows_total, int64_t row_bytes,
                               void* stream);

/*
 * attn_fwd_padded -- unpad gather, varlen attention and pad scatter in one call
 * that never materialises the compact tensors.
 *
 * Passage: page "Lesson 5: IAW model FA2 vs FA3 measured", section 1 (the
 * padded path: gather rows by indices, varlen attention on the compact rows,
 * scatter back by indices) and section 6 (the launches and the movement that
 * path costs); the attention is the one of attn_fwd_varlen.
 *
 * q    (n_rows, num_heads_q, head_dim) bf16, the PADDED tensor (B * total_len
 *      rows, row-major, contiguous); k, v (n_rows, num_heads_k, head_dim) bf16.
 * indices: device int32, n_valid entries, strictly increasing, in [0, n_rows):
 *      compact row r is padded row indices[r].
 * cu_seqlens: device int32, num_seqs+1 offsets over the compact rows (queries
 *      and keys alike); last = n_valid.
 * Precondition: the rows of one sequence are consecutive in the padded tensor,
 *      indices[cu_seqlens[s] + i] == indices[cu_seqlens[s]] + i (true of right-
 *      padded slots and of packed rows).  Violating it gives wrong values for
 *      that sequence but no out-of-range access; in debug mode (ATTN_FWD_DEBUG)
 *      the call returns ATTN_ERR_SHAPE instead.
 * out  (n_rows, num_heads_q, head_dim) fp32: indexed rows get the attention
 *      output, every other row is written with +0.0 bytes.
 * lse  (num_heads_q, n_valid) fp32 over the COMPACT rows, or NULL.
 * max_seqlen, scale, causal, grouped-query heads, alignment and size limits
 *      are those of attn_fwd_varlen (sizes measured on the padded tensors).
 * Two launches: a zero fill of the padding rows, then the attention reading
 * and writing the padded rows in place.  Results equal those of
 * attn_unpad_gather + attn_fwd_varlen + attn_pad_scatter bit for bit.
 */
attn_status_t attn_fwd_padded(const void* q, const void* k, const void* v,
                              const int32_t* indices, const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t n_valid, int32_t n_rows, int32_t num_heads_q,
                              int32_t num_heads_k, int32_t head_dim, int32_t max_seqlen,
                              float scale, int32_t causal, float* out, float* lse, void* stream);

/*
 * attn_fwd_paged -- attention of new queries over a paged KV cache (decode,
 * speculative decode, chunked prefill).
 *
 * Passage: page "why FA is 2x on A100 but 1.5x on Ascend 910", section 5
 * (manage the inference KV cache with PagedAttention; inference is bound by
 * moving K and V), with the attention of page "Intro to FlashAttention on
 * Ascend CANN" (online softmax over key tiles; partial results over disjoint
 * key ranges merge exactly through their log-sum-exps, "the first pitfall").
 *
 * q        (total_q, num_heads_q, head_dim) bf16: the new queries, packed;
 *          sequence s owns rows [cu_seqlens_q[s], cu_seqlens_q[s+1]).
 * k_cache, v_cache (num_pages, page_size, num_heads_k, head_dim) bf16: the
 *          page pool.  Key j of sequence s is row j % page_size of page
 *          block_table[s * max_pages_per_seq + j / page_size], j < seqlens_k[s].
 *          A dense (batch, max_len, H, D) cache is the case page_size = max_len,
 *          block_table[s] = s.
 * seqlens_k (num_seqs) int32: keys of each sequence (the new tokens included).
 * block_table (num_seqs, max_pages_per_seq) int32.  Page numbers outside
 *          [0, num_pages) read as zero keys (never out of bounds); entries past
 *          a sequence's last page are not read.
 * causal: nonzero => query i of Lq sees keys j <= i + (Lk - Lq) (bottom-right:
 *          the new tokens are the last Lq keys).
 * out (total_q, num_heads_q, head_dim) fp32; lse (num_heads_q, total_q) fp32
 *          natural log, or NULL.  A query that sees no key gets 0 and -inf.
 * max_seqlen_q / max_seqlen_k: upper bounds on query / key counts (host);
 *          max_seqlen_k <= max_pages_per_seq * page_size.
 * workspace: optional (may be NULL), 16-byte aligned, at least
 *          attn_fwd_paged_workspace_bytes(...) bytes: lets long key ranges be
 *          split over several workgroups (one more launch merges them).  Too
 *          small or NULL: no split.
 * head_dim 32, 64, 128 or 256; page_size a positive multiple of 16; one page of one
 * tensor (page_size * num_heads_k * head_dim * 2 bytes) under 4 GiB.
 * GQA: the query heads of one KV head are processed together, so each K/V
 * byte is read once per (sequence, KV head).  One or two launches on `stream`.
 */
attn_status_t attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                             const int32_t* block_table, int32_t num_seqs, int32_t total_q,
                             int32_t num_pages, int32_t page_size, int32_t max_pages_per_seq,
                             int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                             int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
                             int32_t causal, float* out, float* lse, void* workspace,
                             int64_t workspace_bytes, void* stream);

/*
 * attn_fwd_paged_fp8kv -- attn_fwd_paged over a cache of 8-bit floats.
 *
 * Passage: page "why FA is 2x on A100 but 1.5x on Ascend 910", section 5 (a
 * narrower KV cache halves the bytes the HBM-bound inference moves), with the
 * E4M3 format and per-tensor factors of attn_fwd_fp8_varlen.
 *
 * k_cache, v_cache (num_pages, page_size, num_heads_k, head_dim): E4M3 bytes;
 * the keys and values are k_scale * K and v_scale * V (factors > 0, finite).
 * q stays bf16.  Every other argument, the workspace and the size rules are
 * those of attn_fwd_paged (the page-size limit counts one byte per element;
 * head_dim 32, 64, 128 or 256).
 * The cache bytes are dequantised to bf16 in registers (E4M3 values are exact
 * in bf16) and the products are the bf16 MFMAs of attn_fwd_paged, so the
 * results carry the same rounding as the bf16 path on the dequantised values.
 */
attn_status_t attn_fwd_paged_fp8kv(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                   const int32_t* block_table, int32_t num_seqs, int32_t total_q,
                                   int32_t num_pages, int32_t page_size, int32_t max_pages_per_seq,
                                   int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
                                   float k_scale, float v_scale, int32_t causal, float* out,
                                   float* lse, void* workspace, int64_t workspace_bytes,
                                   void* stream);

/*
 * attn_fwd_paged_noalloc -- attn_fwd_paged for callers that cannot allocate.
 *
 * For code that must not call hipMalloc: work under HIP graph capture, tight
 * serving (decode) loops, harnesses that forbid allocation.  The same
 * computation, kernels and results as attn_fwd_paged with a workspace of
 * attn_fwd_paged_workspace_bytes; the scratch memory of the key-range split
 * is instead a static device array inside the library, of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the first call on a GPU
 * until the process ends.  Nothing is allocated or freed.
 * Arguments, layouts, preconditions and errors are those of attn_fwd_paged
 * without the workspace.  `stream` must belong to the current HIP device
 * (the array's copy on that device is used).
 * Limit: a shape whose split needs more than ATTN_NOALLOC_SCRATCH_BYTES (only
 * possible under the ATTN_PAGED_CHUNK_TILES test override; every default plan
 * needs at most 16.8 MB at head_dim 256, 8.4 MB at 128) returns
 * ATTN_ERR_SCRATCH before anything is launched.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call writes every slot it reads, so nothing needs clearing):
 * calls that overlap in time on one GPU (different streams, or host threads)
 * race and give wrong results; serialise them.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (17ll << 20)
attn_status_t attn_fwd_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                     const int32_t* block_table, int32_t num_seqs,
                                     int32_t total_q, int32_t num_pages, int32_t page_size,
                                     int32_t max_pages_per_seq, int32_t num_heads_q,
                                     int32_t num_heads_k, int32_t head_dim, int32_t max_seqlen_q,
                                     int32_t max_seqlen_k, float scale, int32_t causal,
                                     float* out, float* lse, void* stream);

/*
 * attn_fwd_paged_workspace_bytes -- workspace that lets attn_fwd_paged split
 * key ranges for this shape; 0 when it would not split (or for invalid
 * arguments).  Pure host computation.
 */
int64_t attn_fwd_paged_workspace_bytes(int32_t num_seqs, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t num_heads_q,
                                       int32_t num_heads_k, int32_t head_dim);

/*
 * attn_fwd_fp8_varlen -- attention on fp8 (OCP E4M3) inputs, packed layout.
 *
 * Passage: the pages name FP8 only as FA-3's direction (page "Lesson 5: IAW
 * model FA2 vs FA3 measured", closing note) and narrower data as a way to halve
 * the bytes moved (page "why FA is 2x on A100 but 1.5x on Ascend 910", section
 * 5); the computation is the attention of attn_fwd_varlen on the dequantised
 * values q_scale * q, k_scale * k, v_scale * v.
 *
 * q (total_q, num_heads_q, head_dim), k, v (total_k, num_heads_k, head_dim):
 *      E4M3 bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *      S.1111.111 is NaN), row-major, contiguous.
 * q_scale, k_scale, v_scale: the per-tensor dequantisation factors (> 0,
 *      finite).  Everything else (cu_seqlens, max_seqlen, scale, causal, out,
 *      lse, GQA, alignment) as in attn_fwd_varlen.
 * Precision: the scores and the row sums are exact products in fp32; the
 * probabilities enter the P*V product as E4M3 (after scaling by 2^8), so the
 * output carries their rounding (at most 2^-4 relative per probability).
 * head_dim 32, 64, 128 or 256 (else ATTN_ERR_UNSUPPORTED; at 32 the fp8
 * MFMA's 64-element reduction runs half empty; at 256 the query block is 128
 * and forcing ATTN_FP8_TILE=256 returns ATTN_ERR_UNSUPPORTED).  One launch.
 */
attn_status_t attn_fwd_fp8_varlen(const void* q, const void* k, const void* v,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t num_seqs, int32_t total_q, int32_t total_k,
                                  int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                                  int32_t max_seqlen, float scale, float q_scale, float k_scale,
                                  float v_scale, int32_t causal, float* out, float* lse,
                                  void* stream);

/*
 * attn_fwd_fp8_dense -- attention on fp8 inputs, dense (batch, seqlen, heads,
 * head_dim) contiguous layout; out (B, Sq, Hq, D) fp32, lse (B, Hq, Sq) fp32.
 * Rules as for attn_fwd_fp8_varlen.
 */
attn_status_t attn_fwd_fp8_dense(const void* q, const void* k, const void* v, int32_t batch,
                                 int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads_q,
                                 int32_t num_heads_k, int32_t head_dim, float scale,
                                 float q_scale, float k_scale, float v_scale, int32_t causal,
                                 float* out, float* lse, void* stream);

/*
 * attn_bwd_varlen -- gradients of attn_fwd_varlen with respect to q, k and v.
 *
 * Passage: page "Intro to FlashAttention on Ascend CANN", section on the
 * second pitfall (backward propagation): the backward pass recomputes the
 * attention probabilities tile by tile from q, k and the forward's
 * log-sum-exp instead of storing them.  The gradients are the exact
 * derivatives of the forward's definition: with P = exp(scale q.k - lse)
 * over the visible keys (0 elsewhere) and dO the gradient of `out`,
 *   dv = P^T dO,  dS = P * (dO v^T - rowsum(dO * out)),
 *   dq = scale dS k,  dk = scale dS^T q,
 * and a grouped key/value head receives the sum over its query heads.
 *
 * q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, the head
 *      counts, scale and causal: exactly as passed to attn_fwd_varlen.
 * out  (total_q, num_heads_q, head_dim) fp32 and lse (num_heads_q, total_q)
 *      fp32: the forward's outputs for these inputs (lse is required here).
 * dout (total_q, num_heads_q, head_dim) bf16: the gradient of out.
 * max_seqlen_q / max_seqlen_k: upper bounds on every query / key length.
 * dq (total_q, num_heads_q, head_dim), dk and dv (total_k, num_heads_k,
 *      head_dim): fp32 outputs, every element written once (keys that no
 *      query sees get 0, as do queries that see no key).
 * workspace: device memory of at least attn_bwd_workspace_bytes(total_q,
 *      num_heads_q) bytes, 16-byte aligned, owned by the caller; it holds
 *      rowsum(dO * out) between the launches and may be reused afterwards.
 * head_dim must be 32, 64, 128 or 256 (else ATTN_ERR_UNSUPPORTED).  Every
 * pointer must be non-NULL and 16-byte aligned (lse and cu_seqlens 4-byte
 * aligned).  Three launches on `stream`, no atomics: rowsum(dO * out), then
 * dq, then dk and dv (at head_dim 256, dv and dk in two launches).  Results
 * are deterministic.
 */
attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const float* out,
                              const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                              int32_t total_k, int32_t num_heads_q, int32_t num_heads_k,
                              int32_t head_dim, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              float scale, int32_t causal, float* dq, float* dk, float* dv,
                              void* workspace, int64_t workspace_bytes, void* stream);

/*
 * attn_bwd_dense -- gradients of attn_fwd_dense (contiguous layouts only).
 *
 * Passage and formulas: those of attn_bwd_varlen.  q, dout (batch, seqlen_q,
 * num_heads_q, head_dim) bf16; k, v (batch, seqlen_k, num_heads_k, head_dim)
 * bf16; out (batch, seqlen_q, num_heads_q, head_dim) fp32 and lse (batch,
 * num_heads_q, seqlen_q) fp32 from attn_fwd_dense; dq, dk, dv fp32 shaped
 * like q, k, v.  Workspace: attn_bwd_workspace_bytes(batch * seqlen_q,
 * num_heads_q) bytes.  Other rules as for attn_bwd_varlen.
 */
attn_status_t attn_bwd_dense(const void* q, const void* k, const void* v, const float* out,
                             const void* dout, const float* lse, int32_t batch, int32_t seqlen_q,
                             int32_t seqlen_k, int32_t num_heads_q, int32_t num_heads_k,
                             int32_t head_dim, float scale, int32_t causal, float* dq, float* dk,
                             float* dv, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * attn_bwd_workspace_bytes -- workspace the backward calls need: 4 bytes per
 * (query row, query head).  Returns 0 for non-positive arguments.  Host only.
 */
int64_t attn_bwd_workspace_bytes(int64_t total_q, int32_t num_heads_q);

/* Human-readable text of a status code (static storage, never NULL). */
const char* attn_status_str(attn_status_t s);

/* ABI version of this header; bumped on any incompatible change. */
int32_t attn_abi_version(void);

#define ATTN_FWD_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
