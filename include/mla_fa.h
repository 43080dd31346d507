/*
 * mla_fa.h -- C ABI of the MI355X (gfx950) MLA flash-attention library.
 *
 * The operation: flash attention for DeepSeek-style multi-head latent attention over
 * the compressed latent cache.  Each cache row holds kv_lora_rank 512 latent values
 * followed by 64 RoPE values (576 in all); with flash attention the cache is K-only
 * and V is the first 512 columns of the same row, shared by every query head
 * ("ik_llama.cpp -mla flag deep-dive", sections "what MLA is" and "the four -mla
 * levels").  Scores are formed tile by tile with an online softmax (running max m,
 * running sum l, earlier terms corrected whenever m grows), so no score matrix is
 * ever written to memory ("Vulkan backend fused Flash Attention: DeepSeek MLA local
 * inference", sections 2.1-2.2).  The optional mask is f16 and additive after
 * scaling; a cell whose mask is -inf is not kept ("baguaai Flash Attention tag page",
 * f16 FA mask digest).  Sparse decoding first compacts each mask row to the ascending
 * list of kept cells with one scan over per-segment ballot counts, then attends only
 * to those rows ("llama.cpp Vulkan backend adds sparse Flash Attention for quantized
 * K/V", commit text).
 *
 * For a query row q (576 values), keys k_j (576 values) and mask b_j:
 *     s_j   = scale * <q, k_j> + b_j           (s_j = -inf when b_j = -inf or j is
 *                                               past the causal edge)
 *     out   = sum_j softmax(s)_j * k_j[0:512]   (all zeros when no key is kept)
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no memory on any of these paths and keeps no pointer after return.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; outputs are valid once the stream reaches that point.
 *   - Arguments are validated on the host before any HIP call.  The return value is
 *     MLA_FA_OK or a negative mla_fa_status; on error nothing was enqueued except
 *     for MLA_FA_ERR_HIP, which reports a failed launch.  No exceptions, no abort,
 *     no host synchronisation.  Calls are reentrant; calls that share a workspace
 *     must be ordered on one stream.
 *   - A call enqueues kernel launches only (no memory set, copy or allocation), so a
 *     call on a capturing stream is recorded into a HIP graph and its replays
 *     reproduce the eager result bit for bit (mla_fa_decode_noalloc: call it once
 *     outside capture first, which looks up the device's scratch address).
 *   - Element types: q is f16 or bf16 (bits, [..][n_head][576] contiguous); the
 *     cache is f16, bf16 or Q8_0.  Supported pairs: f16/f16, bf16/bf16, f16/Q8_0,
 *     bf16/Q8_0.  A Q8_0 row is 18 blocks of {f16 scale d, 32 int8 codes} = 612
 *     bytes; value = code * d.  f16 caches are computed in f16 and bf16 caches in
 *     bf16, with fp32 accumulation.
 *   - Q8_0 range contract: Q8_0 caches are computed with f16 operands.  Each cache
 *     value is f16(code * d), rounded once and saturated to +-65504, and a bf16 query
 *     is converted to f16 with the same saturation (values below f16's subnormal
 *     range become 0).  So the result is the exact one whenever |code * d| <= 65504
 *     (always when |d| < 512: 128 * 511.75 = 65504; a block quantised from values in
 *     f16 range has d <= 516, where only 127 * d may pass 65504, by under 0.05%) and
 *     the query lies within f16's range.  Past that, values are clamped, never
 *     infinite; d must be finite.
 *   - n_head is a multiple of 16 in [16, 128].  Query rows (n_seq * n_tok) times
 *     n_head is at most 2^31 - 1; more is MLA_FA_ERR_INVALID.  Any number of rows
 *     within that runs: calls beyond 65535 rows are issued as several launches.
 *   - Outputs are fp32 [..][n_head][512].
 *   - Tuning overrides, read from the environment at each call (results change by
 *     floating-point reassociation only): MLA_FA_NSPLIT=<1..1024> forces the split
 *     count of automatic plans; MLA_FA_SHAPE=16|32|64|128|p64|p128 forces the
 *     heads-per-workgroup shape; MLA_FA_LOG (any value) prints each call's plan to
 *     stderr.
 *   - Test hook, read at each call: with MLA_FA_FAIL_LAUNCH=<k> (k >= 1) a call
 *     launches no kernel at all; it walks its launch sequence and reports its k-th
 *     launch as failed (MLA_FA_ERR_HIP), or MLA_FA_OK when it has fewer launches.  It
 *     exists so that every launch-error return can be tested without a GPU.
 */
#ifndef MLA_FA_H
#define MLA_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mla_fa_type { MLA_FA_F16 = 1, MLA_FA_BF16 = 2, MLA_FA_Q8_0 = 3 };

enum mla_fa_status {
    MLA_FA_OK = 0,
    MLA_FA_ERR_INVALID = -1,      /* null pointer, bad size, stride or alignment     */
    MLA_FA_ERR_UNSUPPORTED = -2,  /* type pair or head count the library does not do */
    MLA_FA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required       */
    MLA_FA_ERR_HIP = -4           /* a HIP launch failed                              */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char *mla_fa_strerror(int status);

/* Library version as major*10000 + minor*100 + patch (2.0.0: mla_fa_attend takes
 * per-token sparse index lists; 2.1.0: mla_fa_absorbed fuses the split merge with the
 * output projection, three launches per call; mla_fa_attend, mla_fa_absorbed and the
 * sparse mla_fa_decode split rows of device-side lengths in proportion to them). */
int mla_fa_version(void);

/*
 * Number of KV splits the library picks when a call passes n_split = 0, for a call
 * with n_rows = n_seq * n_tok query rows.  Split-KV: each split attends to one range
 * of keys and leaves a partial (m, l, O); the partials are merged with the same
 * rescale-by-new-max rule the online softmax applies between tiles.  The automatic plan
 * fills the current device's compute units (256 on an MI355X, and 256 when no device is
 * visible), so size a workspace with the device the call will run on current.
 */
int mla_fa_auto_splits(int n_rows, int n_head, int64_t n_kv, int kv_type);

/*
 * Workspace bytes a call with these sizes needs (0 when n_split resolves to 1).
 * n_split = 0 means the automatic choice.  The workspace holds the split partials (per
 * split, row and head: fp32 m and l, and the unnormalised O as f16 values with an fp32
 * power-of-two scale per 256-column half, 1040 bytes in all) and a 1 KiB tail (the
 * length-proportional split plan's row table, see mla_fa_attend).  Calls rewrite what
 * they read; it needs no initialisation.
 */
size_t mla_fa_workspace_size(int n_rows, int n_head, int64_t n_kv, int kv_type, int n_split);

/*
 * Decode: n_seq sequences, one query token each.
 *   q              [n_seq][n_head][576] f16/bf16 bits (16-byte aligned).
 *   kv             row j of sequence s at kv + s*kv_seq_stride + j*kv_row_stride
 *                  (bytes).  f16/bf16: 16-byte aligned base and strides; Q8_0:
 *                  4-byte aligned, kv_row_stride at most 2^26.  kv_seq_stride may
 *                  be 0 (shared cache).
 *   n_kv           rows per sequence, 1 .. 2^31-1.
 *   mask           NULL, or f16 bits [n_seq][mask_seq_stride] (elements); element
 *                  (s, j) is added to score j of every head of sequence s.
 *   kv_idx         NULL for dense decoding.  Otherwise the sparse path: per
 *   kv_idx_count   sequence s, kv_idx[s*idx_seq_stride + c] for c < kv_idx_count[s]
 *   idx_seq_stride is an ascending list of cache rows to attend to (as written by
 *                  fa_mask_compact); both arrays live on the device, the count is
 *                  read by the kernels, so there is no host synchronisation.  The
 *                  mask, if given, is still added at the gathered rows.  Entries
 *                  must lie in [0, n_kv); the kernels clamp any that do not (the
 *                  result is then unspecified, but no read leaves the cache).
 *   scale          finite fp32 softmax scale (e.g. 1/sqrt(192)).
 *   out            [n_seq][n_head][512] fp32.
 *   n_split        0 = automatic, else 1 .. 1024 KV splits.  With kv_idx and more than
 *                  one sequence, a split call shares its partial slots out by the lists'
 *                  lengths, as mla_fa_attend describes.
 *   workspace      device buffer of at least mla_fa_workspace_size(n_seq, n_head,
 *                  n_kv, kv_type, n_split) bytes (may be NULL when that is 0).
 */
int mla_fa_decode(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                  int64_t kv_seq_stride, int n_seq, int n_head, int64_t n_kv,
                  const uint16_t *mask, int64_t mask_seq_stride, const int32_t *kv_idx,
                  const int32_t *kv_idx_count, int64_t idx_seq_stride, float scale, float *out,
                  int n_split, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two phases of mla_fa_decode, for callers that time or overlap them.
 * mla_fa_decode_partials runs the split attention and, for n_split > 1, leaves the
 * partials in the workspace (for n_split == 1 it writes `out` directly and there is
 * nothing to merge).  mla_fa_merge_partials combines the partials of a previous
 * mla_fa_decode_partials call with the same n_rows (= n_seq), n_head, n_split and
 * workspace into `out`.  mla_fa_decode is exactly these two calls in order, except with
 * kv_idx over several sequences: there it shares the slots out by the lists' lengths,
 * while the two phases keep n_split pieces per row so that the merge needs only the
 * sizes (the results differ by floating-point reassociation alone).
 */
int mla_fa_decode_partials(const void *q, int q_type, const void *kv, int kv_type,
                           int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq, int n_head,
                           int64_t n_kv, const uint16_t *mask, int64_t mask_seq_stride,
                           const int32_t *kv_idx, const int32_t *kv_idx_count,
                           int64_t idx_seq_stride, float scale, float *out, int n_split,
                           void *workspace, size_t workspace_bytes, void *stream);
int mla_fa_merge_partials(int n_rows, int n_head, int n_split, float *out, const void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * mla_fa_decode for callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * computation, arguments and errors as mla_fa_decode, without the workspace.  The split
 * partials live in a library-owned scratch array of MLA_FA_NOALLOC_SCRATCH_BYTES in
 * device memory, one per GPU, held until the process ends; the call allocates nothing.
 * It uses the scratch of the current device, which must be the device of `stream`.
 *   - The automatic split count (n_split = 0, no MLA_FA_NSPLIT override) always fits:
 *     its partials never exceed 42,598,400 bytes (80 rows of 128 heads, Q8_0, 4 splits).
 *     A call whose partials (mla_fa_workspace_size with the same sizes) exceed the
 *     scratch returns MLA_FA_ERR_WORKSPACE and enqueues nothing.
 *   - Every call on one GPU shares that GPU's scratch and fully rewrites what it reads,
 *     so nothing needs clearing; calls that overlap on one GPU (other streams, other
 *     threads) race on it and must be serialised by the caller.
 *   - The first call on each device looks up the scratch's device address (no
 *     allocation); a failure there returns MLA_FA_ERR_HIP.
 */
#define MLA_FA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
int mla_fa_decode_noalloc(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                          int64_t kv_seq_stride, int n_seq, int n_head, int64_t n_kv, const uint16_t *mask,
                          int64_t mask_seq_stride, const int32_t *kv_idx, const int32_t *kv_idx_count,
                          int64_t idx_seq_stride, float scale, float *out, int n_split, void *stream);

/*
 * Chunked prefill: n_tok query tokens of one sequence against its cache of n_kv rows
 * (the chunk's tokens are the last n_tok positions of the cache).
 *   q        [n_tok][n_head][576] f16/bf16 bits.
 *   kv       row j at kv + j*kv_row_stride (bytes), alignment as for decode.
 *   causal   nonzero: token t attends to keys j <= n_kv - n_tok + t; requires
 *            n_tok <= n_kv.
 *   mask     NULL, or f16 bits [n_tok][mask_row_stride], added per (token, key).
 *   out      [n_tok][n_head][512] fp32.
 *   n_split / workspace as for decode (with n_rows = n_tok).
 */
int mla_fa_prefill(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                   int n_tok, int n_head, int64_t n_kv, int causal, const uint16_t *mask,
                   int64_t mask_row_stride, float scale, float *out, int n_split,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Batched attention over per-sequence caches of different lengths, with the logit
 * softcap, ALiBi slopes and attention sinks that the Metal tensor-API flash-attention
 * kernel supports for the 576/512 shape ("llama.cpp Metal: tensor-API flash attention
 * for F16 KV caches" news item; the pages name the features, the readings below are
 * the plain ones), and sparse attention over one compacted index list per query token
 * ("llama.cpp Vulkan backend adds sparse Flash Attention for quantized K/V": one mask
 * row per query, compacted, feeding the sparse attention).  mla_fa_decode is the
 * special case n_tok = 1, kv_len = NULL, causal = 0 and no extras.
 *   q        [n_seq][n_tok][n_head][576] f16/bf16 bits (device).
 *   kv       row j of sequence s at kv + s*kv_seq_stride + j*kv_row_stride (bytes);
 *            n_kv rows of capacity per sequence; alignment as for decode.
 *   kv_len   NULL (every sequence holds n_kv cells), or int32 [n_seq] (device): the
 *            valid cells of each sequence, clamped to [0, n_kv].
 *   causal   nonzero: token t of sequence s attends to cells j <= L_s - n_tok + t (L_s
 *            its valid length; a row left with no cell outputs 0).  Without kv_len it
 *            requires n_tok <= n_kv.
 *   mask     NULL, or f16 bits, element (s, t, j) at s*mask_seq_stride +
 *            t*mask_tok_stride + j: -inf drops the cell, other values add to the score.
 *   kv_idx   NULL for dense rows.  Otherwise the sparse path: row (s, t) attends only to
 *   kv_idx_count  the cells kv_idx[s*idx_seq_stride + t*idx_tok_stride + c] for
 *   idx_seq_stride, idx_tok_stride   c < kv_idx_count[s*n_tok + t], an ascending list
 *            as fa_mask_compact writes for the n_seq*n_tok mask rows (device arrays,
 *            int32, 4-byte aligned; the counts are read on the device).  The mask, if
 *            given, is still added at the gathered cells.  Entries must lie in
 *            [0, n_kv) (the kernels clamp any that do not; the result is then
 *            unspecified).  Requires causal = 0 and kv_len = NULL: the list alone says
 *            which cells a row sees.  Strides are elements, each at least n_kv where
 *            more than one sequence / token uses it.
 *   alibi_slopes NULL, or fp32 [n_head] (device): the bias of a kept cell for head h is
 *            alibi_slopes[h] times its mask value (dropped cells stay dropped).
 *   sinks    NULL, or fp32 [n_head] (device): a per-head logit that joins the softmax
 *            normaliser as one more term exp(sinks[h] - m) carrying no value.
 *   softcap  0 = off; > 0: the scaled score x = scale * q.k becomes
 *            softcap * tanh(x / softcap) before the mask bias is added.
 *   out      [n_seq][n_tok][n_head][512] fp32 (device).
 *   n_split / workspace as for decode with n_rows = n_seq * n_tok.  When the call
 *            splits (n_split resolves to 2 or more), has kv_len or kv_idx, and
 *            n_seq * n_tok <= 256, the rows' lengths are known on the device only, so
 *            the kernels share the workspace's n_rows * n_split partial slots out in
 *            proportion to them (long rows get more pieces, empty rows none; at most one
 *            piece per workgroup the chip runs at once) instead of cutting every row
 *            into n_split pieces: n_split then sets the workspace size, not a per-row
 *            count.  The results differ only by floating-point reassociation.
 * Errors: as for decode; ERR_INVALID also for a negative or non-finite softcap, for
 * kv_len / alibi_slopes / sinks not 4-byte aligned, and for kv_idx with causal or kv_len.
 */
int mla_fa_attend(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                  int64_t kv_seq_stride, int n_seq, int n_tok, int n_head, int64_t n_kv,
                  const int32_t *kv_len, int causal, const uint16_t *mask, int64_t mask_seq_stride,
                  int64_t mask_tok_stride, const int32_t *kv_idx, const int32_t *kv_idx_count,
                  int64_t idx_seq_stride, int64_t idx_tok_stride, const float *alibi_slopes,
                  const float *sinks, float softcap, float scale, float *out, int n_split, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * Per-head attention with separate keys and values: the non-absorbed MLA shape, where
 * every head has its own 192-wide key (128 dims + 64 RoPE) and 128-wide value
 * ("llama.cpp Metal: tensor-API flash attention for F16 KV caches" news item lists
 * DK=192 / DV=128 beside 576/512; "Vulkan backend fused Flash Attention: DeepSeek MLA
 * local inference", section 3.3, describes the decompressed per-head K and V).  Same
 * online softmax and mask convention as the latent entry points; for token t, head h:
 *     s_j = scale * <q[t][h], k[j][h]> + mask[t][j]     (-inf past the causal edge)
 *     out[t][h] = sum_j softmax(s)_j * v[j][h]           (zeros when no key is kept)
 *   q        [n_tok][n_head][192] f16/bf16 bits (device), 16-byte aligned.
 *   k, v     key j of head h at k + j*k_row_stride + h*384 and v + j*v_row_stride + h*256
 *            (bytes; device; 16-byte aligned, strides multiples of 16 and at least
 *            n_head*384 and n_head*256).  kv_type must equal q_type (f16 or bf16).
 *   causal   nonzero: token t attends to keys j <= n_kv - n_tok + t; requires n_tok <= n_kv.
 *   mask     NULL, or f16 bits, token t's row at mask + t*mask_row_stride (elements),
 *            16-byte aligned with mask_row_stride a multiple of 8 (>= n_kv when n_tok > 1).
 *            It is read in aligned 16-byte blocks: the block holding key n_kv - 1 may reach
 *            up to 7 elements past the row; those values are never used.
 *   out      [n_tok][n_head][128] fp32 (device), 16-byte aligned.
 * One launch, no workspace: a workgroup holds 256 tokens of one head in registers and
 * streams that head's keys and values through LDS.  1 <= n_head <= 65535,
 * 1 <= n_kv <= 2^31-1.  Errors: ERR_INVALID for null pointers, sizes, strides and
 * alignment as above; ERR_UNSUPPORTED for other type pairs.
 */
int mla_fa_prefill_mha(const void *q, int q_type, const void *k, const void *v, int kv_type,
                       int64_t k_row_stride, int64_t v_row_stride, int n_tok, int n_head, int64_t n_kv,
                       int causal, const uint16_t *mask, int64_t mask_row_stride, float scale,
                       float *out, void *stream);

/*
 * Latent attention with the absorbed per-head projections either side, from per-head
 * query parts to per-head outputs.  The per-head up-projection of the latent cache is
 * split into W_UK (128 key dims from the 512 latent) and W_UV (128 value dims from the
 * latent); W_UK is folded into the query and W_UV applied to the attention output
 * instead of decompressing every cached row ("ik_llama.cpp -mla flag deep-dive": wkv_b
 * split per head into wk_b / wv_b; "Vulkan backend fused Flash Attention: DeepSeek MLA
 * local inference", sections 3.2-3.3 and 6.1).  For row r = (s, t) and head h:
 *     q_lat = W_UK[h] q_nope[r][h]                  (512; rounded to q_type on the GPU)
 *     O     = latent attention of [q_lat, q_pe[r][h]] as mla_fa_attend computes it
 *     out[r][h] = W_UV[h] O                         (128; O as a q_type head plus the
 *                                                    q_type rounding of its remainder,
 *                                                    two MFMA operands, fp32 accumulation)
 *   q_nope   [n_seq][n_tok][n_head][128], q_pe [n_seq][n_tok][n_head][64]: q_type bits
 *            (f16 or bf16), device, 16-byte aligned.
 *   w_uk     [n_head][512][128], w_uv [n_head][128][512]: q_type bits, stored
 *            output-major (a linear layer's [out][in]), device, 16-byte aligned.
 *   kv, kv_row_stride, kv_seq_stride, n_kv, kv_len, causal, mask, mask strides, scale:
 *            as for mla_fa_attend (scale is typically 1/sqrt(192)).
 *   out      [n_seq][n_tok][n_head][128] fp32, device, 16-byte aligned.
 *   workspace  device, 256-byte aligned, at least mla_fa_absorbed_workspace_size(
 *            n_seq*n_tok, n_head, n_kv, kv_type, n_split) bytes: it holds the 576-wide
 *            queries, the latent outputs and the split partials.
 * Three launches on `stream`: the query projection (with the q_pe copy), the attention,
 * then the output projection, which for a split plan is fused with the merge of the
 * split partials (the epilogue reads the partials and W_UV; the merged latent output
 * never reaches memory).  With kv_len, a split plan shares its partial slots out by the
 * rows' lengths as mla_fa_attend does.  Errors as for mla_fa_attend; ERR_WORKSPACE when
 * the workspace is missing or short.
 */
size_t mla_fa_absorbed_workspace_size(int n_rows, int n_head, int64_t n_kv, int kv_type, int n_split);
int mla_fa_absorbed(const void *q_nope, const void *q_pe, int q_type, const void *w_uk, const void *w_uv,
                    const void *kv, int kv_type, int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq,
                    int n_tok, int n_head, int64_t n_kv, const int32_t *kv_len, int causal, const uint16_t *mask,
                    int64_t mask_seq_stride, int64_t mask_tok_stride, float scale, float *out, int n_split,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sparse-mask index compaction.  For each of n_rows f16 mask rows (row r at
 * mask + r*mask_row_stride elements, n_kv cells), writes the ascending list of cells
 * whose mask is not -inf (bit pattern != 0xFC00) to idx + r*idx_row_stride and its
 * length to count[r].  Entries of idx past count[r] are left untouched.  One
 * workgroup per row: each wavefront owns one contiguous segment of the row, counts
 * its kept cells with ballots over coalesced loads, one exclusive scan over the
 * segment counts gives every segment its output offset, then each wavefront writes
 * its cells.  idx_row_stride >= n_kv; n_kv <= 2^31-1.
 */
int fa_mask_compact(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                    int32_t *idx, int64_t idx_row_stride, int32_t *count, void *stream);

/*
 * The same compaction (same result, bit for bit) spread over many workgroups per row,
 * for rows of up to 2^22 cells whose rows start 16-byte aligned (mask 16-byte aligned,
 * and mask_row_stride a multiple of 8 when n_rows > 1), and n_rows <= 65535.  Each row
 * is cut into 4096-cell chunks: a first launch counts the kept cells of every chunk into
 * the workspace; a second gives each chunk its output offset (the sum of the counts
 * before it) and writes its cells.  The mask is read twice, by many CUs instead of one.
 *   workspace   device, 4-byte aligned, at least fa_mask_compact_workspace_size(n_rows,
 *               n_kv) bytes (the chunk counts; fully rewritten, no initialisation).
 * Calls outside those limits run fa_mask_compact's kernel and leave the workspace
 * untouched.  Errors as for fa_mask_compact, and ERR_WORKSPACE when the chunked form
 * applies and the workspace is missing or short.  Calls that share a workspace on
 * different streams race.
 */
size_t fa_mask_compact_workspace_size(int n_rows, int64_t n_kv);
int fa_mask_compact_ws(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                       int32_t *idx, int64_t idx_row_stride, int32_t *count, void *workspace,
                       size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_FA_H */
