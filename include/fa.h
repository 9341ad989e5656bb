/*
 * fa.h - C ABI of the MI355X (gfx950) fused exact-attention forward library.
 *
 * The library computes O = softmax(scale * Q K^T) V per (sequence, query head)
 * without writing S or P to memory, and the natural-log log-sum-exp of every
 * row ("Attention kernels: FlashAttention and PagedAttention", sections 2.1,
 * 3.2 and 4.3).  Each entry point enqueues its kernels on the caller's HIP
 * stream and returns; nothing is synchronised.
 *
 * Conventions shared by every entry point
 *   - Element type: Q, K, V and O are bfloat16 (passed as untyped pointers),
 *     LSE is float32.  Head dimension d is 64 or 128.
 *   - Pointers are device pointers owned by the caller.  Inputs are only read.
 *     The library keeps no pointer after the call returns and never frees
 *     caller memory.  The first call on a device queries device attributes
 *     and the kernels' occupancy; no call allocates device memory.
 *   - Strides are in elements; the last (head_dim) dimension must be
 *     contiguous (stride 1) and every row must start 16-byte aligned.
 *   - stream is a hipStream_t (NULL = the null stream).
 *   - Return value: FA_OK, or a negative code with nothing enqueued:
 *       FA_ERR_INVALID_ARG  null pointer, negative or zero size, bad stride or
 *                           alignment, heads_q not a multiple of heads_kv,
 *                           workspace too small, num_splits < 0, a page_size
 *                           that is not a multiple of 16 ("Attention kernels
 *                           ...", section 6.1: pages of 16-multiple tokens);
 *       FA_ERR_UNSUPPORTED  a head_dim other than 64 or 128, a K or V token
 *                           (or cache slot) stride of 2^25 elements or more,
 *                           or a shape the kernels do not cover (stated per
 *                           entry point);
 *       FA_ERR_HIP          a HIP runtime error while launching.
 *     fa_last_error() returns a message for the calling thread's last failure.
 *   - Rows that see no key at all get O = 0 and LSE = -inf (no NaN).
 *   - Results are bitwise reproducible for fixed arguments.
 *
 * Masking options (fa_attn_opts), from the pages' statement of the problem
 * ("FA4 (CuTeDSL) and engineering interfaces", sections 3, 6.2 and 7):
 *   softmax_scale  > 0: used as is; <= 0 or NaN: d^-0.5.
 *   causal         non-zero: query t of a sequence with Lq queries and Lk keys
 *                  sits at key position p = t + Lk - Lq (bottom-right) and sees
 *                  keys j <= p.  Equal to top-left alignment when Lq == Lk.
 *   window_left,   sliding window: row at position p sees keys in
 *   window_right   [p - window_left, p + window_right] (inclusive); a negative
 *                  bound is unbounded on that side.
 *   softcap        > 0: logits become softcap * tanh(scale * q.k / softcap)
 *                  before the softmax; 0 = off.
 *   pack_gqa       > 0: fold the heads_q / heads_kv query heads that share a
 *                  KV head into the rows of one tile so each K/V tile is read
 *                  once for all of them ("FA4 ...", section 5; "Attention
 *                  kernels ...", section 5.3); 0: one tile per query head;
 *                  < 0: pick automatically (on when heads_q > heads_kv).
 *   alibi_slopes   NULL: off.  Else device float32 slopes, slope of (batch b,
 *                  query head h) at alibi_slopes[b * alibi_batch_stride + h]
 *                  (stride 0: one row of heads_q slopes for every batch; in the
 *                  varlen call the batch index is the sequence): the logit of
 *                  a query at position p and key j gets -slope * |p - j|
 *                  ("FA4 ...", section 7, alibi_slopes), p bottom-right as for
 *                  causal.  fa_fwd, fa_fwd_varlen and the kvcache calls
 *                  (fa_fwd_kvcache_paged, its _noalloc and _fp8 variants: the
 *                  batch index is the sequence), without softcap; other entry
 *                  points return FA_ERR_UNSUPPORTED.
 */
#ifndef EXACT_ATTENTION_72_FA_H
#define EXACT_ATTENTION_72_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_ERR_INVALID_ARG (-1)
#define FA_ERR_UNSUPPORTED (-2)
#define FA_ERR_HIP (-3)

typedef struct fa_attn_opts {
  float softmax_scale;
  int causal;
  int window_left;
  int window_right;
  float softcap;
  int pack_gqa;
  const float* alibi_slopes;
  int64_t alibi_batch_stride;
} fa_attn_opts;

/* Dense (padded) attention forward ("FA4 ...", section 3 flash_attn_func).
 *   q   [batch, seqlen_q, heads_q,  head_dim]  strides q_strides  = {batch, seq, head}
 *   k   [batch, seqlen_k, heads_kv, head_dim]  strides k_strides
 *   v   [batch, seqlen_k, heads_kv, head_dim]  strides v_strides
 *   out [batch, seqlen_q, heads_q,  head_dim]  strides o_strides   (written)
 *   lse [batch, heads_q, seqlen_q] float32, dense                  (written; may be NULL)
 * Query head h uses KV head h / (heads_q / heads_kv). */
int fa_fwd(const fa_attn_opts* opts, const void* q, const void* k, const void* v, void* out,
           float* lse, int batch, int seqlen_q, int seqlen_k, int heads_q, int heads_kv,
           int head_dim, const int64_t q_strides[3], const int64_t k_strides[3],
           const int64_t v_strides[3], const int64_t o_strides[3], void* stream);

/* Dense forward with a learned relative-position bias, the first of the two
 * score_mod / mask_mod hooks built into the library ("FA4 ...", sections 1 and 7:
 * a score_mod rewrites each logit after Q K^T, before the softmax; the hook is a
 * compile-time kernel specialisation, declared in fa_mods.h).  The logit of the
 * query at position p (token t, p = t + seqlen_k - seqlen_q) and key j becomes
 *   softmax_scale * q.k + bias[h * (2 * max_distance + 1) + clamp(j - p, -max_distance,
 *   max_distance) + max_distance]
 * with bias a device float32 table [heads_q, 2 * max_distance + 1] (relative
 * distances beyond max_distance share the end entries).  Arguments, masks and
 * results otherwise as fa_fwd (causal and window apply; pack_gqa as fa_fwd).
 * Errors: FA_ERR_INVALID_ARG for a NULL or misaligned bias or max_distance
 * outside [0, 2^30]; FA_ERR_UNSUPPORTED with softcap or alibi_slopes. */
int fa_fwd_relpos_bias(const fa_attn_opts* opts, const void* q, const void* k, const void* v,
                       void* out, float* lse, int batch, int seqlen_q, int seqlen_k, int heads_q,
                       int heads_kv, int head_dim, const float* bias, int max_distance,
                       const int64_t q_strides[3], const int64_t k_strides[3],
                       const int64_t v_strides[3], const int64_t o_strides[3], void* stream);

/* Dense forward with a prefix-LM mask, the second built-in hook (a mask_mod,
 * "FA4 ...", sections 1 and 7): the first prefix_lens[b] keys of batch b are
 * visible to every query (a bidirectional prefix), later keys causally: key j is
 * visible to the query at position p (= t + seqlen_k - seqlen_q) iff
 * j < prefix_lens[b] or j <= p, intersected with the sliding window if one is set.
 * prefix_lens: device int32 [batch] (values <= 0 give plain causal attention,
 * values >= seqlen_k full attention).  opts->causal must be 0 (the mask replaces
 * it; FA_ERR_INVALID_ARG otherwise).  Other arguments and results as fa_fwd.
 * Errors as fa_fwd_relpos_bias, with prefix_lens in place of bias. */
int fa_fwd_prefix_lm(const fa_attn_opts* opts, const void* q, const void* k, const void* v,
                     void* out, float* lse, int batch, int seqlen_q, int seqlen_k, int heads_q,
                     int heads_kv, int head_dim, const int32_t* prefix_lens,
                     const int64_t q_strides[3], const int64_t k_strides[3],
                     const int64_t v_strides[3], const int64_t o_strides[3], void* stream);

/* Variable-length attention forward over packed sequences ("FA4 ...", section 4;
 * "Attention kernels ...", section 7.1).  Sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b], cu_seqlens_k[b+1]);
 * attention never crosses sequences.
 *   q   [total_q, heads_q,  head_dim]  strides q_strides = {token, head}
 *   k,v [total_k, heads_kv, head_dim]  strides k_strides, v_strides
 *   out [total_q, heads_q,  head_dim]  strides o_strides (written)
 *   lse [heads_q, total_q] float32 (written; may be NULL)
 *   cu_seqlens_q, cu_seqlens_k: device int32 [batch + 1], non-decreasing, starting at 0.
 *   max_seqlen_q: an upper bound of the query lengths (sizes the launch).
 * Caller contract, not checked on the device: cu_seqlens_q[batch] == total_q,
 * cu_seqlens_k[batch] <= total_k, every query length <= max_seqlen_q. */
int fa_fwd_varlen(const fa_attn_opts* opts, const void* q, const void* k, const void* v,
                  void* out, float* lse, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int batch, int max_seqlen_q, int total_q,
                  int total_k, int heads_q, int heads_kv, int head_dim,
                  const int64_t q_strides[2], const int64_t k_strides[2],
                  const int64_t v_strides[2], const int64_t o_strides[2], void* stream);

/* Attention of new queries against a paged KV cache, with split-KV
 * ("FA4 ...", sections 6.1 and 6.2; "Attention kernels ...", sections 6.1 and 6.3).
 * Logical key t of sequence b lives in page block_table[b][t / page_size] at slot
 * t % page_size.  The keys are cut into num_splits contiguous page ranges; each
 * range produces a normalised partial O and its LSE, which a combine kernel merges
 * on the same stream.  With num_splits == 1 the result is written directly;
 * num_splits == 0 takes fa_kvcache_num_splits(...).
 * Chunked prefill ("Attention kernels ...", section 5.1): when a sequence has
 * more than 32 packed query rows (seqlen_q * heads_q / heads_kv) the queries
 * run through the prefill kernel over the paged cache, bottom-right aligned
 * (query t sits at key position t + cache_seqlens[b] - seqlen_q); then
 * num_splits must resolve to 1 and page_size must be a multiple of 16.
 *   q        [batch, seqlen_q, heads_q, head_dim]  strides q_strides = {batch, seq, head}
 *   k_cache  [num_pages, page_size, heads_kv, head_dim]  strides k_strides = {page, slot, head}
 *   v_cache  same shape, strides v_strides
 *   block_table  device int32 [batch, max_blocks_per_seq] (row stride max_blocks_per_seq)
 *   cache_seqlens device int32 [batch]: keys per sequence (Lk)
 *   out      [batch, seqlen_q, heads_q, head_dim]  strides o_strides (written)
 *   lse      [batch, heads_q, seqlen_q] float32 (written; may be NULL)
 *   workspace: device memory of at least fa_kvcache_workspace_size(...) bytes
 *              (may be NULL when that size is 0); holds the fp32 partials.
 * opts->pack_gqa applies to chunked prefill only (decode always packs).
 * Errors: FA_ERR_UNSUPPORTED for num_splits > 1 with more than 32 packed rows.
 * Caller contract, not checked on the device: block_table entries of live pages
 * lie in [0, num_pages) and cache_seqlens[b] <= max_blocks_per_seq * page_size. */
int fa_fwd_kvcache_paged(const fa_attn_opts* opts, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table,
                         const int32_t* cache_seqlens, void* out, float* lse, int batch,
                         int seqlen_q, int heads_q, int heads_kv, int head_dim,
                         int64_t num_pages, int page_size, int max_blocks_per_seq,
                         int num_splits, void* workspace, size_t workspace_bytes,
                         const int64_t q_strides[3], const int64_t k_strides[3],
                         const int64_t v_strides[3], const int64_t o_strides[3],
                         void* stream);

/* fa_fwd_kvcache_paged over an FP8 (OCP e4m3) KV cache: the cache holds one byte
 * per element, and logical key / value element x of every row is code * k_scale /
 * code * v_scale ("Attention kernels ...", section 5.2: a KV cache stored in FP8
 * halves the bytes a decode step reads, and decode time is those bytes over the
 * bandwidth).  Q, O and LSE are as in fa_fwd_kvcache_paged.  The codes are
 * widened to bf16 exactly and the products run in bf16 with fp32 accumulation;
 * k_scale multiplies the softmax scale (and the softcap argument) and v_scale
 * multiplies O, so the result is attention over the dequantized cache.
 *   k_cache, v_cache  uint8 [num_pages, page_size, heads_kv, head_dim], strides in
 *                     BYTES {page, slot, head}, every row 16-byte aligned
 *   k_scale, v_scale  finite, > 0 (one scale per tensor)
 * Write the cache with fa_kvcache_append_fp8 (same scales).  The other arguments,
 * the workspace and num_splits are those of fa_fwd_kvcache_paged.
 * Errors: FA_ERR_INVALID_ARG for a scale that is not finite and positive;
 * FA_ERR_UNSUPPORTED for more than 32 packed rows (seqlen_q * heads_q / heads_kv:
 * FP8 caches are read by the decode kernel only).  A NaN code reads
 * as NaN and poisons the rows that see it, like a NaN in a bf16 cache. */
int fa_fwd_kvcache_paged_fp8(const fa_attn_opts* opts, const void* q, const void* k_cache,
                             const void* v_cache, float k_scale, float v_scale,
                             const int32_t* block_table, const int32_t* cache_seqlens, void* out,
                             float* lse, int batch, int seqlen_q, int heads_q, int heads_kv,
                             int head_dim, int64_t num_pages, int page_size,
                             int max_blocks_per_seq, int num_splits, void* workspace,
                             size_t workspace_bytes, const int64_t q_strides[3],
                             const int64_t k_strides[3], const int64_t v_strides[3],
                             const int64_t o_strides[3], void* stream);

/* fa_fwd_kvcache_paged for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results and errors, without the workspace.
 * The split-KV partials and the sequence order go to a static device array of
 * FA_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends; no call allocates or frees anything.  A call whose
 * partials need more than that (fa_kvcache_workspace_size(...) for the resolved
 * split count above FA_NOALLOC_SCRATCH_BYTES) returns FA_ERR_INVALID_ARG with
 * nothing enqueued.  Every call on one device shares that device's array, so
 * calls that overlap on one device (concurrent streams or host threads) race;
 * calls on one stream are ordered and safe.  The first call with num_splits > 1
 * on a device looks the array's address up once (hipGetSymbolAddress). */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int fa_fwd_kvcache_paged_noalloc(const fa_attn_opts* opts, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* cache_seqlens, void* out, float* lse, int batch,
                                 int seqlen_q, int heads_q, int heads_kv, int head_dim,
                                 int64_t num_pages, int page_size, int max_blocks_per_seq,
                                 int num_splits, const int64_t q_strides[3],
                                 const int64_t k_strides[3], const int64_t v_strides[3],
                                 const int64_t o_strides[3], void* stream);

/* Unified prefill + decode batch over a paged KV cache ("Attention kernels ...",
 * section 5.1: a batch mixes requests that prefill a chunk of hundreds or thousands
 * of queries with requests that decode one token, all against a cached prefix plus
 * the new tokens; section 6.1: paged keys).  Sequence b owns the packed query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and the cache_seqlens[b] keys of its pages,
 * the new tokens' keys included (append them first with fa_kvcache_append); its
 * queries are bottom-right aligned (query t at key position t + Lk - Lq).
 *   q        [total_q, heads_q, head_dim]  strides q_strides = {token, head}
 *   k_cache, v_cache [num_pages, page_size, heads_kv, head_dim]  strides {page, slot, head}
 *   out      [total_q, heads_q, head_dim]  strides o_strides (written)
 *   lse      [heads_q, total_q] float32 (written; may be NULL)
 *   cu_seqlens_q device int32 [batch + 1]; block_table device int32 [batch, max_blocks_per_seq];
 *   cache_seqlens device int32 [batch]; max_seqlen_q: an upper bound of the query lengths.
 *   num_splits  split-KV count for the decode requests (>= 1; 0 takes
 *               fa_varlen_paged_num_splits(...)); workspace: device memory of at least
 *               fa_varlen_paged_workspace_size(batch, heads_kv, head_dim, resolved
 *               num_splits) bytes, 16-byte aligned (may be NULL when that is 0).
 * A sequence with at most 32 packed rows (new tokens x heads_q / heads_kv) runs as
 * a decode step, one workgroup per (sequence, KV head, split) with the splits'
 * fp32 partials merged by a combine kernel ("Attention kernels ...", section 6.3);
 * the others in workgroup tiles of 128 packed rows (no split-KV); all launches on
 * the stream.  Caller contract, not checked on the device: cu_seqlens_q
 * non-decreasing from 0 with cu_seqlens_q[batch] == total_q, query lengths <=
 * max_seqlen_q, live block-table entries in [0, num_pages), cache_seqlens[b] <=
 * max_blocks_per_seq * page_size. */
int fa_fwd_varlen_paged(const fa_attn_opts* opts, const void* q, const void* k_cache,
                        const void* v_cache, void* out, float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* block_table, const int32_t* cache_seqlens, int batch,
                        int max_seqlen_q, int total_q, int heads_q, int heads_kv, int head_dim,
                        int64_t num_pages, int page_size, int max_blocks_per_seq, int num_splits,
                        void* workspace, size_t workspace_bytes, const int64_t q_strides[2],
                        const int64_t k_strides[3], const int64_t v_strides[3],
                        const int64_t o_strides[2], void* stream);

/* Split count fa_fwd_varlen_paged takes for num_splits == 0 (host only): the
 * decode requests, at most all batch sequences, are sized as one decode step
 * each, as fa_kvcache_num_splits does for seqlen_q = 1. */
int fa_varlen_paged_num_splits(int batch, int heads_q, int heads_kv, int max_blocks_per_seq);

/* Bytes of workspace fa_fwd_varlen_paged needs for a resolved num_splits >= 1: 0
 * for num_splits == 1, else num_splits * batch * heads_kv * 32 * (head_dim + 1) * 4
 * rounded up to 256 (fp32 partials of every (sequence, KV head) unit's up to 32
 * packed rows), plus, when batch <= 4096, batch * 4 rounded up to 256 (the order in
 * which the split workgroups take the sequences). */
size_t fa_varlen_paged_workspace_size(int batch, int heads_kv, int head_dim, int num_splits);

/* Split count of fa_fwd_kvcache_paged for num_splits == 0 (host only, no device
 * work; it reads the current device's compute-unit count): about 4 workgroups
 * per compute unit over batch * heads_kv and at least 2 when batch <= 4096
 * (the split workgroups then take the sequences longest first), about 32 per
 * compute unit for larger batches; at most 64 and at most max_blocks_per_seq
 * splits, and 1 when the call runs as chunked prefill ("FA4 ...", section 6.2:
 * the split count is chosen to fill the machine). */
int fa_kvcache_num_splits(int batch, int seqlen_q, int heads_q, int heads_kv, int page_size,
                          int max_blocks_per_seq);

/* Bytes of workspace fa_fwd_kvcache_paged needs for a resolved split count
 * num_splits >= 1 (resolve 0 with fa_kvcache_num_splits first; 0 and 1 give 0
 * here, so sizing with 0 under-sizes every call that resolves to more splits):
 * 0 for num_splits == 1, else
 * num_splits * batch * seqlen_q * heads_q * (head_dim + 1) * 4 rounded up to 256
 * (the fp32 partial O and LSE), plus, when batch <= 4096, batch * 4 rounded up
 * to 256 (the order in which the split workgroups take the sequences: longest
 * cache first, computed on the device from cache_seqlens). */
size_t fa_kvcache_workspace_size(int batch, int seqlen_q, int heads_q, int head_dim,
                                 int num_splits);

/* In-place append of new keys and values to a paged cache, for incremental
 * decoding ("FA4 ...", section 6.2: the kvcache call writes the new k and v into
 * the cache; "Attention kernels ...", section 6.1: logical key t of a sequence is
 * slot t % page_size of page block_table[b][t / page_size]).  Token t of
 * sequence b is written at logical position cache_seqlens[b] + t.
 *   k_new, v_new      [batch, seqlen_new, heads_kv, head_dim]  strides {batch, seq, head}
 *   k_cache, v_cache  [num_pages, page_size, heads_kv, head_dim]  strides {page, slot, head}
 *                     (written in place; nothing else in them changes)
 *   block_table       device int32 [batch, max_blocks_per_seq]
 *   cache_seqlens     device int32 [batch]: lengths before the append (read, not updated;
 *                     attend afterwards with cache_seqlens[b] + seqlen_new keys)
 *   rotary_cos, rotary_sin  NULL, or fp32 [positions, rotary_dim / 2] tables: the keys are
 *                     rotated on the way in, as fa_rotary does, at their cache position
 *                     cache_seqlens[b] + t (the values are copied as they are)
 * seqlen_new == 0 is a no-op.  Errors: FA_ERR_INVALID_ARG for one table without the
 * other or a rotary_dim that is not a multiple of 16 in [16, head_dim].  Caller
 * contract, not checked on the device: cache_seqlens[b] + seqlen_new <=
 * max_blocks_per_seq * page_size (and <= the tables' positions), the pages those
 * positions map to lie in [0, num_pages), and no two sequences map a written position
 * to the same slot. */
int fa_kvcache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_table, const int32_t* cache_seqlens, int batch,
                      int seqlen_new, int heads_kv, int head_dim, int64_t num_pages,
                      int page_size, int max_blocks_per_seq, const int64_t kn_strides[3],
                      const int64_t vn_strides[3], const int64_t k_strides[3],
                      const int64_t v_strides[3], const float* rotary_cos,
                      const float* rotary_sin, int rotary_dim, int rotary_interleaved,
                      void* stream);

/* fa_kvcache_append for an FP8 (OCP e4m3) cache: each new bf16 element x is
 * written as the e4m3 code of the fp32 quotient x / k_scale (keys) or x / v_scale
 * (values), rounded to nearest with ties to even and saturated at +-448 ("Attention
 * kernels ...", section 5.2: the KV cache stored in FP8).  The caches are uint8
 * [num_pages, page_size, heads_kv, head_dim] with strides in BYTES, rows 16-byte
 * aligned; the other arguments are those of fa_kvcache_append, without the rotary
 * tables (rotate the new keys first with fa_rotary).  New values must be finite
 * (a NaN is written as a NaN code).
 * Errors: FA_ERR_INVALID_ARG for a scale that is not finite and positive. */
int fa_kvcache_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          float k_scale, float v_scale, const int32_t* block_table,
                          const int32_t* cache_seqlens, int batch, int seqlen_new, int heads_kv,
                          int head_dim, int64_t num_pages, int page_size, int max_blocks_per_seq,
                          const int64_t kn_strides[3], const int64_t vn_strides[3],
                          const int64_t k_strides[3], const int64_t v_strides[3], void* stream);

/* In-place rotary position embedding of x [batch, seqlen, heads, head_dim] (bf16,
 * strides x_strides = {batch, seq, head}), for the new queries of a kvcache step
 * ("FA4 ...", section 6.2: the kvcache call can apply the rotary embedding on the
 * way).  Token t of sequence b sits at position (position_base ? position_base[b] :
 * 0) + t.  Frequency i of that position rotates a pair of dims by the angle whose
 * cosine and sine are cos[pos * rotary_dim / 2 + i] and sin[...] (fp32 tables
 * [positions, rotary_dim / 2], chosen by the caller):
 *   interleaved == 0: dims (i, i + rotary_dim / 2);  interleaved != 0: dims (2i, 2i + 1);
 *   (a, b) -> (a cos - b sin, a sin + b cos), fp32, rounded to bf16 (nearest even).
 * Dims at and past rotary_dim are unchanged.  rotary_dim: a multiple of 16 in
 * [16, head_dim].  Caller contract: every position is a row of the tables. */
int fa_rotary(void* x, int batch, int seqlen, int heads, int head_dim,
              const int64_t x_strides[3], const int32_t* position_base, const float* cos,
              const float* sin, int rotary_dim, int interleaved, void* stream);

/* Backward pass of the dense forward ("Attention kernels ...", section 4.3: the
 * backward recomputes S = Q K^T by blocks and P = exp(S - L) from the saved
 * log-sum-exp L, then dV = P^T dO and dS; "01 FlashAttention project overview &
 * architecture", section 1 directory map: a preprocess forms D_i = rowsum(dO_i * O_i)).  With
 * dP = dO V^T and dS = P (dP - D):  dQ = scale dS K,  dK = scale dS^T Q,
 * dV = P^T dO, where dK and dV of a KV head sum over the query heads that share it.
 *   q, out, dout, dq  [batch, seqlen_q, heads_q, head_dim]  (strides {batch, seq, head})
 *   k, v, dk, dv      [batch, seqlen_k, heads_kv, head_dim]
 *   lse               float32 [batch, heads_q, seqlen_q]: the forward's LSE (natural log)
 *   dq, dk, dv        bf16, written (every element, zeros where nothing flows)
 *   workspace         device memory of at least fa_bwd_workspace_size(...) bytes (holds D and
 *                     the LSE in base-2 units per query row)
 * opts as for fa_fwd (same scale, causal, window, softcap).  With softcap c the logit is
 * c tanh(scale q.k / c), so dS is multiplied by 1 - tanh^2(scale q.k / c) before dQ and dK (the
 * chain rule through the forward's transform, "FA4 ...", section 7); ALiBi is
 * FA_ERR_UNSUPPORTED, and so are a token stride of q or dout of 2^25 elements or more and
 * batch * heads_q * seqlen_q * 4 above 2^31 - 256 bytes (32-bit offsets in the kernels).
 * Two kernels on the stream: dQ (per query block; it also forms D and the base-2 LSE of its
 * rows in the workspace), then dK/dV (per key block).  Deterministic: no atomics. */
int fa_bwd(const fa_attn_opts* opts, const void* q, const void* k, const void* v, const void* out,
           const float* lse, const void* dout, void* dq, void* dk, void* dv, int batch,
           int seqlen_q, int seqlen_k, int heads_q, int heads_kv, int head_dim,
           const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
           const int64_t o_strides[3], const int64_t do_strides[3], const int64_t dq_strides[3],
           const int64_t dk_strides[3], const int64_t dv_strides[3], void* workspace,
           size_t workspace_bytes, void* stream);

/* fa_bwd for packed variable-length sequences (the layout of fa_fwd_varlen):
 * sequence b's queries are tokens cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1 and
 * its keys cu_seqlens_k[b] .. cu_seqlens_k[b + 1] - 1, each sequence bottom-right
 * aligned on its own ("FA4 ...", sections 3 and 4: the varlen call has the same
 * autograd as the dense one).
 *   q, out, dout, dq  [total_q, heads_q, head_dim]  (strides {token, head})
 *   k, v, dk, dv      [total_k, heads_kv, head_dim]
 *   lse               float32 [heads_q, total_q]: fa_fwd_varlen's LSE
 *   cu_seqlens_q/_k   device int32 [batch + 1]; max_seqlen_q / max_seqlen_k: upper
 *                     bounds of the lengths (they size the grids)
 *   workspace         at least fa_bwd_workspace_size(1, total_q, heads_q) bytes
 * Errors and the rest as fa_bwd (also K/V token strides of 2^25 elements or more are
 * FA_ERR_UNSUPPORTED).  Caller contract, not checked on the device: cu_seqlens_q[batch]
 * == total_q, cu_seqlens_k[batch] <= total_k, every length <= its maximum. */
int fa_bwd_varlen(const fa_attn_opts* opts, const void* q, const void* k, const void* v,
                  const void* out, const float* lse, const void* dout, void* dq, void* dk,
                  void* dv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                  int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int heads_q,
                  int heads_kv, int head_dim, const int64_t q_strides[2], const int64_t k_strides[2],
                  const int64_t v_strides[2], const int64_t o_strides[2],
                  const int64_t do_strides[2], const int64_t dq_strides[2],
                  const int64_t dk_strides[2], const int64_t dv_strides[2], void* workspace,
                  size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_bwd needs: twice batch * heads_q * seqlen_q * 4 rounded up to 256
 * (D and the base-2 LSE of every query row). */
size_t fa_bwd_workspace_size(int batch, int seqlen_q, int heads_q);

/* FP8 (OCP e4m3) forward ("Attention kernels ...", section 4.2, the FP8 item;
 * "01 FlashAttention project overview & architecture", section 2.2): Q, K and V
 * enter the matrix products as e4m3 codes (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinity, largest magnitude 448) with fp32 scales: Q per
 * (batch, head, block of FA_FP8_Q_BLOCK rows), K per (batch, KV head, block of
 * FA_FP8_K_BLOCK keys), V per (batch, KV head).  A value is code * scale. */
#define FA_FP8_Q_BLOCK 128
#define FA_FP8_K_BLOCK 64

/* Per-block quantizer.  x bf16 [batch, seqlen, heads, head_dim] (x_strides in
 * elements) -> codes e4m3 [batch, seqlen, heads, head_dim] (codes_strides in
 * bytes; written) and scales float32 [batch, heads, ceil(seqlen / block_rows)]
 * (dense; written).  Per block of block_rows rows of one (batch, head): scale =
 * amax / 448 in fp32 (1 for an all-zero block); code = the e4m3 rounding (to
 * nearest even) of the fp32 quotient x / scale.  Use block_rows =
 * FA_FP8_Q_BLOCK for Q and FA_FP8_K_BLOCK for K.  head_dim 64 or 128; rows
 * 16-byte aligned. */
int fa_fp8_quantize(const void* x, int batch, int seqlen, int heads, int head_dim,
                    const int64_t x_strides[3], int block_rows, void* codes,
                    const int64_t codes_strides[3], float* scales, void* stream);

/* fa_fp8_quantize of rotated rows, for Q and K (incoherent processing,
 * "Attention kernels ...", section 4.2: multiplying Q and K by one random
 * orthogonal matrix spreads an outlier channel over all channels before the
 * FP8 rounding, and leaves Q K^T unchanged).  Every row x is first replaced by
 * x diag(signs) H / sqrt(head_dim) in fp32, H the Sylvester Hadamard matrix of
 * order head_dim, formed by the Walsh-Hadamard butterfly (pairs (i, i + h)
 * become (a + b, a - b) for h = 1, 2, ..., head_dim / 2, then one multiply by
 * fp32(1 / sqrt(head_dim))); the block scales and codes are those of the
 * rotated values.  signs: device float32 [head_dim], each +1 or -1, drawn by
 * the caller and the same for Q and K (then fa_fwd_fp8 over the rotated Q and
 * K codes computes the same attention; V is not rotated).  Other arguments and
 * errors as fa_fp8_quantize; FA_ERR_INVALID_ARG for NULL or unaligned signs. */
int fa_fp8_quantize_rotated(const void* x, int batch, int seqlen, int heads, int head_dim,
                            const int64_t x_strides[3], int block_rows, const float* signs,
                            void* codes, const int64_t codes_strides[3], float* scales,
                            void* stream);

/* Length of a transposed V row: seqlen rounded up to a multiple of FA_FP8_K_BLOCK. */
int fa_fp8_vt_len(int seqlen);

/* V quantizer: one scale per (batch, KV head) (scales float32 [batch, heads_kv],
 * written), codes written transposed into vt (dense, written):
 * vt [batch, heads_kv, head_dim, fa_fp8_vt_len(seqlen)] bytes.  Row d of a head
 * holds V[., d] in groups of 64 keys; position p of group n holds key
 * 64 n + 32 ((p >> 4) & 1) + 8 ((p >> 2) & 3) + 4 (p >> 5) + (p & 3) (the key
 * order in which the P V product reads both of its operands); keys past seqlen
 * hold 0.  Same rounding as fa_fp8_quantize. */
int fa_fp8_quantize_v(const void* v, int batch, int seqlen, int heads_kv, int head_dim,
                      const int64_t v_strides[3], void* vt, float* scales, void* stream);

/* FP8 attention forward.
 *   q   e4m3 [batch, seqlen_q, heads_q, head_dim], q_strides in bytes;
 *       q_scales float32 [batch, heads_q, ceil(seqlen_q / FA_FP8_Q_BLOCK)]
 *   k   e4m3 [batch, seqlen_k, heads_kv, head_dim], k_strides in bytes;
 *       k_scales float32 [batch, heads_kv, ceil(seqlen_k / FA_FP8_K_BLOCK)]
 *   vt, v_scales as fa_fp8_quantize_v writes them for seqlen_k keys
 *   out bf16 [batch, seqlen_q, heads_q, head_dim], o_strides in elements (written)
 *   lse float32 [batch, heads_q, seqlen_q] (natural log; written; may be NULL)
 * opts as for fa_fwd: scale, causal (bottom-right), window; softcap > 0 is
 * FA_ERR_UNSUPPORTED; pack_gqa is ignored.  head_dim 128 (else
 * FA_ERR_UNSUPPORTED).  The scores are exact products of the codes summed in
 * fp32; the probabilities enter the P V product as e4m3 (2^8 p relative to the
 * row maximum, rounded to nearest even) and O is divided by the fp32 row sum. */
int fa_fwd_fp8(const fa_attn_opts* opts, const void* q, const float* q_scales, const void* k,
               const float* k_scales, const void* vt, const float* v_scales, void* out,
               float* lse, int batch, int seqlen_q, int seqlen_k, int heads_q, int heads_kv,
               int head_dim, const int64_t q_strides[3], const int64_t k_strides[3],
               const int64_t o_strides[3], void* stream);

/* Merge of partial attention states ("Attention kernels ...", section 6.3: the
 * partial (O_s, LSE_s) of disjoint key ranges combine with the same rescale as
 * the tiles of one pass):
 *   M = max_s LSE_s,  w_s = exp(LSE_s - M),  LSE = M + ln(sum_s w_s),
 *   O = sum_s (w_s / sum_s w_s) * O_s.
 * A partial whose LSE is -inf has weight 0 and its O is not read; a row whose
 * every LSE_s is -inf gets O = 0 and LSE = -inf.
 *   o_part   float32: row r of split s at o_part + (s * part_stride_rows + r) * head_dim
 *   lse_part float32: row r of split s at lse_part[s * part_stride_rows + r]
 *   part_stride_rows  rows between consecutive splits, >= rows
 *   out      bfloat16, row r at out + r * out_row_stride (written)
 *   lse_out  float32 [rows] (written; may be NULL)
 * Errors: FA_ERR_INVALID_ARG for part_stride_rows < rows, out_row_stride < head_dim,
 * or pointers that are not 4-byte aligned. */
int fa_combine(const float* o_part, const float* lse_part, int num_splits, int64_t rows,
               int head_dim, int64_t part_stride_rows, void* out, int64_t out_row_stride,
               float* lse_out, void* stream);

/* Element types of the states fa_merge_attn_states reads. */
#define FA_DTYPE_FP32 0
#define FA_DTYPE_BF16 1

/* Merge of two attention states held in separate buffers, e.g. attention over a
 * cached prefix and over the new suffix of the same queries ("Attention kernels
 * ...", section 6.3: merge_attn_states(prefix_output, prefix_lse, suffix_output,
 * suffix_lse)); the same formula as fa_combine with two splits.
 *   prefix_out, suffix_out  [batch, seqlen, heads, head_dim] of in_dtype (FA_DTYPE_FP32 or
 *                           FA_DTYPE_BF16), both with strides in_strides = {batch, seq, head}
 *                           in elements, head_dim contiguous (as fa_fwd writes O)
 *   prefix_lse, suffix_lse  float32, element (b, h, t) at b * lse_strides[0] +
 *                           h * lse_strides[1] + t * lse_strides[2] (fa_fwd's [batch, heads,
 *                           seqlen] is {heads * seqlen, seqlen, 1}; fa_fwd_varlen's
 *                           [heads, total] is batch 1 with {0, total, 1})
 *   out      bfloat16 [batch, seqlen, heads, head_dim], strides out_strides (written; may
 *            alias neither input)
 *   lse_out  float32, the same layout as the input LSEs (written; may be NULL)
 * Errors: FA_ERR_UNSUPPORTED for another in_dtype or head_dim; FA_ERR_INVALID_ARG for
 * NULL pointers, negative sizes or strides, or misaligned pointers (out 4-byte aligned
 * with even strides). */
int fa_merge_attn_states(const void* prefix_out, const float* prefix_lse, const void* suffix_out,
                         const float* suffix_lse, int in_dtype, void* out, float* lse_out,
                         int batch, int seqlen, int heads, int head_dim,
                         const int64_t in_strides[3], const int64_t out_strides[3],
                         const int64_t lse_strides[3], void* stream);

/* Host-only helper, no device work: the class of key tile n (keys
 * [n*block_n, n*block_n + block_n)) for query rows at token indices
 * [tok_lo, tok_hi] of a sequence with seqlen_q queries and seqlen_k keys, as the
 * kernels decide it: 0 = skipped; otherwise bit 0 set and bit 1 when the causal
 * diagonal, the right window edge or seqlen_k cuts the tile, bit 2 when the left
 * window edge cuts it ("Attention kernels ...", section 7.2 figure). */
int fa_tile_class(int tok_lo, int tok_hi, int seqlen_q, int seqlen_k, int causal,
                  int window_left, int window_right, int block_n, int n);

/* Message describing the calling thread's last failed call ("" if none). */
const char* fa_last_error(void);

/* Library version (major * 10000 + minor * 100 + patch). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_72_FA_H */
