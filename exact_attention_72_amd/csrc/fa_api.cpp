// C ABI of the attention forward library: argument validation, launch
// parameters, dispatch.  Declarations and the contract live in include/fa.h.
//
// Validation happens before any HIP call, so an invalid call returns an error
// code with nothing enqueued and without touching the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"
#include "fa_blockinfo.h"
#include "fa_internal.h"

#define FA_VERSION_NUMBER 100  // 0.1.0

static_assert(FA_SCRATCH_BYTES == FA_NOALLOC_SCRATCH_BYTES, "scratch size of the header and the kernels differ");

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Options -> score-transform constants.  softmax_scale <= 0 or NaN selects d^-0.5
// ("FA4 (CuTeDSL) and engineering interfaces", section 3).
float resolve_scale(const fa_attn_opts* o, int d) {
  float scale = o->softmax_scale;
  if (!(scale > 0.0f) || isnan(scale) || isinf(scale)) scale = 1.0f / sqrtf((float)d);
  return scale;
}

int fill_opts(const fa_attn_opts* o, int d, FaParams* p, bool* softcap) {
  if (!o) return fail(FA_ERR_INVALID_ARG, "opts is NULL");
  const float scale = resolve_scale(o, d);
  if (isnan(o->softcap) || o->softcap < 0.0f || isinf(o->softcap))
    return fail(FA_ERR_INVALID_ARG, "softcap must be a finite value >= 0");
  const float log2e = 1.4426950408889634f;
  p->scale_log2 = scale * log2e;
  *softcap = o->softcap > 0.0f;
  p->cap_in = *softcap ? scale / o->softcap : 0.0f;
  p->cap_out = *softcap ? o->softcap * log2e : 0.0f;
  p->causal = o->causal ? 1 : 0;
  p->wl = o->window_left < 0 ? -1 : o->window_left;
  p->wr = o->window_right < 0 ? -1 : o->window_right;
  p->alibi = o->alibi_slopes;
  p->alibi_bs = o->alibi_batch_stride;
  p->alibi_inv_scale = 1.0f / scale;
  if (o->alibi_slopes) {
    if ((reinterpret_cast<uintptr_t>(o->alibi_slopes) & 3u) != 0)
      return fail(FA_ERR_INVALID_ARG, "alibi_slopes is not 4-byte aligned");
    if (o->alibi_batch_stride < 0) return fail(FA_ERR_INVALID_ARG, "alibi_batch_stride is negative");
    if (*softcap) return fail(FA_ERR_UNSUPPORTED, "ALiBi together with softcap is not supported");
  }
  return FA_OK;
}

int no_alibi(const FaParams& p, const char* what) {
  if (p.alibi) return fail(FA_ERR_UNSUPPORTED, "ALiBi is not supported by %s", what);
  return FA_OK;
}

int check_dims(int d, int hq, int hkv) {
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d);
  if (hq <= 0 || hkv <= 0) return fail(FA_ERR_INVALID_ARG, "head counts must be positive");
  if (hq % hkv != 0) return fail(FA_ERR_INVALID_ARG, "heads_q %d is not a multiple of heads_kv %d", hq, hkv);
  return FA_OK;
}

// Every row start must be 16-byte aligned: base pointer and all strides * 2 bytes.
// The prefill kernel addresses a 32-key block of K or V through a buffer
// resource with 32-bit byte offsets: 32 token strides must stay below 2^31 bytes.
int check_token_stride(const char* name, int64_t ss) {
  if (ss >= ((int64_t)1 << 25))
    return fail(FA_ERR_UNSUPPORTED, "%s token stride %lld is 2^25 elements or more", name, (long long)ss);
  return FA_OK;
}

int check_strides(const char* name, const void* base, const int64_t* s, int n) {
  if (!s) return fail(FA_ERR_INVALID_ARG, "%s strides are NULL", name);
  if (!aligned16(base)) return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(FA_ERR_INVALID_ARG, "%s stride %d is negative", name, i);
    if ((s[i] * 2) % 16 != 0)
      return fail(FA_ERR_INVALID_ARG, "%s stride %d (%lld elements) breaks 16-byte row alignment", name, i,
                  (long long)s[i]);
  }
  return FA_OK;
}

// Byte strides (FP8 codes): every row start 16-byte aligned.
int check_byte_strides(const char* name, const void* base, const int64_t* s, int n) {
  if (!s) return fail(FA_ERR_INVALID_ARG, "%s strides are NULL", name);
  if (!aligned16(base)) return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(FA_ERR_INVALID_ARG, "%s stride %d is negative", name, i);
    if (s[i] % 16 != 0)
      return fail(FA_ERR_INVALID_ARG, "%s stride %d (%lld bytes) breaks 16-byte row alignment", name, i,
                  (long long)s[i]);
  }
  return FA_OK;
}

// Rotary tables: both or neither; rotated dims a multiple of 16, at most head_dim.
int check_rotary(const float* cos, const float* sin, int dim, int interleaved, int head_dim, FaRotary* r) {
  r->cos = nullptr;
  r->sin = nullptr;
  r->dim = 0;
  r->interleaved = 0;
  if (!cos && !sin) return FA_OK;
  if (!cos || !sin) return fail(FA_ERR_INVALID_ARG, "rotary cos and sin tables go together");
  if (dim < 16 || dim > head_dim || dim % 16 != 0)
    return fail(FA_ERR_INVALID_ARG, "rotary_dim %d must be a multiple of 16 in [16, head_dim]", dim);
  r->cos = cos;
  r->sin = sin;
  r->dim = dim;
  r->interleaved = interleaved ? 1 : 0;
  return FA_OK;
}

bool resolve_pack(const fa_attn_opts* o, int hq, int hkv) {
  if (o->pack_gqa > 0) return true;
  if (o->pack_gqa == 0) return false;
  return hq > hkv;
}

}  // namespace

extern "C" {

const char* fa_last_error(void) { return g_err; }

int fa_version(void) { return FA_VERSION_NUMBER; }

int fa_tile_class(int tok_lo, int tok_hi, int seqlen_q, int seqlen_k, int causal, int window_left,
                  int window_right, int block_n, int n) {
  if (block_n <= 0 || tok_hi < tok_lo) return 0;
  FaRowSpan s;
  s.pos_lo = (int64_t)tok_lo + (seqlen_k - seqlen_q);
  s.pos_hi = (int64_t)tok_hi + (seqlen_k - seqlen_q);
  return fa_tile_class(s, seqlen_k, causal ? 1 : 0, window_left < 0 ? -1 : window_left,
                       window_right < 0 ? -1 : window_right, block_n, n);
}

namespace {

// fa_fwd, and the same with a mod built into the kernel (mod_id != 0, fa_mods.h).
int dense_fwd(const fa_attn_opts* opts, const void* q, const void* k, const void* v, void* out, float* lse,
              int batch, int seqlen_q, int seqlen_k, int heads_q, int heads_kv, int head_dim,
              const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
              const int64_t o_strides[3], int mod_id, const FaModArgs& mod, const char* what, void* stream) {
  int rc;
  if ((rc = check_dims(head_dim, heads_q, heads_kv))) return rc;
  if (!q || !k || !v || !out) return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen_q <= 0 || seqlen_k <= 0)
    return fail(FA_ERR_INVALID_ARG, "batch, seqlen_q and seqlen_k must be positive");
  if ((rc = check_strides("q", q, q_strides, 3)) || (rc = check_strides("k", k, k_strides, 3)) ||
      (rc = check_strides("v", v, v_strides, 3)) || (rc = check_strides("out", out, o_strides, 3)) ||
      (rc = check_token_stride("k", k_strides[1])) || (rc = check_token_stride("v", v_strides[1])))
    return rc;
  FaParams p;
  memset(&p, 0, sizeof p);
  bool softcap = false;
  if ((rc = fill_opts(opts, head_dim, &p, &softcap))) return rc;
  if (mod_id != 0) {
    if (softcap) return fail(FA_ERR_UNSUPPORTED, "%s: softcap is not supported together with a mod", what);
    if ((rc = no_alibi(p, what))) return rc;
  }
  const bool pack = resolve_pack(opts, heads_q, heads_kv);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.q_bs = q_strides[0]; p.q_ss = q_strides[1]; p.q_hs = q_strides[2];
  p.k_bs = k_strides[0]; p.k_ss = k_strides[1]; p.k_hs = k_strides[2];
  p.v_bs = v_strides[0]; p.v_ss = v_strides[1]; p.v_hs = v_strides[2];
  p.o_bs = o_strides[0]; p.o_ss = o_strides[1]; p.o_hs = o_strides[2];
  p.lse_bs = (int64_t)heads_q * seqlen_q;
  p.lse_hs = seqlen_q;
  p.B = batch; p.Nq = seqlen_q; p.Nk = seqlen_k; p.Hq = heads_q; p.Hkv = heads_kv;
  p.g = heads_q / heads_kv;
  p.hg_count = pack ? heads_kv : heads_q;
  p.gp = pack ? p.g : 1;
  p.mod = mod;
  p.scale = resolve_scale(opts, head_dim);
  const int64_t rows = (int64_t)seqlen_q * p.gp;
  if (rows > (int64_t)1 << 30) return fail(FA_ERR_UNSUPPORTED, "too many rows per sequence");
  p.m_blocks = (int)((rows + FA_BLOCK_M - 1) / FA_BLOCK_M);
  p.total_tiles = (int64_t)p.m_blocks * batch * p.hg_count;
  if (p.total_tiles > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "too many tiles");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = mod_id != 0 ? fa_launch_prefill_mod(p, head_dim, pack, mod_id, st)
                             : fa_launch_prefill(p, head_dim, false, false, pack, softcap, st);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return FA_OK;
}

}  // namespace

int fa_fwd(const fa_attn_opts* opts, const void* q, const void* k, const void* v, void* out, float* lse,
           int batch, int seqlen_q, int seqlen_k, int heads_q, int heads_kv, int head_dim,
           const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
           const int64_t o_strides[3], void* stream) {
  g_err[0] = 0;
  const FaModArgs none = {nullptr, 0, 0, 0.0f};
  return dense_fwd(opts, q, k, v, out, lse, batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, q_strides,
                   k_strides, v_strides, o_strides, 0, none, "fa_fwd", stream);
}

int fa_fwd_relpos_bias(const fa_attn_opts* opts, const void* q, const void* k, const void* v, void* out,
                       float* lse, int batch, int seqlen_q, int seqlen_k, int heads_q, int heads_kv, int head_dim,
                       const float* bias, int max_distance, const int64_t q_strides[3],
                       const int64_t k_strides[3], const int64_t v_strides[3], const int64_t o_strides[3],
                       void* stream) {
  g_err[0] = 0;
  if (!bias) return fail(FA_ERR_INVALID_ARG, "bias is NULL");
  if ((reinterpret_cast<uintptr_t>(bias) & 3u) != 0) return fail(FA_ERR_INVALID_ARG, "bias is not 4-byte aligned");
  if (max_distance < 0 || max_distance > (1 << 30))
    return fail(FA_ERR_INVALID_ARG, "max_distance must lie in [0, 2^30]");
  const FaModArgs m = {bias, 2 * (int64_t)max_distance + 1, max_distance, 0.0f};
  return dense_fwd(opts, q, k, v, out, lse, batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, q_strides,
                   k_strides, v_strides, o_strides, FA_MOD_RELPOS_BIAS, m, "fa_fwd_relpos_bias", stream);
}

int fa_fwd_prefix_lm(const fa_attn_opts* opts, const void* q, const void* k, const void* v, void* out, float* lse,
                     int batch, int seqlen_q, int seqlen_k, int heads_q, int heads_kv, int head_dim,
                     const int32_t* prefix_lens, const int64_t q_strides[3], const int64_t k_strides[3],
                     const int64_t v_strides[3], const int64_t o_strides[3], void* stream) {
  g_err[0] = 0;
  if (!prefix_lens) return fail(FA_ERR_INVALID_ARG, "prefix_lens is NULL");
  if ((reinterpret_cast<uintptr_t>(prefix_lens) & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "prefix_lens is not 4-byte aligned");
  if (opts && opts->causal)
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_prefix_lm: the prefix-LM mask replaces causal; pass causal = 0");
  const FaModArgs m = {prefix_lens, 0, 0, 0.0f};
  return dense_fwd(opts, q, k, v, out, lse, batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, q_strides,
                   k_strides, v_strides, o_strides, FA_MOD_PREFIX_LM, m, "fa_fwd_prefix_lm", stream);
}

int fa_fwd_varlen(const fa_attn_opts* opts, const void* q, const void* k, const void* v, void* out,
                  float* lse, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                  int max_seqlen_q, int total_q, int total_k, int heads_q, int heads_kv, int head_dim,
                  const int64_t q_strides[2], const int64_t k_strides[2], const int64_t v_strides[2],
                  const int64_t o_strides[2], void* stream) {
  g_err[0] = 0;
  int rc;
  if ((rc = check_dims(head_dim, heads_q, heads_kv))) return rc;
  if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || max_seqlen_q < 0 || total_q < 0 || total_k < 0)
    return fail(FA_ERR_INVALID_ARG, "batch must be positive and sizes non-negative");
  if ((rc = check_strides("q", q, q_strides, 2)) || (rc = check_strides("k", k, k_strides, 2)) ||
      (rc = check_strides("v", v, v_strides, 2)) || (rc = check_strides("out", out, o_strides, 2)) ||
      (rc = check_token_stride("k", k_strides[0])) || (rc = check_token_stride("v", v_strides[0])))
    return rc;
  FaParams p;
  memset(&p, 0, sizeof p);
  bool softcap = false;
  if ((rc = fill_opts(opts, head_dim, &p, &softcap))) return rc;
  if (total_q == 0 || max_seqlen_q == 0) return FA_OK;  // nothing to compute
  const bool pack = resolve_pack(opts, heads_q, heads_kv);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.q_bs = 0; p.q_ss = q_strides[0]; p.q_hs = q_strides[1];
  p.k_bs = 0; p.k_ss = k_strides[0]; p.k_hs = k_strides[1];
  p.v_bs = 0; p.v_ss = v_strides[0]; p.v_hs = v_strides[1];
  p.o_bs = 0; p.o_ss = o_strides[0]; p.o_hs = o_strides[1];
  p.lse_bs = 0;
  p.lse_hs = total_q;
  p.B = batch; p.Nq = max_seqlen_q; p.Nk = 0; p.Hq = heads_q; p.Hkv = heads_kv;
  p.g = heads_q / heads_kv;
  p.hg_count = pack ? heads_kv : heads_q;
  p.gp = pack ? p.g : 1;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  const int64_t rows = (int64_t)max_seqlen_q * p.gp;
  if (rows > (int64_t)1 << 30) return fail(FA_ERR_UNSUPPORTED, "too many rows per sequence");
  p.m_blocks = (int)((rows + FA_BLOCK_M - 1) / FA_BLOCK_M);
  // upper bound: every row block of every sequence, but no more than the rows exist
  int64_t bound = (int64_t)p.m_blocks * batch;
  int64_t bound2 = ((int64_t)total_q * p.gp + FA_BLOCK_M - 1) / FA_BLOCK_M + batch;
  p.total_tiles = (bound < bound2 ? bound : bound2) * p.hg_count;
  if (p.total_tiles > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "too many tiles");
  // one workgroup per tile index, longest first: the hardware hands out the next
  // tile as a workgroup finishes, which balances unequal sequences (measured
  // 7 % faster than a persistent grid-stride loop on 32 sequences of 64..8192
  // tokens); indices past the real tile count exit at once
  hipError_t e = fa_launch_prefill(p, head_dim, true, false, pack, softcap, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "varlen launch");
  return FA_OK;
}

int fa_kvcache_num_splits(int batch, int seqlen_q, int heads_q, int heads_kv, int page_size,
                          int max_blocks_per_seq) {
  if (batch <= 0 || seqlen_q <= 0 || heads_q <= 0 || heads_kv <= 0 || heads_q % heads_kv != 0 || page_size <= 0 ||
      max_blocks_per_seq <= 0)
    return 1;
  if ((int64_t)seqlen_q * (heads_q / heads_kv) > FA_PAGED_MAX_ROWS) return 1;  // prefill over the cache
  // With more than one split the workgroups take the sequences longest first
  // (batch <= FA_SEQ_ORDER_MAX), so a few workgroups per compute unit level
  // out sequences of very unequal length: about 4 per compute unit and at least
  // 2 splits.  On 64 sequences of 1k-32k keys, 32/8 heads (256-token pages):
  // 1 split 5.01 TB/s, 2 splits 6.64, 3 6.60, 4 6.37, 5 6.59, 6 6.71, 8 6.15.
  // The curve is not monotone because a sequence's pages are cut into
  // ceil(pages / S)-page splits and some counts leave a short last split for
  // many lengths; this host-side choice does not see the lengths (they are on
  // the device) and takes 2, within 1 % of the best count there.  Without the
  // order (larger batches) about 32 per compute unit, so that the lengths level
  // out by number.  Each split keeps at least one page; at most 64 splits.
  const int64_t units = (int64_t)batch * heads_kv;
  const bool ordered = batch <= FA_SEQ_ORDER_MAX;
  const int64_t target = (ordered ? 4 : 32) * (int64_t)fa_device_cus();
  int64_t s = (target + units - 1) / units;
  if (ordered && s < 2) s = 2;
  if (s > 64) s = 64;
  if (s > max_blocks_per_seq) s = max_blocks_per_seq;
  return s < 1 ? 1 : (int)s;
}

// Partial (O, LSE) bytes of the varlen paged decode requests: num_splits x batch x
// heads_kv units of FA_PAGED_MAX_ROWS rows, rounded up to 256; the sequence order
// (one int32 per sequence, batch <= FA_SEQ_ORDER_MAX) follows.
static size_t varlen_paged_partial_bytes(int batch, int heads_kv, int head_dim, int num_splits) {
  size_t rows = (size_t)batch * heads_kv * FA_PAGED_MAX_ROWS;
  size_t bytes = (size_t)num_splits * rows * ((size_t)head_dim + 1) * 4;
  return (bytes + 255) & ~(size_t)255;
}

size_t fa_varlen_paged_workspace_size(int batch, int heads_kv, int head_dim, int num_splits) {
  if (num_splits <= 1 || batch <= 0 || heads_kv <= 0 || head_dim <= 0) return 0;
  size_t bytes = varlen_paged_partial_bytes(batch, heads_kv, head_dim, num_splits);
  if (batch <= FA_SEQ_ORDER_MAX) bytes += ((size_t)batch * 4 + 255) & ~(size_t)255;
  return bytes;
}

int fa_varlen_paged_num_splits(int batch, int heads_q, int heads_kv, int max_blocks_per_seq) {
  // the decode requests of the batch, at most all of its sequences, as one
  // decode step each: the split count fa_kvcache_num_splits gives for them
  return fa_kvcache_num_splits(batch, 1, heads_q, heads_kv, 16, max_blocks_per_seq);
}

int fa_fwd_varlen_paged(const fa_attn_opts* opts, const void* q, const void* k_cache, const void* v_cache,
                        void* out, float* lse, const int32_t* cu_seqlens_q, const int32_t* block_table,
                        const int32_t* cache_seqlens, int batch, int max_seqlen_q, int total_q, int heads_q,
                        int heads_kv, int head_dim, int64_t num_pages, int page_size, int max_blocks_per_seq,
                        int num_splits, void* workspace, size_t workspace_bytes, const int64_t q_strides[2],
                        const int64_t k_strides[3], const int64_t v_strides[3], const int64_t o_strides[2],
                        void* stream) {
  g_err[0] = 0;
  int rc;
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (num_splits == 0 && batch > 0 && heads_q > 0 && heads_kv > 0 && heads_q % heads_kv == 0)
    num_splits = fa_varlen_paged_num_splits(batch, heads_q, heads_kv, max_blocks_per_seq);
  if (num_splits == 0) num_splits = 1;  // invalid sizes: reported below
  if ((rc = check_dims(head_dim, heads_q, heads_kv))) return rc;
  if (!q || !k_cache || !v_cache || !out || !cu_seqlens_q || !block_table || !cache_seqlens)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || max_seqlen_q < 0 || total_q < 0 || num_pages <= 0 || page_size <= 0 || max_blocks_per_seq <= 0)
    return fail(FA_ERR_INVALID_ARG,
                "batch, num_pages, page_size and max_blocks_per_seq must be positive and sizes non-negative");
  if (page_size % 16 != 0) return fail(FA_ERR_INVALID_ARG, "page_size %d is not a multiple of 16", page_size);
  if ((int64_t)max_blocks_per_seq * page_size > ((int64_t)1 << 31) - 1)
    return fail(FA_ERR_UNSUPPORTED, "max_blocks_per_seq * page_size exceeds 2^31 - 1 keys");
  if ((rc = check_strides("q", q, q_strides, 2)) || (rc = check_strides("k_cache", k_cache, k_strides, 3)) ||
      (rc = check_strides("v_cache", v_cache, v_strides, 3)) || (rc = check_strides("out", out, o_strides, 2)) ||
      (rc = check_token_stride("k_cache", k_strides[1])) || (rc = check_token_stride("v_cache", v_strides[1])))
    return rc;
  const size_t need = fa_varlen_paged_workspace_size(batch, heads_kv, head_dim, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes, got %zu", need, workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  FaParams p;
  memset(&p, 0, sizeof p);
  bool softcap = false;
  if ((rc = fill_opts(opts, head_dim, &p, &softcap))) return rc;
  if ((rc = no_alibi(p, "fa_fwd_varlen_paged"))) return rc;
  if (total_q == 0 || max_seqlen_q == 0) return FA_OK;  // nothing to compute
  const bool pack = resolve_pack(opts, heads_q, heads_kv);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.q_bs = 0; p.q_ss = q_strides[0]; p.q_hs = q_strides[1];
  p.k_bs = k_strides[0]; p.k_ss = k_strides[1]; p.k_hs = k_strides[2];
  p.v_bs = v_strides[0]; p.v_ss = v_strides[1]; p.v_hs = v_strides[2];
  p.o_bs = 0; p.o_ss = o_strides[0]; p.o_hs = o_strides[1];
  p.lse_bs = 0;
  p.lse_hs = total_q;
  p.B = batch; p.Nq = max_seqlen_q; p.Nk = 0; p.Hq = heads_q; p.Hkv = heads_kv;
  p.g = heads_q / heads_kv;
  p.hg_count = pack ? heads_kv : heads_q;
  p.gp = pack ? p.g : 1;
  p.cu_q = cu_seqlens_q;
  p.block_table = block_table;
  p.cache_seqlens = cache_seqlens;
  p.page = page_size;
  p.max_blocks = max_blocks_per_seq;
  const int64_t rows = (int64_t)max_seqlen_q * p.gp;
  if (rows > (int64_t)1 << 30) return fail(FA_ERR_UNSUPPORTED, "too many rows per sequence");
  p.m_blocks = (int)((rows + FA_BLOCK_M - 1) / FA_BLOCK_M);
  int64_t bound = (int64_t)p.m_blocks * batch;
  int64_t bound2 = ((int64_t)total_q * p.gp + FA_BLOCK_M - 1) / FA_BLOCK_M + batch;
  p.total_tiles = (bound < bound2 ? bound : bound2) * p.hg_count;
  if (p.total_tiles > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "too many tiles");
  // one workgroup per tile index, longest tiles first (by the keys each sees):
  // with the decode-like sequences in the decode kernel this measured 562
  // against 547 TFLOP/s for a persistent grid-stride loop on a batch of 64
  // one-token requests and 4 chunks of 2048 tokens
  hipStream_t s = static_cast<hipStream_t>(stream);
  // sequences of at most FA_PAGED_MAX_ROWS packed rows (decode steps, short
  // chunks) run in the decode kernel, one workgroup per (sequence, KV head) with
  // its query heads packed into the product columns; the prefill kernel gives
  // them no tiles
  p.skip_rows = FA_PAGED_MAX_ROWS;
  FaParams pd = p;
  pd.num_splits = num_splits;
  if (num_splits > 1) {
    // split-KV for the decode requests: fp32 partials per (sequence, KV head)
    // unit and split, merged by the packed combine; the split workgroups take the
    // sequences longest cache first
    pd.o_part = static_cast<float*>(workspace);
    pd.lse_part = pd.o_part + (size_t)num_splits * batch * heads_kv * FA_PAGED_MAX_ROWS * head_dim;
    if (batch <= FA_SEQ_ORDER_MAX) {
      int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                  varlen_paged_partial_bytes(batch, heads_kv, head_dim, num_splits));
      hipError_t e = fa_launch_seq_order(cache_seqlens, batch, order, s);
      if (e != hipSuccess) return hip_fail(e, "sequence order launch");
      pd.seq_order = order;
    }
  }
  // decode units and prefill tiles in one launch, then the decode splits' merge
  hipError_t e = fa_launch_unified(pd, p, head_dim, pack, softcap, s);
  if (e != hipSuccess) return hip_fail(e, "unified varlen paged launch");
  if (num_splits > 1) {
    e = fa_launch_combine_packed(pd, head_dim, s);
    if (e != hipSuccess) return hip_fail(e, "varlen paged combine launch");
  }
  return FA_OK;
}

// Partial (O, LSE) bytes of a split-KV call, rounded up to 256; the sequence
// order (one int32 per sequence, when batch <= FA_SEQ_ORDER_MAX) follows them.
static size_t kvcache_partial_bytes(int batch, int seqlen_q, int heads_q, int head_dim, int num_splits) {
  size_t rows = (size_t)batch * seqlen_q * heads_q;
  size_t bytes = (size_t)num_splits * rows * ((size_t)head_dim + 1) * 4;
  return (bytes + 255) & ~(size_t)255;
}

size_t fa_kvcache_workspace_size(int batch, int seqlen_q, int heads_q, int head_dim, int num_splits) {
  if (num_splits <= 1 || batch <= 0 || seqlen_q <= 0 || heads_q <= 0 || head_dim <= 0) return 0;
  size_t bytes = kvcache_partial_bytes(batch, seqlen_q, heads_q, head_dim, num_splits);
  if (batch <= FA_SEQ_ORDER_MAX) bytes += ((size_t)batch * 4 + 255) & ~(size_t)255;
  return bytes;
}

namespace {

// FP8 (e4m3) cache of fa_fwd_kvcache_paged_fp8: its two scales.
struct KvFp8 {
  bool on;
  float k_scale, v_scale;
};

// fa_fwd_kvcache_paged, its no-allocation twin and its FP8-cache variant.  With
// use_scratch the partials and the sequence order go to the library's static
// device scratch (after the size check, nothing else touches the device first)
// instead of the workspace.
int kvcache_paged(const fa_attn_opts* opts, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* cache_seqlens, void* out, float* lse, int batch,
                  int seqlen_q, int heads_q, int heads_kv, int head_dim, int64_t num_pages, int page_size,
                  int max_blocks_per_seq, int num_splits, void* workspace, size_t workspace_bytes,
                  bool use_scratch, const int64_t q_strides[3], const int64_t k_strides[3],
                  const int64_t v_strides[3], const int64_t o_strides[3], void* stream,
                  KvFp8 fp8 = {false, 1.0f, 1.0f}) {
  int rc;
  if ((rc = check_dims(head_dim, heads_q, heads_kv))) return rc;
  if (!q || !k_cache || !v_cache || !block_table || !cache_seqlens || !out)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen_q <= 0 || num_pages <= 0 || page_size <= 0 || max_blocks_per_seq <= 0)
    return fail(FA_ERR_INVALID_ARG, "batch, seqlen_q, num_pages, page_size and max_blocks_per_seq must be positive");
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (page_size % 16 != 0) return fail(FA_ERR_INVALID_ARG, "page_size %d is not a multiple of 16", page_size);
  if ((int64_t)max_blocks_per_seq * page_size > ((int64_t)1 << 31) - 1)
    return fail(FA_ERR_UNSUPPORTED, "max_blocks_per_seq * page_size exceeds 2^31 - 1 keys");
  if (fp8.on) {
    if ((rc = check_strides("q", q, q_strides, 3)) || (rc = check_byte_strides("k_cache", k_cache, k_strides, 3)) ||
        (rc = check_byte_strides("v_cache", v_cache, v_strides, 3)) || (rc = check_strides("out", out, o_strides, 3)))
      return rc;
    if (!(fp8.k_scale > 0.0f) || !(fp8.v_scale > 0.0f) || isinf(fp8.k_scale) || isinf(fp8.v_scale))
      return fail(FA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  } else if ((rc = check_strides("q", q, q_strides, 3)) || (rc = check_strides("k_cache", k_cache, k_strides, 3)) ||
             (rc = check_strides("v_cache", v_cache, v_strides, 3)) || (rc = check_strides("out", out, o_strides, 3)) ||
             (rc = check_token_stride("k_cache", k_strides[1])) || (rc = check_token_stride("v_cache", v_strides[1]))) {
    return rc;
  }
  const int g = heads_q / heads_kv;
  if (num_splits == 0)
    num_splits = fa_kvcache_num_splits(batch, seqlen_q, heads_q, heads_kv, page_size, max_blocks_per_seq);
  // more packed query rows than the decode kernel holds: the prefill kernel
  // over the paged cache (chunked prefill), without split-KV
  const bool prefill = (int64_t)seqlen_q * g > FA_PAGED_MAX_ROWS;
  if (prefill && fp8.on)
    return fail(FA_ERR_UNSUPPORTED,
                "fa_fwd_kvcache_paged_fp8 needs seqlen_q * heads_q / heads_kv <= %d (got %lld)",
                FA_PAGED_MAX_ROWS, (long long)seqlen_q * g);
  if (prefill && num_splits != 1)
    return fail(FA_ERR_UNSUPPORTED,
                "num_splits > 1 needs seqlen_q * heads_q / heads_kv <= %d (got %lld); use 1 or 0",
                FA_PAGED_MAX_ROWS, (long long)seqlen_q * g);
  const size_t need = fa_kvcache_workspace_size(batch, seqlen_q, heads_q, head_dim, num_splits);
  if (use_scratch) {
    if (need > FA_SCRATCH_BYTES)
      return fail(FA_ERR_INVALID_ARG,
                  "fa_fwd_kvcache_paged_noalloc: the split partials need %zu bytes, more than the %zu-byte "
                  "static scratch; use fewer splits or fa_fwd_kvcache_paged with a workspace",
                  need, FA_SCRATCH_BYTES);
  } else {
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  }
  FaParams p;
  memset(&p, 0, sizeof p);
  bool softcap = false;
  if ((rc = fill_opts(opts, head_dim, &p, &softcap))) return rc;
  // S = scale q.(k_scale c_k) = (scale k_scale) q.c_k; O = v_scale sum p c_v
  p.scale_log2 *= fp8.k_scale;
  p.cap_in *= fp8.k_scale;
  p.alibi_inv_scale /= fp8.k_scale;   // the bias in raw-score units: q.c_k
  p.v_scale = fp8.v_scale;
  if (use_scratch && need > 0) {
    hipError_t e = fa_scratch_region(&workspace);
    if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
    workspace_bytes = FA_SCRATCH_BYTES;
  }
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.q_bs = q_strides[0]; p.q_ss = q_strides[1]; p.q_hs = q_strides[2];
  p.k_bs = k_strides[0]; p.k_ss = k_strides[1]; p.k_hs = k_strides[2];
  p.v_bs = v_strides[0]; p.v_ss = v_strides[1]; p.v_hs = v_strides[2];
  p.o_bs = o_strides[0]; p.o_ss = o_strides[1]; p.o_hs = o_strides[2];
  p.B = batch; p.Nq = seqlen_q; p.Hq = heads_q; p.Hkv = heads_kv; p.g = g;
  p.block_table = block_table;
  p.cache_seqlens = cache_seqlens;
  p.page = page_size;
  p.max_blocks = max_blocks_per_seq;
  p.num_splits = num_splits;
  p.lse_bs = (int64_t)heads_q * seqlen_q;
  p.lse_hs = seqlen_q;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (prefill) {
    const bool pack = resolve_pack(opts, heads_q, heads_kv);
    p.hg_count = pack ? heads_kv : heads_q;
    p.gp = pack ? g : 1;
    const int64_t rows_seq = (int64_t)seqlen_q * p.gp;
    p.m_blocks = (int)((rows_seq + FA_BLOCK_M - 1) / FA_BLOCK_M);
    p.total_tiles = (int64_t)p.m_blocks * batch * p.hg_count;
    if (p.total_tiles > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "too many tiles");
    hipError_t e = fa_launch_prefill(p, head_dim, false, true, pack, softcap, s);
    if (e != hipSuccess) return hip_fail(e, "paged prefill launch");
    return FA_OK;
  }
  const int64_t rows = (int64_t)batch * heads_q * seqlen_q;
  if (num_splits > 1) {
    p.o_part = static_cast<float*>(workspace);
    p.lse_part = p.o_part + (size_t)num_splits * rows * head_dim;
    if (batch <= FA_SEQ_ORDER_MAX) {
      int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                  kvcache_partial_bytes(batch, seqlen_q, heads_q, head_dim,
                                                                        num_splits));
      hipError_t e = fa_launch_seq_order(cache_seqlens, batch, order, s);
      if (e != hipSuccess) return hip_fail(e, "sequence order launch");
      p.seq_order = order;
    }
  }
  hipError_t e = fa_launch_paged(p, head_dim, softcap, fp8.on, s);
  if (e != hipSuccess) return hip_fail(e, "paged launch");
  if (num_splits > 1) {
    // partial row r = (b * Hq + h) * Nq + t of every split, split after split
    FaCombineParams c;
    memset(&c, 0, sizeof c);
    c.o_in[0] = p.o_part;
    c.lse_in[0] = p.lse_part;
    c.o_split = rows * head_dim;
    c.lse_split = rows;
    c.num_splits = num_splits;
    c.rows = rows;
    c.B = batch;
    c.Hq = heads_q;
    c.Nq = seqlen_q;
    c.i_bs = (int64_t)heads_q * seqlen_q * head_dim; c.i_ss = head_dim; c.i_hs = (int64_t)seqlen_q * head_dim;
    c.il_bs = (int64_t)heads_q * seqlen_q; c.il_hs = seqlen_q; c.il_ss = 1;
    c.o = p.o;
    c.o_bs = p.o_bs; c.o_ss = p.o_ss; c.o_hs = p.o_hs;
    c.lse = lse;
    c.l_bs = p.lse_bs; c.l_hs = p.lse_hs; c.l_ss = 1;
    e = fa_launch_combine(c, head_dim, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return FA_OK;
}

}  // namespace

int fa_fwd_kvcache_paged(const fa_attn_opts* opts, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* cache_seqlens, void* out, float* lse,
                         int batch, int seqlen_q, int heads_q, int heads_kv, int head_dim, int64_t num_pages,
                         int page_size, int max_blocks_per_seq, int num_splits, void* workspace,
                         size_t workspace_bytes, const int64_t q_strides[3], const int64_t k_strides[3],
                         const int64_t v_strides[3], const int64_t o_strides[3], void* stream) {
  g_err[0] = 0;
  return kvcache_paged(opts, q, k_cache, v_cache, block_table, cache_seqlens, out, lse, batch, seqlen_q, heads_q,
                       heads_kv, head_dim, num_pages, page_size, max_blocks_per_seq, num_splits, workspace,
                       workspace_bytes, false, q_strides, k_strides, v_strides, o_strides, stream);
}

int fa_fwd_kvcache_paged_fp8(const fa_attn_opts* opts, const void* q, const void* k_cache, const void* v_cache,
                             float k_scale, float v_scale, const int32_t* block_table,
                             const int32_t* cache_seqlens, void* out, float* lse, int batch, int seqlen_q,
                             int heads_q, int heads_kv, int head_dim, int64_t num_pages, int page_size,
                             int max_blocks_per_seq, int num_splits, void* workspace, size_t workspace_bytes,
                             const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
                             const int64_t o_strides[3], void* stream) {
  g_err[0] = 0;
  return kvcache_paged(opts, q, k_cache, v_cache, block_table, cache_seqlens, out, lse, batch, seqlen_q, heads_q,
                       heads_kv, head_dim, num_pages, page_size, max_blocks_per_seq, num_splits, workspace,
                       workspace_bytes, false, q_strides, k_strides, v_strides, o_strides, stream,
                       KvFp8{true, k_scale, v_scale});
}

int fa_fwd_kvcache_paged_noalloc(const fa_attn_opts* opts, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table, const int32_t* cache_seqlens,
                                 void* out, float* lse, int batch, int seqlen_q, int heads_q, int heads_kv,
                                 int head_dim, int64_t num_pages, int page_size, int max_blocks_per_seq,
                                 int num_splits, const int64_t q_strides[3], const int64_t k_strides[3],
                                 const int64_t v_strides[3], const int64_t o_strides[3], void* stream) {
  g_err[0] = 0;
  return kvcache_paged(opts, q, k_cache, v_cache, block_table, cache_seqlens, out, lse, batch, seqlen_q, heads_q,
                       heads_kv, head_dim, num_pages, page_size, max_blocks_per_seq, num_splits, nullptr, 0, true,
                       q_strides, k_strides, v_strides, o_strides, stream);
}

int fa_kvcache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_table, const int32_t* cache_seqlens, int batch, int seqlen_new,
                      int heads_kv, int head_dim, int64_t num_pages, int page_size, int max_blocks_per_seq,
                      const int64_t kn_strides[3], const int64_t vn_strides[3], const int64_t k_strides[3],
                      const int64_t v_strides[3], const float* rotary_cos, const float* rotary_sin,
                      int rotary_dim, int rotary_interleaved, void* stream) {
  g_err[0] = 0;
  int rc;
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !cache_seqlens)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen_new < 0 || heads_kv <= 0 || num_pages <= 0 || page_size <= 0 || max_blocks_per_seq <= 0)
    return fail(FA_ERR_INVALID_ARG,
                "batch, heads_kv, num_pages, page_size and max_blocks_per_seq must be positive, seqlen_new >= 0");
  if (page_size % 16 != 0) return fail(FA_ERR_INVALID_ARG, "page_size %d is not a multiple of 16", page_size);
  if ((int64_t)max_blocks_per_seq * page_size > ((int64_t)1 << 31) - 1)
    return fail(FA_ERR_UNSUPPORTED, "max_blocks_per_seq * page_size exceeds 2^31 - 1 keys");
  if ((rc = check_strides("k_new", k_new, kn_strides, 3)) || (rc = check_strides("v_new", v_new, vn_strides, 3)) ||
      (rc = check_strides("k_cache", k_cache, k_strides, 3)) || (rc = check_strides("v_cache", v_cache, v_strides, 3)))
    return rc;
  FaRotary rot;
  if ((rc = check_rotary(rotary_cos, rotary_sin, rotary_dim, rotary_interleaved, head_dim, &rot))) return rc;
  if (seqlen_new == 0) return FA_OK;
  FaAppendParams p;
  memset(&p, 0, sizeof p);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.v_cache = static_cast<uint16_t*>(v_cache);
  p.kn_bs = kn_strides[0]; p.kn_ss = kn_strides[1]; p.kn_hs = kn_strides[2];
  p.vn_bs = vn_strides[0]; p.vn_ss = vn_strides[1]; p.vn_hs = vn_strides[2];
  p.k_ps = k_strides[0]; p.k_ss = k_strides[1]; p.k_hs = k_strides[2];
  p.v_ps = v_strides[0]; p.v_ss = v_strides[1]; p.v_hs = v_strides[2];
  p.block_table = block_table;
  p.cache_seqlens = cache_seqlens;
  p.B = batch; p.L = seqlen_new; p.Hkv = heads_kv; p.page = page_size; p.max_blocks = max_blocks_per_seq;
  p.rot = rot;
  hipError_t e = fa_launch_append(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return FA_OK;
}

int fa_kvcache_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache, float k_scale,
                          float v_scale, const int32_t* block_table, const int32_t* cache_seqlens, int batch,
                          int seqlen_new, int heads_kv, int head_dim, int64_t num_pages, int page_size,
                          int max_blocks_per_seq, const int64_t kn_strides[3], const int64_t vn_strides[3],
                          const int64_t k_strides[3], const int64_t v_strides[3], void* stream) {
  g_err[0] = 0;
  int rc;
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !cache_seqlens)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen_new < 0 || heads_kv <= 0 || num_pages <= 0 || page_size <= 0 || max_blocks_per_seq <= 0)
    return fail(FA_ERR_INVALID_ARG,
                "batch, heads_kv, num_pages, page_size and max_blocks_per_seq must be positive, seqlen_new >= 0");
  if (page_size % 16 != 0) return fail(FA_ERR_INVALID_ARG, "page_size %d is not a multiple of 16", page_size);
  if ((int64_t)max_blocks_per_seq * page_size > ((int64_t)1 << 31) - 1)
    return fail(FA_ERR_UNSUPPORTED, "max_blocks_per_seq * page_size exceeds 2^31 - 1 keys");
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale))
    return fail(FA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if ((rc = check_strides("k_new", k_new, kn_strides, 3)) || (rc = check_strides("v_new", v_new, vn_strides, 3)) ||
      (rc = check_byte_strides("k_cache", k_cache, k_strides, 3)) ||
      (rc = check_byte_strides("v_cache", v_cache, v_strides, 3)))
    return rc;
  if (seqlen_new == 0) return FA_OK;
  FaAppendParams p;
  memset(&p, 0, sizeof p);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.v_cache = static_cast<uint16_t*>(v_cache);
  p.kn_bs = kn_strides[0]; p.kn_ss = kn_strides[1]; p.kn_hs = kn_strides[2];
  p.vn_bs = vn_strides[0]; p.vn_ss = vn_strides[1]; p.vn_hs = vn_strides[2];
  p.k_ps = k_strides[0]; p.k_ss = k_strides[1]; p.k_hs = k_strides[2];
  p.v_ps = v_strides[0]; p.v_ss = v_strides[1]; p.v_hs = v_strides[2];
  p.block_table = block_table;
  p.cache_seqlens = cache_seqlens;
  p.B = batch; p.L = seqlen_new; p.Hkv = heads_kv; p.page = page_size; p.max_blocks = max_blocks_per_seq;
  p.fp8 = 1;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  hipError_t e = fa_launch_append(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return FA_OK;
}

int fa_rotary(void* x, int batch, int seqlen, int heads, int head_dim, const int64_t x_strides[3],
              const int32_t* position_base, const float* cos, const float* sin, int rotary_dim, int interleaved,
              void* stream) {
  g_err[0] = 0;
  int rc;
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!x || !cos || !sin) return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen < 0 || heads <= 0)
    return fail(FA_ERR_INVALID_ARG, "batch and heads must be positive, seqlen >= 0");
  if ((rc = check_strides("x", x, x_strides, 3))) return rc;
  FaRotary rot;
  if ((rc = check_rotary(cos, sin, rotary_dim, interleaved, head_dim, &rot))) return rc;
  if (seqlen == 0) return FA_OK;
  FaRotaryParams p;
  memset(&p, 0, sizeof p);
  p.x = static_cast<uint16_t*>(x);
  p.bs = x_strides[0]; p.ss = x_strides[1]; p.hs = x_strides[2];
  p.pos_base = position_base;
  p.B = batch; p.L = seqlen; p.H = heads;
  p.rot = rot;
  hipError_t e = fa_launch_rotary(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rotary launch");
  return FA_OK;
}

// D and the scaled LSE, one fp32 each per query row, each array rounded up to 256
static size_t bwd_row_bytes(int batch, int seqlen_q, int heads_q) {
  const size_t bytes = (size_t)batch * heads_q * seqlen_q * 4;
  return (bytes + 255) & ~(size_t)255;
}

size_t fa_bwd_workspace_size(int batch, int seqlen_q, int heads_q) {
  if (batch <= 0 || seqlen_q <= 0 || heads_q <= 0) return 0;
  return 2 * bwd_row_bytes(batch, seqlen_q, heads_q);
}

int fa_bwd(const fa_attn_opts* opts, const void* q, const void* k, const void* v, const void* out,
           const float* lse, const void* dout, void* dq, void* dk, void* dv, int batch, int seqlen_q, int seqlen_k,
           int heads_q, int heads_kv, int head_dim, const int64_t q_strides[3], const int64_t k_strides[3],
           const int64_t v_strides[3], const int64_t o_strides[3], const int64_t do_strides[3],
           const int64_t dq_strides[3], const int64_t dk_strides[3], const int64_t dv_strides[3], void* workspace,
           size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int rc;
  if ((rc = check_dims(head_dim, heads_q, heads_kv))) return rc;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen_q <= 0 || seqlen_k <= 0)
    return fail(FA_ERR_INVALID_ARG, "batch, seqlen_q and seqlen_k must be positive");
  if ((rc = check_strides("q", q, q_strides, 3)) || (rc = check_strides("k", k, k_strides, 3)) ||
      (rc = check_strides("v", v, v_strides, 3)) || (rc = check_strides("out", out, o_strides, 3)) ||
      (rc = check_strides("dout", dout, do_strides, 3)) || (rc = check_strides("dq", dq, dq_strides, 3)) ||
      (rc = check_strides("dk", dk, dk_strides, 3)) || (rc = check_strides("dv", dv, dv_strides, 3)) ||
      (rc = check_token_stride("q", q_strides[1])) || (rc = check_token_stride("dout", do_strides[1])))
    return rc;
  // the dK/dV kernel reaches the L array from the D array with a 32-bit offset
  if (bwd_row_bytes(batch, seqlen_q, heads_q) > (size_t)0x7fffff00)
    return fail(FA_ERR_UNSUPPORTED, "batch * heads_q * seqlen_q of %lld rows is too many for the backward",
                (long long)batch * heads_q * seqlen_q);
  const size_t need = fa_bwd_workspace_size(batch, seqlen_q, heads_q);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes, got %zu", need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  FaParams f;
  memset(&f, 0, sizeof f);
  bool softcap = false;
  if ((rc = fill_opts(opts, head_dim, &f, &softcap))) return rc;
  if ((rc = no_alibi(f, "fa_bwd"))) return rc;
  FaBwdParams p;
  memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.delta = static_cast<float*>(workspace);
  p.nlse = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_row_bytes(batch, seqlen_q, heads_q));
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.q_bs = q_strides[0]; p.q_ss = q_strides[1]; p.q_hs = q_strides[2];
  p.k_bs = k_strides[0]; p.k_ss = k_strides[1]; p.k_hs = k_strides[2];
  p.v_bs = v_strides[0]; p.v_ss = v_strides[1]; p.v_hs = v_strides[2];
  p.o_bs = o_strides[0]; p.o_ss = o_strides[1]; p.o_hs = o_strides[2];
  p.do_bs = do_strides[0]; p.do_ss = do_strides[1]; p.do_hs = do_strides[2];
  p.dq_bs = dq_strides[0]; p.dq_ss = dq_strides[1]; p.dq_hs = dq_strides[2];
  p.dk_bs = dk_strides[0]; p.dk_ss = dk_strides[1]; p.dk_hs = dk_strides[2];
  p.dv_bs = dv_strides[0]; p.dv_ss = dv_strides[1]; p.dv_hs = dv_strides[2];
  p.B = batch; p.Nq = seqlen_q; p.Nk = seqlen_k; p.Hq = heads_q; p.Hkv = heads_kv; p.g = heads_q / heads_kv;
  p.scale_log2 = f.scale_log2;
  p.scale = resolve_scale(opts, head_dim);
  p.causal = f.causal; p.wl = f.wl; p.wr = f.wr;
  p.softcap = softcap ? 1 : 0; p.cap_in = f.cap_in; p.cap_out = f.cap_out;
  hipError_t e = fa_launch_bwd(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return FA_OK;
}

int fa_bwd_varlen(const fa_attn_opts* opts, const void* q, const void* k, const void* v, const void* out,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                  int total_k, int heads_q, int heads_kv, int head_dim, const int64_t q_strides[2],
                  const int64_t k_strides[2], const int64_t v_strides[2], const int64_t o_strides[2],
                  const int64_t do_strides[2], const int64_t dq_strides[2], const int64_t dk_strides[2],
                  const int64_t dv_strides[2], void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int rc;
  if ((rc = check_dims(head_dim, heads_q, heads_kv))) return rc;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return fail(FA_ERR_INVALID_ARG, "batch must be positive and sizes non-negative");
  if (((reinterpret_cast<uintptr_t>(cu_seqlens_q) | reinterpret_cast<uintptr_t>(cu_seqlens_k)) & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "cu_seqlens are not 4-byte aligned");
  if ((rc = check_strides("q", q, q_strides, 2)) || (rc = check_strides("k", k, k_strides, 2)) ||
      (rc = check_strides("v", v, v_strides, 2)) || (rc = check_strides("out", out, o_strides, 2)) ||
      (rc = check_strides("dout", dout, do_strides, 2)) || (rc = check_strides("dq", dq, dq_strides, 2)) ||
      (rc = check_strides("dk", dk, dk_strides, 2)) || (rc = check_strides("dv", dv, dv_strides, 2)) ||
      (rc = check_token_stride("q", q_strides[0])) || (rc = check_token_stride("dout", do_strides[0])) ||
      (rc = check_token_stride("k", k_strides[0])) || (rc = check_token_stride("v", v_strides[0])))
    return rc;
  // the dK/dV kernel reaches the L array from the D array with a 32-bit offset
  if (bwd_row_bytes(1, total_q, heads_q) > (size_t)0x7fffff00)
    return fail(FA_ERR_UNSUPPORTED, "heads_q * total_q of %lld rows is too many for the backward",
                (long long)heads_q * total_q);
  const size_t need = fa_bwd_workspace_size(1, total_q, heads_q);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes, got %zu", need, workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  FaParams f;
  memset(&f, 0, sizeof f);
  bool softcap = false;
  if ((rc = fill_opts(opts, head_dim, &f, &softcap))) return rc;
  if ((rc = no_alibi(f, "fa_bwd_varlen"))) return rc;
  FaBwdParams p;
  memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.delta = static_cast<float*>(workspace);
  p.nlse = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_row_bytes(1, total_q, heads_q));
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.q_ss = q_strides[0]; p.q_hs = q_strides[1];
  p.k_ss = k_strides[0]; p.k_hs = k_strides[1];
  p.v_ss = v_strides[0]; p.v_hs = v_strides[1];
  p.o_ss = o_strides[0]; p.o_hs = o_strides[1];
  p.do_ss = do_strides[0]; p.do_hs = do_strides[1];
  p.dq_ss = dq_strides[0]; p.dq_hs = dq_strides[1];
  p.dk_ss = dk_strides[0]; p.dk_hs = dk_strides[1];
  p.dv_ss = dv_strides[0]; p.dv_hs = dv_strides[1];
  p.B = batch; p.Nq = max_seqlen_q; p.Nk = max_seqlen_k; p.Hq = heads_q; p.Hkv = heads_kv;
  p.g = heads_q / heads_kv;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.scale_log2 = f.scale_log2;
  p.scale = resolve_scale(opts, head_dim);
  p.causal = f.causal; p.wl = f.wl; p.wr = f.wr;
  p.softcap = softcap ? 1 : 0; p.cap_in = f.cap_in; p.cap_out = f.cap_out;
  hipError_t e = fa_launch_bwd(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return FA_OK;
}

int fa_combine(const float* o_part, const float* lse_part, int num_splits, int64_t rows, int head_dim,
               int64_t part_stride_rows, void* out, int64_t out_row_stride, float* lse_out, void* stream) {
  g_err[0] = 0;
  if (head_dim != 64 && head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!o_part || !lse_part || !out) return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (num_splits < 1 || rows < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 1 and rows >= 0");
  if (part_stride_rows < rows)
    return fail(FA_ERR_INVALID_ARG, "part_stride_rows %lld is below rows %lld (splits would overlap)",
                (long long)part_stride_rows, (long long)rows);
  if (out_row_stride < head_dim || (out_row_stride * 2) % 4 != 0 || (reinterpret_cast<uintptr_t>(out) & 3u))
    return fail(FA_ERR_INVALID_ARG, "out rows must be 4-byte aligned and not overlap");
  if ((reinterpret_cast<uintptr_t>(o_part) & 3u) || (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return fail(FA_ERR_INVALID_ARG, "o_part and lse_part must be 4-byte aligned");
  FaCombineParams c;
  memset(&c, 0, sizeof c);
  c.o_in[0] = o_part;
  c.lse_in[0] = lse_part;
  c.o_split = part_stride_rows * head_dim;
  c.lse_split = part_stride_rows;
  c.num_splits = num_splits;
  c.rows = rows;
  // flat rows: row r is "batch" r of one head and one token
  c.Hq = 1;
  c.Nq = 1;
  c.i_bs = head_dim;
  c.il_bs = 1;
  c.o = static_cast<uint16_t*>(out);
  c.o_bs = out_row_stride;
  c.lse = lse_out;
  c.l_bs = 1;
  hipError_t e = fa_launch_combine(c, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return FA_OK;
}

int fa_merge_attn_states(const void* prefix_out, const float* prefix_lse, const void* suffix_out,
                         const float* suffix_lse, int in_dtype, void* out, float* lse_out, int batch,
                         int seqlen, int heads, int head_dim, const int64_t in_strides[3],
                         const int64_t out_strides[3], const int64_t lse_strides[3], void* stream) {
  g_err[0] = 0;
  if (head_dim != 64 && head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!prefix_out || !prefix_lse || !suffix_out || !suffix_lse || !out || !in_strides || !out_strides || !lse_strides)
    return fail(FA_ERR_INVALID_ARG, "a pointer is NULL");
  if (in_dtype != FA_DTYPE_FP32 && in_dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "in_dtype %d is neither FA_DTYPE_FP32 nor FA_DTYPE_BF16", in_dtype);
  if (batch < 0 || seqlen < 0 || heads < 0) return fail(FA_ERR_INVALID_ARG, "sizes must be >= 0");
  for (int i = 0; i < 3; ++i)
    if (in_strides[i] < 0 || out_strides[i] < 0 || lse_strides[i] < 0)
      return fail(FA_ERR_INVALID_ARG, "strides must be >= 0");
  const uintptr_t ia = (in_dtype == FA_DTYPE_FP32) ? 3u : 1u;
  if ((reinterpret_cast<uintptr_t>(prefix_out) & ia) || (reinterpret_cast<uintptr_t>(suffix_out) & ia) ||
      (reinterpret_cast<uintptr_t>(prefix_lse) & 3u) || (reinterpret_cast<uintptr_t>(suffix_lse) & 3u) ||
      (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)))
    return fail(FA_ERR_INVALID_ARG, "a tensor is not aligned to its element size");
  // the output rows are written as 4-byte pairs of bf16
  if ((reinterpret_cast<uintptr_t>(out) & 3u) || (out_strides[0] | out_strides[1] | out_strides[2]) & 1)
    return fail(FA_ERR_INVALID_ARG, "out must be 4-byte aligned with even strides");
  const int64_t rows = (int64_t)batch * seqlen * heads;
  if (rows == 0) return FA_OK;
  FaCombineParams c;
  memset(&c, 0, sizeof c);
  c.o_in[0] = prefix_out;
  c.o_in[1] = suffix_out;
  c.lse_in[0] = prefix_lse;
  c.lse_in[1] = suffix_lse;
  c.pair = 1;
  c.in_bf16 = in_dtype == FA_DTYPE_BF16;
  c.num_splits = 2;
  c.rows = rows;
  c.B = batch;
  c.Hq = heads;
  c.Nq = seqlen;
  c.i_bs = in_strides[0]; c.i_ss = in_strides[1]; c.i_hs = in_strides[2];
  c.il_bs = lse_strides[0]; c.il_hs = lse_strides[1]; c.il_ss = lse_strides[2];
  c.o = static_cast<uint16_t*>(out);
  c.o_bs = out_strides[0]; c.o_ss = out_strides[1]; c.o_hs = out_strides[2];
  c.lse = lse_out;
  c.l_bs = lse_strides[0]; c.l_hs = lse_strides[1]; c.l_ss = lse_strides[2];
  hipError_t e = fa_launch_combine(c, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return FA_OK;
}


int fa_fp8_vt_len(int seqlen) {
  return seqlen <= 0 ? 0 : (int)(((int64_t)seqlen + FA_FP8_K_BLOCK - 1) / FA_FP8_K_BLOCK * FA_FP8_K_BLOCK);
}

namespace {
int fp8_quantize_rows(const void* x, int batch, int seqlen, int heads, int head_dim, const int64_t x_strides[3],
                      int block_rows, const float* signs, void* codes, const int64_t codes_strides[3], float* scales,
                      void* stream) {
  int rc;
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!x || !codes || !scales) return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen < 0 || heads <= 0) return fail(FA_ERR_INVALID_ARG, "batch and heads must be positive");
  if (block_rows <= 0) return fail(FA_ERR_INVALID_ARG, "block_rows must be positive");
  if ((rc = check_strides("x", x, x_strides, 3)) || (rc = check_byte_strides("codes", codes, codes_strides, 3)))
    return rc;
  if (seqlen == 0) return FA_OK;
  FaFp8QuantParams p;
  memset(&p, 0, sizeof p);
  p.x = static_cast<const uint16_t*>(x);
  p.x_bs = x_strides[0]; p.x_ss = x_strides[1]; p.x_hs = x_strides[2];
  p.codes = static_cast<uint8_t*>(codes);
  p.c_bs = codes_strides[0]; p.c_ss = codes_strides[1]; p.c_hs = codes_strides[2];
  p.scales = scales;
  p.B = batch; p.N = seqlen; p.H = heads; p.rows = block_rows;
  p.signs = signs;
  p.nblk = (int)(((int64_t)seqlen + block_rows - 1) / block_rows);
  if ((int64_t)batch * heads * p.nblk > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "too many blocks");
  hipError_t e = fa_launch_fp8_quant(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  return FA_OK;
}
}  // namespace

int fa_fp8_quantize(const void* x, int batch, int seqlen, int heads, int head_dim, const int64_t x_strides[3],
                    int block_rows, void* codes, const int64_t codes_strides[3], float* scales, void* stream) {
  g_err[0] = 0;
  return fp8_quantize_rows(x, batch, seqlen, heads, head_dim, x_strides, block_rows, nullptr, codes, codes_strides,
                           scales, stream);
}

int fa_fp8_quantize_rotated(const void* x, int batch, int seqlen, int heads, int head_dim,
                            const int64_t x_strides[3], int block_rows, const float* signs, void* codes,
                            const int64_t codes_strides[3], float* scales, void* stream) {
  g_err[0] = 0;
  if (!signs) return fail(FA_ERR_INVALID_ARG, "signs is NULL");
  if ((reinterpret_cast<uintptr_t>(signs) & 3u) != 0) return fail(FA_ERR_INVALID_ARG, "signs is not 4-byte aligned");
  return fp8_quantize_rows(x, batch, seqlen, heads, head_dim, x_strides, block_rows, signs, codes, codes_strides,
                           scales, stream);
}

int fa_fp8_quantize_v(const void* v, int batch, int seqlen, int heads_kv, int head_dim, const int64_t v_strides[3],
                      void* vt, float* scales, void* stream) {
  g_err[0] = 0;
  int rc;
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!v || !vt || !scales) return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen < 0 || heads_kv <= 0)
    return fail(FA_ERR_INVALID_ARG, "batch and heads must be positive");
  if ((rc = check_strides("v", v, v_strides, 3))) return rc;
  if (!aligned16(vt)) return fail(FA_ERR_INVALID_ARG, "vt is not 16-byte aligned");
  if (seqlen == 0) return FA_OK;
  FaFp8QuantParams p;
  memset(&p, 0, sizeof p);
  p.x = static_cast<const uint16_t*>(v);
  p.x_bs = v_strides[0]; p.x_ss = v_strides[1]; p.x_hs = v_strides[2];
  p.vt = static_cast<uint8_t*>(vt);
  p.scales = scales;
  p.B = batch; p.N = seqlen; p.H = heads_kv;
  p.npad = fa_fp8_vt_len(seqlen);
  if ((int64_t)batch * heads_kv * (p.npad / FA_FP8_K_BLOCK) > 0x7fffffff)
    return fail(FA_ERR_UNSUPPORTED, "too many key groups");
  hipError_t e = fa_launch_fp8_quant(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize_v launch");
  return FA_OK;
}

int fa_fwd_fp8(const fa_attn_opts* opts, const void* q, const float* q_scales, const void* k, const float* k_scales,
               const void* vt, const float* v_scales, void* out, float* lse, int batch, int seqlen_q, int seqlen_k,
               int heads_q, int heads_kv, int head_dim, const int64_t q_strides[3], const int64_t k_strides[3],
               const int64_t o_strides[3], void* stream) {
  g_err[0] = 0;
  int rc;
  if ((rc = check_dims(head_dim, heads_q, heads_kv))) return rc;
  if (head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "the FP8 forward is built for head_dim 128");
  if (!q || !k || !vt || !out || !q_scales || !k_scales || !v_scales)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (batch <= 0 || seqlen_q <= 0 || seqlen_k <= 0)
    return fail(FA_ERR_INVALID_ARG, "batch, seqlen_q and seqlen_k must be positive");
  if ((rc = check_byte_strides("q", q, q_strides, 3)) || (rc = check_byte_strides("k", k, k_strides, 3)) ||
      (rc = check_strides("out", out, o_strides, 3)))
    return rc;
  if (!aligned16(vt)) return fail(FA_ERR_INVALID_ARG, "vt is not 16-byte aligned");
  // the kernel addresses a 64-key block of K and a block of V^T with 32-bit byte offsets
  if (k_strides[1] >= ((int64_t)1 << 25))
    return fail(FA_ERR_UNSUPPORTED, "k token stride %lld is 2^25 bytes or more", (long long)k_strides[1]);
  if ((int64_t)head_dim * fa_fp8_vt_len(seqlen_k) >= ((int64_t)1 << 31))
    return fail(FA_ERR_UNSUPPORTED, "seqlen_k %d is too long for the FP8 forward", seqlen_k);
  FaParams tmp;
  memset(&tmp, 0, sizeof tmp);
  bool softcap = false;
  if ((rc = fill_opts(opts, head_dim, &tmp, &softcap))) return rc;
  if ((rc = no_alibi(tmp, "fa_fwd_fp8"))) return rc;
  if (softcap) return fail(FA_ERR_UNSUPPORTED, "softcap is not supported by the FP8 forward");
  FaFp8Params p;
  memset(&p, 0, sizeof p);
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.vt = static_cast<const uint8_t*>(vt);
  p.q_scale = q_scales; p.k_scale = k_scales; p.v_scale = v_scales;
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.q_bs = q_strides[0]; p.q_ss = q_strides[1]; p.q_hs = q_strides[2];
  p.k_bs = k_strides[0]; p.k_ss = k_strides[1]; p.k_hs = k_strides[2];
  p.o_bs = o_strides[0]; p.o_ss = o_strides[1]; p.o_hs = o_strides[2];
  p.lse_bs = (int64_t)heads_q * seqlen_q;
  p.lse_hs = seqlen_q;
  p.B = batch; p.Nq = seqlen_q; p.Nk = seqlen_k; p.Hq = heads_q; p.Hkv = heads_kv;
  p.g = heads_q / heads_kv;
  p.npad = fa_fp8_vt_len(seqlen_k);
  p.q_nblk = (seqlen_q + FA_FP8_Q_BLOCK - 1) / FA_FP8_Q_BLOCK;
  p.k_nblk = (seqlen_k + FA_FP8_K_BLOCK - 1) / FA_FP8_K_BLOCK;
  p.m_blocks = p.q_nblk;
  p.total_tiles = (int64_t)p.m_blocks * batch * heads_q;
  if (p.total_tiles > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "too many tiles");
  p.scale_log2 = tmp.scale_log2;
  p.causal = tmp.causal; p.wl = tmp.wl; p.wr = tmp.wr;
  hipError_t e = fa_launch_fp8_fwd(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 forward launch");
  return FA_OK;
}

}  // extern "C"
