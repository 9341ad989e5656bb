/*
 * fa_mods.h - score_mod / mask_mod hooks of the prefill kernel (HIP device code).
 *
 * "FA4 (CuTeDSL) and engineering interfaces" (sections 1, 3 and the feature
 * table of section 7) describes user functions that rewrite a score after
 * Q K^T and before the softmax (score_mod) or decide whether a key is visible
 * (mask_mod), specialised into the kernel when it is compiled.  Here that
 * specialisation is a C++ template argument of the prefill kernel, fixed when
 * the library is built: a mod is a struct with
 *
 *   static constexpr bool kScore;   // score() is applied
 *   static constexpr bool kMask;    // mask() is applied
 *   __device__ float score(float s, int b, int h, int p, int j, const FaModArgs& a) const;
 *   __device__ bool  mask(int b, int h, int p, int j, const FaModArgs& a) const;
 *
 * where s is the scaled logit softmax_scale * q.k in natural-log units, b the
 * batch index, h the query head, p the query's position on the key axis
 * (token index + seqlen_k - seqlen_q, the bottom-right alignment the causal mask
 * uses) and j the key index.  score() returns the new logit; mask() returns
 * whether key j stays visible.  Both run on every (query, key) pair of every key
 * block the built-in masks (causal, window, sequence length) leave in range; a
 * key the built-in masks drop is dropped whatever mask() says, and score() is
 * not consulted for it.  A key every rule leaves visible enters the softmax with
 * the rewritten logit; a row left with no visible key gets O = 0, LSE = -inf.
 *
 * FaModArgs carries the launch's parameters for the mod (a device pointer and
 * a few scalars), filled by the entry point that instantiates it.  To add a
 * mod: define the struct (here or in a header of your own included by
 * fa_kernels.hip), instantiate the prefill launcher with it and add an entry
 * point, as fa_fwd_relpos_bias and fa_fwd_prefix_lm do for the two mods below.
 */
#ifndef EXACT_ATTENTION_72_FA_MODS_H
#define EXACT_ATTENTION_72_FA_MODS_H

#include <stdint.h>

struct FaModArgs {
  const void* ptr;  // device data of the mod (a table, per-sequence lengths, ...)
  int64_t i0, i1;   // integer parameters
  float f0;         // a float parameter
};

#ifdef __HIPCC__

// No rewrite, no extra mask: the plain kernel.
struct FaNoMod {
  static constexpr bool kScore = false;
  static constexpr bool kMask = false;
  __device__ __forceinline__ float score(float s, int, int, int, int, const FaModArgs&) const { return s; }
  __device__ __forceinline__ bool mask(int, int, int, int, const FaModArgs&) const { return true; }
};

// Learned relative-position bias (score_mod): the logit of query position p and
// key j gets bias[h][clamp(j - p, -R, R) + R] added, from a device fp32 table
// of heads_q rows of 2R + 1 entries (a.ptr, row stride a.i0 = 2R + 1, a.i1 = R).
// Distances beyond R share the end entries.
struct FaRelPosBias {
  static constexpr bool kScore = true;
  static constexpr bool kMask = false;
  __device__ __forceinline__ float score(float s, int, int h, int p, int j, const FaModArgs& a) const {
    const int R = (int)a.i1;
    int r = j - p;
    r = r < -R ? -R : (r > R ? R : r);
    return s + static_cast<const float*>(a.ptr)[(int64_t)h * a.i0 + r + R];
  }
  __device__ __forceinline__ bool mask(int, int, int, int, const FaModArgs&) const { return true; }
};

// Prefix-LM mask (mask_mod): the first prefix_len[b] keys of sequence b are
// visible to every query (a bidirectional prefix), later keys causally (key j
// visible to the query at position p iff j < prefix_len[b] or j <= p).
// a.ptr: device int32 [batch].
struct FaPrefixLM {
  static constexpr bool kScore = false;
  static constexpr bool kMask = true;
  __device__ __forceinline__ float score(float s, int, int, int, int, const FaModArgs&) const { return s; }
  __device__ __forceinline__ bool mask(int b, int, int p, int j, const FaModArgs& a) const {
    return j < static_cast<const int32_t*>(a.ptr)[b] || j <= p;
  }
};

#endif  // __HIPCC__

#endif  // EXACT_ATTENTION_72_FA_MODS_H
