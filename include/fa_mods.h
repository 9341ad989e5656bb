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
 *   static constexpr bool kBlocks;  // key_end() and block_visible() narrow the work
 *   struct Tile;                    // per-tile state
 *   __device__ Tile  tile(int b, const FaModArgs& a) const;
 *   __device__ float score(float s, int b, int h, int p, int j, const Tile& t, const FaModArgs& a) const;
 *   __device__ bool  mask(int b, int h, int p, int j, const Tile& t, const FaModArgs& a) const;
 *   __device__ int   key_end(int p_lo, int p_hi, const Tile& t) const;
 *   __device__ bool  block_visible(int p_lo, int p_hi, int j0, int j1, const Tile& t) const;
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
 * tile() runs once per tile of query rows (all of sequence b) and loads what the
 * mod needs of sequence b, so that score() and mask() touch no memory per score;
 * it must read wave-uniform addresses only (fa_mod_uniform_i32 does a scalar
 * load).  With kBlocks, key_end() bounds the keys mask() can keep for query
 * positions p_lo .. p_hi (keys at or past it are never visible; the kernel skips
 * their blocks) and block_visible() says whether mask() keeps every pair of those
 * positions with keys j0 .. j1 (the kernel then skips mask() on that block).  Both
 * may be conservative (a larger bound, false) but never optimistic.
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

// A 32-bit value at a wave-uniform address, by a scalar load.
__device__ __forceinline__ int32_t fa_mod_uniform_i32(const int32_t* ptr) {
  const uint64_t u = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const int32_t* q = reinterpret_cast<const int32_t*>(((uint64_t)hi << 32) | lo);
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q) : "memory");
  return v;
}

// No rewrite, no extra mask: the plain kernel.
struct FaNoMod {
  static constexpr bool kScore = false;
  static constexpr bool kMask = false;
  static constexpr bool kBlocks = false;
  struct Tile {};
  __device__ __forceinline__ Tile tile(int, const FaModArgs&) const { return {}; }
  __device__ __forceinline__ float score(float s, int, int, int, int, const Tile&, const FaModArgs&) const { return s; }
  __device__ __forceinline__ bool mask(int, int, int, int, const Tile&, const FaModArgs&) const { return true; }
  __device__ __forceinline__ int key_end(int, int, const Tile&) const { return 0x7fffffff; }
  __device__ __forceinline__ bool block_visible(int, int, int, int, const Tile&) const { return true; }
};

// Learned relative-position bias (score_mod): the logit of query position p and
// key j gets bias[h][clamp(j - p, -R, R) + R] added, from a device fp32 table
// of heads_q rows of 2R + 1 entries (a.ptr, row stride a.i0 = 2R + 1, a.i1 = R).
// Distances beyond R share the end entries.
struct FaRelPosBias {
  static constexpr bool kScore = true;
  static constexpr bool kMask = false;
  static constexpr bool kBlocks = false;
  struct Tile {};
  __device__ __forceinline__ Tile tile(int, const FaModArgs&) const { return {}; }
  __device__ __forceinline__ float score(float s, int, int h, int p, int j, const Tile&, const FaModArgs& a) const {
    const int R = (int)a.i1;
    int r = j - p;
    r = r < -R ? -R : (r > R ? R : r);
    return s + static_cast<const float*>(a.ptr)[(int64_t)h * a.i0 + r + R];
  }
  __device__ __forceinline__ bool mask(int, int, int, int, const Tile&, const FaModArgs&) const { return true; }
  __device__ __forceinline__ int key_end(int, int, const Tile&) const { return 0x7fffffff; }
  __device__ __forceinline__ bool block_visible(int, int, int, int, const Tile&) const { return true; }
};

// Prefix-LM mask (mask_mod): the first prefix_len[b] keys of sequence b are
// visible to every query (a bidirectional prefix), later keys causally (key j
// visible to the query at position p iff j < prefix_len[b] or j <= p).
// a.ptr: device int32 [batch].  Keys at or past max(prefix_len[b], p_hi + 1) are
// never visible; a block of keys is visible whole when it ends inside the prefix
// or at or before the first position.
struct FaPrefixLM {
  static constexpr bool kScore = false;
  static constexpr bool kMask = true;
  static constexpr bool kBlocks = true;
  struct Tile {
    int prefix;
  };
  __device__ __forceinline__ Tile tile(int b, const FaModArgs& a) const {
    return {fa_mod_uniform_i32(static_cast<const int32_t*>(a.ptr) + b)};
  }
  __device__ __forceinline__ float score(float s, int, int, int, int, const Tile&, const FaModArgs&) const { return s; }
  __device__ __forceinline__ bool mask(int, int, int p, int j, const Tile& t, const FaModArgs&) const {
    return j < t.prefix || j <= p;
  }
  __device__ __forceinline__ int key_end(int, int p_hi, const Tile& t) const {
    return t.prefix > p_hi + 1 ? t.prefix : p_hi + 1;
  }
  __device__ __forceinline__ bool block_visible(int p_lo, int, int, int j1, const Tile& t) const {
    return j1 < t.prefix || j1 <= p_lo;
  }
};

#endif  // __HIPCC__

#endif  // EXACT_ATTENTION_72_FA_MODS_H
