// Internal launch parameters shared by the C-ABI host code and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fa_mods.h"

// Everything one launch needs, passed by value as the kernel argument.
struct FaParams {
  const uint16_t* q;  // bfloat16 bit patterns
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  // strides in elements: (batch or page, token, head); head_dim is contiguous
  int64_t q_bs, q_ss, q_hs;
  int64_t k_bs, k_ss, k_hs;
  int64_t v_bs, v_ss, v_hs;
  int64_t o_bs, o_ss, o_hs;
  // LSE: element (b, h, token) at lse + b * lse_bs + h * lse_hs + token
  int64_t lse_bs, lse_hs;
  int B, Nq, Nk, Hq, Hkv, g;
  int hg_count;  // tile head axis: heads_kv when GQA heads are packed into rows, else heads_q
  int gp;        // rows per token in a tile: g when packed, else 1
  int m_blocks;  // row blocks per (sequence, head group); for varlen an upper bound
  int64_t total_tiles;  // dense: exact tile count; varlen: an upper bound (one workgroup per tile)
  // varlen
  const int32_t* cu_q;
  const int32_t* cu_k;
  // paged KV
  const int32_t* block_table;
  const int32_t* cache_seqlens;
  int page, max_blocks, num_splits;
  float* o_part;
  float* lse_part;
  // split-KV decode: sequence of the i-th group of workgroups, longest first
  // (NULL: batch order)
  const int32_t* seq_order;
  // varlen batch over a paged cache: sequences with at most this many packed
  // rows (new tokens x g) run in the decode kernel and get no prefill tiles
  // (0: every sequence runs in the prefill kernel)
  int skip_rows;
  // score transform
  float scale_log2;  // softmax_scale * log2(e)
  float cap_in;      // softmax_scale / softcap
  float cap_out;     // softcap * log2(e)
  int causal, wl, wr;
  // ALiBi: slopes[b * alibi_bs + h] (NULL = none), divided by the softmax scale
  const float* alibi;
  int64_t alibi_bs;
  float alibi_inv_scale;
  // score_mod / mask_mod of a kernel built with a mod (fa_mods.h): its
  // parameters, and the softmax scale the mod's logits carry
  FaModArgs mod;
  float scale;
  // paged decode over an FP8 (e4m3) cache: the V scale, which multiplies O (the
  // K scale is folded into scale_log2 / cap_in)
  float v_scale;
};

// Mods the library is built with (fa_mods.h), for fa_launch_prefill_mod.
enum FaModId { FA_MOD_RELPOS_BIAS = 1, FA_MOD_PREFIX_LM = 2 };

// FP8 (OCP e4m3) forward.  Q in blocks of FA_FP8_Q_BLOCK rows and K in blocks
// of FA_FP8_K_BLOCK keys, one fp32 scale per (batch, head, block); V one scale
// per (batch, KV head), stored transposed (V^T rows of FA_FP8_K_BLOCK-key groups
// in the order the P V product reads them).
#ifndef FA_FP8_Q_BLOCK
#define FA_FP8_Q_BLOCK 128
#define FA_FP8_K_BLOCK 64
#endif
struct FaFp8Params {
  const uint8_t* q;   // e4m3 codes; strides in bytes (batch, token, head), head_dim contiguous
  const uint8_t* k;
  const uint8_t* vt;  // [B, Hkv, head_dim, npad]
  const float* q_scale;  // [B, Hq, q_nblk]
  const float* k_scale;  // [B, Hkv, k_nblk]
  const float* v_scale;  // [B, Hkv]
  uint16_t* o;           // bf16; strides in elements
  float* lse;
  int64_t q_bs, q_ss, q_hs;
  int64_t k_bs, k_ss, k_hs;
  int64_t o_bs, o_ss, o_hs;
  int64_t lse_bs, lse_hs;
  int B, Nq, Nk, Hq, Hkv, g, npad;
  int q_nblk, k_nblk, m_blocks;
  int64_t total_tiles;
  float scale_log2;  // softmax_scale * log2(e)
  int causal, wl, wr;
};
// Quantizer of a [B, N, H, head_dim] bf16 tensor: rows in blocks of `rows`
// (per-block scales) or, for vt != NULL, one scale per head and the codes
// written transposed into vt [B, H, head_dim, npad].
struct FaFp8QuantParams {
  const uint16_t* x;
  int64_t x_bs, x_ss, x_hs;  // elements
  uint8_t* codes;            // rows form: [B, N, H, head_dim] codes
  int64_t c_bs, c_ss, c_hs;  // bytes
  uint8_t* vt;               // transposed form
  float* scales;
  int B, N, H, rows, nblk, npad;
  // rows form: fp32 signs [head_dim] of the randomized Hadamard rotation applied
  // to every row before quantization (NULL: none)
  const float* signs;
};

// Rotary position embedding from caller tables: position pos, frequency i
// rotates the pair of dims (i, i + dim / 2) (or (2i, 2i + 1) when interleaved)
// by cos[pos * dim / 2 + i], sin[pos * dim / 2 + i].
struct FaRotary {
  const float* cos;  // [positions, dim / 2] fp32; NULL = no rotation
  const float* sin;
  int dim;           // rotated head dims, a multiple of 16, <= head_dim
  int interleaved;
};

// In-place rotation of x [B, L, H, head_dim]; token t of sequence b sits at
// position (pos_base ? pos_base[b] : 0) + t.
struct FaRotaryParams {
  uint16_t* x;
  int64_t bs, ss, hs;
  const int32_t* pos_base;
  int B, L, H;
  FaRotary rot;
};

// Backward pass (dense BSHD): gradients of q, k, v from dO, O and the
// forward's log-sum-exp.
struct FaBwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;  // [B, Hq, Nq] (varlen: [Hq, total_q]) natural-log LSE of the forward
  float* delta;      // D = rowsum(dO * O), same layout (workspace)
  float* nlse;       // LSE log2(e), +inf for a row that sees no key, same layout (workspace)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  // strides in elements: (batch, token, head)
  int64_t q_bs, q_ss, q_hs, k_bs, k_ss, k_hs, v_bs, v_ss, v_hs, o_bs, o_ss, o_hs;
  int64_t do_bs, do_ss, do_hs, dq_bs, dq_ss, dq_hs, dk_bs, dk_ss, dk_hs, dv_bs, dv_ss, dv_hs;
  int B, Nq, Nk, Hq, Hkv, g;
  float scale, scale_log2;
  int causal, wl, wr;
  // varlen (cu_q != NULL): sequence b's tokens start at cu_q[b] / cu_k[b] of the
  // token axis (batch strides 0), Nq / Nk are the longest lengths, and the LSE-row
  // arrays are [Hq, total_q]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t total_q;
  // softcap (the forward's transform): cap_in = scale / softcap, cap_out =
  // softcap log2(e); softcap == 0: none
  int softcap;
  float cap_in, cap_out;
};

// In-place append of new K/V tokens to a paged cache.
struct FaAppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t kn_bs, kn_ss, kn_hs;  // new tokens: (batch, token, head) strides in elements
  int64_t vn_bs, vn_ss, vn_hs;
  int64_t k_ps, k_ss, k_hs;     // caches: (page, slot, head) strides in elements
  int64_t v_ps, v_ss, v_hs;
  const int32_t* block_table;
  const int32_t* cache_seqlens;  // lengths before the append
  int B, L, Hkv, page, max_blocks;
  FaRotary rot;                  // applied to the keys (rot.cos == NULL: none)
  // fp8: the caches hold e4m3 codes (uint8, strides in bytes), x / scale rounded
  // to nearest even and saturated at +-448; no rotation
  int fp8;
  float k_scale, v_scale;
};

// Merge of partial attention states.  Row r = (b * Hq + h) * Nq + t of
// rows = B * Hq * Nq.  Partial s of row (b, t, h):
//   O   at (in_bf16 ? bf16 : fp32) element  o_in[s'] + s'' * o_split + b * i_bs + t * i_ss + h * i_hs
//   LSE at                                lse_in[s'] + s'' * lse_split + b * il_bs + h * il_hs + t * il_ss
// where (s', s'') = (s, 0) when pair (two separately placed states, num_splits
// == 2) and (0, s) otherwise.  Output O bf16 at o + b * o_bs + t * o_ss + h * o_hs,
// LSE at lse + b * l_bs + h * l_hs + t * l_ss (may be null).
struct FaCombineParams {
  const void* o_in[2];
  const float* lse_in[2];
  int64_t o_split, lse_split;
  int pair;
  int in_bf16;
  int num_splits;
  int64_t rows;
  int B, Hq, Nq;
  int64_t i_bs, i_ss, i_hs;
  int64_t il_bs, il_hs, il_ss;
  uint16_t* o;
  int64_t o_bs, o_ss, o_hs;
  float* lse;
  int64_t l_bs, l_hs, l_ss;
};

// Compute units of the current device (fa_kernels.hip; 256 if the query fails).
int fa_device_cus();

// Device scratch of the no-allocation paged entry point (fa_kernels.hip): a
// static device array of FA_SCRATCH_BYTES on every device the library runs on.
// fa_scratch_region returns the calling thread's current device's address of it
// (looked up once per device with hipGetSymbolAddress).
constexpr size_t FA_SCRATCH_BYTES = (size_t)32 << 20;
hipError_t fa_scratch_region(void** ptr);

// Launchers (fa_kernels.hip).  They return hipSuccess or the launch error.
hipError_t fa_launch_prefill(const FaParams& p, int d, bool varlen, bool paged, bool pack, bool softcap,
                             hipStream_t s);
// fp8: the caches hold e4m3 codes (strides in bytes), p.v_scale multiplies O.
hipError_t fa_launch_paged(const FaParams& p, int d, bool softcap, bool fp8, hipStream_t stream);
// The unified varlen batch over a paged cache in one launch: pp's prefill tiles
// first, then pd's decode units (B * Hkv * num_splits workgroups).
hipError_t fa_launch_unified(const FaParams& pd, const FaParams& pp, int d, bool pack, bool softcap,
                             hipStream_t s);
// The dense prefill kernel built with a shipped mod (no softcap, no ALiBi).
hipError_t fa_launch_prefill_mod(const FaParams& p, int d, bool pack, int mod_id, hipStream_t s);
// Longest-first order of the sequences by cache length (ties by index) into
// order[0, B); B at most FA_SEQ_ORDER_MAX.
constexpr int FA_SEQ_ORDER_MAX = 4096;
hipError_t fa_launch_seq_order(const int32_t* lens, int B, int32_t* order, hipStream_t stream);
hipError_t fa_launch_combine(const FaCombineParams& p, int d, hipStream_t stream);
// Combine of the varlen paged decode partials (packed per (sequence, KV head)
// unit, FA_PAGED_MAX_ROWS rows each) into p.o / p.lse ([total_q, Hq] layouts).
hipError_t fa_launch_combine_packed(const FaParams& p, int d, hipStream_t stream);
hipError_t fa_launch_append(const FaAppendParams& p, int d, hipStream_t stream);
hipError_t fa_launch_rotary(const FaRotaryParams& p, int d, hipStream_t stream);
hipError_t fa_launch_fp8_quant(const FaFp8QuantParams& p, int d, hipStream_t s);
hipError_t fa_launch_fp8_fwd(const FaFp8Params& p, int d, hipStream_t s);
hipError_t fa_launch_bwd(const FaBwdParams& p, int d, hipStream_t stream);

// Tile geometry of the prefill kernel.
constexpr int FA_BLOCK_M = 128;     // query rows per workgroup tile (4 waves x 32)
constexpr int FA_BLOCK_N = 32;      // keys per K/V block (one LDS stage)
constexpr int FA_PAGED_STAGE = 64;  // keys per stage in the paged kernel (4 waves x 16)
constexpr int FA_PAGED_MAX_ROWS = 32;
