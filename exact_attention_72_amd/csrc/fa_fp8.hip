// FP8 (OCP e4m3) attention forward for gfx950: the per-block quantizers and the
// attention kernel.
//
// "Attention kernels: FlashAttention and PagedAttention", section 4.2 (the FP8
// item of FlashAttention-3): Q, K and V enter the matrix products as FP8 e4m3,
// quantized with per-block scales, and V is laid out k-major for the P V
// product.  "01 FlashAttention project overview & architecture", section 2.2:
// an FP8 E4M3 forward.
//
// gfx950 has the 32x32x64 FP8 product (v_mfma_scale_f32_32x32x64_f8f6f4, here
// with unit block scales) and a two-value fp32 -> e4m3 conversion
// (v_cvt_pk_fp8_f32, round to nearest even).  The layout follows the bf16
// kernels (transposed orientation: S^T = K Q^T and O^T = V^T P^T, a lane owns a
// query), with 64-key blocks: a 64-wide product step consumes a whole block.
//
// Scales: a Q block is the 128 query rows of a workgroup, a K block the 64 keys
// of a step, so both fold into the exponent's scalar factor; V has one scale per
// (batch, KV head), applied once to O.  Probabilities enter the P V product as
// 2^8 p relative to the row's reference, which trails the running maximum by
// at most 0.75 in log2 units (so at most 2^8.75 = 430, inside e4m3's 448), and
// keep e4m3's normal range down to 2^-14 of the maximum or less.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_blockinfo.h"
#include "fa_internal.h"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kFp8Max = 448.0f;
constexpr float kPShift = 8.0f;  // log2 of the factor probabilities carry into the P V product
// Largest lead (log2 units) of a score over the row reference left without a
// move: 2^(kPShift + kLazy) = 430 stays inside e4m3's 448.
constexpr float kLazy = 0.75f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// lanes l and l ^ 32 hold the same query column
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// 32x32 fp32 accumulator += A (32 x 64 e4m3) B (64 x 32 e4m3); unit block scales
// (e8m0 127 = 2^0).  Lane l holds row (A) / column (B) l % 32; both operands
// take their 32 k-values per lane in the same order.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four fp32 values -> four e4m3 bytes (round to nearest even), first value lowest.
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// x / scale, clamped to the e4m3 range, as four bytes
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float scale) {
  auto q = [&](float x) { return fminf(fmaxf(x / scale, -kFp8Max), kFp8Max); };
  return pack4(q(a), q(b), q(c), q(d));
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const FA_LDS char*)p);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Each wave has waited (vmcnt) for its DMA of the block the barrier publishes and
// its LDS reads of the buffer about to be refilled have completed; the asm
// statements keep memory operations on their side.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// LDS reads go out as inline assembly (the compiler would otherwise wait for
// every LDS-DMA load in flight before them), each statement with its own wait.
__device__ __forceinline__ i32x8 join(u32x4 a, u32x4 b) {
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
// Scalar load of a float at a wave-uniform address (a vector load would be
// waited for with vmcnt(0), which also drains the LDS-DMA loads in flight).
__device__ __forceinline__ float scalar_load_f32(const float* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const float* u = reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
  float v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(u) : "memory");
  return v;
}

// LDS-DMA through a buffer resource (buffer_load_dwordx4 ... lds): the base in
// scalar registers (taken from the first lane; callers pass wave-uniform
// addresses), a 32-bit byte offset per lane and one per instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, 0x7fffffff, 0x00020000);
}

// Position p of a 64-key group in the product's k order <-> key of the group:
// p = 32 kg + 16 hb + 4 j + i holds key 32 hb + 8 j + 4 kg + i, which is where
// the S^T accumulator of half hb keeps that key for lane half kg (slot 4 j + i).
__device__ __forceinline__ int vt_key_of_position(int p) {
  const int kg = p >> 5, hb = (p >> 4) & 1, j = (p >> 2) & 3, i = p & 3;
  return 32 * hb + 8 * j + 4 * kg + i;
}

// Block maximum of |x| over the workgroup (every thread gets it).
__device__ __forceinline__ float block_amax(float m, float* red) {
  m = wave_max(m);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ------------------------------------------------------------------ quantizers
// Rows form: one workgroup per (batch, head, block of p.rows rows).  The block's
// amax gives scale = amax / 448 (1 for an all-zero block); a code is the e4m3
// rounding of the fp32 quotient x / scale.
//
// ROT (incoherent processing, "Attention kernels...", section 4.2): every row x
// is first replaced by x diag(s) H / sqrt(D) (H the Sylvester Hadamard matrix,
// s the caller's signs), formed in fp32 by the Walsh-Hadamard butterfly: pairs
// (i, i + h) become (a + b, a - b) for h = 1, 2, ..., D / 2 in that order.  A
// thread holds 8 consecutive values of a row and the row's D / 8 chunks sit in
// consecutive lanes, so h = 1, 2, 4 run in registers and h = 8 .. D / 2 across
// lanes (lane bit j = chunk bit j); the amax pass and the code pass both form
// the rotated values (the same operations, so the same numbers).
template <int D, bool ROT>
__global__ __launch_bounds__(kThreads) void fa_fp8_quant_rows_kernel(FaFp8QuantParams p) {
  __shared__ float red[4];
  constexpr int CPR = D / 8;  // 16-byte chunks (8 values) per row
  static_assert(kThreads % CPR == 0 && 64 % CPR == 0, "a row's chunks in consecutive lanes of one wave");
  const int blk = (int)(blockIdx.x % p.nblk);
  const int bh = (int)(blockIdx.x / p.nblk);
  const int b = bh / p.H, h = bh % p.H;
  const int r0 = blk * p.rows;
  const int rows = min(p.rows, p.N - r0);
  const int nch = rows * CPR;
  const int cc = threadIdx.x % CPR;  // this thread's chunk of every row it touches
  const uint16_t* xb = p.x + (int64_t)b * p.x_bs + (int64_t)h * p.x_hs;
  float sg[8];
  if constexpr (ROT) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = p.signs[8 * cc + e];
  }
  // the 8 fp32 values of chunk c (rotated with ROT); every lane of the wave runs
  // this (the butterfly's lane exchanges), lanes past the block load zeros
  auto values = [&](int c, bool valid, float (&y)[8]) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (valid) v = *reinterpret_cast<const u32x4*>(xb + (int64_t)(r0 + c / CPR) * p.x_ss + 8 * cc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = bf16_to_f32(v[e] & 0xFFFFu);
      y[2 * e + 1] = bf16_to_f32(v[e] >> 16);
    }
    if constexpr (ROT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= sg[e];
#pragma unroll
      for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & hh) == 0) {
            const float a = y[i], bb = y[i | hh];
            y[i] = a + bb;
            y[i | hh] = a - bb;
          }
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int m = 1; m < CPR; m <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float o = __shfl_xor(y[e], m);
          y[e] = (lane & m) ? o - y[e] : y[e] + o;   // the low index's value minus the high one's
        }
      constexpr float kInvSqrtD = D == 128 ? (float)0.08838834764831845 : 0.125f;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= kInvSqrtD;
    }
  };
  float m = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += kThreads) {
    const int c = c0 + (int)threadIdx.x;
    float y[8];
    values(c, c < nch, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[e]));
  }
  const float amax = block_amax(m, red);
  const float scale = amax > 0.0f ? amax / kFp8Max : 1.0f;
  if (threadIdx.x == 0) p.scales[(int64_t)bh * p.nblk + blk] = scale;
  uint8_t* cb = p.codes + (int64_t)b * p.c_bs + (int64_t)h * p.c_hs;
  for (int c0 = 0; c0 < nch; c0 += kThreads) {
    const int c = c0 + (int)threadIdx.x;
    float y[8];
    values(c, c < nch, y);
    if (c < nch) {
      u32x2 out;
      out.x = quant4(y[0], y[1], y[2], y[3], scale);
      out.y = quant4(y[4], y[5], y[6], y[7], scale);
      *reinterpret_cast<u32x2*>(cb + (int64_t)(r0 + c / CPR) * p.c_ss + 8 * cc) = out;
    }
  }
}

// Transposed form for V: one scale over each (batch, KV head), codes written to
// vt [B, H, D, npad] row d, group n at bytes 64 n .. + 63, position p holding key
// 64 n + vt_key_of_position(p) (0 past the last key).  Four launches: the head
// maxima are cleared, gathered per 64-key group with an integer atomic maximum
// (non-negative floats order like their bit patterns, so the result does not
// depend on the order), used by every group to write its codes, and finally
// turned into the scales.  The maxima live in the scales array meanwhile.
__global__ __launch_bounds__(kThreads) void fa_fp8_vt_clear_kernel(FaFp8QuantParams p) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < p.B * p.H) p.scales[i] = 0.0f;
}
__global__ __launch_bounds__(kThreads) void fa_fp8_vt_scale_kernel(FaFp8QuantParams p) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < p.B * p.H) {
    const float amax = p.scales[i];
    p.scales[i] = amax > 0.0f ? amax / kFp8Max : 1.0f;
  }
}
// one workgroup per (batch, KV head, 64-key group)
template <int D>
__global__ __launch_bounds__(kThreads) void fa_fp8_vt_amax_kernel(FaFp8QuantParams p) {
  __shared__ float red[4];
  constexpr int CPR = D / 8;
  const int ng = p.npad / 64;
  const int n = (int)(blockIdx.x % ng);
  const int bh = (int)(blockIdx.x / ng);
  const int b = bh / p.H, h = bh % p.H;
  const uint16_t* xb = p.x + (int64_t)b * p.x_bs + (int64_t)h * p.x_hs;
  float m = 0.0f;
  for (int c = threadIdx.x; c < 64 * CPR; c += kThreads) {
    const int key = 64 * n + c / CPR;
    if (key >= p.N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(xb + (int64_t)key * p.x_ss + 8 * (c % CPR));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m = fmaxf(m, fabsf(bf16_to_f32(v[e] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_to_f32(v[e] >> 16)));
    }
  }
  const float amax = block_amax(m, red);
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(p.scales + bh), __float_as_uint(amax));
}
template <int D>
__global__ __launch_bounds__(kThreads) void fa_fp8_vt_write_kernel(FaFp8QuantParams p) {
  __shared__ uint16_t tile[64][D + 8];
  constexpr int CPR = D / 8;
  const int ng = p.npad / 64;
  const int n = (int)(blockIdx.x % ng);
  const int bh = (int)(blockIdx.x / ng);
  const int b = bh / p.H, h = bh % p.H;
  const float amax = p.scales[bh];
  const float scale = amax > 0.0f ? amax / kFp8Max : 1.0f;
  const uint16_t* xb = p.x + (int64_t)b * p.x_bs + (int64_t)h * p.x_hs;
  for (int c = threadIdx.x; c < 64 * CPR; c += kThreads) {
    const int key = 64 * n + c / CPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < p.N) v = *reinterpret_cast<const u32x4*>(xb + (int64_t)key * p.x_ss + 8 * (c % CPR));
    uint16_t* t = &tile[c / CPR][8 * (c % CPR)];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[2 * e] = (uint16_t)(v[e] & 0xFFFFu);
      t[2 * e + 1] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
  uint8_t* vb = p.vt + (int64_t)bh * D * p.npad;
  for (int task = threadIdx.x; task < 2 * D; task += kThreads) {  // (row d, half of the group)
    const int d = task >> 1, half = task & 1;
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int p0 = 32 * half + 4 * q;
      w[q] = quant4(bf16_to_f32(tile[vt_key_of_position(p0)][d]), bf16_to_f32(tile[vt_key_of_position(p0 + 1)][d]),
                    bf16_to_f32(tile[vt_key_of_position(p0 + 2)][d]), bf16_to_f32(tile[vt_key_of_position(p0 + 3)][d]),
                    scale);
    }
    uint8_t* dst = vb + (int64_t)d * p.npad + 64 * n + 32 * half;
    *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(dst + 16) = u32x4{w[4], w[5], w[6], w[7]};
  }
}

// ------------------------------------------------------------------ attention
// One workgroup per (batch, query head, 128-row block), longest row blocks
// first; four waves of 32 query rows; 64-key blocks through a ring of four LDS
// stages filled by LDS-DMA.  A stage holds the block's K rows (64 x D bytes,
// 16-byte chunk c of row r stored at chunk c ^ ((r >> 1) & 7)) and its V^T rows
// (D x 64 bytes, chunk c of row r at c ^ ((r >> 2) & 3)); both swizzles give
// the 16 lanes of a 16-byte read distinct banks.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void fa_fp8_fwd_kernel(FaFp8Params p) {
  static_assert(D == 128, "the FP8 kernel is built for head_dim 128");
  constexpr int BN = FA_FP8_K_BLOCK;  // 64
  constexpr int NBUF = 4;
  constexpr int KT = BN * D;  // K bytes of a block
  constexpr int VT = D * BN;  // V^T bytes of a block
  constexpr int STAGE = KT + VT;
  constexpr int kDmaPerBlock = (KT + VT) / 1024 / 4;  // LDS-DMA instructions per wave and block
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, kg = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- tile
  const int64_t t = blockIdx.x;
  if (t >= p.total_tiles) return;
  const int64_t pairs = (int64_t)p.B * p.Hq;
  const int mb = p.m_blocks - 1 - (int)(t / pairs);
  const int b = (int)((t % pairs) / p.Hq), h = (int)((t % pairs) % p.Hq);
  const int kvh = h / p.g;
  const int Lq = p.Nq, Lk = p.Nk;
  const int m0 = mb * FA_FP8_Q_BLOCK;
  const int m_end = min(m0 + FA_FP8_Q_BLOCK, Lq);
  FaRowSpan span;
  span.pos_lo = (int64_t)m0 + (Lk - Lq);
  span.pos_hi = (int64_t)(m_end - 1) + (Lk - Lq);
  int n_lo, n_hi;
  fa_key_tiles(span, Lk, p.causal, p.wl, p.wr, BN, &n_lo, &n_hi);
  // key blocks [n_full_lo, n_full_hi) need no element mask: the closed-form range
  // of tiles the classifier calls full (one interval), within [n_lo, n_hi)
  int n_full_lo = n_hi, n_full_hi = n_hi;
  {
    int f_lo, f_hi;
    fa_full_tiles(span, Lk, p.causal, p.wl, p.wr, BN, &f_lo, &f_hi);
    f_lo = max(f_lo, n_lo);
    f_hi = min(f_hi, n_hi);
    if (f_lo < f_hi) {
      n_full_lo = f_lo;
      n_full_hi = f_hi;
    }
  }
  const int nb = n_hi - n_lo;

  // ---- this lane's query row: Q as the B operand (32 bytes of each 64-dim chunk)
  const int row = m0 + wave * 32 + col;
  const bool row_ok = row < Lq;
  i32x8 qreg[D / 64];
  {
    const uint8_t* qr = p.q + (int64_t)b * p.q_bs + (int64_t)(row_ok ? row : 0) * p.q_ss + (int64_t)h * p.q_hs;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (row_ok) {
        x = *reinterpret_cast<const u32x4*>(qr + 64 * c + 32 * kg);
        y = *reinterpret_cast<const u32x4*>(qr + 64 * c + 32 * kg + 16);
      }
      qreg[c] = join(x, y);
    }
  }
  const float cq = p.scale_log2 * scalar_load_f32(p.q_scale + ((int64_t)b * p.Hq + h) * p.q_nblk + mb);
  const float v_scale = scalar_load_f32(p.v_scale + (int64_t)b * p.Hkv + kvh);
  const float* kscale = p.k_scale + ((int64_t)b * p.Hkv + kvh) * p.k_nblk;
  const int pos = row + (Lk - Lq);

  // ---- LDS-DMA: instruction j of wave w fills 1 KiB of K (rows (4 j + w) * 8 ..)
  // and 1 KiB of V^T (rows (4 j + w) * 16 ..); this lane's chunk of each
  const uint8_t* kbase = p.k + (int64_t)b * p.k_bs + (int64_t)kvh * p.k_hs;
  const uint8_t* vtbase = p.vt + ((int64_t)b * p.Hkv + kvh) * D * p.npad;
  // A full block goes through buffer resources based at its first key: this
  // lane's row of instruction 0 and its chunk are fixed (the swizzles depend on
  // row bits that the 32- and 64-row steps between instructions leave alone), so
  // each instruction adds only a scalar offset (the host keeps 64 K rows and the
  // D V^T rows below 2^31 bytes).  A final partial block keeps per-lane
  // addresses, its rows clamped to the last key.
  const int kr0 = wave * 8 + lane / 8, vr0 = wave * 16 + lane / 4;
  const uint32_t k_voff = (uint32_t)(kr0 * p.k_ss) + 16u * (uint32_t)((lane & 7) ^ ((kr0 >> 1) & 7));
  const uint32_t v_voff = (uint32_t)(vr0 * p.npad) + 16u * (uint32_t)((lane & 3) ^ ((vr0 >> 2) & 3));
  const uint32_t k_step = (uint32_t)(32 * p.k_ss), v_step = (uint32_t)(64 * p.npad);
  auto issue = [&](int i) __attribute__((always_inline)) {
    char* st = smem + (i % NBUF) * STAGE;
    const int n = n_lo + i;
    if ((n + 1) * BN <= Lk) {
      const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kbase + (int64_t)n * BN * p.k_ss);
      const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vtbase + (int64_t)n * BN);
#pragma unroll
      for (int j = 0; j < KT / 4096; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(st + (4 * j + wave) * 1024), 16, (int)k_voff,
                                                 (int)(j * k_step), 0, 0);
#pragma unroll
      for (int j = 0; j < VT / 4096; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(st + KT + (4 * j + wave) * 1024), 16,
                                                 (int)v_voff, (int)(j * v_step), 0, 0);
      return;
    }
#pragma unroll
    for (int j = 0; j < KT / 4096; ++j) {
      const int r = (4 * j + wave) * 8 + lane / 8;
      const int key = min(n * BN + r, Lk - 1);
      const uint8_t* src = kbase + (int64_t)key * p.k_ss + 16 * ((lane & 7) ^ ((r >> 1) & 7));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (FA_LDS void*)(st + (4 * j + wave) * 1024),
                                       16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < VT / 4096; ++j) {
      const int r = (4 * j + wave) * 16 + lane / 4;
      const uint8_t* src = vtbase + (int64_t)r * p.npad + (int64_t)n * BN + 16 * ((lane & 3) ^ ((r >> 2) & 3));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (FA_LDS void*)(st + KT + (4 * j + wave) * 1024), 16, 0, 0);
    }
  };
  // operand addresses within a stage: K row 32 hb + col, chunks 4 c + 2 kg + e;
  // V^T row 32 db + col, chunks 2 kg + e
  const uint32_t base = lds_addr(smem);
  const uint32_t ka = base + col * D, ksw = (col >> 1) & 7;
  const uint32_t va = base + KT + col * BN, vsw = (col >> 2) & 3;
  // The operand reads go out as one asm statement with the wait for them (and
  // for the block's K scale, loaded in the same statement), so that the
  // compiler sees the results defined only once they have landed: with reads
  // and wait in separate statements it copied read results into the 8-register
  // operand tuples before the wait.  kr[4 hb + 2 c + e]: K row 32 hb + col,
  // chunk 4 c + 2 kg + e (hb is an immediate offset of 32 rows); vr[2 db + e]:
  // V^T row 32 db + col, chunk 2 kg + e (db an immediate offset of 32 rows).
  static_assert(D == 128 && 32 * D == 4096 && 32 * BN == 2048, "the immediate offsets below");
  auto k_addrs = [&](int i, uint32_t (&a)[4]) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)((i % NBUF) * STAGE);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) a[2 * c + e] = ka + so + 16 * ((4 * c + 2 * kg + e) ^ ksw);
  };
  auto v_addrs = [&](int i, uint32_t (&a)[2]) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)((i % NBUF) * STAGE);
#pragma unroll
    for (int e = 0; e < 2; ++e) a[e] = va + so + 16 * ((2 * kg + e) ^ vsw);
  };
  auto s_mfma = [&](const u32x4 (&kr)[8], f32x16 (&sv)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sv[hb] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 64; ++c)
        sv[hb] = mfma_fp8(join(kr[4 * hb + 2 * c], kr[4 * hb + 2 * c + 1]), qreg[c], sv[hb]);
    }
  };
  // block n's K scale address, wave-uniform (for a scalar load)
  auto kscale_ptr = [&](int n) __attribute__((always_inline)) {
    const uint64_t a = reinterpret_cast<uint64_t>(kscale + n);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
  };
  // K of block ik with its scale, and V^T of block iv: reads and wait in one statement
  auto read_kv = [&](int ik, int iv, u32x4 (&kr)[8], u32x4 (&vr)[8], float& ks) __attribute__((always_inline)) {
    uint32_t a[4], b2[2];
    k_addrs(ik, a);
    v_addrs(iv, b2);
    asm volatile(
        "s_load_dword %16, %23, 0x0\n\t"
        "ds_read_b128 %0, %17\n\tds_read_b128 %1, %18\n\tds_read_b128 %2, %19\n\tds_read_b128 %3, %20\n\t"
        "ds_read_b128 %4, %17 offset:4096\n\tds_read_b128 %5, %18 offset:4096\n\t"
        "ds_read_b128 %6, %19 offset:4096\n\tds_read_b128 %7, %20 offset:4096\n\t"
        "ds_read_b128 %8, %21\n\tds_read_b128 %9, %22\n\t"
        "ds_read_b128 %10, %21 offset:2048\n\tds_read_b128 %11, %22 offset:2048\n\t"
        "ds_read_b128 %12, %21 offset:4096\n\tds_read_b128 %13, %22 offset:4096\n\t"
        "ds_read_b128 %14, %21 offset:6144\n\tds_read_b128 %15, %22 offset:6144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7]), "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]),
          "=&v"(vr[6]), "=&v"(vr[7]), "=&s"(ks)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b2[0]), "v"(b2[1]), "s"(kscale_ptr(n_lo + ik))
        : "memory");
  };
  // K of block ik with its scale only (the first block)
  auto read_k = [&](int ik, u32x4 (&kr)[8], float& ks) __attribute__((always_inline)) {
    uint32_t a[4];
    k_addrs(ik, a);
    asm volatile(
        "s_load_dword %8, %13, 0x0\n\t"
        "ds_read_b128 %0, %9\n\tds_read_b128 %1, %10\n\tds_read_b128 %2, %11\n\tds_read_b128 %3, %12\n\t"
        "ds_read_b128 %4, %9 offset:4096\n\tds_read_b128 %5, %10 offset:4096\n\t"
        "ds_read_b128 %6, %11 offset:4096\n\tds_read_b128 %7, %12 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7]), "=&s"(ks)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "s"(kscale_ptr(n_lo + ik))
        : "memory");
  };
  // V^T of block iv only (the last block)
  auto read_v = [&](int iv, u32x4 (&vr)[8]) __attribute__((always_inline)) {
    uint32_t b2[2];
    v_addrs(iv, b2);
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %9 offset:2048\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %9 offset:4096\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %9 offset:6144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7])
        : "v"(b2[0]), "v"(b2[1])
        : "memory");
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;  // m in log2 units (scores times their scales)
  f32x16 x0 = {}, x1 = {};               // 2^8 p of the current block (relative to m_run)

  // Scores of block i (in sv) -> masked, reference moved (O rescaled), exponentials.
  auto softmax = [&](f32x16 (&sv)[2], int i, float cb) __attribute__((always_inline)) {
    const int n = n_lo + i;
    if (n < n_full_lo || n >= n_full_hi) {
      // the row's visible keys in the block are the offsets [lo, hi] from base;
      // slot (hb, a) holds offset 32 hb + 8 (a / 4) + a % 4, a compile-time
      // constant, so a score costs one compare (two with a left window)
      int base = n * BN + 4 * kg;
      asm volatile("" : "+v"(base));  // keeps the offsets out of loop-invariant registers
      int64_t hi = (int64_t)Lk - 1 - base;
      if (p.causal) hi = min(hi, (int64_t)pos - base);
      if (p.wr >= 0) hi = min(hi, (int64_t)pos + p.wr - base);
      int h = (int)max(min(hi, (int64_t)BN), (int64_t)-1);
      asm volatile("" : "+v"(h));  // 32-bit compares below (the bound fits)
      if (p.wl < 0) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int off = 32 * hb + 8 * (a >> 2) + (a & 3);
            sv[hb][a] = off <= h ? sv[hb][a] : kNegInf;
          }
      } else {
        const int64_t lo = (int64_t)pos - p.wl - base;
        int l = (int)max(min(lo, (int64_t)BN), (int64_t)0);
        asm volatile("" : "+v"(l));
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int off = 32 * hb + 8 * (a >> 2) + (a & 3);
            sv[hb][a] = (off <= h && off >= l) ? sv[hb][a] : kNegInf;
          }
      }
    }
    // Exponent arguments relative to the current reference first (multiply-adds,
    // whose results the block maximum then takes without canonicalising each
    // score), the reference moved only when the block's maximum exceeds it by
    // more than kLazy: then 2^8 p stays below 2^(8 + kLazy) < 448 without a move,
    // and a move (which rescales O) is rare once a row has seen a few blocks.
    const float nmc_old = (m_run == kNegInf) ? 0.0f : kPShift - m_run;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      x0[a] = __builtin_fmaf(sv[0][a], cb, nmc_old);
      x1[a] = __builtin_fmaf(sv[1][a], cb, nmc_old);
    }
    float ym = fmaxf(fmaxf(x0[0], x0[1]), x1[0]);
    ym = fmaxf(ym, x1[1]);
#pragma unroll
    for (int a = 2; a < 16; ++a) ym = fmaxf(fmaxf(ym, x0[a]), x1[a]);
    ym = pair_max(ym);
    // the block maximum in log2 units is ym + m_run - kPShift (ym while the row has
    // no reference); -inf - (-inf) is NaN, which compares false: no move while
    // nothing is visible
    const float mx = (m_run == kNegInf) ? ym : ym - nmc_old;
    const bool mv = mx - m_run > kLazy;
    if (__any(mv)) {
      const float m_new = mv ? mx : m_run;
      const float alpha = mv ? exp2_fast(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      m_run = m_new;
      const float nmc = (m_run == kNegInf) ? 0.0f : kPShift - m_run;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        x0[a] = __builtin_fmaf(sv[0][a], cb, nmc);
        x1[a] = __builtin_fmaf(sv[1][a], cb, nmc);
      }
    }
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      x0[a] = exp2_fast(x0[a]);
      x1[a] = exp2_fast(x1[a]);
    }
  };

  // Ring of NBUF stages, the DMA of block i + NBUF - 1 issued at step i.  Step i
  // reads block i + 1's K and forms its scores while block i's P V products run.
  // Wait for a block whose DMA was followed by `after` later blocks' DMAs.
  auto wait_block = [&](int after) __attribute__((always_inline)) {
    switch (after) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<kDmaPerBlock>(); break;
      default: wait_vmcnt<2 * kDmaPerBlock>(); break;
    }
  };
  if (nb > 0) {
    for (int j = 0; j < NBUF - 1 && j < nb; ++j) issue(j);
    wait_block(min(nb - 1, NBUF - 2));  // block 0; blocks 1 .. NBUF - 2 may be in flight
    stage_barrier();
    float ks;
    u32x4 kr[8];
    read_k(0, kr, ks);
    f32x16 sv[2];
    s_mfma(kr, sv);
    softmax(sv, 0, cq * ks);
  }
  for (int i = 0; i < nb; ++i) {
    const bool more = i + 1 < nb;
    if (more) {
      // block i + 1; issued so far: blocks up to i + NBUF - 2
      wait_block(min(nb - 1, i + NBUF - 2) - (i + 1));
      stage_barrier();  // everyone is done with block i - 1's stage
      if (i + NBUF - 1 < nb) issue(i + NBUF - 1);
    }
    // block i's probabilities as the B operand (bytes 16 hb + slot of this lane's 32)
    float rs = 0.0f;
#pragma unroll
    for (int a = 0; a < 16; ++a) rs += x0[a] + x1[a];
    l_run += rs;
    i32x8 pb;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pb[w] = (int)pack4(x0[4 * w], x0[4 * w + 1], x0[4 * w + 2], x0[4 * w + 3]);
      pb[4 + w] = (int)pack4(x1[4 * w], x1[4 * w + 1], x1[4 * w + 2], x1[4 * w + 3]);
    }
    // block i + 1's K (and scale) and block i's V^T, landed when the statement ends
    u32x4 kr[8], vr[8];
    float ks = 1.0f;
    f32x16 sv[2];
    if (more) {
      read_kv(i + 1, i, kr, vr, ks);
      s_mfma(kr, sv);
    } else {
      read_v(i, vr);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = mfma_fp8(join(vr[2 * db], vr[2 * db + 1]), pb, o[db]);
    if (more) softmax(sv, i + 1, cq * ks);
  }

  // ---- epilogue: O = v_scale O^T / l, LSE = (m - 8 + log2 l) ln 2
  const float l_tot = pair_sum(l_run);
  const bool empty = (m_run == kNegInf) || !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : v_scale * rcp_fast(l_tot);
  if (row_ok) {
    uint16_t* ob = p.o + (int64_t)b * p.o_bs + (int64_t)row * p.o_ss + (int64_t)h * p.o_hs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = o[db][4 * q4 + e] * inv;
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        *reinterpret_cast<u32x2*>(ob + 32 * db + 8 * q4 + 4 * kg) = __builtin_bit_cast(u32x2, y);
      }
    if (kg == 0 && p.lse)
      p.lse[(int64_t)b * p.lse_bs + (int64_t)h * p.lse_hs + row] =
          empty ? kNegInf : (m_run - kPShift + log2_fast(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t fa_launch_fp8_quant(const FaFp8QuantParams& p, int d, hipStream_t s) {
  if (d != 128 && d != 64) return hipErrorInvalidValue;
  if (p.vt) {
    const unsigned heads = (unsigned)((p.B * p.H + kThreads - 1) / kThreads);
    const unsigned groups = (unsigned)((int64_t)p.B * p.H * (p.npad / 64));
    hipLaunchKernelGGL(fa_fp8_vt_clear_kernel, dim3(heads), dim3(kThreads), 0, s, p);
    if (d == 128) {
      hipLaunchKernelGGL(fa_fp8_vt_amax_kernel<128>, dim3(groups), dim3(kThreads), 0, s, p);
      hipLaunchKernelGGL(fa_fp8_vt_write_kernel<128>, dim3(groups), dim3(kThreads), 0, s, p);
    } else {
      hipLaunchKernelGGL(fa_fp8_vt_amax_kernel<64>, dim3(groups), dim3(kThreads), 0, s, p);
      hipLaunchKernelGGL(fa_fp8_vt_write_kernel<64>, dim3(groups), dim3(kThreads), 0, s, p);
    }
    hipLaunchKernelGGL(fa_fp8_vt_scale_kernel, dim3(heads), dim3(kThreads), 0, s, p);
  } else {
    const unsigned grid = (unsigned)((int64_t)p.B * p.H * p.nblk);
    if (d == 128 && p.signs)
      hipLaunchKernelGGL((fa_fp8_quant_rows_kernel<128, true>), dim3(grid), dim3(kThreads), 0, s, p);
    else if (d == 128)
      hipLaunchKernelGGL((fa_fp8_quant_rows_kernel<128, false>), dim3(grid), dim3(kThreads), 0, s, p);
    else if (p.signs)
      hipLaunchKernelGGL((fa_fp8_quant_rows_kernel<64, true>), dim3(grid), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((fa_fp8_quant_rows_kernel<64, false>), dim3(grid), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t fa_launch_fp8_fwd(const FaFp8Params& p, int d, hipStream_t s) {
  if (d != 128) return hipErrorInvalidValue;
  if (p.total_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(fa_fp8_fwd_kernel<128>, dim3((unsigned)p.total_tiles), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}
