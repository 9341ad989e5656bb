// gfx950 (CDNA4) kernels for the fused exact-attention forward pass.
//
// Method ("Attention kernels: FlashAttention and PagedAttention", sections 3.1,
// 3.2 and 4.1): a workgroup owns a block of query rows, streams K_j / V_j
// tiles through LDS, forms S_ij = Q_i K_j^T with MFMA, applies scale, softcap
// and mask, updates the running row maximum m and row sum l with the
// exp(m_old - m_new) rescale of the unnormalised output, accumulates
// O += P~_ij V_j with MFMA, and writes O / l and the log-sum-exp once.  S and P
// live only in registers.  Exponentials are base 2 with log2(e) folded into the
// scale, and the division by l happens once at the end (same page, section 4.1).
//
// gfx950 mapping (our design, not the pages'):
//  * v_mfma_f32_32x32x16_bf16 in the transposed orientation S^T = K Q^T and
//    O^T = V^T P^T.  A lane then owns one query column: the 32x32 accumulator
//    puts column j = lane % 32 in lane j and j + 32, so a row maximum or sum is
//    an in-lane reduction plus one exchange with lane ^ 32, and the softmax
//    rescale of O^T is a per-lane scalar.  This is the wave64 counterpart of
//    the pages' "split-Q" rule that each warp owns whole rows (section 4.1).
//  * The S^T accumulator is re-packed in registers as the B operand of the
//    second product (the C-to-A fragment reuse of section 8.5, here C-to-B).
//    Each 16-key chunk of P^T takes accumulator slots {8h..8h+7}; the V^T
//    operand is then read with the same key order.
//  * K and V stages go from global memory straight into LDS with the gfx950
//    LDS-DMA load (global_load_lds_dwordx4: lane l of a wave writes the 16
//    bytes it fetched to LDS at base + 16 l), so no registers stage them.  Both
//    are stored row-major; the source chunk each lane fetches is permuted so
//    that the stored rows carry an XOR swizzle: K by 16-byte chunk (the 32 rows
//    a wave reads with ds_read_b128 per MFMA hit distinct banks), V by 64-byte
//    segment (the rows a transposed read touches hit distinct banks).
//  * The V^T operand comes from ds_read_b64_tr_b16: within each 16-lane group,
//    lane i receives element i % 4 of the 8-byte chunks addressed by lanes
//    i / 4 + 4 k (k = 0..3), so four lanes addressing four consecutive keys of
//    one 4-column span give every lane one column over those four keys.
//  * Workgroup = 4 waves, two workgroups per compute unit.  Prefill: the waves
//    split the 128 query rows (32 each) and share every 32-key stage of a
//    three-stage ring.  Paged decode: the waves share the (at most 32) packed
//    query rows and split each 64-key stage (16 keys each), merging their
//    partial states through LDS at the end.  Chunked prefill over a paged
//    cache is the prefill kernel with K/V addressed through the block table.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa_blockinfo.h"
#include "fa_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// Value of lanes l and l ^ 32 combined: v_permlane32_swap returns the lower half's
// values in one register and the upper half's in the other, for every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the stage pipeline.  __syncthreads() adds a memory fence
// that waits for every outstanding vector-memory operation, including the LDS-DMA
// loads of later blocks that are meant to stay in flight across this barrier.
// Here each wave has already waited (s_waitcnt vmcnt) for the DMA of the block
// the barrier publishes, and its LDS reads of the buffer about to be refilled
// have completed (their results were consumed), so a bare s_barrier suffices;
// the empty asm statements keep the compiler from moving memory operations
// across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ LDS layout
// A stage holds NK rows of K and NK rows of V, each row D bf16 (2D bytes),
// row-major.  Stored 16-byte chunk = logical chunk ^ swizzle(row).
template <int D>
__device__ __forceinline__ int k_swz(int r) {  // distinct chunk per row over 16 rows
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {  // rotates 64-byte segments over 4 rows
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Geometry of a stage load split over four waves: kInstPerWave 1 KiB pieces
// (kRowsPerKiB rows each) per wave and tensor.  In the prefill kernel piece p of
// wave w fills rows (4 p + w) * kRowsPerKiB .. + kRowsPerKiB - 1 of the stage;
// the decode kernel gives each wave its own consecutive rows instead.
template <int D, int NK>
struct DmaGeom {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTensorBytes = NK * kRowBytes;
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kInstPerWave = kTensorBytes / 1024 / 4;
  static constexpr int kRowStep = 4 * kRowsPerKiB;  // rows between instructions of a wave
  static_assert(kInstPerWave >= 1, "stage too small for four waves");
};

// Scalar load of one 32-bit value at a wave-uniform address.  A vector load
// would be waited for with vmcnt(0), which also waits for every LDS-DMA load
// in flight; this waits only for the scalar (and LDS) counter.  The address is
// taken from the first lane: callers pass addresses that are uniform by
// construction, which the compiler cannot always prove (e.g. a sequence index
// found by a ballot).
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int32_t* u = reinterpret_cast<const int32_t*>(((uint64_t)hi << 32) | lo);
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(u) : "memory");
  return v;
}

__device__ __forceinline__ void dma16(const uint16_t* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (FA_LDS void*)lds_dst, 16, 0, 0);
}

// The same LDS-DMA load through a buffer resource (buffer_load_dwordx4 ... lds):
// the base address lives in scalar registers and each lane adds a 32-bit byte
// offset, so a block's source address costs scalar instructions only instead
// of 64-bit vector address arithmetic per load.  Raw buffer (stride 0), 32-bit
// data format (the gfx9 resource word 3).
// The base must be the same in every lane (callers pass wave-uniform addresses);
// it is taken from the first lane, so that the resource lives in scalar registers
// even where the compiler cannot prove the address uniform (a varlen tile found
// by a ballot) and would otherwise wrap each load in a loop over distinct values.
constexpr int kBufRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, 0x7fffffff, kBufRsrcWord3);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds_dst, 16, (int)voff, (int)soff, 0, 0);
}

// ------------------------------------------------------------------ per-wave math
// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const FA_LDS char*)p);
}

// Per-lane LDS byte addresses of the MFMA operands within a stage buffer,
// fixed for the whole kernel.  Both swizzles only flip address bits below the
// row size, so the address of K chunk pair kk is k0 ^ (kk << 5) and that of V
// d-block db is v0 ^ (db << 6); two registers instead of one per operand.
template <int D>
struct LaneOffsets {
  uint32_t k0;  // K row (lane % 32), chunk kg (kk = 0)
  uint32_t v0;  // V transposed-read address for keys 4 kg + (j >> 2), d-block 0
  __device__ __forceinline__ void init(int lane, uint32_t base) { init(lane, base, base); }
  // krows: K rows per operand (32, or 16 with lanes 16..31 repeating rows 0..15)
  __device__ __forceinline__ void init(int lane, uint32_t kbase, uint32_t base, int krows = 32) {
    const int col = lane & (krows - 1), kg = lane >> 5;
    k0 = kbase + col * (2 * D) + ((kg ^ k_swz<D>(col)) << 4);
    const int j = lane & 15, half = (lane >> 4) & 1;
    const int row = 4 * kg + (j >> 2);
    const int c16 = 2 * half + ((j & 3) >> 1);
    v0 = base + row * (2 * D) + ((c16 ^ v_swz<D>(row)) << 4) + (j & 1) * 8;
  }
  __device__ __forceinline__ uint32_t k(int kk) const { return k0 ^ (uint32_t)(kk << 5); }
  __device__ __forceinline__ uint32_t v(int db) const { return v0 ^ (uint32_t)(db << 6); }
};

// LDS operand reads issued as inline assembly.  The compiler cannot tell that
// these reads and an in-flight LDS-DMA load into another stage buffer touch
// different bytes, and would otherwise wait for every outstanding DMA (vmcnt(0))
// before the reads.  The results are waited for explicitly with lgkmcnt(0),
// tied to the result registers.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// S^T for the 32 keys whose K rows start at byte OFF (plus delta) of the stage
// buffers, against the wave's 32 query columns.  Lane (j, kg) gets keys
// 8 (a / 4) + 4 kg + (a % 4) of the block.
template <int D, int OFF>
__device__ __forceinline__ f32x16 qk_block(uint32_t delta, const bf16x8* qreg, const LaneOffsets<D>& off) {
  u32x4 a[D / 16];  // all operand reads in flight before the first product
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) a[kk] = ds_read_b128<OFF>(off.k(kk) + delta);
  if constexpr (D == 128) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                   "+v"(a[7]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
  }
  f32x16 s = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) s = mfma32(__builtin_bit_cast(bf16x8, a[kk]), qreg[kk], s);
  return s;
}

// O^T += V^T P^T for the 16 keys whose V rows start at byte OFF (plus delta) of
// the stage buffers.  pb holds P^T for keys 8 (slot / 4) + 4 kg + (slot % 4) of
// those 16 and of this lane's column; two transposed reads per d-block give the
// V^T operand in the same key order.
template <int D, int OFF>
__device__ __forceinline__ void pv_chunk(uint32_t delta, bf16x8 pb, f32x16* o, const LaneOffsets<D>& off) {
  u32x2 lo[D / 32], hi[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    lo[db] = ds_read_tr16<OFF>(off.v(db) + delta);
    hi[db] = ds_read_tr16<OFF + 8 * (2 * D)>(off.v(db) + delta);
  }
  if constexpr (D == 128) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(lo[0]), "+v"(hi[0]), "+v"(lo[1]), "+v"(hi[1]), "+v"(lo[2]), "+v"(hi[2]),
                   "+v"(lo[3]), "+v"(hi[3]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(lo[0]), "+v"(hi[0]), "+v"(lo[1]), "+v"(hi[1]));
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    u32x4 w = {lo[db].x, lo[db].y, hi[db].x, hi[db].y};
    o[db] = mfma32(__builtin_bit_cast(bf16x8, w), pb, o[db]);
  }
}

// Split forms of qk_block / pv_chunk for the software-pipelined prefill step:
// the reads are issued early, and waited for with an LDS counter that lets the
// reads issued after them stay in flight (LDS reads complete in issue order).
template <int D, int OFF>
__device__ __forceinline__ void read_k(uint32_t delta, const LaneOffsets<D>& off, u32x4 (&a)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) a[kk] = ds_read_b128<OFF>(off.k(kk) + delta);
}
template <int D, int OFF, int K0, int NK>
__device__ __forceinline__ void read_k_part(uint32_t delta, const LaneOffsets<D>& off, u32x4 (&a)[D / 16]) {
#pragma unroll
  for (int kk = K0; kk < K0 + NK; ++kk) a[kk] = ds_read_b128<OFF>(off.k(kk) + delta);
}
template <int D, int OFF, int DB0, int NDB>
__device__ __forceinline__ void read_v_part(uint32_t delta, const LaneOffsets<D>& off, u32x2 (&lo)[NDB],
                                            u32x2 (&hi)[NDB]) {
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    lo[i] = ds_read_tr16<OFF>(off.v(DB0 + i) + delta);
    hi[i] = ds_read_tr16<OFF + 8 * (2 * D)>(off.v(DB0 + i) + delta);
  }
}
template <int D, int OFF>
__device__ __forceinline__ void read_v(uint32_t delta, const LaneOffsets<D>& off, u32x2 (&lo)[D / 32],
                                       u32x2 (&hi)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    lo[db] = ds_read_tr16<OFF>(off.v(db) + delta);
    hi[db] = ds_read_tr16<OFF + 8 * (2 * D)>(off.v(db) + delta);
  }
}
// Wait until at most N LDS operations are outstanding; the listed registers
// are treated as written by the wait, so no use of them moves above it.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4 (&a)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
               : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4 (&a)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x2 (&lo)[4], u32x2 (&hi)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(lo[0]), "+v"(hi[0]), "+v"(lo[1]), "+v"(hi[1]), "+v"(lo[2]), "+v"(hi[2]), "+v"(lo[3]),
                 "+v"(hi[3])
               : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x2 (&lo)[2], u32x2 (&hi)[2]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(lo[0]), "+v"(hi[0]), "+v"(lo[1]), "+v"(hi[1]) : "i"(N));
}
template <int D>
__device__ __forceinline__ f32x16 qk_mma(const u32x4 (&a)[D / 16], const bf16x8* qreg) {
  f32x16 s = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) s = mfma32(__builtin_bit_cast(bf16x8, a[kk]), qreg[kk], s);
  return s;
}

// O^T += V^T P^T product and exponential issued as inline assembly, so that
// the P V phase of the prefill pipeline keeps the order written: one product,
// then the exponentials that fill its 32 cycles.  The compiler does not see
// these as a matrix product, so the asm statement pads the hazard itself: two
// wait states after a VALU write of the operands (the A operand may be
// assembled by moves just before).  Readers of the accumulators wait for the
// last product explicitly (mfma_drain).
__device__ __forceinline__ void pv_mfma_asm(f32x16& acc, u32x4 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ float exp2_asm(float x) {
  float r;
  asm volatile("v_exp_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// Wait states for a VALU access to the accumulators of the last product issued
// by pv_mfma_asm (an 8-pass XDL op).  The accumulators are operands of the
// statement: the compiler does not know the products' latency and would
// otherwise be free to move the (pure arithmetic) accesses above the wait.
template <int N>
__device__ __forceinline__ void mfma_drain(f32x16 (&o)[N]) {
  static_assert(N == 2 || N == 4, "two or four accumulators");
  if constexpr (N == 4) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
  } else {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(o[0]), "+v"(o[1]));
  }
}

// Softcap transform into the log2 domain: c * tanh(scale * s / c) * log2(e),
// tanh(y) = 1 - 2 / (exp(2y) + 1).
__device__ __forceinline__ float softcap_log2(float s, float cap_in, float cap_out) {
  // c tanh(y) log2(e) = c log2(e) - 2 c log2(e) / (exp(2y) + 1), y = scale s / c
  const float t = exp2_fast(s * (cap_in * (2.0f * kLog2e)));
  return __builtin_fmaf(-2.0f * cap_out, rcp_fast(t + 1.0f), cap_out);
}

// Per-lane view of the mask: this lane's query position and the bounds.
struct LaneMask {
  int pos;      // key-axis position of this lane's query row
  int kend;     // keys >= kend are invisible (sequence / split end)
  int kbeg;     // keys < kbeg are invisible (split start)
  int causal, wl, wr;
  __device__ __forceinline__ bool visible(int key) const {  // branch-free
    return (key < kend) & (key >= kbeg) & (!causal | (key <= pos)) & ((wl < 0) | (key >= pos - wl)) &
           ((wr < 0) | (key <= pos + wr));
  }
  // The same predicate for the keys base + off of a 32-key block, off in
  // [0, 32): visible iff lo <= off <= hi.  lo is 0 unless kbeg or a left window
  // cuts the block; the window ends are formed in 64 bits (pos + wr, pos - wl
  // may leave the int range).
  __device__ __forceinline__ int off_hi(int base) const {
    int64_t h = (int64_t)kend - 1 - base;
    if (causal) h = min(h, (int64_t)pos - base);
    if (wr >= 0) h = min(h, (int64_t)pos + wr - base);
    return (int)max(h, (int64_t)-1);
  }
  __device__ __forceinline__ int off_lo(int base) const {
    int64_t l = (int64_t)kbeg - base;
    if (wl >= 0) l = max(l, (int64_t)pos - wl - base);
    return (int)min(max(l, (int64_t)0), (int64_t)32);
  }
};

// Online softmax over one 32-key block held in s.  Scores are in units where
// p = exp2(s * c - m * c): raw scores with c = scale * log2(e), or softcapped
// log2-domain scores with c = 1 (a positive c keeps the maximum where it is).
// Two partial row sums are kept for this lane: l_run of the fp32 probabilities
// (for the log-sum-exp) and l_bf of the bf16-rounded probabilities that enter
// the P V product (for the division of O, so the weights of O sum to one
// exactly).  Masked entries are -inf.
//
// The reference moves only when the running maximum exceeds it by more than
// 2^kRescaleLog2 (or on the first visible key): exponents stay below that bound,
// and since O and l are both relative to the same reference the result is the
// same up to rounding, while the rescale of O (a multiply per accumulator) and
// its exponential are skipped on most blocks.  The decision is wave-uniform.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kRescaleMax = 256.0f;  // 2^kRescaleLog2

// Online softmax of one block of the decode kernel (S^T accumulator s, raw
// scores; c turns them into log2 units).  M is the row's reference in log2
// units (-inf while the row has seen no visible key).  The exponent arguments
// are formed against the current reference first (multiply-adds, whose results
// the block maximum then takes without canonicalising each score); the
// reference moves, rescaling O and the sums, only when the block's maximum
// exceeds it by more than kRescaleLog2 ("Attention kernels...", section 7.3: a
// row with no visible key yet uses 0 as the offset, so exp2(-inf - 0) = 0).
template <int D>
__device__ __forceinline__ void online_softmax(const f32x16& s, float& M, float& l_run, float& l_bf,
                                               f32x16* o, float c, bf16x8& p0, bf16x8& p1) {
  const float nm = (M == kNegInf) ? 0.0f : -M;
  f32x16 y;
#pragma unroll
  for (int a = 0; a < 16; ++a) y[a] = __builtin_fmaf(s[a], c, nm);
  float ym = fmaxf(fmaxf(y[0], y[1]), y[2]);
#pragma unroll
  for (int a = 3; a < 15; a += 2) ym = fmaxf(fmaxf(ym, y[a]), y[a + 1]);
  ym = fmaxf(ym, y[15]);
  ym = pair_max(ym);
  const bool mv = (M == kNegInf) ? (ym != kNegInf) : (ym > kRescaleLog2);
  if (__any(mv)) {
    const float m_new = mv ? ym - nm : M;
    const float alpha = mv ? exp2_fast(M - m_new) : 1.0f;
    l_run *= alpha;
    l_bf *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    M = m_new;
    const float nn = (M == kNegInf) ? 0.0f : -M;
#pragma unroll
    for (int a = 0; a < 16; ++a) y[a] = __builtin_fmaf(s[a], c, nn);
  }
  float rs = 0.0f;
  f32x8 x0, x1;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    x0[a] = exp2_fast(y[a]);
    x1[a] = exp2_fast(y[a + 8]);
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) rs += x0[a] + x1[a];
  l_run += rs;
  p0 = __builtin_convertvector(x0, bf16x8);
  p1 = __builtin_convertvector(x1, bf16x8);
  // the same weights the P V product uses: sum of the bf16-rounded probabilities
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    l_bf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[2 * a], p0[2 * a + 1]}, one, l_bf, false);
    l_bf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[2 * a], p1[2 * a + 1]}, one, l_bf, false);
  }
}

// The same online softmax split into the parts the prefill pipeline places in
// different regions of its loop body (see the prefill kernel).

// Block maximum of s over this lane pair.
__device__ __forceinline__ float block_max(const f32x16& s) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int a = 3; a < 15; a += 2) mx = fmaxf(fmaxf(mx, s[a]), s[a + 1]);
  mx = fmaxf(mx, s[15]);
  return pair_max(mx);
}

// The softmax of a block split in two for the prefill pipeline: the
// exponentials (relative to the reference) run beside the P V products of the
// previous block, their sums and the bf16 MFMA operands beside the S products
// of the next block.
//
// Reference decision for a block with maximum mx: returns true when the
// reference moves (to max(m_run, mx)); then alpha rescales what was
// accumulated relative to the old reference.  m_run is updated here, the
// rescale itself is applied by the caller once the P V products in flight are
// done.
__device__ __forceinline__ bool move_reference(float mx, float& m_run, float c, float& alpha) {
  const float m_cand = fmaxf(m_run, mx);
  alpha = 1.0f;
  if (__any((m_cand - m_run) * c > kRescaleLog2)) {
    // a row that has seen no visible key keeps m = -inf; use 0 as the offset so
    // that exp2(-inf - offset) = 0 instead of NaN ("Attention kernels...", section 7.3)
    const float m_use = (m_cand == kNegInf) ? 0.0f : m_cand;
    alpha = exp2_fast((m_run - m_use) * c);
    m_run = m_cand;
    return true;
  }
  return false;
}
// -m c for the exponentials (0 while the row has seen no visible key).
__device__ __forceinline__ float neg_ref(float m_run, float c) { return (m_run == kNegInf) ? 0.0f : -m_run * c; }
// Sums of the exponentials x into both row sums, and x as two bf16 operands.
__device__ __forceinline__ float lane_sum16(const f32x16& x) {
  const float r0 = (x[0] + x[1]) + (x[2] + x[3]);
  const float r1 = (x[4] + x[5]) + (x[6] + x[7]);
  const float r2 = (x[8] + x[9]) + (x[10] + x[11]);
  const float r3 = (x[12] + x[13]) + (x[14] + x[15]);
  return (r0 + r1) + (r2 + r3);
}
// rs: lane_sum16(x), formed by the caller.
__device__ __forceinline__ void block_sums(const f32x16& x, float rs, float& l_run, float& l_bf, bf16x8& p0,
                                           bf16x8& p1) {
  l_run += rs;
  f32x8 x0, x1;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    x0[a] = x[a];
    x1[a] = x[a + 8];
  }
  p0 = __builtin_convertvector(x0, bf16x8);
  p1 = __builtin_convertvector(x1, bf16x8);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    l_bf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[2 * a], p0[2 * a + 1]}, one, l_bf, false);
    l_bf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[2 * a], p1[2 * a + 1]}, one, l_bf, false);
  }
}

// ------------------------------------------------------------------ tile scheduling
// Linear tile index -> tile, longest first (row blocks nearer the end of a
// sequence see more keys under a causal mask, so they go first); one workgroup
// per tile index, so the hardware hands out the next tile as a workgroup ends.

struct TileId {
  int b, hg, mb;
};

// Row blocks of a varlen sequence with L new tokens: ceil(L gp / BLOCK_M), or
// none when its L g packed rows go to the decode kernel (p.skip_rows).
__device__ __forceinline__ int varlen_mblocks(const FaParams& p, int L) {
  if (p.skip_rows > 0 && L * p.g <= p.skip_rows) return 0;
  return (L * p.gp + FA_BLOCK_M - 1) / FA_BLOCK_M;
}
// Keys before a varlen sequence's first query (its cache or key length minus
// its new tokens), in row-block units: row block m of sequence b sees about
// (P_b + m + 1) blocks' worth of keys under a causal mask.
__device__ __forceinline__ int varlen_prefix_blocks(const FaParams& p, int b, int L) {
  const int Lk = p.cache_seqlens ? p.cache_seqlens[b] : p.cu_k[b + 1] - p.cu_k[b];
  const int pre = Lk - L;
  return pre > 0 ? (int)(((int64_t)pre * p.gp) / FA_BLOCK_M) : 0;
}

// Row blocks M_b and prefix blocks P_b of sequence b (both 0 past the batch).
__device__ __forceinline__ void varlen_seq(const FaParams& p, int b, int& M, int& P) {
  M = 0;
  P = 0;
  if (b < p.B) {
    const int L = p.cu_q[b + 1] - p.cu_q[b];
    M = varlen_mblocks(p, L);
    P = M > 0 ? varlen_prefix_blocks(p, b, L) : 0;
  }
}

// (M, P) of the first kVarlenRegChunks * 64 sequences, read once per tile: lane
// l holds sequences l, l + 64, ...  The binary search over levels then runs on
// registers, and reads memory only for the sequences of larger batches (each
// read is a round trip to the cache, about a microsecond per search step).
constexpr int kVarlenRegChunks = 4;
struct VarlenSeqs {
  int M[kVarlenRegChunks], P[kVarlenRegChunks];
};
__device__ __forceinline__ void varlen_seqs_load(const FaParams& p, int lane, VarlenSeqs& vs) {
#pragma unroll
  for (int j = 0; j < kVarlenRegChunks; ++j) varlen_seq(p, 64 * j + lane, vs.M[j], vs.P[j]);
}

// Varlen tiles are listed by level v = P_b + m, highest first (longest first).
// Number of tiles at levels above v, summed over sequences:
// C(v) = sum_b clamp(M_b + P_b - v - 1, 0, M_b).  With vmax set, also the
// number of levels, max_b (P_b + M_b).
__device__ int64_t varlen_tiles_above(const FaParams& p, const VarlenSeqs& vs, int v, int lane,
                                      int* vmax = nullptr) {
  int64_t acc = 0;
  int top = 0;
  auto add = [&](int M, int P) {
    int c = M + P - v - 1;
    c = c < 0 ? 0 : (c > M ? M : c);
    if (M > 0) top = max(top, P + M);
    acc += wave_sum(c);
  };
#pragma unroll
  for (int j = 0; j < kVarlenRegChunks; ++j)
    if (64 * j < p.B) add(vs.M[j], vs.P[j]);
  for (int b0 = 64 * kVarlenRegChunks; b0 < p.B; b0 += 64) {
    int M, P;
    varlen_seq(p, b0 + lane, M, P);
    add(M, P);
  }
  if (vmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) top = max(top, __shfl_xor(top, off));
    *vmax = top;
  }
  return acc;
}

// Varlen tile t.  Returns false when t is past the last tile.
__device__ bool varlen_tile(const FaParams& p, int64_t t, int lane, TileId* out) {
  const int H = p.hg_count;
  VarlenSeqs vs;
  varlen_seqs_load(p, lane, vs);
  int vmax = 0;
  int64_t total = (int64_t)H * varlen_tiles_above(p, vs, -1, lane, &vmax);
  if (t >= total) return false;
  int lo = 0, hi = vmax - 1;
  while (lo < hi) {  // smallest v with H * C(v) <= t
    int mid = (lo + hi) >> 1;
    if ((int64_t)H * varlen_tiles_above(p, vs, mid, lane) <= t)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int v = lo;
  int64_t j = t - (int64_t)H * varlen_tiles_above(p, vs, v, lane);
  int idx = (int)(j / H);
  out->hg = (int)(j % H);
  out->b = -1;
  // the idx-th sequence (in batch order) with a tile at level v
  auto pick = [&](int b0, int M, int P) -> bool {
    const int m = M > 0 ? v - P : -1;
    const bool f = m >= 0 && m < M;
    const uint64_t mask = __ballot(f);
    const int cnt = __popcll(mask);
    if (idx < cnt) {
      const uint64_t below = (lane == 0) ? 0ull : (mask & (~0ull >> (64 - lane)));
      const bool mine = f && __popcll(below) == idx;
      const uint64_t sel = __ballot(mine);
      const int src = __ffsll((long long)sel) - 1;
      // wave-uniform by construction; made scalar so that everything derived
      // from the tile (bounds, loop counts, addresses) stays in scalar registers
      out->b = __builtin_amdgcn_readfirstlane(b0 + src);
      out->mb = __builtin_amdgcn_readfirstlane(__shfl(m, src));
      return true;
    }
    idx -= cnt;
    return false;
  };
#pragma unroll
  for (int jj = 0; jj < kVarlenRegChunks; ++jj)
    if (64 * jj < p.B && out->b < 0) pick(64 * jj, vs.M[jj], vs.P[jj]);
  for (int b0 = 64 * kVarlenRegChunks; b0 < p.B && out->b < 0; b0 += 64) {
    int M, P;
    varlen_seq(p, b0 + lane, M, P);
    pick(b0, M, P);
  }
  return out->b >= 0;
}

// Dense tiles.  Without a left window, row blocks go longest first, level by
// level over all (sequence, head group) pairs.  With a left window every row
// block has about the same work, and the tiles running together should share
// K/V: workgroup i runs on XCD i % 8, so XCD x takes the pairs x, x + 8, ...
// one after the other, row blocks in order, and its concurrent tiles cover one
// pair's neighbouring windows in that XCD's L2.
__device__ __forceinline__ bool dense_tile(const FaParams& p, int64_t t64, TileId* out) {
  if (t64 >= p.total_tiles) return false;
  // tile counts stay below 2^31 (the host checks), so 32-bit index arithmetic
  const uint32_t t = (uint32_t)t64;
  const uint32_t hgc = (uint32_t)p.hg_count;
  const uint32_t pairs = (uint32_t)p.B * hgc;
  uint32_t bh;
  if (p.wl >= 0 && (pairs & 7) == 0) {
    const uint32_t j = t >> 3, mbs = (uint32_t)p.m_blocks;
    const uint32_t q = j / mbs;
    out->mb = (int)(j - q * mbs);
    bh = q * 8 + (t & 7);
  } else {
    const uint32_t q = t / pairs;
    out->mb = p.m_blocks - 1 - (int)q;
    bh = t - q * pairs;
  }
  const uint32_t b = bh / hgc;
  out->b = (int)b;
  out->hg = (int)(bh - b * hgc);
  return true;
}

// s_waitcnt vmcnt(n * PER) for a wave-uniform n in [0, 5].
template <int PER>
__device__ __forceinline__ void wait_vmcnt_blocks(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER>(); break;
    case 2: wait_vmcnt<2 * PER>(); break;
    case 3: wait_vmcnt<3 * PER>(); break;
    case 4: wait_vmcnt<4 * PER>(); break;
    default: wait_vmcnt<5 * PER>(); break;
  }
}

// ------------------------------------------------------------------ prefill kernel
// Key blocks of 32 stream through a ring of NBUF = 3 LDS stage buffers, the
// DMA of a block issued two iterations before its use.  Iteration i (one
// barrier) issues the DMA of block i + 2, forms the row sums and bf16 operands
// of block i, S^T of block i + 1, and accumulates O^T += V^T P^T of block i
// beside the exponentials of block i + 1, so the matrix products of one block
// and the softmax of the next are independent work within the wave.
//
// PAGED: K and V come from a paged cache ("Attention kernels...", section 6.1):
// key t of sequence b is slot t % page of page block_table[b][t / page], and
// the sequence has cache_seqlens[b] keys.  The rows of one LDS-DMA instruction
// are 1024 / (2 D) consecutive keys starting at a multiple of that count, so
// with page sizes that are multiples of 16 they lie in one page: one scalar
// block-table read per instruction.  VARLEN with PAGED is the unified batch:
// packed queries by cu_seqlens_q, each sequence with its own cache length.
// ALIBI: the logits get the linear positional bias -slope_h |p - key| ("FA4
// (CuTeDSL) and engineering interfaces", section 7), p the query's bottom-right
// position: with the element mask on blocks a boundary cuts, alone on the others.
// MOD: a score_mod / mask_mod (fa_mods.h) applied to every score of every key
// block in range, before the built-in element mask ("FA4 (CuTeDSL) and
// engineering interfaces", sections 1 and 7: the hooks sit between Q K^T and the
// softmax); with a score_mod the scores enter the softmax in log2 units, as with
// softcap.
constexpr int kPrefillStages = 3;  // measured best of 3, 4 and 5 stages
template <int D>
constexpr int prefill_smem_bytes() {
  return 2 * kPrefillStages * DmaGeom<D, FA_BLOCK_N>::kTensorBytes;
}

// The prefill work of one workgroup: tile bid, with its K/V stages in smem
// (prefill_smem_bytes<D>(), 1 KiB aligned).  The kernel below and the unified
// prefill + decode kernel call it.
template <int D, bool VARLEN, bool PACK, bool SOFTCAP, bool PAGED, bool ALIBI = false, class MOD = FaNoMod>
__device__ __forceinline__ void prefill_body(const FaParams& p, char* smem, int bid) {
  constexpr bool kMod = MOD::kScore || MOD::kMask;
  static_assert(!(kMod && (SOFTCAP || ALIBI)), "a mod replaces softcap and ALiBi");
  constexpr int BN = FA_BLOCK_N;  // 32 keys per block
  constexpr int NBUF = kPrefillStages;
  using G = DmaGeom<D, BN>;
  constexpr int T = G::kTensorBytes;  // one tensor of one block
  static_assert(NBUF * T <= 65536, "stage offsets must fit the LDS immediate offset");
  // K stages in the lower half, V stages in the upper half

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int kg = lane >> 5;
  const float c = (SOFTCAP || MOD::kScore) ? 1.0f : p.scale_log2;

  LaneOffsets<D> off;
  off.init(lane, lds_addr(smem), lds_addr(smem) + NBUF * T);
  // DMA geometry of this lane: stage row and the source chunk for K and V
  const int dma_row = wave * G::kRowsPerKiB + lane / G::kChunksPerRow;
  const int dma_pc = lane % G::kChunksPerRow;
  const int k_src = (dma_pc ^ k_swz<D>(dma_row)) * 8;
  const int v_src = (dma_pc ^ v_swz<D>(dma_row)) * 8;

  {
    const int64_t t = bid;
    TileId tile;
    if (VARLEN) {
      if (!varlen_tile(p, t, lane, &tile)) return;
    } else {
      if (!dense_tile(p, t, &tile)) return;
    }

    // ---- sequence view
    int64_t q_start = 0, k_start = 0;
    int Lq = p.Nq, Lk = p.Nk;
    if (VARLEN) {
      q_start = scalar_load_i32(p.cu_q + tile.b);
      Lq = scalar_load_i32(p.cu_q + tile.b + 1) - (int)q_start;
      if (!PAGED) {
        k_start = scalar_load_i32(p.cu_k + tile.b);
        Lk = scalar_load_i32(p.cu_k + tile.b + 1) - (int)k_start;
      }
    }
    if (PAGED) Lk = scalar_load_i32(p.cache_seqlens + tile.b);
    const int kvh = PACK ? tile.hg : tile.hg / p.g;
    const int rows = Lq * p.gp;
    const int m0 = tile.mb * FA_BLOCK_M;
    const int m_end = min(m0 + FA_BLOCK_M, rows);
    FaRowSpan span;
    span.pos_lo = (int64_t)(m0 / p.gp) + (Lk - Lq);
    span.pos_hi = (int64_t)((m_end - 1) / p.gp) + (Lk - Lq);
    int n_lo, n_hi;
    fa_key_tiles(span, Lk, p.causal, p.wl, p.wr, BN, &n_lo, &n_hi);
    // the mod's per-tile state, and the key blocks its mask leaves in range
    const typename MOD::Tile mod_tile = MOD{}.tile(tile.b, p.mod);
    if constexpr (MOD::kBlocks) {
      const int k_end = MOD{}.key_end((int)span.pos_lo, (int)span.pos_hi, mod_tile);
      n_hi = max(n_lo, min(n_hi, (int)(((int64_t)k_end + BN - 1) / BN)));
    }
    // key blocks [n_full_lo, n_full_hi) need no element mask: the closed-form
    // range of tiles the classifier calls full (one interval, checked against the
    // classifier on the host), within [n_lo, n_hi)
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

    // ---- this lane's query row
    const int row = m0 + wave * 32 + col;
    const bool row_ok = row < rows;
    const int tok = row_ok ? (PACK ? row / p.g : row) : 0;
    const int head = PACK ? kvh * p.g + (row_ok ? row % p.g : 0) : tile.hg;
    const uint16_t* qb = p.q + (int64_t)tile.b * p.q_bs + (q_start + tok) * p.q_ss + (int64_t)head * p.q_hs;
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_ok) x = *reinterpret_cast<const u32x4*>(qb + 16 * kk + 8 * kg);
      qreg[kk] = __builtin_bit_cast(bf16x8, x);
    }
    LaneMask mask;
    mask.pos = tok + (Lk - Lq);
    mask.kend = Lk;
    mask.kbeg = 0;
    mask.causal = p.causal;
    mask.wl = p.wl;
    mask.wr = p.wr;
    // ALiBi slope of this lane's head in raw-score units (the scores are scaled later)
    float alibi_k = 0.0f;
    if constexpr (ALIBI) alibi_k = p.alibi[(int64_t)tile.b * p.alibi_bs + head] * p.alibi_inv_scale;

    // DMA sources: this lane's row of every block.  Rows past the last key (only
    // in a final partial block) are clamped to the last key so that they read
    // real (finite) data, which the mask then drops.
    const uint16_t* kbase = p.k + (int64_t)tile.b * p.k_bs + k_start * p.k_ss + (int64_t)kvh * p.k_hs;
    const uint16_t* vbase = p.v + (int64_t)tile.b * p.v_bs + k_start * p.v_ss + (int64_t)kvh * p.v_hs;
    // byte offsets of this lane's row and chunk within a block, and between the
    // instructions of a wave (the host keeps 32 * stride * 2 below 2^31)
    const uint32_t k_voff = (uint32_t)(dma_row * p.k_ss + k_src) * 2u;
    const uint32_t v_voff = (uint32_t)(dma_row * p.v_ss + v_src) * 2u;
    const uint32_t k_step = (uint32_t)(G::kRowStep * p.k_ss) * 2u, v_step = (uint32_t)(G::kRowStep * p.v_ss) * 2u;
    // paged: the lane's row within its instruction's kRowsPerKiB rows, and chunk
    const uint32_t kp_voff = (uint32_t)((lane / G::kChunksPerRow) * p.k_ss + k_src) * 2u;
    const uint32_t vp_voff = (uint32_t)((lane / G::kChunksPerRow) * p.v_ss + v_src) * 2u;
    // block i of this tile (key block n_lo + i) goes to buffer i % NBUF
    auto issue = [&](int i) {
      char* dst = smem + (i % NBUF) * T + wave * 1024;
      const int n0 = (n_lo + i) * BN;
      if constexpr (PAGED) {
        // Keys past the last one are clamped to it; a clamped instruction's rows
        // then all lie in the last key's page.
        const int32_t* bt = p.block_table + (int64_t)tile.b * p.max_blocks;
        if (n0 + BN <= Lk) {
          // a full block: the instruction's rows are consecutive keys of one page,
          // addressed from the page's row (scalar) plus the lane's row offset
#pragma unroll
          for (int j = 0; j < G::kInstPerWave; ++j) {
            const int first = n0 + wave * G::kRowsPerKiB + j * G::kRowStep;
            const int pg = first / p.page;
            const int64_t phys = scalar_load_i32(bt + pg);
            const int slot0 = first - pg * p.page;
            dma16_buf(buf_rsrc(p.k + phys * p.k_bs + (int64_t)slot0 * p.k_ss + (int64_t)kvh * p.k_hs), kp_voff, 0u,
                      dst + j * 4096);
            dma16_buf(buf_rsrc(p.v + phys * p.v_bs + (int64_t)slot0 * p.v_ss + (int64_t)kvh * p.v_hs), vp_voff, 0u,
                      dst + NBUF * T + j * 4096);
          }
          return;
        }
#pragma unroll
        for (int j = 0; j < G::kInstPerWave; ++j) {
          const int first = n0 + wave * G::kRowsPerKiB + j * G::kRowStep;  // first row of the instruction
          const int pg = min(first, Lk - 1) / p.page;
          const int64_t phys = scalar_load_i32(bt + pg);
          const int slot = min(n0 + dma_row + j * G::kRowStep, Lk - 1) - pg * p.page;
          dma16(p.k + phys * p.k_bs + (int64_t)slot * p.k_ss + (int64_t)kvh * p.k_hs + k_src, dst + j * 4096);
          dma16(p.v + phys * p.v_bs + (int64_t)slot * p.v_ss + (int64_t)kvh * p.v_hs + v_src,
                dst + NBUF * T + j * 4096);
        }
      } else if (n0 + BN <= Lk) {
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kbase + (int64_t)n0 * p.k_ss);
        const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vbase + (int64_t)n0 * p.v_ss);
#pragma unroll
        for (int j = 0; j < G::kInstPerWave; ++j) {
          dma16_buf(rk, k_voff, j * k_step, dst + j * 4096);
          dma16_buf(rv, v_voff, j * v_step, dst + NBUF * T + j * 4096);
        }
      } else {
#pragma unroll
        for (int j = 0; j < G::kInstPerWave; ++j) {
          int key = n0 + dma_row + j * G::kRowStep;
          key = key < Lk ? key : Lk - 1;
          dma16(kbase + (int64_t)key * p.k_ss + k_src, dst + j * 4096);
          dma16(vbase + (int64_t)key * p.v_ss + v_src, dst + NBUF * T + j * 4096);
        }
      }
    };
    constexpr int kDmaPerBlock = 2 * G::kInstPerWave;  // this wave's DMA instructions per block

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f, l_bf = 0.0f;

    // Element mask of block i (key block n_lo + i), applied in place.
    auto apply_mask = [&](f32x16& sv, int i) {
      int base = (n_lo + i) * BN + 4 * kg;
      // keep the per-element key offsets inside this (rarely taken) path rather
      // than as sixteen loop-invariant registers
      asm volatile("" : "+v"(base));
      // This row's visible keys in the block form one interval of offsets
      // [lo, hi] from base (the prefill's rows see keys from 0, so kbeg = 0);
      // the offsets of the sixteen scores are compile-time constants.  Without
      // a window the lower end is offset 0 and one compare per score decides
      // (measured 1-2.5 % faster on the 4x16x4096 causal workload than the
      // general predicate); with a window, two.
      auto bias = [&](float x, int off) {
        if constexpr (ALIBI) x = __builtin_fmaf(-alibi_k, (float)abs(mask.pos - (base + off)), x);
        return x;
      };
      if (mask.wl < 0 && mask.wr < 0) {
        const int hi = min(mask.causal ? mask.pos - base : 0x3fffffff, mask.kend - 1 - base);
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int off = 8 * (a >> 2) + (a & 3);
          sv[a] = off <= hi ? bias(sv[a], off) : kNegInf;
        }
      } else {
        const int hi = mask.off_hi(base), lo = mask.off_lo(base);
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int off = 8 * (a >> 2) + (a & 3);
          sv[a] = (off <= hi && off >= lo) ? bias(sv[a], off) : kNegInf;
        }
      }
    };
    auto transform = [&](f32x16& sv) {
      if constexpr (SOFTCAP) {
#pragma unroll
        for (int a = 0; a < 16; ++a) sv[a] = softcap_log2(sv[a], p.cap_in, p.cap_out);
      }
    };
    auto is_masked = [&](int i) { return n_lo + i < n_full_lo || n_lo + i >= n_full_hi; };
    // The mod on block i: the rewritten logit in log2 units, and its mask
    auto apply_mod = [&](f32x16& sv, int i) {
      if constexpr (kMod) {
        const MOD mod{};
        const int base = (n_lo + i) * BN + 4 * kg;
        // the mask only on blocks the mod cannot vouch for as visible whole
        bool masks = MOD::kMask;
        if constexpr (MOD::kMask && MOD::kBlocks)
          masks = !mod.block_visible((int)span.pos_lo, (int)span.pos_hi, (n_lo + i) * BN, (n_lo + i) * BN + BN - 1,
                                     mod_tile);
        if constexpr (MOD::kScore) {
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int key = base + 8 * (a >> 2) + (a & 3);
            sv[a] = mod.score(sv[a] * p.scale, tile.b, head, mask.pos, key, mod_tile, p.mod) * kLog2e;
          }
        }
        if constexpr (MOD::kMask && MOD::kBlocks) {
          // The path that skips the mask loop joins the one that runs it, and
          // the compiler's hazard search (one visit per block) then misses the
          // S product on the shorter path: wait for the product before the
          // branch.
          asm volatile("s_nop 7\n\ts_nop 3" : "+v"(sv));
        }
        if (MOD::kMask && masks) {
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int key = base + 8 * (a >> 2) + (a & 3);
            sv[a] = mod.mask(tile.b, head, mask.pos, key, mod_tile, p.mod) ? sv[a] : kNegInf;
          }
        }
      }
    };
    // ALiBi on a block no boundary cuts: the bias alone, -k |key - pos| with
    // key - pos = fb + (a compile-time offset per slot), exact in fp32
    auto apply_bias = [&](f32x16& sv, int i) {
      if constexpr (ALIBI) {
        const float fb = (float)((n_lo + i) * BN + 4 * kg - mask.pos);
#pragma unroll
        for (int a = 0; a < 16; ++a)
          sv[a] = __builtin_fmaf(-alibi_k, fabsf(fb + (float)(8 * (a >> 2) + (a & 3))), sv[a]);
      }
    };

    // xs: exponentials of the current block relative to m_run, whose sums and
    // bf16 operands are formed at the start of the next step
    f32x16 xs = {};
    // sc: the prepared scores of the block whose exponentials xs holds, kept for
    // the check below.  Exponentials that outgrew the reference (some above 2^8)
    // are caught where they are summed: a per-lane sum above 2^8 (or not finite)
    // sends the wave to the reference decision on the block's maximum, which
    // moves the reference, rescales what was accumulated and redoes the
    // exponentials.  The per-lane sums of a block stay far below 2^8 when the
    // reference is current, so the branch is rarely taken.
    // With softcap sc holds r = 1 / (exp(2 y) + 1) instead (+inf for a hidden
    // key), from which the capped logit is cap_out - 2 cap_out r and the
    // exponential exp2(logit - m) one multiply-add.
    f32x16 sc = {};
    const float cap_k = p.cap_in * (2.0f * kLog2e), cap_m2 = -2.0f * p.cap_out;
    auto softcap_r = [&](float x) { return rcp_fast(exp2_fast(x * cap_k) + 1.0f); };
    // -m c of the current reference (0 while a row has seen no visible key),
    // recomputed only where the reference moves; all_ref: every row of the wave
    // has a reference (once true it stays true: a reference only moves up)
    float nmc_run = 0.0f;
    bool all_ref = false;
    auto check_sums = [&]() -> float {
      float rs = lane_sum16(xs);
      if (__any(!(rs <= kRescaleMax))) {
        float a2;
        f32x16 lg = sc;
        if constexpr (SOFTCAP) {
#pragma unroll
          for (int a = 0; a < 16; ++a) lg[a] = __builtin_fmaf(cap_m2, sc[a], p.cap_out);
        }
        if (move_reference(block_max(lg), m_run, c, a2)) {
          mfma_drain(o);
          l_run *= a2;
          l_bf *= a2;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) o[db] *= a2;
          nmc_run = neg_ref(m_run, c);
          if constexpr (SOFTCAP) {
#pragma unroll
            for (int a = 0; a < 16; ++a) xs[a] = exp2_fast(__builtin_fmaf(cap_m2, sc[a], p.cap_out + nmc_run));
          } else {
#pragma unroll
            for (int a = 0; a < 16; ++a) xs[a] = exp2_fast(__builtin_fmaf(sc[a], c, nmc_run));
          }
          rs = lane_sum16(xs);
        }
      }
      return rs;
    };
    auto exps = [&](const f32x16& sv, float nmc, int a0, int a1) {
#pragma unroll
      for (int a = a0; a < a1; ++a) xs[a] = exp2_fast(__builtin_fmaf(sv[a], c, nmc));
    };
    if (nb > 0) {
      for (int j = 0; j < NBUF - 1 && j < nb; ++j) issue(j);
      // block 0 landed: the DMAs of the blocks after it may still be in flight
      wait_vmcnt_blocks<kDmaPerBlock>(min(NBUF - 2, nb - 1));
      stage_barrier();
      f32x16 s0 = qk_block<D, 0>(0u, qreg, off);
      f32x16 r0 = {};
      if constexpr (SOFTCAP) {
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          r0[a] = softcap_r(s0[a]);
          s0[a] = __builtin_fmaf(cap_m2, r0[a], p.cap_out);
        }
      }
      apply_mod(s0, 0);
      if (is_masked(0))
        apply_mask(s0, 0);
      else
        apply_bias(s0, 0);
      float alpha;
      move_reference(block_max(s0), m_run, c, alpha);  // nothing accumulated yet
      nmc_run = neg_ref(m_run, c);
      all_ref = !__any(m_run == kNegInf);
      exps(s0, nmc_run, 0, 16);
      if constexpr (SOFTCAP) {
#pragma unroll
        for (int a = 0; a < 16; ++a) sc[a] = s0[a] == kNegInf ? __builtin_inff() : r0[a];
      } else {
        sc = s0;
      }
    }

    // Pipeline step for block i (stage B = i % NBUF) when block i + 1 exists.
    // The sums and bf16 operands of block i cover the latency of the K reads of
    // block i + 1; then S^T of block i + 1 (MFMA); its mask, maximum and
    // reference decision; then O^T += V^T P^T of block i, one MFMA at a time
    // beside two exponentials of block i + 1 (the fences keep that order).  A
    // move of the reference rescales O and the sums after the products.
    auto step = [&](auto bufc, int i) {
      constexpr int B = decltype(bufc)::value;
      constexpr int BN1 = (B + 1) % NBUF;
      constexpr int kV = B * T;  // V stage of block i
      // block i + 1 landed (later blocks may still be in flight); everyone is done
      // with block i - 1, whose stages the DMA of block i + NBUF - 1 reuses
      wait_vmcnt_blocks<kDmaPerBlock>(min(i + NBUF - 2, nb - 1) - (i + 1));
      stage_barrier();
      if (i + NBUF - 1 < nb) issue(i + NBUF - 1);
      u32x4 ka[D / 16];
      read_k<D, BN1 * T>(0u, off, ka);
      // the sums of block i run while the K reads are in flight: the empty asm
      // statements (ordered with the reads and waits) pin them there
      asm volatile("" : "+v"(xs));
      const float rs = check_sums();
      bf16x8 p0, p1;
      block_sums(xs, rs, l_run, l_bf, p0, p1);
      asm volatile("" : "+v"(p0), "+v"(p1), "+v"(l_run), "+v"(l_bf));
      u32x2 lo0[D / 32], hi0[D / 32], lo1[D / 32], hi1[D / 32];
      read_v<D, kV>(0u, off, lo0, hi0);
      lgkm_wait<2 * (D / 32)>(ka);  // only the V reads just issued may be outstanding
      // a raised issue priority from the S^T products to the end of the P V
      // phase: measured 1.7-2.5 % faster on the 4x16x4096 causal workload and
      // neutral on the 32k window + softcap one
      __builtin_amdgcn_s_setprio(1);
      f32x16 s_next = qk_mma<D>(ka, qreg);
      read_v<D, kV + 16 * (2 * D)>(0u, off, lo1, hi1);
      // Softcapped scores are transformed inside the product loop below, beside
      // the exponentials, on every block; a cut block's mask then zeroes the
      // exponentials of its hidden keys after that loop.  (As a per-block choice
      // between this and transforming before the loop, the compiler formed the
      // transform on both paths and selected, one select per score; as two
      // copies of the loop, it spilled.)
      const bool masked = is_masked(i + 1);
      const bool first = !all_ref;
      if constexpr (SOFTCAP) {
        // The compiler left 11 wait states between the S product and the
        // transform's first read on one path out of the loop: wait for the
        // product here, before both paths.
        asm volatile("s_nop 7\n\ts_nop 3" : "+v"(s_next));
      } else {
        apply_mod(s_next, i + 1);
        if (masked)
          apply_mask(s_next, i + 1);
        else
          apply_bias(s_next, i + 1);
      }
      // Reference for the exponentials of block i + 1.  While some row of the
      // wave has seen no visible key its reference must be set from this block's
      // maximum first (rare: the first blocks of a tile).  Otherwise the
      // exponentials use the current reference and are checked where they are
      // summed, at the next step (check_sums), off the path between the two
      // products.
      float alpha = 1.0f;
      bool moved = false;
      if (first) {
        // the fence keeps the block maximum inside this rarely taken branch
        f32x16 sv = s_next;
        asm volatile("" : "+v"(sv));
        if constexpr (SOFTCAP) {
          transform(sv);
          if (masked) apply_mask(sv, i + 1);
        }
        moved = move_reference(block_max(sv), m_run, c, alpha);
        nmc_run = neg_ref(m_run, c);
        all_ref = !__any(m_run == kNegInf);
      }
      const float nmc = nmc_run;
      const float cap_nmc = p.cap_out + nmc;
      // P V of block i, each product followed by the exponentials of block i + 1
      constexpr int kPer = 16 / (2 * (D / 32));  // exponentials per product
      auto expo = [&](int a) {
        if constexpr (SOFTCAP) {
          s_next[a] = softcap_r(s_next[a]);
          xs[a] = exp2_asm(__builtin_fmaf(cap_m2, s_next[a], cap_nmc));
        } else {
          xs[a] = exp2_asm(__builtin_fmaf(s_next[a], c, nmc));
        }
      };
      lgkm_wait<2 * (D / 32)>(lo0, hi0);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        pv_mfma_asm(o[db], u32x4{lo0[db].x, lo0[db].y, hi0[db].x, hi0[db].y}, p0);
#pragma unroll
        for (int e = 0; e < kPer; ++e) expo(db * kPer + e);
      }
      lgkm_wait<0>(lo1, hi1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        pv_mfma_asm(o[db], u32x4{lo1[db].x, lo1[db].y, hi1[db].x, hi1[db].y}, p1);
#pragma unroll
        for (int e = 0; e < kPer; ++e) expo(8 + db * kPer + e);
      }
      __builtin_amdgcn_s_setprio(0);
      if constexpr (SOFTCAP) {
        if (masked) {
          // r lies in [0, 1], so -inf marks exactly the hidden keys
          apply_mask(s_next, i + 1);
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const bool hidden = s_next[a] == kNegInf;
            xs[a] = hidden ? 0.0f : xs[a];
            s_next[a] = hidden ? __builtin_inff() : s_next[a];
          }
        }
      }
      sc = s_next;  // r in place (softcap)
      if (moved) {
        mfma_drain(o);
        l_run *= alpha;
        l_bf *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      }
    };
    int i = 0;
    static_assert(NBUF >= 3 && NBUF <= 5, "the unrolled loop below walks three to five stages");
    for (; i + NBUF <= nb - 1; i += NBUF) {
      step(std::integral_constant<int, 0>{}, i);
      step(std::integral_constant<int, 1>{}, i + 1);
      step(std::integral_constant<int, 2>{}, i + 2);
      if constexpr (NBUF > 3) step(std::integral_constant<int, 3 % NBUF>{}, i + 3);
      if constexpr (NBUF > 4) step(std::integral_constant<int, 4 % NBUF>{}, i + 4);
    }
    if (i + 1 <= nb - 1) step(std::integral_constant<int, 0>{}, i), ++i;
    if (i + 1 <= nb - 1) step(std::integral_constant<int, 1>{}, i), ++i;
    if constexpr (NBUF > 3)
      if (i + 1 <= nb - 1) step(std::integral_constant<int, 2 % NBUF>{}, i), ++i;
    if constexpr (NBUF > 4)
      if (i + 1 <= nb - 1) step(std::integral_constant<int, 3 % NBUF>{}, i), ++i;
    // last block (i == nb - 1, stage i % NBUF): sums and P V only
    if (nb > 0) {
      const float rs = check_sums();
      bf16x8 p0, p1;
      block_sums(xs, rs, l_run, l_bf, p0, p1);
      const uint32_t delta = (uint32_t)((i % NBUF) * T);
      pv_chunk<D, 0>(delta, p0, o, off);
      pv_chunk<D, 16 * (2 * D)>(delta, p1, o, off);
    }
    __syncthreads();  // every wave is done with the stage buffers before the next tile

    // ---- epilogue: O / l and LSE = (m c + log2 l) ln 2
    const float l_tot = pair_sum(l_run);
    const float l_o = pair_sum(l_bf);
    const bool empty = (m_run == kNegInf) || !(l_tot > 0.0f) || !(l_o > 0.0f);
    const float inv = empty ? 0.0f : rcp_fast(l_o);
    if (row_ok) {
      uint16_t* ob = p.o + (int64_t)tile.b * p.o_bs + (q_start + tok) * p.o_ss + (int64_t)head * p.o_hs;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x8 x = {};
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = o[db][4 * q4 + e] * inv;
          bf16x8 y = __builtin_convertvector(x, bf16x8);
          u32x4 yb = __builtin_bit_cast(u32x4, y);
          u32x2 z = {yb.x, yb.y};
          *reinterpret_cast<u32x2*>(ob + 32 * db + 8 * q4 + 4 * kg) = z;
        }
      if (kg == 0 && p.lse) {
        const float lse = empty ? kNegInf : (m_run * c + log2_fast(l_tot)) * kLn2;
        p.lse[(int64_t)tile.b * p.lse_bs + (int64_t)head * p.lse_hs + q_start + tok] = lse;
      }
    }
  }
}

template <int D, bool VARLEN, bool PACK, bool SOFTCAP, bool PAGED, bool ALIBI = false, class MOD = FaNoMod>
__global__ __launch_bounds__(kThreads, 2) void fa_prefill_kernel(FaParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[prefill_smem_bytes<D>()];
  prefill_body<D, VARLEN, PACK, SOFTCAP, PAGED, ALIBI, MOD>(p, smem, blockIdx.x);
}

// ------------------------------------------------------------------ sequence order
// Rank of each sequence by cache length, longest first, ties by index: a strict
// total order, so order[] receives a permutation of [0, B).  Each thread ranks
// one sequence against all B lengths, staged through LDS 256 at a time.
__global__ __launch_bounds__(kThreads) void fa_seq_order_kernel(const int32_t* lens, int B, int32_t* order) {
  __shared__ int32_t sl[kThreads];
  const int b = blockIdx.x * kThreads + threadIdx.x;
  const int mine = b < B ? lens[b] : 0;
  int rank = 0;
  for (int c0 = 0; c0 < B; c0 += kThreads) {
    __syncthreads();
    if (c0 + (int)threadIdx.x < B) sl[threadIdx.x] = lens[c0 + threadIdx.x];
    __syncthreads();
    const int n = min(kThreads, B - c0);
    for (int j = 0; j < n; ++j) {
      const int other = sl[j];
      rank += (other > mine) | ((other == mine) & (c0 + j < b));
    }
  }
  if (b < B) order[rank] = b;
}

// ------------------------------------------------------------------ paged split-KV kernel
// One workgroup per (sequence b, KV head, split).  The packed query rows
// (seqlen_q tokens x g heads, at most 32) are the same for all four waves; each
// 64-key stage is split 16 keys per wave, and the waves' partial states are
// merged through LDS at the end ("Attention kernels...", section 6.3: partial
// states combine with the same rescale as the tiles).  Decode is bound by the
// K/V stream: each wave loads its own rows with plain loads one stage ahead and
// two workgroups share a CU (the 64 KiB of LDS the merge needs sets that).  When
// the page size is a multiple of the stage, a stage lies in one page and its
// physical page is one scalar block-table read; otherwise every row looks its
// page up.  Over an FP8 cache a stage is 128 keys, 32 per wave in an LDS buffer
// of the wave's own (the bytes per wave of a bf16 stage, and no key row of the
// products repeated).
constexpr int kPagedStages = 2;  // stages in the paged kernel's ring
// LDS of the paged decode workgroup: the stage ring, reused after the loop for
// the merge of the four waves' states: O [4][32][D] fp32, then m, l and l (bf16
// weights) [3][4][32]
template <int D>
constexpr int paged_smem_bytes() {
  constexpr int kStage = 2 * DmaGeom<D, FA_PAGED_STAGE>::kTensorBytes;
  constexpr int kMerge = 4 * 32 * D * 4 + 3 * 4 * 32 * 4;
  return kPagedStages * kStage > kMerge ? kPagedStages * kStage : kMerge;
}

// Eight e4m3 codes (two dwords, first code lowest) -> eight bf16 values.  Every
// e4m3 value is a bf16 value (3 mantissa bits, exponents 2^-9 .. 2^8), so the
// conversion (unit scale) is exact.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(u32x2 c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], 1.0f, true);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], 1.0f, false);
  const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], 1.0f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, d),
               __builtin_bit_cast(uint32_t, e)};
}

// The decode work of one workgroup: unit `unit` = (sequence, KV head, split),
// LDS in smem (paged_smem_bytes<D>(), 1 KiB aligned).  FP8: the cache holds
// e4m3 codes (strides in bytes), widened to bf16 between the load and the LDS
// store (the stage layout is the bf16 one); the K scale is folded into the
// score scale by the host and the V scale multiplies O here.
template <int D, bool SOFTCAP, bool FP8 = false>
__device__ __forceinline__ void paged_body(const FaParams& p, char* smem, int unit) {
  // keys per stage: four waves of 16 (bf16), or of 32 (FP8, each wave in an LDS
  // buffer of its own)
  constexpr int NK = FP8 ? 2 * FA_PAGED_STAGE : FA_PAGED_STAGE;
  constexpr int NS = kPagedStages;
  using G = DmaGeom<D, FA_PAGED_STAGE>;  // the bf16 stage
  constexpr int kStage = 2 * G::kTensorBytes;
  static_assert(FA_PAGED_STAGE == 4 * 16, "four waves of 16 keys per bf16 stage");
  static_assert(!FP8 || 4 * 2 * (NK / 4) * 2 * D <= NS * kStage, "FP8 wave buffers fit the stages' LDS");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int kg = lane >> 5;
  const float c = SOFTCAP ? 1.0f : p.scale_log2;

  // bf16: a wave's S^T operand covers 16 keys: lanes 16..31 repeat rows 0..15,
  // and the repeated rows (accumulator slots 8..15) are dropped below.  FP8: 32
  // keys, all slots live.
  LaneOffsets<D> off;
  off.init(lane, lds_addr(smem), lds_addr(smem), FP8 ? 32 : 16);
  // Each wave loads the 16 rows it computes on (rows 16 wave .. 16 wave + 15 of a
  // stage; instruction i fills G::kRowsPerKiB of them), so a wave waits only for
  // its own loads and the stages need no workgroup barrier.  The layout and the
  // swizzles are the same as with shared stage loads.
  constexpr int kWaveRows = NK / 4;
  const int dma_row = kWaveRows * wave + lane / G::kChunksPerRow;  // + i * G::kRowsPerKiB
  const int dma_pc = lane % G::kChunksPerRow;
  int k_src[G::kInstPerWave], v_src[G::kInstPerWave];
#pragma unroll
  for (int i = 0; i < G::kInstPerWave; ++i) {
    k_src[i] = (dma_pc ^ k_swz<D>(dma_row + i * G::kRowsPerKiB)) * 8;
    v_src[i] = (dma_pc ^ v_swz<D>(dma_row + i * G::kRowsPerKiB)) * 8;
  }
  // FP8: a lane loads 16 codes, two adjacent 8-element chunks of a row (the even
  // logical chunk E and E + 1), and writes them widened as two 16-byte LDS chunks
  // into the wave's own buffer (its 32 K rows, then its 32 V rows, in the bf16
  // row layout).  LDS chunk c of buffer row r holds logical chunk c ^ swz(r), so
  // E = 2 pp ^ (swz & ~1) fills LDS chunk 2 pp ^ (swz & 1) and E + 1 the other
  // chunk of the pair.
  constexpr int kPairs = D / 16;                     // chunk pairs per row
  constexpr int kRows8 = 64 / kPairs;                // rows per load instruction
  constexpr int kInst8 = FP8 ? kWaveRows / kRows8 : 1;
  int r8[kInst8], k_src8[kInst8], v_src8[kInst8], k_lds8[kInst8], v_lds8[kInst8];
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < kInst8; ++i) {
      const int rw = i * kRows8 + lane / kPairs;     // row among the wave's 32
      const int c2 = 2 * (lane % kPairs);
      const int sk = k_swz<D>(rw), sv = v_swz<D>(rw);
      r8[i] = rw;
      k_src8[i] = (c2 ^ (sk & ~1)) * 8;
      v_src8[i] = (c2 ^ (sv & ~1)) * 8;
      k_lds8[i] = rw * (2 * D) + (c2 ^ (sk & 1)) * 16;
      v_lds8[i] = rw * (2 * D) + (c2 ^ (sv & 1)) * 16;
    }
  }

  const int S = p.num_splits;
  // groups of Hkv * S workgroups take the sequences longest first when an order
  // is given, so that the short ones fill the end of the grid
  const int b = p.seq_order ? scalar_load_i32(p.seq_order + unit / (p.Hkv * S)) : unit / (p.Hkv * S);
  const int kvh = (unit / S) % p.Hkv;
  const int split = unit % S;

  const int Lk = p.cache_seqlens[b];
  int Lq = p.Nq;
  int64_t q_start = 0;
  if (p.cu_q) {
    // a varlen batch: this sequence's new tokens; sequences with more packed
    // rows than a workgroup holds run in the prefill kernel instead
    q_start = p.cu_q[b];
    Lq = p.cu_q[b + 1] - (int)q_start;
    if (Lq <= 0 || Lq * p.g > FA_PAGED_MAX_ROWS) return;
  }
  const int rows = Lq * p.g;
  const int npages = (Lk + p.page - 1) / p.page;
  const int chunk = (npages + S - 1) / S;
  const int p0 = min(split * chunk, npages), p1 = min(p0 + chunk, npages);
  const int k_lo = p0 * p.page;
  const int k_hi = min(p1 * p.page, Lk);

  // rows' key range, intersected with this split
  FaRowSpan span;
  span.pos_lo = (int64_t)(Lk - Lq);
  span.pos_hi = (int64_t)(Lq - 1) + (Lk - Lq);
  int64_t r_lo, r_hi;
  int has = fa_key_range(span, Lk, p.causal, p.wl, p.wr, &r_lo, &r_hi);
  int64_t kb0 = k_lo > r_lo ? k_lo : r_lo;
  int64_t kb1 = k_hi < r_hi + 1 ? k_hi : r_hi + 1;
  if (!has || kb0 >= kb1) {
    kb0 = 0;
    kb1 = 0;
  }
  // stages start at the split start plus multiples of the stage size
  const int st_first = (int)(kb0 > k_lo ? k_lo + ((kb0 - k_lo) / NK) * NK : k_lo);
  const int nst = kb1 > kb0 ? (int)((kb1 - st_first + NK - 1) / NK) : 0;
  const int kend = (int)kb1;

  const bool row_ok = col < rows;
  const int tok = row_ok ? col / p.g : 0;
  const int head = kvh * p.g + (row_ok ? col % p.g : 0);
  const uint16_t* qb = p.q + (int64_t)b * p.q_bs + (q_start + tok) * p.q_ss + (int64_t)head * p.q_hs;
  // ALiBi (not with softcap): this lane's slope in raw-score units
  const bool alibi = !SOFTCAP && p.alibi != nullptr;
  const float alibi_k = alibi ? p.alibi[(int64_t)b * p.alibi_bs + head] * p.alibi_inv_scale : 0.0f;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row_ok) x = *reinterpret_cast<const u32x4*>(qb + 16 * kk + 8 * kg);
    qreg[kk] = __builtin_bit_cast(bf16x8, x);
  }
  LaneMask mask;
  mask.pos = tok + (Lk - Lq);
  mask.kend = kend;
  mask.kbeg = (int)kb0;
  mask.causal = p.causal;
  mask.wl = p.wl;
  mask.wr = p.wr;

  // element offsets scale to bytes by kEs (bf16 2, e4m3 1)
  constexpr int64_t kEs = FP8 ? 1 : 2;
  const char* kpool = reinterpret_cast<const char*>(p.k) + (int64_t)kvh * p.k_hs * kEs;
  const char* vpool = reinterpret_cast<const char*>(p.v) + (int64_t)kvh * p.v_hs * kEs;
  const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;
  // a stage (bf16) or a wave's 32 rows of one (FP8) lies in one page
  const bool page_aligned = (p.page % (FP8 ? NK / 4 : NK)) == 0;
  // rows past the last key read the last key (finite data the mask drops)
  const int last = kend > 0 ? kend - 1 : 0;
  const int64_t phys_last = (page_aligned && nst > 0)
                                ? scalar_load_i32(bt + __builtin_amdgcn_readfirstlane(last / p.page)) : 0;
  const int slot_last = last % p.page;
  // A stage's rows go global -> registers -> LDS: plain loads stream faster than
  // LDS-DMA here (≈6.9 against ≈6.1 TB/s for this pattern in a probe).  Lane l of
  // load i holds the 16 bytes that the stage layout puts at byte l * 16 of the
  // wave's i-th KiB (row dma_row + i * kRowsPerKiB, swizzled chunk).  The loads of
  // stage i + 1 are in flight while stage i is computed.
  u32x4 kr[FP8 ? kInst8 : G::kInstPerWave], vr[FP8 ? kInst8 : G::kInstPerWave];
  auto load8 = [&](int n0, u32x4 (&kr)[FP8 ? kInst8 : G::kInstPerWave], u32x4 (&vr)[FP8 ? kInst8 : G::kInstPerWave]) {
    n0 += kWaveRows * wave;  // this wave's first key
    if (page_aligned) {
      // a wave whose rows all lie past the last key reads the last key's page
      // entry (its rows are clamped to that key), never an entry past the table
      const int64_t phys = scalar_load_i32(bt + __builtin_amdgcn_readfirstlane(min(n0, last) / p.page));
      const int slot0 = n0 % p.page;
#pragma unroll
      for (int i = 0; i < kInst8; ++i) {
        const bool live = n0 + r8[i] < kend;
        const int slot = live ? slot0 + r8[i] : slot_last;
        const int64_t ph = live ? phys : phys_last;
        kr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kpool + ph * p.k_bs + (int64_t)slot * p.k_ss + k_src8[i]));
        vr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(vpool + ph * p.v_bs + (int64_t)slot * p.v_ss + v_src8[i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kInst8; ++i) {
        int key = n0 + r8[i];
        key = key < kend ? key : kend - 1;
        const int64_t phys = bt[key / p.page];
        const int slot = key % p.page;
        kr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kpool + phys * p.k_bs + (int64_t)slot * p.k_ss + k_src8[i]));
        vr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(vpool + phys * p.v_bs + (int64_t)slot * p.v_ss + v_src8[i]));
      }
    }
  };
  auto load = [&](int n0) {
    if constexpr (FP8) {
      load8(n0, kr, vr);
    } else {
      if (page_aligned) {
        // the whole stage is in one page: one scalar table read
        const int64_t phys = scalar_load_i32(bt + __builtin_amdgcn_readfirstlane(n0 / p.page));
        const int slot0 = n0 % p.page;
#pragma unroll
        for (int i = 0; i < G::kInstPerWave; ++i) {
          const int r = dma_row + i * G::kRowsPerKiB;
          const bool live = n0 + r < kend;
          const int slot = live ? slot0 + r : slot_last;
          const int64_t ph = live ? phys : phys_last;
          kr[i] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(kpool + (ph * p.k_bs + (int64_t)slot * p.k_ss + k_src[i]) * kEs));
          vr[i] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(vpool + (ph * p.v_bs + (int64_t)slot * p.v_ss + v_src[i]) * kEs));
        }
      } else {
#pragma unroll
        for (int i = 0; i < G::kInstPerWave; ++i) {
          int key = n0 + dma_row + i * G::kRowsPerKiB;
          key = key < kend ? key : kend - 1;
          const int64_t phys = bt[key / p.page];
          const int slot = key % p.page;
          kr[i] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(kpool + (phys * p.k_bs + (int64_t)slot * p.k_ss + k_src[i]) * kEs));
          vr[i] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(vpool + (phys * p.v_bs + (int64_t)slot * p.v_ss + v_src[i]) * kEs));
        }
      }
    }
  };
  // the wave's buffer: its K rows, then its V rows
  constexpr int kWaveBuf = 2 * kWaveRows * (2 * D);
  constexpr int kWaveV = kWaveRows * (2 * D);
  auto store8 = [&](const u32x4 (&kr)[FP8 ? kInst8 : G::kInstPerWave],
                    const u32x4 (&vr)[FP8 ? kInst8 : G::kInstPerWave]) {
    // the previous stage's operand reads (inline assembly) stay above these
    // stores into the same buffer; LDS operations of one wave complete in order
    asm volatile("" ::: "memory");
    char* wb = smem + wave * kWaveBuf;
#pragma unroll
    for (int i = 0; i < kInst8; ++i) {
      *reinterpret_cast<u32x4*>(wb + k_lds8[i]) = e4m3x8_to_bf16(u32x2{kr[i][0], kr[i][1]});
      *reinterpret_cast<u32x4*>(wb + (k_lds8[i] ^ 16)) = e4m3x8_to_bf16(u32x2{kr[i][2], kr[i][3]});
      *reinterpret_cast<u32x4*>(wb + kWaveV + v_lds8[i]) = e4m3x8_to_bf16(u32x2{vr[i][0], vr[i][1]});
      *reinterpret_cast<u32x4*>(wb + kWaveV + (v_lds8[i] ^ 16)) = e4m3x8_to_bf16(u32x2{vr[i][2], vr[i][3]});
    }
    asm volatile("" ::: "memory");
  };
  auto store = [&](int buf) {
    if constexpr (FP8) {
      store8(kr, vr);
    } else {
      char* dst = smem + buf * kStage + wave * (kWaveRows * 2 * D) + lane * 16;
#pragma unroll
      for (int i = 0; i < G::kInstPerWave; ++i) {
        *reinterpret_cast<u32x4*>(dst + i * 1024) = kr[i];
        *reinterpret_cast<u32x4*>(dst + G::kTensorBytes + i * 1024) = vr[i];
      }
    }
    // the operand reads below are inline assembly: keep the stores above them
    // (LDS operations of one wave complete in order, so no wait is needed)
    asm volatile("" ::: "memory");
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f, l_bf = 0.0f;

  // the products, mask and online softmax of stage i (from LDS buffer buf)
  auto compute = [&](int i, int buf) {
    const int n0 = st_first + i * NK;
    if constexpr (FP8) {
      // this wave's 32 keys, rows 0..31 of its buffer
      const uint32_t delta = wave * kWaveBuf;
      f32x16 s = qk_block<D, 0>(delta, qreg, off);
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = n0 + kWaveRows * wave + 8 * (a >> 2) + 4 * kg + (a & 3);
        float x = s[a];
        if (alibi) x = __builtin_fmaf(-alibi_k, (float)abs(mask.pos - key), x);
        if (SOFTCAP) x = softcap_log2(x, p.cap_in, p.cap_out);
        s[a] = mask.visible(key) ? x : kNegInf;
      }
      bf16x8 p0, p1;
      online_softmax<D>(s, m_run, l_run, l_bf, o, c, p0, p1);
      pv_chunk<D, kWaveV>(delta, p0, o, off);
      pv_chunk<D, kWaveV + 16 * (2 * D)>(delta, p1, o, off);
      return;
    }
    // this wave's 16 keys: rows 16 wave .. 16 wave + 15 of the stage buffer
    const uint32_t delta = buf * kStage + wave * 16 * (2 * D);
    f32x16 s = qk_block<D, 0>(delta, qreg, off);
    if (alibi) {
      // -slope |p - key| on the raw score (the softmax scales both)
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int key = n0 + 16 * wave + 8 * ((a >> 2) & 1) + 4 * kg + (a & 3);
        s[a] = __builtin_fmaf(-alibi_k, (float)abs(mask.pos - key), s[a]);
      }
    }
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int key = n0 + 16 * wave + 8 * ((a >> 2) & 1) + 4 * kg + (a & 3);
      float x = SOFTCAP ? softcap_log2(s[a], p.cap_in, p.cap_out) : s[a];
      s[a] = (a < 8 && mask.visible(key)) ? x : kNegInf;
    }
    bf16x8 p0, p1;
    online_softmax<D>(s, m_run, l_run, l_bf, o, c, p0, p1);
    pv_chunk<D, G::kTensorBytes>(delta, p0, o, off);
  };
  if constexpr (FP8) {
    // An FP8 stage of 32 keys a wave is the bytes of a bf16 stage of 16: the
    // loads of stage i + 1 are in flight while stage i is computed, and each
    // wave stores into and reads from its own buffer only (no barrier).
    if (nst > 0) load8(st_first, kr, vr);
    for (int i = 0; i < nst; ++i) {
      store8(kr, vr);
      if (i + 1 < nst) load8(st_first + (i + 1) * NK, kr, vr);
      compute(i, 0);
    }
  } else {
    if (nst > 0) load(st_first);
    for (int i = 0; i < nst; ++i) {
      const int buf = i % NS;
      // stage i arrives in the registers (the compiler waits for the loads); this
      // wave's reads of the buffer, from stage i - NS, completed before their products
      store(buf);
      if (i + 1 < nst) load(st_first + (i + 1) * NK);
      compute(i, buf);
    }
  }
  __syncthreads();

  // ---- merge the four waves' states through LDS
  float* mo = reinterpret_cast<float*>(smem);               // [4][32 cols][D]
  float* ml = mo + 4 * 32 * D;  // [4][32] m, then [4][32] l (fp32), then [4][32] l (bf16 weights)
  const float l_w = pair_sum(l_run);
  const float lb_w = pair_sum(l_bf);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int d = 32 * db + 8 * (a >> 2) + 4 * kg + (a & 3);
      mo[(wave * 32 + col) * D + d] = o[db][a];
    }
  if (kg == 0) {
    ml[wave * 32 + col] = m_run;       // log2 units
    ml[128 + wave * 32 + col] = l_w;
    ml[256 + wave * 32 + col] = lb_w;
  }
  __syncthreads();

  // thread -> (column, 16 consecutive d values)
  constexpr int kParts = D / 16;             // 8 for D = 128, 4 for D = 64
  const int cc = tid / kParts;
  const int d0 = (tid % kParts) * 16;
  if (cc < 32 && cc < rows) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[w * 32 + cc]);
    float e[4], L = 0.0f, Lb = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = ml[w * 32 + cc];
      e[w] = (mw == kNegInf) ? 0.0f : exp2_fast(mw - M);
      L += e[w] * ml[128 + w * 32 + cc];
      Lb += e[w] * ml[256 + w * 32 + cc];
    }
    const bool empty = (M == kNegInf) || !(L > 0.0f) || !(Lb > 0.0f);
    float inv = empty ? 0.0f : rcp_fast(Lb);
    if constexpr (FP8) inv *= p.v_scale;
    float acc[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) sum += e[w] * mo[(w * 32 + cc) * D + d0 + x];
      acc[x] = sum * inv;
    }
    const float lse = empty ? kNegInf : (M + log2_fast(L)) * kLn2;
    const int ctok = cc / p.g;
    const int chead = kvh * p.g + cc % p.g;
    const int64_t r = ((int64_t)b * p.Hq + chead) * Lq + ctok;  // LSE row order
    if (S == 1) {
      uint16_t* ob = p.o + (int64_t)b * p.o_bs + (q_start + ctok) * p.o_ss + (int64_t)chead * p.o_hs + d0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x8 x;
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) x[e2] = acc[8 * h + e2];
        *reinterpret_cast<bf16x8*>(ob + 8 * h) = __builtin_convertvector(x, bf16x8);
      }
      if (d0 == 0 && p.lse) p.lse[(int64_t)b * p.lse_bs + (int64_t)chead * p.lse_hs + q_start + ctok] = lse;
    } else if (p.cu_q) {
      // varlen batch: partial rows packed per (sequence, KV head) unit, 32 each
      const int64_t rows_all = (int64_t)p.B * p.Hkv * FA_PAGED_MAX_ROWS;
      const int64_t pr = ((int64_t)b * p.Hkv + kvh) * FA_PAGED_MAX_ROWS + cc;
      float* op = p.o_part + ((int64_t)split * rows_all + pr) * D + d0;
#pragma unroll
      for (int x = 0; x < 16; x += 4)
        *reinterpret_cast<float4*>(op + x) = make_float4(acc[x], acc[x + 1], acc[x + 2], acc[x + 3]);
      if (d0 == 0) p.lse_part[(int64_t)split * rows_all + pr] = lse;
    } else {
      const int64_t rows_all = (int64_t)p.B * p.Hq * Lq;
      float* op = p.o_part + ((int64_t)split * rows_all + r) * D + d0;
#pragma unroll
      for (int x = 0; x < 16; x += 4)
        *reinterpret_cast<float4*>(op + x) = make_float4(acc[x], acc[x + 1], acc[x + 2], acc[x + 3]);
      if (d0 == 0) p.lse_part[(int64_t)split * rows_all + r] = lse;
    }
  }
}

template <int D, bool SOFTCAP, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void fa_paged_kernel(FaParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[paged_smem_bytes<D>()];
  paged_body<D, SOFTCAP, FP8>(p, smem, blockIdx.x);
}

// ------------------------------------------------------------------ unified batch
// One launch for a mixed batch over a paged cache ("Attention kernels...",
// section 5.1): the first n_tiles workgroups are the prefill tiles of the
// sequences with many packed rows (prefill_body, longest first), the last ones
// the decode units of the others (paged_body), so that the short HBM-bound
// decode workgroups fill the machine beside the last MFMA-bound tiles instead
// of running before or after them.
template <int D, bool PACK, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void fa_unified_kernel(FaParams pd, FaParams pp, int n_tiles) {
  constexpr int kA = prefill_smem_bytes<D>(), kB = paged_smem_bytes<D>();
  __shared__ __attribute__((aligned(1024))) char smem[kA > kB ? kA : kB];
  const int bid = blockIdx.x;
  if (bid < n_tiles)
    prefill_body<D, true, PACK, SOFTCAP, true>(pp, smem, bid);
  else
    paged_body<D, SOFTCAP>(pd, smem, bid - n_tiles);
}

// ------------------------------------------------------------------ combine kernel
// One wave per row: M = max_s LSE_s, w_s = exp(LSE_s - M), LSE = M + ln sum w_s,
// O = sum_s w_s O_s / sum w_s ("Attention kernels...", section 6.3).  A partial
// whose LSE is -inf has weight 0 (its O is not read).  The partials are fp32
// (split-KV) or bf16 (two attention outputs, e.g. over a cached prefix and the
// new suffix).
template <int D, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void fa_combine_kernel(FaCombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const int t = (int)(r % p.Nq);
  const int h = (int)((r / p.Nq) % p.Hq);
  const int64_t b = r / ((int64_t)p.Nq * p.Hq);
  const int S = p.num_splits;
  const int64_t o_row = b * p.i_bs + (int64_t)t * p.i_ss + (int64_t)h * p.i_hs;
  const int64_t l_row = b * p.il_bs + (int64_t)h * p.il_hs + (int64_t)t * p.il_ss;
  auto lse_of = [&](int s_) -> float {
    return p.pair ? p.lse_in[s_][l_row] : p.lse_in[0][(int64_t)s_ * p.lse_split + l_row];
  };
  float M = kNegInf;
  for (int s_ = 0; s_ < S; ++s_) M = fmaxf(M, lse_of(s_));
  constexpr int E = D / 64;  // elements per lane
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  float W = 0.0f;
  if (M != kNegInf) {
    for (int s_ = 0; s_ < S; ++s_) {
      const float x = lse_of(s_);
      if (x == kNegInf) continue;
      const float w = exp2_fast((x - M) * kLog2e);
      W += w;
      const int64_t off = (p.pair ? 0 : (int64_t)s_ * p.o_split) + o_row + lane * E;
      const void* base = p.pair ? p.o_in[s_] : p.o_in[0];
      if constexpr (IN_BF16) {
        const uint16_t* op = static_cast<const uint16_t*>(base) + off;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * __uint_as_float((uint32_t)op[e] << 16);
      } else {
        const float* op = static_cast<const float*>(base) + off;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * op[e];
      }
    }
  }
  const bool empty = (M == kNegInf) || !(W > 0.0f);
  const float inv = empty ? 0.0f : rcp_fast(W);
  uint16_t* ob = p.o + b * p.o_bs + (int64_t)t * p.o_ss + (int64_t)h * p.o_hs + lane * E;
  if (E == 2) {
    f32x8 x = {acc[0] * inv, acc[E - 1] * inv, 0, 0, 0, 0, 0, 0};
    bf16x8 y = __builtin_convertvector(x, bf16x8);
    *reinterpret_cast<uint32_t*>(ob) = __builtin_bit_cast(u32x4, y).x;
  } else {
    f32x8 x = {acc[0] * inv, 0, 0, 0, 0, 0, 0, 0};
    bf16x8 y = __builtin_convertvector(x, bf16x8);
    *ob = (uint16_t)(__builtin_bit_cast(u32x4, y).x & 0xffffu);
  }
  if (lane == 0 && p.lse)
    p.lse[b * p.l_bs + (int64_t)h * p.l_hs + (int64_t)t * p.l_ss] = empty ? kNegInf : M + __builtin_logf(W);
}

// Combine of the varlen paged decode partials: one wave per packed row of a
// (sequence, KV head) unit (FA_PAGED_MAX_ROWS each); rows of sequences that ran
// in the prefill kernel, and rows past a sequence's new tokens, are skipped.
// Packed row r of sequence b and KV head kvh is token cu_q[b] + r / g of query
// head kvh * g + r % g.
template <int D>
__global__ __launch_bounds__(kThreads) void fa_combine_packed_kernel(FaParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t rows_all = (int64_t)p.B * p.Hkv * FA_PAGED_MAX_ROWS;
  if (u >= rows_all) return;
  const int r = (int)(u % FA_PAGED_MAX_ROWS);
  const int kvh = (int)((u / FA_PAGED_MAX_ROWS) % p.Hkv);
  const int b = (int)(u / ((int64_t)FA_PAGED_MAX_ROWS * p.Hkv));
  const int q0 = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - q0;
  if (Lq <= 0 || Lq * p.g > FA_PAGED_MAX_ROWS || r >= Lq * p.g) return;
  const int S = p.num_splits;
  float M = kNegInf;
  for (int s_ = 0; s_ < S; ++s_) M = fmaxf(M, p.lse_part[(int64_t)s_ * rows_all + u]);
  constexpr int E = D / 64;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  float W = 0.0f;
  if (M != kNegInf) {
    for (int s_ = 0; s_ < S; ++s_) {
      const float x = p.lse_part[(int64_t)s_ * rows_all + u];
      if (x == kNegInf) continue;
      const float w = exp2_fast((x - M) * kLog2e);
      W += w;
      const float* op = p.o_part + ((int64_t)s_ * rows_all + u) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * op[e];
    }
  }
  const bool empty = (M == kNegInf) || !(W > 0.0f);
  const float inv = empty ? 0.0f : rcp_fast(W);
  const int tok = q0 + r / p.g;
  const int head = kvh * p.g + r % p.g;
  uint16_t* ob = p.o + (int64_t)tok * p.o_ss + (int64_t)head * p.o_hs + lane * E;
  if (E == 2) {
    f32x8 x = {acc[0] * inv, acc[E - 1] * inv, 0, 0, 0, 0, 0, 0};
    bf16x8 y = __builtin_convertvector(x, bf16x8);
    *reinterpret_cast<uint32_t*>(ob) = __builtin_bit_cast(u32x4, y).x;
  } else {
    f32x8 x = {acc[0] * inv, 0, 0, 0, 0, 0, 0, 0};
    bf16x8 y = __builtin_convertvector(x, bf16x8);
    *ob = (uint16_t)(__builtin_bit_cast(u32x4, y).x & 0xffffu);
  }
  if (lane == 0 && p.lse) p.lse[(int64_t)head * p.lse_hs + tok] = empty ? kNegInf : M + __builtin_logf(W);
}

// ------------------------------------------------------------------ rotary embedding, K/V append
// Rotary position embedding of one 16-byte chunk (8 dims) of a bf16 row at
// position pos, from the caller's cos/sin tables (the rotation the kvcache call
// can apply on the way into the cache, "FA4 ...", section 6.2; which pairs of
// dims rotate together is the caller's choice, see FaRotary).  src and dst are
// the row (they may alias).  Chunk c of a half-split rotation also owns its
// partner chunk c + dim / 16; the partner's own call does nothing.  fp32
// arithmetic, round-to-nearest-even to bf16.
template <int D>
__device__ __forceinline__ void rope_chunk(const uint16_t* src, uint16_t* dst, int c, int pos, const FaRotary& r) {
  typedef float f32x8_ __attribute__((ext_vector_type(8)));
  const int half = r.dim / 2;
  const float* cs = r.cos + (int64_t)pos * half;
  const float* sn = r.sin + (int64_t)pos * half;
  auto load = [&](int cc) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 8 * cc)), f32x8_);
  };
  auto store = [&](int cc, f32x8_ x) {
    *reinterpret_cast<u32x4*>(dst + 8 * cc) = __builtin_bit_cast(u32x4, __builtin_convertvector(x, bf16x8));
  };
  if (8 * c >= r.dim) {  // past the rotated dims: copy
    if (src != dst) *reinterpret_cast<u32x4*>(dst + 8 * c) = *reinterpret_cast<const u32x4*>(src + 8 * c);
    return;
  }
  if (r.interleaved) {  // pairs (2i, 2i + 1) inside the chunk, i = 4 c + j
    f32x8_ x = load(c), y;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float co = cs[4 * c + j], si = sn[4 * c + j];
      y[2 * j] = x[2 * j] * co - x[2 * j + 1] * si;
      y[2 * j + 1] = x[2 * j] * si + x[2 * j + 1] * co;
    }
    store(c, y);
    return;
  }
  if (8 * c >= half) return;  // written by the chunk c - dim / 16
  const int c2 = c + half / 8;
  f32x8_ a = load(c), b = load(c2), a2, b2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // pairs (i, i + dim / 2), i = 8 c + j
    const float co = cs[8 * c + j], si = sn[8 * c + j];
    a2[j] = a[j] * co - b[j] * si;
    b2[j] = a[j] * si + b[j] * co;
  }
  store(c, a2);
  store(c2, b2);
}

// In-place rotary embedding of a [B, L, H, D] tensor (the new queries of a
// kvcache step), one thread per 16-byte chunk.
template <int D>
__global__ __launch_bounds__(kThreads) void fa_rotary_kernel(FaRotaryParams p) {
  constexpr int C = D / 8;
  const int64_t total = (int64_t)p.B * p.L * p.H * C;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % C);
    int64_t r = i / C;
    const int h = (int)(r % p.H);
    r /= p.H;
    const int t = (int)(r % p.L);
    const int b = (int)(r / p.L);
    const int pos = (p.pos_base ? p.pos_base[b] : 0) + t;
    uint16_t* row = p.x + b * p.bs + t * p.ss + h * p.hs;
    rope_chunk<D>(row, row, c, pos, p.rot);
  }
}

// Incremental decoding writes the new keys and values into the cache in place
// ("FA4 ...", section 6.2): token t of sequence b goes to logical position
// cache_seqlens[b] + t, i.e. slot pos % page of page block_table[b][pos / page]
// ("Attention kernels...", section 6.1); the keys optionally rotated on the
// way.  Bound by memory: one thread per 16-byte chunk of a row, consecutive
// threads on consecutive chunks of a row and then of the next head, so a wave
// writes whole rows.
template <int D>
__global__ __launch_bounds__(kThreads) void fa_append_kernel(FaAppendParams p) {
  constexpr int C = D / 8;  // 16-byte chunks per row
  const int64_t total = (int64_t)p.B * p.L * p.Hkv * C;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % C);
    int64_t r = i / C;
    const int h = (int)(r % p.Hkv);
    r /= p.Hkv;
    const int t = (int)(r % p.L);
    const int b = (int)(r / p.L);
    const int pos = p.cache_seqlens[b] + t;
    const int64_t phys = p.block_table[(int64_t)b * p.max_blocks + pos / p.page];
    const int64_t slot = pos % p.page;
    const uint16_t* ks = p.k_new + b * p.kn_bs + t * p.kn_ss + h * p.kn_hs;
    uint16_t* kd = p.k_cache + phys * p.k_ps + slot * p.k_ss + h * p.k_hs;
    if (p.rot.cos)
      rope_chunk<D>(ks, kd, c, pos, p.rot);
    else
      *reinterpret_cast<u32x4*>(kd + 8 * c) = *reinterpret_cast<const u32x4*>(ks + 8 * c);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(p.v_new + b * p.vn_bs + t * p.vn_ss + h * p.vn_hs + 8 * c);
    *reinterpret_cast<u32x4*>(p.v_cache + phys * p.v_ps + slot * p.v_ss + h * p.v_hs + 8 * c) = vx;
  }
}

// e4m3 code of x / scale, rounded to nearest even and saturated at +-448 (a NaN
// stays NaN), two values per conversion; the quotient is the correctly rounded
// fp32 division.
__device__ __forceinline__ float e4m3_clamp(float x, float scale) {
  const float q = x / scale;
  return q > 448.0f ? 448.0f : (q < -448.0f ? -448.0f : q);
}
// Eight bf16 values (16 bytes, first value lowest) -> eight e4m3 codes.
__device__ __forceinline__ u32x2 bf16x8_to_e4m3(u32x4 x, float scale) {
  u32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t a = x[2 * w], b = x[2 * w + 1];
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(__uint_as_float(a << 16), scale),
                                            e4m3_clamp(__uint_as_float(a & 0xffff0000u), scale), 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(__uint_as_float(b << 16), scale),
                                        e4m3_clamp(__uint_as_float(b & 0xffff0000u), scale), c, true);
    r[w] = (uint32_t)c;
  }
  return r;
}

// Append to an FP8 (e4m3) cache: the same walk as fa_append_kernel, each 16-byte
// chunk of a new bf16 row written as 8 codes (cache strides in bytes).
template <int D>
__global__ __launch_bounds__(kThreads) void fa_append_fp8_kernel(FaAppendParams p) {
  constexpr int C = D / 8;  // 8-element chunks per row
  const int64_t total = (int64_t)p.B * p.L * p.Hkv * C;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint8_t* kc = reinterpret_cast<uint8_t*>(p.k_cache);
  uint8_t* vc = reinterpret_cast<uint8_t*>(p.v_cache);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % C);
    int64_t r = i / C;
    const int h = (int)(r % p.Hkv);
    r /= p.Hkv;
    const int t = (int)(r % p.L);
    const int b = (int)(r / p.L);
    const int pos = p.cache_seqlens[b] + t;
    const int64_t phys = p.block_table[(int64_t)b * p.max_blocks + pos / p.page];
    const int64_t slot = pos % p.page;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(p.k_new + b * p.kn_bs + t * p.kn_ss + h * p.kn_hs + 8 * c);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(p.v_new + b * p.vn_bs + t * p.vn_ss + h * p.vn_hs + 8 * c);
    *reinterpret_cast<u32x2*>(kc + phys * p.k_ps + slot * p.k_ss + h * p.k_hs + 8 * c) = bf16x8_to_e4m3(kx, p.k_scale);
    *reinterpret_cast<u32x2*>(vc + phys * p.v_ps + slot * p.v_ss + h * p.v_hs + 8 * c) = bf16x8_to_e4m3(vx, p.v_scale);
  }
}

// ------------------------------------------------------------------ backward
// "Attention kernels...", section 4.3: the backward recomputes S = Q K^T block by
// block and takes P = exp(S - L) straight from the saved log-sum-exp L, with no
// online reduction; dV = P^T dO, dP = dO V^T, dS = P (dP - D) with
// D = rowsum(dO O) (the pages' preprocess; here the dQ kernel's prologue, which
// also hands D and L to the dK/dV kernel), dQ = scale dS K, dK = scale dS^T Q.
// P and dS enter their products rounded to bf16, like P in the forward.
//
// Two kernels split the work so that each accumulates its gradient in
// registers: the dQ kernel walks key blocks for a block of queries (the
// forward's orientation: a lane owns a query), the dK/dV kernel walks query
// blocks (and the query heads of a KV-head group) for a block of keys, with
// the roles of queries and keys exchanged (a lane owns a key).  Each product
// reads its operands as the forward does: rows of an LDS tile by
// ds_read_b128, or a tile read transposed by ds_read_b64_tr_b16; a tile read
// both ways (K in the dQ kernel, Q and dO in the dK/dV kernel) is staged once,
// in a swizzle that serves both reads.

// 1 KiB LDS-DMA share of a 32-row bf16 tile: rows (row0 + dma_row + 4 RPK j) of
// a tensor whose rows sit at base + r * stride, clamped to the last valid row
// (the mask drops what the clamp duplicates); chunk src of each row.
template <int D>
__device__ __forceinline__ void dma_rows(const uint16_t* base, int64_t stride, int row0, int dma_row, int last,
                                         int src, char* dst) {
  using G = DmaGeom<D, 32>;
#pragma unroll
  for (int j = 0; j < G::kInstPerWave; ++j) {
    int r = row0 + dma_row + j * G::kRowStep;
    r = r < last ? r : last;
    dma16(base + (int64_t)r * stride + src, dst + j * 4096);
  }
}


// The backward kernels read some stage tiles (32 rows of D bf16) both ways: by
// rows with ds_read_b128 and transposed with ds_read_b64_tr_b16 (K in the dQ
// kernel, Q and dO in the dK/dV kernel).  One swizzle serves both reads, so
// each tile is staged once: stored 16-byte chunk =
// logical chunk ^ u_swz(row), where u_swz takes every chunk value over any 16
// aligned rows (the 16 rows a row read serves at once land in distinct banks)
// and its 64-byte-segment bits differ over any 4 aligned rows (the 4 rows of a
// transposed read land in distinct segments).  D = 64: a row is half of the
// 256-byte bank line and the row parity is the extra bank bit; the same two
// rules hold with the segment bit taken from row bit 1.
template <int D>
__device__ __forceinline__ int u_swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Per-lane LDS byte addresses of the reads of one unified tile at a base that is
// a multiple of 256 bytes.  The chunk pair kk of a row read and the d-block db
// of a transposed read only flip address bits 5..7 (bits no row offset, stage
// offset or base touches), so three registers serve every read: row(kk) =
// row0 ^ (kk << 5), tlo(db) = tlo0 ^ (db << 6), thi(db) = thi0 ^ (db << 6).  A
// step adds its stage's offset to the base before the flips; the tensor and
// chunk offsets within the stage are the instructions' immediates.
template <int D>
struct UniOffsets {
  uint32_t row0;        // ds_read_b128: row lane % 32, chunk lane / 32 (kk = 0)
  uint32_t tlo0, thi0;  // ds_read_b64_tr_b16, d-block 0: rows 0..7 / 8..15 of a 16-row chunk
  __device__ __forceinline__ void init(int lane, uint32_t base) {
    const int col = lane & 31, kg = lane >> 5;
    row0 = base + col * (2 * D) + ((kg ^ u_swz<D>(col)) << 4);
    // within a 16-lane group, lanes 4 i .. 4 i + 3 address 32 bytes of row i
    const int j = lane & 15, half = (lane >> 4) & 1;
    const int r = 4 * kg + (j >> 2);
    const int c = 2 * half + ((j & 3) >> 1);
    tlo0 = base + r * (2 * D) + ((c ^ u_swz<D>(r)) << 4) + (j & 1) * 8;
    thi0 = base + (r + 8) * (2 * D) + ((c ^ u_swz<D>(r + 8)) << 4) + (j & 1) * 8;
  }
  // the stage at byte st of the base: row-read and transposed-read addresses
  __device__ __forceinline__ void rows(uint32_t st, uint32_t (&a)[D / 16]) const {
    const uint32_t r = row0 + st;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) a[kk] = r ^ (uint32_t)(kk << 5);
  }
  __device__ __forceinline__ void trs(uint32_t st, uint32_t (&lo)[D / 32], uint32_t (&hi)[D / 32]) const {
    const uint32_t l = tlo0 + st, h = thi0 + st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) lo[db] = l ^ (uint32_t)(db << 6), hi[db] = h ^ (uint32_t)(db << 6);
  }
};
template <int D, int OFF, int K0, int NK>
__device__ __forceinline__ void uni_rows(const uint32_t (&row)[D / 16], u32x4 (&a)[D / 16]) {
#pragma unroll
  for (int kk = K0; kk < K0 + NK; ++kk) a[kk] = ds_read_b128<OFF>(row[kk]);
}
template <int D, int OFF, int DB0, int NDB>
__device__ __forceinline__ void uni_tr(const uint32_t (&tlo)[D / 32], const uint32_t (&thi)[D / 32],
                                       u32x2 (&lo)[NDB], u32x2 (&hi)[NDB]) {
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    lo[i] = ds_read_tr16<OFF>(tlo[DB0 + i]);
    hi[i] = ds_read_tr16<OFF>(thi[DB0 + i]);
  }
}

// dQ: one workgroup per (batch, query head, 128-row block); each wave owns 32
// query rows and walks the key blocks the rows can see.  A stage holds the key
// block's K and V tiles in the unified swizzle: K rows for S^T = K Q^T, K read
// transposed for dQ^T += K^T dS^T, V rows for dP^T = V dO^T.
template <int D, bool VARLEN, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void fa_bwd_dq_kernel(FaBwdParams p) {
  constexpr int BN = 32;
  constexpr int NBUF = 3;
  using G = DmaGeom<D, BN>;
  constexpr int T = G::kTensorBytes;
  constexpr int kStage = 2 * T;  // K tile, V tile
  static_assert(T + 16 * (2 * D) < 65536, "tile offsets must fit the immediate");
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * kStage];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, kg = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float c = p.scale_log2;
  const float cap2 = p.cap_in * (2.0f * kLog2e);  // softcap: exp(2 s cap_in) = exp2(s cap2)
  UniOffsets<D> uo;
  uo.init(lane, lds_addr(smem));
  const int dma_row = wave * G::kRowsPerKiB + lane / G::kChunksPerRow;
  const int u_src = ((lane % G::kChunksPerRow) ^ u_swz<D>(dma_row)) * 8;

  // tile: row blocks longest first (causal rows near the end see more keys)
  const int m_blocks = (p.Nq + 127) / 128;
  const int64_t pairs = (int64_t)p.B * p.Hq;
  const int64_t t = blockIdx.x;
  const int mb = m_blocks - 1 - (int)(t / pairs);
  const int b = (int)((t % pairs) / p.Hq), h = (int)((t % pairs) % p.Hq), kvh = h / p.g;
  const int m0 = mb * 128;
  // the sequence: lengths, token offsets and its (head, row 0) in the LSE-row arrays
  int Lq = p.Nq, Lk = p.Nk;
  int64_t tq = 0, tk = 0, lrow = ((int64_t)b * p.Hq + h) * p.Nq;
  if constexpr (VARLEN) {
    tq = scalar_load_i32(p.cu_q + b);
    Lq = scalar_load_i32(p.cu_q + b + 1) - (int)tq;
    tk = scalar_load_i32(p.cu_k + b);
    Lk = scalar_load_i32(p.cu_k + b + 1) - (int)tk;
    lrow = (int64_t)h * p.total_q + tq;
    if (m0 >= Lq) return;  // past this sequence's rows (the grid covers the longest)
  }
  FaRowSpan span;
  span.pos_lo = (int64_t)m0 + (Lk - Lq);
  span.pos_hi = (int64_t)min(m0 + 128, Lq) - 1 + (Lk - Lq);
  int n_lo, n_hi, f_lo, f_hi;
  fa_key_tiles(span, Lk, p.causal, p.wl, p.wr, BN, &n_lo, &n_hi);
  fa_full_tiles(span, Lk, p.causal, p.wl, p.wr, BN, &f_lo, &f_hi);
  const int nb = n_hi - n_lo;

  const int row = m0 + wave * 32 + col;
  const bool row_ok = row < Lq;
  bf16x8 qreg[D / 16], doreg[D / 16];
  {
    const uint16_t* qb = p.q + b * p.q_bs + (tq + (row_ok ? row : 0)) * p.q_ss + h * p.q_hs;
    const uint16_t* db = p.dout + b * p.do_bs + (tq + (row_ok ? row : 0)) * p.do_ss + h * p.do_hs;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (row_ok) {
        x = *reinterpret_cast<const u32x4*>(qb + 16 * kk + 8 * kg);
        y = *reinterpret_cast<const u32x4*>(db + 16 * kk + 8 * kg);
      }
      qreg[kk] = __builtin_bit_cast(bf16x8, x);
      doreg[kk] = __builtin_bit_cast(bf16x8, y);
    }
  }
  // D = rowsum(dO O) of the row (fp32) and its L in base-2 units; both also go
  // to the workspace for the dK/dV kernel (the grid covers every query row once).
  // P = exp2(s c - L log2 e); a row that sees nothing (L = -inf) gets P = 0.
  const int64_t ri = lrow + (row_ok ? row : 0);
  float dlt, nl = __builtin_inff();
  {
    float acc = 0.0f;
    if (row_ok) {
      const uint16_t* ob = p.o + b * p.o_bs + (tq + row) * p.o_ss + h * p.o_hs;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(ob + 16 * kk + 8 * kg);
        const f32x8 xf = __builtin_convertvector(__builtin_bit_cast(bf16x8, x), f32x8);
        const f32x8 yf = __builtin_convertvector(doreg[kk], f32x8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(xf[e], yf[e], acc);
      }
    }
    dlt = pair_sum(acc);  // the row's other half of the columns sits in lane ^ 32
    if (row_ok) {
      const float l = p.lse[ri];
      nl = (l == kNegInf) ? __builtin_inff() : l * kLog2e;
      if (kg == 0) {
        p.delta[ri] = dlt;
        p.nlse[ri] = nl;
      }
    }
  }
  // Q, dO, O and L land before the first DMA is issued (left pending, their first
  // use in the loop would wait for the DMA of the blocks ahead too)
  wait_vmcnt<0>();
  LaneMask mask;
  mask.pos = row + (Lk - Lq);
  mask.kend = Lk;
  mask.kbeg = 0;
  mask.causal = p.causal;
  mask.wl = p.wl;
  mask.wr = p.wr;

  // DMA of key block n_lo + i into stage i % NBUF: buffer resources based at the
  // block's first key for a full block (the host keeps 32 token strides below
  // 2^31 bytes), rows clamped to the last key for a final partial one.
  const uint16_t* kb = p.k + b * p.k_bs + tk * p.k_ss + kvh * p.k_hs;
  const uint16_t* vb = p.v + b * p.v_bs + tk * p.v_ss + kvh * p.v_hs;
  const uint32_t k_voff = (uint32_t)(dma_row * p.k_ss + u_src) * 2u;
  const uint32_t v_voff = (uint32_t)(dma_row * p.v_ss + u_src) * 2u;
  const uint32_t k_step = (uint32_t)(G::kRowStep * p.k_ss) * 2u, v_step = (uint32_t)(G::kRowStep * p.v_ss) * 2u;
  auto issue = [&](int i) __attribute__((always_inline)) {
    char* st = smem + (i % NBUF) * kStage + wave * 1024;
    const int n0 = (n_lo + i) * BN;
    if (n0 + BN <= Lk) {
      const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kb + (int64_t)n0 * p.k_ss);
      const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vb + (int64_t)n0 * p.v_ss);
#pragma unroll
      for (int j = 0; j < G::kInstPerWave; ++j) {
        dma16_buf(rk, k_voff, j * k_step, st + j * 4096);
        dma16_buf(rv, v_voff, j * v_step, st + T + j * 4096);
      }
    } else {
      dma_rows<D>(kb, p.k_ss, n0, dma_row, Lk - 1, u_src, st);
      dma_rows<D>(vb, p.v_ss, n0, dma_row, Lk - 1, u_src, st + T);
    }
  };
  constexpr int kPer = 2 * G::kInstPerWave;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};
  for (int j = 0; j < NBUF - 1 && j < nb; ++j) issue(j);
  for (int i = 0; i < nb; ++i) {
    // block i landed (block i + 1 may still be in flight); everyone is done with
    // block i - 1, whose stage the DMA of block i + 2 reuses
    if (i + 1 < nb)
      wait_vmcnt<kPer>();
    else
      wait_vmcnt<0>();
    stage_barrier();
    if (i + NBUF - 1 < nb) issue(i + NBUF - 1);
    const uint32_t st = (uint32_t)((i % NBUF) * kStage);
    uint32_t rows[D / 16];
    uo.rows(st, rows);
    u32x4 ka[D / 16];
    uni_rows<D, 0, 0, D / 16>(rows, ka);
    lgkm_wait<0>(ka);
    f32x16 s = qk_mma<D>(ka, qreg);  // S^T = K Q^T
    uni_rows<D, T, 0, D / 16>(rows, ka);
    lgkm_wait<0>(ka);
    const f32x16 dpt = qk_mma<D>(ka, doreg);  // dP^T = V dO^T
    const int n = n_lo + i;
    if (n < f_lo || n >= f_hi) {
      int base = n * BN + 4 * kg;
      asm volatile("" : "+v"(base));
      // the row's visible keys in the block as an interval of offsets
      const int hi = mask.off_hi(base), lo = mask.off_lo(base);
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int off = 8 * (a >> 2) + (a & 3);
        s[a] = (off <= hi && off >= lo) ? s[a] : kNegInf;
      }
    }
    f32x8 x0, x1;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      float ds;
      if constexpr (SOFTCAP) {
        // the forward's logit cap_out (1 - u), u = 2 / (exp(2 s cap_in) + 1), and
        // its derivative in the scaled score, 1 - tanh^2 = u (2 - u)
        const float u = 2.0f * rcp_fast(exp2_fast(s[a] * cap2) + 1.0f);
        const float la = s[a] == kNegInf ? kNegInf : __builtin_fmaf(-p.cap_out, u, p.cap_out);
        ds = exp2_fast(la - nl) * (dpt[a] - dlt) * (u * (2.0f - u));
      } else {
        ds = exp2_fast(__builtin_fmaf(s[a], c, -nl)) * (dpt[a] - dlt);
      }
      if (a < 8)
        x0[a] = ds;
      else
        x1[a - 8] = ds;
    }
    const bf16x8 d0 = __builtin_convertvector(x0, bf16x8), d1 = __builtin_convertvector(x1, bf16x8);
    // dQ^T += K^T dS^T, K read transposed: keys 0..15 of the block, then 16..31
    uint32_t tlo[D / 32], thi[D / 32];
    uo.trs(st, tlo, thi);
    u32x2 lo0[D / 32], hi0[D / 32], lo1[D / 32], hi1[D / 32];
    uni_tr<D, 0, 0, D / 32>(tlo, thi, lo0, hi0);
    uni_tr<D, 16 * (2 * D), 0, D / 32>(tlo, thi, lo1, hi1);
    lgkm_wait<2 * (D / 32)>(lo0, hi0);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const u32x4 w = {lo0[db].x, lo0[db].y, hi0[db].x, hi0[db].y};
      dq[db] = mfma32(__builtin_bit_cast(bf16x8, w), d0, dq[db]);
    }
    lgkm_wait<0>(lo1, hi1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const u32x4 w = {lo1[db].x, lo1[db].y, hi1[db].x, hi1[db].y};
      dq[db] = mfma32(__builtin_bit_cast(bf16x8, w), d1, dq[db]);
    }
  }
  if (row_ok) {
    uint16_t* ob = p.dq + b * p.dq_bs + (tq + row) * p.dq_ss + h * p.dq_hs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x8 x = {};
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dq[db][4 * q4 + e] * p.scale;
        const u32x4 yb = __builtin_bit_cast(u32x4, __builtin_convertvector(x, bf16x8));
        *reinterpret_cast<u32x2*>(ob + 32 * db + 8 * q4 + 4 * kg) = u32x2{yb.x, yb.y};
      }
  }
}

// dV^T or dK^T += X^T Y for one 32-row tile read transposed (X: the tile at byte
// OFF of the stage registers' base, Y: y0 for its rows 0..15, y1 for rows
// 16..31), in four units of D / 64 d-blocks: unit u reads rows 16 (u / 2) ..
// + 15, half u % 2 of the d-blocks.  Three units are in flight while a fourth
// feeds its products, each in registers of its own.
template <int D, int OFF>
__device__ __forceinline__ void tr_products(const uint32_t (&tlo)[D / 32], const uint32_t (&thi)[D / 32],
                                            f32x16 (&acc)[D / 32], bf16x8 y0, bf16x8 y1) {
  constexpr int UD = D / 64, UR = 2 * UD;
  u32x2 lo[4][UD], hi[4][UD];
  auto rd = [&](auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    uni_tr<D, OFF + (u / 2) * 16 * (2 * D), (u % 2) * UD, UD>(tlo, thi, lo[u], hi[u]);
  };
  auto wt = [&lo, &hi](auto uc, auto nc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value, n = decltype(nc)::value;
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(n));
#pragma unroll
    for (int i = 0; i < UD; ++i) asm volatile("" : "+v"(lo[u][i]), "+v"(hi[u][i]));
  };
  auto mm = [&](auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
#pragma unroll
    for (int i = 0; i < UD; ++i)
      acc[(u % 2) * UD + i] = mfma32(__builtin_bit_cast(bf16x8, u32x4{lo[u][i].x, lo[u][i].y, hi[u][i].x, hi[u][i].y}),
                                     u < 2 ? y0 : y1, acc[(u % 2) * UD + i]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using W2 = std::integral_constant<int, 2 * UR>;
  using W1 = std::integral_constant<int, UR>;
  using W0 = std::integral_constant<int, 0>;
  rd(I0{}), rd(I1{}), rd(I2{});
  wt(I0{}, W2{}), rd(I3{}), mm(I0{});
  wt(I1{}, W2{}), mm(I1{});
  wt(I2{}, W1{}), mm(I2{});
  wt(I3{}, W0{}), mm(I3{});
}

template <int OFF>
__device__ __forceinline__ void ds_write_b128(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF));
}

// dK, dV: one workgroup of eight waves per (batch, KV head, 128-key block).  The
// 128 keys are four slices of 32 (a lane owns a key); each slice has two waves,
// s and s + 4, which the hardware places on one SIMD.  The steps walk, for every
// query head of the KV-head group, the query blocks that see the keys.  Wave s
// (the P wave) holds the slice's K rows; for block t it forms S = Q K^T,
// P = exp(S - L) and dV^T += dO^T P, and hands P (fp32) to the other wave
// through LDS.  Wave s + 4 (the dK wave) holds the slice's V rows and, one step
// behind, forms dP = dO V^T, dS = P (dP - D) and dK^T += Q^T dS.  Each wave
// accumulates one gradient, so the two fit one SIMD's registers and issue in
// each other's gaps, with no product computed twice.  A stage holds the query
// block's Q and dO tiles (unified swizzle) and its 32 L and D values; the P
// waves issue its DMA.
template <int D, bool VARLEN, bool SOFTCAP>
__global__ __launch_bounds__(2 * kThreads, 1) void fa_bwd_dkdv_kernel(FaBwdParams p) {
  constexpr int BM = 32;
  constexpr int NBUF = 4;
  using G = DmaGeom<D, BM>;  // four DMA waves
  constexpr int T = G::kTensorBytes;
  constexpr int kLD = NBUF * 256;        // L and D of each stage: 32 + 32 fp32
  constexpr int kPB = 4 * 1024;          // P of one wave: 64 lanes x 16 fp32
  constexpr int kSt = kLD + 8 * kPB;     // P of two steps x four slices, then the stages
  constexpr int kStage = 2 * T;          // Q tile, dO tile
  static_assert(T + 16 * (2 * D) < 65536, "tile offsets must fit the immediate");
  __shared__ __attribute__((aligned(1024))) char smem[kSt + NBUF * kStage];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, kg = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave & 3;
  const bool pwave = wave < 4;
  const float c = p.scale_log2;
  const float cap2 = p.cap_in * (2.0f * kLog2e);  // softcap: exp(2 s cap_in) = exp2(s cap2)
  UniOffsets<D> uo;
  uo.init(lane, lds_addr(smem) + kSt);
  const int dma_row = slot * G::kRowsPerKiB + lane / G::kChunksPerRow;
  const int u_src = ((lane % G::kChunksPerRow) ^ u_swz<D>(dma_row)) * 8;

  const int64_t pairs = (int64_t)p.B * p.Hkv;
  const int64_t t = blockIdx.x;
  const int kbk = (int)(t / pairs);  // key blocks near the start first (they see the most queries)
  const int b = (int)((t % pairs) / p.Hkv), kvh = (int)((t % pairs) % p.Hkv);
  const int j0 = kbk * 128;
  // the sequence: lengths, token offsets, and where its rows of head h sit in the
  // LSE-row arrays (lbase + h * lhead + row)
  int Lq = p.Nq, Lk = p.Nk;
  int64_t tq = 0, tk = 0, lbase = (int64_t)b * p.Hq * p.Nq, lhead = p.Nq;
  if constexpr (VARLEN) {
    tq = scalar_load_i32(p.cu_q + b);
    Lq = scalar_load_i32(p.cu_q + b + 1) - (int)tq;
    tk = scalar_load_i32(p.cu_k + b);
    Lk = scalar_load_i32(p.cu_k + b + 1) - (int)tk;
    lbase = tq;
    lhead = p.total_q;
    if (j0 >= Lk) return;  // past this sequence's keys (the grid covers the longest)
  }
  int64_t i_lo, i_hi;
  fa_query_range(j0, min(j0 + 128, Lk) - 1, Lq, Lk, p.causal, p.wl, p.wr, &i_lo, &i_hi);
  const int qb_lo = (int)(i_lo / BM);
  const int nqb = i_hi > i_lo ? (int)((i_hi + BM - 1) / BM) - qb_lo : 0;
  const int steps = nqb * p.g;

  const int key = j0 + slot * 32 + col;
  const bool key_ok = key < Lk;
  // the P wave holds the slice's K rows (S = Q K^T), the dK wave its V rows (dP = dO V^T)
  bf16x8 kv[D / 16];
  {
    const uint16_t* src = pwave ? p.k + b * p.k_bs + (tk + (key_ok ? key : 0)) * p.k_ss + kvh * p.k_hs
                                : p.v + b * p.v_bs + (tk + (key_ok ? key : 0)) * p.v_ss + kvh * p.v_hs;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key_ok) x = *reinterpret_cast<const u32x4*>(src + 16 * kk + 8 * kg);
      kv[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // K or V lands before the first DMA is issued.  Left pending into the loop,
  // its first use there would make the compiler wait for every outstanding
  // load at each step, the DMA of the blocks ahead included.
  wait_vmcnt<0>();

  // Step t is query head kvh g + t / nqb, query block qb_lo + t % nqb.  A walk
  // advances over (head, block) one block per step with no division: the DMA's
  // walk runs two steps ahead of the P waves'.
  struct Walk {
    int qblk, q0;               // block index within the head's range, first query row
    int64_t qoff, ooff, loff;   // elements to row q0 of the head in Q, dO and the [B, Hq, Nq] rows
  };
  Walk dw;
  dw.qblk = 0;
  dw.q0 = qb_lo * BM;
  {
    const int h0 = kvh * p.g;
    dw.qoff = b * p.q_bs + (int64_t)h0 * p.q_hs + (tq + dw.q0) * p.q_ss;
    dw.ooff = b * p.do_bs + (int64_t)h0 * p.do_hs + (tq + dw.q0) * p.do_ss;
    dw.loff = lbase + h0 * lhead + dw.q0;
  }
  const int64_t q_blk = (int64_t)BM * p.q_ss, o_blk = (int64_t)BM * p.do_ss;
  const int64_t q_wrap = p.q_hs - (int64_t)nqb * q_blk, o_wrap = p.do_hs - (int64_t)nqb * o_blk;
  const int64_t l_wrap = lhead - (int64_t)nqb * BM;
  auto advance = [&](Walk& w) __attribute__((always_inline)) {
    w.q0 += BM, w.qoff += q_blk, w.ooff += o_blk, w.loff += BM;
    if (++w.qblk == nqb) {
      w.qblk = 0, w.q0 = qb_lo * BM;
      w.qoff += q_wrap, w.ooff += o_wrap, w.loff += l_wrap;
    }
  };
  // DMA of the walk's block into stage buf (by the four P waves).  A full block
  // goes through buffer resources based at its first row, each lane adding a
  // fixed byte offset (the host keeps 32 token strides, and the distance from
  // the D array to the L array, below 2^31 bytes); a final partial block clamps
  // its rows to the last query (the P wave's mask drops what the clamp
  // duplicates).  The block's L (lanes 0..31) and D (lanes 32..63) go to the
  // stage's 256-byte area; every P wave writes the same bytes, so every P wave's
  // count of DMAs per step agrees.
  const uint32_t q_voff = (uint32_t)(dma_row * p.q_ss + u_src) * 2u;
  const uint32_t o_voff = (uint32_t)(dma_row * p.do_ss + u_src) * 2u;
  const uint32_t q_step = (uint32_t)(G::kRowStep * p.q_ss) * 2u, o_step = (uint32_t)(G::kRowStep * p.do_ss) * 2u;
  const uint32_t ld_voff =
      (uint32_t)(kg ? 0 : (reinterpret_cast<const char*>(p.nlse) - reinterpret_cast<const char*>(p.delta))) +
      4u * (uint32_t)col;
  auto issue = [&](const Walk& w, int buf) __attribute__((always_inline)) {
    char* st = smem + kSt + buf * kStage + slot * 1024;
    char* ld = smem + buf * 256;
    if (w.q0 + BM <= Lq) {
      const __amdgpu_buffer_rsrc_t rq = buf_rsrc(p.q + w.qoff);
      const __amdgpu_buffer_rsrc_t ro = buf_rsrc(p.dout + w.ooff);
#pragma unroll
      for (int j = 0; j < G::kInstPerWave; ++j) {
        dma16_buf(rq, q_voff, j * q_step, st + j * 4096);
        dma16_buf(ro, o_voff, j * o_step, st + T + j * 4096);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(p.delta + w.loff), (FA_LDS void*)ld, 4, (int)ld_voff, 0, 0,
                                               0);
    } else {
      const int last = Lq - 1 - w.q0;
      dma_rows<D>(p.q + w.qoff, p.q_ss, 0, dma_row, last, u_src, st);
      dma_rows<D>(p.dout + w.ooff, p.do_ss, 0, dma_row, last, u_src, st + T);
      const int r = col < last ? col : last;
      const float* src = (kg ? p.delta : p.nlse) + w.loff + r;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (FA_LDS void*)ld, 4, 0, 0);
    }
  };
  constexpr int kPer = 2 * G::kInstPerWave + 1;

  // The element mask is needed only where the query block cuts the slice's 32
  // keys or runs past Lq.  Every (query i, key j) of blocks q0 .. q0 + 31 and
  // keys kw .. kw + 31 is visible iff kw + 31 < Lk, q0 + 31 < Lq and, with
  // d = Lk - Lq: causal, kw + 31 <= q0 + d; a right window, kw + 31 <= q0 + d + wr;
  // a left window, kw >= q0 + 31 + d - wl.  So q0 in [fq_lo, fq_hi].
  int fq_lo, fq_hi;
  {
    const int64_t kw = j0 + slot * 32, dd = (int64_t)Lk - Lq;
    int64_t lo = 0, hi = (int64_t)Lq - BM;
    if (p.causal) lo = max(lo, kw + 31 - dd);
    if (p.wr >= 0) lo = max(lo, kw + 31 - dd - p.wr);
    if (p.wl >= 0) hi = min(hi, kw - 31 - dd + p.wl);
    if (kw + 32 > Lk) hi = -1;
    fq_lo = (int)min(lo, (int64_t)0x7fffffff);
    fq_hi = (int)max(hi, (int64_t)-1);
  }

  f32x16 acc[D / 32];  // dV (P wave) or dK (dK wave)
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  const uint32_t ld_base = lds_addr(smem) + 16 * kg;  // L of queries 8 j + 4 kg .. + 3 at + 32 j, D at + 128
  // P of this slice, step parity 0, this lane: 16 fp32 as four 16-byte pieces 1 KiB apart
  const uint32_t p_base = lds_addr(smem) + kLD + slot * kPB + 16 * lane;

  // P wave, block t in stage t % NBUF
  int pq0 = qb_lo * BM, pqblk = 0;  // the P waves' walk (first query row only)
  auto p_step = [&](int t_) __attribute__((always_inline)) {
    const int buf = t_ % NBUF;
    const uint32_t st = (uint32_t)(buf * kStage);
    uint32_t rows[D / 16];
    uo.rows(st, rows);
    u32x4 qa[D / 16];
    uni_rows<D, 0, 0, D / 16>(rows, qa);
    lgkm_wait<0>(qa);
    f32x16 sv = qk_mma<D>(qa, kv);  // S = Q K^T: rows queries, lane column = this key
    const uint32_t ldb = ld_base + (uint32_t)(buf * 256);
    u32x4 lr[4];
    lr[0] = ds_read_b128<0>(ldb);
    lr[1] = ds_read_b128<32>(ldb);
    lr[2] = ds_read_b128<64>(ldb);
    lr[3] = ds_read_b128<96>(ldb);
    if (t_ + 2 < steps) {
      issue(dw, (t_ + 2) % NBUF);
      advance(dw);
    }
    lgkm_wait<0>(lr);
    if (!(pq0 >= fq_lo && pq0 <= fq_hi)) {
      // a score the mask drops becomes -inf, so its P (and dS) is 0
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int qi = pq0 + 8 * (a >> 2) + 4 * kg + (a & 3);
        const int pos = qi + (Lk - Lq);
        const bool vis = key_ok & (qi < Lq) & (!p.causal | (key <= pos)) & ((p.wl < 0) | (key >= pos - p.wl)) &
                         ((p.wr < 0) | (key <= pos + p.wr));
        sv[a] = vis ? sv[a] : kNegInf;
      }
    }
    // P = exp2(s c - L), L in base-2 units (+inf for a row that sees no key, so P = 0);
    // the dK wave gets P, or with softcap P times the transform's derivative
    // 1 - tanh^2 = u (2 - u) (the logit is cap_out (1 - u), u = 2 / (exp(2 s cap_in) + 1))
    f32x16 pa, ph;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const float la = -__uint_as_float(lr[a >> 2][a & 3]);
      if constexpr (SOFTCAP) {
        const float u = 2.0f * rcp_fast(exp2_fast(sv[a] * cap2) + 1.0f);
        const float lg = sv[a] == kNegInf ? kNegInf : __builtin_fmaf(-p.cap_out, u, p.cap_out);
        pa[a] = exp2_fast(lg + la);
        ph[a] = pa[a] * (u * (2.0f - u));
      } else {
        pa[a] = exp2_fast(__builtin_fmaf(sv[a], c, la));
        ph[a] = pa[a];
      }
    }
    const uint32_t pw = p_base + (uint32_t)((t_ & 1) * 4 * kPB);
    ds_write_b128<0>(pw, u32x4{__float_as_uint(ph[0]), __float_as_uint(ph[1]), __float_as_uint(ph[2]),
                               __float_as_uint(ph[3])});
    ds_write_b128<1024>(pw, u32x4{__float_as_uint(ph[4]), __float_as_uint(ph[5]), __float_as_uint(ph[6]),
                                  __float_as_uint(ph[7])});
    ds_write_b128<2048>(pw, u32x4{__float_as_uint(ph[8]), __float_as_uint(ph[9]), __float_as_uint(ph[10]),
                                  __float_as_uint(ph[11])});
    ds_write_b128<3072>(pw, u32x4{__float_as_uint(ph[12]), __float_as_uint(ph[13]), __float_as_uint(ph[14]),
                                  __float_as_uint(ph[15])});
    f32x8 x0, x1;
#pragma unroll
    for (int a = 0; a < 8; ++a) x0[a] = pa[a], x1[a] = pa[8 + a];
    const bf16x8 p0 = __builtin_convertvector(x0, bf16x8), p1 = __builtin_convertvector(x1, bf16x8);
    uint32_t tlo[D / 32], thi[D / 32];
    uo.trs(st, tlo, thi);
    tr_products<D, T>(tlo, thi, acc, p0, p1);  // dV^T += dO^T P, dO read transposed
    pq0 += BM;
    if (++pqblk == nqb) pqblk = 0, pq0 = qb_lo * BM;
  };
  // dK wave, block t (one step behind the P wave) in stage t % NBUF
  auto k_step = [&](int t_) __attribute__((always_inline)) {
    const int buf = t_ % NBUF;
    const uint32_t st = (uint32_t)(buf * kStage);
    uint32_t rows[D / 16];
    uo.rows(st, rows);
    u32x4 oa[D / 16];
    uni_rows<D, T, 0, D / 16>(rows, oa);
    lgkm_wait<0>(oa);
    const f32x16 dp = qk_mma<D>(oa, kv);  // dP = dO V^T
    const uint32_t ldb = ld_base + (uint32_t)(buf * 256);
    const uint32_t pr_ = p_base + (uint32_t)((t_ & 1) * 4 * kPB);
    u32x4 dr[4], pr[4];
    dr[0] = ds_read_b128<128>(ldb);
    dr[1] = ds_read_b128<160>(ldb);
    dr[2] = ds_read_b128<192>(ldb);
    dr[3] = ds_read_b128<224>(ldb);
    pr[0] = ds_read_b128<0>(pr_);
    pr[1] = ds_read_b128<1024>(pr_);
    pr[2] = ds_read_b128<2048>(pr_);
    pr[3] = ds_read_b128<3072>(pr_);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(dr[0]), "+v"(dr[1]), "+v"(dr[2]), "+v"(dr[3]), "+v"(pr[0]),
                 "+v"(pr[1]), "+v"(pr[2]), "+v"(pr[3]));
    f32x8 x0, x1;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const float ds = __uint_as_float(pr[a >> 2][a & 3]) * (dp[a] - __uint_as_float(dr[a >> 2][a & 3]));
      if (a < 8)
        x0[a] = ds;
      else
        x1[a - 8] = ds;
    }
    const bf16x8 d0 = __builtin_convertvector(x0, bf16x8), d1 = __builtin_convertvector(x1, bf16x8);
    uint32_t tlo[D / 32], thi[D / 32];
    uo.trs(st, tlo, thi);
    tr_products<D, 0>(tlo, thi, acc, d0, d1);  // dK^T += Q^T dS, Q read transposed
  };

  // Ring of NBUF = 4 stages.  Iteration t: the P waves process block t (its DMA
  // landed; they issue block t + 2's, whose stage last held block t - 2, read
  // by the dK waves in iteration t - 1) and the dK waves block t - 1 (P written
  // by the P waves in iteration t - 1, before this iteration's barrier).  Every
  // wave passes the same steps + 1 barriers.
  // One loop per role (the same steps + 1 barriers in each): a role branch inside
  // one loop would make the compiler give each role's accumulators their own
  // registers and copy them at the join on every step.
  if (pwave) {
    for (int j = 0; j < 2 && j < steps; ++j) {
      issue(dw, j);
      advance(dw);
    }
    for (int it = 0; it <= steps; ++it) {
      if (it < steps) {
        // block it landed; block it + 1 may still be in flight
        if (it + 1 < steps)
          wait_vmcnt<kPer>();
        else
          wait_vmcnt<0>();
      }
      stage_barrier();
      if (it < steps) p_step(it);
    }
  } else {
    for (int it = 0; it <= steps; ++it) {
      stage_barrier();
      if (it > 0) k_step(it - 1);
    }
  }
  if (key_ok) {
    uint16_t* out = pwave ? p.dv + b * p.dv_bs + (tk + key) * p.dv_ss + kvh * p.dv_hs
                          : p.dk + b * p.dk_bs + (tk + key) * p.dk_ss + kvh * p.dk_hs;
    const float sc = pwave ? 1.0f : p.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x8 x = {};
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * q4 + e] * sc;
        const u32x4 xb = __builtin_bit_cast(u32x4, __builtin_convertvector(x, bf16x8));
        *reinterpret_cast<u32x2*>(out + 32 * db + 8 * q4 + 4 * kg) = u32x2{xb.x, xb.y};
      }
  }
}

// ------------------------------------------------------------------ launch helpers
int device_cus() {
  static thread_local int cached_dev = -1;
  static thread_local int cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached_dev = dev;
    cached_cus = n;
  }
  return cached_cus;
}

template <int D, bool VARLEN, bool PACK, bool SOFTCAP, bool PAGED, bool ALIBI = false, class MOD = FaNoMod>
hipError_t launch_prefill_t(const FaParams& p, hipStream_t stream) {
  auto kern = fa_prefill_kernel<D, VARLEN, PACK, SOFTCAP, PAGED, ALIBI, MOD>;
  const int64_t tiles = p.total_tiles;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool SOFTCAP, bool FP8>
hipError_t launch_paged_t(const FaParams& p, hipStream_t stream) {
  int64_t units = (int64_t)p.B * p.Hkv * p.num_splits;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL((fa_paged_kernel<D, SOFTCAP, FP8>), dim3((unsigned)units), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ no-allocation scratch
// The split-KV partials and the sequence order of fa_fwd_kvcache_paged_noalloc
// live here instead of in a caller workspace, for callers that cannot allocate
// device memory.  Each device holds its own copy until the process ends; every
// call on a device shares that copy, so calls that overlap on one device race.
// Nothing in it needs to start at zero: each call writes every partial and the
// whole order before reading them.
static __device__ __align__(256) char scratch[FA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t fa_scratch_region(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the array's name is a host-side stand-in; kernels get this device address
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int fa_device_cus() { return device_cus(); }

hipError_t fa_launch_prefill(const FaParams& p, int d, bool varlen, bool paged, bool pack, bool softcap,
                             hipStream_t s) {
  // ALiBi: dense, varlen and chunked prefill over a paged cache, without softcap
  if (p.alibi) {
    if (softcap || (paged && varlen)) return hipErrorInvalidValue;
#define FA_AL(D_, V_, P_, G_) \
  if (d == D_ && varlen == V_ && pack == P_ && paged == G_) return launch_prefill_t<D_, V_, P_, false, G_, true>(p, s);
    FA_AL(128, false, false, false) FA_AL(128, false, true, false) FA_AL(128, true, false, false)
    FA_AL(128, true, true, false) FA_AL(64, false, false, false) FA_AL(64, false, true, false)
    FA_AL(64, true, false, false) FA_AL(64, true, true, false)
    FA_AL(128, false, false, true) FA_AL(128, false, true, true) FA_AL(64, false, false, true)
    FA_AL(64, false, true, true)
#undef FA_AL
    return hipErrorInvalidValue;
  }
#define FA_PF(D_, V_, G_, P_, S_)                                                    \
  if (d == D_ && varlen == V_ && paged == G_ && pack == P_ && softcap == S_) \
    return launch_prefill_t<D_, V_, P_, S_, G_>(p, s);
#define FA_PF_D(D_)                                                                                        \
  FA_PF(D_, false, false, false, false) FA_PF(D_, false, false, false, true)                              \
  FA_PF(D_, false, false, true, false) FA_PF(D_, false, false, true, true)                                \
  FA_PF(D_, true, false, false, false) FA_PF(D_, true, false, false, true) FA_PF(D_, true, false, true, false) \
  FA_PF(D_, true, false, true, true) FA_PF(D_, false, true, false, false) FA_PF(D_, false, true, false, true)  \
  FA_PF(D_, false, true, true, false) FA_PF(D_, false, true, true, true)                                  \
  FA_PF(D_, true, true, false, false) FA_PF(D_, true, true, false, true) FA_PF(D_, true, true, true, false)    \
  FA_PF(D_, true, true, true, true)
  FA_PF_D(128) FA_PF_D(64)
#undef FA_PF_D
#undef FA_PF
  return hipErrorInvalidValue;
}

hipError_t fa_launch_unified(const FaParams& pd, const FaParams& pp, int d, bool pack, bool softcap,
                             hipStream_t s) {
  const int64_t nd = (int64_t)pd.B * pd.Hkv * pd.num_splits;
  const int64_t grid = nd + pp.total_tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
#define FA_UN(D_, P_, S_)                                                                                  \
  if (d == D_ && pack == P_ && softcap == S_) {                                                         \
    hipLaunchKernelGGL((fa_unified_kernel<D_, P_, S_>), dim3((unsigned)grid), dim3(kThreads), 0, s, pd, pp, \
                       (int)pp.total_tiles);                                                             \
    return hipGetLastError();                                                                            \
  }
  FA_UN(128, true, false) FA_UN(128, true, true) FA_UN(128, false, false) FA_UN(128, false, true)
  FA_UN(64, true, false) FA_UN(64, true, true) FA_UN(64, false, false) FA_UN(64, false, true)
#undef FA_UN
  return hipErrorInvalidValue;
}

hipError_t fa_launch_prefill_mod(const FaParams& p, int d, bool pack, int mod_id, hipStream_t s) {
#define FA_MOD(M_)                                                                         \
  if (d == 128 && pack) return launch_prefill_t<128, false, true, false, false, false, M_>(p, s);   \
  if (d == 128) return launch_prefill_t<128, false, false, false, false, false, M_>(p, s);          \
  if (d == 64 && pack) return launch_prefill_t<64, false, true, false, false, false, M_>(p, s);     \
  if (d == 64) return launch_prefill_t<64, false, false, false, false, false, M_>(p, s);            \
  return hipErrorInvalidValue;
  if (mod_id == FA_MOD_RELPOS_BIAS) { FA_MOD(FaRelPosBias) }
  if (mod_id == FA_MOD_PREFIX_LM) { FA_MOD(FaPrefixLM) }
#undef FA_MOD
  return hipErrorInvalidValue;
}

hipError_t fa_launch_paged(const FaParams& p, int d, bool softcap, bool fp8, hipStream_t s) {
  if (fp8) {
    if (d == 128) return softcap ? launch_paged_t<128, true, true>(p, s) : launch_paged_t<128, false, true>(p, s);
    if (d == 64) return softcap ? launch_paged_t<64, true, true>(p, s) : launch_paged_t<64, false, true>(p, s);
    return hipErrorInvalidValue;
  }
  if (d == 128) return softcap ? launch_paged_t<128, true, false>(p, s) : launch_paged_t<128, false, false>(p, s);
  if (d == 64) return softcap ? launch_paged_t<64, true, false>(p, s) : launch_paged_t<64, false, false>(p, s);
  return hipErrorInvalidValue;
}

hipError_t fa_launch_seq_order(const int32_t* lens, int B, int32_t* order, hipStream_t s) {
  if (B <= 0 || B > FA_SEQ_ORDER_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fa_seq_order_kernel, dim3((unsigned)((B + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     lens, B, order);
  return hipGetLastError();
}

hipError_t fa_launch_combine(const FaCombineParams& p, int d, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t blocks = (p.rows + (kThreads / 64) - 1) / (kThreads / 64);
  if (d == 128 && !p.in_bf16)
    hipLaunchKernelGGL((fa_combine_kernel<128, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 128)
    hipLaunchKernelGGL((fa_combine_kernel<128, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 64 && !p.in_bf16)
    hipLaunchKernelGGL((fa_combine_kernel<64, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL((fa_combine_kernel<64, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t fa_launch_combine_packed(const FaParams& p, int d, hipStream_t s) {
  const int64_t rows_all = (int64_t)p.B * p.Hkv * FA_PAGED_MAX_ROWS;
  if (rows_all <= 0) return hipSuccess;
  const int64_t blocks = (rows_all + (kThreads / 64) - 1) / (kThreads / 64);
  if (d == 128)
    hipLaunchKernelGGL(fa_combine_packed_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL(fa_combine_packed_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t fa_launch_append(const FaAppendParams& p, int d, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.L * p.Hkv * (d / 8);
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  const int64_t cap = 16 * (int64_t)device_cus();  // grid-stride beyond that
  if (blocks > cap) blocks = cap;
  if (p.fp8 && d == 128)
    hipLaunchKernelGGL(fa_append_fp8_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (p.fp8 && d == 64)
    hipLaunchKernelGGL(fa_append_fp8_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 128)
    hipLaunchKernelGGL(fa_append_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL(fa_append_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t fa_launch_rotary(const FaRotaryParams& p, int d, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.L * p.H * (d / 8);
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  const int64_t cap = 16 * (int64_t)device_cus();
  if (blocks > cap) blocks = cap;
  if (d == 128)
    hipLaunchKernelGGL(fa_rotary_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL(fa_rotary_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t fa_launch_bwd(const FaBwdParams& p, int d, hipStream_t s) {
  // varlen: Nq / Nk are the longest lengths; the workgroups past a sequence's
  // rows or keys return at once
  const int64_t dq_tiles = (int64_t)((p.Nq + 127) / 128) * p.B * p.Hq;
  const int64_t dkv_tiles = (int64_t)((p.Nk + 127) / 128) * p.B * p.Hkv;
  if (dq_tiles > 0x7fffffff || dkv_tiles > 0x7fffffff) return hipErrorInvalidValue;
  if (d != 128 && d != 64) return hipErrorInvalidValue;
  // the dQ kernel also writes D and the base-2 LSE that the dK/dV kernel reads
  const bool vl = p.cu_q != nullptr, sc = p.softcap != 0;
#define FA_BWD(K_, D_, T_, N_)                                                                         \
  if (vl && sc) hipLaunchKernelGGL((K_<D_, true, true>), dim3((unsigned)(T_)), dim3(N_), 0, s, p);      \
  else if (vl) hipLaunchKernelGGL((K_<D_, true, false>), dim3((unsigned)(T_)), dim3(N_), 0, s, p);      \
  else if (sc) hipLaunchKernelGGL((K_<D_, false, true>), dim3((unsigned)(T_)), dim3(N_), 0, s, p);      \
  else hipLaunchKernelGGL((K_<D_, false, false>), dim3((unsigned)(T_)), dim3(N_), 0, s, p);
  if (dq_tiles > 0) {
    if (d == 128) { FA_BWD(fa_bwd_dq_kernel, 128, dq_tiles, kThreads) }
    else { FA_BWD(fa_bwd_dq_kernel, 64, dq_tiles, kThreads) }
  }
  if (dkv_tiles > 0) {
    if (d == 128) { FA_BWD(fa_bwd_dkdv_kernel, 128, dkv_tiles, 2 * kThreads) }
    else { FA_BWD(fa_bwd_dkdv_kernel, 64, dkv_tiles, 2 * kThreads) }
  }
#undef FA_BWD
  return hipGetLastError();
}
