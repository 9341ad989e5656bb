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
//  * K is stored row-major in LDS with a 16-byte-chunk XOR swizzle so the 32
//    rows a wave reads per MFMA hit distinct banks.  V is stored transposed in
//    4-key groups, [key/4][d][key%4], written from registers after a 4x4 bf16
//    transpose, so the V^T operand is two 8-byte LDS reads per lane.
//  * Workgroup = 4 waves.  Prefill: the waves split the 128 query rows (32
//    each) and share every 64-key stage.  Paged decode: the waves share the
//    (at most 32) packed query rows and split each 128-key stage (32 keys
//    each), merging their partial states through LDS at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_blockinfo.h"
#include "fa_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ------------------------------------------------------------------ LDS tiles
// K: [key][d] bf16, 16-byte chunk c of row r stored at chunk c ^ swz(r).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

template <int D>
__device__ __forceinline__ int k_lds_offset(int r, int chunk) {
  return r * (D * 2) + ((chunk ^ k_swz<D>(r)) << 4);
}

// V^T: element (key, d) at byte ((key / 4) * D + d) * 8 + (key % 4) * 2.
template <int D>
__device__ __forceinline__ int v_lds_offset(int quad, int d) {
  return (quad * D + d) * 8;
}

// Source rows of one K/V stream: dense / varlen (contiguous keys) or paged.
struct KvSource {
  const uint16_t* kb;  // K base: sequence start (dense / varlen) or pool, plus head offset
  const uint16_t* vb;
  int64_t k_ss, v_ss;  // token strides
  int64_t k_ps, v_ps;  // page strides (paged)
  const int32_t* bt;   // block table row (paged), else null
  int page;
  int kend;            // keys >= kend are not loaded (zero-filled)
};

template <bool PAGED>
__device__ __forceinline__ void kv_row_ptrs(const KvSource& s, int key, const uint16_t** kp,
                                            const uint16_t** vp) {
  if (PAGED) {
    int64_t phys = s.bt[key / s.page];
    int64_t slot = key % s.page;
    *kp = s.kb + phys * s.k_ps + slot * s.k_ss;
    *vp = s.vb + phys * s.v_ps + slot * s.v_ss;
  } else {
    *kp = s.kb + (int64_t)key * s.k_ss;
    *vp = s.vb + (int64_t)key * s.v_ss;
  }
}

// Registers staging one stage of NK keys between the global loads and the LDS
// stores (register double buffering: loads for stage n+1 fly while stage n is
// being computed).
template <int D, int NK>
struct Stage {
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kKChunks = NK * kChunksPerRow;
  static constexpr int kKPer = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVBlocks = (NK / 4) * kChunksPerRow;  // 4 keys x 8 d each
  static constexpr int kVPer = (kVBlocks + kThreads - 1) / kThreads;
  u32x4 k[kKPer];
  u32x4 v[kVPer][4];

  template <bool PAGED>
  __device__ __forceinline__ void load(const KvSource& s, int n0, int tid) {
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      int id = tid + i * kThreads;
      int r = id / kChunksPerRow, c = id % kChunksPerRow;
      int key = n0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if ((kKChunks % kThreads == 0 || id < kKChunks) && key < s.kend) {
        const uint16_t *kp, *vp;
        kv_row_ptrs<PAGED>(s, key, &kp, &vp);
        x = *reinterpret_cast<const u32x4*>(kp + c * 8);
      }
      k[i] = x;
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      int id = tid + i * kThreads;
      int quad = id / kChunksPerRow, dg = id % kChunksPerRow;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int key = n0 + quad * 4 + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if ((kVBlocks % kThreads == 0 || id < kVBlocks) && key < s.kend) {
          const uint16_t *kp, *vp;
          kv_row_ptrs<PAGED>(s, key, &kp, &vp);
          x = *reinterpret_cast<const u32x4*>(vp + dg * 8);
        }
        v[i][r] = x;
      }
    }
  }

  __device__ __forceinline__ void store(char* lk, char* lv, int tid) const {
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      int id = tid + i * kThreads;
      if (kKChunks % kThreads != 0 && id >= kKChunks) continue;
      int r = id / kChunksPerRow, c = id % kChunksPerRow;
      *reinterpret_cast<u32x4*>(lk + k_lds_offset<D>(r, c)) = k[i];
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      int id = tid + i * kThreads;
      if (kVBlocks % kThreads != 0 && id >= kVBlocks) continue;
      int quad = id / kChunksPerRow, dg = id % kChunksPerRow;
      // 4 keys x 8 d -> 8 d-rows of 4 keys: dword w of a key row holds d = 8dg+2w (low
      // half) and 8dg+2w+1 (high half).
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t x0 = v[i][0][w], x1 = v[i][1][w], x2 = v[i][2][w], x3 = v[i][3][w];
        u32x4 out;
        out.x = (x0 & 0xffffu) | (x1 << 16);          // d even: keys 0, 1
        out.y = (x2 & 0xffffu) | (x3 << 16);          // d even: keys 2, 3
        out.z = (x0 >> 16) | (x1 & 0xffff0000u);      // d odd:  keys 0, 1
        out.w = (x2 >> 16) | (x3 & 0xffff0000u);      // d odd:  keys 2, 3
        *reinterpret_cast<u32x4*>(lv + v_lds_offset<D>(quad, dg * 8 + 2 * w)) = out;
      }
    }
  }
};

// ------------------------------------------------------------------ per-wave math
// S^T for the 32 keys [32 kb, 32 kb + 32) of the stage against the wave's 32
// query columns.  Lane (j, kg) gets keys 32 kb + 8 (a / 4) + 4 kg + (a % 4).
template <int D>
__device__ __forceinline__ f32x16 qk_block(const char* lk, int kb, const bf16x8* qreg, int lane) {
  f32x16 s = {};
  const int row = kb * 32 + (lane & 31);
  const int kg = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    bf16x8 a = *reinterpret_cast<const bf16x8*>(lk + k_lds_offset<D>(row, 2 * kk + kg));
    s = mfma32(a, qreg[kk], s);
  }
  return s;
}

// O^T += V^T P^T for the 16 keys [16 c, 16 c + 16) of the stage.  pb holds P^T
// for keys 16 c + 8 (slot / 4) + 4 kg + (slot % 4) of this lane's column.
template <int D>
__device__ __forceinline__ void pv_chunk(const char* lv, int c, bf16x8 pb, f32x16* o, int lane) {
  const int kg = lane >> 5, i = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int d = 32 * db + i;
    u32x2 lo = *reinterpret_cast<const u32x2*>(lv + v_lds_offset<D>(4 * c + kg, d));
    u32x2 hi = *reinterpret_cast<const u32x2*>(lv + v_lds_offset<D>(4 * c + 2 + kg, d));
    u32x4 w = {lo.x, lo.y, hi.x, hi.y};
    o[db] = mfma32(__builtin_bit_cast(bf16x8, w), pb, o[db]);
  }
}

__device__ __forceinline__ bf16x8 pack_p(const f32x16& s, int half) {
  f32x8 x;
#pragma unroll
  for (int t = 0; t < 8; ++t) x[t] = s[8 * half + t];
  return __builtin_convertvector(x, bf16x8);
}

// Score transform into the log2 domain: scale (and softcap), then mask.
struct ScoreXf {
  float scale_log2, cap_in, cap_out;
};

template <bool SOFTCAP>
__device__ __forceinline__ float score(float s, const ScoreXf& x) {
  if (SOFTCAP) {
    // c * tanh(scale * s / c) * log2(e), tanh(y) = 1 - 2 / (exp(2y) + 1)
    float y = s * x.cap_in;
    float t = exp2_fast(y * (2.0f * kLog2e));
    float th = 1.0f - 2.0f * rcp_fast(t + 1.0f);
    return th * x.cap_out;
  }
  return s * x.scale_log2;
}

// Per-lane view of the mask: this lane's query position and the bounds.
struct LaneMask {
  int64_t pos;  // key-axis position of this lane's query row
  int kend;     // keys >= kend are invisible (sequence / split end)
  int kbeg;     // keys < kbeg are invisible (split start)
  int causal, wl, wr;
  __device__ __forceinline__ bool visible(int key) const {
    if (key >= kend || key < kbeg) return false;
    if (causal && key > pos) return false;
    if (wl >= 0 && key < pos - wl) return false;
    if (wr >= 0 && key > pos + wr) return false;
    return true;
  }
};

// Online softmax over NB key blocks held in s[] (already in the log2 domain and
// masked).  m_run is the running maximum, l_run this lane's partial row sum.
template <int NB, int D>
__device__ __forceinline__ void online_softmax(f32x16 (&s)[NB], float& m_run, float& l_run,
                                               f32x16* o) {
  float mx = kNegInf;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s[b][a]);
  mx = fmaxf(mx, xor32(mx));
  const float m_new = fmaxf(m_run, mx);
  // a row that has seen no visible key yet keeps m = -inf; use 0 as the offset so
  // that exp2(-inf - offset) = 0 instead of NaN ("Attention kernels...", section 7.3)
  const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
  const float alpha = exp2_fast(m_run - m_use);
  float rs = 0.0f;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      float p = exp2_fast(s[b][a] - m_use);
      s[b][a] = p;
      rs += p;
    }
  l_run = l_run * alpha + rs;
  if (!__all(alpha == 1.0f)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
  }
  m_run = m_new;
}

// ------------------------------------------------------------------ tile scheduling
// Linear tile index -> tile, longest first (row blocks nearer the end of a
// sequence see more keys under a causal mask, so they go first).  Round r of a
// persistent workgroup w takes index r * G + w on even rounds and the mirror
// index within its XCD group on odd rounds, so that the sum of work per
// workgroup stays level.
__device__ __forceinline__ int64_t tile_index(int64_t round, int w, int G) {
  if ((round & 1) == 0) return round * G + w;
  int mirrored = ((G & 7) == 0) ? (G - 8 - (w & ~7)) + (w & 7) : (G - 1 - w);
  return round * G + mirrored;
}

struct TileId {
  int b, hg, mb;
};

// Varlen: number of tiles at levels above m, summed over sequences:
// C(m) = sum_b max(0, M_b - m - 1), M_b = ceil(L_b * gp / BLOCK_M).
__device__ int64_t varlen_tiles_above(const int32_t* cu_q, int B, int gp, int m, int lane) {
  int64_t acc = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    int b = b0 + lane;
    int c = 0;
    if (b < B) {
      int L = cu_q[b + 1] - cu_q[b];
      int M = (L * gp + FA_BLOCK_M - 1) / FA_BLOCK_M;
      c = M - m - 1;
      if (c < 0) c = 0;
    }
    acc += wave_sum(c);
  }
  return acc;
}

// Varlen tile t (levels m = max..0, each level listing (sequence, head group)).
// Returns false when t is past the last tile.
__device__ bool varlen_tile(const FaParams& p, int64_t t, int lane, TileId* out) {
  const int H = p.hg_count;
  // total = H * C(-1)
  int64_t total = (int64_t)H * varlen_tiles_above(p.cu_q, p.B, p.gp, -1, lane);
  if (t >= total) return false;
  int lo = 0, hi = p.m_blocks - 1;
  while (lo < hi) {  // smallest m with H * C(m) <= t
    int mid = (lo + hi) >> 1;
    if ((int64_t)H * varlen_tiles_above(p.cu_q, p.B, p.gp, mid, lane) <= t)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int m = lo;
  int64_t j = t - (int64_t)H * varlen_tiles_above(p.cu_q, p.B, p.gp, m, lane);
  int idx = (int)(j / H);
  out->hg = (int)(j % H);
  out->mb = m;
  out->b = -1;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    int b = b0 + lane;
    bool f = false;
    if (b < p.B) {
      int L = p.cu_q[b + 1] - p.cu_q[b];
      f = (L * p.gp + FA_BLOCK_M - 1) / FA_BLOCK_M > m;
    }
    uint64_t mask = __ballot(f);
    int cnt = __popcll(mask);
    if (idx < cnt) {
      uint64_t below = (lane == 0) ? 0ull : (mask & (~0ull >> (64 - lane)));
      bool mine = f && __popcll(below) == idx;
      uint64_t sel = __ballot(mine);
      out->b = b0 + (__ffsll((long long)sel) - 1);
      break;
    }
    idx -= cnt;
  }
  return out->b >= 0;
}

__device__ __forceinline__ bool dense_tile(const FaParams& p, int64_t t, TileId* out) {
  if (t >= p.total_tiles) return false;
  const int64_t per_level = (int64_t)p.B * p.hg_count;
  const int level = (int)(t / per_level);
  const int64_t bh = t % per_level;
  out->mb = p.m_blocks - 1 - level;
  out->b = (int)(bh / p.hg_count);
  out->hg = (int)(bh % p.hg_count);
  return true;
}

// ------------------------------------------------------------------ prefill kernel
template <int D, bool VARLEN, bool PACK, bool SOFTCAP>
__global__ __launch_bounds__(kThreads) void fa_prefill_kernel(FaParams p) {
  constexpr int BN = FA_BLOCK_N;
  constexpr int kStageBytes = BN * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kStageBytes];
  // stage buffer `buf` holds K at smem + 2 * buf * kStageBytes and V right after it
  auto lk = [&](int buf) { return smem + 2 * buf * kStageBytes; };
  auto lv = [&](int buf) { return smem + (2 * buf + 1) * kStageBytes; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int kg = lane >> 5;
  const ScoreXf xf = {p.scale_log2, p.cap_in, p.cap_out};

  const int G = gridDim.x;
  for (int64_t round = 0;; ++round) {
    const int64_t t = p.persistent ? tile_index(round, blockIdx.x, G) : (round == 0 ? (int64_t)blockIdx.x : -1);
    if (t < 0) break;
    TileId tile;
    if (VARLEN) {
      if (!varlen_tile(p, t, lane, &tile)) break;
    } else {
      if (!dense_tile(p, t, &tile)) break;
    }

    // ---- sequence view
    int64_t q_start = 0, k_start = 0;
    int Lq = p.Nq, Lk = p.Nk;
    if (VARLEN) {
      q_start = p.cu_q[tile.b];
      Lq = p.cu_q[tile.b + 1] - (int)q_start;
      k_start = p.cu_k[tile.b];
      Lk = p.cu_k[tile.b + 1] - (int)k_start;
    }
    const int kvh = PACK ? tile.hg : tile.hg / p.g;
    const int rows = Lq * p.gp;
    const int m0 = tile.mb * FA_BLOCK_M;
    const int m_end = min(m0 + FA_BLOCK_M, rows);
    FaRowSpan span;
    span.pos_lo = (int64_t)(m0 / p.gp) + (Lk - Lq);
    span.pos_hi = (int64_t)((m_end - 1) / p.gp) + (Lk - Lq);
    int n_lo, n_hi;
    fa_key_tiles(span, Lk, p.causal, p.wl, p.wr, BN, &n_lo, &n_hi);

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
    mask.pos = (int64_t)tok + (Lk - Lq);
    mask.kend = Lk;
    mask.kbeg = 0;
    mask.causal = p.causal;
    mask.wl = p.wl;
    mask.wr = p.wr;

    KvSource src;
    src.kb = p.k + (int64_t)tile.b * p.k_bs + k_start * p.k_ss + (int64_t)kvh * p.k_hs;
    src.vb = p.v + (int64_t)tile.b * p.v_bs + k_start * p.v_ss + (int64_t)kvh * p.v_hs;
    src.k_ss = p.k_ss;
    src.v_ss = p.v_ss;
    src.k_ps = 0;
    src.v_ps = 0;
    src.bt = nullptr;
    src.page = 1;
    src.kend = Lk;

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;

    Stage<D, BN> st;
    if (n_lo < n_hi) {
      st.template load<false>(src, n_lo * BN, tid);
      st.store(lk(0), lv(0), tid);
      __syncthreads();
    }
    for (int n = n_lo; n < n_hi; ++n) {
      const int buf = (n - n_lo) & 1;
      const bool more = n + 1 < n_hi;
      if (more) st.template load<false>(src, (n + 1) * BN, tid);

      f32x16 s[2];
      s[0] = qk_block<D>(lk(buf), 0, qreg, lane);
      s[1] = qk_block<D>(lk(buf), 1, qreg, lane);
      const int cls = fa_tile_class(span, Lk, p.causal, p.wl, p.wr, BN, n);
      if (cls & (FA_TILE_MASK_LEFT | FA_TILE_MASK_RIGHT)) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int key = n * BN + 32 * b + 8 * (a >> 2) + 4 * kg + (a & 3);
            s[b][a] = mask.visible(key) ? score<SOFTCAP>(s[b][a], xf) : kNegInf;
          }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int a = 0; a < 16; ++a) s[b][a] = score<SOFTCAP>(s[b][a], xf);
      }
      online_softmax<2, D>(s, m_run, l_run, o);
#pragma unroll
      for (int c = 0; c < 4; ++c) pv_chunk<D>(lv(buf), c, pack_p(s[c >> 1], c & 1), o, lane);

      if (more) st.store(lk(buf ^ 1), lv(buf ^ 1), tid);
      __syncthreads();
    }

    // ---- epilogue: O / l and LSE = (m + log2 l) ln 2
    const float l_tot = l_run + xor32(l_run);
    const bool empty = (m_run == kNegInf) || !(l_tot > 0.0f);
    const float inv = empty ? 0.0f : rcp_fast(l_tot);
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
        const float lse = empty ? kNegInf : (m_run + log2_fast(l_tot)) * kLn2;
        p.lse[(int64_t)tile.b * p.lse_bs + (int64_t)head * p.lse_hs + q_start + tok] = lse;
      }
    }
    if (!p.persistent) break;
  }
}

// ------------------------------------------------------------------ paged split-KV kernel
// One workgroup per (sequence b, KV head, split).  The packed query rows
// (seqlen_q tokens x g heads, at most 32) are the same for all four waves; each
// 128-key stage is split 32 keys per wave, and the waves' partial states are
// merged through LDS at the end ("Attention kernels...", section 6.3: partial
// states combine with the same rescale as the tiles).
template <int D, bool SOFTCAP>
__global__ __launch_bounds__(kThreads) void fa_paged_kernel(FaParams p) {
  constexpr int NK = FA_PAGED_STAGE;
  constexpr int kStageBytes = NK * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kStageBytes];
  // stage buffer `buf` holds K at smem + 2 * buf * kStageBytes and V right after it
  auto lk = [&](int buf) { return smem + 2 * buf * kStageBytes; };
  auto lv = [&](int buf) { return smem + (2 * buf + 1) * kStageBytes; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int kg = lane >> 5;
  const ScoreXf xf = {p.scale_log2, p.cap_in, p.cap_out};

  const int S = p.num_splits;
  const int unit = blockIdx.x;
  const int b = unit / (p.Hkv * S);
  const int kvh = (unit / S) % p.Hkv;
  const int split = unit % S;

  const int Lk = p.cache_seqlens[b];
  const int Lq = p.Nq;
  const int rows = Lq * p.g;
  const int npages = (Lk + p.page - 1) / p.page;
  const int chunk = (npages + S - 1) / S;
  const int p0 = min(split * chunk, npages), p1 = min(p0 + chunk, npages);
  const int k_lo = p0 * p.page;
  const int k_hi = min(p1 * p.page, Lk);

  // rows' key-range, intersected with this split
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
  // stages start on a page boundary of the split so a stage never crosses splits
  const int st_first = (int)(kb0 > k_lo ? k_lo + ((kb0 - k_lo) / NK) * NK : k_lo);
  const int nst = kb1 > kb0 ? (int)((kb1 - st_first + NK - 1) / NK) : 0;

  const bool row_ok = col < rows;
  const int tok = row_ok ? col / p.g : 0;
  const int head = kvh * p.g + (row_ok ? col % p.g : 0);
  const uint16_t* qb = p.q + (int64_t)b * p.q_bs + (int64_t)tok * p.q_ss + (int64_t)head * p.q_hs;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row_ok) x = *reinterpret_cast<const u32x4*>(qb + 16 * kk + 8 * kg);
    qreg[kk] = __builtin_bit_cast(bf16x8, x);
  }
  LaneMask mask;
  mask.pos = (int64_t)tok + (Lk - Lq);
  mask.kend = (int)kb1;
  mask.kbeg = (int)kb0;
  mask.causal = p.causal;
  mask.wl = p.wl;
  mask.wr = p.wr;

  KvSource src;
  src.kb = p.k + (int64_t)kvh * p.k_hs;
  src.vb = p.v + (int64_t)kvh * p.v_hs;
  src.k_ss = p.k_ss;
  src.v_ss = p.v_ss;
  src.k_ps = p.k_bs;
  src.v_ps = p.v_bs;
  src.bt = p.block_table + (int64_t)b * p.max_blocks;
  src.page = p.page;
  src.kend = (int)kb1;

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  Stage<D, NK> st;
  if (nst > 0) {
    st.template load<true>(src, st_first, tid);
    st.store(lk(0), lv(0), tid);
    __syncthreads();
  }
  for (int i = 0; i < nst; ++i) {
    const int buf = i & 1;
    const bool more = i + 1 < nst;
    const int n0 = st_first + i * NK;
    if (more) st.template load<true>(src, n0 + NK, tid);

    f32x16 s[1];
    s[0] = qk_block<D>(lk(buf), wave, qreg, lane);
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int key = n0 + 32 * wave + 8 * (a >> 2) + 4 * kg + (a & 3);
      s[0][a] = mask.visible(key) ? score<SOFTCAP>(s[0][a], xf) : kNegInf;
    }
    online_softmax<1, D>(s, m_run, l_run, o);
    pv_chunk<D>(lv(buf), 2 * wave, pack_p(s[0], 0), o, lane);
    pv_chunk<D>(lv(buf), 2 * wave + 1, pack_p(s[0], 1), o, lane);

    if (more) st.store(lk(buf ^ 1), lv(buf ^ 1), tid);
    __syncthreads();
  }

  // ---- merge the four waves' states through LDS
  float* mo = reinterpret_cast<float*>(smem);               // [4][32 cols][D]
  float* ml = mo + 4 * 32 * D;                              // [4][32] m, then [4][32] l
  const float l_w = l_run + xor32(l_run);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int d = 32 * db + 8 * (a >> 2) + 4 * kg + (a & 3);
      mo[(wave * 32 + col) * D + d] = o[db][a];
    }
  if (kg == 0) {
    ml[wave * 32 + col] = m_run;
    ml[128 + wave * 32 + col] = l_w;
  }
  __syncthreads();

  // thread -> (column, 16 consecutive d values)
  constexpr int kParts = D / 16;             // 8 for D = 128, 4 for D = 64
  constexpr int kCols = kThreads / kParts;   // 32 for D = 128, 64 for D = 64
  const int c = tid / kParts;
  const int d0 = (tid % kParts) * 16;
  if (kCols >= 32 ? c < 32 : true) {
    if (c < rows) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[w * 32 + c]);
      float e[4], L = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = ml[w * 32 + c];
        e[w] = (mw == kNegInf) ? 0.0f : exp2_fast(mw - M);
        L += e[w] * ml[128 + w * 32 + c];
      }
      const bool empty = (M == kNegInf) || !(L > 0.0f);
      const float inv = empty ? 0.0f : rcp_fast(L);
      float acc[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sum += e[w] * mo[(w * 32 + c) * D + d0 + x];
        acc[x] = sum * inv;
      }
      const float lse = empty ? kNegInf : (M + log2_fast(L)) * kLn2;
      const int ctok = c / p.g;
      const int chead = kvh * p.g + c % p.g;
      const int64_t r = ((int64_t)b * p.Hq + chead) * Lq + ctok;  // LSE row order
      if (S == 1) {
        uint16_t* ob = p.o + (int64_t)b * p.o_bs + (int64_t)ctok * p.o_ss + (int64_t)chead * p.o_hs + d0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x8 x;
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) x[e2] = acc[8 * h + e2];
          *reinterpret_cast<bf16x8*>(ob + 8 * h) = __builtin_convertvector(x, bf16x8);
        }
        if (d0 == 0 && p.lse) p.lse[r] = lse;
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
}

// ------------------------------------------------------------------ combine kernel
// One wave per row: M = max_s LSE_s, w_s = exp(LSE_s - M), LSE = M + ln sum w_s,
// O = sum_s w_s O_s / sum w_s ("Attention kernels...", section 6.3).
template <int D>
__global__ __launch_bounds__(kThreads) void fa_combine_kernel(FaCombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const int S = p.num_splits;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, p.lse_part[(int64_t)s * p.rows + r]);
  constexpr int E = D / 64;  // elements per lane
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  float W = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float x = p.lse_part[(int64_t)s * p.rows + r];
      const float w = (x == kNegInf) ? 0.0f : exp2_fast((x - M) * kLog2e);
      W += w;
      const float* op = p.o_part + ((int64_t)s * p.rows + r) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * op[e];
    }
  }
  const bool empty = (M == kNegInf) || !(W > 0.0f);
  const float inv = empty ? 0.0f : rcp_fast(W);
  const int t = (int)(r % p.Nq);
  const int h = (int)((r / p.Nq) % p.Hq);
  const int64_t b = r / ((int64_t)p.Nq * p.Hq);
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
  if (lane == 0 && p.lse) p.lse[r] = empty ? kNegInf : M + __builtin_logf(W);
}

// ------------------------------------------------------------------ launch helpers
struct DeviceInfo {
  int cus = 0;
};

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

template <typename K>
int occupancy(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess || n <= 0)
    n = 1;
  return n;
}

template <int D, bool VARLEN, bool PACK, bool SOFTCAP>
hipError_t launch_prefill_t(const FaParams& p0, hipStream_t stream) {
  FaParams p = p0;
  auto kern = fa_prefill_kernel<D, VARLEN, PACK, SOFTCAP>;
  int64_t tiles = p.total_tiles;
  if (tiles <= 0) return hipSuccess;
  int64_t grid;
  if (VARLEN || p.persistent) {
    static thread_local int occ = 0;
    if (occ == 0) occ = occupancy(kern);
    int64_t G = (int64_t)device_cus() * occ;
    grid = tiles < G ? tiles : G;
    p.persistent = 1;
  } else {
    grid = tiles;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool SOFTCAP>
hipError_t launch_paged_t(const FaParams& p, hipStream_t stream) {
  int64_t units = (int64_t)p.B * p.Hkv * p.num_splits;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL((fa_paged_kernel<D, SOFTCAP>), dim3((unsigned)units), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t fa_launch_prefill(const FaParams& p, int d, bool varlen, bool pack, bool softcap,
                             hipStream_t s) {
#define FA_PF(D_, V_, P_, S_) \
  if (d == D_ && varlen == V_ && pack == P_ && softcap == S_) return launch_prefill_t<D_, V_, P_, S_>(p, s);
  FA_PF(128, false, false, false) FA_PF(128, false, false, true) FA_PF(128, false, true, false)
  FA_PF(128, false, true, true) FA_PF(128, true, false, false) FA_PF(128, true, false, true)
  FA_PF(128, true, true, false) FA_PF(128, true, true, true)
  FA_PF(64, false, false, false) FA_PF(64, false, false, true) FA_PF(64, false, true, false)
  FA_PF(64, false, true, true) FA_PF(64, true, false, false) FA_PF(64, true, false, true)
  FA_PF(64, true, true, false) FA_PF(64, true, true, true)
#undef FA_PF
  return hipErrorInvalidValue;
}

hipError_t fa_launch_paged(const FaParams& p, int d, bool softcap, hipStream_t s) {
  if (d == 128) return softcap ? launch_paged_t<128, true>(p, s) : launch_paged_t<128, false>(p, s);
  if (d == 64) return softcap ? launch_paged_t<64, true>(p, s) : launch_paged_t<64, false>(p, s);
  return hipErrorInvalidValue;
}

hipError_t fa_launch_combine(const FaCombineParams& p, int d, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t blocks = (p.rows + (kThreads / 64) - 1) / (kThreads / 64);
  if (d == 128)
    hipLaunchKernelGGL(fa_combine_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL(fa_combine_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
