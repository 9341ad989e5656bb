/*
 * oracle.c - fp64 CPU oracle for the exact-attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's compute path may call,
 * link or load this file.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header or table
 * with the HIP path.
 *
 * What it computes is the plain definition of attention, materialised:
 *
 *   For one query row q_i against the keys it may see,
 *     s_j = scale * <q_i, k_j>                      (fp64 dot product)
 *     s_j = c * tanh(s_j / c)          if softcap c > 0
 *     s_j = -inf                       if key j is not visible from row i
 *     m   = max_j s_j
 *     l   = sum_j exp(s_j - m)
 *     P_ij = exp(s_j - m) / l          (the probabilities, materialised)
 *     O_i = sum_j P_ij v_j,  LSE_i = m + ln(l)
 *
 * Sources, cited by page title and section:
 *   - attention definition O = softmax(scale Q K^T) V and the three-pass safe
 *     softmax (max, sum of exponentials, normalise):
 *     "Attention kernels: FlashAttention and PagedAttention", section 2.1.
 *   - the natural-log LSE kept per row for the backward pass:
 *     same page, sections 4.3 and 8.2.
 *   - softcap s' = c * tanh(s / c): "FA4 (CuTeDSL) and engineering interfaces",
 *     section 7 feature table.
 *   - sliding window (left, right): a row at position p sees keys in
 *     [p - left, p + right]: same page, section 7 feature table.
 *   - bottom-right causal alignment (a query is the last tokens of its
 *     sequence): same page, section 6.2; "Attention kernels...", section 5.1.
 *   - varlen packing by cu_seqlens: "FA4 ...", section 4;
 *     "Attention kernels...", section 7.1.
 *   - GQA head map kv_head = q_head / g: "Attention kernels...", sections 5.3
 *     and 8.2.
 *   - paged KV: physical page = block_table[b][t / P], slot t % P:
 *     "Attention kernels...", section 6.1.
 *   - split-KV partials and the merge of partial (O, LSE) states:
 *     "Attention kernels...", section 6.3; "FA4 ...", section 6.2.
 *   - the online (m, l, O) recurrence over key blocks:
 *     "Attention kernels...", sections 2.1 and 3.2.
 *
 * Readings taken where the pages are silent or disagree:
 *   - softcap acts on the scaled logit (scale first, then c*tanh(./c)).
 *   - window bounds are inclusive and a negative bound means unbounded.
 *   - causal alignment is bottom-right everywhere (offset = Lk - Lq); it
 *     equals top-left whenever Lq == Lk.
 *   - a row that sees no key gets O = 0 and LSE = -inf.
 *   - split s of n pages covers pages [s*ceil(n/S), min((s+1)*ceil(n/S), n)).
 *   - partial O is normalised per split; the merge has no epsilon.
 *
 * Inputs are raw bfloat16 bit patterns (uint16); each element is widened
 * exactly to double before any arithmetic.  All arithmetic is fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_VERSION 1

static double bf16_to_double(uint16_t x) {
    uint32_t u = ((uint32_t)x) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Visibility of logical key j from logical query row i of a sequence with
 * Lq queries and Lk keys.  Evaluated for every pair; no block logic. */
static int visible(long i, long j, long Lq, long Lk, int causal, long wl, long wr) {
    long pos = i + (Lk - Lq); /* bottom-right: the query's key-axis position */
    if (j < 0 || j >= Lk) return 0;
    if (causal && j > pos) return 0;
    if (wl >= 0 && j < pos - wl) return 0;
    if (wr >= 0 && j > pos + wr) return 0;
    return 1;
}

/* The definition for one query row.  krows/vrows list the sequence's keys
 * in logical order (nk of them); vis[j] says whether key j is visible.
 * s and p are scratch rows of length nk (the materialised S and P). */
static void attend_row(const uint16_t* q, const uint16_t* const* krows,
                       const uint16_t* const* vrows, const unsigned char* vis,
                       long nk, int d, double scale, double softcap,
                       double* s, double* p, double* o, double* lse) {
    long j;
    int c;
    double m = -INFINITY, l = 0.0;
    for (j = 0; j < nk; ++j) {
        if (!vis[j]) { s[j] = -INFINITY; continue; }
        double dot = 0.0;
        for (c = 0; c < d; ++c) dot += bf16_to_double(q[c]) * bf16_to_double(krows[j][c]);
        double x = scale * dot;
        if (softcap > 0.0) x = softcap * tanh(x / softcap);
        s[j] = x;
    }
    /* pass 1: row maximum */
    for (j = 0; j < nk; ++j) if (s[j] > m) m = s[j];
    for (c = 0; c < d; ++c) o[c] = 0.0;
    if (m == -INFINITY) { *lse = -INFINITY; return; }
    /* pass 2: sum of exponentials */
    for (j = 0; j < nk; ++j) l += (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
    /* pass 3: normalised probabilities, then O = P V */
    for (j = 0; j < nk; ++j) p[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) / l;
    for (j = 0; j < nk; ++j) {
        if (p[j] == 0.0) continue;
        for (c = 0; c < d; ++c) o[c] += p[j] * bf16_to_double(vrows[j][c]);
    }
    *lse = m + log(l);
}

/* ------------------------------------------------------------------------
 * A "problem" describes one call: where each sequence's queries, keys and
 * values live.  Row r (in the caller's output order) is resolved to
 * (sequence b, q head h, query i); the key list of (b, kv head) is built by
 * the oracle's own loops from the layout (dense strides, cu_seqlens, or the
 * block table).
 * ---------------------------------------------------------------------- */
enum { LAYOUT_DENSE = 0, LAYOUT_VARLEN = 1, LAYOUT_PAGED = 2 };

typedef struct {
    int layout;
    const uint16_t *q, *k, *v;
    int B, Hq, Hkv, d;
    long Nq, Nk;                   /* dense: per-sequence lengths; paged: Nq */
    const int32_t *cu_q, *cu_k;    /* varlen */
    long Tq;                       /* varlen: total query rows */
    const int32_t *block_table;    /* paged */
    const int32_t *cache_seqlens;  /* paged */
    long page, max_blocks;
    double scale, softcap;
    int causal;
    long wl, wr;
    /* split mode (paged): num_splits > 0 computes split `split` only */
    int num_splits, split;
} problem;

/* Output row r -> (b, h, i) and the query pointer, plus Lq/Lk. */
static void resolve_row(const problem* P, long r, int* b, int* h, long* i,
                        long* Lq, long* Lk, const uint16_t** qrow) {
    if (P->layout == LAYOUT_DENSE || P->layout == LAYOUT_PAGED) {
        /* r = (b * Hq + h) * Nq + i, the [B, Hq, Nq] LSE order */
        *i = r % P->Nq;
        *h = (int)((r / P->Nq) % P->Hq);
        *b = (int)(r / (P->Nq * P->Hq));
        *Lq = P->Nq;
        *Lk = (P->layout == LAYOUT_DENSE) ? P->Nk : (long)P->cache_seqlens[*b];
        *qrow = P->q + ((((long)*b * P->Nq + *i) * P->Hq) + *h) * P->d;
    } else {
        /* r = h * Tq + t, the [Hq, total_q] LSE order; t -> sequence b */
        long t = r % P->Tq;
        int bb = 0;
        *h = (int)(r / P->Tq);
        while (!(t >= P->cu_q[bb] && t < P->cu_q[bb + 1])) ++bb;
        *b = bb;
        *i = t - P->cu_q[bb];
        *Lq = P->cu_q[bb + 1] - P->cu_q[bb];
        *Lk = P->cu_k[bb + 1] - P->cu_k[bb];
        *qrow = P->q + (t * P->Hq + *h) * P->d;
    }
}

/* Pointer to logical key j of sequence b, kv head kh (K or V tensor). */
static const uint16_t* key_row(const problem* P, const uint16_t* base, int b, int kh, long j) {
    if (P->layout == LAYOUT_DENSE)
        return base + ((((long)b * P->Nk + j) * P->Hkv) + kh) * P->d;
    if (P->layout == LAYOUT_VARLEN)
        return base + (((long)P->cu_k[b] + j) * P->Hkv + kh) * P->d;
    {
        long phys = P->block_table[(long)b * P->max_blocks + j / P->page];
        long slot = j % P->page;
        return base + (((phys * P->page + slot) * P->Hkv) + kh) * P->d;
    }
}

/* Key range [j0, j1) of the current split (paged split mode), else all. */
static void split_range(const problem* P, long Lk, long* j0, long* j1) {
    *j0 = 0; *j1 = Lk;
    if (P->num_splits > 0) {
        long n = (Lk + P->page - 1) / P->page;
        long chunk = (n + P->num_splits - 1) / P->num_splits;
        long p0 = (long)P->split * chunk, p1 = p0 + chunk;
        if (p0 > n) p0 = n;
        if (p1 > n) p1 = n;
        *j0 = p0 * P->page;
        *j1 = p1 * P->page;
        if (*j1 > Lk) *j1 = Lk;
        if (*j0 > *j1) *j0 = *j1;
    }
}

static void compute_row(const problem* P, long r, double* o, double* lse) {
    int b, h;
    long i, Lq, Lk, j, j0, j1;
    const uint16_t* qrow;
    resolve_row(P, r, &b, &h, &i, &Lq, &Lk, &qrow);
    int kh = h / (P->Hq / P->Hkv);
    split_range(P, Lk, &j0, &j1);
    long n = j1 - j0;
    const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
    const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
    unsigned char* vis = (unsigned char*)malloc((size_t)(n > 0 ? n : 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (j = 0; j < n; ++j) {
        kr[j] = key_row(P, P->k, b, kh, j0 + j);
        vr[j] = key_row(P, P->v, b, kh, j0 + j);
        vis[j] = (unsigned char)visible(i, j0 + j, Lq, Lk, P->causal, P->wl, P->wr);
    }
    attend_row(qrow, kr, vr, vis, n, P->d, P->scale, P->softcap, s, p, o, lse);
    free(kr); free(vr); free(vis); free(s); free(p);
}

/* ---------------- threading over independent rows ---------------- */
typedef struct {
    const problem* P;
    const int64_t* rows;
    int64_t nrows, begin, end;
    double *o, *lse;
} work;

static void* worker(void* arg) {
    work* w = (work*)arg;
    int64_t t;
    for (t = w->begin; t < w->end; ++t) {
        long r = w->rows ? (long)w->rows[t] : (long)t;
        compute_row(w->P, r, w->o + (size_t)t * w->P->d, w->lse + t);
    }
    return NULL;
}

static int run_rows(const problem* P, const int64_t* rows, int64_t nrows,
                    double* o, double* lse, int nthreads) {
    int t;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
    pthread_t th[256];
    work w[256];
    for (t = 0; t < nthreads; ++t) {
        w[t].P = P; w[t].rows = rows; w[t].nrows = nrows; w[t].o = o; w[t].lse = lse;
        w[t].begin = nrows * t / nthreads;
        w[t].end = nrows * (t + 1) / nthreads;
        if (pthread_create(&th[t], NULL, worker, &w[t]) != 0) return -1;
    }
    for (t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    return nthreads;
}

/* ---------------- exported entry points ----------------
 * Each computes `nrows` output rows.  rows == NULL means every row, in the
 * natural order given below; otherwise rows[t] names the t-th row to compute.
 * Outputs are compact: o[t * d + c], lse[t].  The return value is the number
 * of threads used (negative on error). */

int oracle_version(void) { return ORACLE_VERSION; }

/* Dense BSHD: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d].  Row order [B, Hq, Nq]. */
int oracle_fwd_dense(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int B, long Nq, long Nk, int Hq, int Hkv, int d,
                     double scale, int causal, long wl, long wr, double softcap,
                     const int64_t* rows, int64_t nrows, double* o, double* lse,
                     int nthreads) {
    problem P;
    memset(&P, 0, sizeof P);
    if (Hkv <= 0 || Hq % Hkv != 0) return -1;
    P.layout = LAYOUT_DENSE; P.q = q; P.k = k; P.v = v;
    P.B = B; P.Hq = Hq; P.Hkv = Hkv; P.d = d; P.Nq = Nq; P.Nk = Nk;
    P.scale = scale; P.softcap = softcap; P.causal = causal; P.wl = wl; P.wr = wr;
    if (!rows) nrows = (int64_t)B * Hq * Nq;
    return run_rows(&P, rows, nrows, o, lse, nthreads);
}

/* Varlen: q [Tq, Hq, d], k/v [Tk, Hkv, d], cu_q/cu_k [B + 1].
 * Row order [Hq, Tq]. */
int oracle_fwd_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* cu_q, const int32_t* cu_k, int B,
                      int Hq, int Hkv, int d,
                      double scale, int causal, long wl, long wr, double softcap,
                      const int64_t* rows, int64_t nrows, double* o, double* lse,
                      int nthreads) {
    problem P;
    memset(&P, 0, sizeof P);
    if (Hkv <= 0 || Hq % Hkv != 0) return -1;
    P.layout = LAYOUT_VARLEN; P.q = q; P.k = k; P.v = v;
    P.B = B; P.Hq = Hq; P.Hkv = Hkv; P.d = d; P.cu_q = cu_q; P.cu_k = cu_k;
    P.Tq = cu_q[B];
    P.scale = scale; P.softcap = softcap; P.causal = causal; P.wl = wl; P.wr = wr;
    if (!rows) nrows = (int64_t)Hq * P.Tq;
    return run_rows(&P, rows, nrows, o, lse, nthreads);
}

/* Paged KV cache: q [B, Nq, Hq, d]; caches [num_pages, page, Hkv, d];
 * block_table [B, max_blocks]; cache_seqlens [B].  Row order [B, Hq, Nq].
 * num_splits == 0: the whole cache.  num_splits > 0: only split `split`,
 * producing that split's normalised O and its LSE. */
int oracle_fwd_paged(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                     const int32_t* block_table, const int32_t* cache_seqlens,
                     int B, long Nq, int Hq, int Hkv, int d, long page, long max_blocks,
                     double scale, int causal, long wl, long wr, double softcap,
                     int num_splits, int split,
                     const int64_t* rows, int64_t nrows, double* o, double* lse,
                     int nthreads) {
    problem P;
    memset(&P, 0, sizeof P);
    if (Hkv <= 0 || Hq % Hkv != 0 || page <= 0) return -1;
    P.layout = LAYOUT_PAGED; P.q = q; P.k = kc; P.v = vc;
    P.B = B; P.Hq = Hq; P.Hkv = Hkv; P.d = d; P.Nq = Nq;
    P.block_table = block_table; P.cache_seqlens = cache_seqlens;
    P.page = page; P.max_blocks = max_blocks;
    P.scale = scale; P.softcap = softcap; P.causal = causal; P.wl = wl; P.wr = wr;
    P.num_splits = num_splits; P.split = split;
    if (!rows) nrows = (int64_t)B * Hq * Nq;
    return run_rows(&P, rows, nrows, o, lse, nthreads);
}

/* Merge S partial states per row ("Attention kernels...", section 6.3):
 *   M = max_s LSE_s;  w_s = exp(LSE_s - M);  LSE = M + ln(sum_s w_s);
 *   O = sum_s (w_s / sum w) O_s.
 * o_part [S, rows, d], lse_part [S, rows]; a row whose every LSE_s is -inf
 * gets O = 0, LSE = -inf. */
void oracle_combine(const double* o_part, const double* lse_part, int S,
                    int64_t rows, int d, double* o, double* lse) {
    int64_t r;
    int s, c;
    for (r = 0; r < rows; ++r) {
        double M = -INFINITY, W = 0.0;
        for (s = 0; s < S; ++s) if (lse_part[(int64_t)s * rows + r] > M) M = lse_part[(int64_t)s * rows + r];
        for (c = 0; c < d; ++c) o[r * d + c] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        for (s = 0; s < S; ++s) {
            double x = lse_part[(int64_t)s * rows + r];
            W += (x == -INFINITY) ? 0.0 : exp(x - M);
        }
        for (s = 0; s < S; ++s) {
            double x = lse_part[(int64_t)s * rows + r];
            double w = (x == -INFINITY) ? 0.0 : exp(x - M) / W;
            if (w == 0.0) continue;
            for (c = 0; c < d; ++c) o[r * d + c] += w * o_part[((int64_t)s * rows + r) * d + c];
        }
        lse[r] = M + log(W);
    }
}

/* The online recurrence over key blocks of `block_n` keys, dense layout
 * ("Attention kernels...", sections 2.1 and 3.2): per block, m_new =
 * max(m, blockmax), alpha = exp(m - m_new), l = alpha l + sum exp(s - m_new),
 * O = alpha O + sum exp(s - m_new) v; at the end O / l, LSE = m + ln l.
 * Row order and outputs as oracle_fwd_dense. */
int oracle_online_dense(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int B, long Nq, long Nk, int Hq, int Hkv, int d,
                        double scale, int causal, long wl, long wr, double softcap,
                        long block_n, const int64_t* rows, int64_t nrows,
                        double* o, double* lse) {
    int64_t t;
    int c;
    if (Hkv <= 0 || Hq % Hkv != 0 || block_n <= 0) return -1;
    if (!rows) nrows = (int64_t)B * Hq * Nq;
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    double* sb = (double*)malloc(sizeof(double) * (size_t)block_n);
    for (t = 0; t < nrows; ++t) {
        long r = rows ? (long)rows[t] : (long)t;
        long i = r % Nq;
        int h = (int)((r / Nq) % Hq);
        int b = (int)(r / (Nq * Hq));
        int kh = h / (Hq / Hkv);
        const uint16_t* qr = q + ((((long)b * Nq + i) * Hq) + h) * d;
        double m = -INFINITY, l = 0.0;
        long j0, j;
        for (c = 0; c < d; ++c) acc[c] = 0.0;
        for (j0 = 0; j0 < Nk; j0 += block_n) {
            long j1 = j0 + block_n < Nk ? j0 + block_n : Nk;
            double bm = -INFINITY;
            for (j = j0; j < j1; ++j) {
                double x = -INFINITY;
                if (visible(i, j, Nq, Nk, causal, wl, wr)) {
                    const uint16_t* kr = k + ((((long)b * Nk + j) * Hkv) + kh) * d;
                    double dot = 0.0;
                    for (c = 0; c < d; ++c) dot += bf16_to_double(qr[c]) * bf16_to_double(kr[c]);
                    x = scale * dot;
                    if (softcap > 0.0) x = softcap * tanh(x / softcap);
                }
                sb[j - j0] = x;
                if (x > bm) bm = x;
            }
            double m_new = m > bm ? m : bm;
            if (m_new == -INFINITY) continue; /* nothing visible yet */
            double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
            l *= alpha;
            for (c = 0; c < d; ++c) acc[c] *= alpha;
            for (j = j0; j < j1; ++j) {
                if (sb[j - j0] == -INFINITY) continue;
                double pj = exp(sb[j - j0] - m_new);
                const uint16_t* vr = v + ((((long)b * Nk + j) * Hkv) + kh) * d;
                l += pj;
                for (c = 0; c < d; ++c) acc[c] += pj * bf16_to_double(vr[c]);
            }
            m = m_new;
        }
        if (m == -INFINITY) {
            for (c = 0; c < d; ++c) o[t * d + c] = 0.0;
            lse[t] = -INFINITY;
        } else {
            for (c = 0; c < d; ++c) o[t * d + c] = acc[c] / l;
            lse[t] = m + log(l);
        }
    }
    free(acc); free(sb);
    return 1;
}

/* The materialised probability row P_i. for one dense row r (length Nk),
 * for the invariant that each non-empty row sums to one. */
int oracle_probs_dense(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       int B, long Nq, long Nk, int Hq, int Hkv, int d,
                       double scale, int causal, long wl, long wr, double softcap,
                       long r, double* p_out) {
    long i = r % Nq, j;
    int h = (int)((r / Nq) % Hq);
    int b = (int)(r / (Nq * Hq));
    int kh;
    double lse;
    if (Hkv <= 0 || Hq % Hkv != 0 || b >= B || Nk <= 0) return -1;
    kh = h / (Hq / Hkv);
    const uint16_t* qr = q + ((((long)b * Nq + i) * Hq) + h) * d;
    const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)Nk);
    const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)Nk);
    unsigned char* vis = (unsigned char*)malloc((size_t)Nk);
    double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    for (j = 0; j < Nk; ++j) {
        kr[j] = k + ((((long)b * Nk + j) * Hkv) + kh) * d;
        vr[j] = v + ((((long)b * Nk + j) * Hkv) + kh) * d;
        vis[j] = (unsigned char)visible(i, j, Nq, Nk, causal, wl, wr);
    }
    attend_row(qr, kr, vr, vis, Nk, d, scale, softcap, s, p_out, o, &lse);
    if (lse == -INFINITY) for (j = 0; j < Nk; ++j) p_out[j] = 0.0;
    free(kr); free(vr); free(vis); free(s); free(o);
    return 0;
}
