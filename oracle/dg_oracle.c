/*
 * dg_oracle.c -- plain CPU fp64 oracle for canvas denoising attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two meet only through the
 * seeded input generator.
 *
 * What it computes (source: "DiffusionGemma Technical Report", paperfeed.app
 * summary page, section "The mechanism: an AR model turned inside out"):
 *
 *  - Canvas step (bidirectional decoder bullet): the 256 canvas positions are
 *    refined with full bidirectional attention inside the canvas while
 *    cross-attending to the KV cache.  For sequence b, query head h, canvas
 *    row i and kv head g = floor(h / G), G = Hq / Hkv, the key set is every
 *    cache row 0..L-1 followed by every canvas row 0..Nc-1, with no mask:
 *        s_j = scale * <q[b,i,h,:], k_j[g,:]>
 *        o   = sum_j exp(s_j - max s) v_j[g,:] / sum_j exp(s_j - max s)
 *
 *  - Commit (causal-encoder bullet and the sentence on freezing a finished
 *    canvas): the frozen block is encoded causally, so block row i sees every
 *    cache row plus block rows 0..i (diagonal included); its K/V rows are then
 *    appended to the cache at rows L..L+Nc-1.  The earlier context is not
 *    re-encoded: cache rows 0..L-1 are left as they are.
 *
 * Precision: every input element is widened exactly to double (bf16, fp32 and
 * e4m3 are subsets of fp64); an e4m3 element is then multiplied by its tensor's
 * scale (the value it stands for).  Scores, exponentials, sums and the weighted
 * sum are all fp64 with libm exp().  Two passes per row: all scores first, then the
 * max-shifted exponentials.  No blocking, no online softmax, no reordering
 * beyond the definition.
 *
 * Layouts (row-major): q and out [B][Nc][Hq][D]; cache K/V [B][cap][Hkv][D];
 * canvas / block K/V [B][Nc][Hkv][D].  prefix_len[b] = L_b, host int32.
 */
#include <math.h>
#include <stdint.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

enum { DGO_BF16 = 0, DGO_F32 = 1, DGO_F64 = 2, DGO_FP8 = 3 };

/*
 * OCP 8-bit floating point, E4M3 variant ("OCP 8-bit Floating Point
 * Specification", E4M3 encoding): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits.  Exponent field 0 holds the subnormals m/8 * 2^-6; the all-ones
 * exponent field is an ordinary binade except mantissa 111, which is NaN (so the
 * largest finite magnitude is 1.75 * 2^8 = 448 and there are no infinities).
 */
static double e4m3_value(uint8_t c) {
  const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* e4m3_value of every byte, filled before the row loops read it. */
static double e4m3_table[256];

static void fill_e4m3_table(void) {
  for (int c = 0; c < 256; c++) e4m3_table[c] = e4m3_value((uint8_t)c);
}

/* Exact widening of one stored element to double. */
static inline __attribute__((always_inline)) double ld(const void* p, int dtype, int64_t i) {
  if (dtype == DGO_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  if (dtype == DGO_F32) return (double)((const float*)p)[i];
  if (dtype == DGO_FP8) return e4m3_table[((const uint8_t*)p)[i]];
  return ((const double*)p)[i];
}

static size_t elem_size(int dtype) {
  return dtype == DGO_FP8 ? 1 : dtype == DGO_BF16 ? 2 : (dtype == DGO_F32 ? 4 : 8);
}

typedef struct {
  int dtype, B, Nc, Hq, Hkv, D;
  double scale;
  const void *q, *k_cache, *v_cache;
  int64_t cap;
  const int32_t* prefix_len;
  const void *k_new, *v_new; /* canvas (step) or block (commit) K/V */
  int causal;                /* 0: canvas step, 1: commit */
  double qs, ks, vs;         /* per-tensor scales of q, K (cache and new) and V: the
                                value of an element is scale * stored value (1 for
                                bf16 / fp32 / fp64 inputs) */
} dgo_args;

/*
 * One output row: query (b, i, h).  `scores` is caller scratch of length
 * >= L + Nc.  Key j < L is cache row j; key j >= L is canvas/block row j - L.
 */
static void attend_row(const dgo_args* a, int b, int i, int h, double* scores, double* out) {
  const int D = a->D, G = a->Hq / a->Hkv, g = h / G;
  const int64_t L = a->prefix_len[b];
  const int64_t n_vis = a->causal ? (int64_t)i + 1 : (int64_t)a->Nc;
  const int64_t n_keys = L + n_vis;
  const int64_t q_off = (((int64_t)b * a->Nc + i) * a->Hq + h) * D;
  /* The tensor scales multiply each stored element; they are applied to the
   * dot product (q and k scales, with the softmax scale) and to the weighted sum
   * of values (v scale), which is the same in exact arithmetic. */
  const double qk_scale = a->qs * a->ks * a->scale;

  /* pass 1: scores and their maximum */
  double m = -INFINITY;
  for (int64_t j = 0; j < n_keys; j++) {
    int64_t k_off;
    const void* kp;
    if (j < L) {
      kp = a->k_cache;
      k_off = (((int64_t)b * a->cap + j) * a->Hkv + g) * D;
    } else {
      kp = a->k_new;
      k_off = (((int64_t)b * a->Nc + (j - L)) * a->Hkv + g) * D;
    }
    double s = 0.0;
    for (int d = 0; d < D; d++) s += ld(a->q, a->dtype, q_off + d) * ld(kp, a->dtype, k_off + d);
    s *= qk_scale;
    scores[j] = s;
    if (s > m) m = s;
  }
  /* pass 2: exponentials, their sum, and the weighted sum of values */
  for (int d = 0; d < D; d++) out[d] = 0.0;
  double l = 0.0;
  for (int64_t j = 0; j < n_keys; j++) {
    const double p = exp(scores[j] - m);
    l += p;
    int64_t v_off;
    const void* vp;
    if (j < L) {
      vp = a->v_cache;
      v_off = (((int64_t)b * a->cap + j) * a->Hkv + g) * D;
    } else {
      vp = a->v_new;
      v_off = (((int64_t)b * a->Nc + (j - L)) * a->Hkv + g) * D;
    }
    for (int d = 0; d < D; d++) out[d] += p * ld(vp, a->dtype, v_off + d);
  }
  for (int d = 0; d < D; d++) out[d] = a->vs * out[d] / l;
}

static int check(const dgo_args* a) {
  if (a->B < 0 || a->Nc <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->D <= 0) return -2;
  if (a->Hq % a->Hkv != 0) return -2;
  if (a->dtype < DGO_BF16 || a->dtype > DGO_FP8) return -3;
  if (!(a->qs > 0) || !(a->ks > 0) || !(a->vs > 0) || isinf(a->qs) || isinf(a->ks) || isinf(a->vs))
    return -2;
  for (int b = 0; b < a->B; b++)
    if (a->prefix_len[b] < 0 || a->prefix_len[b] > a->cap) return -4;
  return 0;
}

/*
 * Runs attend_row over all rows (rows == NULL: out is [B][Nc][Hq][D]) or over
 * the n_rows (b, i, h) triples in `rows` (out is [n_rows][D]).
 */
static int run(const dgo_args* a, int n_rows, const int32_t* rows, double* out) {
  int rc = check(a);
  if (rc) return rc;
  if (a->dtype == DGO_FP8) fill_e4m3_table();
  int64_t max_keys = 0;
  for (int b = 0; b < a->B; b++)
    if (a->prefix_len[b] + a->Nc > max_keys) max_keys = a->prefix_len[b] + a->Nc;
  const int64_t total = rows ? (int64_t)n_rows : (int64_t)a->B * a->Nc * a->Hq;
  if (rows)
    for (int64_t r = 0; r < total; r++)
      if (rows[3 * r] < 0 || rows[3 * r] >= a->B || rows[3 * r + 1] < 0 ||
          rows[3 * r + 1] >= a->Nc || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= a->Hq)
        return -2;
  int failed = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(max_keys > 0 ? max_keys : 1));
    if (!scores) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < total; r++) {
      if (!scores) continue;
      int b, i, h;
      if (rows) {
        b = rows[3 * r];
        i = rows[3 * r + 1];
        h = rows[3 * r + 2];
      } else {
        h = (int)(r % a->Hq);
        i = (int)((r / a->Hq) % a->Nc);
        b = (int)(r / ((int64_t)a->Hq * a->Nc));
      }
      attend_row(a, b, i, h, scores, out + r * a->D);
    }
    free(scores);
  }
  return failed ? -7 : 0;
}

/* Threads the parallel loops above use (the OpenMP default team size). */
int dgo_num_threads(void) { return omp_get_max_threads(); }

/* Threads of the following row loops (n >= 1); timing runs use it for a one-thread figure. */
void dgo_set_num_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
}

/* Canvas step: unmasked attention over [cache rows 0..L-1 ; canvas rows 0..Nc-1].
 * qs, ks, vs: per-tensor scales of the stored q, K and V values. */
int dgo_canvas_attn(int dtype, int B, int Nc, int Hq, int Hkv, int D, double scale,
                    const void* q, const void* k_cache, const void* v_cache, int64_t cap,
                    const int32_t* prefix_len, const void* k_canvas, const void* v_canvas,
                    int n_rows, const int32_t* rows, double* out, double qs, double ks,
                    double vs) {
  dgo_args a = {dtype, B, Nc, Hq, Hkv, D, scale, q, k_cache, v_cache, cap, prefix_len,
                k_canvas, v_canvas, 0, qs, ks, vs};
  return run(&a, n_rows, rows, out);
}

/* Commit attention: block row i sees cache rows 0..L-1 and block rows 0..i. */
int dgo_commit_attn(int dtype, int B, int Nc, int Hq, int Hkv, int D, double scale,
                    const void* q_blk, const void* k_cache, const void* v_cache, int64_t cap,
                    const int32_t* prefix_len, const void* k_blk, const void* v_blk,
                    int n_rows, const int32_t* rows, double* out, double qs, double ks,
                    double vs) {
  dgo_args a = {dtype, B, Nc, Hq, Hkv, D, scale, q_blk, k_cache, v_cache, cap, prefix_len,
                k_blk, v_blk, 1, qs, ks, vs};
  return run(&a, n_rows, rows, out);
}

/*
 * Cache append after a commit: cache rows L_b .. L_b+Nc-1 of sequence b take
 * the block's K/V rows 0..Nc-1, bit for bit; nothing else is written.
 */
int dgo_append_block(int dtype, int B, int Nc, int Hkv, int D, const void* k_blk,
                     const void* v_blk, void* k_cache, void* v_cache, int64_t cap,
                     const int32_t* prefix_len) {
  if (dtype < DGO_BF16 || dtype > DGO_FP8) return -3;
  const size_t es = elem_size(dtype);
  const size_t row = (size_t)Hkv * D * es;
  for (int b = 0; b < B; b++) {
    if (prefix_len[b] < 0 || prefix_len[b] + (int64_t)Nc > cap) return -4;
    for (int i = 0; i < Nc; i++) {
      const size_t src = ((size_t)b * Nc + i) * row;
      const size_t dst = ((size_t)b * cap + prefix_len[b] + i) * row;
      memcpy((char*)k_cache + dst, (const char*)k_blk + src, row);
      memcpy((char*)v_cache + dst, (const char*)v_blk + src, row);
    }
  }
  return 0;
}

/*
 * Partial attention of n_q fp64 query rows (scaled dot products with `scale`)
 * over an explicit fp64 key/value list: returns the running-max triple
 * (m, l, o) with m = max_j s_j, l = sum_j exp(s_j - m), o = sum_j exp(s_j - m) v_j
 * (unnormalised).  An empty key list gives m = -inf, l = 0, o = 0.
 * q [n_q][D], k and v [n_k][D], m and l [n_q], o [n_q][D].
 */
int dgo_partial(int n_q, int n_k, int D, double scale, const double* q, const double* k,
                const double* v, double* m, double* l, double* o) {
  for (int r = 0; r < n_q; r++) {
    double mx = -INFINITY;
    for (int j = 0; j < n_k; j++) {
      double s = 0.0;
      for (int d = 0; d < D; d++) s += q[(int64_t)r * D + d] * k[(int64_t)j * D + d];
      s *= scale;
      if (s > mx) mx = s;
    }
    double sum = 0.0;
    for (int d = 0; d < D; d++) o[(int64_t)r * D + d] = 0.0;
    for (int j = 0; j < n_k; j++) {
      double s = 0.0;
      for (int d = 0; d < D; d++) s += q[(int64_t)r * D + d] * k[(int64_t)j * D + d];
      s *= scale;
      const double p = exp(s - mx);
      sum += p;
      for (int d = 0; d < D; d++) o[(int64_t)r * D + d] += p * v[(int64_t)j * D + d];
    }
    m[r] = mx;
    l[r] = sum;
  }
  return 0;
}

/*
 * Merge of n_parts partial triples for n_q rows into normalised outputs:
 * M = max_s m_s; l = sum_s exp(m_s - M) l_s; out = sum_s exp(m_s - M) o_s / l.
 * Parts with no keys (m = -inf, l = 0) add nothing.  Arrays are
 * m, l [n_parts][n_q] and o [n_parts][n_q][D]; out [n_q][D].
 */
int dgo_merge(int n_parts, int n_q, int D, const double* m, const double* l, const double* o,
              double* out) {
  for (int r = 0; r < n_q; r++) {
    double M = -INFINITY;
    for (int s = 0; s < n_parts; s++)
      if (m[(int64_t)s * n_q + r] > M) M = m[(int64_t)s * n_q + r];
    double lsum = 0.0;
    for (int d = 0; d < D; d++) out[(int64_t)r * D + d] = 0.0;
    if (M == -INFINITY) continue; /* no keys at all: defined as 0 here */
    for (int s = 0; s < n_parts; s++) {
      const double ms = m[(int64_t)s * n_q + r];
      if (ms == -INFINITY) continue;
      const double w = exp(ms - M);
      lsum += w * l[(int64_t)s * n_q + r];
      for (int d = 0; d < D; d++)
        out[(int64_t)r * D + d] += w * o[((int64_t)s * n_q + r) * D + d];
    }
    for (int d = 0; d < D; d++) out[(int64_t)r * D + d] /= lsum;
  }
  return 0;
}
