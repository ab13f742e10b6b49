/*
 * oracle_sanitized.c -- runs every entry point of the CPU oracle (oracle/dg_oracle.c)
 * on small edge-case shapes, built with -fsanitize=address,undefined by
 * tests/test_oracle_sanitized.py.  Every buffer is allocated at exactly the size
 * its layout needs, so a read or write past a tensor's end is caught.
 *
 * Shapes: ragged batches with prefixes 0, 1 and a cache filled to its capacity,
 * grouped-query head ratios 1, 2 and 4, head_dim 8 and 16, every storage format
 * (bf16, fp32, fp64, e4m3), the full output and a row subset, the commit with its
 * append, partial attention over no keys, and a merge with an empty part.
 * Values are checked for finiteness, the row subset against the full output, and
 * the merge of a split key list against partial attention over the whole list.
 * Prints one line and exits 0, or reports the first failure and exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int dgo_canvas_attn(int dtype, int B, int Nc, int Hq, int Hkv, int D, double scale,
                    const void* q, const void* k_cache, const void* v_cache, int64_t cap,
                    const int32_t* prefix_len, const void* k_canvas, const void* v_canvas,
                    int n_rows, const int32_t* rows, double* out, double qs, double ks,
                    double vs);
int dgo_commit_attn(int dtype, int B, int Nc, int Hq, int Hkv, int D, double scale,
                    const void* q_blk, const void* k_cache, const void* v_cache, int64_t cap,
                    const int32_t* prefix_len, const void* k_blk, const void* v_blk,
                    int n_rows, const int32_t* rows, double* out, double qs, double ks,
                    double vs);
int dgo_append_block(int dtype, int B, int Nc, int Hkv, int D, const void* k_blk,
                     const void* v_blk, void* k_cache, void* v_cache, int64_t cap,
                     const int32_t* prefix_len);
int dgo_partial(int n_q, int n_k, int D, double scale, const double* q, const double* k,
                const double* v, double* m, double* l, double* o);
int dgo_merge(int n_parts, int n_q, int D, const double* m, const double* l, const double* o,
              double* out);

#define FAIL(...)                                   \
  do {                                              \
    fprintf(stderr, "FAIL line %d: ", __LINE__);    \
    fprintf(stderr, __VA_ARGS__);                   \
    fprintf(stderr, "\n");                          \
    exit(1);                                        \
  } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 11);
}
static double uniform(void) { return (next_u32() & 0xffffff) / 16777216.0 * 2.0 - 1.0; }

static size_t esize(int dtype) { return dtype == 0 ? 2 : dtype == 1 ? 4 : dtype == 2 ? 8 : 1; }

/* n random finite elements of the format (exactly n * esize bytes) */
static void* random_tensor(int dtype, size_t n) {
  void* p = malloc(n * esize(dtype) + (n == 0));
  if (!p) FAIL("out of memory");
  for (size_t i = 0; i < n; i++) {
    const double x = uniform();
    if (dtype == 0) {
      const float f = (float)x;
      uint32_t u;
      memcpy(&u, &f, 4);
      ((uint16_t*)p)[i] = (uint16_t)(u >> 16);
    } else if (dtype == 1) {
      ((float*)p)[i] = (float)x;
    } else if (dtype == 2) {
      ((double*)p)[i] = x;
    } else {
      uint8_t c = (uint8_t)next_u32();
      if ((c & 0x7f) == 0x7f) c ^= 1; /* not NaN */
      ((uint8_t*)p)[i] = c;
    }
  }
  return p;
}

static void check_finite(const double* x, size_t n, const char* what) {
  for (size_t i = 0; i < n; i++)
    if (!isfinite(x[i])) FAIL("%s: element %zu is %g", what, i, x[i]);
}

static int n_calls = 0;

static void attention_case(int dtype, int B, int Nc, int Hq, int Hkv, int D, const int32_t* L,
                           int64_t cap_extra) {
  int64_t cap = 0;
  for (int b = 0; b < B; b++)
    if (L[b] > cap) cap = L[b];
  cap += cap_extra;
  const size_t nq = (size_t)B * Nc * Hq * D, nkv = (size_t)B * Nc * Hkv * D;
  const size_t ncache = (size_t)B * (size_t)cap * Hkv * D;
  void* q = random_tensor(dtype, nq);
  void* kn = random_tensor(dtype, nkv);
  void* vn = random_tensor(dtype, nkv);
  void* kc = random_tensor(dtype, ncache);
  void* vc = random_tensor(dtype, ncache);
  double* out = (double*)malloc(sizeof(double) * nq);
  double* sub = (double*)malloc(sizeof(double) * 3 * (size_t)D);
  const double s = 1.0 / sqrt((double)D), qs = dtype == 3 ? 0.5 : 1.0, ks = dtype == 3 ? 2.0 : 1.0;
  int32_t rows[9] = {0, 0, 0, B - 1, Nc - 1, Hq - 1, B / 2, Nc / 2, Hq / 2};
  for (int commit = 0; commit < 2; commit++) {
    int rc = commit ? dgo_commit_attn(dtype, B, Nc, Hq, Hkv, D, s, q, kc, vc, cap, L, kn, vn, 0,
                                      NULL, out, qs, ks, 1.0)
                    : dgo_canvas_attn(dtype, B, Nc, Hq, Hkv, D, s, q, kc, vc, cap, L, kn, vn, 0,
                                      NULL, out, qs, ks, 1.0);
    if (rc) FAIL("attention (commit %d, dtype %d) returned %d", commit, dtype, rc);
    check_finite(out, nq, "attention output");
    rc = commit ? dgo_commit_attn(dtype, B, Nc, Hq, Hkv, D, s, q, kc, vc, cap, L, kn, vn, 3, rows,
                                  sub, qs, ks, 1.0)
                : dgo_canvas_attn(dtype, B, Nc, Hq, Hkv, D, s, q, kc, vc, cap, L, kn, vn, 3, rows,
                                  sub, qs, ks, 1.0);
    if (rc) FAIL("row subset returned %d", rc);
    for (int r = 0; r < 3; r++) {
      const int b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
      const double* full = out + (((size_t)b * Nc + i) * Hq + h) * D;
      for (int d = 0; d < D; d++)
        if (sub[r * D + d] != full[d]) FAIL("row subset differs from the full output");
    }
    n_calls += 2;
  }
  /* the append: a cache of capacity max(L) + Nc takes the block at rows L_b.. */
  if (cap_extra >= Nc) {
    if (dgo_append_block(dtype, B, Nc, Hkv, D, kn, vn, kc, vc, cap, L))
      FAIL("append returned an error");
    const size_t row = (size_t)Hkv * D * esize(dtype);
    for (int b = 0; b < B; b++)
      for (int i = 0; i < Nc; i++)
        if (memcmp((char*)kc + ((size_t)b * cap + L[b] + i) * row, (char*)kn + ((size_t)b * Nc + i) * row,
                   row))
          FAIL("appended row differs");
    n_calls++;
  } else {
    /* the append needs L + Nc <= cap: refused without a write */
    int32_t Lbig[8];
    for (int b = 0; b < B; b++) Lbig[b] = (int32_t)cap;
    if (dgo_append_block(dtype, B, Nc, Hkv, D, kn, vn, kc, vc, cap, Lbig) != -4)
      FAIL("append past the capacity was not refused");
  }
  free(q);
  free(kn);
  free(vn);
  free(kc);
  free(vc);
  free(out);
  free(sub);
}

static void merge_case(int n_q, int D, int n_k, int n_split) {
  double* q = (double*)malloc(sizeof(double) * n_q * D);
  double* k = (double*)malloc(sizeof(double) * (n_k ? n_k : 1) * D);
  double* v = (double*)malloc(sizeof(double) * (n_k ? n_k : 1) * D);
  for (int i = 0; i < n_q * D; i++) q[i] = uniform();
  for (int i = 0; i < n_k * D; i++) {
    k[i] = uniform();
    v[i] = uniform();
  }
  /* parts: n_split pieces of the key list (the first empty), then merged */
  const int parts = n_split + 1;
  double* m = (double*)malloc(sizeof(double) * parts * n_q);
  double* l = (double*)malloc(sizeof(double) * parts * n_q);
  double* o = (double*)malloc(sizeof(double) * parts * n_q * D);
  double* out = (double*)malloc(sizeof(double) * n_q * D);
  double* ref = (double*)malloc(sizeof(double) * n_q * D);
  double* mr = (double*)malloc(sizeof(double) * n_q);
  double* lr = (double*)malloc(sizeof(double) * n_q);
  const double scale = 0.5;
  if (dgo_partial(n_q, 0, D, scale, q, k, v, m, l, o)) FAIL("empty partial");
  for (int r = 0; r < n_q; r++)
    if (m[r] != -INFINITY || l[r] != 0.0) FAIL("an empty partial must be (-inf, 0)");
  int j0 = 0;
  for (int p = 1; p < parts; p++) {
    const int j1 = n_k * p / n_split;
    if (dgo_partial(n_q, j1 - j0, D, scale, q, k + (size_t)j0 * D, v + (size_t)j0 * D,
                    m + (size_t)p * n_q, l + (size_t)p * n_q, o + (size_t)p * n_q * D))
      FAIL("partial");
    j0 = j1;
  }
  if (dgo_merge(parts, n_q, D, m, l, o, out)) FAIL("merge");
  if (dgo_partial(n_q, n_k, D, scale, q, k, v, mr, lr, ref)) FAIL("whole partial");
  for (int r = 0; r < n_q; r++)
    for (int d = 0; d < D; d++) {
      const double want = ref[r * D + d] / lr[r];
      if (fabs(out[r * D + d] - want) > 1e-12 * (1.0 + fabs(want)))
        FAIL("merge of %d parts differs from the whole: %g against %g", parts, out[r * D + d], want);
    }
  check_finite(out, (size_t)n_q * D, "merge output");
  n_calls += parts + 2;
  free(q);
  free(k);
  free(v);
  free(m);
  free(l);
  free(o);
  free(out);
  free(ref);
  free(mr);
  free(lr);
}

int main(void) {
  const int32_t L3[3] = {0, 1, 37};
  const int32_t L1[1] = {64};
  const int32_t L2[2] = {5, 0};
  for (int dtype = 0; dtype < 4; dtype++) {
    attention_case(dtype, 3, 8, 4, 2, 16, L3, 0);  /* cache filled to capacity */
    attention_case(dtype, 3, 8, 4, 2, 16, L3, 8);  /* room for the append */
    attention_case(dtype, 1, 4, 4, 1, 8, L1, 4);   /* G = 4 */
    attention_case(dtype, 2, 2, 2, 2, 8, L2, 3);   /* G = 1, a tiny canvas */
  }
  merge_case(5, 8, 23, 4);
  merge_case(3, 16, 1, 1);
  printf("oracle under sanitizers: %d calls, every buffer exactly sized\n", n_calls);
  return 0;
}
