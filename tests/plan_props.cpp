// plan_props.cpp -- host-only property test of the split-key plan (dg_plan.h,
// dg_plan.cpp), built with the address and undefined-behaviour sanitizers by
// tests/test_plan_sanitized.py.  No device is involved: the unit decode and the
// XCD dealing are the same inline functions the kernels run.
//
// Over random shapes, ragged prefixes, device sizes and forced split sizes, for
// the canvas/commit plan and the decode plan:
//   * every unit index decodes to a distinct (b, g, s, rt) in range, and
//     unit_index (the merge kernels' addressing) inverts the decode;
//   * the splits of every (b, g, rt) cover keys 0 .. L_b + n_q - 1 exactly once,
//     each split non-empty and a whole number of key granules but the last;
//   * an accepted plan (the API refuses n_units >= 2^16) keeps every division
//     the kernels make by reciprocal multipliers exact: checked over the whole
//     numerator range of each divisor, and n*d < 2^32 holds there;
//   * the plan's workspace stays within workspace_bound / decode_workspace_bound
//     for the largest prefix, and a plan of natural split size has at most
//     T + B*Hkv*NRT units;
//   * xcd_remap is a bijection of 0..n-1.
// Prints one summary line and exits 0, or reports the first failure and exits 1.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <utility>
#include <vector>

#include "dg_plan.h"

using namespace dg;

static int g_fail = 0;
#define CHECK(cond, ...)                                              \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      fprintf(stderr, __VA_ARGS__);                                   \
      fprintf(stderr, "\n");                                          \
      g_fail = 1;                                                     \
      return false;                                                   \
    }                                                                 \
  } while (0)

// floor(n/d) by the reciprocal multiplier against the true quotient, for every n
// in 0..nmax (and n*d < 2^32 over that range)
static bool exact_division(int64_t nmax, uint32_t d, const char* what) {
  CHECK(d >= 1, "%s: divisor 0", what);
  CHECK((uint64_t)nmax * d < (1ull << 32), "%s: n*d = %lld*%u reaches 2^32", what,
        (long long)nmax, d);
  const uint32_t m = rcp_u32(d);
  for (int64_t n = 0; n <= nmax; n++)
    CHECK(div_rcp((int)n, m) == (int)(n / d), "%s: %lld / %u", what, (long long)n, d);
  return true;
}

struct Case {
  dg_shape s;
  std::vector<int32_t> L;
  int T, forced;
  bool decode;
};

static bool check_plan(const Case& c, long* n_units_seen) {
  const dg_shape& s = c.s;
  Plan p;
  if (c.decode)
    make_decode_plan(&s, c.L.data(), c.T, c.forced, &p);
  else
    make_plan(&s, c.L.data(), c.T, c.forced, &p);
  if (p.n_units >= kMaxUnits) return true;  // refused by the API before any launch
  if (!c.decode && c.forced == 0) {
    // a plan that fits one round of workgroups is the split size W/T itself
    int64_t W = 0;
    for (int b = 0; b < s.batch; b++) W += (int64_t)(c.L[b] + kCanvas);
    const int64_t per = (int64_t)s.n_heads_kv * (kCanvas * (s.n_heads_q / s.n_heads_kv) /
                                                 rows_per_unit(s.dtype));
    if (p.n_units <= c.T) {
      const int gran = key_granule(s.dtype);
      int64_t kappa = (W * per + c.T - 1) / c.T;
      kappa = std::max<int64_t>(((kappa + gran - 1) / gran) * gran, mfma_path(s.dtype) ? 256 : 64);
      for (int b = 0; b < s.batch; b++)
        CHECK(p.seq[b].split_keys <= kappa, "b %d: split of %d keys in a one-round plan of %lld",
              b, p.seq[b].split_keys, (long long)kappa);
    }
  }
  *n_units_seen += p.n_units;
  const int nq = c.decode ? s.n_canvas : kCanvas;
  const int G = s.n_heads_q / s.n_heads_kv, Hkv = s.n_heads_kv;
  const int R = c.decode ? decode_rows(s.dtype) : rows_per_unit(s.dtype);
  const int NRT = (nq * G + R - 1) / R;
  const int gran = key_granule(s.dtype);
  CHECK(p.batch == s.batch && p.n_q == nq && p.g == G && p.rows_per_unit == R &&
            p.n_rowtiles == NRT,
        "plan header");
  CHECK(c.decode || NRT * R == nq * G, "canvas row tiles must be whole: NRT %d R %d", NRT, R);

  // units: the decode is injective, in range, and inverted by unit_index
  std::vector<int> seen((size_t)p.n_units, 0);
  int64_t expect_units = 0;
  for (int b = 0; b < s.batch; b++) {
    CHECK(p.seq[b].unit_base == expect_units, "b %d unit_base %d, expected %lld", b,
          p.seq[b].unit_base, (long long)expect_units);
    expect_units += (int64_t)p.seq[b].n_splits * Hkv * NRT;
  }
  CHECK(expect_units == p.n_units, "n_units %d, sum over sequences %lld", p.n_units,
        (long long)expect_units);
  // key intervals of every (b, g, rt), checked below to tile 0 .. K_b - 1
  std::vector<int64_t> first((size_t)s.batch + 1, 0);
  for (int b = 0; b < s.batch; b++) first[b + 1] = first[b] + (int64_t)Hkv * NRT;
  std::vector<std::vector<std::pair<int64_t, int64_t>>> iv((size_t)first[s.batch]);
  for (int U = 0; U < p.n_units; U++) {
    SeqPlan sp;
    const Unit u = decode_unit(p, U, sp);
    CHECK(u.b >= 0 && u.b < s.batch, "U %d: b %d", U, u.b);
    CHECK(memcmp(&sp, &p.seq[u.b], sizeof sp) == 0, "U %d: sequence plan", U);
    CHECK(u.g >= 0 && u.g < Hkv && u.s >= 0 && u.s < sp.n_splits && u.rt >= 0 && u.rt < NRT,
          "U %d: (g %d, s %d, rt %d) out of range", U, u.g, u.s, u.rt);
    CHECK(unit_index(p, sp, u.g, u.s, u.rt) == U, "U %d: unit_index", U);
    seen[(size_t)U]++;
    const int64_t K = (int64_t)sp.prefix_len + nq;
    const int64_t kbeg = (int64_t)u.s * sp.split_keys;
    const int64_t kstop = std::min<int64_t>(kbeg + sp.split_keys, K);
    CHECK(kbeg < kstop, "U %d: empty split [%lld, %lld) of %lld keys", U, (long long)kbeg,
          (long long)kstop, (long long)K);
    CHECK(sp.split_keys % gran == 0, "split_keys %d not a multiple of %d", sp.split_keys, gran);
    iv[(size_t)(first[u.b] + (int64_t)u.g * NRT + u.rt)].push_back({kbeg, kstop});
  }
  for (int U = 0; U < p.n_units; U++)
    CHECK(seen[(size_t)U] == 1, "U %d decoded %d times", U, seen[(size_t)U]);
  for (int b = 0; b < s.batch; b++)
    for (int64_t t = first[b]; t < first[b + 1]; t++) {
      auto& v = iv[(size_t)t];
      std::sort(v.begin(), v.end());
      int64_t at = 0;
      for (auto& x : v) {
        CHECK(x.first == at, "b %d (g, rt) %lld: split starts at %lld, keys covered to %lld", b,
              (long long)(t - first[b]), (long long)x.first, (long long)at);
        at = x.second;
      }
      CHECK(at == (int64_t)c.L[b] + nq, "b %d (g, rt) %lld: keys covered to %lld of %lld", b,
            (long long)(t - first[b]), (long long)at, (long long)c.L[b] + nq);
    }

  // exact divisions over the numerator ranges the kernels use (each distinct pair once)
  std::vector<std::pair<int64_t, uint32_t>> divs;
  divs.push_back({p.n_units - 1, (uint32_t)NRT});                          // unit / NRT
  for (int b = 0; b < s.batch; b++) {
    const SeqPlan& sp = p.seq[b];
    const int64_t local_max = (int64_t)sp.n_splits * Hkv * NRT - 1;
    CHECK(rcp_u32((uint32_t)sp.n_splits) == sp.rcp_s &&
              rcp_u32((uint32_t)(sp.n_splits * NRT)) == sp.rcp_snrt,
          "b %d reciprocals", b);
    divs.push_back({local_max, (uint32_t)(sp.n_splits * NRT)});            // local / (S*NRT)
    divs.push_back({local_max / NRT, (uint32_t)sp.n_splits});              // (local/NRT) / S
  }
  CHECK(p.rcp_g == rcp_u32((uint32_t)G) && p.rcp_nrt == rcp_u32((uint32_t)NRT) &&
            p.rcp_m == rcp_u32((uint32_t)(nq * G)),
        "plan reciprocals");
  divs.push_back({(int64_t)NRT * R - 1, (uint32_t)G});                     // packed row / G
  divs.push_back({(int64_t)s.n_heads_q * nq - 1, (uint32_t)(nq * G)});     // row / (n_q*G)
  divs.push_back({s.n_heads_q - 1, (uint32_t)G});                          // (row/256) / G
  std::sort(divs.begin(), divs.end());
  divs.erase(std::unique(divs.begin(), divs.end()), divs.end());
  for (auto& d : divs) CHECK(exact_division(d.first, d.second, "kernel division"), "see above");

  // workspace within the bound the API publishes for the largest prefix
  const int64_t Lmax = *std::max_element(c.L.begin(), c.L.end());
  const size_t ws = plan_workspace(&s, p);
  const size_t bound = c.decode ? decode_workspace_bound(&s, Lmax, c.T, c.forced)
                                : workspace_bound(&s, Lmax, c.T, c.forced);
  CHECK(ws <= bound, "workspace %zu above the bound %zu", ws, bound);
  if (c.forced == 0) {
    const int64_t rounds = c.decode ? 1 : kMaxRounds;
    CHECK((int64_t)p.n_units <= rounds * c.T + (int64_t)s.batch * Hkv * NRT,
          "%d units above %lld*T + B*Hkv*NRT = %lld", p.n_units, (long long)rounds,
          (long long)(rounds * c.T + (int64_t)s.batch * Hkv * NRT));
  }
  return true;
}

int main(int argc, char** argv) {
  const int n_cases = argc > 1 ? atoi(argv[1]) : 400;
  const unsigned seed = argc > 2 ? (unsigned)atoi(argv[2]) : 20261203u;
  std::mt19937_64 rng(seed);
  auto pick = [&](std::initializer_list<int> v) {
    return *(v.begin() + std::uniform_int_distribution<size_t>(0, v.size() - 1)(rng));
  };
  auto uni = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };

  // xcd_remap: a bijection of 0..n-1 for every grid size up to the unit limit
  for (int n = 1; n <= kMaxUnits; n += (n < 4096 ? 1 : 97)) {
    std::vector<uint8_t> hit((size_t)n, 0);
    for (int bid = 0; bid < n; bid++) {
      const int u = xcd_remap(bid, n);
      if (u < 0 || u >= n || hit[(size_t)u]) {
        fprintf(stderr, "FAIL xcd_remap(%d, %d) = %d\n", bid, n, u);
        return 1;
      }
      hit[(size_t)u] = 1;
    }
  }

  long units = 0;
  int accepted = 0;
  for (int i = 0; i < n_cases; i++) {
    Case c;
    memset(&c.s, 0, sizeof c.s);
    c.decode = i % 3 == 2;
    c.s.dtype = pick({DG_BF16, DG_BF16, DG_FP8, DG_F32});
    c.s.head_dim = c.s.dtype == DG_FP8 ? 128 : pick({64, 128});
    c.s.n_heads_kv = pick({1, 2, 4, 8, 16});
    const int G = pick({1, 2, 3, 4, 5, 6, 8, 12, 16, 64});
    c.s.n_heads_q = std::min(c.s.n_heads_kv * G, 1024);
    c.s.batch = (int)pick({1, 1, 2, 3, 8, 17, 64});
    c.s.n_canvas = c.decode ? (int)uni(1, DG_MAX_DECODE) : DG_N_CANVAS;
    c.T = pick({256, 256, 304, 80, 1});
    c.forced = 0;
    if (uni(0, 3) == 0) {
      const int gran = key_granule(c.s.dtype);
      c.forced = (int)(((uni(1, 4096) + gran - 1) / gran) * gran);
    }
    // ragged prefixes: empty, tiny, around the granule and the canvas, long
    const int64_t lmax = pick({300, 9000, 140000, 1 << 20});
    for (int b = 0; b < c.s.batch; b++) {
      const int kind = (int)uni(0, 5);
      int64_t L = kind == 0 ? 0 : kind == 1 ? uni(1, 3) : kind == 2 ? 32 * uni(0, 20) + uni(-1, 1)
                                                                    : uni(0, lmax);
      c.L.push_back((int32_t)std::max<int64_t>(L, 0));
    }
    long before = units;
    if (!check_plan(c, &units)) {
      fprintf(stderr,
              "case %d: dtype %d D %d Hq %d Hkv %d B %d n_q %d T %d forced %d decode %d\n", i,
              c.s.dtype, c.s.head_dim, c.s.n_heads_q, c.s.n_heads_kv, c.s.batch, c.s.n_canvas,
              c.T, c.forced, (int)c.decode);
      return 1;
    }
    accepted += units > before;
  }
  printf("plan properties: %d cases (%d accepted plans, %ld units), xcd_remap bijective\n",
         n_cases, accepted, units);
  return g_fail;
}
