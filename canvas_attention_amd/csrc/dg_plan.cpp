// dg_plan.cpp -- the host planners of the split-key decomposition (see dg_plan.h).
// Plain C++: nothing here touches a device, so the same code links into the
// library and into the host-only property test of the plan.
#include "dg_plan.h"

#include <string.h>

#include <algorithm>

namespace dg {

namespace {

// The canvas plan for split size kappa (a multiple of the key granule).
void fill_plan(const dg_shape* s, const int32_t* prefix_len, int64_t kappa, Plan* p) {
  const int R = rows_per_unit(s->dtype);
  const int G = s->n_heads_q / s->n_heads_kv;
  const int NRT = kCanvas * G / R;
  const int per_split = s->n_heads_kv * NRT;  // units per split index
  const int gran = key_granule(s->dtype);
  memset(p, 0, sizeof *p);
  p->batch = s->batch;
  p->n_q = kCanvas;
  p->rcp_m = rcp_u32((uint32_t)(kCanvas * G));
  p->n_rowtiles = NRT;
  p->rows_per_unit = R;
  p->g = G;
  p->rcp_g = rcp_u32((uint32_t)G);
  p->rcp_nrt = rcp_u32((uint32_t)NRT);
  int64_t units = 0;
  for (int b = 0; b < s->batch; b++) {
    const int64_t K = (int64_t)prefix_len[b] + kCanvas;
    int64_t S = (K + kappa - 1) / kappa;
    int64_t sk = (K + S - 1) / S;
    sk = ((sk + gran - 1) / gran) * gran;
    S = (K + sk - 1) / sk;
    p->seq[b].prefix_len = prefix_len[b];
    p->seq[b].n_splits = (int)S;
    p->seq[b].split_keys = (int)sk;
    p->seq[b].unit_base = (int)std::min<int64_t>(units, INT32_MAX);
    p->seq[b].rcp_s = rcp_u32((uint32_t)S);
    p->seq[b].rcp_snrt = rcp_u32((uint32_t)(S * NRT));
    units += S * per_split;
  }
  p->n_units = (int)std::min<int64_t>(units, INT32_MAX);
}

// Keys of the plan's longest unit.
int64_t longest_unit(const dg_shape* s, const int32_t* prefix_len, const Plan& p) {
  int64_t m = 0;
  for (int b = 0; b < s->batch; b++)
    m = std::max<int64_t>(m, std::min<int64_t>(p.seq[b].split_keys, (int64_t)prefix_len[b] + kCanvas));
  return m;
}

}  // namespace

// Split size: the one that fills the device about once, kappa = W/T (W the
// summed keys of all units, T the units that fill the device once).  Each
// sequence rounds its own splits up, so a ragged batch can come out with more
// than T units and spill into a second, mostly idle round of workgroups.  Then
// split sizes aiming at 2 .. kMaxRounds rounds are weighed too, by the cost of
// the longest unit (the tail the greedy dispatch cannot fill) plus kRoundKeys
// per round of workgroups (the prologue and epilogue each round repeats).  The
// choice depends only on the shape, the prefixes and the device, so every entry
// point computes the same split plan for the same call.  The constants come
// from the 8-sequence ragged batch (prefixes 2047..32038, L = 8192-class units
// of the bf16 kernel): over split sizes of 2464..32320 keys its step time fits
// 283 us + 0.0049 us per key of the longest unit + 9.1 us per round within 11 us.
constexpr int64_t kRoundKeys = 1800;

void make_plan(const dg_shape* s, const int32_t* prefix_len, int target_units,
               int forced_split_keys, Plan* p) {
  const int R = rows_per_unit(s->dtype);
  const int G = s->n_heads_q / s->n_heads_kv;
  const int per_split = s->n_heads_kv * (kCanvas * G / R);
  int64_t W = 0;
  for (int b = 0; b < s->batch; b++) W += (int64_t)(prefix_len[b] + kCanvas) * per_split;
  const int64_t T = std::max(target_units, 1);
  const int gran = key_granule(s->dtype);
  const int64_t floor_keys = mfma_path(s->dtype) ? 256 : 64;
  if (forced_split_keys > 0) {
    fill_plan(s, prefix_len, forced_split_keys, p);
    return;
  }
  auto kappa_for = [&](int64_t rounds) {
    int64_t k = (W + rounds * T - 1) / (rounds * T);
    k = ((k + gran - 1) / gran) * gran;
    return std::max<int64_t>(k, floor_keys);
  };
  fill_plan(s, prefix_len, kappa_for(1), p);
  if (p->n_units <= T) return;
  auto cost = [&](const Plan& c) {
    return longest_unit(s, prefix_len, c) + kRoundKeys * ((c.n_units + T - 1) / T);
  };
  int64_t best = cost(*p);
  Plan c;
  for (int rounds = 2; rounds <= kMaxRounds; rounds++) {
    fill_plan(s, prefix_len, kappa_for(rounds), &c);
    if (c.n_units >= kMaxUnits) continue;
    const int64_t cc = cost(c);
    if (cc < best) {
      best = cc;
      *p = c;
    }
  }
}

// With P = B*Hkv*NRT units per split index, splits of kappa >= W / (T - P) keys
// give at most W/kappa + P <= T units (each sequence adds at most one partial
// split per head and tile), so no second round of workgroups waits behind the first.
void make_decode_plan(const dg_shape* s, const int32_t* prefix_len, int target_units,
                      int forced_split_keys, Plan* p) {
  const int nq = s->n_canvas;
  const int R = decode_rows(s->dtype);
  const int G = s->n_heads_q / s->n_heads_kv;
  const int NRT = (nq * G + R - 1) / R;
  const int per_split = s->n_heads_kv * NRT;
  int64_t W = 0;
  for (int b = 0; b < s->batch; b++) W += (int64_t)(prefix_len[b] + nq) * per_split;
  const int64_t T = std::max(target_units, 1);
  const int64_t P = (int64_t)s->batch * per_split;
  const int gran = key_granule(s->dtype);
  const int64_t avail = T > 2 * P ? T - P : T;
  int64_t kappa = (W + avail - 1) / avail;
  kappa = ((kappa + gran - 1) / gran) * gran;
  // at least one chunk per wave of the unit
  kappa = std::max<int64_t>(kappa, mfma_path(s->dtype) ? (int64_t)kDecodeWaves * gran : 64);
  if (forced_split_keys > 0) kappa = forced_split_keys;
  memset(p, 0, sizeof *p);
  p->batch = s->batch;
  p->n_q = nq;
  p->rcp_m = rcp_u32((uint32_t)(nq * G));
  p->n_rowtiles = NRT;
  p->rows_per_unit = R;
  p->g = G;
  p->rcp_g = rcp_u32((uint32_t)G);
  p->rcp_nrt = rcp_u32((uint32_t)NRT);
  int64_t units = 0;
  for (int b = 0; b < s->batch; b++) {
    const int64_t K = (int64_t)prefix_len[b] + nq;
    int64_t S = (K + kappa - 1) / kappa;
    int64_t sk = (K + S - 1) / S;
    sk = ((sk + gran - 1) / gran) * gran;
    S = (K + sk - 1) / sk;
    p->seq[b].prefix_len = prefix_len[b];
    p->seq[b].n_splits = (int)S;
    p->seq[b].split_keys = (int)sk;
    p->seq[b].unit_base = (int)std::min<int64_t>(units, INT32_MAX);
    p->seq[b].rcp_s = rcp_u32((uint32_t)S);
    p->seq[b].rcp_snrt = rcp_u32((uint32_t)(S * NRT));
    units += S * per_split;
  }
  p->n_units = (int)std::min<int64_t>(units, INT32_MAX);
}

size_t partial_row_bytes(const dg_shape* s) {
  return (size_t)s->head_dim * out_elem_size(s->dtype) + 2 * sizeof(float);
}

size_t plan_workspace(const dg_shape* s, const Plan& p) {
  bool any = false;
  for (int b = 0; b < p.batch; b++) any = any || p.seq[b].n_splits > 1;
  if (!any) return 0;
  return (size_t)p.n_units * p.rows_per_unit * partial_row_bytes(s);
}

// A plan aiming at r rounds never exceeds r*T + B*Hkv*NRT units whatever the
// prefixes: each sequence has at most K_b/kappa + 1 splits and kappa >= W/(r*T).
size_t workspace_bound(const dg_shape* s, int64_t max_prefix_len, int target_units,
                       int forced_split_keys) {
  const int R = rows_per_unit(s->dtype);
  const int G = s->n_heads_q / s->n_heads_kv;
  const int NRT = kCanvas * G / R;
  const int64_t per_split = (int64_t)s->n_heads_kv * NRT;
  int64_t units = (int64_t)kMaxRounds * std::max(target_units, 1) + (int64_t)s->batch * per_split;
  if (forced_split_keys > 0) {
    const int64_t S = (max_prefix_len + kCanvas + forced_split_keys - 1) / forced_split_keys;
    units = std::max<int64_t>(units, S * s->batch * per_split);
  }
  return (size_t)units * R * partial_row_bytes(s);
}

// The decode plan never exceeds T + B*Hkv*NRT units (see make_decode_plan).
size_t decode_workspace_bound(const dg_shape* s, int64_t max_prefix_len, int target_units,
                              int forced_split_keys) {
  const int nq = s->n_canvas, R = decode_rows(s->dtype);
  const int G = s->n_heads_q / s->n_heads_kv;
  const int64_t per_split = (int64_t)s->n_heads_kv * ((nq * G + R - 1) / R);
  int64_t units = (int64_t)std::max(target_units, 1) + (int64_t)s->batch * per_split;
  if (forced_split_keys > 0) {
    const int64_t S = (max_prefix_len + nq + forced_split_keys - 1) / forced_split_keys;
    units = std::max<int64_t>(units, S * s->batch * per_split);
  }
  return (size_t)units * R * partial_row_bytes(s);
}

}  // namespace dg
