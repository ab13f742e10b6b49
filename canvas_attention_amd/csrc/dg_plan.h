// dg_plan.h -- the split-key plan of libdg: its types, the unit decode and XCD
// dealing that the kernels run, and the host planners.
//
// Work decomposition.  For every sequence b the key space of one call is the
// concatenation [cache rows 0..L_b-1 ; new rows 0..n_q-1] (the canvas or block of
// 256 rows, or the 1..16 tokens of a decode call): the canvas cross-attends to
// the cache and to itself, and a committed block joins the cache ("DiffusionGemma
// Technical Report", paperfeed.app summary, section "The mechanism: an AR model
// turned inside out").  Query rows of one kv head are packed: packed row
// p = i*G + hh is new row i of query head g*G + hh, so the G query heads sharing
// kv head g form one matrix of n_q*G rows.  A work unit is (sequence b, kv head
// g, key split s, row tile rt): rows [rt*R, rt*R+R) of that packed matrix against
// keys [s*split_keys, min((s+1)*split_keys, end)).  Each unit writes one partial
// result (normalised output rows plus log2-domain max and sum) that a merge
// kernel combines; a sequence with a single split writes its output directly.
//
// Plain C++ with no HIP header: the planners and the decode also build into a
// host-only test (under the address and undefined-behaviour sanitizers) that
// checks the plan's coverage and bounds without a device.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "dg.h"

#if defined(__HIP__)
#define DG_HD __host__ __device__
#else
#define DG_HD
#endif

namespace dg {

constexpr int kCanvas = DG_N_CANVAS;
constexpr int kMaxBatch = DG_MAX_BATCH;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

// Packed rows per unit of the matrix-core canvas/commit kernels (bf16 and fp8):
// eight waves of 32 rows, four row groups x two key groups.
constexpr int kRowsMfma = 128;
// Rows per unit of the fp32 kernel and the key granule of every kernel (fp8
// splits are whole 64-key chunks).
constexpr int kRowsF32 = 64;
constexpr int kKeyGranule = 32;
constexpr int kKeyGranuleFp8 = 64;
// Decode kernel: 32 packed rows per unit, kDecodeWaves waves that stream their own
// chunks; one workgroup per CU.
constexpr int kDecodeRows = 32;
constexpr int kDecodeWaves = 4;
// Unit and row indices stay below 2^16, which keeps every kernel division n/d
// with n*d < 2^32 (the reciprocal-multiplier form below is exact there).
constexpr int kMaxUnits = 1 << 16;

struct SeqPlan {
  int32_t prefix_len;  // L_b
  int32_t n_splits;    // S_b >= 1
  int32_t split_keys;  // keys per split (a multiple of the key granule); the last split may be shorter
  int32_t unit_base;   // first logical unit index of this sequence
  uint32_t rcp_s;      // div_rcp multipliers of S_b and S_b * NRT
  uint32_t rcp_snrt;
};

struct Plan {
  int32_t batch;
  int32_t n_q;          // query rows per sequence and head: 256 (canvas, commit) or the
                        // decode call's new tokens (1..DG_MAX_DECODE)
  uint32_t rcp_m;       // div_rcp multiplier of n_q * G (packed rows per kv head)
  int32_t n_units;      // total logical units = grid size of the attention kernel (< 2^16)
  int32_t n_rowtiles;   // NRT = ceil(n_q*G / R)
  int32_t rows_per_unit;// R
  int32_t g;            // G = query heads per kv head
  uint32_t rcp_g;       // div_rcp multipliers of G and NRT
  uint32_t rcp_nrt;
  SeqPlan seq[kMaxBatch];
};

// Reciprocal multiplier for floor(n / d) when n * d < 2^32: with m = floor(2^32/d) + 1,
// floor(n*m / 2^32) = floor(n/d), because the excess n*(m - 2^32/d)/2^32 < n/2^32 < 1/d
// cannot reach the next multiple of d.  d = 1 is encoded as m = 0.  The kernels divide
// by per-call values (heads per kv head, splits, row tiles) this way: an integer
// division costs tens of dependent instructions before the first load.
inline uint32_t rcp_u32(uint32_t d) { return d <= 1 ? 0u : (uint32_t)((1ull << 32) / d + 1); }

// floor(n / d) from m = rcp_u32(d), for 0 <= n and n*d < 2^32; written without a
// branch so that the scalar loads around it in a kernel stay in one basic block
DG_HD inline int div_rcp(int n, uint32_t m) {
  return (int)(uint32_t)(((uint64_t)(uint32_t)n * m) >> 32) + (m == 0u ? n : 0);
}

// Workgroups are dealt to the 8 XCDs round-robin; workgroup bid of n gets the
// logical index that gives each XCD a contiguous range, so that units sharing K/V
// tiles (the row tiles and splits of one kv head) share an L2.  A bijection of 0..n-1.
DG_HD inline int xcd_remap(int bid, int n) {
  const int x = bid % kNumXcd, j = bid / kNumXcd, r = n % kNumXcd;
  return x * (n / kNumXcd) + (x < r ? x : r) + j;
}

struct Unit {
  int b, g, s, rt;
};

// Unit U of a launch and the plan of its sequence.  Sequence 0's entry is read
// together with the plan header; a unit of a later sequence costs one more
// scalar round trip.  Within a sequence, local = (g*S + s)*NRT + rt.
DG_HD inline Unit decode_unit(const Plan& p, int U, SeqPlan& sp) {
  sp = p.seq[0];
  int b = 0;
  for (int i = 1; i < p.batch; i++)
    if (U >= p.seq[i].unit_base) b = i;
  if (b != 0) sp = p.seq[b];
  const int local = U - sp.unit_base;
  const int S = sp.n_splits, NRT = p.n_rowtiles;
  const int q = div_rcp(local, p.rcp_nrt);  // local / NRT
  Unit u;
  u.b = b;
  u.g = div_rcp(local, sp.rcp_snrt);
  u.s = q - div_rcp(q, sp.rcp_s) * S;
  u.rt = local - q * NRT;
  return u;
}

// The unit index of (g, s, rt) within sequence plan sp: the inverse of decode_unit,
// as the merge kernels address the partials of a row.
DG_HD inline int unit_index(const Plan& p, const SeqPlan& sp, int g, int s, int rt) {
  return sp.unit_base + (g * sp.n_splits + s) * p.n_rowtiles + rt;
}

// ---------------------------------------------------------------- host planners
// (dg_plan.cpp).  target_units is the number of units that fills the device once;
// forced_split_keys > 0 overrides the split size (rounded up to the key granule).

inline bool mfma_path(int dtype) { return dtype != DG_F32; }
inline int key_granule(int dtype) { return dtype == DG_FP8 ? kKeyGranuleFp8 : kKeyGranule; }
inline int rows_per_unit(int dtype) { return mfma_path(dtype) ? kRowsMfma : kRowsF32; }
inline int decode_rows(int dtype) { return mfma_path(dtype) ? kDecodeRows : kRowsF32; }
inline size_t out_elem_size(int dtype) { return dtype == DG_F32 ? 4 : 2; }

// Canvas step and commit: every unit of every sequence gets about the same number
// of keys, chosen so that the units fill the device about once; a ragged batch
// whose plan would spill into a partial second round of workgroups may take a
// smaller split size that aims at up to kMaxRounds full rounds (dg_plan.cpp).
constexpr int kMaxRounds = 4;
void make_plan(const dg_shape* s, const int32_t* prefix_len, int target_units,
               int forced_split_keys, Plan* p);
// Decode: tiles of R packed rows and key splits sized so that the units fill the
// device once.
void make_decode_plan(const dg_shape* s, const int32_t* prefix_len, int target_units,
                      int forced_split_keys, Plan* p);
// Bytes of one partial row: the normalised output (bf16 or fp32) plus max and sum.
size_t partial_row_bytes(const dg_shape* s);
// Workspace a plan's partial rows take (0 when every sequence has one split).
size_t plan_workspace(const dg_shape* s, const Plan& p);
// Workspace that covers every plan of this shape with prefixes up to max_prefix_len
// (the canvas bound allows for plans of up to kMaxRounds rounds).
size_t workspace_bound(const dg_shape* s, int64_t max_prefix_len, int target_units,
                       int forced_split_keys);
size_t decode_workspace_bound(const dg_shape* s, int64_t max_prefix_len, int target_units,
                              int forced_split_keys);

}  // namespace dg
