// dg_internal.h -- types shared by the host API and the gfx950 kernels of libdg.
//
// Work decomposition ("split-key plan").  For every sequence b the key space
// of one call is the concatenation [cache rows 0..L_b-1 ; new rows 0..n_q-1]
// (the canvas or block of 256 rows, or the 1..16 tokens of a decode call).
// Query rows of one kv head are packed: packed row p = i*G + hh is new row i of
// query head g*G + hh, so the G query heads sharing kv head g form one matrix of
// n_q*G rows.  A work unit is (sequence b, kv head g, key
// split s, row tile rt): rows [rt*R, rt*R+R) of that packed matrix against keys
// [s*split_keys, min((s+1)*split_keys, end)).  Each unit writes one partial
// result (normalised output rows plus log2-domain max and sum) that a merge
// kernel combines; a sequence with a single split writes its output directly.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg.h"

namespace dg {

constexpr int kCanvas = DG_N_CANVAS;
constexpr int kMaxBatch = DG_MAX_BATCH;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

struct SeqPlan {
  int32_t prefix_len;  // L_b
  int32_t n_splits;    // S_b >= 1
  int32_t split_keys;  // keys per split (multiple of 32); the last split may be shorter
  int32_t unit_base;   // first logical unit index of this sequence
  uint32_t rcp_s;      // div_rcp multipliers of S_b and S_b * NRT
  uint32_t rcp_snrt;
};

// Reciprocal multiplier for floor(n / d) when n * d < 2^32: with m = floor(2^32/d) + 1,
// floor(n*m / 2^32) = floor(n/d), because the excess n*(m - 2^32/d)/2^32 < n/2^32 < 1/d
// cannot reach the next multiple of d.  d = 1 is encoded as m = 0.  The kernels divide
// by per-call values (heads per kv head, splits, row tiles) this way: a hardware-free
// integer division costs tens of dependent instructions before the first load.
inline uint32_t rcp_u32(uint32_t d) { return d <= 1 ? 0u : (uint32_t)((1ull << 32) / d + 1); }

// bf16 kernel shapes.  R256 and R128: eight waves of 32 packed rows (row groups x
// key groups, waves paired on a SIMD in ping-pong); Free: eight free-running waves
// of 32 rows (256 rows per unit).  The fp8 kernel has the R128 shape.
enum { kVariantR256 = 0, kVariantR128 = 1, kVariantFree = 2, kNumVariants = 3 };
constexpr int kDefaultVariant = kVariantR128;
inline int variant_rows(int v) { return v == kVariantR128 ? 128 : 256; }

struct Plan {
  int32_t batch;
  int32_t n_q;          // query rows per sequence and head: 256 (canvas, commit) or the
                        // decode call's new tokens (1..DG_MAX_DECODE)
  uint32_t rcp_m;       // div_rcp multiplier of n_q * G (packed rows per kv head)
  int32_t variant;      // bf16 kernel shape (kVariant*); rows_per_unit follows from it
  int32_t n_units;      // total logical units = grid size of the attention kernel (< 2^16)
  int32_t n_rowtiles;   // NRT = ceil(n_q*G / R)
  int32_t rows_per_unit;// R
  int32_t g;            // G = query heads per kv head
  uint32_t rcp_g;       // div_rcp multipliers of G and NRT
  uint32_t rcp_nrt;
  SeqPlan seq[kMaxBatch];
};
constexpr int kMaxUnits = 1 << 16;

struct AttnArgs {
  const void* q;        // [B][n_q][Hq][D]
  const void* k_cache;  // [B][cap][Hkv][D]
  const void* v_cache;
  const void* k_new;    // canvas (step), block (commit) or decode K/V [B][n_q][Hkv][D]
  const void* v_new;
  void* k_append;       // commit and decode: cache K/V written at rows L..L+n_q-1 (else null)
  void* v_append;
  void* out;            // [B][n_q][Hq][D]
  void* part_o;         // [n_units][R][D] normalised partial outputs: bf16 for the
                        // bf16 path (the output is rounded to bf16 anyway), fp32 for
                        // the fp32 path
  float* part_ml;       // [n_units][R][2]: max (log2 domain) and sum
  int64_t cap;
  int32_t n_heads_q;
  int32_t n_heads_kv;
  float scale_log2;     // softmax scale * log2(e) (fp8: times the q and k scales)
  float out_scale;      // fp8: the v scale, applied with the normalisation (else 1)
};

// Canvas sampler (dg_sample.hip).
struct SampleArgs {
  const void* logits;      // [B][256][V] bf16
  const int32_t* noise;    // [B][256] re-noise tokens
  const int32_t* prev;     // [B][256] previous step's argmax, or null
  float* entropy;          // [B][256] out, nats
  int32_t* argmax;         // [B][256] out
  int32_t* tokens;         // [B][256] out
  int32_t* accepted;       // [B][256] out, 0/1
  int32_t* stop;           // [B] out, 0/1
  long long qbudget;       // budget in units of 2^-32 nats
  long long qstop;         // stop threshold in units of 2^-32 nats
  float c;                 // log2(e) / tau
  int32_t vocab;
  int32_t batch;
};

// Self-conditioning input (dg_selfcond.hip).  The softmax pass works on vocabulary
// splits of kSelfcondSplit entries and writes blocks of kSelfcondBlock entries.
constexpr int kSelfcondSplit = 8192;
constexpr int kSelfcondBlock = 32;

struct SelfcondArgs {
  const void* logits;  // [M][V] bf16, M = B*256 rows
  const void* embed;   // [V][d] bf16
  const void* w1;      // [d][h] bf16
  const void* w2;      // [h][d] bf16
  void* z;             // [M][d] bf16 out
  void* pblk;          // workspace: exp(x - split max) as bf16, blocked [V/32][M][32]
  float2* stats;       // workspace: [V/8192][M] (log2-domain split max, sum of the weights)
  float* part;         // workspace: fp32 split partials of the products
  void* yblk;          // workspace: softmax(x) E as bf16, blocked [d/32][M][32]
  void* hblk;          // workspace: gelu(y W1) as bf16, blocked [h/32][M][32]
  int32_t rows, vocab, vocab_splits, d_model, d_hidden, split_w1, split_w2;
  // kernel timing hooks of the library (kind 0: the embedding product, 1: the softmax pass)
  void (*time_begin)(int kind, hipStream_t st);
  void (*time_end)(int kind, hipStream_t st);
};

// Host-side launchers (defined next to their kernels).  Each returns the HIP
// error of the launch.
int launch_attn_bf16(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream);
int launch_attn_fp8(const AttnArgs& a, const Plan& p, bool causal, void* stream);
int launch_attn_f32(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream);
int launch_merge(const AttnArgs& a, const Plan& p, int head_dim, bool bf16_out, void* stream);
int launch_sample(const SampleArgs& s, void* stream);
int launch_decode(const AttnArgs& a, const Plan& p, int dtype, int head_dim, void* stream);
int launch_selfcond(const SelfcondArgs& a, void* stream);
// contraction rows per split of a self-conditioning product (a multiple of 32)
int selfcond_splits(int K, int N, int M, int cus);

// Rows per unit of the fp32 kernel and the key granule of every kernel.
constexpr int kRowsF32 = 64;
constexpr int kKeyGranule = 32;

// Decode kernel (dg_attn_mfma.hip): 32 packed rows per unit, kDecodeWaves waves that
// stream their own chunks; one workgroup per CU.
constexpr int kDecodeRows = 32;
constexpr int kDecodeWaves = 4;

}  // namespace dg
