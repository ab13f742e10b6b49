// dg_internal.h -- types shared by the host API and the gfx950 kernels of libdg
// (the split-key plan and its unit decode are in dg_plan.h).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "dg.h"
#include "dg_plan.h"

namespace dg {

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

// Events that a launch records with its own dispatch (hipExtLaunchKernelGGL), so
// that the time between them is the kernel's execution alone; the library's
// kernel timing hooks pass them.  Both null: a plain launch.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Host-side launchers (defined next to their kernels).  Each returns the HIP
// error of the launch.
int launch_attn_bf16(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream,
                     const LaunchEvents& ev);
int launch_attn_fp8(const AttnArgs& a, const Plan& p, bool causal, void* stream,
                    const LaunchEvents& ev);
int launch_attn_f32(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream,
                    const LaunchEvents& ev);
int launch_merge(const AttnArgs& a, const Plan& p, int head_dim, bool bf16_out, void* stream,
                 const LaunchEvents& ev);
int launch_sample(const SampleArgs& s, void* stream);
int launch_decode(const AttnArgs& a, const Plan& p, int dtype, int head_dim, void* stream,
                  const LaunchEvents& ev);
int launch_selfcond(const SelfcondArgs& a, void* stream);
// contraction rows per split of a self-conditioning product (a multiple of 32)
int selfcond_splits(int K, int N, int M, int cus);

}  // namespace dg
