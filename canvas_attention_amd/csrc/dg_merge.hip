// dg_merge.hip -- combines the split-key partials of every query row.
//
// Each split s of a row holds a normalised output O_s, its log2-domain max m_s
// and its sum l_s (relative to m_s).  Attention over the union of the splits'
// keys is
//   M = max_s m_s,  w_s = 2^(m_s - M) * l_s,  out = sum_s w_s O_s / sum_s w_s,
// which is the same softmax as over the concatenated keys: the cache splits and
// the canvas (or block) tile of one row merge into attention over [cache ;
// canvas] ("DiffusionGemma Technical Report", paperfeed.app summary, section
// "The mechanism: an AR model turned inside out").  Splits without keys carry
// l_s = 0 and drop out.  Memory-bound: every thread handles four adjacent
// head_dim elements of one row, so partial reads and output writes are
// contiguous per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

template <int D, bool BF16OUT>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, Plan plan) {
  constexpr int TPR = D / 4;        // threads per row
  constexpr int RPB = 256 / TPR;    // rows per block
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  const int rows_per_seq = Hkv * kCanvas * G;
  const int64_t grow = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int d4 = threadIdx.x % TPR;
  if (grow >= (int64_t)plan.batch * rows_per_seq) return;
  const int b = (int)(grow / rows_per_seq);
  const int rem = (int)(grow % rows_per_seq);
  const int g = rem / (kCanvas * G), p = rem % (kCanvas * G);
  const SeqPlan sp = plan.seq[b];
  if (sp.n_splits == 1) return;  // written directly by the attention kernel
  const int R = plan.rows_per_unit, NRT = plan.n_rowtiles;
  const int rt = p / R, pr = p % R;
  const int u0 = sp.unit_base + g * sp.n_splits * NRT + rt;

  float M = -INFINITY;
  for (int s = 0; s < sp.n_splits; s++)
    M = fmaxf(M, a.part_ml[((int64_t)(u0 + s * NRT) * R + pr) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  for (int s = 0; s < sp.n_splits; s++) {
    const int64_t base = (int64_t)(u0 + s * NRT) * R + pr;
    const float2 ml = *(const float2*)(a.part_ml + base * 2);
    const float w = exp2f(ml.x - M) * ml.y;
    if (w == 0.f) continue;
    const float4 v = *(const float4*)(a.part_o + base * D + 4 * d4);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
    wsum += w;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int i = p / G, hh = p % G;
  const int64_t off = ((int64_t)(b * kCanvas + i) * Hq + g * G + hh) * D + 4 * d4;
  if (BF16OUT) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
    bf16x4 v;
    v[0] = (__bf16)(acc.x * inv);
    v[1] = (__bf16)(acc.y * inv);
    v[2] = (__bf16)(acc.z * inv);
    v[3] = (__bf16)(acc.w * inv);
    *(bf16x4*)((uint16_t*)a.out + off) = v;
  } else {
    *(float4*)((float*)a.out + off) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

template <int D, bool BF16OUT>
int launch_t(const AttnArgs& a, const Plan& p, hipStream_t st) {
  constexpr int RPB = 256 / (D / 4);
  const int64_t rows = (int64_t)p.batch * a.n_heads_q * kCanvas;
  const int blocks = (int)((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((merge_kernel<D, BF16OUT>), dim3(blocks), dim3(256), 0, st, a, p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_merge(const AttnArgs& a, const Plan& p, int head_dim, bool bf16_out, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128)
    return bf16_out ? launch_t<128, true>(a, p, st) : launch_t<128, false>(a, p, st);
  return bf16_out ? launch_t<64, true>(a, p, st) : launch_t<64, false>(a, p, st);
}

}  // namespace dg
