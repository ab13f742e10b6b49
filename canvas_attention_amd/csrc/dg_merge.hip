// dg_merge.hip -- combines the split-key partials of every query row.
//
// Each split s of a row holds a normalised output O_s, its log2-domain max m_s
// and its sum l_s (relative to m_s).  Attention over the union of the splits'
// keys is
//   M = max_s m_s,  w_s = 2^(m_s - M) * l_s,  out = sum_s w_s O_s / sum_s w_s,
// which is the same softmax as over the concatenated keys: the cache splits and
// the canvas (or block, or decode) tile of one row merge into attention over
// [cache ; new rows] ("DiffusionGemma Technical Report", paperfeed.app summary,
// section "The mechanism: an AR model turned inside out").  Splits without keys carry
// l_s = 0 and drop out.  Memory-bound: every thread handles one 16-byte chunk
// of a row (eight bf16 or four fp32 head_dim elements), so partial reads and
// output writes are contiguous per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

// Blocks are dealt like the attention kernel's units (xcd_remap, dg_plan.h):
// contiguous logical blocks on one XCD, so the rows of a kv head are merged on the
// XCD whose L2 holds its partials.

// Partial rows are bf16 for the bf16 path and fp32 for the fp32 path; each thread
// combines 8 (bf16) or 4 (fp32) adjacent head_dim elements of one row.  Block
// (x, y) covers rows x*RPB .. of sequence y.  Index math avoids runtime integer
// division (tens of dependent instructions each, ahead of the first load): G and
// n_q*G through the plan's reciprocals, the rows per unit (a power of two) by a
// shift.  DEC: a decode call (n_q rows per head, 1..16) rather than 256.
template <int D, bool BF16, bool DEC>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, Plan plan) {
  constexpr int EPT = BF16 ? 8 : 4;  // elements per thread
  constexpr int TPR = D / EPT;       // threads per row
  constexpr int RPB = 256 / TPR;     // rows per block
  const int Hq = a.n_heads_q, G = plan.g;
  const int b = blockIdx.y;
  const SeqPlan sp = plan.seq[b];
  if (sp.n_splits == 1) return;  // written directly by the attention kernel
  const int rem = xcd_remap(blockIdx.x, gridDim.x) * RPB + threadIdx.x / TPR;  // row of sequence b
  const int dq = threadIdx.x % TPR;
  const int NQ = DEC ? plan.n_q : kCanvas;
  if (rem >= Hq * NQ) return;
  const int g = DEC ? div_rcp(rem, plan.rcp_m) : div_rcp(rem / kCanvas, plan.rcp_g);
  const int p = rem - g * (NQ * G);
  const int rsh = __builtin_ctz((unsigned)plan.rows_per_unit), NRT = plan.n_rowtiles;
  const int rt = p >> rsh, pr = p & (plan.rows_per_unit - 1);
  const int R = plan.rows_per_unit;
  const int u0 = unit_index(plan, sp, g, 0, rt);  // split s is u0 + s*NRT

  // Splits are visited in batches of 8 with all loads of a batch in flight at
  // once; a running max keeps the weights bounded (partials carry finite maxima).
  constexpr int BATCH = 8;
  float M = -1e30f, wsum = 0.f;
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; e++) acc[e] = 0.f;
  for (int s0 = 0; s0 < sp.n_splits; s0 += BATCH) {
    float2 ml[BATCH];
    uint4 v[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; j++) {
      if (s0 + j < sp.n_splits) {
        const int64_t base = (int64_t)(u0 + (s0 + j) * NRT) * R + pr;
        ml[j] = *(const float2*)(a.part_ml + base * 2);
        v[j] = BF16 ? *(const uint4*)((const uint16_t*)a.part_o + base * D + EPT * dq)
                    : *(const uint4*)((const float*)a.part_o + base * D + EPT * dq);
      } else {
        ml[j] = make_float2(-1e30f, 0.f);
        v[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < BATCH; j++) Mb = fmaxf(Mb, ml[j].x);
    const float r = exp2f(M - Mb);
#pragma unroll
    for (int e = 0; e < EPT; e++) acc[e] *= r;
    wsum *= r;
#pragma unroll
    for (int j = 0; j < BATCH; j++) {
      const float w = exp2f(ml[j].x - Mb) * ml[j].y;
      const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int e = 0; e < EPT; e++) {
        const float x = BF16 ? __uint_as_float((e & 1) ? (wd[e / 2] & 0xffff0000u) : (wd[e / 2] << 16))
                             : __uint_as_float(wd[e]);
        acc[e] = fmaf(w, x, acc[e]);
      }
      wsum += w;
    }
    M = Mb;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int i = div_rcp(p, plan.rcp_g), hh = p - i * G;
  const int64_t off = ((int64_t)(b * NQ + i) * Hq + g * G + hh) * D + EPT * dq;
  if (BF16) {
    typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; e++) o[e] = (__bf16)(acc[e % EPT] * inv);
    *(bf16x8*)((uint16_t*)a.out + off) = o;
  } else {
    *(float4*)((float*)a.out + off) =
        make_float4(acc[0] * inv, acc[1 % EPT] * inv, acc[2 % EPT] * inv, acc[3 % EPT] * inv);
  }
}

// Decode calls (matrix-core kernels: bf16 partial rows, 32 rows per unit) have few
// rows, Hq * n_q per sequence, and many splits: one thread per 8-element chunk would
// walk the splits in a chain of dependent load batches.  Here the sum over splits
// is spread over SG threads per chunk, each with all of its splits' loads in flight
// (splits sg, sg + SG, ...), and the SG partial sums -- each a (max, weight sum,
// weighted values) triple like a split's own -- are combined through LDS.
template <int D>
__global__ __launch_bounds__(256) void merge_dec_kernel(AttnArgs a, Plan plan) {
  constexpr int CPR = D / 8;       // 8-element chunks per row
  constexpr int SG = 8;            // split groups per chunk
  constexpr int IPB = 256 / SG;    // chunks per block
  __shared__ float st[SG][IPB][10];
  const int b = blockIdx.y;
  const SeqPlan sp = plan.seq[b];
  if (sp.n_splits == 1) return;  // written directly by the attention kernel
  const int Hq = a.n_heads_q, G = plan.g, S = sp.n_splits, NRT = plan.n_rowtiles;
  const int ti = threadIdx.x % IPB, sg = threadIdx.x / IPB;
  const int item = blockIdx.x * IPB + ti;
  const int rem = item / CPR, c8 = item % CPR;  // row of sequence b, chunk
  const int M = plan.n_q * G;
  const bool valid = rem < Hq * plan.n_q;
  float mx = -1e30f, wsum = 0.f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; e++) o[e] = 0.f;
  int g = 0, p = 0;
  if (valid) {
    g = div_rcp(rem, plan.rcp_m);
    p = rem - g * M;
    const int rt = p >> 5, pr = p & 31;
    const int u0 = unit_index(plan, sp, g, 0, rt);  // split s is u0 + s*NRT
    for (int s0 = sg; s0 < S; s0 += 8 * SG) {
      float2 ml[8];
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int s = s0 + j * SG;
        if (s < S) {
          const int64_t base = (int64_t)(u0 + s * NRT) * 32 + pr;
          ml[j] = *(const float2*)(a.part_ml + base * 2);
          v[j] = *(const uint4*)((const uint16_t*)a.part_o + base * D + 8 * c8);
        } else {
          ml[j] = make_float2(-1e30f, 0.f);
          v[j] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      float mb = mx;
#pragma unroll
      for (int j = 0; j < 8; j++) mb = fmaxf(mb, ml[j].x);
      const float r = exp2f(mx - mb);
#pragma unroll
      for (int e = 0; e < 8; e++) o[e] *= r;
      wsum *= r;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const float w = exp2f(ml[j].x - mb) * ml[j].y;
        const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int e = 0; e < 8; e++)
          o[e] = fmaf(w, __uint_as_float((e & 1) ? (wd[e / 2] & 0xffff0000u) : (wd[e / 2] << 16)), o[e]);
        wsum += w;
      }
      mx = mb;
    }
  }
  st[sg][ti][0] = mx;
  st[sg][ti][1] = wsum;
#pragma unroll
  for (int e = 0; e < 8; e++) st[sg][ti][2 + e] = o[e];
  __syncthreads();
  if (sg != 0 || !valid) return;
  float M2 = -1e30f;
#pragma unroll
  for (int k = 0; k < SG; k++) M2 = fmaxf(M2, st[k][ti][0]);
  float W = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < SG; k++) {
    const float f = exp2f(st[k][ti][0] - M2);
    W += f * st[k][ti][1];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = fmaf(f, st[k][ti][2 + e], acc[e]);
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int i = div_rcp(p, plan.rcp_g), hh = p - i * G;
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; e++) out[e] = (__bf16)(acc[e] * inv);
  *(bf16x8*)((uint16_t*)a.out + ((int64_t)(b * plan.n_q + i) * Hq + g * G + hh) * D + 8 * c8) = out;
}

template <int D, bool BF16OUT>
int launch_t(const AttnArgs& a, const Plan& p, hipStream_t st, const LaunchEvents& ev) {
  constexpr int RPB = 256 / (D / (BF16OUT ? 8 : 4));
  const int rows = a.n_heads_q * p.n_q;  // per sequence
  const dim3 grid((rows + RPB - 1) / RPB, p.batch);
  if (p.n_q != kCanvas && BF16OUT && p.rows_per_unit == 32) {  // matrix-core decode
    const int chunks = rows * (D / 8);
    hipExtLaunchKernelGGL((merge_dec_kernel<D>), dim3((chunks + 31) / 32, p.batch), dim3(256), 0, st,
                          ev.start, ev.stop, 0, a, p);
  } else if (p.n_q == kCanvas) {
    hipExtLaunchKernelGGL((merge_kernel<D, BF16OUT, false>), grid, dim3(256), 0, st, ev.start, ev.stop,
                          0, a, p);
  } else {
    hipExtLaunchKernelGGL((merge_kernel<D, BF16OUT, true>), grid, dim3(256), 0, st, ev.start, ev.stop,
                          0, a, p);
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_merge(const AttnArgs& a, const Plan& p, int head_dim, bool bf16_out, void* stream,
                 const LaunchEvents& ev) {
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128)
    return bf16_out ? launch_t<128, true>(a, p, st, ev) : launch_t<128, false>(a, p, st, ev);
  return bf16_out ? launch_t<64, true>(a, p, st, ev) : launch_t<64, false>(a, p, st, ev);
}

}  // namespace dg
