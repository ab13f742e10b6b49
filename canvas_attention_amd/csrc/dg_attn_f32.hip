// dg_attn_f32.hip -- split-key canvas / commit attention with fp32 storage and arithmetic.
//
// Same work units, key space, masks and partial format as the bf16 kernel
// (canvas step: unmasked attention over [cache ; canvas]; commit: block row i
// sees block keys 0..i and the block K/V are appended to the cache --
// "DiffusionGemma Technical Report", paperfeed.app summary, section "The
// mechanism: an AR model turned inside out"; decode: the commit's rule for the
// 1..16 new tokens of the same section's AR mode, "AR mode survives").  Products and sums are true fp32
// FMAs on the vector ALU: this path exists for exact-precision checking, not
// speed.  One wave64 per unit, one packed query row per lane; 32-key K/V tiles
// are staged in LDS and read as broadcasts.  Per tile the exact tile max is
// folded in (one rescale per tile).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, Plan plan) {
  constexpr int R = kRowsF32;
  constexpr int TK = 32;
  constexpr int D4 = D / 4;
  __shared__ float4 ks[TK][D4];
  __shared__ float4 vs[TK][D4];

  const int lane = threadIdx.x;
  const int U = xcd_remap(blockIdx.x, gridDim.x);
  SeqPlan sp;
  const Unit u = decode_unit(plan, U, sp);
  const int b = u.b, g = u.g, s = u.s, rt = u.rt, NRT = plan.n_rowtiles;
  const int L = sp.prefix_len;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  const int row0 = rt * R;
  const int NQ = plan.n_q, M = NQ * G;  // new rows per head, packed rows per kv head
  int kend = L + NQ;
  if (CAUSAL) kend = min(kend, L + (row0 + R - 1) / G + 1);
  const int kbeg = s * sp.split_keys;
  const int kstop = min(kbeg + sp.split_keys, kend);

  const float* kc = (const float*)a.k_cache;
  const float* vc = (const float*)a.v_cache;
  const float* kn = (const float*)a.k_new;
  const float* vn = (const float*)a.v_new;

  if (CAUSAL && a.k_append != nullptr) {
    const int cnt = sp.n_splits * NRT;
    const int w = s * NRT + rt;
    const int rpu = (NQ + cnt - 1) / cnt;
    const int r0 = min(NQ, w * rpu), r1 = min(NQ, r0 + rpu);
    const int per = (r1 - r0) * D4;
    for (int idx = lane; idx < 2 * per; idx += 64) {
      const int which = idx / per, rem = idx % per;
      const int r = r0 + rem / D4, c = rem % D4;
      const int64_t src = ((int64_t)(b * NQ + r) * Hkv + g) * D + 4 * c;
      const int64_t dst = (((int64_t)b * a.cap + L + r) * Hkv + g) * D + 4 * c;
      *(float4*)((float*)(which ? a.v_append : a.k_append) + dst) =
          *(const float4*)((which ? vn : kn) + src);
    }
  }

  // lanes past the last packed row (a decode tile) compute on a copy of that row
  // and write nothing
  const int prow = min(row0 + lane, M - 1);
  const bool valid = row0 + lane < M;
  const int qi = prow / G, hh = prow % G;
  float q[D];
  const float* qp = (const float*)a.q + ((int64_t)(b * NQ + qi) * Hq + g * G + hh) * D;
#pragma unroll
  for (int d = 0; d < D; d++) q[d] = qp[d];
  float o[D];
#pragma unroll
  for (int d = 0; d < D; d++) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c2 = a.scale_log2;

  for (int tkey0 = kbeg; tkey0 < kstop; tkey0 += TK) {
    __syncthreads();
    for (int idx = lane; idx < TK * D4; idx += 64) {
      const int r = idx / D4, c = idx % D4;
      const int key = min(tkey0 + r, kstop - 1);
      const float *kp, *vp;
      if (key < L) {
        const int64_t off = (((int64_t)b * a.cap + key) * Hkv + g) * D;
        kp = kc + off;
        vp = vc + off;
      } else {
        const int64_t off = ((int64_t)(b * NQ + key - L) * Hkv + g) * D;
        kp = kn + off;
        vp = vn + off;
      }
      ks[r][c] = *(const float4*)(kp + 4 * c);
      vs[r][c] = *(const float4*)(vp + 4 * c);
    }
    __syncthreads();
    float sc[TK];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; j++) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D4; c++) {
        const float4 k4 = ks[j][c];
        acc = fmaf(q[4 * c + 0], k4.x, acc);
        acc = fmaf(q[4 * c + 1], k4.y, acc);
        acc = fmaf(q[4 * c + 2], k4.z, acc);
        acc = fmaf(q[4 * c + 3], k4.w, acc);
      }
      const int key = tkey0 + j;
      bool ok = key < kstop;
      if (CAUSAL) ok = ok && (key < L || key - L <= qi);
      sc[j] = ok ? acc * c2 : -INFINITY;
      tmax = fmaxf(tmax, sc[j]);
    }
    if (tmax == -INFINITY) continue;  // no visible key in this tile for this row
    const float mnew = fmaxf(m, tmax);
    const float alpha = exp2f(m - mnew);  // m = -inf on the first visible tile -> 0
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; d++) o[d] *= alpha;
    m = mnew;
#pragma unroll
    for (int j = 0; j < TK; j++) {
      const float p = exp2f(sc[j] - m);
      l += p;
#pragma unroll
      for (int c = 0; c < D4; c++) {
        const float4 v4 = vs[j][c];
        o[4 * c + 0] = fmaf(p, v4.x, o[4 * c + 0]);
        o[4 * c + 1] = fmaf(p, v4.y, o[4 * c + 1]);
        o[4 * c + 2] = fmaf(p, v4.z, o[4 * c + 2]);
        o[4 * c + 3] = fmaf(p, v4.w, o[4 * c + 3]);
      }
    }
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (sp.n_splits == 1) {
    if (!valid) return;
    float* op = (float*)a.out + ((int64_t)(b * NQ + qi) * Hq + g * G + hh) * D;
#pragma unroll
    for (int c = 0; c < D4; c++)
      *(float4*)(op + 4 * c) =
          make_float4(o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv, o[4 * c + 3] * inv);
  } else {
    float* po = (float*)a.part_o + ((int64_t)U * R + lane) * D;
#pragma unroll
    for (int c = 0; c < D4; c++)
      *(float4*)(po + 4 * c) =
          make_float4(o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv, o[4 * c + 3] * inv);
    // an empty row reports a very negative max so the merge gives it zero weight
    *(float2*)(a.part_ml + ((int64_t)U * R + lane) * 2) = make_float2(l > 0.f ? m : -1e30f, l);
  }
}

}  // namespace

int launch_attn_f32(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream,
                    const LaunchEvents& ev) {
  hipStream_t st = (hipStream_t)stream;
  if (p.n_units == 0) return 0;
  const dim3 grid(p.n_units), block(64);
  if (head_dim == 128) {
    if (causal)
      hipExtLaunchKernelGGL((attn_f32_kernel<128, true>), grid, block, 0, st, ev.start, ev.stop, 0, a, p);
    else
      hipExtLaunchKernelGGL((attn_f32_kernel<128, false>), grid, block, 0, st, ev.start, ev.stop, 0, a, p);
  } else {
    if (causal)
      hipExtLaunchKernelGGL((attn_f32_kernel<64, true>), grid, block, 0, st, ev.start, ev.stop, 0, a, p);
    else
      hipExtLaunchKernelGGL((attn_f32_kernel<64, false>), grid, block, 0, st, ev.start, ev.stop, 0, a, p);
  }
  return (int)hipGetLastError();
}

}  // namespace dg
