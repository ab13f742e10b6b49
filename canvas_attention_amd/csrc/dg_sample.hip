// dg_sample.hip -- the canvas sampler on gfx950.
//
// After a denoising step's forward pass, every canvas position has logits over
// the vocabulary.  "DiffusionGemma Technical Report" (paperfeed.app summary,
// section "The mechanism: an AR model turned inside out", sampler paragraph):
// tempered logits give per-position entropies, positions are accepted from the
// lowest entropy upwards until a cumulative entropy budget is used up, the rest
// are re-noised to uniformly random tokens, and generation halts once the mean
// entropy is below a threshold with the argmax stable across two steps.
//
// Two launches:
//   * row_stats_kernel: one workgroup per position streams its logits once
//     (bf16, 16-byte loads, four in flight per lane) and forms the entropy of
//     softmax(logits / tau) and the argmax.  HBM-bound: 512 KB per position at a
//     262144-token vocabulary.
//   * select_kernel: one workgroup per canvas: budgeted acceptance, tokens and
//     the stop flag.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

// Bytes in flight: kBatch 16-byte loads per lane and batch, two batches in
// flight, 512 lanes: 32 KB per CU, 8 MB over the chip, about what HBM's
// bandwidth-delay product asks for.  Deeper batches (64 KB or 128 KB per CU, or
// more waves) queue more requests behind each row's stream and measured slower:
// 32.3 us per call at kBatch = 8, 27.9-28.4 us at kBatch = 2.
constexpr int kStatThreads = 512;
constexpr int kBatch = 2;           // 16-byte loads per lane per batch (16 logits)
constexpr float kRefSlack = 16.f;   // log2 units an exponential may exceed 1 by

// Running statistics of a slice of a row.  The exponentials are taken in the
// log2 domain, y = logit * c - r with c = log2(e) / tau and a reference r that is
// raised lazily (only when a batch max exceeds it by more than kRefSlack), so
// every 2^y stays below 2^16 and sums over a row cannot overflow.
//   z = sum 2^y,  s = sum 2^y * y;  entropy (bits) = log2(z) - s / z.
struct RowAcc {
  float best;  // largest logit seen
  int bk;      // first batch of this lane that reached it
  float r;     // reference, log2 domain
  float z, s;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// max of N (even) values as one v_max3 chain (logits are finite or -inf: no NaN
// handling)
template <int N>
__device__ __forceinline__ float max_of(const float (&x)[N]) {
  static_assert(N % 2 == 0 && N >= 2, "an even count");
  float m = x[0];
#pragma unroll
  for (int i = 1; i < N - 1; i += 2) asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(m), "v"(x[i]), "v"(x[i + 1]));
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(m), "v"(x[N - 1]));
  return m;
}


// (a, b) -> a: both slices' sums moved to the larger reference
__device__ __forceinline__ void merge_sums(float& r, float& z, float& s, float r2, float z2, float s2) {
  const float R = fmaxf(r, r2);
  const float fa = __builtin_amdgcn_exp2f(r - R), fb = __builtin_amdgcn_exp2f(r2 - R);
  s = (s + (r - R) * z) * fa + (s2 + (r2 - R) * z2) * fb;
  z = z * fa + z2 * fb;
  r = R;
}

// logits [rows][V] bf16, V a multiple of 8; entropy and argmax [rows].  Lane t's
// batch k holds the 16-byte chunks (k * kBatch + e) * 512 + t, e = 0..kBatch-1:
// every load instruction of a wave reads 1 KB of consecutive logits, and a lane's
// batches come in increasing index order.  -inf logits (masked tokens) are allowed; a
// row needs one finite logit.
__global__ __launch_bounds__(kStatThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void row_stats_kernel(const uint16_t* logits, int vocab,
                                                                 float c, float* entropy,
                                                                 int32_t* argmax) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t row = blockIdx.x;
  const uint4* src = (const uint4*)(logits + row * vocab);
  const int nchunks = vocab / 8;
  const int nbatches = (nchunks + kBatch * kStatThreads - 1) / (kBatch * kStatThreads);
  RowAcc a{-INFINITY, 0, -1e30f, 0.f, 0.f};

  // One batch: 8 * kBatch logits per lane, reduced into the lane's statistics.
  auto reduce_batch = [&](const uint4 (&v)[kBatch], int k) {
    float x[8 * kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; e++) {
      const uint32_t w[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        x[8 * e + 2 * q] = bf16_lo(w[q]);
        x[8 * e + 2 * q + 1] = bf16_hi(w[q]);
      }
    }
    const float cm = max_of(x);
    if (cm > a.best) {  // strict: a lane keeps the first batch that reached its max
      a.best = cm;
      a.bk = k;
    }
    // lazy reference (rare after the first batch): move the sums to cm * c
    const float rc = cm * c;
    if (rc > a.r + kRefSlack) {
      const float f = __builtin_amdgcn_exp2f(a.r - rc);
      a.s = (a.s + (a.r - rc) * a.z) * f;
      a.z *= f;
      a.r = rc;
    }
    float z = 0.f, s = 0.f;
#pragma unroll
    for (int j = 0; j < 8 * kBatch; j++) {
      // clamped so that a -inf logit (masked token) gives p = 0 and p * y = 0
      // (2^-200 is 0 in fp32); the kernel is bound by HBM, not by this max
      const float y = __builtin_fmaxf(__builtin_fmaf(x[j], c, -a.r), -200.f);
      const float p = __builtin_amdgcn_exp2f(y);
      z += p;
      s = __builtin_fmaf(p, y, s);
    }
    a.z += z;
    a.s += s;
  };

  // Batches wholly inside the row: loads without conditions into two register
  // buffers A and B, so that one batch is in flight while the other is reduced
  // (each buffer is refilled only after its reduction has read it, so no copies
  // between iterations are needed; the scheduling barriers keep every refill
  // ahead of the reduction that it is meant to overlap).  A refill past the last
  // full batch requests that batch again, from cache, instead of branching.
  const int nfull = nchunks / (kBatch * kStatThreads);
  auto load_full = [&](int k, uint4 (&v)[kBatch]) {
    const int c0 = min(k, nfull - 1) * kBatch * kStatThreads + t;
#pragma unroll
    for (int e = 0; e < kBatch; e++) v[e] = src[c0 + e * kStatThreads];
  };
  if (nfull > 0) {
    uint4 A[kBatch], B[kBatch];
    load_full(0, A);
    for (int k = 0; k < nfull; k += 2) {
      load_full(k + 1, B);
      __builtin_amdgcn_sched_barrier(0);
      reduce_batch(A, k);
      load_full(k + 2, A);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < nfull) reduce_batch(B, k + 1);
    }
  }
  // the partial last batch: chunks past the end of the row read as logits of
  // -1e30 (bf16 0xf149), for which 2^y is 0
  if (nfull < nbatches) {
    uint4 v[kBatch];
    const int c0 = nfull * kBatch * kStatThreads + t;
#pragma unroll
    for (int e = 0; e < kBatch; e++) {
      const int ci = c0 + e * kStatThreads;
      v[e] = ci < nchunks ? src[ci] : make_uint4(0xf149f149u, 0xf149f149u, 0xf149f149u, 0xf149f149u);
    }
    reduce_batch(v, nfull);
  }

  // ---- workgroup reduction of (max, sums): within each wave, then across waves
  __shared__ float red[4][kStatThreads / 64];
  __shared__ int red_i[kStatThreads / 64];
  float best = a.best, r = a.r, z = a.z, s = a.s;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    best = fmaxf(best, __shfl_xor(best, off));
    const float r2 = __shfl_xor(r, off), z2 = __shfl_xor(z, off), s2 = __shfl_xor(s, off);
    merge_sums(r, z, s, r2, z2, s2);
  }
  if (lane == 0) {
    red[0][wave] = best;
    red[1][wave] = r;
    red[2][wave] = z;
    red[3][wave] = s;
  }
  __syncthreads();
  float M = red[0][0];
  r = red[1][0];
  z = red[2][0];
  s = red[3][0];
#pragma unroll
  for (int w = 1; w < kStatThreads / 64; w++) {
    M = fmaxf(M, red[0][w]);
    merge_sums(r, z, s, red[1][w], red[2][w], red[3][w]);
  }

  // ---- argmax: the lowest index holding M.  A lane whose max is M reloads the
  //      first batch in which it saw it (a few hundred bytes per row in all).
  int cand = 0x7fffffff;
  if (a.best == M) {
    const int k = a.bk;
    const int c0 = k * kBatch * kStatThreads + t;
#pragma unroll
    for (int e = 0; e < kBatch; e++) {
      const int ci = c0 + e * kStatThreads;
      if (ci < nchunks) {
        const uint4 u = src[ci];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
          if (bf16_lo(w[q]) == M) cand = min(cand, ci * 8 + 2 * q);
          if (bf16_hi(w[q]) == M) cand = min(cand, ci * 8 + 2 * q + 1);
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cand = min(cand, __shfl_xor(cand, off));
  if (lane == 0) red_i[wave] = cand;
  __syncthreads();
  if (t == 0) {
    int idx = red_i[0];
#pragma unroll
    for (int w = 1; w < kStatThreads / 64; w++) idx = min(idx, red_i[w]);
    const float hbits = __log2f(z) - s / z;
    entropy[row] = fmaxf(0.f, hbits * 0.69314718055994531f);
    argmax[row] = idx;
  }
}

// kSelGroups workgroups per canvas, each deciding kCanvas / kSelGroups positions.
// Entropies count as integers of 2^-32 nats, q = rint(H * 2^32), so the cumulative
// sums are exact: position i is accepted iff the sum of q over every position
// ordered at or before it -- by (entropy, index) -- is within the budget.  As
// H >= 0 its bits order like its value: j is at or before i iff bits_j < bits_i,
// or bits_j == bits_i and j <= i.  Each of the 16 lanes of a position sums 16 of
// the 256 terms; every workgroup also forms the canvas total and the stability
// test itself (they need all 256 entries, 3 KB), so no workgroup waits for another.
constexpr int kSelGroups = 16;
constexpr int kSelPer = kCanvas / kSelGroups;  // positions per workgroup
static_assert(kSelPer * 16 == kCanvas, "16 lanes per position, 256 threads");

__global__ __launch_bounds__(kCanvas) void select_kernel(const float* entropy, const int32_t* argmax,
                                                         const int32_t* noise, const int32_t* prev,
                                                         long long qbudget, long long qstop,
                                                         int32_t* tokens, int32_t* accepted,
                                                         int32_t* stop) {
  const int t = threadIdx.x, b = blockIdx.y, grp = blockIdx.x;
  const int64_t base = (int64_t)b * kCanvas;
  __shared__ uint32_t bits[kCanvas];
  __shared__ long long qs[kCanvas];
  __shared__ long long wsum[kCanvas / 64];
  __shared__ int wstable[kCanvas / 64];
  {  // thread t loads entry t of the canvas
    const float H = entropy[base + t];
    const long long q = __float2ll_rn(H * 4294967296.0f);
    bits[t] = __float_as_uint(H);
    qs[t] = q;
    const bool same = prev != nullptr && prev[base + t] == argmax[base + t];
    long long sum = q;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    const bool all_same = __all(same);
    if ((t & 63) == 0) {
      wsum[t >> 6] = sum;
      wstable[t >> 6] = all_same ? 1 : 0;
    }
  }
  __syncthreads();
  const int i = grp * kSelPer + (t >> 4), sub = t & 15;  // position, lane within it
  const uint32_t hb = bits[i];
  long long before = 0;
#pragma unroll
  for (int e = 0; e < 16; e++) {
    const int j = sub * 16 + e;
    const uint32_t bj = bits[j];
    before += (bj < hb || (bj == hb && j <= i)) ? qs[j] : 0;
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) before += __shfl_xor(before, off);
  if (sub == 0) {
    const bool acc = before <= qbudget;
    accepted[base + i] = acc ? 1 : 0;
    tokens[base + i] = acc ? argmax[base + i] : noise[base + i];
  }
  if (grp == 0 && t == 0) {
    long long total = 0;
    int stable = 1;
#pragma unroll
    for (int w = 0; w < kCanvas / 64; w++) {
      total += wsum[w];
      stable &= wstable[w];
    }
    stop[b] = (total < (long long)kCanvas * qstop && stable) ? 1 : 0;
  }
}

}  // namespace

int launch_sample(const SampleArgs& s, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int rows = s.batch * kCanvas;
  hipLaunchKernelGGL(row_stats_kernel, dim3(rows), dim3(kStatThreads), 0, st,
                     (const uint16_t*)s.logits, s.vocab, s.c, s.entropy, s.argmax);
  int err = (int)hipGetLastError();
  if (err) return err;
  hipLaunchKernelGGL(select_kernel, dim3(kSelGroups, s.batch), dim3(kCanvas), 0, st, s.entropy, s.argmax,
                     s.noise, s.prev, s.qbudget, s.qstop, s.tokens, s.accepted, s.stop);
  return (int)hipGetLastError();
}

}  // namespace dg
