// dg_selfcond.hip -- the self-conditioning input z = FFW(softmax(logits) E) on gfx950.
//
// "DiffusionGemma Technical Report" (paperfeed.app summary), section "The
// mechanism: an AR model turned inside out", self-conditioning paragraph: the
// decoder also receives z_t = FFW(p0_hat E), the previous step's predicted token
// distribution times the embedding matrix, through a small MLP.  Here p0_hat =
// softmax(logits) (temperature 1) and FFW(y) = gelu(y W1) W2 (GELU in tanh form).
//
// Three kernels, seven launches per call:
//   * softmax_blocks_kernel: one wave per row and vocabulary split (8192
//     entries), four waves per block and one block per CU.  The split's logits
//     stay in registers: the wave takes the max, writes exp(x - max) rounded to
//     bf16, and the split's (max, sum of the rounded weights).  The weights go out in the blocked layout the product
//     kernel reads, [V/32][M][32] -- the 32 entries of a block of every row
//     consecutive -- so a stage of that kernel is one contiguous 16 KB tile; the
//     waves of adjacent rows in one block fill whole 128-byte lines.
//   * gemm_kernel<DT>: C = A B for A blocked as above (M rows, 256 per tile) and
//     B row-major [K][N] (the embedding table, W1, W2), split over K, fp32
//     partials.  Eight waves as 4 row quarters x 2 column halves; 32-row stages
//     stream HBM -> LDS with global_load_lds_dwordx4 through a ring of 5; A
//     operands by ds_read_b128, B operands by the transposing ds_read_b64_tr_b16
//     (B is row-major in K, the matrix cores want K inside a lane); products on
//     v_mfma_f32_32x32x16_bf16.  Units sharing an A tile (same rows and split,
//     other column tiles) are consecutive, so they run on one XCD and share its L2.
//   * reduce_kernel: sums the splits (for the embedding product with the softmax
//     weights 2^(m_s - M) and the division by the total sum), optionally applies
//     GELU, and writes bf16, blocked for the next product or row-major for z.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((ext_vector_type(16))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kTK = kSelfcondBlock;  // contraction rows per stage = entries per block
constexpr int kTileRows = 256;       // rows per product tile
constexpr int kStages = 5;           // LDS ring of the product kernel (160 KB at DT = 256)
constexpr int kMaxSplits = 64;       // splits a reduce takes (the vocabulary limit keeps to it)

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS char*)p;
}

// NL (1 or 2) global_load_lds_dwordx4 from scalar base sb + lane offset vo[e] +
// 1024e into LDS at m0 + 1024e + 16*lane (the instruction offset moves both).
template <int NL>
__device__ __forceinline__ void gll_block(const char* sb, const uint32_t* vo, uint32_t m0) {
  static_assert(NL == 1 || NL == 2, "one or two loads");
  if constexpr (NL == 1)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
                 ::"v"(vo[0]), "s"(m0), "s"(sb) : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %3\n\t"
                 "global_load_lds_dwordx4 %1, %3 offset:1024"
                 ::"v"(vo[0]), "v"(vo[1]), "s"(m0), "s"(sb) : "memory");
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---------------------------------------------------------------- softmax
// Block (split s, row group y): NW waves, RPW rows per wave (rows y*NW*RPW +
// wave*RPW ..).  Lane l holds 16-byte chunks l, l+64, ... of each row's split
// segment.  With one row per wave, two waves of a block write the two 64-byte
// halves of each 128-byte line.
template <int NW, int RPW>
__global__ __launch_bounds__(64 * NW) void softmax_blocks_kernel(SelfcondArgs a) {
  constexpr int CPL = kSelfcondSplit / 8 / 64;  // 16-byte chunks per lane and row
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int s = blockIdx.x, M = a.rows, V = a.vocab;
  const int r0 = NW * RPW * blockIdx.y + RPW * wave;
  const int v0 = s * kSelfcondSplit;
  const int nch = min(kSelfcondSplit, V - v0) / 8;  // valid chunks of the segment
  const float L2E = 1.4426950408889634f;
  // Reserved so that one block runs per CU.  Each wave requests its whole 16 KB
  // segment at once; four waves per CU keep 64 KB in flight (16 MB over the chip),
  // while the 8-wave blocks this replaces kept 128 KB and ran 10% slower: requests
  // beyond what keeps HBM busy only queue.  The store never runs (V >= 32).
  __shared__ char occupancy_pad[96 * 1024];
  if (V < 0) occupancy_pad[threadIdx.x] = 1;
  uint4 x[RPW][CPL];
#pragma unroll
  for (int rr = 0; rr < RPW; rr++) {
    const uint4* src = (const uint4*)((const uint16_t*)a.logits + (int64_t)(r0 + rr) * V + v0);
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      const int c = lane + 64 * j;
      x[rr][j] = c < nch ? src[c] : make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    }
  }
#pragma unroll
  for (int rr = 0; rr < RPW; rr++) {
    const int r = r0 + rr;
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      const uint32_t w[4] = {x[rr][j].x, x[rr][j].y, x[rr][j].z, x[rr][j].w};
#pragma unroll
      for (int q = 0; q < 4; q++)
        m = fmaxf(m, fmaxf(__uint_as_float(w[q] << 16), __uint_as_float(w[q] & 0xffff0000u)));
    }
    m = wave_max(m);
    // log2-domain max; a segment with no finite logit gets a finite sentinel so that
    // its weights are exp2(-inf) = 0 and its split drops out of the merge
    const float mt = m == -INFINITY ? -1e30f : m * L2E;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      const int c = lane + 64 * j;
      const uint32_t w[4] = {x[rr][j].x, x[rr][j].y, x[rr][j].z, x[rr][j].w};
      bf16x8 p;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        p[2 * q] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(w[q] << 16), L2E, -mt));
        p[2 * q + 1] =
            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(w[q] & 0xffff0000u), L2E, -mt));
      }
      if (c < nch) {
#pragma unroll
        for (int e = 0; e < 8; e++) sum += (float)p[e];  // the rounded weights the product uses
        const int64_t kb = (v0 >> 5) + (c >> 2);         // block of 32 entries
        *(bf16x8*)((uint16_t*)a.pblk + ((kb * M + r) << 5) + 8 * (c & 3)) = p;
      }
    }
    sum = wave_sum(sum);
    if (lane == 0) a.stats[(int64_t)s * M + r] = make_float2(mt, sum);
  }
}

// ---------------------------------------------------------------- products
struct GemmArgs {
  const void* a;  // blocked bf16 [K/32][M][32]
  const void* b;  // row-major bf16 [K][N]
  float* part;    // fp32 [S][M][N]
  int M, N, K, split_k, n_splits, n_ntiles;
};

template <int DT>
__global__ __launch_bounds__(512) void gemm_kernel(GemmArgs g) {
  constexpr int ABYTES = kTileRows * kTK * 2;  // 16 KB: A tile of a stage
  constexpr int ROWB = DT * 2;                 // bytes of one B row segment
  constexpr int BBYTES = kTK * ROWB;           // B tile of a stage
  constexpr int SLOT = ABYTES + BBYTES;
  constexpr int CH = ROWB / 16;                // 16-byte chunks per B row
  constexpr int RPL = 1024 / ROWB;             // B rows per 1 KB load
  constexpr int GB = BBYTES / 1024 / 8;        // B loads per wave and stage
  constexpr int GPW = 2 + GB;                  // loads per wave and stage
  constexpr int NCB = DT / 64;                 // 32-column blocks per wave
  static_assert(GB == 1 || GB == 2, "B loads per wave");
  __shared__ __attribute__((aligned(1024))) char ring[kStages * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int n = lane & 31, h = lane >> 5, g16 = lane >> 4;
  const int wr = wave & 3, wc = wave >> 2;
  // unit -> (row tile, split, column tile), column tile fastest
  const int U = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = U % g.n_ntiles, q = U / g.n_ntiles;
  const int s = q % g.n_splits, rt = q / g.n_splits;
  const int k0 = s * g.split_k, k1 = min(g.K, k0 + g.split_k);
  const int nstages = (k1 - k0) / kTK;
  const int n0 = nt * DT, M = g.M, N = g.N;

  // ---- per-lane load offsets (stage independent)
  // A: loads 2w, 2w+1 of the 16 per stage; load e covers tile rows 16e..16e+15,
  // lane l: row 16e + l/4, physical chunk l%4 holding logical chunk ^ ((row>>2)&3)
  uint32_t avo[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    avo[j] = (uint32_t)(row * 64 + 16 * ((lane & 3) ^ ((row >> 2) & 3))) - 2048u * wave - 1024u * j;
  }
  // B: loads GB*w .. ; load e covers rows e*RPL .., lane l: row e*RPL + l/CH,
  // physical chunk l%CH holding logical chunk ^ (4*(row&3) & (CH-1))
  uint32_t bvo[GB];
#pragma unroll
  for (int j = 0; j < GB; j++) {
    const int e = GB * wave + j, row = e * RPL + lane / CH, pc = lane % CH;
    bvo[j] = (uint32_t)row * (uint32_t)(N * 2) + 16u * (uint32_t)(pc ^ ((4 * (row & 3)) & (CH - 1))) -
             1024u * j;
  }
  const char* abase = (const char*)g.a + ((int64_t)rt * kTileRows) * 64;  // + kb*M*64 per stage
  const char* bbase = (const char*)g.b + (int64_t)n0 * 2;                 // + k*N*2 per stage
  const uint32_t lring = lds_addr(ring);
  auto issue = [&](int st, int slot) {
    const int k = k0 + st * kTK;
    const char* at = uniform_ptr(abase + (int64_t)(k >> 5) * M * 64 + 2048 * wave);
    gll_block<2>(at, avo, uniform(lring + slot * SLOT + 2048 * wave));
    const char* bt = uniform_ptr(bbase + (int64_t)k * N * 2);
    gll_block<GB>(bt, bvo, uniform(lring + slot * SLOT + ABYTES + 1024 * GB * wave));
  };

  // ---- operand read offsets within a stage
  // A operand of k-step t, row block rb: row 64wr + 32rb + n, logical chunk 2t + h
  uint32_t aro[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int row = 64 * wr + 32 * rb + n;
      aro[rb][t] = (uint32_t)(row * 64 + 16 * ((2 * t + h) ^ ((row >> 2) & 3)));
    }
  // B operand of k-step t, column block cb: two transposing reads of rows
  // 16t + 8h' + e4 (+4), h' = g16 >> 1; lane 4e4 + c of each 16-lane group supplies
  // columns 4c .. 4c+3 of its row within the group's 16 columns
  const int e4 = (lane & 15) >> 2;
  uint32_t bro[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; cb++)
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int row = 16 * t + 8 * (g16 >> 1) + e4;
      const int col = (DT / 2) * wc + 32 * cb + 16 * (g16 & 1) + 4 * (lane & 3);
      bro[cb][t] = ABYTES + (uint32_t)(row * ROWB + 16 * ((col >> 3) ^ ((4 * e4) & (CH - 1))) + 8 * (lane & 1));
    }

  f32x16 acc[2][NCB];
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[rb][cb][i] = 0.f;

  // ---- the ring: stage k in slot k mod kStages; after the barrier of stage k every
  //      wave is done with stage k-1, whose slot then takes stage k+kStages-1 (so
  //      kStages-1 stages are in flight while one is computed)
#pragma unroll
  for (int st = 0; st < kStages - 1; st++)
    if (st < nstages) issue(st, st);
  for (int k0s = 0; k0s < nstages; k0s += kStages) {
#pragma unroll
    for (int j = 0; j < kStages; j++) {
      const int k = k0s + j;
      if (k >= nstages) break;
      if (k + kStages - 2 < nstages)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kStages - 2) * GPW) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (k + kStages - 1 < nstages) issue(k + kStages - 1, (j + kStages - 1) % kStages);
      const uint32_t sb = lring + (uint32_t)j * SLOT;
#pragma unroll
      for (int t = 0; t < 2; t++) {
        bf16x8 av[2], bv[NCB];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) av[rb] = *(const LDS_AS bf16x8*)(uintptr_t)(sb + aro[rb][t]);
#pragma unroll
        for (int cb = 0; cb < NCB; cb++) {
          const LDS_AS char* p = (const LDS_AS char*)(uintptr_t)(sb + bro[cb][t]);
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 4 * ROWB));
          bv[cb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
          for (int cb = 0; cb < NCB; cb++)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[rb], bv[cb], acc[rb][cb], 0, 0, 0);
      }
    }
  }

  // ---- fp32 partials: lane (n, h) holds column n of rows 8(i/4) + 4h + i%4
  float* out = g.part + ((int64_t)s * M + (int64_t)rt * kTileRows) * N + n0;
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int row = 64 * wr + 32 * rb + 8 * (i >> 2) + 4 * h + (i & 3);
        const int col = (DT / 2) * wc + 32 * cb + n;
        out[(int64_t)row * N + col] = acc[rb][cb][i];
      }
}

// ---------------------------------------------------------------- split sums
struct ReduceArgs {
  const float* part;    // [S][M][N]
  const float2* stats;  // weighted: [S][M] (log2-domain max, sum of weights)
  void* out;            // bf16: blocked [N/32][M][32] or row-major [M][N]
  int M, N, n_splits;
};

// GELU, tanh form, with tanh(u) = 1 - 2 / (exp(2u) + 1)
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  const float t = 1.f - 2.f / (__builtin_amdgcn_exp2f(2.f * 1.4426950408889634f * u) + 1.f);
  return 0.5f * x * (1.f + t);
}

// Block (x, row): 256 threads, thread t sums columns 2048x + 8t .. +7 of the row over
// the splits, eight splits' loads in flight at a time.  The split weights (softmax
// merge: 2^(m_s - M) / sum_s 2^(m_s - M) l_s; otherwise 1) are formed once per
// block by its first wave and shared through LDS.
template <bool WEIGHTED, bool GELU, bool BLOCKED>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs r) {
  __shared__ float wsh[kMaxSplits];
  const int row = blockIdx.y, S = r.n_splits;
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    float w = 0.f;
    if (WEIGHTED) {
      const float2 st = l < S ? r.stats[(int64_t)l * r.M + row] : make_float2(-1e30f, 0.f);
      const float mx = wave_max(st.x);
      w = l < S ? __builtin_amdgcn_exp2f(st.x - mx) : 0.f;
      const float den = wave_sum(w * st.y);
      w = den > 0.f ? w / den : 0.f;
    } else {
      w = 1.f;
    }
    if (l < S) wsh[l] = w;
  }
  __syncthreads();
  const int c = 2048 * blockIdx.x + 8 * threadIdx.x;
  if (c >= r.N) return;
  const float* src = r.part + (int64_t)row * r.N + c;
  const int64_t sstride = (int64_t)r.M * r.N;
  // two float4 accumulators (a local array here ends up in scratch memory)
  float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float4 v0[8], v1[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
      const bool ok = s0 + j < S;
      v0[j] = ok ? *(const float4*)(src + (s0 + j) * sstride) : zero;
      v1[j] = ok ? *(const float4*)(src + (s0 + j) * sstride + 4) : zero;
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float w = s0 + j < S ? wsh[s0 + j] : 0.f;
      a0.x = fmaf(w, v0[j].x, a0.x);
      a0.y = fmaf(w, v0[j].y, a0.y);
      a0.z = fmaf(w, v0[j].z, a0.z);
      a0.w = fmaf(w, v0[j].w, a0.w);
      a1.x = fmaf(w, v1[j].x, a1.x);
      a1.y = fmaf(w, v1[j].y, a1.y);
      a1.z = fmaf(w, v1[j].z, a1.z);
      a1.w = fmaf(w, v1[j].w, a1.w);
    }
  }
  const float o[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; e++) b[e] = (__bf16)(GELU ? gelu_tanh(o[e]) : o[e]);
  const int64_t off = BLOCKED ? (((int64_t)(c >> 5) * r.M + row) << 5) + (c & 31) : (int64_t)row * r.N + c;
  *(bf16x8*)((uint16_t*)r.out + off) = b;
}

template <int DT>
int launch_gemm(const GemmArgs& g, hipStream_t st) {
  const int units = (g.M / kTileRows) * g.n_splits * g.n_ntiles;
  hipLaunchKernelGGL((gemm_kernel<DT>), dim3(units), dim3(512), 0, st, g);
  return (int)hipGetLastError();
}

template <bool W, bool G, bool B>
int launch_reduce(const ReduceArgs& r, hipStream_t st) {
  hipLaunchKernelGGL((reduce_kernel<W, G, B>), dim3((r.N + 2047) / 2048, r.M), dim3(256), 0, st, r);
  return (int)hipGetLastError();
}

// one product plus its split sum; the embedding product (mode 0) takes 256-wide
// column tiles, the MLP's smaller products 128-wide ones (more units to spread)
int product(const void* a, const void* b, int M, int N, int K, int split_k, float* part, const float2* stats,
            void* out, int mode, hipStream_t st, const SelfcondArgs& sa, int timed) {
  const int dt = mode == 0 ? 256 : 128;
  GemmArgs g;
  g.a = a;
  g.b = b;
  g.part = part;
  g.M = M;
  g.N = N;
  g.K = K;
  g.split_k = split_k;
  g.n_splits = (K + split_k - 1) / split_k;
  g.n_ntiles = N / dt;
  if (timed && sa.time_begin) sa.time_begin(0, st);
  int err = dt == 256 ? launch_gemm<256>(g, st) : launch_gemm<128>(g, st);
  if (timed && sa.time_end) sa.time_end(0, st);
  if (err) return err;
  ReduceArgs r;
  r.part = part;
  r.stats = stats;
  r.out = out;
  r.M = M;
  r.N = N;
  r.n_splits = g.n_splits;
  if (mode == 0) return launch_reduce<true, false, true>(r, st);   // y: softmax merge, blocked
  if (mode == 1) return launch_reduce<false, true, true>(r, st);   // gelu(y W1), blocked
  return launch_reduce<false, false, false>(r, st);                // z, row-major
}

}  // namespace

int selfcond_splits(int K, int N, int M, int cus) {
  // splits of an MLP product's contraction (128-wide column tiles) so that its
  // units fill the device about once
  const int tiles = (M / kTileRows) * (N / 128);
  int S = min((cus + tiles - 1) / tiles, kMaxSplits);
  int sk = (K + S - 1) / S;
  sk = ((sk + kTK - 1) / kTK) * kTK;
  return sk;
}

int launch_selfcond(const SelfcondArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int M = a.rows;
  if (a.time_begin) a.time_begin(1, st);
  // one row per wave measured 10% faster than two rows per wave (240 VGPRs), and
  // blocks of four waves held to one per CU 10% faster than blocks of eight
  hipLaunchKernelGGL((softmax_blocks_kernel<4, 1>), dim3(a.vocab_splits, M / 4), dim3(256), 0, st, a);
  if (a.time_end) a.time_end(1, st);
  int err = (int)hipGetLastError();
  if (err) return err;
  err = product(a.pblk, a.embed, M, a.d_model, a.vocab, kSelfcondSplit, a.part, a.stats, a.yblk, 0, st, a, 1);
  if (err) return err;
  err = product(a.yblk, a.w1, M, a.d_hidden, a.d_model, a.split_w1, a.part, nullptr, a.hblk, 1, st, a, 0);
  if (err) return err;
  return product(a.hblk, a.w2, M, a.d_model, a.d_hidden, a.split_w2, a.part, nullptr, a.z, 2, st, a, 0);
}

}  // namespace dg
