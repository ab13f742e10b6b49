// dg_attn_bf16.hip -- split-key canvas / commit attention, bf16 in, fp32 accumulate (gfx950).
//
// Computes, for one work unit (sequence b, kv head g, key split s, row tile rt),
// softmax attention of R packed query rows against the unit's keys, where the
// key space is [cache rows 0..L-1 ; canvas or block rows 0..255]:
//   * canvas step: no mask (bidirectional canvas that cross-attends to the
//     cache; "DiffusionGemma Technical Report", paperfeed.app summary, section
//     "The mechanism: an AR model turned inside out", decoder bullet);
//   * commit: block row i sees block keys 0..i only (the causal encoder bullet
//     of the same section), and the block K/V are copied into cache rows
//     L..L+255 by the same launch (the finished canvas is appended).
//
// Design (CDNA4):
//   * A workgroup is 4 wave64s = WM row groups x WK key groups.  Each wave owns
//     64 packed query rows (two 32-row MFMA blocks); its queries stay in VGPRs.
//   * GQA packing: the G query heads of kv head g are rows p = i*G + hh of one
//     256*G-row matrix, so every K/V tile read from LDS feeds 64 query rows per
//     wave and WM waves per key group.
//   * Scores are computed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//     (M = 32 keys, N = 32 queries): each lane then holds 16 scores of ONE query,
//     so softmax needs no cross-lane reduction except a v_permlane32_swap with
//     the lane holding the other 16 keys.  The score registers, exponentiated and
//     packed to bf16, are used directly as the B operand of O^T += V^T P^T
//     (K = 16 keys per MFMA): the key order inside each MFMA is permuted
//     consistently for P and V, which costs nothing because keys are summed over.
//   * K/V tiles stream HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging)
//     into a 3-slot ring, one workgroup barrier per tile.  Rows are stored densely
//     (D*2 bytes) with an XOR swizzle of the 16-byte chunks so that the K operand
//     reads (ds_read_b128, one key row per lane) and the V operand reads
//     (ds_read_b64_tr_b16, the gfx950 transposing LDS read) are bank-conflict
//     free.  The ring slots are separate LDS objects and the stage loop is
//     unrolled by three, so the compiler can tell the slot being filled from the
//     slot being read and never waits on a prefetch it does not need.
//   * Softmax runs in the log2 domain with a lazily raised reference max: a
//     chunk's exact max is always formed, but the output is rescaled only when it
//     exceeds the reference by more than 64 (so every exponential stays <= 2^64);
//     in steady state a chunk costs max, FMA, exp2, a bf16 pack and a dot2 sum
//     per score.  The result is exact attention; only the point at which the max
//     is folded in moves.
//   * Key groups of a workgroup are merged through LDS at the end; the unit
//     writes its normalised partial rows (fp32) plus (max, sum), or the final
//     bf16 output when the sequence has a single split.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kRescaleThreshold = 64.f;  // log2 units

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // range of logical units so units that share K/V tiles share an L2.
  const int x = bid % kNumXcd, j = bid / kNumXcd;
  return x * (n / kNumXcd) + min(x, n % kNumXcd) + j;
}

struct Unit {
  int b, g, s, rt;
};

__device__ __forceinline__ Unit decode_unit(const Plan& p, int U) {
  int b = 0;
  for (int i = 1; i < p.batch; i++)
    if (U >= p.seq[i].unit_base) b = i;
  const int local = U - p.seq[b].unit_base;
  const int S = p.seq[b].n_splits, NRT = p.n_rowtiles;
  Unit u;
  u.b = b;
  u.g = local / (S * NRT);
  u.s = (local / NRT) % S;
  u.rt = local % NRT;
  return u;
}

__device__ __forceinline__ float partner_max(float x) {
  // lanes l and l^32 exchange through v_permlane32_swap; max of both halves
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float partner_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int NB, int MB>
struct State {
  f32x16 o[NB][MB];  // O^T accumulators: lane (n, h) holds d = 32mb + 8(i/4) + 4h + i%4 of query n
  float mlog[NB];    // reference max of the lane's query, log2 domain
  float lsum[NB];    // sum of this lane's exponentials (the partner lane holds the rest)
};

struct TileSrc {
  const uint16_t *kc, *vc;  // cache K/V of (sequence, kv head), row 0
  const uint16_t *kn, *vn;  // canvas/block K/V of (sequence, kv head), row 0
  int64_t row_stride;       // elements between consecutive rows (Hkv * D)
  int L;                    // cache rows; key j >= L is canvas row j - L
  int kstop;                // end of the unit's keys; later rows are clamped onto kstop-1
};

// Issues this wave's share of the global_load_lds instructions that copy one tile
// (TK keys of K, then TK keys of V) into LDS at kt.  Each instruction moves 1 KB:
// lane l writes 16 bytes at kt + 1024*instr + 16*l, i.e. tile row l / CH, physical
// chunk l % CH; it fetches the logical chunk that the swizzle puts there.
template <int D, int TK, int WM>
__device__ __forceinline__ void issue_tile(char* kt, int tkey0, const TileSrc& t, int rg,
                                           int lane) {
  constexpr int CH = D / 8, RPI = 1024 / (D * 2), IPT = TK / RPI;  // instructions per K tile
  constexpr int GLL = 2 * IPT / WM;
#pragma unroll
  for (int e = 0; e < GLL; e++) {
    const int instr = rg + WM * e;
    const bool isv = instr >= IPT;
    const int ri = instr % IPT;
    const int r = ri * RPI + lane / CH;
    const int p = lane % CH;
    const int c = isv ? (p ^ ((4 * (r & 3)) & (CH - 1))) : (p ^ (r & (CH - 1)));
    const int key = min(tkey0 + r, t.kstop - 1);
    const uint16_t* row = key < t.L ? (isv ? t.vc : t.kc) + (int64_t)key * t.row_stride
                                    : (isv ? t.vn : t.kn) + (int64_t)(key - t.L) * t.row_stride;
    char* dst = kt + (isv ? TK * D * 2 : 0) + ri * 1024;
    __builtin_amdgcn_global_load_lds((const void*)(row + 8 * c), (LDS_AS void*)dst, 16, 0, 0);
  }
}

// One 32-key chunk: S^T = K Q^T, softmax numerators, O^T += V^T P^T.
// kt/vt point at the chunk's first K/V row in LDS (chunks start at multiples of
// 32 tile rows, which keeps the swizzle phase).
template <int D, bool CAUSAL, int NB>
__device__ __forceinline__ void compute_chunk(const char* kt, const char* vt, int key0, int kstop,
                                              int L, int wave_qi_min, const int (&qi)[NB],
                                              const bf16x8 (&qr)[NB][D / 16], float c2, int lane,
                                              State<NB, D / 32>& acc) {
  constexpr int KS = D / 16, CH = D / 8, MB = D / 32, ROWB = D * 2;
  const int n = lane & 31, h = lane >> 5;
  // K operand: lane (n, h) reads key row n, logical chunk (D/16)*h + ks
  bf16x8 kop[KS];
  const char* kp = kt + n * ROWB;
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
    kop[ks] = *(const bf16x8*)(kp + 16 * (((D / 16) * h + ks) ^ (n & (CH - 1))));
  f32x16 s[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++)
#pragma unroll
    for (int i = 0; i < 16; i++) s[nb][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
      s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qr[nb][ks], s[nb], 0, 0, 0);
  // masks: ragged end of the unit's keys and, for the commit, block keys past the diagonal
  const bool tail = key0 + 32 > kstop;
  const bool diag = CAUSAL && (key0 + 31 - L > wave_qi_min);
  if (tail || diag) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int key = key0 + 8 * (i / 4) + 4 * h + (i % 4);
        bool ok = key < kstop;
        if (CAUSAL) ok = ok && (key < L || key - L <= qi[nb]);
        s[nb][i] = ok ? s[nb][i] : -INFINITY;
      }
  }
  // lazily raised reference max
  float cm[NB];
  bool raise = false;
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    float m = s[nb][0];
#pragma unroll
    for (int i = 1; i < 16; i++) m = fmaxf(m, s[nb][i]);
    cm[nb] = m * c2;
    raise = raise || (cm[nb] > acc.mlog[nb] + kRescaleThreshold);
  }
  if (__any(raise)) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const float mnew = fmaxf(acc.mlog[nb], partner_max(cm[nb]));
      const float alpha = __builtin_amdgcn_exp2f(acc.mlog[nb] - mnew);
      acc.mlog[nb] = mnew;
      acc.lsum[nb] *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc.o[nb][mb][i] *= alpha;
    }
  }
  // numerators, packed to bf16 as the B operand; the row sum adds the packed values
  bf16x8 pb[NB][2];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    const float nm = -acc.mlog[nb];
    float sum = acc.lsum[nb];
#pragma unroll
    for (int t = 0; t < 2; t++) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        bf16x2 pr;
        pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][8 * t + j], c2, nm));
        pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][8 * t + j + 1], c2, nm));
        pb[nb][t][j] = pr[0];
        pb[nb][t][j + 1] = pr[1];
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
      }
    }
    acc.lsum[nb] = sum;
  }
  // O^T += V^T P^T; the A operand V^T comes from transposing LDS reads: in each
  // 16-lane group, lane 4e + c supplies 4 head_dim values of key row e, and lane i
  // receives column i of that 4-row block.
  const int g16 = lane >> 4, e4 = (lane & 15) >> 2;
  const int v_row = 4 * (g16 >> 1) + e4;
  const int v_chunk = 2 * (g16 & 1) + ((lane & 3) >> 1);
  const int v_half = (lane & 1) * 8;
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    const int chunk = 4 * mb + v_chunk;
    const char* vb = vt + v_row * ROWB + 16 * (chunk ^ ((4 * e4) & (CH - 1))) + v_half;
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const bf16x4 lo =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + 16 * t * ROWB));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + (16 * t + 8) * ROWB));
      const bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int nb = 0; nb < NB; nb++)
        acc.o[nb][mb] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[nb][t], acc.o[nb][mb], 0, 0, 0);
    }
  }
}

// Everything a pipeline stage needs besides the ring slots.
struct StageCtx {
  TileSrc src;
  int kbeg, kstop, L, ntiles, nstages, kg, rg, lane, wave_qi_min, wave_qi_max;
  float c2;
};

// One stage of the ring: wait for its tile, compute it, refill the slot freed by
// the previous stage.  `cur` and `refill` are this key group's slots.
template <int D, bool CAUSAL, int WM, int WK, int TK, int NB>
__device__ __forceinline__ void run_stage(int st, const char* cur, char* refill, const StageCtx& c,
                                          const int (&qi)[NB], const bf16x8 (&qr)[NB][D / 16],
                                          State<NB, D / 32>& acc) {
  constexpr int ROWB = D * 2, TILEB = TK * ROWB, RPI = 1024 / ROWB;
  constexpr int GLL = 2 * TK / RPI / WM;
  // This wave's loads of stage st must have landed; stage st+1 may stay in flight.
  // The barrier then also certifies that every wave finished stage st-1, whose
  // slot is refilled below.
  const bool next_in_flight = st + 1 < c.nstages && (st + 1) * WK + c.kg < c.ntiles;
  if (next_in_flight)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(GLL) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const int t = st * WK + c.kg;
  if (t < c.ntiles) {
    const int tkey0 = c.kbeg + t * TK;
#pragma unroll
    for (int cc = 0; cc < TK / 32; cc++) {
      const int key0 = tkey0 + 32 * cc;
      if (key0 >= c.kstop) break;
      if (CAUSAL && key0 >= c.L && key0 - c.L > c.wave_qi_max) break;
      compute_chunk<D, CAUSAL>(cur + 32 * cc * ROWB, cur + TILEB + 32 * cc * ROWB, key0, c.kstop,
                               c.L, c.wave_qi_min, qi, qr, c.c2, c.lane, acc);
    }
  }
  const int t2 = (st + 2) * WK + c.kg;
  if (st + 2 < c.nstages && t2 < c.ntiles)
    issue_tile<D, TK, WM>(refill, c.kbeg + t2 * TK, c.src, c.rg, c.lane);
}

template <int D, bool CAUSAL, int WM, int WK, int TK>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(AttnArgs a, Plan plan) {
  static_assert(WM * WK == 4, "four waves per workgroup");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int NB = 2;                 // 32-query MFMA blocks per wave
  constexpr int R = 64 * WM;            // packed rows per unit
  constexpr int KS = D / 16;            // MFMA k-steps over head_dim
  constexpr int CH = D / 8;             // 16-byte chunks per K/V row
  constexpr int MB = D / 32;            // 32-row blocks of O^T
  constexpr int ROWB = D * 2;           // bytes per K/V row
  constexpr int TILEB = TK * ROWB;      // bytes per K (or V) tile
  constexpr int RPI = 1024 / ROWB;      // rows one global_load_lds covers (64 lanes x 16 B)
  static_assert(2 * TK / RPI / WM >= 1 && (2 * TK / RPI) % WM == 0, "tile load split");
  constexpr int SLOTB = WK * 2 * TILEB; // one ring slot: K and V tiles of every key group
  constexpr int MERGEB = (WK - 1) * WM * 64 * (NB * MB * 16 + 2 * NB) * 4;
  static_assert(MERGEB <= SLOTB, "key-group merge fits in one ring slot");
  __shared__ __attribute__((aligned(1024))) char slot0[SLOTB];
  __shared__ __attribute__((aligned(1024))) char slot1[SLOTB];
  __shared__ __attribute__((aligned(1024))) char slot2[SLOTB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int rg = wave % WM, kg = wave / WM;
  const int U = xcd_remap(blockIdx.x, gridDim.x);
  const Unit u = decode_unit(plan, U);
  const SeqPlan sp = plan.seq[u.b];
  const int L = sp.prefix_len;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  const int row0 = u.rt * R;
  int kend = L + kCanvas;
  if (CAUSAL) kend = min(kend, L + (row0 + R - 1) / G + 1);
  const int kbeg = u.s * sp.split_keys;
  const int kstop = min(kbeg + sp.split_keys, kend);
  const int ntiles = kstop > kbeg ? (kstop - kbeg + TK - 1) / TK : 0;
  const int nstages = (ntiles + WK - 1) / WK;

  const int64_t cap = a.cap;
  const uint16_t* kc = (const uint16_t*)a.k_cache;
  const uint16_t* vc = (const uint16_t*)a.v_cache;
  const uint16_t* kn = (const uint16_t*)a.k_new;
  const uint16_t* vn = (const uint16_t*)a.v_new;

  // ---- commit: append the block's K/V rows of head g to cache rows L..L+255
  if (CAUSAL && a.k_append != nullptr) {
    const int cnt = sp.n_splits * plan.n_rowtiles;
    const int w = u.s * plan.n_rowtiles + u.rt;
    const int rpu = (kCanvas + cnt - 1) / cnt;
    const int r0 = min(kCanvas, w * rpu), r1 = min(kCanvas, r0 + rpu);
    const int per = (r1 - r0) * CH;
    for (int idx = tid; idx < 2 * per; idx += 256) {
      const int which = idx / per, rem = idx % per;
      const int r = r0 + rem / CH, c = rem % CH;
      const int64_t src = ((int64_t)(u.b * kCanvas + r) * Hkv + u.g) * D + c * 8;
      const int64_t dst = (((int64_t)u.b * cap + L + r) * Hkv + u.g) * D + c * 8;
      const uint4 val = *(const uint4*)((which ? vn : kn) + src);
      *(uint4*)((uint16_t*)(which ? a.v_append : a.k_append) + dst) = val;
    }
  }

  // ---- queries of this wave: B operand of S^T = K Q^T, lane (n, h) holds
  //      q[row][D/2*h + 8*ks .. +8] for k-step ks (a fixed permutation of head_dim
  //      shared with the K operand)
  bf16x8 qr[NB][KS];
  int qi[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    const int prow = row0 + 64 * rg + 32 * nb + n;
    const int i = prow / G, hh = prow % G;
    qi[nb] = i;
    const uint16_t* qp = (const uint16_t*)a.q +
                         ((int64_t)(u.b * kCanvas + i) * Hq + u.g * G + hh) * D + (D / 2) * h;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qr[nb][ks] = *(const bf16x8*)(qp + 8 * ks);
  }

  StageCtx ctx;
  ctx.src.kc = kc + ((int64_t)u.b * cap * Hkv + u.g) * D;
  ctx.src.vc = vc + ((int64_t)u.b * cap * Hkv + u.g) * D;
  ctx.src.kn = kn + ((int64_t)u.b * kCanvas * Hkv + u.g) * D;
  ctx.src.vn = vn + ((int64_t)u.b * kCanvas * Hkv + u.g) * D;
  ctx.src.row_stride = (int64_t)Hkv * D;
  ctx.src.L = L;
  ctx.src.kstop = kstop;
  ctx.kbeg = kbeg;
  ctx.kstop = kstop;
  ctx.L = L;
  ctx.ntiles = ntiles;
  ctx.nstages = nstages;
  ctx.kg = kg;
  ctx.rg = rg;
  ctx.lane = lane;
  ctx.wave_qi_min = (row0 + 64 * rg) / G;
  ctx.wave_qi_max = (row0 + 64 * rg + 63) / G;
  ctx.c2 = a.scale_log2;

  State<NB, MB> acc;
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc.o[nb][mb][i] = 0.f;
    acc.mlog[nb] = -1e30f;  // log2-domain reference max; finite so rescales never form inf-inf
    acc.lsum[nb] = 0.f;
  }

  // ---- 3-slot ring over the stages; stage st processes tile st*WK + kg
  char* s0 = slot0 + kg * 2 * TILEB;
  char* s1 = slot1 + kg * 2 * TILEB;
  char* s2 = slot2 + kg * 2 * TILEB;
  if (kg < ntiles) issue_tile<D, TK, WM>(s0, kbeg + kg * TK, ctx.src, rg, lane);
  if (1 < nstages && WK + kg < ntiles)
    issue_tile<D, TK, WM>(s1, kbeg + (WK + kg) * TK, ctx.src, rg, lane);
  for (int st = 0; st < nstages; st += 3) {
    run_stage<D, CAUSAL, WM, WK, TK>(st, s0, s2, ctx, qi, qr, acc);
    if (st + 1 < nstages) run_stage<D, CAUSAL, WM, WK, TK>(st + 1, s1, s0, ctx, qi, qr, acc);
    if (st + 2 < nstages) run_stage<D, CAUSAL, WM, WK, TK>(st + 2, s2, s1, ctx, qi, qr, acc);
  }

  // ---- merge the key groups through LDS (group 0 keeps the result)
  if (WK > 1) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float* mbuf = (float*)slot0;
    constexpr int PER = NB * MB * 16 + 2 * NB;  // floats per lane
    if (kg > 0) {
      float* dst = mbuf + ((kg - 1) * WM + rg) * 64 * PER;
      int k = 0;
#pragma unroll
      for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int i = 0; i < 16; i++) dst[(k++) * 64 + lane] = acc.o[nb][mb][i];
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        dst[(k++) * 64 + lane] = acc.mlog[nb];
        dst[(k++) * 64 + lane] = acc.lsum[nb];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kg > 0) return;
#pragma unroll
    for (int og = 1; og < WK; og++) {
      const float* src = mbuf + ((og - 1) * WM + rg) * 64 * PER;
      constexpr int MOFF = NB * MB * 16;
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const float m2 = src[(MOFF + 2 * nb) * 64 + lane];
        const float l2 = src[(MOFF + 2 * nb + 1) * 64 + lane];
        const float mn = fmaxf(acc.mlog[nb], m2);
        const float a1 = __builtin_amdgcn_exp2f(acc.mlog[nb] - mn);
        const float a2 = __builtin_amdgcn_exp2f(m2 - mn);
        acc.mlog[nb] = mn;
        acc.lsum[nb] = acc.lsum[nb] * a1 + l2 * a2;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int i = 0; i < 16; i++)
            acc.o[nb][mb][i] =
                acc.o[nb][mb][i] * a1 + src[((nb * MB + mb) * 16 + i) * 64 + lane] * a2;
      }
    }
  }

  // ---- write the unit's rows
  const bool direct = sp.n_splits == 1;
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    const float lt = partner_sum(acc.lsum[nb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int prow = row0 + 64 * rg + 32 * nb + n;
    if (direct) {
      const int i = prow / G, hh = prow % G;
      uint16_t* op = (uint16_t*)a.out + ((int64_t)(u.b * kCanvas + i) * Hq + u.g * G + hh) * D;
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const int d = 32 * mb + 8 * q4 + 4 * h;
          typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4e;
          bf16x4e v;
#pragma unroll
          for (int j = 0; j < 4; j++) v[j] = (__bf16)(acc.o[nb][mb][4 * q4 + j] * inv);
          *(bf16x4e*)(op + d) = v;
        }
    } else {
      float* po = a.part_o + ((int64_t)U * R + (prow - row0)) * D;
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const int d = 32 * mb + 8 * q4 + 4 * h;
          float4 v;
          v.x = acc.o[nb][mb][4 * q4 + 0] * inv;
          v.y = acc.o[nb][mb][4 * q4 + 1] * inv;
          v.z = acc.o[nb][mb][4 * q4 + 2] * inv;
          v.w = acc.o[nb][mb][4 * q4 + 3] * inv;
          *(float4*)(po + d) = v;
        }
      if (h == 0) {
        float2 ml;
        ml.x = acc.mlog[nb];
        ml.y = lt;
        *(float2*)(a.part_ml + ((int64_t)U * R + (prow - row0)) * 2) = ml;
      }
    }
  }
}

template <int D, bool CAUSAL>
int launch_variant(const AttnArgs& a, const Plan& p, hipStream_t st) {
  // 4 row groups share every K/V tile: 256 rows per unit, 64-key tiles
  hipLaunchKernelGGL((attn_bf16_kernel<D, CAUSAL, 4, 1, 64>), dim3(p.n_units), dim3(256), 0, st,
                     a, p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_attn_bf16(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (p.n_units == 0) return 0;
  if (head_dim == 128)
    return causal ? launch_variant<128, true>(a, p, st) : launch_variant<128, false>(a, p, st);
  return causal ? launch_variant<64, true>(a, p, st) : launch_variant<64, false>(a, p, st);
}

}  // namespace dg
