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
//   * A workgroup is NW wave64s = WM row groups x WK key groups.  Each wave owns
//     32*NB packed query rows held in VGPRs.  With NW = 8 two waves share each
//     SIMD, so one wave's MFMAs overlap the other's softmax arithmetic and the
//     register budget (256 per wave) keeps every MFMA in VGPR form.
//   * GQA packing: the G query heads of kv head g are rows p = i*G + hh of one
//     256*G-row matrix, so every K/V tile read from LDS feeds all query heads of
//     the group at once.
//   * Scores are computed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//     (M = 32 keys, N = 32 queries): each lane then holds 16 scores of ONE query,
//     so softmax needs no cross-lane reduction except a v_permlane32_swap with
//     the lane holding the other 16 keys.  The score registers, exponentiated and
//     packed to bf16, are used directly as the B operand of O^T += V^T P^T
//     (K = 16 keys per MFMA): the key order inside each MFMA is permuted
//     consistently for P and V, which costs nothing because keys are summed over.
//   * K/V tiles stream HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging)
//     into an NST-slot ring, one workgroup barrier per tile.  Whole tiles inside
//     the cache or the canvas use a scalar base plus precomputed 32-bit lane
//     offsets; only a tile that crosses the cache/canvas seam or the end of the
//     unit takes the per-lane path.  Rows are stored densely (D*2 bytes) with an
//     XOR swizzle of the 16-byte chunks so that the K operand reads
//     (ds_read_b128, one key row per lane) and the V operand reads
//     (ds_read_b64_tr_b16, the gfx950 transposing LDS read) are bank-conflict
//     free.
//   * Softmax runs in the log2 domain with a lazily raised reference max: a
//     chunk's exact max is always formed, but the output is rescaled only when it
//     exceeds the reference by more than 64 (so every exponential stays <= 2^64);
//     in steady state a score costs max, FMA, exp2, a bf16 pack and a dot2 sum.
//     The result is exact attention; only the point at which the max is folded
//     in moves.
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS char*)p;
}

template <int MB>
struct State {
  f32x16 o[MB];  // O^T accumulators: lane (n, h) holds d = 32mb + 8(i/4) + 4h + i%4 of query n
  float mlog;    // reference max of the lane's query, log2 domain
  float lsum;    // sum of this lane's exponentials (the partner lane holds the rest)
};

// Where a key group's tiles come from.
struct TileSrc {
  const char *kc, *vc;  // cache K/V of (sequence, kv head), row 0
  const char *kn, *vn;  // canvas/block K/V of (sequence, kv head), row 0
  int rsb;              // bytes between consecutive rows (Hkv * D * 2)
  int L;                // cache rows; key j >= L is canvas row j - L
  int kstop;            // end of the unit's keys; later rows are clamped onto kstop-1
  uint32_t lrs;         // lane row offset (lane / CH) * rsb
  int lp;               // lane physical chunk (lane % CH)
  int lr;               // lane row within one load instruction (lane / CH)
};

// One global_load_lds_dwordx4: every lane copies 16 bytes from its global address
// into LDS at m0 + 16*lane.  Issued from inline asm so that the compiler does not
// see an LDS write it cannot disambiguate from the operand reads of the other
// ring slot (it would otherwise drain every prefetch before the first of them);
// completion is tracked explicitly with s_waitcnt vmcnt before each stage's
// barrier.  Nothing else in the kernel uses m0.
__device__ __forceinline__ void gll_saddr(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds)
               : "memory");
}
__device__ __forceinline__ void gll_vaddr(const char* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vaddr), "s"(lds)
               : "memory");
}

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Issues this wave's share of the global_load_lds instructions that copy one tile
// (TK keys of K, then TK keys of V) into LDS at kt.  Each instruction moves 1 KB:
// lane l writes 16 bytes at kt + 1024*instr + 16*l, i.e. tile row l / CH, physical
// chunk l % CH, and fetches the logical chunk that the swizzle stores there
// (K: chunk ^ (row % CH); V: chunk ^ 4*(row % 4)).
template <int D, int TK, int WM>
__device__ __forceinline__ void issue_tile(uint32_t kt, int tkey0, const TileSrc& t, int rg) {
  constexpr int CH = D / 8, RPI = 1024 / (D * 2), IPT = TK / RPI;  // instructions per K tile
  constexpr int GLL = 2 * IPT / WM;
  const bool in_cache = tkey0 + TK <= t.L && tkey0 + TK <= t.kstop;
  const bool in_canvas = tkey0 >= t.L && tkey0 + TK <= t.kstop;
  if (in_cache || in_canvas) {
    // whole tile from one tensor: scalar base + 32-bit lane offset
    const char* kb = in_cache ? t.kc + (int64_t)tkey0 * t.rsb : t.kn + (int64_t)(tkey0 - t.L) * t.rsb;
    const char* vb = in_cache ? t.vc + (int64_t)tkey0 * t.rsb : t.vn + (int64_t)(tkey0 - t.L) * t.rsb;
#pragma unroll
    for (int e = 0; e < GLL; e++) {
      const int instr = rg + WM * e;
      const bool isv = instr >= IPT;
      const int ri = instr % IPT;
      const int r0 = ri * RPI;  // first tile row of this instruction (uniform)
      const int sw = isv ? ((4 * (t.lr & 3)) & (CH - 1)) : ((r0 + t.lr) & (CH - 1));
      const uint32_t off = t.lrs + 16u * (uint32_t)(t.lp ^ sw);
      const char* base = uniform_ptr((isv ? vb : kb) + (int64_t)r0 * t.rsb);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(kt + (isv ? TK * D * 2 : 0) + ri * 1024);
      gll_saddr(base, off, dst);
    }
  } else {
#pragma unroll
    for (int e = 0; e < GLL; e++) {
      const int instr = rg + WM * e;
      const bool isv = instr >= IPT;
      const int ri = instr % IPT;
      const int r = ri * RPI + t.lr;
      const int c = isv ? (t.lp ^ ((4 * (r & 3)) & (CH - 1))) : (t.lp ^ (r & (CH - 1)));
      const int key = min(tkey0 + r, t.kstop - 1);
      const char* row = key < t.L ? (isv ? t.vc : t.kc) + (int64_t)key * t.rsb
                                  : (isv ? t.vn : t.kn) + (int64_t)(key - t.L) * t.rsb;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(kt + (isv ? TK * D * 2 : 0) + ri * 1024);
      gll_vaddr(row + 16 * c, dst);
    }
  }
}

// V^T operands of one 32-key chunk: vop[mb][t] holds, in lane (d, h), the values
// of keys 16t + 8r + 4h + e (k-slot 4r + e) at head_dim 32mb + d, read with the
// transposing ds_read_b64_tr_b16.
template <int D>
__device__ __forceinline__ void load_v_operands(uint32_t vbase, const uint32_t (&voff)[D / 32],
                                                bf16x8 (&vop)[D / 32][2]) {
  constexpr int ROWB = D * 2, MB = D / 32;
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    const LDS_AS char* p = (const LDS_AS char*)(uintptr_t)(vbase + voff[mb]);
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 16 * t * ROWB));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + (16 * t + 8) * ROWB));
      vop[mb][t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// Per-lane LDS offsets of the K and V operand reads within a 32-key chunk.
template <int D>
struct LaneOffsets {
  uint32_t k[D / 16];  // ds_read_b128 of key row n, logical chunk (D/16)*h + ks
  uint32_t v[D / 32];  // ds_read_b64_tr_b16 of head_dim block mb (row 4*(g16/2) + e)
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int lane) {
  constexpr int CH = D / 8, ROWB = D * 2;
  LaneOffsets<D> o;
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ks++)
    o.k[ks] = n * ROWB + 16 * (((D / 16) * h + ks) ^ (n & (CH - 1)));
  // transposing reads: in each 16-lane group, lane 4e + c supplies 4 head_dim
  // values of key row e, and lane i receives column i of that 4-row block
  const int g16 = lane >> 4, e4 = (lane & 15) >> 2;
  const int v_row = 4 * (g16 >> 1) + e4;
  const int v_chunk = 2 * (g16 & 1) + ((lane & 3) >> 1);
#pragma unroll
  for (int mb = 0; mb < D / 32; mb++)
    o.v[mb] = v_row * ROWB + 16 * ((4 * mb + v_chunk) ^ ((4 * e4) & (CH - 1))) + (lane & 1) * 8;
  return o;
}

// K operands of one 32-key chunk: kop[ks] = key row n, logical chunk
// (D/16)*h + ks (the A operand of S^T = K Q^T).
template <int D>
__device__ __forceinline__ void load_k_operands(uint32_t kbase, const uint32_t (&koff)[D / 16],
                                                bf16x8 (&kop)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ks++)
    kop[ks] = *(const LDS_AS bf16x8*)(uintptr_t)(kbase + koff[ks]);
}

template <int D>
__device__ __forceinline__ void scores(const bf16x8 (&kop)[D / 16], const bf16x8 (&qr)[D / 16],
                                       f32x16& s) {
#pragma unroll
  for (int i = 0; i < 16; i++) s[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ks++)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qr[ks], s, 0, 0, 0);
}

// Masks a chunk's scores (ragged end of the unit; block keys past the diagonal
// for the commit), folds the chunk max into the reference max when it rises by
// more than the threshold, and returns nothing else: the exponentials follow.
template <int MB, bool CAUSAL>
__device__ __forceinline__ void prepare_scores(f32x16& s, int key0, int kstop, int L,
                                               int wave_qi_min, int qi, int h, float c2,
                                               State<MB>& acc) {
  const bool tail = key0 + 32 > kstop;
  const bool diag = CAUSAL && (key0 + 31 - L > wave_qi_min);
  if (tail || diag) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int key = key0 + 8 * (i / 4) + 4 * h + (i % 4);
      bool ok = key < kstop;
      if (CAUSAL) ok = ok && (key < L || key - L <= qi);
      s[i] = ok ? s[i] : -INFINITY;
    }
  }
  float m = s[0];
#pragma unroll
  for (int i = 1; i < 16; i++) m = fmaxf(m, s[i]);
  const float cm = m * c2;
  if (__any(cm > acc.mlog + kRescaleThreshold)) {
    const float mnew = fmaxf(acc.mlog, partner_max(cm));
    const float alpha = __builtin_amdgcn_exp2f(acc.mlog - mnew);
    acc.mlog = mnew;
    acc.lsum *= alpha;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc.o[mb][i] *= alpha;
  }
}

// exp2(s*c - m) packed to bf16 (the B operand of the value product); the row
// sum accumulates the packed values with dot2.
template <int MB>
__device__ __forceinline__ void numerators(const f32x16& s, float c2, State<MB>& acc,
                                           bf16x8 (&pb)[2]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float nm = -acc.mlog;
  float sum = acc.lsum;
#pragma unroll
  for (int t = 0; t < 2; t++) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      bf16x2 pr;
      pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * t + j], c2, nm));
      pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * t + j + 1], c2, nm));
      pb[t][j] = pr[0];
      pb[t][j + 1] = pr[1];
      sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
    }
  }
  acc.lsum = sum;
}

template <int MB>
__device__ __forceinline__ void values(const bf16x8 (&vop)[MB][2], const bf16x8 (&pb)[2],
                                       State<MB>& acc) {
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int t = 0; t < 2; t++)
      acc.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[mb][t], pb[t], acc.o[mb], 0, 0, 0);
}

// The kernel.  Waves process a stream of 32-key chunks; chunk i of a wave lies in
// stage st = i / CPT (tile st*WK + kg of the unit) at position i % CPT.  The
// stream is software-pipelined: while the exponentials of chunk i are formed,
// the score MFMAs of chunk i+1 are issued in the same basic block, interleaved by
// the scheduler (one MFMA per group of VALU instructions), then chunk i's value
// MFMAs follow.  K/V tiles sit in a 2-slot ring: entering a stage waits for its
// tile, then refills the slot of the previous stage, whose last LDS reads (the V
// operands of its final chunk) completed before the barrier.
template <int D, bool CAUSAL, int WM, int WK, int TK>
__global__ __launch_bounds__(512, 2) void attn_bf16_kernel(AttnArgs a, Plan plan) {
  static_assert(WM * WK == 8, "eight waves: row groups x key groups");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int NT = 512;               // threads per workgroup
  constexpr int R = 32 * WM;            // packed rows per unit
  constexpr int KS = D / 16;            // MFMA k-steps over head_dim
  constexpr int CH = D / 8;             // 16-byte chunks per K/V row
  constexpr int MB = D / 32;            // 32-row blocks of O^T
  constexpr int ROWB = D * 2;           // bytes per K/V row
  constexpr int TILEB = TK * ROWB;      // bytes per K (or V) tile
  constexpr int RPI = 1024 / ROWB;      // rows one global_load_lds covers (64 lanes x 16 B)
  constexpr int GLL = 2 * TK / RPI / WM;// global_load_lds per wave per tile
  constexpr int CPT = TK / 32;          // chunks per tile
  static_assert(GLL >= 1 && (2 * TK / RPI) % WM == 0, "tile load split");
  constexpr int SLOTB = WK * 2 * TILEB; // one ring slot: K and V tiles of every key group
  constexpr int PER = MB * 16 + 2;      // floats per lane in the key-group merge
  constexpr int MERGEB = (WK - 1) * WM * 64 * PER * 4;
  static_assert(MERGEB <= 2 * SLOTB, "key-group merge fits in the ring");
  __shared__ __attribute__((aligned(1024))) char ring[2 * SLOTB];

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
    for (int idx = tid; idx < 2 * per; idx += NT) {
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
  bf16x8 qr[KS];
  const int prow = row0 + 32 * rg + n;
  const int qi = prow / G;
  {
    const int hh = prow % G;
    const uint16_t* qp = (const uint16_t*)a.q +
                         ((int64_t)(u.b * kCanvas + qi) * Hq + u.g * G + hh) * D + (D / 2) * h;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qr[ks] = *(const bf16x8*)(qp + 8 * ks);
  }

  TileSrc src;
  src.kc = (const char*)(kc + ((int64_t)u.b * cap * Hkv + u.g) * D);
  src.vc = (const char*)(vc + ((int64_t)u.b * cap * Hkv + u.g) * D);
  src.kn = (const char*)(kn + ((int64_t)u.b * kCanvas * Hkv + u.g) * D);
  src.vn = (const char*)(vn + ((int64_t)u.b * kCanvas * Hkv + u.g) * D);
  src.rsb = Hkv * D * 2;
  src.L = L;
  src.kstop = kstop;
  src.lr = lane / CH;
  src.lp = lane % CH;
  src.lrs = (uint32_t)(lane / CH) * (uint32_t)src.rsb;
  const LaneOffsets<D> lo = lane_offsets<D>(lane);
  const int wave_qi_min = (row0 + 32 * rg) / G;
  const int wave_qi_max = (row0 + 32 * rg + 31) / G;
  const float c2 = a.scale_log2;
  // keys this wave can see: the unit's keys, and for the commit the diagonal
  const int klimit = CAUSAL ? min(kstop, L + wave_qi_max + 1) : kstop;

  State<MB> acc;
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc.o[mb][i] = 0.f;
  acc.mlog = -1e30f;  // log2-domain reference max; finite so rescales never form inf-inf
  acc.lsum = 0.f;

  char* slot0 = ring + kg * 2 * TILEB;
  char* slot1 = ring + SLOTB + kg * 2 * TILEB;
  const uint32_t lslot0 = lds_addr(slot0), lslot1 = lds_addr(slot1);
  // chunk i of this wave: tile (i/CPT)*WK + kg, first key below
  auto chunk_key = [&](int i) { return kbeg + ((i / CPT) * WK + kg) * TK + 32 * (i % CPT); };
  auto chunk_ok = [&](int i) {
    return (i / CPT) * WK + kg < ntiles && chunk_key(i) < klimit;
  };
  auto chunk_lds = [&](int i) {
    return ((i / CPT) & 1 ? lslot1 : lslot0) + 32 * (i % CPT) * ROWB;
  };

  const int nchunks = nstages * CPT;
  if (nstages > 0) {
    if (kg < ntiles) issue_tile<D, TK, WM>(lslot0, kbeg + kg * TK, src, rg);
    const bool second = 1 < nstages && WK + kg < ntiles;
    if (second) issue_tile<D, TK, WM>(lslot1, kbeg + (WK + kg) * TK, src, rg);
    if (second)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(GLL) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  // Consume the query registers before the loop: the compiler's own vmcnt wait for
  // them lands here (it also covers the first prefetches, which were issued after
  // the queries and were needed anyway); inside the loop such a wait would drain
  // prefetches the compiler does not know about.
#pragma unroll
  for (int ks = 0; ks < KS; ks++) asm volatile("" ::"v"(qr[ks]));
  f32x16 s_cur;
  bf16x8 kop[KS];
  if (nchunks > 0 && chunk_ok(0)) {
    load_k_operands<D>(chunk_lds(0), lo.k, kop);
    scores<D>(kop, qr, s_cur);
  }
  for (int i = 0; i < nchunks; i++) {
    const bool ok = chunk_ok(i);
    bf16x8 vop[MB][2];
    if (ok) load_v_operands<D>(chunk_lds(i) + TILEB, lo.v, vop);
    const int i1 = i + 1;
    bool ok1 = false;
    if (i1 < nchunks) {
      if (i1 % CPT == 0) {
        // entering stage st1: its tile must have landed in every wave's share;
        // afterwards the previous stage's slot (all of its reads are done) is
        // refilled with stage st1+1
        const int st1 = i1 / CPT;
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int t2 = (st1 + 1) * WK + kg;
        if (st1 + 1 < nstages && t2 < ntiles)
          issue_tile<D, TK, WM>((st1 + 1) & 1 ? lslot1 : lslot0, kbeg + t2 * TK, src, rg);
      }
      ok1 = chunk_ok(i1);
      if (ok1) load_k_operands<D>(chunk_lds(i1), lo.k, kop);
    }
    f32x16 s_next;
    bf16x8 pb[2];
    if (ok) {
      prepare_scores<MB, CAUSAL>(s_cur, chunk_key(i), kstop, L, wave_qi_min, qi, h, c2, acc);
      if (ok1) {
        // one basic block: next chunk's score MFMAs interleaved with this chunk's
        // exponentials
        scores<D>(kop, qr, s_next);
        numerators<MB>(s_cur, c2, acc, pb);
#pragma unroll
        for (int k = 0; k < KS; k++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
        }
      } else {
        numerators<MB>(s_cur, c2, acc, pb);
      }
      values<MB>(vop, pb, acc);
    } else if (ok1) {
      scores<D>(kop, qr, s_next);
    }
    s_cur = s_next;
  }

  // ---- merge the key groups through LDS (group 0 keeps the result).  Every wave
  //      passes every barrier; only group 0 carries on with the result.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (WK > 1) {
    float* mbuf = (float*)ring;
    if (kg > 0) {
      float* dst = mbuf + ((kg - 1) * WM + rg) * 64 * PER;
      int k = 0;
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int i = 0; i < 16; i++) dst[(k++) * 64 + lane] = acc.o[mb][i];
      dst[(k++) * 64 + lane] = acc.mlog;
      dst[(k++) * 64 + lane] = acc.lsum;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kg == 0) {
#pragma unroll
      for (int og = 1; og < WK; og++) {
        const float* srcm = mbuf + ((og - 1) * WM + rg) * 64 * PER;
        const float m2 = srcm[(MB * 16) * 64 + lane];
        const float l2 = srcm[(MB * 16 + 1) * 64 + lane];
        const float mn = fmaxf(acc.mlog, m2);
        const float a1 = __builtin_amdgcn_exp2f(acc.mlog - mn);
        const float a2 = __builtin_amdgcn_exp2f(m2 - mn);
        acc.mlog = mn;
        acc.lsum = acc.lsum * a1 + l2 * a2;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int i = 0; i < 16; i++)
            acc.o[mb][i] = acc.o[mb][i] * a1 + srcm[(mb * 16 + i) * 64 + lane] * a2;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (kg > 0) return;

  // ---- write the unit's rows: normalised, rounded to bf16, either as the final
  //      output (single split) or as this split's partial rows.  They go out
  //      through a per-wave LDS staging area, 64 columns of head_dim at a time, so
  //      that every store is a whole 128-byte row segment (the accumulator layout
  //      puts one query row in each lane).
  const float lt = partner_sum(acc.lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const bool direct = sp.n_splits == 1;
  constexpr int SROWB = 64 * 2 + 16;  // bytes per staged row (padding spreads banks)
  char* stage = ring + rg * 32 * SROWB;
  const int r_lo = lane / 8, cq = lane % 8;  // 8 lanes cover one 128-byte row segment
  uint16_t* rowp[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int p = row0 + 32 * rg + 8 * k + r_lo;  // packed row stored by this lane
    rowp[k] = direct ? (uint16_t*)a.out +
                           ((int64_t)(u.b * kCanvas + p / G) * Hq + u.g * G + p % G) * D
                     : (uint16_t*)a.part_o + ((int64_t)U * R + (p - row0)) * D;
  }
#pragma unroll
  for (int half = 0; half < MB / 2; half++) {
#pragma unroll
    for (int mbl = 0; mbl < 2; mbl++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4e;
        bf16x4e v;
#pragma unroll
        for (int j = 0; j < 4; j++) v[j] = (__bf16)(acc.o[2 * half + mbl][4 * q4 + j] * inv);
        *(bf16x4e*)(stage + n * SROWB + (32 * mbl + 8 * q4 + 4 * h) * 2) = v;
      }
#pragma unroll
    for (int k = 0; k < 4; k++)
      *(uint4*)(rowp[k] + 64 * half + 8 * cq) =
          *(const uint4*)(stage + (8 * k + r_lo) * SROWB + 16 * cq);
  }
  if (!direct && h == 0)
    *(float2*)(a.part_ml + ((int64_t)U * R + (prow - row0)) * 2) = make_float2(acc.mlog, lt);
}

template <int D, bool CAUSAL, int WM, int WK, int TK>
int launch_one(const AttnArgs& a, const Plan& p, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, CAUSAL, WM, WK, TK>), dim3(p.n_units), dim3(512), 0, st,
                     a, p);
  return (int)hipGetLastError();
}

template <bool CAUSAL>
int launch_d128(const AttnArgs& a, const Plan& p, hipStream_t st) {
  switch (p.variant) {
    case kVariantR256: return launch_one<128, CAUSAL, 8, 1, 64>(a, p, st);
    case kVariantR64: return launch_one<128, CAUSAL, 2, 4, 32>(a, p, st);
    default: return launch_one<128, CAUSAL, 4, 2, 64>(a, p, st);  // kVariantR128
  }
}

}  // namespace

int launch_attn_bf16(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (p.n_units == 0) return 0;
  if (head_dim == 128) return causal ? launch_d128<true>(a, p, st) : launch_d128<false>(a, p, st);
  // head_dim 64 has a single shape: 128 rows per unit
  return causal ? launch_one<64, true, 4, 2, 64>(a, p, st)
                : launch_one<64, false, 4, 2, 64>(a, p, st);
}

}  // namespace dg
