// dg_attn_mfma.hip -- split-key canvas / commit attention on the matrix cores (gfx950):
// bf16 in, or e4m3 (fp8) in; fp32 accumulate; bf16 out.
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
//   * A workgroup is eight wave64s = WM row groups x WK key groups; each wave
//     owns 32 packed query rows (its Q operands stay in VGPRs) and walks its key
//     group's chunks (32 keys in bf16, 64 in fp8).
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
//   * Ping-pong: waves w and w+4 share a SIMD.  Each chunk is split into an MFMA
//     phase X (value product of chunk k, scores of chunk k+1: sixteen MFMAs, with
//     the stage loads and the LDS operand reads of the next chunks between them)
//     and a vector phase Y (softmax of chunk k+1).  One workgroup barrier per
//     chunk, after Y in waves 0-3 and after X in waves 4-7, keeps the two halves of
//     the workgroup half a chunk apart, so on every SIMD one wave runs X while the
//     other runs Y: the matrix pipe and the vector ALU work at the same time.  The
//     MFMA phase runs at raised wave priority.
//   * K/V stream HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a
//     ring of NSLOT stages (one chunk of K and V per key group each); a stage is
//     refilled as soon as the barrier after its last operand read has passed,
//     which keeps NSLOT-2 chunks of loads in flight.  Whole tiles inside the
//     cache or the canvas use a scalar base plus precomputed 32-bit lane offsets;
//     only a tile that crosses the cache/canvas seam or the end of the unit takes
//     the per-lane path.  Rows are stored densely (D*2 bytes) with an XOR swizzle
//     of the 16-byte chunks so that the K operand reads (ds_read_b128, one key row
//     per lane) and the V operand reads (ds_read_b64_tr_b16, the gfx950
//     transposing LDS read) are bank-conflict free.
//   * Softmax runs in the log2 domain with a lazily raised reference max: a
//     chunk's exact max is always formed, but the output is rescaled only when it
//     exceeds the reference by more than 64 (so every exponential stays <= 2^64);
//     in steady state a score costs max, FMA, exp2, a bf16 pack and an fp32 add
//     (fp8: the row sum comes from one more MFMA per chunk instead).
//     The result is exact attention; only the point at which the max is folded
//     in moves.
//   * Key groups of a workgroup are merged through LDS at the end; the unit
//     writes its normalised rows (bf16) plus (max, sum) as a partial, or the final
//     output when the sequence has a single split, through an LDS staging area so
//     that every store is a whole 128-byte row segment.
//
// The fp8 format (OCP e4m3 queries, keys and values with per-tensor scales) runs
// the same kernel with v_mfma_f32_32x32x64_f8f6f4: a chunk is 64 keys (the same
// 8 KB per K or V tile as 32 bf16 keys at head_dim 128), the scores of its two
// 32-key halves feed one value MFMA per 32 head_dim rows, and the exponentials
// are rounded to e4m3 for it.  Its differences are kept in FmtFp8 and the
// overloads taking fp8 operands below.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dg_internal.h"

namespace dg {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
#define LDS_AS __attribute__((address_space(3)))

constexpr float kRescaleThreshold = 64.f;  // log2 units

// Element formats of the ping-pong kernel.  A chunk is the run of keys a wave
// takes per step; both formats move 8 KB of K and 8 KB of V per chunk at
// head_dim 128.  The exponentials of a chunk run up to 2^(kBias + kThreshold)
// relative to the reference max (the lazy rescale below).
struct FmtBf16 {
  static constexpr int ESZ = 2;              // bytes per element
  static constexpr int TK = 32;              // keys per chunk
  static constexpr float kThreshold = 64.f;  // rescale when a chunk max rises this far (log2)
  static constexpr float kBias = 0.f;        // exponent offset of the exponentials
};
// e4m3 tops out at 448 (just under 2^8.81), and the gfx950 conversion returns NaN
// rather than saturating above 464, so the exponentials that become the B
// operand of the value MFMA must stay below that: a bias of 5 plus a threshold of
// 3.5 bounds them by 2^8.5.  The bias also lifts the bulk of a diffuse row (2^-6 ..
// 2^-10 of its max) into e4m3's normal range, where the rounding error is 2^-4
// relative; values below 2^-11 of the reference become subnormal and carry a
// negligible weight.
struct FmtFp8 {
  static constexpr int ESZ = 1;
  static constexpr int TK = 64;
  static constexpr float kThreshold = 3.5f;
  static constexpr float kBias = 5.f;
};
template <class F>
constexpr bool is_fp8 = F::ESZ == 1;

// fp8 rows are 128 bytes, eight 16-byte chunks; logical chunk c of row r is
// stored at physical chunk c ^ swz8(r).  Per cycle the score operand reads take
// one logical chunk of 16 rows {0-7, 16-23} or {8-15, 24-31} of a 32-row half
// (the permuted key rows of kperm8) and the transposing V reads 8 consecutive
// rows of two adjacent chunks: both land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int r) { return 2 * ((r >> 1) & 3) | ((r >> 4) & 1); }

// Key row that fp8 score MFMA row i (0..31) reads within its 32-key half.  The
// MFMA leaves row i of its result in lane half (i / 4) % 2, register 4(i / 8) +
// i % 4; with this permutation lane half h holds keys 16h .. 16h+15 in register
// order, so the e4m3 exponentials of a 64-key chunk are bytes 16t + i = key
// 32t + 16h + i, which two 8-row transposing reads match on the V side.
__device__ __forceinline__ int kperm8(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// Work units come from the plan: xcd_remap, decode_unit and div_rcp (dg_plan.h).

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
  float thr;     // raw score above which a chunk raises the reference:
                 // (mlog + threshold) / c2, kept with mlog
};

// Max of the 16 scores of a lane as one chain of v_max3 (written as a single asm
// block: separate ones each get a wait state).  fmaxf would add canonicalizing
// instructions (IEEE NaN quieting) that nothing here needs: scores are finite or
// -inf.  Dependent vector ALU instructions need no wait states between them.
__device__ __forceinline__ float max16(const f32x16& s) {
  float m;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max3_f32 %0, %0, %10, %11\n\t"
      "v_max3_f32 %0, %0, %12, %13\n\t"
      "v_max3_f32 %0, %0, %14, %15\n\t"
      "v_max_f32 %0, %0, %16"
      : "=&v"(m)
      : "v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]), "v"(s[4]), "v"(s[5]), "v"(s[6]),
        "v"(s[7]), "v"(s[8]), "v"(s[9]), "v"(s[10]), "v"(s[11]), "v"(s[12]), "v"(s[13]),
        "v"(s[14]), "v"(s[15]));
  return m;
}

// global_load_lds_dwordx4: every lane copies 16 bytes from its global address
// into LDS at m0 + instruction offset + 16*lane.  Issued from inline asm so that
// the compiler does not see an LDS write it cannot disambiguate from the operand
// reads of the other ring slots (it would otherwise drain every prefetch before
// the first of them); completion is tracked explicitly with s_waitcnt vmcnt
// before each stage's barrier.  The single-source form is written out in
// issue_stage; this is the per-lane-address form.  Nothing else in the kernel
// uses m0 (the compiler reserves it and takes no clobber of it).
__device__ __forceinline__ void gll_vaddr(const char* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vaddr), "s"(lds)
               : "memory");
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// This wave's share of the global_load_lds instructions that fill one ring stage.
// A stage holds, for every key group kt, one chunk of K and V (F::TK keys); the
// K tiles of the stage are consecutive in LDS and so are its V tiles, so each
// half is a run of 1 KB blocks (block b: keys b*RPI .. b*RPI+RPI-1 of the stage).
// Waves 0 .. NW/2-1 fill the K half and the others the V half, each GPW
// consecutive blocks: one M0 value serves all of a wave's loads, which differ
// only in the instruction offset 1024e (the offset moves the LDS destination and
// the global address alike; the lane offsets take it back out of the latter).
// Writing M0 before every load would stall the wave at each of them.
// Each load moves 1 KB: lane l writes 16 bytes at 16*l of its block, i.e. block
// row l / CH, physical chunk l % CH, and fetches the logical chunk that the
// swizzle stores there (bf16 K: chunk ^ (row % CH); bf16 V: chunk ^ 4*(row % 4);
// fp8 K and V: chunk ^ swz8(row); row within the tile).  Everything that does not depend on the stage is computed
// once per wave; per stage only the byte offset of its first key is formed, and
// a stage lying wholly in the cache or wholly in the canvas (every stage but the
// one at the seam and the unit's last) is issued as scalar base + 32-bit lane
// offsets.
// The ring holds the K tiles of every stage in its first 64 KB and the V tiles in
// the second: stage s, key group kt at s*WK*TILEB + kt*TILEB (+ kVRegion for V),
// so that every operand read is a per-lane base plus an immediate offset.
constexpr uint32_t kVRegion = 65536;

template <class F, int D, int WK, int NW = 8>
struct StageLoads {
  static constexpr int ROWB = D * F::ESZ, CH = ROWB / 16, RPI = 1024 / ROWB, IPT = F::TK / RPI;
  static constexpr int TILEB = F::TK * ROWB, GPW = WK * 2 * IPT / NW;
  static_assert(NW % 2 == 0 && GPW * NW == WK * 2 * IPT && GPW >= 1 && GPW <= 4,
                "whole blocks per wave, instruction offsets below 4 KB");
  uint64_t cb;              // cache K or V base of (sequence, kv head)
  uint64_t nb;              // canvas/block K or V base minus L rows
  uint32_t rowoff;          // first row of the wave's blocks * row stride
  uint32_t dst;             // LDS offset of the wave's first block within a stage
  uint32_t lane[GPW];       // lane byte offset of load e (row, swizzled chunk) less 1024e
  int32_t krow;             // lane's key offset within the stage in load 0 (+RPI per load)
  int32_t rsb, L, kstop;
};

template <class F, int D, int WK, int NW>
__device__ __forceinline__ void stage_loads_init(StageLoads<F, D, WK, NW>& sl, const char* kc,
                                                 const char* vc, const char* kn, const char* vn,
                                                 int rsb, int L, int kstop, int wave, int lane) {
  using SL = StageLoads<F, D, WK, NW>;
  const int lr = lane / SL::CH, lp = lane % SL::CH;
  sl.rsb = rsb;
  sl.L = L;
  sl.kstop = kstop;
  const bool isv = wave >= NW / 2;  // wave-uniform
  const int b0 = (wave % (NW / 2)) * SL::GPW;
  const uint64_t ukc = (uint64_t)(uintptr_t)kc, uvc = (uint64_t)(uintptr_t)vc;
  const uint64_t ukn = (uint64_t)(uintptr_t)kn - (uint64_t)L * (uint64_t)rsb;
  const uint64_t uvn = (uint64_t)(uintptr_t)vn - (uint64_t)L * (uint64_t)rsb;
  sl.cb = uniform64(isv ? uvc : ukc);
  sl.nb = uniform64(isv ? uvn : ukn);
  sl.rowoff = (uint32_t)(b0 * SL::RPI * rsb);
  sl.dst = (uint32_t)((isv ? kVRegion : 0) + b0 * 1024);
  sl.krow = b0 * SL::RPI + lr;
#pragma unroll
  for (int e = 0; e < SL::GPW; e++) {
    const int r = ((b0 + e) % SL::IPT) * SL::RPI + lr;  // row within the tile
    const int sw = is_fp8<F> ? swz8(r) : isv ? ((4 * (r & 3)) & (SL::CH - 1)) : (r & (SL::CH - 1));
    sl.lane[e] = (uint32_t)(e * SL::RPI + lr) * (uint32_t)rsb + 16u * (uint32_t)(lp ^ sw) -
                 1024u * (uint32_t)e;
  }
}

// Where the keys of the stage from skey0 come from: 1 wholly the cache, 2 wholly
// the canvas (both issued as scalar base + lane offsets), 0 both or past the
// unit's end (rows formed per lane).
template <class F, int D, int WK, int NW>
__device__ __forceinline__ int stage_source(int skey0, const StageLoads<F, D, WK, NW>& sl) {
  const int send = skey0 + F::TK * WK;
  if (send <= sl.L && send <= sl.kstop) return 1;
  if (skey0 >= sl.L && send <= sl.kstop) return 2;
  return 0;
}

// NL (1..4) global_load_lds_dwordx4 from scalar base sb + lane offset vo[e] + 1024e
// into LDS at m0 + 1024e + 16*lane: one m0 write serves the whole block.
template <int NL>
__device__ __forceinline__ void gll_block(const char* sb, const uint32_t* vo, uint32_t m0) {
  static_assert(NL >= 1 && NL <= 4, "instruction offsets below 4 KB");
  if constexpr (NL == 1)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
                 ::"v"(vo[0]), "s"(m0), "s"(sb) : "memory");
  else if constexpr (NL == 2)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %3\n\t"
                 "global_load_lds_dwordx4 %1, %3 offset:1024"
                 ::"v"(vo[0]), "v"(vo[1]), "s"(m0), "s"(sb) : "memory");
  else if constexpr (NL == 3)
    asm volatile("s_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %0, %4\n\t"
                 "global_load_lds_dwordx4 %1, %4 offset:1024\n\t"
                 "global_load_lds_dwordx4 %2, %4 offset:2048"
                 ::"v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "s"(m0), "s"(sb) : "memory");
  else
    asm volatile("s_mov_b32 m0, %4\n\tglobal_load_lds_dwordx4 %0, %5\n\t"
                 "global_load_lds_dwordx4 %1, %5 offset:1024\n\t"
                 "global_load_lds_dwordx4 %2, %5 offset:2048\n\t"
                 "global_load_lds_dwordx4 %3, %5 offset:3072"
                 ::"v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(m0), "s"(sb) : "memory");
}

// Issues the wave's loads of one stage (keys from skey0, WK tiles) into the LDS
// slot.  Tiles past the unit's last key are loaded too (rows clamped onto the
// unit's last key) so that each wave always has the same number of loads per
// stage in flight.
template <class F, int D, int WK, int NW>
__device__ __forceinline__ void issue_stage(uint32_t slot, int skey0, const StageLoads<F, D, WK, NW>& sl) {
  using SL = StageLoads<F, D, WK, NW>;
  constexpr int G = SL::GPW;
  const int src = stage_source(skey0, sl);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(slot + sl.dst);
  if (src > 0) {
    const uint64_t tb = (src == 1 ? sl.cb : sl.nb) + (uint64_t)(int64_t)skey0 * (uint64_t)sl.rsb + sl.rowoff;
    gll_block<G>(uniform_ptr((const char*)(uintptr_t)tb), sl.lane, m0);
  } else {
#pragma unroll
    for (int e = 0; e < G; e++) {
      const int key = min(skey0 + sl.krow + e * SL::RPI, sl.kstop - 1);
      const uint64_t base = key < sl.L ? sl.cb : sl.nb;
      const uint64_t row = base + (uint64_t)(int64_t)key * (uint64_t)sl.rsb;
      // the row is the lane's own here: keep only the swizzled chunk of the lane offset
      const uint32_t chunk = sl.lane[e] + 1024u * (uint32_t)e -
                             (uint32_t)(sl.krow - (sl.krow / SL::RPI) * SL::RPI + e * SL::RPI) * (uint32_t)sl.rsb;
      gll_vaddr((const char*)(uintptr_t)(row + chunk), m0 + 1024u * (uint32_t)e);
    }
  }
}

// The scalar half of a stage request, formed one phase ahead of the loads: where
// the stage's keys come from (stage_source) and, for a stage wholly in the cache
// or wholly in the canvas, its scalar base address.  issue_stage_req then costs
// the matrix phase only an m0 write and the loads themselves.
struct StageReq {
  int src;
  uint64_t base;
};

template <class F, int D, int WK, int NW>
__device__ __forceinline__ StageReq stage_req(int skey0, const StageLoads<F, D, WK, NW>& sl) {
  StageReq r;
  r.src = stage_source(skey0, sl);
  r.base = (r.src == 1 ? sl.cb : sl.nb) + (uint64_t)(int64_t)skey0 * (uint64_t)sl.rsb + sl.rowoff;
  return r;
}

template <class F, int D, int WK, int NW>
__device__ __forceinline__ void issue_stage_req(uint32_t slot, int skey0, const StageReq& r,
                                                const StageLoads<F, D, WK, NW>& sl) {
  using SL = StageLoads<F, D, WK, NW>;
  constexpr int G = SL::GPW;
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(slot + sl.dst);
  if (r.src > 0) {
    gll_block<G>(uniform_ptr((const char*)(uintptr_t)r.base), sl.lane, m0);
  } else {
#pragma unroll
    for (int e = 0; e < G; e++) {
      const int key = min(skey0 + sl.krow + e * SL::RPI, sl.kstop - 1);
      const uint64_t base = key < sl.L ? sl.cb : sl.nb;
      const uint64_t row = base + (uint64_t)(int64_t)key * (uint64_t)sl.rsb;
      const uint32_t chunk = sl.lane[e] + 1024u * (uint32_t)e -
                             (uint32_t)(sl.krow - (sl.krow / SL::RPI) * SL::RPI + e * SL::RPI) * (uint32_t)sl.rsb;
      gll_vaddr((const char*)(uintptr_t)(row + chunk), m0 + 1024u * (uint32_t)e);
    }
  }
}

// V^T operands of one 32-key chunk: vop[mb][t] holds, in lane (d, h), the values
// of keys 16t + 8r + 4h + e (k-slot 4r + e) at head_dim 32mb + d, read with the
// transposing ds_read_b64_tr_b16.  vbase[mb] is the lane's address in stage 0;
// off (a compile-time constant in the unrolled loop) selects the stage.
template <int D>
__device__ __forceinline__ void load_v_operands(const uint32_t (&vbase)[D / 32], uint32_t off,
                                                bf16x8 (&vop)[D / 32][2]) {
  constexpr int ROWB = D * 2, MB = D / 32;
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    const LDS_AS char* p = (const LDS_AS char*)(uintptr_t)(vbase[mb] + off);
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
// (D/16)*h + ks (the A operand of S^T = K Q^T); kbase[ks] is the lane's address
// in stage 0 and off selects the stage.
template <int D>
__device__ __forceinline__ void load_k_operands(const uint32_t (&kbase)[D / 16], uint32_t off,
                                                bf16x8 (&kop)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ks++)
    kop[ks] = *(const LDS_AS bf16x8*)(uintptr_t)(kbase[ks] + off);
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

// Masks a chunk's scores when asked (ragged end of the unit; block keys past
// the diagonal for the commit), folds the chunk max into the reference max when
// it rises by more than the threshold, and returns nothing else: the
// exponentials follow.
template <int MB, bool CAUSAL>
__device__ __forceinline__ void prepare_scores(f32x16& s, bool masked, int key0, int kstop, int L,
                                               int qi, int h, float c2, State<MB>& acc) {
  if (masked) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int key = key0 + 8 * (i / 4) + 4 * h + (i % 4);
      bool ok = key < kstop;
      if (CAUSAL) ok = ok && (key < L || key - L <= qi);
      s[i] = ok ? s[i] : -INFINITY;
    }
  }
  const float m = max16(s);
  // m > thr stands for m*c2 > mlog + threshold (c2 > 0); a rounding difference
  // at the boundary moves the exponent bound by far less than its headroom
  if (__any(m > acc.thr)) {
    const float mnew = fmaxf(acc.mlog, partner_max(m * c2));
    const float alpha = __builtin_amdgcn_exp2f(acc.mlog - mnew);
    acc.mlog = mnew;
    acc.thr = (mnew + kRescaleThreshold) / c2;
    acc.lsum *= alpha;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc.o[mb][i] *= alpha;
  }
}

// exp2(s*c - m) packed to bf16 (the B operand of the value product).  The row
// sum adds the fp32 exponentials before rounding, with plain VALU adds: a
// v_dot2_f32_bf16 over the packed values would be one instruction per pair, but
// it does not co-execute with MFMAs of the other wave on the SIMD (measured),
// while adds and packs do.  Computed in place, stage by stage, so that the
// sixteen exponentials are independent and pipeline.
__device__ __forceinline__ void numerators(f32x16& s, float c2, float mlog, float& lsum,
                                           bf16x8 (&pb)[2]) {
  const float nm = -mlog;
#pragma unroll
  for (int i = 0; i < 16; i++) s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, nm));
  float part[4];
#pragma unroll
  for (int q = 0; q < 4; q++) part[q] = (s[4 * q] + s[4 * q + 1]) + (s[4 * q + 2] + s[4 * q + 3]);
  lsum += (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int j = 0; j < 8; j++) pb[t][j] = (__bf16)s[8 * t + j];
}

template <int MB>
__device__ __forceinline__ void numerators(f32x16& s, float c2, State<MB>& acc, bf16x8 (&pb)[2]) {
  numerators(s, c2, acc.mlog, acc.lsum, pb);
}

template <int MB>
__device__ __forceinline__ void values(const bf16x8 (&vop)[MB][2], const bf16x8 (&pb)[2],
                                       f32x16 (&o)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int t = 0; t < 2; t++)
      o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[mb][t], pb[t], o[mb], 0, 0, 0);
}

template <int MB>
__device__ __forceinline__ void values(const bf16x8 (&vop)[MB][2], const bf16x8 (&pb)[2],
                                       State<MB>& acc) {
  values<MB>(vop, pb, acc.o);
}

// The bf16 registers as one group, so that the kernel body below is written
// once for both formats.
template <int D>
struct Ops16 {
  bf16x8 q[D / 16];     // B operands of S^T = K Q^T: lane (n, h), k-step ks holds
                        // q[row][D/2*h + 8*ks .. +8] (the head_dim order the K operands use)
  bf16x8 k[D / 16];     // K operands for the next score MFMAs
  bf16x8 v[D / 32][2];  // V^T operands for the next value MFMAs
  bf16x8 p[2];          // packed exponentials for the next value MFMAs
  f32x16 s[1];          // scores of the chunk the next softmax works on
};

template <int D>
__device__ __forceinline__ void load_k_operands(const uint32_t (&kbase)[D / 16], uint32_t off, Ops16<D>& op) {
  load_k_operands<D>(kbase, off, op.k);
}
template <int D>
__device__ __forceinline__ void scores(Ops16<D>& op) { scores<D>(op.k, op.q, op.s[0]); }
template <int D>
__device__ __forceinline__ void load_v_operands(const uint32_t (&vbase)[D / 32], uint32_t off, Ops16<D>& op) {
  load_v_operands<D>(vbase, off, op.v);
}
template <int MB, bool CAUSAL, int D>
__device__ __forceinline__ void prepare_scores(Ops16<D>& op, bool masked, int key0, int kstop, int L,
                                               int qi, int h, float c2, State<MB>& acc) {
  prepare_scores<MB, CAUSAL>(op.s[0], masked, key0, kstop, L, qi, h, c2, acc);
}
template <int MB, int D>
__device__ __forceinline__ void numerators(Ops16<D>& op, float c2, State<MB>& acc) {
  numerators<MB>(op.s[0], c2, acc, op.p);
}
template <int MB, int D>
__device__ __forceinline__ void values(const Ops16<D>& op, State<MB>& acc) {
  values<MB>(op.v, op.p, acc);
}

// Slices of the matrix phase, so that loads and LDS reads can be placed between
// single MFMAs.  Value MFMA i (0 .. 2*MB-1) adds head_dim block i % MB of keys
// 16*(i / MB) .. +15: the first MB are independent of each other.
template <int D>
constexpr int n_value_mfma(const Ops16<D>*) { return D / 16; }
template <int MB, int D>
__device__ __forceinline__ void value_mfma(int i, const Ops16<D>& op, State<MB>& acc) {
  const int mb = i % MB, t = i / MB;
  acc.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.v[mb][t], op.p[t], acc.o[mb], 0, 0, 0);
}
// Score MFMA ks of the next chunk, then the K operand ks of the chunk after it read
// into the registers the MFMA has just taken (koff: that chunk's stage offset).
template <int D>
__device__ __forceinline__ void score_mfma_and_k(int ks, Ops16<D>& op, const uint32_t (&kbase)[D / 16],
                                                 uint32_t koff, bool read_k) {
  if (ks == 0) {
#pragma unroll
    for (int i = 0; i < 16; i++) op.s[0][i] = 0.f;
  }
  op.s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.k[ks], op.q[ks], op.s[0], 0, 0, 0);
  if (read_k) op.k[ks] = *(const LDS_AS bf16x8*)(uintptr_t)(kbase[ks] + koff);
}
template <int D>
constexpr int n_score_mfma(const Ops16<D>*) { return D / 16; }

// ---------------------------------------------------------------------------
// fp8 operands.  v_mfma_f32_32x32x64_f8f6f4 multiplies byte j of A lane (i, h)
// with byte j of B lane (n, h) (lane = i + 32h) and sums over h and j, so any
// assignment of head_dim (or of keys) to (h, j) works as long as both operands
// use the same one; the result has the 32x32 layout of the bf16 MFMA.

// e4m3 x e4m3 (format code 0 for both operands), no block scales
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Per-lane LDS offsets of the fp8 operand reads (head_dim 128): a 64-key chunk
// is two 32-key halves t of 32 * 128 bytes, and a transposing V read covers 8
// rows, so halves and 8-row blocks are immediate offsets of 4096 and 1024.
struct LaneOffsets8 {
  uint32_t k[2][2];  // K row kperm8(n), logical chunk 4ks + 2h + part (ds_read_b128)
  uint32_t q[2][2];  // query row n, same chunks
  uint32_t v[4];     // ds_read_b64_tr_b8 of head_dim block mb, row 16h + (lane%16)/2
};

__device__ __forceinline__ LaneOffsets8 lane_offsets8(int lane) {
  LaneOffsets8 o;
  const int n = lane & 31, h = lane >> 5, kr = kperm8(n);
#pragma unroll
  for (int ks = 0; ks < 2; ks++)
#pragma unroll
    for (int part = 0; part < 2; part++) {
      const int c = 4 * ks + 2 * h + part;
      o.k[ks][part] = kr * 128 + 16 * (c ^ swz8(kr));
      o.q[ks][part] = n * 128 + 16 * (c ^ swz8(n));
    }
  // transposing read: in each 16-lane group, lane 2e + b supplies bytes 8b .. 8b+7
  // of the group's 16 columns in row e, and lane i receives column i of the 8 rows
  const int i16 = lane & 15, e = i16 >> 1, row = 16 * h + e;
#pragma unroll
  for (int mb = 0; mb < 4; mb++) {
    const int c = 2 * mb + ((lane >> 4) & 1);
    o.v[mb] = row * 128 + 16 * (c ^ swz8(row)) + 8 * (i16 & 1);
  }
  return o;
}

// Registers of the fp8 pipeline (head_dim 128).
struct Ops8 {
  i32x8 q[2];     // B operands of S^T = K Q^T: lane (n, h), k-step ks holds bytes
                  // 64ks + 32h .. +32 of query row n
  i32x8 k[2][2];  // A operands [half t][k-step]: the same bytes of key row 32t + kperm8(n)
  i32x8 v[4];     // A operands of O^T += V^T P^T: lane (d, h), byte 16t + i holds
                  // V[32t + 16h + i][32mb + d]
  i32x8 p;        // B operand: lane (n, h), byte 16t + i holds the e4m3 exponential of
                  // query n and key 32t + 16h + i
  f32x16 s[2];    // scores of the chunk the next softmax works on, per half
  i32x8 ones;     // A operand of e4m3 ones (0x38): ones^T P^T sums the rounded weights
  f32x16 rs;      // row sums of the rounded weights: every element of lane (n, h) holds
                  // query n's sum over all keys so far (the MFMA adds over both halves)
};

// two 16-byte LDS reads joined into one 32-byte operand
__device__ __forceinline__ i32x8 lds_read_2x16(uint32_t a0, uint32_t a1) {
  const i32x4 lo = *(const LDS_AS i32x4*)(uintptr_t)a0;
  const i32x4 hi = *(const LDS_AS i32x4*)(uintptr_t)a1;
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void load_k_operands(const uint32_t (&kbase)[2][2], uint32_t off, Ops8& op) {
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
      op.k[t][ks] = lds_read_2x16(kbase[ks][0] + off + 4096u * t, kbase[ks][1] + off + 4096u * t);
}

__device__ __forceinline__ void scores(Ops8& op) {
#pragma unroll
  for (int t = 0; t < 2; t++) {
#pragma unroll
    for (int i = 0; i < 16; i++) op.s[t][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ks++) op.s[t] = mfma_f8(op.k[t][ks], op.q[ks], op.s[t]);
  }
}

__device__ __forceinline__ void load_v_operands(const uint32_t (&vbase)[4], uint32_t off, Ops8& op) {
#pragma unroll
  for (int mb = 0; mb < 4; mb++) {
    const uint32_t a = vbase[mb] + off;
    i32x2 r[4];
#pragma unroll
    for (int j = 0; j < 4; j++)  // (half, 8-row block) = (j / 2, j % 2)
      r[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (LDS_AS i32x2*)(uintptr_t)(a + 4096u * (j >> 1) + 1024u * (j & 1)));
    op.v[mb] = (i32x8){r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  }
}

// Max of the 32 scores of a lane: one v_max3 chain split over two asm blocks (an
// asm statement takes at most 30 operands).
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  float m;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max3_f32 %0, %0, %10, %11\n\t"
      "v_max3_f32 %0, %0, %12, %13\n\t"
      "v_max3_f32 %0, %0, %14, %15\n\t"
      "v_max3_f32 %0, %0, %16, %17\n\t"
      "v_max3_f32 %0, %0, %18, %19\n\t"
      "v_max3_f32 %0, %0, %20, %21\n\t"
      "v_max3_f32 %0, %0, %22, %23\n\t"
      "v_max3_f32 %0, %0, %24, %25\n\t"
      "v_max3_f32 %0, %0, %26, %27"
      : "=&v"(m)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
        "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
        "v"(a[14]), "v"(a[15]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]),
        "v"(b[5]), "v"(b[6]), "v"(b[7]), "v"(b[8]), "v"(b[9]), "v"(b[10]));
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max_f32 %0, %0, %6"
      : "=&v"(r)
      : "v"(m), "v"(b[11]), "v"(b[12]), "v"(b[13]), "v"(b[14]), "v"(b[15]));
  return r;
}

// fp8 counterpart of prepare_scores: masking with the permuted key order, the
// max of the chunk's 32 scores, and the lazy rescale with the exponent bias (the
// row sums are rescaled with the outputs; only element 0 is ever read).
template <int MB, bool CAUSAL>
__device__ __forceinline__ void prepare_scores(Ops8& op, bool masked, int key0, int kstop, int L,
                                               int qi, int h, float c2, State<MB>& acc) {
  if (masked) {
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int key = key0 + 32 * t + 16 * h + i;
        bool ok = key < kstop;
        if (CAUSAL) ok = ok && (key < L || key - L <= qi);
        op.s[t][i] = ok ? op.s[t][i] : -INFINITY;
      }
  }
  const float m = max32(op.s[0], op.s[1]);
  if (__any(m > acc.thr)) {
    const float mnew = fmaxf(acc.mlog, partner_max(m * c2) - FmtFp8::kBias);
    const float alpha = __builtin_amdgcn_exp2f(acc.mlog - mnew);
    acc.mlog = mnew;
    acc.thr = (mnew + (FmtFp8::kBias + FmtFp8::kThreshold)) / c2;
    op.rs[0] *= alpha;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc.o[mb][i] *= alpha;
  }
}

// exp2(s*c - m) of the 64 keys, packed to e4m3 (v_cvt_pk_fp8_f32 writes two
// bytes, round to nearest even) in key order.  The row sum is taken from the
// rounded bytes by the value MFMAs (values below), so numerator and denominator
// use the same weights: the output is a convex combination of the values, and a
// row whose weight sits on one key is exact.
template <int MB>
__device__ __forceinline__ void numerators(Ops8& op, float c2, State<MB>& acc) {
  const float nm = -acc.mlog;
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) op.s[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(op.s[t][i], c2, nm));
#pragma unroll
  for (int w = 0; w < 8; w++) {
    const f32x16& x = op.s[w >> 2];
    const int b = 4 * (w & 3);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[b], x[b + 1], 0, false);
    op.p[w] = __builtin_amdgcn_cvt_pk_fp8_f32(x[b + 2], x[b + 3], lo, true);
  }
}

template <int MB>
__device__ __forceinline__ void values(Ops8& op, State<MB>& acc) {
#pragma unroll
  for (int mb = 0; mb < MB; mb++) acc.o[mb] = mfma_f8(op.v[mb], op.p, acc.o[mb]);
  op.rs = mfma_f8(op.ones, op.p, op.rs);
}

// fp8 slices: value MFMAs 0 .. MB-1 take head_dim blocks, MFMA MB the row sums;
// score MFMA i = 2t + ks covers key half t, head_dim half ks.
constexpr int n_value_mfma(const Ops8*) { return 5; }
template <int MB>
__device__ __forceinline__ void value_mfma(int i, Ops8& op, State<MB>& acc) {
  if (i < MB) acc.o[i] = mfma_f8(op.v[i], op.p, acc.o[i]);
  else op.rs = mfma_f8(op.ones, op.p, op.rs);
}
__device__ __forceinline__ void score_mfma_and_k(int i, Ops8& op, const uint32_t (&kbase)[2][2],
                                                 uint32_t koff, bool read_k) {
  const int t = i >> 1, ks = i & 1;
  if (ks == 0) {
#pragma unroll
    for (int e = 0; e < 16; e++) op.s[t][e] = 0.f;
  }
  op.s[t] = mfma_f8(op.k[t][ks], op.q[ks], op.s[t]);
  if (read_k)
    op.k[t][ks] = lds_read_2x16(kbase[ks][0] + koff + 4096u * t, kbase[ks][1] + koff + 4096u * t);
}
constexpr int n_score_mfma(const Ops8*) { return 4; }

// The kernel.  Wave (rg, kg) processes chunk k = tile k*WK + kg of the unit for
// k = 0 .. nstages-1; chunk k lives in ring stage k (slot k mod NSLOT).  Per chunk
// a wave runs
//   X(k): O += V(k) P(k) (bf16: 8 MFMAs, fp8: 4 and the row-sum MFMA) with the
//         loads of stage k+NSLOT issued behind the first of them, then
//         S(k+1) = K(k+1) Q^T (bf16: 8 MFMAs, fp8: 4) with the reads of the V(k+1)
//         and K(k+2) operands placed between them;
//   Y(k): softmax of S(k+1) -> P(k+1) (vector ALU only).
// One workgroup barrier per chunk: barrier k follows Y(k) in waves 0-3 (group 0)
// and X(k) in waves 4-7 (group 1), so group 1 runs half a chunk behind and, on
// each SIMD, one wave is in X while the other is in Y.  Between barriers k-1 and
// k group 0 runs X(k), Y(k) and group 1 runs Y(k-1), X(k).
// Ring protocol: every barrier first waits for the wave's LDS reads.  The reads
// of stage s are K(s) in X(s-2) and V(s) in X(s-1), both groups, between barriers
// s-3 and s-1; so all reads of stage k are done at barrier k-1, after which X(k)
// may request stage k+NSLOT into the same slot, and before barrier k every wave
// waits for its own loads of stage k+3, leaving stages k+4 .. k+NSLOT in flight.
// The prologue requests stages 0 .. NSLOT-1 together with the queries (which
// have their own LDS area); barrier A (queries and stage 0 in) precedes the first
// scores and barrier B (stages 1 and 2 in) the first K(2) reads.
// One body serves both formats (F = FmtBf16 or FmtFp8); the entry points are
// attn_bf16_kernel and attn_fp8_kernel below.
template <class F, int D, bool CAUSAL, int WM, int WK, int NSLOT>
__device__ __forceinline__ void attn_body(const AttnArgs& a, const Plan& plan) {
  static_assert(WM * WK == 8, "eight waves: row groups x key groups");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(!is_fp8<F> || D == 128, "fp8: head_dim 128");
  static_assert(NSLOT >= 4, "the ring keeps at least two stages in flight");
  constexpr bool F8 = is_fp8<F>;
  constexpr int TK = F::TK;             // keys per chunk
  constexpr int NT = 512;               // threads per workgroup
  constexpr int R = 32 * WM;            // packed rows per unit
  constexpr int KS = D / 16;            // bf16 MFMA k-steps over head_dim
  constexpr int MB = D / 32;            // 32-row blocks of O^T
  constexpr int ROWB = D * F::ESZ;      // bytes per K/V row
  constexpr int CH = ROWB / 16;         // 16-byte chunks per K/V row
  constexpr int TILEB = TK * ROWB;      // bytes per chunk of K (or V)
  constexpr int SLOTB = WK * 2 * TILEB; // one ring stage: K and V tiles of every key group
  constexpr int GPW = SLOTB / 1024 / 8; // global_load_lds per wave per stage
  static_assert(GPW >= 1 && SLOTB % 8192 == 0, "stage load split");
  constexpr int PER = MB * 16 + 4;      // floats per lane in the key-group merge: O,
                                        // max, sum, padding to whole 16-byte words
  constexpr int MERGEB = (WK - 1) * WM * 64 * PER * 4;
  static_assert(MERGEB <= NSLOT * SLOTB, "key-group merge fits in the ring");
  // score MFMAs per chunk and the V operand reads issued between them
  constexpr int NSM = F8 ? 4 : KS, NVR = 4 * MB;
  static_assert(NVR % NSM == 0, "V reads spread evenly over the score MFMAs");
  constexpr int QBYTES = R * ROWB;      // the unit's query rows, past the ring
  static_assert(NSLOT * SLOTB + QBYTES <= 163840, "ring and queries fit a CU's LDS");
  __shared__ __attribute__((aligned(1024))) char ring[NSLOT * SLOTB + QBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int grp = wave >> 2;  // waves w and w+4 share a SIMD
  const int n = lane & 31, h = lane >> 5;
  const int rg = wave % WM, kg = wave / WM;
  const int U = xcd_remap(blockIdx.x, gridDim.x);
  SeqPlan sp;
  const Unit u = decode_unit(plan, U, sp);
  const int L = sp.prefix_len;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = plan.g;
  const int row0 = u.rt * R;
  int kend = L + kCanvas;
  if (CAUSAL) kend = min(kend, L + div_rcp(row0 + R - 1, plan.rcp_g) + 1);
  const int kbeg = u.s * sp.split_keys;
  const int kstop = min(kbeg + sp.split_keys, kend);
  const int ntiles = kstop > kbeg ? (kstop - kbeg + TK - 1) / TK : 0;
  const int nstages = (ntiles + WK - 1) / WK;

  const int64_t cap = a.cap;
  const char* kc = (const char*)a.k_cache;
  const char* vc = (const char*)a.v_cache;
  const char* kn = (const char*)a.k_new;
  const char* vn = (const char*)a.v_new;

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
      const int64_t src = ((int64_t)(u.b * kCanvas + r) * Hkv + u.g) * ROWB + c * 16;
      const int64_t dst = (((int64_t)u.b * cap + L + r) * Hkv + u.g) * ROWB + c * 16;
      const uint4 val = *(const uint4*)((which ? vn : kn) + src);
      *(uint4*)((char*)(which ? a.v_append : a.k_append) + dst) = val;
    }
  }

  const int prow = row0 + 32 * rg + n;  // packed row of this lane's scores
  const int qi = div_rcp(prow, plan.rcp_g);

  StageLoads<F, D, WK, 8> sl;
  stage_loads_init<F, D, WK, 8>(sl, kc + ((int64_t)u.b * cap * Hkv + u.g) * ROWB,
                                vc + ((int64_t)u.b * cap * Hkv + u.g) * ROWB,
                                kn + ((int64_t)u.b * kCanvas * Hkv + u.g) * ROWB,
                                vn + ((int64_t)u.b * kCanvas * Hkv + u.g) * ROWB,
                                Hkv * ROWB, L, kstop, wave, lane);
  static_assert((NSLOT & (NSLOT - 1)) == 0, "ring of a power-of-two number of stages");
  constexpr uint32_t SSTR = WK * TILEB;  // stage stride within the K (or V) region
  static_assert(NSLOT * SSTR <= kVRegion, "K and V regions of the ring");
  const uint32_t lring = lds_addr(ring);
  auto stage_slot = [&](int slot) { return lring + (uint32_t)slot * SSTR; };
  // The unit's R query rows travel by the same DMA into their own LDS area past
  // the ring, swizzled like a K tile (bf16: chunk ^ row % CH; fp8: chunk ^
  // swz8(row)), so that each wave reads its B operands with conflict-free 16-byte
  // reads.  Loaded per lane straight into registers, every instruction would touch
  // 64 cache lines (32 rows, 16 bytes of each), and both key groups would fetch
  // the same rows.  With the queries out of the ring, every stage of the ring is
  // requested as soon as the unit is known.
  constexpr int QRW = R / 8;              // rows loaded per wave
  constexpr int QPW = QRW * ROWB / 1024;  // loads per wave
  constexpr int QRPI = 1024 / ROWB;       // rows per load
  static_assert(QPW >= 1 && QRW % QRPI == 0, "whole 1 KB query loads per wave");
  auto q_lds = [&](int r) { return lring + (uint32_t)(NSLOT * SLOTB) + (uint32_t)r * ROWB; };
  {
    const char* qb = uniform_ptr((const char*)a.q + ((int64_t)u.b * kCanvas * Hq + u.g * G) * ROWB);
    const int r_first = wave * QRW;
#pragma unroll
    for (int j = 0; j < QPW; j += 4) {
      constexpr int NB4 = QPW < 4 ? QPW : 4;
      uint32_t vo[NB4];
#pragma unroll
      for (int e = 0; e < NB4; e++) {
        const int r = r_first + (j + e) * QRPI + lane / CH;  // row within the unit
        const int pr = row0 + r, qq = div_rcp(pr, plan.rcp_g);
        const int c = (lane % CH) ^ (F8 ? swz8(r) : r % CH);  // logical chunk at this slot
        vo[e] = (uint32_t)((qq * Hq + pr - qq * G) * ROWB + 16 * c) - 1024u * (uint32_t)e;
      }
      gll_block<NB4>(qb, vo, __builtin_amdgcn_readfirstlane(q_lds(r_first + j * QRPI)));
    }
  }
  const int npre = min(NSLOT, nstages);
  for (int st = 0; st < npre; st++) issue_stage<F, D, WK, 8>(stage_slot(st), kbeg + st * WK * TK, sl);

  const auto lo = [&] {
    if constexpr (F8) return lane_offsets8(lane);
    else return lane_offsets<D>(lane);
  }();

  const int wave_qi_min = div_rcp(row0 + 32 * rg, plan.rcp_g);
  const int wave_qi_max = div_rcp(row0 + 32 * rg + 31, plan.rcp_g);
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
  acc.thr = (acc.mlog + (F::kBias + F::kThreshold)) / c2;

  // Chunk k of this wave is tile t = k*WK + kg of the unit (keys kbeg + TK*t ..).
  // It holds visible keys iff k < nok; its scores need masking iff k >= kmask
  // (ragged end of the unit, or for the commit a tile reaching past the
  // diagonal of the wave's first query).
  const int tvis = klimit > kbeg ? (klimit - kbeg + TK - 1) / TK : 0;
  const int nok = tvis > kg ? (tvis - kg + WK - 1) / WK : 0;
  int tmask = (kstop - kbeg) / TK;
  if (CAUSAL) {
    const int x = wave_qi_min + L - (TK - 1) - kbeg;
    tmask = min(tmask, x >= 0 ? x / TK + 1 : 0);
  }
  const int kmask = tmask > kg ? (tmask - kg + WK - 1) / WK : 0;

  auto chunk_key = [&](int k) { return kbeg + (k * WK + kg) * TK; };
  auto stage_key = [&](int st) { return kbeg + st * WK * TK; };
  // per-lane operand addresses in stage 0 of this wave's key group
  using Ops = typename std::conditional<F8, Ops8, Ops16<D>>::type;
  using KAddr = typename std::conditional<F8, uint32_t[2][2], uint32_t[KS]>::type;
  KAddr kaddr;
  uint32_t vaddr[MB];
  Ops op;
  if constexpr (F8) {
#pragma unroll
    for (int i = 0; i < 8; i++) op.ones[i] = 0x38383838;  // e4m3 1.0 in every byte
#pragma unroll
    for (int i = 0; i < 16; i++) op.rs[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int part = 0; part < 2; part++) kaddr[ks][part] = lring + kg * TILEB + lo.k[ks][part];
#pragma unroll
    for (int mb = 0; mb < MB; mb++) vaddr[mb] = lring + kVRegion + kg * TILEB + lo.v[mb];
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) kaddr[ks] = lring + kg * TILEB + lo.k[ks];
#pragma unroll
    for (int mb = 0; mb < MB; mb++) vaddr[mb] = lring + kVRegion + kg * TILEB + lo.v[mb];
  }

  // ---- prologue.  Barrier A: the queries and stage 0 (the wave's oldest loads)
  //      are in LDS; the wave reads its query operands and the scores of chunk 0.
  //      Barrier B: stages 1 and 2 are in (the chunk loop reads K(2) in its first
  //      matrix phase); stages 3.. may still be in flight.
  // (vmcnt counts a wave's loads in issue order: queries, then stages 0, 1, ...)
  if (npre == NSLOT)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((NSLOT - 1) * GPW) : "memory");
  else if (npre == 3)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * GPW) : "memory");
  else if (npre == 2)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(GPW) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (F8) {
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
      op.q[ks] = lds_read_2x16(q_lds(32 * rg) + lo.q[ks][0], q_lds(32 * rg) + lo.q[ks][1]);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
      op.q[ks] = *(const LDS_AS bf16x8*)(uintptr_t)(q_lds(32 * rg) + lo.k[ks]);
  }
  if (0 < nok) {
    load_k_operands(kaddr, 0, op);
    scores(op);
    load_v_operands(vaddr, 0, op);
  }
  if (npre == NSLOT)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NSLOT - 3) * GPW) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (1 < nok) load_k_operands(kaddr, SSTR % (NSLOT * SSTR), op);
  if (0 < nok) {
    prepare_scores<MB, CAUSAL>(op, 0 >= kmask, chunk_key(0), kstop, L, qi, h, c2, acc);
    numerators<MB>(op, c2, acc);
  }
  // the scalar half of X(0)'s stage request
  StageReq req = stage_req(stage_key(NSLOT), sl);

  auto ring_barrier = [&](int k) {  // barrier k (see the kernel comment)
    if (k + NSLOT < nstages)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NSLOT - 3) * GPW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  constexpr int NVM = n_value_mfma((const Ops*)nullptr);  // value (and row-sum) MFMAs per chunk
  constexpr int NSC = n_score_mfma((const Ops*)nullptr);  // score MFMAs per chunk
  constexpr int NRD = (NVR + (F8 ? 8 : KS)) / NSC;         // LDS reads placed after each score MFMA
  static_assert((NVR + (F8 ? 8 : KS)) % NSC == 0, "LDS reads spread evenly over the score MFMAs");

  // The chunk loop is unrolled over the ring so that every stage offset is a
  // compile-time immediate of the LDS instructions.
  for (int k0 = 0; k0 < nstages; k0 += NSLOT) {
#pragma unroll
    for (int j = 0; j < NSLOT; j++) {
      const int k = k0 + j;
      if (k >= nstages) break;
      const uint32_t off1 = ((j + 1) % NSLOT) * SSTR, off2 = ((j + 2) % NSLOT) * SSTR;
      // X(k), the matrix phase: the value product of chunk k with the loads of
      // stage k+NSLOT (into the slot of stage k) behind its first MFMA, then the
      // scores of chunk k+1 with the reads of the V operands of chunk k+1 and of
      // the K operands of chunk k+2 (a chunk past the wave's last is read too and
      // not used) placed between them: the issue slots of an MFMA phase are
      // otherwise idle, and the vector phase keeps only the softmax.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      if (k < nok) value_mfma<MB>(0, op, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (k + NSLOT < nstages) issue_stage_req(stage_slot(j), stage_key(k + NSLOT), req, sl);
      __builtin_amdgcn_sched_barrier(0);
      if (k < nok) {
#pragma unroll
        for (int i = 1; i < NVM; i++) value_mfma<MB>(i, op, acc);
      }
      if (k + 1 < nok) {
        load_v_operands(vaddr, off1, op);
#pragma unroll
        for (int i = 0; i < NSC; i++) score_mfma_and_k(i, op, kaddr, off2, true);
#pragma unroll
        for (int i = 0; i < NSC; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one score MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);  // its share of LDS reads
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if (grp == 1) ring_barrier(k);
      __builtin_amdgcn_sched_barrier(0);
      // Y(k), the vector phase: softmax of chunk k+1, and the scalar half of
      // X(k+1)'s stage request
      if (k + 1 < nok) {
        prepare_scores<MB, CAUSAL>(op, k + 1 >= kmask, chunk_key(k + 1), kstop, L, qi, h, c2, acc);
        numerators<MB>(op, c2, acc);
      }
      req = stage_req(stage_key(k + 1 + NSLOT), sl);
      __builtin_amdgcn_sched_barrier(0);
      if (grp == 0) ring_barrier(k);
    }
  }
  // From here on the ring is free: every operand read and every stage load was
  // waited for at barrier nstages-1 at the latest (group 1's last Y, after it,
  // reads nothing).
  // fp8: both lanes of a query hold its whole row sum; half 0 carries it into the
  // additive per-lane sums of the merge below.
  if constexpr (F8) acc.lsum = h == 0 ? op.rs[0] : 0.f;

  // ---- merge the key groups through LDS: key groups 1.. leave their state,
  //      group 0 folds it into its own and writes the rows (one barrier)
  if (WK > 1) {
    // lane-major, PER floats per lane: 16-byte LDS accesses, and the 4-bank step
    // between lanes keeps each group of 16 lanes on distinct banks
    float4* mbuf = (float4*)ring;
    if (kg > 0) {
      float4* dst = mbuf + (((kg - 1) * WM + rg) * 64 + lane) * (PER / 4);
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int i = 0; i < 4; i++)
          dst[mb * 4 + i] = make_float4(acc.o[mb][4 * i], acc.o[mb][4 * i + 1],
                                        acc.o[mb][4 * i + 2], acc.o[mb][4 * i + 3]);
      dst[MB * 4] = make_float4(acc.mlog, acc.lsum, 0.f, 0.f);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kg > 0) return;
    {
#pragma unroll
      for (int og = 1; og < WK; og++) {
        const float4* srcm = mbuf + (((og - 1) * WM + rg) * 64 + lane) * (PER / 4);
        const float4 ml = srcm[MB * 4];
        const float m2 = ml.x, l2 = ml.y;
        const float mn = fmaxf(acc.mlog, m2);
        const float a1 = __builtin_amdgcn_exp2f(acc.mlog - mn);
        const float a2 = __builtin_amdgcn_exp2f(m2 - mn);
        acc.mlog = mn;
        acc.lsum = acc.lsum * a1 + l2 * a2;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float4 v = srcm[mb * 4 + i];
            acc.o[mb][4 * i] = acc.o[mb][4 * i] * a1 + v.x * a2;
            acc.o[mb][4 * i + 1] = acc.o[mb][4 * i + 1] * a1 + v.y * a2;
            acc.o[mb][4 * i + 2] = acc.o[mb][4 * i + 2] * a1 + v.z * a2;
            acc.o[mb][4 * i + 3] = acc.o[mb][4 * i + 3] * a1 + v.w * a2;
          }
      }
    }
  }

  // ---- write the unit's rows: normalised, rounded to bf16, either as the final
  //      output (single split) or as this split's partial rows.  They go out
  //      through a per-wave LDS staging area, 64 columns of head_dim at a time, so
  //      that every store is a whole 128-byte row segment (the accumulator layout
  //      puts one query row in each lane).  fp8 rows also take the value scale.
  const float lt = partner_sum(acc.lsum);
  float inv;
  if constexpr (F8)
    inv = lt > 0.f ? a.out_scale / lt : 0.f;
  else
    inv = lt > 0.f ? 1.f / lt : 0.f;
  const bool direct = sp.n_splits == 1;
  constexpr int SROWB = 64 * 2 + 16;  // bytes per staged row (padding spreads banks)
  // staging past the merge buffer, so that no wave's staging overwrites state
  // another wave is still merging
  constexpr int STAGE0 = WK > 1 ? kVRegion + 32768 : 0;
  static_assert(WK == 1 || (MERGEB <= STAGE0 && STAGE0 + WM * 32 * SROWB <= NSLOT * SLOTB),
                "output staging clear of the merge buffer");
  char* stage = ring + STAGE0 + rg * 32 * SROWB;
  const int r_lo = lane / 8, cq = lane % 8;  // 8 lanes cover one 128-byte row segment
  uint16_t* rowp[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int p = row0 + 32 * rg + 8 * k + r_lo;  // packed row stored by this lane
    rowp[k] = direct ? (uint16_t*)a.out +
                           ((int64_t)(u.b * kCanvas + div_rcp(p, plan.rcp_g)) * Hq + u.g * G + p - div_rcp(p, plan.rcp_g) * G) * D
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
    // non-temporal: the rows are not read again by this launch, and lines left
    // dirty in L2 lengthen the write-back at the end of the kernel (measured: the
    // launch 0.5-0.8 us shorter at L=8192)
#pragma unroll
    for (int k = 0; k < 4; k++)
      __builtin_nontemporal_store(*(const i32x4*)(stage + (8 * k + r_lo) * SROWB + 16 * cq),
                                  (i32x4*)(rowp[k] + 64 * half + 8 * cq));
  }
  if (!direct && h == 0) {
    const f32x2 ml = {acc.mlog, lt};
    __builtin_nontemporal_store(ml, (f32x2*)(a.part_ml + ((int64_t)U * R + (prow - row0)) * 2));
  }
}

template <int D, bool CAUSAL, int WM, int WK, int NSLOT>
__global__ __launch_bounds__(512, 2) void attn_bf16_kernel(AttnArgs a, Plan plan) {
  attn_body<FmtBf16, D, CAUSAL, WM, WK, NSLOT>(a, plan);
}

template <int D, bool CAUSAL, int WM, int WK, int NSLOT>
__global__ __launch_bounds__(512, 2) void attn_fp8_kernel(AttnArgs a, Plan plan) {
  attn_body<FmtFp8, D, CAUSAL, WM, WK, NSLOT>(a, plan);
}

// ---------------------------------------------------------------------------
// Decode attention: the AR mode of the same weights and cache, and hybrid
// decoding that checks several drafted tokens in one pass ("DiffusionGemma
// Technical Report", paperfeed.app summary, section "The numbers, honestly", the
// AR-mode and concurrency paragraphs).  n_q = 1..16 new tokens per sequence:
// token i attends to every cache row and to new rows 0..i (the commit's causal
// rule), and the new K/V rows are appended to the cache.
//
// With a few query rows per kv head every K/V byte feeds at most 32 packed rows:
// the work is a stream of the cache out of HBM, so the kernel is laid out for
// bytes in flight rather than for matrix-core issue.
//   * A unit is one tile of 32 packed rows (the n_q*G rows of a kv head, padded;
//     more rows make more tiles, which re-read their keys from L2) against one
//     key split.  A workgroup of NW waves per CU.
//   * Wave w takes chunks w, w+NW, ... of the split and streams each into its own
//     ring of NST LDS stages (K tile, then V tile) with global_load_lds_dwordx4:
//     no workgroup barrier inside the loop, NST-1 chunks of K and V per wave in
//     flight while it works on one, and every load instruction covers whole
//     128-byte lines.  The query tile arrives the same way, once, behind one
//     barrier.
//   * Per chunk the arithmetic is the canvas kernel's: transposed scores on the
//     32x32 matrix cores, the lazily rescaled log2-domain softmax, transposing V
//     reads.  Padding rows compute on a copy of the last row and are not written.
//   * The waves' states are merged through LDS at the end, and the unit writes
//     one partial (or the output, when its sequence has a single split).
//   * The first unit of each (sequence, kv head) copies the new K/V rows into the
//     cache: loaded at the start, stored at the end, so that the copy never holds
//     up the stream.  No unit reads cache rows at or past L (new keys come from
//     the new-row buffers), so the copy races with nothing.
template <class F, int D, int NW, int NST>
__global__ __launch_bounds__(64 * NW) void decode_kernel(AttnArgs a, Plan plan) {
  constexpr bool F8 = is_fp8<F>;
  constexpr int TK = F::TK, MB = D / 32, ROWB = D * F::ESZ, CH = ROWB / 16;
  constexpr int TILEB = TK * ROWB;  // bytes of one chunk of K (or V)
  constexpr int RPI = 1024 / ROWB;  // rows per 1 KB load
  constexpr int IPT = TILEB / 1024; // loads per tile
  static_assert(IPT % 4 == 0, "tiles of whole 4 KB load groups");
  constexpr int NG = IPT / 4;
  constexpr int PERCH = 2 * IPT;    // loads per chunk (K and V)
  // outstanding loads issued after the loads of the chunk being waited for
  constexpr int AFTER = (NST - 1) * PERCH;
  static_assert(NST >= 2 && NST * PERCH <= 63, "outstanding loads within the vmcnt range");
  constexpr int SLOTB = 2 * TILEB;  // one stage: K tile, then V tile
  constexpr int WAVEB = NST * SLOTB;
  constexpr int QB = kDecodeRows * ROWB;  // the unit's query rows
  constexpr int QPW = QB / 1024 / NW;     // query loads per wave
  static_assert(QPW >= 1 && QPW * NW * 1024 == QB, "query loads split over the waves");
  constexpr int PER = MB * 16 + 4;        // floats per lane of merge state
  static_assert(64 * PER * 4 <= WAVEB, "a wave's merge state fits in its ring");
  constexpr int NT = 64 * NW;
  constexpr int APT = (2 * DG_MAX_DECODE * CH + NT - 1) / NT;  // appended chunks per thread
  __shared__ __attribute__((aligned(1024))) char lds[NW * WAVEB + QB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int U = xcd_remap(blockIdx.x, gridDim.x);
  SeqPlan sp;
  const Unit u = decode_unit(plan, U, sp);
  const int L = sp.prefix_len, NQ = plan.n_q, G = plan.g, M = NQ * G;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv;
  const int row0 = u.rt * kDecodeRows;
  // keys the tile can see: the cache and the new rows up to its last token
  const int kend = L + min(NQ, div_rcp(min(row0 + kDecodeRows, M) - 1, plan.rcp_g) + 1);
  const int kbeg = u.s * sp.split_keys;
  const int kstop = min(kbeg + sp.split_keys, kend);
  const int ntiles = kstop > kbeg ? (kstop - kbeg + TK - 1) / TK : 0;
  const int nmine = uniform(ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0);

  const uint32_t rsb = (uint32_t)Hkv * ROWB;  // bytes between rows of one kv head
  const char* kc = (const char*)a.k_cache + ((int64_t)u.b * a.cap * Hkv + u.g) * ROWB;
  const char* vc = (const char*)a.v_cache + ((int64_t)u.b * a.cap * Hkv + u.g) * ROWB;
  const char* kn = (const char*)a.k_new + ((int64_t)u.b * NQ * Hkv + u.g) * ROWB;
  const char* vn = (const char*)a.v_new + ((int64_t)u.b * NQ * Hkv + u.g) * ROWB;

  // ---- the cache append, first half: load the new rows of head g
  // (one named register per chunk: an array here is placed in LDS or scratch)
  const bool appender = a.k_append != nullptr && u.s == 0 && u.rt == 0;
  const int napp = appender ? 2 * NQ * CH : 0;  // 16-byte chunks of K and V
  static_assert(APT <= 4, "at most four appended chunks per thread");
  auto app_load = [&](int r) {
    const int idx = tid + NT * r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (idx < napp) {
      const int which = idx >= NQ * CH, rem = idx - which * NQ * CH;
      v = *(const uint4*)((which ? vn : kn) + (int64_t)(rem / CH) * rsb + 16 * (rem % CH));
    }
    return v;
  };
  auto app_store = [&](int r, uint4 v) {
    const int idx = tid + NT * r;
    if (idx < napp) {
      const int which = idx >= NQ * CH, rem = idx - which * NQ * CH;
      const int64_t dst = ((int64_t)u.b * a.cap * Hkv + u.g) * ROWB + (int64_t)(L + rem / CH) * rsb + 16 * (rem % CH);
      *(uint4*)((char*)(which ? a.v_append : a.k_append) + dst) = v;
    }
  };
  const uint4 app0 = app_load(0);
  const uint4 app1 = APT > 1 ? app_load(1) : app0;
  const uint4 app2 = APT > 2 ? app_load(2) : app0;
  const uint4 app3 = APT > 3 ? app_load(3) : app0;

  const uint32_t lbase = lds_addr(lds);
  const uint32_t qarea = lbase + NW * WAVEB;
  const uint32_t wring = lbase + (uint32_t)wave * WAVEB;
  const int lr = lane / CH, lp = lane % CH;
  // swizzle of the 16-byte chunks of tile row r (see lane_offsets, lane_offsets8)
  auto swk = [](int r) { return F8 ? swz8(r) : (r & (CH - 1)); };
  auto swv = [](int r) { return F8 ? swz8(r) : ((4 * (r & 3)) & (CH - 1)); };

  // ---- the query tile: packed row p = i*G + hh of the tile (clamped to the last
  //      row) into row p - row0 of the query area, swizzled like a K tile
  {
    const char* qb = (const char*)a.q + ((int64_t)u.b * NQ * Hq + u.g * G) * ROWB;
#pragma unroll
    for (int e = 0; e < QPW; e++) {
      const int blk = wave * QPW + e, r = blk * RPI + lr;
      const int p = min(row0 + r, M - 1), i = div_rcp(p, plan.rcp_g);
      gll_vaddr(qb + (int64_t)(i * Hq + p - i * G) * ROWB + 16 * (lp ^ swk(r)),
                uniform(qarea + 1024u * blk));
    }
  }

  // ---- chunk loads.  Load e of a tile covers tile rows e*RPI .. e*RPI+RPI-1: lane
  //      l writes 16 bytes at 16l of that 1 KB block (row l / CH, physical chunk
  //      l % CH) and fetches the logical chunk the swizzle stores there.  A chunk
  //      wholly inside the cache is issued as scalar base + lane offsets (offsets
  //      less the 1 KB instruction offsets); a chunk reaching the new rows or the
  //      end of the split forms its rows per lane (rows past the end clamped onto
  //      the last key: loaded, then masked).
  uint32_t kvo[IPT], vvo[IPT];
#pragma unroll
  for (int e = 0; e < IPT; e++) {
    const int r = e * RPI + lr;
    kvo[e] = (uint32_t)r * rsb + 16u * (uint32_t)(lp ^ swk(r)) - 1024u * (uint32_t)(e % 4);
    vvo[e] = (uint32_t)r * rsb + 16u * (uint32_t)(lp ^ swv(r)) - 1024u * (uint32_t)(e % 4);
  }
  const int kclear = min(L, kstop);  // chunks ending at or below this key need no mask
  auto issue_chunk = [&](int c, uint32_t slot) {
    const int key0 = kbeg + (c * NW + wave) * TK;
    if (key0 + TK <= kclear) {
      const char* kb = uniform_ptr(kc + (int64_t)key0 * rsb);
      const char* vb = uniform_ptr(vc + (int64_t)key0 * rsb);
#pragma unroll
      for (int gi = 0; gi < NG; gi++) {
        gll_block<4>(kb, kvo + 4 * gi, uniform(slot + 4096u * gi));
        gll_block<4>(vb, vvo + 4 * gi, uniform(slot + TILEB + 4096u * gi));
      }
    } else {
#pragma unroll
      for (int e = 0; e < IPT; e++) {
        const int r = e * RPI + lr, key = min(key0 + r, kstop - 1);
        const int64_t ro = key < L ? (int64_t)key * rsb : (int64_t)(key - L) * rsb;
        gll_vaddr((key < L ? kc : kn) + ro + 16 * (lp ^ swk(r)), uniform(slot + 1024u * e));
        gll_vaddr((key < L ? vc : vn) + ro + 16 * (lp ^ swv(r)), uniform(slot + TILEB + 1024u * e));
      }
    }
  };

  const auto lo = [&] {
    if constexpr (F8) return lane_offsets8(lane);
    else return lane_offsets<D>(lane);
  }();
  using Ops = typename std::conditional<F8, Ops8, Ops16<D>>::type;
  using KAddr = typename std::conditional<F8, uint32_t[2][2], uint32_t[D / 16]>::type;
  KAddr kaddr;
  uint32_t vaddr[MB];
  Ops op;
  if constexpr (F8) {
#pragma unroll
    for (int i = 0; i < 8; i++) op.ones[i] = 0x38383838;  // e4m3 1.0 in every byte
#pragma unroll
    for (int i = 0; i < 16; i++) op.rs[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int part = 0; part < 2; part++) kaddr[ks][part] = wring + lo.k[ks][part];
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++) kaddr[ks] = wring + lo.k[ks];
  }
#pragma unroll
  for (int mb = 0; mb < MB; mb++) vaddr[mb] = wring + TILEB + lo.v[mb];

  // ---- prologue: the first NST chunks of this wave, then the query tile together
  //      with chunk 0
#pragma unroll
  for (int c = 0; c < NST; c++)
    if (c < nmine) issue_chunk(c, wring + c * SLOTB);
  if (nmine >= NST)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(AFTER) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (F8) {
#pragma unroll
    for (int ks = 0; ks < 2; ks++) op.q[ks] = lds_read_2x16(qarea + lo.q[ks][0], qarea + lo.q[ks][1]);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++) op.q[ks] = *(const LDS_AS bf16x8*)(uintptr_t)(qarea + lo.k[ks]);
  }

  const float c2 = a.scale_log2;
  const int qi = div_rcp(min(row0 + n, M - 1), plan.rcp_g);  // token of this lane's row
  State<MB> acc;
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc.o[mb][i] = 0.f;
  acc.mlog = -1e30f;
  acc.lsum = 0.f;
  acc.thr = (acc.mlog + (F::kBias + F::kThreshold)) / c2;

  // ---- the stream: chunk c of this wave in stage c mod NST; the stage is refilled
  //      with chunk c+NST once the operand reads of chunk c have returned
  for (int c0 = 0; c0 < nmine; c0 += NST) {
#pragma unroll
    for (int j = 0; j < NST; j++) {
      const int c = c0 + j;
      if (c >= nmine) break;
      if (c + NST <= nmine)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(AFTER) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const uint32_t off = (uint32_t)j * SLOTB;
      const int key0 = kbeg + (c * NW + wave) * TK;
      load_k_operands(kaddr, off, op);
      scores(op);
      load_v_operands(vaddr, off, op);
      prepare_scores<MB, true>(op, key0 + TK > kclear, key0, kstop, L, qi, h, c2, acc);
      numerators<MB>(op, c2, acc);
      values<MB>(op, acc);
      if (c + NST < nmine) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_chunk(c + NST, wring + off);
      }
    }
  }
  if constexpr (F8) acc.lsum = h == 0 ? op.rs[0] : 0.f;

  // ---- the cache append, second half
  app_store(0, app0);
  if (APT > 1) app_store(1, app1);
  if (APT > 2) app_store(2, app2);
  if (APT > 3) app_store(3, app3);

  // ---- merge the waves: waves 1.. leave their state in their own ring (all of
  //      their loads and reads are complete), wave 0 folds it in
  if (wave > 0) {
    float4* dst = (float4*)(lds + wave * WAVEB) + lane * (PER / 4);
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        dst[mb * 4 + i] = make_float4(acc.o[mb][4 * i], acc.o[mb][4 * i + 1], acc.o[mb][4 * i + 2],
                                      acc.o[mb][4 * i + 3]);
    dst[MB * 4] = make_float4(acc.mlog, acc.lsum, 0.f, 0.f);
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 1; w < NW; w++) {
    const float4* src = (const float4*)(lds + w * WAVEB) + lane * (PER / 4);
    const float4 ml = src[MB * 4];
    const float mn = fmaxf(acc.mlog, ml.x);
    const float a1 = __builtin_amdgcn_exp2f(acc.mlog - mn);
    const float a2 = __builtin_amdgcn_exp2f(ml.x - mn);
    acc.mlog = mn;
    acc.lsum = acc.lsum * a1 + ml.y * a2;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float4 v = src[mb * 4 + i];
        acc.o[mb][4 * i] = acc.o[mb][4 * i] * a1 + v.x * a2;
        acc.o[mb][4 * i + 1] = acc.o[mb][4 * i + 1] * a1 + v.y * a2;
        acc.o[mb][4 * i + 2] = acc.o[mb][4 * i + 2] * a1 + v.z * a2;
        acc.o[mb][4 * i + 3] = acc.o[mb][4 * i + 3] * a1 + v.w * a2;
      }
  }

  // ---- the tile's rows: normalised, rounded to bf16; lane (n, h) holds head_dim
  //      32mb + 8q + 4h .. +3 of row n for every (mb, q)
  const float lt = partner_sum(acc.lsum);
  const float inv = lt > 0.f ? (F8 ? a.out_scale : 1.f) / lt : 0.f;
  const int p = row0 + n;
  if (p >= M) return;
  const bool direct = sp.n_splits == 1;
  const int i = div_rcp(p, plan.rcp_g);
  uint16_t* dst = direct ? (uint16_t*)a.out + ((int64_t)(u.b * NQ + i) * Hq + u.g * G + p - i * G) * D
                         : (uint16_t*)a.part_o + ((int64_t)U * kDecodeRows + n) * D;
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4e;
      bf16x4e v;
#pragma unroll
      for (int j = 0; j < 4; j++) v[j] = (__bf16)(acc.o[mb][4 * q4 + j] * inv);
      *(bf16x4e*)(dst + 32 * mb + 8 * q4 + 4 * h) = v;
    }
  if (!direct && h == 0)
    *(float2*)(a.part_ml + ((int64_t)U * kDecodeRows + n) * 2) = make_float2(acc.mlog, lt);
}

template <class F, int D, int NST>
int launch_decode_t(const AttnArgs& a, const Plan& p, hipStream_t st, const LaunchEvents& ev) {
  hipExtLaunchKernelGGL((decode_kernel<F, D, kDecodeWaves, NST>), dim3(p.n_units),
                        dim3(64 * kDecodeWaves), 0, st, ev.start, ev.stop, 0, a, p);
  return (int)hipGetLastError();
}

template <int D, bool CAUSAL, int WM, int WK, int NSLOT>
int launch_one(const AttnArgs& a, const Plan& p, hipStream_t st, const LaunchEvents& ev) {
  hipExtLaunchKernelGGL((attn_bf16_kernel<D, CAUSAL, WM, WK, NSLOT>), dim3(p.n_units), dim3(512), 0,
                        st, ev.start, ev.stop, 0, a, p);
  return (int)hipGetLastError();
}


template <bool CAUSAL>
int launch_fp8(const AttnArgs& a, const Plan& p, hipStream_t st, const LaunchEvents& ev) {
  hipExtLaunchKernelGGL((attn_fp8_kernel<128, CAUSAL, 4, 2, 4>), dim3(p.n_units), dim3(512), 0, st,
                        ev.start, ev.stop, 0, a, p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_attn_fp8(const AttnArgs& a, const Plan& p, bool causal, void* stream,
                    const LaunchEvents& ev) {
  hipStream_t st = (hipStream_t)stream;
  if (p.n_units == 0) return 0;
  return causal ? launch_fp8<true>(a, p, st, ev) : launch_fp8<false>(a, p, st, ev);
}

int launch_decode(const AttnArgs& a, const Plan& p, int dtype, int head_dim, void* stream,
                  const LaunchEvents& ev) {
  hipStream_t st = (hipStream_t)stream;
  if (p.n_units == 0) return 0;
  // two stages of 16 KB (K and V chunk) per wave at head_dim 128, four of 8 KB at 64
  if (dtype == DG_FP8) return launch_decode_t<FmtFp8, 128, 2>(a, p, st, ev);
  if (head_dim == 128) return launch_decode_t<FmtBf16, 128, 2>(a, p, st, ev);
  return launch_decode_t<FmtBf16, 64, 4>(a, p, st, ev);
}

int launch_attn_bf16(const AttnArgs& a, const Plan& p, int head_dim, bool causal, void* stream,
                     const LaunchEvents& ev) {
  hipStream_t st = (hipStream_t)stream;
  if (p.n_units == 0) return 0;
  // 128 packed rows per unit: four row groups x two key groups
  if (head_dim == 128)
    return causal ? launch_one<128, true, 4, 2, 4>(a, p, st, ev)
                  : launch_one<128, false, 4, 2, 4>(a, p, st, ev);
  return causal ? launch_one<64, true, 4, 2, 8>(a, p, st, ev)
                : launch_one<64, false, 4, 2, 8>(a, p, st, ev);
}

}  // namespace dg
