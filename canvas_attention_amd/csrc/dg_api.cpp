// dg_api.cpp -- the C ABI of libdg: argument checks, the split-key plan and launches.
//
// Entry points follow the two attention modes of "DiffusionGemma Technical
// Report" (paperfeed.app summary, section "The mechanism: an AR model turned
// inside out"): the bidirectional canvas step over [cache ; canvas] and the
// causal block commit that appends the block to the cache; and the AR mode of
// the same weights (section "The numbers, honestly"): causal decoding of 1..16
// new tokens over the same cache.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "dg.h"
#include "dg_internal.h"

namespace {

using dg::AttnArgs;
using dg::key_granule;
using dg::make_decode_plan;
using dg::make_plan;
using dg::mfma_path;
using dg::out_elem_size;
using dg::partial_row_bytes;
using dg::Plan;
using dg::plan_workspace;

thread_local std::string g_last_error;

dg_status fail(dg_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dg_status fail(dg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Bytes of one stored input element (q, K, V).
size_t elem_size(int dtype) { return dtype == DG_FP8 ? 1 : dtype == DG_BF16 ? 2 : 4; }

// Call kinds: the canvas step, the block commit and decode attention.
enum Mode { kCanvasStep = 0, kCommit = 1, kDecode = 2 };

dg_status check_shape(const dg_shape* s, Mode mode = kCanvasStep) {
  if (!s) return fail(DG_ERR_NULL, "shape is NULL");
  if (s->dtype != DG_BF16 && s->dtype != DG_F32 && s->dtype != DG_FP8)
    return fail(DG_ERR_DTYPE, "unknown dtype %d (DG_BF16=0, DG_F32=1, DG_FP8=2)", s->dtype);
  if (s->batch < 1 || s->batch > DG_MAX_BATCH)
    return fail(DG_ERR_SHAPE, "batch %d outside 1..%d", s->batch, DG_MAX_BATCH);
  if (mode == kDecode) {
    if (s->n_canvas < 1 || s->n_canvas > DG_MAX_DECODE)
      return fail(DG_ERR_SHAPE, "decode of %d new tokens, must be 1..%d", s->n_canvas,
                  DG_MAX_DECODE);
  } else if (s->n_canvas != DG_N_CANVAS) {
    return fail(DG_ERR_SHAPE, "n_canvas %d, must be %d", s->n_canvas, DG_N_CANVAS);
  }
  if (s->n_heads_kv < 1 || s->n_heads_q < 1 || s->n_heads_q > 1024)
    return fail(DG_ERR_SHAPE, "head counts Hq=%d Hkv=%d invalid", s->n_heads_q, s->n_heads_kv);
  if (s->n_heads_q % s->n_heads_kv != 0)
    return fail(DG_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", s->n_heads_q, s->n_heads_kv);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(DG_ERR_SHAPE, "head_dim %d, must be 64 or 128", s->head_dim);
  if (!(s->scale == s->scale) || isinf(s->scale))
    return fail(DG_ERR_SHAPE, "scale is not finite");
  if (s->dtype == DG_FP8) {
    if (s->head_dim != 128)
      return fail(DG_ERR_SHAPE, "head_dim %d, DG_FP8 supports 128 only", s->head_dim);
    const float sc[3] = {s->q_scale, s->k_scale, s->v_scale};
    for (float x : sc)
      if (!(x == x) || isinf(x)) return fail(DG_ERR_SHAPE, "an fp8 tensor scale is not finite");
  }
  return DG_OK;
}

// Per-tensor scale of an fp8 tensor: <= 0 selects 1.
float tensor_scale(float x) { return x > 0.f ? x : 1.f; }

float effective_scale(const dg_shape* s) {
  return s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
}

// Keys per split forced through the environment (tests use it to exercise many
// splits and ragged split ends), rounded up to the dtype's key granule; 0 when
// unset.
int forced_split_keys(int dtype) {
  const char* e = getenv("DG_SPLIT_KEYS");
  if (!e || !*e) return 0;
  const long v = strtol(e, nullptr, 10);
  if (v <= 0) return 0;
  const int g = key_granule(dtype);
  return (int)(((v + g - 1) / g) * g);
}

// Target number of units: one workgroup per CU for the matrix-core kernels
// (eight waves, two per SIMD), one wave per SIMD for the fp32 kernel.
int target_units(int dtype) { return device_cu_count() * (mfma_path(dtype) ? 1 : 4); }

int decode_target_units(int dtype) {
  // the matrix-core decode kernel takes one workgroup per CU (its LDS rings); the
  // fp32 kernel runs one wave per unit, four per CU
  return device_cu_count() * (mfma_path(dtype) ? 1 : 4);
}

// ------------------------------------------------------------ kernel timing
constexpr int kMaxTimed = 4096;
struct Timing {
  bool enabled = false;
  hipEvent_t ev[2][kMaxTimed][2];  // [attn/merge][launch][begin/end]
  bool created[2][kMaxTimed] = {};
  int count[2] = {0, 0};
} g_timing;

void time_begin(int kind, hipStream_t st) {
  if (!g_timing.enabled) return;
  const int k = g_timing.count[kind];
  if (k >= kMaxTimed) return;
  if (!g_timing.created[kind][k]) {
    if (hipEventCreate(&g_timing.ev[kind][k][0]) != hipSuccess ||
        hipEventCreate(&g_timing.ev[kind][k][1]) != hipSuccess)
      return;
    g_timing.created[kind][k] = true;
  }
  hipEventRecord(g_timing.ev[kind][k][0], st);
}

void time_end(int kind, hipStream_t st) {
  if (!g_timing.enabled) return;
  const int k = g_timing.count[kind];
  if (k >= kMaxTimed || !g_timing.created[kind][k]) return;
  hipEventRecord(g_timing.ev[kind][k][1], st);
  g_timing.count[kind] = k + 1;
}

// The event pair of the next timed launch of `kind`, recorded by the launch itself
// with its dispatch (so the interval is the kernel's own execution, without the
// time a separate event marker spends in the queue); null events when timing is
// off or the record is full.  timing_commit keeps the pair once the launch has
// been enqueued.
dg::LaunchEvents timing_events(int kind) {
  dg::LaunchEvents ev;
  if (!g_timing.enabled) return ev;
  const int k = g_timing.count[kind];
  if (k >= kMaxTimed) return ev;
  if (!g_timing.created[kind][k]) {
    if (hipEventCreate(&g_timing.ev[kind][k][0]) != hipSuccess ||
        hipEventCreate(&g_timing.ev[kind][k][1]) != hipSuccess)
      return ev;
    g_timing.created[kind][k] = true;
  }
  ev.start = g_timing.ev[kind][k][0];
  ev.stop = g_timing.ev[kind][k][1];
  return ev;
}

void timing_commit(int kind, const dg::LaunchEvents& ev) {
  if (ev.start) g_timing.count[kind]++;
}

struct Call {
  dg_shape shape;
  Plan plan;
  AttnArgs args;
  bool causal;
  Mode mode;
};

// Partial rows [n_units][R][D] at the start of the workspace, then (max, sum) pairs.
void set_workspace(Call* c, void* workspace) {
  c->args.part_o = workspace;
  c->args.part_ml = workspace ? (float*)((char*)workspace + (size_t)c->plan.n_units *
                                                               c->plan.rows_per_unit *
                                                               c->shape.head_dim *
                                                               out_elem_size(c->shape.dtype))
                              : nullptr;
}

dg_status prepare(const dg_shape* shape, const void* q, const dg_kv* kv_cache,
                  const int32_t* prefix_len, const dg_kv* kv_new, void* out, void* workspace,
                  size_t ws_bytes, Mode mode, Call* c) {
  dg_status st = check_shape(shape, mode);
  if (st) return st;
  const bool commit = mode != kCanvasStep;  // causal, and the new rows join the cache
  const int nq = mode == kDecode ? shape->n_canvas : DG_N_CANVAS;
  if (!q || !out || !kv_cache || !kv_new || !prefix_len)
    return fail(DG_ERR_NULL, "a required argument is NULL (q, out, caches or prefix_len)");
  if (!kv_new->k || !kv_new->v) return fail(DG_ERR_NULL, "canvas/block/new K or V is NULL");
  if (kv_new->capacity != nq)
    return fail(DG_ERR_SHAPE, "canvas/block/new K/V capacity %lld, must be %d",
                (long long)kv_new->capacity, nq);
  if (kv_cache->capacity < 0) return fail(DG_ERR_CAPACITY, "negative cache capacity");
  if ((!kv_cache->k || !kv_cache->v) && (kv_cache->capacity > 0 || commit))
    return fail(DG_ERR_NULL, "cache K or V is NULL");
  const void* ptrs[] = {q, out, kv_new->k, kv_new->v, kv_cache->k, kv_cache->v, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DG_ERR_ALIGN, "device pointer %p is not 16-byte aligned", p);
  for (int b = 0; b < shape->batch; b++) {
    const int64_t L = prefix_len[b];
    if (L < 0) return fail(DG_ERR_CAPACITY, "prefix_len[%d] = %lld is negative", b, (long long)L);
    const int64_t need = commit ? L + nq : L;
    if (need > kv_cache->capacity)
      return fail(DG_ERR_CAPACITY, "prefix_len[%d] = %lld%s exceeds cache capacity %lld", b,
                  (long long)L, commit ? (mode == kDecode ? " + new tokens" : " + 256") : "",
                  (long long)kv_cache->capacity);
    if (L + DG_N_CANVAS > INT32_MAX / 2)
      return fail(DG_ERR_CAPACITY, "prefix_len[%d] too large", b);
  }
  c->shape = *shape;
  c->causal = commit;
  c->mode = mode;
  if (mode == kDecode)
    make_decode_plan(shape, prefix_len, decode_target_units(shape->dtype),
                     forced_split_keys(shape->dtype), &c->plan);
  else
    make_plan(shape, prefix_len, target_units(shape->dtype), forced_split_keys(shape->dtype),
              &c->plan);
  // unit and row indices stay below 2^16, which keeps every kernel division n/d with
  // n*d < 2^32 (the reciprocal-multiplier form is exact there)
  if (c->plan.n_units >= dg::kMaxUnits)
    return fail(DG_ERR_SHAPE, "%d work units, at most %d", c->plan.n_units, dg::kMaxUnits - 1);
  const size_t need_ws = plan_workspace(shape, c->plan);
  if (need_ws > ws_bytes)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes, this call needs %zu", ws_bytes, need_ws);
  if (need_ws > 0 && !workspace) return fail(DG_ERR_NULL, "workspace is NULL");
  AttnArgs& a = c->args;
  a.q = q;
  a.k_cache = kv_cache->k;
  a.v_cache = kv_cache->v;
  a.k_new = kv_new->k;
  a.v_new = kv_new->v;
  a.k_append = commit ? kv_cache->k : nullptr;
  a.v_append = commit ? kv_cache->v : nullptr;
  a.out = out;
  set_workspace(c, workspace);
  a.cap = kv_cache->capacity;
  a.n_heads_q = shape->n_heads_q;
  a.n_heads_kv = shape->n_heads_kv;
  a.scale_log2 = effective_scale(shape) * 1.4426950408889634f;
  a.out_scale = 1.f;
  if (shape->dtype == DG_FP8) {
    a.scale_log2 *= tensor_scale(shape->q_scale) * tensor_scale(shape->k_scale);
    a.out_scale = tensor_scale(shape->v_scale);
  }
  return DG_OK;
}

dg_status launch(const Call& c, void* stream, bool timed = true) {
  const int dt = c.shape.dtype;
  const dg::LaunchEvents none;
  dg::LaunchEvents ev = timed && c.plan.n_units > 0 ? timing_events(0) : none;
  int err;
  if (c.mode == kDecode && mfma_path(dt))
    err = dg::launch_decode(c.args, c.plan, dt, c.shape.head_dim, stream, ev);
  else if (dt == DG_BF16)
    err = dg::launch_attn_bf16(c.args, c.plan, c.shape.head_dim, c.causal, stream, ev);
  else if (dt == DG_FP8)
    err = dg::launch_attn_fp8(c.args, c.plan, c.causal, stream, ev);
  else
    err = dg::launch_attn_f32(c.args, c.plan, c.shape.head_dim, c.causal, stream, ev);
  if (err != 0)
    return fail(DG_ERR_HIP, "attention kernel launch failed: %s",
                hipGetErrorString((hipError_t)err));
  timing_commit(0, ev);
  bool any = false;
  for (int b = 0; b < c.plan.batch; b++) any = any || c.plan.seq[b].n_splits > 1;
  if (any) {
    ev = timed ? timing_events(1) : none;
    err = dg::launch_merge(c.args, c.plan, c.shape.head_dim, dt != DG_F32, stream, ev);
    if (err != 0)
      return fail(DG_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString((hipError_t)err));
    timing_commit(1, ev);
  }
  if (getenv("DG_LOG")) {
    static const char* const kModeName[] = {"canvas", "commit", "decode"};
    fprintf(stderr, "[dg] %s dtype=%d units=%d R=%d NRT=%d", kModeName[c.mode], dt,
            c.plan.n_units, c.plan.rows_per_unit, c.plan.n_rowtiles);
    for (int b = 0; b < c.plan.batch; b++)
      fprintf(stderr, " | b%d L=%d S=%d keys/split=%d", b, c.plan.seq[b].prefix_len,
              c.plan.seq[b].n_splits, c.plan.seq[b].split_keys);
    fprintf(stderr, "\n");
  }
  return DG_OK;
}

// ------------------------------------------------ no-allocation entry point
// dg_canvas_attn_noalloc keeps its partial results in this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` is only a stand-in for the
// symbol: the device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = DG_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// The scratch address on the GPU that `stream` belongs to (the current device for
// the null stream), looked up once per device with that device current.
dg_status scratch_address(void* stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(DG_ERR_HIP, "device index %d outside 0..63", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(DG_ERR_HIP, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      e = hipSetDevice(cur);
      if (e != hipSuccess)
        return fail(DG_ERR_HIP, "hipSetDevice(%d) failed: %s", cur, hipGetErrorString(e));
    }
    if (r != hipSuccess || !p)
      return fail(DG_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s",
                  hipGetErrorString(r));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

}  // namespace

extern "C" {

size_t dg_workspace_bytes(const dg_shape* shape, int64_t max_prefix_len) {
  if (check_shape(shape) != DG_OK || max_prefix_len < 0 || max_prefix_len > INT32_MAX / 2)
    return 0;
  return dg::workspace_bound(shape, max_prefix_len, target_units(shape->dtype),
                             forced_split_keys(shape->dtype));
}

dg_status dg_canvas_attn(const dg_shape* shape, const void* q, const dg_kv* kv_cache,
                         const int32_t* prefix_len, const dg_kv* kv_canvas, void* out,
                         void* workspace, size_t ws_bytes, void* stream) {
  Call c;
  dg_status st = prepare(shape, q, kv_cache, prefix_len, kv_canvas, out, workspace, ws_bytes,
                         kCanvasStep, &c);
  if (st) return st;
  return launch(c, stream);
}

dg_status dg_canvas_attn_noalloc(const dg_shape* shape, const void* q, const dg_kv* kv_cache,
                                 const int32_t* prefix_len, const dg_kv* kv_canvas, void* out,
                                 void* stream) {
  // Validate and plan against a stand-in workspace of the scratch's size (never
  // dereferenced), so that a call the scratch cannot hold is rejected before any
  // HIP call; then point the partial results at this device's scratch array.
  Call c;
  void* const stand_in = (void*)(uintptr_t)256;
  dg_status st = prepare(shape, q, kv_cache, prefix_len, kv_canvas, out, stand_in, kScratchBytes,
                         kCanvasStep, &c);
  if (st == DG_ERR_WORKSPACE)
    return fail(DG_ERR_WORKSPACE,
                "this call needs %zu bytes of partial results, more than the %zu-byte scratch "
                "of dg_canvas_attn_noalloc (use dg_canvas_attn with a workspace)",
                plan_workspace(shape, c.plan), kScratchBytes);
  if (st) return st;
  void* ws = nullptr;
  if (plan_workspace(shape, c.plan) > 0) {
    st = scratch_address(stream, &ws);
    if (st) return st;
  }
  set_workspace(&c, ws);
  return launch(c, stream, false);
}

dg_status dg_commit_block(const dg_shape* shape, const void* q_blk, const dg_kv* kv_blk,
                          dg_kv* kv_cache, const int32_t* prefix_len, void* out,
                          void* workspace, size_t ws_bytes, void* stream) {
  Call c;
  dg_status st = prepare(shape, q_blk, kv_cache, prefix_len, kv_blk, out, workspace, ws_bytes,
                         kCommit, &c);
  if (st) return st;
  return launch(c, stream);
}

size_t dg_decode_workspace_bytes(const dg_shape* shape, int64_t max_prefix_len) {
  if (check_shape(shape, kDecode) != DG_OK || max_prefix_len < 0 ||
      max_prefix_len > INT32_MAX / 2)
    return 0;
  return dg::decode_workspace_bound(shape, max_prefix_len, decode_target_units(shape->dtype),
                                    forced_split_keys(shape->dtype));
}

dg_status dg_decode_attn(const dg_shape* shape, const void* q, const dg_kv* kv_new,
                         dg_kv* kv_cache, const int32_t* prefix_len, void* out,
                         void* workspace, size_t ws_bytes, void* stream) {
  Call c;
  dg_status st = prepare(shape, q, kv_cache, prefix_len, kv_new, out, workspace, ws_bytes,
                         kDecode, &c);
  if (st) return st;
  return launch(c, stream);
}

dg_status dg_canvas_step_loop(const dg_shape* shape, int32_t n_steps, const void* q,
                              int64_t q_step_stride, const dg_kv* kv_canvas,
                              int64_t kv_step_stride, const dg_kv* kv_cache,
                              const int32_t* prefix_len, void* out, int64_t out_step_stride,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (n_steps < 0) return fail(DG_ERR_SHAPE, "n_steps %d is negative", n_steps);
  if (q_step_stride < 0 || kv_step_stride < 0 || out_step_stride < 0)
    return fail(DG_ERR_SHAPE, "step strides must be >= 0");
  Call c;
  dg_status st = prepare(shape, q, kv_cache, prefix_len, kv_canvas, out, workspace, ws_bytes,
                         kCanvasStep, &c);
  if (st) return st;
  const size_t es = elem_size(shape->dtype), eo = out_elem_size(shape->dtype);
  if (((q_step_stride * (int64_t)es) & 15) || ((kv_step_stride * (int64_t)es) & 15) ||
      ((out_step_stride * (int64_t)eo) & 15))
    return fail(DG_ERR_ALIGN, "step strides must keep 16-byte alignment");
  for (int s = 0; s < n_steps; s++) {
    Call cs = c;
    cs.args.q = (const char*)q + (int64_t)s * q_step_stride * es;
    cs.args.k_new = (const char*)kv_canvas->k + (int64_t)s * kv_step_stride * es;
    cs.args.v_new = (const char*)kv_canvas->v + (int64_t)s * kv_step_stride * es;
    cs.args.out = (char*)out + (int64_t)s * out_step_stride * eo;
    st = launch(cs, stream);
    if (st) return st;
  }
  return DG_OK;
}

dg_status dg_canvas_sample(const dg_sample_shape* shape, const void* logits,
                           const int32_t* noise_tokens, const int32_t* prev_argmax,
                           float* entropy, int32_t* argmax, int32_t* tokens,
                           int32_t* accepted, int32_t* stop, void* stream) {
  if (!shape) return fail(DG_ERR_NULL, "shape is NULL");
  if (shape->batch < 1 || shape->batch > DG_MAX_BATCH)
    return fail(DG_ERR_SHAPE, "batch %d outside 1..%d", shape->batch, DG_MAX_BATCH);
  if (shape->n_canvas != DG_N_CANVAS)
    return fail(DG_ERR_SHAPE, "n_canvas %d, must be %d", shape->n_canvas, DG_N_CANVAS);
  if (shape->vocab < 8 || shape->vocab % 8 != 0 || shape->vocab > (1 << 27))
    return fail(DG_ERR_SHAPE, "vocab %d: a multiple of 8 in 8..2^27", shape->vocab);
  if (!(shape->tau > 0.f) || isinf(shape->tau))
    return fail(DG_ERR_SHAPE, "tau must be finite and > 0");
  if (!(shape->budget >= 0.f) || shape->budget > 1e6f)
    return fail(DG_ERR_SHAPE, "budget must be in 0..1e6");
  if (!(shape->stop_entropy >= 0.f) || shape->stop_entropy > 1e6f)
    return fail(DG_ERR_SHAPE, "stop_entropy must be in 0..1e6");
  if (!logits || !noise_tokens || !entropy || !argmax || !tokens || !accepted || !stop)
    return fail(DG_ERR_NULL, "a required argument is NULL (only prev_argmax may be)");
  if (!aligned16(logits)) return fail(DG_ERR_ALIGN, "logits %p is not 16-byte aligned", logits);
  const void* words[] = {noise_tokens, prev_argmax, entropy, argmax, tokens, accepted, stop};
  for (const void* p : words)
    if (((uintptr_t)p & 3u) != 0) return fail(DG_ERR_ALIGN, "pointer %p is not 4-byte aligned", p);
  dg::SampleArgs a;
  a.logits = logits;
  a.noise = noise_tokens;
  a.prev = prev_argmax;
  a.entropy = entropy;
  a.argmax = argmax;
  a.tokens = tokens;
  a.accepted = accepted;
  a.stop = stop;
  a.qbudget = llrint((double)shape->budget * 4294967296.0);
  a.qstop = llrint((double)shape->stop_entropy * 4294967296.0);
  a.c = (float)(1.4426950408889634 / (double)shape->tau);
  a.vocab = shape->vocab;
  a.batch = shape->batch;
  const int err = dg::launch_sample(a, stream);
  if (err != 0)
    return fail(DG_ERR_HIP, "sampler launch failed: %s", hipGetErrorString((hipError_t)err));
  return DG_OK;
}

// Workspace layout of dg_self_condition: every part 256-byte aligned.
struct SelfcondLayout {
  size_t pblk, stats, part, yblk, hblk, total;
  int vocab_splits, split_w1, split_w2;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static dg_status selfcond_layout(const dg_selfcond_shape* s, SelfcondLayout* l) {
  if (!s) return fail(DG_ERR_NULL, "shape is NULL");
  if (s->batch < 1 || s->batch > DG_MAX_BATCH)
    return fail(DG_ERR_SHAPE, "batch %d outside 1..%d", s->batch, DG_MAX_BATCH);
  if (s->n_canvas != DG_N_CANVAS)
    return fail(DG_ERR_SHAPE, "n_canvas %d, must be %d", s->n_canvas, DG_N_CANVAS);
  if (s->vocab < dg::kSelfcondBlock || s->vocab % dg::kSelfcondBlock != 0 ||
      s->vocab > DG_SELFCOND_MAX_VOCAB)
    return fail(DG_ERR_SHAPE, "vocab %d: a multiple of 32 in 32..%d", s->vocab, DG_SELFCOND_MAX_VOCAB);
  if (s->d_model < 256 || s->d_model % 256 != 0 || s->d_model > 16384)
    return fail(DG_ERR_SHAPE, "d_model %d: a multiple of 256 in 256..16384", s->d_model);
  if (s->d_hidden < 128 || s->d_hidden % 128 != 0 || s->d_hidden > 16384)
    return fail(DG_ERR_SHAPE, "d_hidden %d: a multiple of 128 in 128..16384", s->d_hidden);
  const size_t M = (size_t)s->batch * DG_N_CANVAS;
  const int cus = device_cu_count();
  l->vocab_splits = (s->vocab + dg::kSelfcondSplit - 1) / dg::kSelfcondSplit;
  l->split_w1 = dg::selfcond_splits(s->d_model, s->d_hidden, (int)M, cus);
  l->split_w2 = dg::selfcond_splits(s->d_hidden, s->d_model, (int)M, cus);
  const size_t s1 = (size_t)l->vocab_splits;
  const size_t s2 = (size_t)((s->d_model + l->split_w1 - 1) / l->split_w1);
  const size_t s3 = (size_t)((s->d_hidden + l->split_w2 - 1) / l->split_w2);
  const size_t part = std::max({s1 * M * s->d_model, s2 * M * s->d_hidden, s3 * M * s->d_model}) * 4;
  l->pblk = 0;
  l->stats = align256(l->pblk + M * s->vocab * 2);
  l->part = align256(l->stats + s1 * M * 8);
  l->yblk = align256(l->part + part);
  l->hblk = align256(l->yblk + M * s->d_model * 2);
  l->total = align256(l->hblk + M * s->d_hidden * 2);
  return DG_OK;
}

static void hook_begin(int kind, hipStream_t st) { time_begin(kind, st); }
static void hook_end(int kind, hipStream_t st) { time_end(kind, st); }

size_t dg_selfcond_workspace_bytes(const dg_selfcond_shape* shape) {
  SelfcondLayout l;
  return selfcond_layout(shape, &l) == DG_OK ? l.total : 0;
}

dg_status dg_self_condition(const dg_selfcond_shape* shape, const void* logits, const void* embed,
                            const void* w1, const void* w2, void* z, void* workspace, size_t ws_bytes,
                            void* stream) {
  SelfcondLayout l;
  dg_status st = selfcond_layout(shape, &l);
  if (st) return st;
  if (!logits || !embed || !w1 || !w2 || !z || !workspace)
    return fail(DG_ERR_NULL, "a required argument is NULL (logits, embed, w1, w2, z, workspace)");
  const void* ptrs[] = {logits, embed, w1, w2, z, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DG_ERR_ALIGN, "device pointer %p is not 16-byte aligned", p);
  if (ws_bytes < l.total)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes, this call needs %zu", ws_bytes, l.total);
  dg::SelfcondArgs a;
  char* ws = (char*)workspace;
  a.logits = logits;
  a.embed = embed;
  a.w1 = w1;
  a.w2 = w2;
  a.z = z;
  a.pblk = ws + l.pblk;
  a.stats = (float2*)(ws + l.stats);
  a.part = (float*)(ws + l.part);
  a.yblk = ws + l.yblk;
  a.hblk = ws + l.hblk;
  a.rows = shape->batch * DG_N_CANVAS;
  a.vocab = shape->vocab;
  a.vocab_splits = l.vocab_splits;
  a.d_model = shape->d_model;
  a.d_hidden = shape->d_hidden;
  a.split_w1 = l.split_w1;
  a.split_w2 = l.split_w2;
  a.time_begin = hook_begin;
  a.time_end = hook_end;
  const int err = dg::launch_selfcond(a, stream);
  if (err != 0)
    return fail(DG_ERR_HIP, "self-conditioning launch failed: %s", hipGetErrorString((hipError_t)err));
  return DG_OK;
}

const char* dg_status_string(dg_status status) {
  switch (status) {
    case DG_OK: return "DG_OK";
    case DG_ERR_NULL: return "DG_ERR_NULL";
    case DG_ERR_SHAPE: return "DG_ERR_SHAPE";
    case DG_ERR_DTYPE: return "DG_ERR_DTYPE";
    case DG_ERR_CAPACITY: return "DG_ERR_CAPACITY";
    case DG_ERR_WORKSPACE: return "DG_ERR_WORKSPACE";
    case DG_ERR_HIP: return "DG_ERR_HIP";
    case DG_ERR_ALIGN: return "DG_ERR_ALIGN";
    default: return "DG_ERR_UNKNOWN";
  }
}

const char* dg_last_error(void) { return g_last_error.c_str(); }

dg_status dg_kernel_timing_enable(int32_t enable) {
  g_timing.enabled = enable != 0;
  return DG_OK;
}

dg_status dg_kernel_timing_samples(float* attn_ms, float* merge_ms, int32_t max_n,
                                   int32_t* n_attn, int32_t* n_merge) {
  float* dst[2] = {attn_ms, merge_ms};
  for (int kind = 0; kind < 2; kind++) {
    for (int k = 0; k < g_timing.count[kind]; k++) {
      if (hipEventSynchronize(g_timing.ev[kind][k][1]) != hipSuccess)
        return fail(DG_ERR_HIP, "hipEventSynchronize failed");
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, g_timing.ev[kind][k][0], g_timing.ev[kind][k][1]) !=
          hipSuccess)
        return fail(DG_ERR_HIP, "hipEventElapsedTime failed");
      if (dst[kind] && k < max_n) dst[kind][k] = ms;
    }
  }
  if (n_attn) *n_attn = g_timing.count[0];
  if (n_merge) *n_merge = g_timing.count[1];
  g_timing.count[0] = g_timing.count[1] = 0;
  return DG_OK;
}

dg_status dg_kernel_timing_read(int32_t* n_attn, double* attn_ms, int32_t* n_merge,
                                double* merge_ms) {
  double tot[2] = {0, 0};
  for (int kind = 0; kind < 2; kind++) {
    for (int k = 0; k < g_timing.count[kind]; k++) {
      if (hipEventSynchronize(g_timing.ev[kind][k][1]) != hipSuccess)
        return fail(DG_ERR_HIP, "hipEventSynchronize failed");
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, g_timing.ev[kind][k][0], g_timing.ev[kind][k][1]) !=
          hipSuccess)
        return fail(DG_ERR_HIP, "hipEventElapsedTime failed");
      tot[kind] += ms;
    }
  }
  if (n_attn) *n_attn = g_timing.count[0];
  if (n_merge) *n_merge = g_timing.count[1];
  if (attn_ms) *attn_ms = tot[0];
  if (merge_ms) *merge_ms = tot[1];
  g_timing.count[0] = g_timing.count[1] = 0;
  return DG_OK;
}

}  // extern "C"
