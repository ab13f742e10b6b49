/*
 * dg.h -- C ABI of the canvas denoising attention library (libdg.so, gfx950).
 *
 * The operations come from "DiffusionGemma Technical Report" (paperfeed.app
 * summary page), section "The mechanism: an AR model turned inside out":
 *   - a single transformer is run in two attention modes: the prompt and all
 *     committed text are encoded causally into a KV cache, and a 256-token
 *     canvas is refined with full bidirectional attention within itself while
 *     cross-attending to that cache (dg_canvas_attn, dg_canvas_step_loop);
 *   - once a canvas is fully denoised it is frozen, encoded causally and
 *     appended to the cache, so the growing context is never re-encoded
 *     (dg_commit_block).
 * The same weights also decode causally, token by token, over the same cache
 * (AR mode, section "The numbers, honestly"; dg_decode_attn, which also takes
 * several drafted tokens at once for hybrid decoding).  After each step the
 * sampler (dg_canvas_sample) accepts or re-noises positions, and the predicted
 * distribution feeds the next step through the self-conditioning input
 * (dg_self_condition).
 * The same page (section "The numbers, honestly") and the report's abstract
 * give the block size (256 positions) and the ~12 refinement passes per block
 * that dg_canvas_step_loop is meant for.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Element type: DG_BF16 (bf16 storage, fp32 accumulation, bf16 output rounded
 * to nearest-even), DG_F32 (fp32 storage and arithmetic throughout) or DG_FP8
 * (queries, keys and values stored as OCP e4m3 -- 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals, largest finite value 448, bytes 0x7f and
 * 0xff NaN, no infinities -- each tensor with a per-tensor scale, so that the
 * value an element stands for is scale * e4m3 value; fp32 accumulation, the
 * softmax weights rounded to e4m3 for the value product, bf16 output rounded to
 * nearest-even; head_dim 128 only).  The fp8 element type is the deployment
 * precision of the report's throughput figures (section "The numbers, honestly":
 * H100, FP8).
 *
 * Layouts (all row-major, element strides implied by the shape):
 *   queries q, q_blk, out ......... [B][Nc][Hq][D]   (out is bf16 for DG_FP8)
 *   canvas / block / new K, V ..... [B][Nc][Hkv][D]     (dg_kv.capacity = Nc)
 *   cache K, V .................... [B][capacity][Hkv][D]
 * Query head h reads kv head h / (Hq / Hkv) (grouped-query attention with
 * consecutive query heads sharing a kv head).  prefix_len[b] (host int32
 * array of B entries) is the number of valid cache rows of sequence b.
 *
 * Ownership: the caller owns every buffer (inputs, outputs, cache, workspace)
 * and keeps it alive until the work enqueued on `stream` has completed.  All
 * device pointers must be 16-byte aligned.  The library allocates no device
 * memory and keeps no state between calls, apart from the scratch array of
 * dg_canvas_attn_noalloc and the record of the kernel timing hooks (both below).
 *
 * Streams and errors: `stream` is a hipStream_t passed as void* (NULL = the
 * default stream).  Every argument is validated on the host before any HIP
 * call; a rejected call enqueues nothing and returns a negative status.  DG_OK
 * means the work was enqueued, not that it has finished.  Device faults surface
 * at the caller's next synchronisation.  dg_last_error() gives a thread-local
 * description of the last failure.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dg_status;

enum {
  DG_OK = 0,
  DG_ERR_NULL = -1,      /* a required pointer is NULL                          */
  DG_ERR_SHAPE = -2,     /* unsupported or inconsistent shape                   */
  DG_ERR_DTYPE = -3,     /* unknown element type                                */
  DG_ERR_CAPACITY = -4,  /* prefix_len negative or beyond the cache capacity    */
  DG_ERR_WORKSPACE = -5, /* workspace smaller than dg_workspace_bytes() asks    */
  DG_ERR_HIP = -6,       /* a HIP runtime call or kernel launch failed          */
  DG_ERR_ALIGN = -7      /* a device pointer is not 16-byte aligned             */
};

enum { DG_BF16 = 0, DG_F32 = 1, DG_FP8 = 2 };

/* Limits checked by every entry point. */
#define DG_N_CANVAS 256  /* canvas / block length: fixed at 256 positions      */
#define DG_MAX_BATCH 64  /* sequences per call                                  */
#define DG_MAX_DECODE 16 /* new tokens per sequence of one dg_decode_attn call  */

typedef struct {
  int32_t dtype;      /* DG_BF16, DG_F32 or DG_FP8                               */
  int32_t batch;      /* B, 1..DG_MAX_BATCH                                      */
  int32_t n_canvas;   /* Nc, must equal DG_N_CANVAS (dg_decode_attn: the number  */
                      /* of new tokens k, 1..DG_MAX_DECODE)                      */
  int32_t n_heads_q;  /* Hq >= 1, a multiple of n_heads_kv                       */
  int32_t n_heads_kv; /* Hkv >= 1                                               */
  int32_t head_dim;   /* D: 64 or 128 (DG_FP8: 128)                             */
  float scale;        /* softmax scale; <= 0 selects 1/sqrt(D)                   */
  /* DG_FP8 only (ignored otherwise): the per-tensor scales of q (canvas or block
   * queries), of K (cache and canvas or block keys alike: the commit appends block
   * rows to the cache bit for bit) and of V; <= 0 selects 1.  Must be finite.    */
  float q_scale;
  float k_scale;
  float v_scale;
} dg_shape;

/* A pair of K and V buffers, each [B][capacity][Hkv][D]. */
typedef struct {
  void* k;
  void* v;
  int64_t capacity; /* rows per sequence (Nc for canvas/block buffers)           */
} dg_kv;

/*
 * Workspace bytes that any call with this shape and every prefix_len[b] <=
 * max_prefix_len needs (partial results of the split-key plan).  Returns 0 for
 * an invalid shape.  Sizing once for the largest prefix a caller will reach
 * makes one workspace serve a whole generation.  The plan itself depends only on
 * the shape, the prefix lengths and the device: about one unit of work per CU,
 * or, for a ragged batch whose units would spill into a partial second round of
 * workgroups, a smaller split that fills up to four rounds.
 */
size_t dg_workspace_bytes(const dg_shape* shape, int64_t max_prefix_len);

/*
 * Canvas denoising step (bidirectional decoder of the mechanism section).
 * For every sequence b, query head h and canvas row i:
 *   out[b,i,h,:] = softmax_j(scale * <q[b,i,h,:], k_j>) v_j
 * (with DG_FP8, q, k_j and v_j are the scaled e4m3 values and out is bf16)
 * over j in { cache rows 0..prefix_len[b]-1 } U { canvas rows 0..Nc-1 } of kv
 * head h / (Hq/Hkv); no mask.  The cache is only read.
 *   q          [B][Nc][Hq][D] device
 *   kv_cache   device cache (k, v, capacity), capacity >= prefix_len[b]
 *   prefix_len host int32[B], 0 <= prefix_len[b] <= kv_cache->capacity
 *   kv_canvas  device canvas K/V, capacity must equal Nc
 *   out        [B][Nc][Hq][D] device, written completely
 *   workspace  device scratch of ws_bytes >= dg_workspace_bytes(shape, max_b L_b)
 *              (may be NULL when that is 0); contents are overwritten
 */
dg_status dg_canvas_attn(const dg_shape* shape, const void* q, const dg_kv* kv_cache,
                         const int32_t* prefix_len, const dg_kv* kv_canvas, void* out,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * dg_canvas_attn without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, result and validation as dg_canvas_attn,
 * bit for bit, except that the split partial results live in a file-scope
 * device array of the library of DG_NOALLOC_SCRATCH_BYTES bytes: one copy per
 * GPU, held from the library's first use on that GPU until the process ends; a
 * call uses the copy of the GPU its stream belongs to (the current device for
 * the null stream).
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the first call on a device looks up that device's scratch address
 * once.  A call whose partial results exceed the scratch is rejected with
 * DG_ERR_WORKSPACE before any HIP call (at Hq=16, Hkv=8, D=128 the scratch holds
 * every batch up to 8 sequences at any prefix length).  Every call on one GPU
 * shares its scratch, and each call overwrites what the last one left: calls
 * that overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  No kernel timing hooks run on this path.
 */
#define DG_NOALLOC_SCRATCH_BYTES (48u << 20)
dg_status dg_canvas_attn_noalloc(const dg_shape* shape, const void* q, const dg_kv* kv_cache,
                                 const int32_t* prefix_len, const dg_kv* kv_canvas, void* out,
                                 void* stream);

/*
 * Block commit (causal encoder of the mechanism section).  Block row i of
 * sequence b attends to cache rows 0..prefix_len[b]-1 and block rows 0..i
 * (diagonal included):
 *   out[b,i,h,:] = softmax_j(scale * <q_blk[b,i,h,:], k_j>) v_j
 * and the block's K/V rows are written, bit for bit, into cache rows
 * prefix_len[b] .. prefix_len[b]+Nc-1.  Cache rows below prefix_len[b] are not
 * modified.  prefix_len itself is not changed: the caller advances it by Nc.
 *   q_blk      [B][Nc][Hq][D] device
 *   kv_blk     device block K/V, capacity must equal Nc
 *   kv_cache   device cache; requires prefix_len[b] + Nc <= capacity
 *   prefix_len host int32[B]
 *   out        [B][Nc][Hq][D] device
 *   workspace  as for dg_canvas_attn
 */
dg_status dg_commit_block(const dg_shape* shape, const void* q_blk, const dg_kv* kv_blk,
                          dg_kv* kv_cache, const int32_t* prefix_len, void* out,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * n_steps canvas steps against one fixed cache (the ~12 refinement passes of
 * a block), enqueued in order on `stream`.  Step s reads
 *   q + s*q_step_stride, kv_canvas->k + s*kv_step_stride,
 *   kv_canvas->v + s*kv_step_stride
 * and writes out + s*out_step_stride (all strides in elements of the tensor
 * they step: input elements for q and K/V, output elements for out; each step
 * laid out as for dg_canvas_attn).  The result is bit for bit that of n_steps
 * separate dg_canvas_attn calls: in the model each step's queries depend on
 * the previous step's output, so steps are never fused; the loop plans once
 * and only removes per-call host work.  n_steps >= 0 and every stride >= 0
 * (DG_ERR_SHAPE otherwise); the workspace is reused by every step.
 */
dg_status dg_canvas_step_loop(const dg_shape* shape, int32_t n_steps, const void* q,
                              int64_t q_step_stride, const dg_kv* kv_canvas,
                              int64_t kv_step_stride, const dg_kv* kv_cache,
                              const int32_t* prefix_len, void* out, int64_t out_step_stride,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode attention ("DiffusionGemma Technical Report", paperfeed.app summary,
 * section "The numbers, honestly": the AR-mode paragraph runs the same weights
 * causally over the same cache, and the concurrency paragraph serves several
 * sequences at once).  shape->n_canvas is the number k of new tokens per
 * sequence, 1..DG_MAX_DECODE: one for plain AR decoding, more for a hybrid
 * decoder that checks drafted tokens in one pass.  New token i of sequence b
 * attends to cache rows 0..prefix_len[b]-1 and new rows 0..i (diagonal
 * included):
 *   out[b,i,h,:] = softmax_j(scale * <q[b,i,h,:], k_j>) v_j
 * and the new K/V rows are written, bit for bit, into cache rows
 * prefix_len[b] .. prefix_len[b]+k-1, as dg_commit_block does for a block.
 * prefix_len itself is not changed: the caller advances it by the number of
 * tokens it keeps (rows past the kept ones are overwritten by the next call).
 * Every element type; head_dim 64 or 128 (DG_FP8: 128).
 *   q          [B][k][Hq][D] device
 *   kv_new     device K/V of the new tokens, [B][k][Hkv][D]; capacity must equal k
 *   kv_cache   device cache; requires prefix_len[b] + k <= capacity
 *   prefix_len host int32[B]
 *   out        [B][k][Hq][D] device (bf16 for DG_FP8), written completely
 *   workspace  device scratch of ws_bytes >= dg_decode_workspace_bytes(shape,
 *              max_b L_b) (may be NULL when that is 0); contents are overwritten
 */
size_t dg_decode_workspace_bytes(const dg_shape* shape, int64_t max_prefix_len);
dg_status dg_decode_attn(const dg_shape* shape, const void* q, const dg_kv* kv_new,
                         dg_kv* kv_cache, const int32_t* prefix_len, void* out,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Canvas sampler ("DiffusionGemma Technical Report", paperfeed.app summary,
 * section "The mechanism: an AR model turned inside out", sampler paragraph).
 * After a denoising step, for every sequence b and canvas position i:
 *   entropy[b,i] = -sum_v q_v ln q_v,  q = softmax(logits[b,i,:] / tau)   (nats)
 *   argmax[b,i]  = the lowest v with the largest logit
 * Positions are then taken in ascending (entropy, i) order and accepted while the
 * cumulative entropy of the accepted ones stays <= budget (possibly none);
 *   tokens[b,i] = accepted ? argmax[b,i] : noise_tokens[b,i]
 * (noise_tokens: the caller's uniformly random tokens for re-noised positions),
 * and stop[b] = 1 iff the mean entropy of the canvas is < stop_entropy and every
 * argmax equals prev_argmax (the previous step's argmax; NULL: no previous step,
 * stop = 0).  The acceptance and stop decisions count each fp32 entropy as an
 * integer number of 2^-32 nats, so the cumulative sums are exact and do not
 * depend on any summation order.
 *   logits        [B][Nc][V] bf16 device, 16-byte aligned; V a multiple of 8,
 *                 8 <= V <= 2^27; finite or -inf (masked) values, one finite
 *                 value per row
 *   noise_tokens, prev_argmax [B][Nc] int32 device (prev_argmax may be NULL)
 *   entropy       [B][Nc] float device (out); argmax, tokens, accepted (0/1)
 *                 [B][Nc] int32 device (out); stop [B] int32 device (out)
 * Two kernel launches on `stream`; no workspace.  The tempered logits the report
 * anneals (tau from 0.8 to 0.4 over the steps) are the caller's schedule: tau is
 * per call.
 */
typedef struct {
  int32_t batch;        /* B, 1..DG_MAX_BATCH                                     */
  int32_t n_canvas;     /* Nc, must equal DG_N_CANVAS                             */
  int32_t vocab;        /* V                                                      */
  float tau;            /* temperature, > 0                                       */
  float budget;         /* cumulative entropy budget in nats, 0..1e6 (report: 0.1) */
  float stop_entropy;   /* mean-entropy threshold in nats, 0..1e6 (report: 0.005)  */
} dg_sample_shape;

dg_status dg_canvas_sample(const dg_sample_shape* shape, const void* logits,
                           const int32_t* noise_tokens, const int32_t* prev_argmax,
                           float* entropy, int32_t* argmax, int32_t* tokens,
                           int32_t* accepted, int32_t* stop, void* stream);

/*
 * Self-conditioning input ("DiffusionGemma Technical Report", paperfeed.app
 * summary, section "The mechanism: an AR model turned inside out",
 * self-conditioning paragraph): next to the noisy canvas the decoder receives
 * z = FFW(p0 E), the previous step's predicted token distribution p0 pushed
 * through the embedding matrix E and a small MLP.  Readings of what the page
 * leaves open: p0 = softmax(logits) at temperature 1 (the annealed temperature
 * belongs to the sampler); FFW(y) = gelu(y W1) W2 with no biases and GELU in its
 * tanh form.  For every sequence b and canvas position i:
 *   y[b,i,:] = sum_v softmax(logits[b,i,:])_v E[v,:]
 *   z[b,i,:] = gelu(y[b,i,:] W1) W2
 * Precision: p0, y and gelu(y W1) are rounded to bf16 before the product that
 * consumes them; products accumulate in fp32; z is bf16.
 *   logits     [B][Nc][V] bf16 device; finite or -inf (a row needs one finite value)
 *   embed      E [V][d] bf16 device
 *   w1         [d][h] bf16 device;  w2 [h][d] bf16 device
 *   z          [B][Nc][d] bf16 device (out)
 *   workspace  device scratch of ws_bytes >= dg_selfcond_workspace_bytes(shape)
 *              (the blocked softmax weights, split partials, y and the hidden
 *              activations); contents are overwritten
 * All pointers 16-byte aligned.  Seven kernel launches on `stream`.  With
 * dg_kernel_timing_enable, the embedding product is recorded in the attention
 * slot and the softmax pass in the merge slot.
 */
#define DG_SELFCOND_MAX_VOCAB 524288

typedef struct {
  int32_t batch;     /* B, 1..DG_MAX_BATCH                                        */
  int32_t n_canvas;  /* Nc, must equal DG_N_CANVAS                                */
  int32_t vocab;     /* V, a multiple of 32, 32..DG_SELFCOND_MAX_VOCAB            */
  int32_t d_model;   /* d, a multiple of 256, 256..16384                          */
  int32_t d_hidden;  /* h, the MLP's hidden width, a multiple of 128, 128..16384  */
} dg_selfcond_shape;

size_t dg_selfcond_workspace_bytes(const dg_selfcond_shape* shape);
dg_status dg_self_condition(const dg_selfcond_shape* shape, const void* logits, const void* embed,
                            const void* w1, const void* w2, void* z, void* workspace,
                            size_t ws_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* dg_status_string(dg_status status);

/* Thread-local description of the last failed call on this thread ("" if none). */
const char* dg_last_error(void);

/*
 * Kernel timing for measurement.  While enabled, every attention kernel the
 * library launches is bracketed by HIP events recorded on the launch stream.
 * dg_kernel_timing_read() waits for the recorded events, returns the number of
 * launches and the summed milliseconds of the split-key attention kernels
 * (attn_ms) and of the merge kernels (merge_ms) since the last read, and
 * clears the record.  At most 4096 launches are kept between reads; later ones
 * are not timed.  Not thread-safe; for benchmarks only.
 */
dg_status dg_kernel_timing_enable(int32_t enable);
dg_status dg_kernel_timing_read(int32_t* n_attn, double* attn_ms, int32_t* n_merge,
                                double* merge_ms);
/*
 * Like dg_kernel_timing_read, but returns the duration of every recorded launch
 * (milliseconds, in launch order) instead of sums: up to max_n attention kernels
 * into attn_ms and up to max_n merge kernels into merge_ms (host arrays owned by
 * the caller; either may be NULL to skip that kind).  *n_attn and *n_merge get
 * the numbers recorded, which may exceed max_n.  Clears the record.
 */
dg_status dg_kernel_timing_samples(float* attn_ms, float* merge_ms, int32_t max_n,
                                   int32_t* n_attn, int32_t* n_merge);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
