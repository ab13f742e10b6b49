"""Thin Python binding of libdg.so (the gfx950 canvas-attention library).

Argument marshalling only: every tensor is passed to the C ABI in
include/dg.h as ``data_ptr()`` plus the current HIP stream; all of the
arithmetic runs in the library's kernels.  torch provides device memory and
streams.  Importing this module raises if libdg.so has not been built -- there
is no CPU fallback.

Functions mirror the C entry points: ``canvas_attn``, ``commit_block``,
``canvas_step_loop``, ``canvas_sample``, ``workspace_bytes``,
``kernel_timing_enable`` and ``kernel_timing_read``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DG_LIBRARY selects another build of the same library (for example a variant
# compiled with different tuning flags); the default is the in-tree build.
LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(_HERE, "libdg.so")

DG_BF16, DG_F32, DG_FP8 = 0, 1, 2
N_CANVAS = 256
MAX_DECODE = 16
STATUS = {0: "DG_OK", -1: "DG_ERR_NULL", -2: "DG_ERR_SHAPE", -3: "DG_ERR_DTYPE",
          -4: "DG_ERR_CAPACITY", -5: "DG_ERR_WORKSPACE", -6: "DG_ERR_HIP", -7: "DG_ERR_ALIGN"}


class DgShape(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_canvas", ctypes.c_int32), ("n_heads_q", ctypes.c_int32),
                ("n_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("q_scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class DgSampleShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_canvas", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tau", ctypes.c_float), ("budget", ctypes.c_float),
                ("stop_entropy", ctypes.c_float)]


class DgSelfcondShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_canvas", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_hidden", ctypes.c_int32)]


class DgKv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int64)]


class DgError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {detail}")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m canvas_attention_amd.build` "
                      "(there is no CPU fallback for the GPU path)")

lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_P = ctypes.POINTER
lib.dg_workspace_bytes.argtypes = [_P(DgShape), _i64]
lib.dg_workspace_bytes.restype = _sz
lib.dg_canvas_attn.argtypes = [_P(DgShape), _vp, _P(DgKv), _vp, _P(DgKv), _vp, _vp, _sz, _vp]
lib.dg_canvas_attn.restype = _i32
lib.dg_canvas_attn_noalloc.argtypes = [_P(DgShape), _vp, _P(DgKv), _vp, _P(DgKv), _vp, _vp]
lib.dg_canvas_attn_noalloc.restype = _i32
lib.dg_commit_block.argtypes = [_P(DgShape), _vp, _P(DgKv), _P(DgKv), _vp, _vp, _vp, _sz, _vp]
lib.dg_commit_block.restype = _i32
lib.dg_canvas_step_loop.argtypes = [_P(DgShape), _i32, _vp, _i64, _P(DgKv), _i64, _P(DgKv), _vp,
                                    _vp, _i64, _vp, _sz, _vp]
lib.dg_canvas_step_loop.restype = _i32
lib.dg_decode_workspace_bytes.argtypes = [_P(DgShape), _i64]
lib.dg_decode_workspace_bytes.restype = _sz
lib.dg_decode_attn.argtypes = [_P(DgShape), _vp, _P(DgKv), _P(DgKv), _vp, _vp, _vp, _sz, _vp]
lib.dg_decode_attn.restype = _i32
lib.dg_selfcond_workspace_bytes.argtypes = [_P(DgSelfcondShape)]
lib.dg_selfcond_workspace_bytes.restype = _sz
lib.dg_self_condition.argtypes = [_P(DgSelfcondShape), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.dg_self_condition.restype = _i32
lib.dg_canvas_sample.argtypes = [_P(DgSampleShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
lib.dg_canvas_sample.restype = _i32
lib.dg_status_string.argtypes = [_i32]
lib.dg_status_string.restype = ctypes.c_char_p
lib.dg_last_error.argtypes = []
lib.dg_last_error.restype = ctypes.c_char_p
lib.dg_kernel_timing_enable.argtypes = [_i32]
lib.dg_kernel_timing_enable.restype = _i32
lib.dg_kernel_timing_read.argtypes = [_P(_i32), _P(ctypes.c_double), _P(_i32),
                                      _P(ctypes.c_double)]
lib.dg_kernel_timing_read.restype = _i32
lib.dg_kernel_timing_samples.argtypes = [_P(ctypes.c_float), _P(ctypes.c_float), _i32, _P(_i32),
                                         _P(_i32)]
lib.dg_kernel_timing_samples.restype = _i32

EXPORTS = ["dg_workspace_bytes", "dg_canvas_attn", "dg_canvas_attn_noalloc", "dg_commit_block",
           "dg_canvas_step_loop",
           "dg_canvas_sample", "dg_decode_workspace_bytes", "dg_decode_attn",
           "dg_selfcond_workspace_bytes", "dg_self_condition",
           "dg_status_string", "dg_last_error", "dg_kernel_timing_enable",
           "dg_kernel_timing_read", "dg_kernel_timing_samples"]


def _check(fn, status):
    if status != 0:
        raise DgError(fn, status, lib.dg_last_error().decode())


def _dtype_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return DG_BF16
    if dtype == torch.float32:
        return DG_F32
    if dtype == torch.float8_e4m3fn:
        return DG_FP8
    raise TypeError(f"unsupported dtype {dtype}; bfloat16, float32 or float8_e4m3fn")


def out_dtype(dtype):
    """Output element type for inputs of `dtype` (fp8 inputs give bf16 rows)."""
    return torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype


def _shape(q: torch.Tensor, hkv: int, scale, tensor_scales=None) -> DgShape:
    B, Nc, Hq, D = q.shape
    qs, ks, vs = tensor_scales if tensor_scales is not None else (0.0, 0.0, 0.0)
    return DgShape(_dtype_code(q.dtype), B, Nc, Hq, hkv, D, float(scale) if scale else 0.0,
                   float(qs), float(ks), float(vs))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t: torch.Tensor, name: str, dtype, dims: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != dims or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dims}-d tensor")


def _check_attn(q, k_cache, v_cache, k_new, v_new, out, names):
    """Shape agreement of one attention call's tensors.  The C ABI sees only
    pointers and the sizes in dg_shape / dg_kv, so a cache or K/V tensor with
    another batch, kv-head count or head_dim than those sizes would be read (and
    for the commit and decode, written) past its end: reject it here, before any
    launch.  q and out are [..., B, n, Hq, D]; the caches [B, cap, Hkv, D]; the
    new K/V [..., B, n, Hkv, D] with q's leading dimensions."""
    lead, (B, n, Hq, D) = tuple(q.shape[:-4]), tuple(q.shape[-4:])
    Hkv = k_cache.shape[2]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"{names[0]} has {Hq} heads, not a multiple of the cache's {Hkv}")
    if tuple(k_cache.shape) != tuple(v_cache.shape):
        raise ValueError(f"k_cache {tuple(k_cache.shape)} and v_cache {tuple(v_cache.shape)} differ")
    if k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"cache {tuple(k_cache.shape)} does not match {names[0]} "
                         f"{tuple(q.shape)}: expected [{B}, cap, Hkv, {D}]")
    want = lead + (B, n, Hkv, D)
    for name, t in ((names[1], k_new), (names[2], v_new)):
        if tuple(t.shape) != want:
            raise ValueError(f"{name} is {tuple(t.shape)}, expected {want}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out is {tuple(out.shape)}, expected {tuple(q.shape)}")
    dev = q.device
    for t in (k_cache, v_cache, k_new, v_new, out):
        if t.device != dev:
            raise ValueError(f"tensors on different devices ({t.device} and {dev})")


def _check_workspace(workspace, device):
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError(f"workspace must be a tensor on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _prefix(prefix_len, batch):
    if len(prefix_len) != batch:
        raise ValueError(f"prefix_len has {len(prefix_len)} entries, batch is {batch}")
    return (ctypes.c_int32 * batch)(*[int(x) for x in prefix_len])


def _check_like(items, device):
    """Each (name, tensor, dtype, shape) must be a contiguous tensor of exactly that
    type and shape on `device`: the kernels read and write these per position, with
    only the sizes in the call's shape struct to go by."""
    for name, t, dtype, shape in items:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name} is {tuple(t.shape)}, expected a contiguous {tuple(shape)}")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_sample(logits, noise_tokens, prev_argmax, out):
    """Sampler call: noise_tokens, prev_argmax (optional) and the five outputs
    (entropy, argmax, tokens, accepted, stop) against logits [B, n, V]."""
    B, Nc, _ = logits.shape
    if not isinstance(out, (tuple, list)) or len(out) != 5:
        raise ValueError("out must hold five tensors: entropy, argmax, tokens, accepted, stop")
    items = [("noise_tokens", noise_tokens, torch.int32, (B, Nc))]
    if prev_argmax is not None:
        items.append(("prev_argmax", prev_argmax, torch.int32, (B, Nc)))
    names = ("entropy", "argmax", "tokens", "accepted", "stop")
    types = (torch.float32, torch.int32, torch.int32, torch.int32, torch.int32)
    shapes = ((B, Nc), (B, Nc), (B, Nc), (B, Nc), (B,))
    items += list(zip(names, out, types, shapes))
    _check_like(items, logits.device)


def _check_selfcond(logits, embed, w1, w2, out):
    """Self-conditioning call: E [V, d], W1 [d, h], W2 [h, d] and z [B, n, d]
    against logits [B, n, V], all bf16 on the logits' device."""
    B, nc, V = logits.shape
    if not isinstance(w1, torch.Tensor) or w1.dim() != 2:
        raise ValueError("w1 must be a 2-d tensor")
    d, h = w1.shape
    bf = torch.bfloat16
    _check_like([("embed", embed, bf, (V, d)), ("w1", w1, bf, (d, h)), ("w2", w2, bf, (h, d)),
                 ("out", out, bf, (B, nc, d))], logits.device)


def workspace_bytes(batch, n_heads_q, n_heads_kv, head_dim, max_prefix_len,
                    dtype=torch.bfloat16) -> int:
    """Bytes of workspace any call of this shape needs (see dg_workspace_bytes)."""
    shape = DgShape(_dtype_code(dtype), batch, N_CANVAS, n_heads_q, n_heads_kv, head_dim, 0.0)
    return int(lib.dg_workspace_bytes(ctypes.byref(shape), int(max_prefix_len)))


def alloc_workspace(q: torch.Tensor, n_heads_kv: int, max_prefix_len: int) -> torch.Tensor:
    B, _, Hq, D = q.shape
    n = workspace_bytes(B, Hq, n_heads_kv, D, max_prefix_len, q.dtype)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def canvas_attn(q, k_cache, v_cache, prefix_len, k_canvas, v_canvas, out=None, workspace=None,
                scale=None, stream=None, tensor_scales=None):
    """dg_canvas_attn: q [B,256,Hq,D]; caches [B,cap,Hkv,D]; canvas K/V [B,256,Hkv,D].
    float8_e4m3fn inputs take tensor_scales = (q_scale, k_scale, v_scale) and give
    a bfloat16 output."""
    dt = q.dtype
    _need(q, "q", dt, 4)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_canvas", k_canvas),
                    ("v_canvas", v_canvas)):
        _need(t, name, dt, 4)
    hkv = k_cache.shape[2]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype(dt), device=q.device)
    _need(out, "out", out_dtype(dt), 4)
    _check_attn(q, k_cache, v_cache, k_canvas, v_canvas, out, ("q", "k_canvas", "v_canvas"))
    if workspace is None:
        workspace = alloc_workspace(q, hkv, max(int(x) for x in prefix_len))
    _check_workspace(workspace, q.device)
    shape = _shape(q, hkv, scale, tensor_scales)
    cache = DgKv(k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[1])
    canv = DgKv(k_canvas.data_ptr(), v_canvas.data_ptr(), k_canvas.shape[1])
    st = lib.dg_canvas_attn(ctypes.byref(shape), _ptr(q), ctypes.byref(cache),
                            _prefix(prefix_len, q.shape[0]), ctypes.byref(canv), _ptr(out),
                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream))
    _check("dg_canvas_attn", st)
    return out


def canvas_attn_noalloc(q, k_cache, v_cache, prefix_len, k_canvas, v_canvas, out, scale=None,
                        stream=None, tensor_scales=None):
    """dg_canvas_attn_noalloc: dg_canvas_attn with its partial results in the
    library's per-GPU scratch array instead of a workspace; the caller passes
    `out`, so nothing is allocated on this path."""
    dt = q.dtype
    _need(q, "q", dt, 4)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_canvas", k_canvas),
                    ("v_canvas", v_canvas)):
        _need(t, name, dt, 4)
    _need(out, "out", out_dtype(dt), 4)
    _check_attn(q, k_cache, v_cache, k_canvas, v_canvas, out, ("q", "k_canvas", "v_canvas"))
    shape = _shape(q, k_cache.shape[2], scale, tensor_scales)
    cache = DgKv(k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[1])
    canv = DgKv(k_canvas.data_ptr(), v_canvas.data_ptr(), k_canvas.shape[1])
    st = lib.dg_canvas_attn_noalloc(ctypes.byref(shape), _ptr(q), ctypes.byref(cache),
                                    _prefix(prefix_len, q.shape[0]), ctypes.byref(canv), _ptr(out),
                                    _stream(stream))
    _check("dg_canvas_attn_noalloc", st)
    return out


def commit_block(q_blk, k_blk, v_blk, k_cache, v_cache, prefix_len, out=None, workspace=None,
                 scale=None, stream=None, tensor_scales=None):
    """dg_commit_block: causal block attention, then block K/V appended to the cache."""
    dt = q_blk.dtype
    _need(q_blk, "q_blk", dt, 4)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_blk", k_blk),
                    ("v_blk", v_blk)):
        _need(t, name, dt, 4)
    hkv = k_cache.shape[2]
    if out is None:
        out = torch.empty(q_blk.shape, dtype=out_dtype(dt), device=q_blk.device)
    _need(out, "out", out_dtype(dt), 4)
    _check_attn(q_blk, k_cache, v_cache, k_blk, v_blk, out, ("q_blk", "k_blk", "v_blk"))
    if workspace is None:
        workspace = alloc_workspace(q_blk, hkv, max(int(x) for x in prefix_len))
    _check_workspace(workspace, q_blk.device)
    shape = _shape(q_blk, hkv, scale, tensor_scales)
    blk = DgKv(k_blk.data_ptr(), v_blk.data_ptr(), k_blk.shape[1])
    cache = DgKv(k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[1])
    st = lib.dg_commit_block(ctypes.byref(shape), _ptr(q_blk), ctypes.byref(blk),
                             ctypes.byref(cache), _prefix(prefix_len, q_blk.shape[0]),
                             _ptr(out), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dg_commit_block", st)
    return out



def decode_workspace_bytes(batch, n_new, n_heads_q, n_heads_kv, head_dim, max_prefix_len,
                           dtype=torch.bfloat16) -> int:
    """Bytes of workspace any decode call of this shape needs (dg_decode_workspace_bytes)."""
    shape = DgShape(_dtype_code(dtype), batch, n_new, n_heads_q, n_heads_kv, head_dim, 0.0)
    return int(lib.dg_decode_workspace_bytes(ctypes.byref(shape), int(max_prefix_len)))


def decode_attn(q, k_new, v_new, k_cache, v_cache, prefix_len, out=None, workspace=None,
                scale=None, stream=None, tensor_scales=None):
    """dg_decode_attn: k = q.shape[1] new tokens per sequence (1..16) attend causally
    to the cache and to each other; their K/V are appended to the cache."""
    dt = q.dtype
    _need(q, "q", dt, 4)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new),
                    ("v_new", v_new)):
        _need(t, name, dt, 4)
    B, k, Hq, D = q.shape
    hkv = k_cache.shape[2]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype(dt), device=q.device)
    _need(out, "out", out_dtype(dt), 4)
    _check_attn(q, k_cache, v_cache, k_new, v_new, out, ("q", "k_new", "v_new"))
    if workspace is None:
        n = decode_workspace_bytes(B, k, Hq, hkv, D, max(int(x) for x in prefix_len), dt)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    shape = _shape(q, hkv, scale, tensor_scales)
    new = DgKv(k_new.data_ptr(), v_new.data_ptr(), k_new.shape[1])
    cache = DgKv(k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[1])
    st = lib.dg_decode_attn(ctypes.byref(shape), _ptr(q), ctypes.byref(new), ctypes.byref(cache),
                            _prefix(prefix_len, B), _ptr(out), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dg_decode_attn", st)
    return out

def canvas_step_loop(q_steps, k_steps, v_steps, k_cache, v_cache, prefix_len, out=None,
                     workspace=None, scale=None, stream=None, tensor_scales=None):
    """dg_canvas_step_loop over N steps: q_steps [N,B,256,Hq,D], k/v_steps [N,B,256,Hkv,D]."""
    dt = q_steps.dtype
    _need(q_steps, "q_steps", dt, 5)
    _need(k_steps, "k_steps", dt, 5)
    _need(v_steps, "v_steps", dt, 5)
    _need(k_cache, "k_cache", dt, 4)
    _need(v_cache, "v_cache", dt, 4)
    n = q_steps.shape[0]
    hkv = k_cache.shape[2]
    if out is None:
        out = torch.empty(q_steps.shape, dtype=out_dtype(dt), device=q_steps.device)
    _need(out, "out", out_dtype(dt), 5)
    _check_attn(q_steps, k_cache, v_cache, k_steps, v_steps, out, ("q_steps", "k_steps", "v_steps"))
    if n == 0:
        return out
    q0 = q_steps[0]
    if workspace is None:
        workspace = alloc_workspace(q0, hkv, max(int(x) for x in prefix_len))
    _check_workspace(workspace, q0.device)
    shape = _shape(q0, hkv, scale, tensor_scales)
    canv = DgKv(k_steps.data_ptr(), v_steps.data_ptr(), k_steps.shape[2])
    cache = DgKv(k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[1])
    st = lib.dg_canvas_step_loop(ctypes.byref(shape), n, _ptr(q_steps), q_steps[0].numel(),
                                 ctypes.byref(canv), k_steps[0].numel(), ctypes.byref(cache),
                                 _prefix(prefix_len, q0.shape[0]), _ptr(out), out[0].numel(),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    _check("dg_canvas_step_loop", st)
    return out


def canvas_sample(logits, noise_tokens, prev_argmax=None, tau=0.8, budget=0.1,
                  stop_entropy=0.005, out=None, stream=None):
    """dg_canvas_sample: logits [B,256,V] bf16, noise_tokens and prev_argmax [B,256]
    int32 (prev_argmax may be None).  Returns (entropy float32 [B,256], argmax,
    tokens, accepted int32 [B,256], stop int32 [B]); `out` may supply those five
    tensors."""
    _need(logits, "logits", torch.bfloat16, 3)
    B, Nc, V = logits.shape
    if out is None:
        dev = logits.device
        out = (torch.empty(B, Nc, dtype=torch.float32, device=dev),
               torch.empty(B, Nc, dtype=torch.int32, device=dev),
               torch.empty(B, Nc, dtype=torch.int32, device=dev),
               torch.empty(B, Nc, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    _check_sample(logits, noise_tokens, prev_argmax, out)
    entropy, argmax, tokens, accepted, stop = out
    shape = DgSampleShape(B, Nc, V, float(tau), float(budget), float(stop_entropy))
    st = lib.dg_canvas_sample(ctypes.byref(shape), _ptr(logits), _ptr(noise_tokens),
                              _ptr(prev_argmax), _ptr(entropy), _ptr(argmax), _ptr(tokens),
                              _ptr(accepted), _ptr(stop), _stream(stream))
    _check("dg_canvas_sample", st)
    return entropy, argmax, tokens, accepted, stop



def selfcond_workspace_bytes(batch, vocab, d_model, d_hidden) -> int:
    """Bytes of workspace a self-conditioning call of this shape needs."""
    shape = DgSelfcondShape(batch, N_CANVAS, vocab, d_model, d_hidden)
    return int(lib.dg_selfcond_workspace_bytes(ctypes.byref(shape)))


def self_condition(logits, embed, w1, w2, out=None, workspace=None, stream=None):
    """dg_self_condition: z = gelu(softmax(logits) E W1) W2 for bf16 logits
    [B, 256, V], E [V, d], W1 [d, h], W2 [h, d]; returns z [B, 256, d] bf16."""
    _need(logits, "logits", torch.bfloat16, 3)
    _need(w1, "w1", torch.bfloat16, 2)
    B, nc, V = logits.shape
    d, h = w1.shape
    if out is None:
        out = torch.empty((B, nc, d), dtype=torch.bfloat16, device=logits.device)
    _check_selfcond(logits, embed, w1, w2, out)
    shape = DgSelfcondShape(B, nc, V, d, h)
    if workspace is None:
        n = int(lib.dg_selfcond_workspace_bytes(ctypes.byref(shape)))
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=logits.device)
    _check_workspace(workspace, logits.device)
    st = lib.dg_self_condition(ctypes.byref(shape), _ptr(logits), _ptr(embed), _ptr(w1), _ptr(w2),
                               _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dg_self_condition", st)
    return out

def kernel_timing_enable(on: bool = True):
    _check("dg_kernel_timing_enable", lib.dg_kernel_timing_enable(1 if on else 0))


def kernel_timing_samples(max_n: int = 4096):
    """(attn_ms list, merge_ms list): per-launch durations since the previous read."""
    a = (ctypes.c_float * max_n)()
    m = (ctypes.c_float * max_n)()
    na, nm = ctypes.c_int32(), ctypes.c_int32()
    _check("dg_kernel_timing_samples",
           lib.dg_kernel_timing_samples(a, m, max_n, ctypes.byref(na), ctypes.byref(nm)))
    return list(a[:min(na.value, max_n)]), list(m[:min(nm.value, max_n)])


def kernel_timing_read():
    """(n_attn, attn_ms, n_merge, merge_ms) since the previous read."""
    na, nm = ctypes.c_int32(), ctypes.c_int32()
    ta, tm = ctypes.c_double(), ctypes.c_double()
    _check("dg_kernel_timing_read", lib.dg_kernel_timing_read(ctypes.byref(na), ctypes.byref(ta),
                                                              ctypes.byref(nm), ctypes.byref(tm)))
    return na.value, ta.value, nm.value, tm.value
