"""CPU fp64 oracle for canvas denoising attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
shares no code with the GPU library.

The arithmetic lives in ``dg_oracle.c`` (plain C, fp64, OpenMP over output
rows); this module only builds it with gcc and marshals numpy arrays through
ctypes.  What it computes follows "DiffusionGemma Technical Report"
(paperfeed.app summary), section "The mechanism: an AR model turned inside
out": the canvas is refined with full bidirectional attention within itself
while cross-attending to the causal KV cache, and a finished canvas is frozen,
encoded causally and appended to the cache.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dg_oracle.c")
_LIB = os.path.join(_HERE, "libdg_oracle.so")

BF16, F32, F64, FP8 = 0, 1, 2, 3
# bf16 and e4m3 travel as their bit patterns (uint16, uint8)
_DTYPE_OF = {np.dtype(np.uint16): BF16, np.dtype(np.float32): F32, np.dtype(np.float64): F64,
             np.dtype(np.uint8): FP8}

_lib = None


def build(force: bool = True) -> str:
    """Compile dg_oracle.c into libdg_oracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        attn_args = [i32, i32, i32, i32, i32, i32, dbl, vp, vp, vp, i64, vp, vp, vp, i32, vp, vp,
                     dbl, dbl, dbl]
        for name in ("dgo_canvas_attn", "dgo_commit_attn"):
            fn = getattr(lib, name)
            fn.argtypes = attn_args
            fn.restype = i32
        lib.dgo_append_block.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i64, vp]
        lib.dgo_append_block.restype = i32
        lib.dgo_partial.argtypes = [i32, i32, i32, dbl, vp, vp, vp, vp, vp, vp]
        lib.dgo_partial.restype = i32
        lib.dgo_merge.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        lib.dgo_merge.restype = i32
        lib.dgo_num_threads.argtypes = []
        lib.dgo_num_threads.restype = i32
        lib.dgo_set_num_threads.argtypes = [i32]
        lib.dgo_set_num_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype(*arrays) -> int:
    dts = {a.dtype for a in arrays}
    if len(dts) != 1:
        raise TypeError(f"mixed element types: {dts}")
    dt = dts.pop()
    if dt not in _DTYPE_OF:
        raise TypeError(f"unsupported element type {dt} (bf16 bits as uint16, e4m3 bits as "
                        "uint8, float32, float64)")
    return _DTYPE_OF[dt]


def _attn(fn_name, q, k_cache, v_cache, prefix_len, k_new, v_new, scale, rows, tensor_scales):
    lib = _load()
    arrays = [np.ascontiguousarray(x) for x in (q, k_cache, v_cache, k_new, v_new)]
    q, k_cache, v_cache, k_new, v_new = arrays
    dt = _dtype(*arrays)
    B, Nc, Hq, D = q.shape
    _, cap, Hkv, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pl = np.ascontiguousarray(np.asarray(prefix_len, dtype=np.int32).reshape(B))
    if rows is None:
        out = np.empty((B, Nc, Hq, D), np.float64)
        rows_arr, n_rows = None, 0
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        n_rows = rows_arr.shape[0]
        out = np.empty((n_rows, D), np.float64)
    qs, ks, vs = (1.0, 1.0, 1.0) if tensor_scales is None else (float(x) for x in tensor_scales)
    rc = getattr(lib, fn_name)(dt, B, Nc, Hq, Hkv, D, float(scale), _ptr(q), _ptr(k_cache),
                               _ptr(v_cache), cap, _ptr(pl), _ptr(k_new), _ptr(v_new), n_rows,
                               _ptr(rows_arr) if rows_arr is not None else None, _ptr(out),
                               qs, ks, vs)
    if rc != 0:
        raise ValueError(f"{fn_name} rejected its arguments (code {rc})")
    return out


def num_threads() -> int:
    """OpenMP threads the oracle's row loops run on."""
    return int(_load().dgo_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls in this process (OpenMP, n >= 1)."""
    _load().dgo_set_num_threads(int(n))


def canvas_attn(q, k_cache, v_cache, prefix_len, k_canvas, v_canvas, scale=None, rows=None,
                tensor_scales=None):
    """Canvas step: every canvas row attends, unmasked, to cache rows 0..L-1 and
    canvas rows 0..Nc-1.  Returns fp64 [B,Nc,Hq,D], or [len(rows),D] for a list
    of (b, i, h) rows.  tensor_scales = (q, k, v) multiplies the stored values
    (for e4m3 inputs; default 1)."""
    return _attn("dgo_canvas_attn", q, k_cache, v_cache, prefix_len, k_canvas, v_canvas,
                 scale, rows, tensor_scales)


def commit_attn(q_blk, k_cache, v_cache, prefix_len, k_blk, v_blk, scale=None, rows=None,
                tensor_scales=None):
    """Commit attention: block row i attends to cache rows 0..L-1 and block rows
    0..i (causal).  Same output convention as canvas_attn."""
    return _attn("dgo_commit_attn", q_blk, k_cache, v_cache, prefix_len, k_blk, v_blk,
                 scale, rows, tensor_scales)



def decode_attn(q, k_cache, v_cache, prefix_len, k_new, v_new, scale=None, rows=None,
                tensor_scales=None):
    """AR-mode decode of k new tokens per sequence ("DiffusionGemma Technical
    Report", paperfeed.app summary, section "The numbers, honestly": the same
    weights decode causally over the same cache; several drafted tokens at once
    for hybrid decoding): new token i attends to cache rows 0..L-1 and new rows
    0..i.  That is the commit's causal rule with k rows in place of 256, so this
    runs the same fp64 definition with Nc = k = q.shape[1].  The cache append
    that follows is append_block with the k new rows."""
    return _attn("dgo_commit_attn", q, k_cache, v_cache, prefix_len, k_new, v_new,
                 scale, rows, tensor_scales)

def append_block(k_blk, v_blk, k_cache, v_cache, prefix_len):
    """Copy block K/V rows into cache rows L_b..L_b+Nc-1 in place (bitwise)."""
    lib = _load()
    for a in (k_cache, v_cache):
        if not a.flags.c_contiguous:
            raise ValueError("cache arrays must be C-contiguous")
    k_blk = np.ascontiguousarray(k_blk)
    v_blk = np.ascontiguousarray(v_blk)
    dt = _dtype(k_blk, v_blk, k_cache, v_cache)
    B, Nc, Hkv, D = k_blk.shape
    cap = k_cache.shape[1]
    pl = np.ascontiguousarray(np.asarray(prefix_len, dtype=np.int32).reshape(B))
    rc = lib.dgo_append_block(dt, B, Nc, Hkv, D, _ptr(k_blk), _ptr(v_blk), _ptr(k_cache),
                              _ptr(v_cache), cap, _ptr(pl))
    if rc != 0:
        raise ValueError(f"dgo_append_block rejected its arguments (code {rc})")


def partial(q, k, v, scale):
    """(m, l, o) of fp64 query rows q [n_q,D] over keys k, v [n_k,D]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64).reshape(-1, q.shape[1])
    v = np.ascontiguousarray(v, dtype=np.float64).reshape(-1, q.shape[1])
    n_q, D = q.shape
    m = np.empty(n_q)
    l_ = np.empty(n_q)
    o = np.empty((n_q, D))
    lib.dgo_partial(n_q, k.shape[0], D, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(m),
                    _ptr(l_), _ptr(o))
    return m, l_, o


def merge(ms, ls, os_):
    """Normalised output from stacked partials m, l [S,n_q] and o [S,n_q,D]."""
    lib = _load()
    ms = np.ascontiguousarray(ms, dtype=np.float64)
    ls = np.ascontiguousarray(ls, dtype=np.float64)
    os_ = np.ascontiguousarray(os_, dtype=np.float64)
    S, n_q, D = os_.shape
    out = np.empty((n_q, D))
    lib.dgo_merge(S, n_q, D, _ptr(ms), _ptr(ls), _ptr(os_), _ptr(out))
    return out
