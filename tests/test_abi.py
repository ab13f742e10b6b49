"""CPU-only checks of the C ABI: the library loads, exports every entry point
declared in include/dg.h, and rejects bad arguments on the host before any HIP
call (fake device pointers are never dereferenced on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


@pytest.fixture(scope="module")
def dg():
    from canvas_attention_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    import canvas_attention_amd.dg as dg_mod
    return dg_mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("dg_canvas_attn", "dg_commit_block", "dg_canvas_step_loop", "dg_workspace_bytes",
              "dg_decode_attn", "dg_decode_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(dg):
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(dg.lib, n), f"libdg.so does not export {n}"
    assert set(dg.EXPORTS) == set(names)


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced by the rejected calls


def shape(dg, **kw):
    d = dict(dtype=0, batch=1, n_canvas=256, n_heads_q=16, n_heads_kv=8, head_dim=128, scale=0.0)
    d.update(kw)
    return dg.DgShape(**d)


def call_canvas(dg, sh, q=FAKE, cache=None, prefix=(0,), canvas=None, out=FAKE, ws=FAKE,
                ws_bytes=1 << 40):
    cache = cache or dg.DgKv(FAKE, FAKE, 4096)
    canvas = canvas or dg.DgKv(FAKE, FAKE, 256)
    pl = (ctypes.c_int32 * len(prefix))(*prefix)
    return dg.lib.dg_canvas_attn(ctypes.byref(sh), q, ctypes.byref(cache), pl,
                                 ctypes.byref(canvas), out, ws, ws_bytes, None)


def call_commit(dg, sh, cache=None, prefix=(0,), ws_bytes=1 << 40):
    cache = cache or dg.DgKv(FAKE, FAKE, 4096)
    blk = dg.DgKv(FAKE, FAKE, 256)
    pl = (ctypes.c_int32 * len(prefix))(*prefix)
    return dg.lib.dg_commit_block(ctypes.byref(sh), FAKE, ctypes.byref(blk), ctypes.byref(cache),
                                  pl, FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -3),
    (dict(batch=0), -2),
    (dict(batch=65), -2),
    (dict(n_canvas=128), -2),
    (dict(n_heads_q=12, n_heads_kv=8), -2),
    (dict(head_dim=96), -2),
    (dict(n_heads_kv=0), -2),
    (dict(scale=float("nan")), -2),
    (dict(dtype=2, head_dim=64), -2),
    (dict(dtype=2, q_scale=float("inf")), -2),
    (dict(dtype=2, v_scale=float("nan")), -2),
])
def test_shape_errors(dg, kw, code):
    st = call_canvas(dg, shape(dg, **kw), prefix=(0,) * max(1, kw.get("batch", 1) or 1))
    assert st == code, (st, dg.lib.dg_last_error())
    assert dg.lib.dg_last_error().decode()


def test_null_and_alignment_errors(dg):
    sh = shape(dg)
    assert call_canvas(dg, sh, q=None) == -1
    assert call_canvas(dg, sh, out=None) == -1
    assert call_canvas(dg, sh, canvas=dg.DgKv(None, FAKE, 256)) == -1
    assert call_canvas(dg, sh, cache=dg.DgKv(None, FAKE, 64)) == -1
    assert call_canvas(dg, sh, q=FAKE + 8) == -7
    assert call_canvas(dg, sh, cache=dg.DgKv(FAKE + 2, FAKE, 64)) == -7


def test_capacity_errors(dg):
    sh = shape(dg)
    assert call_canvas(dg, sh, prefix=(-1,)) == -4
    assert call_canvas(dg, sh, cache=dg.DgKv(FAKE, FAKE, 100), prefix=(101,)) == -4
    assert call_canvas(dg, sh, canvas=dg.DgKv(FAKE, FAKE, 255)) == -2
    # commit needs room for the whole block behind the prefix
    assert call_commit(dg, sh, cache=dg.DgKv(FAKE, FAKE, 300), prefix=(45,)) == -4
    assert "exceeds cache capacity" in dg.lib.dg_last_error().decode()
    # a commit may never run on a cache without storage
    assert call_commit(dg, sh, cache=dg.DgKv(None, None, 0), prefix=(0,)) in (-1, -4)


def test_workspace_too_small(dg):
    sh = shape(dg)
    st = call_canvas(dg, sh, prefix=(4000,), ws_bytes=1024)
    assert st == -5
    assert "workspace" in dg.lib.dg_last_error().decode()


def test_step_loop_errors(dg):
    sh = shape(dg)
    cache = dg.DgKv(FAKE, FAKE, 4096)
    canv = dg.DgKv(FAKE, FAKE, 256)
    pl = (ctypes.c_int32 * 1)(0)
    st = dg.lib.dg_canvas_step_loop(ctypes.byref(sh), -1, FAKE, 0, ctypes.byref(canv), 0,
                                    ctypes.byref(cache), pl, FAKE, 0, FAKE, 1 << 40, None)
    assert st == -2
    st = dg.lib.dg_canvas_step_loop(ctypes.byref(sh), 2, FAKE, 3, ctypes.byref(canv), 0,
                                    ctypes.byref(cache), pl, FAKE, 0, FAKE, 1 << 40, None)
    assert st == -7
    for strides in ((-8, 0, 0), (0, -8, 0), (0, 0, -8)):
        st = dg.lib.dg_canvas_step_loop(ctypes.byref(sh), 2, FAKE, strides[0], ctypes.byref(canv),
                                        strides[1], ctypes.byref(cache), pl, FAKE, strides[2],
                                        FAKE, 1 << 40, None)
        assert st == -2 and b"stride" in dg.lib.dg_last_error()


def test_fp8_step_strides(dg):
    # fp8 steps q and K/V in 1-byte elements and out in 2-byte (bf16) elements
    sh = shape(dg, dtype=2)
    cache = dg.DgKv(FAKE, FAKE, 4096)
    canv = dg.DgKv(FAKE, FAKE, 256)
    pl = (ctypes.c_int32 * 1)(0)
    for qs, kvs, os_ in ((8, 16, 8), (16, 24, 8), (16, 16, 4)):
        st = dg.lib.dg_canvas_step_loop(ctypes.byref(sh), 2, FAKE, qs, ctypes.byref(canv), kvs,
                                        ctypes.byref(cache), pl, FAKE, os_, FAKE, 1 << 40, None)
        assert st == -7, (qs, kvs, os_, st)


def test_workspace_bytes(dg):
    assert dg.lib.dg_workspace_bytes(ctypes.byref(shape(dg, head_dim=96)), 1000) == 0
    assert dg.lib.dg_workspace_bytes(ctypes.byref(shape(dg)), -1) == 0
    n = dg.lib.dg_workspace_bytes(ctypes.byref(shape(dg)), 8192)
    assert n > 0 and n % 4 == 0
    n32 = dg.lib.dg_workspace_bytes(ctypes.byref(shape(dg, dtype=1, head_dim=64)), 64)
    assert n32 > 0
    # fp8 partial rows are bf16, as for the bf16 path
    n8 = dg.lib.dg_workspace_bytes(ctypes.byref(shape(dg, dtype=2)), 8192)
    assert n8 == n
    assert dg.lib.dg_workspace_bytes(ctypes.byref(shape(dg, dtype=2, head_dim=64)), 64) == 0


def test_status_strings(dg):
    for code, name in dg.STATUS.items():
        assert dg.lib.dg_status_string(code).decode() == name
    assert dg.lib.dg_status_string(-99).decode() == "DG_ERR_UNKNOWN"


def sample_shape(dg, **kw):
    d = dict(batch=1, n_canvas=256, vocab=262144, tau=0.8, budget=0.1, stop_entropy=0.005)
    d.update(kw)
    return dg.DgSampleShape(**d)


def call_sample(dg, sh, logits=FAKE, noise=FAKE, prev=None, outs=(FAKE, FAKE, FAKE, FAKE, FAKE)):
    return dg.lib.dg_canvas_sample(ctypes.byref(sh), logits, noise, prev, *outs, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -2), (dict(batch=65), -2), (dict(n_canvas=255), -2),
    (dict(vocab=4), -2), (dict(vocab=1001), -2), (dict(vocab=(1 << 27) + 8), -2),
    (dict(tau=0.0), -2), (dict(tau=float("inf")), -2), (dict(tau=float("nan")), -2),
    (dict(budget=-0.1), -2), (dict(budget=float("nan")), -2), (dict(stop_entropy=-1.0), -2),
])
def test_sample_shape_errors(dg, kw, code):
    assert call_sample(dg, sample_shape(dg, **kw)) == code, dg.lib.dg_last_error()


def test_sample_null_and_alignment(dg):
    sh = sample_shape(dg)
    assert call_sample(dg, sh, logits=None) == -1
    assert call_sample(dg, sh, noise=None) == -1
    assert call_sample(dg, sh, outs=(FAKE, None, FAKE, FAKE, FAKE)) == -1
    assert call_sample(dg, sh, logits=FAKE + 8) == -7
    assert call_sample(dg, sh, prev=FAKE + 2) == -7


def call_decode(dg, sh, q=FAKE, new=None, cache=None, prefix=(0,), out=FAKE, ws=FAKE,
                ws_bytes=1 << 40):
    new = new or dg.DgKv(FAKE, FAKE, sh.n_canvas)
    cache = cache or dg.DgKv(FAKE, FAKE, 4096)
    pl = (ctypes.c_int32 * len(prefix))(*prefix)
    return dg.lib.dg_decode_attn(ctypes.byref(sh), q, ctypes.byref(new), ctypes.byref(cache), pl,
                                 out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_canvas=0), -2), (dict(n_canvas=17), -2), (dict(n_canvas=256), -2),
    (dict(dtype=7, n_canvas=1), -3), (dict(n_canvas=4, head_dim=96), -2),
    (dict(n_canvas=4, n_heads_q=12), -2), (dict(n_canvas=4, dtype=2, head_dim=64), -2),
    (dict(n_canvas=2, batch=65), -2),
])
def test_decode_shape_errors(dg, kw, code):
    assert call_decode(dg, shape(dg, **kw)) == code


def test_decode_argument_errors(dg):
    sh = shape(dg, n_canvas=4)
    assert call_decode(dg, sh, q=None) == -1
    assert call_decode(dg, sh, new=dg.DgKv(FAKE, None, 4)) == -1
    assert call_decode(dg, sh, q=FAKE + 4) == -7
    # the new K/V hold exactly the k new rows
    assert call_decode(dg, sh, new=dg.DgKv(FAKE, FAKE, 256)) == -2
    # the cache needs room for the new rows behind the prefix
    assert call_decode(dg, sh, cache=dg.DgKv(FAKE, FAKE, 100), prefix=(97,)) == -4
    assert "new tokens" in dg.lib.dg_last_error().decode()
    assert call_decode(dg, sh, prefix=(-3,)) == -4
    st = call_decode(dg, sh, prefix=(4000,), ws_bytes=64)
    assert st == -5 and "workspace" in dg.lib.dg_last_error().decode()


def test_decode_workspace_bytes(dg):
    f = dg.lib.dg_decode_workspace_bytes
    assert f(ctypes.byref(shape(dg, n_canvas=0)), 100) == 0
    assert f(ctypes.byref(shape(dg, n_canvas=1)), -1) == 0
    n1 = f(ctypes.byref(shape(dg, n_canvas=1)), 8192)
    n16 = f(ctypes.byref(shape(dg, n_canvas=16)), 8192)
    # 32 packed rows per tile: Hq/Hkv = 2 heads per kv head gives one tile up to 16 tokens
    assert n1 > 0 and n1 == n16
    n_g8 = f(ctypes.byref(shape(dg, n_canvas=16, n_heads_q=32, n_heads_kv=4)), 8192)
    assert n_g8 > n16
    assert f(ctypes.byref(shape(dg, n_canvas=3, dtype=1, head_dim=64)), 64) > 0


def sc_shape(dg, **kw):
    d = dict(batch=1, n_canvas=256, vocab=262144, d_model=2048, d_hidden=1920)
    d.update(kw)
    return dg.DgSelfcondShape(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -2), (dict(n_canvas=255), -2), (dict(vocab=100), -2), (dict(vocab=16), -2),
    (dict(vocab=524288 + 32), -2), (dict(d_model=200), -2), (dict(d_model=384), -2),
    (dict(d_hidden=0), -2), (dict(d_hidden=200), -2),
])
def test_selfcond_shape_errors(dg, kw, code):
    sh = sc_shape(dg, **kw)
    assert dg.lib.dg_selfcond_workspace_bytes(ctypes.byref(sh)) == 0
    st = dg.lib.dg_self_condition(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code


def test_selfcond_argument_errors(dg):
    sh = sc_shape(dg)
    n = dg.lib.dg_selfcond_workspace_bytes(ctypes.byref(sh))
    # the blocked softmax weights alone are 256 x 262144 bf16
    assert n >= 256 * 262144 * 2
    f = dg.lib.dg_self_condition
    assert f(ctypes.byref(sh), None, FAKE, FAKE, FAKE, FAKE, FAKE, n, None) == -1
    assert f(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, n, None) == -7
    assert f(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n - 1, None) == -5


# ---------------------------------------------------------------- binding checks
# The C ABI sees only pointers and the sizes in dg_shape / dg_kv, so the binding
# must reject tensors whose shapes disagree before anything is launched: a cache
# with another batch, kv-head count or head_dim would be read past its end (and
# written, for the commit and decode).  _check_attn inspects shapes and devices
# only, so CPU tensors exercise it here.

def _attn_tensors(torch, B=2, n=256, Hq=16, Hkv=8, D=128, cap=300, lead=()):
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)  # noqa: E731
    return dict(q=z(*lead, B, n, Hq, D), kc=z(B, cap, Hkv, D), vc=z(B, cap, Hkv, D),
                kn=z(*lead, B, n, Hkv, D), vn=z(*lead, B, n, Hkv, D), out=z(*lead, B, n, Hq, D))


def _check(dg, t, names=("q", "k_canvas", "v_canvas")):
    dg._check_attn(t["q"], t["kc"], t["vc"], t["kn"], t["vn"], t["out"], names)


def test_binding_accepts_matching_shapes(dg):
    torch = pytest.importorskip("torch")
    _check(dg, _attn_tensors(torch))
    _check(dg, _attn_tensors(torch, lead=(3,)), ("q_steps", "k_steps", "v_steps"))
    _check(dg, _attn_tensors(torch, n=4, Hq=4, Hkv=2, D=64), ("q", "k_new", "v_new"))


@pytest.mark.parametrize("keys,shape,msg", [
    (("kc", "vc"), (1, 300, 8, 128), "does not match"),  # caches of a smaller batch than q's
    (("kc", "vc"), (2, 300, 8, 64), "does not match"),   # caches of another head_dim
    (("vc",), (2, 300, 4, 128), "differ"),               # V cache with other kv heads
    (("kc",), (2, 300, 8, 64), "differ"),                # K cache with another head_dim
    (("kn",), (2, 256, 4, 128), "expected"),             # canvas K with other kv heads
    (("vn",), (1, 256, 8, 128), "expected"),             # canvas V with another batch
    (("kn",), (2, 128, 8, 128), "expected"),             # canvas K with fewer rows
    (("out",), (2, 256, 16, 64), "expected"),            # output of another shape
])
def test_binding_rejects_mismatched_shapes(dg, keys, shape, msg):
    torch = pytest.importorskip("torch")
    t = _attn_tensors(torch)
    for key in keys:
        t[key] = torch.zeros(*shape, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=msg):
        _check(dg, t)


def test_binding_rejects_head_counts_that_do_not_divide(dg):
    torch = pytest.importorskip("torch")
    t = _attn_tensors(torch, Hkv=6)
    with pytest.raises(ValueError, match="multiple"):
        _check(dg, t)


def test_binding_step_tensors_hold_n_steps(dg):
    torch = pytest.importorskip("torch")
    t = _attn_tensors(torch, lead=(12,))
    t["kn"] = torch.zeros(11, 2, 256, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="expected"):
        _check(dg, t, ("q_steps", "k_steps", "v_steps"))
    t = _attn_tensors(torch, lead=(12,))
    t["out"] = torch.zeros(11, 2, 256, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="expected"):
        _check(dg, t, ("q_steps", "k_steps", "v_steps"))


def test_noalloc_rejects_before_any_hip_call(dg):
    """A shape whose partial results exceed the scratch array is refused on the host
    (fake device pointers, never dereferenced), as are the usual argument errors."""
    # 63 empty prefixes and one of 8192 rows: 2016 single-split units plus a split
    # sequence, so every unit writes partial rows (about 71 MB at this shape)
    big = shape(dg, batch=64)
    pl = (ctypes.c_int32 * 64)(*([0] * 63 + [8192]))
    cache = dg.DgKv(FAKE, FAKE, 8192 + 256)
    canvas = dg.DgKv(FAKE, FAKE, 256)
    st = dg.lib.dg_canvas_attn_noalloc(ctypes.byref(big), FAKE, ctypes.byref(cache), pl,
                                       ctypes.byref(canvas), FAKE, None)
    assert st == -5 and b"scratch" in dg.lib.dg_last_error()
    one = (ctypes.c_int32 * 1)(100)
    st = dg.lib.dg_canvas_attn_noalloc(ctypes.byref(shape(dg, head_dim=96)), FAKE,
                                       ctypes.byref(cache), one, ctypes.byref(canvas), FAKE, None)
    assert st == -2
    st = dg.lib.dg_canvas_attn_noalloc(ctypes.byref(shape(dg)), None, ctypes.byref(cache), one,
                                       ctypes.byref(canvas), FAKE, None)
    assert st == -1


def _sample_tensors(torch, B=2, n=256, V=64):
    return dict(logits=torch.zeros(B, n, V, dtype=torch.bfloat16),
                noise=torch.zeros(B, n, dtype=torch.int32),
                prev=torch.zeros(B, n, dtype=torch.int32),
                out=[torch.zeros(B, n, dtype=torch.float32)]
                + [torch.zeros(B, n, dtype=torch.int32) for _ in range(3)]
                + [torch.zeros(B, dtype=torch.int32)])


def test_binding_sampler_checks(dg):
    """The sampler writes entropy, argmax, tokens and accepted per position and stop
    per canvas: caller-supplied outputs of another shape or type are refused."""
    torch = pytest.importorskip("torch")
    t = _sample_tensors(torch)
    dg._check_sample(t["logits"], t["noise"], t["prev"], t["out"])
    dg._check_sample(t["logits"], t["noise"], None, t["out"])
    bad = [
        ("noise", torch.zeros(2, 255, dtype=torch.int32), ValueError),
        ("noise", torch.zeros(2, 256, dtype=torch.int64), TypeError),
        ("prev", torch.zeros(1, 256, dtype=torch.int32), ValueError),
        (0, torch.zeros(2, 256, dtype=torch.float16), TypeError),
        (1, torch.zeros(2, 128, dtype=torch.int32), ValueError),
        (4, torch.zeros(1, dtype=torch.int32), ValueError),
        (2, torch.zeros(256, 2, dtype=torch.int32).t(), ValueError),  # not contiguous
    ]
    for key, val, exc in bad:
        u = _sample_tensors(torch)
        if isinstance(key, int):
            u["out"][key] = val
        else:
            u[key] = val
        with pytest.raises(exc):
            dg._check_sample(u["logits"], u["noise"], u["prev"], u["out"])
    with pytest.raises(ValueError, match="five"):
        dg._check_sample(t["logits"], t["noise"], None, t["out"][:4])


def test_binding_selfcond_checks(dg):
    """z and the weights must agree with the logits' batch and vocabulary and with
    each other's widths: a smaller z would be written past its end."""
    torch = pytest.importorskip("torch")
    bf = torch.bfloat16
    B, V, d, h = 1, 64, 256, 128
    lg = torch.zeros(B, 256, V, dtype=bf)
    ok = dict(embed=torch.zeros(V, d, dtype=bf), w1=torch.zeros(d, h, dtype=bf),
              w2=torch.zeros(h, d, dtype=bf), out=torch.zeros(B, 256, d, dtype=bf))
    dg._check_selfcond(lg, **ok)
    bad = [("embed", torch.zeros(V + 32, d, dtype=bf)), ("w2", torch.zeros(h, d + 256, dtype=bf)),
           ("out", torch.zeros(B, 128, d, dtype=bf)), ("out", torch.zeros(B, 256, d, dtype=torch.float32))]
    for key, val in bad:
        kw = dict(ok)
        kw[key] = val
        with pytest.raises((ValueError, TypeError)):
            dg._check_selfcond(lg, **kw)


def test_binding_prefix_length_checked_first(dg):
    with pytest.raises(ValueError, match="entries"):
        dg._prefix([1, 2, 3], 2)
