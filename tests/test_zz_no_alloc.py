"""dg_canvas_attn_noalloc (partial results in the library's per-GPU scratch array)
against dg_canvas_attn (partial results in a caller workspace): the same kernels
on the same plan, so the outputs must agree bit for bit; also against the oracle
at the bf16 gate.  Two calls in a row, the second with a smaller input, so the
second call runs on scratch the first one left behind."""
import numpy as np
import pytest

from canvas_attention_amd import synth
from helpers import TOL_BF16, record, row_err, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU machines skip the module
    pytest.skip("needs a GPU", allow_module_level=True)

import canvas_attention_amd.dg as dg  # noqa: E402  (loads libdg.so; raises if missing)


def _inputs(seed, L, B, Hq=16, Hkv=8, D=128):
    L = np.asarray(L, np.int32)
    kc, vc = synth.cache(seed, L, int(L.max()) + 256, Hkv, D, "bf16")
    q, kn, vn = synth.canvas(seed, B, Hq, Hkv, D, "bf16")
    return L, kc, vc, q, kn, vn


def test_noalloc_matches_the_workspace_entry_point(oracle_lib):
    # the second call is smaller: fewer sequences and units, a shorter prefix
    for seed, L in ((41, [8192, 3000]), (42, [700])):
        L, kc, vc, q, kn, vn = _inputs(seed, L, len(L))
        args = (to_dev(q), to_dev(kc), to_dev(vc), L, to_dev(kn), to_dev(vn))
        ref = dg.canvas_attn(*args)
        out = torch.empty_like(ref)
        got = dg.canvas_attn_noalloc(*args, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), f"L={L.tolist()}: noalloc differs from dg_canvas_attn"
        err = record(f"noalloc L={L.tolist()}",
                     row_err(to_host_f64(got), oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)), TOL_BF16)
        assert err <= TOL_BF16


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """63 empty prefixes and one of 8192 rows: every one of the 2000-odd units then
    writes partial rows (about 71 MB), more than the scratch holds.  The call is
    refused on the host with a clear error and the output is left untouched (the
    tensors' contents do not matter: nothing is launched)."""
    B, Hq, Hkv, D = 64, 16, 8, 128
    L = np.array([0] * 63 + [8192], np.int32)
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    args = (z(B, 256, Hq, D), z(B, 8192 + 256, Hkv, D), z(B, 8192 + 256, Hkv, D), L,
            z(B, 256, Hkv, D), z(B, 256, Hkv, D))
    out = z(B, 256, Hq, D)
    with pytest.raises(dg.DgError, match="scratch"):
        dg.canvas_attn_noalloc(*args, out=out)
    torch.cuda.synchronize()
    assert not out.any()


def test_noalloc_replayed_from_a_captured_graph():
    """The callers this entry point is for include code under HIP graph capture:
    captured once, the call is replayed three times with other eager launches of
    the library (which also use the scratch's GPU) and synchronizations between
    the replays; every replay must equal the eager workspace call bit for bit."""
    L, kc, vc, q, kn, vn = _inputs(43, [3000], 1)
    args = (to_dev(q), to_dev(kc), to_dev(vc), L, to_dev(kn), to_dev(vn))
    ref = dg.canvas_attn(*args)
    out = torch.empty_like(ref)
    dg.canvas_attn_noalloc(*args, out=out)  # first call on the device: scratch address lookup
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    L2, kc2, vc2, q2, kn2, vn2 = _inputs(44, [5000], 1)
    other = (to_dev(q2), to_dev(kc2), to_dev(vc2), L2, to_dev(kn2), to_dev(vn2))
    ref2 = dg.canvas_attn(*other)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dg.canvas_attn_noalloc(*args, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        # eager work between replays, on the same scratch: another no-allocation call
        got2 = dg.canvas_attn_noalloc(*other, out=torch.empty_like(ref2))
        torch.cuda.synchronize()
        assert torch.equal(got2, ref2), f"replay {rep}: eager call between replays differs"
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager call"
