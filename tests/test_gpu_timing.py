"""The kernel timing hooks (dg_kernel_timing_enable, _samples, _read): every
timed launch records an event pair with its own dispatch.  Checks that each
attention and merge launch is counted once, that every duration is positive and
that together they fit inside a pair of stream events around the calls, that a
read clears the record, and that nothing is recorded while the hooks are off or
on the no-allocation path (which runs no hooks)."""
import numpy as np
import pytest

from canvas_attention_amd import synth
from helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU machines skip the module
    pytest.skip("needs a GPU", allow_module_level=True)

import canvas_attention_amd.dg as dg  # noqa: E402

EMPTY = (0, 0.0, 0, 0.0)


def _inputs(L=2048):
    Lv = np.asarray([L], np.int32)
    kc, vc = synth.cache(7, Lv, L + 256, 8, 128, "bf16")
    q, kn, vn = synth.canvas(7, 1, 16, 8, 128, "bf16")
    return [to_dev(x) for x in (q, kc, vc, kn, vn)], Lv


def test_timing_hooks_count_and_bound_every_launch(monkeypatch):
    monkeypatch.setenv("DG_SPLIT_KEYS", "512")  # several splits: every call also merges
    (q, kc, vc, kn, vn), L = _inputs()
    out = torch.empty_like(q)
    ws = dg.alloc_workspace(q, 8, int(L[0]))
    dg.canvas_attn(q, kc, vc, L, kn, vn, out=out, workspace=ws)
    torch.cuda.synchronize()
    dg.kernel_timing_read()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    dg.kernel_timing_enable(True)
    try:
        ev[0].record(stream)
        for _ in range(5):
            dg.canvas_attn(q, kc, vc, L, kn, vn, out=out, workspace=ws)
        ev[1].record(stream)
        torch.cuda.synchronize()
        attn, merge = dg.kernel_timing_samples(64)
    finally:
        dg.kernel_timing_enable(False)
    total = ev[0].elapsed_time(ev[1])
    print(f"attention {np.round(attn, 4)} ms, merge {np.round(merge, 4)} ms, calls {total:.4f} ms")
    assert len(attn) == 5 and len(merge) == 5
    assert all(x > 0 for x in attn + merge)
    # the kernels run one after another on the stream, inside the outer events
    assert sum(attn) + sum(merge) <= total * 1.01 + 1e-3
    assert dg.kernel_timing_read() == EMPTY


def test_timing_hooks_record_nothing_when_off_or_without_allocation():
    (q, kc, vc, kn, vn), L = _inputs()
    out = torch.empty_like(q)
    dg.kernel_timing_read()
    dg.canvas_attn(q, kc, vc, L, kn, vn, out=out)
    torch.cuda.synchronize()
    assert dg.kernel_timing_read() == EMPTY
    dg.kernel_timing_enable(True)
    try:
        dg.canvas_attn_noalloc(q, kc, vc, L, kn, vn, out)
        torch.cuda.synchronize()
        assert dg.kernel_timing_read() == EMPTY
    finally:
        dg.kernel_timing_enable(False)
