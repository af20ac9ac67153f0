"""readyStateReaderStatic, the entry point with no workspace argument (for
callers that cannot allocate), against readyStateReader with a workspace of
its own.

Both run the same kernels, so every output must agree bit for bit; the
static call's outputs also meet the oracle's parity bar.  Calls follow each
other on one stream with different plans -- a larger one, then a smaller one
(fewer rows, the 16-row kernel form), the all-fp32 four-launch path, then the
first plan again -- since every call shares the device's one static array.
"""
import sys

import numpy as np
import pytest

import synth
from synth.gen import make_shape

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _both(inp, dev):
    """One readyStateReader call and one readyStateReaderStatic call on the
    same inputs; returns both sets of host outputs."""
    from hla_recurrent_state_amd import StateReader
    from synth.device import to_device, to_numpy_bits
    from tests.gpu_util import alloc_outputs, reader_shape
    cfg = inp.cfg
    d = to_device(inp, dev)
    reader = StateReader(reader_shape(cfg), cfg.slots)
    res = []
    for static in (False, True):
        o = alloc_outputs(cfg, dev)
        for k in ("gathered", "out", "logrms", "delta", "feat"):
            o[k].view(torch.uint8).fill_(0x5A)  # the same fill under both, so untouched values match too
        args = (d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"])
        kw = dict(logrms=o["logrms"], delta=o["delta"], feat=o["feat"], dev_status=o["dev_status"])
        if static:
            reader.call_static(*args, **kw)
        else:
            reader(*args, **kw)
        torch.cuda.synchronize()
        res.append({
            "gathered": to_numpy_bits(o["gathered"], cfg.state_dtype),
            "out": to_numpy_bits(o["out"], cfg.act_dtype),
            "logrms": o["logrms"].cpu().numpy(),
            "delta": o["delta"].cpu().numpy(),
            "feat": o["feat"].cpu().numpy(),
            "dev_status": int(o["dev_status"].item()),
        })
    reader.close()
    return res


def _check(inp, dev):
    from tests.gpu_util import compare, oracle_reference
    cfg = inp.cfg
    _say("case", cfg.name, "B", cfg.B, "M", cfg.M, "r", cfg.r, cfg.state_dtype)
    ws, st = _both(inp, dev)
    for k in ("gathered", "out", "logrms", "delta", "feat"):
        assert np.array_equal(ws[k].view(np.uint8), st[k].view(np.uint8)), k
    assert ws["dev_status"] == 0 and st["dev_status"] == 0
    rep = compare(inp, st, oracle_reference(inp))
    _say("  report", rep)
    assert rep["ok"], rep


def test_static_scratch_matches_workspace_calls():
    dev = _dev()
    big = synth.make(make_shape("batched", B=12, t=16), seed=91)      # 84 rows: the large-row form
    small = synth.make(make_shape("paper", B=2, t=16), seed=92)       # 14 rows: the 16-row form
    fp32 = synth.make(make_shape("tiny", B=2, H=3, t=16), seed=93)    # general path, four launches
    for inp in (big, small, fp32, big):
        _check(inp, dev)


def test_static_scratch_rejects_plans_beyond_its_size():
    """The rank workload's general path needs more scratch than the array
    holds: refused before anything is launched, outputs untouched."""
    from hla_recurrent_state_amd import (READY_ERR_STATIC_SCRATCH_TOO_SMALL, READY_STATIC_SCRATCH_BYTES,
                                         ReadyError, StateReader)
    from tests.gpu_util import reader_shape
    dev = _dev()
    cfg = make_shape("rank", B=256)
    reader = StateReader(reader_shape(cfg), cfg.slots)
    assert reader.workspace_bytes > READY_STATIC_SCRATCH_BYTES
    one = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    states = torch.zeros((1, 1, 1, 1, 128, 128), dtype=torch.bfloat16, device=dev)
    acc = torch.zeros(1, dtype=torch.int32, device=dev)
    w = {k: one for k in ("wq", "u", "v", "w1", "w2")}
    with pytest.raises(ReadyError) as e:
        reader.call_static(states, acc, one, w, one, one)
    assert e.value.code == READY_ERR_STATIC_SCRATCH_TOO_SMALL
    reader.close()
