"""GPU parity of the fp32 single-launch reader (k_reader_f32): fp32 states,
activations and weights at serving sizes (at most 16 rows B n, r <= 16).

Every case calls libready.so through its C ABI and compares with the
float64 CPU oracle on the same stored values: bit-exact gather, Delta h and
the features within 1e-4 (normwise), out within one fp32 ulp of the oracle
sum plus that tolerance, log-RMS within 1e-5.  Each case also checks that
the plan runs as one launch, so that it is this kernel that is tested.
"""
import sys

import numpy as np
import pytest

import synth
from synth.gen import make_shape

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32 = dict(state_dtype="f32", act_dtype="f32", weight_dtype="f32")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _launches(cfg, path="fused"):
    import hla_recurrent_state_amd as R
    from tests.gpu_util import reader_shape
    st, plan = R.readyPlanCreate(reader_shape(cfg, path=path), list(cfg.slots))
    assert st == R.READY_OK
    st, n = R.readyPlanLaunches(plan)
    R.readyPlanDestroy(plan)
    assert st == R.READY_OK
    return n


def _check(inp, path="fused", debug=True, inplace=False, seqs=None):
    from tests.gpu_util import compare, oracle_reference, run_reader
    dev = _dev()
    cfg = inp.cfg
    n = _launches(cfg, path)
    _say("case", cfg.name, "B", cfg.B, "n", cfg.n, "M", cfg.M, "r", cfg.r, "d", cfg.d, "Hm", cfg.Hm, path,
         "launches", n, "debug" if debug else "no debug outputs")
    assert n == (1 if path == "fused" else 4)
    res = run_reader(inp, dev, inplace=inplace, path=path, debug=debug)
    rep = compare(inp, res, oracle_reference(inp, seqs))
    _say("  report", rep)
    assert rep["ok"], rep
    return res


def _with_gain_and_biases(inp, seed):
    cfg = inp.cfg
    rng = np.random.default_rng(seed)
    store = synth.gen._store
    inp.gamma = store(1.0 + 0.1 * rng.standard_normal(cfg.d), "f32")
    inp.b1 = store(0.2 * rng.standard_normal(cfg.Hm), "f32")
    inp.b2 = store(0.2 * rng.standard_normal(cfg.d), "f32")
    return inp


@pytest.mark.parametrize("name", ["tiny", "wide"])
def test_fused_and_four_launch_paths_agree(name):
    """The two fp32 configurations on the single launch and on the general
    path's four launches: both within the oracle's bar, and within the same
    tolerance of each other."""
    inp = synth.make(name, seed=3)
    a = _check(inp)
    b = _check(inp, path="unfused")
    assert np.array_equal(a["gathered"], b["gathered"])
    scale = max(float(np.max(np.abs(b["delta"]))), 1e-30)
    assert float(np.max(np.abs(a["delta"] - b["delta"]))) <= 2e-4 * scale


@pytest.mark.parametrize("name", ["tiny", "wide"])
def test_timed_configuration_without_debug_outputs(name):
    _check(synth.make(name, seed=4), debug=False)


@pytest.mark.parametrize("B,n,r,H,act", [
    (1, 1, 8, 3, "silu"),        # one row
    (2, 8, 16, 3, "gelu_tanh"),  # 16 rows, the most this kernel takes
    (3, 5, 8, 5, "relu"),        # 15 rows: the 16-row form with a ragged tail
    (16, 1, 16, 2, "silu"),      # 16 sequences of one position
    (2, 3, 8, 24, "silu"),       # 48 pairs: z in 6 column blocks of 64
])
def test_rows_ranks_and_ragged_sizes(B, n, r, H, act):
    """d = 1048 (the last K chunk of the query sums has 24 values), Hm = 100
    (the last A item has 4 of its 16 columns, W2 rows padded to 128 in LDS),
    scattered layer slots, gain and biases."""
    cfg = make_shape("tiny", B=B, n=n, P=8, H=H, L_tot=4, slots=(3, 1), t=12, r=r, d=1048, Hm=100, act=act, **F32)
    _check(_with_gain_and_biases(synth.make(cfg, seed=50 + B + r), seed=B * n))


def test_shared_reader_parameters():
    cfg = make_shape("tiny", B=2, n=7, H=4, t=8, d=512, Hm=32, shared=True, **F32)
    _check(synth.make(cfg, seed=61))


def test_in_place_output():
    _check(synth.make(make_shape("tiny", B=2, t=16), seed=62), inplace=True)


def test_zero_w2_gives_out_equal_h_bitwise():
    from tests.gpu_util import run_reader
    inp = synth.make(make_shape("wide", t=64), seed=63)
    inp.w2 = np.zeros_like(inp.w2)
    res = run_reader(inp, _dev())
    assert np.array_equal(res["out"], inp.h)
    assert np.all(res["delta"] == 0.0)


def test_out_of_range_accept_index_sets_status_and_skips_sequence():
    import tests.gpu_util as gu
    from hla_recurrent_state_amd import READY_ERR_ACCEPT_IDX, StateReader
    from tests.gpu_util import compare, oracle_reference
    dev = _dev()
    cfg = make_shape("tiny", B=3, n=5, H=4, t=16)
    assert _launches(cfg) == 1
    inp = synth.make(cfg, seed=64)
    inp.accept_idx = np.array([2, 8, -1], dtype=np.int32)
    d = synth.device.to_device(inp, dev)
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    o = gu.alloc_outputs(cfg, dev)
    sentinel = 0x7FC12345
    o["gathered"].view(torch.int32).fill_(sentinel)
    o["out"].view(torch.int32).fill_(sentinel)
    o["delta"].view(torch.int32).fill_(sentinel)
    reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"],
           logrms=o["logrms"], delta=o["delta"], feat=o["feat"], dev_status=o["dev_status"])
    torch.cuda.synchronize()
    assert int(o["dev_status"].item()) == READY_ERR_ACCEPT_IDX
    for k in ("gathered", "out", "delta"):
        assert bool(torch.all(o[k][1:].view(torch.int32) == sentinel)), k
    assert bool(torch.all(o["feat"][1:] == 0.0))
    res = {"gathered": o["gathered"].cpu().numpy(), "out": o["out"].cpu().numpy(),
           "logrms": o["logrms"].cpu().numpy(), "delta": o["delta"].cpu().numpy(),
           "feat": o["feat"].cpu().numpy(), "dev_status": 0}
    ok = synth.make(cfg, seed=64)
    ok.accept_idx = inp.accept_idx.copy()
    ok.accept_idx[1:] = 0
    rep = compare(ok, res, oracle_reference(ok, [0]))
    assert rep["ok"], rep


def test_repeated_calls_on_one_workspace_and_determinism():
    """Each call leaves its counters cleared for the next: calls with changed
    accept indices in between reproduce the first call bit for bit."""
    import tests.gpu_util as gu
    from hla_recurrent_state_amd import StateReader
    dev = _dev()
    cfg = make_shape("wide", t=32)
    assert _launches(cfg) == 1
    inp = synth.make(cfg, seed=65)
    d = synth.device.to_device(inp, dev)
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    ws = reader.new_workspace(dev)
    o = gu.alloc_outputs(cfg, dev)

    def call(acc):
        d["accept_idx"].copy_(torch.from_numpy(acc.astype(np.int32)))
        reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"], logrms=o["logrms"],
               delta=o["delta"], feat=o["feat"], dev_status=o["dev_status"], workspace=ws)
        torch.cuda.synchronize()
        return {k: o[k].cpu().numpy().copy() for k in ("gathered", "out", "logrms", "delta", "feat")}

    first = call(inp.accept_idx)
    other = call((inp.accept_idx + 3) % cfg.P)
    again = call(inp.accept_idx)
    for k in first:
        assert np.array_equal(first[k], again[k]), k
    assert not np.array_equal(first["logrms"], other["logrms"])
    assert int(o["dev_status"].item()) == 0
    from tests.gpu_util import compare, oracle_reference
    rep = compare(inp, dict(first, dev_status=0), oracle_reference(inp))
    assert rep["ok"], rep


def test_static_entry_matches_workspace_call():
    """readyStateReaderStatic (the library's own scratch array) on this path:
    bit for bit the workspace call's outputs, on two calls in a row, the
    second with a smaller batch."""
    import tests.gpu_util as gu
    from hla_recurrent_state_amd import StateReader
    dev = _dev()
    for B, seed in ((2, 66), (1, 67)):
        cfg = make_shape("wide", B=B, H=24, t=32)
        assert _launches(cfg) == 1
        inp = synth.make(cfg, seed=seed)
        d = synth.device.to_device(inp, dev)
        reader = StateReader(gu.reader_shape(cfg), cfg.slots)
        outs = []
        for static in (False, True):
            o = gu.alloc_outputs(cfg, dev)
            args = (d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"])
            kw = dict(logrms=o["logrms"], delta=o["delta"], feat=o["feat"], dev_status=o["dev_status"])
            if static:
                reader.call_static(*args, **kw)
            else:
                reader(*args, **kw)
            torch.cuda.synchronize()
            assert int(o["dev_status"].item()) == 0
            outs.append({k: o[k].cpu().numpy() for k in ("gathered", "out", "logrms", "delta", "feat")})
        for k in outs[0]:
            assert np.array_equal(outs[0][k], outs[1][k]), (B, k)
        reader.close()


def test_graph_capture_replays_match_eager():
    import tests.gpu_util as gu
    from hla_recurrent_state_amd import StateReader
    dev = _dev()
    cfg = make_shape("wide", t=32)
    inp = synth.make(cfg, seed=68)
    d = synth.device.to_device(inp, dev)
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    ws = reader.workspace(dev)
    o = gu.alloc_outputs(cfg, dev)
    reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"], delta=o["delta"],
           workspace=ws)
    torch.cuda.synchronize()
    eager = {k: o[k].clone() for k in ("gathered", "out", "delta")}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"],
                   delta=o["delta"], workspace=ws, stream=s.cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in ("gathered", "out", "delta"):
            o[k].zero_()
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("gathered", "out", "delta"):
            assert torch.equal(o[k], eager[k]), (rep, k)
        del junk


def test_two_concurrent_calls_on_two_streams():
    """Two calls at once on two streams, each with its own workspace: both
    complete and each equals the same call made alone, bit for bit."""
    import tests.gpu_util as gu
    from hla_recurrent_state_amd import StateReader
    dev = _dev()
    cfg = make_shape("wide", t=32)
    inps = [synth.make(cfg, seed=s) for s in (69, 70)]
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    ds = [synth.device.to_device(inp, dev) for inp in inps]
    wss = [reader.new_workspace(dev, st.cuda_stream) for st in streams]
    torch.cuda.synchronize()

    def call(k, o, stream):
        d = ds[k]
        reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"],
               dev_status=o["dev_status"], workspace=wss[k], stream=stream.cuda_stream)

    alone = []
    for k in range(2):
        o = gu.alloc_outputs(cfg, dev)
        call(k, o, streams[k])
        torch.cuda.synchronize()
        alone.append(o)
    together = [gu.alloc_outputs(cfg, dev) for _ in range(2)]
    for k in range(2):
        call(k, together[k], streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        assert int(together[k]["dev_status"].item()) == 0
        for key in ("out", "gathered"):
            assert torch.equal(together[k][key], alone[k][key]), (k, key)
