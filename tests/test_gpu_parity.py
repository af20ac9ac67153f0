"""GPU parity of the HIP state reader against the float64 CPU oracle.

Every case calls libready.so through its C ABI (ctypes) on seeded synthetic
inputs and compares element by element with the oracle run on the same
stored values: bit-exact gather, Delta h within the normwise tolerance, out
within one ulp of the rounded oracle sum, log-RMS within 1e-5.
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


def _check(inp, seqs=None, inplace=False, expect_ok=True, path="fused", debug=True):
    from tests.gpu_util import compare, oracle_reference, run_reader
    dev = _dev()
    _say("case", inp.cfg.name, "B", inp.cfg.B, "M", inp.cfg.M, "r", inp.cfg.r, inp.cfg.state_dtype, path,
         "debug outputs" if debug else "no debug outputs")
    res = run_reader(inp, dev, inplace=inplace, path=path, debug=debug)
    ref = oracle_reference(inp, seqs)
    rep = compare(inp, res, ref)
    _say("  report", rep)
    if expect_ok:
        assert rep["ok"], rep
    return res, ref, rep


# ------------------------------------------------------------ the five configurations

def test_tiny():
    _check(synth.make("tiny", seed=1))


def test_paper_shape():
    _check(synth.make("paper", seed=1))


def test_wide_heads():
    _check(synth.make("wide", seed=1))


def test_batched():
    _check(synth.make("batched", seed=1))


@pytest.mark.parametrize("name", ["paper", "batched"])
def test_timed_configuration_without_debug_outputs(name):
    """The call exactly as the benchmark times it: logrms, delta and feat
    are NULL.  gathered is bit-exact and out is within one bf16 ulp of
    RNE(h + Delta h_ref) plus the tolerance, at the full shapes (short state
    histories, t = 64: the values change, the launch does not)."""
    cfg = make_shape(name, t=64)
    _check(synth.make(cfg, seed=21), debug=False)


# ------------------------------------------------------------ the unfused path (four launches)

def test_paper_shape_unfused_path():
    _check(synth.make("paper", seed=1), path="unfused")


def test_batched_unfused_path_matches_fused():
    # the four-launch path on the single-kernel path's workload: within
    # tolerance of the oracle, the gather bit-identical to the single kernel's,
    # log-RMS equal up to the order of the sum of squares (8 waves against 4)
    from tests.gpu_util import run_reader
    inp = synth.make("batched", seed=2)
    res_u, _, _ = _check(inp, seqs=[0, 31, 63], path="unfused")
    res_f = run_reader(inp, _dev())
    assert np.array_equal(res_u["gathered"], res_f["gathered"])
    assert np.max(np.abs(res_u["logrms"] - res_f["logrms"])) <= 1e-6 * max(1.0, np.max(np.abs(res_f["logrms"])))


def test_rank_ablation_sampled():
    """B = 256, 48 pairs, r = 128: the oracle checks a sample of sequences,
    and the gather is checked bit-exact for all of them."""
    inp = synth.make("rank", seed=1)
    res, ref, rep = _check(inp, seqs=[0, 1, 97, 128, 200, 255])
    want = inp.buf[np.arange(inp.cfg.B), inp.accept_idx][:, list(inp.cfg.slots)]
    want = want.reshape(inp.cfg.B, inp.cfg.M, 128, 128)
    assert np.array_equal(res["gathered"], want)


def test_large_row_count_residual_epilogue():
    """B = 256 (1792 rows), d = 2560, r = 64: the second MLP layer runs on
    the 128 x 128 matrix-core GEMM with its 16-byte residual epilogue.  In
    place (out is h), then with two out-of-range accept indices: those
    sequences' out rows stay untouched, the sampled others match the oracle."""
    cfg = make_shape("paper", B=256, H=1, t=8, r=64, d=2560, Hm=64)
    inp = synth.make(cfg, seed=71)
    _check(inp, seqs=[0, 1, 130, 255], inplace=True)
    dev = _dev()
    bad = synth.make(cfg, seed=71)
    bad.accept_idx = bad.accept_idx.copy()
    bad.accept_idx[[5, 200]] = cfg.P
    import tests.gpu_util as gu
    d = synth.device.to_device(bad, dev)
    from hla_recurrent_state_amd import StateReader, READY_ERR_ACCEPT_IDX
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    o = gu.alloc_outputs(cfg, dev)
    sentinel_bits = 0x7FC1
    o["out"].view(torch.int16).fill_(sentinel_bits)
    reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"],
           logrms=o["logrms"], delta=o["delta"], feat=o["feat"], dev_status=o["dev_status"])
    torch.cuda.synchronize()
    reader.close()
    assert int(o["dev_status"].item()) == READY_ERR_ACCEPT_IDX
    out = o["out"].view(torch.int16).cpu().numpy()
    assert np.all(out[[5, 200]] == sentinel_bits)
    from tests.gpu_util import compare, oracle_reference
    res = {"gathered": o["gathered"].view(torch.int16).cpu().numpy().view(np.uint16),
           "out": out.view(np.uint16), "logrms": o["logrms"].cpu().numpy(),
           "delta": o["delta"].cpu().numpy(), "feat": o["feat"].cpu().numpy(), "dev_status": 0}
    rep = compare(bad, res, oracle_reference(bad, [0, 4, 6, 199, 201, 255]))
    assert rep["ok"], rep


# ------------------------------------------------------------ multi-tile cases with ragged tails

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "relu"])
def test_ragged_shapes(dt, act):
    """Rows B*n = 15 (two row blocks, ragged), d = 1048 (ragged K splits),
    Hm = 100 (unaligned rows: scalar weight path), scattered layer slots,
    r = 16, with gain and biases."""
    cfg = make_shape("tiny", B=3, n=5, H=3, L_tot=4, slots=(3, 1), t=12, r=16, d=1048, Hm=100,
                     state_dtype=dt, act_dtype=dt, weight_dtype=dt, act=act)
    inp = synth.make(cfg, seed=7)
    rng = np.random.default_rng(3)
    store = synth.gen._store
    inp.gamma = store(1.0 + 0.1 * rng.standard_normal(cfg.d), dt)
    inp.b1 = store(0.2 * rng.standard_normal(cfg.Hm), dt)
    inp.b2 = store(0.2 * rng.standard_normal(cfg.d), dt)
    _check(inp)


@pytest.mark.parametrize("r", [8, 16, 24, 32])
@pytest.mark.parametrize("rows", ["one_tile", "several_tiles"])
def test_bf16_fast_path_ragged(r, rows):
    """All-bf16 path: B*n = 15 (one 16-row tile) or 35 (one ragged 64-row
    tile, several sequences per tile), d = 1048 (ragged K chunks), Hm = 72
    (ragged 64-column tiles of the first MLP layer), scattered layer slots,
    with gain and biases."""
    B, n = (3, 5) if rows == "one_tile" else (5, 7)
    cfg = make_shape("paper", B=B, n=n, H=8, L_tot=5, slots=(4, 1), t=12, r=r, d=1048, Hm=72)
    inp = synth.make(cfg, seed=8 + r)
    rng = np.random.default_rng(r)
    store = synth.gen._store
    inp.gamma = store(1.0 + 0.1 * rng.standard_normal(cfg.d), "bf16")
    inp.b1 = store(0.2 * rng.standard_normal(cfg.Hm), "bf16")
    inp.b2 = store(0.2 * rng.standard_normal(cfg.d), "bf16")
    _check(inp)


@pytest.mark.parametrize("slots,B", [((4, 1, 3), 2), ((4, 1, 3), 5), ((4, 1, 3, 0, 2), 5)])
def test_bf16_fast_path_many_pairs_rank_8(slots, B):
    """r = 8 with 48 or 80 layer-head pairs: more (pair, output) items of f
    than threads in a workgroup (384 or 640 against 256), so threads build
    two or three of them, at 14 rows (one 16-row tile) and 35 rows (a ragged
    32-row block of out)."""
    cfg = make_shape("paper", B=B, n=7, H=16, L_tot=5, slots=slots, t=12, r=8, d=1048, Hm=72)
    assert cfg.M * cfg.r > 256
    from hla_recurrent_state_amd import StateReader
    from tests.gpu_util import reader_shape
    sr = StateReader(reader_shape(cfg), cfg.slots)
    sr.prep_size(1)  # raises unless the plan takes the single-kernel path
    sr.close()
    _check(synth.make(cfg, seed=60 + len(slots) + B))


@pytest.mark.parametrize("act", ["gelu_tanh", "relu"])
def test_bf16_fast_path_activations(act):
    cfg = make_shape("paper", B=2, t=12, act=act)
    _check(synth.make(cfg, seed=14))


@pytest.mark.parametrize("r", [8, 24, 128])
def test_ranks_and_mixed_dtypes(r):
    cfg = make_shape("tiny", B=2, H=2, t=8, r=r, d=640, Hm=64, state_dtype="bf16", act_dtype="f32",
                     weight_dtype="bf16")
    _check(synth.make(cfg, seed=11))


def test_shared_reader_parameters():
    cfg = make_shape("tiny", B=2, H=4, t=8, d=512, Hm=32, shared=True, state_dtype="bf16",
                     act_dtype="bf16", weight_dtype="bf16")
    _check(synth.make(cfg, seed=12))


def test_long_block_and_many_rows():
    """n = 16 positions and B*n = 48 rows with fp32 states and bf16 weights."""
    cfg = make_shape("tiny", B=3, n=16, P=16, H=2, t=20, d=256, Hm=48, state_dtype="f32",
                     act_dtype="bf16", weight_dtype="bf16")
    _check(synth.make(cfg, seed=13))


# ------------------------------------------------------------ matrix-core per-state kernel (bf16, r > 32)

@pytest.mark.parametrize("r", [40, 64, 96, 128])
def test_bf16_general_ranks_many_tiles(r):
    """bf16 states and weights with r > 32: 640 state tiles, so each
    persistent workgroup walks two or three tiles and crosses layer-head pairs;
    r = 40 and 96 leave part of the last 32-rank step padded.  Gain and
    biases set."""
    cfg = make_shape("paper", B=20, t=8, r=r, d=512, Hm=64)
    inp = synth.make(cfg, seed=50 + r)
    rng = np.random.default_rng(r)
    store = synth.gen._store
    inp.gamma = store(1.0 + 0.1 * rng.standard_normal(cfg.d), "bf16")
    inp.b1 = store(0.2 * rng.standard_normal(cfg.Hm), "bf16")
    inp.b2 = store(0.2 * rng.standard_normal(cfg.d), "bf16")
    _check(inp)


@pytest.mark.parametrize("act_dtype", ["bf16", "f32"])
def test_bf16_general_many_rows_large_tiles(act_dtype):
    """B n = 259 rows (three 128-row tiles, the last ragged) with bf16 states
    and weights and r = 64: the 128 x 128 tile GEMMs of the general path
    (query sums split over K when the activations are bf16, the first MLP
    layer split over K with a separate sum, bias and activation), d = 1048 and
    Hm = 200 ragged against the 32-wide K steps and 128-wide column tiles.
    The oracle checks a sample of sequences; the gather is checked for all."""
    cfg = make_shape("paper", B=37, t=8, r=64, d=1048, Hm=200, act_dtype=act_dtype)
    inp = synth.make(cfg, seed=70)
    rng = np.random.default_rng(70)
    store = synth.gen._store
    inp.gamma = store(1.0 + 0.1 * rng.standard_normal(cfg.d), "bf16")
    inp.b1 = store(0.2 * rng.standard_normal(cfg.Hm), "bf16")
    inp.b2 = store(0.2 * rng.standard_normal(cfg.d), "bf16")
    res, ref, rep = _check(inp, seqs=[0, 17, 18, 36])
    want = inp.buf[np.arange(cfg.B), inp.accept_idx][:, list(cfg.slots)].reshape(cfg.B, cfg.M, 128, 128)
    assert np.array_equal(res["gathered"], want)


@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_rank_32_at_the_paper_pair_count(path):
    """r = 32 with the pages' 32 layer-head pairs (arXiv section 4.4,
    Table 3) at the batched shape, on the single kernel (the default plan)
    and on the four-launch path (the matrix-core per-state kernel at exactly
    r = 32).  The oracle checks a sample of sequences; the gather is checked
    for all."""
    from hla_recurrent_state_amd import READY_ERR_UNSUPPORTED, ReadyError, StateReader
    from tests.gpu_util import reader_shape
    cfg = make_shape("batched", t=16, r=32)
    assert cfg.M == 32
    sr = StateReader(reader_shape(cfg, path=path), cfg.slots)
    try:
        sr.prep_size(1)
        single = True
    except ReadyError as e:
        assert e.code == READY_ERR_UNSUPPORTED
        single = False
    sr.close()
    assert single == (path == "fused")
    _say("r = 32, M = 32:", "single kernel" if single else "four launches")
    inp = synth.make(cfg, seed=33)
    res, ref, rep = _check(inp, seqs=[0, 1, 31, 62, 63], path=path)
    want = inp.buf[np.arange(cfg.B), inp.accept_idx][:, list(cfg.slots)].reshape(cfg.B, cfg.M, 128, 128)
    assert np.array_equal(res["gathered"], want)


def test_bf16_general_long_block_full_rank():
    """n = 16 positions (every row of the padded query block used), r = 128."""
    cfg = make_shape("paper", B=3, n=16, P=16, H=4, t=20, r=128, d=384, Hm=48)
    _check(synth.make(cfg, seed=61))


def test_bf16_general_shared_parameters():
    cfg = make_shape("paper", B=5, H=6, t=8, r=64, d=256, Hm=32, shared=True)
    _check(synth.make(cfg, seed=62))


# ------------------------------------------------------------ accept index edge cases

@pytest.mark.parametrize("pattern", ["zeros", "last", "mixed"])
def test_accept_index_edges(pattern):
    cfg = make_shape("paper", B=5, t=16)
    inp = synth.make(cfg, seed=21)
    inp.accept_idx = {"zeros": np.zeros(5), "last": np.full(5, cfg.P - 1),
                      "mixed": np.array([0, 7, 3, 7, 0])}[pattern].astype(np.int32)
    _check(inp)


@pytest.mark.parametrize("r", [8, 64])
def test_out_of_range_accept_index_sets_status_and_skips_sequence(r):
    """r = 8 runs the single-kernel path, r = 64 the matrix-core per-state
    kernel of the general path."""
    dev = _dev()
    cfg = make_shape("paper", B=3, t=16, r=r)
    inp = synth.make(cfg, seed=22)
    inp.accept_idx = np.array([2, 8, -1], dtype=np.int32)
    import tests.gpu_util as gu
    d = synth.device.to_device(inp, dev)
    from hla_recurrent_state_amd import StateReader
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    o = gu.alloc_outputs(cfg, dev)
    sentinel_bits = 0x7FC1
    o["gathered"].view(torch.int16).fill_(sentinel_bits)
    o["out"].view(torch.int16).fill_(sentinel_bits)
    reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"],
           logrms=o["logrms"], delta=o["delta"], feat=o["feat"], dev_status=o["dev_status"])
    torch.cuda.synchronize()
    from hla_recurrent_state_amd import READY_ERR_ACCEPT_IDX
    assert int(o["dev_status"].item()) == READY_ERR_ACCEPT_IDX
    g = o["gathered"].view(torch.int16).cpu().numpy()
    out = o["out"].view(torch.int16).cpu().numpy()
    assert np.all(g[1:] == sentinel_bits) and np.all(out[1:] == sentinel_bits)
    # the valid sequence is still computed correctly
    from tests.gpu_util import compare, oracle_reference
    res = {"gathered": g.view(np.uint16), "out": out.view(np.uint16),
           "logrms": o["logrms"].cpu().numpy(), "delta": o["delta"].cpu().numpy(),
           "feat": o["feat"].cpu().numpy(), "dev_status": 0}
    ok = synth.make(cfg, seed=22)
    ok.accept_idx = inp.accept_idx.copy()
    ok.accept_idx[1:] = 0
    rep = compare(ok, res, oracle_reference(ok, [0]))
    assert rep["ok"], rep


# ------------------------------------------------------------ properties

def test_fast_path_large_batch():
    # 512 sequences (16384 state tiles, 3584 draft rows): many tiles per
    # workgroup and many row blocks of the query and MLP items; the oracle
    # checks sequences across the batch
    _check(synth.make(make_shape("batched", B=512, t=8), seed=35), seqs=[0, 1, 255, 300, 511])


def test_in_place_output():
    _check(synth.make(make_shape("paper", B=2, t=16), seed=31), inplace=True)


def test_zero_w2_gives_out_equal_h_bitwise():
    from tests.gpu_util import run_reader
    inp = synth.make(make_shape("paper", B=2, t=16), seed=32)
    inp.w2 = np.zeros_like(inp.w2)
    res = run_reader(inp, _dev())
    assert np.array_equal(res["out"], inp.h)
    assert np.all(res["delta"] == 0.0)


def test_run_to_run_bitwise_determinism():
    from tests.gpu_util import run_reader
    inp = synth.make(make_shape("batched", B=8, t=16), seed=33)
    a = run_reader(inp, _dev())
    b = run_reader(inp, _dev())
    for k in ("gathered", "out", "logrms", "delta", "feat"):
        assert np.array_equal(a[k], b[k]), k


def test_batch_permutation_equivariance():
    from tests.gpu_util import run_reader
    inp = synth.make(make_shape("batched", B=6, t=16), seed=34)
    a = run_reader(inp, _dev())
    perm = np.array([3, 0, 5, 1, 4, 2])
    inp.buf = np.ascontiguousarray(inp.buf[perm])
    inp.accept_idx = inp.accept_idx[perm]
    inp.h = np.ascontiguousarray(inp.h[perm])
    b = run_reader(inp, _dev())
    for k in ("gathered", "out", "logrms", "delta", "feat"):
        assert np.array_equal(a[k][perm], b[k]), k


def test_zero_batch_is_a_no_op():
    from hla_recurrent_state_amd import StateReader
    import tests.gpu_util as gu
    dev = _dev()
    cfg = make_shape("paper", B=1, t=4)
    inp = synth.make(cfg, seed=35)
    d = synth.device.to_device(inp, dev)
    reader = StateReader(gu.reader_shape(cfg, B=0), cfg.slots)
    o = gu.alloc_outputs(cfg, dev, B=1)
    o["out"].fill_(3.0)
    reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"])
    torch.cuda.synchronize()
    assert torch.all(o["out"] == 3.0)


def test_graph_capture_replays_match_eager():
    """The call captured into a HIP graph, replayed several times with eager
    work and synchronisations in between; every replay equals the eager run."""
    from hla_recurrent_state_amd import StateReader
    import tests.gpu_util as gu
    dev = _dev()
    cfg = make_shape("batched", B=4, t=16)
    inp = synth.make(cfg, seed=40)
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
        junk = torch.randn(1 << 20, device=dev).sum()     # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("gathered", "out", "delta"):
            assert torch.equal(o[k].view(torch.int8) if o[k].dtype != torch.float32 else o[k], 
                               eager[k].view(torch.int8) if eager[k].dtype != torch.float32 else eager[k]), (rep, k)
        del junk


# ------------------------------------------------------------ workspace contract

def test_unprepared_workspace_is_reported_and_computes_nothing():
    """A workspace that readyWorkspaceInit did not prepare: the call stores
    READY_ERR_WORKSPACE_UNINIT and leaves every output untouched."""
    from hla_recurrent_state_amd import READY_ERR_WORKSPACE_UNINIT, StateReader
    import tests.gpu_util as gu
    dev = _dev()
    cfg = make_shape("paper", B=2, t=8)
    inp = synth.make(cfg, seed=41)
    d = synth.device.to_device(inp, dev)
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    ws = torch.zeros(max(reader.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    o = gu.alloc_outputs(cfg, dev)
    o["out"].view(torch.int16).fill_(0x7FC1)
    o["gathered"].view(torch.int16).fill_(0x7FC1)
    reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"],
           dev_status=o["dev_status"], workspace=ws)
    torch.cuda.synchronize()
    assert int(o["dev_status"].item()) == READY_ERR_WORKSPACE_UNINIT
    assert bool(torch.all(o["out"].view(torch.int16) == 0x7FC1))
    assert bool(torch.all(o["gathered"].view(torch.int16) == 0x7FC1))


def test_repeated_calls_on_one_workspace():
    """Calls on one prepared workspace: each call leaves its counters cleared
    for the next, so repeated calls (with changed accept indices in between)
    reproduce single-call results bit for bit."""
    from hla_recurrent_state_amd import StateReader
    import tests.gpu_util as gu
    from synth.device import to_numpy_bits
    dev = _dev()
    cfg = make_shape("batched", B=6, t=16)
    inp = synth.make(cfg, seed=42)
    d = synth.device.to_device(inp, dev)
    reader = StateReader(gu.reader_shape(cfg), cfg.slots)
    ws = reader.new_workspace(dev)
    o = gu.alloc_outputs(cfg, dev)

    def call(acc):
        d["accept_idx"].copy_(torch.from_numpy(acc.astype(np.int32)))
        reader(d["states"], d["accept_idx"], d["h"], d["weights"], o["gathered"], o["out"],
               logrms=o["logrms"], delta=o["delta"], dev_status=o["dev_status"], workspace=ws)
        torch.cuda.synchronize()
        return {k: (to_numpy_bits(o[k], cfg.act_dtype) if k == "out" else o[k].cpu().numpy().copy())
                for k in ("out", "logrms", "delta")}

    first = call(inp.accept_idx)
    other = call((inp.accept_idx + 3) % cfg.P)
    again = call(inp.accept_idx)
    for k in first:
        assert np.array_equal(first[k], again[k]), k
    assert not np.array_equal(first["logrms"], other["logrms"])
    assert int(o["dev_status"].item()) == 0
    rep = __import__("tests.gpu_util", fromlist=["compare"]).compare(
        inp, {"gathered": to_numpy_bits(o["gathered"], cfg.state_dtype), "out": first["out"],
              "logrms": first["logrms"], "delta": first["delta"],
              "feat": np.zeros((cfg.B, cfg.n, cfg.F), np.float32), "dev_status": 0},
        __import__("tests.gpu_util", fromlist=["oracle_reference"]).oracle_reference(inp))
    assert rep["gather_bitexact"] and rep["dh_rel"] <= rep["tol"] and rep["logrms_err"] <= 1e-5, rep
    assert rep["out_excess"] <= 0.0, rep


def test_two_concurrent_calls_on_two_streams():
    """Two batched calls at once, each on its own stream with its own
    workspace and buffers: the work items of each launch are claimed from
    its own counters and a launch never needs its whole grid resident at
    once, so both complete, and each gives bit for bit the outputs of the
    same call made alone."""
    from hla_recurrent_state_amd import StateReader
    import tests.gpu_util as gu
    from synth.device import to_numpy_bits
    dev = _dev()
    cfg = make_shape("batched", t=16)
    inps = [synth.make(cfg, seed=s) for s in (81, 82)]
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
        call(k, together[k], streams[k])   # both enqueued before either is waited for
    torch.cuda.synchronize()
    for k in range(2):
        _say("stream", k, "status", int(together[k]["dev_status"].item()))
        assert int(together[k]["dev_status"].item()) == 0
        for key, dt in (("out", cfg.act_dtype), ("gathered", cfg.state_dtype)):
            assert np.array_equal(to_numpy_bits(together[k][key], dt), to_numpy_bits(alone[k][key], dt)), key
    rep = gu.compare(inps[0], {"gathered": to_numpy_bits(together[0]["gathered"], cfg.state_dtype),
                               "out": to_numpy_bits(together[0]["out"], cfg.act_dtype), "logrms": None,
                               "delta": None, "feat": None, "dev_status": 0},
                     gu.oracle_reference(inps[0], seqs=[0, 31, 63]))
    assert rep["ok"], rep
    reader.close()
