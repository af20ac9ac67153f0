"""GPU parity of several readers sharing one gather (readyStatePrepare once,
then readyStateApply per reader) against the float64 oracle's multi_reader,
and against single readyStateReader calls with each reader's weights.

The bar is the single reader's: gather bit-exact, log-RMS within 1e-5,
f and Delta h within the normwise 1e-2 (bf16), out within one bf16 ulp of
the rounded oracle sum plus that tolerance.  Each apply call must also give
bit for bit what one readyStateReader call gives with that reader's weights
and h: the same kernels do the same arithmetic on the same values.
"""
import sys

import numpy as np
import pytest

import synth
from tests.gpu_util import reader_shape
from synth.device import tensor, to_device, to_numpy_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _reader_dev(rd, cfg, device):
    w = {k: tensor(rd[k], cfg.weight_dtype, device) for k in ("wq", "u", "v", "w1", "w2")}
    for src, dst in (("gamma", "h_gamma"), ("b1", "b1"), ("b2", "b2")):
        if src in rd:
            w[dst] = tensor(rd[src], cfg.weight_dtype, device)
    return tensor(rd["h"], cfg.act_dtype, device), w


def _run_multi(inp, readers, device, inplace=False, sr=None):
    """prepare once, apply per reader; host copies of every output.  `sr`
    (a StateReader) is reused with its workspace when given."""
    from hla_recurrent_state_amd import StateReader
    from tests.gpu_util import alloc_outputs, reader_shape
    cfg = inp.cfg
    d = to_device(inp, device)
    rdev = [_reader_dev(rd, cfg, device) for rd in readers]
    own = sr is None
    if own:
        sr = StateReader(reader_shape(cfg), cfg.slots)
    n_inj = len(readers)
    prep = sr.new_prep(n_inj, device)
    o = alloc_outputs(cfg, device)
    sr.prepare(d["states"], d["accept_idx"], [w for _, w in rdev], o["gathered"], prep, logrms=o["logrms"],
               dev_status=o["dev_status"])
    res = []
    for i, (h, w) in enumerate(rdev):
        oi = alloc_outputs(cfg, device)
        oi["out"].fill_(7.0)  # sentinel for rows that must stay unwritten
        if inplace:
            oi["out"] = h.clone()
            h = oi["out"]
        sr.apply(prep, n_inj, i, h, w, oi["out"], delta=oi["delta"], feat=oi["feat"], dev_status=oi["dev_status"])
        res.append(oi)
    torch.cuda.synchronize(device)
    host = []
    for oi in res:
        host.append({
            "gathered": to_numpy_bits(o["gathered"], cfg.state_dtype),
            "logrms": o["logrms"].cpu().numpy(),
            "out": to_numpy_bits(oi["out"], cfg.act_dtype),
            "delta": oi["delta"].cpu().numpy(),
            "feat": oi["feat"].cpu().numpy(),
            "dev_status": int(o["dev_status"].item()) | int(oi["dev_status"].item()),
        })
    if own:
        sr.close()
    return host


def _run_single(inp, rd, device):
    """One readyStateReader call with reader rd's weights and h."""
    from tests.gpu_util import run_reader
    d = to_device(inp, device)
    h, w = _reader_dev(rd, inp.cfg, device)
    d["h"], d["weights"] = h, w
    return run_reader(inp, device, dev_inputs=d)


def _oracle(inp, readers, seqs):
    from oracle import reader as orc
    cfg = inp.cfg
    buf = orc.decode(inp.buf[seqs], cfg.state_dtype)
    hs = [orc.decode(rd["h"][seqs], cfg.act_dtype) for rd in readers]
    ws = [{"Wq": orc.decode(rd["wq"], cfg.weight_dtype), "U": orc.decode(rd["u"], cfg.weight_dtype),
           "V": orc.decode(rd["v"], cfg.weight_dtype), "W1": orc.decode(rd["w1"], cfg.weight_dtype),
           "W2": orc.decode(rd["w2"], cfg.weight_dtype)} for rd in readers]
    for w, rd in zip(ws, readers):
        for k in ("gamma", "b1", "b2"):
            if k in rd:
                w[k] = orc.decode(rd[k], cfg.weight_dtype)
    ref = orc.multi_reader(buf, inp.accept_idx[seqs], list(cfg.slots), cfg.H, hs, ws, act=cfg.act,
                           state_eps=cfg.state_eps, h_eps=cfg.h_eps, shared=cfg.shared)
    out = []
    for i in range(len(readers)):
        r = dict(ref["readers"][i])
        r.update(G=ref["G"], ell=ref["ell"], seqs=list(seqs))
        out.append(r)
    return out


def _check(inp, n_readers, seqs=None, seed=5, extras=False):
    from tests.gpu_util import compare
    dev = _dev()
    cfg = inp.cfg
    seqs = list(range(cfg.B)) if seqs is None else list(seqs)
    _say("multi case", cfg.name, "B", cfg.B, "M", cfg.M, "r", cfg.r, "readers", n_readers, "act", cfg.act,
         "shared", cfg.shared, "extras", extras)
    readers = synth.make_readers(inp, n_readers, seed=seed, extras=extras)
    res = _run_multi(inp, readers, dev)
    refs = _oracle(inp, readers, seqs)
    for i in range(n_readers):
        rep = compare(inp, res[i], refs[i])
        _say("  reader", i, rep)
        assert rep["ok"], (i, rep)
    return readers, res


def test_paper_shape_three_readers():
    _check(synth.make("paper", seed=3), 3)


def test_batched_sample_five_readers():
    # all 64 sequences on the GPU, the oracle on a sample spanning the batch
    _check(synth.make("batched", seed=3), 5, seqs=[0, 17, 40, 63])


@pytest.mark.parametrize("r", [16, 24])
def test_ranks_two_readers(r):
    _check(synth.make("paper", seed=4, r=r, B=3), 2)


def test_several_row_blocks_ragged():
    # 77 rows: the apply launch's query sums in three 32-row tiles (the last
    # one ragged) and its output in two 64-row tiles, against the one-reader
    # launch's 64-row query tiles and 32-row output tiles
    inp = synth.make("paper", seed=17, B=11)
    _check(inp, 2, seqs=[0, 5, 10])


@pytest.mark.parametrize("n_readers", [1, 8])
def test_one_and_the_most_readers(n_readers):
    # a single reader through prepare/apply, and the most readers one prepare serves
    _check(synth.make("paper", seed=16, B=2), n_readers)


def test_gain_biases_and_gelu():
    # every reader with its own RMSNorm gain and MLP biases, GELU (tanh form)
    _check(synth.make("paper", seed=14, B=3, act="gelu_tanh"), 3, extras=True)


def test_shared_reader_parameters_relu():
    # one W_q, U, V per reader shared by all pairs, ReLU
    _check(synth.make("paper", seed=15, B=2, shared=True, act="relu"), 2, extras=True)


def test_rank_32_at_the_paper_pair_count_two_readers():
    # r = 32 with the pages' 32 pairs runs as the single kernel, so its P can
    # be shared: checked against the oracle and against single calls
    dev = _dev()
    inp = synth.make("paper", seed=16, r=32, B=3)
    sr_shape = reader_shape(inp.cfg)
    from hla_recurrent_state_amd import StateReader
    assert StateReader(sr_shape, inp.cfg.slots).prep_size(2) > 0
    readers, res = _check(inp, 2)
    for i, rd in enumerate(readers):
        single = _run_single(inp, rd, dev)
        for key in ("gathered", "logrms", "out", "delta", "feat"):
            assert np.array_equal(res[i][key].view(np.uint8), single[key].view(np.uint8)), (i, key)


def test_rank_40_is_unsupported():
    # r = 40 runs as four kernels, so there is no P to share
    from hla_recurrent_state_amd import READY_ERR_UNSUPPORTED, StateReader, ReadyError
    cfg = synth.make_shape("paper", r=40)
    sr = StateReader(reader_shape(cfg), cfg.slots)
    with pytest.raises(ReadyError) as e:
        sr.prep_size(2)
    assert e.value.code == READY_ERR_UNSUPPORTED


def test_apply_equals_single_reader_bitwise():
    dev = _dev()
    inp = synth.make("paper", seed=6, B=5)
    readers = synth.make_readers(inp, 3, seed=7)
    multi = _run_multi(inp, readers, dev)
    for i, rd in enumerate(readers):
        single = _run_single(inp, rd, dev)
        for key in ("gathered", "logrms", "out", "delta", "feat"):
            assert np.array_equal(multi[i][key].view(np.uint8), single[key].view(np.uint8)), (i, key)
        _say("  reader", i, "bit-identical to the single call")


def test_apply_in_place():
    dev = _dev()
    inp = synth.make("paper", seed=8, B=2)
    readers = synth.make_readers(inp, 2, seed=9)
    a = _run_multi(inp, readers, dev)
    b = _run_multi(inp, readers, dev, inplace=True)
    for i in range(2):
        assert np.array_equal(a[i]["out"], b[i]["out"])


def test_invalid_accept_index_leaves_that_sequence():
    dev = _dev()
    inp = synth.make("paper", seed=10, B=3)
    inp.accept_idx[1] = inp.cfg.P + 2  # out of range: reported, sequence 1 left alone
    readers = synth.make_readers(inp, 2, seed=11)
    res = _run_multi(inp, readers, dev)
    from oracle import reader as orc
    from tests.gpu_util import compare
    refs = _oracle(inp, readers, [0, 2])
    for i in range(2):
        assert res[i]["dev_status"] == 9  # READY_ERR_ACCEPT_IDX
        assert np.all(orc.decode(res[i]["out"][1], inp.cfg.act_dtype) == 7.0)
        assert np.all(res[i]["feat"][1] == 0.0)
        rep = compare(inp, dict(res[i], dev_status=0), refs[i])
        assert rep["ok"], (i, rep)


def test_prepare_then_apply_repeated_calls():
    # the counters in the workspace are left cleared by every launch: a second
    # round of prepare + apply on the same workspace gives the same outputs
    from hla_recurrent_state_amd import StateReader
    from tests.gpu_util import reader_shape
    dev = _dev()
    inp = synth.make("paper", seed=12, B=2)
    readers = synth.make_readers(inp, 3, seed=13)
    sr = StateReader(reader_shape(inp.cfg), inp.cfg.slots)
    a = _run_multi(inp, readers, dev, sr=sr)
    b = _run_multi(inp, readers, dev, sr=sr)
    sr.close()
    for i in range(3):
        for key in ("out", "delta", "feat"):
            assert np.array_equal(a[i][key], b[i][key]), (i, key)


def test_producer_feeds_several_readers():
    # verify-state producer -> prepare -> apply per reader, against the
    # oracle's multi_reader on the produced states
    from tests.gpu_util import compare
    from tests.test_gpu_verify import _bits, _run as run_producer
    dev = _dev()
    cfg = synth.make_shape("paper", B=3, H=4, t=12)
    inp = synth.make(cfg, seed=43)
    vi = synth.make_verify(B=cfg.B, P=cfg.P, L=cfg.L_tot, H=cfg.H, t=12, seed=44)
    buf = run_producer(vi, dev)
    inp.buf = _bits(buf, "bf16").reshape(cfg.B, cfg.P, cfg.L_tot, cfg.H, 128, 128)
    readers = synth.make_readers(inp, 3, seed=45)
    res = _run_multi(inp, readers, dev)
    refs = _oracle(inp, readers, list(range(cfg.B)))
    for i in range(3):
        rep = compare(inp, res[i], refs[i])
        _say("  reader", i, rep)
        assert rep["ok"], (i, rep)
