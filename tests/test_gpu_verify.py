"""GPU parity of the verify-state producer (readyVerifyStates) against the
float64 oracle of the gated delta rule (oracle.gdn.gdn_run).

Position 0 is a bit copy of S_t.  Later positions: fp32 states within a
normwise 1e-5 of the oracle (fp32 arithmetic over at most 63 rank-one updates
of unit-norm keys); bf16 states within one bf16 ulp of the oracle value plus
4e-6 of the state's largest entry (the kernel rounds its fp32 state once, and
that state carries the fp32 chain's error, which matters next to a rounding
boundary or for entries near zero).
"""
import sys

import numpy as np
import pytest

import synth
from synth.gen import decode

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tensor(x, dtype, dev):
    from synth.device import tensor
    return tensor(x, dtype, dev)


def _run(vi, dev, out=None, H=None):
    import hla_recurrent_state_amd as R
    from synth.device import torch_dtype
    st = _tensor(vi.state_t, vi.state_dtype, dev)
    steps = vi.P - 1
    k = _tensor(vi.k, vi.kv_dtype, dev) if steps else None
    v = _tensor(vi.v, vi.kv_dtype, dev) if steps else None
    al = torch.from_numpy(vi.alpha).to(dev) if steps else None
    be = torch.from_numpy(vi.beta).to(dev) if steps else None
    if out is None:
        out = torch.empty((vi.B, vi.P, vi.L, vi.H, 128, 128), dtype=torch_dtype(vi.state_dtype), device=dev)
    R.verify_states(st, k, v, al, be, out, vi.H if H is None else H)
    torch.cuda.synchronize()
    return out


def _bits(t, dtype):
    from synth.device import to_numpy_bits
    return to_numpy_bits(t, dtype)


def _oracle(vi):
    """[B][P][M][128][128] float64 states from the oracle's recurrence."""
    from oracle.gdn import gdn_run
    M = vi.L * vi.H
    s0 = decode(vi.state_t, vi.state_dtype).astype(np.float64)
    ks = decode(vi.k, vi.kv_dtype).astype(np.float64)
    vs = decode(vi.v, vi.kv_dtype).astype(np.float64)
    ref = np.empty((vi.B, vi.P, M, 128, 128))
    for b in range(vi.B):
        for m in range(M):
            seq = gdn_run(s0[b, m], vi.alpha[b, :, m].astype(np.float64), vi.beta[b, :, m].astype(np.float64),
                          [ks[b, p, m] for p in range(vi.P - 1)], [vs[b, p, m] for p in range(vi.P - 1)])
            for p in range(vi.P):
                ref[b, p, m] = seq[p]
    return ref


def _check(vi, got_bits):
    B, P, M = vi.B, vi.P, vi.L * vi.H
    got = got_bits.reshape(B, P, M, 128, 128)
    # position 0: bit copy of S_t
    assert np.array_equal(got[:, 0], vi.state_t), "position 0 is not a bit copy of S_t"
    ref = _oracle(vi)
    g = decode(got, vi.state_dtype).astype(np.float64)
    worst = 0.0
    for p in range(1, P):
        err = np.abs(g[:, p] - ref[:, p])
        if vi.state_dtype == "f32":
            rel = err.max() / np.abs(ref[:, p]).max()
            worst = max(worst, rel)
            assert rel <= 1e-5, (p, rel)
        else:
            # one bf16 ulp of the exact value (8 significant bits), plus the fp32
            # chain's error, which is relative to the state's largest entries
            mag = np.maximum(np.abs(ref[:, p]), 1e-30)
            ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
            allow = ulp + 4e-6 * np.abs(ref[:, p]).max()
            ratio = (err / allow).max()
            worst = max(worst, ratio)
            assert ratio <= 1.0, (p, ratio)
    _say("  worst", worst)


@pytest.mark.parametrize("sdt,kdt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")])
def test_verify_states_parity(sdt, kdt):
    dev = _dev()
    vi = synth.make_verify(B=3, P=8, L=2, H=3, t=16, state_dtype=sdt, kv_dtype=kdt, seed=5)
    _say("case verify", sdt, kdt, "B", vi.B, "P", vi.P, "M", vi.L * vi.H)
    out = _run(vi, dev)
    _check(vi, _bits(out, sdt))


def test_verify_long_block():
    """P = 64 positions (the largest supported block, 63 updates)."""
    dev = _dev()
    vi = synth.make_verify(B=1, P=64, L=1, H=2, t=8, state_dtype="f32", kv_dtype="f32", seed=6)
    _say("case verify long block")
    _check(vi, _bits(_run(vi, dev), "f32"))


def test_verify_single_position_is_a_copy():
    dev = _dev()
    vi = synth.make_verify(B=2, P=1, L=2, H=2, t=8, seed=7)
    _say("case verify P=1")
    out = _run(vi, dev)
    assert np.array_equal(_bits(out, "bf16").reshape(2, 1, 4, 128, 128)[:, 0], vi.state_t)


def test_verify_identity_gates_keep_the_state_bitwise():
    """alpha = 1, beta = 0: every position equals S_t exactly."""
    dev = _dev()
    for sdt in ("bf16", "f32"):
        vi = synth.make_verify(B=2, P=5, L=1, H=3, t=8, state_dtype=sdt, kv_dtype=sdt, seed=8)
        vi.alpha[:] = 1.0
        vi.beta[:] = 0.0
        got = _bits(_run(vi, dev), sdt).reshape(2, 5, 3, 128, 128)
        for p in range(5):
            assert np.array_equal(got[:, p], vi.state_t), (sdt, p)


def test_verify_full_write_stores_the_value():
    """beta = 1: S_{t+p} k_p = v_p (the delta rule overwrites the value at key k_p)."""
    dev = _dev()
    vi = synth.make_verify(B=2, P=4, L=1, H=2, t=8, state_dtype="f32", kv_dtype="f32", seed=9)
    vi.beta[:] = 1.0
    got = _bits(_run(vi, dev), "f32").reshape(2, 4, 2, 128, 128).astype(np.float64)
    for b in range(2):
        for p in range(1, 4):
            for m in range(2):
                sk = got[b, p, m] @ vi.k[b, p - 1, m].astype(np.float64)
                assert np.abs(sk - vi.v[b, p - 1, m]).max() < 1e-4, (b, p, m)


def test_verify_into_strided_buffer_leaves_other_slots():
    """Write layers into slots 1 and 2 of a buffer with 4 layer slots; the
    other slots keep their sentinel bits."""
    dev = _dev()
    vi = synth.make_verify(B=2, P=6, L=2, H=3, t=8, seed=10)
    big = torch.empty((2, 6, 4, 3, 128, 128), dtype=torch.bfloat16, device=dev)
    big.view(torch.int16).fill_(0x7FC1)
    _run(vi, dev, out=big[:, :, 1:3])
    bits = _bits(big, "bf16")
    assert np.all(bits[:, :, 0] == 0x7FC1) and np.all(bits[:, :, 3] == 0x7FC1)
    _check(vi, np.ascontiguousarray(bits[:, :, 1:3]))


def test_producer_feeds_the_reader():
    """The producer's buffer read by the state reader gives the reader's
    oracle result on the oracle-produced states (steps 1-5 downstream of f1)."""
    from tests.gpu_util import compare, oracle_reference, run_reader
    dev = _dev()
    cfg = synth.make_shape("paper", B=3, H=4, t=12)
    inp = synth.make(cfg, seed=41)
    vi = synth.make_verify(B=cfg.B, P=cfg.P, L=cfg.L_tot, H=cfg.H, t=12, seed=42)
    buf = _run(vi, dev)
    inp.buf = _bits(buf, "bf16").reshape(cfg.B, cfg.P, cfg.L_tot, cfg.H, 128, 128)
    res = run_reader(inp, dev)
    rep = compare(inp, res, oracle_reference(inp))
    _say("  report", rep)
    assert rep["ok"], rep
