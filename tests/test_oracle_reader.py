"""Pins for the float64 reader oracle (CPU only).

Each test checks the oracle against something other than itself: a value
worked out by hand on a tiny non-symmetric example, a closed form, an
invariant the pages' definitions imply, or a special case that reduces to a
library routine.  The examples are chosen so that a dropped term, a wrong
sign or index, or a transposed operand changes the result.
"""
import math

import numpy as np
import pytest

from oracle import reader as R


# ---------------------------------------------------------------- formats

def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x0000, 0x8000], dtype=np.uint16)
    got = R.decode(bits, "bf16")
    assert got[0] == 1.0
    assert got[1] == -2.0
    assert got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 2.0 ** -133            # smallest subnormal
    assert math.isinf(got[4]) and got[4] > 0
    assert got[5] == 0.0 and got[6] == 0.0 and math.copysign(1.0, got[6]) < 0


def test_round_to_bf16_hand_cases():
    x = np.array([1.0 + 2.0 ** -8,               # tie between 1 and 1+2^-7: even is 1
                  1.0 + 3 * 2.0 ** -8,           # tie between 1+2^-7 and 1+2^-6: even is 1+2^-6
                  1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above the tie: up
                  -(1.0 + 2.0 ** -8 + 2.0 ** -20),
                  3.0,                           # representable
                  (2.0 - 2.0 ** -7) * 2.0 ** 127,        # largest finite
                  (2.0 - 2.0 ** -8) * 2.0 ** 127,        # tie above the largest: to even -> overflow
                  2.0 ** -134,                   # half the smallest subnormal: tie to 0 (even)
                  3 * 2.0 ** -134])              # tie between 1 and 2 subnormal units: to 2
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 3.0,
                     (2.0 - 2.0 ** -7) * 2.0 ** 127, np.inf, 0.0, 2 * 2.0 ** -133])
    got = R.round_to_bf16(x)
    assert np.array_equal(got, want)
    assert np.isnan(R.round_to_bf16(np.array([np.nan])))[0]


def test_round_to_bf16_brute_force_nearest():
    """Against an exhaustive search over every finite bfloat16 value."""
    all_bits = np.arange(0, 0x7F80, dtype=np.uint32)              # +0 .. largest finite
    table = (all_bits << np.uint32(16)).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                        table[rng.integers(1, table.size - 1, 500)] * (1 + 2.0 ** -8)])
    x = x[np.abs(x) < table[-1]]
    a = np.abs(x)
    hi = np.searchsorted(table, a)                               # table[hi-1] < a <= table[hi]
    lo = hi - 1
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (all_bits[hi] % 2 == 0))
    want = np.where(pick_hi, table[hi], table[lo]) * np.sign(x)
    exact = table[np.minimum(hi, table.size - 1)] == a
    want = np.where(exact, x, want)
    assert np.array_equal(R.round_to_bf16(x), want)


# ---------------------------------------------------------------- step 1

def test_gather_selects_accept_position_layer_and_head():
    """Each buffer entry encodes its own (b, p, l, a) so the source of every
    gathered tile can be read back from its values."""
    B, P, L_tot, H, dv, dk = 3, 8, 5, 2, 2, 3
    buf = np.zeros((B, P, L_tot, H, dv, dk))
    for b in range(B):
        for p in range(P):
            for l in range(L_tot):
                for a in range(H):
                    buf[b, p, l, a] = 1000 * b + 100 * p + 10 * l + a + np.arange(dv * dk).reshape(dv, dk) / 100
    accept = np.array([7, 0, 3])
    layer_ids = [4, 1]                      # not sorted, not contiguous
    G = R.gather_committed(buf, accept, layer_ids, H)
    assert G.shape == (B, 4, dv, dk)
    for b in range(B):
        for l, lid in enumerate(layer_ids):
            for a in range(H):
                tag = 1000 * b + 100 * accept[b] + 10 * lid + a
                assert np.array_equal(np.floor(G[b, l * H + a]), np.full((dv, dk), tag))
                assert np.allclose(G[b, l * H + a] - tag, np.arange(dv * dk).reshape(dv, dk) / 100)


# ---------------------------------------------------------------- step 2

def test_prepare_state_hand_example():
    S = np.array([[3.0, 4.0], [0.0, 0.0]])           # mean of squares 25/4, rms 2.5
    S_bar, ell = R.prepare_state(S, 0.0)
    assert np.allclose(S_bar, [[1.2, 1.6], [0.0, 0.0]], rtol=0, atol=1e-15)
    assert ell == pytest.approx(math.log(2.5), rel=1e-15)


def test_prepare_state_eps_and_zero_state():
    S_bar, ell = R.prepare_state(np.zeros((4, 4)), 1e-6)
    assert np.all(S_bar == 0.0)
    assert ell == pytest.approx(0.5 * math.log(1e-6), rel=1e-14)
    S = np.array([[3.0, 4.0], [0.0, 0.0]])
    _, ell = R.prepare_state(S, 0.75)                  # sqrt(25/4 + 3/4) = sqrt(7)
    assert ell == pytest.approx(0.5 * math.log(7.0), rel=1e-14)


def test_prepare_state_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(0)
    S = rng.standard_normal((16, 16)) * 3.7
    S_bar, ell = R.prepare_state(S, 0.0)
    assert np.mean(S_bar ** 2) == pytest.approx(1.0, rel=1e-14)
    for c in (0.01, 2.0, 123.0):
        S_bar_c, ell_c = R.prepare_state(c * S, 0.0)
        assert np.allclose(S_bar_c, S_bar, rtol=1e-13, atol=0)
        assert ell_c == pytest.approx(ell + math.log(c), abs=1e-12)
    S_bar_n, ell_n = R.prepare_state(-2.0 * S, 0.0)    # negative scale flips the sign
    assert np.allclose(S_bar_n, -S_bar, rtol=1e-13, atol=0)
    assert ell_n == pytest.approx(ell + math.log(2.0), abs=1e-12)


# ---------------------------------------------------------------- step 3

def test_project_state_hand_example():
    V = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 0.0]])   # d_v=3, r=2
    S_bar = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])  # d_v=3, d_k=2
    # row i of T is sum_v V[v, i] * S_bar[v, :]
    assert np.array_equal(R.project_state(V, S_bar), [[11.0, 14.0], [3.0, 4.0]])


# ---------------------------------------------------------------- step 4

def test_rmsnorm_hand_example_and_gain():
    out = R.rmsnorm(np.array([3.0, 4.0]), None, 0.0)     # mean square 12.5
    assert np.allclose(out, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    out = R.rmsnorm(np.array([3.0, 4.0]), np.array([2.0, -1.0]), 0.0)
    assert np.allclose(out, [6 / math.sqrt(12.5), -4 / math.sqrt(12.5)], rtol=1e-15)
    assert np.allclose(R.rmsnorm(np.full(10, -7.5), None, 0.0), -np.ones(10), rtol=1e-15)
    out = R.rmsnorm(np.array([1.0, 1.0]), None, 3.0)     # sqrt(1 + 3) = 2
    assert np.allclose(out, [0.5, 0.5], rtol=1e-15)


def test_query_hand_example():
    Wq = np.array([[1.0, 0.0, 2.0], [0.0, 1.0, 0.0]])    # r=2, d=3
    U = np.array([[1.0, 2.0], [0.0, 1.0]])                # r=2, d_k=2
    z, q = R.query(Wq, U, np.array([1.0, 2.0, 3.0]))
    assert np.array_equal(z, [7.0, 2.0])
    assert np.array_equal(q, [7.0, 16.0])                 # q_k = sum_i U[i, k] z_i


def test_readout_hand_example():
    T = np.array([[11.0, 14.0], [3.0, 4.0]])
    u = R.readout(T, np.array([7.0, 16.0]), 2)
    assert np.allclose(u, [301 / math.sqrt(2), 85 / math.sqrt(2)], rtol=1e-15)


def test_special_case_reduces_to_gdn_readout():
    """With r = d_k = d_v = d, W_q = U = V = I and unit gain the reader's
    readout is the textbook raw readout o = S q of the normalised state,
    with q = RMSNorm(h), scaled by 1/sqrt(d_k)."""
    rng = np.random.default_rng(1)
    d = 6
    S = rng.standard_normal((d, d))
    h = rng.standard_normal(d)
    I = np.eye(d)
    S_bar, _ = R.prepare_state(S, 0.0)
    T = R.project_state(I, S_bar)
    _, q = R.query(I, I, R.rmsnorm(h, None, 0.0))
    u = R.readout(T, q, d)
    h_hat = h / np.sqrt(np.mean(h ** 2))
    want = np.matmul(S / np.sqrt(np.mean(S ** 2)), h_hat) / math.sqrt(d)
    assert np.allclose(u, want, rtol=1e-13, atol=1e-14)


def test_readout_linear_in_state():
    rng = np.random.default_rng(2)
    dv, dk, r = 8, 8, 3
    V = rng.standard_normal((dv, r))
    q = rng.standard_normal(dk)
    S1, S2 = rng.standard_normal((dv, dk)), rng.standard_normal((dv, dk))
    a, b = 0.7, -2.5
    lhs = R.readout(R.project_state(V, a * S1 + b * S2), q, dk)
    rhs = a * R.readout(R.project_state(V, S1), q, dk) + b * R.readout(R.project_state(V, S2), q, dk)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- step 5

def test_activation_closed_forms():
    assert R.silu(np.array([0.0]))[0] == 0.0
    assert R.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert R.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-14)
    x = np.linspace(-6, 6, 25)
    assert np.allclose(R.silu(-x), R.silu(x) - x, atol=1e-14)        # x*sig(-x) = x - x*sig(x)
    assert R.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert R.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(R.gelu_tanh(x) - R.gelu_tanh(-x), x, atol=1e-14)   # odd part is x/2
    assert R.gelu_tanh(np.array([1.0]))[0] == pytest.approx(0.8411919906082768, rel=1e-12)
    assert np.array_equal(R.relu(np.array([-2.0, 0.0, 3.0])), [0.0, 0.0, 3.0])


def test_pack_order_is_per_pair_interleaved():
    f = R.pack([np.array([1.0, 2.0]), np.array([3.0, 4.0])], [10.0, 20.0])
    assert np.array_equal(f, [1.0, 2.0, 10.0, 3.0, 4.0, 20.0])


def test_mlp_hand_example():
    W1 = np.array([[1.0, -1.0], [2.0, 0.0]])               # Hm=2, F=2
    W2 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])    # d=3, Hm=2
    f = np.array([3.0, 1.0])
    assert np.array_equal(R.mlp(f, W1, None, W2, None, "relu"), [2.0, 6.0, 8.0])
    assert np.array_equal(R.mlp(f, W1, np.array([-3.0, 0.0]), W2, None, "relu"), [0.0, 6.0, 6.0])
    assert np.array_equal(R.mlp(f, W1, np.array([-3.0, 0.0]), W2, np.ones(3), "relu"), [1.0, 7.0, 7.0])
    # W1 applied as W1 f (a transposed W1 would give [2, -3] before the ReLU)
    assert np.array_equal(R.mlp(np.array([1.0, 1.0]), W1, None, np.eye(2), None, "relu"), [0.0, 2.0])


# ---------------------------------------------------------------- whole path

def _tiny_inputs(seed, B=2, P=8, L_tot=3, H=2, d=16, r=3, Hm=5, n=4, dk=8, shared=False):
    rng = np.random.default_rng(seed)
    layer_ids = [2, 0]
    M = len(layer_ids) * H
    buf = rng.standard_normal((B, P, L_tot, H, dk, dk))
    accept = rng.integers(0, P, B)
    h = rng.standard_normal((B, n, d))
    shp = (lambda *s: s) if shared else (lambda *s: (M,) + s)
    Wq = rng.standard_normal(shp(r, d))
    U = rng.standard_normal(shp(r, dk))
    V = rng.standard_normal(shp(dk, r))
    F = M * (r + 1)
    W1 = rng.standard_normal((Hm, F))
    W2 = rng.standard_normal((d, Hm))
    return dict(buf=buf, accept_idx=accept, layer_ids=layer_ids, H=H, h=h, Wq=Wq, U=U, V=V,
                W1=W1, W2=W2, shared=shared)


def _einsum_reader(buf, accept_idx, layer_ids, H, h, Wq, U, V, W1, W2, shared=False,
                   eps_s=1e-6, eps_h=1e-6):
    """A second, vectorised reading of steps 1-5 (einsum over all pairs)."""
    B, n, d = h.shape
    G = buf[np.arange(B)[:, None, None], accept_idx[:, None, None],
            np.asarray(layer_ids)[None, :, None], np.arange(H)[None, None, :]]
    G = G.reshape(B, len(layer_ids) * H, buf.shape[4], buf.shape[5])
    rms = np.sqrt(np.mean(G ** 2, axis=(2, 3)) + eps_s)
    Sb = G / rms[:, :, None, None]
    if shared:
        T = np.einsum("vi,bmvk->bmik", V, Sb)
    else:
        T = np.einsum("mvi,bmvk->bmik", V, Sb)
    hh = h / np.sqrt(np.mean(h ** 2, axis=2, keepdims=True) + eps_h)
    if shared:
        z = np.einsum("id,bjd->bji", Wq, hh)[:, :, None, :].repeat(G.shape[1], axis=2)
        q = np.einsum("ik,bjmi->bjmk", U, z)
    else:
        z = np.einsum("mid,bjd->bjmi", Wq, hh)
        q = np.einsum("mik,bjmi->bjmk", U, z)
    u = np.einsum("bmik,bjmk->bjmi", T, q) / np.sqrt(buf.shape[5])
    ell = np.log(rms)
    f = np.concatenate([u, np.broadcast_to(ell[:, None, :, None], u.shape[:3] + (1,))], axis=3)
    f = f.reshape(B, n, -1)
    pre = np.einsum("hf,bjf->bjh", W1, f)
    a = pre / (1 + np.exp(-pre))
    dh = np.einsum("dh,bjh->bjd", W2, a)
    return dict(ell=ell, T=T, z=z, q=q, u=u, f=f, dh=dh)


@pytest.mark.parametrize("shared", [False, True])
def test_state_reader_matches_vectorised_reading(shared):
    inp = _tiny_inputs(3, shared=shared)
    got = R.state_reader(**inp)
    want = _einsum_reader(**inp)
    for key in ("ell", "T", "z", "q", "u", "f", "dh"):
        assert np.allclose(got[key], want[key], rtol=1e-12, atol=1e-12), key
    assert np.allclose(got["h_new"], inp["h"] + want["dh"], rtol=1e-12, atol=1e-12)


def test_state_reader_invariants():
    inp = _tiny_inputs(4)
    base = R.state_reader(**inp)
    # scaling every state of the buffer by c > 0 leaves u unchanged and shifts ell by ln c
    scaled = dict(inp, buf=inp["buf"] * 3.0)
    out = R.state_reader(**scaled, state_eps=0.0)
    ref = R.state_reader(**inp, state_eps=0.0)
    assert np.allclose(out["u"], ref["u"], rtol=1e-12, atol=1e-12)
    assert np.allclose(out["ell"], ref["ell"] + math.log(3.0), rtol=0, atol=1e-12)
    # T and ell do not depend on the draft position: duplicated h rows give identical rows
    h = inp["h"].copy()
    h[:, 2] = h[:, 0]
    dup = R.state_reader(**dict(inp, h=h))
    for key in ("u", "f", "dh"):
        assert np.array_equal(dup[key][:, 2], dup[key][:, 0]), key
    n = h.shape[1]
    M = base["ell"].shape[1]
    r = base["u"].shape[3]
    for j in range(n):
        assert np.array_equal(base["f"][:, j].reshape(-1, M, r + 1)[:, :, r], base["ell"])
    # W2 = 0 gives Delta h = 0 and h' = h exactly
    zero = R.state_reader(**dict(inp, W2=np.zeros_like(inp["W2"])))
    assert np.all(zero["dh"] == 0.0) and np.array_equal(zero["h_new"], inp["h"])
    # W1 = 0: Delta h_j = W2 act(b1) + b2 is the same for every j
    b1 = np.linspace(-1, 1, inp["W1"].shape[0])
    w1z = R.state_reader(**dict(inp, W1=np.zeros_like(inp["W1"])), b1=b1)
    want = inp["W2"] @ R.silu(b1)
    for b in range(h.shape[0]):
        for j in range(n):
            assert np.allclose(w1z["dh"][b, j], want, rtol=1e-13, atol=1e-13)


def test_state_reader_seq_subset_leaves_others_nan():
    inp = _tiny_inputs(6, B=3)
    full = R.state_reader(**inp)
    part = R.state_reader(**inp, seqs=[1])
    assert np.array_equal(part["dh"][1], full["dh"][1])
    assert np.all(np.isnan(part["dh"][0])) and np.all(np.isnan(part["dh"][2]))


# ---------------------------------------------------------------- several readers, one gather

def _readers(seed, n_readers, base):
    """Per-reader weights and h of the same shapes as `base` (_tiny_inputs)."""
    rng = np.random.default_rng(seed)
    readers, hs = [], []
    for _ in range(n_readers):
        readers.append({k: rng.standard_normal(base[k].shape) for k in ("Wq", "U", "V", "W1", "W2")})
        hs.append(rng.standard_normal(base["h"].shape))
    return readers, hs


@pytest.mark.parametrize("shared", [False, True])
def test_multi_reader_each_reader_matches_vectorised_reading(shared):
    inp = _tiny_inputs(8, shared=shared)
    readers, hs = _readers(9, 3, inp)
    got = R.multi_reader(inp["buf"], inp["accept_idx"], inp["layer_ids"], inp["H"], hs, readers,
                         shared=shared)
    for i, (w, h) in enumerate(zip(readers, hs)):
        want = _einsum_reader(inp["buf"], inp["accept_idx"], inp["layer_ids"], inp["H"], h, w["Wq"], w["U"],
                              w["V"], w["W1"], w["W2"], shared=shared)
        assert np.allclose(got["ell"], want["ell"], rtol=1e-12, atol=1e-12)
        for key in ("T", "z", "q", "u", "f", "dh"):
            assert np.allclose(got["readers"][i][key], want[key], rtol=1e-12, atol=1e-12), (i, key)
        assert np.allclose(got["readers"][i]["h_new"], h + want["dh"], rtol=1e-12, atol=1e-12)


def test_multi_reader_shares_the_gather_and_orders_readers():
    inp = _tiny_inputs(10)
    readers, hs = _readers(11, 3, inp)
    args = (inp["buf"], inp["accept_idx"], inp["layer_ids"], inp["H"])
    got = R.multi_reader(*args, hs, readers)
    # the gathered states are the brute-force selection of the single reader
    single = R.state_reader(*args, hs[0], readers[0]["Wq"], readers[0]["U"], readers[0]["V"],
                            readers[0]["W1"], readers[0]["W2"])
    assert np.array_equal(got["G"], single["G"])
    assert np.array_equal(got["ell"], single["ell"])
    # every ell column of every reader's f is the shared ell
    M, r = got["ell"].shape[1], got["readers"][0]["u"].shape[3]
    for out in got["readers"]:
        for j in range(hs[0].shape[1]):
            assert np.array_equal(out["f"][:, j].reshape(-1, M, r + 1)[:, :, r], got["ell"])
    # reversing the readers reverses the outputs
    rev = R.multi_reader(*args, hs[::-1], readers[::-1])
    for i in range(3):
        assert np.array_equal(rev["readers"][i]["dh"], got["readers"][2 - i]["dh"])
    # two identical readers on identical h give identical outputs
    twin = R.multi_reader(*args, [hs[0], hs[0]], [readers[0], readers[0]])
    assert np.array_equal(twin["readers"][0]["dh"], twin["readers"][1]["dh"])
