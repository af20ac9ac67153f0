"""Tests of the seeded input generator (CPU only).

The generator is pinned to things other than itself: Philox4x32-10's
published known-answer vectors, the float64 oracle recurrence driven by the
very coefficients the generator drew, the Proposition 2 identity relative to
buffer position 0, special gate values, and the oracle's own bf16 rounding.
"""
import numpy as np
import pytest

import synth
from synth.gen import bf16_bits_to_f32, gdn_states, make_shape
from oracle import gdn as ogdn
from oracle import reader as oreader


def test_philox_known_answers():
    """Known-answer vectors of Philox4x32 with 10 rounds, as published with the
    reference implementation of Salmon et al. (SC 2011)."""
    assert synth.philox4x32_10([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert synth.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert synth.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344],
                               [0xA4093822, 0x299F31D0]) == [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def _small(**kw):
    base = dict(B=2, H=3, d_k=8, d_v=6, t=5, r=4, d=16, Hm=8)
    base.update(kw)
    return make_shape("tiny", **base)


def test_deterministic_and_thread_count_independent():
    cfg = _small(B=3, t=20)
    a = gdn_states(cfg, 11, nthreads=1)
    b = gdn_states(cfg, 11, nthreads=4)
    c = gdn_states(cfg, 12, nthreads=4)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_recurrence_matches_float64_oracle():
    """Buffer position p equals the fp64 gated delta rule run from zero with
    the generator's own coefficients, to fp32 accuracy."""
    cfg = _small()
    buf, coef = gdn_states(cfg, 3, with_coef=True)
    dk, dv, t, P = cfg.d_k, cfg.d_v, cfg.t, cfg.P
    for s in range(cfg.B * cfg.M):
        b, l, a = s // cfg.M, (s // cfg.H) % cfg.L_sel, s % cfg.H
        c = coef[s].astype(np.float64)
        ks, vs, al, be = c[:, :dk], c[:, dk:dk + dv], c[:, dk + dv], c[:, dk + dv + 1]
        states = ogdn.gdn_run(np.zeros((dv, dk)), al, be, ks, vs)
        for p in range(P):
            ref = states[t + p]
            got = buf[b, p, cfg.slots[l], a].astype(np.float64)
            assert np.max(np.abs(got - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref))), (s, p)


def test_buffer_positions_satisfy_proposition2():
    """S_{t+p} = S_t P_p + W_p relative to position 0 of the verify buffer."""
    cfg = _small(d_k=16, d_v=16, t=40, B=1)
    buf, coef = gdn_states(cfg, 5, with_coef=True)
    dk, dv, t, P = cfg.d_k, cfg.d_v, cfg.t, cfg.P
    for s in range(cfg.M):
        a = s % cfg.H
        c = coef[s].astype(np.float64)
        tail = slice(t, t + P - 1)                 # coefficients of steps t+1 .. t+P-1
        Ps, Ws = ogdn.unrolled_products(c[tail, dk + dv], c[tail, dk + dv + 1], c[tail, :dk],
                                        c[tail, dk:dk + dv], dv)
        St = buf[0, 0, cfg.slots[s // cfg.H], a].astype(np.float64)
        for p in range(P):
            ref = buf[0, p, cfg.slots[s // cfg.H], a].astype(np.float64)
            err = np.max(np.abs(St @ Ps[p] + Ws[p] - ref)) / np.max(np.abs(ref))
            assert err <= 1e-4, (s, p, err)


def test_coefficient_distributions():
    cfg = _small(B=4, t=200, d_k=32, d_v=32, alpha_lo=0.9)
    _, coef = gdn_states(cfg, 9, with_coef=True)
    dk, dv = cfg.d_k, cfg.d_v
    k, v = coef[..., :dk], coef[..., dk:dk + dv]
    al, be = coef[..., dk + dv], coef[..., dk + dv + 1]
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-5)       # unit keys
    assert abs(v.mean()) < 0.02 and abs(v.var() - 1.0) < 0.03            # v ~ N(0, 1)
    assert al.min() > 0.9 and al.max() < 1.0 and abs(al.mean() - 0.95) < 0.005
    assert be.min() > 0.0 and be.max() < 1.0 and abs(be.mean() - 0.5) < 0.02
    # raw key draws are Gaussian too: their norms^2 average d_k before normalisation
    # (checked through the value stream which uses the same normal generator)
    assert abs(np.mean(v ** 4) - 3.0) < 0.15                            # Gaussian kurtosis


def test_forced_gates():
    cfg = _small(B=1, t=6, d_k=8, d_v=8)
    # beta = 1: the state written at step i maps k_i to v_i exactly (alpha is free)
    buf, coef = gdn_states(cfg, 1, beta_fixed=1.0, with_coef=True)
    dk, dv = cfg.d_k, cfg.d_v
    for s in range(cfg.M):
        for p in range(1, cfg.P):
            i = cfg.t + p                                   # step that produced position p
            k = coef[s, i - 1, :dk].astype(np.float64)
            v = coef[s, i - 1, dk:dk + dv].astype(np.float64)
            S = buf[0, p, cfg.slots[s // cfg.H], s % cfg.H].astype(np.float64)
            assert np.allclose(S @ k, v, atol=1e-5)
    # beta = 0 from the zero state: nothing is ever written
    buf0 = gdn_states(cfg, 1, alpha_fixed=1.0, beta_fixed=0.0)
    assert np.all(buf0[:, :, list(cfg.slots)] == 0.0)


def test_layer_slots_and_noise_in_unselected_slots():
    cfg = make_shape("tiny", B=2, H=2, t=4, L_tot=5, slots=(3, 1), d_k=8, d_v=8)
    buf = gdn_states(cfg, 2)
    assert buf.shape == (2, 8, 5, 2, 8, 8)
    sel = buf[:, :, [3, 1]]
    rest = buf[:, :, [0, 2, 4]]
    assert np.abs(rest).mean() > 1.0                 # N(0, 4) noise
    # the recurrence slots differ per layer (independent streams)
    assert not np.array_equal(sel[:, :, 0], sel[:, :, 1])


def test_bf16_packing_matches_oracle_rounding():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    x = np.concatenate([x, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)])
    bits = synth.gen.to_bf16_bits(x)
    got = bf16_bits_to_f32(bits).astype(np.float64)
    want = oreader.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_states_are_rounded_fp32_states():
    cfg32 = _small(B=1, t=10)
    cfg16 = make_shape("tiny", B=1, H=3, d_k=8, d_v=6, t=10, r=4, d=16, Hm=8, state_dtype="bf16")
    a = gdn_states(cfg32, 8)
    b = gdn_states(cfg16, 8)
    assert b.dtype == np.uint16
    assert np.array_equal(bf16_bits_to_f32(b), bf16_bits_to_f32(synth.gen.to_bf16_bits(a)))


@pytest.mark.parametrize("name", ["tiny", "paper"])
def test_make_shapes_and_scales(name):
    x = synth.make(name, seed=1)
    c = x.cfg
    assert x.buf.shape == (c.B, c.P, c.L_tot, c.H, 128, 128)
    assert x.h.shape == (c.B, c.n, c.d) and x.wq.shape == (c.M, c.r, c.d)
    assert x.u.shape == (c.M, c.r, c.d_k) and x.v.shape == (c.M, c.d_v, c.r)
    assert x.w1.shape == (c.Hm, c.F) and x.w2.shape == (c.d, c.Hm)
    assert x.accept_idx.dtype == np.int32 and np.all((0 <= x.accept_idx) & (x.accept_idx < c.P))
    wq = synth.gen.decode(x.wq, c.weight_dtype)
    assert abs(wq.std() * np.sqrt(c.d) - 1.0) < 0.05                      # N(0, 1/d)
    w2 = synth.gen.decode(x.w2, c.weight_dtype)
    assert abs(w2.std() * np.sqrt(c.Hm) - 1.0) < 0.05


def test_config_shapes_follow_the_pages():
    """Shape constants the pages state (see tests/golden/paper_shapes.txt)."""
    import os
    gold = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "paper_shapes.txt")
    for line in open(path, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=", 1)
            gold[k.strip()] = v.strip()
    p = synth.CONFIGS["paper"]
    assert p.d_k == p.d_v == int(gold["d_k"]) == int(gold["d_v"])
    assert p.r == int(gold["rank"]) and p.d == int(gold["draft_width"])
    assert p.n == int(gold["block"]) and p.P == int(gold["block"]) + 1
    assert tuple(p.layer_ids) == tuple(int(s) for s in gold["state_layers"].split(","))
    assert tuple(synth.CONFIGS["rank"].layer_ids) == tuple(int(s) for s in gold["ablation_layers"].split(","))
    assert synth.CONFIGS["rank"].r == int(gold["full_rank"])
    # every selected layer is a recurrent layer of the 3 GDN : 1 attention pattern
    n_layers, period = int(gold["target_layers"]), int(gold["pattern_period"])
    attn = [i for i in range(n_layers) if i % period == period - 1]
    assert len(attn) == int(gold["full_attention_layers"])
    assert n_layers - len(attn) == int(gold["recurrent_layers"])
    for cfg in synth.CONFIGS.values():
        for lid in cfg.layer_ids:
            assert lid % period != period - 1
