"""Seeded synthetic inputs at the pages' shapes.

Shapes (ReaDy arXiv text, section 3.1 "Position-conditioned reading" and
section 4.1 "Inference settings"; Appendix D.3 "Hybrid target model"):
128 x 128 value-by-key states, draft width 5120, block of 7 drafts verified
with a root token (8 buffer positions), rank 8, state layers (30, 62) or
(2, 30, 62).  Heads per selected layer are not on the pages; 16 are assumed
(48 for the wide-heads case).  The bottleneck MLP width is not on the pages
either (64 for the tiny case, 256 otherwise).

Value distributions: states come from the fp32 gated delta rule run for t
steps from zero (C generator, gdn_gen.c); h ~ N(0, 1); every weight matrix
~ N(0, 1/fan_in) with fan_in the input width of the map it applies (d for
W_q, r for U since q = U^T z, d_v for V since T = V^T S, F for W1, Hm for W2);
gamma = 1 and no biases unless a test sets them; accept index ~ U{0..P-1}.
bf16 configurations store every value rounded to nearest even from fp32.
"""
import ctypes
import dataclasses
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth.so")
SRC_PATH = os.path.join(HERE, "gdn_gen.c")


@dataclasses.dataclass
class Shape:
    name: str
    B: int
    P: int
    n: int
    layer_ids: tuple          # target layer IDs (labels)
    L_tot: int                # slots on the buffer's layer axis
    slots: tuple              # slot of each selected layer
    H: int
    d_k: int
    d_v: int
    r: int
    d: int
    Hm: int
    t: int
    alpha_lo: float
    state_dtype: str          # "f32" | "bf16"
    act_dtype: str
    weight_dtype: str
    act: str = "silu"
    state_eps: float = 1e-6
    h_eps: float = 1e-6
    shared: bool = False      # one W_q/U/V shared by every pair

    @property
    def L_sel(self):
        return len(self.slots)

    @property
    def M(self):
        return self.L_sel * self.H

    @property
    def F(self):
        return self.M * (self.r + 1)


def _shape(name, **kw):
    base = dict(P=8, n=7, d_k=128, d_v=128, r=8, d=5120, Hm=256, t=4096, alpha_lo=0.9)
    base.update(kw)
    if "slots" not in base:
        base["slots"] = tuple(range(len(base["layer_ids"])))
    if "L_tot" not in base:
        base["L_tot"] = len(base["slots"])
    return Shape(name=name, **base)


CONFIGS = {
    # 1 layer x 2 heads, t = 64, fp32 throughout, MLP 18 -> 64 -> 5120, batch 1
    "tiny": _shape("tiny", B=1, layer_ids=(62,), H=2, t=64, Hm=64,
                   state_dtype="f32", act_dtype="f32", weight_dtype="f32"),
    # layers (30, 62) x 16 heads, bf16, t = 4096, MLP 288 -> 256 -> 5120, batch 1
    "paper": _shape("paper", B=1, layer_ids=(30, 62), H=16,
                    state_dtype="bf16", act_dtype="bf16", weight_dtype="bf16"),
    # 2 layers x 48 heads, fp32 states, t = 16384, alpha ~ U(0.95, 1), batch 1
    "wide": _shape("wide", B=1, layer_ids=(30, 62), H=48, t=16384, alpha_lo=0.95,
                   state_dtype="f32", act_dtype="f32", weight_dtype="f32"),
    # 64 independent sequences of the paper shape
    "batched": _shape("batched", B=64, layer_ids=(30, 62), H=16,
                      state_dtype="bf16", act_dtype="bf16", weight_dtype="bf16"),
    # layers (2, 30, 62) x 16 heads, r = 128, batch 256
    "rank": _shape("rank", B=256, layer_ids=(2, 30, 62), H=16, r=128,
                   state_dtype="bf16", act_dtype="bf16", weight_dtype="bf16"),
}


def make_shape(name="tiny", **overrides):
    """A configuration, optionally with fields replaced (e.g. B, t, r, L_tot, slots)."""
    cfg = CONFIGS[name]
    if not overrides:
        return cfg
    kw = dataclasses.asdict(cfg)
    kw.update(overrides)
    if "slots" in overrides and "layer_ids" not in overrides:
        kw["layer_ids"] = tuple(kw["layer_ids"][i % len(cfg.layer_ids)] for i in range(len(kw["slots"])))
    if "layer_ids" in overrides and "slots" not in overrides:
        kw["slots"] = tuple(range(len(overrides["layer_ids"])))
    if "L_tot" not in overrides:
        kw["L_tot"] = max(kw["L_tot"], max(kw["slots"]) + 1)
    return Shape(**kw)


# ---------------------------------------------------------------- C generator

_lib = None


def build(force=False):
    """Compile the C generator (gcc, OpenMP) next to this file."""
    if os.path.exists(LIB_PATH) and not force:
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-mavx2", "-mfma", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-o", tmp, SRC_PATH, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        lib.synth_philox4x32_10.restype = None
        lib.synth_gdn_states.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_uint64,
            ctypes.c_void_p, ctypes.c_int]
        lib.synth_gdn_states.restype = ctypes.c_int
        lib.synth_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.synth_to_bf16.restype = None
        _lib = lib
    return _lib


def philox4x32_10(ctr, key):
    """Philox4x32-10 of one counter block (exposed for known-answer tests)."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib.synth_philox4x32_10(c, k, o)
    return list(o)


def to_bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_to_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gdn_states(cfg, seed, out=None, alpha_fixed=-1.0, beta_fixed=-1.0, with_coef=False,
               nthreads=0):
    """Fill a [B][P][L_tot][H][d_v][d_k] buffer (fp32, or bf16 bit patterns).

    Only the selected slots are written by the recurrence; the other slots of a
    freshly allocated buffer are filled with N(0, 4) noise so that a read of
    the wrong slot cannot go unnoticed.
    """
    lib = _load()
    dt = np.uint16 if cfg.state_dtype == "bf16" else np.float32
    shape = (cfg.B, cfg.P, cfg.L_tot, cfg.H, cfg.d_v, cfg.d_k)
    if out is None:
        out = np.empty(shape, dtype=dt)
        unselected = [s for s in range(cfg.L_tot) if s not in cfg.slots]
        if unselected:
            rng = np.random.default_rng([seed, 77])
            for s in unselected:
                noise = (2.0 * rng.standard_normal((cfg.B, cfg.P, cfg.H, cfg.d_v, cfg.d_k))).astype(np.float32)
                out[:, :, s] = to_bf16_bits(noise) if dt == np.uint16 else noise
    assert out.shape == shape and out.dtype == dt and out.flags.c_contiguous
    st = [x // out.itemsize for x in out.strides[:4]]
    slots = (ctypes.c_int32 * cfg.L_sel)(*cfg.slots)
    coef = None
    if with_coef:
        steps = cfg.t + cfg.P - 1
        coef = np.zeros((cfg.B * cfg.M, steps, cfg.d_k + cfg.d_v + 2), dtype=np.float32)
    rc = lib.synth_gdn_states(out.ctypes.data, int(dt == np.uint16), st[0], st[1], st[2], st[3],
                              cfg.B, cfg.P, cfg.L_sel, slots, cfg.H, cfg.d_k, cfg.d_v, cfg.t,
                              float(cfg.alpha_lo), float(alpha_fixed), float(beta_fixed),
                              int(seed) & (2 ** 64 - 1),
                              None if coef is None else coef.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError("synth_gdn_states failed")
    return (out, coef) if with_coef else out


# ---------------------------------------------------------------- the rest

@dataclasses.dataclass
class Inputs:
    cfg: Shape
    buf: np.ndarray           # [B][P][L_tot][H][d_v][d_k]  fp32 or bf16 bits
    accept_idx: np.ndarray    # int32 [B]
    h: np.ndarray             # [B][n][d]
    wq: np.ndarray            # [M][r][d] (or [r][d] when shared)
    u: np.ndarray             # [M][r][d_k]
    v: np.ndarray             # [M][d_v][r]
    w1: np.ndarray            # [Hm][F]
    w2: np.ndarray            # [d][Hm]
    gamma: np.ndarray = None  # [d]
    b1: np.ndarray = None     # [Hm]
    b2: np.ndarray = None     # [d]


def _rng(seed, tag):
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([int(seed), tag])))


def _store(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return to_bf16_bits(x) if dtype == "bf16" else x


def make(cfg="tiny", seed=0, states=True, nthreads=0, **overrides):
    """All inputs of one reader call.  `cfg` is a config name or a Shape."""
    if isinstance(cfg, str):
        cfg = make_shape(cfg, **overrides)
    elif overrides:
        raise ValueError("overrides need a config name")
    M, r, d, dk, dv, F, Hm = cfg.M, cfg.r, cfg.d, cfg.d_k, cfg.d_v, cfg.F, cfg.Hm
    buf = gdn_states(cfg, seed, nthreads=nthreads) if states else None
    accept = _rng(seed, 1).integers(0, cfg.P, cfg.B).astype(np.int32)
    h = _rng(seed, 2).standard_normal((cfg.B, cfg.n, d), dtype=np.float32)
    pre = () if cfg.shared else (M,)
    wq = _rng(seed, 3).standard_normal(pre + (r, d), dtype=np.float32) / np.float32(np.sqrt(d))
    u = _rng(seed, 4).standard_normal(pre + (r, dk), dtype=np.float32) / np.float32(np.sqrt(r))
    v = _rng(seed, 5).standard_normal(pre + (dv, r), dtype=np.float32) / np.float32(np.sqrt(dv))
    w1 = _rng(seed, 6).standard_normal((Hm, F), dtype=np.float32) / np.float32(np.sqrt(F))
    w2 = _rng(seed, 7).standard_normal((d, Hm), dtype=np.float32) / np.float32(np.sqrt(Hm))
    wd, ad = cfg.weight_dtype, cfg.act_dtype
    return Inputs(cfg=cfg, buf=buf, accept_idx=accept, h=_store(h, ad), wq=_store(wq, wd),
                  u=_store(u, wd), v=_store(v, wd), w1=_store(w1, wd), w2=_store(w2, wd))


def make_readers(inp, n_readers, seed=0, extras=False):
    """Weights and draft representations of n_readers readers that share the
    committed states of `inp` (one reader per injection site).  Reader 0 is
    inp's own (h, wq, u, v, w1, w2); the others are drawn independently with
    the same distributions.  With extras, every reader also gets a gain
    gamma ~ N(1, 0.1^2) and biases b1, b2 ~ N(0, 0.1^2) (reader 0's drawn
    here too).  Returns a list of dicts of stored arrays."""
    cfg = inp.cfg
    M, r, d, dk, dv, F, Hm = cfg.M, cfg.r, cfg.d, cfg.d_k, cfg.d_v, cfg.F, cfg.Hm
    pre = () if cfg.shared else (M,)
    wd, ad = cfg.weight_dtype, cfg.act_dtype
    out = [dict(h=inp.h, wq=inp.wq, u=inp.u, v=inp.v, w1=inp.w1, w2=inp.w2)]
    for i in range(1, n_readers):
        g = lambda tag: _rng(seed, 100 * i + tag)
        out.append(dict(
            h=_store(g(2).standard_normal((cfg.B, cfg.n, d), dtype=np.float32), ad),
            wq=_store(g(3).standard_normal(pre + (r, d), dtype=np.float32) / np.float32(np.sqrt(d)), wd),
            u=_store(g(4).standard_normal(pre + (r, dk), dtype=np.float32) / np.float32(np.sqrt(r)), wd),
            v=_store(g(5).standard_normal(pre + (dv, r), dtype=np.float32) / np.float32(np.sqrt(dv)), wd),
            w1=_store(g(6).standard_normal((Hm, F), dtype=np.float32) / np.float32(np.sqrt(F)), wd),
            w2=_store(g(7).standard_normal((d, Hm), dtype=np.float32) / np.float32(np.sqrt(Hm)), wd)))
    if extras:
        for i, rd in enumerate(out):
            g = lambda tag: _rng(seed, 100 * i + tag)
            rd["gamma"] = _store(1.0 + 0.1 * g(8).standard_normal(d, dtype=np.float32), wd)
            rd["b1"] = _store(0.1 * g(9).standard_normal(Hm, dtype=np.float32), wd)
            rd["b2"] = _store(0.1 * g(10).standard_normal(d, dtype=np.float32), wd)
    return out


@dataclasses.dataclass
class VerifyInputs:
    """Inputs of one verify-state producer call (stored values)."""
    B: int
    P: int
    L: int
    H: int
    state_dtype: str
    kv_dtype: str
    state_t: np.ndarray   # [B][L*H][128][128] committed states S_t
    k: np.ndarray         # [B][P-1][L*H][128] unit-norm keys of steps 1 .. P-1
    v: np.ndarray         # [B][P-1][L*H][128]
    alpha: np.ndarray     # [B][P-1][L*H] fp32 decay gates
    beta: np.ndarray      # [B][P-1][L*H] fp32 write strengths


def make_verify(B=2, P=8, L=2, H=3, t=16, state_dtype="bf16", kv_dtype="bf16", seed=0, alpha_lo=0.9):
    """Seeded inputs for the verify-state producer: S_t from the fp32 gated
    delta rule run t steps from zero (stored in state_dtype), and the block's
    steps drawn like the rule's own inputs (keys k = g / |g| with g ~ N(0, I),
    values ~ N(0, 1), alpha ~ U(alpha_lo, 1), beta ~ U(0, 1))."""
    cfg = _shape("verify", B=B, P=1, layer_ids=tuple(range(L)), H=H, t=t, alpha_lo=alpha_lo,
                 state_dtype=state_dtype, act_dtype=state_dtype, weight_dtype=state_dtype)
    buf = gdn_states(cfg, seed)                                      # [B][1][L][H][128][128]
    st = np.ascontiguousarray(buf.reshape(B, L * H, 128, 128))
    steps, M = P - 1, L * H
    rng = _rng(seed, 11)
    g = rng.standard_normal((B, steps, M, 128))
    k = (g / np.linalg.norm(g, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, steps, M, 128), dtype=np.float32)
    alpha = rng.uniform(alpha_lo, 1.0, (B, steps, M)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, steps, M)).astype(np.float32)
    return VerifyInputs(B=B, P=P, L=L, H=H, state_dtype=state_dtype, kv_dtype=kv_dtype, state_t=st,
                        k=_store(k, kv_dtype), v=_store(v, kv_dtype), alpha=alpha, beta=beta)


def decode(x, dtype):
    """fp32 view of a stored array (bf16 bit patterns are widened)."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
