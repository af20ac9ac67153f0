"""Float64 oracle of the ReaDy state reader, steps 1-5, written from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function works in
numpy float64 on exact (decoded) input values, in the order the pages give,
with no blocking, fusion or reordering.  Loops over sequences and
layer-head pairs are plain Python loops so each line can be checked against
the definitions by eye.

Readings of points the pages leave open are marked "Reading:" below.

Parity pins: every function here is pinned by a test in
tests/test_oracle_reader.py against closed forms, invariants or special cases
that reduce to a textbook routine.  The numeric values of the complete Delta-h
at the benchmark shapes have no printed worked example on the pages; beyond
those pins they are "parity unpinned" (the pages print no test vector).
"""
import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats.  The GPU path stores states/activations/weights either as
# IEEE float32 or as bfloat16 (the upper 16 bits of a float32).  The oracle
# decodes them exactly to float64 and never rounds in between (the pages fix
# no intermediate precision; fp64 is the reference).
# ---------------------------------------------------------------------------


def decode(x, dtype):
    """Exact float64 value of a stored array.

    dtype "f32": x holds float32 values.
    dtype "bf16": x holds the raw 16-bit patterns (uint16); a bfloat16 value
    is the float32 whose upper half is those bits and whose lower half is 0.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError("unknown dtype %r" % (dtype,))


def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Written from the definition of round-to-nearest-even on an 8-bit
    significand: for a finite nonzero x with binary exponent e (so that
    2**e <= |x| < 2**(e+1)), representable neighbours are spaced
    2**(e-7) apart; pick the nearer one, and on an exact tie the one whose
    last significand bit is 0.  Values beyond the largest finite bfloat16
    (rounding up past it) become infinity; NaN stays NaN.  Subnormal bfloat16
    values use the fixed spacing 2**-133.  Returns float64 values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()                              # NaN, +-inf and zeros pass through
    a = np.abs(x)
    ok = np.isfinite(x) & (x != 0.0)
    _, e2 = np.frexp(np.where(ok, a, 1.0))      # a = m * 2**e2, 0.5 <= m < 1
    e = np.maximum(e2 - 1, -126)                # 2**e <= a < 2**(e+1); fixed below normal range
    spacing = np.ldexp(1.0, e - 7)
    qv = np.where(ok, a, 0.0) / spacing         # exact: spacing is a power of two
    lo = np.floor(qv)
    frac = qv - lo
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(lo, 2.0) == 1.0))
    r = (lo + up) * spacing
    max_finite = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(r > max_finite, np.inf, r)
    out[ok] = np.copysign(r, x)[ok]
    return out


# ---------------------------------------------------------------------------
# Step 1: gather the committed state of each selected (layer, head) at the
# sequence's accept index.
# arXiv text, section 3.1 "Drafting, verification, and commitment" (only
# states of committed tokens are kept) and section 3.2 "Avoiding redundant
# data movement" (a gather writes the selected committed states into a
# preallocated buffer); rainbus summary, 方法步骤详情, step (4).
# Reading: position p of the verify buffer holds the state after the root and
# p accepted drafts; accept index a selects position a directly.  Pairs are
# ordered layer-major in the order of layer_ids, then by head: m = l*H + a.
# ---------------------------------------------------------------------------


def gather_committed(buf, accept_idx, layer_ids, H):
    """buf: float64 [B][P][L_tot][H][d_v][d_k]; returns G [B][M][d_v][d_k]."""
    B = buf.shape[0]
    M = len(layer_ids) * H
    G = np.empty((B, M) + buf.shape[4:], dtype=np.float64)
    for b in range(B):
        p = int(accept_idx[b])
        for l, lid in enumerate(layer_ids):
            for a in range(H):
                G[b, l * H + a] = buf[b, p, lid, a]
    return G


# ---------------------------------------------------------------------------
# Step 2: state preparation -- RMS normalisation and the log-RMS scale.
# arXiv text, section 3.1 "Position-conditioned reading" (S-bar is an
# RMS-normalised state) and "Fusion and residual injection" (log-RMS state
# scales keep the magnitude removed by normalisation); rainbus summary,
# 方法步骤详情, step (1).
# Reading: one RMS per d_v x d_k matrix over all its entries, no learnable
# gain, rms = sqrt(mean(S^2) + eps); the log is the natural log of rms.
# ---------------------------------------------------------------------------


def prepare_state(S, eps):
    """S: one d_v x d_k state.  Returns (S_bar, ell) with ell = ln(rms)."""
    ms = float(np.sum(S * S)) / S.size
    rms = math.sqrt(ms + eps)
    return S / rms, math.log(rms)


# ---------------------------------------------------------------------------
# Step 3: the shared low-rank projection T = V^T S_bar (r x d_k), formed once
# per state and shared by every draft position of the block.
# arXiv text, section 3.1 "Position-conditioned reading" (V in R^{d_v x r}
# compresses the value dimension, giving T in R^{r x d_k}) and section 3.2
# "State-access footprint" (T is independent of the draft position);
# rainbus summary, 方法步骤详情, step (2).
# ---------------------------------------------------------------------------


def project_state(V, S_bar):
    """V: [d_v][r]; S_bar: [d_v][d_k].  Returns T = V^T S_bar, [r][d_k]."""
    return V.T @ S_bar


# ---------------------------------------------------------------------------
# Step 4: per-position query and readout.
# z_j = W_q RMSNorm(h_j), q_j = U^T z_j, u_j = T q_j / sqrt(d_k).
# arXiv text, section 3.1 "Position-conditioned reading" (W_q in R^{r x d},
# U in R^{r x d_k}; the Eq. (3) display is lost in extraction); rainbus
# summary, 方法步骤详情, step (2), which writes the four formulas out;
# onedev summary, 어떻게 동작하나.
# Reading: RMSNorm(h) = gamma * h / sqrt(mean(h^2) + eps) over the d entries
# of one position, gamma defaulting to ones; it is applied although h is
# already post-norm, as written.  The scale is 1/sqrt(d_k), not 1/sqrt(r).
# ---------------------------------------------------------------------------


def rmsnorm(h_j, gamma, eps):
    """h_j: [d].  gamma: [d] or None (ones)."""
    ms = float(np.sum(h_j * h_j)) / h_j.size
    out = h_j / math.sqrt(ms + eps)
    if gamma is not None:
        out = gamma * out
    return out


def query(Wq, U, h_hat_j):
    """Wq: [r][d], U: [r][d_k], h_hat_j: [d].  Returns (z_j [r], q_j [d_k])."""
    z = Wq @ h_hat_j
    q = U.T @ z
    return z, q


def readout(T, q_j, d_k):
    """u_j = T q_j / sqrt(d_k), [r]."""
    return (T @ q_j) / math.sqrt(d_k)


# ---------------------------------------------------------------------------
# Step 5: packing, bottleneck MLP and residual.
# arXiv text, section 3.1 "Fusion and residual injection" (readouts of the
# selected layers and heads are concatenated with their log-RMS scales to
# form f_j; a bottleneck maps it back to the draft width; the Eq. (4) display
# is lost); rainbus summary, 方法步骤详情, step (3) (h'_j = h_j + Delta h_j).
# Reading: f_j = [u^0, ell_0, u^1, ell_1, ...] per pair in pair order;
# Delta h = W2 act(W1 f + b1) + b2 with act = SiLU unless chosen otherwise;
# the sum h + Delta h is exact here and is rounded to the activation dtype
# only by the caller (round_to_bf16 for bf16 activations).
# ---------------------------------------------------------------------------


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x ** 3)))


def relu(x):
    return np.maximum(x, 0.0)


ACTIVATIONS = {"silu": silu, "gelu_tanh": gelu_tanh, "relu": relu}


def pack(u_pairs, ell_pairs):
    """u_pairs: list over pairs of [r]; ell_pairs: list of scalars -> f [M(r+1)]."""
    parts = []
    for u, ell in zip(u_pairs, ell_pairs):
        parts.append(np.asarray(u, dtype=np.float64))
        parts.append(np.array([ell], dtype=np.float64))
    return np.concatenate(parts)


def mlp(f_j, W1, b1, W2, b2, act):
    """Delta h_j = W2 act(W1 f_j + b1) + b2.  W1: [Hm][F]; W2: [d][Hm]."""
    pre = W1 @ f_j
    if b1 is not None:
        pre = pre + b1
    a = ACTIVATIONS[act](pre)
    dh = W2 @ a
    if b2 is not None:
        dh = dh + b2
    return dh


# ---------------------------------------------------------------------------
# The whole path.
# ---------------------------------------------------------------------------


def pair_params(P, m, shared):
    """Reader parameters of pair m: stacked per pair unless shared."""
    return P if shared else P[m]


def state_reader(buf, accept_idx, layer_ids, H, h, Wq, U, V, W1, W2,
                 gamma=None, b1=None, b2=None, act="silu",
                 state_eps=1e-6, h_eps=1e-6, shared=False, seqs=None):
    """Run steps 1-5 in float64 on decoded inputs.

    buf [B][P][L_tot][H][d_v][d_k]; accept_idx [B]; h [B][n][d];
    Wq [M][r][d], U [M][r][d_k], V [M][d_v][r] (or unstacked when shared);
    W1 [Hm][F]; W2 [d][Hm].  `seqs` optionally restricts the work to a list
    of sequence indices (outputs of the others are left as NaN).

    Returns a dict with gathered G, ell [B][M], T [B][M][r][d_k],
    z [B][n][M][r], q [B][n][M][d_k], u [B][n][M][r], f [B][n][F],
    dh [B][n][d], h_new = h + dh [B][n][d] (exact, unrounded).
    """
    B, n, d = h.shape
    M = len(layer_ids) * H
    d_v, d_k = buf.shape[4], buf.shape[5]
    r = (Wq.shape[0] if shared else Wq.shape[1])
    F = M * (r + 1)
    if seqs is None:
        seqs = range(B)
    nan = np.nan
    G = np.full((B, M, d_v, d_k), nan)
    ell = np.full((B, M), nan)
    T = np.full((B, M, r, d_k), nan)
    z = np.full((B, n, M, r), nan)
    q = np.full((B, n, M, d_k), nan)
    u = np.full((B, n, M, r), nan)
    f = np.full((B, n, F), nan)
    dh = np.full((B, n, d), nan)
    for b in seqs:
        Gb = gather_committed(buf[b:b + 1], accept_idx[b:b + 1], layer_ids, H)[0]
        G[b] = Gb
        for m in range(M):
            S_bar, ell[b, m] = prepare_state(Gb[m], state_eps)
            T[b, m] = project_state(pair_params(V, m, shared), S_bar)
        for j in range(n):
            h_hat = rmsnorm(h[b, j], gamma, h_eps)
            for m in range(M):
                z[b, j, m], q[b, j, m] = query(pair_params(Wq, m, shared),
                                               pair_params(U, m, shared), h_hat)
                u[b, j, m] = readout(T[b, m], q[b, j, m], d_k)
            f[b, j] = pack([u[b, j, m] for m in range(M)], [ell[b, m] for m in range(M)])
            dh[b, j] = mlp(f[b, j], W1, b1, W2, b2, act)
    return {"G": G, "ell": ell, "T": T, "z": z, "q": q, "u": u, "f": f,
            "dh": dh, "h_new": h + dh}


# ---------------------------------------------------------------------------
# Several readers sharing one gather.
# arXiv text, section 4, "Number of injections" and Table 5: the drafter may
# carry readers in its draft layers (0, 2, 4) or in all five instead of only
# in the final one.
# Reading: every reader is a complete reader (steps 3-5) with its own W_q, U,
# V, gain, W1, b1, W2, b2, fed with the draft representations h of its own
# layer; steps 1-2 (the committed states, S_bar and ell) depend only on the
# target's states and are the same for all of them, so they are done once.
# ---------------------------------------------------------------------------


def multi_reader(buf, accept_idx, layer_ids, H, hs, readers, act="silu",
                 state_eps=1e-6, h_eps=1e-6, shared=False, seqs=None):
    """Run steps 1-2 once and steps 3-5 for each reader, float64.

    hs: list over readers of h [B][n][d] (each reader's own injection site).
    readers: list of dicts with Wq, U, V, W1, W2 and optionally gamma, b1, b2
    (layouts as in state_reader).
    Returns {"G": gathered, "ell": [B][M], "readers": [per-reader dicts with
    T, z, q, u, f, dh, h_new as in state_reader]}.
    """
    B = hs[0].shape[0]
    M = len(layer_ids) * H
    d_v, d_k = buf.shape[4], buf.shape[5]
    if seqs is None:
        seqs = range(B)
    G = np.full((B, M, d_v, d_k), np.nan)
    S_bar = np.full((B, M, d_v, d_k), np.nan)
    ell = np.full((B, M), np.nan)
    # steps 1-2, once
    for b in seqs:
        G[b] = gather_committed(buf[b:b + 1], accept_idx[b:b + 1], layer_ids, H)[0]
        for m in range(M):
            S_bar[b, m], ell[b, m] = prepare_state(G[b, m], state_eps)
    # steps 3-5, per reader
    outs = []
    for h, w in zip(hs, readers):
        n, d = h.shape[1], h.shape[2]
        Wq, U, V = w["Wq"], w["U"], w["V"]
        r = Wq.shape[0] if shared else Wq.shape[1]
        F = M * (r + 1)
        T = np.full((B, M, r, d_k), np.nan)
        z = np.full((B, n, M, r), np.nan)
        q = np.full((B, n, M, d_k), np.nan)
        u = np.full((B, n, M, r), np.nan)
        f = np.full((B, n, F), np.nan)
        dh = np.full((B, n, d), np.nan)
        for b in seqs:
            for m in range(M):
                T[b, m] = project_state(pair_params(V, m, shared), S_bar[b, m])
            for j in range(n):
                h_hat = rmsnorm(h[b, j], w.get("gamma"), h_eps)
                for m in range(M):
                    z[b, j, m], q[b, j, m] = query(pair_params(Wq, m, shared),
                                                   pair_params(U, m, shared), h_hat)
                    u[b, j, m] = readout(T[b, m], q[b, j, m], d_k)
                f[b, j] = pack([u[b, j, m] for m in range(M)], [ell[b, m] for m in range(M)])
                dh[b, j] = mlp(f[b, j], w["W1"], w.get("b1"), w["W2"], w.get("b2"), act)
        outs.append({"T": T, "z": z, "q": q, "u": u, "f": f, "dh": dh, "h_new": h + dh})
    return {"G": G, "ell": ell, "readers": outs}
