"""Float64 oracle of the Gated DeltaNet algebra the reader rests on.

TEST INFRASTRUCTURE ONLY (see the package docstring).

  * gdn_step / gdn_run -- the gated delta rule S_i = S_{i-1} A_i + B_i with
    A_i = alpha_i (I - beta_i k_i k_i^T) and B_i = beta_i v_i k_i^T.
    arXiv text, Appendix D.1 (Eqs. D.2-D.3: decay gate alpha, write strength
    beta, normalised keys, zero initial state) and Appendix A.2 (the
    coefficients); rainbus summary, 前置知识 "Gated DeltaNet 循环状态".
  * unrolled_products -- P_j = A_{t+1} ... A_{t+j} and the accumulated writes
    W_j of Proposition 2 (arXiv text, Appendix A.2 and section 2
    "Revisiting the committed state", Eq. (2)).
    Reading: the display defining W_j is lost in extraction; the plainest
    reading consistent with S_{t+j} = S_t P_j + W_j and "an empty product is
    the identity" is W_j = sum_{i=1..j} B_{t+i} A_{t+i+1} ... A_{t+j},
    equivalently W_{j+1} = W_j A_{t+j+1} + B_{t+j+1}, W_0 = 0.
  * query_span_split -- Proposition 1's split
    S q* = (S Q) Q^+ q* + S (I - Pi_Q) q*, Pi_Q = Q Q^+ (arXiv text,
    section 2 "Query-dependent context", Appendix A.1; the Eq. (1) display
    is lost, the split is written out in the rainbus summary, 前置知识
    "查询空间投影").
  * footprint -- state elements M d_v d_k against token-wise KV elements
    M t (d_k + d_v) (arXiv text, section 3.2 "State-access footprint";
    onedev summary, 무엇과 다른가).

Parity pins: tests/test_oracle_gdn.py (induction identity on tiny inputs,
special gates, the constructive counter-example of the Proposition 1 proof,
closed-form counts).
"""
import numpy as np


def transition(alpha, beta, k):
    """A_i = alpha (I - beta k k^T)  (d_k x d_k)."""
    d_k = k.shape[0]
    return alpha * (np.eye(d_k) - beta * np.outer(k, k))


def write(beta, v, k):
    """B_i = beta v k^T  (d_v x d_k)."""
    return beta * np.outer(v, k)


def gdn_step(S, alpha, beta, k, v):
    """One update of the gated delta rule in product form S A + B."""
    return S @ transition(alpha, beta, k) + write(beta, v, k)


def gdn_run(S0, alphas, betas, ks, vs):
    """Apply the rule for i = 1..len(alphas); returns the list [S_0, S_1, ...]."""
    out = [np.array(S0, dtype=np.float64)]
    for a, b, k, v in zip(alphas, betas, ks, vs):
        out.append(gdn_step(out[-1], a, b, k, v))
    return out


def readout(S, q):
    """Raw attention readout o = S q."""
    return S @ q


def unrolled_products(alphas, betas, ks, vs, d_v):
    """P_j and W_j for j = 0..J of the continuation whose coefficients are given
    (index 0 of each list is step t+1).  Returns lists Ps, Ws of length J+1."""
    d_k = ks[0].shape[0] if len(ks) else 0
    Ps = [np.eye(d_k)]
    Ws = [np.zeros((d_v, d_k))]
    for a, b, k, v in zip(alphas, betas, ks, vs):
        A = transition(a, b, k)
        Ps.append(Ps[-1] @ A)
        Ws.append(Ws[-1] @ A + write(b, v, k))
    return Ps, Ws


def pinv(Q):
    """Moore-Penrose pseudoinverse (library routine, via SVD)."""
    return np.linalg.pinv(Q)


def query_span_split(S, Q, q_star):
    """Return (in_span_term, out_of_span_term) of S q* for known queries Q."""
    Qp = pinv(Q)
    Pi = Q @ Qp
    first = (S @ Q) @ (Qp @ q_star)
    second = S @ ((np.eye(Q.shape[0]) - Pi) @ q_star)
    return first, second


def footprint(M, t, d_k, d_v):
    """(state elements, token-wise KV elements) for M layer-head pairs."""
    return M * d_v * d_k, M * t * (d_k + d_v)
