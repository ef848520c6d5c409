"""Float64 CPU oracle for the LaCT chunk-wise SwiGLU fast-weight layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never imports it, and this
module imports nothing from the product.

Source: "Test-Time Training Done Right" (LaCT), as given on the OpenReview
rebuttal page (paperhub.cn, "qae8I9PSoo"), section "Python-style pseudocode"
(functions ``zeropower_via_newtonschulz5``, ``block_causal_lact_swiglu`` and
``bidirectional_lact_swiglu``), and the bud-325 summary page of the same paper
(Key claims: section 3.1 / Fig. 3 orderings, section 3.2 Eq. 6, 8, 9, 10).

Everything is the plain definition, in float64, one (batch, head) at a time:

* fast-weight function  f_W(x) = W2 (silu(W1 x) * (W3 x)), no biases
  (rebuttal page, docstring of the block-causal function; summary page
  section 3.2 Eq. 6).  W1, W3 are [dh, d]; W2 is [d, dh].
* read  (apply):  o_t = f_W(q_t)                      (rebuttal page, apply
  step of both functions).
* write (update): descent direction of the associative loss
  L_j = -sum_t eta_{j,t} <f_W(k_t), v_t>, one eta per matrix j (rebuttal
  page, the gradient block inside the chunk loop of the block-causal
  function; summary page section 3.2 Eq. 4-5).  G_j = -dL_j/dW_j, summed
  over the tokens.
* momentum: beta = mean over the written tokens of the per-token momentum,
  G <- G + beta M, M <- G, M = 0 at sequence start, before Muon
  (rebuttal page, momentum block of the block-causal function).
* Muon: five quintic Newton-Schulz steps with five coefficient triples after
  Frobenius normalisation with eps 1e-7 (rebuttal page,
  ``zeropower_via_newtonschulz5``; summary page section 3.2 Eq. 9-10).  A
  quintic step is an odd matrix polynomial, so it keeps the singular vectors
  and maps each singular value through the scalar quintic; the oracle
  computes exactly that from an SVD.
* step + L2 row renorm: W <- W + G, then each row rescaled to its norm at
  sequence start, with eps 1e-5 added to the current norm (rebuttal page,
  end of the chunk loop; summary page section 3.2 Eq. 8).
* variant "master" (uTTT page section C.1): the steps accumulate into a
  master state S <- S + G that is never rescaled, and the weights that reads
  and gradients use are a fast copy, S with every row rescaled to its
  sequence-start norm after each write (W0 itself before the first write).
* orderings (summary page section 3.1 / Fig. 3; rebuttal page, the two
  functions and the answer on the video experiment).

Readings where the pages are silent or inconsistent are listed in the design doc
("Readings of the pages"); the ones that matter here:

* ``silu_backprop`` is not defined on the page; it is read as the
  derivative of x*sigmoid(x):  sigmoid(x) * (1 + x * (1 - sigmoid(x))).
* The bidirectional function's Muon branch overwrites the weights with the
  orthogonalised update and then adds the raw gradient; it is read as the
  block-causal function's rule  W <- W + NS(G).
* The causal loop writes every chunk that starts before T - C; the segment
  that ends at T is read only.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(finite differences, linearity, the matrix iteration of Newton-Schulz
written in the other Gram orientation, its singular-value band and rank-one
closed form, norm and momentum closed forms, the momentum buffer and the
renorm targets across two writes, brute force, causality invariants).
"""
from __future__ import annotations

import numpy as np

# Newton-Schulz quintic coefficients (a, b, c), one triple per iteration, as
# printed in ``zeropower_via_newtonschulz5`` on the rebuttal page.
NS_COEFFS = (
    (4.0848, -6.8946, 2.9270),
    (3.9505, -6.3029, 2.6377),
    (3.7418, -5.5913, 2.3037),
    (2.8769, -3.1427, 1.2046),
    (2.8366, -3.0525, 1.2012),
)
NS_EPS = 1e-7       # added to the Frobenius norm before dividing
RENORM_EPS = 1e-5   # added to the current row norm before rescaling

ORDER_APPLY_THEN_UPDATE = 0  # causal LM / AR video (shifted block-causal mask)
ORDER_UPDATE_THEN_APPLY = 1  # bidirectional per chunk (NVS: whole sequence)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """silu(x) = x * sigmoid(x)."""
    x = _f64(x)
    return x * sigmoid(x)


def silu_grad(x):
    """d/dx [x sigmoid(x)] = sigmoid(x) (1 + x (1 - sigmoid(x)))."""
    x = _f64(x)
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def row_norms(W):
    """L2 norm of every row of W (the renorm targets are these, taken once)."""
    W = _f64(W)
    return np.sqrt(np.sum(W * W, axis=-1))


# ---------------------------------------------------------------- read ----
def apply(W1, W3, W2, X):
    """Read: rows of X are tokens [n, d]; returns f_W(x_t) for each row [n, d].

    f_W(x) = W2 (silu(W1 x) * (W3 x)).
    """
    W1, W3, W2, X = _f64(W1), _f64(W3), _f64(W2), _f64(X)
    gate = X @ W1.T          # [n, dh]   (W1 x_t)
    up = X @ W3.T            # [n, dh]   (W3 x_t)
    hidden = silu(gate) * up
    return hidden @ W2.T     # [n, d]    (W2 h_t)


# --------------------------------------------------------------- write ----
def chunk_gradient(W1, W3, W2, K, V, eta1, eta3, eta2):
    """Descent directions of the associative loss over the tokens given.

    For L_j = -sum_t eta_{j,t} <f_W(k_t), v_t> this returns G_j = -dL_j/dW_j:

      g_t = W1 k_t, u_t = W3 k_t, e_t = W2^T v_t          (back-prop of <., v>)
      G2  = sum_t eta2_t v_t (silu(g_t) * u_t)^T          [d, dh]
      G3  = sum_t eta3_t (e_t * silu(g_t)) k_t^T          [dh, d]
      G1  = sum_t eta1_t (e_t * u_t * silu'(g_t)) k_t^T   [dh, d]

    Per-channel variant (rebuttal page: the learning-rate tensors of the
    block-causal function are [b, l, d] or [b, l, 1]): eta1, eta3 of shape
    [n, d] scale k_t channel by channel (G1 = sum_t (e u silu') (eta1_t * k_t)^T,
    likewise G3) and eta2 of shape [n, dh] scales the hidden activations
    (G2 = sum_t v_t (eta2_t * h_t)^T), which is where the page multiplies
    them in; with one value per token the two forms coincide.
    """
    W1, W3, W2, K, V = _f64(W1), _f64(W3), _f64(W2), _f64(K), _f64(V)

    def per(eta):
        eta = _f64(eta)
        return eta if eta.ndim == 2 else eta.reshape(-1)[:, None]

    eta1, eta3, eta2 = per(eta1), per(eta3), per(eta2)
    g = K @ W1.T                      # [n, dh]
    u = K @ W3.T                      # [n, dh]
    e = V @ W2                        # [n, dh]  rows are (W2^T v_t)^T
    s = silu(g)
    h = s * u
    d_up = e * s
    d_gate = e * u * silu_grad(g)
    G2 = V.T @ (h * eta2)             # [d, dh]
    G3 = d_up.T @ (K * eta3)          # [dh, d]
    G1 = d_gate.T @ (K * eta1)        # [dh, d]
    return G1, G3, G2


def momentum_step(G, M, beta):
    """G <- G + beta M; the new buffer is the new G (pre-Muon sum)."""
    G = _f64(G) + float(beta) * _f64(M)
    return G, G.copy()


def newton_schulz5(G, eps=NS_EPS, coeffs=NS_COEFFS):
    """Muon orthogonalisation of one matrix.

    The iterate starts at X0 = G / (||G||_F + eps).  One step with
    coefficients (a, b, c) replaces X by a X + b (X X^T) X + c (X X^T)^2 X.
    Writing X = U diag(s) V^T (thin SVD), (X X^T)^k X = U diag(s^(2k+1)) V^T,
    so the step keeps U and V and sends every singular value s to
    a s + b s^3 + c s^5.  Five steps therefore give U diag(phi(s0)) V^T, with
    s0 the singular values of X0 and phi the five scalar quintics applied in
    order.  (The page transposes tall matrices first; that only changes which
    side the Gram matrix is formed on, not the result.)
    """
    G = _f64(G)
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s = S / (np.linalg.norm(G) + eps)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


def step_renorm(W, U, n0, eps=RENORM_EPS):
    """W <- W + U, then every row r <- r / (||r|| + eps) * n0[row]."""
    W = _f64(W) + _f64(U)
    nr = row_norms(W)
    return W / (nr + eps)[:, None] * _f64(n0)[:, None]


# ------------------------------------------------------- one head state ----
RENORM_OFF, RENORM_ROWS, RENORM_MASTER = 0, 1, 2


def renorm_mode(renorm):
    """True / False / "master" (or the mode number) -> RENORM_* mode."""
    if renorm == "master" or renorm == RENORM_MASTER:
        return RENORM_MASTER
    return RENORM_ROWS if renorm else RENORM_OFF


class HeadState:
    """Fast-weight state of one (batch, head): W (the weights reads and
    gradients use), the sequence-start row norms, the momentum buffers (zero
    at sequence start) and, once a "master" write has happened, the master
    state S1, S3, S2 (None before)."""

    def __init__(self, W1, W3, W2):
        self.W1, self.W3, self.W2 = _f64(W1).copy(), _f64(W3).copy(), _f64(W2).copy()
        self.n1, self.n3, self.n2 = row_norms(self.W1), row_norms(self.W3), row_norms(self.W2)
        self.M1 = np.zeros_like(self.W1)
        self.M3 = np.zeros_like(self.W3)
        self.M2 = np.zeros_like(self.W2)
        self.S1 = self.S3 = self.S2 = None

    def copy(self):
        c = HeadState.__new__(HeadState)
        for k, v in self.__dict__.items():
            c.__dict__[k] = None if v is None else v.copy()
        return c


def update(state, K, V, eta1, eta3, eta2, mom=None, use_muon=False,
           use_momentum=False, renorm=True, return_parts=False):
    """One write on the tokens (K, V) given; returns the new state.

    mom: per-token momentum coefficients of the written tokens (their mean is
    beta).  With return_parts the raw gradient, the post-momentum gradient
    and the final step are returned too.
    """
    s = state.copy()
    G1, G3, G2 = chunk_gradient(s.W1, s.W3, s.W2, K, V, eta1, eta3, eta2)
    raw = (G1.copy(), G3.copy(), G2.copy())
    if use_momentum:
        beta = float(np.mean(_f64(mom))) if mom is not None and np.size(mom) else 0.0
        G1, s.M1 = momentum_step(G1, s.M1, beta)
        G3, s.M3 = momentum_step(G3, s.M3, beta)
        G2, s.M2 = momentum_step(G2, s.M2, beta)
    pre_ns = (G1.copy(), G3.copy(), G2.copy())
    if use_muon:
        G1, G3, G2 = newton_schulz5(G1), newton_schulz5(G3), newton_schulz5(G2)
    mode = renorm_mode(renorm)
    if mode == RENORM_MASTER:
        if s.S1 is None:   # the master starts at the weights of the first write
            s.S1, s.S3, s.S2 = s.W1.copy(), s.W3.copy(), s.W2.copy()
        s.S1, s.S3, s.S2 = s.S1 + G1, s.S3 + G3, s.S2 + G2
        zero = np.zeros_like
        s.W1 = step_renorm(s.S1, zero(s.S1), s.n1)
        s.W3 = step_renorm(s.S3, zero(s.S3), s.n3)
        s.W2 = step_renorm(s.S2, zero(s.S2), s.n2)
    elif mode == RENORM_ROWS:
        s.W1 = step_renorm(s.W1, G1, s.n1)
        s.W3 = step_renorm(s.W3, G3, s.n3)
        s.W2 = step_renorm(s.W2, G2, s.n2)
    else:
        s.W1, s.W3, s.W2 = s.W1 + G1, s.W3 + G3, s.W2 + G2
    if return_parts:
        return s, {"raw": raw, "pre_ns": pre_ns, "step": (G1, G3, G2)}
    return s


def chunk_bounds(T, chunk):
    """[(s, e)] chunks of length `chunk`; the last one ends at T (may be short)."""
    if T <= 0:
        return []
    return [(s, min(s + chunk, T)) for s in range(0, T, chunk)]


def sequence(W1, W3, W2, Q, K, V, eta1, eta3, eta2, chunk, mom=None,
             order=ORDER_APPLY_THEN_UPDATE, subset=None, update_last=False,
             use_muon=False, use_momentum=False, renorm=True, state=None,
             return_states=False):
    """Whole-sequence layer for one (batch, head).

    Q, K, V: [T, d]; eta*, mom: [T].  subset = (offset, length) of the
    written tokens inside every chunk (None = the whole chunk).

    * apply-then-update: chunk c is read with W_c, then written -> W_{c+1};
      the chunk that ends at T is read only unless update_last.
    * update-then-apply: chunk c is written first, then read with the result.
    Returns O [T, d] and the final state (and the per-chunk states W_c).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    T = Q.shape[0]
    st = HeadState(W1, W3, W2) if state is None else state.copy()
    O = np.zeros((T, W2.shape[0]), dtype=np.float64)
    states = []
    bounds = chunk_bounds(T, chunk)

    def write(s, e):
        if subset is not None:
            a, b = s + subset[0], min(s + subset[0] + subset[1], e)
        else:
            a, b = s, e
        if b <= a:
            return st
        m = None if mom is None else _f64(mom)[a:b]
        return update(st, K[a:b], V[a:b], _f64(eta1)[a:b], _f64(eta3)[a:b],
                      _f64(eta2)[a:b], mom=m, use_muon=use_muon,
                      use_momentum=use_momentum, renorm=renorm)

    for ci, (s, e) in enumerate(bounds):
        last = ci == len(bounds) - 1
        states.append(st.copy())
        if order == ORDER_APPLY_THEN_UPDATE:
            O[s:e] = apply(st.W1, st.W3, st.W2, Q[s:e])
            if not last or update_last:
                st = write(s, e)
        elif order == ORDER_UPDATE_THEN_APPLY:
            st = write(s, e)
            O[s:e] = apply(st.W1, st.W3, st.W2, Q[s:e])
        else:
            raise ValueError("unknown order")
    if return_states:
        return O, st, states
    return O, st



# ------------------------------------------- linear fast-weight variant ----
# The rebuttal page compares fast-weight networks (Fig. 8(a)); the simplest
# is linear, f_W(x) = W x with one d x d matrix per head.  Its associative
# loss L = -sum_t eta_t <W k_t, v_t> has the descent direction
# G = sum_t eta_t v_t k_t^T, which does not depend on W; momentum, Muon, the
# step and the row renorm are those of the SwiGLU layer.

def linear_apply(W, X):
    """Read of the linear variant: rows of X are tokens; returns W x_t."""
    return _f64(X) @ _f64(W).T


def linear_gradient(K, V, eta):
    """G = sum_t eta_t v_t k_t^T  [d, d]."""
    K, V = _f64(K), _f64(V)
    return (V * _f64(eta).reshape(-1)[:, None]).T @ K


def linear_sequence(W, Q, K, V, eta, chunk, mom=None, order=ORDER_APPLY_THEN_UPDATE,
                    subset=None, update_last=False, use_muon=False, use_momentum=False,
                    renorm=True):
    """Whole sequence of the linear variant for one head, with the orderings
    and renorm modes of ``sequence``.  Returns O [T, d] and the final
    (W, M) - W being the master state in the "master" mode."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    W = _f64(W).copy()
    n0 = row_norms(W)
    M = np.zeros_like(W)
    mode = renorm_mode(renorm)
    S = W.copy()   # the master state of the "master" mode
    T = Q.shape[0]
    O = np.zeros((T, W.shape[0]))
    bounds = chunk_bounds(T, chunk)
    for ci, (s, e) in enumerate(bounds):
        last = ci == len(bounds) - 1
        a, b = (s, e) if subset is None else (s + subset[0], min(s + subset[0] + subset[1], e))
        writes = (order == ORDER_UPDATE_THEN_APPLY or not last or update_last) and b > a
        if order == ORDER_APPLY_THEN_UPDATE:
            O[s:e] = linear_apply(W, Q[s:e])
        if writes:
            G = linear_gradient(K[a:b], V[a:b], _f64(eta)[a:b])
            if use_momentum:
                beta = float(np.mean(_f64(mom)[a:b]))
                G, M = momentum_step(G, M, beta)
            if use_muon:
                G = newton_schulz5(G)
            if mode == RENORM_MASTER:
                S = S + G
                W = step_renorm(S, np.zeros_like(S), n0)
            elif mode == RENORM_ROWS:
                W = step_renorm(W, G, n0)
            else:
                W = W + G
        if order == ORDER_UPDATE_THEN_APPLY:
            O[s:e] = linear_apply(W, Q[s:e])
    return O, (S if mode == RENORM_MASTER else W, M)
