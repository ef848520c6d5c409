"""Float64 CPU oracle of the outer-loop backward of the LaCT fast-weight layer.

TEST INFRASTRUCTURE ONLY, like lact_oracle.py: only ``tests/`` (and the
smoke / cpu_baseline legs) may import it; it imports nothing from the product.

The layer's outputs O depend on q, k, v, the learning rates eta, the momentum
coefficients and the initial weights W0 through the chunk recurrence: every
write changes the weights that later chunks read.  A model that trains the
layer's inputs by gradient descent (how LaCT is trained; the uTTT page,
section 2, notes that the task-loss gradients flow back through the earlier
writes) needs the vector-Jacobian product of the whole sequence: given dO,
the gradients of <O, dO> with respect to all of those inputs.

This module computes that product by the chain rule, written out step by
step in reverse order of the forward computation of ``lact_oracle.sequence``
(one (batch, head) at a time, float64):

* read      O = W2 (silu(W1 q) * (W3 q))
* write     G = chunk gradient of -sum eta <f_W(k), v> (its derivative needs
            the second derivative of silu)
* momentum  G~ = G + beta M, M <- G~, beta = mean of the chunk's coefficients
* Muon      U = NS(G~): the five quintic steps X <- a X + b (X X^T) X +
            c (X X^T)^2 X after X0 = G~ / (||G~||_F + 1e-7), on the wide
            orientation, differentiated as matrix products
* step      W <- (W + U) row by row rescaled to n0 / (||row|| + 1e-5), with
            n0 the row norms of W0 (so W0 also receives gradient through n0)

Every forward state is kept (the oracle is for small cases), then the chunks
are walked backwards.  The forward formulas and readings are those of
lact_oracle.py (rebuttal page pseudocode; summary page section 3.1-3.2).

Parity status: pinned by tests/test_backward_pins.py - central finite
differences of the oracle's own forward sequence along random directions of
every input, and torch.autograd in float64 on an independent torch version
of the forward.
"""
from __future__ import annotations

import numpy as np

from oracle import lact_oracle as F

NS_EPS = F.NS_EPS
RENORM_EPS = F.RENORM_EPS


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def silu_grad2(x):
    """d^2/dx^2 [x sigmoid(x)] = s (1 - s) (2 + x (1 - 2 s)), s = sigmoid(x)."""
    s = F.sigmoid(x)
    return s * (1.0 - s) * (2.0 + x * (1.0 - 2.0 * s))


# ---------------------------------------------------------------- read ----
def apply_vjp(W1, W3, W2, X, dO):
    """Cotangents of the read O = W2 (silu(W1 x) * (W3 x)) for the rows x of
    X: returns dX, dW1, dW3, dW2."""
    W1, W3, W2, X, dO = map(_f64, (W1, W3, W2, X, dO))
    g = X @ W1.T
    u = X @ W3.T
    s = F.silu(g)
    h = s * u
    dW2 = dO.T @ h                       # O = h W2^T
    dh = dO @ W2
    du = dh * s
    dg = dh * u * F.silu_grad(g)
    dW1 = dg.T @ X
    dW3 = du.T @ X
    dX = dg @ W1 + du @ W3
    return dX, dW1, dW3, dW2


# ------------------------------------------------------- chunk gradient ----
def chunk_gradient_vjp(W1, W3, W2, K, V, eta1, eta3, eta2, dG1, dG3, dG2):
    """Cotangents of (G1, G3, G2) = lact_oracle.chunk_gradient(...): returns
    dW1, dW3, dW2, dK, dV, deta1, deta3, deta2."""
    W1, W3, W2, K, V = map(_f64, (W1, W3, W2, K, V))
    dG1, dG3, dG2 = map(_f64, (dG1, dG3, dG2))
    e1, e3, e2 = (_f64(x).reshape(-1) for x in (eta1, eta3, eta2))
    g = K @ W1.T
    u = K @ W3.T
    e = V @ W2
    s = F.silu(g)
    s1 = F.silu_grad(g)
    h = s * u                 # G2 = V^T (e2 h)
    a = e * s                 # G3 = (e3 a)^T K
    b = e * u * s1            # G1 = (e1 b)^T K
    # G2 = sum_t e2_t v_t h_t^T
    dV = e2[:, None] * (h @ dG2.T)
    dh = e2[:, None] * (V @ dG2)
    de2 = np.einsum("ti,ij,tj->t", V, dG2, h)
    # G3 = sum_t e3_t a_t k_t^T
    da = e3[:, None] * (K @ dG3.T)
    dK = e3[:, None] * (a @ dG3)
    de3 = np.einsum("tj,ji,ti->t", a, dG3, K)
    # G1 = sum_t e1_t b_t k_t^T
    db = e1[:, None] * (K @ dG1.T)
    dK = dK + e1[:, None] * (b @ dG1)
    de1 = np.einsum("tj,ji,ti->t", b, dG1, K)
    # elementwise: h = s u, a = e s, b = e u s'(g), s = silu(g)
    ds = dh * u + da * e
    du = dh * s + db * e * s1
    dE = da * s + db * u * s1
    dg = ds * s1 + db * e * u * silu_grad2(g)
    # g = K W1^T, u = K W3^T, e = V W2
    dW1 = dg.T @ K
    dW3 = du.T @ K
    dW2 = V.T @ dE
    dK = dK + dg @ W1 + du @ W3
    dV = dV + dE @ W2.T
    return dW1, dW3, dW2, dK, dV, de1, de3, de2


# -------------------------------------------------------- Newton-Schulz ----
def newton_schulz5_vjp(G, dU, eps=NS_EPS, coeffs=F.NS_COEFFS):
    """Cotangent of U = NS(G) (the five quintic steps of lact_oracle, as
    matrix products on the wide orientation) given dU: returns dG."""
    G, dU = _f64(G), _f64(dU)
    tall = G.shape[0] > G.shape[1]
    if tall:
        G, dU = G.T, dU.T
    r = float(np.linalg.norm(G))
    X = G / (r + eps)
    xs = [X]
    for a, b, c in coeffs:
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
        xs.append(X)
    dX = dU
    for k in range(len(coeffs) - 1, -1, -1):
        a, b, c = coeffs[k]
        X = xs[k]
        A = X @ X.T
        B = b * A + c * (A @ A)
        # Y = a X + B X
        dB = dX @ X.T
        dXn = a * dX + B.T @ dX
        dA = b * dB + c * (dB @ A.T + A.T @ dB)
        dXn = dXn + (dA + dA.T) @ X
        dX = dXn
    # X0 = G / (r + eps), r = ||G||_F
    dG = dX / (r + eps)
    if r > 0.0:
        dG = dG - (np.sum(dX * G) / ((r + eps) ** 2 * r)) * G
    return dG.T.copy() if tall else dG


# ------------------------------------------------------- step + renorm ----
def step_renorm_vjp(W, U, n0, dWn, eps=RENORM_EPS):
    """Cotangent of Wn = rows of (W + U) rescaled to n0 / (||row|| + eps):
    returns d(W + U) (the cotangent of both W and U) and dn0."""
    W, U, n0, dWn = map(_f64, (W, U, n0, dWn))
    R = W + U
    r = np.sqrt(np.sum(R * R, axis=1))
    f = n0 / (r + eps)
    proj = np.sum(dWn * R, axis=1)
    dR = f[:, None] * dWn - (n0 / (r + eps) ** 2 / np.where(r > 0, r, 1.0) * proj)[:, None] * R
    dn0 = proj / (r + eps)
    return dR, dn0


# ------------------------------------------------------------- one write ----
def update_vjp(state, K, V, eta1, eta3, eta2, dnew, mom=None, use_muon=False,
               use_momentum=False, renorm=True):
    """Cotangents of one write (lact_oracle.update) from state ``state`` on
    tokens K, V.  dnew: dict of cotangents of the new state's W1, W3, W2, M1,
    M3, M2 (missing keys = 0).  Returns (dold, dK, dV, deta1, deta3, deta2,
    dmom, dn0) with dold the cotangents of the old state's W and M."""
    s = state
    G = F.chunk_gradient(s.W1, s.W3, s.W2, K, V, eta1, eta3, eta2)
    beta = 0.0
    if use_momentum:
        beta = float(np.mean(_f64(mom))) if mom is not None and np.size(mom) else 0.0
        Gt = tuple(g + beta * m for g, m in zip(G, (s.M1, s.M3, s.M2)))
    else:
        Gt = G
    Us = tuple(F.newton_schulz5(g) for g in Gt) if use_muon else Gt
    Ws = (s.W1, s.W3, s.W2)
    ns = (s.n1, s.n3, s.n2)
    dWn = tuple(_f64(dnew.get(k, np.zeros_like(w))) for k, w in zip(("W1", "W3", "W2"), Ws))
    dold = {}
    dU, dn0 = [], []
    for W, U, n, d in zip(Ws, Us, ns, dWn):
        if renorm:
            dR, dn = step_renorm_vjp(W, U, n, d)
        else:
            dR, dn = d, np.zeros_like(n)
        dU.append(dR)
        dn0.append(dn)
    for key, dR in zip(("W1", "W3", "W2"), dU):
        dold[key] = dR.copy()
    # through Newton-Schulz
    dGt = [newton_schulz5_vjp(g, du) for g, du in zip(Gt, dU)] if use_muon else list(dU)
    dmom = None
    if use_momentum:
        # M_new = G~, and G~ feeds the step: both cotangents add up
        for i, key in enumerate(("M1", "M3", "M2")):
            if key in dnew:
                dGt[i] = dGt[i] + _f64(dnew[key])
        dbeta = sum(float(np.sum(d * m)) for d, m in zip(dGt, (s.M1, s.M3, s.M2)))
        for key, d in zip(("M1", "M3", "M2"), dGt):
            dold[key] = beta * d
        n = np.size(mom) if mom is not None else 0
        dmom = np.full(n, dbeta / n) if n else np.zeros(0)
    dW1, dW3, dW2, dK, dV, de1, de3, de2 = chunk_gradient_vjp(s.W1, s.W3, s.W2, K, V, eta1, eta3, eta2,
                                                              *dGt)
    dold["W1"] += dW1
    dold["W3"] += dW3
    dold["W2"] += dW2
    return dold, dK, dV, de1, de3, de2, dmom, tuple(dn0)


# ------------------------------------------------------------ sequence ----
def sequence_vjp(W1, W3, W2, Q, K, V, eta1, eta3, eta2, chunk, dO, mom=None,
                 order=F.ORDER_APPLY_THEN_UPDATE, subset=None, update_last=False,
                 use_muon=False, use_momentum=False, renorm=True):
    """Gradients of <O, dO> for O = lact_oracle.sequence(...) (same
    arguments) with respect to Q, K, V, eta1, eta3, eta2, the momentum
    coefficients (None without momentum) and the initial W1, W3, W2.
    Returns a dict with keys Q, K, V, eta1, eta3, eta2, mom, W1, W3, W2."""
    Q, K, V, dO = map(_f64, (Q, K, V, dO))
    e1, e3, e2 = (_f64(x).reshape(-1) for x in (eta1, eta3, eta2))
    T = Q.shape[0]
    bounds = F.chunk_bounds(T, chunk)
    st = F.HeadState(W1, W3, W2)
    # forward, keeping the state before every chunk and its write range
    plan = []
    for ci, (s0, e0) in enumerate(bounds):
        last = ci == len(bounds) - 1
        a0, a1 = (s0, e0) if subset is None else (s0 + subset[0], min(s0 + subset[0] + subset[1], e0))
        writes = (order == F.ORDER_UPDATE_THEN_APPLY or not last or update_last) and a1 > a0
        before = st.copy()
        if writes:
            m = None if mom is None else _f64(mom)[a0:a1]
            st = F.update(st, K[a0:a1], V[a0:a1], e1[a0:a1], e3[a0:a1], e2[a0:a1], mom=m,
                          use_muon=use_muon, use_momentum=use_momentum, renorm=renorm)
        plan.append((s0, e0, a0, a1, writes, before, st.copy()))
    g = {"Q": np.zeros_like(Q), "K": np.zeros_like(K), "V": np.zeros_like(V),
         "eta1": np.zeros_like(e1), "eta3": np.zeros_like(e3), "eta2": np.zeros_like(e2),
         "mom": None if mom is None else np.zeros(np.size(mom))}
    dn0 = [np.zeros(W.shape[0]) for W in (W1, W3, W2)]
    dstate = {}   # cotangent of the state after the chunk being walked
    for s0, e0, a0, a1, writes, before, after in reversed(plan):
        # the read of this chunk sees `before` (apply then update) or `after`
        read_state = before if order == F.ORDER_APPLY_THEN_UPDATE else after
        dX, dW1, dW3, dW2 = apply_vjp(read_state.W1, read_state.W3, read_state.W2, Q[s0:e0], dO[s0:e0])
        g["Q"][s0:e0] += dX
        if order == F.ORDER_UPDATE_THEN_APPLY:
            for key, d in (("W1", dW1), ("W3", dW3), ("W2", dW2)):
                dstate[key] = dstate.get(key, 0.0) + d
        if writes:
            m = None if mom is None else _f64(mom)[a0:a1]
            dold, dK, dV, d1, d3, d2, dm, dn = update_vjp(
                before, K[a0:a1], V[a0:a1], e1[a0:a1], e3[a0:a1], e2[a0:a1], dstate, mom=m,
                use_muon=use_muon, use_momentum=use_momentum, renorm=renorm)
            g["K"][a0:a1] += dK
            g["V"][a0:a1] += dV
            g["eta1"][a0:a1] += d1
            g["eta3"][a0:a1] += d3
            g["eta2"][a0:a1] += d2
            if dm is not None and g["mom"] is not None:
                g["mom"][a0:a1] += dm
            for i in range(3):
                dn0[i] += dn[i]
            dstate = dold
        if order == F.ORDER_APPLY_THEN_UPDATE:
            for key, d in (("W1", dW1), ("W3", dW3), ("W2", dW2)):
                dstate[key] = dstate.get(key, 0.0) + d
    # W0: its own cotangent plus the renorm targets n0 = row norms of W0
    for i, (key, W) in enumerate((("W1", W1), ("W3", W3), ("W2", W2))):
        W = _f64(W)
        r = np.sqrt(np.sum(W * W, axis=1))
        d = _f64(dstate.get(key, np.zeros_like(W)))
        g[key] = d + (dn0[i] / np.where(r > 0, r, 1.0))[:, None] * W
    return g
