"""Pins of the outer-loop backward oracle (oracle/lact_backward.py) to facts
that do not come from it: central finite differences of the forward oracle's
own sequence along random directions of every input, and torch.autograd in
float64 on a torch version of the forward written here (matrix-form
Newton-Schulz, its own loop over chunks).  CPU only."""
import math

import zlib

import numpy as np
import pytest

from oracle import lact_backward as B
from oracle import lact_oracle as F

CASES = {
    # name: (T, chunk, order, subset, muon, momentum, renorm)
    "causal-muon-momentum": (17, 5, F.ORDER_APPLY_THEN_UPDATE, None, True, True, True),
    "causal-plain": (12, 4, F.ORDER_APPLY_THEN_UPDATE, None, False, False, True),
    "causal-no-renorm": (12, 4, F.ORDER_APPLY_THEN_UPDATE, None, True, True, False),
    "video-subset": (16, 8, F.ORDER_APPLY_THEN_UPDATE, (4, 4), True, False, True),
    "bidirectional-subset": (10, 10, F.ORDER_UPDATE_THEN_APPLY, (0, 7), False, False, True),
}


def _inputs(rng, T, d=4, dh=6):
    s = 1.0 / math.sqrt(d)
    W = [rng.standard_normal((dh, d)) * s, rng.standard_normal((dh, d)) * s, rng.standard_normal((d, dh)) * s]
    Q, K, V = (rng.standard_normal((T, d)) for _ in range(3))
    Q /= np.linalg.norm(Q, axis=1, keepdims=True)
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    e = [np.log1p(np.exp(rng.standard_normal(T))) * 0.3 for _ in range(3)]
    mom = rng.uniform(0.5, 0.95, T)
    dO = rng.standard_normal((T, d))
    return W, Q, K, V, e, mom, dO


def _loss(W, Q, K, V, e, mom, dO, case):
    T, C, order, subset, muon, momentum, renorm = CASES[case]
    O, _ = F.sequence(*W, Q, K, V, *e, C, mom=mom if momentum else None, order=order, subset=subset,
                      use_muon=muon, use_momentum=momentum, renorm=renorm)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_finite_differences(case):
    T, C, order, subset, muon, momentum, renorm = CASES[case]
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    W, Q, K, V, e, mom, dO = _inputs(rng, T)
    g = B.sequence_vjp(*W, Q, K, V, *e, C, dO, mom=mom if momentum else None, order=order, subset=subset,
                       use_muon=muon, use_momentum=momentum, renorm=renorm)
    base = dict(W1=W[0], W3=W[1], W2=W[2], Q=Q, K=K, V=V, eta1=e[0], eta3=e[1], eta2=e[2], mom=mom)
    keys = ["W1", "W3", "W2", "Q", "K", "V", "eta1", "eta3", "eta2"] + (["mom"] if momentum else [])
    h = 1e-5
    for key in keys:
        for trial in range(2):
            delta = rng.standard_normal(base[key].shape)
            def at(sign):
                x = dict(base)
                x[key] = base[key] + sign * h * delta
                return _loss([x["W1"], x["W3"], x["W2"]], x["Q"], x["K"], x["V"], [x["eta1"], x["eta3"], x["eta2"]],
                             x["mom"], dO, case)
            # fourth-order central stencil: the Newton-Schulz steps make the
            # loss strongly curved, and the two-point stencil's h^2 error
            # alone is about 1e-6 here
            fd = (8 * (at(1) - at(-1)) - (at(2) - at(-2))) / (12 * h)
            an = float(np.sum(g[key] * delta))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (case, key, trial, fd, an)


def _torch_forward(torch, W, Q, K, V, e, mom, case):
    """The layer in torch float64, from the definitions (not the oracle's
    code): matrix-form Newton-Schulz with the Gram matrix on the row side of
    the wide orientation."""
    T, C, order, subset, muon, momentum, renorm = CASES[case]
    W1, W3, W2 = W
    n = [w.norm(dim=1) for w in (W1, W3, W2)]
    M = [torch.zeros_like(w) for w in (W1, W3, W2)]
    coeffs = F.NS_COEFFS

    def ns(G):
        X = G.T if G.shape[0] > G.shape[1] else G
        X = X / (X.norm() + 1e-7)
        for a, b, c in coeffs:
            A = X @ X.T
            X = a * X + (b * A + c * A @ A) @ X
        return X.T if G.shape[0] > G.shape[1] else X

    def read(W1, W3, W2, x):
        return (torch.nn.functional.silu(x @ W1.T) * (x @ W3.T)) @ W2.T

    outs = []
    for s0 in range(0, T, C):
        e0 = min(s0 + C, T)
        last = e0 == T
        a0, a1 = (s0, e0) if subset is None else (s0 + subset[0], min(s0 + subset[0] + subset[1], e0))
        writes = (order == F.ORDER_UPDATE_THEN_APPLY or not last) and a1 > a0
        if order == F.ORDER_APPLY_THEN_UPDATE:
            outs.append(read(W1, W3, W2, Q[s0:e0]))
        if writes:
            k, v = K[a0:a1], V[a0:a1]
            # G_j = -dL_j/dW_j of L_j = -sum eta_j <f(k), v>, written out so
            # that it stays a differentiable function of the weights
            G1 = _regrad(torch, W1, W3, W2, k, v, e[0][a0:a1], 0)
            G3 = _regrad(torch, W1, W3, W2, k, v, e[1][a0:a1], 1)
            G2 = _regrad(torch, W1, W3, W2, k, v, e[2][a0:a1], 2)
            G = [G1, G3, G2]
            if momentum:
                beta = mom[a0:a1].mean()
                G = [g + beta * m for g, m in zip(G, M)]
                M = G
            U = [ns(g) for g in G] if muon else G
            Wn = []
            for w, u, nn in zip((W1, W3, W2), U, n):
                r = w + u
                Wn.append(r / (r.norm(dim=1, keepdim=True) + 1e-5) * nn[:, None] if renorm else r)
            W1, W3, W2 = Wn
        if order == F.ORDER_UPDATE_THEN_APPLY:
            outs.append(read(W1, W3, W2, Q[s0:e0]))
    return torch.cat(outs)


def _regrad(torch, W1, W3, W2, k, v, et, j):
    """G_j = -dL_j/dW_j written out (the SwiGLU backward), as a differentiable
    function of the weights."""
    g, u, ev = k @ W1.T, k @ W3.T, v @ W2
    sg = torch.sigmoid(g)
    s = g * sg
    if j == 2:
        return v.T @ (et[:, None] * s * u)
    if j == 1:
        return (et[:, None] * ev * s).T @ k
    return (et[:, None] * ev * u * sg * (1 + g * (1 - sg))).T @ k


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_torch_autograd(case):
    torch = pytest.importorskip("torch")
    T, C, order, subset, muon, momentum, renorm = CASES[case]
    rng = np.random.default_rng(7 + len(case))
    W, Q, K, V, e, mom, dO = _inputs(rng, T)
    g = B.sequence_vjp(*W, Q, K, V, *e, C, dO, mom=mom if momentum else None, order=order, subset=subset,
                       use_muon=muon, use_momentum=momentum, renorm=renorm)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Wt = [t(w) for w in W]
    Qt, Kt, Vt = t(Q), t(K), t(V)
    et = [t(x) for x in e]
    mt = t(mom)
    O = _torch_forward(torch, Wt, Qt, Kt, Vt, et, mt, case)
    # the torch forward agrees with the oracle's
    ref, _ = F.sequence(*W, Q, K, V, *e, C, mom=mom if momentum else None, order=order, subset=subset,
                        use_muon=muon, use_momentum=momentum, renorm=renorm)
    assert np.max(np.abs(O.detach().numpy() - ref)) < 1e-12
    (O * torch.tensor(dO)).sum().backward()
    pairs = [("W1", Wt[0]), ("W3", Wt[1]), ("W2", Wt[2]), ("Q", Qt), ("K", Kt), ("V", Vt),
             ("eta1", et[0]), ("eta3", et[1]), ("eta2", et[2])] + ([("mom", mt)] if momentum else [])
    for key, x in pairs:
        want = x.grad.numpy()
        scale = max(1e-12, float(np.max(np.abs(want))))
        assert np.max(np.abs(g[key] - want)) < 1e-9 * scale, (case, key, np.max(np.abs(g[key] - want)), scale)
