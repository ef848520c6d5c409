"""Pins of the float64 oracle to facts that do not come from the oracle.

Each test checks one oracle function against something fixed by the pages or
by mathematics: central finite differences of the associative loss, the
linearity of the chunk gradient in its tokens, brute-force scalar loops, the
Newton-Schulz matrix iteration written with the Gram matrix on the other
side (the oracle uses the singular-value form), its singular-value band and
rank-one closed form, closed forms of the renorm and of momentum, the
momentum buffer and renorm targets over two writes, the printed constants,
and the causality structure of the orderings.  CPU only.
"""
import math
import os

import numpy as np
import pytest

from oracle import lact_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_state(rng, d, dh, scale=None):
    s = 1.0 / math.sqrt(d) if scale is None else scale
    return (rng.standard_normal((dh, d)) * s, rng.standard_normal((dh, d)) * s,
            rng.standard_normal((d, dh)) * s)


# ------------------------------------------------------------ scalars ----
def test_silu_and_derivative():
    x = np.linspace(-12, 12, 2001)
    h = 1e-5
    fd = (O.silu(x + h) - O.silu(x - h)) / (2 * h)
    assert np.max(np.abs(fd - O.silu_grad(x))) < 1e-9
    assert O.silu(0.0) == 0.0 and O.silu_grad(0.0) == 0.5
    # silu(x) = x / (1 + e^-x) written with math.exp
    for v in (-3.0, -0.5, 0.25, 2.0, 7.0):
        assert abs(O.silu(v) - v / (1.0 + math.exp(-v))) < 1e-15


# -------------------------------------------------------------- apply ----
def test_apply_brute_force():
    rng = np.random.default_rng(1)
    d, dh, n = 4, 6, 5
    W1, W3, W2 = _rand_state(rng, d, dh)
    X = rng.standard_normal((n, d))
    out = O.apply(W1, W3, W2, X)
    for t in range(n):
        hidden = []
        for j in range(dh):
            g = sum(W1[j][i] * X[t][i] for i in range(d))
            u = sum(W3[j][i] * X[t][i] for i in range(d))
            hidden.append(g / (1.0 + math.exp(-g)) * u)
        for i in range(d):
            ref = sum(W2[i][j] * hidden[j] for j in range(dh))
            assert abs(out[t][i] - ref) < 1e-13


# ----------------------------------------------------------- gradient ----
def _loss(W1, W3, W2, K, V, eta):
    """L = -sum_t eta_t <f_W(k_t), v_t>, scalar loops (no oracle code)."""
    total = 0.0
    d, dh = W2.shape
    for t in range(K.shape[0]):
        h = []
        for j in range(dh):
            g = float(np.dot(W1[j], K[t]))
            u = float(np.dot(W3[j], K[t]))
            h.append(g / (1.0 + math.exp(-g)) * u)
        f = [sum(W2[i][j] * h[j] for j in range(dh)) for i in range(d)]
        total -= eta[t] * sum(f[i] * V[t][i] for i in range(d))
    return total


def test_gradient_finite_differences():
    rng = np.random.default_rng(2)
    d, dh, n = 3, 5, 7
    W1, W3, W2 = _rand_state(rng, d, dh, scale=0.7)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    e1, e3, e2 = (np.abs(rng.standard_normal(n)) + 0.1 for _ in range(3))
    G1, G3, G2 = O.chunk_gradient(W1, W3, W2, K, V, e1, e3, e2)
    h = 1e-6
    for G, idx, eta in ((G1, 0, e1), (G3, 1, e3), (G2, 2, e2)):
        Ws = [W1, W3, W2]
        fd = np.zeros_like(G)
        for a in range(G.shape[0]):
            for b in range(G.shape[1]):
                Wp = [w.copy() for w in Ws]
                Wm = [w.copy() for w in Ws]
                Wp[idx][a, b] += h
                Wm[idx][a, b] -= h
                fd[a, b] = -(_loss(*Wp, K, V, eta) - _loss(*Wm, K, V, eta)) / (2 * h)
        rel = np.linalg.norm(G - fd) / np.linalg.norm(fd)
        assert rel < 1e-7, (idx, rel)


def test_gradient_matches_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    d, dh, n = 16, 40, 33
    W1, W3, W2 = _rand_state(rng, d, dh)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    eta = np.abs(rng.standard_normal(n)) * 1e-2
    G1, G3, G2 = O.chunk_gradient(W1, W3, W2, K, V, eta, eta, eta)
    t = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in (W1, W3, W2)]
    Kt, Vt, Et = (torch.tensor(a, dtype=torch.float64) for a in (K, V, eta))
    hid = torch.nn.functional.silu(Kt @ t[0].T) * (Kt @ t[1].T)
    L = -(Et[:, None] * (hid @ t[2].T) * Vt).sum()
    L.backward()
    for G, w in zip((G1, G3, G2), t):
        assert np.max(np.abs(G + w.grad.numpy())) < 1e-13 * max(1.0, np.max(np.abs(G)))


def test_gradient_linearity_and_permutation():
    rng = np.random.default_rng(4)
    d, dh, n = 8, 24, 50
    W1, W3, W2 = _rand_state(rng, d, dh)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    e1, e3, e2 = (np.abs(rng.standard_normal(n)) for _ in range(3))
    full = O.chunk_gradient(W1, W3, W2, K, V, e1, e3, e2)
    a = O.chunk_gradient(W1, W3, W2, K[:17], V[:17], e1[:17], e3[:17], e2[:17])
    b = O.chunk_gradient(W1, W3, W2, K[17:], V[17:], e1[17:], e3[17:], e2[17:])
    p = rng.permutation(n)
    perm = O.chunk_gradient(W1, W3, W2, K[p], V[p], e1[p], e3[p], e2[p])
    for f, x, y, z in zip(full, a, b, perm):
        assert np.max(np.abs(f - (x + y))) < 1e-12 * np.max(np.abs(f))
        assert np.max(np.abs(f - z)) < 1e-12 * np.max(np.abs(f))


def test_gradient_eta_selects_matrix():
    """eta1 only reaches G1, eta3 only G3, eta2 only G2 (page: lr0/lr1/lr2)."""
    rng = np.random.default_rng(5)
    d, dh, n = 4, 8, 9
    W1, W3, W2 = _rand_state(rng, d, dh)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    z, one = np.zeros(n), np.ones(n)
    G1, G3, G2 = O.chunk_gradient(W1, W3, W2, K, V, one, z, z)
    assert np.abs(G1).max() > 0 and np.abs(G3).max() == 0 and np.abs(G2).max() == 0
    G1, G3, G2 = O.chunk_gradient(W1, W3, W2, K, V, z, z, one)
    assert np.abs(G1).max() == 0 and np.abs(G3).max() == 0 and np.abs(G2).max() > 0


def test_gradient_per_channel_eta_brute_force():
    """Per-channel learning rates: scalar loops of the definition
    G1[j][i] = sum_t (e u silu')_tj eta1_ti k_ti (likewise G3 with e s) and
    G2[i][j] = sum_t v_ti eta2_tj h_tj; and constant channels reduce to the
    per-token form."""
    rng = np.random.default_rng(21)
    d, dh, n = 3, 5, 4
    W1, W3, W2 = _rand_state(rng, d, dh)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    e1, e3 = np.abs(rng.standard_normal((n, d))), np.abs(rng.standard_normal((n, d)))
    e2 = np.abs(rng.standard_normal((n, dh)))
    G1, G3, G2 = O.chunk_gradient(W1, W3, W2, K, V, e1, e3, e2)
    for j in range(dh):
        for i in range(d):
            a1 = a3 = 0.0
            for t in range(n):
                g = sum(W1[j][x] * K[t][x] for x in range(d))
                u = sum(W3[j][x] * K[t][x] for x in range(d))
                e = sum(W2[x][j] * V[t][x] for x in range(d))
                sg = 1.0 / (1.0 + math.exp(-g))
                a1 += e * u * sg * (1 + g * (1 - sg)) * e1[t][i] * K[t][i]
                a3 += e * g * sg * e3[t][i] * K[t][i]
            assert abs(G1[j][i] - a1) < 1e-13 and abs(G3[j][i] - a3) < 1e-13
    for i in range(d):
        for j in range(dh):
            a2 = 0.0
            for t in range(n):
                g = sum(W1[j][x] * K[t][x] for x in range(d))
                u = sum(W3[j][x] * K[t][x] for x in range(d))
                a2 += V[t][i] * e2[t][j] * g / (1.0 + math.exp(-g)) * u
            assert abs(G2[i][j] - a2) < 1e-13
    c = np.abs(rng.standard_normal(n))
    per_tok = O.chunk_gradient(W1, W3, W2, K, V, c, c, c)
    per_ch = O.chunk_gradient(W1, W3, W2, K, V, np.repeat(c[:, None], d, 1), np.repeat(c[:, None], d, 1),
                              np.repeat(c[:, None], dh, 1))
    for a, b in zip(per_tok, per_ch):
        assert np.max(np.abs(a - b)) < 1e-14


# ----------------------------------------------------- Newton-Schulz ----
def _golden_coeffs():
    rows = []
    with open(os.path.join(GOLDEN, "ns_coefficients.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(tuple(float(x) for x in line.split()))
    return rows


def _phi(x):
    for a, b, c in _golden_coeffs():
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def test_ns_coefficients_are_the_pages():
    assert [tuple(c) for c in O.NS_COEFFS] == _golden_coeffs()
    assert O.NS_EPS == 1e-7 and O.RENORM_EPS == 1e-5


def _ns_matrix_iteration(G):
    """The five quintic steps as matrix products, written here with the Gram
    matrix on the column side: X <- X (a I + b X^T X + c (X^T X)^2), which
    equals a X + b (X X^T) X + c (X X^T)^2 X, in the orientation G has."""
    X = np.array(G, dtype=np.float64)
    X = X / (math.sqrt(float(np.sum(X * X))) + 1e-7)
    eye = np.eye(X.shape[1])
    for a, b, c in _golden_coeffs():
        S = X.T @ X
        X = X @ (a * eye + b * S + c * (S @ S))
    return X


@pytest.mark.parametrize("shape", [(12, 30), (30, 12), (16, 16), (128, 512), (1024, 256)])
def test_ns_matches_matrix_iteration(shape):
    """The oracle's singular-value form equals the matrix iteration."""
    rng = np.random.default_rng(6)
    G = rng.standard_normal(shape) * 3.0
    ref = _ns_matrix_iteration(G)
    out = O.newton_schulz5(G)
    assert out.shape == G.shape
    assert np.max(np.abs(out - ref)) < 1e-12


def test_ns_zero_and_low_rank():
    """A zero gradient gives a zero step; a rank-deficient one keeps its rank
    (phi(0) = 0) and its row and column spaces."""
    assert np.array_equal(O.newton_schulz5(np.zeros((8, 20))), np.zeros((8, 20)))
    rng = np.random.default_rng(17)
    G = rng.standard_normal((16, 3)) @ rng.standard_normal((3, 40))
    out = O.newton_schulz5(G)
    assert np.max(np.abs(out - _ns_matrix_iteration(G))) < 1e-12
    sv = np.linalg.svd(out, compute_uv=False)
    assert sv[3] < 1e-12 * sv[0]


def test_ns_singular_values_approach_one():
    rng = np.random.default_rng(7)
    m, n = 32, 96
    U, _ = np.linalg.qr(rng.standard_normal((m, m)))
    V, _ = np.linalg.qr(rng.standard_normal((n, m)))
    s = np.geomspace(0.02, 1.0, m)
    G = (U * s) @ V.T
    out = O.newton_schulz5(G)
    sv = np.linalg.svd(out, compute_uv=False)
    grid = np.linspace(0.01, 1.0, 200001)
    lo, hi = _phi(grid).min(), _phi(grid).max()
    assert 0.977 < lo < 0.978 and 1.031 < hi < 1.032
    assert sv.min() >= lo - 1e-12 and sv.max() <= hi + 1e-12
    # a rank-1 input maps to phi(||G|| / (||G|| + eps)) u v^T
    u, v = rng.standard_normal(m), rng.standard_normal(n)
    r1 = np.outer(u, v)
    out1 = O.newton_schulz5(r1)
    nr = np.linalg.norm(r1)
    ref = _phi(nr / (nr + 1e-7)) * r1 / nr
    assert np.max(np.abs(out1 - ref)) < 1e-13


def test_ns_scale_invariance():
    rng = np.random.default_rng(8)
    G = rng.standard_normal((20, 50))
    a, b = O.newton_schulz5(G), O.newton_schulz5(G * 37.0)
    assert np.max(np.abs(a - b)) < 1e-6


# ----------------------------------------------------- renorm, momentum ----
def test_step_renorm_closed_form():
    rng = np.random.default_rng(9)
    W, U = rng.standard_normal((10, 7)), rng.standard_normal((10, 7)) * 0.3
    n0 = np.abs(rng.standard_normal(10)) + 0.5
    out = O.step_renorm(W, U, n0)
    r = W + U
    nr = np.sqrt((r * r).sum(1))
    assert np.max(np.abs(np.sqrt((out * out).sum(1)) - n0 * nr / (nr + 1e-5))) < 1e-14
    # direction unchanged
    cos = (out * r).sum(1) / (np.sqrt((out * out).sum(1)) * nr)
    assert np.max(np.abs(cos - 1.0)) < 1e-14


def test_momentum_closed_form():
    rng = np.random.default_rng(10)
    beta = 0.9
    Gs = [rng.standard_normal((5, 6)) for _ in range(6)]
    M = np.zeros((5, 6))
    for c, G in enumerate(Gs):
        out, M = O.momentum_step(G, M, beta)
        ref = sum(beta ** (c - s) * Gs[s] for s in range(c + 1))
        assert np.max(np.abs(out - ref)) < 1e-12
        assert np.max(np.abs(M - ref)) < 1e-12


def test_update_eta_zero_is_pure_renorm():
    rng = np.random.default_rng(11)
    d, dh, n = 8, 16, 12
    W1, W3, W2 = _rand_state(rng, d, dh)
    st = O.HeadState(W1, W3, W2)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    z = np.zeros(n)
    new = O.update(st, K, V, z, z, z, use_muon=False)
    for W, Wn in ((W1, new.W1), (W3, new.W3), (W2, new.W2)):
        nr = np.sqrt((W * W).sum(1))
        assert np.max(np.abs(Wn - W * (nr / (nr + 1e-5))[:, None])) < 1e-15


def test_update_momentum_beta_is_chunk_mean():
    rng = np.random.default_rng(12)
    d, dh, n = 4, 8, 10
    W1, W3, W2 = _rand_state(rng, d, dh)
    st = O.HeadState(W1, W3, W2)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    eta = np.full(n, 0.01)
    mom = rng.uniform(0.5, 1.0, n)
    st.M1 = rng.standard_normal(st.M1.shape)
    _, parts = O.update(st, K, V, eta, eta, eta, mom=mom, use_momentum=True, return_parts=True)
    raw1 = parts["raw"][0]
    assert np.max(np.abs(parts["pre_ns"][0] - (raw1 + mom.mean() * st.M1))) < 1e-15


def test_momentum_buffer_holds_pre_muon_sum():
    """Two writes with momentum and Muon: after the second write the buffer
    is G2 + beta G1, both raw chunk gradients (before Newton-Schulz), G1 at
    the initial weights and G2 at the weights after the first write."""
    rng = np.random.default_rng(18)
    d, dh, n = 6, 14, 11
    W1, W3, W2 = _rand_state(rng, d, dh)
    st0 = O.HeadState(W1, W3, W2)
    ks = [rng.standard_normal((n, d)) for _ in range(2)]
    vs = [rng.standard_normal((n, d)) for _ in range(2)]
    eta = np.full(n, 0.02)
    mom = rng.uniform(0.6, 0.95, (2, n))
    st1 = O.update(st0, ks[0], vs[0], eta, eta, eta, mom=mom[0], use_muon=True, use_momentum=True)
    st2 = O.update(st1, ks[1], vs[1], eta, eta, eta, mom=mom[1], use_muon=True, use_momentum=True)
    g1 = O.chunk_gradient(st0.W1, st0.W3, st0.W2, ks[0], vs[0], eta, eta, eta)
    g2 = O.chunk_gradient(st1.W1, st1.W3, st1.W2, ks[1], vs[1], eta, eta, eta)
    beta2 = float(np.mean(mom[1]))
    for M, a, b in zip((st2.M1, st2.M3, st2.M2), g1, g2):
        want = b + beta2 * a
        assert np.max(np.abs(M - want)) < 1e-13 * np.max(np.abs(want))
    # the buffer after the first write is the first raw gradient itself
    for M, a in zip((st1.M1, st1.M3, st1.M2), g1):
        assert np.max(np.abs(M - a)) < 1e-15 * np.max(np.abs(a)) + 1e-300


@pytest.mark.parametrize("muon", [False, True])
def test_renorm_targets_are_sequence_start_norms(muon):
    """Over two writes every row ends at n0 ||r|| / (||r|| + 1e-5), with n0
    the row norms of the initial weights (not of the weights before the
    write) and r the row after the step.  The initial rows are made short
    (norm ~1e-5) so that the two readings differ by a factor near two."""
    rng = np.random.default_rng(19)
    d, dh, n = 5, 9, 13
    W1, W3, W2 = _rand_state(rng, d, dh, scale=1e-5 if not muon else None)
    n0 = [np.sqrt((W * W).sum(1)) for W in (W1, W3, W2)]
    st = O.HeadState(W1, W3, W2)
    for c in range(2):
        K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
        eta = np.full(n, 1e-9 if not muon else 0.01)
        new, parts = O.update(st, K, V, eta, eta, eta, use_muon=muon, return_parts=True)
        for W_prev, U, W_new, tgt in zip((st.W1, st.W3, st.W2), parts["step"], (new.W1, new.W3, new.W2), n0):
            r = W_prev + U
            nr = np.sqrt((r * r).sum(1))
            got = np.sqrt((W_new * W_new).sum(1))
            assert np.max(np.abs(got / (tgt * nr / (nr + 1e-5)) - 1.0)) < 1e-13, c
            if not muon and c == 1:
                # recomputing the targets from the weights before the write
                # would give rows about half as long
                prev = np.sqrt((W_prev * W_prev).sum(1))
                assert np.min(np.abs(got - prev * nr / (nr + 1e-5)) / got) > 0.2
        st = new


def test_master_state_variant():
    """Variant with a master state (uTTT page section C.1): over two writes
    the master is W0 + U1 + U2 (the Newton-Schulz steps, never rescaled),
    the weights used afterwards are the master's rows rescaled to
    n0 ||S|| / (||S|| + 1e-5), and the second write's gradient is taken at
    that rescaled copy, not at the master."""
    rng = np.random.default_rng(20)
    d, dh, n = 5, 9, 13
    W1, W3, W2 = _rand_state(rng, d, dh)
    n0 = [np.sqrt((W * W).sum(1)) for W in (W1, W3, W2)]
    st0 = O.HeadState(W1, W3, W2)
    ks = [rng.standard_normal((n, d)) for _ in range(2)]
    vs = [rng.standard_normal((n, d)) for _ in range(2)]
    eta = np.full(n, 0.02)
    st1, p1 = O.update(st0, ks[0], vs[0], eta, eta, eta, use_muon=True, renorm="master", return_parts=True)
    st2, p2 = O.update(st1, ks[1], vs[1], eta, eta, eta, use_muon=True, renorm="master", return_parts=True)
    for i, (W0, S, Wf) in enumerate(zip((W1, W3, W2), (st2.S1, st2.S3, st2.S2), (st2.W1, st2.W3, st2.W2))):
        assert np.max(np.abs(S - (W0 + p1["step"][i] + p2["step"][i]))) < 1e-14
        ns = np.sqrt((S * S).sum(1))
        want = S * (n0[i] / (ns + 1e-5))[:, None]
        assert np.max(np.abs(Wf - want)) < 1e-14
    g2 = O.chunk_gradient(st1.W1, st1.W3, st1.W2, ks[1], vs[1], eta, eta, eta)
    for a, b in zip(p2["raw"], g2):
        assert np.max(np.abs(a - b)) < 1e-15 * max(1.0, np.max(np.abs(b)))
    # it differs from rescaling in place (rows of W1 + U2 from the rescaled W1)
    inplace = O.update(st1, ks[1], vs[1], eta, eta, eta, use_muon=True, renorm=True)
    assert np.max(np.abs(inplace.W1 - st2.W1)) > 1e-3


def test_linear_variant_gradient_and_sequence():
    """Linear fast weight f_W(x) = W x: the gradient is -dL/dW of
    L = -sum eta <W k, v> (central differences), and one write from W0
    followed by a read is, written out by hand, the rows of W0 + NS(G)
    rescaled to their initial norms, applied to the next chunk's queries."""
    rng = np.random.default_rng(22)
    d, n = 4, 6
    W = rng.standard_normal((d, d)) * 0.5
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    eta = np.abs(rng.standard_normal(n))
    G = O.linear_gradient(K, V, eta)
    loss = lambda W_: -sum(eta[t] * float(np.dot(W_ @ K[t], V[t])) for t in range(n))
    h = 1e-6
    for i in range(d):
        for j in range(d):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            assert abs(-(loss(Wp) - loss(Wm)) / (2 * h) - G[i, j]) < 1e-7
    Q = rng.standard_normal((2 * n, d))
    Kk = np.concatenate([K, rng.standard_normal((n, d))])
    Vv = np.concatenate([V, rng.standard_normal((n, d))])
    ee = np.concatenate([eta, eta])
    out, (Wf, _) = O.linear_sequence(W, Q, Kk, Vv, ee, n, use_muon=True)
    assert np.max(np.abs(out[:n] - Q[:n] @ W.T)) < 1e-14
    R = W + _ns_matrix_iteration(G)
    n0 = np.sqrt((W * W).sum(1))
    W1 = R / (np.sqrt((R * R).sum(1)) + 1e-5)[:, None] * n0[:, None]
    assert np.max(np.abs(out[n:] - Q[n:] @ W1.T)) < 1e-12
    assert np.max(np.abs(Wf - W1)) < 1e-12   # the last chunk is not written


# ---------------------------------------------------------- orderings ----
def _seq_inputs(rng, T, d, dh):
    W = _rand_state(rng, d, dh)
    Q = rng.standard_normal((T, d))
    Q /= np.linalg.norm(Q, axis=1, keepdims=True)
    K = rng.standard_normal((T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((T, d))
    eta = np.log1p(np.exp(rng.standard_normal(T))) * 1e-2
    return W, Q, K, V, eta


def test_causal_ordering_is_shifted_block_causal():
    rng = np.random.default_rng(13)
    T, C, d, dh = 80, 16, 8, 16
    W, Q, K, V, eta = _seq_inputs(rng, T, d, dh)
    mom = np.full(T, 0.9)
    kw = dict(chunk=C, mom=mom, use_muon=True, use_momentum=True)
    base, st = O.sequence(*W, Q, K, V, eta, eta, eta, **kw)
    # chunk 0 is read with the initial weights
    assert np.max(np.abs(base[:C] - O.apply(*W, Q[:C]))) < 1e-15
    for c in range(T // C):
        K2, V2, e2 = K.copy(), V.copy(), eta.copy()
        K2[c * C:] += 1.0
        V2[c * C:] -= 0.5
        e2[c * C:] *= 3.0
        out, _ = O.sequence(*W, Q, K2, V2, e2, e2, e2, **kw)
        # outputs of chunks <= c do not see keys/values of chunk c or later
        assert np.array_equal(out[: (c + 1) * C], base[: (c + 1) * C])
        if c < T // C - 1:
            assert not np.allclose(out[(c + 1) * C:], base[(c + 1) * C:])
    # the last chunk is never written: final state == state before the last chunk
    _, st_last, states = O.sequence(*W, Q, K, V, eta, eta, eta, return_states=True, **kw)
    assert np.array_equal(st_last.W1, states[-1].W1)


def test_causal_loop_bound_ragged():
    """Chunks that start before T - C are written; the tail is read only."""
    rng = np.random.default_rng(14)
    d, dh, C = 6, 12, 10
    T = 35
    W, Q, K, V, eta = _seq_inputs(rng, T, d, dh)
    out, st, states = O.sequence(*W, Q, K, V, eta, eta, eta, chunk=C, return_states=True)
    assert len(states) == 4   # chunks [0,10) [10,20) [20,30) [30,35)
    K2 = K.copy()
    K2[30:] += 1.0
    out2, st2 = O.sequence(*W, Q, K2, V, eta, eta, eta, chunk=C)
    assert np.array_equal(out, out2) and np.array_equal(st.W1, st2.W1)


def test_ar_video_subset_ordering():
    rng = np.random.default_rng(15)
    T, C, d, dh = 64, 16, 8, 16
    W, Q, K, V, eta = _seq_inputs(rng, T, d, dh)
    kw = dict(chunk=C, subset=(8, 8), use_muon=True)
    base, _ = O.sequence(*W, Q, K, V, eta, eta, eta, **kw)
    K2, V2 = K.copy(), V.copy()
    for s in range(0, T, C):
        K2[s:s + 8] += 2.0   # noisy half never writes
        V2[s:s + 8] *= -1.0
    out, _ = O.sequence(*W, Q, K2, V2, eta, eta, eta, **kw)
    assert np.array_equal(out, base)
    # the clean half of chunk 0 reaches chunk 1's reads
    K3 = K.copy()
    K3[8:16] += 1.0
    out3, _ = O.sequence(*W, Q, K3, V, eta, eta, eta, **kw)
    assert np.array_equal(out3[:C], base[:C]) and not np.allclose(out3[C:2 * C], base[C:2 * C])


def test_bidirectional_subset_ordering():
    rng = np.random.default_rng(16)
    T, d, dh = 48, 8, 16
    W, Q, K, V, eta = _seq_inputs(rng, T, d, dh)
    kw = dict(chunk=T, order=O.ORDER_UPDATE_THEN_APPLY, subset=(0, 36))
    base, st = O.sequence(*W, Q, K, V, eta, eta, eta, **kw)
    K2 = K.copy()
    K2[36:] += 1.0   # target tokens do not write
    out, _ = O.sequence(*W, Q, K2, V, eta, eta, eta, **kw)
    assert np.array_equal(out, base)
    # every token, including the first, sees the write of the input tokens
    out_nowrite = O.apply(*W, Q)
    assert not np.allclose(out[:1], out_nowrite[:1])


def test_page_flops_model():
    vals = {}
    with open(os.path.join(GOLDEN, "flops_model.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    # count the multiply-adds of one token through the oracle's contractions
    d, dh = 1, 1
    fwd_key = 2 * (2 * d * dh)          # W1 k, W3 k
    backward = 2 * (d * dh) + 3 * 2 * (d * dh)   # W2^T v, three outer products
    fwd_query = 3 * 2 * d * dh           # W1 q, W3 q, W2 h
    assert (fwd_key, backward, fwd_query) == (vals["forward_with_key"], vals["backward"], vals["forward_with_query"])
    assert fwd_key + backward + fwd_query == vals["total"]
