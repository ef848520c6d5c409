"""CPU model of where the HIP path rounds (test infrastructure only).

The float64 oracle computes the layer exactly.  The HIP path computes it in
fp32 with bf16 MFMA operands, so with Muon on it drifts from the oracle chunk
by chunk: the Newton-Schulz polynomial maps the gradient's small singular
directions to unit length and so amplifies any perturbation along them.
This module replays a sequence in float32 and rounds to bf16 exactly where
the kernels do, so that the end-to-end drift of the GPU run can be told
apart from a kernel bug: the GPU's per-chunk error curve against the oracle
must follow this model's curve within a stated factor.

Rounding points (they follow the kernels):

* weights: fp32 masters, bf16 operand copies (W1, W3, W2 and W2^T) written
  after every step;
* read: g = W1 q, u = W3 q accumulate in fp32; h = silu(g) u is rounded to
  bf16 as the operand of W2 h; the output is rounded to bf16;
* gradient: g, u, e = W2^T v in fp32; the SwiGLU backward in fp32; the three
  eta-scaled products eta h, eta e s, eta e u silu'(g) are rounded to bf16 as
  the operands of the token contractions, which accumulate in fp32;
* momentum, step and renorm in fp32;
* Newton-Schulz (wide orientation, Frobenius normalisation in fp32), per
  ``ns`` (the library's lact_ns_prec):
    - "bf16": every product takes bf16 operands; the iterate stays fp32
      between steps; A and B are stored as bf16; the b A term reads the
      stored A (one-workgroup kernels) or an fp32 copy of it (the batched
      GEMM path for larger matrices, ``gemm_path``);
    - "bf16-shifted": the same, except that steps 2, 3 and 4 subtract
      mu I from A before it is stored, mu = trace(A) / rows (batched path:
      ||X||_F^2 / rows, the same number up to rounding), and take
      B_s = (b + 2 c mu) A_s + c A_s A_s,  X <- (a + b mu + c mu^2) X + B_s X;
    - "f32": fp32 operands ("f32-shifted": with the shift, to check that the
      shift leaves the step unchanged in exact arithmetic).
  The one-workgroup kernel keeps the iterate divided by the product of the
  a's; that rescaling does not change how it rounds and is not modelled.

Shapes follow the oracle's convention: one head, W1, W3 [dh, d], W2 [d, dh],
tokens as rows.  The functions here share no code with the oracle or the
kernels; they are written from the same definitions, with the kernels'
rounding added.
"""
from __future__ import annotations

import numpy as np

NS_COEFFS = ((4.0848, -6.8946, 2.9270), (3.9505, -6.3029, 2.6377), (3.7418, -5.5913, 2.3037),
             (2.8769, -3.1427, 1.2046), (2.8366, -3.0525, 1.2012))


def bf(x):
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _sig(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _op(x, mode):
    """A matrix as the MFMA sees it: rounded to bf16 unless mode is "f32"."""
    return _f32(x) if mode == "f32" else bf(x)


def newton_schulz(G, ns="bf16", gemm_path=False, eps=1e-7):
    """Newton-Schulz-5 of one matrix with the kernels' rounding (module
    docstring); G in either orientation, fp32 result."""
    X = _f32(G)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T.copy()
    n = X.shape[0]
    eye = np.eye(n, dtype=np.float32)
    mode = "f32" if ns.startswith("f32") else "bf16"
    shift = ns.endswith("-shifted")
    nrm = np.float32(np.sqrt(np.sum(X.astype(np.float64) ** 2)))
    X = (X * np.float32(1.0 / (nrm + eps))).astype(np.float32)
    for it, (a, b, c) in enumerate(NS_COEFFS):
        Xo = _op(X, mode)
        A = (Xo @ Xo.T).astype(np.float32)
        mu = np.float32(0.0)
        if shift and it >= 2:
            tr = np.sum(X.astype(np.float64) ** 2) if gemm_path else np.trace(A.astype(np.float64))
            mu = np.float32(tr / n)
        As = (A - mu * eye).astype(np.float32)
        Ao = _op(As, mode)
        AA = (Ao @ Ao).astype(np.float32)
        bterm = As if gemm_path else Ao
        B = _op(np.float32(b + 2 * c * mu) * bterm + np.float32(c) * AA, mode)
        X = (np.float32(a + (b + c * mu) * mu) * X + B @ Xo).astype(np.float32)
    return X.T.copy() if tall else X


class State:
    """fp32 masters, sequence-start row norms, momentum, bf16 operand copies."""

    def __init__(self, W1, W3, W2, op="bf16"):
        self.op = op
        self.W1, self.W3, self.W2 = _f32(W1).copy(), _f32(W3).copy(), _f32(W2).copy()
        self.n1, self.n3, self.n2 = (np.sqrt(np.sum(w.astype(np.float64) ** 2, axis=1)).astype(np.float32)
                                     for w in (self.W1, self.W3, self.W2))
        self.M1 = np.zeros_like(self.W1)
        self.M3 = np.zeros_like(self.W3)
        self.M2 = np.zeros_like(self.W2)
        self.refresh()

    def refresh(self):
        r = (lambda x: x) if self.op == "f32" else bf
        self.s1, self.s3, self.s2 = r(self.W1), r(self.W3), r(self.W2)


def apply(st: State, Q):
    Q = _f32(Q)
    g = Q @ st.s1.T
    u = Q @ st.s3.T
    h = g * _sig(g) * u
    if st.op != "f32":
        h = bf(h)
    o = (h @ st.s2.T).astype(np.float32)
    return o if st.op == "f32" else bf(o)


def gradient(st: State, K, V, eta):
    K, V, eta = _f32(K), _f32(V), _f32(eta)[:, None]
    g = K @ st.s1.T
    u = K @ st.s3.T
    e = V @ st.s2
    sg = _sig(g)
    s = g * sg
    dsl = sg * (1.0 + g * (1.0 - sg))
    r = (lambda x: x) if st.op == "f32" else bf
    fh = r(eta * s * u)
    fu = r(eta * s * e)
    fg = r(eta * dsl * (e * u))
    G2 = (V.T @ fh).astype(np.float32)
    G3 = (fu.T @ K).astype(np.float32)
    G1 = (fg.T @ K).astype(np.float32)
    return G1, G3, G2


def update(st: State, K, V, eta, mom=None, use_muon=False, use_momentum=False, renorm=True,
           ns="bf16", gemm_path=False):
    G = list(gradient(st, K, V, eta))
    if use_momentum:
        beta = np.float32(np.mean(_f32(mom))) if mom is not None and len(mom) else np.float32(0)
        st.M1 = (G[0] + beta * st.M1).astype(np.float32)
        st.M3 = (G[1] + beta * st.M3).astype(np.float32)
        st.M2 = (G[2] + beta * st.M2).astype(np.float32)
        G = [st.M1, st.M3, st.M2]
    if use_muon:
        G = [newton_schulz(x, ns=ns, gemm_path=gemm_path) for x in G]
    for name, nname, U in (("W1", "n1", G[0]), ("W3", "n3", G[1]), ("W2", "n2", G[2])):
        W = (getattr(st, name) + U).astype(np.float32)
        if renorm:
            nr = np.sqrt(np.sum(W.astype(np.float64) ** 2, axis=1)).astype(np.float32)
            W = (W * (getattr(st, nname) / (nr + np.float32(1e-5)))[:, None]).astype(np.float32)
        setattr(st, name, W)
    st.refresh()


def sequence(W1, W3, W2, Q, K, V, eta, chunk, mom=None, order=0, subset=None, update_last=False,
             use_muon=False, use_momentum=False, renorm=True, ns="bf16", op="bf16", n_chunks=None):
    """Whole sequence of one head with the kernels' rounding; returns the
    outputs [T, d] (float32) and the final State.  Matrices with more than
    128 rows in the wide orientation (d = 256) take the batched GEMM path."""
    gemm_path = W2.shape[0] > 128
    st = State(W1, W3, W2, op=op)
    T = Q.shape[0]
    O = np.zeros((T, W2.shape[0]), dtype=np.float32)
    bounds = [(s, min(s + chunk, T)) for s in range(0, T, chunk)]
    if n_chunks is not None:
        bounds = bounds[:n_chunks]

    def write(s, e):
        a, b = (s, e) if subset is None else (s + subset[0], min(s + subset[0] + subset[1], e))
        if b > a:
            update(st, K[a:b], V[a:b], eta[a:b], None if mom is None else mom[a:b], use_muon=use_muon,
                   use_momentum=use_momentum, renorm=renorm, ns=ns, gemm_path=gemm_path)

    for ci, (s, e) in enumerate(bounds):
        last = s + chunk >= T
        if order == 0:
            O[s:e] = apply(st, Q[s:e])
            if not last or update_last:
                write(s, e)
        else:
            write(s, e)
            O[s:e] = apply(st, Q[s:e])
    return O, st
