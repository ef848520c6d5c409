"""GPU parity of every C-ABI entry point against the float64 oracle, at sizes
the oracle finishes in seconds that still span several tiles and a ragged
tail.  Bar: relative Frobenius error 2e-2 (bf16 operands) / 1e-4 (fp32)."""
import numpy as np
import pytest

from chunk_test_head_amd import _lib as L
from chunk_test_head_amd import workloads as WL
from oracle import lact_oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

# one reduced case per workload family: (workload, bh, n_tok)
FAMILIES = {
    0: dict(heads=1, batch=1),
    1: dict(heads=2, batch=1),
    2: dict(heads=2, batch=1),
    3: dict(heads=2, batch=1),
    4: dict(heads=1, batch=2),
}


def small(wi, T, chunk, subset=None):
    w = WL.WORKLOADS[wi]
    kw = dict(FAMILIES[wi])
    kw.update(T=T, chunk=chunk)
    if w.subset is not None or subset is not None:
        kw["subset"] = subset if subset is not None else (w.subset and (0, 0))
    return w.scaled(**kw)


def inputs(w):
    return WL.weights(w), WL.tokens(w)


@pytest.mark.parametrize("wi", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("n_tok", [1, 300, 613])
def test_apply(device, wi, n_tok):
    import torch
    w = small(wi, n_tok, n_tok, subset=(0, n_tok))
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    q = H.act_to_dev(w, inp, "q", device)
    out = H.out_buffer(w, n_tok, device)
    print(f"apply wl={wi} bh={w.bh} n={n_tok}", flush=True)
    L.lact_apply(fw.shape, fw, q, out)
    torch.cuda.synchronize()
    got = H.to64(out)
    for b in range(w.bh):
        ref = O.apply(W[0][b], W[1][b], W[2][b], inp["q"][b])
        assert H.rel(got[b], ref) < H.TOL[w.dtype], (b, H.rel(got[b], ref))
    # state untouched and the shadow consistent with it
    assert np.array_equal(H.to64(fw.w1), W[0].astype(np.float64))


@pytest.mark.parametrize("wi", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("n_tok", [37, 700])
def test_gradient(device, wi, n_tok):
    import torch
    w = small(wi, n_tok, n_tok, subset=(0, n_tok))
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    k = H.act_to_dev(w, inp, "k", device)
    v = H.act_to_dev(w, inp, "v", device)
    eta = torch.from_numpy(inp["eta"]).to(device)
    g = [torch.full((w.bh, w.d, w.dh), float("nan"), device=device) for _ in range(3)]
    ws = H.workspace(w, n_tok, device, muon=False)
    print(f"gradient wl={wi} bh={w.bh} n={n_tok}", flush=True)
    L.lact_gradient(fw.shape, fw, k, v, eta, eta, eta, g[0], g[1], g[2], ws)
    torch.cuda.synchronize()
    got = [H.to64(x) for x in g]
    for b in range(w.bh):
        e = inp["eta"][b]
        G1, G3, G2 = O.chunk_gradient(W[0][b], W[1][b], W[2][b], inp["k"][b], inp["v"][b], e, e, e)
        for name, x, ref in (("G1", got[0][b].T, G1), ("G3", got[1][b].T, G3), ("G2", got[2][b], G2)):
            assert H.rel(x, ref) < H.TOL[w.dtype], (name, b, H.rel(x, ref))


@pytest.mark.parametrize("dh", [256, 320, 448])
def test_d256_hidden_sizes(device, dh):
    """d = 256 with hidden sizes other than the workloads' 1024: the read
    streams dh / 32 hidden blocks through its two LDS stages of W1 / W3 rows
    and of W2 (8, 10 and 14 blocks here), the gradient launches dh / 64
    hidden-block workgroups; ragged token counts span several tiles and,
    for the gradient, several splits."""
    import dataclasses
    import torch
    base = dataclasses.replace(WL.WORKLOADS[4], dh=dh, name=f"long-context-dh{dh}")
    for n_tok in (130, 613):
        w = base.scaled(heads=1, batch=2, T=n_tok, chunk=n_tok)
        W, inp = inputs(w)
        fw = H.make_state(w, W, device)
        q = H.act_to_dev(w, inp, "q", device)
        out = H.out_buffer(w, n_tok, device)
        print(f"apply d=256 dh={dh} bh={w.bh} n={n_tok}", flush=True)
        L.lact_apply(fw.shape, fw, q, out)
        torch.cuda.synchronize()
        got = H.to64(out)
        for b in range(w.bh):
            ref = O.apply(W[0][b], W[1][b], W[2][b], inp["q"][b])
            assert H.rel(got[b], ref) < H.TOL[w.dtype], ("apply", n_tok, b, H.rel(got[b], ref))
    n_tok = 1500
    w = base.scaled(heads=1, batch=2, T=n_tok, chunk=n_tok)
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    k = H.act_to_dev(w, inp, "k", device)
    v = H.act_to_dev(w, inp, "v", device)
    eta = torch.from_numpy(inp["eta"]).to(device)
    g = [torch.full((w.bh, w.d, w.dh), float("nan"), device=device) for _ in range(3)]
    ws = H.workspace(w, n_tok, device, muon=False)
    print(f"gradient d=256 dh={dh} bh={w.bh} n={n_tok}", flush=True)
    L.lact_gradient(fw.shape, fw, k, v, eta, eta, eta, g[0], g[1], g[2], ws)
    torch.cuda.synchronize()
    got = [H.to64(x) for x in g]
    for b in range(w.bh):
        e = inp["eta"][b]
        G1, G3, G2 = O.chunk_gradient(W[0][b], W[1][b], W[2][b], inp["k"][b], inp["v"][b], e, e, e)
        for name, x, ref in (("G1", got[0][b].T, G1), ("G3", got[1][b].T, G3), ("G2", got[2][b], G2)):
            assert H.rel(x, ref) < H.TOL[w.dtype], (name, b, H.rel(x, ref))


def test_gradient_distinct_etas(device):
    """eta1 / eta3 / eta2 reach only their own matrix."""
    import torch
    w = small(1, 200, 200, subset=(0, 200))
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    k = H.act_to_dev(w, inp, "k", device)
    v = H.act_to_dev(w, inp, "v", device)
    rng = np.random.default_rng(5)
    etas = [np.abs(rng.standard_normal((w.bh, w.T))).astype(np.float32) * 0.01 for _ in range(3)]
    et = [torch.from_numpy(e).to(device) for e in etas]
    g = [torch.empty((w.bh, w.d, w.dh), device=device) for _ in range(3)]
    ws = H.workspace(w, w.T, device, muon=False)
    L.lact_gradient(fw.shape, fw, k, v, et[0], et[1], et[2], g[0], g[1], g[2], ws)
    torch.cuda.synchronize()
    for b in range(w.bh):
        G1, G3, G2 = O.chunk_gradient(W[0][b], W[1][b], W[2][b], inp["k"][b], inp["v"][b],
                                      etas[0][b], etas[1][b], etas[2][b])
        assert H.rel(H.to64(g[0])[b].T, G1) < 2e-2
        assert H.rel(H.to64(g[1])[b].T, G3) < 2e-2
        assert H.rel(H.to64(g[2])[b], G2) < 2e-2


NS_PRECS = [(L.NS_BF16_SHIFTED, 2e-2), (L.NS_BF16, 2e-2), (L.NS_F32, 1e-4)]


@pytest.mark.parametrize("prec,tol", NS_PRECS)
@pytest.mark.parametrize("rows,cols", [(128, 512), (128, 256), (256, 1024), (64, 128), (64, 256), (64, 512),
                                       (128, 192), (192, 320)])
def test_newton_schulz(device, prec, tol, rows, cols):
    import torch
    # a gradient-like input: oracle chunk gradient of a random head
    w = WL.WORKLOADS[1].scaled(heads=1, batch=1, T=512, chunk=512)
    rng = np.random.default_rng(rows + cols)
    Gs = []
    for i in range(3):
        A = rng.standard_normal((rows, 8)) @ rng.standard_normal((8, cols))
        Gs.append(A + 0.05 * rng.standard_normal((rows, cols)))
    g = torch.from_numpy(np.stack(Gs).astype(np.float32)).to(device)
    u = torch.full_like(g, float("nan"))
    ws = torch.empty(L.ns_workspace_bytes(3, rows, cols) // 4 + 1, device=device)
    print(f"ns prec={L.NS_PREC_NAMES[prec]} {rows}x{cols}", flush=True)
    L.lact_newton_schulz(g, u, ws, prec=prec)
    torch.cuda.synchronize()
    got = H.to64(u)
    for i in range(3):
        ref = O.newton_schulz5(g[i].cpu().numpy().astype(np.float64))
        assert H.rel(got[i], ref) < tol, (i, H.rel(got[i], ref))


@pytest.mark.parametrize("prec,tol", NS_PRECS)
@pytest.mark.parametrize("rows,cols", [(128, 512), (128, 256), (256, 1024)])
def test_newton_schulz_degenerate(device, prec, tol, rows, cols):
    """Degenerate inputs (Muon orthogonalisation, quintic Newton-Schulz of the
    LaCT pages): a zero gradient stays exactly zero (the norm guard eps keeps
    the scale finite), a rank-one gradient, and one whose norm is far below
    eps (its Gram products underflow; the iterate is then the scaled input
    times the product of the a coefficients, as in the oracle)."""
    import torch
    rng = np.random.default_rng(7 + cols)
    Gs = [np.zeros((rows, cols)),
          np.outer(rng.standard_normal(rows), rng.standard_normal(cols)),
          1e-30 * rng.standard_normal((rows, cols))]
    g = torch.from_numpy(np.stack(Gs).astype(np.float32)).to(device)
    u = torch.full_like(g, float("nan"))
    ws = torch.empty(L.ns_workspace_bytes(3, rows, cols) // 4 + 1, device=device)
    print(f"ns degenerate prec={L.NS_PREC_NAMES[prec]} {rows}x{cols}", flush=True)
    L.lact_newton_schulz(g, u, ws, prec=prec)
    torch.cuda.synchronize()
    got = H.to64(u)
    assert np.all(got[0] == 0.0)
    for i in (1, 2):
        ref = O.newton_schulz5(g[i].cpu().numpy().astype(np.float64))
        if i == 1 and prec == L.NS_F32:
            # rank one: the result is phi(1) u v^T.  Its u v^T component must
            # hold the fp32 bar; the rest is fp32 rounding noise in the null
            # directions, which the quintics grow by up to the product of the
            # a coefficients (about 493) as they grow any small singular
            # value, so it is bounded by 1e-3 instead.
            u_, s_, vt_ = np.linalg.svd(ref, full_matrices=False)
            uu, vv = u_[:, 0], vt_[0]
            coef = float(uu @ got[i] @ vv)
            assert abs(coef - s_[0]) < 1e-4 * s_[0], (coef, s_[0])
            resid = got[i] - coef * np.outer(uu, vv)
            assert np.linalg.norm(resid) < 1e-3 * np.linalg.norm(ref), np.linalg.norm(resid)
            continue
        assert H.rel(got[i], ref) < tol, (i, H.rel(got[i], ref))


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("wi", [0, 1, 2, 3, 4])
def test_step_renorm(device, wi, renorm):
    """W <- W + U (+ row renorm) on the masters, then a read through the
    operand copies the step rewrote (W1, W3, W2 and W2^T) against the oracle's
    read with the new weights."""
    import torch
    w = small(wi, 64, 64, subset=(0, 64))
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    rng = np.random.default_rng(wi)
    U = [rng.standard_normal((w.bh, w.d, w.dh)).astype(np.float32) * 0.05 for _ in range(3)]
    u = [torch.from_numpy(x).to(device) for x in U]
    ws = H.workspace(w, 0, device)
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=renorm)
    L.lact_step_renorm(fw.shape, fw, u[0], u[1], u[2], o, ws)
    q = H.act_to_dev(w, inp, "q", device)
    out = H.out_buffer(w, w.T, device)
    L.lact_apply(fw.shape, fw, q, out)
    torch.cuda.synchronize()
    W1, W3, W2 = H.to64(fw.w1), H.to64(fw.w3), H.to64(fw.w2)
    got = H.to64(out)
    tol_o = 2e-2 if w.dtype == "bf16" else 1e-4
    for b in range(w.bh):
        if renorm:
            n1, n3, n2 = O.row_norms(W[0][b]), O.row_norms(W[1][b]), O.row_norms(W[2][b])
            e1 = O.step_renorm(W[0][b], U[0][b].T, n1)
            e3 = O.step_renorm(W[1][b], U[1][b].T, n3)
            e2 = O.step_renorm(W[2][b], U[2][b], n2)
        else:
            e1 = W[0][b].astype(np.float64) + U[0][b].T
            e3 = W[1][b].astype(np.float64) + U[1][b].T
            e2 = W[2][b].astype(np.float64) + U[2][b]
        assert H.rel(W1[b], e1) < 1e-5
        assert H.rel(W3[b], e3) < 1e-5
        assert H.rel(W2[b], e2) < 1e-5
        ref = O.apply(e1, e3, e2, WL.token_values(inp, "q", b, 0, w.T))
        assert H.rel(got[b], ref) < tol_o, (b, H.rel(got[b], ref))
    assert H.rel(H.to64(fw.n1), np.stack([O.row_norms(x) for x in W[0]])) < 1e-6
    H.check_shadow(fw)


@pytest.mark.parametrize("wi", [0, 1, 3, 4])
def test_update_twice(device, wi):
    """Two writes (momentum buffer non-zero on the second) from the same state."""
    import torch
    w = small(wi, 2 * 320, 320, subset=(0, 320))
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    k = H.act_to_dev(w, inp, "k", device)
    v = H.act_to_dev(w, inp, "v", device)
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    ws = H.workspace(w, 320, device)
    o = H.opts_of(w)
    sts = [O.HeadState(W[0][b], W[1][b], W[2][b]) for b in range(w.bh)]
    for c in range(2):
        sl = slice(320 * c, 320 * (c + 1))
        L.lact_update(fw.shape, fw, k[:, sl], v[:, sl], eta[:, sl], eta[:, sl], eta[:, sl],
                      None if mom is None else mom[:, sl], o, ws)
        torch.cuda.synchronize()
        W1, W3, W2, M1, M3, M2 = H.state64(fw)
        for b in range(w.bh):
            e = inp["eta"][b, sl]
            m = None if inp["mom"] is None else inp["mom"][b, sl]
            # teacher-forced: the oracle step starts from the GPU's W_c
            ref = O.update(sts[b], inp["k"][b, sl], inp["v"][b, sl], e, e, e, mom=m,
                           use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
            for name, x, y in (("W1", W1[b], ref.W1), ("W3", W3[b], ref.W3), ("W2", W2[b], ref.W2)):
                assert H.rel(x, y) < H.TOL[w.dtype], (c, name, b, H.rel(x, y))
            if w.use_momentum:
                assert H.rel(M1[b], ref.M1) < H.TOL[w.dtype]
                assert H.rel(M2[b], ref.M2) < H.TOL[w.dtype]
            st = H.oracle_state(O, W1[b], W3[b], W2[b], sts[b].n1, sts[b].n3, sts[b].n2,
                                None if M1 is None else (M1[b], M3[b], M2[b]))
            sts[b] = st
        H.check_shadow(fw)


@pytest.mark.parametrize("wi,n", [(0, 320), (1, 320), (1, 1), (3, 320), (3, 17), (4, 320)])
def test_chunk_step(device, wi, n):
    """One chunk step (read with W_c, then write): with Newton-Schulz on and
    d = 128 the read shares the Newton-Schulz launch (its workgroups after
    the matrices'), otherwise it runs first.  Both results against the oracle
    (also a one-token and a 17-token chunk)."""
    import torch
    w = small(wi, n, n, subset=(0, n))
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    q = H.act_to_dev(w, inp, "q", device)
    k = H.act_to_dev(w, inp, "k", device)
    v = H.act_to_dev(w, inp, "v", device)
    out = H.out_buffer(w, n, device)
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    ws = H.workspace(w, n, device)
    print(f"chunk_step wl={wi} n={n}", flush=True)
    L.lact_chunk_step(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, H.opts_of(w), ws)
    torch.cuda.synchronize()
    got = H.to64(out)
    W1, W3, W2, M1, M3, M2 = H.state64(fw)
    for b in range(w.bh):
        ref_o = O.apply(W[0][b], W[1][b], W[2][b], WL.token_values(inp, "q", b, 0, n))
        assert H.rel(got[b], ref_o) < H.TOL[w.dtype], (b, H.rel(got[b], ref_o))
        e = inp["eta"][b]
        m = None if inp["mom"] is None else inp["mom"][b]
        ref = O.update(O.HeadState(W[0][b], W[1][b], W[2][b]), inp["k"][b], inp["v"][b], e, e, e,
                       mom=m, use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
        for name, x, y in (("W1", W1[b], ref.W1), ("W3", W3[b], ref.W3), ("W2", W2[b], ref.W2)):
            assert H.rel(x, y) < H.TOL[w.dtype], (name, b, H.rel(x, y))
    H.check_shadow(fw)


SEQ_CASES = {
    # workload: (T, chunk, subset)
    0: (1024, 256, None),
    1: (4 * 256 + 100, 256, None),
    2: (1024, 1024, (0, 768)),
    3: (3 * 512, 512, (256, 256)),
    4: (3 * 384, 384, None),
}


@pytest.mark.parametrize("wi", [0, 1, 2, 3, 4])
def test_sequence_end_to_end(device, wi):
    T, C, sub = SEQ_CASES[wi]
    w = small(wi, T, C, subset=sub)
    if wi == 0:
        w = WL.WORKLOADS[0]   # the tiny fp32 workload at its full size
    W, inp = inputs(w)
    print(f"sequence wl={wi} T={w.T} C={w.chunk}", flush=True)
    got, fw = H.run_sequence(w, inp, W, device)
    W1, W3, W2, *_ = H.state64(fw)
    for b in range(w.bh):
        m = None if inp["mom"] is None else inp["mom"][b]
        e = inp["eta"][b]
        ref, st = O.sequence(W[0][b], W[1][b], W[2][b], inp["q"][b], inp["k"][b], inp["v"][b], e, e, e,
                             w.chunk, mom=m, order=w.order, subset=w.subset, update_last=w.update_last,
                             use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
        assert H.rel(got[b], ref) < H.TOL[w.dtype], (b, H.rel(got[b], ref))
        assert H.rel(W1[b], st.W1) < H.TOL[w.dtype]
        assert H.rel(W2[b], st.W2) < H.TOL[w.dtype]
    H.check_shadow(fw)


@pytest.mark.parametrize("dh", [256, 512])
def test_sequence_bf16_d64(device, dh):
    """bf16 operands at d = 64 (a supported shape no workload uses): the
    d = 64 read and gradient kernels, the one-launch Newton-Schulz of 64 x dh,
    momentum and renorm, over a causal sequence with a ragged last chunk,
    against the oracle."""
    import dataclasses
    w = dataclasses.replace(WL.WORKLOADS[1], d=64, dh=dh, heads=2, batch=1, T=3 * 128 + 50, chunk=128,
                            name=f"lm-causal-d64-dh{dh}")
    W, inp = inputs(w)
    print(f"sequence bf16 d=64 dh={dh} T={w.T} C={w.chunk}", flush=True)
    got, fw = H.run_sequence(w, inp, W, device)
    W1, W3, W2, *_ = H.state64(fw)
    for b in range(w.bh):
        m = None if inp["mom"] is None else inp["mom"][b]
        e = inp["eta"][b]
        ref, st = O.sequence(W[0][b], W[1][b], W[2][b], inp["q"][b], inp["k"][b], inp["v"][b], e, e, e,
                             w.chunk, mom=m, order=w.order, subset=w.subset, update_last=w.update_last,
                             use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
        assert H.rel(got[b], ref) < H.TOL[w.dtype], (b, H.rel(got[b], ref))
        assert H.rel(W1[b], st.W1) < H.TOL[w.dtype]
        assert H.rel(W2[b], st.W2) < H.TOL[w.dtype]
    H.check_shadow(fw)


def test_sequence_f32_d128(device):
    """fp32 activations and operands at d = 128 (the fp32 read and gradient
    kernels, Newton-Schulz with fp32 operands, momentum, renorm) over a
    causal sequence with a ragged last chunk, against the oracle (bar 1e-4)."""
    import dataclasses
    w = dataclasses.replace(WL.WORKLOADS[1], dtype="f32", d=128, dh=256, heads=2, batch=1,
                            T=3 * 128 + 50, chunk=128, name="lm-causal-f32-d128")
    W, inp = inputs(w)
    print(f"sequence f32 d=128 T={w.T} C={w.chunk}", flush=True)
    got, fw = H.run_sequence(w, inp, W, device)
    W1, W3, W2, *_ = H.state64(fw)
    for b in range(w.bh):
        m = None if inp["mom"] is None else inp["mom"][b]
        e = inp["eta"][b]
        ref, st = O.sequence(W[0][b], W[1][b], W[2][b], inp["q"][b], inp["k"][b], inp["v"][b], e, e, e,
                             w.chunk, mom=m, order=w.order, subset=w.subset, update_last=w.update_last,
                             use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
        assert H.rel(got[b], ref) < H.TOL[w.dtype], (b, H.rel(got[b], ref))
        assert H.rel(W1[b], st.W1) < H.TOL[w.dtype], (b, H.rel(W1[b], st.W1))
        assert H.rel(W2[b], st.W2) < H.TOL[w.dtype], (b, H.rel(W2[b], st.W2))


@pytest.mark.parametrize("wi", [1, 3])
def test_zero_tokens_write_nothing(device, wi):
    """Reads, writes and chunk steps of zero tokens return LACT_OK and leave
    the state (weights, norms, momentum, operand copies) and the output
    buffer bitwise unchanged."""
    import torch
    w = small(wi, 64, 64, subset=(0, 64))
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    q = H.act_to_dev(w, inp, "q", device)
    k = H.act_to_dev(w, inp, "k", device)
    v = H.act_to_dev(w, inp, "v", device)
    out = H.out_buffer(w, 64, device)
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    ws = H.workspace(w, 64, device)
    torch.cuda.synchronize()
    bufs = [fw.w1, fw.w3, fw.w2, fw.n1, fw.n3, fw.n2, fw.shadow] + \
        [m for m in (fw.m1, fw.m3, fw.m2) if m is not None]
    before = [b.clone() for b in bufs]
    print(f"zero tokens wl={wi}", flush=True)
    L.lact_apply(fw.shape, fw, q, out, n_tok=0)
    L.lact_update(fw.shape, fw, k, v, eta, eta, eta, mom, H.opts_of(w), ws, n_tok=0)
    L.lact_chunk_step(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, H.opts_of(w), ws, n_tok=0)
    torch.cuda.synchronize()
    for a, b in zip(bufs, before):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert torch.isnan(out.float()).all()



@pytest.mark.parametrize("wi,renorm", [(1, True), (3, True), (4, True), (2, False)])
def test_nonfinite_flag(device, wi, renorm):
    """lact_update_opts.nonfinite: a clean write leaves the flag at zero
    (lact_check_finite -> OK); a write whose values hold a NaN makes the new
    weights non-finite and sets it (-> LACT_ERR_NONFINITE).  Covers the
    fused Newton-Schulz + step epilogue (d = 128, Muon) and the step kernel."""
    import dataclasses
    import torch
    w = dataclasses.replace(small(wi, 96, 96, subset=(0, 96)), renorm=renorm)
    W, inp = inputs(w)
    fw = H.make_state(w, W, device)
    k = H.act_to_dev(w, inp, "k", device)
    v = H.act_to_dev(w, inp, "v", device)
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    ws = H.workspace(w, 96, device)
    flag = torch.zeros(4, dtype=torch.int32, device=device)
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=renorm, nonfinite=flag)
    print(f"nonfinite flag wl={wi} renorm={renorm}", flush=True)
    L.lact_update(fw.shape, fw, k, v, eta, eta, eta, mom, o, ws)
    assert L.lact_check_finite(flag) == L.OK
    v_bad = v.clone()
    v_bad[0, 5, 3] = float("nan")
    L.lact_update(fw.shape, fw, k, v_bad, eta, eta, eta, mom, o, ws)
    assert L.lact_check_finite(flag) == L.ERR_NONFINITE
    assert int(flag[0].item()) == 1 and not torch.isfinite(fw.w1[0]).all()
    # other heads are independent: their weights stay finite
    if w.bh > 1:
        assert torch.isfinite(fw.w1[1:]).all() and torch.isfinite(fw.w2[1:]).all()


@pytest.mark.parametrize("wi", [1, 2, 3, 4])
def test_sequence_master_variant(device, wi):
    """Master-state variant (renorm = 2; uTTT page section C.1): the fp32
    state accumulates W + U unscaled and the operand copies that reads and
    gradients use hold its rows rescaled to the sequence-start norms.  Whole
    sequences against the oracle's "master" mode: outputs, and the master
    state itself; the copies are the rescaled master rows."""
    import dataclasses
    import torch
    T, C, sub = SEQ_CASES[wi]
    w = small(wi, T, C, subset=sub)
    W, inp = inputs(w)
    q, k, v = (H.act_to_dev(w, inp, n, device) for n in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    out = H.out_buffer(w, w.T, device)
    fw = H.make_state(w, W, device)
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=2)
    max_upd = max(z - a for _, a, z in w.writes())
    ws = torch.full(((L.workspace_bytes(fw.shape, max_upd, o) + 3) // 4,), float("nan"), device=device)
    print(f"master variant wl={wi} T={w.T} C={w.chunk}", flush=True)
    L.lact_sequence(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, w.T, w.chunk, w.order, w.subset,
                    int(w.update_last), o, ws)
    torch.cuda.synchronize()
    got = H.to64(out)
    W1, W3, W2, *_ = H.state64(fw)
    for b in range(w.bh):
        m = None if inp["mom"] is None else inp["mom"][b]
        e = inp["eta"][b]
        ref, st = O.sequence(W[0][b], W[1][b], W[2][b], inp["q"][b], inp["k"][b], inp["v"][b], e, e, e,
                             w.chunk, mom=m, order=w.order, subset=w.subset, update_last=w.update_last,
                             use_muon=w.use_muon, use_momentum=w.use_momentum, renorm="master")
        assert H.rel(got[b], ref) < 2e-2, (b, H.rel(got[b], ref))
        assert H.rel(W1[b], st.S1) < 2e-2 and H.rel(W2[b], st.S2) < 2e-2
        # the master is not rescaled: its rows drift from the sequence-start
        # norms by far more than the renorm eps would (1e-5 relative)
        assert np.max(np.abs(np.sqrt((W1[b] ** 2).sum(1)) / st.n1 - 1.0)) > 1e-3
    m = w.d * w.dh
    sh = fw.shadow.view(torch.bfloat16).view(w.bh, 4, m).float().cpu().numpy().astype(np.float64)
    n1 = H.to64(fw.n1)
    for b in range(w.bh):
        want = W1[b] * (n1[b] / (np.sqrt((W1[b] ** 2).sum(1)) + 1e-5))[:, None]
        assert H.rel(sh[b, 0].reshape(w.dh, w.d), want) < 1e-2


@pytest.mark.parametrize("wi", [0, 1, 3])
def test_sequence_per_channel_eta(device, wi):
    """Per-channel learning rates (the rebuttal page's [b, l, d] learning-rate
    tensors): eta1, eta3 [bh, T, d] scale k channel by channel, eta2
    [bh, T, dh] the hidden units.  Whole sequences (Muon, momentum, subset
    as the family has them) against the oracle with the same rates."""
    import torch
    T, C, sub = SEQ_CASES[wi]
    w = small(wi, T, C, subset=sub)
    if wi == 0:
        w = WL.WORKLOADS[0].scaled(T=3 * 128 + 40, chunk=128)
    W, inp = inputs(w)
    rng = np.random.default_rng(40 + wi)
    sp = lambda shape: (np.log1p(np.exp(rng.standard_normal(shape))) * 1e-2).astype(np.float32)
    e1, e3, e2 = sp((w.bh, w.T, w.d)), sp((w.bh, w.T, w.d)), sp((w.bh, w.T, w.dh))
    q, k, v = (H.act_to_dev(w, inp, n, device) for n in ("q", "k", "v"))
    et = [torch.from_numpy(x).to(device) for x in (e1, e3, e2)]
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    out = H.out_buffer(w, w.T, device)
    fw = H.make_state(w, W, device)
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm, eta_per_channel=True)
    max_upd = max(z - a for _, a, z in w.writes())
    ws = torch.full(((L.workspace_bytes(fw.shape, max_upd, o) + 3) // 4,), float("nan"), device=device)
    print(f"per-channel eta wl={wi} T={w.T} C={w.chunk}", flush=True)
    L.lact_sequence(fw.shape, fw, q, k, v, out, et[0], et[1], et[2], mom, w.T, w.chunk, w.order, w.subset,
                    int(w.update_last), o, ws)
    torch.cuda.synchronize()
    got = H.to64(out)
    W1, W3, W2, *_ = H.state64(fw)
    for b in range(w.bh):
        m = None if inp["mom"] is None else inp["mom"][b]
        ref, st = O.sequence(W[0][b], W[1][b], W[2][b], inp["q"][b], inp["k"][b], inp["v"][b], e1[b], e3[b],
                             e2[b], w.chunk, mom=m, order=w.order, subset=w.subset, update_last=w.update_last,
                             use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
        assert H.rel(got[b], ref) < H.TOL[w.dtype], (b, H.rel(got[b], ref))
        assert H.rel(W1[b], st.W1) < H.TOL[w.dtype] and H.rel(W2[b], st.W2) < H.TOL[w.dtype]
    H.check_shadow(fw)


def test_sequence_forked_read_is_bitwise_the_plain_read(device):
    """d = 256 with Muon: lact_sequence runs each chunk's read on the
    library's second stream beside the write's Newton-Schulz, with fewer
    workgroups than 128-token tiles (each loops over several).  Chunks of
    16384 tokens on two heads (256 tiles) take that path; the outputs and
    the final state must equal, bit for bit, the same sequence composed of
    lact_apply (one workgroup per tile, caller's stream) and lact_update."""
    import torch
    C = 16384
    w = WL.WORKLOADS[4].scaled(heads=2, batch=1, T=2 * C + 300, chunk=C)
    W, inp = inputs(w)
    q, k, v = (H.act_to_dev(w, inp, n, device) for n in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device)
    o = H.opts_of(w)
    print(f"forked read T={w.T} chunk={C} bh={w.bh}", flush=True)
    out_seq, fw_seq = H.run_sequence(w, inp, W, device)
    fw = H.make_state(w, W, device)
    out = H.out_buffer(w, w.T, device)
    ws = H.workspace(w, C, device)
    lay = L.layout_of(q)
    for s0, e0 in w.chunk_bounds():
        L.lact_apply(fw.shape, fw, q[:, s0:e0], out[:, s0:e0], q_layout=lay, o_layout=L.layout_of(out))
        if e0 < w.T:
            L.lact_update(fw.shape, fw, k[:, s0:e0], v[:, s0:e0], eta[:, s0:e0], eta[:, s0:e0], eta[:, s0:e0],
                          mom[:, s0:e0], o, ws, k_layout=lay, v_layout=lay)
    torch.cuda.synchronize()
    assert np.array_equal(H.to64(out), out_seq)
    for name in ("w1", "w3", "w2", "m1", "m3", "m2", "shadow"):
        a, b = getattr(fw, name), getattr(fw_seq, name)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
