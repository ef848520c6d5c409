"""Parity at the workloads' full sizes, in the launch configuration that
bench.py times (one lact_sequence call over the whole sequence).

The oracle cannot replay a full sequence in seconds, so:
  1. the whole sequence runs once through lact_sequence (as bench.py does);
  2. it runs again one chunk per lact_sequence call, continuing the state
     (resume), and must give bitwise the same outputs and final state;
  3. at sampled chunks of the second run the GPU state W_c (and M_c) is copied
     back and, on sampled heads, the oracle computes that chunk from it
     (teacher forcing): the chunk's outputs and the state W_{c+1} (M_{c+1})
     must match within the bf16 bar (relative Frobenius 2e-2).
"""
import numpy as np
import pytest

from chunk_test_head_amd import _lib as L
from chunk_test_head_amd import workloads as WL
from oracle import lact_oracle as O
from tests import gpu_helpers as H
from tests import rounding_model as RM

pytestmark = pytest.mark.gpu

# workload -> (sampled chunks, sampled heads, sampled apply tokens per head)
SAMPLES = {
    1: ([0, 7, 14, 15], [0, 31], None),
    2: ([0], [0, 5], 4096),
    3: ([0, 3, 6], [0, 39], None),
    4: ([0, 40, 62, 63], [0, 3], 4096),
}


def _dev_inputs(w, inp, dev):
    import torch
    q, k, v = (torch.from_numpy(inp[n + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
               for n in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(dev)
    mom = torch.from_numpy(inp["mom"]).to(dev) if inp["mom"] is not None else None
    return q, k, v, eta, mom


def _snapshot(fw):
    W1, W3, W2, M1, M3, M2 = H.state64(fw)
    n = (H.to64(fw.n1), H.to64(fw.n3), H.to64(fw.n2))
    return (W1, W3, W2), (M1, M3, M2), n


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wi", [1, 2, 3, 4])
def test_full_size_sampled_chunks(device, wi):
    import torch
    w = WL.WORKLOADS[wi]
    chunks, heads, n_apply = SAMPLES[wi]
    print(f"full size {w.name}: generating inputs", flush=True)
    W = WL.weights(w)
    inp = WL.tokens(w, threads=16, values=False)
    q, k, v, eta, mom = _dev_inputs(w, inp, device)
    shape = H.shape_of(w)
    o = H.opts_of(w)
    max_upd = max(z - a for _, a, z in w.writes())
    ws = torch.empty(L.workspace_bytes(shape, max_upd, o), dtype=torch.uint8, device=device)

    # 1. whole sequence, as bench.py runs it
    print(f"full size {w.name}: whole sequence", flush=True)
    out_full = torch.empty_like(q)
    fw_full = H.make_state(w, W, device)
    L.lact_sequence(shape, fw_full, q, k, v, out_full, eta, eta, eta, mom, w.T, w.chunk, w.order,
                    w.subset, int(w.update_last), o, ws)
    torch.cuda.synchronize()

    # 2. one chunk per call, continuing the state
    print(f"full size {w.name}: chunk by chunk", flush=True)
    out_step = torch.empty_like(q)
    fw = H.make_state(w, W, device)
    bounds = w.chunk_bounds()
    snaps = {}
    for ci, (s, e) in enumerate(bounds):
        if ci in chunks:
            torch.cuda.synchronize()
            snaps[ci] = _snapshot(fw)
        last = ci == len(bounds) - 1
        mom_c = mom[:, s:] if mom is not None else None
        L.lact_sequence(shape, fw, q[:, s:], k[:, s:], v[:, s:], out_step[:, s:], eta[:, s:], eta[:, s:],
                        eta[:, s:], mom_c, e - s, w.chunk, w.order, w.subset,
                        0 if last else 1, o, ws,
                        layouts=(L.layout_of(q), L.layout_of(k), L.layout_of(v), L.layout_of(out_step)))
        if ci in chunks:
            torch.cuda.synchronize()
            snaps[ci] = snaps[ci] + (_snapshot(fw),)
    torch.cuda.synchronize()
    assert torch.equal(out_full.view(torch.int16), out_step.view(torch.int16)), "resume is not bitwise"
    assert torch.equal(fw_full.w1, fw.w1) and torch.equal(fw_full.w2, fw.w2)

    # 3. teacher-forced oracle steps at the sampled chunks
    got = out_step
    for ci in chunks:
        (Wc, Mc, n0, (Wn, Mn, _)) = snaps[ci]
        s, e = bounds[ci]
        last = ci == len(bounds) - 1
        for b in heads:
            st = O.HeadState(Wc[0][b], Wc[1][b], Wc[2][b])
            st.n1, st.n3, st.n2 = n0[0][b], n0[1][b], n0[2][b]
            if Mc[0] is not None:
                st.M1, st.M3, st.M2 = Mc[0][b], Mc[1][b], Mc[2][b]
            if w.subset is not None:
                a0, a1 = s + w.subset[0], min(s + w.subset[0] + w.subset[1], e)
            else:
                a0, a1 = s, e
            write = (w.order == WL.ORDER_UPDATE_THEN_APPLY) or not last
            new = st
            if write:
                ev = inp["eta"][b, a0:a1]
                mv = None if inp["mom"] is None else inp["mom"][b, a0:a1]
                new = O.update(st, WL.token_values(inp, "k", b, a0, a1), WL.token_values(inp, "v", b, a0, a1),
                               ev, ev, ev, mom=mv, use_muon=w.use_muon, use_momentum=w.use_momentum,
                               renorm=w.renorm)
                for name, x, y in (("W1", Wn[0][b], new.W1), ("W3", Wn[1][b], new.W3), ("W2", Wn[2][b], new.W2)):
                    err = H.rel(x, y)
                    print(f"  {w.name} chunk {ci} head {b} {name}_next rel err {err:.2e}", flush=True)
                    assert err < 2e-2, (ci, b, name, err)
                if w.use_momentum:
                    assert H.rel(Mn[0][b], new.M1) < 2e-2 and H.rel(Mn[2][b], new.M2) < 2e-2
            # outputs of this chunk: read with W_c (apply-then-update) or with
            # the oracle's own W_{c+1} (update-then-apply; with one chunk that
            # is the oracle's end-to-end result from the exact initial state)
            rd = st if w.order == WL.ORDER_APPLY_THEN_UPDATE else new
            if n_apply is not None and e - s > n_apply:
                rng = np.random.default_rng(ci * 1000 + b)
                toks = np.sort(rng.choice(np.arange(s, e), n_apply, replace=False))
            else:
                toks = np.arange(s, e)
            qv = np.stack([WL.token_values(inp, "q", b, t, t + 1)[0] for t in toks]) if n_apply else \
                WL.token_values(inp, "q", b, s, e)
            ref = O.apply(rd.W1, rd.W3, rd.W2, qv)
            gv = got[b, torch.from_numpy(toks).to(got.device)].float().cpu().numpy()
            err = H.rel(gv, ref)
            print(f"  {w.name} chunk {ci} head {b} outputs rel err {err:.2e}", flush=True)
            assert err < 2e-2, (ci, b, err)


# workload -> heads replayed end to end by the oracle
E2E = {1: [0, 17], 3: [0, 21]}


def _gpu_run(w, W, q, k, v, eta, mom, device, prec):
    """Whole sequence on the GPU with Newton-Schulz precision `prec`;
    returns (outputs, float64 state)."""
    import torch
    max_upd = max(z - a for _, a, z in w.writes())
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm, ns_prec=prec)
    ws = torch.empty(L.workspace_bytes(H.shape_of(w), max_upd, o), dtype=torch.uint8, device=device)
    out = torch.empty_like(q)
    fw = H.make_state(w, W, device)
    L.lact_sequence(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, w.T, w.chunk, w.order, w.subset,
                    int(w.update_last), o, ws)
    torch.cuda.synchronize()
    return out, H.state64(fw)


def _oracle_head(w, W, inp, b):
    m = None if inp["mom"] is None else inp["mom"][b]
    e = inp["eta"][b]
    return O.sequence(W[0][b], W[1][b], W[2][b], WL.token_values(inp, "q", b, 0, w.T),
                      WL.token_values(inp, "k", b, 0, w.T), WL.token_values(inp, "v", b, 0, w.T), e, e, e,
                      w.chunk, mom=m, order=w.order, subset=w.subset, update_last=w.update_last,
                      use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)


def _model_head(w, W, inp, b, ns):
    m = None if inp["mom"] is None else inp["mom"][b]
    return RM.sequence(W[0][b], W[1][b], W[2][b], WL.token_values(inp, "q", b, 0, w.T),
                       WL.token_values(inp, "k", b, 0, w.T), WL.token_values(inp, "v", b, 0, w.T),
                       inp["eta"][b], w.chunk, mom=m, order=w.order, subset=w.subset,
                       update_last=w.update_last, use_muon=w.use_muon, use_momentum=w.use_momentum,
                       renorm=w.renorm, ns=ns)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wi", [1, 3])
def test_full_size_end_to_end(device, wi):
    """Whole sequence on the GPU, in the Newton-Schulz precision bench.py
    times (bf16 operands with the shifted last steps), against the oracle's
    own whole sequence from the exact initial state, on sampled heads: the
    outputs of every token and the final W1, W3, W2 (and momentum) within the
    bf16 bar.  The page's plain bf16 Newton-Schulz is run and reported too:
    with Muon every write maps the gradient through a polynomial that
    amplifies perturbations along small singular directions, so it drifts
    from the oracle chunk by chunk; its curve must follow the rounding
    model's (tests/rounding_model.py) within a factor of 1.2."""
    w = WL.WORKLOADS[wi]
    print(f"end to end {w.name}: inputs", flush=True)
    W = WL.weights(w)
    inp = WL.tokens(w, threads=16, values=False)
    q, k, v, eta, mom = _dev_inputs(w, inp, device)
    runs = {}
    for prec in (L.NS_BF16_SHIFTED, L.NS_BF16):
        runs[prec] = _gpu_run(w, W, q, k, v, eta, mom, device, prec)
    bounds = w.chunk_bounds()
    for b in E2E[wi]:
        ref, st = _oracle_head(w, W, inp, b)
        for prec, ns in ((L.NS_BF16_SHIFTED, "bf16-shifted"), (L.NS_BF16, "bf16")):
            out, (W1g, W3g, W2g, M1g, M3g, M2g) = runs[prec]
            got = out[b].float().cpu().numpy()
            err_o = H.rel(got, ref)
            errs_w = [H.rel(W1g[b], st.W1), H.rel(W3g[b], st.W3), H.rel(W2g[b], st.W2)]
            mod_o, mod_st = _model_head(w, W, inp, b, ns)
            err_m = H.rel(mod_o, ref)
            curve = [H.rel(got[s:e], ref[s:e]) for s, e in bounds]
            print(f"  {w.name} head {b} ns={ns}: outputs {err_o:.2e} (model {err_m:.2e}), final "
                  f"W1 {errs_w[0]:.2e} W3 {errs_w[1]:.2e} W2 {errs_w[2]:.2e} (model W1 "
                  f"{H.rel(mod_st.W1, st.W1):.2e}); per chunk " + " ".join(f"{x:.1e}" for x in curve),
                  flush=True)
            assert 1 / 1.2 < err_o / err_m < 1.2, (b, ns, err_o, err_m)
            if prec == L.NS_BF16_SHIFTED:
                assert err_o < 2e-2, (b, err_o)
                assert max(errs_w) < 2e-2, (b, errs_w)
                if M1g is not None:
                    assert H.rel(M1g[b], st.M1) < 2e-2 and H.rel(M2g[b], st.M2) < 2e-2


@pytest.mark.timeout(900)
def test_long_context_drift_is_the_rounding_models(device):
    """Long-context (63 writes of 16384 tokens, d = 256, Muon + momentum):
    no Newton-Schulz precision holds the 2e-2 bar end to end, because the
    bf16 operands of the read and gradient contractions alone (weights and
    SwiGLU intermediates) drift by about 8e-2 over 63 writes in the rounding
    model with fp32-accurate Newton-Schulz.  So this test pins the drift
    instead: on one head, the GPU's error curve against the oracle (outputs
    of every chunk, cumulative, and the final weights) for the benched and
    the page's precision must stay within a factor of 1.2 of the rounding
    model's curve at chunks 1, 8, 16, 32 and 63; the first chunk, read with
    the exact initial weights, is within 2e-2; and the per-step error
    (test_full_size_sampled_chunks) stays within 2e-2 everywhere."""
    w = WL.WORKLOADS[4]
    b = 2
    print(f"long-context drift: inputs", flush=True)
    W = WL.weights(w)
    inp = WL.tokens(w, threads=16, values=False)
    q, k, v, eta, mom = _dev_inputs(w, inp, device)
    runs = {prec: _gpu_run(w, W, q, k, v, eta, mom, device, prec) for prec in (L.NS_BF16_SHIFTED, L.NS_BF16)}
    got = {prec: r[0][b].float().cpu().numpy() for prec, r in runs.items()}
    fin = {prec: r[1] for prec, r in runs.items()}
    del runs
    print("long-context drift: oracle", flush=True)
    ref, st = _oracle_head(w, W, inp, b)
    bounds = w.chunk_bounds()
    marks = [1, 8, 16, 32, 63]
    for prec, ns in ((L.NS_BF16_SHIFTED, "bf16-shifted"), (L.NS_BF16, "bf16")):
        print(f"long-context drift: rounding model {ns}", flush=True)
        mod_o, mod_st = _model_head(w, W, inp, b, ns)
        g = got[prec]
        cum_g = [H.rel(g[:bounds[c][1]], ref[:bounds[c][1]]) for c in marks]
        cum_m = [H.rel(mod_o[:bounds[c][1]], ref[:bounds[c][1]]) for c in marks]
        curve = [H.rel(g[s:e], ref[s:e]) for s, e in bounds]
        W1g = fin[prec][0][b]
        print(f"  long-context head {b} ns={ns}: cumulative outputs at chunks {marks}: GPU "
              + " ".join(f"{x:.2e}" for x in cum_g) + " model " + " ".join(f"{x:.2e}" for x in cum_m)
              + f"; final W1 GPU {H.rel(W1g, st.W1):.2e} model {H.rel(mod_st.W1, st.W1):.2e}; per chunk "
              + " ".join(f"{x:.1e}" for x in curve[::4]), flush=True)
        assert curve[0] < 2e-2
        for c, x, y in zip(marks, cum_g, cum_m):
            assert 1 / 1.2 < x / y < 1.2, (ns, c, x, y)
        assert 1 / 1.2 < H.rel(W1g, st.W1) / H.rel(mod_st.W1, st.W1) < 1.2
