"""Shared set-up of GPU parity tests: upload the seeded inputs, run the HIP
path through the C ABI, bring results back as float64 for the oracle."""
from __future__ import annotations

import numpy as np

from chunk_test_head_amd import _lib as L
from chunk_test_head_amd import workloads as WL

TOL = {"bf16": 2e-2, "f32": 1e-4}


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def shape_of(w):
    return L.Shape(w.bh, w.d, w.dh, L.BF16 if w.dtype == "bf16" else L.F32)


def opts_of(w):
    return L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)


def act_to_dev(w, inp, name, dev):
    import torch
    if w.dtype == "bf16":
        bits = inp[name + "_bits"]
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(inp[name]).to(dev)


def out_buffer(w, T, dev):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return torch.full((w.bh, T, w.d), float("nan"), dtype=dt, device=dev)


def to64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def make_state(w, W, dev, momentum=None):
    import torch
    W1, W3, W2 = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in W)
    fw = L.FastWeights(shape_of(w), W1, W3, W2, momentum=w.use_momentum if momentum is None else momentum)
    L.lact_init_state(fw.shape, fw)
    return fw


def workspace(w, max_tok, dev, muon=None):
    import torch
    o = opts_of(w)
    if muon is not None:
        o.use_muon = int(muon)
    n = L.workspace_bytes(shape_of(w), max_tok, o)
    # NaN-filled: a kernel that reads scratch it never wrote shows up as NaN
    return torch.full(((n + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)


def run_sequence(w, inp, W, dev, stream=None):
    """Whole sequence through lact_sequence; returns (O float64, FastWeights)."""
    import torch
    q, k, v = (act_to_dev(w, inp, n, dev) for n in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(dev)
    mom = torch.from_numpy(inp["mom"]).to(dev) if inp["mom"] is not None else None
    out = out_buffer(w, w.T, dev)
    fw = make_state(w, W, dev)
    max_upd = min(w.chunk, w.T) if w.subset is None else min(w.subset[1], w.chunk - w.subset[0], w.T)
    ws = workspace(w, max_upd, dev)
    L.lact_sequence(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, w.T, w.chunk, w.order, w.subset,
                    int(w.update_last), opts_of(w), ws, stream=stream)
    torch.cuda.synchronize()
    return to64(out), fw


def state64(fw):
    """GPU state as float64 numpy, per head: (W1, W3, W2, M1, M3, M2) with M in
    the natural orientation of its matrix (the device stores it wide)."""
    W1, W3, W2 = to64(fw.w1), to64(fw.w3), to64(fw.w2)
    if fw.m1 is not None:
        M1 = np.transpose(to64(fw.m1), (0, 2, 1))
        M3 = np.transpose(to64(fw.m3), (0, 2, 1))
        M2 = to64(fw.m2)
    else:
        M1 = M3 = M2 = None
    return W1, W3, W2, M1, M3, M2


def check_shadow(fw):
    """The operand copies must be the fp32 weights rounded to the operand type
    (round to nearest even), bit for bit: W1, W3 [dh][d], W2 [d][dh] and W2^T
    [dh][d] per head."""
    import torch
    sh = fw.shape
    dt = torch.bfloat16 if sh.dtype == L.BF16 else torch.float32
    m = sh.d * sh.dh
    s = fw.shadow.view(dt).view(sh.bh, 4, m)
    want = (fw.w1.reshape(sh.bh, m), fw.w3.reshape(sh.bh, m), fw.w2.reshape(sh.bh, m),
            fw.w2.transpose(1, 2).reshape(sh.bh, m))
    for x, (name, ref) in enumerate(zip(("W1", "W3", "W2", "W2T"), want)):
        assert torch.equal(s[:, x], ref.to(dt)), f"shadow {name} differs from the weights"


def oracle_state(O, W1, W3, W2, n1=None, n3=None, n2=None, M=None):
    """An oracle HeadState with the given weights (and norms / momentum)."""
    st = O.HeadState(W1, W3, W2)
    if n1 is not None:
        st.n1, st.n3, st.n2 = n1, n3, n2
    if M is not None:
        st.M1, st.M3, st.M2 = M
    return st
