"""Outer-loop backward on the GPU: lact_sequence_backward (the
vector-Jacobian product of a whole sequence with respect to q, k, v, the
learning rates, the momentum coefficients and W0) against the float64
backward oracle (oracle/lact_backward.py, itself pinned to finite
differences and torch autograd), head by head, on multi-chunk ragged
sequences of every ordering and option the backward supports.

The GPU recomputes the forward and runs the chain rule in fp32; the bar is
the fp32 bar of the forward, a relative Frobenius error of 1e-4 per
gradient (fp32 products over up to a few thousand tokens, through up to
five Newton-Schulz VJP steps; measured 3e-7 without Muon, up to 4e-5 with
it), and 1e-3 for the momentum coefficients (below)."""
import math

import zlib

import numpy as np
import pytest

from chunk_test_head_amd import _lib as L
from oracle import lact_backward as B
from oracle import lact_oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

A2U, U2A = O.ORDER_APPLY_THEN_UPDATE, O.ORDER_UPDATE_THEN_APPLY
CASES = {
    # name: (d, dh, dtype, T, chunk, order, subset, muon, momentum, renorm)
    "causal-muon-momentum": (64, 128, "f32", 3 * 64 + 21, 64, A2U, None, True, True, True),
    "causal-plain": (64, 128, "f32", 2 * 64 + 10, 64, A2U, None, False, False, True),
    "causal-no-renorm": (64, 128, "f32", 3 * 64, 64, A2U, None, True, True, False),
    "video-subset-bf16": (128, 256, "bf16", 4 * 64, 64, A2U, (32, 32), True, False, True),
    "bidirectional-subset": (64, 192, "f32", 160, 160, U2A, (0, 100), False, False, True),
    "d256-muon-momentum": (256, 512, "f32", 2 * 96 + 30, 96, A2U, None, True, True, True),
    # 2048-token chunks: the token contractions split K (partial sums added
    # in split order by a second launch)
    "long-chunks-split-k": (64, 128, "f32", 2 * 2048 + 100, 2048, A2U, None, True, True, True),
    # eight heads of the lm-causal shape: the token contractions take the
    # 128 x 128 tile kernel (512 tiles), split-K included; two heads checked
    "lm-shape-128-tiles": (128, 512, "bf16", 2 * 2048 + 64, 2048, A2U, None, True, True, True),
}
# (number of heads, heads compared with the oracle); default 2, all
HEADS = {"lm-shape-128-tiles": (8, (0, 7))}
TOL = 1e-4
# dL/dmom is one number per write (the momentum buffer projected on the
# cotangent of the pre-Newton-Schulz sum, spread over the write's tokens):
# when the two are nearly orthogonal its relative error is the cotangent's
# divided by that cosine (measured up to 2.8e-4 on 2048-token chunks)
TOL_MOM = 1e-3


def _inputs(rng, bh, T, d, dh):
    s = 1.0 / math.sqrt(d)
    W = [rng.standard_normal((bh, dh, d)) * s, rng.standard_normal((bh, dh, d)) * s,
         rng.standard_normal((bh, d, dh)) * s]
    Q, K = (rng.standard_normal((bh, T, d)) for _ in range(2))
    Q /= np.linalg.norm(Q, axis=2, keepdims=True)
    K /= np.linalg.norm(K, axis=2, keepdims=True)
    V = rng.standard_normal((bh, T, d))
    e = [np.log1p(np.exp(rng.standard_normal((bh, T)))) * 0.1 for _ in range(3)]
    mom = rng.uniform(0.5, 0.95, (bh, T))
    dO = rng.standard_normal((bh, T, d))
    f32 = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    return [f32(w) for w in W], f32(Q), f32(K), f32(V), [f32(x) for x in e], f32(mom), f32(dO)


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_oracle(device, case):
    import torch
    d, dh, dt, T, C, order, subset, muon, momentum, renorm = CASES[case]
    bh, check = HEADS.get(case, (2, (0, 1)))
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    W, Q, K, V, e, mom, dO = _inputs(rng, bh, T, d, dh)
    act = torch.bfloat16 if dt == "bf16" else torch.float32
    dev = lambda x, t=torch.float32: torch.from_numpy(x).to(device, t)
    q, k, v = dev(Q, act), dev(K, act), dev(V, act)
    # the oracle reads the activations the GPU reads
    Q64, K64, V64 = (x.double().cpu().numpy() for x in (q, k, v))
    shape = L.Shape(bh, d, dh, L.BF16 if dt == "bf16" else L.F32)
    o = L.opts(use_muon=muon, use_momentum=momentum, renorm=renorm)
    grads = {"dq": torch.empty(bh, T, d, device=device), "dk": torch.empty(bh, T, d, device=device),
             "dv": torch.empty(bh, T, d, device=device)}
    for n in ("deta1", "deta3", "deta2"):
        grads[n] = torch.empty(bh, T, device=device)
    grads["dmom"] = torch.empty(bh, T, device=device) if momentum else None
    for n, w in zip(("dw1", "dw3", "dw2"), W):
        grads[n] = torch.empty(w.shape, device=device)
    # NaN-filled: a read of an unwritten value shows up
    for t in grads.values():
        if t is not None:
            t.fill_(float("nan"))
    ws = torch.full(((L.backward_workspace_bytes(shape, T, C, o) + 3) // 4,), float("nan"), device=device)
    print(f"backward {case}: bh={bh} d={d} dh={dh} T={T} chunk={C}", flush=True)
    L.lact_sequence_backward(shape, dev(W[0]), dev(W[1]), dev(W[2]), q, k, v, dev(dO), dev(e[0]), dev(e[1]),
                             dev(e[2]), dev(mom) if momentum else None, T, C, order, subset, 0, o, grads, ws)
    torch.cuda.synchronize()
    got = {n: t.double().cpu().numpy() for n, t in grads.items() if t is not None}
    keys = {"Q": "dq", "K": "dk", "V": "dv", "eta1": "deta1", "eta3": "deta3", "eta2": "deta2", "W1": "dw1",
            "W3": "dw3", "W2": "dw2"}
    if momentum:
        keys["mom"] = "dmom"
    for b in check:
        ref = B.sequence_vjp(W[0][b], W[1][b], W[2][b], Q64[b], K64[b], V64[b], e[0][b], e[1][b], e[2][b], C,
                             dO[b], mom=mom[b] if momentum else None, order=order, subset=subset,
                             use_muon=muon, use_momentum=momentum, renorm=renorm)
        errs = {key: H.rel(got[name][b], ref[key]) for key, name in keys.items()}
        print("  head", b, " ".join(f"{key} {x:.1e}" for key, x in errs.items()), flush=True)
        for key, x in errs.items():
            assert x < (TOL_MOM if key == "mom" else TOL), (case, b, key, x)


def test_backward_zero_tokens(device):
    """T = 0: every gradient of the tokens is empty and dW0 is zero (no
    output depends on W0)."""
    import torch
    bh, d, dh = 1, 64, 128
    shape = L.Shape(bh, d, dh, L.F32)
    o = L.opts(use_muon=True, use_momentum=True)
    W = [torch.randn(bh, dh, d, device=device), torch.randn(bh, dh, d, device=device),
         torch.randn(bh, d, dh, device=device)]
    z = torch.zeros(bh, 1, d, device=device)
    e = torch.zeros(bh, 1, device=device)
    grads = {"dq": z.clone(), "dk": z.clone(), "dv": z.clone(), "deta1": e.clone(), "deta3": e.clone(),
             "deta2": e.clone(), "dmom": e.clone(),
             "dw1": torch.full_like(W[0], float("nan")), "dw3": torch.full_like(W[1], float("nan")),
             "dw2": torch.full_like(W[2], float("nan"))}
    ws = torch.zeros(max(256, L.backward_workspace_bytes(shape, 0, 64, o)), dtype=torch.uint8, device=device)
    L.lact_sequence_backward(shape, W[0], W[1], W[2], z, z, z, z, e, e, e, e, 0, 64, A2U, None, 0, o, grads, ws)
    torch.cuda.synchronize()
    for n in ("dw1", "dw3", "dw2"):
        assert torch.count_nonzero(grads[n]) == 0
