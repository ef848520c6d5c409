"""The linear fast-weight variant (f_W(x) = W x, one d x d matrix per head;
the rebuttal page's comparison of fast-weight networks, Fig. 8(a)) through
lact_linear_sequence against the oracle's linear_sequence."""
import math

import numpy as np
import pytest

from chunk_test_head_amd import _lib as L
from chunk_test_head_amd import workloads as WL
from oracle import lact_oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CASES = [
    # (d, dtype, T, chunk, order, subset, muon, momentum, renorm)
    (128, "bf16", 3 * 256 + 90, 256, O.ORDER_APPLY_THEN_UPDATE, None, True, True, 1),
    (256, "bf16", 3 * 192 + 40, 192, O.ORDER_APPLY_THEN_UPDATE, None, True, True, 1),
    (128, "bf16", 4 * 128, 128, O.ORDER_APPLY_THEN_UPDATE, (64, 64), True, False, 1),
    (64, "bf16", 300, 300, O.ORDER_UPDATE_THEN_APPLY, (0, 200), False, False, 1),
    (64, "f32", 3 * 128 + 17, 128, O.ORDER_APPLY_THEN_UPDATE, None, False, False, 1),
    (128, "bf16", 3 * 256, 256, O.ORDER_APPLY_THEN_UPDATE, None, True, True, 2),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_linear_sequence(device, case):
    import torch
    d, dt, T, C, order, subset, muon, momentum, renorm = CASES[case]
    bh = 3
    w = WL.WORKLOADS[1].scaled(heads=bh, batch=1, T=T, chunk=C)
    inp = WL.tokens(WL.Workload(**{**w.__dict__, "d": d, "dtype": dt}))
    rng = np.random.default_rng(case)
    W0 = (rng.standard_normal((bh, d, d)) / math.sqrt(d)).astype(np.float32)
    mom = np.full((bh, T), 0.9, np.float32)
    shape = L.Shape(bh, d, d, L.BF16 if dt == "bf16" else L.F32)
    lw = L.LinearWeights(shape, torch.from_numpy(W0).to(device), momentum=momentum)
    L.lact_linear_init_state(shape, lw)
    wl = WL.Workload(**{**w.__dict__, "d": d, "dtype": dt})
    q, k, v = (H.act_to_dev(wl, inp, n, device) for n in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(device)
    mt = torch.from_numpy(mom).to(device) if momentum else None
    out = H.out_buffer(wl, T, device)
    o = L.opts(use_muon=muon, use_momentum=momentum, renorm=renorm)
    ws = torch.full(((L.linear_workspace_bytes(shape, o) + 3) // 4,), float("nan"), device=device)
    print(f"linear d={d} {dt} T={T} C={C} order={order} subset={subset} muon={muon} renorm={renorm}", flush=True)
    L.lact_linear_sequence(shape, lw, q, k, v, out, eta, mt, T, C, order, subset, 0, o, ws)
    torch.cuda.synchronize()
    got = H.to64(out)
    wg = H.to64(lw.w)
    tol = H.TOL[dt]
    for b in range(bh):
        ref, (Wf, _) = O.linear_sequence(W0[b], inp["q"][b], inp["k"][b], inp["v"][b], inp["eta"][b], C,
                                         mom=mom[b] if momentum else None, order=order, subset=subset,
                                         use_muon=muon, use_momentum=momentum,
                                         renorm="master" if renorm == 2 else True)
        assert H.rel(got[b], ref) < tol, (b, H.rel(got[b], ref))
        assert H.rel(wg[b], Wf) < tol, (b, H.rel(wg[b], Wf))
