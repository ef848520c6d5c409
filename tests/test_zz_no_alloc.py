"""GPU check of lact_sequence_noalloc (the sequence driver with the
library's own device scratch instead of a caller workspace) against
lact_sequence with a caller workspace: two calls in a row on one GPU, the
second with a smaller input, each bitwise equal to the workspace entry point
on the same input (same kernels, same order of every sum)."""
import numpy as np
import pytest

from chunk_test_head_amd import _lib as L
from chunk_test_head_amd import workloads as WL
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _run(w, device, noalloc):
    import torch
    W = WL.weights(w)
    inp = WL.tokens(w)
    q, k, v = (H.act_to_dev(w, inp, n, device) for n in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    out = H.out_buffer(w, w.T, device)
    fw = H.make_state(w, W, device)
    o = H.opts_of(w)
    if noalloc:
        L.lact_sequence_noalloc(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, w.T, w.chunk, w.order, w.subset,
                                int(w.update_last), o)
    else:
        max_upd = max(z - a for _, a, z in w.writes())
        ws = torch.full(((L.workspace_bytes(fw.shape, max_upd, o) + 3) // 4,), float("nan"), device=device)
        L.lact_sequence(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, w.T, w.chunk, w.order, w.subset,
                        int(w.update_last), o, ws)
    torch.cuda.synchronize()
    bufs = [out, fw.w1, fw.w3, fw.w2, fw.shadow] + [m for m in (fw.m1, fw.m3, fw.m2) if m is not None]
    return [b.clone() for b in bufs]


def test_noalloc_matches_workspace_entry_point(device):
    import torch
    cases = [
        # lm-causal family (fused Newton-Schulz + step + read), 4 heads, ragged last chunk
        WL.WORKLOADS[1].scaled(heads=4, batch=1, T=3 * 512 + 100, chunk=512),
        # smaller: long-context family (batched Newton-Schulz, d = 256), 2 heads
        WL.WORKLOADS[4].scaled(heads=2, batch=1, T=2 * 256 + 64, chunk=256),
    ]
    for w in cases:
        print(f"noalloc {w.name} bh={w.bh} T={w.T} chunk={w.chunk}", flush=True)
        want = _run(w, device, noalloc=False)
        got = _run(w, device, noalloc=True)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (w.name, i)
