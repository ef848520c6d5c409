"""The ABI allocates nothing, never synchronises and records no memset nodes,
so a caller can capture a whole sequence (state initialisation + every chunk
step) into a HIP graph.  Each replay, with the caller's own eager work and a
synchronisation between replays, must reproduce the eager run bitwise (every
reduction in the path has a fixed order)."""
import numpy as np
import pytest

from chunk_test_head_amd import _lib as L
from tests import gpu_helpers as H
from tests.test_gpu_parity import SEQ_CASES, inputs, small

pytestmark = pytest.mark.gpu


# 1: d = 128 with Muon + momentum (Newton-Schulz fused with the read),
# 2: d = 256 update-then-apply on a subset, 4: d = 256 with Muon (batched GEMMs)
@pytest.mark.parametrize("wi", [1, 2, 4])
def test_sequence_graph_replay(device, wi):
    import torch
    T, C, sub = SEQ_CASES[wi]
    w = small(wi, T, C, subset=sub)
    W, inp = inputs(w)
    print(f"graph wl={wi} T={w.T} C={w.chunk}", flush=True)
    q, k, v = (H.act_to_dev(w, inp, n, device) for n in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    W0 = [torch.from_numpy(np.ascontiguousarray(x)).to(device) for x in W]
    fw = H.make_state(w, W, device)
    out = H.out_buffer(w, w.T, device)
    max_upd = min(w.chunk, w.T) if w.subset is None else min(w.subset[1], w.chunk - w.subset[0], w.T)
    ws = H.workspace(w, max_upd, device)
    o = H.opts_of(w)

    def restore():
        fw.w1.copy_(W0[0])
        fw.w2.copy_(W0[2])
        fw.w3.copy_(W0[1])
        out.fill_(float("nan"))

    def run(stream):
        L.lact_init_state(fw.shape, fw, stream)
        L.lact_sequence(fw.shape, fw, q, k, v, out, eta, eta, eta, mom, w.T, w.chunk, w.order, w.subset,
                        int(w.update_last), o, ws, stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (out, fw.w1, fw.w3, fw.w2)]

    side = torch.cuda.Stream()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        run(side)
    ref = snapshot()

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run(side)
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for name, x, y in zip(("o", "W1", "W3", "W2"), got, ref):
            assert torch.equal(x, y), (rep, name)
