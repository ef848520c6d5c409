"""Streaming decode on the GPU: lact_decode_apply (the weight-streaming read
of a few tokens per head) against the float64 oracle's read, and the
streaming pattern - every token read as it arrives, a write only when a
chunk of keys and values has filled (uTTT page section 2; the causal
function's chunk loop on the rebuttal page) - against lact_sequence and the
oracle's causal sequence."""
import numpy as np
import pytest

from chunk_test_head_amd import _lib as L
from chunk_test_head_amd import workloads as WL
from oracle import lact_oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

# family -> reduced workload (heads) with the family's d, dh and dtype
FAMILIES = {0: dict(heads=2, batch=1), 1: dict(heads=4, batch=1), 2: dict(heads=2, batch=1),
            3: dict(heads=3, batch=1), 4: dict(heads=2, batch=1)}


@pytest.mark.parametrize("wi", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("n", [1, 3, 8])
def test_decode_read(device, wi, n):
    import torch
    w = WL.WORKLOADS[wi].scaled(T=n, chunk=n, subset=(0, n) if WL.WORKLOADS[wi].subset else None,
                                **FAMILIES[wi])
    W, inp = WL.weights(w), WL.tokens(w)
    fw = H.make_state(w, W, device)
    q = H.act_to_dev(w, inp, "q", device)
    out = H.out_buffer(w, n, device)
    # NaN-filled: no partial is read before it is written
    ws = torch.full(((L.decode_workspace_bytes(fw.shape, n) + 3) // 4,), float("nan"), device=device)
    print(f"decode wl={wi} bh={w.bh} n={n}", flush=True)
    L.lact_decode_apply(fw.shape, fw, q, out, ws)
    torch.cuda.synchronize()
    got = H.to64(out)
    for b in range(w.bh):
        ref = O.apply(W[0][b], W[1][b], W[2][b], inp["q"][b])
        assert H.rel(got[b], ref) < H.TOL[w.dtype], (b, H.rel(got[b], ref))
    # a second call on the same workspace gives the same bits
    again = torch.full_like(out, float("nan"))
    L.lact_decode_apply(fw.shape, fw, q, again, ws)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.uint8), out.view(torch.uint8))


def test_decode_strided_layout(device):
    """q and o in a [B, T, H, d] layout (token stride = heads x d)."""
    import torch
    w = WL.WORKLOADS[1].scaled(heads=4, batch=1, T=2, chunk=2)
    W, inp = WL.weights(w), WL.tokens(w)
    fw = H.make_state(w, W, device)
    q = H.act_to_dev(w, inp, "q", device)                 # [bh, 2, d]
    q_bthd = q.permute(1, 0, 2).contiguous()              # [2, bh, d]
    o_bthd = torch.full_like(q_bthd, float("nan"))
    lay = L.Layout(w.d, w.bh * w.d)
    ws = torch.zeros(L.decode_workspace_bytes(fw.shape, 2), dtype=torch.uint8, device=device)
    L.lact_decode_apply(fw.shape, fw, q_bthd, o_bthd, ws, n_tok=2, q_layout=lay, o_layout=lay)
    torch.cuda.synchronize()
    got = H.to64(o_bthd.permute(1, 0, 2))
    for b in range(w.bh):
        ref = O.apply(W[0][b], W[1][b], W[2][b], inp["q"][b])
        assert H.rel(got[b], ref) < 2e-2


@pytest.mark.parametrize("wi", [1, 4])
def test_streaming_read_each_token_write_when_full(device, wi):
    """Tokens arrive one at a time: each is read with the current weights
    (decode read), and when a chunk of keys and values has filled it is
    written (lact_update).  The outputs are the causal sequence's: against
    lact_sequence (same weights at every read) and the oracle."""
    import torch
    C = 64
    w = WL.WORKLOADS[wi].scaled(heads=2, batch=1, T=3 * C + 17, chunk=C)
    W, inp = WL.weights(w), WL.tokens(w)
    q, k, v = (H.act_to_dev(w, inp, nm, device) for nm in ("q", "k", "v"))
    eta = torch.from_numpy(inp["eta"]).to(device)
    mom = torch.from_numpy(inp["mom"]).to(device) if inp["mom"] is not None else None
    o_opts = H.opts_of(w)
    fw = H.make_state(w, W, device)
    out = H.out_buffer(w, w.T, device)
    ws_dec = torch.zeros(L.decode_workspace_bytes(fw.shape, 1), dtype=torch.uint8, device=device)
    ws_upd = H.workspace(w, C, device)
    lay = L.layout_of(q)
    print(f"streaming wl={wi} T={w.T} chunk={C}", flush=True)
    for t in range(w.T):
        L.lact_decode_apply(fw.shape, fw, q[:, t:t + 1], out[:, t:t + 1], ws_dec, n_tok=1, q_layout=lay,
                            o_layout=L.layout_of(out))
        if (t + 1) % C == 0 and t + 1 < w.T:
            s0 = t + 1 - C
            L.lact_update(fw.shape, fw, k[:, s0:t + 1], v[:, s0:t + 1], eta[:, s0:t + 1], eta[:, s0:t + 1],
                          eta[:, s0:t + 1], None if mom is None else mom[:, s0:t + 1], o_opts, ws_upd,
                          k_layout=lay, v_layout=lay)
    torch.cuda.synchronize()
    got = H.to64(out)
    seq, _ = H.run_sequence(w, inp, W, device)
    for b in range(w.bh):
        e = inp["eta"][b]
        m = None if inp["mom"] is None else inp["mom"][b]
        ref, _ = O.sequence(W[0][b], W[1][b], W[2][b], inp["q"][b], inp["k"][b], inp["v"][b], e, e, e, C,
                            mom=m, use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
        assert H.rel(got[b], ref) < 2e-2, (b, H.rel(got[b], ref))
        # same weights at every read: only the read kernels' rounding differs
        assert H.rel(got[b], seq[b]) < 1e-2, (b, H.rel(got[b], seq[b]))
