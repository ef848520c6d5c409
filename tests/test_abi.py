"""Host-only checks of the C ABI: the library loads, exports every function
that include/lact.h declares, and rejects bad arguments with the documented
status before touching the device (no GPU needed: every call here fails
validation, so nothing is enqueued)."""
import ctypes

import pytest

from chunk_test_head_amd import _lib as L


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_declared_function(lib):
    names = L.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(7):
        assert lib.lact_status_string(s)
    assert lib.lact_status_string(6) != lib.lact_status_string(99)


def test_opts_and_finite_checks(lib):
    """Bad Newton-Schulz precision and a misaligned non-finite flag are
    rejected before anything is enqueued; lact_check_finite rejects a NULL or
    misaligned flag without touching the device."""
    sh = _shape()
    st = L.State(*([256] * 10))
    lay = L.Layout(512 * 128, 128)
    for prec, flag, code in ((3, None, 1), (-1, None, 1), (L.NS_F32, 1026, 3)):
        o = L.opts(use_muon=True, ns_prec=prec, nonfinite=flag)
        need = 1 << 30
        assert lib.lact_update(ctypes.byref(sh), ctypes.byref(st), 256, lay, 512, lay, 1024, 1024, 1024,
                               None, 100, 100, ctypes.byref(o), 4096, need, None) == code
    assert lib.lact_check_finite(None, None) == 1
    assert lib.lact_check_finite(1026, None) == 3
    assert lib.lact_newton_schulz(1, 128, 512, 7, 256, 256, 1e-7, 256, 1 << 30, None) == 1


def _shape(bh=2, d=128, dh=512, dtype=L.BF16):
    return L.Shape(bh, d, dh, dtype)


def test_shadow_and_workspace_sizes(lib):
    sh = _shape()
    assert L.shadow_bytes(sh) == 2 * 4 * 128 * 512 * 2
    o = L.opts(use_muon=True, use_momentum=True)
    a = L.workspace_bytes(sh, 2048, o)
    b = L.workspace_bytes(sh, 4096, o)
    assert 0 < a <= b
    assert L.shadow_bytes(_shape(d=96)) == 0
    # d = 256: Newton-Schulz runs as batched GEMMs with buffers of their own
    big = _shape(bh=4, d=256, dh=1024)
    assert L.workspace_bytes(big, 16384, L.opts()) < L.workspace_bytes(big, 16384, L.opts(use_muon=True))
    # d = 128, dh = 512 with Muon: the Newton-Schulz workgroups sum the split
    # partials and step, so the write needs the partials, the per-head beta
    # and the second operand copy (2 d dh per head, 4 bytes) and nothing else
    plain = L.workspace_bytes(sh, 2048, L.opts())
    fused = L.workspace_bytes(sh, 2048, o)
    assert fused - plain == 2 * 2 * 128 * 512 * 4 - 2 * 3 * 128 * 512 * 4


@pytest.mark.parametrize("d,dh,dtype,code", [
    (96, 512, L.BF16, 2), (128, 96, L.BF16, 2), (128, 64, L.BF16, 2), (256, 8192, L.BF16, 2),
    (256, 1024, L.F32, 2), (128, 512, 7, 1), (0, 512, L.BF16, 1),
])
def test_bad_shapes(lib, d, dh, dtype, code):
    sh = L.Shape(1, d, dh, dtype)
    st = L.State(*([16] * 10))
    assert lib.lact_init_state(ctypes.byref(sh), ctypes.byref(st), None) == code


def test_null_and_alignment(lib):
    sh = _shape()
    st = L.State(*([256] * 10))
    lay = L.Layout(512 * 128, 128)
    # null state pointer
    bad = L.State(*([256] * 9 + [0]))
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(bad), 256, lay, 512, lay, 10, None) == 1
    # misaligned activation
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(st), 258, lay, 512, lay, 10, None) == 3
    # token stride shorter than a token
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(st), 256, L.Layout(512 * 128, 127), 512,
                          lay, 10, None) == 1
    # token stride long enough but not a multiple of 16 bytes (132 bf16 = 264 bytes)
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(st), 256, L.Layout(512 * 132, 132), 512,
                          lay, 10, None) == 3
    # head stride not a multiple of 16 bytes
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(st), 256, L.Layout(512 * 128 + 4, 128), 512,
                          lay, 10, None) == 3
    # o aliasing q
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(st), 256, lay, 256, lay, 10, None) == 1
    # negative token count
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(st), 256, lay, 512, lay, -1, None) == 1


def test_update_workspace_and_momentum_checks(lib):
    sh = _shape()
    lay = L.Layout(512 * 128, 128)
    o = L.opts(use_momentum=True)
    st_nom = L.State(*([256] * 6 + [0, 0, 0] + [256]))
    need = L.workspace_bytes(sh, 100, o)
    args = lambda st, mom, ws, wsb: (ctypes.byref(sh), ctypes.byref(st), 256, lay, 512, lay, 1024, 1024,
                                     1024, mom, 100, 100, ctypes.byref(o), ws, wsb, None)
    # momentum on but no momentum buffers
    assert lib.lact_update(*args(st_nom, 1024, 4096, need)) == 1
    st = L.State(*([256] * 10))
    # momentum on but no coefficients
    assert lib.lact_update(*args(st, None, 4096, need)) == 1
    # workspace too small / missing
    assert lib.lact_update(*args(st, 1024, 4096, need - 1)) == 4
    assert lib.lact_update(*args(st, 1024, None, need)) == 4


def test_sequence_argument_checks(lib):
    sh = _shape()
    st = L.State(*([256] * 10))
    lay = L.Layout(512 * 128, 128)
    o = L.opts()
    ws_need = L.workspace_bytes(sh, 64, o)
    base = [ctypes.byref(sh), ctypes.byref(st), 256, lay, 256, lay, 256, lay, 512, lay, 1024, 1024, 1024,
            None, 100]
    def call(T, chunk, order, so, sl, wsb=ws_need):
        return lib.lact_sequence(*base, T, chunk, order, so, sl, 0, ctypes.byref(o), 4096, wsb, None)
    assert call(100, 0, 0, 0, -1) == 1          # chunk < 1
    assert call(100, 64, 5, 0, -1) == 1         # bad order
    assert call(100, 64, 0, 64, 10) == 1        # subset offset outside the chunk
    assert call(100, 64, 0, 0, -1, ws_need - 1) == 4


def test_newton_schulz_checks(lib):
    assert lib.lact_newton_schulz(0, 128, 512, L.BF16, 256, 256, 1e-7, 256, 1 << 30, None) == 1
    assert lib.lact_newton_schulz(1, 512, 128, L.BF16, 256, 256, 1e-7, 256, 1 << 30, None) == 2
    assert lib.lact_newton_schulz(1, 100, 128, L.BF16, 256, 256, 1e-7, 256, 1 << 30, None) == 2
    need = L.ns_workspace_bytes(1, 128, 512)
    assert lib.lact_newton_schulz(1, 128, 512, L.BF16, 256, 256, 1e-7, 256, need - 1, None) == 4


def test_sequence_noalloc_checks(lib):
    """The entry point without a workspace checks its arguments like
    lact_sequence, and a sequence whose writes need more workspace than the
    library's scratch returns LACT_ERR_WORKSPACE, before any device call."""
    lay = L.Layout(512 * 128, 128)
    st = L.State(*([256] * 10))
    o = L.opts(use_muon=True, use_momentum=True)
    def call(sh, T, chunk, order=0):
        return lib.lact_sequence_noalloc(ctypes.byref(sh), ctypes.byref(st), 256, lay, 256, lay, 256, lay, 512, lay,
                                         1024, 1024, 1024, 1024, 100, T, chunk, order, 0, -1, 0, ctypes.byref(o),
                                         None)
    assert call(_shape(bh=4), 100, 0) == 1                  # chunk < 1
    assert call(_shape(bh=4), 100, 64, order=9) == 1        # bad order
    big = _shape(bh=256)                                    # lm-causal shape with 256 heads
    assert L.workspace_bytes(big, 2048, o) > L.NOALLOC_SCRATCH_BYTES
    assert call(big, 4096, 2048) == 4
    assert L.workspace_bytes(_shape(bh=32), 2048, o) <= L.NOALLOC_SCRATCH_BYTES


def test_decode_checks(lib):
    """Decode reads: more than LACT_DECODE_MAX_TOKENS tokens, a missing or
    short workspace and o aliasing q are rejected before any device call."""
    sh = _shape(bh=4)
    st = L.State(*([256] * 10))
    lay = L.Layout(512 * 128, 128)
    need = L.decode_workspace_bytes(sh, 1)
    assert need > 0 and L.decode_workspace_bytes(sh, 9) == 0 and L.decode_workspace_bytes(sh, 0) == 0
    call = lambda n, ws, wsb, o=512: lib.lact_decode_apply(ctypes.byref(sh), ctypes.byref(st), 256, lay, o, lay,
                                                           n, ws, wsb, None)
    assert call(9, 4096, 1 << 20) == 1
    assert call(1, 4096, need - 1) == 4
    assert call(1, None, need) == 4
    assert call(1, 4096, need, o=256) == 1
    assert call(0, None, 0) == 0          # nothing to read: nothing enqueued


def test_per_channel_eta_checks(lib):
    """Per-channel learning rates are for d <= 128; other values of the flag
    are invalid."""
    lay = L.Layout(512 * 256, 256)
    st = L.State(*([256] * 10))
    for d, flag, code in ((256, 1, 2), (128, 2, 1)):
        sh = L.Shape(2, d, 1024, L.BF16)
        o = L.opts(eta_per_channel=flag)
        assert lib.lact_update(ctypes.byref(sh), ctypes.byref(st), 256, lay, 512, lay, 1024, 1024, 1024, None,
                               100, 100, ctypes.byref(o), 4096, 1 << 30, None) == code


def test_linear_variant_checks(lib):
    """The linear variant has one d x d matrix: shape.dh must equal d; a
    missing momentum buffer or a short workspace is rejected on the host."""
    st = L.LinearState(256, 256, 0, 256)
    assert lib.lact_linear_init_state(ctypes.byref(L.Shape(2, 128, 512, L.BF16)), ctypes.byref(st), None) == 2
    sh = L.Shape(2, 128, 128, L.BF16)
    assert L.linear_workspace_bytes(L.Shape(2, 128, 512, L.BF16), L.opts()) == 0
    lay = L.Layout(512 * 128, 128)
    def call(o, wsb):
        return lib.lact_linear_sequence(ctypes.byref(sh), ctypes.byref(st), 256, lay, 512, lay, 768, lay, 1024, lay,
                                        2048, 2048, 100, 100, 50, 0, 0, -1, 0, ctypes.byref(o), 4096, wsb, None)
    assert call(L.opts(use_momentum=True), 1 << 30) == 1          # no momentum buffer
    o = L.opts(use_muon=True)
    assert call(o, L.linear_workspace_bytes(sh, o) - 1) == 4


def test_backward_checks(lib):
    """The outer-loop backward: workspace size grows with the number of
    chunks (one fp32 state each); the master renorm variant and per-channel
    rates are unsupported; NULL gradients, a missing momentum output and a
    short workspace are rejected on the host."""
    sh = L.Shape(2, 128, 512, L.F32)
    o = L.opts(use_muon=True, use_momentum=True)
    a = L.backward_workspace_bytes(sh, 1024, 256, o)
    b = L.backward_workspace_bytes(sh, 2048, 256, o)
    assert 0 < a < b
    assert L.backward_workspace_bytes(L.Shape(2, 96, 512, L.F32), 1024, 256, o) == 0
    assert L.backward_workspace_bytes(L.Shape(2, 256, 1024, L.F32), 1024, 256, o) > 0
    lay = L.Layout(1024 * 128, 128)
    g = L.Grads(*([4096] * 10))
    def call(o, grads=g, wsb=1 << 34, mom=4096, T=1024):
        return lib.lact_sequence_backward(ctypes.byref(sh), 256, 256, 256, 512, lay, 768, lay, 1024, lay, 2048,
                                          4096, 4096, 4096, mom, 1024, T, 256, 0, 0, -1, 0, ctypes.byref(o),
                                          None if grads is None else ctypes.byref(grads), 8192, wsb, None)
    assert call(L.opts(use_muon=True, renorm=2)) == 2
    assert call(L.opts(eta_per_channel=True)) == 2
    assert call(o, grads=None) == 1
    assert call(o, mom=None) == 1
    assert call(o, grads=L.Grads(*([4096] * 6 + [0] + [4096] * 3))) == 1   # no dmom with momentum
    assert call(o, wsb=a - 1) == 4
    assert call(o, T=-1) == 1
