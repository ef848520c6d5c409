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
    for s in range(6):
        assert lib.lact_status_string(s)


def _shape(bh=2, d=128, dh=512, dtype=L.BF16):
    return L.Shape(bh, d, dh, dtype)


def test_shadow_and_workspace_sizes(lib):
    sh = _shape()
    assert L.shadow_bytes(sh) == 2 * 4 * 128 * 512 * 2
    o = L.opts(use_muon=True, use_momentum=True)
    a = L.workspace_bytes(sh, 2048, o)
    b = L.workspace_bytes(sh, 4096, o)
    assert 0 < a <= b
    assert L.workspace_bytes(sh, 2048, L.opts()) < a  # no Muon buffers
    assert L.shadow_bytes(_shape(d=96)) == 0


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
    # misaligned token stride (127 bf16 = 254 bytes)
    assert lib.lact_apply(ctypes.byref(sh), ctypes.byref(st), 256, L.Layout(512 * 128, 127), 512,
                          lay, 10, None) == 1
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
