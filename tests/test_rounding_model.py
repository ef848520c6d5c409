"""CPU checks of the rounding model (tests/rounding_model.py) that the
end-to-end GPU drift is calibrated against: without bf16 rounding it must be
the oracle's computation, and the shifted Newton-Schulz steps must be the
same polynomial as the plain ones."""
import numpy as np
import pytest

from chunk_test_head_amd import workloads as WL
from oracle import lact_oracle as O
from tests import rounding_model as R


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


@pytest.mark.parametrize("shape", [(128, 512), (512, 128), (64, 256), (256, 1024)])
@pytest.mark.parametrize("ns", ["f32", "f32-shifted"])
def test_model_newton_schulz_fp32_is_the_oracle(shape, ns):
    rng = np.random.default_rng(shape[0] + shape[1])
    G = (rng.standard_normal((shape[0], 12)) @ rng.standard_normal((12, shape[1]))
         + 0.1 * rng.standard_normal(shape)).astype(np.float32)
    ref = O.newton_schulz5(G.astype(np.float64))
    for gemm_path in (False, True):
        assert _rel(R.newton_schulz(G, ns=ns, gemm_path=gemm_path), ref) < 2e-5


def test_model_bf16_rounds_and_shift_helps_near_one():
    """bf16 operands cost about 2^-9 relative per step; on a gradient whose
    singular values are spread over [0.3, 1] the shifted steps round less."""
    rng = np.random.default_rng(3)
    U, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    V, _ = np.linalg.qr(rng.standard_normal((512, 128)))
    G = ((U * np.linspace(0.3, 1.0, 128)) @ V.T).astype(np.float32)
    ref = O.newton_schulz5(G.astype(np.float64))
    e_b = _rel(R.newton_schulz(G, ns="bf16"), ref)
    e_s = _rel(R.newton_schulz(G, ns="bf16-shifted"), ref)
    assert 5e-4 < e_b < 2e-2
    assert e_s < 0.5 * e_b


def test_model_sequence_fp32_is_the_oracle():
    w = WL.WORKLOADS[1].scaled(heads=1, batch=1, T=3 * 128 + 40, chunk=128)
    w = WL.Workload(**{**w.__dict__, "d": 64, "dh": 128})
    W = WL.weights(w)
    inp = WL.tokens(w)
    e, m = inp["eta"][0], inp["mom"][0]
    ref, st = O.sequence(W[0][0], W[1][0], W[2][0], inp["q"][0], inp["k"][0], inp["v"][0], e, e, e, w.chunk,
                         mom=m, use_muon=True, use_momentum=True)
    out, sm = R.sequence(W[0][0], W[1][0], W[2][0], inp["q"][0], inp["k"][0], inp["v"][0], e, w.chunk, mom=m,
                         use_muon=True, use_momentum=True, ns="f32", op="f32")
    assert _rel(out, ref) < 1e-4
    assert _rel(sm.W1, st.W1) < 1e-4 and _rel(sm.M2, st.M2) < 1e-4
