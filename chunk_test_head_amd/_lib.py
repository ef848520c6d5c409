"""Thin Python binding of liblact.so (include/lact.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  PyTorch supplies device memory (tensor.data_ptr()) and the
HIP stream (torch.cuda.current_stream().cuda_stream); it computes nothing on
the layer's path.  There is no fallback: if the library is missing or fails
to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblact.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "lact.h")

F32, BF16 = 0, 1
APPLY_THEN_UPDATE, UPDATE_THEN_APPLY = 0, 1
NS_BF16_SHIFTED, NS_BF16, NS_F32 = 0, 1, 2
NS_PREC_NAMES = {NS_BF16_SHIFTED: "bf16-shifted", NS_BF16: "bf16", NS_F32: "f32"}
OK, ERR_NONFINITE = 0, 6
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "alignment",
          4: "workspace", 5: "HIP error", 6: "non-finite weights"}


class Shape(ctypes.Structure):
    _fields_ = [("bh", ctypes.c_int32), ("d", ctypes.c_int32), ("dh", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class State(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w3", "w2", "n1", "n3", "n2", "m1", "m3", "m2", "shadow")]


class Layout(ctypes.Structure):
    _fields_ = [("stride_bh", ctypes.c_int64), ("stride_tok", ctypes.c_int64)]


class UpdateOpts(ctypes.Structure):
    _fields_ = [("use_muon", ctypes.c_int32), ("use_momentum", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("renorm_eps", ctypes.c_float),
                ("ns_eps", ctypes.c_float), ("ns_prec", ctypes.c_int32),
                ("nonfinite", ctypes.c_void_p), ("eta_per_channel", ctypes.c_int32)]


class LactError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_lib = None


def load():
    """Load liblact.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    try:
        import torch  # noqa: F401  (its libamdhip64 must be the one in use)
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is not built; run chunk_test_head_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    pS, pSt, pO = ctypes.POINTER(Shape), ctypes.POINTER(State), ctypes.POINTER(UpdateOpts)
    L = Layout
    sig = {
        "lact_shadow_bytes": (SZ, [pS]),
        "lact_workspace_bytes": (SZ, [pS, I64, pO]),
        "lact_ns_workspace_bytes": (SZ, [I32, I32, I32]),
        "lact_init_state": (I32, [pS, pSt, P]),
        "lact_apply": (I32, [pS, pSt, P, L, P, L, I64, P]),
        "lact_gradient": (I32, [pS, pSt, P, L, P, L, P, P, P, I64, I64, P, P, P, P, SZ, P]),
        "lact_newton_schulz": (I32, [I32, I32, I32, I32, P, P, F, P, SZ, P]),
        "lact_step_renorm": (I32, [pS, pSt, P, P, P, pO, P, SZ, P]),
        "lact_update": (I32, [pS, pSt, P, L, P, L, P, P, P, P, I64, I64, pO, P, SZ, P]),
        "lact_chunk_step": (I32, [pS, pSt, P, L, P, L, P, L, P, L, P, P, P, P, I64, I64, pO, P, SZ, P]),
        "lact_sequence": (I32, [pS, pSt, P, L, P, L, P, L, P, L, P, P, P, P, I64, I64, I64, I32,
                                I64, I64, I32, pO, P, SZ, P]),
        "lact_sequence_noalloc": (I32, [pS, pSt, P, L, P, L, P, L, P, L, P, P, P, P, I64, I64, I64, I32,
                                        I64, I64, I32, pO, P]),
        "lact_decode_workspace_bytes": (SZ, [pS, I64]),
        "lact_decode_apply": (I32, [pS, pSt, P, L, P, L, I64, P, SZ, P]),
        "lact_linear_shadow_bytes": (SZ, [pS]),
        "lact_linear_workspace_bytes": (SZ, [pS, pO]),
        "lact_linear_init_state": (I32, [pS, P, P]),
        "lact_linear_sequence": (I32, [pS, P, P, L, P, L, P, L, P, L, P, P, I64, I64, I64, I32, I64, I64, I32,
                                       pO, P, SZ, P]),
        "lact_backward_workspace_bytes": (SZ, [pS, I64, I64, pO]),
        "lact_sequence_backward": (I32, [pS, P, P, P, P, L, P, L, P, L, P, P, P, P, P, I64, I64, I64, I32, I64,
                                         I64, I32, pO, ctypes.POINTER(Grads), P, SZ, P]),
        "lact_prof_begin": (I32, [I32, I32]),
        "lact_prof_end": (I32, [ctypes.POINTER(I32), ctypes.POINTER(F), ctypes.POINTER(F),
                                ctypes.POINTER(F)]),
        "lact_check_finite": (I32, [P, P]),
        "lact_status_string": (ctypes.c_char_p, [I32]),
        "lact_last_hip_error": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions():
    """Names of every function that include/lact.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(lact_[a-z_]+)\s*\(", text, re.M)))


# ---------------------------------------------------------------- helpers --
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st, where):
    if st != 0:
        raise LactError(st, where)


def _eta_stride(eta):
    """eta_stride_bh of a [bh, T] (per token) or [bh, T, channels] (per
    channel) learning-rate tensor: tokens between heads."""
    return eta.stride(0) // eta.shape[2] if eta.dim() == 3 else eta.stride(0)


def layout_of(t):
    """Layout of a [bh, T, d] (or [bh, T, d]-strided) tensor."""
    return Layout(t.stride(0), t.stride(1))


def opts(use_muon=False, use_momentum=False, renorm=True, renorm_eps=1e-5, ns_eps=1e-7,
         ns_prec=NS_BF16_SHIFTED, nonfinite=None, eta_per_channel=False):
    """lact_update_opts; nonfinite: a device int32 tensor (or None); renorm:
    False / True / 2 (master state with a rescaled operand copy)."""
    return UpdateOpts(int(use_muon), int(use_momentum), int(renorm), renorm_eps, ns_eps, int(ns_prec),
                      _ptr(nonfinite), int(eta_per_channel))


def shadow_bytes(shape):
    return load().lact_shadow_bytes(ctypes.byref(shape))


def workspace_bytes(shape, max_update_tokens, o):
    return load().lact_workspace_bytes(ctypes.byref(shape), int(max_update_tokens), ctypes.byref(o))


def ns_workspace_bytes(count, rows, cols):
    return load().lact_ns_workspace_bytes(count, rows, cols)


class FastWeights:
    """Device buffers of one lact_state, allocated with torch."""

    def __init__(self, shape, w1, w3, w2, momentum=True):
        import torch
        dev = w1.device
        self.shape = shape
        self.w1 = w1.detach().to(dev, torch.float32).contiguous().clone()
        self.w3 = w3.detach().to(dev, torch.float32).contiguous().clone()
        self.w2 = w2.detach().to(dev, torch.float32).contiguous().clone()
        bh, d, dh = shape.bh, shape.d, shape.dh
        self.n1 = torch.empty(bh, dh, device=dev)
        self.n3 = torch.empty(bh, dh, device=dev)
        self.n2 = torch.empty(bh, d, device=dev)
        if momentum:
            self.m1 = torch.empty(bh, d, dh, device=dev)
            self.m3 = torch.empty(bh, d, dh, device=dev)
            self.m2 = torch.empty(bh, d, dh, device=dev)
        else:
            self.m1 = self.m3 = self.m2 = None
        self.shadow = torch.empty(shadow_bytes(shape), dtype=torch.uint8, device=dev)
        self.struct = State(*(_ptr(x) for x in (self.w1, self.w3, self.w2, self.n1, self.n3, self.n2,
                                                 self.m1, self.m3, self.m2, self.shadow)))

    def ref(self):
        return ctypes.byref(self.struct)


PROF_APPLY, PROF_GRAD, PROF_REDUCE, PROF_NS, PROF_STEP = 1, 2, 3, 4, 5


def lact_prof_begin(kind, max_launches):
    _check(load().lact_prof_begin(kind, max_launches), "lact_prof_begin")


def lact_prof_end():
    """-> (launches, total_ms, min_ms, max_ms)"""
    n = ctypes.c_int32()
    t, lo, hi = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    _check(load().lact_prof_end(ctypes.byref(n), ctypes.byref(t), ctypes.byref(lo), ctypes.byref(hi)),
           "lact_prof_end")
    return n.value, t.value, lo.value, hi.value


# ------------------------------------------------------------ entry points --
def lact_init_state(shape, fw, stream=None):
    _check(load().lact_init_state(ctypes.byref(shape), fw.ref(), _stream(stream)), "lact_init_state")


def lact_apply(shape, fw, q, o, n_tok=None, stream=None, q_layout=None, o_layout=None):
    n = q.shape[1] if n_tok is None else n_tok
    _check(load().lact_apply(ctypes.byref(shape), fw.ref(), _ptr(q), q_layout or layout_of(q), _ptr(o),
                             o_layout or layout_of(o), int(n), _stream(stream)), "lact_apply")


DECODE_MAX_TOKENS = 8


def decode_workspace_bytes(shape, n_tok):
    return load().lact_decode_workspace_bytes(ctypes.byref(shape), int(n_tok))


def lact_decode_apply(shape, fw, q, o, ws, n_tok=None, stream=None, q_layout=None, o_layout=None):
    n = q.shape[1] if n_tok is None else n_tok
    _check(load().lact_decode_apply(ctypes.byref(shape), fw.ref(), _ptr(q), q_layout or layout_of(q), _ptr(o),
                                    o_layout or layout_of(o), int(n), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)), "lact_decode_apply")


def lact_gradient(shape, fw, k, v, eta1, eta3, eta2, g1, g3, g2, ws, n_tok=None, stream=None,
                  k_layout=None, v_layout=None):
    n = k.shape[1] if n_tok is None else n_tok
    _check(load().lact_gradient(ctypes.byref(shape), fw.ref(), _ptr(k), k_layout or layout_of(k), _ptr(v),
                                v_layout or layout_of(v), _ptr(eta1), _ptr(eta3), _ptr(eta2),
                                _eta_stride(eta1), int(n), _ptr(g1), _ptr(g3), _ptr(g2), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "lact_gradient")


def lact_newton_schulz(g, u, ws, prec=NS_BF16_SHIFTED, eps=1e-7, stream=None):
    count, rows, cols = g.shape
    _check(load().lact_newton_schulz(count, rows, cols, prec, _ptr(g), _ptr(u), eps, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "lact_newton_schulz")


def lact_check_finite(flag, stream=None):
    """Waits for the stream; returns the status (OK or ERR_NONFINITE)."""
    st = load().lact_check_finite(_ptr(flag), _stream(stream))
    if st not in (OK, ERR_NONFINITE):
        raise LactError(st, "lact_check_finite")
    return st


def lact_step_renorm(shape, fw, u1, u3, u2, o, ws, stream=None):
    _check(load().lact_step_renorm(ctypes.byref(shape), fw.ref(), _ptr(u1), _ptr(u3), _ptr(u2),
                                   ctypes.byref(o), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "lact_step_renorm")


def lact_update(shape, fw, k, v, eta1, eta3, eta2, mom, o, ws, n_tok=None, stream=None,
                k_layout=None, v_layout=None):
    n = k.shape[1] if n_tok is None else n_tok
    _check(load().lact_update(ctypes.byref(shape), fw.ref(), _ptr(k), k_layout or layout_of(k), _ptr(v),
                              v_layout or layout_of(v), _ptr(eta1), _ptr(eta3), _ptr(eta2), _ptr(mom),
                              _eta_stride(eta1), int(n), ctypes.byref(o), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "lact_update")


def lact_chunk_step(shape, fw, q, k, v, out, eta1, eta3, eta2, mom, o, ws, n_tok=None, stream=None):
    n = q.shape[1] if n_tok is None else n_tok
    _check(load().lact_chunk_step(ctypes.byref(shape), fw.ref(), _ptr(q), layout_of(q), _ptr(k), layout_of(k),
                                  _ptr(v), layout_of(v), _ptr(out), layout_of(out), _ptr(eta1), _ptr(eta3),
                                  _ptr(eta2), _ptr(mom), _eta_stride(eta1), int(n), ctypes.byref(o), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "lact_chunk_step")


def lact_sequence(shape, fw, q, k, v, out, eta1, eta3, eta2, mom, T, chunk, order, subset, update_last,
                  o, ws, stream=None, layouts=None):
    sub_off, sub_len = (0, -1) if subset is None else subset
    ql, kl, vl, ol = layouts or (layout_of(q), layout_of(k), layout_of(v), layout_of(out))
    _check(load().lact_sequence(ctypes.byref(shape), fw.ref(), _ptr(q), ql, _ptr(k), kl, _ptr(v), vl,
                                _ptr(out), ol, _ptr(eta1), _ptr(eta3), _ptr(eta2), _ptr(mom),
                                _eta_stride(eta1), int(T), int(chunk), int(order), int(sub_off), int(sub_len),
                                int(update_last), ctypes.byref(o), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "lact_sequence")


NOALLOC_SCRATCH_BYTES = 160 * 1024 * 1024


def lact_sequence_noalloc(shape, fw, q, k, v, out, eta1, eta3, eta2, mom, T, chunk, order, subset, update_last,
                          o, stream=None, layouts=None):
    """lact_sequence with the library's own scratch instead of a workspace."""
    sub_off, sub_len = (0, -1) if subset is None else subset
    ql, kl, vl, ol = layouts or (layout_of(q), layout_of(k), layout_of(v), layout_of(out))
    _check(load().lact_sequence_noalloc(ctypes.byref(shape), fw.ref(), _ptr(q), ql, _ptr(k), kl, _ptr(v), vl,
                                        _ptr(out), ol, _ptr(eta1), _ptr(eta3), _ptr(eta2), _ptr(mom),
                                        _eta_stride(eta1), int(T), int(chunk), int(order), int(sub_off),
                                        int(sub_len), int(update_last), ctypes.byref(o), _stream(stream)),
           "lact_sequence_noalloc")


# ------------------------------------------------ outer-loop backward ----
class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dq", "dk", "dv", "deta1", "deta3", "deta2", "dmom", "dw1", "dw3",
                                                 "dw2")]


def backward_workspace_bytes(shape, T, chunk, o):
    return load().lact_backward_workspace_bytes(ctypes.byref(shape), int(T), int(chunk), ctypes.byref(o))


def lact_sequence_backward(shape, w1, w3, w2, q, k, v, dout, eta1, eta3, eta2, mom, T, chunk, order, subset,
                           update_last, o, grads, ws, stream=None, layouts=None):
    """grads: dict with fp32 tensors dq, dk, dv ([bh, T, d]), deta1, deta3,
    deta2, dmom ([bh, T], dmom None without momentum), dw1, dw3, dw2."""
    sub_off, sub_len = (0, -1) if subset is None else subset
    ql, kl, vl = layouts or (layout_of(q), layout_of(k), layout_of(v))
    g = Grads(*(_ptr(grads.get(n)) for n, _ in Grads._fields_))
    _check(load().lact_sequence_backward(ctypes.byref(shape), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(q), ql, _ptr(k),
                                         kl, _ptr(v), vl, _ptr(dout), _ptr(eta1), _ptr(eta3), _ptr(eta2), _ptr(mom),
                                         _eta_stride(eta1), int(T), int(chunk), int(order), int(sub_off),
                                         int(sub_len), int(update_last), ctypes.byref(o), ctypes.byref(g), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)), "lact_sequence_backward")


# ---------------------------------------------------- linear variant ----
class LinearState(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w", "n", "m", "shadow")]


class LinearWeights:
    """Device buffers of one lact_linear_state (w [bh, d, d] fp32)."""

    def __init__(self, shape, w, momentum=True):
        import torch
        dev = w.device
        self.shape = shape
        self.w = w.detach().to(dev, torch.float32).contiguous().clone()
        self.n = torch.empty(shape.bh, shape.d, device=dev)
        self.m = torch.empty_like(self.w) if momentum else None
        self.shadow = torch.empty(load().lact_linear_shadow_bytes(ctypes.byref(shape)), dtype=torch.uint8,
                                  device=dev)
        self.struct = LinearState(*(_ptr(x) for x in (self.w, self.n, self.m, self.shadow)))

    def ref(self):
        return ctypes.byref(self.struct)


def linear_workspace_bytes(shape, o):
    return load().lact_linear_workspace_bytes(ctypes.byref(shape), ctypes.byref(o))


def lact_linear_init_state(shape, lw, stream=None):
    _check(load().lact_linear_init_state(ctypes.byref(shape), lw.ref(), _stream(stream)), "lact_linear_init_state")


def lact_linear_sequence(shape, lw, q, k, v, out, eta, mom, T, chunk, order, subset, update_last, o, ws,
                         stream=None):
    sub_off, sub_len = (0, -1) if subset is None else subset
    _check(load().lact_linear_sequence(ctypes.byref(shape), lw.ref(), _ptr(q), layout_of(q), _ptr(k), layout_of(k),
                                       _ptr(v), layout_of(v), _ptr(out), layout_of(out), _ptr(eta), _ptr(mom),
                                       eta.stride(0), int(T), int(chunk), int(order), int(sub_off), int(sub_len),
                                       int(update_last), ctypes.byref(o), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)), "lact_linear_sequence")
