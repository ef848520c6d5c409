"""Workload registry and seeded synthetic inputs for the fast-weight layer.

This module holds no arithmetic of the method: it only describes the five
synthetic workloads and draws their inputs.  Both the HIP path (through the
binding) and the float64 oracle are fed from here, so they see the same
values.

Input recipe (the workload descriptions of the LaCT pages: LM 2K chunks at
32K context, NVS full-sequence chunk with input and target views, AR-video
chunks of three latent frames with a noisy/clean interleave):

* q, k: N(0, 1) per element, then every token's d-vector divided by its L2
  norm;  v: N(0, 1);
* eta: softplus(N(0, 1)) * 1e-2 per token, one value shared by the three
  matrices;  per-token momentum coefficient: the constant 0.9 where momentum
  is on;
* W1, W3, W2: N(0, 1/d) (variance 1/d), independent per head;
* bf16 workloads round q, k, v once to bfloat16 (round to nearest even);
  both sides read those rounded values.

Streams are keyed ``numpy.random.default_rng([workload, tensor, chunk])``
(tensor ids q=1, k=2, v=3, eta=4, W1=5, W3=6, W2=7, momentum=8), so any chunk
can be drawn on its own.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ORDER_APPLY_THEN_UPDATE = 0
ORDER_UPDATE_THEN_APPLY = 1

TID_Q, TID_K, TID_V, TID_ETA, TID_W1, TID_W3, TID_W2, TID_MOM = 1, 2, 3, 4, 5, 6, 7, 8


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    heads: int
    d: int
    dh: int
    T: int
    chunk: int
    dtype: str                 # "f32" or "bf16": activations and MFMA operands
    order: int
    subset: tuple | None       # (offset, length) of written tokens per chunk
    use_muon: bool
    use_momentum: bool
    momentum: float = 0.9
    renorm: bool = True
    update_last: bool = False

    @property
    def bh(self):
        return self.batch * self.heads

    def chunk_bounds(self):
        return [(s, min(s + self.chunk, self.T)) for s in range(0, self.T, self.chunk)]

    def writes(self):
        """(chunk index, first, last) of every written token range."""
        out = []
        b = self.chunk_bounds()
        for ci, (s, e) in enumerate(b):
            last = ci == len(b) - 1
            if self.order == ORDER_APPLY_THEN_UPDATE and last and not self.update_last:
                continue
            a, z = (s, e) if self.subset is None else (s + self.subset[0], min(s + self.subset[0] + self.subset[1], e))
            if z > a:
                out.append((ci, a, z))
        return out

    def scaled(self, T=None, chunk=None, heads=None, batch=None, subset=None, name=None):
        """Same workload at other sizes (parity cases that the oracle runs fast)."""
        kw = dataclasses.asdict(self)
        if T is not None:
            kw["T"] = T
        if chunk is not None:
            kw["chunk"] = chunk
        if heads is not None:
            kw["heads"] = heads
        if batch is not None:
            kw["batch"] = batch
        if subset is not None:
            kw["subset"] = subset
        if name is not None:
            kw["name"] = name
        return Workload(**kw)


WORKLOADS = [
    Workload(0, "tiny-causal-f32", 1, 1, 64, 128, 1024, 256, "f32",
             ORDER_APPLY_THEN_UPDATE, None, False, False),
    Workload(1, "lm-causal", 4, 8, 128, 512, 32768, 2048, "bf16",
             ORDER_APPLY_THEN_UPDATE, None, True, True),
    Workload(2, "nvs-bidirectional", 2, 4, 256, 1024, 65536, 65536, "bf16",
             ORDER_UPDATE_THEN_APPLY, (0, 49152), False, False),
    Workload(3, "ar-video", 1, 40, 128, 256, 57344, 8192, "bf16",
             ORDER_APPLY_THEN_UPDATE, (4096, 4096), True, False),
    Workload(4, "long-context", 1, 4, 256, 1024, 1048576, 16384, "bf16",
             ORDER_APPLY_THEN_UPDATE, None, True, True),
]


def algorithmic_flops(w: Workload):
    """Contraction flops of one whole sequence: 6 d dh per read token and
    12 d dh per written token (LaCT rebuttal page, FLOPS note of the
    bidirectional function), plus with Muon, per write and per matrix, five
    iterations of 4 d^2 dh + 2 d^3 on the wide d x dh orientation."""
    d, dh = w.d, w.dh
    writes = w.writes()
    n_written = sum(z - a for _, a, z in writes)
    f = 6.0 * d * dh * w.T + 12.0 * d * dh * n_written
    if w.use_muon:
        f += len(writes) * 3 * 5 * (4.0 * d * d * dh + 2.0 * d ** 3)
    return f * w.bh


def page_convention_flops(w: Workload):
    """18 D H L B convention of the page (every token read once and written
    once, Muon ignored); reported beside the algorithmic count."""
    return 18.0 * w.d * w.dh * w.T * w.bh


# ------------------------------------------------------------ bf16 ----
def round_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------- generators ----
def _rng(w, tid, key):
    return np.random.default_rng([w.index, tid, key])


def _draw_tokens(w, tid, ci, s, e):
    g = _rng(w, tid, ci)
    x = g.standard_normal((w.bh, e - s, w.d), dtype=np.float32)
    if tid in (TID_Q, TID_K):
        n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
        x = (x / n).astype(np.float32)
    return x


def _draw_eta(w, ci, s, e):
    g = _rng(w, TID_ETA, ci)
    z = g.standard_normal((w.bh, e - s)).astype(np.float64)
    sp = np.where(z > 20, z, np.log1p(np.exp(np.minimum(z, 20))))
    return (sp * 1e-2).astype(np.float32)


def weights(w: Workload):
    """Initial fast weights: W1, W3 [bh, dh, d]; W2 [bh, d, dh]; fp32."""
    sd = math.sqrt(1.0 / w.d)
    W1 = (_rng(w, TID_W1, 0).standard_normal((w.bh, w.dh, w.d)) * sd).astype(np.float32)
    W3 = (_rng(w, TID_W3, 0).standard_normal((w.bh, w.dh, w.d)) * sd).astype(np.float32)
    W2 = (_rng(w, TID_W2, 0).standard_normal((w.bh, w.d, w.dh)) * sd).astype(np.float32)
    return W1, W3, W2


def tokens(w: Workload, threads: int = 8, values: bool = True):
    """q, k, v as [bh, T, d] arrays (float32 values; for bf16 workloads also
    the uint16 bit patterns), eta [bh, T] and momentum [bh, T] (or None).

    Returns a dict: q, k, v (float32 values, already bf16-representable for
    bf16 workloads), q_bits/k_bits/v_bits (uint16, bf16 workloads only),
    eta, mom.  values=False (bf16 workloads only) skips the float32 copies;
    token_values() widens any token range of the bits on demand.
    """
    bounds = w.chunk_bounds()
    out = {}
    for name, tid in (("q", TID_Q), ("k", TID_K), ("v", TID_V)):
        keep = values or w.dtype != "bf16"
        arr = np.empty((w.bh, w.T, w.d), dtype=np.float32) if keep else None
        bits = np.empty((w.bh, w.T, w.d), dtype=np.uint16) if w.dtype == "bf16" else None

        def fill(args, tid=tid, arr=arr, bits=bits):
            ci, (s, e) = args
            x = _draw_tokens(w, tid, ci, s, e)
            if bits is not None:
                b = round_to_bf16_bits(x)
                bits[:, s:e] = b
                if arr is not None:
                    arr[:, s:e] = bf16_bits_to_f32(b)
            else:
                arr[:, s:e] = x

        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(fill, list(enumerate(bounds))))
        if arr is not None:
            out[name] = arr
        if bits is not None:
            out[name + "_bits"] = bits
    eta = np.empty((w.bh, w.T), dtype=np.float32)
    for ci, (s, e) in enumerate(bounds):
        eta[:, s:e] = _draw_eta(w, ci, s, e)
    out["eta"] = eta
    out["mom"] = np.full((w.bh, w.T), w.momentum, dtype=np.float32) if w.use_momentum else None
    return out


def token_values(inp, name, b, s, e):
    """float32 values of tokens [s, e) of head b (from the bf16 bits when the
    float32 copy was not kept)."""
    if name in inp:
        return inp[name][b, s:e]
    return bf16_bits_to_f32(inp[name + "_bits"][b, s:e])


def get(index_or_name):
    for w in WORKLOADS:
        if w.index == index_or_name or w.name == index_or_name:
            return w
    raise KeyError(index_or_name)
