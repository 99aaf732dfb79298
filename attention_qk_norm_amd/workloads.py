"""Seeded synthetic inputs for layerwise QK-Norm.

This module only draws random numbers: it holds none of the normalisation
arithmetic, and both the HIP path and the CPU oracle consume exactly the
tensors it returns.

The five workloads stand in for the projected query/key activations of the
OLMo-series models the SwiftQK review evaluates (section 4: OLMoE-7B,
OLMo2-13B, OLMo3-32B; Fig. 2(a) uses inputs of 64 and of 4096 tokens). The
pages' activations come from vLLM serving ShareGPT traffic; neither the
weights nor the dataset are available, so seeded draws of the same shapes
and value spreads are used instead.

Recipe: numpy `default_rng([workload_id, tensor_id])` with tensor ids
q=0, k=1, gamma_q=2, gamma_k=3, outlier mask for q=4, for k=5, and the
per-head weights of the headwise form q=6, k=7. Values are
drawn in float32; bf16 and fp8 (OCP e4m3) tensors are then rounded to
nearest-even by torch. The rounded values are the problem instance.
"""
from dataclasses import dataclass, field
from typing import Tuple

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}

TENSOR_Q, TENSOR_K, TENSOR_GQ, TENSOR_GK, MASK_Q, MASK_K, TENSOR_HGQ, TENSOR_HGK = range(8)

# Head width of each workload's model, for the headwise form (the OLMo2
# shapes use 128-wide heads; the tiny fp32 case cuts its rows into 4 heads).
HEAD_DIM = {"c1": 64, "c2": 128, "c3": 128, "c4": 128, "c5": 128, "c4f8": 128, "c5f8": 128}


@dataclass(frozen=True)
class Workload:
    wid: int                 # workload id, first seed word
    name: str
    T: int                   # tokens
    hq: int                  # query row width
    hk: int                  # key row width
    dtype: str               # "f32" or "bf16" (activations and weights)
    dist: str                # "normal" or "laplace"
    scale: float             # normal: standard deviation; laplace: scale b
    outlier_p: float         # probability an element is an outlier
    outlier_mult: float      # outlier elements are multiplied by this
    gamma_lo: float
    gamma_hi: float
    eps: float
    slices: Tuple[int, ...]  # slice counts exercised; the first is the primary one
    in_place: bool           # output overwrites the input
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def elem_bytes(self):
        return ELEM_BYTES[self.dtype]

    @property
    def gamma_dtype(self):
        """The weights' dtype: bf16 for FP8 rows, else the rows' own."""
        return "bf16" if self.dtype == "fp8" else self.dtype

    def algorithmic_bytes(self):
        """Bytes a single fused pass must move: every q and k element read once
        and written once, and each gamma read once."""
        s = self.elem_bytes
        return 2 * self.T * (self.hq + self.hk) * s + (self.hq + self.hk) * ELEM_BYTES[self.gamma_dtype]


WORKLOADS = {
    "c1": Workload(1, "tiny-f32", 4, 256, 256, "f32", "normal", 1.0, 0.0, 1.0,
                   0.5, 1.5, 1e-6, (1, 4), False,
                   "T=4, rows of 256, fp32; oracle finishes in milliseconds"),
    "c2": Workload(2, "olmo2-7b-decode", 64, 4096, 4096, "bf16", "normal", 1.0,
                   0.01, 20.0, 0.5, 1.5, 1e-6, (1,), False,
                   "decode step, 32 heads x 128, 1% outliers x20"),
    "c3": Workload(3, "olmo2-13b-decode-batch", 256, 5120, 5120, "bf16",
                   "normal", float(np.sqrt(2.0)), 0.0, 1.0, 0.8, 1.2, 1e-6,
                   (4, 1), False,
                   "40 heads x 128; 4 slices of 1280 = a 4-way tensor-parallel shard"),
    "c4": Workload(4, "olmo2-32b-gqa-prefill", 2048, 5120, 1024, "bf16",
                   "normal", 1.0, 0.0, 1.0, 0.5, 1.5, 1e-6, (1,), False,
                   "40 query heads, 8 kv heads of 128"),
    "c5": Workload(5, "large-prefill", 16384, 4096, 4096, "bf16", "laplace",
                   1.0, 0.0, 1.0, 0.5, 1.5, 1e-6, (8, 1), True,
                   "in-place output; 8 slices of 512"),
    # FP8-E4M3 activations (the review's Fig. 2(b) FP8 runs) on the two
    # prefill shapes; the weights stay bf16
    "c4f8": Workload(14, "olmo2-32b-gqa-prefill-fp8", 2048, 5120, 1024, "fp8",
                     "normal", 1.0, 0.0, 1.0, 0.5, 1.5, 1e-6, (1,), False,
                     "C4's shape with e4m3 rows"),
    "c5f8": Workload(15, "large-prefill-fp8", 16384, 4096, 4096, "fp8", "laplace",
                     1.0, 0.0, 1.0, 0.5, 1.5, 1e-6, (8, 1), True,
                     "C5's shape with e4m3 rows, in place; 8 slices of 512"),
}


def _draw(rng, n, dist, scale):
    if dist == "normal":
        return rng.standard_normal(n, dtype=np.float32) * np.float32(scale)
    if dist == "laplace":
        return rng.laplace(0.0, scale, n).astype(np.float32)
    raise ValueError(dist)


def _finish(a32, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a32))
    return t.to(DTYPES[dtype]) if dtype != "f32" else t


def activations(w, which):
    """Seeded [T, width] activations of workload `w` for tensor "q" or "k"."""
    tid, mid, width = ((TENSOR_Q, MASK_Q, w.hq) if which == "q"
                       else (TENSOR_K, MASK_K, w.hk))
    n = w.T * width
    a = _draw(np.random.default_rng([w.wid, tid]), n, w.dist, w.scale)
    if w.outlier_p > 0.0:
        mask = np.random.default_rng([w.wid, mid]).random(n) < w.outlier_p
        a[mask] *= np.float32(w.outlier_mult)
    return _finish(a.reshape(w.T, width), w.dtype)


def weights(w, which):
    """Seeded gamma of workload `w` for tensor "q" or "k"."""
    tid, width = (TENSOR_GQ, w.hq) if which == "q" else (TENSOR_GK, w.hk)
    g = np.random.default_rng([w.wid, tid]).uniform(w.gamma_lo, w.gamma_hi, width)
    return _finish(g.astype(np.float32), w.gamma_dtype)


def head_weights(w, which, head_dim):
    """Seeded weights of one head (head_dim of them, shared by every head of
    the tensor) for the headwise form; tensor ids 6 (q) and 7 (k)."""
    tid = TENSOR_HGQ if which == "q" else TENSOR_HGK
    g = np.random.default_rng([w.wid, tid]).uniform(w.gamma_lo, w.gamma_hi, head_dim)
    return _finish(g.astype(np.float32), w.gamma_dtype)


def generate(name):
    """All inputs of a named workload: dict with q, k, gamma_q, gamma_k (CPU
    tensors) and the Workload record under "w"."""
    w = WORKLOADS[name]
    return {"w": w, "q": activations(w, "q"), "k": activations(w, "k"),
            "gamma_q": weights(w, "q"), "gamma_k": weights(w, "k")}


def random_rows(T, H, dtype, seed, dist="normal", scale=1.0):
    """Generic seeded [T, H] rows for edge-case tests."""
    a = _draw(np.random.default_rng(seed), T * H, dist, scale)
    return _finish(a.reshape(T, H), dtype)


def device_rows(T, H, dtype, seed, device):
    """Seeded N(0,1) [T, H] rows drawn on the device (torch's generator), for
    inputs too large to draw on the host; tests copy back the rows they check."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn((T, H), generator=g, device=device, dtype=torch.float32).to(DTYPES[dtype])


def random_weights(H, dtype, seed, lo=0.5, hi=1.5):
    g = np.random.default_rng(seed).uniform(lo, hi, H).astype(np.float32)
    return _finish(g, dtype)


def exact_sum_rows(T, H, dtype, seed):
    """Rows whose sums of squares are exact in fp32 in any order: x = n/16 with
    integer n uniform in [-16, 16]. Every square is a multiple of 2^-8 and, for
    H <= 16384, every partial sum stays below 2^14, so fp32 holds all of them
    exactly. The values are exact in bf16 too."""
    n = np.random.default_rng(seed).integers(-16, 17, size=(T, H))
    return _finish((n.astype(np.float32) / np.float32(16.0)), dtype)
