"""Seeded synthetic inputs for the MoE layer forward and backward.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the layer's arithmetic.  Both the HIP path (through the
tests and bench.py) and the CPU oracle are fed from it.

Recipe (one independent numpy PCG64 stream per tensor block, so blocks can be
drawn in parallel and any block can be regenerated on its own):

* ``hidden [T, d]``      ~ N(0, 1)                stream ``[seed, 0]``
* ``w_router [d, N]``    ~ N(0, 1) / sqrt(d)      stream ``[seed, 1]``
* ``w1[e] [d, f]``       ~ N(0, 1) / sqrt(d)      stream ``[seed, 2, e]``
* ``w3[e] [d, f]``       ~ N(0, 1) / sqrt(d)      stream ``[seed, 3, e]``
* ``w2[e] [f, d]``       ~ N(0, 1) / sqrt(f)      stream ``[seed, 4, e]``
* shared experts (optional, s = 0 .. Ns-1, hidden size fs):
  ``w1s[s] [d, fs]``, ``w3s[s] [d, fs]`` ~ N(0, 1) / sqrt(d), streams
  ``[seed, 5, s]``, ``[seed, 6, s]``; ``w2s[s] [fs, d]`` ~ N(0, 1) / sqrt(fs),
  stream ``[seed, 7, s]``
* backward: the output gradient ``dy [T, d]`` ~ N(0, 1), stream ``[seed, 8]``

Normals are drawn as float32, scaled in float32, and for bf16 workloads
rounded to bfloat16 with round-to-nearest-even (the bit patterns are kept as
``uint16``).  The skewed workload adds a per-expert router bias
``b_e = 2.0 * ln(z_{e+1})`` with ``z_r = r^-1.1 / sum_q q^-1.1`` (a Zipf
rank weight, expert 0 hottest), which makes some experts hot and others idle.

The workload shapes stand in for the pages' examples: a Mixtral-8x7B layer
(8 experts, top-2, d 4096, f 14336), a 16-expert top-2 router, 64 experts,
fine-grained expert counts, and a decode batch where most experts get a
handful of tokens.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "MoEInputs", "make_inputs", "make_workload_inputs",
    "bf16_bits_to_f32", "f32_to_bf16_bits", "zipf_bias", "make_dy",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    N: int
    k: int
    f: int
    dtype: str                 # "f32" or "bf16": storage/compute type of hidden, weights, y
    capacity_factor: float     # <= 0 means no capacity limit
    zipf_bias: bool = False


# The five shapes the layer is exercised on.  Keys are short handles; the
# ``name`` spells out the sizes.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32_T64_d128_N8_k2_f256_nocap", 64, 128, 8, 2, 256, "f32", 0.0),
    "n16_cf125": Workload("n16_T4096_d2048_N16_k2_f5632_cf1.25", 4096, 2048, 16, 2, 5632, "bf16", 1.25),
    "mixtral": Workload("mixtral_T8192_d4096_N8_k2_f14336_nodrop", 8192, 4096, 8, 2, 14336, "bf16", 0.0),
    "skewed_zipf": Workload("zipf_skew_T16384_d4096_N64_k2_f2048_cf1.5", 16384, 4096, 64, 2, 2048, "bf16", 1.5, True),
    "decode": Workload("decode_T256_d4096_N128_k2_f1536_nocap", 256, 4096, 128, 2, 1536, "bf16", 0.0),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_bias(N: int, s: float = 1.1, scale: float = 2.0) -> np.ndarray:
    r = np.arange(1, N + 1, dtype=np.float64)
    z = r ** (-s)
    z /= z.sum()
    return (scale * np.log(z)).astype(np.float32)


@dataclasses.dataclass
class MoEInputs:
    """Host arrays.  For bf16 the arrays hold uint16 bit patterns."""
    T: int
    d: int
    N: int
    k: int
    f: int
    dtype: str
    capacity_factor: float
    hidden: np.ndarray            # [T, d]
    w_router: np.ndarray          # [d, N]
    w1: np.ndarray                # [N, d, f]
    w3: np.ndarray                # [N, d, f]
    w2: np.ndarray                # [N, f, d]
    bias: Optional[np.ndarray] = None   # [N] float32 or None
    w1s: Optional[np.ndarray] = None    # [Ns, d, fs] shared experts, or None
    w3s: Optional[np.ndarray] = None    # [Ns, d, fs]
    w2s: Optional[np.ndarray] = None    # [Ns, fs, d]

    @property
    def n_shared(self) -> int:
        return 0 if self.w1s is None else self.w1s.shape[0]

    def values(self, name: str) -> np.ndarray:
        """float32 values of a tensor (exact for bf16 storage)."""
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a

    def expert_values(self, name: str, e: int) -> np.ndarray:
        a = getattr(self, name)[e]
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


def _draw(key, shape, scale, dtype):
    rng = np.random.default_rng(key)
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(T, d, N, k, f, dtype="bf16", capacity_factor=0.0, seed=0,
                bias: Optional[np.ndarray] = None, zipf=False, n_shared=0,
                f_shared: Optional[int] = None) -> MoEInputs:
    """Draw one layer's inputs with the recipe in the module docstring."""
    assert dtype in ("f32", "bf16")
    st = np.uint16 if dtype == "bf16" else np.float32
    w1 = np.empty((N, d, f), st)
    w3 = np.empty((N, d, f), st)
    w2 = np.empty((N, f, d), st)
    sd, sf = 1.0 / math.sqrt(d), 1.0 / math.sqrt(f)

    def fill(job):
        which, e = job
        if which == 2:
            w1[e] = _draw([seed, 2, e], (d, f), sd, dtype)
        elif which == 3:
            w3[e] = _draw([seed, 3, e], (d, f), sd, dtype)
        else:
            w2[e] = _draw([seed, 4, e], (f, d), sf, dtype)

    jobs = [(w, e) for w in (2, 3, 4) for e in range(N)]
    with ThreadPoolExecutor(_threads()) as ex:
        fh = ex.submit(_draw, [seed, 0], (T, d), 1.0, dtype)
        fr = ex.submit(_draw, [seed, 1], (d, N), sd, dtype)
        list(ex.map(fill, jobs))
        hidden, w_router = fh.result(), fr.result()
    if zipf and bias is None:
        bias = zipf_bias(N)
    inp = MoEInputs(T, d, N, k, f, dtype, float(capacity_factor), hidden, w_router, w1, w3, w2,
                    None if bias is None else np.asarray(bias, np.float32))
    if n_shared > 0:
        fs = f if f_shared is None else f_shared
        ss = 1.0 / math.sqrt(fs)
        inp.w1s = np.stack([_draw([seed, 5, q], (d, fs), sd, dtype) for q in range(n_shared)])
        inp.w3s = np.stack([_draw([seed, 6, q], (d, fs), sd, dtype) for q in range(n_shared)])
        inp.w2s = np.stack([_draw([seed, 7, q], (fs, d), ss, dtype) for q in range(n_shared)])
    return inp


def make_dy(T: int, d: int, dtype: str = "bf16", seed: int = 0) -> np.ndarray:
    """The output gradient of a backward pass (recipe in the module docstring);
    bf16 bit patterns as uint16 for bf16, else float32."""
    return _draw([seed, 8], (T, d), 1.0, dtype)


def make_workload_inputs(key: str, seed: int = 0, n_shared: int = 0,
                         f_shared: Optional[int] = None) -> MoEInputs:
    w = WORKLOADS[key]
    return make_inputs(w.T, w.d, w.N, w.k, w.f, w.dtype, w.capacity_factor, seed, zipf=w.zipf_bias,
                       n_shared=n_shared, f_shared=f_shared)
