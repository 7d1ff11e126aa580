"""Seeded synthetic inputs shared by the GPU tests, the oracle and the benchmark.

Holds no arithmetic of the method: it only draws keys, values, queries, new
tokens and the initial-centroid shuffle, and rounds them once to their
storage type. The draws are counter-based (SplitMix64 outputs indexed by
element), implemented in ``synth.c`` and run with OpenMP.

Workloads (``WORKLOADS``) follow the five synthetic configurations the
ClusterKV pages' 32k-context settings are modelled on; see ``workload()``.
Arrays of bf16 values are ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

F32, BF16 = 0, 1


def compile_lib(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", _SRC, "-o", tmp,
                        "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            compile_lib(force=False)
        lib = C.CDLL(_LIB)
        p, i, ll, d, u64 = C.c_void_p, C.c_int, C.c_longlong, C.c_double, C.c_uint64
        lib.synth_stream_seed.argtypes = [u64, u64, u64]
        lib.synth_stream_seed.restype = u64
        lib.synth_config_seed.argtypes = [i, i]
        lib.synth_config_seed.restype = u64
        lib.synth_round_bf16.argtypes = [p, C.c_size_t, p]
        lib.synth_mixture_keys.argtypes = [u64, i, i, i, i, i, d, i, d, i, p, ll, p, p]
        lib.synth_values.argtypes = [u64, i, i, i, i, d, i, p, ll]
        lib.synth_init_idx.argtypes = [u64, i, i, i, p]
        lib.synth_queries_noisy_key.argtypes = [u64, i, i, i, i, i, p, i, ll, d, p]
        lib.synth_queries_mixture.argtypes = [u64, i, i, i, i, i, p, d, i, p]
        lib.synth_queries_drift.argtypes = [u64, i, i, i, i, i, p, d, d, i, p]
        lib.synth_normal_array.argtypes = [u64, C.c_size_t, d, i, p]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _np(dtype: int):
    return np.uint16 if dtype == BF16 else np.float32


def config_seed(config: int, layer: int = 0) -> int:
    return int(_load().synth_config_seed(config, layer))


def stream_seed(base: int, a: int, b: int) -> int:
    return int(_load().synth_stream_seed(base, a, b))


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_round_bf16(_p(x), x.size, _p(out))
    return out


def normal_array(seed: int, shape, sigma: float = 1.0, dtype: int = F32) -> np.ndarray:
    out = np.empty(shape, dtype=_np(dtype))
    _load().synth_normal_array(seed, out.size, sigma, dtype, _p(out))
    return out


def mixture_keys(base: int, H: int, n: int, d: int, M: int, sigma: float, n_out: int = 0,
                 out_scale: float = 1.0, dtype: int = BF16, i0: int = 0, out: np.ndarray | None = None,
                 rows: int | None = None, want_means: bool = False, want_comp: bool = False):
    """Keys of tokens i0 .. i0+n-1 of each head's mixture stream.

    Writes rows 0..n-1 of ``out`` [H, rows, d] (allocated when None).
    Returns (keys, comp [H, n] or None, key-space means [H, M, d] or None).
    """
    rows = n if rows is None else rows
    if out is None:
        out = np.zeros((H, rows, d), dtype=_np(dtype))
    assert out.shape == (H, rows, d) and out.flags.c_contiguous and out.dtype == _np(dtype)
    comp = np.empty((H, n), dtype=np.int32) if want_comp else None
    means = np.empty((H, M, d), dtype=np.float64) if want_means else None
    _load().synth_mixture_keys(base, H, i0, n, d, M, sigma, n_out, out_scale, dtype, _p(out), rows * d, _p(comp),
                               _p(means))
    return out, comp, means


def mixture_means(base: int, H: int, d: int, M: int, n_out: int, out_scale: float) -> np.ndarray:
    """Key-space component means (outlier scaling applied), fp64 [H, M, d]."""
    scratch = np.zeros((H, 1, d), dtype=np.float32)
    means = np.empty((H, M, d), dtype=np.float64)
    _load().synth_mixture_keys(base, H, 0, 0, d, M, 0.0, n_out, out_scale, F32, _p(scratch), d, None, _p(means))
    return means


def values(base: int, H: int, n: int, d: int, dtype: int = BF16, i0: int = 0, out: np.ndarray | None = None,
           rows: int | None = None, sigma: float = 1.0) -> np.ndarray:
    rows = n if rows is None else rows
    if out is None:
        out = np.zeros((H, rows, d), dtype=_np(dtype))
    assert out.shape == (H, rows, d) and out.flags.c_contiguous and out.dtype == _np(dtype)
    _load().synth_values(base, H, i0, n, d, sigma, dtype, _p(out), rows * d)
    return out


def init_idx(base: int, H: int, L: int, C: int) -> np.ndarray:
    """The first C positions of a seeded shuffle of [0, L), per head [H, C]."""
    out = np.empty((H, C), dtype=np.int32)
    _load().synth_init_idx(base, H, L, C, _p(out))
    return out


def queries_noisy_key(base: int, step: int, Hq: int, G: int, keys: np.ndarray, n_cur: int,
                      sigma: float) -> np.ndarray:
    """q = a random current key of the query head's KV head + N(0, sigma^2)."""
    H, rows, d = keys.shape
    dtype = BF16 if keys.dtype == np.uint16 else F32
    keys = np.ascontiguousarray(keys)
    out = np.empty((Hq, d), dtype=keys.dtype)
    _load().synth_queries_noisy_key(base, step, Hq, G, d, n_cur, _p(keys), dtype, rows * d, sigma, _p(out))
    return out


def queries_drift(base: int, step: int, Hq: int, G: int, means: np.ndarray, sigma: float, p_change: float,
                  dtype: int = BF16) -> np.ndarray:
    """Mixture queries whose three components persist across steps, each
    replaced with probability p_change per step; fresh N(0, sigma^2) noise."""
    H, M, d = means.shape
    means = np.ascontiguousarray(means, dtype=np.float64)
    out = np.empty((Hq, d), dtype=_np(dtype))
    _load().synth_queries_drift(base, step, Hq, G, d, M, _p(means), sigma, float(p_change), dtype, _p(out))
    return out


def queries_mixture(base: int, step: int, Hq: int, G: int, means: np.ndarray, sigma: float,
                    dtype: int = BF16) -> np.ndarray:
    """q = Dirichlet(1,1,1) mixture of three distinct component means + N(0, sigma^2)."""
    H, M, d = means.shape
    means = np.ascontiguousarray(means, dtype=np.float64)
    out = np.empty((Hq, d), dtype=_np(dtype))
    _load().synth_queries_mixture(base, step, Hq, G, d, M, _p(means), sigma, dtype, _p(out))
    return out


@dataclass
class Workload:
    """One synthetic configuration (shapes follow the pages' 32k-context settings)."""
    name: str
    config: int
    heads: int           # KV heads per layer (batch x kv_heads)
    G: int               # query heads per KV head
    L: int               # prompt tokens clustered at prefill
    d: int
    dtype: int
    M: int               # mixture components per head
    sigma: float
    n_out: int           # outlier channels per head
    out_scale: float
    C: int
    iters: int
    B: int
    steps: int           # decode steps
    query: str           # "noisy_key" or "mixture"
    q_sigma: float
    append: bool = False  # one new token per head before each decode step
    layers: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def q_heads(self) -> int:
        return self.heads * self.G

    @property
    def capacity(self) -> int:
        return self.L + (self.steps if self.append else 0)


WORKLOADS = {
    1: Workload("single_head_L1k_fp32", 1, heads=1, G=1, L=1024, d=128, dtype=F32, M=16, sigma=0.3, n_out=0,
                out_scale=1.0, C=16, iters=10, B=128, steps=1, query="noisy_key", q_sigma=0.1),
    2: Workload("llama2_layer_32h_L8k", 2, heads=32, G=1, L=8192, d=128, dtype=BF16, M=256, sigma=0.3, n_out=4,
                out_scale=10.0, C=128, iters=10, B=1024, steps=1, query="noisy_key", q_sigma=0.1),
    3: Workload("append_32h_L32k_B2k", 3, heads=32, G=1, L=32768, d=128, dtype=BF16, M=256, sigma=0.3, n_out=4,
                out_scale=10.0, C=400, iters=10, B=2048, steps=256, query="noisy_key", q_sigma=0.1,
                append=True),
    4: Workload("gqa_b16_L32k_B1k", 4, heads=128, G=4, L=32768, d=128, dtype=BF16, M=256, sigma=0.3, n_out=4,
                out_scale=10.0, C=400, iters=10, B=1024, steps=128, query="mixture", q_sigma=0.2),
    5: Workload("stack32_b8_L32k_B1k", 5, heads=64, G=4, L=32768, d=128, dtype=BF16, M=256, sigma=0.3, n_out=4,
                out_scale=10.0, C=400, iters=10, B=1024, steps=64, query="mixture", q_sigma=0.2, layers=32),
}


def workload(n: int) -> Workload:
    return WORKLOADS[n]
