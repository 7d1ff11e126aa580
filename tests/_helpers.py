"""Shared helpers of the GPU tests: host<->device transfer of the generator's
arrays and construction of one workload's inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy array (uint16 = bf16 bits, float32, int32) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def torch_dtype(w) -> torch.dtype:
    return torch.bfloat16 if w.dtype == synth.BF16 else torch.float32


def make_inputs(w, layer: int = 0, heads: int | None = None):
    """Keys/values [H, capacity, d] (prompt rows plus, for append workloads,
    the decode-time tokens at rows L..), the initial positions the seeded
    shuffle draws (the oracle's, from seed = base; the GPU build draws its own
    from the same seed) and the key-space means."""
    H = w.heads if heads is None else heads
    base = synth.config_seed(w.config, layer)
    cap = w.capacity
    K, _, means = synth.mixture_keys(base, H, cap, w.d, w.M, w.sigma, w.n_out, w.out_scale, w.dtype,
                                     want_means=(w.query == "mixture"))
    V = synth.values(base, H, cap, w.d, w.dtype)
    init = oracle.init_positions(H, w.L, w.C, base)
    return base, K, V, init, means


def queries(w, base, step: int, K: np.ndarray, n_cur: int, means, heads: int | None = None):
    H = w.heads if heads is None else heads
    if w.query == "mixture":
        return synth.queries_mixture(base, step, H * w.G, w.G, means, w.q_sigma, w.dtype)
    return synth.queries_noisy_key(base, step, H * w.G, w.G, K, n_cur, w.q_sigma)


def split_ws(idx, q_heads: int) -> torch.Tensor:
    """Workspace for the token split of the fused selection and attention: the per-head arrival
    counters zero, the partial results filled with NaN bytes (their contents must not matter)."""
    import clustered_sparse_attention_kv_amd as kvc
    ws = torch.full((kvc.select_decode_workspace_bytes(idx.heads, q_heads, idx.d),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    ws[:(4 * idx.heads + 255) // 256 * 256] = 0
    return ws
