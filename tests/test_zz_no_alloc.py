"""The allocation-free entry point kv_sparse_decode_noalloc, through the C
ABI, against kv_sparse_decode (its workspace-taking twin) on two calls in a
row, the second smaller than the first: the same kernels, so the outputs
match bit for bit; and both within 2e-3 of the oracle's attention."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _helpers import to_dev, to_np

pytestmark = pytest.mark.gpu
kvc = pytest.importorskip("clustered_sparse_attention_kv_amd")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def one_call(H, G, cap, B, seed):
    base = synth.config_seed(60, seed)
    d = 128
    K = synth.normal_array(synth.stream_seed(base, 0, 1), (H, cap, d), 1.0, synth.BF16)
    V = synth.normal_array(synth.stream_seed(base, 0, 2), (H, cap, d), 1.0, synth.BF16)
    q = synth.normal_array(synth.stream_seed(base, 0, 3), (H * G, d), 1.0, synth.BF16)
    rng = np.random.default_rng(seed)
    sel = np.stack([rng.permutation(cap)[:B] for _ in range(H)]).astype(np.int32)
    cnt = rng.integers(1, B + 1, H).astype(np.int32)
    cnt[0] = B
    scale = 1.0 / math.sqrt(d)
    qd, Kd, Vd, sd, cd = to_dev(q), to_dev(K), to_dev(V), to_dev(sel), to_dev(cnt)
    out_na = torch.full((H * G, d), float("nan"), dtype=torch.float32, device="cuda")
    kvc.sparse_decode_noalloc(qd, Kd, Vd, sd, cd, scale, out=out_na)
    ref = kvc.sparse_decode(qd, Kd, Vd, sd, cd, scale)
    torch.cuda.synchronize()
    assert torch.equal(out_na, ref), "noalloc differs from kv_sparse_decode"
    od = oracle.decode(q, G, K, V, sel, cnt, scale)
    err = float(np.abs(to_np(out_na) - od).max())
    say(f"  heads={H} G={G} B={B}: bit-identical to kv_sparse_decode, max abs err vs oracle {err:.2e}")
    assert err <= 2e-3


def test_noalloc_matches_workspace_decode_twice():
    # first call: 64 KV heads x 8 query heads x 1024 selected (4.26 MB of partials)
    one_call(H=64, G=8, cap=3000, B=1024, seed=1)
    # second call, smaller: fewer heads, splits and query heads; the scratch
    # keeps the first call's contents, which must not matter
    one_call(H=5, G=2, cap=700, B=130, seed=2)
