"""Parity at the full sizes of the synthetic workloads, in the configuration
the benchmark times (kv_cluster_build, then kv_cluster_select_decode per
decode step; the split select + decode path is checked beside it).

The GPU runs every head, and the oracle re-runs the k-means of every head of
the layers it checks (all 32 heads of workloads 2 and 3, all 128 of workload
4, all 64 of four of workload 5's 32 layers); the cluster index, selection and
decode are checked for every head given the GPU's own clustering (integer
results bit-exact, attention within 2e-3)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _helpers import queries, split_ws, to_dev, to_np

pytestmark = pytest.mark.gpu
kvc = pytest.importorskip("clustered_sparse_attention_kv_amd")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gen(w, layer=0):
    base = synth.config_seed(w.config, layer)
    K, _, means = synth.mixture_keys(base, w.heads, w.capacity, w.d, w.M, w.sigma, w.n_out, w.out_scale, w.dtype,
                                     want_means=(w.query == "mixture"))
    V = synth.values(base, w.heads, w.capacity, w.d, w.dtype)
    init = oracle.init_positions(w.heads, w.L, w.C, base)
    return base, K, V, init, means


def check_build(w, K, init, idx, heads=None):
    """The oracle's k-means of the given heads (all by default) against the
    GPU's: label agreement, centroids of clusters with identical membership,
    operand from the GPU's centroids; the index bit-exact given the GPU's
    labels on every head."""
    gl = to_np(idx.labels)[:, :w.L]
    gc = to_np(idx.centroids)
    opt = oracle.BF16 if w.dtype == synth.BF16 else oracle.F32
    sizes, offsets, ids = to_np(idx.sizes), to_np(idx.offsets), to_np(idx.token_ids)[:, :w.L]
    for h in range(w.heads):
        s, o, i = oracle.csr(gl[h], w.C)
        assert np.array_equal(sizes[h], s) and np.array_equal(offsets[h], o) and np.array_equal(ids[h], i), h
    sample = list(range(w.heads)) if heads is None else list(heads)
    Ks = np.ascontiguousarray(K[sample, :w.L])
    ref = oracle.build(Ks, w.C, w.iters, np.ascontiguousarray(init[sample]))
    agree = (gl[sample] == ref["labels"]).mean()
    worst, same, total = 0.0, 0, 0
    gop = to_np(idx.centroids_op)
    for a, h in enumerate(sample):
        ro, ri = ref["offsets"][a], ref["token_ids"][a]
        for k in range(w.C):
            total += 1
            if ro[k + 1] - ro[k] == offsets[h, k + 1] - offsets[h, k] and np.array_equal(
                    ri[ro[k]:ro[k + 1]], ids[h, offsets[h, k]:offsets[h, k + 1]]):
                same += 1
                nrm = max(np.linalg.norm(ref["c"][a, k]), 1e-30)
                worst = max(worst, np.linalg.norm(gc[h, k] - ref["c"][a, k]) / nrm)
        assert np.array_equal(gop[h, :w.C], oracle.normalize(gc[h], opt))
    say(f"  {len(sample)} heads: label agreement {agree:.6f}, {same}/{total} clusters with identical members, "
        f"centroid rel err {worst:.2e}")
    assert agree >= 0.999 and worst <= 1e-3


def check_step(w, idx, K, V, Kd, Vd, q, B, scale, c=None, sizes=None, offsets=None, token_ids=None, split=True):
    H = w.heads
    qd = to_dev(q)
    fsel = torch.empty(H, B, dtype=torch.int32, device="cuda")
    fcnt = torch.empty(H, dtype=torch.int32, device="cuda")
    fout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, sel_ids=fsel, sel_count=fcnt)
    # the token split (its own copies of the selection)
    tsel = torch.empty(H, B, dtype=torch.int32, device="cuda")
    tcnt = torch.empty(H, dtype=torch.int32, device="cuda")
    tout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, sel_ids=tsel, sel_count=tcnt,
                             workspace=split_ws(idx, H * w.G))
    # and without ids to return (the clusters above the cut gathered before the ranking)
    eout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, workspace=split_ws(idx, H * w.G))
    if split:
        sel, cnt = kvc.select(idx, qd, B)
        out = kvc.sparse_decode(qd, Kd, Vd, sel, cnt, scale)
    torch.cuda.synchronize()
    c = to_np(idx.centroids) if c is None else c
    sizes = to_np(idx.sizes) if sizes is None else sizes
    offsets = to_np(idx.offsets) if offsets is None else offsets
    token_ids = to_np(idx.token_ids) if token_ids is None else token_ids
    osel, ocnt, _, _ = oracle.select(q, w.G, c, sizes, offsets, token_ids, B)
    assert np.array_equal(to_np(fcnt), ocnt) and np.array_equal(to_np(fsel), osel)
    assert np.array_equal(to_np(tcnt), ocnt) and np.array_equal(to_np(tsel), osel)
    od = oracle.decode(q, w.G, K, V, osel, ocnt, scale)
    ferr = max(float(np.abs(to_np(fout) - od).max()), float(np.abs(to_np(tout) - od).max()),
               float(np.abs(to_np(eout) - od).max()))
    err = float(np.abs(to_np(out) - od).max()) if split else 0.0
    if split:
        assert np.array_equal(to_np(sel), osel) and np.array_equal(to_np(cnt), ocnt)
    assert ferr <= 2e-3 and err <= 2e-3
    return ferr, err


@pytest.mark.parametrize("cfg", [2, 4])
def test_full_size_build_select_decode(cfg):
    w = synth.workload(cfg)
    say(f"[full size] {w.name}: {w.heads} heads x {w.L} keys, C={w.C}, B={w.B}")
    base, K, V, init, means = gen(w)
    idx = kvc.ClusterIndex(w.heads, w.C, w.capacity, torch.bfloat16, packed=True)
    Kd, Vd = to_dev(K), to_dev(V)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    assert int(to_np(idx.dev_flags)[0]) == 0
    check_build(w, K, init, idx)
    scale = 1.0 / math.sqrt(w.d)
    for step in (0, 1, w.steps - 1):
        q = queries(w, base, step, K, w.L, means)
        ferr, err = check_step(w, idx, K, V, Kd, Vd, q, w.B, scale)
        say(f"  step {step}: decode max abs err fused {ferr:.2e}, split {err:.2e}")
    # the benchmark's configuration: the fused path reading the packed copy
    kvc.pack(idx, Kd, Vd)
    for step in (2, w.steps - 2):
        q = queries(w, base, step, K, w.L, means)
        ferr, _ = check_step(w, idx, K, V, Kd, Vd, q, w.B, scale, split=False)
        say(f"  step {step} (packed): decode max abs err fused {ferr:.2e}")


def test_full_size_dense_decode():
    """The full-KV comparator at the benchmark's size: every KV head, all
    32768 rows, against the oracle's attention."""
    w = synth.workload(4)
    base, K, V, init, means = gen(w)
    Kd, Vd = to_dev(K), to_dev(V)
    scale = 1.0 / math.sqrt(w.d)
    q = queries(w, base, 0, K, w.L, means)
    out = kvc.dense_decode(to_dev(q), Kd, Vd, w.L, scale)
    torch.cuda.synchronize()
    allsel = np.tile(np.arange(w.L, dtype=np.int32), (w.heads, 1))
    od = oracle.decode(q, w.G, K, V, allsel, np.full(w.heads, w.L, np.int32), scale)
    err = float(np.abs(to_np(out) - od).max())
    say(f"[full size dense] {w.heads} heads x {w.L} rows: max abs err {err:.2e}")
    assert err <= 2e-3


def test_full_size_append_workload():
    w = synth.workload(3)
    say(f"[full size] {w.name}: {w.heads} heads x {w.L} keys + {w.steps} appended, C={w.C}, B={w.B}")
    base, K, V, init, means = gen(w)
    Kp, Vp = K.copy(), V.copy()
    Kp[:, w.L:] = 0
    Vp[:, w.L:] = 0
    idx = kvc.ClusterIndex(w.heads, w.C, w.capacity, torch.bfloat16)
    Kd, Vd = to_dev(Kp), to_dev(Vp)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    check_build(w, K, init, idx)
    built = dict(labels=to_np(idx.labels)[:, :w.L], sizes=to_np(idx.sizes), offsets=to_np(idx.offsets),
                 token_ids=to_np(idx.token_ids)[:, :w.L], c=to_np(idx.centroids),
                 chat=to_np(idx.centroids_op)[:, :w.C])
    oi = oracle.Index(built, w.capacity)
    scale = 1.0 / math.sqrt(w.d)
    for s in range(w.steps):
        n = w.L + s
        kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n])), to_dev(np.ascontiguousarray(V[:, n])))
        oi.append(np.ascontiguousarray(K[:, n]))
        if s % 64 == 0 or s == w.steps - 1:
            q = queries(w, base, s, K, n + 1, means)
            assert np.array_equal(to_np(idx.labels)[:, :n + 1], oi.labels[:, :n + 1])
            off, ids = kvc.export_csr(idx)
            assert np.array_equal(to_np(off), oi.offsets) and np.array_equal(to_np(ids)[:, :n + 1],
                                                                              oi.token_ids[:, :n + 1])
            ferr, err = check_step(w, idx, K, V, Kd, Vd, q, w.B, scale, c=oi.c, sizes=oi.sizes,
                                   offsets=oi.offsets, token_ids=oi.token_ids)
            say(f"  step {s}: {n + 1} tokens, decode max abs err fused {ferr:.2e}, split {err:.2e}")


@pytest.mark.parametrize("layer", [0, 10, 21, 31])
def test_full_size_layer_stack(layer):
    """The 32-layer stack runs layer by layer through the same calls; four
    layers (independent seeded mixtures, the first and the last among them)
    are built and checked at their full size: the k-means of all 64 KV heads
    against the oracle's, then 8 of the 64 decode steps on the benchmark's
    configuration (the fused kernel reading the packed copy, and the token
    split), every head."""
    w = synth.workload(5)
    scale = 1.0 / math.sqrt(w.d)
    say(f"[full size] {w.name} layer {layer}: {w.heads} heads x {w.L} keys, C={w.C}, B={w.B}")
    base, K, V, init, means = gen(w, layer)
    idx = kvc.ClusterIndex(w.heads, w.C, w.capacity, torch.bfloat16, packed=True)
    Kd, Vd = to_dev(K), to_dev(V)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    check_build(w, K, init, idx)
    kvc.pack(idx, Kd, Vd)
    worst = 0.0
    for step in range(0, w.steps, 8):
        q = queries(w, base, step, K, w.L, means)
        ferr, _ = check_step(w, idx, K, V, Kd, Vd, q, w.B, scale, split=(step == 0))
        worst = max(worst, ferr)
    say(f"  8 decode steps: decode max abs err {worst:.2e}")
    del Kd, Vd, idx
    torch.cuda.empty_cache()
