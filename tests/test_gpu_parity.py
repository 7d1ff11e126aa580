"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same
seeded inputs: each kernel step on its own, then the whole path.

Bars: cluster index and selection bit-exact given identical inputs; labels
bit-exact given an identical operand (the certified argmax resolves every
near-tie in fp64); centroids within 1e-3 relative; attention within 2e-3
max-abs (bf16 inputs, fp32 accumulation)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _helpers import split_ws, make_inputs, queries, to_dev, to_np, torch_dtype

pytestmark = pytest.mark.gpu

kvc = pytest.importorskip("clustered_sparse_attention_kv_amd")

SMALL = synth.Workload("small_bf16_ragged", 90, heads=3, G=2, L=1500, d=128, dtype=synth.BF16, M=20, sigma=0.3,
                       n_out=4, out_scale=10.0, C=40, iters=6, B=200, steps=3, query="noisy_key", q_sigma=0.1)
SMALL_APPEND = synth.Workload("small_bf16_append", 91, heads=2, G=1, L=1100, d=128, dtype=synth.BF16, M=24,
                              sigma=0.3, n_out=4, out_scale=10.0, C=37, iters=5, B=300, steps=20, query="noisy_key",
                              q_sigma=0.1, append=True)
LONG_APPEND = synth.Workload("long_append_bf16", 94, heads=2, G=1, L=600, d=128, dtype=synth.BF16, M=12,
                             sigma=0.3, n_out=4, out_scale=10.0, C=9, iters=3, B=300, steps=4400, query="noisy_key",
                             q_sigma=0.1, append=True)
SMALL_WINDOW = synth.Workload("small_bf16_window", 92, heads=3, G=2, L=1100, d=128, dtype=synth.BF16, M=24,
                              sigma=0.3, n_out=4, out_scale=10.0, C=37, iters=5, B=300, steps=130,
                              query="noisy_key", q_sigma=0.1, append=True)
CASES = {"cfg1_fp32": synth.workload(1), "small_bf16": SMALL}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pad_op(chat: np.ndarray, cpad: int) -> np.ndarray:
    H, C, d = chat.shape
    out = np.zeros((H, cpad, d), dtype=chat.dtype)
    out[:, :C] = chat
    return out


def built_gpu(w, K, seed, packed=False):
    idx = kvc.ClusterIndex(K.shape[0], w.C, w.capacity, torch_dtype(w), packed=packed)
    Kd = to_dev(K)
    kvc.build(idx, Kd, w.L, w.iters, seed=seed)
    torch.cuda.synchronize()
    return idx, Kd


@pytest.mark.parametrize("case", list(CASES))
def test_assign_step_bit_exact(case):
    w = CASES[case]
    say(f"[assign step] {case}")
    base, K, V, init, _ = make_inputs(w)
    H = K.shape[0]
    opt = oracle.BF16 if w.dtype == synth.BF16 else oracle.F32
    # operand: normalised initial centroids, then one oracle iteration later
    c0 = np.stack([K[h, init[h]].astype(np.float32) if w.dtype == synth.F32 else oracle.to_f64(K[h, init[h]])
                   .astype(np.float32) for h in range(H)])
    for it in range(2):
        chat = np.stack([oracle.normalize(c0[h], opt) for h in range(H)])
        want = np.stack([oracle.assign(K[h, :w.L], chat[h])[0] for h in range(H)])
        idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w))
        labels, top2, flagged = kvc.debug_assign(idx, to_dev(K), w.L, to_dev(pad_op(chat, kvc.cpad(w.C))),
                                                 want_top2=(w.dtype == synth.BF16))
        got = to_np(labels)[:, :w.L]
        say(f"  iter {it}: flagged per head {to_np(flagged).tolist()}, mismatches {(got != want).sum()}")
        assert np.array_equal(got, want)
        if top2 is not None:
            # the matrix-core best score is within the certification bound of the exact one
            t2 = to_np(top2)
            best = np.stack([oracle.assign(K[h, :w.L], chat[h])[1] for h in range(H)])
            kn = np.linalg.norm(oracle.to_f64(K[:, :w.L]), axis=2)
            bound = 4 * (w.d + 16) * 2.0 ** -24 * kn * 1.004
            err = np.abs(t2[..., 0] - best)
            say(f"  max |fp32 best - fp64 best| / bound = {(err / bound).max():.3e}")
            assert np.all(err <= bound)
            # the kernel certifies exactly the keys whose best and runner-up are
            # further apart than the threshold from the exact key norm (up to
            # keys on the threshold itself): a wrong norm in the kernel shows up
            # as a different number of queued keys
            m1, m2 = t2[..., 0].astype(np.float64), t2[..., 1].astype(np.float64)
            thr = (2 * 4 * (w.d + 16) * 2.0 ** -24 * 1.02) * kn + 2.0 ** -15 * 1.02 * np.maximum(np.abs(m1), np.abs(m2))
            want_flag = (~(m1 - m2 > thr)).sum(axis=1)
            got_flag = to_np(flagged)
            say(f"  queued per head: kernel {got_flag.tolist()}, from exact norms {want_flag.tolist()}")
            assert np.all(np.abs(got_flag - want_flag) <= np.maximum(2, want_flag // 100))
        c0 = np.stack([oracle.update(K[h, :w.L], want[h], c0[h])[0] for h in range(H)])


@pytest.mark.parametrize("case", list(CASES))
def test_update_step_bit_exact(case):
    w = CASES[case]
    say(f"[update step] {case}")
    base, K, V, init, _ = make_inputs(w)
    H = K.shape[0]
    rng = np.random.default_rng(11)
    labels = rng.integers(0, w.C, (H, w.L)).astype(np.int32)
    labels[labels == 3] = 4  # cluster 3 empty: keeps its previous centroid
    prev = rng.standard_normal((H, w.C, w.d)).astype(np.float32)
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w))
    lab_full = np.full((H, w.capacity), -1, np.int32)
    lab_full[:, :w.L] = labels
    idx.labels.copy_(to_dev(lab_full))
    idx.centroids.copy_(to_dev(prev))
    kvc.debug_update(idx, to_dev(K), w.L)
    torch.cuda.synchronize()
    opt = oracle.BF16 if w.dtype == synth.BF16 else oracle.F32
    for h in range(H):
        s, o, i = oracle.csr(labels[h], w.C)
        assert np.array_equal(to_np(idx.sizes)[h], s)
        assert np.array_equal(to_np(idx.offsets)[h], o)
        assert np.array_equal(to_np(idx.token_ids)[h, :w.L], i)
        c, _ = oracle.update(K[h, :w.L], labels[h], prev[h])
        assert np.array_equal(to_np(idx.centroids)[h], c)
        assert np.array_equal(to_np(idx.centroids_op)[h, :w.C], oracle.normalize(c, opt))


@pytest.mark.parametrize("case", list(CASES))
def test_build_select_decode_end_to_end(case):
    w = CASES[case]
    say(f"[end to end] {case}")
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    idx, Kd = built_gpu(w, K, base, packed=True)
    assert int(to_np(idx.dev_flags)[0]) == 0
    ref = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, init)
    gl = to_np(idx.labels)[:, :w.L]
    agree = (gl == ref["labels"]).mean()
    say(f"  label agreement {agree:.6f}")
    assert agree >= 0.999
    gc = to_np(idx.centroids)
    same = [(h, k) for h in range(H) for k in range(w.C)
            if np.array_equal(np.flatnonzero(gl[h] == k), np.flatnonzero(ref["labels"][h] == k))]
    rel = max(np.linalg.norm(gc[h, k] - ref["c"][h, k]) / max(np.linalg.norm(ref["c"][h, k]), 1e-30)
              for h, k in same)
    say(f"  centroid rel err (same membership, {len(same)} clusters) {rel:.3e}")
    assert rel <= 1e-3
    # index bit-exact given the GPU's labels; operand bit-exact given its centroids
    opt = oracle.BF16 if w.dtype == synth.BF16 else oracle.F32
    for h in range(H):
        s, o, i = oracle.csr(gl[h], w.C)
        assert np.array_equal(to_np(idx.sizes)[h], s) and np.array_equal(to_np(idx.offsets)[h], o)
        assert np.array_equal(to_np(idx.token_ids)[h, :w.L], i)
        assert np.array_equal(to_np(idx.centroids_op)[h, :w.C], oracle.normalize(gc[h], opt))
    # selection (bit-exact given the GPU's index) and sparse decode (<= 2e-3)
    Vd = to_dev(V)
    ws = torch.zeros(kvc.decode_workspace_bytes(H, H * w.G, max(w.B, 1)) + 4096, dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(w.d)
    cases = [(step, B) for step, B in enumerate([w.B, 1, 7, w.L + 50])]
    for pk in (False, True):
        if pk:
            # the packed copy: row i of head h is the cache row token_ids[h][i]
            kvc.pack(idx, Kd, Vd)
            torch.cuda.synchronize()
            ids = to_np(idx.token_ids)[:, :w.L]
            for h in range(H):
                assert np.array_equal(to_np(idx.k_packed)[h, :w.L], K[h, ids[h]])
                assert np.array_equal(to_np(idx.v_packed)[h, :w.L], V[h, ids[h]])
        for step, B in cases:
            check_step(w, idx, base, K, V, Kd, Vd, means, gc, step, B, scale, pk)
    del ws


def check_step(w, idx, base, K, V, Kd, Vd, means, gc, step, B, scale, packed):
    H = K.shape[0]
    q = queries(w, base, step, K, w.L, means)
    sel, cnt = kvc.select(idx, to_dev(q), B)
    ws_b = torch.zeros(kvc.decode_workspace_bytes(H, H * w.G, B), dtype=torch.uint8, device="cuda")
    out = kvc.sparse_decode(to_dev(q), Kd, Vd, sel, cnt, scale, workspace=ws_b)
    torch.cuda.synchronize()
    osel, ocnt, _, _ = oracle.select(q, w.G, gc, to_np(idx.sizes), to_np(idx.offsets), to_np(idx.token_ids), B)
    assert np.array_equal(to_np(cnt), ocnt), B
    assert np.array_equal(to_np(sel), osel), B
    od = oracle.decode(q, w.G, K, V, to_np(sel), to_np(cnt), scale)
    err = np.abs(to_np(out) - od).max()
    # the fused kernel (one kernel, then the token split and its merge): same
    # selection, same attention
    ferrs = []
    for ws in (None, split_ws(idx, H * w.G)):
        fsel = torch.full((H, B), -7, dtype=torch.int32, device="cuda")
        fcnt = torch.empty(H, dtype=torch.int32, device="cuda")
        fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, B, scale, sel_ids=fsel, sel_count=fcnt, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(fcnt), ocnt) and np.array_equal(to_np(fsel), osel), (B, ws is None)
        ferrs.append(np.abs(to_np(fout) - od).max())
        if ws is not None:  # no ids to return: the clusters above the cut are gathered before the ranking
            fcnt2 = torch.empty(H, dtype=torch.int32, device="cuda")
            fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, B, scale, sel_count=fcnt2, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(fcnt2), ocnt), B
            ferrs.append(np.abs(to_np(fout) - od).max())
    say(f"  B={B}{' packed' if packed else ''}: count {to_np(cnt).tolist()[:4]}, decode max abs err {err:.3e}, "
        f"fused {ferrs[0]:.3e}, token split {ferrs[1]:.3e}")
    assert err <= 2e-3 and max(ferrs) <= 2e-3


def test_append_long_lists():
    """Long appended lists: two calls of 2200 tokens per head (one launch
    each, the tokens inserted in order, every insert shifting the later
    clusters' entries); the labels, sizes and exported index equal the
    oracle's after each call."""
    w = LONG_APPEND
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), packed=True)
    Kc, Vc = np.zeros_like(K), np.zeros_like(V)
    Kc[:, :w.L], Vc[:, :w.L] = K[:, :w.L], V[:, :w.L]
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    built = dict(labels=to_np(idx.labels)[:, :w.L], sizes=to_np(idx.sizes), offsets=to_np(idx.offsets),
                 token_ids=to_np(idx.token_ids)[:, :w.L], c=to_np(idx.centroids),
                 chat=to_np(idx.centroids_op)[:, :w.C])
    oi = oracle.Index(built, w.capacity)
    n = w.L
    for nn in (2200, 2200):
        kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + nn])),
                   to_dev(np.ascontiguousarray(V[:, n:n + nn])))
        for t in range(nn):
            oi.append(np.ascontiguousarray(K[:, n + t]))
        n += nn
        torch.cuda.synchronize()
        assert np.array_equal(to_np(idx.labels)[:, :n], oi.labels[:, :n]), n
        assert np.array_equal(to_np(idx.sizes), oi.sizes), n
        off, ids = kvc.export_csr(idx)
        assert np.array_equal(to_np(off), oi.offsets), n
        assert np.array_equal(to_np(ids)[:, :n], oi.token_ids[:, :n]), n
    say(f"[long append] {n - w.L} tokens per head, sizes {oi.sizes[0].tolist()}")


def test_append_then_select_decode():
    w = SMALL_APPEND
    say("[append]")
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), packed=True)
    Kc = np.zeros_like(K)
    Vc = np.zeros_like(V)
    Kc[:, :w.L], Vc[:, :w.L] = K[:, :w.L], V[:, :w.L]
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    kvc.pack(idx, Kd, Vd)
    torch.cuda.synchronize()
    assert idx._s.packed == 1
    # the oracle index continues from the GPU's built state (identical centroids)
    built = dict(labels=to_np(idx.labels)[:, :w.L], sizes=to_np(idx.sizes), offsets=to_np(idx.offsets),
                 token_ids=to_np(idx.token_ids)[:, :w.L], c=to_np(idx.centroids),
                 chat=to_np(idx.centroids_op)[:, :w.C])
    oi = oracle.Index(built, w.capacity)
    n = w.L
    scale = 1.0 / math.sqrt(w.d)
    steps = [1] * 12 + [3, 1, 4]
    for s, nn in enumerate(steps):
        kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + nn])),
                   to_dev(np.ascontiguousarray(V[:, n:n + nn])))
        for t in range(nn):
            oi.append(np.ascontiguousarray(K[:, n + t]))
        n += nn
        assert idx.n_tokens == n
        q = queries(w, base, s, K, n, means)
        sel, cnt = kvc.select(idx, to_dev(q), w.B)
        out = kvc.sparse_decode(to_dev(q), Kd, Vd, sel, cnt, scale)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(idx.labels)[:, :n], oi.labels[:, :n])
        assert np.array_equal(to_np(idx.sizes), oi.sizes)
        osel, ocnt, _, _ = oracle.select(q, w.G, oi.c, oi.sizes, oi.offsets, oi.token_ids, w.B)
        assert np.array_equal(to_np(sel), osel) and np.array_equal(to_np(cnt), ocnt)
        od = oracle.decode(q, w.G, K, V, osel, ocnt, scale)
        assert np.abs(to_np(out) - od).max() <= 2e-3
        # fused, from the packed copy plus the appended rows, then from the caches alone
        for pk, ws in ((1, None), (0, None), (1, split_ws(idx, H * w.G)), (0, split_ws(idx, H * w.G))):
            idx._s.packed = pk
            fsel = torch.full((H, w.B), -7, dtype=torch.int32, device="cuda")
            fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, w.B, scale, sel_ids=fsel, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(fsel), osel), (pk, ws is None)
            assert np.abs(to_np(fout) - od).max() <= 2e-3, (pk, ws is None)
        idx._s.packed = 1
    off, ids = kvc.export_csr(idx)
    assert np.array_equal(to_np(off), oi.offsets)
    assert np.array_equal(to_np(ids)[:, :n], oi.token_ids[:, :n])
    assert np.array_equal(to_np(Kd)[:, :n], K[:, :n]) and np.array_equal(to_np(Vd)[:, :n], V[:, :n])
    with pytest.raises(kvc.KvcError):
        kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, :w.capacity - n + 1])),
                   to_dev(np.ascontiguousarray(V[:, :w.capacity - n + 1])))
    say(f"  appended {n - w.L} tokens; final sizes sum {to_np(idx.sizes).sum(axis=1).tolist()}")


def test_dense_decode_matches_full_attention():
    """The full-KV comparator: attention over every one of the first n rows
    (II.A) against the oracle's, for ragged n and a single row."""
    w = SMALL
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    Kd, Vd = to_dev(K), to_dev(V)
    scale = 1.0 / math.sqrt(w.d)
    for n in (w.L, 1, 777):
        q = queries(w, base, n, K, n, means)
        out = kvc.dense_decode(to_dev(q), Kd, Vd, n, scale)
        torch.cuda.synchronize()
        allsel = np.tile(np.arange(n, dtype=np.int32), (H, 1))
        od = oracle.decode(q, w.G, K, V, allsel, np.full(H, n, np.int32), scale)
        err = float(np.abs(to_np(out) - od).max())
        say(f"  dense n={n}: max abs err {err:.2e}")
        assert err <= 2e-3


def test_attention_sinks_end_to_end():
    """III.B: the first tokens are attention sinks, kept out of the clustering
    and always recalled. Build, selection (split and fused, from the caches and
    from the packed copy, budgets below, at and above the sink count), attention
    and appends against the oracle with the same n_sink."""
    w, n_sink = SMALL_APPEND, 16
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    init = oracle.init_positions(H, w.L, w.C, base, n_sink)
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), packed=True, n_sink=n_sink)
    Kc, Vc = K.copy(), V.copy()
    Kc[:, w.L:], Vc[:, w.L:] = 0, 0
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    assert int(to_np(idx.dev_flags)[0]) == 0
    ref = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, init, n_sink=n_sink)
    gl = to_np(idx.labels)[:, :w.L]
    assert np.all(gl[:, :n_sink] == -1)
    assert np.array_equal(gl, ref["labels"])
    assert np.array_equal(to_np(idx.centroids), ref["c"])
    nc = w.L - n_sink
    assert np.array_equal(to_np(idx.sizes), ref["sizes"]) and np.array_equal(to_np(idx.offsets), ref["offsets"])
    assert np.array_equal(to_np(idx.token_ids)[:, :nc], ref["token_ids"])
    built = dict(labels=gl, sizes=to_np(idx.sizes), offsets=to_np(idx.offsets),
                 token_ids=to_np(idx.token_ids)[:, :nc], c=to_np(idx.centroids), chat=to_np(idx.centroids_op)[:, :w.C])
    oi = oracle.Index(built, w.capacity)
    scale = 1.0 / math.sqrt(w.d)
    n = w.L
    for step in range(4):
        if step > 0:  # append one token per head
            kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + 1])),
                       to_dev(np.ascontiguousarray(V[:, n:n + 1])))
            oi.append(np.ascontiguousarray(K[:, n]))
            n += 1
        if step == 0:
            kvc.pack(idx, Kd, Vd)
        q = queries(w, base, step, K, n, means)
        for B in (w.B, 5, n_sink, n + 40):
            osel, ocnt, _, _ = oracle.select(q, w.G, oi.c, oi.sizes, oi.offsets, oi.token_ids, B, n_sink=n_sink)
            od = oracle.decode(q, w.G, K, V, osel, ocnt, scale)
            sel, cnt = kvc.select(idx, to_dev(q), B)
            out = kvc.sparse_decode(to_dev(q), Kd, Vd, sel, cnt, scale)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(sel), osel) and np.array_equal(to_np(cnt), ocnt), (step, B)
            assert np.abs(to_np(out) - od).max() <= 2e-3
            for pk, ws in ((1, None), (0, None), (1, split_ws(idx, H * w.G))):
                idx._s.packed = pk
                fsel = torch.full((H, B), -7, dtype=torch.int32, device="cuda")
                fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, B, scale, sel_ids=fsel, workspace=ws)
                torch.cuda.synchronize()
                assert np.array_equal(to_np(fsel), osel), (step, B, pk, ws is None)
                assert np.abs(to_np(fout) - od).max() <= 2e-3, (step, B, pk, ws is None)
                if ws is not None:
                    fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, B, scale, workspace=ws)
                    torch.cuda.synchronize()
                    assert np.abs(to_np(fout) - od).max() <= 2e-3, (step, B, pk, "no ids")
            idx._s.packed = 1
        say(f"  sinks: step {step}, {n} tokens, count {ocnt.tolist()}")


def test_window_clustering_end_to_end():
    """III.B / Sys-A: generated tokens join a window that every selection
    recalls (after the attention sinks), and every m tokens the window alone is
    clustered into nc new clusters. Each clustering is checked bit-exact
    against the oracle (labels, centroids, operand, sizes, offsets, member ids,
    the packed copy's new rows); selections (split and fused, from the caches
    and from the packed copy, budgets that cut inside the window, after it and
    past every token) and attention are checked along the way; a
    nearest-centroid append after a clustering may pick a new cluster."""
    w, n_sink, m, nc = SMALL_WINDOW, 8, 40, 4
    base, K, V, _, means = make_inputs(w)
    H = K.shape[0]
    init = oracle.init_positions(H, w.L, w.C, base, n_sink)
    slots = w.C + 3 * nc
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), packed=True, n_sink=n_sink, c_slots=slots)
    Kc, Vc = K.copy(), V.copy()
    Kc[:, w.L:], Vc[:, w.L:] = 0, 0
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    kvc.pack(idx, Kd, Vd)
    torch.cuda.synchronize()
    ref = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, init, n_sink=n_sink)
    assert np.array_equal(to_np(idx.labels)[:, :w.L], ref["labels"])
    assert np.array_equal(to_np(idx.centroids)[:, :w.C], ref["c"])
    assert idx.c_active == w.C and idx.window_start == w.L
    oi = oracle.Index(ref, w.capacity)
    scale = 1.0 / math.sqrt(w.d)
    n, step, windows = w.L, 0, 0

    def check_index():
        ca, nt = oi.C, oi.n
        assert idx.c_active == ca and idx.window_start == oi.window_start and idx.n_tokens == nt
        assert np.array_equal(to_np(idx.labels)[:, :nt], oi.labels[:, :nt])
        assert np.array_equal(to_np(idx.centroids)[:, :ca], oi.c)
        assert np.array_equal(to_np(idx.centroids_op)[:, :ca], oi.chat)
        assert np.array_equal(to_np(idx.sizes)[:, :ca], oi.sizes)
        off, ids = kvc.export_csr(idx)
        off, ids = to_np(off), to_np(ids)
        assert np.array_equal(off[:, :ca + 1], oi.offsets) and np.all(off[:, ca + 1:] == oi.offsets[:, -1:])
        total = int(oi.offsets[0, -1])
        assert np.array_equal(ids[:, :total], oi.token_ids[:, :total])

    def check_select(q, B):
        win = (oi.window_start, oi.n)
        osel, ocnt, _, _ = oracle.select(q, w.G, oi.c, oi.sizes, oi.offsets, oi.token_ids, B, n_sink=n_sink,
                                         window=win)
        od = oracle.decode(q, w.G, K, V, osel, ocnt, scale)
        sel, cnt = kvc.select(idx, to_dev(q), B)
        out = kvc.sparse_decode(to_dev(q), Kd, Vd, sel, cnt, scale)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(sel), osel) and np.array_equal(to_np(cnt), ocnt), (step, B)
        assert np.abs(to_np(out) - od).max() <= 2e-3, (step, B)
        for pk, ws in ((1, None), (0, None), (1, split_ws(idx, H * w.G))):
            idx._s.packed = pk
            fsel = torch.full((H, B), -7, dtype=torch.int32, device="cuda")
            fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, B, scale, sel_ids=fsel, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(fsel), osel), (step, B, pk, ws is None)
            assert np.abs(to_np(fout) - od).max() <= 2e-3, (step, B, pk, ws is None)
            if ws is not None:
                fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, B, scale, workspace=ws)
                torch.cuda.synchronize()
                assert np.abs(to_np(fout) - od).max() <= 2e-3, (step, B, pk, "no ids")
        idx._s.packed = 1

    while n < w.capacity:
        kvc.append_window(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + 1])),
                          to_dev(np.ascontiguousarray(V[:, n:n + 1])))
        oi.add_window(1)
        n += 1
        step += 1
        if n - oi.window_start == m and oi.C + nc <= slots:
            init_w = synth.init_idx(synth.stream_seed(base, 7, windows), H, m, nc) + np.int32(n - m)
            kvc.cluster_window(idx, Kd, Vd, nc, w.iters, to_dev(init_w))
            oi.cluster_window(K, nc, w.iters, init_w)
            torch.cuda.synchronize()
            windows += 1
            assert int(to_np(idx.dev_flags)[0]) == 0
            check_index()
            # the packed copy holds every member of the main part, in index order
            total = int(oi.offsets[0, -1])
            kp, vp = to_np(idx.k_packed), to_np(idx.v_packed)
            for h in range(H):
                rows = oi.token_ids[h, :total]
                assert np.array_equal(kp[h, :total], K[h, rows]) and np.array_equal(vp[h, :total], V[h, rows])
            say(f"  window {windows} clustered at {n} tokens: {oi.C} clusters, sizes of the new ones "
                f"{oi.sizes[:, -nc:].tolist()}")
            if windows == 3 and n < w.capacity:
                # a nearest-centroid append, with the window empty
                kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + 1])),
                           to_dev(np.ascontiguousarray(V[:, n:n + 1])))
                oi.append(np.ascontiguousarray(K[:, n]))
                n += 1
                torch.cuda.synchronize()
                check_index()
        if step % 9 == 1 or n == w.capacity:
            q = queries(w, base, step, K, n, means)
            for B in (w.B, n_sink + 10, n + 40):
                check_select(q, B)
    assert windows == 3


@pytest.mark.parametrize("metric", ["cosine", "l2", "inner_product"])
@pytest.mark.parametrize("nc", [4, 40])
def test_window_clustering_one_launch_and_general(metric, nc):
    """Clustering a window of generated tokens takes one launch per call for
    up to 32 new clusters and the build's kernels beyond that; under each
    distance both give the oracle's result bit for bit (labels, centroids,
    operand, sizes, offsets, member ids)."""
    w, m = SMALL_WINDOW, 64
    mk, om = {"cosine": (kvc.COSINE, oracle.COSINE), "l2": (kvc.L2, oracle.L2),
              "inner_product": (kvc.INNER_PRODUCT, oracle.IP)}[metric]
    say(f"[window clustering] {metric}, {nc} clusters")
    base, K, V, init, _ = make_inputs(w)
    H = K.shape[0]
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), c_slots=w.C + nc, metric=mk)
    Kc, Vc = K.copy(), V.copy()
    Kc[:, w.L:], Vc[:, w.L:] = 0, 0
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    ref = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, init, metric=om)
    oi = oracle.Index(ref, w.capacity, metric=om)
    for n in range(w.L, w.L + m):
        kvc.append_window(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + 1])),
                          to_dev(np.ascontiguousarray(V[:, n:n + 1])))
        oi.add_window(1)
    init_w = synth.init_idx(synth.stream_seed(base, 11, nc), H, m, nc) + np.int32(w.L)
    kvc.cluster_window(idx, Kd, Vd, nc, w.iters, to_dev(init_w))
    oi.cluster_window(K, nc, w.iters, init_w)
    torch.cuda.synchronize()
    assert int(to_np(idx.dev_flags)[0]) == 0
    ca, nt = oi.C, oi.n
    assert idx.c_active == ca == w.C + nc and idx.n_tokens == nt
    assert np.array_equal(to_np(idx.labels)[:, :nt], oi.labels[:, :nt])
    assert np.array_equal(to_np(idx.centroids)[:, :ca], oi.c)
    assert np.array_equal(to_np(idx.centroids_op)[:, :ca], oi.chat)
    assert np.array_equal(to_np(idx.sizes)[:, :ca], oi.sizes)
    off, ids = kvc.export_csr(idx)
    off, ids = to_np(off), to_np(ids)
    assert np.array_equal(off[:, :ca + 1], oi.offsets)
    total = int(oi.offsets[0, -1])
    assert np.array_equal(ids[:, :total], oi.token_ids[:, :total])
    say(f"  new clusters' sizes {oi.sizes[:, -nc:].sum(axis=1).tolist()} (of {m} tokens per head)")


@pytest.mark.parametrize("metric", ["l2", "inner_product"])
@pytest.mark.parametrize("case", ["small_bf16_append", "cfg1_fp32"])
def test_distance_variants_end_to_end(case, metric):
    """III.B's alternatives to the cosine (L2 and inner-product distance): one
    assignment against a given operand (labels bit-exact; matrix-core scores
    within the certificate's bound), the whole build (labels, centroids,
    operand, index bit-exact), nearest-centroid appends under the same
    distance, and the selection and attention on the result."""
    w = SMALL_APPEND if case == "small_bf16_append" else synth.workload(1)
    m, om = {"l2": (kvc.L2, oracle.L2), "inner_product": (kvc.INNER_PRODUCT, oracle.IP)}[metric]
    say(f"[distance variant] {case} {metric}")
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    bf = w.dtype == synth.BF16
    opt = oracle.BF16 if bf else oracle.F32
    # one assignment against the operand of the initial centroids
    c0 = np.stack([oracle.to_f64(K[h, init[h]]).astype(np.float32) for h in range(H)])
    chat = np.stack([oracle.operand(c0[h], opt, om) for h in range(H)])
    want = np.stack([oracle.assign(K[h, :w.L], chat[h], om)[0] for h in range(H)])
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), metric=m)
    labels, top2, flagged = kvc.debug_assign(idx, to_dev(K), w.L, to_dev(pad_op(chat, kvc.cpad(w.C))), want_top2=bf)
    got = to_np(labels)[:, :w.L]
    say(f"  assign: flagged per head {to_np(flagged).tolist()}, mismatches {(got != want).sum()}")
    assert np.array_equal(got, want)
    if bf:
        best = np.stack([oracle.assign(K[h, :w.L], chat[h], om)[1] for h in range(H)])
        kn = np.linalg.norm(oracle.to_f64(K[:, :w.L]), axis=2)
        A = np.linalg.norm(oracle.to_f64(chat), axis=2).max(axis=1)[:, None]
        bmax = 0.5 * A * A if om == oracle.L2 else 0.0 * A
        bound = 4 * 2.0 ** -24 * ((w.d + 17) * kn * A + 2 * bmax) * 1.004
        err = np.abs(to_np(top2)[..., 0] - best)
        say(f"  max |fp32 best - fp64 best| / bound = {(err / bound).max():.3e}")
        assert np.all(err <= bound)
        # queued keys: exactly those within the threshold built from the exact
        # key norms, the largest operand norm and the largest bias
        t2 = to_np(top2).astype(np.float64)
        m1, m2 = t2[..., 0], t2[..., 1]
        thr = (2 * 4 * 2.0 ** -24 * 1.02) * ((w.d + 17) * kn * A + 2 * bmax) + \
            2.0 ** -15 * 1.02 * np.maximum(np.abs(m1), np.abs(m2))
        want_flag = (~(m1 - m2 > thr)).sum(axis=1)
        got_flag = to_np(flagged)
        say(f"  queued per head: kernel {got_flag.tolist()}, from exact norms {want_flag.tolist()}")
        assert np.all(np.abs(got_flag - want_flag) <= np.maximum(2, want_flag // 100))
    # the whole build
    Kc, Vc = K.copy(), V.copy()
    Kc[:, w.L:], Vc[:, w.L:] = 0, 0
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    assert int(to_np(idx.dev_flags)[0]) == 0
    ref = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, init, metric=om)
    gl = to_np(idx.labels)[:, :w.L]
    say(f"  build: label agreement {(gl == ref['labels']).mean():.6f}")
    assert np.array_equal(gl, ref["labels"])
    assert np.array_equal(to_np(idx.centroids), ref["c"])
    assert np.array_equal(to_np(idx.centroids_op)[:, :w.C], ref["chat"])
    assert np.array_equal(to_np(idx.sizes), ref["sizes"]) and np.array_equal(to_np(idx.offsets), ref["offsets"])
    assert np.array_equal(to_np(idx.token_ids)[:, :w.L], ref["token_ids"])
    oi = oracle.Index(ref, w.capacity, metric=om)
    n = w.L
    scale = 1.0 / math.sqrt(w.d)
    for step in range(3):
        if w.append and step > 0:
            kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + 1])),
                       to_dev(np.ascontiguousarray(V[:, n:n + 1])))
            oi.append(np.ascontiguousarray(K[:, n]))
            n += 1
            torch.cuda.synchronize()
            assert np.array_equal(to_np(idx.labels)[:, :n], oi.labels[:, :n])
        q = queries(w, base, step, K, n, means)
        osel, ocnt, _, _ = oracle.select(q, w.G, oi.c, oi.sizes, oi.offsets, oi.token_ids, w.B)
        od = oracle.decode(q, w.G, K, V, osel, ocnt, scale)
        fsel = torch.full((H, w.B), -7, dtype=torch.int32, device="cuda")
        fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, w.B, scale, sel_ids=fsel)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(fsel), osel), step
        assert np.abs(to_np(fout) - od).max() <= 2e-3, step


@pytest.mark.parametrize("where", ["device", "host"])
def test_cluster_cache_matches_uncached_path(where):
    """Sys-A / Sys-D: the KV lives in HBM or in pinned host memory (read by the
    kernels over the host link), and each decode step assembles the selected
    clusters through the R-step GPU cache. Every step, for R = 1 and 2 and with
    attention sinks: the selection equals the oracle's; the attention equals
    kv_sparse_decode over the same tokens bit for bit (the same kernel reads
    the same rows in the same order) and the oracle's within 2e-3; the cache's
    counters equal the oracle's simulation of the cache. The query sequence
    repeats and drifts so that steps hit, partly hit and miss."""
    w, n_sink = SMALL, 4
    base, K, V, _, means = make_inputs(w)
    H = K.shape[0]
    host = where == "host"
    init = oracle.init_positions(H, w.L, w.C, base, n_sink)
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), packed=True, n_sink=n_sink, packed_on_host=host)
    Kd, Vd = to_dev(K), to_dev(V)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    Ks, Vs = (Kd.cpu().pin_memory(), Vd.cpu().pin_memory()) if host else (Kd, Vd)
    kvc.pack(idx, Ks, Vs)
    torch.cuda.synchronize()
    if host:
        ids = to_np(idx.token_ids)[:, :w.L - n_sink]
        for h in range(H):
            assert np.array_equal(to_np(idx.k_packed)[h, :w.L - n_sink], K[h, ids[h]])
    labels, c = to_np(idx.labels), to_np(idx.centroids)
    sizes, offsets, token_ids = to_np(idx.sizes), to_np(idx.offsets), to_np(idx.token_ids)
    scale = 1.0 / math.sqrt(w.d)
    pattern = [0, 0, 1, 0, 2, 2, 1, 3, 3, 0]
    for R in (1, 2):
        cache = kvc.ClusterCache(idx, R, w.B)
        kvc.cache_reset(idx, cache)
        sim = oracle.ClusterCache(H, R)
        for t, qs in enumerate(pattern):
            q = queries(w, base, qs, K, w.L, means)
            sel = torch.full((H, w.B), -7, dtype=torch.int32, device="cuda")
            cnt = torch.empty(H, dtype=torch.int32, device="cuda")
            out = kvc.cached_select_decode(idx, cache, to_dev(q), Ks, Vs, scale, sel_ids=sel, sel_count=cnt)
            osel, ocnt, _, _ = oracle.select(q, w.G, c, sizes, offsets, token_ids, w.B, n_sink=n_sink)
            ref = kvc.sparse_decode(to_dev(q), Kd, Vd, to_dev(osel), to_dev(ocnt), scale)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(sel), osel) and np.array_equal(to_np(cnt), ocnt), (R, t)
            assert torch.equal(out, ref), (R, t)
            assert np.abs(to_np(out) - oracle.decode(q, w.G, K, V, osel, ocnt, scale)).max() <= 2e-3
            sim.step(osel, ocnt, labels)
            assert np.array_equal(to_np(cache.stats), sim.stats), (R, t, to_np(cache.stats), sim.stats)
        assert cache.step == len(pattern)
        say(f"  {where}, R={R}: {cache.hit_rates()}")


MANY = synth.Workload("many_clusters_bf16", 93, heads=3, G=2, L=3000, d=128, dtype=synth.BF16, M=40, sigma=0.3,
                      n_out=4, out_scale=10.0, C=100, iters=4, B=300, steps=4, query="noisy_key", q_sigma=0.1)


def test_selection_merge_and_full_ranking():
    """Selection orders only the clusters that can be selected (a size-weighted
    score histogram finds them) with one wave while there are at most 64 (a
    sorting network over 16, 32 or 64 lanes), and sorts every cluster beyond
    that: with 100 clusters, budgets needing a few, about 20, about 40, more
    than 64 and all clusters (and sinks) select exactly as the oracle, split
    and fused."""
    w, n_sink = MANY, 5
    base, K, V, _, means = make_inputs(w)
    H = K.shape[0]
    init = oracle.init_positions(H, w.L, w.C, base, n_sink)
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), packed=True, n_sink=n_sink)
    Kd, Vd = to_dev(K), to_dev(V)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    kvc.pack(idx, Kd, Vd)
    torch.cuda.synchronize()
    c, sizes, offsets, token_ids = (to_np(idx.centroids), to_np(idx.sizes), to_np(idx.offsets),
                                    to_np(idx.token_ids))
    scale = 1.0 / math.sqrt(w.d)
    for step, B in enumerate([3, 40, 300, 700, 1300, 2500, w.L + 60]):
        q = queries(w, base, step, K, w.L, means)
        osel, ocnt, _, order = oracle.select(q, w.G, c, sizes, offsets, token_ids, B, n_sink=n_sink)
        # clusters the budget reaches (the count of ranks the selection needs)
        ranks = [int(np.searchsorted(np.cumsum(sizes[h][order[h]]), max(B - n_sink, 0), side="left")) + 1
                 for h in range(H)]
        sel, cnt = kvc.select(idx, to_dev(q), B)
        torch.cuda.synchronize()
        say(f"  B={B}: clusters reached per head {ranks}, count {ocnt.tolist()}")
        assert np.array_equal(to_np(sel), osel) and np.array_equal(to_np(cnt), ocnt), B
        od = oracle.decode(q, w.G, K, V, osel, ocnt, scale)
        for ws in (None, split_ws(idx, H * w.G)):
            fsel = torch.full((H, B), -7, dtype=torch.int32, device="cuda")
            fout = kvc.select_decode(idx, to_dev(q), Kd, Vd, B, scale, sel_ids=fsel, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(fsel), osel), (B, ws is None)
            assert np.abs(to_np(fout) - od).max() <= 2e-3, (B, ws is None)


def test_graph_replay_matches_eager():
    """The benchmark captures a pass's decode steps (append, then fused
    selection and attention, with or without the token split and its merge
    kernel) in a HIP graph after a build and replays it after each new build.
    Every replay, with eager builds and synchronisations between replays,
    gives the eager run's outputs bit for bit."""
    w = SMALL_APPEND
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch_dtype(w), packed=True)
    Kc, Vc = K.copy(), V.copy()
    Kc[:, w.L:], Vc[:, w.L:] = 0, 0
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    initd = to_dev(init)
    ws = torch.empty(kvc.build_workspace_bytes(H, w.L, w.C, w.iters), dtype=torch.uint8, device="cuda")
    steps = 6
    Knew = [to_dev(np.ascontiguousarray(K[:, w.L + s:w.L + s + 1])) for s in range(steps)]
    Vnew = [to_dev(np.ascontiguousarray(V[:, w.L + s:w.L + s + 1])) for s in range(steps)]
    Q = [to_dev(queries(w, base, s, K, w.L + s + 1, means)) for s in range(steps)]
    outs = [torch.empty(H * w.G, w.d, dtype=torch.float32, device="cuda") for _ in range(steps)]
    scale = 1.0 / math.sqrt(w.d)

    def prepare():
        kvc.build(idx, Kd, w.L, w.iters, init_idx=initd, workspace=ws)
        kvc.pack(idx, Kd, Vd)

    wsd = split_ws(idx, H * w.G)

    def run():
        for s in range(steps):
            kvc.append(idx, Kd, Vd, Knew[s], Vnew[s])
            # every other step with the token split (its second kernel in the graph too)
            kvc.select_decode(idx, Q[s], Kd, Vd, w.B, scale, out=outs[s], workspace=wsd if s % 2 == 0 else None)

    prepare()
    run()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    prepare()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        prepare()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s], want[s]), (rep, s)
    say(f"  {steps} captured steps, 3 replays identical to the eager run")


def test_init_index_out_of_range_flag():
    w = SMALL
    base, K, V, init, _ = make_inputs(w)
    bad = init.copy()
    bad[1, 5] = w.L + 3
    idx = kvc.ClusterIndex(K.shape[0], w.C, w.capacity, torch.bfloat16)
    kvc.build(idx, to_dev(K), w.L, 1, init_idx=to_dev(bad))
    torch.cuda.synchronize()
    assert int(to_np(idx.dev_flags)[0]) & 1
