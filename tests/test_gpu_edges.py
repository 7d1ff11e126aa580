"""Parity of the HIP path with the oracle on the edge cases of the method and
of the GPU path's limits, through the C ABI:

- the seeded initial positions (device shuffle against the oracle's);
- the selection scores themselves (fp64, bit for bit);
- eight query heads per KV head on every decode path;
- exact ties in the assignment (duplicated initial keys: the lowest cluster
  wins and the other cluster empties and keeps its centroid) and in the
  selection (duplicated centroids: the lowest id ranks first);
- one cluster, and the largest cluster count the path supports (512);
- zero and NaN key rows;
- non-finite scores in the nearest-centroid append (a NaN operand row of
  cluster 0 or of a later cluster, an infinite one, a NaN key);
- a caller's selected count outside [0, B] in the standalone decode.

Integer results bit-exact; attention within 2e-3 max-abs."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _helpers import make_inputs, queries, split_ws, to_dev, to_np

pytestmark = pytest.mark.gpu
kvc = pytest.importorskip("clustered_sparse_attention_kv_amd")

G8 = synth.Workload("g8_bf16", 95, heads=4, G=8, L=2000, d=128, dtype=synth.BF16, M=24, sigma=0.3, n_out=4,
                    out_scale=10.0, C=48, iters=5, B=256, steps=3, query="mixture", q_sigma=0.2)
APPEND_NF = synth.Workload("append_nonfinite_bf16", 97, heads=3, G=1, L=700, d=128, dtype=synth.BF16, M=12,
                           sigma=0.3, n_out=4, out_scale=10.0, C=20, iters=4, B=100, steps=12, query="noisy_key",
                           q_sigma=0.1, append=True)
TIES = synth.Workload("ties_bf16", 96, heads=3, G=2, L=1300, d=128, dtype=synth.BF16, M=16, sigma=0.3, n_out=4,
                      out_scale=10.0, C=24, iters=6, B=200, steps=2, query="noisy_key", q_sigma=0.1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_build_exact(w, K, idx, ref):
    """Labels, centroids, operand and index equal to the oracle's, bit for bit."""
    L = w.L
    assert np.array_equal(to_np(idx.labels)[:, :L], ref["labels"])
    assert np.array_equal(to_np(idx.centroids), ref["c"])
    assert np.array_equal(to_np(idx.centroids_op)[:, :w.C], ref["chat"])
    assert np.array_equal(to_np(idx.sizes), ref["sizes"])
    assert np.array_equal(to_np(idx.offsets), ref["offsets"])
    assert np.array_equal(to_np(idx.token_ids)[:, :L], ref["token_ids"])


def check_decode_paths(w, idx, K, V, Kd, Vd, q, B, packed_too=True):
    """Selection on every path bit-exact with the oracle given the GPU's index;
    attention within 2e-3 on the split, fused, token-split and packed paths."""
    H = K.shape[0]
    scale = 1.0 / math.sqrt(w.d)
    qd = to_dev(q)
    c, sizes, offsets, ids = to_np(idx.centroids), to_np(idx.sizes), to_np(idx.offsets), to_np(idx.token_ids)
    osel, ocnt, _, _ = oracle.select(q, w.G, c, sizes, offsets, ids, B)
    od = oracle.decode(q, w.G, K, V, osel, ocnt, scale)
    sel, cnt = kvc.select(idx, qd, B)
    out = kvc.sparse_decode(qd, Kd, Vd, sel, cnt, scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(sel), osel) and np.array_equal(to_np(cnt), ocnt)
    errs = [float(np.abs(to_np(out) - od).max())]
    wss = [None] + ([split_ws(idx, H * w.G)] if w.G <= 4 else [])
    for ws in wss:
        fsel = torch.full((H, B), -7, dtype=torch.int32, device="cuda")
        fcnt = torch.empty(H, dtype=torch.int32, device="cuda")
        fout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, sel_ids=fsel, sel_count=fcnt, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(fsel), osel) and np.array_equal(to_np(fcnt), ocnt)
        errs.append(float(np.abs(to_np(fout) - od).max()))
        if ws is not None:  # no ids to return: the clusters above the cut are gathered before the ranking
            fout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, workspace=ws)
            torch.cuda.synchronize()
            errs.append(float(np.abs(to_np(fout) - od).max()))
    if packed_too and idx.k_packed is not None:
        kvc.pack(idx, Kd, Vd)
        for ws in wss:
            fsel = torch.full((H, B), -7, dtype=torch.int32, device="cuda")
            fcnt = torch.empty(H, dtype=torch.int32, device="cuda")
            fout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, sel_ids=fsel, sel_count=fcnt, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(fsel), osel) and np.array_equal(to_np(fcnt), ocnt)
            errs.append(float(np.abs(to_np(fout) - od).max()))
            if ws is not None:
                fout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, workspace=ws)
                torch.cuda.synchronize()
                errs.append(float(np.abs(to_np(fout) - od).max()))
    assert max(errs) <= 2e-3, errs
    return errs


@pytest.mark.parametrize("L,C,n_sink", [(1500, 40, 0), (1500, 400, 0), (32768, 40, 0), (32768, 400, 0),
                                        (32768, 400, 16), (600, 1, 0), (700, 512, 3), (512, 512, 0)])
def test_init_positions_match_oracle(L, C, n_sink):
    """The device's seeded partial Fisher-Yates shuffle (all swaps drawn at
    once, then resolved) gives the oracle's sequential positions bit for bit,
    including C = L - n_sink (a full shuffle) and heads whose draws collide."""
    H = 16
    seed = 0x5EED0000 + L + C
    got = to_np(kvc.init_positions(H, L, C, seed, n_sink=n_sink))
    torch.cuda.synchronize()
    want = oracle.init_positions(H, L, C, seed, n_sink)
    say(f"[init positions] L={L} C={C} n_sink={n_sink}: {H} heads")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case", ["cfg1", "g8", "cfg4"])
def test_debug_scores_bit_exact(case):
    """The selection's fp64 scores (III.C: clusters rank by their centroid's
    attention weight to the query) equal the oracle's chains bit for bit,
    given the GPU's centroids: workload 1 (fp32), eight query heads per KV
    head, and the benchmark workload at full size (128 KV heads, C = 400)."""
    w = {"cfg1": synth.workload(1), "g8": G8, "cfg4": synth.workload(4)}[case]
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    tdt = torch.bfloat16 if w.dtype == synth.BF16 else torch.float32
    idx = kvc.ClusterIndex(H, w.C, w.capacity, tdt)
    kvc.build(idx, to_dev(K), w.L, w.iters, seed=base)
    for step in (0, 1):
        q = queries(w, base, step, K, w.L, means)
        sc = to_np(kvc.debug_scores(idx, to_dev(q)))
        torch.cuda.synchronize()
        _, _, osc, _ = oracle.select(q, w.G, to_np(idx.centroids), to_np(idx.sizes), to_np(idx.offsets),
                                     to_np(idx.token_ids), w.B)
        say(f"[debug scores] {w.name} step {step}: {H} heads x {w.C} clusters")
        assert np.array_equal(sc.view(np.uint64), osc.view(np.uint64))


def test_eight_query_heads_every_path():
    """G = 8 (the largest query-head group the path supports): build from the
    seed, then selection and attention on the split path, the fused kernel
    and the fused kernel reading the packed copy; the dense comparator too."""
    w = G8
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch.bfloat16, packed=True)
    Kd, Vd = to_dev(K), to_dev(V)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    ref = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, init)
    check_build_exact(w, K, idx, ref)
    for step, B in ((0, w.B), (1, 1), (2, w.L + 9)):
        q = queries(w, base, step, K, w.L, means)
        errs = check_decode_paths(w, idx, K, V, Kd, Vd, q, B, packed_too=(step == 0))
        say(f"  G=8 step {step} B={B}: max abs err {max(errs):.2e}")
    scale = 1.0 / math.sqrt(w.d)
    q = queries(w, base, 0, K, w.L, means)
    out = kvc.dense_decode(to_dev(q), Kd, Vd, w.L, scale)
    torch.cuda.synchronize()
    allsel = np.tile(np.arange(w.L, dtype=np.int32), (H, 1))
    od = oracle.decode(q, w.G, K, V, allsel, np.full(H, w.L, np.int32), scale)
    assert float(np.abs(to_np(out) - od).max()) <= 2e-3


def test_exact_ties_and_an_emptied_cluster():
    """Ties are decided by the lowest id (the reading of the silent tie rule).
    Assignment: two initial positions hold bit-identical keys, so the two
    operand rows are identical and every key ties between them; all go to the
    lower cluster, and after the first iteration the other is empty and keeps
    its centroid (the build continues from that state, bit-exact with the
    oracle). Selection: two clusters given bit-identical centroids score the
    same, and the lower id ranks first on every path."""
    w = TIES
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    init = init.copy()
    # head h: the key at init[h, 3] is copied over the one at init[h, 9]
    for h in range(H):
        K[h, init[h, 9]] = K[h, init[h, 3]]
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch.bfloat16, packed=True)
    Kd, Vd = to_dev(K), to_dev(V)
    Ks = np.ascontiguousarray(K[:, :w.L])
    # after one iteration cluster 9 is empty (every key tied it with cluster 3)
    # and keeps its initial centroid
    kvc.build(idx, Kd, w.L, 1, init_idx=to_dev(init))
    torch.cuda.synchronize()
    check_build_exact(w, K, idx, oracle.build(Ks, w.C, 1, init))
    sizes, c = to_np(idx.sizes), to_np(idx.centroids)
    for h in range(H):
        assert sizes[h, 9] == 0, sizes[h]
        assert np.array_equal(c[h, 9], oracle.to_f64(K[h, init[h, 9]]).astype(np.float32))
    say(f"  after one iteration: cluster 9 sizes {sizes[:, 9].tolist()}, cluster 3 sizes {sizes[:, 3].tolist()}")
    # the whole build, whose later iterations start from the emptied cluster
    kvc.build(idx, Kd, w.L, w.iters, init_idx=to_dev(init))
    torch.cuda.synchronize()
    check_build_exact(w, K, idx, oracle.build(Ks, w.C, w.iters, init))
    sizes = to_np(idx.sizes)
    # selection ties: cluster 5's centroid := cluster 2's (both layouts), so the
    # two score identically; the ids of cluster 5 then come right after 2's
    cen = idx.centroids.clone()
    cen[:, 5] = cen[:, 2]
    idx.centroids.copy_(cen)
    ct = idx.centroids_t.clone()
    ct[:, :, 5, :] = ct[:, :, 2, :]
    idx.centroids_t.copy_(ct)
    torch.cuda.synchronize()
    for step in range(w.steps):
        q = queries(w, base, step, K, w.L, means)
        _, _, osc, order = oracle.select(q, w.G, to_np(idx.centroids), sizes, to_np(idx.offsets),
                                         to_np(idx.token_ids), w.B)
        for h in range(H):
            r2 = int(np.flatnonzero(order[h] == 2)[0])
            assert order[h, r2 + 1] == 5 and osc[h, 2] == osc[h, 5]
        errs = check_decode_paths(w, idx, K, V, Kd, Vd, q, w.L, packed_too=(step == 0))
        say(f"  tie step {step}: max abs err {max(errs):.2e}")


@pytest.mark.parametrize("C", [1, 512])
def test_one_cluster_and_the_largest_count(C):
    """C = 1: the whole context is one cluster, so any budget takes the first
    min(B, N) tokens. C = 512: the largest operand the assignment stages and
    the largest selection."""
    w = synth.Workload(f"c{C}_bf16", 97, heads=2, G=4, L=4096, d=128, dtype=synth.BF16, M=64, sigma=0.3, n_out=4,
                       out_scale=10.0, C=C, iters=4, B=700, steps=2, query="mixture", q_sigma=0.2)
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch.bfloat16, packed=True)
    Kd, Vd = to_dev(K), to_dev(V)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    ref = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, init)
    agree = (to_np(idx.labels)[:, :w.L] == ref["labels"]).mean()
    say(f"[C={C}] label agreement {agree:.6f}")
    assert agree >= 0.999
    if C == 1:
        check_build_exact(w, K, idx, ref)
    for step, B in ((0, w.B), (1, 3)):
        q = queries(w, base, step, K, w.L, means)
        errs = check_decode_paths(w, idx, K, V, Kd, Vd, q, B, packed_too=(step == 0))
        if C == 1:
            sel = to_np(kvc.select(idx, to_dev(q), B)[0])
            assert np.array_equal(sel, np.tile(np.arange(B, dtype=np.int32), (H, 1)))
        say(f"  C={C} step {step} B={B}: max abs err {max(errs):.2e}")


def test_zero_and_nan_key_rows():
    """A zero key scores 0 against every centroid and goes to cluster 0 (the
    reading of the tie rule); a key of NaN scores NaN everywhere and stays in
    cluster 0 under the sequential argmax rule. One assignment step of the
    matrix-core pass with its exact fallback, bit-exact with the oracle, then a
    full build whose labels and index stay in range."""
    w = TIES
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    K = K.copy()
    K[:, 17] = 0                       # zero key rows
    K[1, 40] = 0x7FC0                  # a NaN key row (bf16 quiet NaN)
    opt = oracle.BF16
    c0 = np.stack([oracle.to_f64(K[h, init[h]]).astype(np.float32) for h in range(H)])
    chat = np.stack([oracle.normalize(c0[h], opt) for h in range(H)])
    want = np.stack([oracle.assign(K[h, :w.L], chat[h])[0] for h in range(H)])
    cp = kvc.cpad(w.C)
    op = np.zeros((H, cp, w.d), dtype=np.uint16)
    op[:, :w.C] = chat
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch.bfloat16)
    labels, _, flagged = kvc.debug_assign(idx, to_dev(K), w.L, to_dev(op))
    torch.cuda.synchronize()
    got = to_np(labels)[:, :w.L]
    assert np.array_equal(got, want)
    assert np.all(got[:, 17] == 0) and got[1, 40] == 0
    say(f"  zero and NaN rows: labels {got[:, 17].tolist()} / {got[1, 40]}, queued {to_np(flagged).tolist()}")
    # a full build with those rows: the NaN key makes its cluster's mean NaN;
    # every label and index entry stays in range
    idx2 = kvc.ClusterIndex(H, w.C, w.capacity, torch.bfloat16)
    kvc.build(idx2, to_dev(K), w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    lab = to_np(idx2.labels)[:, :w.L]
    assert lab.min() >= 0 and lab.max() < w.C
    sizes, offsets, ids = to_np(idx2.sizes), to_np(idx2.offsets), to_np(idx2.token_ids)[:, :w.L]
    for h in range(H):
        assert sizes[h].sum() == w.L and offsets[h, -1] == w.L
        assert np.array_equal(np.sort(ids[h]), np.arange(w.L))
        s, o, i = oracle.csr(lab[h], w.C)
        assert np.array_equal(sizes[h], s) and np.array_equal(ids[h], i)


def test_append_non_finite_scores():
    """The append's argmax follows the sequential rule (start from cluster 0,
    move only to a strictly larger score) when scores are not finite: a NaN
    operand row of a later cluster never wins (head 0), a NaN row of cluster 0
    keeps every token there (head 1), an infinite component makes its cluster
    score +-inf or NaN by the key's sign (head 2), and a NaN key goes to
    cluster 0. Labels, sizes and index bit-exact with the oracle."""
    w = APPEND_NF
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    K = K.copy()
    K[2, w.L + 3] = 0x7FC0                  # a NaN key (bf16 quiet NaN)
    idx = kvc.ClusterIndex(H, w.C, w.capacity, torch.bfloat16)
    Kc, Vc = np.zeros_like(K), np.zeros_like(V)
    Kc[:, :w.L], Vc[:, :w.L] = K[:, :w.L], V[:, :w.L]
    Kd, Vd = to_dev(Kc), to_dev(Vc)
    kvc.build(idx, Kd, w.L, w.iters, seed=base)
    torch.cuda.synchronize()
    op = to_np(idx.centroids_op)
    op[0, 5] = 0x7FC0                       # NaN row of a later cluster
    op[1, 0] = 0x7FC0                       # NaN row of cluster 0
    op[2, 3, 7] = 0x7F80                    # +inf in one channel
    idx.centroids_op.copy_(to_dev(op))
    built = dict(labels=to_np(idx.labels)[:, :w.L], sizes=to_np(idx.sizes), offsets=to_np(idx.offsets),
                 token_ids=to_np(idx.token_ids)[:, :w.L], c=to_np(idx.centroids), chat=op[:, :w.C])
    oi = oracle.Index(built, w.capacity)
    labs = []
    for t in range(w.steps):
        n = w.L + t
        kvc.append(idx, Kd, Vd, to_dev(np.ascontiguousarray(K[:, n:n + 1])),
                   to_dev(np.ascontiguousarray(V[:, n:n + 1])))
        labs.append(oi.append(np.ascontiguousarray(K[:, n])))
    torch.cuda.synchronize()
    n = w.L + w.steps
    assert np.array_equal(to_np(idx.labels)[:, :n], oi.labels[:, :n])
    assert np.array_equal(to_np(idx.sizes), oi.sizes)
    off, ids = kvc.export_csr(idx)
    assert np.array_equal(to_np(off), oi.offsets)
    assert np.array_equal(to_np(ids)[:, :n], oi.token_ids[:, :n])
    labs = np.stack(labs, axis=1)
    assert np.all(labs[1] == 0) and np.all(labs[0] != 5) and labs[2, 3] == 0
    say(f"  non-finite append labels: {labs.tolist()}")


@pytest.mark.parametrize("seed", range(6))
def test_fused_decode_random_shapes(seed):
    """The fused selection and attention with the token split, with and
    without selected ids to return (without them, the clusters above the cut
    bin are gathered before the candidates are ranked), from the caches and
    from the packed copy, on seeded random shapes: head counts, query heads
    per KV head, context lengths, cluster counts from 1 to 400, budgets from 1
    token to more than the context, with and without attention sinks.
    Selection bit-exact and attention within 2e-3 of the oracle."""
    rng = np.random.default_rng(4000 + seed)
    H = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4]))
    L = int(rng.integers(300, 3000))
    n_sink = int(rng.choice([0, 5]))
    C = int(min(rng.choice([1, 7, 40, 150, 400]), L - n_sink))
    w = synth.Workload(f"random_{seed}", 200 + seed, heads=H, G=G, L=L, d=128, dtype=synth.BF16, M=16, sigma=0.3,
                       n_out=4, out_scale=10.0, C=C, iters=3, B=1, steps=3, query="noisy_key", q_sigma=0.1)
    base, K, V, init, means = make_inputs(w)
    idx = kvc.ClusterIndex(H, C, L, torch.bfloat16, packed=True, n_sink=n_sink)
    Kd, Vd = to_dev(K), to_dev(V)
    kvc.build(idx, Kd, L, w.iters, seed=base)
    torch.cuda.synchronize()
    c, sizes, offsets, ids = to_np(idx.centroids), to_np(idx.sizes), to_np(idx.offsets), to_np(idx.token_ids)
    scale = 1.0 / math.sqrt(w.d)
    budgets = sorted({1, int(rng.integers(2, 64)), int(rng.integers(64, L)), L + 50})
    errs = []
    for step, B in enumerate(budgets):
        q = queries(w, base, step, K, L, means)
        qd = to_dev(q)
        osel, ocnt, _, _ = oracle.select(q, G, c, sizes, offsets, ids, B, n_sink=n_sink)
        od = oracle.decode(q, G, K, V, osel, ocnt, scale)
        for pk in (0, 1):
            if pk:
                kvc.pack(idx, Kd, Vd)
            idx._s.packed = pk
            ws = split_ws(idx, H * G)
            fsel = torch.full((H, B), -7, dtype=torch.int32, device="cuda")
            fcnt = torch.empty(H, dtype=torch.int32, device="cuda")
            fout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, sel_ids=fsel, sel_count=fcnt, workspace=ws)
            ecnt = torch.empty(H, dtype=torch.int32, device="cuda")
            eout = kvc.select_decode(idx, qd, Kd, Vd, B, scale, sel_count=ecnt, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(fsel), osel) and np.array_equal(to_np(fcnt), ocnt), (B, pk)
            assert np.array_equal(to_np(ecnt), ocnt), (B, pk)
            errs += [float(np.abs(to_np(fout) - od).max()), float(np.abs(to_np(eout) - od).max())]
    say(f"  H={H} G={G} L={L} C={C} sinks={n_sink} budgets={budgets}: max abs err {max(errs):.2e}")
    assert max(errs) <= 2e-3, errs


def test_sparse_decode_clamps_the_count():
    """kv_sparse_decode takes a count above B as B and a negative one as 0,
    and gives entries outside [0, capacity) no weight."""
    w = TIES
    base, K, V, init, means = make_inputs(w)
    H = K.shape[0]
    Kd, Vd = to_dev(K), to_dev(V)
    scale = 1.0 / math.sqrt(w.d)
    B = 96
    rng = np.random.default_rng(3)
    sel = np.stack([rng.permutation(w.L)[:B] for _ in range(H)]).astype(np.int32)
    q = queries(w, base, 0, K, w.L, means)
    cnt = np.array([B + 1000, -5, B], dtype=np.int32)
    bad = sel.copy()
    bad[2, 7] = w.capacity + 50
    bad[2, 8] = -3
    out = kvc.sparse_decode(to_dev(q), Kd, Vd, to_dev(bad), to_dev(cnt), scale)
    torch.cuda.synchronize()
    keep = np.ones((H, B), bool)
    keep[2, 7:9] = False
    o = to_np(out)
    for h, n in ((0, B), (1, 0)):
        od = oracle.decode(q[h * w.G:(h + 1) * w.G], w.G, K[h:h + 1], V[h:h + 1], sel[h:h + 1],
                           np.array([n], np.int32), scale)
        assert np.abs(o[h * w.G:(h + 1) * w.G] - od).max() <= 2e-3
    s2 = sel[2][keep[2]][None]
    od = oracle.decode(q[2 * w.G:3 * w.G], w.G, K[2:3], V[2:3], np.ascontiguousarray(s2),
                       np.array([s2.shape[1]], np.int32), scale)
    assert np.abs(o[2 * w.G:3 * w.G] - od).max() <= 2e-3
