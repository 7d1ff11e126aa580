"""Pins of the CPU oracle against brute force, closed forms, library routines and
invariants. Each test names the rule (ClusterKV summary page section) it pins.
Runs on the CPU only."""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import BF16, F32, F64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


# ----------------------------------------------------------------- rounding

def test_round_bf16_hand_cases(orc):
    """Round-to-nearest-even from fp64, including a case that double rounding
    through fp32 would get wrong."""
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2 ** -8, 0x3F80),                 # exact tie -> even (down)
        (1.0 + 3 * 2 ** -8, 0x3F82),             # exact tie -> even (up)
        (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),      # above the tie; fp32 first would tie
        (-2.0, 0xC000),
        (-0.0, 0x8000),
        (0.0, 0x0000),
        (3.3895313892515355e38, 0x7F7F),         # largest finite bf16
        (3.40282346638528859811704183484516925440e38, 0x7F80),  # rounds up to inf
        (2.0 ** -133, 0x0001),                    # smallest subnormal
        (2.0 ** -134, 0x0000),                    # tie with zero -> even
        (3 * 2.0 ** -134, 0x0002),                # 1.5 ulp tie -> even 2
        (float("inf"), 0x7F80),
        (2.0 ** -126, 0x0080),
    ]
    for x, want in cases:
        got = int(orc.round_bf16(np.array([x]))[0])
        assert got == want, (x, hex(got), hex(want))
    assert (int(orc.round_bf16(np.array([float("nan")]))[0]) & 0x7FC0) == 0x7FC0


def test_round_bf16_matches_torch_and_synth(orc, syn):
    """On fp32-representable values (no double-rounding question) the oracle,
    torch's float32->bfloat16 conversion and the input generator agree."""
    rng = np.random.default_rng(5)
    x32 = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 3000),
                          np.array([1.00390625, 1.01171875, -1.00390625], np.float32)])
    x = x32.astype(np.float64)
    t = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    o = orc.round_bf16(x)
    s = syn.round_bf16(x)
    assert np.array_equal(o, t)
    assert np.array_equal(s, t)


# --------------------------------------------------------------- normalise

def test_normalize_unit_direction(orc):
    """III.B: only a centroid's direction matters to cosine assignment."""
    rng = np.random.default_rng(1)
    c = rng.standard_normal((7, 16)).astype(np.float32)
    c[3] = 0.0
    e = orc.normalize(c, F64)
    nrm = np.linalg.norm(c.astype(np.float64), axis=1)
    for k in range(7):
        if k == 3:
            assert np.all(e[k] == 0.0)
            continue
        assert abs(np.linalg.norm(e[k]) - 1.0) < 1e-14
        np.testing.assert_allclose(e[k], c[k] / nrm[k], rtol=1e-15, atol=0)
    b = orc.to_f64(orc.normalize(c, BF16))
    ref = c.astype(np.float64) / np.where(nrm > 0, nrm, 1.0)[:, None]
    # each bf16 component is within half an ulp (2^-9 relative) of the direction
    assert np.all(np.abs(b - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-300)
    f = orc.normalize(c, F32)
    assert f.dtype == np.float32
    assert np.all(np.abs(f.astype(np.float64) - ref) <= np.abs(ref) * 2.0 ** -24 + 1e-300)


# ------------------------------------------------------------------ assign

def test_assign_brute_force_cosine(orc):
    """III.B: nearest centroid by cosine similarity (brute force in numpy on
    normalised keys and centroids)."""
    rng = np.random.default_rng(2)
    K = (rng.standard_normal((300, 12)) * rng.uniform(0.1, 50, (300, 1))).astype(np.float32)
    c = rng.standard_normal((9, 12))
    chat = orc.normalize(c, F64)
    labels, best = orc.assign(K, chat)
    Kn = K.astype(np.float64) / np.linalg.norm(K.astype(np.float64), axis=1, keepdims=True)
    cn = c / np.linalg.norm(c, axis=1, keepdims=True)
    cos = Kn @ cn.T
    assert np.array_equal(labels, np.argmax(cos, axis=1))
    # the winning score is K . chat (the cosine times ||K||)
    np.testing.assert_allclose(best, np.max(K.astype(np.float64) @ chat.T, axis=1), rtol=1e-13)


def test_assign_ties_and_scale_invariance(orc):
    """Exact ties go to the lowest cluster id; scaling a key does not move it
    (a smaller cosine distance wins, III.B)."""
    chat = np.array([[0.0, 1.0], [1.0, 0.0], [1.0, 0.0], [0.6, 0.8]], dtype=np.float64)
    K = np.array([[1.0, 0.0], [3.0, 4.0], [300.0, 400.0], [0.0, 0.0], [-1.0, 0.0]], dtype=np.float32)
    labels, _ = orc.assign(K, chat)
    # (1,0): tie between clusters 1 and 2 -> 1. (3,4) and its multiple -> 3.
    # zero key scores 0 everywhere -> 0. (-1,0): scores 0,-1,-1,-0.6 -> 0.
    assert labels.tolist() == [1, 3, 3, 0, 0]


# ------------------------------------------------------------------ update

def test_update_closed_form_means(orc):
    """III.B / Sys-B: a centroid is the mean of its keys; C = 1 gives the global
    mean; an empty cluster keeps its centroid."""
    rng = np.random.default_rng(3)
    K = rng.standard_normal((500, 8)).astype(np.float32)
    labels = rng.integers(0, 6, 500).astype(np.int32)
    labels[labels == 4] = 5  # cluster 4 empty
    c0 = rng.standard_normal((6, 8)).astype(np.float32)
    c, counts = orc.update(K, labels, c0)
    assert counts.tolist() == np.bincount(labels, minlength=6).tolist()
    for k in range(6):
        if counts[k] == 0:
            assert np.array_equal(c[k], c0[k])
        else:
            want = K[labels == k].astype(np.float64).mean(axis=0).astype(np.float32)
            assert np.max(np.abs(c[k].view(np.int32) - want.view(np.int32))) <= 1
    g, _ = orc.update(K, np.zeros(500, np.int32), c0[:1])
    np.testing.assert_allclose(g[0], K.astype(np.float64).mean(axis=0), rtol=1e-6, atol=1e-7)


# --------------------------------------------------------------------- csr

def test_csr_matches_stable_argsort(orc):
    """Sys-C: sizes, prefix sums and cluster-sorted token ids (a stable counting
    sort is numpy's stable argsort by label)."""
    rng = np.random.default_rng(4)
    for C in (1, 3, 17, 400):
        labels = rng.integers(0, C, 2000).astype(np.int32)
        sizes, offsets, ids = orc.csr(labels, C)
        assert np.array_equal(sizes, np.bincount(labels, minlength=C))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(labels, minlength=C))]))
        assert np.array_equal(ids, np.argsort(labels, kind="stable"))


# ------------------------------------------------------------------- build

def _check_index(orc, K, r, C):
    H, L = r["labels"].shape
    for h in range(H):
        lab, sz, off, ids = r["labels"][h], r["sizes"][h], r["offsets"][h], r["token_ids"][h]
        assert sz.sum() == L and off[0] == 0 and off[-1] == L
        assert np.array_equal(np.diff(off), sz)
        assert np.array_equal(np.sort(ids), np.arange(L))
        for k in range(C):
            seg = ids[off[k]:off[k + 1]]
            assert np.all(np.diff(seg) > 0)
            assert np.all(lab[seg] == k)
        # centroids are exactly the means of the final labels (recomputed)
        c2, _ = orc.update(K[h, :L], lab, r["c"][h])
        assert np.array_equal(c2, r["c"][h])
        # chat is the normalised final centroid
        assert np.array_equal(orc.normalize(r["c"][h], F64 if r["c"].dtype == np.float64 else
                                            (BF16 if K.dtype == np.uint16 else F32)), r["chat"][h])


@pytest.mark.parametrize("cfgdtype", ["f32", "bf16"])
def test_build_invariants(orc, syn, cfgdtype):
    dt = syn.F32 if cfgdtype == "f32" else syn.BF16
    base = syn.config_seed(90)
    H, L, d, C = 3, 700, 32, 12
    K, _, _ = syn.mixture_keys(base, H, L, d, 10, 0.3, 2, 10.0, dt)
    init = syn.init_idx(base, H, L, C)
    r = orc.build(K, C, 10, init, early_exit=False)
    _check_index(orc, K, r, C)
    # without early exit every iteration runs; with it the result is identical
    r2 = orc.build(K, C, 10, init, early_exit=True)
    for key in ("c", "chat", "labels", "sizes", "offsets", "token_ids"):
        assert np.array_equal(r[key], r2[key]), key


def test_inertia_non_increasing_exact_mode(orc, syn):
    """Norm-weighted cosine distance sum_i ||K_i||(1 - cos) never increases: the
    assignment step minimises each term and the raw-mean direction maximises
    sum_i K_i . chat over unit chat."""
    base = syn.config_seed(91)
    H, L, d, C = 4, 1500, 24, 20
    K, _, _ = syn.mixture_keys(base, H, L, d, 30, 0.6, 3, 10.0, syn.BF16)
    init = syn.init_idx(base, H, L, C)
    r = orc.build(K, C, 25, init, mode=1, early_exit=False)
    for h in range(H):
        I = r["inertia"][h]
        assert np.all(np.diff(I) <= 1e-12 * I[0]), I
    rb = orc.build(K, C, 25, init, mode=0, early_exit=False)
    tot = sum(np.linalg.norm(orc.to_f64(K[h]), axis=1).sum() for h in range(H)) / H
    for h in range(H):
        assert np.all(np.diff(rb["inertia"][h]) <= 2.0 ** -8 * tot)


def test_converged_fixed_point(orc, syn):
    """III.B: iterate until assignments stop changing; once they repeat, one
    more iteration changes nothing."""
    base = syn.config_seed(92)
    K, _, _ = syn.mixture_keys(base, 2, 600, 16, 6, 0.3, 0, 1.0, syn.F32)
    init = syn.init_idx(base, 2, 600, 6)
    r = orc.build(K, 6, 50, init, early_exit=True)
    assert np.all(r["iters_run"] < 50)
    for h in range(2):
        lab, _ = orc.assign(K[h], r["chat"][h])
        assert np.array_equal(lab, r["labels"][h])


def test_well_separated_mixture_recovered(orc, syn):
    """With one initial key per component of a well separated mixture, the
    clusters are exactly the generator's components."""
    base = syn.config_seed(93)
    H, L, d, M = 2, 800, 32, 8
    K, comp, _ = syn.mixture_keys(base, H, L, d, M, 0.05, 0, 1.0, syn.F32, want_comp=True)
    init = np.stack([[int(np.flatnonzero(comp[h] == m)[0]) for m in range(M)] for h in range(H)]).astype(np.int32)
    r = orc.build(K, M, 10, init)
    for h in range(H):
        assert np.array_equal(r["labels"][h], comp[h])


def test_every_key_its_own_cluster_and_exact_top_b(orc):
    """C = N with the keys as initial centroids: each key forms its own cluster,
    and cluster selection reduces to exact top-B by q . k (III.A's formulation,
    here the textbook top-k with ties to the lower index)."""
    rng = np.random.default_rng(7)
    N, d = 96, 16
    K = rng.integers(-8, 9, (1, N, d)).astype(np.float32)
    Kn = K[0] / np.linalg.norm(K[0], axis=1, keepdims=True)
    cosm = Kn @ Kn.T - np.eye(N) * 10
    assert cosm.max() < 1 - 1e-9  # no two keys share a direction
    r = orc.build(K, N, 3, np.arange(N, dtype=np.int32)[None])
    assert np.array_equal(r["labels"][0], np.arange(N))
    assert np.array_equal(r["c"][0], K[0])
    q = rng.integers(-4, 5, (1, d)).astype(np.float32)
    s = (K[0].astype(np.float64) @ q[0].astype(np.float64))
    for B in (1, 7, 40, N, N + 5):
        sel, cnt, _, _ = orc.select(q, 1, r["c"], r["sizes"], r["offsets"], r["token_ids"], B)
        want = np.lexsort((np.arange(N), -s))[:min(B, N)]
        assert cnt[0] == min(B, N)
        assert np.array_equal(sel[0, :cnt[0]], want)


# ------------------------------------------------------------------ select

def _brute_select(q, G, c, sizes, offsets, ids, B):
    """Independent brute force: exact scores with Python integers (inputs are
    integer-valued), full sort, walk."""
    H, C, d = c.shape
    out, cnts = [], []
    for h in range(H):
        qbar = [sum(int(q[h * G + g, j]) for g in range(G)) for j in range(d)]
        sc = [sum(qbar[j] * int(c[h, k, j]) for j in range(d)) for k in range(C)]
        order = sorted(range(C), key=lambda k: (-sc[k], k))
        sel = []
        for k in order:
            members = list(ids[h, offsets[h, k]:offsets[h, k + 1]])
            sel.extend(members[:max(0, B - len(sel))])
            if len(sel) >= B:
                break
        cnts.append(len(sel))
        out.append(sel + [-1] * (B - len(sel)))
    return np.array(out, np.int32), np.array(cnts, np.int32)


@pytest.mark.parametrize("G", [1, 4])
def test_select_brute_force(orc, G):
    """III.C / Sys-C: clusters ranked by attention to q (summed over the query
    heads sharing the KV head), taken until the budget, the last trimmed."""
    rng = np.random.default_rng(8 + G)
    H, C, d, N = 3, 23, 8, 200
    c = rng.integers(-3, 4, (H, C, d)).astype(np.float32)
    q = rng.integers(-3, 4, (H * G, d)).astype(np.float32)
    labels = rng.integers(0, C, (H, N)).astype(np.int32)
    S, O, I = zip(*[orc.csr(labels[h], C) for h in range(H)])
    S, O, I = np.stack(S), np.stack(O), np.stack(I)
    for B in (1, 5, 17, 64, 150, 200, 250):
        sel, cnt, scores, order = orc.select(q, G, c, S, O, I, B)
        bs, bc = _brute_select(q, G, c, S, O, I, B)
        assert np.array_equal(cnt, bc) and np.array_equal(sel, bs), B
        assert np.all(cnt == min(B, N))
        for h in range(H):
            got = sel[h, :cnt[h]]
            assert len(set(got.tolist())) == cnt[h]
            # clusters appear as a prefix of the ranking, only the last partial
            ranks = [int(np.flatnonzero(order[h] == labels[h, t])[0]) for t in got]
            assert ranks == sorted(ranks)
            used = sorted(set(ranks))
            assert used == list(range(len(used)))
            for r in used[:-1]:
                k = order[h, r]
                assert sum(1 for t in got if labels[h, t] == k) == S[h, k]


def test_select_single_cluster(orc):
    """C = 1: the selection is the first min(B, N) tokens in position order."""
    rng = np.random.default_rng(9)
    N = 50
    c = rng.standard_normal((1, 1, 8)).astype(np.float32)
    q = rng.standard_normal((1, 8)).astype(np.float32)
    s, o, i = orc.csr(np.zeros(N, np.int32), 1)
    for B in (1, 10, 50, 80):
        sel, cnt, _, _ = orc.select(q, 1, c, s[None], o[None], i[None], B)
        assert cnt[0] == min(B, N) and np.array_equal(sel[0, :cnt[0]], np.arange(min(B, N)))


# ------------------------------------------------------------------ decode

def _sdpa(q, K, V, scale, mask=None):
    """torch's scaled dot-product attention in float64 on the CPU."""
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1)
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)[0, :, 0, :].numpy()


def test_decode_dense_when_budget_covers_all(orc, syn):
    """II.A: with B >= N the sparse decode is textbook softmax attention over
    all tokens (torch SDPA in float64)."""
    base = syn.config_seed(94)
    H, G, N, d = 2, 4, 300, 32
    K = syn.normal_array(syn.stream_seed(base, 0, 0), (H, N, d), 1.0, syn.BF16)
    V = syn.normal_array(syn.stream_seed(base, 0, 1), (H, N, d), 1.0, syn.BF16)
    q = syn.normal_array(syn.stream_seed(base, 0, 2), (H * G, d), 1.0, syn.BF16)
    B = 512
    sel = np.full((H, B), -1, np.int32)
    rng = np.random.default_rng(0)
    for h in range(H):
        sel[h, :N] = rng.permutation(N)
    cnt = np.full(H, N, np.int32)
    scale = 1.0 / math.sqrt(d)
    out = orc.decode(q, G, K, V, sel, cnt, scale)
    Kf, Vf, qf = orc.to_f64(K), orc.to_f64(V), orc.to_f64(q)
    for g in range(H * G):
        h = g // G
        ref = _sdpa(qf[g:g + 1], Kf[h], Vf[h], scale)[0]
        np.testing.assert_allclose(out[g], ref, rtol=0, atol=2e-7)


def test_decode_masked_attention(orc, syn):
    """III.A: attention restricted to the selected tokens equals dense attention
    with every other token masked out."""
    base = syn.config_seed(95)
    H, G, N, d, B = 2, 2, 400, 16, 57
    K = syn.normal_array(syn.stream_seed(base, 1, 0), (H, N, d), 1.0, syn.F32)
    V = syn.normal_array(syn.stream_seed(base, 1, 1), (H, N, d), 1.0, syn.F32)
    q = syn.normal_array(syn.stream_seed(base, 1, 2), (H * G, d), 1.0, syn.F32)
    rng = np.random.default_rng(1)
    sel = np.stack([rng.choice(N, B, replace=False) for _ in range(H)]).astype(np.int32)
    cnt = np.array([B, 20], np.int32)
    scale = 0.3
    out = orc.decode(q, G, K, V, sel, cnt, scale)
    for g in range(H * G):
        h = g // G
        mask = np.zeros(N, bool)
        mask[sel[h, :cnt[h]]] = True
        ref = _sdpa(q[g:g + 1].astype(np.float64), K[h].astype(np.float64), V[h].astype(np.float64), scale, mask)[0]
        np.testing.assert_allclose(out[g], ref, rtol=0, atol=2e-7)
    # no selected token: zero output
    z = orc.decode(q, G, K, V, sel, np.zeros(H, np.int32), scale)
    assert np.all(z == 0)


# ------------------------------------------------------------------ append

def test_append_nearest_centroid_and_index(orc, syn):
    """A decode-time token joins its nearest existing centroid (cosine); the
    canonical index equals the one rebuilt from all labels."""
    base = syn.config_seed(96)
    H, L, d, C, A = 2, 500, 16, 9, 40
    K, _, _ = syn.mixture_keys(base, H, L + A, d, 12, 0.3, 2, 10.0, syn.BF16)
    init = syn.init_idx(base, H, L, C)
    r = orc.build(np.ascontiguousarray(K[:, :L]), C, 10, init)
    idx = orc.Index(r, L + A)
    for t in range(A):
        labs = idx.append(K[:, L + t])
        for h in range(H):
            kf = orc.to_f64(K[h, L + t])
            ch = orc.to_f64(r["chat"][h])
            assert labs[h] == int(np.argmax(ch @ kf))
    for h in range(H):
        s, o, i = orc.csr(idx.labels[h, :L + A], C)
        assert np.array_equal(s, idx.sizes[h]) and np.array_equal(o, idx.offsets[h])
        assert np.array_equal(i, idx.token_ids[h, :L + A])


# ------------------------------------------------------------------ golden

def test_worked_example(orc):
    with open(os.path.join(GOLDEN, "worked_example_d2.json")) as f:
        g = json.load(f)
    e = g["expect"]
    K = np.array(g["keys"], np.float32)[None]
    V = np.array(g["values"], np.float32)[None]
    r = orc.build(K, g["C"], g["iters"], np.array(g["init_idx"], np.int32)[None])
    assert r["labels"][0].tolist() == e["labels"]
    assert r["c"][0].astype(np.float64).tolist() == e["centroids"]
    assert r["sizes"][0].tolist() == e["sizes"]
    assert r["offsets"][0].tolist() == e["offsets"]
    assert r["token_ids"][0].tolist() == e["token_ids"]
    q = np.array([e["query"]], np.float32)
    sel, cnt, scores, _ = orc.select(q, 1, r["c"], r["sizes"], r["offsets"], r["token_ids"], e["B"])
    assert scores[0].tolist() == e["scores"]
    assert sel[0].tolist() == e["sel_ids"] and int(cnt[0]) == e["sel_count"]
    out = orc.decode(q, 1, K, V, sel, cnt, e["scale"])
    np.testing.assert_allclose(out[0], e["out"], rtol=0, atol=e["out_atol"])
    assert f32(e["scale"]) == e["scale"]


# ------------------------------------------------------------------ recall

def test_recall_hand_case(orc):
    """III.A: the reference set is the B tokens of largest attention weight.
    Logits 3, 2, 1, 0 -> the top 2 are tokens 0 and 1."""
    K = np.array([[[3, 0], [2, 0], [1, 0], [0, 0]]], np.float32)
    q = np.array([[1, 0]], np.float32)
    for sel, want in (([0, 3], 0.5), ([1, 0], 1.0), ([2, 3], 0.0)):
        r = orc.recall(q, 1, K, 4, np.array([sel], np.int32), np.array([2], np.int32))
        assert r.tolist() == [want], sel
    # a budget covering every token recalls everything
    r = orc.recall(q, 1, K, 4, np.array([[3, 2, 1, 0, -1]], np.int32), np.array([4], np.int32))
    assert r.tolist() == [1.0]


def test_recall_one_key_per_cluster_is_exact(orc):
    """With C = N (every key its own cluster, centroid = the key) the cluster
    selection is the exact top-B by q . k (III.A), ties included, so its recall
    is 1 for every budget."""
    rng = np.random.default_rng(21)
    H, N, d = 2, 60, 8
    K = rng.integers(-3, 4, (H, N, d)).astype(np.float32)
    q = rng.integers(-3, 4, (H, d)).astype(np.float32)
    S, O, I = zip(*[orc.csr(np.arange(N, dtype=np.int32), N) for _ in range(H)])
    S, O, I = np.stack(S), np.stack(O), np.stack(I)
    for B in (1, 5, 17, 60, 80):
        sel, cnt, _, _ = orc.select(q, 1, K, S, O, I, B)
        assert np.all(orc.recall(q, 1, K, N, sel, cnt) == 1.0), B


def test_recall_brute_force(orc):
    """Against an independent count: exact logits from Python integers on
    integer-valued inputs, ranking by (logit desc, position asc)."""
    rng = np.random.default_rng(22)
    H, G, N, d, B = 2, 2, 40, 6, 9
    K = rng.integers(-4, 5, (H, N, d)).astype(np.float32)
    q = rng.integers(-4, 5, (H * G, d)).astype(np.float32)
    sel = np.stack([rng.permutation(N)[:B] for _ in range(H)]).astype(np.int32)
    cnt = np.array([B, B - 2], np.int32)
    r = orc.recall(q, G, K, N, sel, cnt)
    for g in range(H * G):
        h = g // G
        z = [sum(int(q[g, j]) * int(K[h, t, j]) for j in range(d)) for t in range(N)]
        top = set(sorted(range(N), key=lambda t: (-z[t], t))[:B])
        want = len(top & set(sel[h, :cnt[h]].tolist())) / B
        assert r[g] == want, g


# ------------------------------------------------------------------- sinks

def test_sinks_stay_out_of_clusters_and_are_always_selected(orc, syn):
    """III.B: the first tokens are kept as attention sinks and only the rest
    are clustered. Building with n_sink equals building the remaining rows
    alone (ids shifted by n_sink); the selection always starts with the sinks,
    which count toward B, and the clusters fill the rest."""
    n_sink, C, L, B = 16, 9, 300, 64
    base = syn.config_seed(95)
    K, _, _ = syn.mixture_keys(base, 2, L, 8, 6, 0.3, 0, 1.0, syn.F32)
    init = syn.init_idx(base, 2, L - n_sink, C) + n_sink
    r = orc.build(K, C, 5, init, n_sink=n_sink)
    alone = orc.build(np.ascontiguousarray(K[:, n_sink:]), C, 5, init - n_sink)
    assert np.all(r["labels"][:, :n_sink] == -1)
    assert np.array_equal(r["labels"][:, n_sink:], alone["labels"])
    assert np.array_equal(r["token_ids"], alone["token_ids"] + n_sink)
    assert np.array_equal(r["c"], alone["c"]) and r["sizes"].sum(axis=1).tolist() == [L - n_sink] * 2
    q = syn.normal_array(syn.stream_seed(base, 0, 9), 2 * 8, 1.0, syn.F32).reshape(2, 8)
    sel, cnt, _, _ = orc.select(q, 1, r["c"], r["sizes"], r["offsets"], r["token_ids"], B, n_sink=n_sink)
    rest, rcnt, _, _ = orc.select(q, 1, r["c"], r["sizes"], r["offsets"], r["token_ids"], B - n_sink)
    assert cnt.tolist() == [B, B]
    assert np.all(sel[:, :n_sink] == np.arange(n_sink))
    assert np.array_equal(sel[:, n_sink:], rest)
    # a budget within the sinks recalls sinks only
    sel, cnt, _, _ = orc.select(q, 1, r["c"], r["sizes"], r["offsets"], r["token_ids"], 5, n_sink=n_sink)
    assert cnt.tolist() == [5, 5] and np.all(sel == np.arange(5))


# ------------------------------------------------- generated-token clustering

def _canonical(labels: np.ndarray, C: int):
    """Stable sort of the clustered tokens (label >= 0) by label, with numpy."""
    ids = np.flatnonzero(labels >= 0)
    order = np.argsort(labels[ids], kind="stable")
    sizes = np.bincount(labels[ids], minlength=C)
    return sizes, np.concatenate([[0], np.cumsum(sizes)]), ids[order].astype(np.int32)


def test_window_clustering_extends_the_index(orc, syn):
    """III.B: tokens generated during decoding are clustered on their own, into
    a few new centroids, and until then stay uncompressed in a window that is
    always recalled. The existing clusters do not change; the new clusters are
    the prefill k-means of the window's keys alone, with the next ids; their
    centroids are the exact means of their members; the canonical index equals
    the stable sort of all labels; sinks and window come first in a selection,
    as many as the budget allows."""
    n_sink, C, L, d, m, nc, B = 4, 9, 300, 16, 40, 4, 64
    H = 2
    base = syn.config_seed(97)
    K, _, _ = syn.mixture_keys(base, H, L + 2 * m + 3, d, 6, 0.3, 0, 1.0, syn.BF16)
    init = syn.init_idx(base, H, L - n_sink, C) + n_sink
    r = orc.build(np.ascontiguousarray(K[:, :L]), C, 5, init, n_sink=n_sink)
    idx = orc.Index(r, K.shape[1])
    idx.add_window(m)
    assert np.all(idx.labels[:, L:L + m] == -1) and idx.window_start == L and idx.n == L + m
    q = syn.normal_array(syn.stream_seed(base, 0, 9), H * d, 1.0, syn.BF16).reshape(H, d)
    # selection with an open window: sinks, then the window, then the clusters
    sel, cnt, _, _ = orc.select(q, 1, idx.c, idx.sizes, idx.offsets, idx.token_ids, B, n_sink=n_sink,
                                window=(L, L + m))
    rest, rcnt, _, _ = orc.select(q, 1, idx.c, idx.sizes, idx.offsets, idx.token_ids, B - n_sink - m)
    assert cnt.tolist() == [B, B]
    assert np.all(sel[:, :n_sink] == np.arange(n_sink)) and np.all(sel[:, n_sink:n_sink + m] == np.arange(L, L + m))
    assert np.array_equal(sel[:, n_sink + m:], rest)
    small, scnt, _, _ = orc.select(q, 1, idx.c, idx.sizes, idx.offsets, idx.token_ids, 10, n_sink=n_sink,
                                   window=(L, L + m))
    assert scnt.tolist() == [10, 10] and np.all(small == np.concatenate([np.arange(n_sink), np.arange(L, L + 6)]))
    # cluster the window
    before = dict(c=idx.c.copy(), sizes=idx.sizes.copy(), offsets=idx.offsets.copy(), ids=idx.token_ids.copy())
    init_w = syn.init_idx(syn.config_seed(98), H, m, nc) + L
    rw = idx.cluster_window(K, nc, 6, init_w)
    assert idx.C == C + nc and idx.window_start == L + m
    assert np.array_equal(idx.c[:, :C], before["c"]) and np.array_equal(idx.sizes[:, :C], before["sizes"])
    assert np.array_equal(idx.offsets[:, :C + 1], before["offsets"])
    nbuilt = L - n_sink
    assert np.array_equal(idx.token_ids[:, :nbuilt], before["ids"][:, :nbuilt])
    alone = orc.build(np.ascontiguousarray(K[:, L:L + m]), nc, 6, init_w - L)
    assert np.array_equal(rw["labels"], alone["labels"]) and np.array_equal(rw["c"], alone["c"])
    # the window's keys alone decide: other keys changed, same clustering
    K2 = K.copy()
    K2[:, :L] = K[:, ::-1][:, :L]
    idx2 = orc.Index(r, K.shape[1])
    idx2.add_window(m)
    assert np.array_equal(idx2.cluster_window(K2, nc, 6, init_w)["labels"], rw["labels"])
    kf = orc.to_f64(K)
    for h in range(H):
        lab = idx.labels[h, :L + m]
        assert np.all(lab[:n_sink] == -1) and np.all((lab[L:] >= C) & (lab[L:] < C + nc))
        s, o, i = _canonical(lab, C + nc)
        assert np.array_equal(s, idx.sizes[h]) and np.array_equal(o, idx.offsets[h])
        assert np.array_equal(i, idx.token_ids[h, :L + m - n_sink])
        for k in range(C, C + nc):
            mem = np.flatnonzero(lab == k)
            if mem.size:  # exact mean of bf16 values, rounded once to fp32
                want = np.array([math.fsum(kf[h, mem, j]) for j in range(d)]) / mem.size
                assert np.array_equal(idx.c[h, k], want.astype(np.float32)), (h, k)
    # an empty window recalls nothing extra; a nearest-centroid append may pick a new cluster
    sel2, cnt2, _, _ = orc.select(q, 1, idx.c, idx.sizes, idx.offsets, idx.token_ids, B, n_sink=n_sink,
                                  window=(L + m, L + m))
    sel3, cnt3, _, _ = orc.select(q, 1, idx.c, idx.sizes, idx.offsets, idx.token_ids, B, n_sink=n_sink)
    assert np.array_equal(sel2, sel3) and np.array_equal(cnt2, cnt3)
    labs = idx.append(K[:, L + m])
    for h in range(H):
        assert labs[h] == int(np.argmax(orc.to_f64(idx.chat[h]) @ kf[h, L + m]))


def test_window_clustering_two_groups_closed_form(orc):
    """A window of two tight, orthogonal groups clustered into two centroids,
    one started in each group: each group becomes a cluster and each centroid is
    its group's mean (hand-computable values)."""
    d, H = 4, 1
    pre = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [-1, 1, -1, 1], [1, 1, -1, -1]], np.float32)
    win = np.array([[2, 0, 0, 0], [0, 0, 3, 0], [4, 0.5, 0, 0], [0, 0, 5, 0.5], [3, -0.5, 0, 0], [0, 0.25, 2, 0]],
                   np.float32)
    K = np.concatenate([pre, win])[None]
    r = orc.build(np.ascontiguousarray(K[:, :4]), 2, 3, np.array([[0, 1]], np.int32))
    idx = orc.Index(r, 10)
    idx.add_window(6)
    idx.cluster_window(K, 2, 4, np.array([[4, 5]], np.int32))
    assert idx.labels[0, 4:10].tolist() == [2, 3, 2, 3, 2, 3]
    assert np.array_equal(idx.c[0, 2], np.array([3, 0, 0, 0], np.float32))
    assert np.array_equal(idx.c[0, 3], np.array([0, 0.25 / 3, 10 / 3, 0.5 / 3], np.float32))
    assert idx.sizes[0].tolist()[2:] == [3, 3] and idx.offsets[0].tolist()[2:] == [4, 7, 10]
    assert idx.token_ids[0, 4:10].tolist() == [4, 6, 8, 5, 7, 9]


# ------------------------------------------------------------ distance variants

def test_distance_variants_hand_cases(orc):
    """III.B prefers the cosine to L2 and inner-product distance. Two small
    cases worked by hand, where the three distances disagree:
    (a) keys [1,0], [10,0], [0,1], [0,10], centroids started at the first two:
        L2 keeps [10,0] alone, since the three others are closer to [1/3, 11/3],
        while cosine and inner product split by direction;
    (b) key [1, 0.5] against centroids [1,0] and [0,5]: cosine and L2 pick the
        first, the inner product the longer second."""
    K = np.array([[[1, 0], [10, 0], [0, 1], [0, 10]]], np.float32)
    init = np.array([[0, 1]], np.int32)
    got = {m: orc.build(K, 2, 6, init, metric=m)["labels"][0].tolist() for m in (orc.COSINE, orc.L2, orc.IP)}
    assert got[orc.L2] == [0, 1, 0, 0]
    assert got[orc.COSINE] == [1, 1, 0, 0] and got[orc.IP] == [1, 1, 0, 0]
    r = orc.build(K, 2, 6, init, metric=orc.L2)
    assert np.array_equal(r["c"][0], np.array([[1 / 3, 11 / 3], [10, 0]], np.float32))
    assert np.array_equal(r["chat"][0], r["c"][0])  # L2 operand: the centroid itself (fp32 keys)
    c = np.array([[1, 0], [0, 5]], np.float32)
    k = np.array([[1, 0.5]], np.float32)
    assert orc.assign(k, orc.operand(c, orc.F32, orc.COSINE), orc.COSINE)[0].tolist() == [0]
    assert orc.assign(k, orc.operand(c, orc.F32, orc.L2), orc.L2)[0].tolist() == [0]
    assert orc.assign(k, orc.operand(c, orc.F32, orc.IP), orc.IP)[0].tolist() == [1]
    # the L2 score is K.c - ||c||^2 / 2: 1 - 0.5 and 2.5 - 12.5
    assert orc.assign(k, c, orc.L2)[1].tolist() == [0.5]


def test_distance_variants_brute_force(orc):
    """L2: argmin of the squared distance; inner product: argmax of the dot
    product; lowest index on ties. Small integer data keep every fp64 sum exact,
    so numpy's brute force decides the same way."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        d, C, L = int(rng.integers(1, 9)), int(rng.integers(1, 12)), 60
        K = rng.integers(-4, 5, (L, d)).astype(np.float32)
        c = rng.integers(-4, 5, (C, d)).astype(np.float32)
        lab, best = orc.assign(K, c, orc.L2)
        dist = ((K[:, None, :].astype(np.float64) - c[None].astype(np.float64)) ** 2).sum(-1)
        assert np.array_equal(lab, np.argmin(dist, axis=1)), trial
        kn = (K.astype(np.float64) ** 2).sum(1)
        assert np.allclose(best, (kn - dist.min(1)) / 2, rtol=0, atol=0), trial  # K.c - |c|^2/2 = (|K|^2 - dist)/2
        lab, best = orc.assign(K, c, orc.IP)
        dots = K.astype(np.float64) @ c.T.astype(np.float64)
        assert np.array_equal(lab, np.argmax(dots, axis=1)) and np.array_equal(best, dots.max(1)), trial
    # the operand of L2 and inner product is the centroid rounded once (bf16 here), no normalisation
    cf = rng.standard_normal((9, 16)).astype(np.float32)
    want = torch.from_numpy(cf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for m in (orc.L2, orc.IP):
        assert np.array_equal(orc.operand(cf, orc.BF16, m), want)
    assert np.array_equal(orc.operand(cf, orc.BF16, orc.COSINE), orc.normalize(cf, orc.BF16))


def test_l2_kmeans_objective_non_increasing_exact_mode(orc, syn):
    """Lloyd's k-means under L2: assigning to the nearest centroid and moving
    each centroid to its members' mean never raise sum ||K_i - c_label||^2
    (exact mode: fp64 centroids and operand)."""
    base = syn.config_seed(99)
    K, _, _ = syn.mixture_keys(base, 2, 700, 16, 10, 0.3, 2, 10.0, syn.F32)
    init = syn.init_idx(base, 2, 700, 12)
    r = orc.build(K, 12, 15, init, mode=1, early_exit=False, metric=orc.L2)
    for h in range(2):
        I = r["inertia"][h]
        assert np.all(np.diff(I) <= 1e-12 * I[:-1]), I
        # the recorded objective is the plain sum of squared distances
        lab = orc.assign(K[h], r["chat"][h], orc.L2)[0]
        direct = sum(float(((orc.to_f64(K[h, i]) - r["c"][h, lab[i]]) ** 2).sum()) for i in range(700))
        assert math.isclose(orc.inertia(K[h], r["chat"][h], lab, orc.L2), direct, rel_tol=1e-12)


# ------------------------------------------------------------- cluster cache

def test_cluster_cache_counts_hand_case(orc):
    """Sys-D: a cluster selected within the last R steps is not loaded again;
    a hand-worked sequence of selections (clusters a, b, c = labels 0, 1, 2;
    label -1 is a sink) and its hits for R = 1 and R = 2."""
    labels = np.array([[0, 0, 0, 0, 0, 1, 1, 2, -1]])
    steps = [[8, 0, 1, 2, 5, 6],   # a:3 b:2  (the sink 8 is not counted); nothing cached yet
             [0, 1, 2, 7],         # a:3 c:1  a was taken at step 0: a hit, 3 tokens
             [5, 6, 0],            # b:2 a:1  R=1: a (1 token); R=2: also b, taken at step 0 (2 tokens)
             [0, 1, 2, 3, 4]]      # a:5      a was taken at step 2 with 1 member: 1 token
    # clusters selected, cluster hits, cluster tokens selected, token hits
    want = {1: [2 + 2 + 2 + 1, 1 + 1 + 1, 5 + 4 + 3 + 5, 3 + 1 + 1],
            2: [2 + 2 + 2 + 1, 1 + 2 + 1, 5 + 4 + 3 + 5, 3 + 3 + 1]}
    for R in (1, 2):
        sim = orc.ClusterCache(1, R)
        for s in steps:
            sel = np.full((1, 8), -1, np.int32)
            sel[0, :len(s)] = s
            sim.step(sel, np.array([len(s)]), labels)
        st = sim.stats[0]
        assert st.tolist() == want[R], (R, st)


# -------------------------------------------------------- initialisation

def _golden_init():
    with open(os.path.join(GOLDEN, "init_shuffle_L10.json")) as f:
        return json.load(f)


def test_init_shuffle_hand_worked(orc):
    """The seeded partial Fisher-Yates shuffle that picks the initial centroids
    (the reading of the open initialisation of III.B), against permutations
    worked step by step, including a draw that lands on a position an earlier
    swap moved, a draw with no swap, and the attention sinks kept apart."""
    g = _golden_init()
    for case in g["cases"] + [g["published_vector"]]:
        seed, h = int(case["seed"], 16), case["head"]
        got = orc.init_positions(h + 1, case["L"], case["C"], seed, n_sink=case["n_sink"])[h]
        assert got.tolist() == case["positions"], case


def test_init_shuffle_generator_is_published_splitmix64(orc):
    """Head 0 of seed 0x9E3779B97F4A7C15 starts from state 0, so its draws are
    SplitMix64's published seed-0 outputs; with n rows a draw r picks
    i + r mod (n - i). Checked over several n, so that every bit of the three
    outputs matters to some modulus."""
    pub = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    for n in (3, 10, 97, 1000, 65521, 1 << 20):
        perm = list(range(n))
        for i, r in enumerate(pub):
            j = i + r % (n - i)
            perm[i], perm[j] = perm[j], perm[i]
        got = orc.init_positions(1, n, 3, 0x9E3779B97F4A7C15)[0]
        assert got.tolist() == perm[:3], n


def test_init_shuffle_full_permutation_uniform(orc):
    """With C = n the shuffle is a full Fisher-Yates shuffle: every one of the
    n! orders is equally likely. Over 48,000 heads (independent streams) each
    of the 24 orders of n = 4 appears about 2,000 times (chi-square, p = 1e-6);
    the classic mistake j = r mod n (not i + r mod (n - i)) fails this."""
    from scipy.stats import chi2
    H = 48000
    p = orc.init_positions(H, 4, 4, 12345)
    assert np.all(np.sort(p, axis=1) == np.arange(4))
    code = p[:, 0] * 64 + p[:, 1] * 16 + p[:, 2] * 4 + p[:, 3]
    _, counts = np.unique(code, return_counts=True)
    assert counts.size == 24
    exp = H / 24
    stat = float(((counts - exp) ** 2 / exp).sum())
    assert stat < chi2.ppf(1 - 1e-6, 23), stat


def test_init_shuffle_distinct_in_range(orc):
    """Positions are distinct clustered rows (n_sink .. L-1); with C = 1 the
    first draw alone decides (uniform over the rows: every row is hit over
    many heads)."""
    p = orc.init_positions(16, 1500, 400, 7, n_sink=5)
    for row in p:
        assert len(set(row.tolist())) == 400
        assert row.min() >= 5 and row.max() < 1500
    one = orc.init_positions(20000, 25, 1, 99, n_sink=5)[:, 0]
    assert set(one.tolist()) == set(range(5, 25))
    with pytest.raises(ValueError):
        orc.init_positions(1, 10, 11, 1)


def test_build_from_seed_uses_the_shuffle(orc, syn):
    """A build given a seed starts from the keys at init_positions(seed)."""
    K, _, _ = syn.mixture_keys(syn.config_seed(91), 3, 600, 16, 8, 0.3, 0, 1.0, syn.F32, want_means=False)
    a = orc.build(K, 12, 4, seed=2024)
    b = orc.build(K, 12, 4, orc.init_positions(3, 600, 12, 2024))
    for k in ("labels", "c", "token_ids"):
        assert np.array_equal(a[k], b[k])


# ----------------------------------------------------------- objectives

def test_inertia_hand_cases_all_distances(orc):
    """The k-means objective of each distance (III.B: cosine; L2 and inner
    product are the alternatives) on a case worked by hand:
    K = (3, 4), (0, -2); operand rows (1, 0), (0, 1); labels 0, 1.
      cosine: sum ||K_i|| - K_i . chat = (5 - 3) + (2 - (-2)) = 6
      L2: ||(2, 4)||^2 + ||(0, -3)||^2 = 20 + 9 = 29
      inner product: -(3 + (-2)) = -1."""
    K = np.array([[3.0, 4.0], [0.0, -2.0]], dtype=np.float32)
    chat = np.array([[1.0, 0.0], [0.0, 1.0]], dtype=np.float64)
    lab = np.array([0, 1], dtype=np.int32)
    assert orc.inertia(K, chat, lab, orc.COSINE) == 6.0
    assert orc.inertia(K, chat, lab, orc.L2) == 29.0
    assert orc.inertia(K, chat, lab, orc.IP) == -1.0
    # the inner-product objective is minus the sum of the chosen products
    lab2 = np.array([1, 0], dtype=np.int32)
    assert orc.inertia(K, chat, lab2, orc.IP) == -(4.0 + 0.0)


def test_normalize_bf16_rounds_once_from_fp64(orc):
    """The bf16 operand is the fp64 quotient c_j / ||c|| rounded once (RNE), with
    ||c||^2 the ascending sum of exact squares: bit for bit, on rows chosen so
    that rounding through fp32 first would differ on some components."""
    rng = np.random.default_rng(11)
    c = (rng.standard_normal((4000, 64)) * rng.uniform(0.01, 40, (4000, 1))).astype(np.float32)
    got = orc.normalize(c, BF16)
    q = np.empty(c.shape, dtype=np.float64)
    for k in range(c.shape[0]):
        s = 0.0
        for v in c[k].tolist():
            s += v * v  # exact square of an fp32 value, summed in ascending order
        n = math.sqrt(s)
        q[k] = [v / n for v in c[k].tolist()]
    want = orc.round_bf16(q)
    assert np.array_equal(got, want)
    # the case is sensitive: rounding through fp32 changes some components
    via32 = orc.round_bf16(q.astype(np.float32).astype(np.float64))
    assert int((via32 != want).sum()) >= 1
