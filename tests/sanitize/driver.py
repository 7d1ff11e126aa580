"""Runs the oracle, the input generator and the C ABI's host code, built with
AddressSanitizer and UndefinedBehaviorSanitizer, over small inputs that reach
every function: argv = sanitized liboracle, libsynth, ABI library. Exits
non-zero (the sanitizers abort) on any report. numpy and ctypes only."""
import ctypes as C
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

oracle._LIB, synth._LIB, abi_path = sys.argv[1], sys.argv[2], sys.argv[3]
oracle._lib = synth._lib = None


def generator_and_oracle():
    base = synth.config_seed(3)
    H, L, d, Cn = 3, 300, 16, 9
    K, _, means = synth.mixture_keys(base, H, L + 4, d, 6, 0.3, 2, 10.0, synth.BF16, want_means=True)
    V = synth.values(base, H, L + 4, d, synth.BF16)
    Kf, _, _ = synth.mixture_keys(base, H, L, d, 6, 0.3, 0, 1.0, synth.F32)
    synth.normal_array(synth.stream_seed(base, 1, 2), (5, 7), 1.0, synth.F32)
    synth.init_idx(base, H, L, Cn)
    synth.round_bf16(np.linspace(-3, 3, 50))
    qn = synth.queries_noisy_key(base, 0, H * 2, 2, K, L, 0.1)
    qm = synth.queries_mixture(base, 1, H * 2, 2, means, 0.2, synth.BF16)
    synth.queries_drift(base, 2, H * 2, 2, means, 0.2, 0.1, synth.BF16)
    oracle.round_bf16(np.array([1.0, -2.5e-40, float("inf"), float("nan"), 3.4e38]))
    pos = oracle.init_positions(H, L, Cn, 77, n_sink=4)
    oracle.init_positions(2, 6, 6, 5)
    for metric in (oracle.COSINE, oracle.L2, oracle.IP):
        for kk in (K[:, :L], Kf):
            r = oracle.build(np.ascontiguousarray(kk), Cn, 4, seed=11, metric=metric)
            oracle.build(np.ascontiguousarray(kk), Cn, 3, mode=1, seed=11, metric=metric)
        oracle.build(np.ascontiguousarray(K[:, :L]), Cn, 3, pos, n_sink=4, metric=metric)
        chat = oracle.operand(r["c"][0], oracle.BF16, metric)
        oracle.assign(K[0, :L], chat, metric)
        oracle.inertia(K[0, :L], chat, r["labels"][0], metric)
    oracle.normalize(r["c"][0], oracle.F32)
    oracle.update(K[0, :L], r["labels"][0], r["c"][0])
    oracle.csr(r["labels"][0], Cn)
    idx = oracle.Index(r, L + 4)
    idx.append(np.ascontiguousarray(K[:, L]))
    idx.add_window(3)
    idx.cluster_window(K, 2, 3, np.tile(np.array([L + 1, L + 3], np.int32), (H, 1)))
    for q, B in ((qn, 40), (qm, 1), (qm, 10 * L)):
        sel, cnt, _, _ = oracle.select(q, 2, idx.c, idx.sizes, idx.offsets, idx.token_ids, B, n_sink=2,
                                       window=(L + 4, L + 4))
        oracle.decode(q, 2, K, V, sel, cnt, 1.0 / math.sqrt(d))
        oracle.recall(q, 2, K, L, sel, cnt)
    cache = oracle.ClusterCache(H, 1)
    cache.step(sel, cnt, idx.labels)


class Index(C.Structure):
    _fields_ = [("heads", C.c_int32), ("d", C.c_int32), ("C", C.c_int32), ("capacity", C.c_int32),
                ("dtype", C.c_int32), ("n_build", C.c_int32), ("n_tokens", C.c_int32), ("packed", C.c_int32),
                ("centroids", C.c_void_p), ("centroids_op", C.c_void_p), ("labels", C.c_void_p),
                ("sizes", C.c_void_p), ("offsets", C.c_void_p), ("token_ids", C.c_void_p),
                ("app_offsets", C.c_void_p), ("app_ids", C.c_void_p), ("dev_flags", C.c_void_p),
                ("centroids_t", C.c_void_p), ("k_packed", C.c_void_p), ("v_packed", C.c_void_p),
                ("n_sink", C.c_int32), ("c_slots", C.c_int32), ("c_active", C.c_int32),
                ("window_start", C.c_int32), ("metric", C.c_int32)]


class Cache(C.Structure):
    _fields_ = [("R", C.c_int32), ("B", C.c_int32), ("step", C.c_int32), ("reserved", C.c_int32),
                ("k", C.c_void_p), ("v", C.c_void_p), ("table", C.c_void_p), ("stats", C.c_void_p)]


def abi():
    """Every entry point with valid arguments (the launchers are no-ops) and
    with arguments each check must refuse; the pointers are never
    dereferenced on the host."""
    L = C.CDLL(abi_path)
    p = C.c_void_p(0x10000)
    u64, sz, f = C.c_uint64, C.c_size_t, C.c_float
    L.kv_cluster_index_bytes.restype = sz
    for fn in ("kv_cluster_build_workspace_bytes", "kv_sparse_decode_workspace_bytes",
               "kv_cluster_select_decode_workspace_bytes", "kv_dense_decode_workspace_bytes",
               "kv_cluster_window_workspace_bytes", "kv_cluster_cache_workspace_bytes"):
        getattr(L, fn).restype = sz
    L.kv_cluster_status_string.restype = C.c_char_p
    for s in range(8):
        L.kv_cluster_status_string(s)
    for heads, Cn, cap, dt, slots in ((4, 16, 256, 1, 0), (2, 512, 4096, 0, 0), (3, 40, 1500, 1, 64), (0, 1, 1, 1, 0)):
        L.kv_cluster_index_bytes(heads, 128, Cn, cap, dt, slots)
    idx = Index()
    nb = L.kv_cluster_index_bytes(4, 128, 16, 256, 1, 32)
    assert L.kv_cluster_index_init(C.byref(idx), 4, 128, 16, 256, 1, 32, 2, 0, p, sz(nb), None) == 0
    assert L.kv_cluster_index_init(C.byref(idx), 4, 128, 16, 256, 1, 32, 2, 0, p, sz(nb - 1), None) == 3
    ws = sz(1 << 40)
    L.kv_cluster_build_workspace_bytes(4, 200, 16, 10)
    assert L.kv_cluster_build(C.byref(idx), p, 200, 10, u64(7), p, ws, None) == 0
    assert L.kv_cluster_build_from(C.byref(idx), p, 200, 10, p, p, ws, None) == 0
    ev = (C.c_void_p * 20)(*([0x20000] * 20))
    assert L.kv_cluster_build_timed(C.byref(idx), p, 200, 10, u64(7), None, p, ws, ev, None) == 0
    assert L.kv_cluster_build(C.byref(idx), p, 10, 10, u64(7), p, ws, None) != 0
    assert L.kv_cluster_init_positions(4, 2, 200, 16, u64(9), p, None) == 0
    assert L.kv_cluster_append(C.byref(idx), p, p, p, p, 1, None) == 0
    assert L.kv_cluster_append(C.byref(idx), p, p, p, p, 1000, None) == 4
    assert L.kv_cluster_append_window(C.byref(idx), p, p, p, p, 3, None) == 0
    assert L.kv_cluster_cluster_window(C.byref(idx), p, p, 2, 3, p, p, ws, None) == 0
    assert L.kv_cluster_select(C.byref(idx), p, 16, 64, p, p, None) == 0
    assert L.kv_cluster_debug_scores(C.byref(idx), p, 16, p, None) == 0
    assert L.kv_cluster_debug_assign(C.byref(idx), p, 100, p, p, p, p, p, ws, None) == 0
    assert L.kv_cluster_debug_update(C.byref(idx), p, 100, p, ws, None) != 0  # sinks: refused
    for G, B in ((1, 1), (4, 1024), (8, 4096)):
        assert L.kv_sparse_decode(p, 4 * G, p, p, 1, 4, 256, 128, p, p, B, f(0.1), p, p, ws, None) == 0
        assert L.kv_sparse_decode_noalloc(p, 4 * G, p, p, 1, 4, 256, 128, p, p, B, f(0.1), p, None) == 0
        assert L.kv_cluster_select_decode(C.byref(idx), p, 4 * G, p, p, B, f(0.1), p, p, p, p, ws, None) == 0
        assert L.kv_dense_decode(p, 4 * G, p, p, 1, 4, 256, 128, 200, f(0.1), p, p, ws, None) == 0
    assert L.kv_sparse_decode_noalloc(p, 8192 * 8, p, p, 1, 8192, 256, 128, p, p, 1024, f(0.1), p, None) == 6
    idx.k_packed = idx.v_packed = 0x30000
    assert L.kv_cluster_pack(C.byref(idx), p, p, None) == 0
    assert L.kv_cluster_export_csr(C.byref(idx), p, p, None) == 0
    cache = Cache(1, 64, 0, 0, 0x40000, 0x40000, 0x40000, 0x40000)
    assert L.kv_cluster_cache_reset(C.byref(idx), C.byref(cache), None) == 0
    assert L.kv_cluster_cached_select_decode(C.byref(idx), C.byref(cache), p, 16, p, p, f(0.1), p, p, p, p, ws,
                                             None) == 0
    bad = Index()
    assert L.kv_cluster_select(C.byref(bad), p, 16, 64, p, p, None) != 0
    assert L.kv_cluster_cpad(0) == 0 and L.kv_cluster_cpad(513) == 544


generator_and_oracle()
abi()
print("sanitized run clean", flush=True)
