"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects invalid arguments with the documented status codes
before anything is enqueued (every call here fails validation, so no GPU is
touched)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvcluster.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, CAPACITY = 0, 1, 2, 3, 4
FAKE = 0x10000  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def kvc():
    import clustered_sparse_attention_kv_amd as m
    if not os.path.exists(m.LIB_PATH):
        m.build_lib()
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t|kvc_status|const char\*)\s+(kv_\w+)\(", text, re.M)))


def test_every_declared_function_is_exported(kvc):
    names = declared_functions()
    assert len(names) >= 25
    for n in ("kv_cluster_build", "kv_cluster_append", "kv_cluster_select", "kv_sparse_decode",
              "kv_cluster_index_bytes", "kv_cluster_debug_scores", "kv_cluster_init_positions"):
        assert n in names, n
    for n in names:
        assert hasattr(kvc.lib(), n), n


def make_index(kvc, heads=4, d=128, Cn=16, cap=256, dtype=1, n_build=0, n_tokens=0, null=None, window=0):
    """A descriptor with fake pointers; a "built" one (n_build > 0) has C
    clusters in use and `window` tokens in its window."""
    ptrs = [FAKE] * 10
    s = kvc._Index(heads, d, Cn, cap, dtype, n_build, n_tokens, 0, *ptrs)
    if n_build:
        s.c_active = Cn
        s.window_start = n_tokens - window
    if null:
        setattr(s, null, None)
    return s


def test_status_strings_and_sizes(kvc):
    L = kvc.lib()
    for code in range(7):
        assert L.kv_cluster_status_string(code) != b"unknown status"
    assert L.kv_cluster_status_string(99) == b"unknown status"
    assert [L.kv_cluster_cpad(c) for c in (1, 32, 33, 400, 512)] == [32, 32, 64, 416, 512]
    a = L.kv_cluster_build_workspace_bytes(128, 32768, 400, 10)
    b = L.kv_cluster_build_workspace_bytes(128, 32768, 400, 20)
    assert 0 < a < b and a % 256 == 0
    assert L.kv_cluster_build_workspace_bytes(0, 10, 1, 1) == 0
    assert L.kv_sparse_decode_workspace_bytes(128, 512, 128, 1024) >= 128 * 16 * 4 * 130 * 4


def test_build_rejects(kvc):
    L = kvc.lib()
    p = C.c_void_p(FAKE)

    def build(idx, Lk=200, iters=10, ws_bytes=1 << 40, keys=p, seed=5):
        return L.kv_cluster_build(C.byref(idx) if idx is not None else None, keys, Lk, iters, seed, p, ws_bytes, None)

    assert build(None) == INVALID
    assert build(make_index(kvc), keys=None) == INVALID
    assert L.kv_cluster_build_from(C.byref(make_index(kvc)), p, 200, 10, None, p, 1 << 40, None) == INVALID
    for field in ("centroids", "centroids_op", "labels", "sizes", "offsets", "token_ids", "app_offsets", "app_ids",
                  "dev_flags", "centroids_t"):
        assert build(make_index(kvc, null=field)) == INVALID, field
    assert build(make_index(kvc, d=64)) == UNSUPPORTED
    assert build(make_index(kvc, Cn=600)) == UNSUPPORTED
    assert build(make_index(kvc, dtype=7)) == INVALID
    assert build(make_index(kvc, Cn=16), Lk=15) == INVALID          # L < C
    assert build(make_index(kvc, cap=256), Lk=257) == INVALID       # L > capacity
    assert build(make_index(kvc), iters=0) == INVALID
    sinks = make_index(kvc, Cn=16)
    sinks.n_sink = -1
    assert build(sinks) == INVALID                                  # negative sink count
    sinks.n_sink = 190
    assert build(sinks, Lk=200) == INVALID                          # fewer clustered rows than C
    need = L.kv_cluster_build_workspace_bytes(4, 200, 16, 10)
    assert build(make_index(kvc), ws_bytes=need - 1) == WORKSPACE
    # the timed variant takes positions or (NULL positions) the seed, with the same checks
    assert L.kv_cluster_build_timed(C.byref(make_index(kvc)), p, 200, 10, 5, None, p, need - 1, None,
                                    None) == WORKSPACE


def test_init_positions_rejects(kvc):
    L = kvc.lib()
    p = C.c_void_p(FAKE)
    assert L.kv_cluster_init_positions(4, 0, 100, 10, 1, None, None) == INVALID
    assert L.kv_cluster_init_positions(0, 0, 100, 10, 1, p, None) == INVALID
    assert L.kv_cluster_init_positions(4, 0, 100, 0, 1, p, None) == INVALID
    assert L.kv_cluster_init_positions(4, 95, 100, 6, 1, p, None) == INVALID   # 5 rows for 6 positions
    assert L.kv_cluster_init_positions(4, -1, 100, 6, 1, p, None) == INVALID
    assert L.kv_cluster_init_positions(4, 0, 1000, 513, 1, p, None) == UNSUPPORTED


def test_index_layout(kvc):
    """kv_cluster_index_bytes covers every array of the index (each 256-byte
    aligned), and kv_cluster_index_init rejects bad sizes and small memory
    before it enqueues anything."""
    L = kvc.lib()
    H, d, Cn, cap = 3, 128, 40, 1000

    def al(x):
        return (x + 255) // 256 * 256

    for dt, e in ((1, 2), (0, 4)):
        for S in (0, 64):
            s_ = S or Cn
            cpad = (s_ + 31) // 32 * 32
            want = (al(4 * H * s_ * d) + al(e * H * cpad * d) + al(4 * H * cap) + al(4 * H * s_) + al(4 * H * (s_ + 1))
                    + al(4 * H * cap) + al(4 * H * (s_ + 1)) + al(4 * H * cap) + al(4) + al(4 * H * s_ * d))
            assert L.kv_cluster_index_bytes(H, d, Cn, cap, dt, S) == want, (dt, S)
    assert L.kv_cluster_index_bytes(H, 64, Cn, cap, 1, 0) == 0
    assert L.kv_cluster_index_bytes(H, d, 600, cap, 1, 0) == 0
    assert L.kv_cluster_index_bytes(H, d, Cn, cap, 1, 20) == 0       # fewer slots than clusters
    assert L.kv_cluster_index_bytes(0, d, Cn, cap, 1, 0) == 0
    idx = kvc._Index()
    p = C.c_void_p(FAKE)
    need = L.kv_cluster_index_bytes(H, d, Cn, cap, 1, 0)
    assert L.kv_cluster_index_init(C.byref(idx), H, d, Cn, cap, 1, 0, 0, 0, p, need - 1, None) == WORKSPACE
    assert L.kv_cluster_index_init(C.byref(idx), H, d, Cn, cap, 1, 0, 0, 0, None, need, None) == INVALID
    assert L.kv_cluster_index_init(None, H, d, Cn, cap, 1, 0, 0, 0, p, need, None) == INVALID
    assert L.kv_cluster_index_init(C.byref(idx), H, 64, Cn, cap, 1, 0, 0, 0, p, need, None) == UNSUPPORTED
    assert L.kv_cluster_index_init(C.byref(idx), H, d, Cn, cap, 1, 0, -1, 0, p, need, None) == INVALID
    assert L.kv_cluster_index_init(C.byref(idx), H, d, Cn, cap, 1, 0, 0, 3, p, need, None) == INVALID
    assert idx.centroids is None   # untouched on error


def test_debug_scores_rejects(kvc):
    L = kvc.lib()
    p = C.c_void_p(FAKE)
    built = make_index(kvc, heads=4, n_build=200, n_tokens=200)
    assert L.kv_cluster_debug_scores(C.byref(built), p, 6, p, None) == INVALID          # 6 % 4 != 0
    assert L.kv_cluster_debug_scores(C.byref(built), p, 36, p, None) == UNSUPPORTED     # G = 9
    assert L.kv_cluster_debug_scores(C.byref(built), p, 16, None, None) == INVALID
    assert L.kv_cluster_debug_scores(C.byref(make_index(kvc)), p, 16, p, None) == INVALID  # never built


def test_append_select_decode_reject(kvc):
    L = kvc.lib()
    p = C.c_void_p(FAKE)
    full = make_index(kvc, cap=256, n_build=200, n_tokens=250)
    assert L.kv_cluster_append(C.byref(full), p, p, p, p, 7, None) == CAPACITY
    assert L.kv_cluster_append(C.byref(full), p, p, p, p, 0, None) == INVALID
    assert L.kv_cluster_append(C.byref(make_index(kvc)), p, p, p, p, 1, None) == INVALID  # never built
    built = make_index(kvc, heads=4, n_build=200, n_tokens=200)
    assert L.kv_cluster_select(C.byref(built), p, 6, 64, p, p, None) == INVALID       # 6 % 4 != 0
    assert L.kv_cluster_select(C.byref(built), p, 4 * 9, 64, p, p, None) == UNSUPPORTED  # G = 9
    assert L.kv_cluster_select(C.byref(built), p, 16, 0, p, p, None) == INVALID
    assert L.kv_cluster_select(C.byref(make_index(kvc)), p, 16, 64, p, p, None) == INVALID
    f = C.c_float(0.1)
    assert L.kv_cluster_select_decode(C.byref(built), p, 12, p, p, 64, f, p, None, None, None, 0, None) == UNSUPPORTED
    assert L.kv_cluster_select_decode(C.byref(built), p, 16, None, p, 64, f, p, None, None, None, 0, None) == INVALID
    sd_ws = L.kv_cluster_select_decode_workspace_bytes(4, 16, 128)
    assert sd_ws >= 4 * 8 * 4 * 130 * 4  # 4 heads x 8 blocks x 4 query heads x (128 + 2) floats
    assert L.kv_cluster_select_decode(C.byref(built), p, 16, p, p, 64, f, p, None, None, p, sd_ws - 1,
                                      None) == WORKSPACE
    ws = L.kv_sparse_decode_workspace_bytes(4, 16, 128, 64)
    dec = lambda **k: L.kv_sparse_decode(p, k.get("qh", 16), p, p, k.get("dt", 1), 4, 256, k.get("d", 128), p, p,
                                         k.get("B", 64), f, p, p, k.get("ws", ws), None)
    assert dec(d=64) == UNSUPPORTED
    assert dec(qh=12) == UNSUPPORTED
    assert dec(qh=10) == INVALID
    assert dec(dt=3) == INVALID
    assert dec(ws=ws - 1) == WORKSPACE
    assert dec(B=0) == INVALID
    assert dec(qh=32, B=4096 + 64, ws=1 << 40) == UNSUPPORTED   # 65 splits x 8 heads > 512 pairs
    # the allocation-free variant: the same checks, and requests beyond its
    # fixed scratch are refused before anything is enqueued
    na = lambda **k: L.kv_sparse_decode_noalloc(p, k.get("qh", 16), p, p, 1, k.get("heads", 4), 256, k.get("d", 128),
                                                p, p, k.get("B", 64), f, k.get("out", p), None)
    assert na(d=64) == UNSUPPORTED and na(qh=10) == INVALID and na(B=0) == INVALID and na(out=None) == INVALID
    assert L.kv_sparse_decode_workspace_bytes(8192, 8192 * 8, 128, 1024) > 16 << 20
    assert na(heads=8192, qh=8192 * 8, B=1024) == 6  # KVC_ERR_TOO_LARGE
    assert L.kv_cluster_export_csr(C.byref(built), None, p, None) == INVALID
    # the dense comparator: bf16 only, 1 <= n <= capacity, enough workspace
    dws = L.kv_dense_decode_workspace_bytes(4, 16, 128, 200)
    assert dws > 0 and L.kv_dense_decode_workspace_bytes(4, 16, 64, 200) == 0
    dd = lambda **k: L.kv_dense_decode(p, k.get("qh", 16), p, p, k.get("dt", 1), 4, 256, k.get("d", 128),
                                       k.get("n", 200), f, p, p, k.get("ws", dws), None)
    assert dd(dt=0) == UNSUPPORTED
    assert dd(d=64) == UNSUPPORTED
    assert dd(qh=12) == UNSUPPORTED
    assert dd(n=0) == INVALID and dd(n=257) == INVALID
    assert dd(ws=dws - 1) == WORKSPACE
    # packing needs both packed arrays and a built index
    assert L.kv_cluster_pack(C.byref(built), p, p, None) == INVALID           # no packed arrays
    unbuilt = make_index(kvc)
    unbuilt.k_packed, unbuilt.v_packed = FAKE, FAKE
    assert L.kv_cluster_pack(C.byref(unbuilt), p, p, None) == INVALID         # not built
    withp = make_index(kvc, n_build=200, n_tokens=200)
    withp.k_packed = FAKE
    assert L.kv_cluster_pack(C.byref(withp), p, None, None) == INVALID        # no v_cache


def test_window_calls_reject(kvc):
    """Generated-token window: appends, clustering and slot counts are checked
    against the index state before anything is enqueued."""
    L = kvc.lib()
    p = C.c_void_p(FAKE)
    # a nearest-centroid append needs an empty window
    open_w = make_index(kvc, cap=256, n_build=200, n_tokens=210, window=10)
    assert L.kv_cluster_append(C.byref(open_w), p, p, p, p, 1, None) == INVALID
    assert L.kv_cluster_append_window(C.byref(open_w), p, p, p, p, 47, None) == CAPACITY
    assert L.kv_cluster_append_window(C.byref(open_w), p, p, p, p, 0, None) == INVALID
    assert L.kv_cluster_append_window(C.byref(make_index(kvc)), p, p, p, p, 1, None) == INVALID  # never built
    # clustering the window: 1 <= n_clusters <= window, free slots, iters >= 1, workspace
    ws = L.kv_cluster_window_workspace_bytes(4, 10, 2, 3)
    assert ws > 0 and ws % 256 == 0 and L.kv_cluster_window_workspace_bytes(4, 0, 2, 3) == 0
    slotted = make_index(kvc, Cn=16, cap=256, n_build=200, n_tokens=210, window=10)
    slotted.c_slots = 20
    cw = lambda idx, nc=2, it=3, b=ws: L.kv_cluster_cluster_window(C.byref(idx), p, p, nc, it, p, p, b, None)
    assert cw(open_w) == INVALID                      # no free slot (c_slots = C)
    assert cw(slotted, nc=0) == INVALID
    assert cw(slotted, nc=11) == INVALID              # more clusters than window tokens
    assert cw(slotted, nc=5) == INVALID               # 16 + 5 > 20 slots
    assert cw(slotted, it=0) == INVALID
    assert cw(slotted, b=ws - 1) == WORKSPACE
    empty = make_index(kvc, Cn=16, cap=256, n_build=200, n_tokens=200)
    empty.c_slots = 20
    assert cw(empty, nc=1) == INVALID                 # empty window
    assert cw(make_index(kvc), nc=1) == INVALID       # never built
    # slot counts: at least C, at most 512
    few = make_index(kvc, Cn=16)
    few.c_slots = 8
    assert L.kv_cluster_build(C.byref(few), p, 200, 3, 1, p, 1 << 40, None) == INVALID
    many = make_index(kvc, Cn=16)
    many.c_slots = 600
    assert L.kv_cluster_build(C.byref(many), p, 200, 3, 1, p, 1 << 40, None) == UNSUPPORTED
    # the assignment distance is one of cosine, L2, inner product
    for bad in (-1, 3):
        odd = make_index(kvc, Cn=16)
        odd.metric = bad
        assert L.kv_cluster_build(C.byref(odd), p, 200, 3, 1, p, 1 << 40, None) == INVALID


def test_cluster_cache_calls_reject(kvc):
    """The cluster cache: descriptor fields, index state, G, B and the
    workspace are checked before anything is enqueued."""
    L = kvc.lib()
    p = C.c_void_p(FAKE)
    built = make_index(kvc, heads=4, Cn=16, cap=256, n_build=200, n_tokens=200)
    f = C.c_float(0.1)
    ws = L.kv_cluster_cache_workspace_bytes(4, 16, 128, 64)
    assert ws >= L.kv_sparse_decode_workspace_bytes(4, 16, 128, 64) + 4 * 64 * 4
    assert L.kv_cluster_cache_workspace_bytes(0, 16, 128, 64) == 0

    def cache(R=1, B=64, null=None):
        c = kvc._Cache(R, B, 0, 0, FAKE, FAKE, FAKE, FAKE)
        if null:
            setattr(c, null, None)
        return c

    def run(idx=built, c=None, qh=16, b=ws):
        return L.kv_cluster_cached_select_decode(C.byref(idx), C.byref(c or cache()), p, qh, p, p, f, p, None, None, p,
                                                 b, None)
    assert run(c=cache(R=0)) == INVALID
    assert run(c=cache(B=0)) == INVALID
    for field in ("k", "v", "table", "stats"):
        assert run(c=cache(null=field)) == INVALID, field
    assert run(idx=make_index(kvc)) == INVALID          # never built
    assert run(qh=12) == UNSUPPORTED                    # G = 3
    assert run(qh=10) == INVALID                        # 10 % 4 != 0
    assert run(b=ws - 1) == WORKSPACE
    assert run(c=cache(B=8192 + 64), b=1 << 40) == UNSUPPORTED  # 129 splits x 4 heads > 512 pairs
    assert L.kv_cluster_cache_reset(C.byref(built), C.byref(cache(null="table")), None) == INVALID


def test_binding_fails_loudly_without_library(kvc, monkeypatch):
    """The product path never falls back to anything else: no library, no call."""
    import clustered_sparse_attention_kv_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "LIB_PATH", "/nonexistent/libkvcluster.so")
    with pytest.raises(RuntimeError):
        m.lib()
