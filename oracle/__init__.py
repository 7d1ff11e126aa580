"""CPU oracle for the clustered sparse-KV hot path (ClusterKV, arXiv 2412.03213).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The GPU library never
imports or links this package, and there is no fallback from the GPU path to it.

The arithmetic lives in ``kvc_oracle.c`` (plain C, fp64, fixed-order chains);
this module compiles it with gcc and marshals numpy arrays through ctypes.
Arrays of bf16 values are passed as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2
COSINE, L2, IP = 0, 1, 2  # assignment distance (III.B: cosine; L2 and inner product are the alternatives)

_lib = None


def compile_lib(force: bool = True) -> str:
    """Compile the oracle with gcc (fp contraction off, explicit fma only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-mavx2", "-mfma", "-ffp-contract=off", "-fopenmp", "-shared",
               "-fPIC", "-std=c11", "-Wall", "-Wno-unused-variable", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            compile_lib(force=False)
        lib = C.CDLL(_LIB)
        p, i, ll, d = C.c_void_p, C.c_int, C.c_longlong, C.c_double
        lib.orc_round_bf16.argtypes = [d]
        lib.orc_round_bf16.restype = C.c_uint16
        lib.orc_normalize.argtypes = [i, i, p, i, p, i]
        lib.orc_operand.argtypes = [i, i, p, i, p, i, i]
        lib.orc_assign.argtypes = [i, i, i, p, i, ll, p, i, i, p, p]
        lib.orc_update.argtypes = [i, i, i, p, i, ll, p, p, i, p]
        lib.orc_csr.argtypes = [i, i, p, p, p, p]
        lib.orc_inertia.argtypes = [i, i, p, i, ll, p, i, i, p]
        lib.orc_inertia.restype = d
        lib.orc_build.argtypes = [i, i, i, i, i, i, i, i, p, ll, p, p, p, p, p, p, p, p, p, i]
        lib.orc_build.restype = i
        lib.orc_append.argtypes = [i, i, i, p, i, p, i, i, p, p, p, p]
        lib.orc_append.restype = i
        lib.orc_select.argtypes = [i, i, i, i, i, p, i, p, p, p, p, ll, p, p, p, p]
        lib.orc_decode.argtypes = [i, i, i, p, i, p, p, i, ll, p, p, i, d, p]
        lib.orc_recall.argtypes = [i, i, i, i, i, p, i, p, i, ll, p, p, p]
        lib.orc_init.argtypes = [i, i, i, i, C.c_uint64, p]
        lib.orc_init.restype = i
        _lib = lib
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported element type {a.dtype}")


def _np_of(dt: int):
    return {F32: np.float32, BF16: np.uint16, F64: np.float64}[dt]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def round_bf16(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns, round to nearest even (scalar C routine per element)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for t in range(flat_in.size):
        flat_out[t] = lib.orc_round_bf16(float(flat_in[t]))
    return out


def to_f64(a: np.ndarray) -> np.ndarray:
    """Values of an array as fp64 (bf16 bit patterns decoded exactly)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def normalize(c: np.ndarray, optype: int) -> np.ndarray:
    """c [C, d] (fp32 or fp64) -> unit-length operand in ``optype``."""
    lib = _load()
    c = _c(c)
    Cn, d = c.shape
    out = np.empty((Cn, d), dtype=_np_of(optype))
    lib.orc_normalize(Cn, d, _ptr(c), _dt(c), _ptr(out), optype)
    return out


def operand(c: np.ndarray, optype: int, metric: int = COSINE) -> np.ndarray:
    """c [C, d] -> the assignment operand in ``optype``: the unit direction
    (cosine) or the centroid itself (L2, inner product), rounded once."""
    lib = _load()
    c = _c(c)
    Cn, d = c.shape
    out = np.empty((Cn, d), dtype=_np_of(optype))
    lib.orc_operand(Cn, d, _ptr(c), _dt(c), _ptr(out), optype, metric)
    return out


def assign(K: np.ndarray, chat: np.ndarray, metric: int = COSINE):
    """K [L, d], chat [C, d] -> (labels int32 [L], best score fp64 [L])."""
    lib = _load()
    K, chat = _c(K), _c(chat)
    L, d = K.shape
    labels = np.empty(L, dtype=np.int32)
    best = np.empty(L, dtype=np.float64)
    lib.orc_assign(L, d, chat.shape[0], _ptr(K), _dt(K), d, _ptr(chat), _dt(chat), metric, _ptr(labels),
                   _ptr(best))
    return labels, best


def update(K: np.ndarray, labels: np.ndarray, c: np.ndarray):
    """Means of the assigned keys; returns (new c, counts). c is not modified."""
    lib = _load()
    K, c = _c(K), _c(c).copy()
    labels = _c(labels, np.int32)
    L, d = K.shape
    counts = np.empty(c.shape[0], dtype=np.int32)
    lib.orc_update(L, d, c.shape[0], _ptr(K), _dt(K), d, _ptr(labels), _ptr(c), _dt(c), _ptr(counts))
    return c, counts


def csr(labels: np.ndarray, C: int):
    """labels [L] -> (sizes [C], offsets [C+1], token_ids [L])."""
    lib = _load()
    labels = _c(labels, np.int32)
    L = labels.shape[0]
    sizes = np.empty(C, dtype=np.int32)
    offsets = np.empty(C + 1, dtype=np.int32)
    ids = np.empty(L, dtype=np.int32)
    lib.orc_csr(L, C, _ptr(labels), _ptr(sizes), _ptr(offsets), _ptr(ids))
    return sizes, offsets, ids


def inertia(K: np.ndarray, chat: np.ndarray, labels: np.ndarray, metric: int = COSINE) -> float:
    lib = _load()
    K, chat = _c(K), _c(chat)
    labels = _c(labels, np.int32)
    L, d = K.shape
    return lib.orc_inertia(L, d, _ptr(K), _dt(K), d, _ptr(chat), _dt(chat), metric, _ptr(labels))


def init_positions(H: int, L: int, C: int, seed: int, n_sink: int = 0) -> np.ndarray:
    """Initial centroid positions [H, C] int32: per head, the first C entries of
    a partial Fisher-Yates shuffle of the clustered rows n_sink .. L-1, driven
    by SplitMix64 from state seed ^ (0x9E3779B97F4A7C15 * (h + 1))."""
    lib = _load()
    out = np.empty((H, C), dtype=np.int32)
    if lib.orc_init(H, n_sink, L, C, seed & ((1 << 64) - 1), _ptr(out)) != 0:
        raise ValueError("init_positions needs 1 <= C <= L - n_sink")
    return out


def build(K: np.ndarray, C: int, iters: int, init_idx: np.ndarray | None = None, L: int | None = None,
          mode: int = 0, early_exit: bool = True, n_sink: int = 0, metric: int = COSINE,
          seed: int | None = None) -> dict:
    """Prefill clustering of every head of K [H, rows, d] over its first L rows.

    The initial centroids are the keys at init_idx [H, C], or, with init_idx
    None, at init_positions(H, L, C, seed, n_sink) (the seeded shuffle).

    mode 0: centroids fp32, operand in the key type; mode 1: exact (fp64).
    metric: assignment distance, COSINE (the method's), L2 or IP.
    n_sink: the first n_sink rows are attention sinks (III.B keeps the first
    tokens apart and clusters the rest): they get label -1, stay out of every
    cluster, and init_idx holds positions >= n_sink. token_ids hold the
    clustered tokens' positions (L - n_sink of them).
    Returns a dict with c, chat, labels, sizes, offsets, token_ids, inertia,
    iters_run.
    """
    if init_idx is None:
        if seed is None:
            raise ValueError("build needs init_idx or a seed")
        init_idx = init_positions(K.shape[0], K.shape[1] if L is None else L, C, seed, n_sink)
    if n_sink:
        H, rows, _ = K.shape
        L = rows if L is None else L
        r = build(np.ascontiguousarray(K[:, n_sink:L]), C, iters, np.asarray(init_idx, np.int32) - n_sink,
                  mode=mode, early_exit=early_exit, metric=metric)
        labels = np.full((H, L), -1, dtype=np.int32)
        labels[:, n_sink:] = r["labels"]
        r["labels"] = labels
        r["token_ids"] = r["token_ids"] + np.int32(n_sink)
        return r
    lib = _load()
    K = _c(K)
    H, rows, d = K.shape
    L = rows if L is None else L
    init_idx = _c(init_idx, np.int32).reshape(H, C)
    kdt = _dt(K)
    cdt = F64 if mode == 1 else F32
    optype = F64 if mode == 1 else kdt
    c = np.empty((H, C, d), dtype=_np_of(cdt))
    chat = np.empty((H, C, d), dtype=_np_of(optype))
    labels = np.empty((H, L), dtype=np.int32)
    sizes = np.empty((H, C), dtype=np.int32)
    offsets = np.empty((H, C + 1), dtype=np.int32)
    ids = np.empty((H, L), dtype=np.int32)
    inert = np.empty((H, iters), dtype=np.float64)
    iters_run = np.empty(H, dtype=np.int32)
    rc = lib.orc_build(H, L, d, C, iters, kdt, mode, metric, _ptr(K), rows * d, _ptr(init_idx), _ptr(c), _ptr(chat),
                       _ptr(labels), _ptr(sizes), _ptr(offsets), _ptr(ids), _ptr(inert), _ptr(iters_run),
                       1 if early_exit else 0)
    if rc != 0:
        raise ValueError("init index out of range")
    return dict(c=c, chat=chat, labels=labels, sizes=sizes, offsets=offsets, token_ids=ids,
                inertia=inert, iters_run=iters_run)


class Index:
    """Canonical host-side cluster index of one build, grown by append()
    (nearest centroid) or by add_window() + cluster_window() (generated tokens
    clustered on their own, III.B)."""

    def __init__(self, built: dict, capacity: int, metric: int = COSINE):
        H, L = built["labels"].shape
        self.metric = metric
        self.H, self.C = built["sizes"].shape
        self.n = L  # tokens, sinks included; the next one gets position n
        self.window_start = L  # tokens window_start .. n-1 are in no cluster yet
        self.c = built["c"]
        self.chat = built["chat"]
        self.labels = np.full((H, capacity), -1, dtype=np.int32)
        self.labels[:, :L] = built["labels"]
        self.sizes = built["sizes"].copy()
        self.offsets = built["offsets"].copy()
        self.token_ids = np.full((H, capacity), -1, dtype=np.int32)
        nc = built["token_ids"].shape[1]
        self.token_ids[:, :nc] = built["token_ids"]

    def append(self, knew: np.ndarray) -> np.ndarray:
        """knew [H, d]: one new key per head; returns the labels."""
        if self.window_start != self.n:
            raise ValueError("the window of generated tokens is not empty: cluster it first")
        lib = _load()
        knew = _c(knew)
        H, d = knew.shape
        out = np.empty(H, dtype=np.int32)
        for h in range(H):
            kh = np.ascontiguousarray(knew[h])
            ch = np.ascontiguousarray(self.chat[h])
            lab = self.labels[h]
            sz = self.sizes[h]
            off = self.offsets[h]
            ids = self.token_ids[h]
            out[h] = lib.orc_append(d, self.C, self.n, _ptr(kh), _dt(kh), _ptr(ch), _dt(ch), self.metric, _ptr(lab),
                                    _ptr(sz), _ptr(off), _ptr(ids))
        self.n += 1
        self.window_start = self.n
        return out

    def add_window(self, n_new: int = 1):
        """n_new generated tokens per head join the window (label -1)."""
        self.n += n_new

    def cluster_window(self, K: np.ndarray, n_clusters: int, iters: int, init_idx: np.ndarray) -> dict:
        """III.B: the window's tokens (positions window_start .. n-1 of the keys
        K [H, rows, d]) are clustered on their own by the prefill k-means into
        n_clusters new clusters, starting from the keys at init_idx ([H,
        n_clusters] positions in the window). The new clusters get the next
        ids, C .. C + n_clusters - 1; the existing ones do not change. Since
        their ids are the largest, their members follow every existing member
        in the canonical index. Returns the window's own build result."""
        lo, hi = self.window_start, self.n
        r = build(np.ascontiguousarray(K[:, lo:hi]), n_clusters, iters,
                  np.asarray(init_idx, np.int32) - np.int32(lo), metric=self.metric)
        C0, m = self.C, hi - lo
        total = self.offsets[:, C0]
        self.labels[:, lo:hi] = C0 + r["labels"]
        self.c = np.concatenate([self.c, r["c"]], axis=1)
        self.chat = np.concatenate([self.chat, r["chat"]], axis=1)
        self.sizes = np.concatenate([self.sizes, r["sizes"]], axis=1)
        self.offsets = np.concatenate([self.offsets, total[:, None] + r["offsets"][:, 1:]], axis=1)
        for h in range(self.H):
            self.token_ids[h, total[h]:total[h] + m] = r["token_ids"][h] + lo
        self.C += n_clusters
        self.window_start = hi
        return r


def select(q: np.ndarray, G: int, c: np.ndarray, sizes: np.ndarray, offsets: np.ndarray,
           token_ids: np.ndarray, B: int, n_sink: int = 0, window: tuple | None = None):
    """q [H*G, d]; c fp32 [H, C, d]; CSR arrays per head. Returns
    (sel_ids [H, B], sel_count [H], scores [H, C], order [H, C]).

    Tokens recalled ahead of every cluster, as many as B allows, in this
    order: n_sink attention sinks (III.B; tokens 0 .. n_sink - 1), then the
    window of generated tokens not yet clustered (window = (lo, hi): tokens lo
    .. hi - 1). The clusters fill the remaining entries as on their own."""
    fixed = np.arange(n_sink, dtype=np.int32)
    if window is not None:
        fixed = np.concatenate([fixed, np.arange(window[0], window[1], dtype=np.int32)])
    nf = fixed.shape[0]
    if nf:
        H = c.shape[0]
        ns = min(B, nf)
        rest = max(B - nf, 1)
        s2, c2, scores, order = select(q, G, c, sizes, offsets, token_ids, rest)
        sel = np.full((H, B), -1, dtype=np.int32)
        sel[:, :ns] = fixed[:ns]
        cnt = np.full(H, ns, dtype=np.int32)
        if B > nf:
            sel[:, nf:] = s2
            cnt = cnt + c2
        return sel, cnt, scores, order
    lib = _load()
    q = _c(q)
    c = _c(c, np.float32)
    sizes, offsets, token_ids = _c(sizes, np.int32), _c(offsets, np.int32), _c(token_ids, np.int32)
    H, Cn, d = c.shape
    sel = np.empty((H, B), dtype=np.int32)
    cnt = np.empty(H, dtype=np.int32)
    scores = np.empty((H, Cn), dtype=np.float64)
    order = np.empty((H, Cn), dtype=np.int32)
    lib.orc_select(H, G, d, Cn, B, _ptr(q), _dt(q), _ptr(c), _ptr(sizes), _ptr(offsets), _ptr(token_ids),
                   token_ids.shape[1], _ptr(sel), _ptr(cnt), _ptr(scores), _ptr(order))
    return sel, cnt, scores, order


def decode(q: np.ndarray, G: int, Kc: np.ndarray, Vc: np.ndarray, sel_ids: np.ndarray,
           sel_count: np.ndarray, scale: float) -> np.ndarray:
    """q [H*G, d]; Kc, Vc [H, rows, d]; sel_ids [H, B] -> out fp32 [H*G, d]."""
    lib = _load()
    q, Kc, Vc = _c(q), _c(Kc), _c(Vc)
    sel_ids, sel_count = _c(sel_ids, np.int32), _c(sel_count, np.int32)
    H, rows, d = Kc.shape
    B = sel_ids.shape[1]
    if _dt(Kc) != _dt(Vc):
        raise TypeError("K and V caches must share a type")
    out = np.empty((H * G, d), dtype=np.float32)
    lib.orc_decode(H, G, d, _ptr(q), _dt(q), _ptr(Kc), _ptr(Vc), _dt(Kc), rows * d, _ptr(sel_ids),
                   _ptr(sel_count), B, float(scale), _ptr(out))
    return out


def recall(q: np.ndarray, G: int, Kc: np.ndarray, N: int, sel_ids: np.ndarray, sel_count: np.ndarray) -> np.ndarray:
    """Fraction of the exact top-min(B, N) attention tokens of each query head
    (q [H*G, d], keys Kc [H, rows, d], first N rows) that the selection
    sel_ids [H, B] (sel_count [H] valid entries) recalls -> float64 [H*G]."""
    lib = _load()
    q, Kc = _c(q), _c(Kc)
    sel_ids, sel_count = _c(sel_ids, np.int32), _c(sel_count, np.int32)
    H, rows, d = Kc.shape
    B = sel_ids.shape[1]
    out = np.empty(H * G, dtype=np.float64)
    lib.orc_recall(H, G, d, int(N), B, _ptr(q), _dt(q), _ptr(Kc), _dt(Kc), rows * d, _ptr(sel_ids),
                   _ptr(sel_count), _ptr(out))
    return out


class ClusterCache:
    """Counters of the GPU cluster cache (Sys-D: the GPU keeps the selected KV
    and cluster labels of the last R decoding steps, and only clusters absent
    from it are loaded), simulated from the selections.

    Per head, the cache remembers for each cluster the step of its most recent
    selection and how many members were taken then (selection takes a prefix
    of each cluster's members in index order). At step t a selected cluster k
    taking m members is found in the cache when its last selection was at a
    step in [t - R, t - 1]; then min(m, members taken then) of its tokens are
    cache hits. Sinks and window tokens (label -1) are not counted."""

    def __init__(self, H: int, R: int):
        self.R, self.t = R, 0
        self.last = [dict() for _ in range(H)]
        self.stats = np.zeros((H, 4), dtype=np.int64)  # clusters, cluster hits, tokens, token hits

    def step(self, sel_ids: np.ndarray, sel_count: np.ndarray, labels: np.ndarray):
        """sel_ids [H, B] token ids, sel_count [H], labels [H, rows] of the index."""
        for h, last in enumerate(self.last):
            ids = sel_ids[h, :sel_count[h]]
            labs = labels[h, ids]
            ks, ms = np.unique(labs[labs >= 0], return_counts=True)
            for k, m in zip(ks.tolist(), ms.tolist()):
                self.stats[h, 0] += 1
                self.stats[h, 2] += m
                if k in last and self.t - self.R <= last[k][0] < self.t:
                    self.stats[h, 1] += 1
                    self.stats[h, 3] += min(m, last[k][1])
            for k, m in zip(ks.tolist(), ms.tolist()):
                last[k] = (self.t, m)
        self.t += 1
