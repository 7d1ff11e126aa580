"""Cluster-granular sparse KV recall on AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libkvcluster.so`` (C ABI declared in
``include/kvcluster.h``). Every step of the path runs in the library's HIP
kernels; this module only checks tensor shapes, passes device pointers and the
current stream, and turns status codes into exceptions. PyTorch supplies the
device memory and streams.

There is no CPU fallback: when the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvcluster.so")

KVC_F32, KVC_BF16 = 0, 1
COSINE, L2, INNER_PRODUCT = 0, 1, 2  # assignment distance (kvc_metric)
HEAD_DIM, MAX_C, MAX_G = 128, 512, 8

_lib = None


class KvcError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class _Index(C.Structure):
    _fields_ = [("heads", C.c_int32), ("d", C.c_int32), ("C", C.c_int32), ("capacity", C.c_int32),
                ("dtype", C.c_int32), ("n_build", C.c_int32), ("n_tokens", C.c_int32), ("packed", C.c_int32),
                ("centroids", C.c_void_p), ("centroids_op", C.c_void_p), ("labels", C.c_void_p),
                ("sizes", C.c_void_p), ("offsets", C.c_void_p), ("token_ids", C.c_void_p),
                ("app_offsets", C.c_void_p), ("app_ids", C.c_void_p), ("dev_flags", C.c_void_p),
                ("centroids_t", C.c_void_p), ("k_packed", C.c_void_p), ("v_packed", C.c_void_p),
                ("n_sink", C.c_int32), ("c_slots", C.c_int32), ("c_active", C.c_int32),
                ("window_start", C.c_int32), ("metric", C.c_int32)]


class _Cache(C.Structure):
    _fields_ = [("R", C.c_int32), ("B", C.c_int32), ("step", C.c_int32), ("reserved", C.c_int32),
                ("k", C.c_void_p), ("v", C.c_void_p), ("table", C.c_void_p), ("stats", C.c_void_p)]


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with clustered_sparse_attention_kv_amd.build_lib()")
        L = C.CDLL(LIB_PATH)
        p, i, sz, f = C.c_void_p, C.c_int, C.c_size_t, C.c_float
        L.kv_cluster_cpad.argtypes = [i]
        L.kv_cluster_cpad.restype = i
        L.kv_cluster_build_workspace_bytes.argtypes = [i, i, i, i]
        L.kv_cluster_build_workspace_bytes.restype = sz
        u64 = C.c_uint64
        L.kv_cluster_index_bytes.argtypes = [i, i, i, i, i, i]
        L.kv_cluster_index_bytes.restype = sz
        L.kv_cluster_index_init.argtypes = [p, i, i, i, i, i, i, i, i, p, sz, p]
        L.kv_cluster_init_positions.argtypes = [i, i, i, i, u64, p, p]
        L.kv_cluster_build.argtypes = [p, p, i, i, u64, p, sz, p]
        L.kv_cluster_build_from.argtypes = [p, p, i, i, p, p, sz, p]
        L.kv_cluster_build_timed.argtypes = [p, p, i, i, u64, p, p, sz, p, p]
        L.kv_cluster_debug_scores.argtypes = [p, p, i, p, p]
        L.kv_cluster_append.argtypes = [p, p, p, p, p, i, p]
        L.kv_cluster_append_window.argtypes = [p, p, p, p, p, i, p]
        L.kv_cluster_window_workspace_bytes.argtypes = [i, i, i, i]
        L.kv_cluster_window_workspace_bytes.restype = sz
        L.kv_cluster_cluster_window.argtypes = [p, p, p, i, i, p, p, sz, p]
        L.kv_cluster_select.argtypes = [p, p, i, i, p, p, p]
        L.kv_sparse_decode_workspace_bytes.argtypes = [i, i, i, i]
        L.kv_sparse_decode_workspace_bytes.restype = sz
        L.kv_sparse_decode.argtypes = [p, i, p, p, i, i, i, i, p, p, i, f, p, p, sz, p]
        L.kv_sparse_decode_noalloc.argtypes = [p, i, p, p, i, i, i, i, p, p, i, f, p, p]
        L.kv_cluster_select_decode_workspace_bytes.argtypes = [i, i, i]
        L.kv_cluster_select_decode_workspace_bytes.restype = sz
        L.kv_cluster_select_decode.argtypes = [p, p, i, p, p, i, f, p, p, p, p, sz, p]
        L.kv_cluster_export_csr.argtypes = [p, p, p, p]
        L.kv_cluster_pack.argtypes = [p, p, p, p]
        L.kv_dense_decode_workspace_bytes.argtypes = [i, i, i, i]
        L.kv_dense_decode_workspace_bytes.restype = sz
        L.kv_dense_decode.argtypes = [p, i, p, p, i, i, i, i, i, f, p, p, sz, p]
        L.kv_cluster_debug_assign.argtypes = [p, p, i, p, p, p, p, p, sz, p]
        L.kv_cluster_debug_update.argtypes = [p, p, i, p, sz, p]
        L.kv_cluster_cache_reset.argtypes = [p, p, p]
        L.kv_cluster_cache_workspace_bytes.argtypes = [i, i, i, i]
        L.kv_cluster_cache_workspace_bytes.restype = sz
        L.kv_cluster_cached_select_decode.argtypes = [p, p, p, i, p, p, f, p, p, p, p, sz, p]
        L.kv_cluster_status_string.argtypes = [i]
        L.kv_cluster_status_string.restype = C.c_char_p
        for name in ("kv_cluster_index_init", "kv_cluster_init_positions", "kv_cluster_build_from",
                     "kv_cluster_debug_scores", "kv_cluster_build", "kv_cluster_build_timed", "kv_cluster_append", "kv_cluster_append_window",
                     "kv_cluster_cluster_window", "kv_cluster_select", "kv_sparse_decode", "kv_sparse_decode_noalloc",
                     "kv_cluster_select_decode",
                     "kv_cluster_export_csr", "kv_cluster_pack", "kv_dense_decode", "kv_cluster_debug_assign",
                     "kv_cluster_debug_update", "kv_cluster_cache_reset", "kv_cluster_cached_select_decode"):
            getattr(L, name).restype = i
        _lib = L
    return _lib


def build_lib() -> str:
    from ._build import build
    return build()


def status_string(status: int) -> str:
    return lib().kv_cluster_status_string(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise KvcError(status, what)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KVC_BF16
    if t == torch.float32:
        return KVC_F32
    raise TypeError(f"unsupported element type {t} (bfloat16 or float32)")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return C.c_void_p(t.data_ptr())


_hip_rt = None


def _hip():
    """The HIP runtime that torch has loaded (for host-memory pointers)."""
    global _hip_rt
    if _hip_rt is None:
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        rt = C.CDLL(path or "libamdhip64.so")
        rt.hipHostGetDevicePointer.argtypes = [C.POINTER(C.c_void_p), C.c_void_p, C.c_uint]
        rt.hipHostGetDevicePointer.restype = C.c_int
        _hip_rt = rt
    return _hip_rt


def _ptr_kv(t: torch.Tensor | None):
    """Device-visible address of a K/V array: device memory, or pinned host
    memory (``pin_memory=True``) mapped into the GPU's address space, for KV
    that lives on the host."""
    if t is None:
        return None
    if t.is_cuda:
        return _ptr(t)
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    if not t.is_pinned():
        raise ValueError("host K/V arrays must be pinned (allocate them with pin_memory=True)")
    dptr = C.c_void_p()
    rc = _hip().hipHostGetDevicePointer(C.byref(dptr), C.c_void_p(t.data_ptr()), 0)
    if rc != 0 or not dptr.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({rc})")
    return dptr


def _stream(stream) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def cpad(C_: int) -> int:
    return lib().kv_cluster_cpad(C_)


def build_workspace_bytes(heads: int, L: int, C_: int, iters: int) -> int:
    return lib().kv_cluster_build_workspace_bytes(heads, L, C_, iters)


def decode_workspace_bytes(heads: int, q_heads: int, B: int, d: int = HEAD_DIM) -> int:
    return lib().kv_sparse_decode_workspace_bytes(heads, q_heads, d, B)


class ClusterIndex:
    """Device memory of one cluster index (``kvc_index``), allocated with torch."""

    def __init__(self, heads: int, C_: int, capacity: int, dtype: torch.dtype = torch.bfloat16,
                 d: int = HEAD_DIM, device="cuda", packed: bool = False, n_sink: int = 0, c_slots: int = 0,
                 metric: int = COSINE, packed_on_host: bool = False):
        """packed: also allocate the cluster-ordered copies of the keys and
        values (``kv_cluster_pack``), two more arrays of the caches' size.
        n_sink: attention sinks, kept out of the clustering and always
        selected first. c_slots: cluster slots per head (>= C; 0 for C), room
        for the clusters that ``cluster_window`` adds. metric: assignment
        distance, COSINE (the method's), L2 or INNER_PRODUCT. packed_on_host:
        the packed copies live in pinned host memory (offloaded KV)."""
        self.heads, self.C, self.capacity, self.d, self.dtype = heads, C_, capacity, d, dtype
        S = c_slots if c_slots else C_
        self.slots = S
        # one allocation laid out by the library (kv_cluster_index_bytes / kv_cluster_index_init)
        nbytes = lib().kv_cluster_index_bytes(heads, d, C_, capacity, _dtype_code(dtype), c_slots)
        if nbytes == 0:
            raise ValueError(f"invalid index sizes heads={heads} d={d} C={C_} capacity={capacity} c_slots={c_slots}")
        self._mem = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self._s = _Index()
        _check(lib().kv_cluster_index_init(C.byref(self._s), heads, d, C_, capacity, _dtype_code(dtype), c_slots,
                                           n_sink, metric, C.c_void_p(self._mem.data_ptr()), nbytes,
                                           _stream(None)), "kv_cluster_index_init")
        base = self._mem.data_ptr()

        def arr(ptr, t, shape):
            n = 1
            for x in shape:
                n *= x
            off = ptr - base
            return self._mem[off:off + n * torch.empty((), dtype=t).element_size()].view(t).view(shape)

        self.centroids = arr(self._s.centroids, torch.float32, (heads, S, d))
        self.centroids_op = arr(self._s.centroids_op, dtype, (heads, cpad(S), d))
        self.labels = arr(self._s.labels, torch.int32, (heads, capacity))
        self.sizes = arr(self._s.sizes, torch.int32, (heads, S))
        self.offsets = arr(self._s.offsets, torch.int32, (heads, S + 1))
        self.token_ids = arr(self._s.token_ids, torch.int32, (heads, capacity))
        self.app_offsets = arr(self._s.app_offsets, torch.int32, (heads, S + 1))
        self.app_ids = arr(self._s.app_ids, torch.int32, (heads, capacity))
        self.dev_flags = arr(self._s.dev_flags, torch.int32, (1,))
        self.centroids_t = arr(self._s.centroids_t, torch.float32, (heads, d // 4, S, 4))
        if packed and packed_on_host:
            self.k_packed = torch.empty(heads, capacity, d, dtype=dtype, pin_memory=True)
            self.v_packed = torch.empty(heads, capacity, d, dtype=dtype, pin_memory=True)
        elif packed:
            self.k_packed = torch.empty(heads, capacity, d, dtype=dtype, device=device)
            self.v_packed = torch.empty(heads, capacity, d, dtype=dtype, device=device)
        else:
            self.k_packed = self.v_packed = None
        if packed:
            self._s.k_packed = _ptr_kv(self.k_packed).value
            self._s.v_packed = _ptr_kv(self.v_packed).value
        self.metric = metric
        self.n_sink = n_sink

    @property
    def n_build(self) -> int:
        return self._s.n_build

    @property
    def n_tokens(self) -> int:
        return self._s.n_tokens

    @property
    def c_active(self) -> int:
        return self._s.c_active

    @property
    def window_start(self) -> int:
        return self._s.window_start

    def ref(self):
        return C.byref(self._s)


def _cache_check(idx: ClusterIndex, t: torch.Tensor, name: str):
    if t.dtype != idx.dtype or tuple(t.shape) != (idx.heads, idx.capacity, idx.d):
        raise ValueError(f"{name} must be {idx.dtype} [{idx.heads}, {idx.capacity}, {idx.d}], got "
                         f"{t.dtype} {list(t.shape)}")


def init_positions(heads: int, L: int, C_: int, seed: int, n_sink: int = 0, device="cuda", stream=None):
    """kv_cluster_init_positions: the seeded initial centroid positions, int32 [heads, C]."""
    out = torch.empty(heads, C_, dtype=torch.int32, device=device)
    _check(lib().kv_cluster_init_positions(heads, n_sink, L, C_, seed & ((1 << 64) - 1), _ptr(out),
                                           _stream(stream)), "kv_cluster_init_positions")
    return out


def build(idx: ClusterIndex, keys: torch.Tensor, L: int, iters: int, seed: int | None = None,
          init_idx: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
          assign_events=None):
    """kv_cluster_build: cluster the first L rows of keys [heads, capacity, d],
    from the seeded initial positions (seed) or from init_idx int32 [heads, C]
    (kv_cluster_build_from).

    assign_events: optional ctypes array of 2*iters hipEvent_t handles
    (kv_cluster_build_timed) recorded around each assignment kernel."""
    _cache_check(idx, keys, "keys")
    if (seed is None) == (init_idx is None):
        raise ValueError("build takes exactly one of seed and init_idx")
    if init_idx is not None and (init_idx.dtype != torch.int32 or tuple(init_idx.shape) != (idx.heads, idx.C)):
        raise ValueError("init_idx must be int32 [heads, C]")
    need = build_workspace_bytes(idx.heads, L, idx.C, iters)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=keys.device)
    seed = 0 if seed is None else seed & ((1 << 64) - 1)
    if assign_events is not None:
        if len(assign_events) < 2 * iters:
            raise ValueError("assign_events needs 2 * iters handles")
        _check(lib().kv_cluster_build_timed(idx.ref(), _ptr(keys), L, iters, seed, _ptr(init_idx),
                                            _ptr(workspace), workspace.numel(), assign_events, _stream(stream)),
               "kv_cluster_build_timed")
    elif init_idx is None:
        _check(lib().kv_cluster_build(idx.ref(), _ptr(keys), L, iters, seed, _ptr(workspace), workspace.numel(),
                                      _stream(stream)), "kv_cluster_build")
    else:
        _check(lib().kv_cluster_build_from(idx.ref(), _ptr(keys), L, iters, _ptr(init_idx), _ptr(workspace),
                                           workspace.numel(), _stream(stream)), "kv_cluster_build_from")
    return workspace


def debug_scores(idx: ClusterIndex, q: torch.Tensor, stream=None) -> torch.Tensor:
    """kv_cluster_debug_scores: the fp64 selection scores [heads, c_active] of q [q_heads, d]."""
    if q.dtype != idx.dtype or q.dim() != 2 or q.shape[1] != idx.d:
        raise ValueError(f"q must be {idx.dtype} [q_heads, {idx.d}]")
    out = torch.empty(idx.heads, max(idx.c_active, 1), dtype=torch.float64, device=q.device)
    _check(lib().kv_cluster_debug_scores(idx.ref(), _ptr(q), q.shape[0], _ptr(out), _stream(stream)),
           "kv_cluster_debug_scores")
    return out


def append(idx: ClusterIndex, k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
           v_new: torch.Tensor, stream=None):
    """kv_cluster_append: k_new, v_new [heads, n_new, d]."""
    _cache_check(idx, k_cache, "k_cache")
    _cache_check(idx, v_cache, "v_cache")
    k_new, v_new, n_new = _new_rows(idx, k_new, v_new)
    _check(lib().kv_cluster_append(idx.ref(), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), n_new,
                                   _stream(stream)), "kv_cluster_append")


def _new_rows(idx: ClusterIndex, k_new: torch.Tensor, v_new: torch.Tensor):
    if k_new.dim() == 2:
        k_new, v_new = k_new.unsqueeze(1), v_new.unsqueeze(1)
    n_new = k_new.shape[1]
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        if t.dtype != idx.dtype or tuple(t.shape) != (idx.heads, n_new, idx.d):
            raise ValueError(f"{nm} must be {idx.dtype} [{idx.heads}, n_new, {idx.d}]")
    return k_new, v_new, n_new


def append_window(idx: ClusterIndex, k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                  v_new: torch.Tensor, stream=None):
    """kv_cluster_append_window: k_new, v_new [heads, n_new, d] join the window
    of generated tokens (recalled whole until cluster_window)."""
    _cache_check(idx, k_cache, "k_cache")
    _cache_check(idx, v_cache, "v_cache")
    k_new, v_new, n_new = _new_rows(idx, k_new, v_new)
    _check(lib().kv_cluster_append_window(idx.ref(), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), n_new,
                                          _stream(stream)), "kv_cluster_append_window")


def window_workspace_bytes(heads: int, m: int, n_clusters: int, iters: int) -> int:
    return lib().kv_cluster_window_workspace_bytes(heads, m, n_clusters, iters)


def cluster_window(idx: ClusterIndex, k_cache: torch.Tensor, v_cache: torch.Tensor, n_clusters: int, iters: int,
                   init_idx: torch.Tensor, workspace: torch.Tensor | None = None, stream=None):
    """kv_cluster_cluster_window: the window's tokens become n_clusters new
    clusters; init_idx int32 [heads, n_clusters] holds token positions in the
    window."""
    _cache_check(idx, k_cache, "k_cache")
    _cache_check(idx, v_cache, "v_cache")
    if init_idx.dtype != torch.int32 or tuple(init_idx.shape) != (idx.heads, n_clusters):
        raise ValueError("init_idx must be int32 [heads, n_clusters]")
    m = idx.n_tokens - idx.window_start
    need = window_workspace_bytes(idx.heads, max(m, 1), max(n_clusters, 1), max(iters, 1))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=k_cache.device)
    _check(lib().kv_cluster_cluster_window(idx.ref(), _ptr(k_cache), _ptr(v_cache), n_clusters, iters,
                                           _ptr(init_idx), _ptr(workspace), workspace.numel(), _stream(stream)),
           "kv_cluster_cluster_window")
    return workspace


def select(idx: ClusterIndex, q: torch.Tensor, B: int, sel_ids: torch.Tensor | None = None,
           sel_count: torch.Tensor | None = None, stream=None):
    """kv_cluster_select: q [q_heads, d] -> (sel_ids [heads, B], sel_count [heads])."""
    if q.dtype != idx.dtype or q.dim() != 2 or q.shape[1] != idx.d:
        raise ValueError(f"q must be {idx.dtype} [q_heads, {idx.d}]")
    if sel_ids is None:
        sel_ids = torch.empty(idx.heads, B, dtype=torch.int32, device=q.device)
    if sel_count is None:
        sel_count = torch.empty(idx.heads, dtype=torch.int32, device=q.device)
    if sel_ids.dtype != torch.int32 or tuple(sel_ids.shape) != (idx.heads, B) or sel_count.numel() != idx.heads:
        raise ValueError("sel_ids must be int32 [heads, B], sel_count int32 [heads]")
    _check(lib().kv_cluster_select(idx.ref(), _ptr(q), q.shape[0], B, _ptr(sel_ids), _ptr(sel_count),
                                   _stream(stream)), "kv_cluster_select")
    return sel_ids, sel_count


def sparse_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, sel_ids: torch.Tensor,
                  sel_count: torch.Tensor, scale: float, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None):
    """kv_sparse_decode: attention of q [q_heads, d] over the selected rows -> fp32 [q_heads, d]."""
    heads, capacity, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q, k_cache and v_cache must share a type; k and v caches a shape")
    B = sel_ids.shape[1]
    if sel_ids.dtype != torch.int32 or sel_ids.shape[0] != heads or sel_count.numel() != heads:
        raise ValueError("sel_ids must be int32 [heads, B], sel_count int32 [heads]")
    if out is None:
        out = torch.empty(q.shape[0], d, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(decode_workspace_bytes(heads, q.shape[0], B, d), 1), dtype=torch.uint8,
                                device=q.device)
    _check(lib().kv_sparse_decode(_ptr(q), q.shape[0], _ptr(k_cache), _ptr(v_cache), _dtype_code(q.dtype), heads,
                                  capacity, d, _ptr(sel_ids), _ptr(sel_count), B, float(scale), _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream(stream)), "kv_sparse_decode")
    return out


def sparse_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, sel_ids: torch.Tensor,
                          sel_count: torch.Tensor, scale: float, out: torch.Tensor | None = None, stream=None):
    """kv_sparse_decode_noalloc: kv_sparse_decode with the partial results in
    the library's fixed device scratch (no workspace) -> fp32 [q_heads, d]."""
    heads, capacity, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q, k_cache and v_cache must share a type; k and v caches a shape")
    B = sel_ids.shape[1]
    if sel_ids.dtype != torch.int32 or sel_ids.shape[0] != heads or sel_count.numel() != heads:
        raise ValueError("sel_ids must be int32 [heads, B], sel_count int32 [heads]")
    if out is None:
        out = torch.empty(q.shape[0], d, dtype=torch.float32, device=q.device)
    _check(lib().kv_sparse_decode_noalloc(_ptr(q), q.shape[0], _ptr(k_cache), _ptr(v_cache), _dtype_code(q.dtype),
                                          heads, capacity, d, _ptr(sel_ids), _ptr(sel_count), B, float(scale),
                                          _ptr(out), _stream(stream)), "kv_sparse_decode_noalloc")
    return out


def select_decode_workspace_bytes(heads: int, q_heads: int, d: int = HEAD_DIM) -> int:
    return int(lib().kv_cluster_select_decode_workspace_bytes(heads, q_heads, d))


def select_decode(idx: ClusterIndex, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, B: int,
                  scale: float, out: torch.Tensor | None = None, sel_ids: torch.Tensor | None = None,
                  sel_count: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """kv_cluster_select_decode: selection and sparse attention -> fp32 [q_heads, d]. Without a workspace
    one kernel; with one (select_decode_workspace_bytes, its arrival counters zero before the first call), the
    blocks of a head split the tokens and the last of them merges their partial results."""
    _cache_check(idx, k_cache, "k_cache")
    _cache_check(idx, v_cache, "v_cache")
    if q.dtype != idx.dtype or q.dim() != 2 or q.shape[1] != idx.d:
        raise ValueError(f"q must be {idx.dtype} [q_heads, {idx.d}]")
    if out is None:
        out = torch.empty(q.shape[0], idx.d, dtype=torch.float32, device=q.device)
    if sel_ids is not None and (sel_ids.dtype != torch.int32 or tuple(sel_ids.shape) != (idx.heads, B)):
        raise ValueError("sel_ids must be int32 [heads, B]")
    if sel_count is not None and (sel_count.dtype != torch.int32 or sel_count.numel() != idx.heads):
        raise ValueError("sel_count must be int32 [heads]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kv_cluster_select_decode(idx.ref(), _ptr(q), q.shape[0], _ptr_kv(k_cache), _ptr_kv(v_cache), B,
                                          float(scale), _ptr(out), _ptr(sel_ids), _ptr(sel_count), _ptr(workspace),
                                          ws_bytes, _stream(stream)),
           "kv_cluster_select_decode")
    return out


def pack(idx: ClusterIndex, k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None):
    """kv_cluster_pack: cluster-ordered copies of the built tokens' rows (the
    index must have been created with packed=True)."""
    _cache_check(idx, k_cache, "k_cache")
    _cache_check(idx, v_cache, "v_cache")
    if idx.k_packed is None:
        raise ValueError("the index has no packed arrays (create it with packed=True)")
    _check(lib().kv_cluster_pack(idx.ref(), _ptr_kv(k_cache), _ptr_kv(v_cache), _stream(stream)), "kv_cluster_pack")


class ClusterCache:
    """Device memory of a cluster cache (``kvc_cluster_cache``) for one index:
    the rows of the last R + 1 steps, the per-cluster table and counters."""

    def __init__(self, idx: ClusterIndex, R: int, B: int, device="cuda"):
        self.R, self.B = R, B
        self.k = torch.empty(idx.heads, (R + 1) * B, idx.d, dtype=idx.dtype, device=device)
        self.v = torch.empty_like(self.k)
        self.table = torch.empty(idx.heads, idx.slots, 3, dtype=torch.int32, device=device)
        self.stats = torch.zeros(idx.heads, 4, dtype=torch.int64, device=device)
        self._s = _Cache(R, B, 0, 0, self.k.data_ptr(), self.v.data_ptr(), self.table.data_ptr(),
                         self.stats.data_ptr())

    @property
    def step(self) -> int:
        return self._s.step

    def ref(self):
        return C.byref(self._s)

    def hit_rates(self) -> dict:
        """Cluster and token hit rates accumulated since the last reset."""
        s = self.stats.sum(dim=0).tolist()
        return {"clusters": s[0], "cluster_hits": s[1], "tokens": s[2], "token_hits": s[3],
                "cluster_hit_rate": s[1] / max(s[0], 1), "token_hit_rate": s[3] / max(s[2], 1)}


def cache_reset(idx: ClusterIndex, cache: ClusterCache, stream=None):
    """kv_cluster_cache_reset."""
    _check(lib().kv_cluster_cache_reset(idx.ref(), cache.ref(), _stream(stream)), "kv_cluster_cache_reset")


def cache_workspace_bytes(heads: int, q_heads: int, B: int, d: int = HEAD_DIM) -> int:
    return lib().kv_cluster_cache_workspace_bytes(heads, q_heads, d, B)


def cached_select_decode(idx: ClusterIndex, cache: ClusterCache, q: torch.Tensor, k_cache: torch.Tensor,
                         v_cache: torch.Tensor, scale: float, out: torch.Tensor | None = None,
                         sel_ids: torch.Tensor | None = None, sel_count: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None):
    """kv_cluster_cached_select_decode: selection through the cluster cache and
    attention over the assembled rows -> fp32 [q_heads, d]. k_cache, v_cache
    may be pinned host tensors (offloaded KV)."""
    _cache_check(idx, k_cache, "k_cache")
    _cache_check(idx, v_cache, "v_cache")
    if q.dtype != idx.dtype or q.dim() != 2 or q.shape[1] != idx.d:
        raise ValueError(f"q must be {idx.dtype} [q_heads, {idx.d}]")
    if out is None:
        out = torch.empty(q.shape[0], idx.d, dtype=torch.float32, device=q.device)
    if sel_ids is not None and (sel_ids.dtype != torch.int32 or tuple(sel_ids.shape) != (idx.heads, cache.B)):
        raise ValueError("sel_ids must be int32 [heads, B]")
    if sel_count is not None and (sel_count.dtype != torch.int32 or sel_count.numel() != idx.heads):
        raise ValueError("sel_count must be int32 [heads]")
    if workspace is None:
        workspace = torch.empty(max(cache_workspace_bytes(idx.heads, q.shape[0], cache.B, idx.d), 1),
                                dtype=torch.uint8, device=q.device)
    _check(lib().kv_cluster_cached_select_decode(idx.ref(), cache.ref(), _ptr(q), q.shape[0], _ptr_kv(k_cache),
                                                 _ptr_kv(v_cache), float(scale), _ptr(out), _ptr(sel_ids),
                                                 _ptr(sel_count), _ptr(workspace), workspace.numel(),
                                                 _stream(stream)), "kv_cluster_cached_select_decode")
    return out


def dense_decode_workspace_bytes(heads: int, q_heads: int, n: int, d: int = HEAD_DIM) -> int:
    return lib().kv_dense_decode_workspace_bytes(heads, q_heads, d, n)


def dense_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, n: int, scale: float,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """kv_dense_decode: full attention of q [q_heads, d] over the first n rows -> fp32 [q_heads, d]."""
    heads, capacity, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q, k_cache and v_cache must share a type; k and v caches a shape")
    if out is None:
        out = torch.empty(q.shape[0], d, dtype=torch.float32, device=q.device)
    need = dense_decode_workspace_bytes(heads, q.shape[0], n, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().kv_dense_decode(_ptr(q), q.shape[0], _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache.dtype), heads,
                                 capacity, d, n, scale, _ptr(out), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "kv_dense_decode")
    return out


def export_csr(idx: ClusterIndex, stream=None):
    """Canonical index (main + appended parts): (offsets [heads, slots+1], token_ids [heads, capacity])."""
    off = torch.empty(idx.heads, idx.slots + 1, dtype=torch.int32, device=idx.labels.device)
    ids = torch.full((idx.heads, idx.capacity), -1, dtype=torch.int32, device=idx.labels.device)
    _check(lib().kv_cluster_export_csr(idx.ref(), _ptr(off), _ptr(ids), _stream(stream)), "kv_cluster_export_csr")
    return off, ids


def debug_assign(idx: ClusterIndex, keys: torch.Tensor, L: int, chat: torch.Tensor, want_top2: bool = False,
                 stream=None):
    """One assignment under the operand chat [heads, cpad(C), d] -> (labels, top2, flagged per head)."""
    _cache_check(idx, keys, "keys")
    if chat.dtype != idx.dtype or tuple(chat.shape) != (idx.heads, cpad(idx.C), idx.d):
        raise ValueError("chat must match centroids_op")
    labels = torch.full((idx.heads, idx.capacity), -1, dtype=torch.int32, device=keys.device)
    top2 = torch.empty(idx.heads, L, 2, dtype=torch.float32, device=keys.device) if want_top2 else None
    flagged = torch.zeros(idx.heads, dtype=torch.int32, device=keys.device)
    ws = torch.empty(max(build_workspace_bytes(idx.heads, L, idx.C, 1), 1), dtype=torch.uint8, device=keys.device)
    _check(lib().kv_cluster_debug_assign(idx.ref(), _ptr(keys), L, _ptr(chat), _ptr(labels), _ptr(top2),
                                         _ptr(flagged), _ptr(ws), ws.numel(), _stream(stream)),
           "kv_cluster_debug_assign")
    return labels, top2, flagged


def debug_update(idx: ClusterIndex, keys: torch.Tensor, L: int, stream=None):
    """Index arrays and centroid update from idx.labels (first L tokens)."""
    _cache_check(idx, keys, "keys")
    ws = torch.empty(max(build_workspace_bytes(idx.heads, L, idx.C, 1), 1), dtype=torch.uint8, device=keys.device)
    _check(lib().kv_cluster_debug_update(idx.ref(), _ptr(keys), L, _ptr(ws), ws.numel(), _stream(stream)),
           "kv_cluster_debug_update")
