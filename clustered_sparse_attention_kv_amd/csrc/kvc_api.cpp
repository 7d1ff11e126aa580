// C ABI of kvcluster: argument checks (before anything is enqueued),
// workspace carving and launch sequencing on the caller's stream. The library
// allocates nothing and never synchronises.
#include "kvcluster.h"

#include <hip/hip_runtime.h>

#include "kvc_internal.h"

using namespace kvc;

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// cluster slots per head: the stride of every per-cluster array
int slots(const kvc_index* idx) { return idx->c_slots ? idx->c_slots : idx->C; }

bool index_ok(const kvc_index* idx) {
  return idx && idx->centroids && idx->centroids_op && idx->labels && idx->sizes && idx->offsets && idx->token_ids &&
         idx->app_offsets && idx->app_ids && idx->dev_flags && idx->centroids_t && idx->heads >= 1 &&
         idx->capacity >= 1 && idx->C >= 1 && (idx->dtype == KVC_F32 || idx->dtype == KVC_BF16) &&
         idx->n_sink >= 0 && (idx->c_slots == 0 || idx->c_slots >= idx->C) && idx->metric >= KVC_COSINE &&
         idx->metric <= KVC_INNER_PRODUCT;
}

kvc_status index_support(const kvc_index* idx) {
  if (idx->d != KVC_HEAD_DIM || idx->C > KVC_MAX_C || slots(idx) > KVC_MAX_C) return KVC_ERR_UNSUPPORTED;
  if ((long long)idx->heads * idx->capacity >= (1ll << 31)) return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}

// the host mirrors of a built index are consistent
bool built_ok(const kvc_index* idx) {
  return idx->n_build >= 1 && idx->c_active >= 1 && idx->c_active <= slots(idx) && idx->n_sink <= idx->n_build &&
         idx->window_start >= idx->n_build && idx->window_start <= idx->n_tokens && idx->n_tokens <= idx->capacity;
}

// the index as the selection kernels read it
IndexView view(const kvc_index* idx) {
  IndexView x{};
  x.cent_t = idx->centroids_t;
  x.sizes = idx->sizes;
  x.offsets = idx->offsets;
  x.token_ids = idx->token_ids;
  x.app_offsets = idx->app_offsets;
  x.app_ids = idx->app_ids;
  x.cap = idx->capacity;
  x.cs = slots(idx);
  x.ca = idx->c_active;
  x.n_sink = idx->n_sink;
  x.wlo = idx->window_start;
  x.nw = idx->n_tokens - idx->window_start;
  return x;
}

struct BuildWs {
  int32_t* init;     // [heads, C]: initial centroid positions drawn from the seed
  uint32_t* qcount;  // [iters, heads]
  int32_t* queue;    // [heads, L]
  int32_t* hist;     // [heads, nblk, C]
  void* op_t;        // [heads, d / 8, cpad(C)] 16-byte chunks: the bf16 operand chunk-major
  int32_t* dirty;    // [iters, heads, C]: clusters a key entered or left in that iteration
  float* norm2;      // [heads, L]: each key's squared norm, from the first iteration on
  size_t bytes;
};

BuildWs carve_build(void* base, int heads, int L, int C, int iters) {
  BuildWs w{};
  size_t o = 0;
  char* b = static_cast<char*>(base);
  w.init = reinterpret_cast<int32_t*>(b + o);
  o = align_up(o + sizeof(int32_t) * (size_t)heads * C);
  w.qcount = reinterpret_cast<uint32_t*>(b + o);
  o = align_up(o + sizeof(uint32_t) * (size_t)iters * heads);
  w.queue = reinterpret_cast<int32_t*>(b + o);
  o = align_up(o + sizeof(int32_t) * (size_t)heads * L);
  w.hist = reinterpret_cast<int32_t*>(b + o);
  o = align_up(o + sizeof(int32_t) * (size_t)heads * csr_blocks(L) * C);
  w.op_t = b + o;
  o = align_up(o + sizeof(uint16_t) * (size_t)heads * kv_cluster_cpad(C) * KVC_HEAD_DIM);
  w.dirty = reinterpret_cast<int32_t*>(b + o);
  o = align_up(o + sizeof(int32_t) * (size_t)iters * heads * C);
  w.norm2 = reinterpret_cast<float*>(b + o);
  o = align_up(o + sizeof(float) * (size_t)heads * L);
  w.bytes = o;
  return w;
}

// Workspace of the window clustering: the build's scratch for m keys and nc
// clusters, then the window's own clustering (nc clusters with strides nc and
// cpad(nc), m tokens).
struct WindowWs {
  BuildWs b;
  float *cent, *cent_t;
  void* chat;
  int32_t *labels, *sizes, *offsets, *ids;
  size_t bytes;
};

WindowWs carve_window(void* base, int heads, int m, int nc, int iters) {
  WindowWs w{};
  w.b = carve_build(base, heads, m, nc, iters);
  size_t o = w.b.bytes;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* p = b + o;
    o = align_up(o + bytes);
    return p;
  };
  w.cent = reinterpret_cast<float*>(take(sizeof(float) * (size_t)heads * nc * KVC_HEAD_DIM));
  w.cent_t = reinterpret_cast<float*>(take(sizeof(float) * (size_t)heads * nc * KVC_HEAD_DIM));
  w.chat = take(sizeof(float) * (size_t)heads * kv_cluster_cpad(nc) * KVC_HEAD_DIM);
  w.labels = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)heads * m));
  w.sizes = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)heads * nc));
  w.offsets = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)heads * (nc + 1)));
  w.ids = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)heads * m));
  w.bytes = o;
  return w;
}

size_t elem_bytes(int dtype) { return dtype == KVC_BF16 ? 2 : 4; }

kvc_status status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_HIP; }

}  // namespace

extern "C" {

int kv_cluster_cpad(int C) { return C < 1 ? 0 : (C + 31) / 32 * 32; }

namespace {
// The arrays of one index in one allocation (256-byte aligned each).
struct IndexLayout {
  size_t centroids, centroids_op, labels, sizes, offsets, token_ids, app_offsets, app_ids, dev_flags, centroids_t,
      bytes;
};
IndexLayout index_layout(int heads, int d, int C, int capacity, int dtype, int c_slots) {
  IndexLayout l{};
  const size_t H = (size_t)heads, S = (size_t)(c_slots ? c_slots : C), cap = (size_t)capacity;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  l.centroids = take(sizeof(float) * H * S * d);
  l.centroids_op = take(elem_bytes(dtype) * H * (size_t)kv_cluster_cpad((int)S) * d);
  l.labels = take(sizeof(int32_t) * H * cap);
  l.sizes = take(sizeof(int32_t) * H * S);
  l.offsets = take(sizeof(int32_t) * H * (S + 1));
  l.token_ids = take(sizeof(int32_t) * H * cap);
  l.app_offsets = take(sizeof(int32_t) * H * (S + 1));
  l.app_ids = take(sizeof(int32_t) * H * cap);
  l.dev_flags = take(sizeof(int32_t));
  l.centroids_t = take(sizeof(float) * H * S * d);
  l.bytes = o;
  return l;
}
bool index_sizes_ok(int heads, int d, int C, int capacity, int dtype, int c_slots) {
  return heads >= 1 && d == KVC_HEAD_DIM && C >= 1 && C <= KVC_MAX_C && capacity >= 1 &&
         (dtype == KVC_F32 || dtype == KVC_BF16) && (c_slots == 0 || (c_slots >= C && c_slots <= KVC_MAX_C)) &&
         (long long)heads * capacity < (1ll << 31);
}
}  // namespace

size_t kv_cluster_index_bytes(int heads, int d, int C, int capacity, kvc_dtype dtype, int c_slots) {
  if (!index_sizes_ok(heads, d, C, capacity, dtype, c_slots)) return 0;
  return index_layout(heads, d, C, capacity, dtype, c_slots).bytes;
}

kvc_status kv_cluster_index_init(kvc_index* idx, int heads, int d, int C, int capacity, kvc_dtype dtype, int c_slots,
                                 int n_sink, kvc_metric metric, void* mem, size_t mem_bytes, void* stream) {
  if (!idx || !mem || n_sink < 0 || metric < KVC_COSINE || metric > KVC_INNER_PRODUCT) return KVC_ERR_INVALID_ARG;
  if (heads >= 1 && C >= 1 && capacity >= 1 && (d != KVC_HEAD_DIM || C > KVC_MAX_C || c_slots > KVC_MAX_C))
    return KVC_ERR_UNSUPPORTED;
  if (!index_sizes_ok(heads, d, C, capacity, dtype, c_slots)) return KVC_ERR_INVALID_ARG;
  const IndexLayout l = index_layout(heads, d, C, capacity, dtype, c_slots);
  if (mem_bytes < l.bytes) return KVC_ERR_WORKSPACE;
  char* b = static_cast<char*>(mem);
  kvc_index x{};
  x.heads = heads;
  x.d = d;
  x.C = C;
  x.capacity = capacity;
  x.dtype = dtype;
  x.centroids = reinterpret_cast<float*>(b + l.centroids);
  x.centroids_op = b + l.centroids_op;
  x.labels = reinterpret_cast<int32_t*>(b + l.labels);
  x.sizes = reinterpret_cast<int32_t*>(b + l.sizes);
  x.offsets = reinterpret_cast<int32_t*>(b + l.offsets);
  x.token_ids = reinterpret_cast<int32_t*>(b + l.token_ids);
  x.app_offsets = reinterpret_cast<int32_t*>(b + l.app_offsets);
  x.app_ids = reinterpret_cast<int32_t*>(b + l.app_ids);
  x.dev_flags = reinterpret_cast<int32_t*>(b + l.dev_flags);
  x.centroids_t = reinterpret_cast<float*>(b + l.centroids_t);
  x.n_sink = n_sink;
  x.c_slots = c_slots;
  x.metric = metric;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t cap = (size_t)heads * capacity;
  hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(b), l.bytes / sizeof(int32_t), 0, st);
  if (e == hipSuccess) e = launch_fill_i32(x.labels, cap, -1, st);
  if (e == hipSuccess) e = launch_fill_i32(x.token_ids, cap, -1, st);
  if (e == hipSuccess) e = launch_fill_i32(x.app_ids, cap, -1, st);
  if (e != hipSuccess) return KVC_ERR_HIP;
  *idx = x;
  return KVC_OK;
}

size_t kv_cluster_build_workspace_bytes(int heads, int L, int C, int iters) {
  if (heads < 1 || L < 1 || C < 1 || iters < 1) return 0;
  return carve_build(nullptr, heads, L, C, iters).bytes;
}

kvc_status kv_cluster_build(kvc_index* idx, const void* keys, int L, int iters, uint64_t seed, void* ws,
                            size_t ws_bytes, void* stream) {
  return kv_cluster_build_timed(idx, keys, L, iters, seed, nullptr, ws, ws_bytes, nullptr, stream);
}

kvc_status kv_cluster_build_from(kvc_index* idx, const void* keys, int L, int iters, const int32_t* init_idx,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!init_idx) return KVC_ERR_INVALID_ARG;
  return kv_cluster_build_timed(idx, keys, L, iters, 0, init_idx, ws, ws_bytes, nullptr, stream);
}

kvc_status kv_cluster_init_positions(int heads, int n_sink, int L, int C, uint64_t seed, int32_t* out,
                                     void* stream) {
  if (!out || heads < 1 || n_sink < 0 || C < 1 || L < 1 || (long long)L - n_sink < C) return KVC_ERR_INVALID_ARG;
  if (C > KVC_MAX_C) return KVC_ERR_UNSUPPORTED;
  return status(launch_init_positions(heads, n_sink, L, C, seed, out, static_cast<hipStream_t>(stream)));
}

kvc_status kv_cluster_build_timed(kvc_index* idx, const void* keys, int L, int iters, uint64_t seed,
                                  const int32_t* init_idx, void* ws, size_t ws_bytes, void* const* assign_events,
                                  void* stream) {
  if (!index_ok(idx) || !keys || !ws) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  const int H = idx->heads, C = idx->C, cap = idx->capacity, cpad = kv_cluster_cpad(C);
  const int cs = slots(idx), cps = kv_cluster_cpad(cs);
  const int ns = idx->n_sink;
  if (ns < 0 || L - ns < C || L > cap || iters < 1 || iters > 100000) return KVC_ERR_INVALID_ARG;
  // the clustered rows: [ns, L); their labels start at labels + ns, and the
  // index stores their absolute positions
  const int Lc = L - ns;
  const void* keys_c = static_cast<const char*>(keys) + (size_t)ns * KVC_HEAD_DIM * elem_bytes(idx->dtype);
  const BuildWs w = carve_build(ws, H, Lc, C, iters);
  if (ws_bytes < w.bytes) return KVC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long hs = (long long)cap * KVC_HEAD_DIM;
  idx->packed = 0;  // the index changes: any packed copy is stale
  hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(w.qcount), (size_t)iters * H, 0, st);
  if (e == hipSuccess) e = launch_fill_i32(w.dirty, (size_t)iters * H * C, 0, st);
  if (e == hipSuccess) e = launch_fill_i32(idx->app_offsets, (size_t)H * (cs + 1), 0, st);
  if (e == hipSuccess) e = launch_fill2d_i32(idx->labels, H, cap, ns, -1, st);  // sinks: in no cluster
  // without explicit positions, the seeded shuffle draws them into the workspace
  if (e == hipSuccess && !init_idx) {
    e = launch_init_positions(H, ns, L, C, seed, w.init, st);
    init_idx = w.init;
  }
  if (e == hipSuccess)
    e = launch_init_centroids(idx->dtype, keys, hs, H, ns, L, init_idx, C, cpad, cs, cps, idx->metric, idx->centroids,
                              idx->centroids_t, idx->centroids_op, idx->dev_flags, st);
  for (int t = 0; t < iters && e == hipSuccess; ++t) {
    hipEvent_t* ev = assign_events ? (hipEvent_t*)assign_events + 2 * t : nullptr;
    // from the second iteration on, the assignment marks the clusters keys
    // entered or left and the update recomputes only those
    int32_t* dirty = t == 0 ? nullptr : w.dirty + (size_t)t * H * C;
    // the keys' norms (for the certificate) are computed once and kept
    e = launch_assign(idx->dtype, keys_c, hs, H, Lc, idx->centroids_op, C, cpad, cps, idx->metric, idx->labels + ns,
                      cap, w.queue, w.qcount + (size_t)t * H, w.op_t, dirty, w.norm2, t == 0 ? 1 : 2, nullptr, ev,
                      st);
    if (e == hipSuccess)
      e = launch_csr(idx->labels + ns, cap, H, Lc, C, cs, w.hist, idx->sizes, idx->offsets, idx->token_ids, cap, ns,
                     st);
    if (e == hipSuccess)
      e = launch_update(idx->dtype, keys, hs, H, C, cs, cps, idx->metric, idx->sizes, idx->offsets, idx->token_ids,
                        cap, idx->centroids, idx->centroids_t, idx->centroids_op, dirty, st);
  }
  if (e != hipSuccess) return KVC_ERR_HIP;
  idx->n_build = L;
  idx->n_tokens = L;
  idx->window_start = L;
  idx->c_active = C;
  return KVC_OK;
}

kvc_status kv_cluster_debug_assign(const kvc_index* idx, const void* keys, int L, const void* chat, int32_t* labels,
                            float* top2, int32_t* flagged, void* ws, size_t ws_bytes, void* stream) {
  if (!index_ok(idx) || !keys || !chat || !labels || !ws) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  const int H = idx->heads, C = idx->C, cap = idx->capacity, cpad = kv_cluster_cpad(C);
  if (L < 1 || L > cap) return KVC_ERR_INVALID_ARG;
  const BuildWs w = carve_build(ws, H, L, C, 1);
  if (ws_bytes < w.bytes) return KVC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(w.qcount), (size_t)H, 0, st);
  if (e == hipSuccess)
    e = launch_assign(idx->dtype, keys, (long long)cap * KVC_HEAD_DIM, H, L, chat, C, cpad, cpad, idx->metric, labels,
                      cap, w.queue, w.qcount, w.op_t, nullptr, nullptr, 0, top2, nullptr, st);
  if (e == hipSuccess && flagged)
    e = hipMemcpyAsync(flagged, w.qcount, sizeof(int32_t) * H, hipMemcpyDeviceToDevice, st);
  return status(e);
}

kvc_status kv_cluster_debug_scores(const kvc_index* idx, const void* q, int q_heads, double* scores, void* stream) {
  if (!index_ok(idx) || !q || !scores || q_heads < 1) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx) || q_heads % idx->heads != 0) return KVC_ERR_INVALID_ARG;
  const int G = q_heads / idx->heads;
  if (G > KVC_MAX_G) return KVC_ERR_UNSUPPORTED;
  return status(launch_debug_scores(idx->dtype, q, G, view(idx), idx->heads, scores, static_cast<hipStream_t>(stream)));
}

kvc_status kv_cluster_debug_update(kvc_index* idx, const void* keys, int L, void* ws, size_t ws_bytes, void* stream) {
  if (!index_ok(idx) || !keys || !ws || idx->n_sink != 0) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  const int H = idx->heads, C = idx->C, cap = idx->capacity;
  const int cs = slots(idx), cps = kv_cluster_cpad(cs);
  if (L < 1 || L > cap) return KVC_ERR_INVALID_ARG;
  const BuildWs w = carve_build(ws, H, L, C, 1);
  if (ws_bytes < w.bytes) return KVC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  idx->packed = 0;  // the index changes: any packed copy is stale
  hipError_t e =
      launch_csr(idx->labels, cap, H, L, C, cs, w.hist, idx->sizes, idx->offsets, idx->token_ids, cap, 0, st);
  if (e == hipSuccess)
    e = launch_update(idx->dtype, keys, (long long)cap * KVC_HEAD_DIM, H, C, cs, cps, idx->metric, idx->sizes,
                      idx->offsets, idx->token_ids, cap, idx->centroids, idx->centroids_t, idx->centroids_op, nullptr,
                      st);
  return status(e);
}

kvc_status kv_cluster_append(kvc_index* idx, void* k_cache, void* v_cache, const void* k_new, const void* v_new, int n_new,
                      void* stream) {
  if (!index_ok(idx) || !k_cache || !v_cache || !k_new || !v_new || n_new < 1) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx)) return KVC_ERR_INVALID_ARG;
  if ((long long)idx->n_tokens + n_new > idx->capacity) return KVC_ERR_CAPACITY;
  if (idx->window_start != idx->n_tokens) return KVC_ERR_INVALID_ARG;  // an open window: cluster it first
  const int cs = slots(idx), cap = idx->capacity;
  hipError_t e = launch_append(idx->dtype, k_cache, v_cache, (long long)cap * KVC_HEAD_DIM, idx->heads, k_new, v_new,
                               n_new, idx->n_tokens, idx->centroids_op, idx->c_active, cs, kv_cluster_cpad(cs),
                               idx->metric, idx->labels, cap, idx->sizes, idx->app_offsets, idx->app_ids,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return KVC_ERR_HIP;
  idx->n_tokens += n_new;
  idx->window_start = idx->n_tokens;
  return KVC_OK;
}

kvc_status kv_cluster_append_window(kvc_index* idx, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                             int n_new, void* stream) {
  if (!index_ok(idx) || !k_cache || !v_cache || !k_new || !v_new || n_new < 1) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx)) return KVC_ERR_INVALID_ARG;
  if ((long long)idx->n_tokens + n_new > idx->capacity) return KVC_ERR_CAPACITY;
  hipError_t e = launch_window_append(idx->dtype, k_cache, v_cache, idx->capacity, idx->heads, k_new, v_new, n_new,
                                      idx->n_tokens, idx->labels, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return KVC_ERR_HIP;
  idx->n_tokens += n_new;
  return KVC_OK;
}

size_t kv_cluster_window_workspace_bytes(int heads, int m, int n_clusters, int iters) {
  if (heads < 1 || m < 1 || n_clusters < 1 || iters < 1) return 0;
  return carve_window(nullptr, heads, m, n_clusters, iters).bytes;
}

kvc_status kv_cluster_cluster_window(kvc_index* idx, const void* k_cache, const void* v_cache, int n_clusters, int iters,
                              const int32_t* init_idx, void* ws, size_t ws_bytes, void* stream) {
  if (!index_ok(idx) || !k_cache || !v_cache || !init_idx || !ws) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx)) return KVC_ERR_INVALID_ARG;
  const int H = idx->heads, cap = idx->capacity, cs = slots(idx), cps = kv_cluster_cpad(cs);
  const int wlo = idx->window_start, m = idx->n_tokens - wlo, nc = n_clusters, ca = idx->c_active;
  if (nc < 1 || nc > m || ca + nc > cs || iters < 1 || iters > 100000) return KVC_ERR_INVALID_ARG;
  const bool packed = idx->packed == 1;
  if (packed && (!idx->k_packed || !idx->v_packed)) return KVC_ERR_INVALID_ARG;
  const WindowWs w = carve_window(ws, H, m, nc, iters);
  if (ws_bytes < w.bytes) return KVC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long hs = (long long)cap * KVC_HEAD_DIM;
  const int cpw = kv_cluster_cpad(nc);
  // the window's keys: rows wlo .. n_tokens-1; the index stores absolute positions
  const void* keys_w = static_cast<const char*>(k_cache) + (size_t)wlo * KVC_HEAD_DIM * elem_bytes(idx->dtype);
  hipError_t e = hipSuccess;
  // a small window: its whole k-means in one launch, same arithmetic
  const bool fused = window_kmeans_fits(m, nc);
  if (fused)
    e = launch_window_kmeans(idx->dtype, k_cache, hs, H, wlo, idx->n_tokens, m, nc, cpw, iters, init_idx, idx->metric,
                             w.cent, w.cent_t, w.chat, w.labels, w.sizes, w.offsets, w.ids, idx->dev_flags, st);
  if (!fused && e == hipSuccess) e = launch_fill_i32(reinterpret_cast<int32_t*>(w.b.qcount), (size_t)iters * H, 0, st);
  if (!fused && e == hipSuccess)
    e = launch_init_centroids(idx->dtype, k_cache, hs, H, wlo, idx->n_tokens, init_idx, nc, cpw, nc, cpw, idx->metric,
                              w.cent, w.cent_t, w.chat, idx->dev_flags, st);
  for (int t = 0; !fused && t < iters && e == hipSuccess; ++t) {
    e = launch_assign(idx->dtype, keys_w, hs, H, m, w.chat, nc, cpw, cpw, idx->metric, w.labels, m, w.b.queue,
                      w.b.qcount + (size_t)t * H, w.b.op_t, nullptr, nullptr, 0, nullptr, nullptr, st);
    if (e == hipSuccess) e = launch_csr(w.labels, m, H, m, nc, nc, w.b.hist, w.sizes, w.offsets, w.ids, m, wlo, st);
    if (e == hipSuccess)
      e = launch_update(idx->dtype, k_cache, hs, H, nc, nc, cpw, idx->metric, w.sizes, w.offsets, w.ids, m, w.cent,
                        w.cent_t, w.chat, nullptr, st);
  }
  if (e == hipSuccess)
    e = launch_merge_window(idx->dtype, H, nc, m, wlo, w.cent, w.chat, w.labels, w.sizes, w.offsets, w.ids, ca, cs, cps,
                            idx->centroids, idx->centroids_t, idx->centroids_op, idx->sizes, idx->offsets,
                            idx->token_ids, idx->labels, cap, st);
  // the packed copy gains the new members' rows, right after the existing ones
  if (e == hipSuccess && packed)
    e = launch_pack(idx->dtype, k_cache, v_cache, cap, H, idx->token_ids, m, idx->offsets + ca, nullptr, cs + 1,
                    idx->k_packed, idx->v_packed, st);
  if (e != hipSuccess) return KVC_ERR_HIP;
  idx->c_active = ca + nc;
  idx->window_start = idx->n_tokens;
  return KVC_OK;
}

kvc_status kv_cluster_select(const kvc_index* idx, const void* q, int q_heads, int B, int32_t* sel_ids, int32_t* sel_count,
                      void* stream) {
  if (!index_ok(idx) || !q || !sel_ids || !sel_count || B < 1 || q_heads < 1) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx) || q_heads % idx->heads != 0) return KVC_ERR_INVALID_ARG;
  const int G = q_heads / idx->heads;
  if (G > KVC_MAX_G) return KVC_ERR_UNSUPPORTED;
  if ((long long)idx->heads * B >= (1ll << 31)) return KVC_ERR_INVALID_ARG;
  const IndexView x = view(idx);
  return status(launch_select(idx->dtype, q, G, x, idx->heads, B, sel_ids, sel_count,
                                  static_cast<hipStream_t>(stream)));
}

size_t kv_sparse_decode_workspace_bytes(int heads, int q_heads, int d, int B) {
  if (heads < 1 || q_heads < heads || d < 1 || B < 1) return 0;
  const int G = q_heads / heads;
  const size_t nsplit = (size_t)(B + DEC_TOK - 1) / DEC_TOK;
  return align_up(sizeof(float) * heads * nsplit * G * (d + 2));
}

namespace {
kvc_status sparse_decode_check(const void* q, int q_heads, const void* k_cache, const void* v_cache, int dtype,
                               int heads, int capacity, int d, const int32_t* sel_ids, const int32_t* sel_count,
                               int B, const float* out) {
  if (!q || !k_cache || !v_cache || !sel_ids || !sel_count || !out) return KVC_ERR_INVALID_ARG;
  if (heads < 1 || q_heads < 1 || capacity < 1 || B < 1 || q_heads % heads != 0) return KVC_ERR_INVALID_ARG;
  if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_INVALID_ARG;
  if (d != KVC_HEAD_DIM) return KVC_ERR_UNSUPPORTED;
  const int G = q_heads / heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if ((long long)heads * B >= (1ll << 31)) return KVC_ERR_INVALID_ARG;
  if ((long long)((B + DEC_TOK - 1) / DEC_TOK) * G > DEC_MAX_PAIRS) return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}
}  // namespace

kvc_status kv_sparse_decode(const void* q, int q_heads, const void* k_cache, const void* v_cache, int dtype,
                            int heads, int capacity, int d, const int32_t* sel_ids, const int32_t* sel_count, int B,
                            float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (kvc_status s = sparse_decode_check(q, q_heads, k_cache, v_cache, dtype, heads, capacity, d, sel_ids,
                                         sel_count, B, out))
    return s;
  if (!ws) return KVC_ERR_INVALID_ARG;
  if (ws_bytes < kv_sparse_decode_workspace_bytes(heads, q_heads, d, B)) return KVC_ERR_WORKSPACE;
  return status(launch_decode(dtype, q, q_heads / heads, k_cache, v_cache, (long long)capacity * d, heads, sel_ids,
                              sel_count, B, scale, out, static_cast<float*>(ws), static_cast<hipStream_t>(stream)));
}

kvc_status kv_sparse_decode_noalloc(const void* q, int q_heads, const void* k_cache, const void* v_cache, int dtype,
                                    int heads, int capacity, int d, const int32_t* sel_ids, const int32_t* sel_count,
                                    int B, float scale, float* out, void* stream) {
  if (kvc_status s = sparse_decode_check(q, q_heads, k_cache, v_cache, dtype, heads, capacity, d, sel_ids,
                                         sel_count, B, out))
    return s;
  if (kv_sparse_decode_workspace_bytes(heads, q_heads, d, B) > KVC_NOALLOC_SCRATCH_BYTES) return KVC_ERR_TOO_LARGE;
  void* part = nullptr;
  if (noalloc_scratch(&part) != hipSuccess) return KVC_ERR_HIP;
  return status(launch_decode(dtype, q, q_heads / heads, k_cache, v_cache, (long long)capacity * d, heads, sel_ids,
                              sel_count, B, scale, out, static_cast<float*>(part), static_cast<hipStream_t>(stream)));
}

size_t kv_cluster_select_decode_workspace_bytes(int heads, int q_heads, int d) {
  if (heads < 1 || q_heads < heads || d < 1) return 0;
  const int G = q_heads / heads;
  // the arrival counters [heads], then the partial results [heads, P, G, d + 2]
  return align_up(sizeof(int32_t) * heads) + align_up(sizeof(float) * heads * fused_blocks_per_head(heads) * G * (d + 2));
}

kvc_status kv_cluster_select_decode(const kvc_index* idx, const void* q, int q_heads, const void* k_cache,
                             const void* v_cache, int B, float scale, float* out, int32_t* sel_ids,
                             int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  if (!index_ok(idx) || !q || !k_cache || !v_cache || !out || B < 1 || q_heads < 1) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx) || q_heads % idx->heads != 0) return KVC_ERR_INVALID_ARG;
  const int G = q_heads / idx->heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if ((long long)idx->heads * B >= (1ll << 31)) return KVC_ERR_INVALID_ARG;
  if (ws && ws_bytes < kv_cluster_select_decode_workspace_bytes(idx->heads, q_heads, idx->d)) return KVC_ERR_WORKSPACE;
  const IndexView x = view(idx);
  const bool packed = idx->packed == 1 && idx->k_packed && idx->v_packed;
  // the token split exists for bf16 and at most 4 query heads per KV head
  const bool ts = ws && idx->dtype == KVC_BF16 && G <= 4;
  int32_t* arrive = ts ? static_cast<int32_t*>(ws) : nullptr;
  float* part =
      ts ? reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(sizeof(int32_t) * idx->heads)) : nullptr;
  return status(launch_select_decode(idx->dtype, q, G, x, idx->heads, k_cache, v_cache,
                                         packed ? idx->k_packed : nullptr, packed ? idx->v_packed : nullptr, B, scale,
                                         out, sel_ids, sel_count, part, arrive, static_cast<hipStream_t>(stream)));
}

kvc_status kv_cluster_pack(kvc_index* idx, const void* k_cache, const void* v_cache, void* stream) {
  if (!index_ok(idx) || !k_cache || !v_cache || !idx->k_packed || !idx->v_packed) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx)) return KVC_ERR_INVALID_ARG;
  // rows 0 .. offsets[h][c_active]-1: the main part, at most n_tokens - n_sink rows
  const int cs = slots(idx);
  const kvc_status e = status(launch_pack(idx->dtype, k_cache, v_cache, idx->capacity, idx->heads, idx->token_ids,
                                       idx->n_tokens - idx->n_sink, nullptr, idx->offsets + idx->c_active, cs + 1,
                                       idx->k_packed, idx->v_packed, static_cast<hipStream_t>(stream)));
  if (e == KVC_OK) idx->packed = 1;
  return e;
}

kvc_status kv_cluster_export_csr(const kvc_index* idx, int32_t* offsets, int32_t* token_ids, void* stream) {
  if (!index_ok(idx) || !offsets || !token_ids) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx)) return KVC_ERR_INVALID_ARG;
  return status(launch_export_csr(idx->heads, idx->c_active, slots(idx), idx->offsets, idx->token_ids,
                                      idx->app_offsets, idx->app_ids, idx->capacity, offsets, token_ids,
                                      static_cast<hipStream_t>(stream)));
}

kvc_status kv_cluster_cache_reset(const kvc_index* idx, kvc_cluster_cache* cache, void* stream) {
  if (!index_ok(idx) || !cache || !cache->table || !cache->stats) return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = idx->heads, cs = slots(idx);
  // table entries (step, row, members) = (never, 0, 0); counters 0
  hipError_t e = launch_fill_i32(cache->table, (size_t)H * cs * 3, 0, st);
  if (e == hipSuccess) e = launch_fill2d_i32(cache->table, H * cs, 3, 1, -(1 << 30), st);
  if (e == hipSuccess) e = launch_fill_i32(reinterpret_cast<int32_t*>(cache->stats), (size_t)H * 4 * 2, 0, st);
  if (e != hipSuccess) return KVC_ERR_HIP;
  cache->step = 0;
  return KVC_OK;
}

size_t kv_cluster_cache_workspace_bytes(int heads, int q_heads, int d, int B) {
  if (heads < 1 || q_heads < heads || d < 1 || B < 1) return 0;
  return align_up(sizeof(int32_t) * (size_t)heads * B) + align_up(sizeof(int32_t) * (size_t)heads) +
         kv_sparse_decode_workspace_bytes(heads, q_heads, d, B);
}

kvc_status kv_cluster_cached_select_decode(const kvc_index* idx, kvc_cluster_cache* cache, const void* q, int q_heads,
                                    const void* k_cache, const void* v_cache, float scale, float* out,
                                    int32_t* sel_ids, int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  if (!index_ok(idx) || !cache || !q || !k_cache || !v_cache || !out || !ws || q_heads < 1) return KVC_ERR_INVALID_ARG;
  if (!cache->k || !cache->v || !cache->table || !cache->stats || cache->R < 1 || cache->B < 1 || cache->step < 0)
    return KVC_ERR_INVALID_ARG;
  if (kvc_status s = index_support(idx)) return s;
  if (!built_ok(idx) || q_heads % idx->heads != 0) return KVC_ERR_INVALID_ARG;
  const int H = idx->heads, G = q_heads / H, B = cache->B, R = cache->R;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if ((long long)H * (R + 1) * B >= (1ll << 31)) return KVC_ERR_INVALID_ARG;
  if ((long long)((B + DEC_TOK - 1) / DEC_TOK) * G > DEC_MAX_PAIRS) return KVC_ERR_UNSUPPORTED;
  if (ws_bytes < kv_cluster_cache_workspace_bytes(H, q_heads, KVC_HEAD_DIM, B)) return KVC_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  int32_t* rows = reinterpret_cast<int32_t*>(w);
  int32_t* count = reinterpret_cast<int32_t*>(w + align_up(sizeof(int32_t) * (size_t)H * B));
  float* part = reinterpret_cast<float*>(w + align_up(sizeof(int32_t) * (size_t)H * B) + align_up(sizeof(int32_t) * H));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool packed = idx->packed == 1 && idx->k_packed && idx->v_packed;
  hipError_t e = launch_cache_assemble(idx->dtype, q, G, view(idx), H, k_cache, v_cache,
                                       packed ? idx->k_packed : nullptr, packed ? idx->v_packed : nullptr, B, R,
                                       cache->step, cache->k, cache->v, cache->table,
                                       reinterpret_cast<long long*>(cache->stats), rows, count, sel_ids, sel_count,
                                       st);
  if (e == hipSuccess)
    e = launch_decode(idx->dtype, q, G, cache->k, cache->v, (long long)(R + 1) * B * KVC_HEAD_DIM, H, rows, count, B,
                      scale, out, part, st);
  if (e != hipSuccess) return KVC_ERR_HIP;
  cache->step += 1;
  return KVC_OK;
}

size_t kv_dense_decode_workspace_bytes(int heads, int q_heads, int d, int n) {
  if (heads < 1 || q_heads < heads || q_heads % heads != 0 || d != KVC_HEAD_DIM || n < 1) return 0;
  const int G = q_heads / heads;
  if (G > KVC_MAX_G) return 0;
  int nsplit, T;
  dense_split(n, G, &nsplit, &T);
  return align_up(sizeof(float) * (size_t)heads * nsplit * G * (KVC_HEAD_DIM + 2));
}

kvc_status kv_dense_decode(const void* q, int q_heads, const void* k_cache, const void* v_cache, int dtype, int heads,
                    int capacity, int d, int n, float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !out || !ws || heads < 1 || q_heads < 1) return KVC_ERR_INVALID_ARG;
  if (dtype != KVC_BF16 && dtype != KVC_F32) return KVC_ERR_INVALID_ARG;
  if (d != KVC_HEAD_DIM || dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
  if (q_heads % heads != 0) return KVC_ERR_INVALID_ARG;
  const int G = q_heads / heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if (n < 1 || n > capacity) return KVC_ERR_INVALID_ARG;
  if ((long long)heads * capacity >= (1ll << 31)) return KVC_ERR_UNSUPPORTED;
  if (ws_bytes < kv_dense_decode_workspace_bytes(heads, q_heads, d, n)) return KVC_ERR_WORKSPACE;
  return status(launch_dense_decode(q, G, k_cache, v_cache, capacity, heads, n, scale, out,
                                        static_cast<float*>(ws), static_cast<hipStream_t>(stream)));
}

const char* kv_cluster_status_string(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARG: return "invalid argument";
    case KVC_ERR_UNSUPPORTED: return "unsupported by the GPU path (d must be 128, C <= 512, G in {1,2,4,8})";
    case KVC_ERR_WORKSPACE: return "workspace too small";
    case KVC_ERR_CAPACITY: return "index capacity exceeded";
    case KVC_ERR_HIP: return "HIP launch failure";
    case KVC_ERR_TOO_LARGE: return "request larger than the fixed device scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
