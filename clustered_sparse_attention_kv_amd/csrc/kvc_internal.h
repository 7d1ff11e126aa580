// Host-side launchers of the kvcluster kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

enum { DT_F32 = 0, DT_BF16 = 1 };
// assignment distance: the cosine (the method's), L2, inner product
enum { M_COSINE = 0, M_L2 = 1, M_IP = 2 };

constexpr int MAX_C = 512;       // largest cluster count (slots) per head
constexpr int DEC_TOK = 64;      // selected tokens per decode block (split)
constexpr int DEC_MAX_PAIRS = 512;  // splits x query heads one merge block holds

// Host-side sizing shared by the launchers and the workspace arithmetic of the
// C ABI (kvc_host.cpp).
constexpr int CSR_BLOCK_TOKENS = 4096;  // tokens per block of the counting sort
int csr_blocks(int L);
// Blocks per KV head of the fused selection and attention: enough that the
// grid covers the 256 compute units.
int fused_blocks_per_head(int heads);
// 16-row tiles per slice of the token split (4, 2 or 1).
int fused_slice_tiles(int B, int P);
// Split of the dense pass over n rows: nsplit blocks of T rows.
void dense_split(int n, int G, int* nsplit, int* T);

// Bytes of the fixed device scratch of kv_sparse_decode_noalloc.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
// The current device's address of that scratch (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

// The index as the selection kernels read it: device arrays with per-head
// strides of cs cluster slots (cs + 1 for the prefix arrays) and cap tokens;
// clusters 0 .. ca-1 in use; ahead of the clusters, the n_sink attention sinks
// (tokens 0 .. n_sink-1) and the nw window tokens wlo .. wlo+nw-1 are recalled.
struct IndexView {
  const float* cent_t;  // [heads, d/4, cs, 4]
  const int32_t *sizes, *offsets, *token_ids, *app_offsets, *app_ids;
  long long cap;
  int cs, ca, n_sink, wlo, nw;
};

hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t v, hipStream_t st);
// Initial centroid positions [heads, C] of the seeded partial shuffle of rows lo .. L-1.
hipError_t launch_init_positions(int heads, int lo, int L, int C, unsigned long long seed, int32_t* out,
                                 hipStream_t st);
hipError_t launch_init_centroids(int dtype, const void* keys, long long head_stride, int heads, int lo, int L,
                                 const int32_t* init_idx, int C, int cpad, int cs, int cps, int metric, float* cent,
                                 float* cent_t, void* chat, int32_t* flags, hipStream_t st);
hipError_t launch_assign(int dtype, const void* keys, long long head_stride, int heads, int L, const void* chat, int C,
                         int cpad, int cps, int metric, int32_t* labels, long long label_stride, int32_t* queue,
                         uint32_t* qcount, void* op_t, int32_t* dirty, float* norm2, int norm_mode, float* top2,
                         hipEvent_t* events, hipStream_t st);
hipError_t launch_fill2d_i32(int32_t* p, int rows, long long stride, int cols, int value, hipStream_t st);
hipError_t launch_csr(const int32_t* labels, long long label_stride, int heads, int L, int C, int cs, int32_t* hist,
                      int32_t* sizes, int32_t* offsets, int32_t* token_ids, long long ids_stride, int id_base,
                      hipStream_t st);
hipError_t launch_update(int dtype, const void* keys, long long head_stride, int heads, int C, int cs, int cps,
                         int metric, const int32_t* sizes, const int32_t* offsets, const int32_t* token_ids, long long ids_stride,
                         float* cent, float* cent_t, void* chat, const int32_t* dirty, hipStream_t st);
// Moves the window's clustering (nc clusters of the m tokens wlo .. wlo+m-1,
// in arrays of stride nc / cpad(nc) / m per head) into the index as clusters
// ca .. ca+nc-1.
// The window's whole k-means in one launch, for windows whose labels fit the
// kernel's LDS (at most 16384 tokens) and at most WINDOW_KMEANS_MAX_C clusters.
constexpr int WINDOW_KMEANS_MAX_C = 32;
bool window_kmeans_fits(int m, int nc);
hipError_t launch_window_kmeans(int dtype, const void* keys, long long head_stride, int heads, int wlo, int n_tokens,
                                int m, int nc, int cpw, int iters, const int32_t* init_idx, int metric, float* cent,
                                float* cent_t, void* chat, int32_t* labels, int32_t* sizes, int32_t* offsets,
                                int32_t* ids, int32_t* flags, hipStream_t st);
hipError_t launch_merge_window(int dtype, int heads, int nc, int m, int wlo, const float* cent_w, const void* chat_w,
                               const int32_t* labels_w, const int32_t* sizes_w, const int32_t* offsets_w,
                               const int32_t* ids_w, int ca, int cs, int cps, float* cent, float* cent_t, void* chat,
                               int32_t* sizes, int32_t* offsets, int32_t* token_ids, int32_t* labels, long long cap,
                               hipStream_t st);

hipError_t launch_append(int dtype, void* kc, void* vc, long long head_stride, int heads, const void* knew,
                         const void* vnew, int n_new, int n0, const void* chat, int ca, int cs, int cps, int metric,
                         int32_t* labels, long long cap, int32_t* sizes, int32_t* app_offsets, int32_t* app_ids,
                         hipStream_t st);
hipError_t launch_window_append(int dtype, void* kc, void* vc, long long cap, int heads, const void* knew,
                                const void* vnew, int n_new, int n0, int32_t* labels, hipStream_t st);
hipError_t launch_debug_scores(int dtype, const void* q, int G, const IndexView& x, int heads, double* scores,
                               hipStream_t st);
hipError_t launch_select(int dtype, const void* q, int G, const IndexView& x, int heads, int B, int32_t* sel_ids,
                         int32_t* sel_count, hipStream_t st);
hipError_t launch_decode(int dtype, const void* q, int G, const void* kc, const void* vc, long long head_stride,
                         int heads, const int32_t* sel_ids, const int32_t* sel_count, int B, float scale, float* out,
                         float* part, hipStream_t st);
hipError_t launch_select_decode(int dtype, const void* q, int G, const IndexView& x, int heads, const void* kc,
                                const void* vc, const void* kp, const void* vp, int B, float scale, float* out,
                                int32_t* sel_ids, int32_t* sel_count, float* part, int32_t* arrive,
                                hipStream_t st);
// The selection's scores of the clusters in use: scores[h * stride + k].
hipError_t launch_scores(int dtype, const void* q, int G, const IndexView& x, int heads, double* scores, int stride,
                         hipStream_t st);
// kp, vp: the packed copies (both non-null) or null (rows from the caches).
// The cluster cache's step: selection, then the selected rows assembled into
// region t mod (R + 1) of ck / cv ([heads, (R + 1) * B, d]) from the cache or
// their source; rows / count receive the decode's row list and counts.
hipError_t launch_cache_assemble(int dtype, const void* q, int G, const IndexView& x, int heads, const void* kc,
                                 const void* vc, const void* kp, const void* vp, int B, int R, int t, void* ck,
                                 void* cv, int32_t* table, long long* stats, int32_t* rows, int32_t* count,
                                 int32_t* sel_ids, int32_t* sel_count, hipStream_t st);
hipError_t launch_dense_decode(const void* q, int G, const void* kc, const void* vc, long long cap, int heads, int n,
                               float scale, float* out, float* part, hipStream_t st);
// Rows i in [r0, r1) of the packed copies from the cache rows token_ids[h][i]:
// r0 = row0[h * stride] (0 without row0), r1 = row1[h * stride] (r0 + n
// without row1; n bounds r1 - r0 and sizes the grid).
hipError_t launch_pack(int dtype, const void* kc, const void* vc, long long cap, int heads, const int32_t* token_ids,
                       int n, const int32_t* row0, const int32_t* row1, long long stride, void* kp, void* vp,
                       hipStream_t st);
hipError_t launch_export_csr(int heads, int ca, int cs, const int32_t* offsets, const int32_t* token_ids,
                             const int32_t* app_offsets, const int32_t* app_ids, long long cap, int32_t* out_offsets,
                             int32_t* out_ids, hipStream_t st);

}  // namespace kvc
