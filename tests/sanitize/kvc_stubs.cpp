// No-op stand-ins for the kernel launchers of kvc_internal.h, so that the C
// ABI's argument checks and workspace arithmetic (kvc_api.cpp, kvc_host.cpp)
// build as host-only code and run under AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU. Every launcher returns success and
// touches no memory; hipMemcpyAsync likewise.
#include <hip/hip_runtime.h>

#include "kvc_internal.h"

namespace kvc {

hipError_t noalloc_scratch(void** ptr) {
  static char fake[16];
  *ptr = fake;
  return hipSuccess;
}

hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t v, hipStream_t st) { return hipSuccess; }

hipError_t launch_init_positions(int heads, int lo, int L, int C, unsigned long long seed, int32_t* out, hipStream_t st) { return hipSuccess; }

hipError_t launch_init_centroids(int dtype, const void* keys, long long head_stride, int heads, int lo, int L, const int32_t* init_idx, int C, int cpad, int cs, int cps, int metric, float* cent, float* cent_t, void* chat, int32_t* flags, hipStream_t st) { return hipSuccess; }

hipError_t launch_assign(int dtype, const void* keys, long long head_stride, int heads, int L, const void* chat, int C, int cpad, int cps, int metric, int32_t* labels, long long label_stride, int32_t* queue, uint32_t* qcount, void* op_t, int32_t* dirty, float* norm2, int norm_mode, float* top2, hipEvent_t* events, hipStream_t st) { return hipSuccess; }

hipError_t launch_fill2d_i32(int32_t* p, int rows, long long stride, int cols, int value, hipStream_t st) { return hipSuccess; }

hipError_t launch_csr(const int32_t* labels, long long label_stride, int heads, int L, int C, int cs, int32_t* hist, int32_t* sizes, int32_t* offsets, int32_t* token_ids, long long ids_stride, int id_base, hipStream_t st) { return hipSuccess; }

hipError_t launch_update(int dtype, const void* keys, long long head_stride, int heads, int C, int cs, int cps, int metric, const int32_t* sizes, const int32_t* offsets, const int32_t* token_ids, long long ids_stride, float* cent, float* cent_t, void* chat, const int32_t* dirty, hipStream_t st) { return hipSuccess; }

hipError_t launch_window_kmeans(int dtype, const void* keys, long long head_stride, int heads, int wlo, int n_tokens, int m, int nc, int cpw, int iters, const int32_t* init_idx, int metric, float* cent, float* cent_t, void* chat, int32_t* labels, int32_t* sizes, int32_t* offsets, int32_t* ids, int32_t* flags, hipStream_t st) { return hipSuccess; }

hipError_t launch_merge_window(int dtype, int heads, int nc, int m, int wlo, const float* cent_w, const void* chat_w, const int32_t* labels_w, const int32_t* sizes_w, const int32_t* offsets_w, const int32_t* ids_w, int ca, int cs, int cps, float* cent, float* cent_t, void* chat, int32_t* sizes, int32_t* offsets, int32_t* token_ids, int32_t* labels, long long cap, hipStream_t st) { return hipSuccess; }

hipError_t launch_append(int dtype, void* kc, void* vc, long long head_stride, int heads, const void* knew, const void* vnew, int n_new, int n0, const void* chat, int ca, int cs, int cps, int metric, int32_t* labels, long long cap, int32_t* sizes, int32_t* app_offsets, int32_t* app_ids, hipStream_t st) { return hipSuccess; }

hipError_t launch_window_append(int dtype, void* kc, void* vc, long long cap, int heads, const void* knew, const void* vnew, int n_new, int n0, int32_t* labels, hipStream_t st) { return hipSuccess; }

hipError_t launch_debug_scores(int dtype, const void* q, int G, const IndexView& x, int heads, double* scores, hipStream_t st) { return hipSuccess; }

hipError_t launch_select(int dtype, const void* q, int G, const IndexView& x, int heads, int B, int32_t* sel_ids, int32_t* sel_count, hipStream_t st) { return hipSuccess; }

hipError_t launch_decode(int dtype, const void* q, int G, const void* kc, const void* vc, long long head_stride, int heads, const int32_t* sel_ids, const int32_t* sel_count, int B, float scale, float* out, float* part, hipStream_t st) { return hipSuccess; }

hipError_t launch_select_decode(int dtype, const void* q, int G, const IndexView& x, int heads, const void* kc, const void* vc, const void* kp, const void* vp, int B, float scale, float* out, int32_t* sel_ids, int32_t* sel_count, float* part, int32_t* arrive, hipStream_t st) { return hipSuccess; }

hipError_t launch_scores(int dtype, const void* q, int G, const IndexView& x, int heads, double* scores, int stride, hipStream_t st) { return hipSuccess; }

hipError_t launch_cache_assemble(int dtype, const void* q, int G, const IndexView& x, int heads, const void* kc, const void* vc, const void* kp, const void* vp, int B, int R, int t, void* ck, void* cv, int32_t* table, long long* stats, int32_t* rows, int32_t* count, int32_t* sel_ids, int32_t* sel_count, hipStream_t st) { return hipSuccess; }

hipError_t launch_dense_decode(const void* q, int G, const void* kc, const void* vc, long long cap, int heads, int n, float scale, float* out, float* part, hipStream_t st) { return hipSuccess; }

hipError_t launch_pack(int dtype, const void* kc, const void* vc, long long cap, int heads, const int32_t* token_ids, int n, const int32_t* row0, const int32_t* row1, long long stride, void* kp, void* vp, hipStream_t st) { return hipSuccess; }

hipError_t launch_export_csr(int heads, int ca, int cs, const int32_t* offsets, const int32_t* token_ids, const int32_t* app_offsets, const int32_t* app_ids, long long cap, int32_t* out_offsets, int32_t* out_ids, hipStream_t st) { return hipSuccess; }

}  // namespace kvc

extern "C" hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipSuccess; }
