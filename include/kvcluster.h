/*
 * kvcluster: cluster-granular sparse KV recall on AMD Instinct MI355X (gfx950).
 *
 * The method is ClusterKV, "Manipulating LLM KV Cache in Semantic Space for
 * Recallable Compression" (arXiv 2412.03213). Section names below refer to
 * the paper summary page (paperlayer.ai, 2412.03213v2).
 *
 *  - At prefill, each head's keys are grouped into C semantic clusters by
 *    cosine k-means (III.B "Clustering in the Semantic Space", Sys-B
 *    "Semantic Clustering"). The result is an index: centroids, cluster
 *    sizes, prefix sums and the token ids sorted by cluster (Sys-C
 *    "Selection and Indexing").
 *  - At each decode step, the query scores the centroids and whole clusters
 *    are taken in score order until the token budget B is met, with the last
 *    cluster trimmed (III.C, Sys-C with Fig. 8). Single-query attention then
 *    runs over only the recalled tokens (II.A, III.A "Problem Formulation").
 *
 * Conventions shared by every call:
 *  - Memory. Every pointer argument is DEVICE memory unless stated otherwise,
 *    owned by the caller. The library never allocates, frees or
 *    synchronises. Its one piece of device state is the fixed scratch
 *    array of kv_sparse_decode_noalloc (below), which that call alone uses.
 *  - Streams. `stream` is a hipStream_t passed as void* (NULL is the null
 *    stream). Every call only enqueues work on it; results are valid once
 *    the stream has been synchronised.
 *  - Errors. Arguments are checked on the host before anything is enqueued.
 *    On any error nothing is enqueued and the call returns a nonzero
 *    kvc_status. A kernel launch failure returns KVC_ERR_HIP. Faults inside
 *    kernels surface through HIP at the caller's next synchronisation.
 *  - Layout. heads = batch x KV heads, flattened. K/V caches are row-major
 *    [heads, capacity, d] with head stride capacity*d. Query heads are
 *    [q_heads, d] with q_heads = G * heads; query head g reads KV head g / G.
 *    The GPU path supports d = 128 and C <= 512.
 *  - Element types. KVC_BF16 (the production path; bf16 inputs, fp32
 *    accumulation) or KVC_F32. Keys, values, queries and new tokens of one
 *    index share the type.
 */
#ifndef KVCLUSTER_H
#define KVCLUSTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_HEAD_DIM 128 /* the only head dimension the GPU path supports */
#define KVC_MAX_C 512    /* largest cluster count per head */
#define KVC_MAX_G 8      /* largest number of query heads per KV head */

typedef enum kvc_dtype { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* Assignment distance (III.B measures semantic distance by the cosine and
 * names L2 and inner-product distance as the alternatives it is preferred to;
 * the model-accuracy section compares the three). */
typedef enum kvc_metric {
  KVC_COSINE = 0,        /* argmax_k K . c_k / ||c_k|| (the method's) */
  KVC_L2 = 1,            /* argmin_k ||K - c_k||^2 = argmax_k (K . c_k - ||c_k||^2 / 2) */
  KVC_INNER_PRODUCT = 2  /* argmax_k K . c_k */
} kvc_metric;

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1, /* a null pointer, a size out of range, ... */
  KVC_ERR_UNSUPPORTED = 2, /* valid for the method, not for this GPU path (d != 128, C > 512, G > 8) */
  KVC_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_workspace_bytes() */
  KVC_ERR_CAPACITY = 4,    /* an append would pass the index capacity */
  KVC_ERR_HIP = 5,         /* a kernel launch failed */
  KVC_ERR_TOO_LARGE = 6    /* larger than the fixed scratch of kv_sparse_decode_noalloc */
} kvc_status;

/*
 * The cluster index of `heads` independent heads: centroids plus the
 * cluster-to-token metadata that Sys-C keeps after clustering (sizes, prefix
 * sums, token indices sorted by cluster). The caller allocates every array
 * (device memory) and fills in the pointers and sizes; kv_cluster_build
 * writes the contents.
 *
 * Tokens appended at decode time (kv_cluster_append) are kept in a second,
 * cluster-major list so that no append moves the built index: the members of
 * cluster k are token_ids[offsets[k] .. offsets[k+1]) followed by
 * app_ids[app_offsets[k] .. app_offsets[k+1]), in ascending token order.
 *
 * Generated tokens can instead be clustered periodically (III.B; Sys-A): they
 * join a window (kv_cluster_append_window) that every selection recalls whole,
 * and kv_cluster_cluster_window turns the window into a few new clusters with
 * ids c_active, c_active+1, ... . Every per-cluster array therefore has a
 * per-head stride of c_slots cluster slots, of which the first c_active are in
 * use.
 */
typedef struct kvc_index {
  int32_t heads;    /* independent problems (batch x KV heads) */
  int32_t d;        /* head dimension; must be 128 */
  int32_t C;        /* clusters per head, 1 <= C <= 512 */
  int32_t capacity; /* rows per head of the K/V caches (and of labels/token_ids/app_ids) */
  int32_t dtype;    /* kvc_dtype of keys, queries and the centroid operand */
  int32_t n_build;  /* host mirror: tokens clustered by the last build */
  int32_t n_tokens; /* host mirror: n_build + tokens appended since */
  int32_t packed;   /* host mirror: 1 once kv_cluster_pack has filled k_packed/v_packed for
                       the current build (kv_cluster_build resets it to 0) */
  float* centroids;       /* [heads, C, d] fp32: mean of each cluster's keys */
  void* centroids_op;     /* [heads, kv_cluster_cpad(C), d] unit-length centroids in `dtype`
                             (the assignment operand); rows C .. cpad(C)-1 are zero after a build */
  int32_t* labels;        /* [heads, capacity] cluster of every token (-1: none) */
  int32_t* sizes;         /* [heads, C] members per cluster, appended tokens included */
  int32_t* offsets;       /* [heads, C+1] prefix sums of the main part's sizes (the built
                             clusters, then clusters made from windows) */
  int32_t* token_ids;     /* [heads, capacity] the main part: members sorted by cluster, ascending
                             within */
  int32_t* app_offsets;   /* [heads, C+1] prefix sums of the appended part */
  int32_t* app_ids;       /* [heads, capacity] appended tokens, cluster-major, ascending within */
  int32_t* dev_flags;     /* [1] error bits set by kernels (bit 0: an init index out of range) */
  float* centroids_t;     /* [heads, d/4, C, 4] fp32: the same centroids with 4-channel chunks
                             cluster-minor, written by the build and read by selection */
  void* k_packed;         /* optional (NULL): [heads, capacity, d] in dtype; kv_cluster_pack writes
                             the built tokens' key rows in index order (row i = token_ids[i]) */
  void* v_packed;         /* optional (NULL): the value rows in the same order */
  int32_t n_sink;         /* attention sinks (III.B): tokens 0 .. n_sink-1 are kept out of the
                             clustering (label -1) and always selected first; 0 = none. Set by
                             the caller before kv_cluster_build. */
  int32_t c_slots;        /* cluster slots per head, C <= c_slots <= 512, or 0 for C: the per-head
                             stride S of centroids [heads, S, d], centroids_op [heads,
                             kv_cluster_cpad(S), d], sizes [heads, S], offsets and app_offsets
                             [heads, S+1] and centroids_t [heads, d/4, S, 4] (the sizes written
                             above for C hold when c_slots is 0) */
  int32_t c_active;       /* host mirror: clusters in use, ids 0 .. c_active-1 (C after a build) */
  int32_t window_start;   /* host mirror: first token of the window; tokens window_start ..
                             n_tokens-1 are in no cluster yet (label -1) and every selection
                             recalls them (n_build after a build) */
  int32_t metric;         /* kvc_metric of every assignment (build, window clustering, append);
                             KVC_COSINE (0) is the method's. Under L2 and inner product the
                             operand centroids_op holds the centroids themselves, rounded once
                             to dtype, instead of their unit directions. */
} kvc_index;

/* Rows of centroids_op per head: C rounded up to the matrix-core tile (32). */
int kv_cluster_cpad(int C);

/*
 * Device memory of one index (every array of kvc_index except the optional
 * packed copies), for `heads` heads of dimension d, C clusters, `capacity`
 * tokens per head, element type dtype and c_slots cluster slots (0 for C).
 * The caller allocates it (one allocation); 0 for invalid sizes.
 */
size_t kv_cluster_index_bytes(int heads, int d, int C, int capacity, kvc_dtype dtype, int c_slots);

/*
 * Lays an index out in caller memory: sets the size fields of *idx (heads,
 * d, C, capacity, dtype, c_slots, n_sink, metric; host mirrors 0; k_packed
 * and v_packed NULL, for the caller to set) and points every array into mem
 * (device memory of at least kv_cluster_index_bytes(...) bytes, each array
 * 256-byte aligned). Enqueues on stream the fills that give a fresh index:
 * labels, token_ids and app_ids -1, every other array 0. Requires d = 128,
 * 1 <= C <= c_slots (or c_slots 0) <= 512, capacity >= 1, n_sink >= 0.
 */
kvc_status kv_cluster_index_init(kvc_index* idx, int heads, int d, int C, int capacity, kvc_dtype dtype, int c_slots,
                                 int n_sink, kvc_metric metric, void* mem, size_t mem_bytes, void* stream);

/* Bytes of workspace kv_cluster_build needs for these sizes. */
size_t kv_cluster_build_workspace_bytes(int heads, int L, int C, int iters);

/*
 * Initial centroid positions (the pages leave the initialisation open; III.B
 * only says that the k-means iterates until the assignment settles; the
 * reading here is a seeded random choice of C distinct keys). For every head
 * h, the clustered rows are n_sink .. L-1 (n = L - n_sink of them) and the
 * positions are n_sink + perm[0 .. C-1] of a partial Fisher-Yates shuffle:
 * perm = (0, 1, ..., n-1); for i = 0 .. C-1, j = i + (r_i mod (n - i)) and
 * perm[i], perm[j] swap, with r_i the i-th output of SplitMix64 (Steele, Lea
 * and Flood 2014: the state advances by 0x9E3779B97F4A7C15, then z ^= z >> 30,
 * z *= 0xBF58476D1CE4E5B9, z ^= z >> 27, z *= 0x94D049BB133111EB, z ^= z >> 31)
 * started from state seed ^ (0x9E3779B97F4A7C15 * (h + 1)), arithmetic mod
 * 2^64. out is [heads, C] int32 (device). Requires 1 <= C <= min(512, n)
 * (KVC_ERR_UNSUPPORTED above 512); enqueues one kernel on stream.
 */
kvc_status kv_cluster_init_positions(int heads, int n_sink, int L, int C, uint64_t seed, int32_t* out, void* stream);

/*
 * Prefill clustering (III.B; Sys-B). For every head, the first L rows of
 * `keys` ([heads, capacity, d], idx->dtype) are clustered into idx->C
 * clusters by `iters` iterations of cosine k-means:
 *   - only rows idx->n_sink .. L-1 are clustered: the attention sinks before
 *     them keep label -1 and are not in the index (kv_cluster_select puts them
 *     first). Requires 0 <= n_sink and C <= L - n_sink;
 *   - the initial centroids are the keys at the positions
 *     kv_cluster_init_positions(heads, n_sink, L, C, seed) gives, drawn on the
 *     device into the workspace;
 *   - each iteration normalises the centroids (rounded once to idx->dtype),
 *     assigns every key to the centroid of largest cosine similarity (lowest
 *     id on an exact tie; a key whose scores are all NaN or -inf goes to
 *     cluster 0) and replaces each centroid by the mean of its keys (an empty
 *     cluster keeps its centroid). Under idx->metric KVC_L2 or
 *     KVC_INNER_PRODUCT the operand is the centroid itself (rounded once) and
 *     a key joins the centroid of least L2 distance (largest K . c - ||c||^2
 *     / 2, both fp64 chains over ascending channels, then their fp64
 *     difference) or of largest inner product.
 * On return (after synchronisation) the index holds the means of the final
 * assignment, their normalised operand, labels, sizes, offsets and
 * token_ids; the appended part is empty. idx->n_build, idx->n_tokens and
 * idx->window_start are set to L and idx->c_active to C on the host.
 * Requires 1 <= C <= L <= capacity, iters >= 1, C <= 512, and a workspace of
 * kv_cluster_build_workspace_bytes(heads, L, C, iters) bytes (contents need
 * not be initialised).
 */
kvc_status kv_cluster_build(kvc_index* idx, const void* keys, int L, int iters, uint64_t seed, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * kv_cluster_build from caller-chosen initial positions instead of the
 * seeded shuffle: init_idx ([heads, C] int32, device) holds distinct token
 * positions in [n_sink, L). An index out of range sets bit 0 of
 * *idx->dev_flags and row 0 is used instead. Otherwise identical.
 */
kvc_status kv_cluster_build_from(kvc_index* idx, const void* keys, int L, int iters, const int32_t* init_idx,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * kv_cluster_build with timing: initial positions from init_idx, or from the
 * seed when init_idx is NULL. assign_events (host array of 2*iters
 * hipEvent_t handles created by the caller, or NULL) receives, for iteration
 * t, events recorded on `stream` right before and right after the launch of
 * that iteration's assignment kernel (the matrix-core pass for bf16 keys, the
 * fp64 pass for fp32 keys). Otherwise identical to kv_cluster_build.
 */
kvc_status kv_cluster_build_timed(kvc_index* idx, const void* keys, int L, int iters, uint64_t seed,
                                  const int32_t* init_idx, void* ws, size_t ws_bytes, void* const* assign_events,
                                  void* stream);

/*
 * Decode-time append of n_new tokens per head (rows idx->n_tokens ..
 * idx->n_tokens+n_new-1). k_new and v_new are [heads, n_new, d] in
 * idx->dtype and are written into the caches; each new key joins the cluster
 * of largest cosine similarity under the current centroid operand, whose
 * centroids do not move. Sizes, labels and the appended list are updated;
 * idx->n_tokens (and idx->window_start with it) advances on the host. The
 * clusters in use are the candidates (idx->c_active). Returns
 * KVC_ERR_CAPACITY, enqueuing nothing, if the tokens would not fit, and
 * KVC_ERR_INVALID_ARG while a window is open (window_start < n_tokens). (The
 * pages cluster generated tokens periodically instead, III.B: see
 * kv_cluster_append_window; joining the nearest centroid is the per-token
 * alternative this call provides.)
 */
kvc_status kv_cluster_append(kvc_index* idx, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      int n_new, void* stream);

/*
 * Decode-time append of n_new generated tokens per head to the window
 * (III.B: generated tokens are clustered on their own, every m decoding
 * steps; Sys-A): k_new and v_new ([heads, n_new, d], idx->dtype) become rows
 * idx->n_tokens .. idx->n_tokens+n_new-1 of the caches with label -1, and
 * idx->n_tokens advances on the host. Every selection recalls the window's
 * tokens right after the attention sinks until kv_cluster_cluster_window
 * clusters them. Requires a built index; KVC_ERR_CAPACITY if the tokens would
 * not fit.
 */
kvc_status kv_cluster_append_window(kvc_index* idx, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                             int n_new, void* stream);

/* Bytes of workspace kv_cluster_cluster_window needs for a window of m tokens. */
size_t kv_cluster_window_workspace_bytes(int heads, int m, int n_clusters, int iters);

/*
 * Clustering of the window (III.B: the generated tokens alone, into a few new
 * centroids, 4 every 320 steps on the pages; Sys-A): the m = n_tokens -
 * window_start window tokens of every head are clustered into n_clusters
 * clusters by `iters` iterations of the same cosine k-means as
 * kv_cluster_build, from the initial centroids at init_idx ([heads,
 * n_clusters] int32 token positions, distinct, in [window_start, n_tokens);
 * one out of range sets bit 0 of *idx->dev_flags and row 0 is used instead).
 * The new clusters take ids c_active .. c_active+n_clusters-1 (centroids,
 * operand, sizes, offsets after those of the existing clusters, members
 * after the existing members, labels); the existing clusters do not change.
 * With idx->packed set, the new members' rows are added to the packed copy
 * (read from k_cache and v_cache). Then c_active grows by n_clusters and the
 * window is empty (window_start = n_tokens). Requires 1 <= n_clusters <= m,
 * c_active + n_clusters <= the slots per head, iters >= 1, and a workspace of
 * kv_cluster_window_workspace_bytes(heads, m, n_clusters, iters) bytes
 * (contents need not be initialised).
 */
kvc_status kv_cluster_cluster_window(kvc_index* idx, const void* k_cache, const void* v_cache, int n_clusters, int iters,
                              const int32_t* init_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Cluster-granular selection (III.C; Sys-C, Fig. 8) for every KV head h:
 *   - the G = q_heads / heads query heads of h are summed (fp64),
 *   - score_k = fp64 dot product of that sum with centroid k (ascending
 *     channel order), the logit of the centroid's attention weight,
 *   - the idx->n_sink attention sinks come first (tokens 0 .. n_sink-1),
 *     then the window (tokens window_start .. n_tokens-1), in position
 *     order and as many as B allows; then the clusters in use are taken in
 *     order of (score descending, id ascending), each contributing its
 *     tokens in ascending position order, until B tokens are taken; the last
 *     cluster is trimmed.
 * q is [q_heads, d] in idx->dtype. sel_ids [heads, B] receives the selected
 * token positions (in that order; -1 past the count) and sel_count [heads]
 * receives min(B, n_sink + window + tokens in the clusters). Requires B >= 1
 * and G <= 8.
 */
kvc_status kv_cluster_select(const kvc_index* idx, const void* q, int q_heads, int B, int32_t* sel_ids,
                      int32_t* sel_count, void* stream);

/* Bytes of workspace kv_sparse_decode needs. */
size_t kv_sparse_decode_workspace_bytes(int heads, int q_heads, int d, int B);

/*
 * Single-query attention over the recalled tokens (II.A; III.A); requires
 * ceil(B / 64) * G <= 512 (B <= 4096 at G = 8). For query head g (KV head
 * h = g / G):
 *   out[g] = sum_i softmax_i(scale * q_g . K[h, i]) V[h, i]
 * over i in sel_ids[h*B .. h*B + sel_count[h]) (fp32 accumulation, fp32
 * output [q_heads, d]; zero when sel_count[h] is 0). k_cache and v_cache are
 * [heads, capacity, d] in `dtype`, q is [q_heads, d] in `dtype`. A count
 * outside [0, B] is taken as its nearest bound, and entries outside [0,
 * capacity) are skipped (they get no weight). The selected set is split into blocks
 * of 64 tokens whose partial results (running max, sum, output) go to the
 * workspace (kv_sparse_decode_workspace_bytes(heads, q_heads, d, B) bytes,
 * contents need not be initialised) and are merged by a second kernel.
 */
kvc_status kv_sparse_decode(const void* q, int q_heads, const void* k_cache, const void* v_cache, int dtype, int heads,
                     int capacity, int d, const int32_t* sel_ids, const int32_t* sel_count, int B, float scale,
                     float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * kv_sparse_decode for callers that cannot allocate device memory or hand
 * over a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The same kernels and the same result;
 * the split-K partial results go to a fixed device scratch of
 * KVC_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends (a static device array; no allocation, no
 * allocating library call). The caller still passes inputs and output.
 * Returns KVC_ERR_TOO_LARGE, enqueuing nothing, when the request needs more
 * than that (kv_sparse_decode_workspace_bytes(heads, q_heads, d, B) >
 * KVC_NOALLOC_SCRATCH_BYTES), and the other status codes as
 * kv_sparse_decode. Every call on one GPU shares its scratch, so calls that
 * overlap on one GPU (concurrent streams) race; calls ordered on one stream
 * do not. Nothing in the scratch needs clearing between calls.
 */
#define KVC_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
kvc_status kv_sparse_decode_noalloc(const void* q, int q_heads, const void* k_cache, const void* v_cache, int dtype,
                                    int heads, int capacity, int d, const int32_t* sel_ids,
                                    const int32_t* sel_count, int B, float scale, float* out, void* stream);

/*
 * Cluster-ordered copy of the keys and values of the index's main part: row i
 * of head h of idx->k_packed / idx->v_packed becomes row token_ids[h][i] of
 * k_cache / v_cache ([heads, capacity, d], idx->dtype), for i <
 * offsets[h][c_active] (the built tokens and those clustered from windows).
 * The members of each cluster then lie in consecutive rows, and
 * kv_cluster_select_decode reads the selected main-part tokens from the copy
 * (sinks, window tokens and tokens appended by kv_cluster_append still come
 * from the caches). Sets idx->packed to 1; kv_cluster_build resets it, and
 * kv_cluster_cluster_window extends the copy. Costs a second copy of that
 * part of the caches. Requires a built index and both packed arrays;
 * otherwise KVC_ERR_INVALID_ARG.
 */
kvc_status kv_cluster_pack(kvc_index* idx, const void* k_cache, const void* v_cache, void* stream);

/*
 * kv_cluster_select followed by kv_sparse_decode in one kernel (several
 * blocks per KV head, each making the selection): the same selection and the
 * same attention, without the selected ids leaving the chip. With
 * idx->packed set, the selected built tokens are read from the packed copy
 * (the same values, consecutive rows per cluster). k_cache and v_cache are
 * [heads, idx->capacity, d] in idx->dtype; q is [q_heads, d]; out is fp32
 * [q_heads, d]. sel_ids [heads, B] and sel_count [heads] are optional (NULL)
 * copies of the selection. Requires G = q_heads / heads in {1, 2, 4, 8}.
 * ws is optional. Without it, every block of a head scores all the selected
 * keys and weights a share of the value channels. With it (at least
 * kv_cluster_select_decode_workspace_bytes(heads, q_heads, d) bytes; bf16 and
 * G <= 4 only, otherwise unused), the blocks of a head split the selected
 * tokens instead and write partial results (running maximum, sum and output);
 * the last block of each head to finish merges them: the same attention up
 * to fp32 summation order. The workspace starts with one arrival counter per
 * KV head (int32, the first 4 * heads bytes rounded up to 256), which must be
 * zero before the first call on that workspace; every call leaves them zero
 * (the rest need not be initialised). Calls that share a workspace must not
 * overlap. ws_bytes is ignored when ws is
 * NULL; a smaller ws gives KVC_ERR_WORKSPACE.
 */
size_t kv_cluster_select_decode_workspace_bytes(int heads, int q_heads, int d);
kvc_status kv_cluster_select_decode(const kvc_index* idx, const void* q, int q_heads, const void* k_cache,
                             const void* v_cache, int B, float scale, float* out, int32_t* sel_ids,
                             int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/*
 * GPU cache of selected clusters for offloaded KV (Sys-A: the KV lives in CPU
 * memory and the selected clusters are loaded at each decoding step; Sys-D: a
 * GPU cache keeps the selected KV and cluster labels of the last R decoding
 * steps, and only clusters absent from it are loaded; the pages choose R = 1).
 * The caller allocates every array (device memory) and sets R and B;
 * kv_cluster_cache_reset fills the table and counters.
 */
typedef struct kvc_cluster_cache {
  int32_t R;        /* decoding steps whose selections stay cached, R >= 1 */
  int32_t B;        /* token budget of every cached step (the rows of one step) */
  int32_t step;     /* host mirror: cached steps since the last reset */
  int32_t reserved; /* 0 */
  void* k;          /* [heads, (R + 1) * B, d] in the index's dtype: step t's rows are region
                       t mod (R + 1), in selection order */
  void* v;          /* the value rows, same layout */
  int32_t* table;   /* [heads, S, 3] (S = cluster slots per head): for each cluster, the step of its
                       last selection, its first row in the cache and the members taken then */
  int64_t* stats;   /* [heads, 4], accumulated over steps: clusters selected, clusters found in the
                       cache, cluster tokens selected, tokens copied from the cache */
} kvc_cluster_cache;

/* Empties the cache (no cluster cached, counters 0, step 0). Also needed
 * after every kv_cluster_build of the index: cluster ids change meaning. */
kvc_status kv_cluster_cache_reset(const kvc_index* idx, kvc_cluster_cache* cache, void* stream);

/* Bytes of workspace kv_cluster_cached_select_decode needs. */
size_t kv_cluster_cache_workspace_bytes(int heads, int q_heads, int d, int B);

/*
 * kv_cluster_select_decode through the cluster cache, for KV that lives in
 * host memory: k_cache / v_cache (and the packed copy, when idx->packed is
 * set) may be pinned host memory mapped into the GPU's address space (or
 * device memory). At step t = cache->step, for every KV head:
 *   - the selection of kv_cluster_select with B = cache->B;
 *   - the selected rows are assembled, in selection order, into region
 *     t mod (R + 1) of the cache. A member of cluster k is copied from the
 *     cache when k was last selected at a step in [t - R, t - 1] with at
 *     least that many members taken (members are taken in index order, so the
 *     cached ones are a prefix); every other row (and every sink and window
 *     token) is read from its source. The table and counters are updated;
 *   - attention over the assembled rows (the split path of kv_sparse_decode),
 *     fp32 out [q_heads, d].
 * cache->step then advances on the host. sel_ids [heads, B] and sel_count
 * [heads] (optional) receive the selection as token ids. Requires G =
 * q_heads / heads in {1, 2, 4, 8}, ceil(B / 64) * G <= 512, R >= 1, B >= 1,
 * and a workspace of kv_cluster_cache_workspace_bytes(heads, q_heads, d, B)
 * bytes (contents need not be initialised).
 */
kvc_status kv_cluster_cached_select_decode(const kvc_index* idx, kvc_cluster_cache* cache, const void* q, int q_heads,
                                    const void* k_cache, const void* v_cache, float scale, float* out,
                                    int32_t* sel_ids, int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace kv_dense_decode needs. */
size_t kv_dense_decode_workspace_bytes(int heads, int q_heads, int d, int n);

/*
 * Full single-query attention over the first n rows of every head, the
 * computation that cluster-granular recall approximates (II.A; III.A) and the
 * full-KV comparator of the decode benchmark: for query head g (KV head
 * h = g / G),
 *   out[g] = sum_{i < n} softmax_i(scale * q_g . K[h, i]) V[h, i]
 * with bf16 inputs, fp32 accumulation and fp32 output [q_heads, d].
 * k_cache and v_cache are [heads, capacity, d] bf16 (KVC_BF16 only; KVC_F32
 * returns KVC_ERR_UNSUPPORTED), q is [q_heads, d]. The rows are split into
 * blocks whose partial results go to the workspace
 * (kv_dense_decode_workspace_bytes(heads, q_heads, d, n) bytes, contents need
 * not be initialised) and are merged by a second kernel. Requires
 * 1 <= n <= capacity and G in {1, 2, 4, 8}.
 */
kvc_status kv_dense_decode(const void* q, int q_heads, const void* k_cache, const void* v_cache, int dtype, int heads,
                    int capacity, int d, int n, float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * The canonical index of every head (main and appended parts merged):
 * offsets [heads, S+1] (S = slots per head; entries past c_active hold the
 * total) and token_ids [heads, capacity] with each cluster's members in
 * ascending order, as a stable counting sort of all labels of clustered
 * tokens would give (Sys-C). For tests and checkpoints.
 */
kvc_status kv_cluster_export_csr(const kvc_index* idx, int32_t* offsets, int32_t* token_ids, void* stream);

/*
 * Single steps of the build, for checking each kernel on its own (an index
 * without attention sinks: kv_cluster_debug_update rejects n_sink != 0).
 *  - kv_cluster_debug_assign: labels [heads, capacity] of the first L keys
 *    under the given operand chat [heads, cpad(C), d] (same rule as the
 *    build; this chat has cpad(C) rows per head whatever the slot count). top2 (optional, [heads, L, 2] fp32) receives the matrix-core
 *    best and runner-up scores of bf16 keys; flagged (optional, [1]) the
 *    number of keys whose order the fp32 scores could not certify and which
 *    were re-scored in fp64. ws as for the build.
 *  - kv_cluster_debug_update: from labels [heads, capacity] of the first L
 *    keys, the index arrays (sizes, offsets, token_ids) and the centroid
 *    update plus normalisation, writing idx->centroids (in: previous
 *    centroids, kept for empty clusters) and idx->centroids_op.
 */
kvc_status kv_cluster_debug_assign(const kvc_index* idx, const void* keys, int L, const void* chat, int32_t* labels,
                            float* top2, int32_t* flagged, void* ws, size_t ws_bytes, void* stream);
kvc_status kv_cluster_debug_update(kvc_index* idx, const void* keys, int L, void* ws, size_t ws_bytes, void* stream);

/*
 * The selection scores of kv_cluster_select (III.C; Sys-C: clusters rank by
 * the attention weight of their centroid to the query): scores [heads,
 * c_active] (device, fp64) receives, for KV head h and cluster k, the fp64
 * chain over ascending channels j of qbar_j * centroids[h][k][j], where
 * qbar_j is the fp64 sum over g = 0 .. G-1 (ascending) of q[h*G + g][j] and G
 * = q_heads / heads; the very values the selection orders. For tests.
 */
kvc_status kv_cluster_debug_scores(const kvc_index* idx, const void* q, int q_heads, double* scores, void* stream);

/* Static text for a status code. */
const char* kv_cluster_status_string(kvc_status s);

#ifdef __cplusplus
}
#endif

#endif /* KVCLUSTER_H */
