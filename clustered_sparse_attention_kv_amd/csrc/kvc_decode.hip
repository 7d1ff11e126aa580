// Decode-time kernels: nearest-centroid append, cluster-granular selection,
// and split-K single-query attention over the recalled tokens.
//
// Method: ClusterKV (arXiv 2412.03213), paper summary page sections III.C
// "Selection at the Granularity of Semantic Clusters", Sys-C "Selection and
// Indexing" (Fig. 8: sizes and prefix sums decide which clusters fit; the last
// one is trimmed; indexing works per KV head), II.A "LLM Inference and KV
// Cache" (the latest query attends to the cached keys and values) and III.A
// "Problem Formulation" (attention over the B selected tokens).
#include <mutex>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// ---------------------------------------------------------------------------
// a6: append n_new tokens per head. One block per head; tokens in order.
// label = argmax_k of the fp64 chain k_new . chat_k (ascending channel order,
// lowest k on ties), the same rule as the build's assignment, over the C
// clusters in use (per-head strides: cs slots, cps operand rows); under the
// L2 distance the score is the chain minus half the fp64 chain of chat_kj^2. The token id
// joins the end of its cluster's appended list (ids only grow, so lists stay
// ascending), shifting the later clusters' entries right by one; the prefix
// entries of every slot after the cluster advance, so unused slots keep the
// list's total.
constexpr int APP_THREADS = 512;  // one thread per cluster (C <= 512)
template <typename KT>
__global__ __launch_bounds__(APP_THREADS) void append_kernel(KT* __restrict__ kc, KT* __restrict__ vc, long long head_stride,
                                                     const KT* __restrict__ knew, const KT* __restrict__ vnew,
                                                     int n_new, int n0, const KT* __restrict__ chat, int C, int cs,
                                                     int cps, int metric, int32_t* __restrict__ labels, long long cap,
                                                     int32_t* __restrict__ sizes, int32_t* __restrict__ app_offsets,
                                                     int32_t* __restrict__ app_ids) {
  __shared__ double kv[D];
  __shared__ double rs[APP_THREADS / WAVE];
  __shared__ int rk[APP_THREADS / WAVE];
  __shared__ double s_score0;  // cluster 0's score
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t* aoff = app_offsets + (size_t)h * (cs + 1);
  int32_t* aids = app_ids + (size_t)h * cap;
  const KT* Ch = chat + (size_t)h * cps * D;
  for (int t = 0; t < n_new; ++t) {
    const int pos = n0 + t;
    const KT* ks = knew + ((size_t)h * n_new + t) * D;
    const KT* vs = vnew + ((size_t)h * n_new + t) * D;
    if (tid < D) {
      kc[(size_t)h * head_stride + (size_t)pos * D + tid] = ks[tid];
      vc[(size_t)h * head_stride + (size_t)pos * D + tid] = vs[tid];
      kv[tid] = (double)load_f32(ks, tid);
    }
    __syncthreads();
    // thread tid scores centroid tid (C <= 512): half rows requested at once
    // in 16-byte pieces, then the fp64 chain over ascending j
    double best = -INFINITY;
    int bi = 0x7FFFFFFF;
    {
      constexpr int EPP = 16 / (int)sizeof(KT);  // elements per 16-byte piece
      constexpr int HP = D / EPP / 2;            // pieces per half row
      const int c0 = tid;
      const u32x4* r0 = reinterpret_cast<const u32x4*>(Ch + (size_t)(c0 < C ? c0 : 0) * D);
      double s0 = 0.0, nn0 = 0.0;
      const bool l2 = metric == M_L2;
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        u32x4 x0[HP];
#pragma unroll
        for (int i = 0; i < HP; ++i) x0[i] = r0[half * HP + i];
#pragma unroll
        for (int i = 0; i < HP; ++i)
#pragma unroll
          for (int e = 0; e < EPP; ++e) {
            float a;
            if constexpr (sizeof(KT) == 2)
              a = (e & 1) ? __uint_as_float(x0[i][e >> 1] & 0xFFFF0000u) : __uint_as_float(x0[i][e >> 1] << 16);
            else
              a = __uint_as_float(x0[i][e]);
            const double kj = kv[(half * HP + i) * EPP + e];
            s0 = fma(kj, (double)a, s0);
            if (l2) nn0 = fma((double)a, (double)a, nn0);
          }
      }
      if (l2) s0 = s0 - 0.5 * nn0;
      if (c0 < C && s0 > best) {  // a NaN or -inf score never leads
        best = s0;
        bi = c0;
      }
      if (tid == 0) s_score0 = s0;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bi, off);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (lane == 0) {
      rs[w] = best;
      rk[w] = bi;
    }
    __syncthreads();
    best = rs[0];
    bi = rk[0];
    for (int v = 1; v < APP_THREADS / WAVE; ++v)
      if (rs[v] > best || (rs[v] == best && rk[v] < bi)) {
        best = rs[v];
        bi = rk[v];
      }
    // non-finite scores follow the sequential rule (start from cluster 0, move
    // only to a strictly larger score): when cluster 0 scores NaN, or no score
    // exceeds -inf, the token joins cluster 0
    const double sc0 = s_score0;
    const int lab = (bi >= C || sc0 != sc0) ? 0 : bi;
    // insert pos at the end of cluster lab's appended segment
    const int a = aoff[cs];            // entries before this append
    const int p = aoff[lab + 1];
    // every thread holds both bounds before any thread moves them (the prefix
    // increments below), so all threads run the shift loop the same number of
    // times and meet its barriers together
    __syncthreads();
    for (int hiend = a; hiend > p; hiend -= APP_THREADS) {  // shift right to left, one chunk at a time
      const int lo = hiend - APP_THREADS > p ? hiend - APP_THREADS : p;
      const int e = lo + tid;
      int v = 0;
      if (e < hiend) v = aids[e];
      __syncthreads();
      if (e < hiend) aids[e + 1] = v;
      __syncthreads();
    }
    if (tid == 0) {
      aids[p] = pos;
      sizes[(size_t)h * cs + lab] += 1;
      labels[(size_t)h * cap + pos] = lab;
    }
    for (int k = lab + 1 + tid; k <= cs; k += APP_THREADS) aoff[k] += 1;
    __syncthreads();
  }
}

// Tokens that join the window of generated tokens (III.B; they are clustered
// later, together): rows n0 .. n0+n_new-1 of the caches, label -1.
template <typename KT>
__global__ __launch_bounds__(256) void window_append_kernel(KT* __restrict__ kc, KT* __restrict__ vc, long long cap,
                                                            const KT* __restrict__ knew,
                                                            const KT* __restrict__ vnew, int n_new, int n0,
                                                            int32_t* __restrict__ labels) {
  const int h = blockIdx.y;
  for (int e = blockIdx.x * 256 + threadIdx.x; e < n_new * D; e += gridDim.x * 256) {
    const int t = e / D, j = e % D;
    const size_t dst = ((size_t)h * cap + n0 + t) * D + j, src = ((size_t)h * n_new + t) * D + j;
    kc[dst] = knew[src];
    vc[dst] = vnew[src];
    if (j == 0) labels[(size_t)h * cap + n0 + t] = -1;
  }
}

// ---------------------------------------------------------------------------
// a7-a9: selection, computed by one block of 512 threads per KV head (C <= 512).
//  1. qbar_j = fp64 sum over the head's G query heads (ascending g).
//  2. score_k = fp64 chain qbar . c_k over ascending j; thread k owns cluster k.
//  3. Order (score, k) by score descending, k ascending. Only clusters that
//     can be selected need an order: a histogram of the scores (256 equal bins
//     between the lowest and the highest, each cluster counted with its size)
//     gives the bin where the size summed from the top first reaches the
//     budget left for clusters (B less the sinks and the window); the clusters
//     in that bin and above are the candidates, every other one ranks below
//     them. Up to 64 candidates are sorted by one wave (bitonic, wave
//     shuffles only); more fall back to a bitonic sort of all 512 entries,
//     strides below 64 through wave shuffles, larger ones through LDS.
//  4. Exclusive prefix W_r of sizes in rank order: rank r starts at W_r.
//  5. Output position p < min(B, N) belongs to the last rank r with W_r <= p
//     and takes member p - W_r of that cluster (built part, then appended
//     part), so every cluster before the cut is whole and the last is trimmed.
//     The attention sinks and the window of unclustered generated tokens come
//     before every cluster.
constexpr int SEL_THREADS = 512;

struct SelShared {
  double qbar[D];
  unsigned long long xkey[SEL_THREADS];
  int xid[SEL_THREADS];
  int W[SEL_THREADS];      // exclusive prefix of sizes in rank order
  int obase[SEL_THREADS];  // offsets[k_r]
  int nbase[SEL_THREADS];  // built members of k_r
  int abase[SEL_THREADS];  // app_offsets[k_r]
  int mn[SEL_THREADS], mo[SEL_THREADS], mb[SEL_THREADS], ma[SEL_THREADS];  // per cluster k: size, offset, built, app offset
  int wsum[SEL_THREADS / WAVE];
  int total;
  double wlo[SEL_THREADS / WAVE], whi[SEL_THREADS / WAVE];  // per wave: lowest and highest score
  int hist[256];                                            // cluster sizes per score bin
  unsigned long long ckey[WAVE];                            // candidates (any order)
  int cid[WAVE];
  int ncand;
  int nrank;  // ranks that can hold clusters: 64 after the candidates' sort, else all
  // early gather (select_phase<true>): clusters above the cut bin, one ballot
  // per wave, and the flag wave 0 raises once the ranks are in LDS
  unsigned long long cmask[SEL_THREADS / WAVE];
  int ready;
};

// Value of lane (lane ^ S) within the wave, with lane operations only (no
// LDS): DPP quad permutes for S = 1, 2; for S = 4, 8 the partner lies in the
// same row of 16, S lanes up or down, so two DPP row shifts and a select; for
// S = 16 and 32 a swap of 16-lane rows or 32-lane halves (v_permlane16_swap /
// v_permlane32_swap of the value with itself gives the lower partner rows in
// one result and the upper ones in the other) and a select.
template <int S>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (S == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  else if constexpr (S == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  else if constexpr (S == 4 || S == 8) {
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x100 + S, 0xF, 0xF, false);  // row_shl: lane + S
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x110 + S, 0xF, 0xF, false);  // row_shr: lane - S
    return (threadIdx.x & S) ? dn : up;
  } else if constexpr (S == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 16) ? p[0] : p[1]);
  } else {
    static_assert(S == 32, "lane distance");
    const auto p = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 32) ? p[0] : p[1]);
  }
}

// fp64 minimum and maximum over the wave (every lane gets them): DPP steps on
// both 32-bit halves, as wave_max below.
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ double dpp64(double v) {
  const unsigned long long x = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, RM, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(x >> 32), (int)(x >> 32), CTRL, RM, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ __forceinline__ void wave_min_max(double& lo, double& hi) {
  lo = fmin(lo, dpp64<0xB1>(lo));
  hi = fmax(hi, dpp64<0xB1>(hi));
  lo = fmin(lo, dpp64<0x4E>(lo));
  hi = fmax(hi, dpp64<0x4E>(hi));
  lo = fmin(lo, dpp64<0x141>(lo));
  hi = fmax(hi, dpp64<0x141>(hi));
  lo = fmin(lo, dpp64<0x140>(lo));
  hi = fmax(hi, dpp64<0x140>(hi));
  lo = fmin(lo, dpp64<0x142, 0xA>(lo));
  hi = fmax(hi, dpp64<0x142, 0xA>(hi));
  lo = fmin(lo, dpp64<0x143, 0xC>(lo));
  hi = fmax(hi, dpp64<0x143, 0xC>(hi));
  const unsigned long long l = (unsigned long long)__double_as_longlong(lo);
  const unsigned long long u = (unsigned long long)__double_as_longlong(hi);
  lo = __longlong_as_double((long long)(((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(l >> 32), 63) << 32) |
                                        (unsigned)__builtin_amdgcn_readlane((int)l, 63)));
  hi = __longlong_as_double((long long)(((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(u >> 32), 63) << 32) |
                                        (unsigned)__builtin_amdgcn_readlane((int)u, 63)));
}

// Inclusive prefix sum over the 64 lanes: row shifts by 1, 2, 4, 8 (zero
// shifted in) scan each row of 16, then the last lane of row 0 (2) is added
// to row 1 (3), and the last lane of row 1 to rows 2 and 3 (DPP, no LDS).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// One compare-exchange stage of the bitonic sort over the block (thread t
// holds element t): partner t ^ STRIDE, through LDS when it lies in another
// wave. Sub-sequences of SIZE end up best-first where t & SIZE == 0.
template <int SIZE, int STRIDE, typename Sh>
__device__ __forceinline__ void bitonic_stage(Sh& S, unsigned long long& key, int& id, int tid) {
  unsigned long long ok;
  int oi;
  if constexpr (STRIDE >= WAVE) {
    S.xkey[tid] = key;
    S.xid[tid] = id;
    __syncthreads();
    ok = S.xkey[tid ^ STRIDE];
    oi = S.xid[tid ^ STRIDE];
    __syncthreads();
  } else {
    const int lo = lane_xor<STRIDE>((int)(key & 0xFFFFFFFFull));
    const int hi = lane_xor<STRIDE>((int)(key >> 32));
    ok = ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
    oi = lane_xor<STRIDE>(id);
  }
  const bool want_better = ((tid & SIZE) == 0) == ((tid & STRIDE) == 0);
  const bool partner_better = ok > key || (ok == key && oi < id);
  if (want_better == partner_better) {
    key = ok;
    id = oi;
  }
  if constexpr (STRIDE > 1) bitonic_stage<SIZE, STRIDE / 2>(S, key, id, tid);
}


template <int SIZE, int N, typename Sh>
__device__ __forceinline__ void bitonic_sort(Sh& S, unsigned long long& key, int& id, int tid) {
  bitonic_stage<SIZE, SIZE / 2>(S, key, id, tid);
  if constexpr (SIZE < N) bitonic_sort<SIZE * 2, N>(S, key, id, tid);
}

// qbar_j of KV head h: the fp64 sum over its G query heads in ascending order
// (III.C ranks clusters by their centroid's attention weight to the query; the
// query heads sharing a KV head share one selection).
// (all G values are requested before the sum, which runs in ascending g)
template <typename QT>
__device__ __forceinline__ double query_sum(const QT* __restrict__ q, int G, int h, int j) {
  float v[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) v[g] = g < G ? load_f32(q, ((size_t)h * G + g) * D + j) : 0.f;
  double s = 0.0;
#pragma unroll
  for (int g = 0; g < 8; ++g)
    if (g < G) s = s + (double)v[g];
  return s;
}

// Score of cluster k: the fp64 chain over ascending j of qbar_j * c_kj. The
// centroids come from the chunk-major copy [d/4, cs, 4] of the head: chunk jj
// of row k sits at ((jj * cs) + k) * 16 bytes, so the 64 lanes of a wave
// scoring consecutive clusters read 1 KiB contiguously. The row's 32 chunks
// are requested together (centroid_load), so that a caller can issue them
// before it waits for anything else, and then chained (centroid_chain).
struct CentroidRow {
  f32x4 v[D / 4];
};
__device__ __forceinline__ void centroid_load(CentroidRow& r, const float* __restrict__ cent_t_head, int cs, int k) {
  const f32x4* ct = reinterpret_cast<const f32x4*>(cent_t_head) + k;
#pragma unroll
  for (int jj = 0; jj < D / 4; ++jj) r.v[jj] = ct[(size_t)jj * cs];
}
__device__ __forceinline__ double centroid_chain(const double* qbar, const CentroidRow& r) {
  double sc = 0.0;
#pragma unroll
  for (int jj = 0; jj < D / 4; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc = fma(qbar[4 * jj + i], (double)r.v[jj][i], sc);
  return sc;
}

// Returns the cluster id of rank tid (ids >= X.ca are padding).
// EARLY (with early_ok): when at most 64 candidates need an order, wave 0
// sorts them while the other waves return at once; *early is then true, the
// ranks (W, obase, ..., total, nrank) are valid once S.ready is 1 (wave 0
// sets it after writing them, with a release fence), and cmask marks the
// clusters in bins above the cut: their sizes sum to less than the budget
// left for clusters, so each is selected whole and they hold the first ranks.
// Otherwise *early is false and every rank is in LDS on return (block
// barrier), as without EARLY.
template <bool EARLY = false, typename QT>
__device__ __forceinline__ int select_phase(SelShared& S, const QT* __restrict__ q, int G, const IndexView& X, int h,
                                            int B, bool early_ok = false, bool* early = nullptr) {
  if constexpr (EARLY) *early = false;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int C = X.ca, cs = X.cs;
  // Requests in this order: the query and the per-cluster metadata, then the
  // thread's centroid row (32 chunks at once). Loads complete in order, so the
  // LDS stores of the query sum and the metadata wait for their own loads
  // only, and the centroid rows arrive while the block meets at the barrier.
  // (Every block of a head streams the head's whole centroids and runs every
  // chain: sharing the scores between a head's blocks through device memory
  // costs several device-coherent round trips, more than the reads it saves,
  // and streaming the block's own share first with the rest after a barrier,
  // to find the rest in L2, serialises the fp64 chains and is slower too.)
  double qs = 0.0;
  if (tid < D) qs = query_sum(q, G, h, tid);
  int mn = 0, mo = 0, mo1 = 0, ma = 0;
  if (tid < C) {
    mn = X.sizes[(size_t)h * cs + tid];
    mo = X.offsets[(size_t)h * (cs + 1) + tid];
    mo1 = X.offsets[(size_t)h * (cs + 1) + tid + 1];
    ma = X.app_offsets[(size_t)h * (cs + 1) + tid];
  }
  CentroidRow crow;
  if (tid < C) centroid_load(crow, X.cent_t + (size_t)h * cs * D, cs, tid);
  if (tid < C) {  // per-cluster metadata
    S.mn[tid] = mn;
    S.mo[tid] = mo;
    S.mb[tid] = mo1 - mo;
    S.ma[tid] = ma;
  }
  if (tid < D) S.qbar[tid] = qs;
  if (tid < 256) S.hist[tid] = 0;
  if (tid == 0) {
    S.ncand = 0;
    S.ready = 0;
  }
  __syncthreads();
  unsigned long long key = 0;
  int id = C + tid;  // padding entries: worst key, distinct ids past the clusters
  double sc = 0.0;
  if (tid < C) sc = centroid_chain(S.qbar, crow);
  if (tid < C) {
    key = ordered_key(sc);
    id = tid;
  }
  // lowest and highest score of the head
  {
    double lo = tid < C ? sc : INFINITY, hi = tid < C ? sc : -INFINITY;
    wave_min_max(lo, hi);
    if (lane == 0) {
      S.wlo[w] = lo;
      S.whi[w] = hi;
    }
  }
  __syncthreads();
  double smin = S.wlo[0], smax = S.whi[0];
#pragma unroll
  for (int v = 1; v < SEL_THREADS / WAVE; ++v) {
    smin = fmin(smin, S.wlo[v]);
    smax = fmax(smax, S.whi[v]);
  }
  // bin of each cluster: monotone in the score (rounding is monotone)
  int bin = 0;
  if (tid < C && smax > smin) {
    const double x = (sc - smin) * (256.0 / (smax - smin));
    bin = x >= 255.0 ? 255 : (int)x;
  }
  if (tid < C && S.mn[tid] > 0) atomicAdd(&S.hist[bin], S.mn[tid]);
  __syncthreads();
  const int bc = B - X.n_sink - X.nw;  // entries left for clusters
  int bstar;
  {
    // every wave: size in bins >= b for lane's bins 4 lane .. 4 lane + 3;
    // b* = the highest bin whose sum reaches bc (all bins when the clusters
    // hold fewer)
    int hb[4], t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hb[i] = S.hist[4 * lane + i];
      t += hb[i];
    }
    const int pre = wave_incl_scan(t);
    int suf = __builtin_amdgcn_readlane(pre, WAVE - 1) - pre;  // size in the bins of later lanes
    int nq = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      suf += hb[i];
      nq += suf >= bc ? 1 : 0;
    }
    nq = __builtin_amdgcn_readlane(wave_incl_scan(nq), WAVE - 1);
    bstar = bc <= 0 ? 256 : (nq > 0 ? nq - 1 : 0);
  }
  if constexpr (EARLY) {
    const unsigned long long cm = __ballot(tid < C && bin > bstar && S.mn[tid] > 0);
    if (lane == 0) S.cmask[w] = cm;
  }
  if (tid < C && bin >= bstar) {
    const int slot = atomicAdd(&S.ncand, 1);
    if (slot < WAVE) {
      S.ckey[slot] = key;
      S.cid[slot] = id;
    }
  }
  __syncthreads();
  const int ncand = S.ncand;
  if (ncand <= WAVE) {
    // one wave orders the candidates; every other rank is padding
    int fid = C + tid;
    if (w == 0) {
      unsigned long long k2 = lane < ncand ? S.ckey[lane] : 0ull;
      int i2 = lane < ncand ? S.cid[lane] : C + lane;
      // a network over the smallest power of two lanes that holds them (lanes
      // past it hold padding, which keeps its place at the end)
      if (ncand <= 16) bitonic_sort<2, 16>(S, k2, i2, lane);
      else if (ncand <= 32) bitonic_sort<2, 32>(S, k2, i2, lane);
      else bitonic_sort<2, WAVE>(S, k2, i2, lane);
      int n = 0, ob = 0, nb = 0, ab = 0;
      if (i2 < C) {
        n = S.mn[i2];
        ob = S.mo[i2];
        nb = S.mb[i2];
        ab = S.ma[i2];
      }
      const int x = wave_incl_scan(n);
      const int tot = __builtin_amdgcn_readlane(x, WAVE - 1);
      S.W[lane] = x - n;
      S.obase[lane] = ob;
      S.nbase[lane] = nb;
      S.abase[lane] = ab;
      for (int r = WAVE + lane; r < SEL_THREADS; r += WAVE) S.W[r] = tot;
      if (lane == 0) {
        S.total = tot;
        S.nrank = WAVE;
      }
      fid = i2;
      if constexpr (EARLY) {
        if (early_ok) {  // the ranks are in LDS: raise the flag after them
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          if (lane == 0) __hip_atomic_store(&S.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
    if constexpr (EARLY) {
      if (early_ok) {
        *early = true;
        return fid;
      }
    }
    __syncthreads();
    return fid;
  }
  if constexpr (EARLY) *early = false;
  // bitonic sort of all entries, best first ("better" = larger key, then smaller id)
  bitonic_sort<2, SEL_THREADS>(S, key, id, tid);
  // thread r now holds rank r; prefix of sizes in rank order
  int n = 0, ob = 0, nb = 0, ab = 0;
  if (id < C) {
    n = S.mn[id];
    ob = S.mo[id];
    nb = S.mb[id];
    ab = S.ma[id];
  }
  const int x = wave_incl_scan(n);
  if (lane == WAVE - 1) S.wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int v = 0; v < SEL_THREADS / WAVE; ++v) {
    base += v < w ? S.wsum[v] : 0;
    tot += S.wsum[v];
  }
  S.W[tid] = base + x - n;
  S.obase[tid] = ob;
  S.nbase[tid] = nb;
  S.abase[tid] = ab;
  if (tid == 0) {
    S.total = tot;
    S.nrank = SEL_THREADS;
  }
  __syncthreads();
  return id;
}

// Entry of member e of the cluster at rank r (built members first, then the
// appended ones).
__device__ __forceinline__ int rank_entry(const SelShared& S, int r, int e, const int32_t* __restrict__ ids_h,
                                          const int32_t* __restrict__ app_h, bool packed) {
  const int nb = S.nbase[r];
  if (e < nb) return packed ? S.obase[r] + e : ids_h[S.obase[r] + e];
  const int a = app_h[S.abase[r] + (e - nb)];
  return packed ? ~a : a;
}

// Entry at a position below n_sink + nw: a sink or a window token.
__device__ __forceinline__ int fixed_entry(int p, bool packed, const IndexView& X) {
  const int t = p < X.n_sink ? p : X.wlo + (p - X.n_sink);
  return packed ? ~t : t;
}

// Entry of member e of cluster k (built members first, then the appended
// ones): rank_entry with the cluster's own offsets.
__device__ __forceinline__ int cluster_entry(const SelShared& S, int k, int e, const int32_t* __restrict__ ids_h,
                                             const int32_t* __restrict__ app_h, bool packed) {
  const int nb = S.mb[k];
  if (e < nb) return packed ? S.mo[k] + e : ids_h[S.mo[k] + e];
  const int a = app_h[S.ma[k] + (e - nb)];
  return packed ? ~a : a;
}

// Position of the set bit of rank r (from 0) in m (r < popcount(m)).
__device__ __forceinline__ int nth_set_bit(unsigned long long m, int r) {
  int pos = 0;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) {
    const unsigned long long lo = m & ((1ull << sh) - 1ull);
    const int c = __popcll(lo);
    if (r >= c) {
      r -= c;
      m >>= sh;
      pos += sh;
    } else {
      m = lo;
    }
  }
  return pos;
}

// Entry at output position p (< n_sink + nw + total) of the ranked, trimmed
// selection: positions below n_sink are the attention sinks (tokens 0 ..
// n_sink - 1, always recalled first), the next nw the window of generated
// tokens not yet clustered (wlo .. wlo + nw - 1), the rest come from the
// clusters. The entry is the token id, or with a packed copy (packed = true)
// the row of the copy for a member of the index's main part (its position in
// the index, offset + member) and ~token for a sink, a window token or a token
// appended to a cluster (all read from the caches).
__device__ __forceinline__ int select_emit(const SelShared& S, int p, const int32_t* __restrict__ ids_h,
                                           const int32_t* __restrict__ app_h, bool packed, const IndexView& X) {
  if (p < X.n_sink + X.nw) return fixed_entry(p, packed, X);
  p -= X.n_sink + X.nw;
  int lo = 0, hi = S.nrank - 1;  // last r with W[r] <= p
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.W[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  return rank_entry(S, lo, p - S.W[lo], ids_h, app_h, packed);
}

// select_emit for two positions (p2 < 0: none), the two searches over the
// ranks interleaved so that their LDS round trips overlap.
__device__ __forceinline__ void select_emit2(const SelShared& S, int p1, int p2, const int32_t* __restrict__ ids_h,
                                             const int32_t* __restrict__ app_h, bool packed, const IndexView& X,
                                             int& e1, int& e2) {
  const int fixed = X.n_sink + X.nw;
  const int q1 = p1 - fixed, q2 = p2 - fixed;
  int r1 = 0, r2 = 0;  // last r with W[r] <= q (the ranks' starts do not decrease)
  for (int step = S.nrank >> 1; step >= 1; step >>= 1) {
    const int w1 = S.W[r1 + step], w2 = S.W[r2 + step];
    r1 += w1 <= q1 ? step : 0;
    r2 += w2 <= q2 ? step : 0;
  }
  e1 = q1 < 0 ? fixed_entry(p1, packed, X) : rank_entry(S, r1, q1 - S.W[r1], ids_h, app_h, packed);
  if (p2 >= 0) e2 = q2 < 0 ? fixed_entry(p2, packed, X) : rank_entry(S, r2, q2 - S.W[r2], ids_h, app_h, packed);
}

// Calls f(p, entry) for every position p in [p0, p1) of the selection (p1 <=
// the selected count): the sinks and the window by thread, then the clusters
// by wave, wave v taking ranks v, v + 8, ... and its lanes their members, so
// no position needs a search over the ranks.
template <typename F>
__device__ __forceinline__ void select_expand(const SelShared& S, int p0, int p1, const int32_t* __restrict__ ids_h,
                                              const int32_t* __restrict__ app_h, bool packed, const IndexView& X,
                                              F&& f) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fixed = X.n_sink + X.nw;
  for (int p = p0 + tid; p < p1 && p < fixed; p += SEL_THREADS) f(p, fixed_entry(p, packed, X));
  for (int r = w; r < SEL_THREADS; r += SEL_THREADS / WAVE) {
    const int st = fixed + S.W[r];  // position of the rank's first member
    if (st >= p1) break;            // the starts do not decrease
    const int en = fixed + (r + 1 < SEL_THREADS ? S.W[r + 1] : S.total);
    const int lo = st > p0 ? st : p0, hi = en < p1 ? en : p1;
    for (int p = lo + lane; p < hi; p += WAVE) f(p, rank_entry(S, r, p - st, ids_h, app_h, packed));
  }
}

// Row of a staged selection entry: a row of the packed copy (id >= 0) or the
// cache row ~id of an appended token (id < 0). Without a packed copy the
// entries are token ids and both bases are the cache.
template <typename KT>
__device__ __forceinline__ const KT* sel_row(const KT* packed_h, const KT* cache_h, int id) {
  return id >= 0 ? packed_h + (size_t)id * D : cache_h + (size_t)(~id) * D;
}

// Token id of a staged selection entry (for the optional copy of the selection).
__device__ __forceinline__ int sel_token(const int32_t* __restrict__ ids_h, int id, bool packed) {
  return packed ? (id >= 0 ? ids_h[id] : ~id) : id;
}

// Selected entries of a head: sinks and window first, then min(B, ...) in all.
__device__ __forceinline__ int select_count(const SelShared& S, const IndexView& X, int B) {
  const int n = X.n_sink + X.nw + S.total;
  return n < B ? n : B;
}

// The selection's scores of the clusters in use, spread over the whole chip:
// block (y, h) scores clusters 64 y .. 64 y + 63 of KV head h with the same
// query sum and chains as select_phase, into scores[h * stride + k], which the
// debug export returns.
constexpr int SCORE_THREADS = 64;
template <typename QT>
__global__ __launch_bounds__(SCORE_THREADS) void scores_kernel(const QT* __restrict__ q, int G, const IndexView X,
                                                               double* __restrict__ scores, int stride) {
  __shared__ double qbar[D];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int k = blockIdx.y * SCORE_THREADS + tid;
  CentroidRow crow;
  if (k < X.ca) centroid_load(crow, X.cent_t + (size_t)h * X.cs * D, X.cs, k);
  for (int j = tid; j < D; j += SCORE_THREADS) qbar[j] = query_sum(q, G, h, j);
  __syncthreads();
  if (k < X.ca) scores[(size_t)h * stride + k] = centroid_chain(qbar, crow);
}

hipError_t launch_scores(int dtype, const void* q, int G, const IndexView& x, int heads, double* scores, int stride,
                         hipStream_t st) {
  const dim3 grid(heads, (x.ca + SCORE_THREADS - 1) / SCORE_THREADS);
  if (dtype == DT_BF16)
    scores_kernel<uint16_t><<<grid, SCORE_THREADS, 0, st>>>((const uint16_t*)q, G, x, scores, stride);
  else
    scores_kernel<float><<<grid, SCORE_THREADS, 0, st>>>((const float*)q, G, x, scores, stride);
  return hipGetLastError();
}

hipError_t launch_debug_scores(int dtype, const void* q, int G, const IndexView& x, int heads, double* scores,
                               hipStream_t st) {
  return launch_scores(dtype, q, G, x, heads, scores, x.ca, st);
}

template <typename QT>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const QT* __restrict__ q, int G, const IndexView X,
                                                             int B, int32_t* __restrict__ sel_ids,
                                                             int32_t* __restrict__ sel_count) {
  __shared__ SelShared S;
  const int h = blockIdx.x, tid = threadIdx.x;
  select_phase(S, q, G, X, h, B);
  const int cnt = select_count(S, X, B);
  const int32_t* ids_h = X.token_ids + (size_t)h * X.cap;
  const int32_t* app_h = X.app_ids + (size_t)h * X.cap;
  select_expand(S, 0, cnt, ids_h, app_h, false, X, [&](int p, int ent) { sel_ids[(size_t)h * B + p] = ent; });
  for (int p = cnt + tid; p < B; p += SEL_THREADS) sel_ids[(size_t)h * B + p] = -1;
  if (tid == 0) sel_count[h] = cnt;
}

// ---------------------------------------------------------------------------
// Cluster cache for offloaded KV (Sys-A: the KV lives in CPU memory and the
// selected clusters are loaded at each decoding step; Sys-D: a GPU cache keeps
// the selected KV and the cluster labels of the last R decoding steps, so only
// clusters absent from it are loaded). One block per KV head, decode step t:
//  1. the selection of select_kernel (sinks, window, ranked clusters, trim);
//  2. region t mod (R + 1) of the head's cache buffer ([(R + 1) * B, d])
//     receives the selected rows in selection order (row region * B + p for
//     entry p). A member e of cluster k comes from the cache when k's table
//     entry was written at a step in [t - R, t - 1] and holds more than e
//     members (those rows sit in that step's region, never the current one);
//     every other row is read from its source: the packed copy or the caches,
//     in host memory when the KV is offloaded;
//  3. each selected cluster's entry becomes (t, its first row, members taken),
//     and the head's counters add: clusters selected, clusters found in the
//     cache, cluster tokens selected, tokens copied from the cache.
// Sinks and window tokens are read from their source at every step and are
// not counted. The decode then reads the region's rows in order.
template <typename KT>
__global__ __launch_bounds__(SEL_THREADS) void cache_assemble_kernel(
    const KT* __restrict__ q, int G, const IndexView X, const KT* __restrict__ kc, const KT* __restrict__ vc,
    const KT* __restrict__ kp, const KT* __restrict__ vp, int packed, int B, int R, int t, KT* __restrict__ ck,
    KT* __restrict__ cv, int32_t* __restrict__ table, long long* __restrict__ stats, int32_t* __restrict__ rows,
    int32_t* __restrict__ count, int32_t* __restrict__ sel_ids, int32_t* __restrict__ sel_count) {
  __shared__ SelShared S;
  __shared__ int hitlen[SEL_THREADS], hitrow[SEL_THREADS];  // per rank: cached members and their first row
  __shared__ long long red[4][SEL_THREADS / WAVE];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int id = select_phase(S, q, G, X, h, B);
  const int cnt = select_count(S, X, B);
  const int fixed = X.n_sink + X.nw;
  const int nclus = cnt > fixed ? cnt - fixed : 0;  // entries taken from clusters
  const int region = t % (R + 1);
  int32_t* tab = table + (size_t)h * X.cs * 3;
  // rank tid: members taken from its cluster and that cluster's cached entry
  int m = 0;
  if (id < X.ca) {
    m = nclus - S.W[tid];
    m = m < S.mn[id] ? m : S.mn[id];
    m = m > 0 ? m : 0;
  }
  int es = 0, er = 0, el = 0;
  if (m > 0) {
    es = tab[(size_t)id * 3];
    er = tab[(size_t)id * 3 + 1];
    el = tab[(size_t)id * 3 + 2];
  }
  const bool hit = m > 0 && es >= t - R && es < t && el > 0;
  hitlen[tid] = hit ? el : 0;
  hitrow[tid] = er;
  __syncthreads();
  if (m > 0) {  // the entry now points at this step's rows
    tab[(size_t)id * 3] = t;
    tab[(size_t)id * 3 + 1] = region * B + fixed + S.W[tid];
    tab[(size_t)id * 3 + 2] = m;
  }
  {
    long long v[4] = {m > 0 ? 1 : 0, hit ? 1 : 0, m, hit ? (el < m ? el : m) : 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v[i] += __shfl_xor(v[i], off);
      if (lane == 0) red[i][w] = v[i];
    }
  }
  const int32_t* ids_h = X.token_ids + (size_t)h * X.cap;
  const int32_t* app_h = X.app_ids + (size_t)h * X.cap;
  const size_t hb = (size_t)h * (R + 1) * B;
  KT* ckh = ck + hb * D;
  KT* cvh = cv + hb * D;
  const KT* kch = kc + (size_t)h * X.cap * D;
  const KT* vch = vc + (size_t)h * X.cap * D;
  const KT* kph = kp + (size_t)h * X.cap * D;
  const KT* vph = vp + (size_t)h * X.cap * D;
  constexpr int LPR = D * (int)sizeof(KT) / 16;  // lanes per row, 16 bytes each
  constexpr int RPP = SEL_THREADS / LPR;         // rows per pass
  const int l = tid % LPR;
  for (int p = tid / LPR; p < cnt; p += RPP) {
    const int ent = select_emit(S, p, ids_h, app_h, packed, X);
    const KT* sk = sel_row(kph, kch, ent);
    const KT* sv = sel_row(vph, vch, ent);
    if (p >= fixed) {
      const int pc = p - fixed;
      int lo = 0, hi = SEL_THREADS - 1;  // rank of entry p: last r with W[r] <= pc
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (S.W[mid] <= pc) lo = mid;
        else hi = mid - 1;
      }
      const int e = pc - S.W[lo];
      if (e < hitlen[lo]) {
        sk = ckh + (size_t)(hitrow[lo] + e) * D;
        sv = cvh + (size_t)(hitrow[lo] + e) * D;
      }
    }
    const u32x4 a = reinterpret_cast<const u32x4*>(sk)[l];
    const u32x4 b = reinterpret_cast<const u32x4*>(sv)[l];
    const size_t dst = ((size_t)region * B + p) * D;
    reinterpret_cast<u32x4*>(ckh + dst)[l] = a;
    reinterpret_cast<u32x4*>(cvh + dst)[l] = b;
    if (l == 0) {
      rows[(size_t)h * B + p] = region * B + p;
      if (sel_ids) sel_ids[(size_t)h * B + p] = sel_token(ids_h, ent, packed);
    }
  }
  if (sel_ids)
    for (int p = cnt + tid; p < B; p += SEL_THREADS) sel_ids[(size_t)h * B + p] = -1;
  __syncthreads();
  if (tid == 0) {
    count[h] = cnt;
    if (sel_count) sel_count[h] = cnt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      long long sum = 0;
#pragma unroll
      for (int v = 0; v < SEL_THREADS / WAVE; ++v) sum += red[i][v];
      stats[(size_t)h * 4 + i] += sum;
    }
  }
}

// Max / sum over the whole wave, result in every lane: row reductions by DPP,
// then row broadcasts (rows 0-1, then 0-3 into the upper half), and a read of
// lane 63.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over each row of 16 lanes, left in every lane of the row: quad swaps,
// then the mirrored half-row, then the mirrored row (DPP, no LDS traffic).
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// ---------------------------------------------------------------------------
// Rows of 8 channels as loaded: bf16 rows stay packed (4 VGPRs), fp32 rows are
// two 16-byte vectors.
template <typename KT>
struct Row8;
template <>
struct Row8<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ float at(int c) const {
    const uint32_t u = v[c >> 1];
    return (c & 1) ? __uint_as_float(u & 0xFFFF0000u) : __uint_as_float(u << 16);
  }
};
template <>
struct Row8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ float at(int c) const { return c < 4 ? a[c] : b[c - 4]; }
};

// ---------------------------------------------------------------------------
// a7-a11 fused: selection, gather and single-query attention of one KV head
// in one block of 512 threads, with no exchange between blocks.
// After the selection phase, the selected tokens are processed in chunks of
// 512: each wave gathers 64 rows (16 lanes per 128-channel row, 8 channels
// per lane, 16-byte loads), scores them against the G query heads sharing the
// KV head (q pre-scaled by scale * log2 e), and the block keeps an online
// softmax (running max and sum per query head, block-uniform) with per-lane
// partial outputs rescaled at each chunk. The waves' partial outputs are
// summed through LDS at the end.
template <typename KT, int G>
__global__ __launch_bounds__(SEL_THREADS) void select_decode_kernel(
    const KT* __restrict__ q, const IndexView X, const KT* __restrict__ kc, const KT* __restrict__ vc,
    const KT* __restrict__ kp, const KT* __restrict__ vp, int packed, int B, float qscale, float* __restrict__ out,
    int32_t* __restrict__ sel_ids, int32_t* __restrict__ sel_count) {
  constexpr int NW = SEL_THREADS / WAVE;                       // 8 waves
  constexpr int RS = (G <= 4 && sizeof(KT) == 2) ? 16 : (G <= 2 ? 8 : 4);  // row steps per load batch
  constexpr int NB = 16 / RS;                                  // batches per chunk
  constexpr bool V_EARLY = NB == 1;                            // V gathered together with K
  __shared__ SelShared S;
  __shared__ int sel[SEL_THREADS];
  __shared__ float sc[G][SEL_THREADS];
  __shared__ float wred[NW][G];
  __shared__ float ored[NW][G][D];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = lane >> 4, gl = lane & 15;
  select_phase(S, q, G, X, h, B);
  const int cnt = select_count(S, X, B);
  const long long cap = X.cap;
  if (sel_count && tid == 0) sel_count[h] = cnt;
  if (sel_ids)
    for (int p = cnt + tid; p < B; p += SEL_THREADS) sel_ids[(size_t)h * B + p] = -1;
  const int32_t* ids_h = X.token_ids + (size_t)h * cap;
  const int32_t* app_h = X.app_ids + (size_t)h * cap;
  const KT* Kh = kc + (size_t)h * cap * D + 8 * gl;
  const KT* Vh = vc + (size_t)h * cap * D + 8 * gl;
  const KT* Kph = kp + (size_t)h * cap * D + 8 * gl;
  const KT* Vph = vp + (size_t)h * cap * D + 8 * gl;

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    load8(q + ((size_t)h * G + g) * D + 8 * gl, qv[g]);
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[g][c] *= qscale;
  }
  float o[G][8];
  float m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[g][c] = 0.f;
  }

  for (int c0 = 0; c0 < cnt; c0 += SEL_THREADS) {
    const int nchunk = cnt - c0 < SEL_THREADS ? cnt - c0 : SEL_THREADS;
    {
      const int p = c0 + tid;
      const int ent = tid < nchunk ? select_emit(S, p, ids_h, app_h, packed, X) : 0;
      sel[tid] = ent;
      if (sel_ids && tid < nchunk) sel_ids[(size_t)h * B + p] = sel_token(ids_h, ent, packed);
    }
    __syncthreads();
    Row8<KT> vrow[V_EARLY ? RS : 1];
#pragma unroll 1
    for (int b = 0; b < NB; ++b) {
      Row8<KT> krow[RS];
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        const int t = w * 64 + (b * RS + r) * 4 + grp;
        const int id = t < nchunk ? sel[t] : 0;
        krow[r].load(sel_row(Kph, Kh, id));
        if constexpr (V_EARLY) vrow[r].load(sel_row(Vph, Vh, id));
      }
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        const int t = w * 64 + (b * RS + r) * 4 + grp;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) s = fmaf(qv[g][c], krow[r].at(c), s);
          s = row16_sum(s);
          if (gl == 0) sc[g][t] = t < nchunk ? s : -INFINITY;
        }
      }
    }
    __syncthreads();
    float mnew[G], f[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = sc[g][w * 64 + lane];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      if (lane == 0) wred[w][g] = m;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = m_run[g];
#pragma unroll
      for (int v = 0; v < NW; ++v) m = fmaxf(m, wred[v][g]);
      mnew[g] = m;
      f[g] = m_run[g] == -INFINITY ? 0.f : exp2f(m_run[g] - m);
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = sc[g][w * 64 + lane];
      const float p = mnew[g] == -INFINITY ? 0.f : exp2f(s - mnew[g]);
      sc[g][w * 64 + lane] = p;
      float l = p;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
      if (lane == 0) wred[w][g] = l;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float l = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) l += wred[v][g];
      l_run[g] = l_run[g] * f[g] + l;
      m_run[g] = mnew[g];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[g][c] *= f[g];
    }
#pragma unroll 1
    for (int b = 0; b < NB; ++b) {
      Row8<KT> vb[V_EARLY ? 1 : RS];
      if constexpr (!V_EARLY) {
#pragma unroll
        for (int r = 0; r < RS; ++r) {
          const int t = w * 64 + (b * RS + r) * 4 + grp;
          const int id = t < nchunk ? sel[t] : 0;
          vb[r].load(sel_row(Vph, Vh, id));
        }
      }
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        const int t = w * 64 + (b * RS + r) * 4 + grp;
        const Row8<KT>& vr = V_EARLY ? vrow[r] : vb[r];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = sc[g][t];
#pragma unroll
          for (int c = 0; c < 8; ++c) o[g][c] = fmaf(p, vr.at(c), o[g][c]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = o[g][c];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[g][c] = v;
    }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) ored[w][g][8 * gl + c] = o[g][c];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += SEL_THREADS) {
    const int g = e / D, j = e % D;
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) s += ored[v][g][j];
    out[((size_t)h * G + g) * D + j] = l_run[g] > 0.f ? s / l_run[g] : 0.f;
  }
}

// ---------------------------------------------------------------------------
// a7-a11 fused, bf16. After the selection phase each wave runs on its own
// over 64-token slices (wave w takes the block's slices w, w + 8, ...): it
// stages a slice's selected entries in its own part of LDS and keeps an
// online softmax per query head (running max, sum and partial output); the
// waves' states are merged once at the end. Per slice:
//  - query-key products on the matrix cores: the 64 keys form the A operand
//    of four v_mfma_f32_16x16x32_bf16 tiles of 16 rows (lane = row lane % 16,
//    16-byte piece 32 s + 8 (lane / 16) of the row, so one load instruction
//    reads 64 contiguous bytes of 16 rows); the B operand holds the G query
//    heads in its first columns; bf16 inputs, fp32 accumulation, and the
//    scale (times log2 e) multiplies the fp32 result;
//  - the scores go through wave-private LDS to a lane-per-token layout for
//    the max and sum (DPP reductions), and back as weights;
//  - the value rows are gathered and weighted in fp32 on the vector units.
// P blocks share each KV head (P = 2, or 4 and 8 when there are few heads,
// so that the grid still covers the chip), and all of them select. Then
// either (TS false) all score all keys, and block `part` gathers and weights
// channels [part D / P, (part + 1) D / P) of the values (8 channels per
// lane), writing those output channels; or (TS true) block `part` takes the
// slices part, part + P, ... (16 NT entries each) with all channels and
// writes its partial result (running maximum, sum, unnormalised output per
// query head) to part_out [heads, P, G, D + 2], and the last of the head's
// blocks to arrive merges the P partial results (below). The
// blocks of a head get block indices 8 apart, so the round-robin dispatch
// over the 8 XCDs places them on one XCD and its L2 serves the repeated reads
// of the keys and centroids; results do not depend on the placement.
template <int G, int P, bool TS, int NT = 4>
__global__ __launch_bounds__(SEL_THREADS) void select_decode_bf16_kernel(
    const uint16_t* __restrict__ q, const IndexView X, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp, int packed,
    int heads, int B, float qscale, float* __restrict__ out, int32_t* __restrict__ sel_ids,
    int32_t* __restrict__ sel_count, float* __restrict__ part_out, int32_t* __restrict__ arrive) {
  static_assert(G <= 8, "at most 8 query heads per KV head");
  constexpr int NW = SEL_THREADS / WAVE;
  constexpr int EMIT = 2048;                 // selected ids staged per pass
  constexpr int HC = TS ? D : D / P;         // value channels per block
  constexpr int RPS = WAVE / (HC / 8);       // value rows per load instruction (8 with 64 channels)
  constexpr int ST = 16 * NT;                // tokens per slice (NT tiles of 16 rows)
  static_assert(TS || NT == 4, "slices of 64 tokens without the token split");
  constexpr int VR = ST / RPS;               // value rows per lane per slice
  __shared__ SelShared S;
  __shared__ int sel[EMIT];
  constexpr int GP = G < 4 ? 4 : G;          // floats per token in pw (16-byte rows)
  __shared__ __align__(16) float pw[NW][64][GP];  // wave-private: scores, then weights, token-major
  __shared__ float ored[NW][G][HC];
  __shared__ float wm[NW][G], wl[NW][G];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int within = blockIdx.x % (8 * P);
  const int part = within / 8;
  const int h = blockIdx.x / (8 * P) * 8 + within % 8;
  if (h >= heads) return;  // whole block: the grid covers heads rounded up to 8
  const int vgrp = lane / (HC / 8), vgl = lane % (HC / 8);  // value row in the load, 8-channel chunk
  const int j16 = lane & 15, kb4 = lane >> 4;
  // queries as the B operand: column = query head (lane % 16 < G), k-step s
  // holds channels 32 s + 8 (lane / 16) .. + 7; read first, so that their
  // latency passes during the selection
  bf16x8 qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j16 < G) v = *reinterpret_cast<const u32x4*>(q + ((size_t)h * G + j16) * D + 32 * s + 8 * kb4);
    qb[s] = __builtin_bit_cast(bf16x8, v);
  }
  // with the token split and no selected ids to return, the gather of the
  // clusters above the cut starts before the candidates are ranked (below)
  bool early = false;
  select_phase<TS>(S, q, G, X, h, B, TS && sel_ids == nullptr, &early);
  const int cnt = early ? 0 : select_count(S, X, B);  // (early: known once the ranks are)
  const long long cap = X.cap;
  // one block per head publishes the count and the unused entries; the
  // selected entries come from the block that stages them (all from block 0
  // without the token split)
  const bool writer = part == 0;
  if (writer && sel_count && tid == 0) sel_count[h] = select_count(S, X, B);  // wave 0 holds the ranks
  if (writer && sel_ids)
    for (int p = cnt + tid; p < B; p += SEL_THREADS) sel_ids[(size_t)h * B + p] = -1;
  const int32_t* ids_h = X.token_ids + (size_t)h * cap;
  const int32_t* app_h = X.app_ids + (size_t)h * cap;
  const int vch = TS ? 0 : HC * part;  // the block's first value channel
  const uint16_t* Kh = kc + (size_t)h * cap * D + 8 * kb4;
  const uint16_t* Vh = vc + (size_t)h * cap * D + vch + 8 * vgl;
  const uint16_t* Kph = kp + (size_t)h * cap * D + 8 * kb4;
  const uint16_t* Vph = vp + (size_t)h * cap * D + vch + 8 * vgl;

  // per query head: the wave's running maximum (uniform), this lane's share
  // of the sum of weights, and the partial output of this lane's channels
  float o[G][8], m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[g][c] = 0.f;
  }

  // one slice: the n64 (<= ST) entries staged at ss, gathered, scored and
  // folded into the wave's running state
  auto do_slice = [&](const int* ss, int n64) {
    bf16x8 ka[NT][4];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      const int t = T * 16 + j16;
      const int id = t < n64 ? ss[t] : 0;
      const uint16_t* src = sel_row(Kph, Kh, id);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        ka[T][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 32 * s));
    }
    Row8<uint16_t> vrow[VR];
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int t = r * RPS + vgrp;
      const int id = t < n64 ? ss[t] : 0;
      vrow[r].load(sel_row(Vph, Vh, id));
    }
    f32x4 acc[NT] = {};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int T = 0; T < NT; ++T) acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[T][s], qb[s], acc[T], 0, 0, 0);
    // score of (row 16 T + 4 (lane / 16) + r, query head lane % 16) -> pw[w][row][g]
    if (j16 < G) {
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = T * 16 + 4 * kb4 + r;
          pw[w][t][j16] = t < n64 ? acc[T][r] * qscale : -INFINITY;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane = token of the slice: its G scores become weights. The running
    // maximum moves (and the partial results are rescaled) only when the
    // slice holds a larger score; the sums stay per lane until the end.
    {
      float sv[GP];
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&pw[w][lane][g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[g4 + i] = lane < ST ? x[i] : -INFINITY;  // lanes past the slice: no token
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float smax = wave_max(sv[g]);
        if (smax > m_run[g]) {  // uniform over the wave
          const float f = m_run[g] == -INFINITY ? 0.f : exp2f(m_run[g] - smax);
          l_run[g] *= f;
#pragma unroll
          for (int c = 0; c < 8; ++c) o[g][c] *= f;
          m_run[g] = smax;
        }
        const float pv = m_run[g] == -INFINITY ? 0.f : exp2f(sv[g] - m_run[g]);
        sv[g] = pv;
        l_run[g] += pv;
      }
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4)
        *reinterpret_cast<f32x4*>(&pw[w][lane][g4]) = f32x4{sv[g4], sv[g4 + 1], sv[g4 + 2], sv[g4 + 3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int t = r * RPS + vgrp;
      float pv[GP];
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&pw[w][t][g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[g4 + i] = x[i];
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[g][c] = fmaf(pv[g], vrow[r].at(c), o[g][c]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if constexpr (!TS) {
    for (int base = 0; base < cnt; base += EMIT) {
      const int nb = cnt - base < EMIT ? cnt - base : EMIT;
      // each wave stages the entries of its own slices (w, w + 8, ... of 64),
      // one search over the ranks per entry, and starts on them with no block
      // barrier: no wave reads another's part of sel
      for (int t = w * 64 + lane; t < nb; t += 2 * NW * 64) {
        const int t2 = t + NW * 64;  // the next slice's entry, searched alongside
        int e1, e2 = 0;
        select_emit2(S, base + t, t2 < nb ? base + t2 : -1, ids_h, app_h, packed, X, e1, e2);
        sel[t] = e1;
        if (t2 < nb) sel[t2] = e2;
        if (writer && sel_ids) {
          sel_ids[(size_t)h * B + base + t] = sel_token(ids_h, e1, packed);
          if (t2 < nb) sel_ids[(size_t)h * B + base + t2] = sel_token(ids_h, e2, packed);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int t0 = w * 64; t0 < nb; t0 += NW * 64) do_slice(sel + t0, nb - t0 < 64 ? nb - t0 : 64);
    }
  } else {
    // Early: output positions [0, P1) hold the sinks, the window and then the
    // clusters above the cut bin in id order (each selected whole, together the
    // first ranks), and the rank order takes over from P1. The softmax and the
    // weighted sum do not depend on the order of the tokens, so a slice inside
    // [0, P1) is staged and gathered before the candidates are ranked; a slice
    // reaching past P1 waits for wave 0's flag. Every wave builds the same list
    // of those clusters: lane i holds the i-th (ck) and its exclusive prefix of
    // sizes (cpre).
    const int nfix = X.n_sink + X.nw < B ? X.n_sink + X.nw : B;
    int P1 = 0, ck = 0, cpre = 0, ncl = 0;
    if (early) {
      unsigned long long cmv[NW];
      int cbase[NW + 1];
      cbase[0] = 0;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        cmv[v] = S.cmask[v];
        cbase[v + 1] = cbase[v] + __popcll(cmv[v]);
      }
      ncl = cbase[NW];
      P1 = nfix;
      if (ncl <= WAVE) {
        unsigned long long m = 0;
        int r = 0, kb = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v)
          if (lane >= cbase[v] && lane < cbase[v + 1]) {
            m = cmv[v];
            r = lane - cbase[v];
            kb = v * WAVE;
          }
        ck = lane < ncl ? kb + nth_set_bit(m, r) : 0;
        const int n = lane < ncl ? S.mn[ck] : 0;
        const int x = wave_incl_scan(n);
        cpre = x - n;
        P1 = nfix + __builtin_amdgcn_readlane(x, WAVE - 1);
      }
    }
    bool ranked = !early;
    int lim_r = cnt;  // the selected count once ranked
    // slices part, part + P, ...: wave w takes the block's slices w, w + 8, ...
    // and stages each one's entries in its own 64 words of sel
    for (int sl = part + P * w;; sl += P * NW) {
      const int t0 = sl * ST;
      if (!ranked && t0 + ST > P1) {  // the slice needs the ranks
        while (__hip_atomic_load(&S.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
          __builtin_amdgcn_s_sleep(1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        ranked = true;
        lim_r = select_count(S, X, B);
      }
      const int lim = ranked ? lim_r : P1;
      if (t0 >= lim) break;
      const int n64 = lim - t0 < ST ? lim - t0 : ST;
      const int p = t0 + lane;
      int ent = 0;
      if (lane < n64 && (p < nfix || p >= P1)) ent = select_emit(S, p, ids_h, app_h, packed, X);
      // positions of the clusters above the cut in the slice: q in [qa, qb)
      const int qa = (t0 > nfix ? t0 : nfix) - nfix;
      const int qb = (t0 + n64 < P1 ? t0 + n64 : P1) - nfix;
      if (qa < qb) {
        // the clusters that overlap the slice, one at a time (wave-uniform
        // loop; lane 0's prefix is 0 <= qa, so both ballots hold lane 0)
        const unsigned long long lo = __ballot(lane < ncl && cpre <= qa);
        const unsigned long long hi = __ballot(lane < ncl && cpre <= qb - 1);
        const int ilo = 63 - __clzll(lo), ihi = 63 - __clzll(hi);
        const int qq = p - nfix;
        for (int i = ilo; i <= ihi; ++i) {
          const int k = __builtin_amdgcn_readlane(ck, i), pre = __builtin_amdgcn_readlane(cpre, i);
          if (lane < n64 && p >= nfix && p < P1 && qq >= pre && qq < pre + S.mn[k])
            ent = cluster_entry(S, k, qq - pre, ids_h, app_h, packed);
        }
      }
      if (lane < n64) {
        sel[w * 64 + lane] = ent;
        if (sel_ids) sel_ids[(size_t)h * B + t0 + lane] = sel_token(ids_h, ent, packed);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      do_slice(sel + w * 64, n64);
    }
  }
  // merge: the row groups of each wave (lanes HC / 8 apart share channels), then the 8 waves
  if constexpr (TS) {
    // four row groups of 16 lanes (vgrp = lane / 16), each lane NV = 8 G
    // values: a transposed reduction. Swapping the 32-lane halves of values i
    // and i + NV / 2 and adding leaves value i summed over the halves in lanes
    // 0-31 and value i + NV / 2 in lanes 32-63; swapping 16-lane rows of those
    // sums pairwise (i, i + NV / 4) and adding leaves row r holding value
    // i + r NV / 4, summed over all four row groups. Each lane then writes its
    // NV / 4 values: lane operations only, no LDS round trip.
    constexpr int NV = G * 8;
    float r1[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) {
      const int j = i + NV / 2;
      const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[i >> 3][i & 7]),
                                                      __float_as_uint(o[j >> 3][j & 7]), false, false);
      r1[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) {
      const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(r1[i]), __float_as_uint(r1[i + NV / 4]), false,
                                                      false);
      const float r2 = __uint_as_float(p[0]) + __uint_as_float(p[1]);
      const int v = i + vgrp * (NV / 4);
      ored[w][v >> 3][8 * vgl + (v & 7)] = r2;
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float v = o[g][c];
#pragma unroll
        for (int m = HC / 8; m < WAVE; m <<= 1) v += __shfl_xor(v, m);
        o[g][c] = v;
      }
    if (vgrp == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) ored[w][g][8 * vgl + c] = o[g][c];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) l_run[g] = wave_sum(l_run[g]);
  if (lane < G) {
    // the running maximum and the reduced sum are the same in every lane;
    // lane g publishes head g's
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g == lane) {
        wm[w][g] = m_run[g];
        wl[w][g] = l_run[g];
      }
  }
  __syncthreads();
  for (int e = tid; e < G * HC; e += SEL_THREADS) {
    const int g = e / HC, j = e % HC;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, wm[v][g]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float f = wm[v][g] == -INFINITY ? 0.f : exp2f(wm[v][g] - M);
        L = fmaf(f, wl[v][g], L);
        O = fmaf(f, ored[v][g][j], O);
      }
    }
    if constexpr (TS) {
      // device-coherent stores (written through this XCD's L2), read below by
      // whichever block of the head merges
      float* pd = part_out + (((size_t)h * P + part) * G + g) * (D + 2);
      __hip_atomic_store(pd + j, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (j == 0) {
        __hip_atomic_store(pd + D, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pd + D + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      out[((size_t)h * G + g) * D + HC * part + j] = L > 0.f ? O / L : 0.f;
    }
  }
  if constexpr (TS) {
    // The last of the head's P blocks to arrive merges the P partial results
    // in block order. Each block's partial results were stored device-coherent
    // (above); every thread waits for its stores to complete before the block
    // arrives, and the merging block reads them device-coherent after it has
    // seen the other P - 1 arrivals. No cache-wide write-back or invalidate is
    // involved (both cost tens of microseconds per launch here). The merging
    // block resets the counter for the next call.
    __shared__ int last;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are complete
    __syncthreads();
    if (tid == 0) last = __hip_atomic_fetch_add(arrive + h, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P - 1;
    __syncthreads();
    if (last) {
      const float* ph = part_out + (size_t)h * P * G * (D + 2);
      auto ld = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
      for (int e = tid; e < G * D; e += SEL_THREADS) {
        const int g = e / D, j = e % D;
        float mp[P], lp[P], op[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const float* pp = ph + (p * G + g) * (D + 2);
          mp[p] = ld(pp + D);
          lp[p] = ld(pp + D + 1);
          op[p] = ld(pp + j);
        }
        float M = -INFINITY;
#pragma unroll
        for (int p = 0; p < P; ++p) M = fmaxf(M, mp[p]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const float f = mp[p] == -INFINITY ? 0.f : exp2f(mp[p] - M);
          L = fmaf(f, lp[p], L);
          O = fmaf(f, op[p], O);
        }
        out[((size_t)h * G + g) * D + j] = L > 0.f ? O / L : 0.f;
      }
      if (tid == 0) arrive[h] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// a10 + a11 standalone: gather + split-K attention over given selections.
// Grid (ceil(B / 64), heads); block = 4 waves over 64 selected tokens, 16
// lanes per 128-channel row. Each block writes (m, l, o[d]) per query head
// (log2 domain; q pre-scaled by scale * log2 e); a second kernel merges the
// splits of each head in split order.
template <typename KT, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(const KT* __restrict__ q, const KT* __restrict__ kc,
                                                           const KT* __restrict__ vc, long long head_stride,
                                                           const int32_t* __restrict__ sel_ids,
                                                           const int32_t* __restrict__ sel_count, int B,
                                                           float qscale, float* __restrict__ part) {
  __shared__ float ps[G][DEC_TOK];
  __shared__ float ored[4][G][D];
  __shared__ float sm[G], sl[G];
  const int h = blockIdx.y, sp = blockIdx.x, nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = lane >> 4, gl = lane & 15;
  // the caller's count, clamped to the row of B entries; entries outside
  // [0, capacity) are skipped
  const int cnt = min(max(sel_count[h], 0), B);
  const long long cap = head_stride / D;
  const int t0 = sp * DEC_TOK;
  const int ntok = cnt - t0 < 0 ? 0 : (cnt - t0 > DEC_TOK ? DEC_TOK : cnt - t0);

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    load8(q + ((size_t)h * G + g) * D + 8 * gl, qv[g]);
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[g][c] *= qscale;
  }
  const KT* Kh = kc + (size_t)h * head_stride + 8 * gl;
  const KT* Vh = vc + (size_t)h * head_stride + 8 * gl;
  Row8<KT> kr[4], vr[4];
  bool ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = w * 16 + r * 4 + grp;
    int id = t < ntok ? sel_ids[(size_t)h * B + t0 + t] : 0;
    ok[r] = t < ntok && id >= 0 && id < cap;
    id = ok[r] ? id : 0;
    kr[r].load(Kh + (size_t)id * D);
    vr[r].load(Vh + (size_t)id * D);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = w * 16 + r * 4 + grp;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) s = fmaf(qv[g][c], kr[r].at(c), s);
      s = row16_sum(s);
      if (gl == 0) ps[g][t] = ok[r] ? s : -INFINITY;
    }
  }
  __syncthreads();
  for (int g = w; g < G; g += 4) {
    const float v = ps[g][lane];
    float m = v;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float p = m == -INFINITY ? 0.f : exp2f(v - m);
    float l = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    ps[g][lane] = p;
    if (lane == 0) {
      sm[g] = m;
      sl[g] = l;
    }
  }
  __syncthreads();
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[g][c] = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = w * 16 + r * 4 + grp;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = ps[g][t];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[g][c] = fmaf(p, vr[r].at(c), o[g][c]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = o[g][c];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[g][c] = v;
    }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) ored[w][g][8 * gl + c] = o[g][c];
  }
  __syncthreads();
  float* pp = part + ((size_t)h * nsplit + sp) * G * (D + 2);
  for (int e = tid; e < G * D; e += 256) {
    const int g = e / D, j = e % D;
    pp[g * (D + 2) + j] = ored[0][g][j] + ored[1][g][j] + ored[2][g][j] + ored[3][g][j];
  }
  if (tid < G) {
    pp[tid * (D + 2) + D] = sm[tid];
    pp[tid * (D + 2) + D + 1] = sl[tid];
  }
}

// Merge of the splits of one head, in split order: M = max m_s,
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s (zero without tokens).
// The (m, l) pairs and the split weights go through LDS first so that every
// thread's loads of the partial outputs are independent.
constexpr int COMB_MAX = DEC_MAX_PAIRS;  // (split, query head) pairs held in LDS
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ part, int nsplit, int G,
                                                             float* __restrict__ out) {
  __shared__ float wt[COMB_MAX];
  __shared__ float Ls[8];  // query heads per KV head (at most 8)
  const int h = blockIdx.x;
  const float* ph = part + (size_t)h * nsplit * G * (D + 2);
  for (int e = threadIdx.x; e < nsplit * G; e += 256) wt[e] = ph[(size_t)e * (D + 2) + D];
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, wt[s * G + g]);
    float L = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = wt[s * G + g];
      const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);
      L = fmaf(f, ph[((size_t)s * G + g) * (D + 2) + D + 1], L);
      wt[s * G + g] = f;
    }
    Ls[g] = L;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int g = e / D, j = e % D;
    float O = 0.f;
    int s = 0;
    for (; s + 4 <= nsplit; s += 4) {
      const float o0 = ph[((size_t)(s + 0) * G + g) * (D + 2) + j];
      const float o1 = ph[((size_t)(s + 1) * G + g) * (D + 2) + j];
      const float o2 = ph[((size_t)(s + 2) * G + g) * (D + 2) + j];
      const float o3 = ph[((size_t)(s + 3) * G + g) * (D + 2) + j];
      O = fmaf(wt[(s + 0) * G + g], o0, O);
      O = fmaf(wt[(s + 1) * G + g], o1, O);
      O = fmaf(wt[(s + 2) * G + g], o2, O);
      O = fmaf(wt[(s + 3) * G + g], o3, O);
    }
    for (; s < nsplit; ++s) O = fmaf(wt[s * G + g], ph[((size_t)s * G + g) * (D + 2) + j], O);
    out[((size_t)h * G + g) * D + j] = Ls[g] > 0.f ? O / Ls[g] : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Full attention over the first n rows of each head (the dense computation
// that cluster-granular recall approximates; the full-KV comparator). Grid
// (nsplit, heads), 4 waves per block; split s covers tokens [s T, s T + T).
// Each wave takes 64-token slices w, w + 4, ... of its split: query-key
// products on the matrix cores (the 64 keys as the A operand of four
// 16x16x32 bf16 tiles, the G queries as B), an online softmax per wave with
// one token per lane, and the value rows weighted on the vector units, 16
// lanes per row (8 channels each) and 4 rows per load instruction. The waves'
// states merge in LDS and the block writes its partial (o[d], m, l), which
// decode_combine_kernel merges over the splits.
template <int G>
__global__ __launch_bounds__(256) void dense_decode_bf16_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ kc,
                                                                const uint16_t* __restrict__ vc, long long cap, int n,
                                                                int T, float qscale, float* __restrict__ part) {
  constexpr int NW = 4;
  constexpr int GP = G < 4 ? 4 : G;
  constexpr int VR = 16;  // value rows per lane per slice (4 per load instruction)
  __shared__ __align__(16) float pw[NW][64][GP];
  __shared__ float ored[NW][G][D];
  __shared__ float wm[NW][G], wl[NW][G];
  const int h = blockIdx.y, sp = blockIdx.x, nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j16 = lane & 15, kb4 = lane >> 4;     // key tiles: row lane % 16, 16-byte piece lane / 16
  const int grp = lane >> 4, gl = lane & 15;      // value rows: row lane / 16 of each 4, channels 8 (lane % 16)
  const int tb = sp * T, te = tb + T < n ? tb + T : n;
  const uint16_t* Kh = kc + (size_t)h * cap * D + 8 * kb4;
  const uint16_t* Vh = vc + (size_t)h * cap * D + 8 * gl;
  bf16x8 qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j16 < G) v = *reinterpret_cast<const u32x4*>(q + ((size_t)h * G + j16) * D + 32 * s + 8 * kb4);
    qb[s] = __builtin_bit_cast(bf16x8, v);
  }
  float o[G][8], m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[g][c] = 0.f;
  }
  for (int t0 = tb + w * 64; t0 < te; t0 += NW * 64) {
    const int n64 = te - t0 < 64 ? te - t0 : 64;
    bf16x8 ka[4][4];
#pragma unroll
    for (int T4 = 0; T4 < 4; ++T4) {
      const int t = T4 * 16 + j16;
      const uint16_t* src = Kh + (size_t)(t0 + (t < n64 ? t : 0)) * D;
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[T4][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 32 * s));
    }
    u32x4 vr[VR];
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int t = r * 4 + grp;
      vr[r] = t < n64 ? *reinterpret_cast<const u32x4*>(Vh + (size_t)(t0 + t) * D) : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 acc[4] = {};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int T4 = 0; T4 < 4; ++T4) acc[T4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[T4][s], qb[s], acc[T4], 0, 0, 0);
    if (j16 < G) {
#pragma unroll
      for (int T4 = 0; T4 < 4; ++T4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = T4 * 16 + 4 * kb4 + r;
          pw[w][t][j16] = t < n64 ? acc[T4][r] * qscale : -INFINITY;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      float sv[GP];
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&pw[w][lane][g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[g4 + i] = x[i];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float smax = wave_max(sv[g]);
        if (smax > m_run[g]) {  // uniform over the wave
          const float f = m_run[g] == -INFINITY ? 0.f : exp2f(m_run[g] - smax);
          l_run[g] *= f;
#pragma unroll
          for (int c = 0; c < 8; ++c) o[g][c] *= f;
          m_run[g] = smax;
        }
        const float pv = m_run[g] == -INFINITY ? 0.f : exp2f(sv[g] - m_run[g]);
        sv[g] = pv;
        l_run[g] += pv;
      }
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4)
        *reinterpret_cast<f32x4*>(&pw[w][lane][g4]) = f32x4{sv[g4], sv[g4 + 1], sv[g4 + 2], sv[g4 + 3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int t = r * 4 + grp;
      float pv[GP];
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&pw[w][t][g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[g4 + i] = x[i];
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t u = vr[r][c >> 1];
        const float vv = (c & 1) ? __uint_as_float(u & 0xFFFF0000u) : __uint_as_float(u << 16);
#pragma unroll
        for (int g = 0; g < G; ++g) o[g][c] = fmaf(pv[g], vv, o[g][c]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // merge: the 4 row groups of each wave (lanes 16 apart share channels), then the waves
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = wave_sum(l_run[g]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = o[g][c];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[g][c] = v;
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) ored[w][g][8 * gl + c] = o[g][c];
  }
  if (lane < G) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g == lane) {
        wm[w][g] = m_run[g];
        wl[w][g] = l_run[g];
      }
  }
  __syncthreads();
  float* ph = part + ((size_t)h * nsplit + sp) * G * (D + 2);
  for (int e = tid; e < G * D; e += 256) {
    const int g = e / D, j = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, wm[v][g]);
    float O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < NW; ++v) O = fmaf(wm[v][g] == -INFINITY ? 0.f : exp2f(wm[v][g] - M), ored[v][g][j], O);
    }
    ph[(size_t)g * (D + 2) + j] = O;
    if (j == 0) {
      float Ls = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int v = 0; v < NW; ++v) Ls = fmaf(wm[v][g] == -INFINITY ? 0.f : exp2f(wm[v][g] - M), wl[v][g], Ls);
      }
      ph[(size_t)g * (D + 2) + D] = M;
      ph[(size_t)g * (D + 2) + D + 1] = Ls;
    }
  }
}

// ---------------------------------------------------------------------------
// Packed copy of the index's key and value rows in index order: row i of head
// h is the cache row token_ids[h][i], for i in [r0, r1): r0 = row0[h * stride]
// (or 0 without row0), r1 = row1[h * stride] (or r0 + n without row1). 16
// bytes per lane, one row per D * sizeof(KT) / 16 lanes.
template <typename KT>
__global__ __launch_bounds__(256) void pack_kernel(const KT* __restrict__ kc, const KT* __restrict__ vc, long long cap,
                                                   const int32_t* __restrict__ token_ids, int n,
                                                   const int32_t* __restrict__ row0, const int32_t* __restrict__ row1,
                                                   long long stride, KT* __restrict__ kp, KT* __restrict__ vp) {
  constexpr int LPR = D * (int)sizeof(KT) / 16;  // lanes per row
  constexpr int RPB = 256 / LPR;                 // rows per block and pass
  const int h = blockIdx.y;
  const int l = threadIdx.x % LPR, rr = threadIdx.x / LPR;
  const size_t hb = (size_t)h * cap;
  const int r0 = row0 ? row0[(size_t)h * stride] : 0;
  const int r1 = row1 ? row1[(size_t)h * stride] : r0 + n;
  for (int i = r0 + blockIdx.x * RPB + rr; i < r1; i += gridDim.x * RPB) {
    const size_t src = (hb + (size_t)token_ids[hb + i]) * D, dst = (hb + (size_t)i) * D;
    const u32x4 k = reinterpret_cast<const u32x4*>(kc + src)[l];
    const u32x4 v = reinterpret_cast<const u32x4*>(vc + src)[l];
    reinterpret_cast<u32x4*>(kp + dst)[l] = k;
    reinterpret_cast<u32x4*>(vp + dst)[l] = v;
  }
}

// ---------------------------------------------------------------------------
// Canonical index (main and appended parts merged) of the C clusters in use,
// one block per head; prefix entries of unused slots hold the total.
__global__ __launch_bounds__(256) void export_csr_kernel(int C, int cs, const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ token_ids,
                                                         const int32_t* __restrict__ app_offsets,
                                                         const int32_t* __restrict__ app_ids, long long cap,
                                                         int32_t* __restrict__ out_offsets,
                                                         int32_t* __restrict__ out_ids) {
  const int h = blockIdx.x;
  const int32_t* off = offsets + (size_t)h * (cs + 1);
  const int32_t* aoff = app_offsets + (size_t)h * (cs + 1);
  for (int k = threadIdx.x; k <= cs; k += 256)
    out_offsets[(size_t)h * (cs + 1) + k] = k <= C ? off[k] + aoff[k] : off[C] + aoff[C];
  for (int k = threadIdx.x; k < C; k += 256) {
    int dst = off[k] + aoff[k];
    for (int e = off[k]; e < off[k + 1]; ++e) out_ids[(size_t)h * cap + dst++] = token_ids[(size_t)h * cap + e];
    for (int e = aoff[k]; e < aoff[k + 1]; ++e) out_ids[(size_t)h * cap + dst++] = app_ids[(size_t)h * cap + e];
  }
}

// ---------------------------------------------------------------------------
// Host launchers.

hipError_t launch_append(int dtype, void* kc, void* vc, long long head_stride, int heads, const void* knew,
                         const void* vnew, int n_new, int n0, const void* chat, int ca, int cs, int cps, int metric,
                         int32_t* labels, long long cap, int32_t* sizes, int32_t* app_offsets, int32_t* app_ids,
                         hipStream_t st) {
  if (dtype == DT_BF16)
    append_kernel<uint16_t><<<heads, APP_THREADS, 0, st>>>((uint16_t*)kc, (uint16_t*)vc, head_stride, (const uint16_t*)knew,
                                                   (const uint16_t*)vnew, n_new, n0, (const uint16_t*)chat, ca, cs, cps,
                                                   metric, labels, cap, sizes, app_offsets, app_ids);
  else
    append_kernel<float><<<heads, APP_THREADS, 0, st>>>((float*)kc, (float*)vc, head_stride, (const float*)knew,
                                                (const float*)vnew, n_new, n0, (const float*)chat, ca, cs, cps, metric,
                                                labels, cap, sizes, app_offsets, app_ids);
  return hipGetLastError();
}

hipError_t launch_window_append(int dtype, void* kc, void* vc, long long cap, int heads, const void* knew,
                                const void* vnew, int n_new, int n0, int32_t* labels, hipStream_t st) {
  const long long elems = (long long)n_new * D;
  const dim3 grid((unsigned)((elems + 255) / 256 < 64 ? (elems + 255) / 256 : 64), heads);
  if (dtype == DT_BF16)
    window_append_kernel<uint16_t><<<grid, 256, 0, st>>>((uint16_t*)kc, (uint16_t*)vc, cap, (const uint16_t*)knew,
                                                         (const uint16_t*)vnew, n_new, n0, labels);
  else
    window_append_kernel<float><<<grid, 256, 0, st>>>((float*)kc, (float*)vc, cap, (const float*)knew,
                                                      (const float*)vnew, n_new, n0, labels);
  return hipGetLastError();
}

hipError_t launch_select(int dtype, const void* q, int G, const IndexView& x, int heads, int B, int32_t* sel_ids,
                         int32_t* sel_count, hipStream_t st) {
  if (dtype == DT_BF16)
    select_kernel<uint16_t><<<heads, SEL_THREADS, 0, st>>>((const uint16_t*)q, G, x, B, sel_ids, sel_count);
  else
    select_kernel<float><<<heads, SEL_THREADS, 0, st>>>((const float*)q, G, x, B, sel_ids, sel_count);
  return hipGetLastError();
}

hipError_t launch_cache_assemble(int dtype, const void* q, int G, const IndexView& x, int heads, const void* kc,
                                 const void* vc, const void* kp, const void* vp, int B, int R, int t, void* ck,
                                 void* cv, int32_t* table, long long* stats, int32_t* rows, int32_t* count,
                                 int32_t* sel_ids, int32_t* sel_count, hipStream_t st) {
  const int packed = kp && vp ? 1 : 0;
  if (dtype == DT_BF16)
    cache_assemble_kernel<uint16_t><<<heads, SEL_THREADS, 0, st>>>(
        (const uint16_t*)q, G, x, (const uint16_t*)kc, (const uint16_t*)vc, (const uint16_t*)(packed ? kp : kc),
        (const uint16_t*)(packed ? vp : vc), packed, B, R, t, (uint16_t*)ck, (uint16_t*)cv, table, stats, rows, count,
        sel_ids, sel_count);
  else
    cache_assemble_kernel<float><<<heads, SEL_THREADS, 0, st>>>(
        (const float*)q, G, x, (const float*)kc, (const float*)vc, (const float*)(packed ? kp : kc),
        (const float*)(packed ? vp : vc), packed, B, R, t, (float*)ck, (float*)cv, table, stats, rows, count, sel_ids,
        sel_count);
  return hipGetLastError();
}

struct FusedArgs {
  const void* q;
  IndexView x;
  int heads;
  const void *kc, *vc, *kp, *vp;  // kp, vp: packed copies, or the caches when not packed
  int packed, B;
  float qscale;
  float* out;
  int32_t *sel_ids, *sel_count;
  float* part;      // partial results of the token split, or null
  int32_t* arrive;  // [heads] arrival counters of the token split (zero between calls)
};

template <typename KT, int G>
static void launch_fused(const FusedArgs& a, hipStream_t st) {
  if constexpr (sizeof(KT) == 2) {
    // enough blocks per head that the grid covers the 256 compute units
    const int P = fused_blocks_per_head(a.heads);
    const int nb = (a.heads + 7) / 8 * 8 * P;
#define KVC_FUSED_ARGS                                                                                          \
  (const uint16_t*)a.q, a.x, (const uint16_t*)a.kc, (const uint16_t*)a.vc, (const uint16_t*)a.kp,             \
      (const uint16_t*)a.vp, a.packed, a.heads, a.B, a.qscale, a.out, a.sel_ids, a.sel_count, a.part, a.arrive
    if constexpr (G <= 4) {
      if (a.part) {  // token split; the last block of each head merges
        // slices of 64, 32 or 16 tokens: the longest that still gives each of
        // a block's 8 waves one slice (short budgets take 16)
        const int nt = fused_slice_tiles(a.B, P);
#define KVC_TS_LAUNCH(PP)                                                                                       \
  {                                                                                                               \
    if (nt == 4) select_decode_bf16_kernel<G, PP, true, 4><<<nb, SEL_THREADS, 0, st>>>(KVC_FUSED_ARGS);            \
    else if (nt == 2) select_decode_bf16_kernel<G, PP, true, 2><<<nb, SEL_THREADS, 0, st>>>(KVC_FUSED_ARGS);       \
    else select_decode_bf16_kernel<G, PP, true, 1><<<nb, SEL_THREADS, 0, st>>>(KVC_FUSED_ARGS);                    \
  }
        if (P == 2) KVC_TS_LAUNCH(2)
        else if (P == 4) KVC_TS_LAUNCH(4)
        else KVC_TS_LAUNCH(8)
#undef KVC_TS_LAUNCH
        return;
      }
    }
    if (P == 2) select_decode_bf16_kernel<G, 2, false><<<nb, SEL_THREADS, 0, st>>>(KVC_FUSED_ARGS);
    else if (P == 4) select_decode_bf16_kernel<G, 4, false><<<nb, SEL_THREADS, 0, st>>>(KVC_FUSED_ARGS);
    else select_decode_bf16_kernel<G, 8, false><<<nb, SEL_THREADS, 0, st>>>(KVC_FUSED_ARGS);
#undef KVC_FUSED_ARGS
  }
  else
    select_decode_kernel<KT, G><<<a.heads, SEL_THREADS, 0, st>>>(
        (const KT*)a.q, a.x, (const KT*)a.kc, (const KT*)a.vc, (const KT*)a.kp, (const KT*)a.vp, a.packed, a.B,
        a.qscale, a.out, a.sel_ids, a.sel_count);
}

template <typename KT>
static hipError_t fused_dispatch(int G, const FusedArgs& a, hipStream_t st) {
  switch (G) {
    case 1: launch_fused<KT, 1>(a, st); break;
    case 2: launch_fused<KT, 2>(a, st); break;
    case 4: launch_fused<KT, 4>(a, st); break;
    case 8: launch_fused<KT, 8>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Blocks per KV head of the fused kernel: enough that the grid covers the
// 256 compute units.

hipError_t launch_select_decode(int dtype, const void* q, int G, const IndexView& x, int heads, const void* kc,
                                const void* vc, const void* kp, const void* vp, int B, float scale, float* out,
                                int32_t* sel_ids, int32_t* sel_count, float* part, int32_t* arrive,
                                hipStream_t st) {
  FusedArgs a{q, x, heads, kc, vc, kp ? kp : kc, vp ? vp : vc, kp && vp ? 1 : 0, B, scale * 1.4426950408889634f,
              out, sel_ids, sel_count, part, arrive};
  if (dtype == DT_BF16) return fused_dispatch<uint16_t>(G, a, st);
  return fused_dispatch<float>(G, a, st);
}

template <typename KT>
static hipError_t decode_dispatch(const void* q, int G, const void* kc, const void* vc, long long head_stride,
                                  int heads, const int32_t* sel_ids, const int32_t* sel_count, int B, float qscale,
                                  float* out, float* part, hipStream_t st) {
  dim3 grid((B + DEC_TOK - 1) / DEC_TOK, heads);
  const KT* qq = (const KT*)q;
  const KT* kk = (const KT*)kc;
  const KT* vv = (const KT*)vc;
  switch (G) {
    case 1: decode_split_kernel<KT, 1><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, part); break;
    case 2: decode_split_kernel<KT, 2><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, part); break;
    case 4: decode_split_kernel<KT, 4><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, part); break;
    case 8: decode_split_kernel<KT, 8><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, part); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<<<heads, 256, 0, st>>>(part, (int)grid.x, G, out);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, const void* q, int G, const void* kc, const void* vc, long long head_stride,
                         int heads, const int32_t* sel_ids, const int32_t* sel_count, int B, float scale, float* out,
                         float* part, hipStream_t st) {
  const float qscale = scale * 1.4426950408889634f;
  if (dtype == DT_BF16)
    return decode_dispatch<uint16_t>(q, G, kc, vc, head_stride, heads, sel_ids, sel_count, B, qscale, out, part, st);
  return decode_dispatch<float>(q, G, kc, vc, head_stride, heads, sel_ids, sel_count, B, qscale, out, part, st);
}

// ---------------------------------------------------------------------------
// Fixed device scratch of the allocation-free decode entry point: the split-K
// partial results live in this file-scope array, which every GPU the library
// runs on holds until the process ends. In host code the array's name is a
// stand-in, not a device address: host code reaches the memory only through
// the address hipGetSymbolAddress returns with the device current, looked up
// once per device and kept.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_export_csr(int heads, int ca, int cs, const int32_t* offsets, const int32_t* token_ids,
                             const int32_t* app_offsets, const int32_t* app_ids, long long cap, int32_t* out_offsets,
                             int32_t* out_ids, hipStream_t st) {
  export_csr_kernel<<<heads, 256, 0, st>>>(ca, cs, offsets, token_ids, app_offsets, app_ids, cap, out_offsets,
                                           out_ids);
  return hipGetLastError();
}


hipError_t launch_dense_decode(const void* q, int G, const void* kc, const void* vc, long long cap, int heads, int n,
                               float scale, float* out, float* part, hipStream_t st) {
  int nsplit, T;
  dense_split(n, G, &nsplit, &T);
  const float qscale = scale * 1.4426950408889634f;
  const dim3 grid(nsplit, heads);
  switch (G) {
#define KVC_DENSE_CASE(GG)                                                                                        \
  case GG:                                                                                                      \
    dense_decode_bf16_kernel<GG><<<grid, 256, 0, st>>>((const uint16_t*)q, (const uint16_t*)kc,                \
                                                       (const uint16_t*)vc, cap, n, T, qscale, part);           \
    break;
    KVC_DENSE_CASE(1)
    KVC_DENSE_CASE(2)
    KVC_DENSE_CASE(4)
    KVC_DENSE_CASE(8)
#undef KVC_DENSE_CASE
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<<<heads, 256, 0, st>>>(part, nsplit, G, out);
  return hipGetLastError();
}

hipError_t launch_pack(int dtype, const void* kc, const void* vc, long long cap, int heads, const int32_t* token_ids,
                       int n, const int32_t* row0, const int32_t* row1, long long stride, void* kp, void* vp,
                       hipStream_t st) {
  if (n < 1) return hipSuccess;
  const int bx = (n + 15) / 16 < 64 ? (n + 15) / 16 : 64;
  if (dtype == DT_BF16)
    pack_kernel<uint16_t><<<dim3(bx, heads), 256, 0, st>>>((const uint16_t*)kc, (const uint16_t*)vc, cap, token_ids,
                                                          n, row0, row1, stride, (uint16_t*)kp, (uint16_t*)vp);
  else
    pack_kernel<float><<<dim3(bx, heads), 256, 0, st>>>((const float*)kc, (const float*)vc, cap, token_ids, n, row0,
                                                       row1, stride, (float*)kp, (float*)vp);
  return hipGetLastError();
}

}  // namespace kvc
