// Decode-time kernels: nearest-centroid append, cluster-granular selection,
// and split-K single-query attention over the recalled tokens.
//
// Method: ClusterKV (arXiv 2412.03213), paper summary page sections III.C
// "Selection at the Granularity of Semantic Clusters", Sys-C "Selection and
// Indexing" (Fig. 8: sizes and prefix sums decide which clusters fit; the last
// one is trimmed; indexing works per KV head), II.A "LLM Inference and KV
// Cache" (the latest query attends to the cached keys and values) and III.A
// "Problem Formulation" (attention over the B selected tokens).
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// ---------------------------------------------------------------------------
// a6: append n_new tokens per head. One block per head; tokens in order.
// label = argmax_k of the fp64 chain k_new . chat_k (ascending channel order,
// lowest k on ties), the same rule as the build's assignment. The token id
// joins the end of its cluster's appended list (ids only grow, so lists stay
// ascending), shifting the later clusters' entries right by one.
template <typename KT>
__global__ __launch_bounds__(256) void append_kernel(KT* __restrict__ kc, KT* __restrict__ vc, long long head_stride,
                                                     const KT* __restrict__ knew, const KT* __restrict__ vnew,
                                                     int n_new, int n0, int n_build, const KT* __restrict__ chat,
                                                     int C, int cpad, int32_t* __restrict__ labels, long long cap,
                                                     int32_t* __restrict__ sizes, int32_t* __restrict__ app_offsets,
                                                     int32_t* __restrict__ app_ids) {
  __shared__ double kv[D];
  __shared__ double rs[4];
  __shared__ int rk[4];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t* aoff = app_offsets + (size_t)h * (C + 1);
  int32_t* aids = app_ids + (size_t)h * cap;
  const KT* Ch = chat + (size_t)h * cpad * D;
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
    double best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int c = tid; c < C; c += 256) {
      double s = 0.0;
      for (int j = 0; j < D; ++j) s = fma(kv[j], (double)load_f32(Ch, (size_t)c * D + j), s);
      if (s > best) {
        best = s;
        bi = c;
      }
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
    for (int v = 1; v < 4; ++v)
      if (rs[v] > best || (rs[v] == best && rk[v] < bi)) {
        best = rs[v];
        bi = rk[v];
      }
    const int lab = bi;
    // insert pos at the end of cluster lab's appended segment
    const int a = pos - n_build;       // entries before this append
    const int p = aoff[lab + 1];
    for (int hiend = a; hiend > p; hiend -= 256) {  // shift right to left, one chunk at a time
      const int lo = hiend - 256 > p ? hiend - 256 : p;
      const int e = lo + tid;
      int v = 0;
      if (e < hiend) v = aids[e];
      __syncthreads();
      if (e < hiend) aids[e + 1] = v;
      __syncthreads();
    }
    if (tid == 0) {
      aids[p] = pos;
      sizes[(size_t)h * C + lab] += 1;
      labels[(size_t)h * cap + pos] = lab;
    }
    for (int k = lab + 1 + tid; k <= C; k += 256) aoff[k] += 1;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// a7-a9: selection, one block of 512 threads per KV head (C <= 512).
//  1. qbar_j = fp64 sum over the head's G query heads (ascending g).
//  2. score_k = fp64 chain qbar . c_k over ascending j; thread k owns cluster k.
//  3. Bitonic sort of (score, k) into (score descending, k ascending) order.
//  4. Exclusive prefix W_r of sizes in rank order: rank r starts at W_r.
//  5. Output position p < min(B, N) belongs to the last rank r with W_r <= p;
//     it takes member p - W_r of that cluster (built part, then appended part),
//     so every cluster before the cut is whole and the last one is trimmed.
template <typename QT>
__global__ __launch_bounds__(512) void select_kernel(const QT* __restrict__ q, int G, const float* __restrict__ cent,
                                                     int C, const int32_t* __restrict__ sizes,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ token_ids,
                                                     const int32_t* __restrict__ app_offsets,
                                                     const int32_t* __restrict__ app_ids, long long cap, int B,
                                                     int32_t* __restrict__ sel_ids, int32_t* __restrict__ sel_count) {
  __shared__ double qbar[D];
  __shared__ unsigned long long key[512];
  __shared__ int kid[512];
  __shared__ int W[512];
  const int h = blockIdx.x, tid = threadIdx.x;
  if (tid < D) {
    double s = 0.0;
    for (int g = 0; g < G; ++g) s = s + (double)load_f32(q, ((size_t)h * G + g) * D + tid);
    qbar[tid] = s;
  }
  __syncthreads();
  unsigned long long u = 0;
  int k = 0x7FFFFFFF;
  if (tid < C) {
    const f32x4* cr = reinterpret_cast<const f32x4*>(cent + ((size_t)h * C + tid) * D);
    double s = 0.0;
#pragma unroll 4
    for (int jj = 0; jj < D / 4; ++jj) {
      const f32x4 v = cr[jj];
      s = fma(qbar[4 * jj], (double)v[0], s);
      s = fma(qbar[4 * jj + 1], (double)v[1], s);
      s = fma(qbar[4 * jj + 2], (double)v[2], s);
      s = fma(qbar[4 * jj + 3], (double)v[3], s);
    }
    u = ordered_key(s);
    k = tid;
  }
  key[tid] = u;
  kid[tid] = k;
  __syncthreads();
  // bitonic sort, best first: "better" = larger key, then smaller id
  for (int size = 2; size <= 512; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int o = tid ^ stride;
      if (o > tid) {
        const unsigned long long ua = key[tid], ub = key[o];
        const int ka = kid[tid], kb = kid[o];
        const bool a_better = ua > ub || (ua == ub && ka < kb);
        const bool swap = (tid & size) == 0 ? !a_better : a_better;
        if (swap) {
          key[tid] = ub;
          key[o] = ua;
          kid[tid] = kb;
          kid[o] = ka;
        }
      }
      __syncthreads();
    }
  }
  const int kr = kid[tid];
  const int nr = kr < C ? sizes[(size_t)h * C + kr] : 0;
  W[tid] = nr;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    const int v = tid >= off ? W[tid - off] : 0;
    __syncthreads();
    W[tid] += v;
    __syncthreads();
  }
  const int total = W[511];
  const int incl = W[tid];
  __syncthreads();
  W[tid] = incl - nr;  // exclusive
  __syncthreads();
  const int cnt = total < B ? total : B;
  const int32_t* off = offsets + (size_t)h * (C + 1);
  const int32_t* aoff = app_offsets + (size_t)h * (C + 1);
  for (int p = tid; p < B; p += 512) {
    int tok = -1;
    if (p < cnt) {
      int lo = 0, hi = 511;  // last r with W[r] <= p
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (W[mid] <= p) lo = mid;
        else hi = mid - 1;
      }
      const int kk = kid[lo];
      const int e = p - W[lo];
      const int nb = off[kk + 1] - off[kk];
      tok = e < nb ? token_ids[(size_t)h * cap + off[kk] + e] : app_ids[(size_t)h * cap + aoff[kk] + (e - nb)];
    }
    sel_ids[(size_t)h * B + p] = tok;
  }
  if (tid == 0) sel_count[h] = cnt;
}

// ---------------------------------------------------------------------------
// a10 + a11: gather + split-K single-query attention.
// Grid (ceil(B / 64), heads); block = 4 waves over 64 selected tokens. In a
// wave, 16 lanes cover one 128-channel row (8 channels each), so one load
// instruction gathers 4 rows of K (or V) with 16-byte accesses per lane. The
// G query heads of the KV head share every gathered row. Each block writes
// (m, l, o[d]) per query head in the log2 domain (q is pre-scaled by
// scale * log2 e); the last block of a head to finish merges the splits in
// split order (a per-head arrival counter, reset by that block).
template <typename KT, int G>
__global__ __launch_bounds__(256) void decode_kernel(const KT* __restrict__ q, const KT* __restrict__ kc,
                                                     const KT* __restrict__ vc, long long head_stride,
                                                     const int32_t* __restrict__ sel_ids,
                                                     const int32_t* __restrict__ sel_count, int B, float qscale,
                                                     float* __restrict__ out, float* __restrict__ part,
                                                     uint32_t* __restrict__ counters) {
  __shared__ float ps[G][DEC_TOK];
  __shared__ float ored[4][G][D];
  __shared__ int s_last;
  const int h = blockIdx.y, sp = blockIdx.x, nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = lane >> 4, gl = lane & 15;
  const int cnt = sel_count[h];
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
  float kr[4][8], vr[4][8];
  bool valid[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = w * 16 + r * 4 + grp;
    valid[r] = t < ntok;
    const int id = valid[r] ? sel_ids[(size_t)h * B + t0 + t] : 0;
    load8(Kh + (size_t)id * D, kr[r]);
    load8(Vh + (size_t)id * D, vr[r]);
  }
  // scores
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) s = fmaf(qv[g][c], kr[r][c], s);
      s += __shfl_xor(s, 8);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 1);
      if (gl == 0) ps[g][w * 16 + r * 4 + grp] = valid[r] ? s : -INFINITY;
    }
  }
  __syncthreads();
  // per query head: split max, weights, sum (one wave per head)
  __shared__ float sm[G], sl[G];
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
      for (int c = 0; c < 8; ++c) o[g][c] = fmaf(p, vr[r][c], o[g][c]);
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
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(counters + h, 1u) == (uint32_t)(nsplit - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* ph = part + (size_t)h * nsplit * G * (D + 2);
  for (int e = tid; e < G * D; e += 256) {
    const int g = e / D, j = e % D;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, __builtin_nontemporal_load(ph + ((size_t)s * G + g) * (D + 2) + D));
    float Ls = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float* ps2 = ph + ((size_t)s * G + g) * (D + 2);
        const float ms = __builtin_nontemporal_load(ps2 + D);
        const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);
        Ls = fmaf(f, __builtin_nontemporal_load(ps2 + D + 1), Ls);
        O = fmaf(f, __builtin_nontemporal_load(ps2 + j), O);
      }
    }
    out[((size_t)h * G + g) * D + j] = Ls > 0.f ? O / Ls : 0.f;
  }
  if (tid == 0) counters[h] = 0;
}

// ---------------------------------------------------------------------------
// Canonical index (built + appended parts merged), one block per head.
__global__ __launch_bounds__(256) void export_csr_kernel(int C, const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ token_ids,
                                                         const int32_t* __restrict__ app_offsets,
                                                         const int32_t* __restrict__ app_ids, long long cap,
                                                         int32_t* __restrict__ out_offsets,
                                                         int32_t* __restrict__ out_ids) {
  const int h = blockIdx.x;
  const int32_t* off = offsets + (size_t)h * (C + 1);
  const int32_t* aoff = app_offsets + (size_t)h * (C + 1);
  for (int k = threadIdx.x; k <= C; k += 256) out_offsets[(size_t)h * (C + 1) + k] = off[k] + aoff[k];
  for (int k = threadIdx.x; k < C; k += 256) {
    int dst = off[k] + aoff[k];
    for (int e = off[k]; e < off[k + 1]; ++e) out_ids[(size_t)h * cap + dst++] = token_ids[(size_t)h * cap + e];
    for (int e = aoff[k]; e < aoff[k + 1]; ++e) out_ids[(size_t)h * cap + dst++] = app_ids[(size_t)h * cap + e];
  }
}

// ---------------------------------------------------------------------------
// Host launchers.

hipError_t launch_append(int dtype, void* kc, void* vc, long long head_stride, int heads, const void* knew,
                         const void* vnew, int n_new, int n0, int n_build, const void* chat, int C, int cpad,
                         int32_t* labels, long long cap, int32_t* sizes, int32_t* app_offsets, int32_t* app_ids,
                         hipStream_t st) {
  if (dtype == DT_BF16)
    append_kernel<uint16_t><<<heads, 256, 0, st>>>((uint16_t*)kc, (uint16_t*)vc, head_stride, (const uint16_t*)knew,
                                                   (const uint16_t*)vnew, n_new, n0, n_build,
                                                   (const uint16_t*)chat, C, cpad, labels, cap, sizes, app_offsets,
                                                   app_ids);
  else
    append_kernel<float><<<heads, 256, 0, st>>>((float*)kc, (float*)vc, head_stride, (const float*)knew,
                                                (const float*)vnew, n_new, n0, n_build, (const float*)chat, C, cpad,
                                                labels, cap, sizes, app_offsets, app_ids);
  return hipGetLastError();
}

hipError_t launch_select(int dtype, const void* q, int G, const float* cent, int heads, int C, const int32_t* sizes,
                         const int32_t* offsets, const int32_t* token_ids, const int32_t* app_offsets,
                         const int32_t* app_ids, long long cap, int B, int32_t* sel_ids, int32_t* sel_count,
                         hipStream_t st) {
  if (dtype == DT_BF16)
    select_kernel<uint16_t><<<heads, 512, 0, st>>>((const uint16_t*)q, G, cent, C, sizes, offsets, token_ids,
                                                   app_offsets, app_ids, cap, B, sel_ids, sel_count);
  else
    select_kernel<float><<<heads, 512, 0, st>>>((const float*)q, G, cent, C, sizes, offsets, token_ids, app_offsets,
                                                app_ids, cap, B, sel_ids, sel_count);
  return hipGetLastError();
}

template <typename KT>
static hipError_t decode_dispatch(const void* q, int G, const void* kc, const void* vc, long long head_stride,
                                  int heads, const int32_t* sel_ids, const int32_t* sel_count, int B, float qscale,
                                  float* out, float* part, uint32_t* counters, hipStream_t st) {
  dim3 grid((B + DEC_TOK - 1) / DEC_TOK, heads);
  const KT* qq = (const KT*)q;
  const KT* kk = (const KT*)kc;
  const KT* vv = (const KT*)vc;
  switch (G) {
    case 1: decode_kernel<KT, 1><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, out, part, counters); break;
    case 2: decode_kernel<KT, 2><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, out, part, counters); break;
    case 4: decode_kernel<KT, 4><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, out, part, counters); break;
    case 8: decode_kernel<KT, 8><<<grid, 256, 0, st>>>(qq, kk, vv, head_stride, sel_ids, sel_count, B, qscale, out, part, counters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, const void* q, int G, const void* kc, const void* vc, long long head_stride,
                         int heads, const int32_t* sel_ids, const int32_t* sel_count, int B, float scale, float* out,
                         float* part, uint32_t* counters, hipStream_t st) {
  const float qscale = scale * 1.4426950408889634f;
  if (dtype == DT_BF16)
    return decode_dispatch<uint16_t>(q, G, kc, vc, head_stride, heads, sel_ids, sel_count, B, qscale, out, part,
                                     counters, st);
  return decode_dispatch<float>(q, G, kc, vc, head_stride, heads, sel_ids, sel_count, B, qscale, out, part, counters,
                                st);
}

hipError_t launch_export_csr(int heads, int C, const int32_t* offsets, const int32_t* token_ids,
                             const int32_t* app_offsets, const int32_t* app_ids, long long cap, int32_t* out_offsets,
                             int32_t* out_ids, hipStream_t st) {
  export_csr_kernel<<<heads, 256, 0, st>>>(C, offsets, token_ids, app_offsets, app_ids, cap, out_offsets, out_ids);
  return hipGetLastError();
}

}  // namespace kvc
