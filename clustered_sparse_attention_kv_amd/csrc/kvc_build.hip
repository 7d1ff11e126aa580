// Prefill clustering kernels: initial centroids, cosine assignment on the
// matrix cores with a certified argmax, fp64 re-scoring of uncertified keys,
// the stable counting sort that builds the cluster index, and the centroid
// update fused with normalisation.
//
// Method: ClusterKV (arXiv 2412.03213), paper summary page sections III.B
// "Clustering in the Semantic Space" (cosine k-means over keys), Sys-B
// "Semantic Clustering" (batched per-head clustering; accumulate assigned keys
// and counts, then divide) and Sys-C "Selection and Indexing" (sizes, prefix
// sums, token ids sorted by cluster).
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// ---------------------------------------------------------------------------
// Normalisation of one centroid row held by one wave (2 channels per lane).
// norm = sqrt(fp64 sum of c_j^2 over ascending j); chat_j = c_j / norm rounded
// once to the operand type (zero when the norm is zero). The ascending sum is
// one lane's chain so its order is fixed (its loads are batched). Returns the
// two rounded values this lane stored.
template <typename OT>
__device__ __forceinline__ double2 normalize_row(const float c0, const float c1, float* lds_row, OT* out_row) {
  const int lane = lane_id();
  lds_row[2 * lane] = c0;
  lds_row[2 * lane + 1] = c1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double ss = 0.0;
  if (lane == 0) {
#pragma unroll 16
    for (int j = 0; j < D; ++j) {
      const double v = (double)lds_row[j];
      ss = fma(v, v, ss);
    }
  }
  // broadcast lane 0's sum
  const int lo = __builtin_amdgcn_readfirstlane((int)(__double_as_longlong(ss) & 0xFFFFFFFFll));
  const int hi = __builtin_amdgcn_readfirstlane((int)(__double_as_longlong(ss) >> 32));
  ss = __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
  const double nrm = sqrt(ss);
  const double v0 = nrm > 0.0 ? (double)c0 / nrm : 0.0;
  const double v1 = nrm > 0.0 ? (double)c1 / nrm : 0.0;
  store_op(out_row, 2 * lane, v0);
  store_op(out_row, 2 * lane + 1, v1);
  return double2{rounded_op(out_row, v0), rounded_op(out_row, v1)};
}

// The assignment operand of one centroid row under each distance (III.B
// defines the semantic distance by the cosine and names L2 and inner product
// as the alternatives): the unit direction for the cosine, the centroid itself
// for L2 and inner product, rounded once to the operand type. metric is
// uniform over the wave.
template <typename OT>
__device__ __forceinline__ double2 operand_row(int metric, const float c0, const float c1, float* lds_row,
                                               OT* out_row) {
  if (metric == M_COSINE) return normalize_row(c0, c1, lds_row, out_row);
  const int lane = lane_id();
  store_op(out_row, 2 * lane, (double)c0);
  store_op(out_row, 2 * lane + 1, (double)c1);
  return double2{rounded_op(out_row, (double)c0), rounded_op(out_row, (double)c1)};
}

// ---------------------------------------------------------------------------
// a1: initial centroid positions by a seeded partial Fisher-Yates shuffle of
// the n = L - lo clustered rows (the pages leave the initialisation open;
// III.B only says that the k-means iterates until the assignment settles).
// Swap i (i = 0 .. C-1) exchanges entries i and j_i = i + (r_i mod (n - i)) of
// the permutation, with r_i the i-th SplitMix64 output from state
// seed ^ (0x9E3779B97F4A7C15 * (h + 1)); position k is lo + perm[k].
//
// SplitMix64's i-th output depends only on i (the state after i + 1 steps is
// the start plus (i + 1) increments), so all j_i are drawn at once, one thread
// per swap. The sequential result then follows from which earlier swap last
// wrote a position: before swap i, entry p (p >= i) holds p unless an earlier
// swap i' targeted it (j_i' = p), in which case it holds a_i', the value entry
// i' had when swap i' ran. With P_i the last i' < i with j_i' = i and Q_i the
// last i' < i with j_i' = j_i:
//   a_i = P_i < 0 ? i : a_{P_i},      perm[i] = Q_i < 0 ? j_i : a_{Q_i}.
// a_i refers only to smaller indices, so repeated substitution settles it (at
// least the smallest unsettled index settles per round). One block per head.
constexpr int INIT_THREADS = 512;  // one thread per swap (C <= 512)
__global__ __launch_bounds__(INIT_THREADS) void init_positions_kernel(unsigned long long seed, int lo, int L, int C,
                                                                      int32_t* __restrict__ out) {
  __shared__ int J[INIT_THREADS];
  __shared__ int A[INIT_THREADS];
  __shared__ int unsettled;
  const int h = blockIdx.x, i = threadIdx.x;
  const unsigned long long gamma = 0x9E3779B97F4A7C15ull;
  const long long n = (long long)L - lo;
  if (i < C) {
    unsigned long long z = (seed ^ (gamma * (unsigned long long)(h + 1))) + gamma * (unsigned long long)(i + 1);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    J[i] = i + (int)(z % (unsigned long long)(n - i));
  }
  __syncthreads();
  int P = -1, Q = -1;
  if (i < C) {
    const int ji = J[i];
    for (int t = 0; t < i; ++t) {
      const int jt = J[t];
      P = jt == i ? t : P;
      Q = jt == ji ? t : Q;
    }
    A[i] = P < 0 ? i : -1;
  }
  for (;;) {
    if (i == 0) unsettled = 0;
    __syncthreads();
    if (i < C && A[i] < 0) {
      const int v = A[P];
      if (v >= 0) A[i] = v;
      else unsettled = 1;
    }
    __syncthreads();
    const int more = unsettled;
    __syncthreads();
    if (!more) break;
  }
  if (i < C) out[(size_t)h * C + i] = lo + (Q < 0 ? J[i] : A[Q]);
}

hipError_t launch_init_positions(int heads, int lo, int L, int C, unsigned long long seed, int32_t* out,
                                 hipStream_t st) {
  if (C < 1 || C > INIT_THREADS || lo < 0 || (long long)L - lo < C) return hipErrorInvalidValue;
  init_positions_kernel<<<heads, INIT_THREADS, 0, st>>>(seed, lo, L, C, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a1 + a2: initial centroids c_k = K[init_idx[k]] (exact copy to fp32) and
// their normalised operand. One wave per centroid row, 4 rows per block.
// Rows k in [C, cpad) of the operand are zeroed. Per-cluster arrays have a
// per-head stride of cs cluster slots (cs >= C; the operand has cps =
// cpad(cs) rows per head), which leaves room for clusters added later.
// The centroid pair (c0, c1) of channels 2*lane, 2*lane+1 of cluster k, also
// stored in the chunk-major copy [d/4, cs, 4] that selection reads coalesced.
__device__ __forceinline__ void store_centroid(float* cent_row, float* cent_t_head, int cs, int k, float c0, float c1) {
  const int lane = lane_id();
  cent_row[2 * lane] = c0;
  cent_row[2 * lane + 1] = c1;
  const int j = 2 * lane;
  float* t = cent_t_head + ((size_t)(j >> 2) * cs + k) * 4 + (j & 3);
  t[0] = c0;
  t[1] = c1;
}

template <typename KT>
__global__ __launch_bounds__(256) void init_centroids_kernel(const KT* __restrict__ keys, long long head_stride,
                                                             int lo, int L, const int32_t* __restrict__ init_idx, int C,
                                                             int cpad, int cs, int cps, int metric,
                                                             float* __restrict__ cent, float* __restrict__ cent_t,
                                                             KT* __restrict__ chat, int32_t* __restrict__ dev_flags) {
  __shared__ float rows[4][D];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y;
  const int k = blockIdx.x * 4 + w;
  if (k >= cpad) return;
  KT* out = chat + ((size_t)h * cps + k) * D;
  if (k >= C) {
    store_op(out, 2 * lane, 0.0);
    store_op(out, 2 * lane + 1, 0.0);
    return;
  }
  int tok = init_idx[(size_t)h * C + k];
  if (tok < lo || tok >= L) {
    if (lane == 0) atomicOr(dev_flags, 1);
    tok = 0;
  }
  const KT* src = keys + (size_t)h * head_stride + (size_t)tok * D;
  const float c0 = load_f32(src, 2 * lane), c1 = load_f32(src, 2 * lane + 1);
  store_centroid(cent + ((size_t)h * cs + k) * D, cent_t + (size_t)h * cs * D, cs, k, c0, c1);
  operand_row(metric, c0, c1, rows[w], out);
}

// ---------------------------------------------------------------------------
// a3: assignment of bf16 keys on the matrix cores.
//
// v_mfma_f32_16x16x32_bf16 with the normalised centroids as the A operand
// (16 centroids x 32 channels per tile, staged once per block in LDS) and the
// keys as the B operand (32 channels x 16 keys): lane l holds key l % 16 of
// its tile and channels 32 s + 8 (l / 16) .. + 7 at k-step s, so one load
// instruction reads 64 contiguous bytes of 16 key rows. D[centroid][key]
// gives each lane 4 centroids (4 (l / 16) + r) of one key per tile.
//
// Block = 12 waves x 64 keys (4 tiles of 16 per wave); the grid holds about
// one block per compute unit and each block walks over 768-key groups of one
// head, so the head's operand is staged in LDS once per block (row r's 16-byte
// chunk c at c ^ (r & 15): the 16 rows one read instruction touches land in
// distinct banks).
//
// Each lane keeps the best and the runner-up score of each of its keys; the
// 4 lanes of a key merge at the end. A score's place in the tile loop, the
// code ((31 - tile) << 2) | (3 - r), replaces its seven low mantissa bits, so
// the running maximum carries its own centroid id. Two scores fold at a time:
// with best m1 >= runner-up m2, the top two of {m1, m2, e1, e2} are
// max3(m1, e1, e2) and max(med3(m1, e1, e2), m2), so a score costs one
// v_and_or_b32 and one and a half further instructions. The code moves a value
// by at most 127 units in the last place. The fp32 order is certified against the exact
// (fp64) order when
//   best - runner_up > 2 * 4 * (d + 16) * 2^-24 * ||K_i|| * max||chat_k|| * 1.02
//                      + 2^-15 * max(|best|, |runner_up|) * 1.02,
// a bound on the error of any fp32 accumulation of d exact products (the
// products of bf16 operands are exact) with a safety factor of 4, plus the
// code bits. Keys that fail it are queued for exact re-scoring (fix-up
// kernel below). Ties and near-ties therefore always resolve by the fp64
// rule, lowest id first. Only the tiles that hold centroids are computed; a
// partial last tile masks its padding rows.
//
// The L2 and inner-product variants (METRIC) use centroids that are not unit
// length. The score is K_i . chat_k (inner product) or K_i . chat_k + b_k with
// b_k = -||chat_k||^2 / 2 rounded to fp32 (L2, argmin of the distance), and the
// certificate uses the head's largest operand norm A and largest |b_k|:
//   best - runner_up > 2 * 4 * 2^-24 * ((d + 17) * ||K_i|| * A + 2 max|b_k|) * 1.02,
// which also covers the rounding of b_k and of the addition.
// A key that changed cluster marks both clusters (flags per head, C of them;
// old is the previous iteration's label, anything outside [0, C) is skipped):
// the update recomputes only marked clusters, since a cluster whose member set
// is unchanged gets the same centroid from the same ascending chain.
__device__ __forceinline__ void mark_moved(int32_t* flags, int C, int old_label, int new_label) {
  if ((unsigned)old_label < (unsigned)C) flags[old_label] = 1;
  flags[new_label] = 1;
}

constexpr int AS_WAVES = 12;
constexpr int AS_THREADS = AS_WAVES * WAVE;
constexpr int AS_TILE = AS_WAVES * 64;

// Running best and runner-up with two more scores (code bits in place; all
// values finite or -inf). The maximum of the bit-built operands is a plain
// v_max3_f32: the compiler would otherwise canonicalise each operand first.
// max(x, m2) of finite values is med3(x, m2, FLT_MAX).
__device__ __forceinline__ void top2_push2(float e1, float e2, float& m1, float& m2) {
  const float mid = __builtin_amdgcn_fmed3f(m1, e1, e2);
  m2 = __builtin_amdgcn_fmed3f(mid, m2, 3.40282347e38f);
  float mx;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx) : "v"(m1), "v"(e1), "v"(e2));
  m1 = mx;
}

template <int METRIC>
__global__ __launch_bounds__(AS_THREADS) void assign_bf16_mfma_kernel(
    const uint16_t* __restrict__ keys, long long head_stride, int L, const uint16_t* __restrict__ chat, int C,
    int cpad, int cps, int32_t* __restrict__ labels, long long label_stride, int32_t* __restrict__ queue,
    uint32_t* __restrict__ qcount, u32x4* __restrict__ op_t, int32_t* __restrict__ dirty, float* __restrict__ norm2,
    int norm_mode, float* __restrict__ top2) {
  extern __shared__ u32x4 sC[];  // cpad rows x 16 chunks of 16 B, chunk c of row r at c ^ (r & 15)
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, kb4 = lane >> 4;

  const u32x4* Cg = reinterpret_cast<const u32x4*>(chat + (size_t)h * cps * D);
  // block 0 of each head also stores the chunk-major copy [16][cpad] that the
  // exact pass reads (rows of one chunk contiguous)
  u32x4* Ot = blockIdx.x == 0 ? op_t + (size_t)h * 16 * cpad : nullptr;
  // a non-finite component in operand row 0 (possible under L2 and inner
  // product) makes cluster 0's score NaN for some keys, and the sequential
  // argmax rule then keeps them in cluster 0 where the fold below would skip
  // the NaN: every key of such a head goes to the exact pass
  // (one 16-byte slot after the zero tile: the kernel keeps all of its LDS in
  // the dynamic allocation, whose size limit leaves no room for static LDS)
  int& row0_bad = *reinterpret_cast<int*>(sC + (cpad + 16) * 16);
  if (tid == 0) row0_bad = 0;
  __syncthreads();
  for (int e = tid; e < cpad * 16; e += AS_THREADS) {
    const int r = e >> 4, c = e & 15;
    const u32x4 v = Cg[e];
    sC[r * 16 + (c ^ (r & 15))] = v;
    if (Ot) Ot[(size_t)c * cpad + r] = v;
    if (r == 0) {
      bool bad = false;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bad |= (v[q] & 0x7F80u) == 0x7F80u || (v[q] & 0x7F800000u) == 0x7F800000u;
      if (bad) row0_bad = 1;
    }
  }
  // one zero tile past the operand: the tile loop reads one tile ahead without
  // a bound
  for (int e = tid; e < 16 * 16; e += AS_THREADS) sC[cpad * 16 + e] = u32x4{0u, 0u, 0u, 0u};
  // variants: after the operand, the per-centroid bias (L2; cpad floats) and
  // the largest operand norm (one word), all in the dynamic allocation so the
  // kernel has no static LDS
  float* sBias = reinterpret_cast<float*>(sC + (cpad + 16) * 16 + 1);
  unsigned& sMaxNorm = *reinterpret_cast<unsigned*>(sBias + cpad);
  float normA = 1.0f, biasM = 0.0f;
  if constexpr (METRIC != M_COSINE) {
    if (tid == 0) sMaxNorm = 0u;
    __syncthreads();
    for (int k = tid; k < cpad; k += AS_THREADS) {
      double nn = 0.0;
      if (k < C)
        for (int c = 0; c < 16; ++c) {
          const u32x4 v = Cg[(size_t)k * 16 + c];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const double lo = (double)__uint_as_float(v[q] << 16), hi = (double)__uint_as_float(v[q] & 0xFFFF0000u);
            nn = fma(lo, lo, nn);
            nn = fma(hi, hi, nn);
          }
        }
      if constexpr (METRIC == M_L2) sBias[k] = (float)(-0.5 * nn);
      atomicMax(&sMaxNorm, __float_as_uint((float)sqrt(nn) * 1.0000001f));
    }
  }
  __syncthreads();
  if constexpr (METRIC != M_COSINE) {
    normA = __uint_as_float(sMaxNorm);
    biasM = METRIC == M_L2 ? 0.5f * normA * normA * 1.0000001f : 0.0f;
  }

  const uint16_t* Kh = keys + (size_t)h * head_stride + 8 * kb4;
  const int ngroups = (L + AS_TILE - 1) / AS_TILE;
  // the and-mask of the code bits, held in a vector register so that one
  // v_and_or_b32 (which reads a single scalar operand) takes it beside the
  // scalar code
  unsigned vmask;
  asm volatile("v_mov_b32 %0, 0xffffff80" : "=v"(vmask));
  const int ntl = (C + 15) >> 4;          // tiles holding centroids
  const bool partial = (C & 15) != 0;     // the last of them holds padding rows
  const float gamma = 2.0f * 4.0f * (float)(D + 16) * 5.9604644775390625e-8f * 1.02f;
  const float gbits = 3.0517578125e-5f * 1.02f;  // 2^-15: the code bits of best and runner-up
  // variants: threshold = g2 * ((d + 17) * A * ||K_i|| + 2 max|b_k|)
  const float g2 = 2.0f * 4.0f * 5.9604644775390625e-8f * 1.02f;
  const float gA = g2 * (float)(D + 17) * normA, gB = g2 * 2.0f * biasM;
  const u32x4* sA[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) sA[s] = sC + j16 * 16 + ((4 * s + kb4) ^ j16);
  for (int grpi = blockIdx.x; grpi < ngroups; grpi += gridDim.x) {
    const int row0 = grpi * AS_TILE + wave * 64;
    // the label this lane's key had after the previous iteration, read early
    const int prow = row0 + kb4 * 16 + j16;
    const int old_label = dirty && prow < L ? labels[(size_t)h * label_stride + prow] : -1;
    // ||K||^2 of that key from an earlier iteration (norm_mode 2)
    const float kept_n2 = norm_mode == 2 && prow < L ? norm2[(size_t)h * L + prow] : 0.f;
    u32x4 kn[4][4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      int row = row0 + T * 16 + j16;
      row = row < L ? row : L - 1;  // the tail tile repeats the last key; its results are not stored
      const uint16_t* src = Kh + (size_t)row * D;
#pragma unroll
      for (int s = 0; s < 4; ++s) kn[T][s] = *reinterpret_cast<const u32x4*>(src + 32 * s);
    }
    bf16x8 kb[4][4];
    float n2[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 v = kn[T][s];
        kb[T][s] = __builtin_bit_cast(bf16x8, v);
        if (norm_mode == 2) continue;
        // the four words as scalars first: a bit cast of an indexed vector
        // element inside this unrolled loop compiles to the first word four
        // times
        const unsigned e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // two channels per packed dot product
          const bf16x2 x = __builtin_bit_cast(bf16x2, e[q]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
        }
      }
      n2[T] = ss;
    }
    float m1[4], m2[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      m1[T] = -INFINITY;
      m2[T] = -INFINITY;
    }
    // centroid tiles in a pipeline: while the products of tile ct + 1 run on
    // the matrix cores, the vector units fold tile ct into the running best
    // and runner-up, and the operand of tile ct + 2 is read from LDS. The
    // instruction scheduler is asked to alternate one product with four
    // vector instructions so that both units stay busy within a wave. The
    // tile count (cpad / 16) is even and only the last two tiles can hold
    // padding rows, so the loop body folds full tiles without masks.
    // row ct * 16 + j16 of the operand: its chunk 4 s + kb4 sits at
    // (4 s + kb4) ^ j16, the same for every tile, so only the tile's base moves
    auto load_a = [&](int ct, bf16x8 (&a)[4]) {
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = __builtin_bit_cast(bf16x8, sA[s][ct * 256]);
    };
    auto mma = [&](const bf16x8 (&a)[4], f32x4 (&acc)[4]) {
#pragma unroll
      for (int T = 0; T < 4; ++T) acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], kb[T][s], acc[T], 0, 0, 0);
    };
    auto fold = [&](int ct, const f32x4 (&acc)[4], bool masked) {
      const int u0 = ct * 16;  // centroid of register r in this lane: u0 + 4 (lane / 16) + r
      const unsigned tcode = (unsigned)(31 - ct) << 2;
      f32x4 bias = {0.f, 0.f, 0.f, 0.f};
      if constexpr (METRIC == M_L2) bias = *reinterpret_cast<const f32x4*>(sBias + u0 + 4 * kb4);
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float sc = acc[T][r];
          if constexpr (METRIC == M_L2) sc += bias[r];
          e[r] = __uint_as_float((__float_as_uint(sc) & vmask) | (tcode | (unsigned)(3 - r)));
          if (masked && u0 + 4 * kb4 + r >= C) e[r] = -INFINITY;
        }
        top2_push2(e[0], e[1], m1[T], m2[T]);
        top2_push2(e[2], e[3], m1[T], m2[T]);
      }
    };
    auto interleave = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the operand reads first
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix product
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four vector instructions
      }
    };
    bf16x8 aA[4], aB[4];
    f32x4 accA[4], accB[4];
    load_a(0, aA);
    mma(aA, accA);
    load_a(ntl > 1 ? 1 : 0, aB);
    int ct = 0;
    for (; ct + 2 < ntl; ct += 2) {
      mma(aB, accB);       // tile ct + 1
      load_a(ct + 2, aA);
      fold(ct, accA, false);
      interleave();
      mma(aA, accA);       // tile ct + 2
      load_a(ct + 3, aB);  // the next tile, or (unused) the zero tile past the operand
      fold(ct + 1, accB, false);
      interleave();
    }
    // accA holds tile ct; tile ct + 1, when there is one, is the last
    if (ct + 1 < ntl) {
      mma(aB, accB);
      fold(ct, accA, false);
      if (partial) fold(ct + 1, accB, true);
      else fold(ct + 1, accB, false);
    } else {
      if (partial) fold(ct, accA, true);
      else fold(ct, accA, false);
    }
    // centroid ids from the code bits (tile, register) and the lane group,
    // then merge the 4 lanes of each key (lanes 16 apart) and certify
    int i1[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const unsigned code = __float_as_uint(m1[T]) & 127u;
      i1[T] = 16 * (31 - (int)(code >> 2)) + 4 * kb4 + 3 - (int)(code & 3u);
#pragma unroll
      for (int m = 16; m <= 32; m <<= 1) {
        const float o1 = __shfl_xor(m1[T], m), o2 = __shfl_xor(m2[T], m);
        const int oi = __shfl_xor(i1[T], m);
        const float M2 = fmaxf(fminf(m1[T], o1), fmaxf(m2[T], o2));
        i1[T] = m1[T] > o1 ? i1[T] : (o1 > m1[T] ? oi : min(i1[T], oi));
        m1[T] = fmaxf(m1[T], o1);
        m2[T] = M2;
        if (norm_mode != 2) n2[T] += __shfl_xor(n2[T], m);
      }
    }
    // lane kb4 == T publishes key j16 of tile T
    int my_label = 0;
    bool my_flag = false;
    float my_m1 = 0.f, my_m2 = 0.f, my_n2 = 0.f;
#pragma unroll
    for (int T = 0; T < 4; ++T)
      if (T == kb4) {
        my_label = i1[T];
        const float nn = norm_mode == 2 ? kept_n2 : n2[T];
        if (norm_mode == 1) my_n2 = nn;
        const float thr = (METRIC == M_COSINE ? gamma * sqrtf(nn) : gA * sqrtf(nn) + gB) +
                          gbits * fmaxf(fabsf(m1[T]), fabsf(m2[T]));
        my_flag = !((m1[T] - m2[T]) > thr) || row0_bad;  // true for NaN and ties
        my_m1 = m1[T];
        my_m2 = m2[T];
      }
    const int row = prow;
    const bool valid = row < L;
    if (valid) {
      // a queued key's label is written by the exact pass, which also marks it
      if (!my_flag) {
        labels[(size_t)h * label_stride + row] = my_label;
        if (dirty && old_label != my_label) mark_moved(dirty + (size_t)h * C, C, old_label, my_label);
      }
      if (norm_mode == 1) norm2[(size_t)h * L + row] = my_n2;
      if (top2) {
        top2[((size_t)h * L + row) * 2] = my_m1;
        top2[((size_t)h * L + row) * 2 + 1] = my_m2;
      }
    }
    const bool push = valid && my_flag;
    const unsigned long long bal = __ballot(push);
    if (bal) {
      const int n = __popcll(bal);
      const int first = __ffsll((long long)bal) - 1;
      int base = 0;
      if (lane == first) base = (int)atomicAdd(qcount + h, (uint32_t)n);
      base = __shfl(base, first);
      const int slot = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (push) queue[(size_t)h * L + slot] = row;
    }
  }
}

// ---------------------------------------------------------------------------
// a3 exact path: label_i = argmax_k of the fp64 chain sum_j K_ij * chat_kj over
// ascending j, lowest k on ties. Used for keys the matrix-core pass could not
// certify, and for every key of fp32 inputs. One wave per block and EX_NK keys
// per wave and pass; lane c owns centroids c, c+64, ... The wave's keys are
// written to LDS in fp64 and every lane reads channel j of a key from the same
// address (a broadcast, a vector operand of the fp64 fma). bf16 operands are
// read from the chunk-major copy [d/8][cpad] of 16-byte chunks that the
// matrix-core pass stores, so the 64 lanes' rows at one chunk are one
// contiguous kilobyte; the next chunk's loads are issued before the current
// chunk's arithmetic. fp32 operands are read row by row. Grid (heads, waves
// per head): blocks go to the 8 XCDs round robin, so with a multiple of 8 heads
// the waves of head h share one XCD, whose L2 holds that head's operand. Rows
// come from the per-head queue (queue != null) or are all rows. Under the L2
// distance (L2D) the score is the chain minus nn_k / 2, nn_k the fp64 chain of
// chat_kj^2 over ascending j, accumulated beside the products.
constexpr int EX_NK = 2;
template <typename KT, int MAXT, bool L2D>
__global__ __launch_bounds__(64) void assign_exact_kernel(const KT* __restrict__ keys, long long head_stride, int L,
                                                          const KT* __restrict__ chat, int C, int cpad, int cps,
                                                          int32_t* __restrict__ labels, long long label_stride,
                                                          const int32_t* __restrict__ queue,
                                                          const uint32_t* __restrict__ qcount,
                                                          const u32x4* __restrict__ op_t,
                                                          int32_t* __restrict__ dirty) {
  constexpr bool BF = sizeof(KT) == 2;
  constexpr int CHUNKS = D * (int)sizeof(KT) / 16;  // 16-byte chunks per operand row
  constexpr int EPC = 16 / (int)sizeof(KT);         // elements per chunk
  constexpr int NK = EX_NK;
  __shared__ __align__(16) double kl[NK * D];
  const int h = blockIdx.x, lane = threadIdx.x;
  const int n = queue ? (int)__atomic_load_n(qcount + h, __ATOMIC_RELAXED) : L;
  if ((int)blockIdx.y * NK >= n) return;  // no key for this wave
  const KT* Kh = keys + (size_t)h * head_stride;
  const u32x4* Cg = reinterpret_cast<const u32x4*>(chat + (size_t)h * cps * D);
  const u32x4* Ct = BF ? op_t + (size_t)h * CHUNKS * cpad : nullptr;
  // lane's centroid rows; rows past cpad read the last (zero) padding row and
  // are excluded from the argmax, so no branch separates the chains
  int crow[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) crow[t] = min(lane + 64 * t, cpad - 1);
  auto load = [&](int q, int t) {
    if constexpr (BF) return Ct[(size_t)q * cpad + crow[t]];
    else return Cg[(size_t)crow[t] * CHUNKS + q];
  };
  for (int e = (int)blockIdx.y * NK; e < n; e += (int)gridDim.y * NK) {
    int row[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int ee = min(e + kk, n - 1);
      row[kk] = queue ? queue[(size_t)h * L + ee] : ee;
    }
    // the previous pass's reads of kl are done (one wave, in order) before
    // these writes, and the writes before the reads below
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      kl[kk * D + lane] = (double)load_f32(Kh, (size_t)row[kk] * D + lane);
      kl[kk * D + 64 + lane] = (double)load_f32(Kh, (size_t)row[kk] * D + 64 + lane);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    double s[NK][MAXT], nn[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      nn[t] = 0.0;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) s[kk][t] = 0.0;
    }
    u32x4 cur[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) cur[t] = load(0, t);
#pragma unroll 1
    for (int q = 0; q < CHUNKS; ++q) {
      u32x4 nxt[MAXT];
      if (q + 1 < CHUNKS)
#pragma unroll
        for (int t = 0; t < MAXT; ++t) nxt[t] = load(q + 1, t);
      double kj[NK][EPC];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int i = 0; i < EPC; i += 2) {
          const double2 v = *reinterpret_cast<const double2*>(kl + kk * D + q * EPC + i);
          kj[kk][i] = v.x;
          kj[kk][i + 1] = v.y;
        }
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
#pragma unroll
        for (int i = 0; i < EPC; ++i) {
          float x;
          if constexpr (BF)
            x = (i & 1) ? __uint_as_float(cur[t][i >> 1] & 0xFFFF0000u) : __uint_as_float(cur[t][i >> 1] << 16);
          else
            x = __uint_as_float(cur[t][i]);
          const double xd = (double)x;
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) s[kk][t] = fma(kj[kk][i], xd, s[kk][t]);
          if constexpr (L2D) nn[t] = fma(xd, xd, nn[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < MAXT; ++t) cur[t] = nxt[t];
    }
    if constexpr (L2D)
#pragma unroll
      for (int t = 0; t < MAXT; ++t)
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) s[kk][t] = s[kk][t] - 0.5 * nn[t];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      double best = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        const int c = lane + 64 * t;
        if (c < C && s[kk][t] > best) {
          best = s[kk][t];
          bi = c;
        }
      }
      // wave argmax: larger score, then smaller id
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (ob > best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      // non-finite scores follow the sequential rule (start from cluster 0,
      // move only to a strictly larger score): when cluster 0 scores NaN, or
      // no score exceeds -inf, the key stays in cluster 0
      const double s0 = __shfl(s[kk][0], 0);  // cluster 0's score (lane 0 owns it)
      if (bi >= C || s0 != s0) bi = 0;
      if (lane == 0 && e + kk < n) {
        int32_t* lp = labels + (size_t)h * label_stride + row[kk];
        if (dirty) {
          const int old_label = *lp;
          if (old_label != bi) mark_moved(dirty + (size_t)h * C, C, old_label, bi);
        }
        *lp = bi;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a5: stable counting sort of labels into the cluster index.
// Blocks of CS_BLOCK tokens. count: per-block histograms. scan: per cluster
// the exclusive prefix over blocks (block bases within the cluster), sizes,
// and offsets as the exclusive prefix of sizes over clusters. scatter: wave w
// of a block owns CS_BLOCK / 16 consecutive tokens, walked in chunks of 64 in
// token order; the waves' histograms give each wave's base per cluster (after
// the cluster offset and the block base), a lane's rank among lower lanes of
// the same label in its chunk comes from matching label bits with ballots, and
// the last lane of each label in a chunk advances the wave's running position.
// Position = offset + block base + wave base + earlier chunks + rank keeps
// token order.
constexpr int CS_BLOCK = CSR_BLOCK_TOKENS;
constexpr int CS_THREADS = 1024;

__global__ __launch_bounds__(256) void csr_count_kernel(const int32_t* __restrict__ labels, long long label_stride,
                                                        int L, int C, int nblk, int32_t* __restrict__ hist) {
  __shared__ int cnt[512];
  const int h = blockIdx.y, b = blockIdx.x;
  for (int c = threadIdx.x; c < C; c += 256) cnt[c] = 0;
  __syncthreads();
  const int32_t* lab = labels + (size_t)h * label_stride;
  for (int i = b * CS_BLOCK + threadIdx.x; i < min(L, (b + 1) * CS_BLOCK); i += 256) atomicAdd(&cnt[lab[i]], 1);
  __syncthreads();
  int32_t* out = hist + ((size_t)h * nblk + b) * C;
  for (int c = threadIdx.x; c < C; c += 256) out[c] = cnt[c];
}

__global__ __launch_bounds__(512) void csr_scan_kernel(int C, int cs, int nblk, int32_t* __restrict__ hist,
                                                       int32_t* __restrict__ sizes, int32_t* __restrict__ offsets) {
  constexpr int U = 16;  // block counts requested together
  __shared__ int sc[512];
  const int h = blockIdx.x, c = threadIdx.x;
  int32_t* hh = hist + (size_t)h * nblk * C;
  int run = 0;
  if (c < C) {
    for (int b0 = 0; b0 < nblk; b0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = b0 + u < nblk ? hh[(size_t)(b0 + u) * C + c] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b0 + u < nblk) {
          hh[(size_t)(b0 + u) * C + c] = run;
          run += v[u];
        }
    }
    sizes[(size_t)h * cs + c] = run;
  }
  sc[c] = c < C ? run : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over 512 entries
  for (int off = 1; off < 512; off <<= 1) {
    const int v = c >= off ? sc[c - off] : 0;
    __syncthreads();
    sc[c] += v;
    __syncthreads();
  }
  if (c < C) offsets[(size_t)h * (cs + 1) + c] = sc[c] - run;
  if (c == C - 1) offsets[(size_t)h * (cs + 1) + C] = sc[c];
}

__global__ __launch_bounds__(CS_THREADS) void csr_scatter_kernel(const int32_t* __restrict__ labels,
                                                                 long long label_stride, int L, int C, int cs,
                                                                 int nblk, const int32_t* __restrict__ hist,
                                                                 const int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ token_ids,
                                                                 long long ids_stride, int id_base) {
  constexpr int NW = CS_THREADS / WAVE;
  constexpr int PER = CS_BLOCK / CS_THREADS;  // chunks of 64 tokens per wave
  __shared__ int wh[NW][512];
  const int h = blockIdx.y, b = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int e = tid; e < NW * 512; e += CS_THREADS) (&wh[0][0])[e] = 0;
  const int t0 = b * CS_BLOCK + w * (PER * WAVE) + lane;
  int lab[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = t0 + u * WAVE;
    lab[u] = i < L ? labels[(size_t)h * label_stride + i] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (lab[u] >= 0) atomicAdd(&wh[w][lab[u]], 1);
  __syncthreads();
  // per cluster: the cluster's offset plus the block base, then the waves in order
  const int32_t* base = hist + ((size_t)h * nblk + b) * C;
  for (int c = tid; c < C; c += CS_THREADS) {
    int run = base[c] + offsets[(size_t)h * (cs + 1) + c];
    int t[NW];
#pragma unroll
    for (int v = 0; v < NW; ++v) t[v] = wh[v][c];
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      wh[v][c] = run;
      run += t[v];
    }
  }
  __syncthreads();
  const int nbits = 32 - __clz(C > 1 ? C - 1 : 1);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int l = lab[u];
    unsigned long long same = __ballot(l >= 0);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = l >= 0 && ((l >> bit) & 1);
      const unsigned long long bal = __ballot(set);
      same &= set ? bal : ~bal;
    }
    if (l >= 0) {
      // every lane reads the running position before the last lane of its
      // label moves it (one wave; LDS operations in program order)
      const int pos = wh[w][l] + __popcll(same & ((1ull << lane) - 1ull));
      token_ids[(size_t)h * ids_stride + pos] = id_base + t0 + u * WAVE;
      if ((same >> lane) == 1ull) wh[w][l] = pos + 1;
    }
  }
}

// ---------------------------------------------------------------------------
// a4 + a2: centroid update fused with normalisation. One wave per cluster,
// lane = channels 2 lane, 2 lane + 1. The member ids come in groups of 64
// (one per lane, the next group requested before the current one is summed);
// each member's id reaches the wave through a lane read, the group's rows are
// all requested at once, and then summed in fp64 in ascending member order
// (the index order). The mean is the fp64 sum / count rounded once to fp32 (an
// empty cluster keeps its centroid); the new operand row is the normalised
// mean.
template <typename KT>
struct UpdRow;  // one row's two channels as loaded
template <>
struct UpdRow<uint16_t> {
  static constexpr int GROUP = 32;
  uint32_t v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ float a() const { return __uint_as_float(v << 16); }
  __device__ __forceinline__ float b() const { return __uint_as_float(v & 0xFFFF0000u); }
};
template <>
struct UpdRow<float> {
  static constexpr int GROUP = 32;
  float2 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ float a() const { return v.x; }
  __device__ __forceinline__ float b() const { return v.y; }
};

template <typename KT>
__global__ __launch_bounds__(256) void update_kernel(const KT* __restrict__ keys, long long head_stride, int C,
                                                     int cs, int cps, int metric, const int32_t* __restrict__ sizes,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ token_ids, long long ids_stride,
                                                     float* __restrict__ cent, float* __restrict__ cent_t,
                                                     KT* __restrict__ chat, const int32_t* __restrict__ dirty) {
  constexpr int GR = UpdRow<KT>::GROUP;
  __shared__ float rows[4][D];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y;
  const int k = blockIdx.x * 4 + w;
  if (k >= C) return;
  // with flags, a cluster no key entered or left keeps its centroid as it is
  if (dirty && __builtin_amdgcn_readfirstlane(dirty[(size_t)h * C + k]) == 0) return;
  // the same value in every lane: scalar registers, uniform branches
  const int n = __builtin_amdgcn_readfirstlane(sizes[(size_t)h * cs + k]);
  const int off = __builtin_amdgcn_readfirstlane(offsets[(size_t)h * (cs + 1) + k]);
  const int32_t* ids = token_ids + (size_t)h * ids_stride + off;
  const KT* Kh = keys + (size_t)h * head_stride + 2 * lane;
  float* cr = cent + ((size_t)h * cs + k) * D;
  float c0, c1;
  if (n > 0) {
    double a0 = 0.0, a1 = 0.0;
    auto load_ids = [&](int m0) { return m0 + lane < n && lane < GR ? ids[m0 + lane] : 0; };
    auto sum_group = [&](int m0, int idc) {
      const int cnt = n - m0 < GR ? n - m0 : GR;
      UpdRow<KT> x[GR];
#pragma unroll
      for (int u = 0; u < GR; ++u)
        if (u < cnt) x[u].load(Kh + (size_t)__builtin_amdgcn_readlane(idc, u) * D);
#pragma unroll
      for (int u = 0; u < GR; ++u)
        if (u < cnt) {
          a0 += (double)x[u].a();
          a1 += (double)x[u].b();
        }
    };
    // groups of GR members, two id registers so the next group's ids are in
    // flight while the current group's rows are loaded and summed
    int idA = load_ids(0), idB = 0;
    for (int m0 = 0; m0 < n; m0 += 2 * GR) {
      if (m0 + GR < n) idB = load_ids(m0 + GR);
      sum_group(m0, idA);
      if (m0 + GR >= n) break;
      if (m0 + 2 * GR < n) idA = load_ids(m0 + 2 * GR);
      sum_group(m0 + GR, idB);
    }
    c0 = (float)(a0 / (double)n);
    c1 = (float)(a1 / (double)n);
    store_centroid(cr, cent_t + (size_t)h * cs * D, cs, k, c0, c1);
  } else {
    c0 = cr[2 * lane];
    c1 = cr[2 * lane + 1];
  }
  operand_row(metric, c0, c1, rows[w], chat + ((size_t)h * cps + k) * D);
}

// ---------------------------------------------------------------------------
// Clustering of a small window of generated tokens in one launch (nc <= 32
// clusters): one block per head runs the whole k-means of the window's m keys
// with the build's arithmetic. Initial centroids are the keys at init_idx;
// a key's label is the argmax of the fp64 chains over ascending channels
// against the operand rows (lowest cluster on ties; under the L2 distance the
// chain minus half the fp64 chain of the row's squares); a cluster's mean is
// the fp64 sum of its members in ascending token order divided by the count,
// rounded once (an empty cluster keeps its centroid); operand rows as in the
// build. The member lists are written once, after the last iteration. The
// outputs are the arrays the window merge reads: centroids (both layouts),
// operand rows (padding rows zeroed), labels, sizes, offsets and ids.
constexpr int WK_MAXC = WINDOW_KMEANS_MAX_C;
template <typename KT>
__global__ __launch_bounds__(256) void window_kmeans_kernel(
    const KT* __restrict__ keys, long long head_stride, int wlo, int n_tokens, int m, int nc, int cpw, int iters,
    const int32_t* __restrict__ init_idx, int metric, float* __restrict__ cent, float* __restrict__ cent_t,
    KT* __restrict__ chat, int32_t* __restrict__ labels, int32_t* __restrict__ sizes,
    int32_t* __restrict__ offsets, int32_t* __restrict__ ids, int32_t* __restrict__ flags) {
  constexpr int EPC = 16 / (int)sizeof(KT);  // elements per 16-byte chunk
  constexpr int CH = D / EPC;                // chunks per row
  constexpr int BATCH = 16;                  // member rows requested together
  extern __shared__ int lab[];               // the m labels
  __shared__ __align__(16) double op[WK_MAXC][D];  // operand rows in fp64 (exact)
  __shared__ double hnn[WK_MAXC];            // half the fp64 chain of each row's squares (L2)
  __shared__ float rows[4][D];
  __shared__ int cnt[WK_MAXC];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const KT* Kw = keys + (size_t)h * head_stride + (size_t)wlo * D;  // row i of the window
  float* cent_h = cent + (size_t)h * nc * D;
  float* ct_h = cent_t + (size_t)h * nc * D;
  KT* chat_h = chat + (size_t)h * cpw * D;
  // operand row k (the values this wave just stored) into LDS in fp64, and nn_k / 2
  auto refresh = [&](int k, double2 r) {
    op[k][2 * lane] = r.x;
    op[k][2 * lane + 1] = r.y;
    if (metric == M_L2) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane == 0) {
        double nn = 0.0;
#pragma unroll 16
        for (int j = 0; j < D; ++j) nn = fma(op[k][j], op[k][j], nn);
        hnn[k] = 0.5 * nn;
      }
    }
  };
  // initial centroids (padding operand rows zeroed)
  for (int k = w; k < cpw; k += 4) {
    KT* out = chat_h + (size_t)k * D;
    if (k >= nc) {
      store_op(out, 2 * lane, 0.0);
      store_op(out, 2 * lane + 1, 0.0);
      continue;
    }
    int tok = init_idx[(size_t)h * nc + k];
    if (tok < wlo || tok >= n_tokens) {
      if (lane == 0) atomicOr(flags, 1);
      tok = 0;
    }
    const KT* src = keys + (size_t)h * head_stride + (size_t)tok * D;
    const float c0 = load_f32(src, 2 * lane), c1 = load_f32(src, 2 * lane + 1);
    store_centroid(cent_h + (size_t)k * D, ct_h, nc, k, c0, c1);
    refresh(k, operand_row(metric, c0, c1, rows[w], out));
  }
  __syncthreads();
  for (int t = 0; t < iters; ++t) {
    // assignment: one thread per key (its row in registers), one cluster's
    // chain at a time over ascending channels
    for (int i = tid; i < m; i += 256) {
      const u32x4* kr = reinterpret_cast<const u32x4*>(Kw + (size_t)i * D);
      u32x4 kv[CH];
#pragma unroll
      for (int q = 0; q < CH; ++q) kv[q] = kr[q];
      double best = -INFINITY;
      int bi = 0;
      for (int k = 0; k < nc; ++k) {
        // the row's words enter each cluster's pass afresh, so their fp64
        // conversions are not hoisted out of this loop (128 doubles would
        // leave no registers to batch the operand reads)
#pragma unroll
        for (int q = 0; q < CH; ++q) asm volatile("" : "+v"(kv[q]));
        double sk = 0.0;
        // the operand row in batches of 32 values, all requested before use
        constexpr int OB = 32;
#pragma unroll
        for (int j0 = 0; j0 < D; j0 += OB) {
          double ob[OB];
#pragma unroll
          for (int u = 0; u < OB; u += 2) {
            const double2 t2 = *reinterpret_cast<const double2*>(&op[k][j0 + u]);
            ob[u] = t2.x;
            ob[u + 1] = t2.y;
          }
          __builtin_amdgcn_sched_barrier(0);  // keep the batch's reads ahead of its uses
#pragma unroll
          for (int u = 0; u < OB; ++u) {
            const int j = j0 + u, q = j / EPC, e = j % EPC;
            double x;
            if constexpr (sizeof(KT) == 2)
              x = (double)((e & 1) ? __uint_as_float(kv[q][e >> 1] & 0xFFFF0000u)
                                   : __uint_as_float(kv[q][e >> 1] << 16));
            else
              x = (double)__uint_as_float(kv[q][e]);
            sk = fma(x, ob[u], sk);
          }
        }
        if (metric == M_L2) sk = sk - hnn[k];
        if (sk > best) {
          best = sk;
          bi = k;
        }
      }
      lab[i] = bi;
    }
    __syncthreads();
    // update: one wave per cluster; members in ascending token order, rows
    // requested BATCH at a time and summed in that order
    for (int k = w; k < nc; k += 4) {
      double a0 = 0.0, a1 = 0.0;
      int n = 0;
      for (int c0 = 0; c0 < m; c0 += 64) {
        unsigned long long bits = __ballot(c0 + lane < m && lab[c0 + lane] == k);
        while (bits) {
          int mi[BATCH];
          int nb = 0;
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            mi[b] = 0;
            if (bits) {
              mi[b] = c0 + __ffsll((long long)bits) - 1;
              bits &= bits - 1;
              ++nb;
            }
          }
          float v0[BATCH], v1[BATCH];
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            const KT* r = Kw + (size_t)mi[b] * D;
            v0[b] = b < nb ? load_f32(r, 2 * lane) : 0.f;
            v1[b] = b < nb ? load_f32(r, 2 * lane + 1) : 0.f;
          }
#pragma unroll
          for (int b = 0; b < BATCH; ++b)
            if (b < nb) {
              a0 += (double)v0[b];
              a1 += (double)v1[b];
            }
          n += nb;
        }
      }
      float c0, c1;
      if (n > 0) {
        c0 = (float)(a0 / (double)n);
        c1 = (float)(a1 / (double)n);
        store_centroid(cent_h + (size_t)k * D, ct_h, nc, k, c0, c1);
      } else {
        c0 = cent_h[(size_t)k * D + 2 * lane];
        c1 = cent_h[(size_t)k * D + 2 * lane + 1];
      }
      refresh(k, operand_row(metric, c0, c1, rows[w], chat_h + (size_t)k * D));
    }
    __syncthreads();
  }
  // labels, sizes, offsets and member lists of the last assignment
  for (int i = tid; i < m; i += 256) labels[(size_t)h * m + i] = lab[i];
  if (tid < nc) {
    int n = 0;
    for (int i = 0; i < m; ++i) n += lab[i] == tid ? 1 : 0;
    cnt[tid] = n;
  }
  __syncthreads();
  if (tid < nc) {
    int o = 0;
    for (int k = 0; k < tid; ++k) o += cnt[k];
    sizes[(size_t)h * nc + tid] = cnt[tid];
    offsets[(size_t)h * (nc + 1) + tid] = o;
    if (tid == nc - 1) offsets[(size_t)h * (nc + 1) + nc] = o + cnt[tid];
    for (int i = 0; i < m; ++i)
      if (lab[i] == tid) ids[(size_t)h * m + o++] = wlo + i;
  }
}

hipError_t launch_window_kmeans(int dtype, const void* keys, long long head_stride, int heads, int wlo, int n_tokens,
                                int m, int nc, int cpw, int iters, const int32_t* init_idx, int metric, float* cent,
                                float* cent_t, void* chat, int32_t* labels, int32_t* sizes, int32_t* offsets,
                                int32_t* ids, int32_t* flags, hipStream_t st) {
  if (!window_kmeans_fits(m, nc)) return hipErrorInvalidValue;
  const size_t lds = (size_t)m * sizeof(int);
  if (dtype == DT_BF16)
    window_kmeans_kernel<uint16_t><<<heads, 256, lds, st>>>((const uint16_t*)keys, head_stride, wlo, n_tokens, m, nc,
                                                            cpw, iters, init_idx, metric, cent, cent_t,
                                                            (uint16_t*)chat, labels, sizes, offsets, ids, flags);
  else
    window_kmeans_kernel<float><<<heads, 256, lds, st>>>((const float*)keys, head_stride, wlo, n_tokens, m, nc, cpw,
                                                         iters, init_idx, metric, cent, cent_t, (float*)chat, labels,
                                                         sizes, offsets, ids, flags);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Clustering of generated tokens (III.B: the tokens generated since the last
// clustering are clustered on their own into a few new centroids). The window
// is clustered by the kernels above into workspace arrays of nc clusters
// (strides nc, cpad(nc) operand rows, m tokens per head); this kernel moves
// the result into the index as clusters ca .. ca+nc-1: centroid rows (both
// layouts and the operand), sizes, offsets continuing the prefix of the
// existing clusters, member ids after the existing members (so the index
// order stays the stable sort by label), and the window tokens' labels. One
// block per head.
template <typename KT>
__global__ __launch_bounds__(256) void merge_window_kernel(
    int nc, int m, int wlo, const float* __restrict__ cent_w, const KT* __restrict__ chat_w,
    const int32_t* __restrict__ labels_w, const int32_t* __restrict__ sizes_w, const int32_t* __restrict__ offsets_w,
    const int32_t* __restrict__ ids_w, int ca, int cs, int cps, float* __restrict__ cent, float* __restrict__ cent_t,
    KT* __restrict__ chat, int32_t* __restrict__ sizes, int32_t* __restrict__ offsets, int32_t* __restrict__ token_ids,
    int32_t* __restrict__ labels, long long cap) {
  const int h = blockIdx.x, tid = threadIdx.x;
  const int cpw = (nc + 31) / 32 * 32;
  int32_t* off = offsets + (size_t)h * (cs + 1);
  const int base = off[ca];  // members so far; entries ca+1 .. are written below, entry ca is not
  for (int e = tid; e < nc * D; e += 256) {
    const int k = e / D, j = e % D;
    const float v = cent_w[((size_t)h * nc + k) * D + j];
    cent[((size_t)h * cs + ca + k) * D + j] = v;
    cent_t[(size_t)h * cs * D + ((size_t)(j >> 2) * cs + ca + k) * 4 + (j & 3)] = v;
    chat[((size_t)h * cps + ca + k) * D + j] = chat_w[((size_t)h * cpw + k) * D + j];
  }
  for (int k = tid; k < nc; k += 256) {
    sizes[(size_t)h * cs + ca + k] = sizes_w[(size_t)h * nc + k];
    off[ca + k + 1] = base + offsets_w[(size_t)h * (nc + 1) + k + 1];
  }
  for (int i = tid; i < m; i += 256) {
    token_ids[(size_t)h * cap + base + i] = ids_w[(size_t)h * m + i];
    labels[(size_t)h * cap + wlo + i] = ca + labels_w[(size_t)h * m + i];
  }
}

// rows x cols int32 values at a row stride (the attention sinks' labels)
__global__ void fill2d_i32_kernel(int32_t* __restrict__ p, long long stride, int cols, int value) {
  for (int c = threadIdx.x; c < cols; c += blockDim.x) p[(size_t)blockIdx.x * stride + c] = value;
}

hipError_t launch_fill2d_i32(int32_t* p, int rows, long long stride, int cols, int value, hipStream_t st) {
  if (rows < 1 || cols < 1) return hipSuccess;
  fill2d_i32_kernel<<<rows, 256, 0, st>>>(p, stride, cols, value);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, size_t n, int32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------
// Host launchers.

static int grid1(size_t n, int per) { return (int)((n + per - 1) / per); }

hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int blocks = grid1(n, 256) < 1024 ? grid1(n, 256) : 1024;
  fill_i32_kernel<<<blocks, 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_init_centroids(int dtype, const void* keys, long long head_stride, int heads, int lo, int L,
                                 const int32_t* init_idx, int C, int cpad, int cs, int cps, int metric, float* cent,
                                 float* cent_t, void* chat, int32_t* flags, hipStream_t st) {
  dim3 grid(grid1(cpad, 4), heads);
  if (dtype == DT_BF16)
    init_centroids_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)keys, head_stride, lo, L, init_idx, C, cpad,
                                                          cs, cps, metric, cent, cent_t, (uint16_t*)chat, flags);
  else
    init_centroids_kernel<float><<<grid, 256, 0, st>>>((const float*)keys, head_stride, lo, L, init_idx, C, cpad, cs,
                                                       cps, metric, cent, cent_t, (float*)chat, flags);
  return hipGetLastError();
}

// The exact pass instantiated for the number of 64-centroid groups a lane owns
// and the distance; grid (heads, waves per head).
template <typename KT, int MAXT>
hipError_t launch_exact_t(const KT* keys, long long head_stride, int L, const KT* chat, int C, int cpad, int cps,
                          int metric, int32_t* labels, long long label_stride, const int32_t* queue, const uint32_t* qcount,
                          const u32x4* op_t, int32_t* dirty, dim3 grid, hipStream_t st) {
  if (metric == M_L2)
    assign_exact_kernel<KT, MAXT, true><<<grid, 64, 0, st>>>(keys, head_stride, L, chat, C, cpad, cps, labels,
                                                             label_stride, queue, qcount, op_t, dirty);
  else
    assign_exact_kernel<KT, MAXT, false><<<grid, 64, 0, st>>>(keys, head_stride, L, chat, C, cpad, cps, labels,
                                                              label_stride, queue, qcount, op_t, dirty);
  return hipGetLastError();
}

template <typename KT>
hipError_t launch_exact(const KT* keys, long long head_stride, int L, const KT* chat, int C, int cpad, int cps,
                        int metric, int32_t* labels, long long label_stride, const int32_t* queue, const uint32_t* qcount,
                        const u32x4* op_t, int32_t* dirty, dim3 grid, hipStream_t st) {
  switch ((C + 63) / 64) {
#define KVC_EXACT_CASE(T) \
  case T:                 \
    return launch_exact_t<KT, T>(keys, head_stride, L, chat, C, cpad, cps, metric, labels, label_stride, queue,  \
                                 qcount, op_t, dirty, grid, st);
    KVC_EXACT_CASE(1)
    KVC_EXACT_CASE(2)
    KVC_EXACT_CASE(3)
    KVC_EXACT_CASE(4)
    KVC_EXACT_CASE(5)
    KVC_EXACT_CASE(6)
    KVC_EXACT_CASE(7)
    KVC_EXACT_CASE(8)
#undef KVC_EXACT_CASE
    default:
      return hipErrorInvalidValue;
  }
}

template <int METRIC>
static hipError_t launch_mfma_t(dim3 grid, size_t lds, const uint16_t* keys, long long head_stride, int L,
                                const uint16_t* chat, int C, int cpad, int cps, int32_t* labels,
                                long long label_stride, int32_t* queue, uint32_t* qcount, u32x4* op_t,
                                int32_t* dirty, float* norm2, int norm_mode, float* top2, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)assign_bf16_mfma_kernel<METRIC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  assign_bf16_mfma_kernel<METRIC><<<grid, AS_THREADS, lds, st>>>(keys, head_stride, L, chat, C, cpad, cps, labels,
                                                                 label_stride, queue, qcount, op_t, dirty, norm2,
                                                                 norm_mode, top2);
  return hipGetLastError();
}

hipError_t launch_assign(int dtype, const void* keys, long long head_stride, int heads, int L, const void* chat, int C,
                         int cpad, int cps, int metric, int32_t* labels, long long label_stride, int32_t* queue,
                         uint32_t* qcount, void* op_t, int32_t* dirty, float* norm2, int norm_mode, float* top2,
                         hipEvent_t* events, hipStream_t st) {
  u32x4* ot = static_cast<u32x4*>(op_t);
  if (dtype == DT_BF16) {
    const size_t lds = (size_t)(cpad + 16) * D * 2 + 16;  // the operand, one zero tile and a flag
    // about one block per compute unit; each walks over 768-key groups of one head
    const int ngroups = grid1(L, AS_TILE);
    int gx = (256 + heads - 1) / heads;
    gx = gx < 1 ? 1 : (gx > ngroups ? ngroups : gx);
    dim3 grid(gx, heads);
    if (events) {
      hipError_t e0 = hipEventRecord(events[0], st);
      if (e0 != hipSuccess) return e0;
    }
    const uint16_t* kk = (const uint16_t*)keys;
    const uint16_t* cc = (const uint16_t*)chat;
    hipError_t e;
    // variants: the fp32 biases and the largest norm follow the staged operand
    const size_t lds_var = lds + (size_t)cpad * 4 + 16;
    if (metric == M_L2)
      e = launch_mfma_t<M_L2>(grid, lds_var, kk, head_stride, L, cc, C, cpad, cps, labels, label_stride, queue,
                              qcount, ot, dirty, norm2, norm_mode, top2, st);
    else if (metric == M_IP)
      e = launch_mfma_t<M_IP>(grid, lds_var, kk, head_stride, L, cc, C, cpad, cps, labels, label_stride, queue,
                              qcount, ot, dirty, norm2, norm_mode, top2, st);
    else
      e = launch_mfma_t<M_COSINE>(grid, lds, kk, head_stride, L, cc, C, cpad, cps, labels, label_stride, queue,
                                  qcount, ot, dirty, norm2, norm_mode, top2, st);
    if (e != hipSuccess) return e;
    if (events) {
      e = hipEventRecord(events[1], st);
      if (e != hipSuccess) return e;
    }
    // exact re-scoring of the uncertified keys: 64 waves per head (128 keys a
    // pass); waves without a key exit at once
    return launch_exact<uint16_t>((const uint16_t*)keys, head_stride, L, (const uint16_t*)chat, C, cpad, cps, metric,
                                  labels, label_stride, queue, qcount, ot, dirty, dim3(heads, 64), st);
  }
  dim3 g2(heads, grid1(L, EX_NK) < 512 ? grid1(L, EX_NK) : 512);
  if (events) {
    hipError_t e0 = hipEventRecord(events[0], st);
    if (e0 != hipSuccess) return e0;
  }
  hipError_t e = launch_exact<float>((const float*)keys, head_stride, L, (const float*)chat, C, cpad, cps, metric,
                                     labels, label_stride, nullptr, nullptr, nullptr, dirty, g2, st);
  if (e == hipSuccess && events) e = hipEventRecord(events[1], st);
  return e;
}

hipError_t launch_csr(const int32_t* labels, long long label_stride, int heads, int L, int C, int cs, int32_t* hist,
                      int32_t* sizes, int32_t* offsets, int32_t* token_ids, long long ids_stride, int id_base,
                      hipStream_t st) {
  const int nblk = csr_blocks(L);
  csr_count_kernel<<<dim3(nblk, heads), 256, 0, st>>>(labels, label_stride, L, C, nblk, hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  csr_scan_kernel<<<heads, 512, 0, st>>>(C, cs, nblk, hist, sizes, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  csr_scatter_kernel<<<dim3(nblk, heads), CS_THREADS, 0, st>>>(labels, label_stride, L, C, cs, nblk, hist, offsets,
                                                               token_ids, ids_stride, id_base);
  return hipGetLastError();
}

hipError_t launch_update(int dtype, const void* keys, long long head_stride, int heads, int C, int cs, int cps,
                         int metric, const int32_t* sizes, const int32_t* offsets, const int32_t* token_ids, long long ids_stride,
                         float* cent, float* cent_t, void* chat, const int32_t* dirty, hipStream_t st) {
  dim3 grid(grid1(C, 4), heads);
  if (dtype == DT_BF16)
    update_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)keys, head_stride, C, cs, cps, metric, sizes,
                                                  offsets, token_ids, ids_stride, cent, cent_t, (uint16_t*)chat, dirty);
  else
    update_kernel<float><<<grid, 256, 0, st>>>((const float*)keys, head_stride, C, cs, cps, metric, sizes, offsets,
                                               token_ids, ids_stride, cent, cent_t, (float*)chat, dirty);
  return hipGetLastError();
}

hipError_t launch_merge_window(int dtype, int heads, int nc, int m, int wlo, const float* cent_w, const void* chat_w,
                               const int32_t* labels_w, const int32_t* sizes_w, const int32_t* offsets_w,
                               const int32_t* ids_w, int ca, int cs, int cps, float* cent, float* cent_t, void* chat,
                               int32_t* sizes, int32_t* offsets, int32_t* token_ids, int32_t* labels, long long cap,
                               hipStream_t st) {
  if (dtype == DT_BF16)
    merge_window_kernel<uint16_t><<<heads, 256, 0, st>>>(nc, m, wlo, cent_w, (const uint16_t*)chat_w, labels_w,
                                                         sizes_w, offsets_w, ids_w, ca, cs, cps, cent, cent_t,
                                                         (uint16_t*)chat, sizes, offsets, token_ids, labels, cap);
  else
    merge_window_kernel<float><<<heads, 256, 0, st>>>(nc, m, wlo, cent_w, (const float*)chat_w, labels_w, sizes_w,
                                                      offsets_w, ids_w, ca, cs, cps, cent, cent_t, (float*)chat, sizes,
                                                      offsets, token_ids, labels, cap);
  return hipGetLastError();
}

}  // namespace kvc
