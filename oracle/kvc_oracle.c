/*
 * CPU oracle for the clustered sparse-KV hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file. The GPU library
 * shares no code with it, and it is never a fallback for the GPU path.
 *
 * The method is ClusterKV, "Manipulating LLM KV Cache in Semantic Space for
 * Recallable Compression" (arXiv 2412.03213). Citations below name the
 * section of the paper summary page (paperlayer.ai, 2412.03213v2) that
 * defines each step:
 *   - III.A  Problem Formulation and Design Rationale
 *   - III.B  Clustering in the Semantic Space
 *   - III.C  Selection at the Granularity of Semantic Clusters
 *   - Sys-B  "B. Semantic Clustering" (system part)
 *   - Sys-C  "C. Selection and Indexing" (system part, Fig. 8)
 *   - II.A   "A. LLM Inference and KV Cache"
 *
 * Numerics. Every reduction that feeds a discrete decision (an argmax, a
 * ranking) is a fixed-order fp64 chain s = fma(a_j, b_j, s) over ascending j.
 * Products of bf16 or fp32 operands are exact in fp64, so that chain is a
 * complete definition of the score. Continuous outputs are computed in fp64
 * and rounded once to their storage type.
 *
 * Element types: 0 = fp32, 1 = bf16 (raw 16-bit patterns), 2 = fp64 (the
 * "exact" mode, where the normalised centroid is not rounded at all).
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * brute force, closed forms or invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2

/* Assignment distance. III.B defines the semantic distance by the cosine and
 * names L2 and inner-product distance as the alternatives it is preferred to;
 * the model-accuracy section compares the three. */
#define ORC_COSINE 0
#define ORC_L2 1
#define ORC_IP 2

/* ---------------------------------------------------------------- scalars */

static double bf16_bits_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double ld(const void* p, int dt, size_t i) {
  if (dt == ORC_BF16) return bf16_bits_to_f64(((const uint16_t*)p)[i]);
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  return ((const double*)p)[i];
}

/* fp64 -> bf16, round to nearest with ties to even, from the fp64 fields. */
uint16_t orc_round_bf16(double x) {
  uint64_t u;
  memcpy(&u, &x, 8);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  int E = (int)((u >> 52) & 0x7FF);
  uint64_t M = u & ((1ULL << 52) - 1);
  if (E == 0x7FF) return M ? (uint16_t)(sign | 0x7FC0) : (uint16_t)(sign | 0x7F80);
  if (E == 0) return sign; /* fp64 subnormal or zero: far below bf16's range */
  int e = E - 1023;        /* |x| = 1.M * 2^e */
  if (e >= -126) {
    uint64_t keep = M >> 45, rest = M & ((1ULL << 45) - 1), half = 1ULL << 44;
    if (rest > half || (rest == half && (keep & 1))) keep += 1;
    if (keep == 128) { keep = 0; e += 1; }
    if (e > 127) return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint16_t)((e + 127) << 7) | (uint16_t)keep);
  }
  /* bf16 subnormal: count units of 2^-133 in S * 2^(e-52), S = 1.M scaled. */
  uint64_t S = (1ULL << 52) | M;
  int shift = 52 - (e + 133);
  if (shift >= 64) return sign;
  uint64_t q = S >> shift, rest = S & ((1ULL << shift) - 1), half = 1ULL << (shift - 1);
  if (rest > half || (rest == half && (q & 1))) q += 1;
  return (uint16_t)(sign | (uint16_t)q); /* q == 128 encodes the smallest normal */
}

static void st(void* p, int dt, size_t i, double v) {
  if (dt == ORC_BF16) ((uint16_t*)p)[i] = orc_round_bf16(v);
  else if (dt == ORC_F32) ((float*)p)[i] = (float)v;
  else ((double*)p)[i] = v;
}

/* fp64 chain over ascending j: sum_j a[j] * b[j]. */
static double chain_dot(int d, const void* a, int adt, size_t ao, const void* b, int bdt, size_t bo) {
  double s = 0.0;
  for (int j = 0; j < d; ++j) s = fma(ld(a, adt, ao + j), ld(b, bdt, bo + j), s);
  return s;
}

/* ------------------------------------------------------------- clustering */

/*
 * Normalise centroids to unit length (III.B: the semantic distance is the
 * cosine, so only a centroid's direction matters to the assignment).
 * norm_k = sqrt(fp64 chain of c_kj^2); chat_kj = round_op(c_kj / norm_k);
 * a zero centroid gives chat_k = 0.
 */
void orc_normalize(int C, int d, const void* c, int cdt, void* chat, int optype) {
  for (int k = 0; k < C; ++k) {
    size_t o = (size_t)k * d;
    double ss = chain_dot(d, c, cdt, o, c, cdt, o);
    double nrm = sqrt(ss);
    for (int j = 0; j < d; ++j) {
      double v = nrm > 0.0 ? ld(c, cdt, o + j) / nrm : 0.0;
      st(chat, optype, o + j, v);
    }
  }
}

/*
 * The assignment operand of C centroids, rounded once to optype.
 *  - cosine: the unit direction (orc_normalize);
 *  - L2 and inner product: the centroid itself, chat_kj = round_op(c_kj).
 */
void orc_operand(int C, int d, const void* c, int cdt, void* chat, int optype, int metric) {
  if (metric == ORC_COSINE) {
    orc_normalize(C, d, c, cdt, chat, optype);
    return;
  }
  for (size_t e = 0; e < (size_t)C * d; ++e) st(chat, optype, e, ld(c, cdt, e));
}

/*
 * Assignment (III.B: each key joins its nearest centroid under the semantic
 * distance). Exact ties go to the lowest k.
 *  - cosine: ||K_i|| is a positive per-key constant, so the cosine argmax is
 *    argmax_k K_i . chat_k (chat the unit direction);
 *  - inner product: argmax_k K_i . chat_k (chat the centroid);
 *  - L2: argmin_k ||K_i - chat_k||^2 = argmax_k (K_i . chat_k - nn_k / 2),
 *    since ||K_i||^2 is a per-key constant; nn_k = fp64 chain of chat_kj^2
 *    over ascending j, and the score is the fp64 difference.
 *
 * The loop nest computes the chains of all k for one key together: each
 * s[k] is still the chain over ascending j, so the scores are the chain's.
 * best (optional) receives the winning score.
 */
void orc_assign(int L, int d, int C, const void* K, int kdt, long long row_stride, const void* chat,
                int optype, int metric, int32_t* labels, double* best) {
  double* cT = (double*)malloc(sizeof(double) * (size_t)d * C);
  double* s = (double*)malloc(sizeof(double) * (size_t)C);
  double* half_nn = (double*)calloc((size_t)C, sizeof(double));
  for (int k = 0; k < C; ++k)
    for (int j = 0; j < d; ++j) cT[(size_t)j * C + k] = ld(chat, optype, (size_t)k * d + j);
  if (metric == ORC_L2)
    for (int k = 0; k < C; ++k)
      half_nn[k] = 0.5 * chain_dot(d, chat, optype, (size_t)k * d, chat, optype, (size_t)k * d);
  for (int i = 0; i < L; ++i) {
    size_t ro = (size_t)i * (size_t)row_stride;
    for (int k = 0; k < C; ++k) s[k] = 0.0;
    for (int j = 0; j < d; ++j) {
      double kij = ld(K, kdt, ro + j);
      const double* cj = cT + (size_t)j * C;
      for (int k = 0; k < C; ++k) s[k] = fma(kij, cj[k], s[k]);
    }
    if (metric == ORC_L2)
      for (int k = 0; k < C; ++k) s[k] = s[k] - half_nn[k];
    int arg = 0;
    for (int k = 1; k < C; ++k)
      if (s[k] > s[arg]) arg = k;
    labels[i] = arg;
    if (best) best[i] = s[arg];
  }
  free(cT);
  free(s);
  free(half_nn);
}

/*
 * Centroid update (III.B: each centroid becomes the mean of the keys
 * assigned to it; Sys-B: the kernel accumulates the assigned keys and counts
 * them, then divides). Raw keys are averaged. The sum runs in fp64 over
 * members in ascending token order and is rounded once to the centroid type
 * after the division. An empty cluster keeps its previous centroid.
 */
void orc_update(int L, int d, int C, const void* K, int kdt, long long row_stride,
                const int32_t* labels, void* c, int cdt, int32_t* counts) {
  double* sum = (double*)calloc((size_t)C * d, sizeof(double));
  int32_t* n = (int32_t*)calloc((size_t)C, sizeof(int32_t));
  for (int i = 0; i < L; ++i) {
    int k = labels[i];
    n[k] += 1;
    for (int j = 0; j < d; ++j) sum[(size_t)k * d + j] += ld(K, kdt, (size_t)i * (size_t)row_stride + j);
  }
  for (int k = 0; k < C; ++k) {
    if (n[k] > 0)
      for (int j = 0; j < d; ++j) st(c, cdt, (size_t)k * d + j, sum[(size_t)k * d + j] / (double)n[k]);
    if (counts) counts[k] = n[k];
  }
  free(sum);
  free(n);
}

/*
 * Cluster index (Sys-C: after clustering, the metadata kept is the cluster
 * sizes, their prefix sums and the token indices sorted by cluster).
 * A stable counting sort: within a cluster, token ids ascend.
 */
void orc_csr(int L, int C, const int32_t* labels, int32_t* sizes, int32_t* offsets, int32_t* token_ids) {
  for (int k = 0; k < C; ++k) sizes[k] = 0;
  for (int i = 0; i < L; ++i) sizes[labels[i]] += 1;
  offsets[0] = 0;
  for (int k = 0; k < C; ++k) offsets[k + 1] = offsets[k] + sizes[k];
  int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
  for (int k = 0; k < C; ++k) cur[k] = offsets[k];
  for (int i = 0; i < L; ++i) token_ids[cur[labels[i]]++] = i;
  free(cur);
}

/*
 * The k-means objective of an assignment under each distance:
 *  - cosine: the norm-weighted cosine distance
 *    I = sum_i (||K_i|| - K_i . chat_{label_i}) = sum_i ||K_i|| (1 - cos);
 *  - L2: I = sum_i ||K_i - chat_{label_i}||^2;
 *  - inner product: I = -sum_i K_i . chat_{label_i}.
 */
double orc_inertia(int L, int d, const void* K, int kdt, long long row_stride, const void* chat,
                   int optype, int metric, const int32_t* labels) {
  double I = 0.0;
  for (int i = 0; i < L; ++i) {
    size_t ro = (size_t)i * (size_t)row_stride, co = (size_t)labels[i] * d;
    if (metric == ORC_L2) {
      double e = 0.0;
      for (int j = 0; j < d; ++j) {
        double t = ld(K, kdt, ro + j) - ld(chat, optype, co + j);
        e = fma(t, t, e);
      }
      I += e;
    } else if (metric == ORC_IP) {
      I -= chain_dot(d, K, kdt, ro, chat, optype, co);
    } else {
      double nk = sqrt(chain_dot(d, K, kdt, ro, K, kdt, ro));
      I += nk - chain_dot(d, K, kdt, ro, chat, optype, co);
    }
  }
  return I;
}

static size_t esize(int dt) { return dt == ORC_BF16 ? 2 : (dt == ORC_F32 ? 4 : 8); }

/*
 * Initial centroids by a seeded shuffle (the pages leave the initialisation
 * open; III.B only says that the k-means iterates until the assignment
 * settles). The reading: the initial centroids are the keys at the first C
 * positions of a seeded random permutation of the clustered rows.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; the widely used 64-bit
 * finaliser constants): the state advances by the golden-ratio increment
 * 0x9E3779B97F4A7C15 and each output is the state after the advance, mixed by
 *   z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
 *   z ^= z >> 31.
 * Head h starts from state seed ^ (0x9E3779B97F4A7C15 * (h + 1)) (mod 2^64).
 *
 * Shuffle: the clustered rows are lo .. L-1 (lo = the attention sinks kept
 * apart), n = L - lo of them. perm = (0, 1, ..., n-1); for i = 0 .. C-1 in
 * order, j = i + (next output mod (n - i)) and perm[i], perm[j] swap (a
 * partial Fisher-Yates shuffle). out[h*C + k] = lo + perm[k].
 * Requires 1 <= C <= n.
 */
static uint64_t splitmix64_next(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ULL;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

int orc_init(int H, int lo, int L, int C, uint64_t seed, int32_t* out) {
  int n = L - lo;
  if (lo < 0 || C < 1 || C > n) return -1;
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  for (int h = 0; h < H; ++h) {
    uint64_t state = seed ^ (0x9E3779B97F4A7C15ULL * (uint64_t)(h + 1));
    for (int i = 0; i < n; ++i) perm[i] = i;
    for (int i = 0; i < C; ++i) {
      uint64_t r = splitmix64_next(&state);
      int j = i + (int)(r % (uint64_t)(n - i));
      int32_t t = perm[i];
      perm[i] = perm[j];
      perm[j] = t;
      out[(size_t)h * C + i] = lo + perm[i];
    }
  }
  free(perm);
  return 0;
}

/*
 * Prefill clustering of H independent heads (III.B; Sys-B batches heads).
 * K: keys [H, *, d] with head stride head_stride elements and row stride d;
 * the first L rows of each head are clustered.
 * init_idx [H, C]: the token positions whose keys are the initial centroids
 * (the seeded shuffle is an input; the oracle copies those keys exactly).
 * mode: 0 = operand type of the input (fp32 centroids, chat in the key type),
 *       1 = exact (fp64 centroids, fp64 chat).
 * metric: the assignment distance (cosine, the method's; L2 or inner product).
 * Per iteration t: chat = operand(c); labels = assign(chat); c = update.
 * With early_exit, stops when labels repeat (every later iteration would
 * reproduce the same state). The outputs are the final centroids (means of
 * the final labels), chat_final = normalise(final c), labels and the
 * cluster index. inertia [H, iters] gets I_t for each run iteration
 * (NaN after an early exit); iters_run [H] the count.
 * Returns 0, or -1 if an init index is out of range.
 */
int orc_build(int H, int L, int d, int C, int iters, int kdt, int mode, int metric, const void* K,
              long long head_stride, const int32_t* init_idx, void* c_out, void* chat_out,
              int32_t* labels, int32_t* sizes, int32_t* offsets, int32_t* token_ids, double* inertia,
              int32_t* iters_run, int early_exit) {
  int cdt = mode == 1 ? ORC_F64 : ORC_F32;
  int optype = mode == 1 ? ORC_F64 : kdt;
  for (int h = 0; h < H; ++h)
    for (int k = 0; k < C; ++k)
      if (init_idx[(size_t)h * C + k] < 0 || init_idx[(size_t)h * C + k] >= L) return -1;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < H; ++h) {
    const char* Kh = (const char*)K + (size_t)h * (size_t)head_stride * esize(kdt);
    char* ch = (char*)c_out + (size_t)h * C * d * esize(cdt);
    char* chh = (char*)chat_out + (size_t)h * C * d * esize(optype);
    int32_t* lab = labels + (size_t)h * L;
    int32_t* prev = (int32_t*)malloc(sizeof(int32_t) * (size_t)L);
    for (int k = 0; k < C; ++k)
      for (int j = 0; j < d; ++j)
        st(ch, cdt, (size_t)k * d + j, ld(Kh, kdt, (size_t)init_idx[(size_t)h * C + k] * d + j));
    int t = 0;
    for (; t < iters; ++t) {
      orc_operand(C, d, ch, cdt, chh, optype, metric);
      orc_assign(L, d, C, Kh, kdt, d, chh, optype, metric, lab, NULL);
      if (inertia) inertia[(size_t)h * iters + t] = orc_inertia(L, d, Kh, kdt, d, chh, optype, metric, lab);
      orc_update(L, d, C, Kh, kdt, d, lab, ch, cdt, NULL);
      if (early_exit && t > 0 && memcmp(prev, lab, sizeof(int32_t) * (size_t)L) == 0) { ++t; break; }
      memcpy(prev, lab, sizeof(int32_t) * (size_t)L);
    }
    if (inertia)
      for (int u = t; u < iters; ++u) inertia[(size_t)h * iters + u] = NAN;
    if (iters_run) iters_run[h] = t;
    orc_operand(C, d, ch, cdt, chh, optype, metric);
    orc_csr(L, C, lab, sizes + (size_t)h * C, offsets + (size_t)h * (C + 1), token_ids + (size_t)h * L);
    free(prev);
  }
  return err;
}

/*
 * Decode-time append of one token per head: the new key joins its nearest
 * existing centroid under the assignment rule above (chat_final); centroids
 * do not move. The token id n_cur goes to the end of its cluster's segment,
 * so segments stay in ascending order. The canonical index arrays
 * (sizes [C], offsets [C+1], token_ids [n_cur + 1]) are updated in place.
 * Returns the label.
 */
int orc_append(int d, int C, int n_cur, const void* knew, int kdt, const void* chat, int optype, int metric,
               int32_t* labels, int32_t* sizes, int32_t* offsets, int32_t* token_ids) {
  int32_t lab;
  orc_assign(1, d, C, knew, kdt, d, chat, optype, metric, &lab, NULL);
  int pos = offsets[lab + 1];
  for (int p = n_cur; p > pos; --p) token_ids[p] = token_ids[p - 1];
  token_ids[pos] = n_cur;
  for (int k = lab + 1; k <= C; ++k) offsets[k] += 1;
  sizes[lab] += 1;
  labels[n_cur] = lab;
  return lab;
}

typedef struct { double s; int k; } scored;

static int cmp_scored(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->k > y->k) - (x->k < y->k);
}

/*
 * Cluster-granular selection for H KV heads (III.C: rank the centroids by
 * attention weight to the query and take tokens from the top clusters until
 * the budget B is met; Sys-C, Fig. 8: sizes and prefix sums decide which
 * clusters fit, and the last one is trimmed).
 *  - G query heads share KV head h (query head g maps to h = g / G); their
 *    query is summed: qbar_j = fp64 sum over ascending g.
 *  - score_k = fp64 chain qbar . c_k (c the fp32 means). softmax(x / sqrt(d))
 *    is increasing in x, so the logit ranks the same as the weight.
 *  - Order by (score descending, k ascending); walk that order, taking
 *    min(n_k, B - taken) tokens of each cluster, i.e. the first tokens of
 *    its ascending segment, until B tokens are taken or clusters run out.
 * sel_ids [H, B] receives the ids in that order (-1 past sel_count);
 * sel_count [H] = min(B, tokens). scores [H, C] and order [H, C] (optional)
 * receive the scores and the full ranking.
 */
void orc_select(int H, int G, int d, int C, int B, const void* q, int qdt, const float* c,
                const int32_t* sizes, const int32_t* offsets, const int32_t* token_ids,
                long long ids_stride, int32_t* sel_ids, int32_t* sel_count, double* scores,
                int32_t* order) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < H; ++h) {
    double* qbar = (double*)calloc((size_t)d, sizeof(double));
    scored* sc = (scored*)malloc(sizeof(scored) * (size_t)C);
    for (int g = 0; g < G; ++g)
      for (int j = 0; j < d; ++j) qbar[j] = qbar[j] + ld(q, qdt, ((size_t)h * G + g) * d + j);
    for (int k = 0; k < C; ++k) {
      sc[k].s = chain_dot(d, qbar, ORC_F64, 0, c, ORC_F32, ((size_t)h * C + k) * d);
      sc[k].k = k;
      if (scores) scores[(size_t)h * C + k] = sc[k].s;
    }
    qsort(sc, (size_t)C, sizeof(scored), cmp_scored);
    const int32_t* sz = sizes + (size_t)h * C;
    const int32_t* off = offsets + (size_t)h * (C + 1);
    const int32_t* ids = token_ids + (size_t)h * (size_t)ids_stride;
    int32_t* out = sel_ids + (size_t)h * B;
    int taken = 0;
    for (int r = 0; r < C; ++r) {
      if (order) order[(size_t)h * C + r] = sc[r].k;
      if (taken >= B) continue;
      int k = sc[r].k;
      int m = sz[k] < B - taken ? sz[k] : B - taken;
      for (int t = 0; t < m; ++t) out[taken + t] = ids[off[k] + t];
      taken += m;
    }
    for (int t = taken; t < B; ++t) out[t] = -1;
    sel_count[h] = taken;
    free(qbar);
    free(sc);
  }
}

/*
 * Single-query attention over the recalled tokens only (II.A: the latest
 * query attends to the cached keys and values through softmax of the
 * query-key scores applied to the values; III.A: attention over the B
 * selected tokens approximates the full computation).
 * For query head g (KV head h = g / G):
 *   z_i = scale * (fp64 chain q_g . K_i) over the selected i,
 *   o   = sum_i exp(z_i - max z) V_i / sum_i exp(z_i - max z), rounded to fp32.
 * With no selected token the output is zero.
 */
void orc_decode(int H, int G, int d, const void* q, int qdt, const void* Kc, const void* Vc, int kdt,
                long long head_stride, const int32_t* sel_ids, const int32_t* sel_count, int B,
                double scale, float* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int g = 0; g < H * G; ++g) {
    int h = g / G;
    int n = sel_count[h];
    const int32_t* sel = sel_ids + (size_t)h * B;
    double* z = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* num = (double*)calloc((size_t)d, sizeof(double));
    double m = -INFINITY, den = 0.0;
    for (int t = 0; t < n; ++t) {
      size_t ro = (size_t)h * (size_t)head_stride + (size_t)sel[t] * d;
      z[t] = scale * chain_dot(d, q, qdt, (size_t)g * d, Kc, kdt, ro);
      if (z[t] > m) m = z[t];
    }
    for (int t = 0; t < n; ++t) {
      double w = exp(z[t] - m);
      size_t ro = (size_t)h * (size_t)head_stride + (size_t)sel[t] * d;
      den += w;
      for (int j = 0; j < d; ++j) num[j] += w * ld(Vc, kdt, ro + j);
    }
    for (int j = 0; j < d; ++j) out[(size_t)g * d + j] = n > 0 ? (float)(num[j] / den) : 0.0f;
    free(z);
    free(num);
  }
}

/*
 * Selection quality (III.A: the selection that attention over B tokens
 * should approximate is the B tokens with the largest attention weights).
 * For query head g (KV head h = g / G) over the first N rows of the head:
 * the exact top min(B, N) tokens by the fp64 chain q_g . K_t (equal logits:
 * the lower position first; softmax is increasing, so logits rank like the
 * weights), and recall[g] = |top set and selected set of h| / min(B, N),
 * where the selected set is sel_ids[h, 0 .. sel_count[h]).
 */
typedef struct {
  double s;
  int t;
} logit_t;

static int cmp_logit(const void* a, const void* b) {
  const logit_t* x = (const logit_t*)a;
  const logit_t* y = (const logit_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->t > y->t) - (x->t < y->t);
}

void orc_recall(int H, int G, int d, int N, int B, const void* q, int qdt, const void* Kc, int kdt,
                long long head_stride, const int32_t* sel_ids, const int32_t* sel_count, double* recall) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int g = 0; g < H * G; ++g) {
    const int h = g / G;
    const int top = B < N ? B : N;
    logit_t* z = (logit_t*)malloc(sizeof(logit_t) * (size_t)(N > 0 ? N : 1));
    unsigned char* in_top = (unsigned char*)calloc((size_t)(N > 0 ? N : 1), 1);
    for (int t = 0; t < N; ++t) {
      z[t].s = chain_dot(d, q, qdt, (size_t)g * d, Kc, kdt, (size_t)h * (size_t)head_stride + (size_t)t * d);
      z[t].t = t;
    }
    qsort(z, (size_t)N, sizeof(logit_t), cmp_logit);
    for (int r = 0; r < top; ++r) in_top[z[r].t] = 1;
    int hit = 0;
    for (int i = 0; i < sel_count[h]; ++i) {
      const int t = sel_ids[(size_t)h * B + i];
      if (t >= 0 && t < N && in_top[t]) ++hit;
    }
    recall[g] = top > 0 ? (double)hit / (double)top : 1.0;
    free(z);
    free(in_top);
  }
}

