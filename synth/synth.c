/*
 * Seeded synthetic inputs for the clustered sparse-KV path.
 *
 * This module only draws data. It holds none of the method's arithmetic, and
 * both the GPU library's tests and the CPU oracle consume the bytes it
 * writes. Every draw is counter-based, so any element can be produced
 * independently of the others (and in parallel):
 *
 *   SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014): the i-th output of a stream with seed s is
 *   mix(s + (i + 1) * 0x9E3779B97F4A7C15), where mix is the 64-bit finaliser.
 *
 *   uniform(s, i) = (top 53 bits of the i-th output + 1) * 2^-53, in (0, 1].
 *   normal(s, i)  = Box-Muller on the pair (uniform(s, 2p), uniform(s, 2p+1)),
 *                   p = i / 2; even i takes the cosine, odd i the sine.
 *   below(s, i, n) = floor(output * n / 2^64)   (multiply-shift, n < 2^32).
 *
 * Every stream's seed is stream_seed(base, a, b) = mix(base ^ mix(a * 2^16 + b)).
 * The generated values are rounded once, from fp64, to the requested storage
 * type (round to nearest, ties to even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t draw(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1) * GOLDEN); }

static double uniform01(uint64_t seed, uint64_t i) {
  return (double)((draw(seed, i) >> 11) + 1) * (1.0 / 9007199254740992.0);
}

static double normal01(uint64_t seed, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = uniform01(seed, 2 * p), u2 = uniform01(seed, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

static uint32_t below(uint64_t seed, uint64_t i, uint32_t n) {
  return (uint32_t)(((unsigned __int128)draw(seed, i) * n) >> 64);
}

uint64_t synth_stream_seed(uint64_t base, uint64_t a, uint64_t b) {
  return mix64(base ^ mix64((a << 16) + b));
}

uint64_t synth_config_seed(int config, int layer) {
  return mix64(0xC1A57E55ULL + 1000ULL * (uint64_t)config + (uint64_t)layer);
}

/* fp64 -> bf16 bits, round to nearest even (NaN kept quiet). */
static uint16_t to_bf16(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  if (isnan(x)) return 0x7FC0;
  /* Round directly from the fp64 bits: keep sign, exponent and the top 7
   * mantissa bits of the bf16 result. */
  uint32_t sign = (uint32_t)(b >> 63);
  double a = fabs(x);
  if (a == 0.0) return (uint16_t)(sign << 15);
  int e;
  (void)frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  /* bf16 normal range: exponent field 1..254, i.e. a in [2^-126, 2^128). */
  int ue = e - 1; /* a = (2m) * 2^ue, 2m in [1, 2) */
  double scaled;
  int q_exp = ue < -126 ? -126 : ue; /* subnormals share the 2^-126 scale */
  scaled = ldexp(a, 7 - q_exp);      /* integer part = significand in ulps */
  double fl = floor(scaled);
  double rem = scaled - fl; /* exact: scaled has <= 53 bits */
  uint64_t sig = (uint64_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (sig & 1))) sig += 1;
  /* sig counts ulps of 2^(q_exp-7); renormalise a carry into the exponent. */
  uint32_t out;
  if (ue < -126) {
    /* subnormal range: sig in [0, 128]; 128 becomes the smallest normal. */
    out = (uint32_t)sig; /* exponent field 0, or 1 when sig == 128 */
  } else {
    if (sig == 256) { sig = 128; q_exp += 1; }
    if (q_exp > 127) return (uint16_t)((sign << 15) | 0x7F80); /* overflow: inf */
    out = ((uint32_t)(q_exp + 127) << 7) | (uint32_t)(sig - 128);
  }
  return (uint16_t)((sign << 15) | out);
}

static void store(void* out, int dtype, size_t at, double v) {
  if (dtype == 1) ((uint16_t*)out)[at] = to_bf16(v);
  else ((float*)out)[at] = (float)v;
}

/* Round an fp64 array to bf16 bits (exposed for the tests of this module). */
void synth_round_bf16(const double* x, size_t n, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = to_bf16(x[i]);
}

/*
 * Gaussian-mixture keys, per head h (stream seeds derived from (base, h, s)):
 *   s=0  component means mu[m][j] ~ N(0, 1)             (index m*d + j)
 *   s=1  component of token i: below(.., i, M)
 *   s=2  noise eps[i][j] ~ N(0, 1)                      (index i*d + j)
 *   s=3  outlier channels: partial Fisher-Yates over [0, d), n_out picks
 *   key[i][j] = (mu[comp_i][j] + sigma * eps[i][j]) * (j outlier ? out_scale : 1)
 * Tokens i0 .. i0+n-1 are written to rows 0 .. n-1 of each head
 * (row stride d, head stride head_stride elements). means_out (optional) gets
 * the key-space means (outlier scaling applied), fp64 [H, M, d];
 * comp_out (optional) gets the component ids [H, n].
 */
void synth_mixture_keys(uint64_t base, int H, int i0, int n, int d, int M, double sigma,
                        int n_out, double out_scale, int dtype, void* out, long long head_stride,
                        int32_t* comp_out, double* means_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < H; ++h) {
    uint64_t s_mu = synth_stream_seed(base, (uint64_t)h, 0);
    uint64_t s_z = synth_stream_seed(base, (uint64_t)h, 1);
    uint64_t s_e = synth_stream_seed(base, (uint64_t)h, 2);
    uint64_t s_o = synth_stream_seed(base, (uint64_t)h, 3);
    double* mu = (double*)malloc(sizeof(double) * (size_t)M * d);
    double* scale = (double*)malloc(sizeof(double) * (size_t)d);
    int* perm = (int*)malloc(sizeof(int) * (size_t)d);
    for (size_t t = 0; t < (size_t)M * d; ++t) mu[t] = normal01(s_mu, t);
    for (int j = 0; j < d; ++j) { perm[j] = j; scale[j] = 1.0; }
    for (int t = 0; t < n_out && t < d; ++t) {
      int r = t + (int)below(s_o, (uint64_t)t, (uint32_t)(d - t));
      int tmp = perm[t]; perm[t] = perm[r]; perm[r] = tmp;
      scale[perm[t]] = out_scale;
    }
    if (means_out)
      for (int m = 0; m < M; ++m)
        for (int j = 0; j < d; ++j)
          means_out[((size_t)h * M + m) * d + j] = mu[(size_t)m * d + j] * scale[j];
    for (int r = 0; r < n; ++r) {
      uint64_t i = (uint64_t)i0 + (uint64_t)r;
      int comp = (int)below(s_z, i, (uint32_t)M);
      if (comp_out) comp_out[(size_t)h * n + r] = comp;
      size_t row = (size_t)h * (size_t)head_stride + (size_t)r * d;
      for (int j = 0; j < d; ++j) {
        double v = (mu[(size_t)comp * d + j] + sigma * normal01(s_e, i * (uint64_t)d + j)) * scale[j];
        store(out, dtype, row + j, v);
      }
    }
    free(mu); free(scale); free(perm);
  }
}

/* Values ~ N(0, sigma^2), per head stream (base, h, 4), index i*d + j. */
void synth_values(uint64_t base, int H, int i0, int n, int d, double sigma, int dtype, void* out,
                  long long head_stride) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < H; ++h) {
    uint64_t s_v = synth_stream_seed(base, (uint64_t)h, 4);
    for (int r = 0; r < n; ++r) {
      uint64_t i = (uint64_t)i0 + (uint64_t)r;
      size_t row = (size_t)h * (size_t)head_stride + (size_t)r * d;
      for (int j = 0; j < d; ++j) store(out, dtype, row + j, sigma * normal01(s_v, i * (uint64_t)d + j));
    }
  }
}

/*
 * Seeded shuffle for the initial centroids: per head h, a partial
 * Fisher-Yates over [0, L) driven by stream (base, h, 5); the first C
 * positions of the shuffled order are written to out[h*C .. h*C + C).
 */
void synth_init_idx(uint64_t base, int H, int L, int C, int32_t* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < H; ++h) {
    uint64_t s = synth_stream_seed(base, (uint64_t)h, 5);
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)L);
    for (int i = 0; i < L; ++i) perm[i] = i;
    for (int i = 0; i < C && i < L; ++i) {
      int j = i + (int)below(s, (uint64_t)i, (uint32_t)(L - i));
      int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
      out[(size_t)h * C + i] = perm[i];
    }
    free(perm);
  }
}

/*
 * Queries that are noisy copies of a random current key: for query head g
 * (KV head g / G) at decode step `step`, stream (base ^ mix(step + 1), g, 6):
 * draw 0 picks r = below(.., 0, n_cur), then q[j] = key[r][j] + sigma * N(0,1)
 * (normal index 2 + j). keys holds the stored (already rounded) keys of each
 * KV head with the given head stride.
 */
void synth_queries_noisy_key(uint64_t base, int step, int Hq, int G, int d, int n_cur,
                             const void* keys, int dtype, long long head_stride, double sigma,
                             void* out) {
  uint64_t sb = base ^ mix64((uint64_t)step + 1);
  for (int g = 0; g < Hq; ++g) {
    uint64_t s = synth_stream_seed(sb, (uint64_t)g, 6);
    int h = g / G;
    uint32_t r = below(s, 0, (uint32_t)n_cur);
    size_t row = (size_t)h * (size_t)head_stride + (size_t)r * d;
    for (int j = 0; j < d; ++j) {
      double kv;
      if (dtype == 1) {
        uint32_t bits = (uint32_t)((const uint16_t*)keys)[row + j] << 16;
        float f; memcpy(&f, &bits, 4); kv = f;
      } else {
        kv = ((const float*)keys)[row + j];
      }
      store(out, dtype, (size_t)g * d + j, kv + sigma * normal01(s, 2 + (uint64_t)j));
    }
  }
}

/*
 * Queries that are a random mixture of three component means: for query head
 * g (KV head h = g / G) at step `step`, stream (base ^ mix(step + 1), g, 7):
 * draws 0..2 pick three distinct components by a partial Fisher-Yates over
 * [0, M); uniforms 3..5 give Dirichlet(1,1,1) weights w_a = e_a / sum(e),
 * e_a = -log(u); q[j] = sum_a w_a * means[h][m_a][j] + sigma * N(0,1)
 * (normal index 8 + j). means are the key-space component means.
 */
void synth_queries_mixture(uint64_t base, int step, int Hq, int G, int d, int M,
                           const double* means, double sigma, int dtype, void* out) {
  uint64_t sb = base ^ mix64((uint64_t)step + 1);
  for (int g = 0; g < Hq; ++g) {
    uint64_t s = synth_stream_seed(sb, (uint64_t)g, 7);
    int h = g / G;
    int pick[3];
    int* perm = (int*)malloc(sizeof(int) * (size_t)M);
    for (int m = 0; m < M; ++m) perm[m] = m;
    int na = M < 3 ? M : 3;
    for (int a = 0; a < na; ++a) {
      int r = a + (int)below(s, (uint64_t)a, (uint32_t)(M - a));
      int t = perm[a]; perm[a] = perm[r]; perm[r] = t;
      pick[a] = perm[a];
    }
    free(perm);
    double e[3], se = 0.0;
    for (int a = 0; a < na; ++a) { e[a] = -log(uniform01(s, 3 + (uint64_t)a)); se += e[a]; }
    for (int j = 0; j < d; ++j) {
      double v = 0.0;
      for (int a = 0; a < na; ++a) v += (e[a] / se) * means[((size_t)h * M + pick[a]) * d + j];
      store(out, dtype, (size_t)g * d + j, v + sigma * normal01(s, 8 + (uint64_t)j));
    }
  }
}

/*
 * Mixture queries that drift over decoding steps: query head g mixes three
 * component means of its KV head, as synth_queries_mixture does, but each of
 * the three slots keeps its component and weight until a change event (an
 * independent per-slot, per-step draw below p_change), and only the noise is
 * new at every step. Consecutive steps therefore attend to overlapping parts of
 * the context. Stateless: the epoch of slot a at step t is the number of events
 * in steps 1 .. t, recounted from the seed.
 */
void synth_queries_drift(uint64_t base, int step, int Hq, int G, int d, int M, const double* means, double sigma,
                         double p_change, int dtype, void* out) {
  const uint64_t nb = base ^ mix64((uint64_t)step + 0x5151);
  for (int g = 0; g < Hq; ++g) {
    const int h = g / G;
    int pick[3];
    double e[3], se = 0.0;
    for (int a = 0; a < 3; ++a) {
      const uint64_t slot = synth_stream_seed(base, (uint64_t)g, 100 + (uint64_t)a);
      uint64_t epoch = 0;
      for (int u = 1; u <= step; ++u)
        if (uniform01(slot, (uint64_t)u) < p_change) ++epoch;
      const uint64_t es = synth_stream_seed(slot, epoch, 1);
      pick[a] = (int)below(es, 0, (uint32_t)M);
      e[a] = -log(uniform01(es, 1));
      se += e[a];
    }
    const uint64_t ns = synth_stream_seed(nb, (uint64_t)g, 9);
    for (int j = 0; j < d; ++j) {
      double v = 0.0;
      for (int a = 0; a < 3; ++a) v += (e[a] / se) * means[((size_t)h * M + pick[a]) * d + j];
      store(out, dtype, (size_t)g * d + j, v + sigma * normal01(ns, (uint64_t)j));
    }
  }
}

/* Plain N(0, sigma^2) array from one stream (used for tiny test cases). */
void synth_normal_array(uint64_t seed, size_t n, double sigma, int dtype, void* out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) store(out, dtype, (size_t)i, sigma * normal01(seed, (uint64_t)i));
}
