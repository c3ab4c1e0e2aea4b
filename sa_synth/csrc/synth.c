/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file produces the input tensors (queries, key/value caches, planted
 * positions, projections) that both the GPU path and the CPU oracle consume.
 * It holds none of the attention method's arithmetic: no scoring, no
 * selection, no softmax.  Every value is a pure function of
 * (seed, stream, counter), so any slice of any tensor can be regenerated on
 * its own, in any order, by any number of threads, with identical bits.
 *
 * Generator definition (published algorithms, restated here):
 *   - mix64: the SplitMix64 output function (Steele, Lea and Flood,
 *     "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014):
 *       z ^= z >> 30; z *= 0xbf58476d1ce4e5b9;
 *       z ^= z >> 27; z *= 0x94d049bb133111eb;
 *       z ^= z >> 31.
 *   - key(seed, stream)   = mix64(mix64(seed) ^ mix64(stream + GAMMA))
 *     with GAMMA = 0x9e3779b97f4a7c15 (the SplitMix64 increment).
 *   - word(key, c)        = mix64(key + (c + 1) * GAMMA)      (counter mode)
 *   - uniform(key, c)     = ((word >> 11) + 0.5) * 2^-53, in (0, 1).
 *   - normal(key, i):     Box-Muller (1958) on the pair j = i >> 1:
 *       u1 = uniform(key, 2j), u2 = uniform(key, 2j + 1),
 *       r = sqrt(-2 ln u1), th = 2 pi u2,
 *       normal = r cos th  for even i,  r sin th  for odd i   (fp64, libm).
 *   - storage: fp64 -> fp32 by round-to-nearest-even (the C cast);
 *              fp32 -> bf16 by round-to-nearest-even on the bit pattern.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9e3779b97f4a7c15ULL

enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2 };

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t make_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ mix64(stream + GAMMA));
}

static inline uint64_t word_at(uint64_t key, uint64_t c) { return mix64(key + (c + 1) * GAMMA); }

static inline double uniform_at(uint64_t key, uint64_t c) {
  return ((double)(word_at(key, c) >> 11) + 0.5) * 0x1.0p-53;
}

static inline double normal_at(uint64_t key, uint64_t i) {
  const uint64_t j = i >> 1;
  const double u1 = uniform_at(key, 2 * j);
  const double u2 = uniform_at(key, 2 * j + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* Both members of pair j: normal(key, 2j) and normal(key, 2j + 1). */
static inline void normal_pair(uint64_t key, uint64_t j, double* z0, double* z1) {
  const double u1 = uniform_at(key, 2 * j);
  const double u2 = uniform_at(key, 2 * j + 1);
  const double r = sqrt(-2.0 * log(u1));
  double sn, cs;
  sincos(6.283185307179586476925286766559 * u2, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline void store(void* out, int kind, int64_t pos, double v) {
  if (kind == OUT_F64) {
    ((double*)out)[pos] = v;
  } else if (kind == OUT_F32) {
    ((float*)out)[pos] = (float)v;
  } else {
    ((uint16_t*)out)[pos] = f32_to_bf16_rne((float)v);
  }
}

/* out[pos0 + (c - c0)] = mean + sd * normal(key, c) for c in [c0, c1). */
static void fill_range(uint64_t key, uint64_t c0, uint64_t c1, double mean, double sd, int kind,
                       void* out, int64_t pos0) {
  uint64_t c = c0;
  if (c < c1 && (c & 1)) {
    store(out, kind, pos0, mean + sd * normal_at(key, c));
    ++c;
  }
  for (; c + 1 < c1; c += 2) {
    double z0, z1;
    normal_pair(key, c >> 1, &z0, &z1);
    store(out, kind, pos0 + (int64_t)(c - c0), mean + sd * z0);
    store(out, kind, pos0 + (int64_t)(c - c0) + 1, mean + sd * z1);
  }
  if (c < c1) store(out, kind, pos0 + (int64_t)(c - c0), mean + sd * normal_at(key, c));
}

/* Stream id of one (tensor tag, layer, batch, head) slab. */
uint64_t synth_stream_id(uint32_t tag, uint32_t layer, uint32_t b, uint32_t h) {
  uint64_t s = mix64((uint64_t)tag + 0x100000001b3ULL);
  s = mix64(s ^ ((uint64_t)layer + 0x51ULL));
  s = mix64(s ^ ((uint64_t)b + 0x9dULL));
  s = mix64(s ^ ((uint64_t)h + 0x3bULL));
  return s;
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t c) {
  return word_at(make_key(seed, stream), c);
}

/* out[k] = mean + sd * normal(key, start + k), k < count, stored as `kind`. */
void synth_normal(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, double mean,
                  double sd, int kind, void* out) {
  const uint64_t key = make_key(seed, stream);
  const int64_t chunk = 8192;
  const int64_t n_chunks = (count + chunk - 1) / chunk;
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < n_chunks; ++w) {
    const int64_t k0 = w * chunk;
    const int64_t k1 = k0 + chunk < count ? k0 + chunk : count;
    fill_range(key, start + (uint64_t)k0, start + (uint64_t)k1, mean, sd, kind, out, k0);
  }
}

/* Fill a [B, H, per_slab] tensor holding sequences b0 .. b0+B-1: slab (b, h)
 * uses stream (tag, layer, b0 + b, h), counters 0 .. per_slab-1. */
void synth_fill_normal(uint64_t seed, uint32_t tag, uint32_t layer, int64_t b0, int64_t B, int64_t H,
                       int64_t per_slab, double mean, double sd, int kind, void* out) {
  const int64_t n_slab = B * H;
  const int64_t chunk = 4096;
  const int64_t chunks_per_slab = (per_slab + chunk - 1) / chunk;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t w = 0; w < n_slab * chunks_per_slab; ++w) {
    const int64_t slab = w / chunks_per_slab;
    const int64_t c0 = (w % chunks_per_slab) * chunk;
    const int64_t c1 = c0 + chunk < per_slab ? c0 + chunk : per_slab;
    const uint64_t key =
        make_key(seed, synth_stream_id(tag, layer, (uint32_t)(b0 + slab / H), (uint32_t)(slab % H)));
    fill_range(key, (uint64_t)c0, (uint64_t)c1, mean, sd, kind, out, slab * per_slab + c0);
  }
}

/* out[k] = lo + (hi - lo) * uniform(key, start + k)  (fp64). */
void synth_uniform(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, double lo,
                   double hi, double* out) {
  const uint64_t key = make_key(seed, stream);
  for (int64_t k = 0; k < count; ++k) out[k] = lo + (hi - lo) * uniform_at(key, start + (uint64_t)k);
}

typedef struct {
  uint64_t w;
  int64_t t;
} keyed_pos;

static int cmp_keyed(const void* a, const void* b) {
  const keyed_pos* x = (const keyed_pos*)a;
  const keyed_pos* y = (const keyed_pos*)b;
  if (x->w != y->w) return x->w < y->w ? -1 : 1;
  return x->t < y->t ? -1 : (x->t > y->t);
}

static int cmp_i32(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* m distinct positions of [0, n): the m smallest word(key, t) (ties by t),
 * returned in ascending position order.  Returns 0, or -1 on bad sizes. */
int synth_choose(uint64_t seed, uint64_t stream, int64_t n, int64_t m, int32_t* out) {
  if (m < 0 || m > n) return -1;
  keyed_pos* tmp = (keyed_pos*)malloc(sizeof(keyed_pos) * (size_t)(n > 0 ? n : 1));
  if (!tmp) return -1;
  const uint64_t key = make_key(seed, stream);
  for (int64_t t = 0; t < n; ++t) {
    tmp[t].w = word_at(key, (uint64_t)t);
    tmp[t].t = t;
  }
  qsort(tmp, (size_t)n, sizeof(keyed_pos), cmp_keyed);
  for (int64_t j = 0; j < m; ++j) out[j] = (int32_t)tmp[j].t;
  qsort(out, (size_t)m, sizeof(int32_t), cmp_i32);
  free(tmp);
  return 0;
}

/* Round fp64 values to the storage kind (RNE). */
void synth_round(const double* in, int64_t n, int kind, void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) store(out, kind, k, in[k]);
}

/*
 * Layer-correlated keys: latent x_0 = z_0, x_l = rho * x_{l-1} + sqrt(1 - rho^2) * z_l
 * (z_l from stream (tag, l, b, h)), each layer stored from its fp64 latent.
 * Fills layer `layer` of a [B, H, per_slab] tensor holding sequences b0 .. b0+B-1.
 */
int synth_fill_ar1(uint64_t seed, uint32_t tag, uint32_t layer, double rho, int64_t b0, int64_t B,
                    int64_t H, int64_t per_slab, int kind, void* out) {
  if (layer >= 64) return -1;
  const int64_t n_slab = B * H;
  const int64_t chunk = 4096;
  const int64_t chunks_per_slab = (per_slab + chunk - 1) / chunk;
  const double innov = sqrt(1.0 - rho * rho);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t w = 0; w < n_slab * chunks_per_slab; ++w) {
    const int64_t slab = w / chunks_per_slab;
    const uint32_t b = (uint32_t)(b0 + slab / H), h = (uint32_t)(slab % H);
    const int64_t c0 = (w % chunks_per_slab) * chunk;
    const int64_t c1 = c0 + chunk < per_slab ? c0 + chunk : per_slab;
    uint64_t keys[64];
    const uint32_t nl = layer + 1;
    for (uint32_t l = 0; l < nl; ++l) keys[l] = make_key(seed, synth_stream_id(tag, l, b, h));
    for (int64_t c = c0; c < c1; ++c) {
      double x = normal_at(keys[0], (uint64_t)c);
      for (uint32_t l = 1; l < nl; ++l) x = rho * x + innov * normal_at(keys[l], (uint64_t)c);
      store(out, kind, slab * per_slab + c, x);
    }
  }
  return 0;
}

/*
 * The same chain with a correlation per layer:
 *   x_0 = z_0,  x_l = rhos[l] * x_{l-1} + sqrt(1 - rhos[l]^2) * z_l  (rhos[0] unused).
 */
int synth_fill_ar1_sched(uint64_t seed, uint32_t tag, uint32_t layer, const double* rhos,
                         int64_t b0, int64_t B, int64_t H, int64_t per_slab, int kind, void* out) {
  if (layer >= 64) return -1;
  const int64_t n_slab = B * H;
  const int64_t chunk = 4096;
  const int64_t chunks_per_slab = (per_slab + chunk - 1) / chunk;
  double innov[64];
  for (uint32_t l = 1; l <= layer; ++l) innov[l] = sqrt(1.0 - rhos[l] * rhos[l]);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t w = 0; w < n_slab * chunks_per_slab; ++w) {
    const int64_t slab = w / chunks_per_slab;
    const uint32_t b = (uint32_t)(b0 + slab / H), h = (uint32_t)(slab % H);
    const int64_t c0 = (w % chunks_per_slab) * chunk;
    const int64_t c1 = c0 + chunk < per_slab ? c0 + chunk : per_slab;
    uint64_t keys[64];
    const uint32_t nl = layer + 1;
    for (uint32_t l = 0; l < nl; ++l) keys[l] = make_key(seed, synth_stream_id(tag, l, b, h));
    for (int64_t c = c0; c < c1; ++c) {
      double x = normal_at(keys[0], (uint64_t)c);
      for (uint32_t l = 1; l < nl; ++l) x = rhos[l] * x + innov[l] * normal_at(keys[l], (uint64_t)c);
      store(out, kind, slab * per_slab + c, x);
    }
  }
  return 0;
}

static inline double bf16_bits_to_f64(uint16_t v) {
  uint32_t u = (uint32_t)v << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/*
 * Random projection of token-major features plus noise:
 *   out[t, m] = bf16( sum_j P[m, j] * X(t, j) + noise_sd * normal(key, t * M + m) )
 * where X(t, j) for j = r * D + i is the stored bf16 value x[r * x_stride_h + t * D + i]
 * (x is a [H, N, D] slab set, head-major), P is [M, H*D] fp64 row-major.
 * Sums run in fp64 in ascending j.
 */
void synth_project_bf16(const uint16_t* x, int64_t H, int64_t N, int64_t D, int64_t x_stride_h,
                        const double* P, int64_t M, double noise_sd, uint64_t seed, uint64_t stream,
                        uint16_t* out) {
  const uint64_t key = make_key(seed, stream);
  const int64_t J = H * D;
  /* P transposed to [J, M] so that the M accumulators of one token update together;
   * each accumulator still sums its own terms in ascending j. */
  double* PT = (double*)malloc(sizeof(double) * (size_t)(J * M));
  if (!PT) return;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t j = 0; j < J; ++j) PT[j * M + m] = P[m * J + j];
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)M);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < N; ++t) {
      for (int64_t m = 0; m < M; ++m) acc[m] = 0.0;
      for (int64_t r = 0; r < H; ++r) {
        const uint16_t* xr = x + r * x_stride_h + t * D;
        for (int64_t i = 0; i < D; ++i) {
          const double f = bf16_bits_to_f64(xr[i]);
          const double* pt = PT + (r * D + i) * M;
          for (int64_t m = 0; m < M; ++m) acc[m] += pt[m] * f;
        }
      }
      for (int64_t m = 0; m < M; ++m) {
        double v = acc[m];
        if (noise_sd != 0.0) v += noise_sd * normal_at(key, (uint64_t)(t * M + m));
        out[t * M + m] = f32_to_bf16_rne((float)v);
      }
    }
    free(acc);
  }
  free(PT);
}

/*
 * Planted rows: for each position t in pos[0..n_pos), row t of a [N, D] slab becomes
 *   out[t * D + i] = scale * base[i] + noise_sd * normal(key, t * D + i)
 * i.e. a direction `base` (fp64) plus the slab's own noise at those counters.
 */
void synth_plant_rows(uint64_t seed, uint64_t stream, const int32_t* pos, int64_t n_pos, int64_t D,
                      const double* base, double scale, double noise_sd, int kind, void* out) {
  const uint64_t key = make_key(seed, stream);
  for (int64_t p = 0; p < n_pos; ++p) {
    const int64_t t = pos[p];
    for (int64_t i = 0; i < D; ++i)
      store(out, kind, t * D + i, scale * base[i] + noise_sd * normal_at(key, (uint64_t)(t * D + i)));
  }
}
