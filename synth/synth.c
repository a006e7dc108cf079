/*
 * Seeded synthetic inputs for the Phi-3-style prefill and the K16/V8 decode
 * attention workloads.
 *
 * This file produces input BYTES only: random normal weights and activations,
 * uniform token ids, random page permutations, and the storage encodings the
 * inputs are handed over in (IEEE binary16, per-row int8 + binary16 scale,
 * OCP E4M3FN bytes).  It holds none of the forward arithmetic.  Both the CPU
 * oracle and the GPU path consume exactly the bytes written here.
 *
 * Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The stream of a tensor is
 * keyed by key = mix(seed ^ fnv1a64(name)); element i takes output i of the
 * SplitMix64 sequence started at that key, i.e. mix(key + (i + 1) * gamma).
 * Generation is therefore counter based: any slice can be produced on its own
 * and in parallel, and the result does not depend on the thread count.
 * Normals: Box-Muller on pairs (2j, 2j+1) in double precision.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_fnv1a64(const char* s) {
  uint64_t h = 0xcbf29ce484222325ULL;
  for (; *s; ++s) {
    h ^= (uint8_t)*s;
    h *= 0x100000001b3ULL;
  }
  return h;
}

uint64_t synth_key(uint64_t seed, const char* name) { return mix64(seed ^ synth_fnv1a64(name)); }

static inline uint64_t bits_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* ---- IEEE 754 binary16, round to nearest even, from double ---------------- */
uint16_t synth_f64_to_f16(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  uint64_t a = b & 0x7FFFFFFFFFFFFFFFULL;
  if (a >= 0x7FF0000000000000ULL) /* inf / nan */
    return sign | 0x7C00u | (a > 0x7FF0000000000000ULL ? 0x200u : 0u);
  if (a == 0) return sign;
  int e = (int)(a >> 52) - 1023;
  uint64_t mant = (a & 0xFFFFFFFFFFFFFULL) | (e == -1023 ? 0 : (1ULL << 52));
  if (e == -1023) return sign; /* double subnormal: far below binary16's range */
  if (e > 15) return sign | 0x7C00u;
  int shift;
  if (e >= -14) shift = 42;           /* normal: keep 11 significant bits */
  else if (e >= -26) shift = 28 - e;  /* subnormal: unit 2^-24 */
  else return sign;                   /* below half the smallest subnormal */
  uint64_t q = mant >> shift;
  uint64_t rem = mant & ((1ULL << shift) - 1);
  uint64_t half = 1ULL << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  if (e >= -14) {
    int ee = e + 15;
    if (q == 2048) { q = 1024; ee++; }
    if (ee >= 31) return sign | 0x7C00u;
    return sign | (uint16_t)(ee << 10) | (uint16_t)(q & 0x3FF);
  }
  return sign | (uint16_t)q; /* q == 1024 is the smallest normal, encoded the same way */
}

double synth_f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* ---- OCP 8-bit floating point, E4M3FN (bias 7, max 448, no inf) ----------
 * Round to nearest even, saturating to +-448.  S.1111.111 (NaN) is never
 * produced for finite input. */
uint8_t synth_f64_to_e4m3(double x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int E;
  (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) */
  int ue = E - 1;     /* a in [2^ue, 2^(ue+1)) */
  if (ue < -6) {      /* subnormal: unit 2^-9 */
    double q = nearbyint(ldexp(a, 9));
    return sign | (uint8_t)q; /* q == 8 is the smallest normal, encoded the same way */
  }
  double q = nearbyint(ldexp(a, 3 - ue)); /* in [8, 16] */
  if (q == 16.0) { q = 8.0; ue++; }
  int code = ((ue + 7) << 3) | ((int)q - 8);
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

/* ---- threaded fill ------------------------------------------------------- */
enum { OUT_F64 = 0, OUT_F32 = 1, OUT_F16 = 2 };

typedef struct {
  uint64_t key;
  double std;
  int64_t begin, end;
  int kind;
  void* out;
} normal_job;

static inline void store_at(int kind, void* out, int64_t i, double v) {
  if (kind == OUT_F64) ((double*)out)[i] = v;
  else if (kind == OUT_F32) ((float*)out)[i] = (float)v;
  else ((uint16_t*)out)[i] = synth_f64_to_f16(v);
}

/* Fills [begin, end); begin is even, so each Box-Muller pair is drawn once. */
static void* normal_worker(void* p) {
  normal_job* j = (normal_job*)p;
  for (int64_t i = j->begin; i < j->end; i += 2) {
    uint64_t jj = (uint64_t)i >> 1;
    double u1 = (double)((bits_at(j->key, 2 * jj) >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(bits_at(j->key, 2 * jj + 1) >> 11) * 0x1.0p-53;
    double r = j->std * sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    store_at(j->kind, j->out, i, r * cos(t));
    if (i + 1 < j->end) store_at(j->kind, j->out, i + 1, r * sin(t));
  }
  return NULL;
}

#define MAX_THREADS 64

static void run_normal(uint64_t key, double std, int64_t n, int kind, void* out, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > MAX_THREADS) nthreads = MAX_THREADS;
  if (n < 65536) nthreads = 1;
  normal_job jobs[MAX_THREADS];
  pthread_t th[MAX_THREADS];
  int64_t chunk = (n + nthreads - 1) / nthreads;
  chunk += chunk & 1;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = t * chunk, e = b + chunk < n ? b + chunk : n;
    if (b >= e) break;
    jobs[t] = (normal_job){key, std, b, e, kind, out};
    if (nthreads == 1) { normal_worker(&jobs[t]); continue; }
    pthread_create(&th[t], NULL, normal_worker, &jobs[t]);
    started++;
  }
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}

/* out[i] = std * (element i of the unit-normal stream named `name`), i in [0, n). */
void synth_normal_f64(uint64_t seed, const char* name, double std, int64_t n, double* out, int nthreads) {
  run_normal(synth_key(seed, name), std, n, OUT_F64, out, nthreads);
}
void synth_normal_f32(uint64_t seed, const char* name, double std, int64_t n, float* out, int nthreads) {
  run_normal(synth_key(seed, name), std, n, OUT_F32, out, nthreads);
}
void synth_normal_f16(uint64_t seed, const char* name, double std, int64_t n, uint16_t* out, int nthreads) {
  run_normal(synth_key(seed, name), std, n, OUT_F16, out, nthreads);
}

/* Uniform integers in [0, range): (bits * range) >> 64 (Lemire's multiply-shift map). */
void synth_uniform_i32(uint64_t seed, const char* name, int64_t n, int32_t range, int32_t* out) {
  uint64_t key = synth_key(seed, name);
  for (int64_t i = 0; i < n; ++i) {
    unsigned __int128 p = (unsigned __int128)bits_at(key, (uint64_t)i) * (uint64_t)range;
    out[i] = (int32_t)(uint64_t)(p >> 64);
  }
}

/* Uniform random permutation of 0..n-1 (Fisher-Yates, draws from the named stream). */
void synth_permutation(uint64_t seed, const char* name, int32_t n, int32_t* out) {
  uint64_t key = synth_key(seed, name);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    unsigned __int128 p = (unsigned __int128)bits_at(key, (uint64_t)i) * (uint64_t)(i + 1);
    int32_t j = (int32_t)(uint64_t)(p >> 64);
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

void synth_encode_f16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = synth_f64_to_f16(x[i]);
}

void synth_decode_f16(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = synth_f16_to_f64(h[i]);
}

/* x[i] / scale, encoded as E4M3FN (RNE, saturating). */
void synth_encode_e4m3(const double* x, int64_t n, double scale, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = synth_f64_to_e4m3(x[i] / scale);
}

/* Symmetric per-row int8 of binary16 weights w[rows][cols]:
 * s_r = f16(max_k |w[r][k]| / 127), q = clamp(rne(w / s_r), -127, 127);
 * an all-zero row takes s_r = 1 and q = 0. */
typedef struct {
  const uint16_t* w;
  int64_t cols, r0, r1;
  int8_t* q;
  uint16_t* s;
} quant_job;

static void* quant_worker(void* p) {
  quant_job* j = (quant_job*)p;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    const uint16_t* row = j->w + r * j->cols;
    double amax = 0.0;
    for (int64_t k = 0; k < j->cols; ++k) {
      double v = fabs(synth_f16_to_f64(row[k]));
      if (v > amax) amax = v;
    }
    uint16_t sh = amax > 0.0 ? synth_f64_to_f16(amax / 127.0) : (uint16_t)0x3C00;
    double s = synth_f16_to_f64(sh);
    j->s[r] = sh;
    for (int64_t k = 0; k < j->cols; ++k) {
      double v = amax > 0.0 ? nearbyint(synth_f16_to_f64(row[k]) / s) : 0.0;
      if (v > 127.0) v = 127.0;
      if (v < -127.0) v = -127.0;
      j->q[r * j->cols + k] = (int8_t)v;
    }
  }
  return NULL;
}

void synth_quantize_rows_i8(const uint16_t* w, int64_t rows, int64_t cols, int8_t* q, uint16_t* s,
                            int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > MAX_THREADS) nthreads = MAX_THREADS;
  if (rows < 256) nthreads = 1;
  quant_job jobs[MAX_THREADS];
  pthread_t th[MAX_THREADS];
  int64_t chunk = (rows + nthreads - 1) / nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = t * chunk, e = b + chunk < rows ? b + chunk : rows;
    if (b >= e) break;
    jobs[t] = (quant_job){w, cols, b, e, q, s};
    if (nthreads == 1) { quant_worker(&jobs[t]); continue; }
    pthread_create(&th[t], NULL, quant_worker, &jobs[t]);
    started++;
  }
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}
