/*
 * Seeded synthetic-input generator for tree speculative-decoding verification
 * workloads.  It draws random numbers only: it holds none of the verification
 * arithmetic (no softmax, no attention, no acceptance rule).
 *
 * Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used as a counter-based
 * generator: the i-th draw of stream `key` is mix(key + (i+1)*GAMMA), which is
 * exactly the i-th output of a SplitMix64 sequence whose state starts at `key`.
 * A stream key is derived from (seed, stream id) with the same mixer, so any
 * element of any tensor can be regenerated independently and in parallel.
 *
 * Normals: Box-Muller (cosine branch) in fp64 from two 53-bit uniforms taken at
 * draw indices 2i and 2i+1, then rounded to fp32 (round-to-nearest-even) and,
 * for bf16 outputs, from fp32 to bf16 (round-to-nearest-even).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC svgen.c -o libsvgen.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t svg_stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* uniform in (0,1] with 53 bits */
static inline double u53_open0(uint64_t v) { return ((double)(v >> 11) + 1.0) * (1.0 / 9007199254740992.0); }
/* uniform in [0,1) with 53 bits */
static inline double u53(uint64_t v) { return (double)(v >> 11) * (1.0 / 9007199254740992.0); }

static inline double normal_at(uint64_t key, uint64_t i) {
  double u1 = u53_open0(draw(key, 2 * i));
  double u2 = u53(draw(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  if ((x & 0x7f800000u) == 0x7f800000u) return (uint16_t)(x >> 16); /* inf/nan: not produced here */
  uint32_t lsb = (x >> 16) & 1u;
  x += 0x7fffu + lsb;
  return (uint16_t)(x >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t x = (uint32_t)h << 16;
  float f;
  memcpy(&f, &x, 4);
  return f;
}

/* raw 64-bit draws */
void svg_u64(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, uint64_t* out) {
  uint64_t key = svg_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, offset + (uint64_t)i);
}

/* 24-bit uniforms k/2^24 in [0,1), exactly representable in fp32 */
void svg_uniform24_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, float* out) {
  uint64_t key = svg_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(draw(key, offset + (uint64_t)i) >> 40) * (1.0f / 16777216.0f);
}

/* mean + sigma * N(0,1), rounded to fp32 */
void svg_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double mean, double sigma, float* out) {
  uint64_t key = svg_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + sigma * normal_at(key, offset + (uint64_t)i));
}

/* mean + sigma * N(0,1), rounded to fp32 then to bf16 (bit pattern in uint16) */
void svg_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double mean, double sigma, uint16_t* out) {
  uint64_t key = svg_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne((float)(mean + sigma * normal_at(key, offset + (uint64_t)i)));
}

/* out = bf16(float(base) + sigma * N(0,1)): a perturbed copy of a bf16 tensor */
void svg_perturb_bf16(uint64_t seed, uint64_t stream, int64_t n, const uint16_t* base, double sigma, uint16_t* out) {
  uint64_t key = svg_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne((float)((double)bf16_to_f32(base[i]) + sigma * normal_at(key, (uint64_t)i)));
}

/* out = float(base) + sigma * N(0,1) rounded to fp32 */
void svg_perturb_f32(uint64_t seed, uint64_t stream, int64_t n, const float* base, double sigma, float* out) {
  uint64_t key = svg_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)((double)base[i] + sigma * normal_at(key, (uint64_t)i));
}

/*
 * Draft sampling for the input recipe (the drafter's side, not verification):
 * for each requested row, draw one token from softmax(logits[row]/T) with the
 * Gumbel-max construction, token = argmax_v (logits[row][v]/T + G_v) with
 * G_v = -log(-log(U_v)) and U_v a 53-bit uniform in (0,1).  The noise for
 * (request j, vocabulary entry v) is draw index j*V + v of the stream.
 * For T <= 0 the noise is skipped and the plain argmax (lowest id on ties) is
 * returned, which is greedy drafting.
 * dtype: 0 = fp32 rows, 1 = bf16 rows.
 */
void svg_draft_tokens(uint64_t seed, uint64_t stream, const void* logits, int dtype, int64_t V,
                      const int64_t* row_index, int64_t n_req, double T, int32_t* out) {
  uint64_t key = svg_stream_key(seed, stream);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < n_req; ++j) {
    int64_t row = row_index[j];
    double best = -INFINITY;
    int32_t arg = 0;
    for (int64_t v = 0; v < V; ++v) {
      double l = dtype == 0 ? (double)((const float*)logits)[row * V + v]
                            : (double)bf16_to_f32(((const uint16_t*)logits)[row * V + v]);
      double s;
      if (T > 0.0) {
        double u = ((double)(draw(key, (uint64_t)(j * V + v)) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
        s = l / T - log(-log(u));
      } else {
        s = l;
      }
      if (s > best) { best = s; arg = (int32_t)v; }
    }
    out[j] = arg;
  }
}
