/*
 * Seeded synthetic inputs for the GSA layer (test and benchmark infrastructure).
 *
 * This module produces the Q/K/V/W_g tensors that both the CPU oracle and the
 * HIP library consume.  It holds none of the attention arithmetic: it only
 * draws numbers and writes them in the token layout [N][T_f][H][d]
 * (T_f = P special tokens followed by the h*w image tokens of a frame,
 * row-major over the image grid).
 *
 * Generator: counter based, so every element depends only on
 * (seed, stream, flat index) and the output is identical for any thread count.
 *   key      = mix64(mix64(seed) + stream)
 *   a_i, b_i = mix64(key + (2i+1)*G), mix64(key + (2i+2)*G)
 * where mix64 is the SplitMix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) and
 * G = 0x9E3779B97F4A7C15 its golden-ratio increment.  A standard normal is
 * obtained from (a_i, b_i) with the Box-Muller transform
 *   z = sqrt(-2 ln u1) * cos(2 pi u2),  u1 in (0,1], u2 in [0,1),
 * evaluated in double, scaled, cast to float and, for bf16 output, rounded
 * to nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GEN_BF16 0
#define GEN_F32 1

static const uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) + stream);
}

/* Standard normal for counter i of the stream with key `key`. */
static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t a = mix64(key + (2 * i + 1) * GOLDEN);
  uint64_t b = mix64(key + (2 * i + 2) * GOLDEN);
  double u1 = ((double)(a >> 11) + 1.0) * (1.0 / 9007199254740992.0); /* (0,1] */
  double u2 = (double)(b >> 11) * (1.0 / 9007199254740992.0);         /* [0,1) */
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* Uniform integer in [0, n) for counter i. */
static inline uint32_t uniform_int_at(uint64_t key, uint64_t i, uint32_t n) {
  uint64_t a = mix64(key + (i + 1) * GOLDEN);
  return (uint32_t)(((a >> 32) * (uint64_t)n) >> 32);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0; /* NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline void store(void* dst, int dtype, int64_t i, double v) {
  float f = (float)v;
  if (dtype == GEN_F32)
    ((float*)dst)[i] = f;
  else
    ((uint16_t*)dst)[i] = f32_to_bf16_rne(f);
}

/* dst[i] = std * N(0,1)_(offset+i) for i in [0, n). */
void gen_normal(void* dst, int64_t n, int dtype, uint64_t seed, uint64_t stream, double std,
                int64_t offset) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) store(dst, dtype, i, std * normal_at(key, (uint64_t)(offset + i)));
}

/*
 * Clustered ("peaky") tokens.  For each s x s window of the image grid and
 * each head, one cluster id c is drawn uniformly from [0, n_clusters) with
 * the map stream; every image token of that window and head is
 *   centroid[c][h][:] + noise_std * N(0,1)
 * with the centroid table [n_clusters][H][d] ~ N(0,1) drawn from the
 * centroid stream.  Special tokens are N(0,1) from the noise stream.
 * Layout of dst: [N][T_f][H][d].
 */
void gen_clustered(void* dst, int dtype, int n_frames, int n_special, int grid_h, int grid_w,
                   int n_heads, int head_dim, int pool, uint64_t seed, uint64_t stream_noise,
                   uint64_t stream_centroid, uint64_t stream_map, int n_clusters,
                   double noise_std) {
  const int64_t tf = (int64_t)n_special + (int64_t)grid_h * grid_w;
  const int64_t row = (int64_t)n_heads * head_dim;
  const int64_t wins_x = grid_w / pool, wins_per_frame = (int64_t)(grid_h / pool) * wins_x;
  const uint64_t kn = stream_key(seed, stream_noise);
  const uint64_t kc = stream_key(seed, stream_centroid);
  const uint64_t km = stream_key(seed, stream_map);
  const int64_t ntok = (int64_t)n_frames * tf;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < ntok; ++t) {
    int64_t f = t / tf, p = t % tf;
    for (int hh = 0; hh < n_heads; ++hh) {
      for (int c = 0; c < head_dim; ++c) {
        int64_t i = t * row + (int64_t)hh * head_dim + c;
        double noise = normal_at(kn, (uint64_t)i);
        double v;
        if (p < n_special) {
          v = noise;
        } else {
          int64_t y = (p - n_special) / grid_w, x = (p - n_special) % grid_w;
          int64_t win = f * wins_per_frame + (y / pool) * wins_x + (x / pool);
          uint32_t cl = uniform_int_at(km, (uint64_t)(win * n_heads + hh), (uint32_t)n_clusters);
          double cen = normal_at(kc, (uint64_t)(((int64_t)cl * n_heads + hh) * head_dim + c));
          v = cen + noise_std * noise;
        }
        store(dst, dtype, i, v);
      }
    }
  }
}

/* Expose the raw stream for tests of the generator itself. */
uint64_t gen_mix64(uint64_t z) { return mix64(z); }
double gen_normal_at(uint64_t seed, uint64_t stream, uint64_t i) {
  return normal_at(stream_key(seed, stream), i);
}
