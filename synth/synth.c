/*
 * Seeded synthetic inputs for the quantized attention forward.
 *
 * This module only makes test and benchmark inputs. It holds none of the
 * method's arithmetic and is the one piece of code shared by the CPU oracle
 * side and the GPU side: both consume the BF16 bit patterns it writes.
 *
 * Generator (counter based, so any element can be produced on its own):
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): output n of the stream with seed s is
 *     mix64(s + (n + 1) * 0x9E3779B97F4A7C15) with the published finaliser.
 *   - uniform in (0,1): ((x >> 11) + 0.5) * 2^-53, never 0 or 1.
 *   - standard normal by the Box-Muller transform in double precision: the
 *     pair (2p, 2p+1) of uniforms gives normals p*2 (cosine) and p*2+1 (sine).
 *   - each value is transformed in double, rounded to float, then to BF16
 *     with round-to-nearest-even.
 *
 * Tensors are [B,S,H,D] with D fastest; element (b,s,h,d) has linear index
 * ((b*S + s)*H + h)*D + d, and that index is the normal's counter.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_splitmix64(uint64_t seed, uint64_t n) { return mix64(seed + (n + 1) * SYNTH_GAMMA); }

double synth_uniform(uint64_t seed, uint64_t n) {
  return ((double)(synth_splitmix64(seed, n) >> 11) + 0.5) * 0x1.0p-53;
}

double synth_normal(uint64_t seed, uint64_t n) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t p = n >> 1;
  double u1 = synth_uniform(seed, 2 * p), u2 = synth_uniform(seed, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  return (n & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
}

static uint16_t to_bf16(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Kinds of tensor (the transform applied to the normal z at element (b,s,h,d)). */
enum {
  SYNTH_NORMAL = 0,       /* z */
  SYNTH_HEAD_SCALE = 1,   /* z * a[h],  a[h] = lo + (hi - lo) * U(aux_seed, h)          */
  SYNTH_CHANNEL_BIAS = 2, /* z + sigma * N(aux_seed, h*D + d)  (shared over b and s)    */
  SYNTH_OUTLIERS = 3      /* z, replaced with probability p by sigma * N(aux_seed, idx) */
};

typedef struct {
  int32_t kind;
  uint64_t seed;     /* stream of the base normal */
  uint64_t aux_seed; /* stream of the per-head scale, bias or outlier values */
  uint64_t mask_seed;/* stream deciding which entries are outliers */
  double p0, p1;     /* HEAD_SCALE: lo, hi.  CHANNEL_BIAS: sigma.  OUTLIERS: probability, sigma */
} synth_spec;

/* Per-element transform; tab holds the per-head scales (HEAD_SCALE) or the
 * per-(h,d) biases (CHANNEL_BIAS), precomputed from their own stream. */
static double transform(const synth_spec* sp, const double* tab, int64_t idx, int64_t h, int64_t d, int64_t D,
                        double z) {
  switch (sp->kind) {
    case SYNTH_HEAD_SCALE: return z * tab[h];
    case SYNTH_CHANNEL_BIAS: return z + tab[h * D + d];
    case SYNTH_OUTLIERS:
      if (synth_uniform(sp->mask_seed, (uint64_t)idx) < sp->p0) return sp->p1 * synth_normal(sp->aux_seed, (uint64_t)idx);
      return z;
    default: return z;
  }
}

static double* make_table(const synth_spec* sp, int64_t H, int64_t D) {
  double* tab = NULL;
  if (sp->kind == SYNTH_HEAD_SCALE) {
    tab = (double*)malloc((size_t)H * sizeof(double));
    for (int64_t h = 0; h < H; ++h) tab[h] = sp->p0 + (sp->p1 - sp->p0) * synth_uniform(sp->aux_seed, (uint64_t)h);
  } else if (sp->kind == SYNTH_CHANNEL_BIAS) {
    tab = (double*)malloc((size_t)(H * D) * sizeof(double));
    for (int64_t i = 0; i < H * D; ++i) tab[i] = sp->p0 * synth_normal(sp->aux_seed, (uint64_t)i);
  }
  return tab;
}

/* Both normals of Box-Muller pair p. */
static void normal_pair(uint64_t seed, uint64_t p, double* z0, double* z1) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = synth_uniform(seed, 2 * p), u2 = synth_uniform(seed, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1)), sn, cs;
  sincos(two_pi * u2, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

/* Fill linear elements [start, end) of a [B,S,H,D] tensor (out points at element 0). */
void synth_fill(const synth_spec* sp, int64_t S, int64_t H, int64_t D, int64_t start, int64_t end, uint16_t* out) {
  (void)S;
  if (start >= end) return;
  double* tab = make_table(sp, H, D);
  int64_t d = start % D, h = (start / D) % H; /* coordinates of element i, advanced incrementally */
  double z[2];
  normal_pair(sp->seed, (uint64_t)(start >> 1), &z[0], &z[1]);
  for (int64_t i = start; i < end; ++i) {
    if (!(i & 1) && i != start) normal_pair(sp->seed, (uint64_t)(i >> 1), &z[0], &z[1]);
    out[i] = sp->kind == SYNTH_NORMAL ? to_bf16(z[i & 1]) : to_bf16(transform(sp, tab, i, h, d, D, z[i & 1]));
    if (++d == D) { d = 0; if (++h == H) h = 0; }
  }
  free(tab);
}

/* Fill rows [s0, s1) of head (b,h) as a dense [s1-s0][D] block. */
void synth_fill_head(const synth_spec* sp, int64_t S, int64_t H, int64_t D, int64_t b, int64_t h,
                     int64_t s0, int64_t s1, uint16_t* out) {
  double* tab = make_table(sp, H, D);
  for (int64_t s = s0; s < s1; ++s)
    for (int64_t d = 0; d < D; ++d) {
      int64_t idx = ((b * S + s) * H + h) * D + d;
      out[(s - s0) * D + d] = to_bf16(transform(sp, tab, idx, h, d, D, synth_normal(sp->seed, (uint64_t)idx)));
    }
  free(tab);
}
