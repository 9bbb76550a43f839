/*
 * msagen.c -- seeded synthetic inputs for MSA decode, written straight into
 * the paged device layout documented in include/msa.h.
 *
 * This file is input preparation only: random draws and the quantisers that
 * turn fp32 draws into stored codes (NVFP4, FP8 E4M3, bf16). It holds none of
 * the decode path's arithmetic (no decoding, scoring, pooling, selection or
 * attention). Both the HIP path and the CPU oracle read the bytes it writes.
 *
 * Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) evaluated at a counter, so any
 * element is a pure function of (seed, tensor tag, logical index) and the
 * output does not depend on the thread count or on the page permutation.
 * Normals: Box-Muller (1958) from two such uniforms; the cache generators use
 * both outputs (r cos, r sin) of each pair.
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
/* Output number `ctr` of the SplitMix64 sequence started at `key`. */
static inline uint64_t rng_at(uint64_t key, uint64_t ctr) { return mix64(key + (ctr + 1) * GAMMA); }
/* Uniform in (0, 1) with 53 random bits. */
static inline double unif_at(uint64_t key, uint64_t ctr) {
  return ((double)(rng_at(key, ctr) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
static inline double normal_at(uint64_t key, uint64_t ctr) {
  double u1 = unif_at(key, 2 * ctr), u2 = unif_at(key, 2 * ctr + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}
/* Both Box-Muller outputs of pair `ctr`: out[0] = r cos, out[1] = r sin. */
static inline void normal_pair_at(uint64_t key, uint64_t ctr, double* out) {
  double u1 = unif_at(key, 2 * ctr), u2 = unif_at(key, 2 * ctr + 1);
  double r = sqrt(-2.0 * log(u1)), th = 6.283185307179586476925 * u2;
  out[0] = r * cos(th);
  out[1] = r * sin(th);
}

uint64_t msagen_stream_key(uint64_t seed, uint64_t tag) {
  return mix64(mix64(seed + GAMMA) ^ (tag * 0xD1B54A32D192ED03ULL));
}

/* ---------------------------------------------------------------- encoders */

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static inline uint16_t bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* |x| -> OCP E4M3 (e4m3fn) magnitude code, round to nearest even, saturating
 * at 448 (code 0x7E). */
static inline uint8_t e4m3_mag_rne(double a) {
  if (!(a > 0.0)) return 0;
  if (a >= 448.0) return 0x7E;
  if (a < 0.015625) { /* below the smallest normal 2^-6: subnormal step 2^-9 */
    double m = nearbyint(a * 512.0);
    return (uint8_t)m; /* m == 8 gives 0x08 = 2^-6, the smallest normal */
  }
  int e;
  double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  double mant = f * 2.0 - 1.0; /* a = (1 + mant) * 2^(e-1) */
  int E = e - 1;
  double m = nearbyint(mant * 8.0);
  if (m >= 8.0) { m = 0.0; E += 1; }
  int biased = E + 7;
  if (biased > 15 || (biased == 15 && m > 6.0)) return 0x7E;
  return (uint8_t)((biased << 3) | (int)m);
}
static inline uint8_t e4m3_rne(double x) {
  uint8_t c = e4m3_mag_rne(fabs(x));
  return (uint8_t)(x < 0.0 ? (c | 0x80) : c);
}
/* Value of an E4M3 code -- encoder-side copy used only to form x / scale. */
static inline double e4m3_val_enc(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return (c & 0x80) ? -v : v;
}
/* |x| -> E2M1 magnitude code (0..7 for 0,.5,1,1.5,2,3,4,6), nearest, ties to
 * the even code, saturating at 6. */
static inline uint8_t e2m1_mag_rne(double a) {
  if (a <= 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2;
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;
  return 7;
}
static inline uint8_t e2m1_rne(double x) {
  uint8_t c = e2m1_mag_rne(fabs(x));
  return (uint8_t)((x < 0.0 && c != 0) ? (c | 8) : c);
}

/* Exported scalar encoders (for round-trip tests of the generator). */
uint16_t msagen_bf16_rne(float x) { return bf16_rne(x); }
uint8_t msagen_e4m3_rne(double x) { return e4m3_rne(x); }
uint8_t msagen_e2m1_rne(double x) { return e2m1_rne(x); }

/* ------------------------------------------------------------ dense tensors */

/* out[i] = bf16(sigma * N(key, start + i)). */
void msagen_normal_bf16(uint64_t key, int64_t start, int64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = bf16_rne((float)(sigma * normal_at(key, (uint64_t)(start + i))));
}
/* out[i] = (float)U(key, start + i), uniform in (0,1). */
void msagen_uniform_f32(uint64_t key, int64_t start, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = (float)unif_at(key, (uint64_t)(start + i));
}
/* out[i] = (float)(sigma * N(key, start + i)). */
void msagen_normal_f32(uint64_t key, int64_t start, int64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = (float)(sigma * normal_at(key, (uint64_t)(start + i)));
}

/* ------------------------------------------------------------ paged caches */

/* Logical element counter of token `tok` of sequence `b`, channel `ch` of
 * `nch` channels: independent of the page the token is stored in. */
static inline uint64_t tok_ctr(int64_t b, int64_t tok, int64_t nch, int64_t ch) {
  return ((((uint64_t)b << 32) | (uint64_t)tok) * (uint64_t)nch) + (uint64_t)ch;
}

/*
 * K and V caches. For every sequence b and token tok < ctx_lens[b]:
 *   K[b,tok,g,d] = N(key_k, ...) * kmul[g*128 + d],  V likewise with key_v, vmul
 * (kmul/vmul hold 1.0 except for outlier channels), quantised per 16-element
 * group of one token: scale = E4M3_RNE(amax / 6), code = E2M1_RNE(x / scale)
 * (scale 0 -> all codes +0). Written to page block_table[b][tok / 128] at slot
 * tok % 128 in the NVFP4 layout of msa.h (K token-major, V dim-major), or as
 * bf16 when nvfp4 == 0 (k_scale / v_scale unused). Pages a sequence does not
 * use are left untouched.
 */
void msagen_kv_cache(uint64_t key_k, uint64_t key_v, int32_t nseq, const int32_t* ctx_lens,
                     const int32_t* block_table, int32_t max_blocks, int32_t n_kv_heads,
                     const float* kmul, const float* vmul, int32_t nvfp4, void* k_data,
                     uint8_t* k_scale, void* v_data, uint8_t* v_scale) {
  int64_t total = 0;
  for (int32_t b = 0; b < nseq; b++) total += (ctx_lens[b] + 127) / 128;
  /* flatten (b, blk) pairs */
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t flat = 0; flat < total; flat++) {
    int64_t rem = flat;
    int32_t b = 0;
    while (rem >= (ctx_lens[b] + 127) / 128) { rem -= (ctx_lens[b] + 127) / 128; b++; }
    int32_t blk = (int32_t)rem;
    int64_t page = block_table[(int64_t)b * max_blocks + blk];
    int32_t ntok = ctx_lens[b] - blk * 128;
    if (ntok > 128) ntok = 128;
    const int G = n_kv_heads;
    for (int g = 0; g < G; g++) {
      for (int slot = 0; slot < ntok; slot++) {
        int64_t tok = (int64_t)blk * 128 + slot;
        for (int which = 0; which < 2; which++) {
          uint64_t key = which == 0 ? key_k : key_v;
          const float* mul = which == 0 ? kmul : vmul;
          double x[128];
          for (int d = 0; d < 128; d += 2) {
            normal_pair_at(key, tok_ctr(b, tok, (int64_t)G * 64, (int64_t)g * 64 + d / 2), x + d);
            x[d] *= mul[g * 128 + d];
            x[d + 1] *= mul[g * 128 + d + 1];
          }
          if (!nvfp4) {
            uint16_t* base = (uint16_t*)(which == 0 ? k_data : v_data) + (page * G + g) * 128 * 128;
            for (int d = 0; d < 128; d++) {
              uint16_t h = bf16_rne((float)x[d]);
              if (which == 0) base[slot * 128 + d] = h; else base[d * 128 + slot] = h;
            }
            continue;
          }
          uint8_t* data = (uint8_t*)(which == 0 ? k_data : v_data) + (page * G + g) * 128 * 64;
          uint8_t* sc = (which == 0 ? k_scale : v_scale) + (page * G + g) * 128 * 8;
          for (int c = 0; c < 8; c++) {
            double amax = 0.0;
            for (int i = 0; i < 16; i++) amax = fmax(amax, fabs(x[16 * c + i]));
            uint8_t scode = e4m3_rne(amax / 6.0);
            double s = e4m3_val_enc(scode);
            if (which == 0) sc[slot * 8 + c] = scode; else sc[c * 128 + slot] = scode;
            for (int i = 0; i < 16; i++) {
              int d = 16 * c + i;
              uint8_t code = s > 0.0 ? e2m1_rne(x[d] / s) : 0;
              if (which == 0) {
                uint8_t* byte = data + slot * 64 + d / 2;
                if (d & 1) *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
                else *byte = (uint8_t)((*byte & 0xF0) | code);
              } else {
                uint8_t* byte = data + d * 64 + slot / 2;
                if (slot & 1) *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
                else *byte = (uint8_t)((*byte & 0xF0) | code);
              }
            }
          }
        }
      }
    }
  }
}

/*
 * Indexer keys. For every sequence b and token tok < ctx_lens[b]:
 *   k[d] = sigma * N(key, ...) + (plant[b*max_blocks + tok/128] ? shift[b*64 + d] : 0)
 * fmt 1 (FP8): per-token scale s = amax / 448 (fp32; 1.0 when amax == 0),
 * code = E4M3_RNE(k / s) saturating; written idx_k[page][slot][64] and
 * (float) idx_scale[page][slot]. fmt 2 (NVFP4): per 16-dim group scale
 * E4M3_RNE(amax / 6) and codes E2M1_RNE(k / scale) as for K; written
 * idx_k[page][slot][32] (dim 2i in the low nibble) and (u8)
 * idx_scale[page][slot][4]. fmt 0 (BF16): idx_k holds bf16 codes.
 */
void msagen_idx_cache(uint64_t key, int32_t nseq, const int32_t* ctx_lens, const int32_t* block_table,
                      int32_t max_blocks, double sigma, const uint8_t* plant, const float* shift,
                      int32_t fmt, void* idx_k, void* idx_scale) {
  int64_t total = 0;
  for (int32_t b = 0; b < nseq; b++) total += (ctx_lens[b] + 127) / 128;
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t flat = 0; flat < total; flat++) {
    int64_t rem = flat;
    int32_t b = 0;
    while (rem >= (ctx_lens[b] + 127) / 128) { rem -= (ctx_lens[b] + 127) / 128; b++; }
    int32_t blk = (int32_t)rem;
    int64_t page = block_table[(int64_t)b * max_blocks + blk];
    int planted = plant ? plant[(int64_t)b * max_blocks + blk] : 0;
    int32_t ntok = ctx_lens[b] - blk * 128;
    if (ntok > 128) ntok = 128;
    for (int slot = 0; slot < ntok; slot++) {
      int64_t tok = (int64_t)blk * 128 + slot;
      float x[64];
      float amax = 0.0f;
      double nrm[64];
      for (int d = 0; d < 64; d += 2) normal_pair_at(key, tok_ctr(b, tok, 32, d / 2), nrm + d);
      for (int d = 0; d < 64; d++) {
        double v = sigma * nrm[d];
        if (planted) v += shift[(int64_t)b * 64 + d];
        x[d] = (float)v;
        amax = fmaxf(amax, fabsf(x[d]));
      }
      if (fmt == 1) {
        float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        uint8_t* row = (uint8_t*)idx_k + (page * 128 + slot) * 64;
        for (int d = 0; d < 64; d++) row[d] = e4m3_rne((double)x[d] / (double)s);
        ((float*)idx_scale)[page * 128 + slot] = s;
      } else if (fmt == 2) {
        uint8_t* row = (uint8_t*)idx_k + (page * 128 + slot) * 32;
        uint8_t* sc = (uint8_t*)idx_scale + (page * 128 + slot) * 4;
        for (int c = 0; c < 4; c++) {
          double gmax = 0.0;
          for (int i = 0; i < 16; i++) gmax = fmax(gmax, fabs((double)x[16 * c + i]));
          uint8_t scode = e4m3_rne(gmax / 6.0);
          double sv = e4m3_val_enc(scode);
          sc[c] = scode;
          for (int i = 0; i < 16; i += 2) {
            uint8_t lo = sv > 0.0 ? e2m1_rne((double)x[16 * c + i] / sv) : 0;
            uint8_t hi = sv > 0.0 ? e2m1_rne((double)x[16 * c + i + 1] / sv) : 0;
            row[(16 * c + i) / 2] = (uint8_t)(lo | (hi << 4));
          }
        }
      } else {
        uint16_t* row = (uint16_t*)idx_k + (page * 128 + slot) * 64;
        for (int d = 0; d < 64; d++) row[d] = bf16_rne(x[d]);
      }
    }
  }
}
