/* Seeded synthetic input generator shared by the tests, the bench and the
 * oracle's callers.  It produces the bytes of the host expert pool, the
 * hidden activations and the router weights.  It holds none of the MoE
 * layer's arithmetic: it only draws numbers and stores them in the formats
 * the pool is laid out in.
 *
 * Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: word i of stream `key` is the SplitMix64 finaliser applied to
 * key + (i+1)*0x9E3779B97F4A7C15.  Each 64-bit word gives four 16-bit
 * uniforms; a uniform u indexes a caller-supplied table of 65536 quantiles
 * of N(0,1) (inverse-transform sampling at 2^-16 resolution).
 *
 * Storage formats written here (the layout of one expert blob, gate, up and
 * down as row-major [out,in] matrices followed by their scale arrays):
 *   bf16 : round-to-nearest-even of the fp32 sample.
 *   fp8  : OCP E4M3FN code of w/s, s = fp32 amax/448 per 128x128 block.
 *   mxfp4: OCP E2M1 code of w*2^-x per 32 consecutive inputs, x =
 *          floor(log2 amax) - 2 stored as E8M0 (x+127); two codes per byte,
 *          the even element in the low nibble.
 *   nvfp4: E2M1 code of w/(s_b*t) per 16 consecutive inputs, s_b = E4M3 of
 *          amax_b/(6t), t = fp32 amax_matrix/(6*448) per matrix; codes as
 *          mxfp4, then the E4M3 block scales, then the three t.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_word(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

uint64_t synth_key(uint64_t a, uint64_t b) { return mix64(mix64(a + GOLDEN) ^ (b * 0xD1B54A32D192ED03ULL + 1)); }

static inline uint16_t uniform16(uint64_t key, uint64_t i) {
  uint64_t w = synth_word(key, i >> 2);
  return (uint16_t)(w >> (16 * (i & 3)));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP E4M3FN encoder, round-to-nearest-even, saturating at +-448. */
static uint8_t enc_e4m3(float v) {
  uint8_t s = (v < 0.0f || (v == 0.0f && signbit(v))) ? 0x80 : 0;
  double a = fabs((double)v);
  if (a >= 448.0) return s | 0x7E;
  if (a < ldexp(1.0, -6)) {            /* subnormal range: step 2^-9 */
    double q = a / ldexp(1.0, -9);
    double r = nearbyint(q);           /* default rounding mode is RNE */
    return s | (uint8_t)r;             /* r == 8 lands on the min normal code */
  }
  int e;
  double m = frexp(a, &e);             /* a = m*2^e, m in [0.5,1) */
  int E = e - 1;                       /* a = (2m)*2^E, 2m in [1,2) */
  double frac = (2.0 * m - 1.0) * 8.0; /* 3 mantissa bits */
  double r = nearbyint(frac);
  if (r >= 8.0) { r = 0.0; E += 1; }
  int code = ((E + 7) << 3) | (int)r;
  if (code > 0x7E) code = 0x7E;
  return s | (uint8_t)code;
}

/* OCP E2M1 encoder, round-to-nearest-even on the grid {0,.5,1,1.5,2,3,4,6}. */
static uint8_t enc_e2m1(float v) {
  static const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  uint8_t s = (v < 0.0f) ? 8 : 0;
  float a = fabsf(v);
  if (a >= 6.0f) return s | 7;
  int lo = 0;
  while (lo < 7 && grid[lo + 1] <= a) lo++;
  if (lo == 7) return s | 7;
  float d0 = a - grid[lo], d1 = grid[lo + 1] - a;
  int c;
  if (d0 < d1) c = lo;
  else if (d1 < d0) c = lo + 1;
  else c = (lo & 1) ? lo + 1 : lo;     /* tie: even code (even mantissa bit) */
  return s | (uint8_t)c;
}

/* n values of N(0, sigma^2) rounded to bf16. */
void synth_normal_bf16(uint16_t* out, size_t n, uint64_t key, const float* table, float sigma) {
  for (size_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(table[uniform16(key, i)] * sigma);
}

/* n values of N(0, sigma^2) as fp32. */
void synth_normal_f32(float* out, size_t n, uint64_t key, const float* table, float sigma) {
  for (size_t i = 0; i < n; ++i) out[i] = table[uniform16(key, i)] * sigma;
}

/* keys[i] = synth_key(base, first + i). */
void synth_keys(uint64_t* out, size_t n, uint64_t base, uint64_t first) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < (long)n; ++i) out[i] = synth_key(base, first + (uint64_t)i);
}

/* n rows of H bf16 values, row i drawn from stream keys[i]. */
void synth_rows_bf16(uint16_t* out, const uint64_t* keys, size_t n, int H, const float* table, float sigma) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < (long)n; ++i) synth_normal_bf16(out + (size_t)i * H, (size_t)H, keys[i], table, sigma);
}

/* n uniforms in [0,1) with 53 bits. */
void synth_uniform_f64(double* out, size_t n, uint64_t key) {
  for (size_t i = 0; i < n; ++i) out[i] = (double)(synth_word(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

static void fill_matrix_fp8(uint8_t* q, float* scale, int rows, int cols, uint64_t key,
                            const float* table, float sigma) {
  const int rb = rows / 128, cb = cols / 128;
  for (int br = 0; br < rb; ++br)
    for (int bc = 0; bc < cb; ++bc) {
      float amax = 0.0f;
      for (int r = 0; r < 128; ++r)
        for (int c = 0; c < 128; ++c) {
          size_t idx = (size_t)(br * 128 + r) * cols + bc * 128 + c;
          float w = table[uniform16(key, idx)] * sigma;
          float a = fabsf(w);
          if (a > amax) amax = a;
        }
      float s = amax > 0.0f ? amax / 448.0f : 1.0f;
      scale[br * cb + bc] = s;
      for (int r = 0; r < 128; ++r)
        for (int c = 0; c < 128; ++c) {
          size_t idx = (size_t)(br * 128 + r) * cols + bc * 128 + c;
          float w = table[uniform16(key, idx)] * sigma;
          q[idx] = enc_e4m3(w / s);
        }
    }
}

static void fill_matrix_mxfp4(uint8_t* packed, uint8_t* e8m0, int rows, int cols, uint64_t key,
                              const float* table, float sigma) {
  const int nb = cols / 32;
  for (int r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b) {
      float w[32];
      float amax = 0.0f;
      for (int c = 0; c < 32; ++c) {
        size_t idx = (size_t)r * cols + b * 32 + c;
        w[c] = table[uniform16(key, idx)] * sigma;
        if (fabsf(w[c]) > amax) amax = fabsf(w[c]);
      }
      int x;
      if (amax == 0.0f) x = 0;
      else {
        int e;
        frexpf(amax, &e);
        x = (e - 1) - 2;
        if (x < -127) x = -127;
        if (x > 127) x = 127;
      }
      e8m0[(size_t)r * nb + b] = (uint8_t)(x + 127);
      for (int c = 0; c < 32; c += 2) {
        uint8_t lo = enc_e2m1(ldexpf(w[c], -x));
        uint8_t hi = enc_e2m1(ldexpf(w[c + 1], -x));
        packed[((size_t)r * cols + b * 32 + c) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
}

static void fill_matrix_nvfp4(uint8_t* packed, uint8_t* e4m3, float* tensor_scale, int rows, int cols,
                              uint64_t key, const float* table, float sigma) {
  const size_t n = (size_t)rows * cols;
  float amax = 0.0f;
  for (size_t i = 0; i < n; ++i) {
    const float a = fabsf(table[uniform16(key, i)] * sigma);
    if (a > amax) amax = a;
  }
  const float t = amax > 0.0f ? amax / (6.0f * 448.0f) : 1.0f;
  *tensor_scale = t;
  const int nb = cols / 16;
  for (int r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b) {
      float w[16];
      float bmax = 0.0f;
      for (int c = 0; c < 16; ++c) {
        w[c] = table[uniform16(key, (size_t)r * cols + b * 16 + c)] * sigma;
        if (fabsf(w[c]) > bmax) bmax = fabsf(w[c]);
      }
      const uint8_t sc = enc_e4m3(bmax / (6.0f * t));
      e4m3[(size_t)r * nb + b] = sc;
      /* the decoded scale (E4M3: bias 7, subnormal step 2^-9) */
      const int e = (sc >> 3) & 15, m = sc & 7;
      const float sv = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + m / 8.0f, e - 7);
      const float d = sv * t;
      for (int c = 0; c < 16; c += 2) {
        const uint8_t lo = d > 0.0f ? enc_e2m1(w[c] / d) : 0;
        const uint8_t hi = d > 0.0f ? enc_e2m1(w[c + 1] / d) : 0;
        packed[((size_t)r * cols + b * 16 + c) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
}

/* Bytes of one expert blob for format fmt (0 bf16, 1 fp8 e4m3 + 128x128 fp32
 * block scales, 2 mxfp4 + e8m0 per 32, 3 nvfp4 + e4m3 per 16 + 3 fp32
 * tensor scales padded to 16 bytes). */
size_t synth_expert_bytes(int fmt, int H, int I) {
  size_t n = (size_t)H * I;
  if (fmt == 0) return 3 * n * 2;
  if (fmt == 1) return 3 * n + 3 * (n / (128 * 128)) * 4;
  if (fmt == 3) return 3 * n / 2 + 3 * n / 16 + 16;
  return 3 * n / 2 + 3 * n / 32;
}

/* One expert blob: gate [I,H], up [I,H], down [H,I] then (fp8/mxfp4) the
 * scale arrays in the same order.  key selects the expert's streams. */
void synth_expert_blob(uint8_t* out, int fmt, int H, int I, uint64_t key, const float* table, float sigma) {
  size_t n = (size_t)H * I;
  uint64_t kg = synth_key(key, 1), ku = synth_key(key, 2), kd = synth_key(key, 3);
  if (fmt == 0) {
    uint16_t* w = (uint16_t*)out;
    synth_normal_bf16(w, n, kg, table, sigma);
    synth_normal_bf16(w + n, n, ku, table, sigma);
    synth_normal_bf16(w + 2 * n, n, kd, table, sigma);
  } else if (fmt == 1) {
    size_t ns = n / (128 * 128);
    float* sc = (float*)(out + 3 * n);
    fill_matrix_fp8(out, sc, I, H, kg, table, sigma);
    fill_matrix_fp8(out + n, sc + ns, I, H, ku, table, sigma);
    fill_matrix_fp8(out + 2 * n, sc + 2 * ns, H, I, kd, table, sigma);
  } else if (fmt == 3) {
    size_t np = n / 2, ns = n / 16;
    uint8_t* sc = out + 3 * np;
    float ts[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    fill_matrix_nvfp4(out, sc, &ts[0], I, H, kg, table, sigma);
    fill_matrix_nvfp4(out + np, sc + ns, &ts[1], I, H, ku, table, sigma);
    fill_matrix_nvfp4(out + 2 * np, sc + 2 * ns, &ts[2], H, I, kd, table, sigma);
    memcpy(out + 3 * np + 3 * ns, ts, sizeof(ts));
  } else {
    size_t np = n / 2, ns = n / 32;
    uint8_t* sc = out + 3 * np;
    fill_matrix_mxfp4(out, sc, I, H, kg, table, sigma);
    fill_matrix_mxfp4(out + np, sc + ns, I, H, ku, table, sigma);
    fill_matrix_mxfp4(out + 2 * np, sc + 2 * ns, H, I, kd, table, sigma);
  }
}

/* Experts [first, first+count) of a pool laid out [L*E][S]; expert id g =
 * l*E+e uses key synth_key(seed_key, g).  Parallel over experts. */
void synth_pool(uint8_t* pool, size_t S, long first, long count, int fmt, int H, int I,
                uint64_t seed_key, const float* table, float sigma) {
#pragma omp parallel for schedule(dynamic, 1)
  for (long g = first; g < first + count; ++g)
    synth_expert_blob(pool + (size_t)(g - first) * S, fmt, H, I, synth_key(seed_key, (uint64_t)g), table, sigma);
}
