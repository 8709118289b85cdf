/*
 * Seeded synthetic inputs for the quantized MoE grouped-GEMM path.
 *
 * This module produces the bytes that both the CPU oracle and the GPU library
 * consume: BF16 activations, fp32 router logits (optionally Zipf-biased), and
 * 4-bit expert weights already encoded in the frozen base formats (MXFP4 or
 * group-32 INT4).  It holds none of the method's arithmetic: no routing, no
 * permutation, no decoding of weights, no matrix products.
 *
 * Random source: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
 * Counter = (block index lo, block index hi, stream id, 0), key = seed.  One
 * Philox block yields four 32-bit words = eight 16-bit draws; element i of a
 * stream uses draw i % 8 of block i / 8, so any sub-range of a tensor (for
 * example one expert's weights) regenerates to the same bytes on its own.
 *
 * Normal deviates: a 16-bit draw u indexes a 65536-entry table of standard
 * normal quantiles at the bin mid-points, Phi^-1((u + 0.5) / 65536), built once
 * by bisection on Phi(z) = erfc(-z / sqrt 2) / 2.  This is inverse-transform
 * sampling with 65536 levels (|z| <= 4.42), far finer than BF16 spacing near
 * the mode, and it is cheap enough to fill ~17e9 weights in seconds.
 *
 * Encoders (the storage formats of the frozen base):
 *  - MXFP4: 32-element groups along K share one E8M0 exponent; the exponent is
 *    floor(log2(group amax)) - 2, clamped to the E8M0 range [-127, 127]; each
 *    element is w / 2^exp rounded to the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}
 *    (round to nearest, ties to the even code, saturating at 6, sign kept so a
 *    negative value that rounds to zero is code 8).
 *  - INT4: 32-element groups along K share one BF16 scale s = bf16(amax / 7);
 *    q = clamp(round_half_even(w / s), -8, 7) in two's complement; s = 0 gives
 *    q = 0.
 * Packing: element k of a row lives in byte k >> 1, low nibble for even k.
 * Layouts: packed [E][N][K/2] bytes, scales [E][N][K/32] (u8 E8M0 or u16 BF16).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- Philox */

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t n0 = hi1 ^ c[1] ^ k[0];
  const uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

/* Philox4x32 with 10 rounds; the key is bumped by the Weyl constants between
 * rounds. */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                         uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof c);
}

/* Eight 16-bit draws of block `blk` of stream `sid`. */
static inline void draws16(uint64_t seed, uint32_t sid, uint64_t blk,
                           uint16_t d[8]) {
  const uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), sid, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t o[4];
  synth_philox4x32_10(ctr, key, o);
  for (int i = 0; i < 4; ++i) {
    d[2 * i] = (uint16_t)(o[i] & 0xFFFFu);
    d[2 * i + 1] = (uint16_t)(o[i] >> 16);
  }
}

/* ------------------------------------------------------- normal quantiles */

static float g_qtab[65536];
static int g_qtab_ready = 0;

static double std_normal_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

void synth_init(void) {
  if (g_qtab_ready) return;
  for (int u = 0; u < 65536; ++u) {
    const double p = (u + 0.5) / 65536.0;
    double lo = -10.0, hi = 10.0;
    for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (mid == lo || mid == hi) break;
      if (std_normal_cdf(mid) < p) lo = mid; else hi = mid;
    }
    g_qtab[u] = (float)(0.5 * (lo + hi));
  }
  g_qtab_ready = 1;
}

const float* synth_quantile_table(void) {
  synth_init();
  return g_qtab;
}

/* ------------------------------------------------------------ BF16 bits */

static inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static inline float bf16_bits_to_f32(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------- dense tensors */

/* out[i] = bf16(mean + std * z_i), i in [i0, i0 + n) of stream `sid`. */
void synth_normal_bf16(uint64_t seed, uint32_t sid, int64_t i0, int64_t n,
                       float mean, float std, uint16_t* out) {
  synth_init();
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < (n + 7) / 8 + 1; ++b) {
    const int64_t first = (i0 / 8 + b) * 8;
    uint16_t d[8];
    draws16(seed, sid, (uint64_t)(first / 8), d);
    for (int j = 0; j < 8; ++j) {
      const int64_t i = first + j;
      if (i < i0 || i >= i0 + n) continue;
      out[i - i0] = f32_to_bf16_bits(mean + std * g_qtab[d[j]]);
    }
  }
}

/* out[i] = std * z_i (+ bias[i % ncols] if bias != NULL), fp32. */
void synth_normal_f32(uint64_t seed, uint32_t sid, int64_t i0, int64_t n,
                      float std, const float* bias, int64_t ncols, float* out) {
  synth_init();
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < (n + 7) / 8 + 1; ++b) {
    const int64_t first = (i0 / 8 + b) * 8;
    uint16_t d[8];
    draws16(seed, sid, (uint64_t)(first / 8), d);
    for (int j = 0; j < 8; ++j) {
      const int64_t i = first + j;
      if (i < i0 || i >= i0 + n) continue;
      float v = std * g_qtab[d[j]];
      if (bias) v += bias[i % ncols];
      out[i - i0] = v;
    }
  }
}

/* Zipf popularity bias: a seeded uniform permutation assigns each expert a
 * rank r in 1..E (Fisher-Yates driven by stream `sid`), and
 * bias[e] = -s * ln(r_e), so exp(bias) is proportional to r^-s. */
void synth_zipf_bias(uint64_t seed, uint32_t sid, int E, double s,
                     int32_t* rank_out, float* bias_out) {
  int32_t perm[65536];
  if (E > 65536) return;
  for (int i = 0; i < E; ++i) perm[i] = i;
  for (int i = E - 1; i > 0; --i) {
    const uint32_t ctr[4] = {(uint32_t)i, 0u, sid, 1u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t o[4];
    synth_philox4x32_10(ctr, key, o);
    const uint64_t r = ((uint64_t)o[0] << 32) | o[1];
    const int j = (int)(r % (uint64_t)(i + 1));
    const int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  /* perm[position] = expert; rank = position + 1 */
  for (int pos = 0; pos < E; ++pos) {
    const int e = perm[pos];
    if (rank_out) rank_out[e] = pos + 1;
    bias_out[e] = (float)(-s * log((double)(pos + 1)));
  }
}

/* ---------------------------------------------------------- encoders */

/* E2M1 code (0..15) of a value already divided by its group scale. */
static inline uint8_t e2m1_encode(double v) {
  const int neg = signbit(v) ? 1 : 0;
  const double a = fabs(v);
  uint8_t m;
  if (a <= 0.25) m = 0;        /* tie at .25 -> code 0 (even) */
  else if (a < 0.75) m = 1;    /* 0.5 */
  else if (a <= 1.25) m = 2;   /* 1.0; ties .75 and 1.25 -> code 2 */
  else if (a < 1.75) m = 3;    /* 1.5 */
  else if (a <= 2.5) m = 4;    /* 2.0; ties 1.75 and 2.5 -> code 4 */
  else if (a < 3.5) m = 5;     /* 3.0 */
  else if (a <= 5.0) m = 6;    /* 4.0; ties 3.5 and 5 -> code 6 */
  else m = 7;                  /* 6.0, saturating */
  return (uint8_t)((neg << 3) | m);
}

/* Encode one 32-element group of fp32 weights to MXFP4. Writes 16 bytes of
 * nibbles and returns the E8M0 scale byte. */
uint8_t synth_encode_mxfp4_group(const float* w, uint8_t* nib16) {
  float amax = 0.f;
  for (int i = 0; i < 32; ++i) {
    const float a = fabsf(w[i]);
    if (a > amax) amax = a;
  }
  int code = 0, se = -127;
  if (amax > 0.f && isfinite(amax)) {
    int ex;
    frexp((double)amax, &ex); /* amax = m * 2^ex, m in [0.5, 1) */
    se = (ex - 1) - 2;        /* floor(log2 amax) - 2 */
    if (se < -127) se = -127;
    if (se > 127) se = 127;
    code = se + 127;
  }
  for (int i = 0; i < 16; ++i) {
    uint8_t lo = 0, hi = 0;
    if (amax > 0.f) {
      lo = e2m1_encode(ldexp((double)w[2 * i], -se));
      hi = e2m1_encode(ldexp((double)w[2 * i + 1], -se));
    } else {
      lo = signbit(w[2 * i]) ? 8 : 0;
      hi = signbit(w[2 * i + 1]) ? 8 : 0;
    }
    nib16[i] = (uint8_t)(lo | (hi << 4));
  }
  return (uint8_t)code;
}

/* Encode one 32-element group to INT4 with a BF16 scale. Writes 16 bytes and
 * returns the scale's BF16 bits. */
uint16_t synth_encode_int4_group(const float* w, uint8_t* nib16) {
  float amax = 0.f;
  for (int i = 0; i < 32; ++i) {
    const float a = fabsf(w[i]);
    if (a > amax) amax = a;
  }
  const uint16_t sb = f32_to_bf16_bits(amax / 7.0f);
  const float s = bf16_bits_to_f32(sb);
  for (int i = 0; i < 16; ++i) {
    int q[2] = {0, 0};
    for (int h = 0; h < 2; ++h) {
      if (s != 0.f) {
        double r = nearbyint((double)w[2 * i + h] / (double)s);
        if (r < -8) r = -8;
        if (r > 7) r = 7;
        q[h] = (int)r;
      }
    }
    nib16[i] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
  }
  return sb;
}

/* Expert weights W[e][n][k] = std * z, for experts [e0, e1) of an E x N x K
 * tensor, encoded group by group.  fmt 1 = MXFP4 (scales u8), 2 = INT4 (scales
 * u16 BF16).  Outputs are laid out for the requested expert range only:
 * packed[(e-e0)][N][K/2], scales[(e-e0)][N][K/32].  Returns 0 on success. */
int synth_qweights(uint64_t seed, uint32_t sid, int fmt, int64_t E, int64_t N,
                   int64_t K, int64_t e0, int64_t e1, float std,
                   uint8_t* packed, void* scales) {
  if (K % 32 != 0 || e0 < 0 || e1 > E || e0 > e1) return 1;
  if (fmt != 1 && fmt != 2) return 2;
  synth_init();
  const int64_t rows = (e1 - e0) * N;
  const int64_t G = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t grow = e0 * N + r; /* global row index e * N + n */
    float w[32];
    for (int64_t g = 0; g < G; ++g) {
      const int64_t base = grow * K + g * 32; /* element index, multiple of 8 */
      for (int b = 0; b < 4; ++b) {
        uint16_t d[8];
        draws16(seed, sid, (uint64_t)(base / 8 + b), d);
        for (int j = 0; j < 8; ++j) w[b * 8 + j] = std * g_qtab[d[j]];
      }
      uint8_t* dst = packed + r * (K / 2) + g * 16;
      if (fmt == 1)
        ((uint8_t*)scales)[r * G + g] = synth_encode_mxfp4_group(w, dst);
      else
        ((uint16_t*)scales)[r * G + g] = synth_encode_int4_group(w, dst);
    }
  }
  return 0;
}

/* The fp32 weights before encoding, for a row range of the flattened [E*N][K]
 * tensor (used to check the encoders, never by the path). */
void synth_weights_f32(uint64_t seed, uint32_t sid, int64_t K, int64_t row0,
                       int64_t nrows, float std, float* out) {
  synth_init();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int64_t b = 0; b < K / 8; ++b) {
      uint16_t d[8];
      draws16(seed, sid, (uint64_t)(((row0 + r) * K) / 8 + b), d);
      for (int j = 0; j < 8; ++j) out[r * K + b * 8 + j] = std * g_qtab[d[j]];
    }
  }
}

int synth_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
