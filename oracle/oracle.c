/*
 * CPU oracle for the quantized MoE grouped-GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the bench's CPU
 * baseline do.  It shares no code with the HIP library.
 *
 * What it computes (plain definitions, double precision, no blocking):
 *
 *  route    Orbit page, 时刻细节 "Active-expert-chunked dequantization": every
 *           token activates only the experts its router selects.  Per token:
 *           order experts by (logit descending, expert id ascending), keep the
 *           first k; softmax over all E logits in double; renormalise the k
 *           kept probabilities so they sum to 1.
 *  permute  Same passage: the selected experts are grouped before the grouped
 *           GEMM.  Pairs p = t*k + j are listed expert by expert (ascending
 *           id), ascending p inside an expert (a stable counting sort).
 *  decode   "超大规模开放权重模型技术解析", 三 微缩放量化的原理: 4-bit elements in
 *           groups of 32 sharing one scale.  MXFP4: E2M1 value table times
 *           2^(e8m0 - 127) (code 255 is NaN); INT4: two's-complement nibble
 *           times its BF16 scale.  Both products are formed in fp32, where
 *           they are exact unless they overflow.
 *  project  y[pair][n] = sum over k ascending of x[t][k] * W_e[n][k], double;
 *           the transposed form sums over W's rows: y[i][c] = sum_n a[i][n] W_e[n][c].
 *  ffn      h = W_gu,e x (rows [0,I) gate, [I,2I) up); a = silu(gate) * up;
 *           o = W_down,e a; y[t] = sum over j ascending of g[t,j] * o[t,j].
 *  dx       Orbit page, 时刻细节: the backward for a frozen base forms no weight
 *           gradient.  dO = g * dY[t]; dA = W_down^T dO; dH = [dA * up *
 *           silu'(gate) | dA * silu(gate)]; dXp = W_gu^T dH; dX[t] = sum over
 *           j ascending of dXp[t,j].  Gates are constants.
 *  lora     Orbit page, opening section: a BF16 adapter on the frozen base.
 *           LoRA form y = x W_e^T + alpha (x A_e^T) B_e^T, in double; its
 *           backward gives the adapter's weight gradients and its part of dx.
 *  router_bwd  The gradient the base hands back to a trainable router (the
 *           pages freeze the base, not the router): dg[t,j] = <dY[t], o[t,j]>,
 *           then reverse mode through the gate definition of route.  The
 *           pages give no formula for this step; it is the chain rule
 *           applied to the forward above.
 *
 * Weight layout: packed [E][N][K/2] (element k in byte k>>1, low nibble for
 * even k), scales [E][N][K/32] (u8 E8M0 for MXFP4, u16 BF16 bits for INT4).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { FMT_MXFP4 = 1, FMT_INT4 = 2 };

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------- scalars */

static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round-to-nearest-even fp32 -> BF16 bits; NaN stays NaN (quiet). */
static uint16_t float_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t rounding = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + rounding) >> 16);
}

void oracle_bf16_view(const float* w, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16(w[i]);
}

void oracle_bf16_to_f64(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (double)bf16_to_float(h[i]);
}

/* E2M1 values by code: sign bit 3, then the eight magnitudes. */
static const float kE2M1[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                                -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

static float e8m0_value(uint8_t code) {
  if (code == 255) return NAN;
  return ldexpf(1.0f, (int)code - 127);
}

static float decode_one(int fmt, uint8_t nib, const void* scales, int64_t sidx) {
  if (fmt == FMT_MXFP4) return kE2M1[nib] * e8m0_value(((const uint8_t*)scales)[sidx]);
  int q = (int)(nib & 0xF);
  if (q >= 8) q -= 16;
  return (float)q * bf16_to_float(((const uint16_t*)scales)[sidx]);
}

/* Decode one expert's [N][K] weights to fp32. */
int oracle_decode(int fmt, const uint8_t* packed, const void* scales, int64_t N, int64_t K,
                  float* w) {
  if ((fmt != FMT_MXFP4 && fmt != FMT_INT4) || K % 32) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t byte = packed[n * (K / 2) + k / 2];
      const uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
      w[n * K + k] = decode_one(fmt, nib, scales, n * (K / 32) + k / 32);
    }
  }
  return 0;
}

static int64_t scale_bytes(int fmt) { return fmt == FMT_MXFP4 ? 1 : 2; }

static void expert_ptrs(int fmt, const uint8_t* packed, const void* scales, int64_t N, int64_t K,
                        int e, const uint8_t** pe, const void** se) {
  *pe = packed + (int64_t)e * N * (K / 2);
  *se = (const uint8_t*)scales + (int64_t)e * N * (K / 32) * scale_bytes(fmt);
}

/* --------------------------------------------------------------- route */

int oracle_route(const float* logits, int T, int E, int k, int32_t* ids, double* gates) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return 1;
  for (int64_t i = 0; i < (int64_t)T * E; ++i)
    if (!isfinite(logits[i])) return 2;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (int64_t)t * E;
    char* taken = (char*)calloc((size_t)E, 1);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    if (!taken || !p) {
      bad = 1;
      free(taken);
      free(p);
      continue;
    }
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        /* strictly greater logit wins; equal logits keep the lower id */
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
    double m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmax(m, (double)l[e]);
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = exp((double)l[e] - m);
      z += p[e];
    }
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += p[ids[(int64_t)t * k + j]] / z;
    for (int j = 0; j < k; ++j) gates[(int64_t)t * k + j] = (p[ids[(int64_t)t * k + j]] / z) / s;
    free(taken);
    free(p);
  }
  return bad ? 3 : 0;
}

/* ------------------------------------------------------------- permute */

int oracle_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                   int32_t* perm, int32_t* inv_perm, int32_t* active, int32_t* n_active) {
  const int64_t P = (int64_t)T * k;
  for (int64_t p = 0; p < P; ++p)
    if (ids[p] < 0 || ids[p] >= E) return 1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) counts[ids[p]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t pos = 0;
  for (int e = 0; e < E; ++e)
    for (int64_t p = 0; p < P; ++p)
      if (ids[p] == e) perm[pos++] = (int32_t)p;
  for (int64_t i = 0; i < P; ++i) inv_perm[perm[i]] = (int32_t)i;
  int a = 0;
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0) active[a++] = e;
  for (int i = a; i < E; ++i) active[i] = -1;
  *n_active = a;
  return 0;
}

/* ---------------------------------------------------------- projection */

static double dot_f64(const double* a, const float* b, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += a[i] * (double)b[i];
  return s;
}

/* y[i][n] = sum_k x[tok[i]][k] * W_{exp[i]}[n][k] for npairs pairs.
 * x is BF16 [T][K]; weights [E][N][K] in fmt; y is double [npairs][N]. */
int oracle_project(int fmt, const uint8_t* packed, const void* scales, int E, int64_t N,
                   int64_t K, const uint16_t* x, int64_t npairs, const int32_t* tok,
                   const int32_t* expert, double* y) {
  float* w = (float*)malloc(sizeof(float) * (size_t)(N * K));
  double* xr = (double*)malloc(sizeof(double) * (size_t)K);
  if (!w || !xr) {
    free(w);
    free(xr);
    return 3;
  }
  for (int e = 0; e < E; ++e) {
    int used = 0;
    for (int64_t i = 0; i < npairs && !used; ++i) used = expert[i] == e;
    if (!used) continue;
    const uint8_t* pe;
    const void* se;
    expert_ptrs(fmt, packed, scales, N, K, e, &pe, &se);
    if (oracle_decode(fmt, pe, se, N, K, w)) {
      free(w);
      free(xr);
      return 1;
    }
    for (int64_t i = 0; i < npairs; ++i) {
      if (expert[i] != e) continue;
      oracle_bf16_to_f64(x + (int64_t)tok[i] * K, K, xr);
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < N; ++n) y[i * N + n] = dot_f64(xr, w + n * K, K);
    }
  }
  free(w);
  free(xr);
  return 0;
}

/* Transposed access, as the input-gradient backward reads the frozen base:
 * y[i][c] = sum over n ascending of a[i][n] * W_{expert[i]}[n][c].  a is BF16
 * [npairs][N] (one row per pair), y is double [npairs][K]. */
int oracle_project_t(int fmt, const uint8_t* packed, const void* scales, int E, int64_t N,
                     int64_t K, const uint16_t* a, int64_t npairs, const int32_t* expert,
                     double* y) {
  float* w = (float*)malloc(sizeof(float) * (size_t)(N * K));
  double* ar = (double*)malloc(sizeof(double) * (size_t)N);
  if (!w || !ar) {
    free(w);
    free(ar);
    return 3;
  }
  for (int e = 0; e < E; ++e) {
    int used = 0;
    for (int64_t i = 0; i < npairs && !used; ++i) used = expert[i] == e;
    if (!used) continue;
    const uint8_t* pe;
    const void* se;
    expert_ptrs(fmt, packed, scales, N, K, e, &pe, &se);
    if (oracle_decode(fmt, pe, se, N, K, w)) {
      free(w);
      free(ar);
      return 1;
    }
    for (int64_t i = 0; i < npairs; ++i) {
      if (expert[i] != e) continue;
      oracle_bf16_to_f64(a + i * N, N, ar);
#pragma omp parallel for schedule(static)
      for (int64_t c = 0; c < K; ++c) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += ar[n] * (double)w[n * K + c];
        y[i * K + c] = acc;
      }
    }
  }
  free(w);
  free(ar);
  return 0;
}

/* ----------------------------------------------------------------- FFN */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
double oracle_silu(double z) { return z * sigmoid(z); }
double oracle_silu_grad(double z) {
  const double s = sigmoid(z);
  return s * (1.0 + z * (1.0 - s));
}

/* Shared driver: for every selected token and each of its k slots, decode the
 * slot's expert (once per expert) and evaluate the per-pair quantities.
 * mode 0: forward  -> o[slot][d] (and h[slot][2I] if h != NULL)
 * mode 1: backward -> dxp[slot][d] (and dA[slot][I] if da != NULL) */
static int ffn_pairs(int mode, int fmt, const uint8_t* gu_p, const void* gu_s,
                     const uint8_t* dn_p, const void* dn_s, int E, int64_t d, int64_t I,
                     const uint16_t* x, const uint16_t* dy, int k, const int32_t* ids,
                     const double* gates, int64_t ntok, const int32_t* toks, double* out,
                     double* h_out, double* da_out) {
  const int64_t N2 = 2 * I;
  float* wgu = (float*)malloc(sizeof(float) * (size_t)(N2 * d));
  float* wdn = (float*)malloc(sizeof(float) * (size_t)(d * I));
  double* xr = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)N2);
  double* a = (double*)malloc(sizeof(double) * (size_t)N2);
  int rc = 0;
  if (!wgu || !wdn || !xr || !h || !a) rc = 3;
  for (int e = 0; e < E && !rc; ++e) {
    int used = 0;
    for (int64_t s = 0; s < ntok * k && !used; ++s)
      used = ids[(int64_t)toks[s / k] * k + s % k] == e;
    if (!used) continue;
    const uint8_t* pe;
    const void* se;
    expert_ptrs(fmt, gu_p, gu_s, N2, d, e, &pe, &se);
    rc |= oracle_decode(fmt, pe, se, N2, d, wgu);
    expert_ptrs(fmt, dn_p, dn_s, d, I, e, &pe, &se);
    rc |= oracle_decode(fmt, pe, se, d, I, wdn);
    if (rc) break;
    for (int64_t s = 0; s < ntok * k; ++s) {
      const int64_t t = toks[s / k];
      const int64_t j = s % k;
      if (ids[t * k + j] != e) continue;
      oracle_bf16_to_f64(x + t * d, d, xr);
      /* h = W_gu x */
#pragma omp parallel for schedule(static)
      for (int64_t r = 0; r < N2; ++r) h[r] = dot_f64(xr, wgu + r * d, d);
      if (h_out) memcpy(h_out + s * N2, h, sizeof(double) * (size_t)N2);
      double* o = out + s * d;
      if (mode == 0) {
        for (int64_t i = 0; i < I; ++i) a[i] = oracle_silu(h[i]) * h[I + i];
        /* o = W_down a */
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < d; ++n) {
          double acc = 0.0;
          for (int64_t i = 0; i < I; ++i) acc += (double)wdn[n * I + i] * a[i];
          o[n] = acc;
        }
      } else {
        const double g = gates[t * k + j];
        double* dO = (double*)malloc(sizeof(double) * (size_t)d);
        double* dA = (double*)malloc(sizeof(double) * (size_t)I);
        if (!dO || !dA) {
          free(dO);
          free(dA);
          rc = 3;
          break;
        }
        for (int64_t n = 0; n < d; ++n) dO[n] = g * (double)bf16_to_float(dy[t * d + n]);
        /* dA = W_down^T dO: every dA[i] sums its terms over n ascending;
           a thread takes 64 consecutive i at a time and runs n outside, so
           that W_down is read along its rows */
#pragma omp parallel for schedule(static)
        for (int64_t i0 = 0; i0 < I; i0 += 64) {
          const int64_t i1 = i0 + 64 < I ? i0 + 64 : I;
          for (int64_t i = i0; i < i1; ++i) dA[i] = 0.0;
          for (int64_t n = 0; n < d; ++n)
            for (int64_t i = i0; i < i1; ++i) dA[i] += dO[n] * (double)wdn[n * I + i];
        }
        if (da_out) memcpy(da_out + s * I, dA, sizeof(double) * (size_t)I);
        /* dH = [dA * up * silu'(gate) | dA * silu(gate)] */
        for (int64_t i = 0; i < I; ++i) {
          a[i] = dA[i] * h[I + i] * oracle_silu_grad(h[i]);
          a[I + i] = dA[i] * oracle_silu(h[i]);
        }
        /* dXp = W_gu^T dH: every o[c] sums its terms over r ascending
           (64 consecutive c per thread at a time, r outside, as above) */
#pragma omp parallel for schedule(static)
        for (int64_t c0 = 0; c0 < d; c0 += 64) {
          const int64_t c1 = c0 + 64 < d ? c0 + 64 : d;
          for (int64_t c = c0; c < c1; ++c) o[c] = 0.0;
          for (int64_t r = 0; r < N2; ++r)
            for (int64_t c = c0; c < c1; ++c) o[c] += a[r] * (double)wgu[r * d + c];
        }
        free(dO);
        free(dA);
      }
    }
  }
  free(wgu);
  free(wdn);
  free(xr);
  free(h);
  free(a);
  return rc;
}

/* y[s][n] for the selected tokens toks[0..ntok): sum over j ascending of
 * g[t,j] * o[t,j][n].  h_out (nullable) receives h per (token, slot):
 * [ntok*k][2I]. */
int oracle_ffn(int fmt, const uint8_t* gu_p, const void* gu_s, const uint8_t* dn_p,
               const void* dn_s, int E, int64_t d, int64_t I, const uint16_t* x, int k,
               const int32_t* ids, const double* gates, int64_t ntok, const int32_t* toks,
               double* y, double* h_out) {
  double* o = (double*)malloc(sizeof(double) * (size_t)(ntok * k * d));
  if (!o) return 3;
  int rc = ffn_pairs(0, fmt, gu_p, gu_s, dn_p, dn_s, E, d, I, x, NULL, k, ids, gates, ntok, toks,
                     o, h_out, NULL);
  if (!rc) {
    for (int64_t s = 0; s < ntok; ++s) {
      const int64_t t = toks[s];
      for (int64_t n = 0; n < d; ++n) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += gates[t * k + j] * o[(s * k + j) * d + n];
        y[s * d + n] = acc;
      }
    }
  }
  free(o);
  return rc;
}

/* dX[s][c] for the selected tokens: sum over j ascending of dXp[t,j][c].
 * da_out (nullable) receives dA per (token, slot): [ntok*k][I]. */
int oracle_dx(int fmt, const uint8_t* gu_p, const void* gu_s, const uint8_t* dn_p,
              const void* dn_s, int E, int64_t d, int64_t I, const uint16_t* x,
              const uint16_t* dy, int k, const int32_t* ids, const double* gates, int64_t ntok,
              const int32_t* toks, double* dx, double* da_out) {
  double* dxp = (double*)malloc(sizeof(double) * (size_t)(ntok * k * d));
  if (!dxp) return 3;
  int rc = ffn_pairs(1, fmt, gu_p, gu_s, dn_p, dn_s, E, d, I, x, dy, k, ids, gates, ntok, toks,
                     dxp, NULL, da_out);
  if (!rc) {
    for (int64_t s = 0; s < ntok; ++s) {
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += dxp[(s * k + j) * d + c];
        dx[s * d + c] = acc;
      }
    }
  }
  free(dxp);
  return rc;
}

/* ------------------------------------------------------ router backward */

/* Gradient of L = <dY, y> with respect to the gates and the router logits,
 * the base and the routing choice held fixed (the top-k selection is
 * piecewise constant in the logits, so it passes no gradient).
 *
 * dg[s][j] = sum over n ascending of dY[t][n] * o[t,j][n], o from the forward
 * definition above.  The logit gradient runs reverse mode through the gate
 * definition of oracle_route, step by step: p = softmax over all E logits,
 * S = sum of the kept p, g_j = p[id_j] / S; so
 *   dS = -sum_j dg_j p[id_j] / S^2,
 *   dp_e = (e kept as slot j ? dg_j / S : 0) + (e kept ? dS : 0),
 *   dl_e = p_e (dp_e - sum_e' p_e' dp_e').
 * Outputs for the selected tokens: dgates [ntok][k], dlogits [ntok][E]
 * (either may be NULL). */
int oracle_router_bwd(int fmt, const uint8_t* gu_p, const void* gu_s, const uint8_t* dn_p,
                      const void* dn_s, int E, int64_t d, int64_t I, const uint16_t* x,
                      const uint16_t* dy, const float* logits, int k, const int32_t* ids,
                      int64_t ntok, const int32_t* toks, double* dgates, double* dlogits) {
  double* o = (double*)malloc(sizeof(double) * (size_t)(ntok * k * d));
  double* dg = (double*)malloc(sizeof(double) * (size_t)(ntok * k));
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  double* dp = (double*)malloc(sizeof(double) * (size_t)E);
  int rc = (!o || !dg || !p || !dp) ? 3 : 0;
  if (!rc)
    rc = ffn_pairs(0, fmt, gu_p, gu_s, dn_p, dn_s, E, d, I, x, NULL, k, ids, NULL, ntok, toks, o,
                   NULL, NULL);
  for (int64_t s = 0; s < ntok && !rc; ++s) {
    const int64_t t = toks[s];
    for (int j = 0; j < k; ++j) {
      double acc = 0.0;
      for (int64_t n = 0; n < d; ++n)
        acc += (double)bf16_to_float(dy[t * d + n]) * o[(s * k + j) * d + n];
      dg[s * k + j] = acc;
      if (dgates) dgates[s * k + j] = acc;
    }
    if (!dlogits) continue;
    const float* l = logits + t * E;
    double m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmax(m, (double)l[e]);
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = exp((double)l[e] - m);
      z += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= z;
    double S = 0.0;
    for (int j = 0; j < k; ++j) S += p[ids[t * k + j]];
    double dS = 0.0;
    for (int j = 0; j < k; ++j) dS -= dg[s * k + j] * p[ids[t * k + j]] / (S * S);
    for (int e = 0; e < E; ++e) dp[e] = 0.0;
    for (int j = 0; j < k; ++j) dp[ids[t * k + j]] += dg[s * k + j] / S + dS;
    double pdp = 0.0;
    for (int e = 0; e < E; ++e) pdp += p[e] * dp[e];
    for (int e = 0; e < E; ++e) dlogits[s * E + e] = p[e] * (dp[e] - pdp);
  }
  free(o);
  free(dg);
  free(p);
  free(dp);
  return rc;
}

/* ------------------------------------------------------ adapter (LoRA) */

/* Orbit page, opening section: the base is frozen in its low-precision
 * format and one BF16 adapter on top of it is what trains.  Which adapter is
 * a reading: on the Orbit issue page the maintainers make orthogonal
 * finetuning (OFT / QOFT) the default and prefer it to LoRA, the feature the
 * question mentions; no OFT formula is on the pages, so the additive
 * low-rank (LoRA) form is what is built.  LoRA form of one expert
 * projection:
 *   y[i][n] = sum_k x[t][k] W_e[n][k] + alpha * sum_j u[i][j] B_e[n][j],
 *   u[i][j] = sum_k x[t][k] A_e[j][k]
 * with t = tok[i], e = expert[i]; A is BF16 [E][rank][K], B BF16 [E][N][rank].
 * Everything in double; u (nullable) receives alpha * u, as [npairs][rank]. */
int oracle_lora_project(int fmt, const uint8_t* packed, const void* scales, int E, int64_t N,
                        int64_t K, const uint16_t* x, int64_t npairs, const int32_t* tok,
                        const int32_t* expert, int rank, double alpha, const uint16_t* A,
                        const uint16_t* B, double* y, double* u_out) {
  if (rank <= 0) return 1;
  int rc = oracle_project(fmt, packed, scales, E, N, K, x, npairs, tok, expert, y);
  if (rc) return rc;
  double* xr = (double*)malloc(sizeof(double) * (size_t)K);
  double* u = (double*)malloc(sizeof(double) * (size_t)rank);
  if (!xr || !u) {
    free(xr);
    free(u);
    return 3;
  }
  for (int64_t i = 0; i < npairs; ++i) {
    const int64_t e = expert[i];
    oracle_bf16_to_f64(x + (int64_t)tok[i] * K, K, xr);
    for (int j = 0; j < rank; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += xr[k] * (double)bf16_to_float(A[(e * rank + j) * K + k]);
      u[j] = acc;
      if (u_out) u_out[i * rank + j] = alpha * acc;
    }
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int j = 0; j < rank; ++j) acc += u[j] * (double)bf16_to_float(B[(e * N + n) * rank + j]);
      y[i * N + n] += alpha * acc;
    }
  }
  free(xr);
  free(u);
  return 0;
}

/* Backward of oracle_lora_project's adapter term for L = <dY, y>, base frozen
 * (chain rule through y = x W^T + alpha (x A^T) B^T; the pages give no
 * formula for this step).  Per pair i (t = tok[i], e = expert[i]):
 *   u_i = alpha x_t A_e^T,  du_i = dY_i B_e,  dx_i = alpha du_i A_e,
 *   dA_e = alpha sum_i du_i (x) x_t,  dB_e = sum_i dY_i (x) u_i.
 * dy BF16 [npairs][N]; outputs double: dx [npairs][K], dA [E][rank][K],
 * dB [E][N][rank] (each nullable; dA, dB are overwritten, zero for experts no
 * pair uses). */
int oracle_lora_bwd(int E, int64_t N, int64_t K, const uint16_t* x, const uint16_t* dy,
                    int64_t npairs, const int32_t* tok, const int32_t* expert, int rank,
                    double alpha, const uint16_t* A, const uint16_t* B, double* dx, double* dA,
                    double* dB) {
  if (rank <= 0) return 1;
  double* xr = (double*)malloc(sizeof(double) * (size_t)K);
  double* u = (double*)malloc(sizeof(double) * (size_t)rank);
  double* du = (double*)malloc(sizeof(double) * (size_t)rank);
  if (!xr || !u || !du) {
    free(xr);
    free(u);
    free(du);
    return 3;
  }
  if (dA) memset(dA, 0, sizeof(double) * (size_t)(E * rank * K));
  if (dB) memset(dB, 0, sizeof(double) * (size_t)(E * N * rank));
  for (int64_t i = 0; i < npairs; ++i) {
    const int64_t e = expert[i];
    oracle_bf16_to_f64(x + (int64_t)tok[i] * K, K, xr);
    for (int j = 0; j < rank; ++j) {
      double su = 0.0, sd = 0.0;
      for (int64_t k = 0; k < K; ++k) su += xr[k] * (double)bf16_to_float(A[(e * rank + j) * K + k]);
      for (int64_t n = 0; n < N; ++n)
        sd += (double)bf16_to_float(dy[i * N + n]) * (double)bf16_to_float(B[(e * N + n) * rank + j]);
      u[j] = alpha * su;
      du[j] = sd;
    }
    if (dx)
      for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int j = 0; j < rank; ++j) acc += du[j] * (double)bf16_to_float(A[(e * rank + j) * K + k]);
        dx[i * K + k] = alpha * acc;
      }
    if (dA)
      for (int j = 0; j < rank; ++j)
        for (int64_t k = 0; k < K; ++k) dA[(e * rank + j) * K + k] += alpha * du[j] * xr[k];
    if (dB)
      for (int64_t n = 0; n < N; ++n) {
        const double g = (double)bf16_to_float(dy[i * N + n]);
        for (int j = 0; j < rank; ++j) dB[(e * N + n) * rank + j] += g * u[j];
      }
  }
  free(xr);
  free(u);
  free(du);
  return 0;
}

/* The SwiGLU FFN of oracle_ffn with a LoRA adapter on each projection (null
 * adapter pointers: none on that projection), in double:
 *   h = W_gu x + alpha_gu B_gu (A_gu x),  a = silu(h[:I]) * h[I:],
 *   o = W_dn a + alpha_dn B_dn (A_dn a),  y[t] = sum over j ascending of g o.
 * A_gu [E][rank][d], B_gu [E][2I][rank], A_dn [E][rank][I], B_dn [E][d][rank]. */
int oracle_ffn_lora(int fmt, const uint8_t* gu_p, const void* gu_s, const uint8_t* dn_p,
                    const void* dn_s, int E, int64_t d, int64_t I, const uint16_t* x, int k,
                    const int32_t* ids, const double* gates, int64_t ntok, const int32_t* toks,
                    int rank, double alpha_gu, double alpha_dn, const uint16_t* Agu,
                    const uint16_t* Bgu, const uint16_t* Adn, const uint16_t* Bdn, double* y) {
  if (rank <= 0) return 1;
  const int64_t N2 = 2 * I;
  float* wgu = (float*)malloc(sizeof(float) * (size_t)(N2 * d));
  float* wdn = (float*)malloc(sizeof(float) * (size_t)(d * I));
  double* xr = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)N2);
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  double* op = (double*)malloc(sizeof(double) * (size_t)(ntok * k * d));   /* per pair */
  double* u = (double*)malloc(sizeof(double) * (size_t)rank);
  int rc = (!wgu || !wdn || !xr || !h || !a || !op || !u) ? 3 : 0;
  for (int e = 0; e < E && !rc; ++e) {
    int used = 0;
    for (int64_t s = 0; s < ntok * k && !used; ++s)
      used = ids[(int64_t)toks[s / k] * k + s % k] == e;
    if (!used) continue;
    const uint8_t* pe;
    const void* se;
    expert_ptrs(fmt, gu_p, gu_s, N2, d, e, &pe, &se);
    rc |= oracle_decode(fmt, pe, se, N2, d, wgu);
    expert_ptrs(fmt, dn_p, dn_s, d, I, e, &pe, &se);
    rc |= oracle_decode(fmt, pe, se, d, I, wdn);
    if (rc) break;
    for (int64_t s = 0; s < ntok * k; ++s) {
      const int64_t t = toks[s / k];
      const int64_t j = s % k;
      if (ids[t * k + j] != e) continue;
      oracle_bf16_to_f64(x + t * d, d, xr);
      for (int64_t r = 0; r < N2; ++r) h[r] = dot_f64(xr, wgu + r * d, d);
      if (Agu && Bgu) {
        for (int q = 0; q < rank; ++q) {
          double acc = 0.0;
          for (int64_t c = 0; c < d; ++c)
            acc += xr[c] * (double)bf16_to_float(Agu[((int64_t)e * rank + q) * d + c]);
          u[q] = acc;
        }
        for (int64_t r = 0; r < N2; ++r) {
          double acc = 0.0;
          for (int q = 0; q < rank; ++q)
            acc += u[q] * (double)bf16_to_float(Bgu[((int64_t)e * N2 + r) * rank + q]);
          h[r] += alpha_gu * acc;
        }
      }
      for (int64_t i = 0; i < I; ++i) a[i] = oracle_silu(h[i]) * h[I + i];
      double* o = op + s * d;
      for (int64_t n = 0; n < d; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i) acc += (double)wdn[n * I + i] * a[i];
        o[n] = acc;
      }
      if (Adn && Bdn) {
        for (int q = 0; q < rank; ++q) {
          double acc = 0.0;
          for (int64_t i = 0; i < I; ++i)
            acc += a[i] * (double)bf16_to_float(Adn[((int64_t)e * rank + q) * I + i]);
          u[q] = acc;
        }
        for (int64_t n = 0; n < d; ++n) {
          double acc = 0.0;
          for (int q = 0; q < rank; ++q)
            acc += u[q] * (double)bf16_to_float(Bdn[((int64_t)e * d + n) * rank + q]);
          o[n] += alpha_dn * acc;
        }
      }
    }
  }
  for (int64_t s = 0; s < ntok && !rc; ++s) {
    const int64_t t = toks[s];
    for (int64_t n = 0; n < d; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += gates[t * k + j] * op[(s * k + j) * d + n];
      y[s * d + n] = acc;
    }
  }
  free(wgu);
  free(wdn);
  free(xr);
  free(h);
  free(a);
  free(op);
  free(u);
  return rc;
}

/* Backward of oracle_ffn_lora for L = <dY, y>, the base and the gates held
 * fixed: the gradients of both adapters and the input gradient through them
 * and the frozen base.  Orbit page, opening section: the base stays frozen and
 * the BF16 adapter is what trains; section 时刻细节: no gradient is formed for
 * the frozen base.  The pages give no formula for this step; it is the chain
 * rule through the forward above, per (token, slot) pair with e = ids[t][j],
 * g = gates[t][j], the forward quantities recomputed in double:
 *   u_gu = alpha_gu A_gu x,  h = W_gu x + B_gu u_gu,  a = silu(h_g) h_u,
 *   u_dn = alpha_dn A_dn a,  o = W_dn a + B_dn u_dn,
 * then, from dO = g dY[t]:
 *   dB_dn += dO (x) u_dn,  du_dn = B_dn^T dO,  dA_dn += alpha_dn du_dn (x) a,
 *   da = W_dn^T dO + alpha_dn A_dn^T du_dn,
 *   dH = [da h_u silu'(h_g) | da silu(h_g)],
 *   dB_gu += dH (x) u_gu,  du_gu = B_gu^T dH,  dA_gu += alpha_gu du_gu (x) x,
 *   dXp = W_gu^T dH + alpha_gu A_gu^T du_gu,
 * and dX[s] = sum over j ascending of dXp[t,j] for the selected tokens.
 * A null A or B leaves that projection without an adapter.  Shapes: A_gu
 * [E][r_gu][d], B_gu [E][2I][r_gu], A_dn [E][r_dn][I], B_dn [E][d][r_dn];
 * outputs (each nullable; the weight gradients are overwritten, zero for
 * experts no pair uses): dx [ntok][d], dA_gu [E][r_gu][d], dB_gu
 * [E][2I][r_gu], dA_dn [E][r_dn][I], dB_dn [E][d][r_dn]. */
int oracle_ffn_lora_bwd(int fmt, const uint8_t* gu_p, const void* gu_s, const uint8_t* dn_p,
                        const void* dn_s, int E, int64_t d, int64_t I, const uint16_t* x,
                        const uint16_t* dy, int k, const int32_t* ids, const double* gates,
                        int64_t ntok, const int32_t* toks, int r_gu, int r_dn, double alpha_gu,
                        double alpha_dn, const uint16_t* Agu, const uint16_t* Bgu,
                        const uint16_t* Adn, const uint16_t* Bdn, double* dx, double* dAgu,
                        double* dBgu, double* dAdn, double* dBdn) {
  const int has_gu = Agu && Bgu, has_dn = Adn && Bdn;
  if ((has_gu && r_gu <= 0) || (has_dn && r_dn <= 0)) return 1;
  const int64_t N2 = 2 * I;
  const int rmax = (r_gu > r_dn ? r_gu : r_dn) > 0 ? (r_gu > r_dn ? r_gu : r_dn) : 1;
  float* wgu = (float*)malloc(sizeof(float) * (size_t)(N2 * d));
  float* wdn = (float*)malloc(sizeof(float) * (size_t)(d * I));
  double* xr = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)N2);
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  double* dO = (double*)malloc(sizeof(double) * (size_t)d);
  double* da = (double*)malloc(sizeof(double) * (size_t)I);
  double* dH = (double*)malloc(sizeof(double) * (size_t)N2);
  double* ugu = (double*)malloc(sizeof(double) * (size_t)rmax);
  double* udn = (double*)malloc(sizeof(double) * (size_t)rmax);
  double* du = (double*)malloc(sizeof(double) * (size_t)rmax);
  double* dxp = (double*)malloc(sizeof(double) * (size_t)(ntok * k * d));
  int rc = (!wgu || !wdn || !xr || !h || !a || !dO || !da || !dH || !ugu || !udn || !du || !dxp)
               ? 3 : 0;
  if (dAgu && has_gu) memset(dAgu, 0, sizeof(double) * (size_t)(E * r_gu * d));
  if (dBgu && has_gu) memset(dBgu, 0, sizeof(double) * (size_t)(E * N2 * r_gu));
  if (dAdn && has_dn) memset(dAdn, 0, sizeof(double) * (size_t)(E * r_dn * I));
  if (dBdn && has_dn) memset(dBdn, 0, sizeof(double) * (size_t)(E * d * r_dn));
  for (int e = 0; e < E && !rc; ++e) {
    int used = 0;
    for (int64_t s = 0; s < ntok * k && !used; ++s)
      used = ids[(int64_t)toks[s / k] * k + s % k] == e;
    if (!used) continue;
    const uint8_t* pe;
    const void* se;
    expert_ptrs(fmt, gu_p, gu_s, N2, d, e, &pe, &se);
    rc |= oracle_decode(fmt, pe, se, N2, d, wgu);
    expert_ptrs(fmt, dn_p, dn_s, d, I, e, &pe, &se);
    rc |= oracle_decode(fmt, pe, se, d, I, wdn);
    if (rc) break;
    const uint16_t* Ag = has_gu ? Agu + (int64_t)e * r_gu * d : NULL;
    const uint16_t* Bg = has_gu ? Bgu + (int64_t)e * N2 * r_gu : NULL;
    const uint16_t* Ad = has_dn ? Adn + (int64_t)e * r_dn * I : NULL;
    const uint16_t* Bd = has_dn ? Bdn + (int64_t)e * d * r_dn : NULL;
    for (int64_t s = 0; s < ntok * k; ++s) {
      const int64_t t = toks[s / k];
      const int64_t j = s % k;
      if (ids[t * k + j] != e) continue;
      /* forward */
      oracle_bf16_to_f64(x + t * d, d, xr);
#pragma omp parallel for schedule(static)
      for (int64_t r = 0; r < N2; ++r) h[r] = dot_f64(xr, wgu + r * d, d);
      if (has_gu) {
        for (int q = 0; q < r_gu; ++q) {
          double acc = 0.0;
          for (int64_t c = 0; c < d; ++c) acc += (double)bf16_to_float(Ag[q * d + c]) * xr[c];
          ugu[q] = alpha_gu * acc;
        }
        for (int64_t r = 0; r < N2; ++r) {
          double acc = 0.0;
          for (int q = 0; q < r_gu; ++q) acc += (double)bf16_to_float(Bg[r * r_gu + q]) * ugu[q];
          h[r] += acc;
        }
      }
      for (int64_t i = 0; i < I; ++i) a[i] = oracle_silu(h[i]) * h[I + i];
      if (has_dn) {
        for (int q = 0; q < r_dn; ++q) {
          double acc = 0.0;
          for (int64_t i = 0; i < I; ++i) acc += (double)bf16_to_float(Ad[q * I + i]) * a[i];
          udn[q] = alpha_dn * acc;
        }
      }
      /* backward */
      const double g = gates[t * k + j];
      for (int64_t n = 0; n < d; ++n) dO[n] = g * (double)bf16_to_float(dy[t * d + n]);
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < I; ++i) {
        double acc = 0.0;
        for (int64_t n = 0; n < d; ++n) acc += dO[n] * (double)wdn[n * I + i];
        da[i] = acc;
      }
      if (has_dn) {
        for (int q = 0; q < r_dn; ++q) {
          double acc = 0.0;
          for (int64_t n = 0; n < d; ++n) acc += (double)bf16_to_float(Bd[n * r_dn + q]) * dO[n];
          du[q] = acc;
        }
        if (dBdn)
          for (int64_t n = 0; n < d; ++n)
            for (int q = 0; q < r_dn; ++q) dBdn[((int64_t)e * d + n) * r_dn + q] += dO[n] * udn[q];
        if (dAdn)
          for (int q = 0; q < r_dn; ++q)
            for (int64_t i = 0; i < I; ++i)
              dAdn[((int64_t)e * r_dn + q) * I + i] += alpha_dn * du[q] * a[i];
        for (int64_t i = 0; i < I; ++i) {
          double acc = 0.0;
          for (int q = 0; q < r_dn; ++q) acc += (double)bf16_to_float(Ad[q * I + i]) * du[q];
          da[i] += alpha_dn * acc;
        }
      }
      for (int64_t i = 0; i < I; ++i) {
        dH[i] = da[i] * h[I + i] * oracle_silu_grad(h[i]);
        dH[I + i] = da[i] * oracle_silu(h[i]);
      }
      double* o = dxp + s * d;
#pragma omp parallel for schedule(static)
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t r = 0; r < N2; ++r) acc += dH[r] * (double)wgu[r * d + c];
        o[c] = acc;
      }
      if (has_gu) {
        for (int q = 0; q < r_gu; ++q) {
          double acc = 0.0;
          for (int64_t r = 0; r < N2; ++r) acc += (double)bf16_to_float(Bg[r * r_gu + q]) * dH[r];
          du[q] = acc;
        }
        if (dBgu)
          for (int64_t r = 0; r < N2; ++r)
            for (int q = 0; q < r_gu; ++q)
              dBgu[((int64_t)e * N2 + r) * r_gu + q] += dH[r] * ugu[q];
        if (dAgu)
          for (int q = 0; q < r_gu; ++q)
            for (int64_t c = 0; c < d; ++c)
              dAgu[((int64_t)e * r_gu + q) * d + c] += alpha_gu * du[q] * xr[c];
        for (int64_t c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int q = 0; q < r_gu; ++q) acc += (double)bf16_to_float(Ag[q * d + c]) * du[q];
          o[c] += alpha_gu * acc;
        }
      }
    }
  }
  if (!rc && dx) {
    for (int64_t s = 0; s < ntok; ++s)
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += dxp[(s * k + j) * d + c];
        dx[s * d + c] = acc;
      }
  }
  free(wgu);
  free(wdn);
  free(xr);
  free(h);
  free(a);
  free(dO);
  free(da);
  free(dH);
  free(ugu);
  free(udn);
  free(du);
  free(dxp);
  return rc;
}
