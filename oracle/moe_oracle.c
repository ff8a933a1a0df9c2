/*
 * moe_oracle.c -- CPU oracle for one Hunyuan-style mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * reference that the GPU path is checked against.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * What it computes (sources are the three pages this project follows):
 *   - Routing: "Hy3 on CANN NPU" deployment guide, section 1 (model overview):
 *     192 routed experts, top-8, sigmoid scores (moe_router_use_sigmoid),
 *     route_norm, router_scaling_factor = 2.826.  Hy4-preview tutorial,
 *     section 1: 256 routed experts, top-8, one shared expert.
 *   - Pipeline order: Hy3 guide section 8.5 (Gating -> InitRouting ->
 *     grouped GMM -> FinalizeRouting -> add of the shared expert).
 *   - Shared expert add: HunyuanImage-3.0 multi-stream article, source
 *     walkthrough part 3 (output = shared-MLP output + combined output).
 *   - Expert FFN: SwiGLU, W_d( silu(W_g x) * (W_u x) ), weights stored
 *     [out, in] (a reading: the pages give only the sizes).
 *   - MX-fp8: OCP Microscaling Formats (MX) v1.0 specification, 32-element
 *     blocks, E8M0 shared scale, E4M3 (FN variant) elements.
 *   - Static per-tensor FP8 W8A8 (the FP8 checkpoints of the Hy3 guide,
 *     section 2, and the Hy4 tutorial's w8a8 weights): one scale per weight
 *     tensor, max|w| / 448, and fixed activation scales.
 *   - MXFP4 (W4A8 routed experts, Hy3 guide section 8.2): the same
 *     specification's E2M1 elements with the same 32-element E8M0 blocks;
 *     activations stay MX-fp8 and the shared expert stays W8A8.
 *
 * Numerics.  Every stage boundary is stored as fp32.  Every dot product and
 * every sum accumulates in double in ascending index order and is rounded
 * once to fp32.  Transcendentals are evaluated in double.  Results are
 * therefore independent of the number of OpenMP threads.
 *
 * Error behaviour: functions return 0 on success and -1 on a bad argument.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* Threads an OpenMP region of this library runs with (for reporting). */
ORC_EXPORT int oracle_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------ */
/* Element decoding                                                    */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Weight element loader: wdtype 0 = fp32 array, 1 = bf16 bit patterns. */
static double load_w(const void *base, int wdtype, int64_t i) {
  if (wdtype == 1) return (double)bf16_bits_to_float(((const uint16_t *)base)[i]);
  return (double)((const float *)base)[i];
}

/* ------------------------------------------------------------------ */
/* OCP MX: E4M3 (FN) element format and E8M0 block scale               */
/* ------------------------------------------------------------------ */

/* E4M3 FN value of a code (OCP MX v1.0, element format table): exponent
 * bias 7, three mantissa bits, subnormals at exponent field 0, no
 * infinities, S.1111.111 is NaN.  Returns NaN for the two NaN codes. */
ORC_EXPORT double oracle_e4m3_decode(uint8_t code) {
  int sign = (code >> 7) & 1;
  int ef = (code >> 3) & 15;
  int mf = code & 7;
  double mag;
  if (ef == 15 && mf == 7) return NAN;
  if (ef == 0)
    mag = ldexp((double)mf, -9);             /* m/8 * 2^(1-7) */
  else
    mag = ldexp(1.0 + mf / 8.0, ef - 7);
  return sign ? -mag : mag;
}

/* Round v to E4M3 FN, round-to-nearest-even, saturating to +-448.  The
 * sign bit is copied from v (so -0.0 and tiny negatives give 0x80). */
ORC_EXPORT uint8_t oracle_e4m3_encode(double v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9 */
    double q = nearbyint(ldexp(a, 9));     /* exact scaling, RNE */
    return sign | (uint8_t)q;                /* q == 8 is the smallest normal */
  }
  int e2;
  double f = frexp(a, &e2);                  /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;                            /* a = (2f) * 2^e, 2f in [1, 2) */
  double m = nearbyint((2.0 * f - 1.0) * 8.0);
  if (m == 8.0) { m = 0.0; e += 1; }
  if (e > 8 || (e == 8 && m == 7.0)) return sign | 0x7E;   /* above 448 */
  return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* Quantise nblk blocks of 32 fp32 values (contiguous) to MX-fp8.
 * Scale rule (OCP MX v1.0, conversion section): X = floor(log2(max|v|)) -
 * emax_elem with emax_elem = 8 for E4M3, clamped to the E8M0 range
 * [-127, 127]; an all-zero block takes X = -127.  Element i is the E4M3
 * rounding of v_i / 2^X.  The scale byte is X + 127. */
ORC_EXPORT int oracle_mxq(int64_t nblk, const float *v, uint8_t *q, uint8_t *scale) {
  if (nblk < 0 || (nblk > 0 && (!v || !q || !scale))) return -1;
  for (int64_t b = 0; b < nblk; ++b) {
    const float *vb = v + b * 32;
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double a = fabs((double)vb[i]);
      if (a > amax) amax = a;
    }
    int X;
    if (amax == 0.0) {
      X = -127;
    } else {
      int e2;
      frexp(amax, &e2);
      X = (e2 - 1) - 8;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    scale[b] = (uint8_t)(X + 127);
    for (int i = 0; i < 32; ++i) q[b * 32 + i] = oracle_e4m3_encode(ldexp((double)vb[i], -X));
  }
  return 0;
}

/* Dequantise: v = E4M3(q) * 2^(scale - 127). */
ORC_EXPORT int oracle_mx_dequant(int64_t nblk, const uint8_t *q, const uint8_t *scale, float *v) {
  if (nblk < 0 || (nblk > 0 && (!v || !q || !scale))) return -1;
  for (int64_t b = 0; b < nblk; ++b)
    for (int i = 0; i < 32; ++i)
      v[b * 32 + i] = (float)ldexp(oracle_e4m3_decode(q[b * 32 + i]), (int)scale[b] - 127);
  return 0;
}

/* Round a row of n fp32 values through MX-fp8 (quantise then dequantise). */
static void mx_roundtrip_row(int64_t n, const float *in, float *out) {
  uint8_t q[32], s;
  for (int64_t b = 0; b < n / 32; ++b) {
    oracle_mxq(1, in + b * 32, q, &s);
    oracle_mx_dequant(1, q, &s, out + b * 32);
  }
}

/* ------------------------------------------------------------------ */
/* OCP MX: E2M1 (FP4) element format, for the W4A8 expert weights       */
/* ------------------------------------------------------------------ */

/* E2M1 value of a 4-bit code (OCP MX v1.0, element format table): bit 3 is
 * the sign, bits 2-1 the exponent field (bias 1), bit 0 the mantissa; an
 * exponent field of 0 is subnormal (m/2 * 2^0).  No infinities, no NaN.  The
 * eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4 and 6. */
ORC_EXPORT double oracle_e2m1_decode(uint8_t code) {
  int sign = (code >> 3) & 1;
  int ef = (code >> 1) & 3;
  int mf = code & 1;
  double mag = (ef == 0) ? 0.5 * mf : ldexp(1.0 + 0.5 * mf, ef - 1);
  return sign ? -mag : mag;
}

/* Round v to E2M1: the nearest of the eight magnitudes; a value exactly
 * between two of them goes to the one whose code has mantissa bit 0 (round
 * to nearest even); values beyond 6 become 6 (saturation, the nearest
 * magnitude).  The sign bit is copied from v. */
ORC_EXPORT uint8_t oracle_e2m1_encode(double v) {
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  double a = fabs(v);
  /* saturate first: far above 6 every distance rounds to the same double */
  if (a >= 6.0) return sign | 0x7;
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(a - oracle_e2m1_decode((uint8_t)c));
    /* codes ascend in magnitude, so a tie is between c - 1 and c */
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return sign | (uint8_t)best;
}

/* Quantise nblk blocks of 32 fp32 values to MXFP4, one code per output
 * byte (values 0..15).  Scale rule as for MX-fp8 with E2M1's largest normal
 * exponent: X = floor(log2(max|v|)) - 2 (6 = 1.5 * 2^2), clamped to
 * [-127, 127]; an all-zero block takes X = -127.  Element i is the E2M1
 * rounding of v_i / 2^X; the scale byte is X + 127. */
ORC_EXPORT int oracle_mxq4(int64_t nblk, const float *v, uint8_t *q, uint8_t *scale) {
  if (nblk < 0 || (nblk > 0 && (!v || !q || !scale))) return -1;
  for (int64_t b = 0; b < nblk; ++b) {
    const float *vb = v + b * 32;
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double a = fabs((double)vb[i]);
      if (a > amax) amax = a;
    }
    int X;
    if (amax == 0.0) {
      X = -127;
    } else {
      int e2;
      frexp(amax, &e2);
      X = (e2 - 1) - 2;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    scale[b] = (uint8_t)(X + 127);
    for (int i = 0; i < 32; ++i) q[b * 32 + i] = oracle_e2m1_encode(ldexp((double)vb[i], -X));
  }
  return 0;
}

/* Dequantise MXFP4: v = E2M1(q) * 2^(scale - 127). */
ORC_EXPORT int oracle_mx4_dequant(int64_t nblk, const uint8_t *q, const uint8_t *scale, float *v) {
  if (nblk < 0 || (nblk > 0 && (!v || !q || !scale))) return -1;
  for (int64_t b = 0; b < nblk; ++b)
    for (int i = 0; i < 32; ++i)
      v[b * 32 + i] =
          (float)ldexp(oracle_e2m1_decode(q[b * 32 + i] & 0xF), (int)scale[b] - 127);
  return 0;
}

/* Round a row of n fp32 values through MXFP4. */
static void mx4_roundtrip_row(int64_t n, const float *in, float *out) {
  uint8_t q[32], s;
  for (int64_t b = 0; b < n / 32; ++b) {
    oracle_mxq4(1, in + b * 32, q, &s);
    oracle_mx4_dequant(1, q, &s, out + b * 32);
  }
}

/* ------------------------------------------------------------------ */
/* Step 1-4: gating (router GEMM, sigmoid, top-k, route_norm, scale)   */
/* ------------------------------------------------------------------ */

/* Router logits z[t,e] = fp32( sum_h x[t,h] * W_r[e,h] + b[e] ).
 * x: [T,H] fp32, W_r: [E,H] fp32, bias: [E] or NULL. */
ORC_EXPORT int oracle_router_logits(int64_t T, int64_t H, int64_t E, const float *x,
                                    const float *Wr, const float *bias, float *z) {
  if (T < 0 || H <= 0 || E <= 0 || (T > 0 && (!x || !Wr || !z))) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += (double)x[t * H + h] * (double)Wr[e * H + h];
      if (bias) acc += (double)bias[e];
      z[t * E + e] = (float)acc;
    }
  }
  return 0;
}

/* Sigmoid score s = fp32( 1 / (1 + exp(-z)) ), evaluated in double. */
static float sigmoid_score(float z) { return (float)(1.0 / (1.0 + exp(-(double)z))); }

/* True when expert a ranks before expert b: higher score first, and the
 * lower expert index first among equal scores. */
static int ranks_before(float sa, int a, float sb, int b) {
  if (sa != sb) return sa > sb;
  return a < b;
}

/* Step 4 for one token: w[j] = fp32( rho * s[idx_j] / sum_j s[idx_j] ) with
 * the denominator summed in double over j ascending (route_norm = 1), or
 * fp32( rho * s[idx_j] ) (route_norm = 0).  route_norm and
 * router_scaling_factor: Hy3 guide, section 1. */
static void route_weights_row(int64_t k, const float *s, const int32_t *idx, float rho,
                              int route_norm, float *w) {
  double den = 0.0;
  for (int64_t j = 0; j < k; ++j) den += (double)s[idx[j]];
  for (int64_t j = 0; j < k; ++j) {
    double sj = (double)s[idx[j]];
    double wj = route_norm ? (double)rho * sj / den : (double)rho * sj;
    w[j] = (float)wj;
  }
}

/* Step 4 on selections given from outside (a selection another gating
 * produced, e.g. one that differs from this oracle's only by near-equal
 * scores): scores [T,E] are this oracle's sigmoid scores, idx [T,k] the
 * selected experts.  Returns -1 unless every row holds k distinct experts
 * in [0, E). */
ORC_EXPORT int oracle_route_weights(int64_t T, int64_t E, int64_t k, const float *scores,
                                    const int32_t *idx, float rho, int route_norm, float *w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  if (T == 0) return 0;
  if (!scores || !idx || !w) return -1;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = idx[t * k + j];
      if (e < 0 || e >= E) return -1;
      for (int64_t i = 0; i < j; ++i)
        if (idx[t * k + i] == e) return -1;
    }
  for (int64_t t = 0; t < T; ++t)
    route_weights_row(k, scores + t * E, idx + t * k, rho, route_norm, w + t * k);
  return 0;
}

/* Full gating for T tokens.
 *   topk_idx [T,k] int32 : selected experts, best first
 *   topk_w   [T,k] fp32  : rho * s / sum(selected s)   (route_norm = 1)
 *                          rho * s                      (route_norm = 0)
 *   scores   [T,E] fp32  : optional, the sigmoid scores
 *   gap      [T]   fp32  : optional, s(k-th) - s(k+1-th), +inf when k == E
 * rho is the router scaling factor, applied to the routed weights only. */
ORC_EXPORT int oracle_route(int64_t T, int64_t H, int64_t E, int64_t k, const float *x,
                            const float *Wr, const float *bias, float rho, int route_norm,
                            int32_t *topk_idx, float *topk_w, float *scores, float *gap) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E) return -1;
  if (T == 0) return 0;
  if (!x || !Wr || !topk_idx || !topk_w) return -1;
  float *z = (float *)malloc(sizeof(float) * (size_t)(T * E));
  if (!z) return -1;
  oracle_router_logits(T, H, E, x, Wr, bias, z);
  int rc = 0;
#pragma omp parallel
  {
    float *s = (float *)malloc(sizeof(float) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    if (!s || !taken) {
#pragma omp atomic write
      rc = -1;
    } else {
#pragma omp for schedule(static)
      for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
          s[e] = sigmoid_score(z[t * E + e]);
          taken[e] = 0;
          if (scores) scores[t * E + e] = s[e];
        }
        /* k rounds of "pick the best remaining expert". */
        for (int64_t j = 0; j < k; ++j) {
          int best = -1;
          for (int e = 0; e < (int)E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || ranks_before(s[e], e, s[best], best)) best = e;
          }
          taken[best] = 1;
          topk_idx[t * k + j] = best;
        }
        if (gap) {
          if (k == E) {
            gap[t] = INFINITY;
          } else {
            int next = -1;
            for (int e = 0; e < (int)E; ++e) {
              if (taken[e]) continue;
              if (next < 0 || ranks_before(s[e], e, s[next], next)) next = e;
            }
            gap[t] = s[topk_idx[t * k + k - 1]] - s[next];
          }
        }
        route_weights_row(k, s, topk_idx + t * k, rho, route_norm, topk_w + t * k);
      }
    }
    free(s);
    free(taken);
  }
  free(z);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Step 5: InitRouting -- group (token, slot) pairs by expert          */
/* ------------------------------------------------------------------ */

/* Pairs are numbered f = t*k + j.  counts[e] is the number of pairs routed
 * to e; offsets is the exclusive prefix sum (offsets[E] = T*k).  Walking f in
 * ascending order, pair f goes to row r = offsets[e] + (number of earlier
 * pairs with the same expert): sorted_src[r] = f and dest[f] = r.  Rows inside
 * one expert's segment are therefore in ascending token order.
 * Returns -1 if an index is outside [0, E). */
ORC_EXPORT int oracle_permute(int64_t T, int64_t E, int64_t k, const int32_t *topk_idx,
                              int32_t *counts, int32_t *offsets, int32_t *sorted_src,
                              int32_t *dest) {
  if (T < 0 || E <= 0 || k <= 0 || !counts || !offsets) return -1;
  int64_t P = T * k;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < P; ++f) {
    int32_t e = topk_idx[f];
    if (e < 0 || e >= E) return -1;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *cursor = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!cursor) return -1;
  for (int64_t f = 0; f < P; ++f) {
    int32_t e = topk_idx[f];
    int32_t r = offsets[e] + cursor[e]++;
    sorted_src[r] = (int32_t)f;
    dest[f] = r;
  }
  free(cursor);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Step 6-8: one expert's SwiGLU FFN over a set of rows                */
/* ------------------------------------------------------------------ */

/* For M input rows xr [M,H] (fp32) and one expert whose weights are
 *   Wg [I,H], Wu [I,H], Wd [H,I]   (wdtype 0 = fp32, 1 = bf16 bits),
 * compute
 *   g_i = sum_h x~_h Wg[i,h],  u_i = sum_h x~_h Wu[i,h]     (double)
 *   h_i = fp32( silu(g_i) * u_i ),  silu(g) = g / (1 + exp(-g))
 *   y_n = fp32( sum_i h~_i Wd[n,i] )
 * where x~ = x and h~ = h, except with mx = 1 (MX-fp8, W8A8): x~ = MXQ(x)
 * along H and h~ = MXQ(h) along I, and the weights are MXQ'd along their
 * reduction axis (each Wg/Wu row along H, each Wd row along I) before use;
 * and with mx = 2 (W4A8: MXFP4 weights, MX-fp8 activations) the same, except
 * that the weights are rounded through MXFP4 instead.
 * h_out [M,I] (optional) receives h before any MX rounding; y [M,H]. */
ORC_EXPORT int oracle_swiglu_rows(int64_t M, int64_t H, int64_t I, const float *xr, int wdtype,
                                  const void *Wg, const void *Wu, const void *Wd, int mx,
                                  float *h_out, float *y) {
  if (M < 0 || H <= 0 || I <= 0 || (wdtype != 0 && wdtype != 1)) return -1;
  if (mx < 0 || mx > 2 || (mx && (wdtype != 0 || H % 32 || I % 32))) return -1;
  if (M == 0) return 0;
  if (!xr || !Wg || !Wu || !Wd || !y) return -1;

  /* MX: pre-round the weights once (dequantised fp32 copies). */
  void (*wround)(int64_t, const float *, float *) = (mx == 2) ? mx4_roundtrip_row
                                                               : mx_roundtrip_row;
  float *wg_q = NULL, *wu_q = NULL, *wd_q = NULL;
  const void *g_src = Wg, *u_src = Wu, *d_src = Wd;
  if (mx) {
    wg_q = (float *)malloc(sizeof(float) * (size_t)(I * H));
    wu_q = (float *)malloc(sizeof(float) * (size_t)(I * H));
    wd_q = (float *)malloc(sizeof(float) * (size_t)(H * I));
    if (!wg_q || !wu_q || !wd_q) { free(wg_q); free(wu_q); free(wd_q); return -1; }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
      wround(H, (const float *)Wg + i * H, wg_q + i * H);
      wround(H, (const float *)Wu + i * H, wu_q + i * H);
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < H; ++n) wround(I, (const float *)Wd + n * I, wd_q + n * I);
    g_src = wg_q; u_src = wu_q; d_src = wd_q;
  }

  /* Rows one after another; inside a row every output element is one
   * thread's fixed-order sum, so results do not depend on the thread count. */
  int rc = 0;
  float *xt = (float *)malloc(sizeof(float) * (size_t)H);
  float *hr = (float *)malloc(sizeof(float) * (size_t)I);
  float *ht = (float *)malloc(sizeof(float) * (size_t)I);
  if (!xt || !hr || !ht) {
    rc = -1;
  } else {
    const int gdt = mx ? 0 : wdtype;
    for (int64_t m = 0; m < M; ++m) {
      if (mx) mx_roundtrip_row(H, xr + m * H, xt);
      else memcpy(xt, xr + m * H, sizeof(float) * (size_t)H);
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
          g += (double)xt[h] * load_w(g_src, gdt, i * H + h);
          u += (double)xt[h] * load_w(u_src, gdt, i * H + h);
        }
        double silu = g / (1.0 + exp(-g));
        hr[i] = (float)(silu * u);
      }
      if (h_out) memcpy(h_out + m * I, hr, sizeof(float) * (size_t)I);
      if (mx) mx_roundtrip_row(I, hr, ht);
      else memcpy(ht, hr, sizeof(float) * (size_t)I);
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i) acc += (double)ht[i] * load_w(d_src, gdt, n * I + i);
        y[m * H + n] = (float)acc;
      }
    }
  }
  free(xt);
  free(hr);
  free(ht);
  free(wg_q);
  free(wu_q);
  free(wd_q);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Static per-tensor FP8 (W8A8 with one scale per tensor)               */
/* ------------------------------------------------------------------ */

/* Per-tensor scale of a weight matrix: s = fp32(max|w| / 448), so the
 * largest element maps to E4M3's largest normal; an all-zero tensor takes
 * s = 1.  (FP8 checkpoints of the Hy3 and Hy4 families carry one such scale
 * per weight tensor; the pages name the format only.) */
ORC_EXPORT float oracle_fp8_tensor_scale(int64_t n, const float *w) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(w[i]);
    if (a > amax) amax = a;
  }
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

/* E4M3 codes of v under a per-tensor scale s: code = E4M3(fp32(v / s)),
 * round to nearest even, saturating. */
ORC_EXPORT int oracle_fp8_quantize(int64_t n, const float *v, float s, uint8_t *q) {
  if (n < 0 || (n > 0 && (!v || !q)) || !(s > 0.0f)) return -1;
  for (int64_t i = 0; i < n; ++i) {
    float scaled = v[i] / s;
    q[i] = oracle_e4m3_encode((double)scaled);
  }
  return 0;
}

/* Dequantised values E4M3(q) * s, in double (exact: at most 4 + 24
 * significant bits). */
static void fp8_dequant_d(int64_t n, const float *v, float s, double *out) {
  for (int64_t i = 0; i < n; ++i) {
    float scaled = v[i] / s;
    out[i] = oracle_e4m3_decode(oracle_e4m3_encode((double)scaled)) * (double)s;
  }
}

/* One expert's SwiGLU FFN with static per-tensor FP8: each weight matrix
 * (fp32 masters Wg [I,H], Wu [I,H], Wd [H,I]) quantised with its own
 * oracle_fp8_tensor_scale, the rows x [M,H] with the static activation
 * scale s_x, and h with the static scale s_h:
 *   g_i = sum_h x~_h Wg~[i,h],  u_i = sum_h x~_h Wu~[i,h]      (double)
 *   h_i = fp32( silu(g_i) * u_i )
 *   y_n = fp32( sum_i h~_i Wd~[n,i] )
 * where a~ is the dequantised E4M3 value of a.  h_out [M,I] (optional)
 * receives h before quantisation; y [M,H]. */
ORC_EXPORT int oracle_swiglu_rows_fp8(int64_t M, int64_t H, int64_t I, const float *xr,
                                      const float *Wg, const float *Wu, const float *Wd, float s_x,
                                      float s_h, float *h_out, float *y) {
  if (M < 0 || H <= 0 || I <= 0 || !(s_x > 0.0f) || !(s_h > 0.0f)) return -1;
  if (M == 0) return 0;
  if (!xr || !Wg || !Wu || !Wd || !y) return -1;
  double *wg = (double *)malloc(sizeof(double) * (size_t)(I * H));
  double *wu = (double *)malloc(sizeof(double) * (size_t)(I * H));
  double *wd = (double *)malloc(sizeof(double) * (size_t)(H * I));
  double *xt = (double *)malloc(sizeof(double) * (size_t)H);
  float *hr = (float *)malloc(sizeof(float) * (size_t)I);
  double *ht = (double *)malloc(sizeof(double) * (size_t)I);
  int rc = -1;
  if (!wg || !wu || !wd || !xt || !hr || !ht) goto done;
  fp8_dequant_d(I * H, Wg, oracle_fp8_tensor_scale(I * H, Wg), wg);
  fp8_dequant_d(I * H, Wu, oracle_fp8_tensor_scale(I * H, Wu), wu);
  fp8_dequant_d(H * I, Wd, oracle_fp8_tensor_scale(H * I, Wd), wd);
  for (int64_t m = 0; m < M; ++m) {
    fp8_dequant_d(H, xr + m * H, s_x, xt);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
      double g = 0.0, u = 0.0;
      for (int64_t h = 0; h < H; ++h) {
        g += xt[h] * wg[i * H + h];
        u += xt[h] * wu[i * H + h];
      }
      hr[i] = (float)(g / (1.0 + exp(-g)) * u);
    }
    if (h_out) memcpy(h_out + m * I, hr, sizeof(float) * (size_t)I);
    fp8_dequant_d(I, hr, s_h, ht);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int64_t i = 0; i < I; ++i) acc += ht[i] * wd[n * I + i];
      y[m * H + n] = (float)acc;
    }
  }
  rc = 0;
done:
  free(wg);
  free(wu);
  free(wd);
  free(xt);
  free(hr);
  free(ht);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Step 9: FinalizeRouting -- weighted combine plus the shared expert  */
/* ------------------------------------------------------------------ */

/* out[t,n] = fp32( (sum_{j<k} w[t,j] * y[dest[t*k+j], n]) + zsh[t,n] ),
 * j ascending, in double.  zsh may be NULL (no shared expert). */
ORC_EXPORT int oracle_combine(int64_t T, int64_t H, int64_t k, const float *y, const int32_t *dest,
                              const float *topk_w, const float *zsh, float *out) {
  if (T < 0 || H <= 0 || k <= 0) return -1;
  if (T == 0) return 0;
  if (!y || !dest || !topk_w || !out) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j)
        acc += (double)topk_w[t * k + j] * (double)y[(int64_t)dest[t * k + j] * H + n];
      if (zsh) acc += (double)zsh[t * H + n];
      out[t * H + n] = (float)acc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* The whole layer, in the pages' order                                */
/* ------------------------------------------------------------------ */

/* Gating -> InitRouting -> per-expert SwiGLU FFN over each expert's rows ->
 * FinalizeRouting -> + shared expert.
 *   x [T,H] fp32 (bf16 inputs are passed already widened, which is exact)
 *   Wr [E,H] fp32, bias [E] or NULL
 *   Wg, Wu [E,I,H]; Wd [E,H,I]    (wdtype 0 fp32 / 1 bf16 bits; fp32 if mx)
 *   Sg, Su [Is,H]; Sd [H,Is]      (shared expert; NULL or Is == 0: none)
 *   mx: 0 none, 1 MX-fp8 experts (W8A8), 2 W4A8: MXFP4 routed experts with
 *       MX-fp8 activations, and an MX-fp8 (W8A8) shared expert -- the hybrid
 *       recipe of the Hy3 guide, section 8.2 (routed W4A8, shared W8A8)
 * Outputs: out [T,H]; optional intermediates (any may be NULL):
 *   topk_idx [T,k], topk_w [T,k], counts [E], offsets [E+1],
 *   sorted_src [T*k], dest [T*k], h [T*k, I] (pre-MX), y [T*k, H],
 *   zsh [T,H]. */
ORC_EXPORT int oracle_layer_forward(int64_t T, int64_t H, int64_t E, int64_t k, int64_t I,
                                    int64_t Is, float rho, int route_norm, const float *x,
                                    const float *Wr, const float *bias, int wdtype, const void *Wg,
                                    const void *Wu, const void *Wd, const void *Sg, const void *Su,
                                    const void *Sd, int mx, float *out, int32_t *topk_idx_o,
                                    float *topk_w_o, int32_t *counts_o, int32_t *offsets_o,
                                    int32_t *sorted_src_o, int32_t *dest_o, float *h_o, float *y_o,
                                    float *zsh_o) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E || I <= 0 || Is < 0) return -1;
  if (T == 0) return 0;
  if (!x || !Wr || !Wg || !Wu || !Wd || !out) return -1;
  int64_t P = T * k;
  size_t esz = (mx || wdtype == 0) ? sizeof(float) : sizeof(uint16_t);
  int rc = -1;
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
  float *w = (float *)malloc(sizeof(float) * (size_t)P);
  int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t *src = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
  int32_t *dest = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
  float *xrows = (float *)malloc(sizeof(float) * (size_t)(P * H));
  float *y = (float *)malloc(sizeof(float) * (size_t)(P * H));
  float *h = h_o ? h_o : NULL;
  float *zsh = NULL;
  int have_shared = (Is > 0 && Sg && Su && Sd);
  if (have_shared) zsh = (float *)malloc(sizeof(float) * (size_t)(T * H));
  if (!idx || !w || !counts || !offsets || !src || !dest || !xrows || !y ||
      (have_shared && !zsh))
    goto done;

  /* Gating. */
  if (oracle_route(T, H, E, k, x, Wr, bias, rho, route_norm, idx, w, NULL, NULL)) goto done;
  /* InitRouting. */
  if (oracle_permute(T, E, k, idx, counts, offsets, src, dest)) goto done;
  /* Gather each permuted row's token activations. */
  for (int64_t r = 0; r < P; ++r)
    memcpy(xrows + r * H, x + (int64_t)(src[r] / k) * H, sizeof(float) * (size_t)H);
  /* Grouped FFN: expert e owns rows [offsets[e], offsets[e+1]). */
  for (int64_t e = 0; e < E; ++e) {
    int64_t r0 = offsets[e], m = counts[e];
    if (m == 0) continue;
    const char *g = (const char *)Wg + (size_t)(e * I * H) * esz;
    const char *u = (const char *)Wu + (size_t)(e * I * H) * esz;
    const char *d = (const char *)Wd + (size_t)(e * H * I) * esz;
    if (oracle_swiglu_rows(m, H, I, xrows + r0 * H, wdtype, g, u, d, mx, h ? h + r0 * I : NULL,
                           y + r0 * H))
      goto done;
  }
  /* Shared expert on every token. */
  if (have_shared &&
      oracle_swiglu_rows(T, H, Is, x, wdtype, Sg, Su, Sd, mx == 2 ? 1 : mx, NULL, zsh))
    goto done;
  /* FinalizeRouting + add. */
  if (oracle_combine(T, H, k, y, dest, w, zsh, out)) goto done;

  if (topk_idx_o) memcpy(topk_idx_o, idx, sizeof(int32_t) * (size_t)P);
  if (topk_w_o) memcpy(topk_w_o, w, sizeof(float) * (size_t)P);
  if (counts_o) memcpy(counts_o, counts, sizeof(int32_t) * (size_t)E);
  if (offsets_o) memcpy(offsets_o, offsets, sizeof(int32_t) * (size_t)(E + 1));
  if (sorted_src_o) memcpy(sorted_src_o, src, sizeof(int32_t) * (size_t)P);
  if (dest_o) memcpy(dest_o, dest, sizeof(int32_t) * (size_t)P);
  if (y_o) memcpy(y_o, y, sizeof(float) * (size_t)(P * H));
  if (zsh_o && have_shared) memcpy(zsh_o, zsh, sizeof(float) * (size_t)(T * H));
  rc = 0;
done:
  free(idx);
  free(w);
  free(counts);
  free(offsets);
  free(src);
  free(dest);
  free(xrows);
  free(y);
  free(zsh);
  return rc;
}
