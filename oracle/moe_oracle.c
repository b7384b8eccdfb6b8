/*
 * CPU oracle for the MXFP4 routed-expert MoE layer -- TEST INFRASTRUCTURE.
 *
 * Plain, slow and written to be checked by eye against the definition:
 *   - MXFP4 element: E2M1, 1 sign bit, 2 exponent bits, 1 mantissa bit; the 16
 *     codes form a fixed codebook (XFP blog, section "路线二：硬件格式（NVFP4 /
 *     MXFP4）").  Exponent bias 1, e = 0 is the subnormal row, and no code is
 *     reserved for inf or NaN, so the largest magnitude is 6.
 *   - MXFP4 block: 32 elements along K share one 8-bit power-of-two exponent
 *     (UE8M0, bias 127, 0xFF = NaN), as the OCP Microscaling format that the
 *     same section names defines it.
 *   - Storage: two codes per byte, so a packed row is K/2 bytes, with a separate
 *     scale tensor beside the packed tensor (campaign page "glm53-mxfp4-mi355x",
 *     sections "A fused tensor with two dtypes in it" and "The model card and
 *     the metadata disagree").
 *   - Expert MLP: gate and up stacked into one weight whose output feeds the
 *     SwiGLU (TensorFold PR #1050, commit notes: a dense layer runs "[gate | up]"
 *     stacked), with the clamp the MI355X experts keep (model card
 *     "GLM-5.3-Flash-MXFP4", section "Verification compute and EAGLE").
 *   - Routing: top-k of the router's softmax with renormalised weights; only the
 *     experts the router picked are read (campaign page, section "A file is a
 *     census; a decode step is a sample").
 *   - Shared expert (optional): an MXFP4 MLP of the same shape that every token
 *     reads, packed codes with a scale tensor beside them (campaign page,
 *     section "The model card and the metadata disagree"), in the always-active
 *     set of the census formula (section "A file is a census; a decode step is
 *     a sample").  It enters the combine with weight 1 as one more slot per
 *     token, after the k routed ones.
 *   - Per-expert exclusions (optional): an expert kept in bf16 inside a fused
 *     buffer whose other experts are packed MXFP4, so the exclusion set is
 *     carried per expert (campaign page, section "A fused tensor with two
 *     dtypes in it").  Such an expert's contractions read its bf16 weights.
 *
 * Activation formats: bf16 (W4A16), or x and the SwiGLU output quantised per 32
 * along K to MXFP4 (A4) or MXFP8 with E4M3 elements (A8) before the contraction
 * that reads them.
 *
 * Precision: x is bf16, every contraction accumulates in fp32 in increasing K
 * order from +0.0f, the SwiGLU output is rounded to bf16, the combine adds
 * w*y in fp32 in increasing slot order, and the output is rounded to bf16.
 * Build with -ffp-contract=off and no fast-math so each step rounds as written.
 *
 * Nothing here is shared with the GPU library.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* malloc size that is never zero */
static size_t nz(int64_t n) { return n > 0 ? (size_t)n : 1; }

/* ---------------------------------------------------------------- codec */

/* E2M1 value of a 4-bit code: bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 * mantissa.  e = 0 holds the subnormals 0 and 0.5. */
double orc_e2m1_value(int32_t code) {
  int s = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double mag;
  if (e == 0)
    mag = 0.5 * m;
  else
    mag = ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* UE8M0 scale byte: 2^(S-127); 0xFF encodes NaN. */
double orc_ue8m0_value(int32_t s) {
  if (s == 255) return NAN;
  return ldexp(1.0, s - 127);
}

static int code_at(const uint8_t* row_codes, int64_t k) {
  uint8_t byte = row_codes[k / 2];
  return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

void orc_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                 float* out) {
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* rc = codes + r * (K / 2);
    const uint8_t* rs = scales + r * (K / 32);
    for (int64_t k = 0; k < K; ++k) {
      double v = orc_e2m1_value(code_at(rc, k)) * orc_ue8m0_value(rs[k / 32]);
      out[r * K + k] = (float)v;
    }
  }
}

/* ---------------------------------------------------------------- bf16 */

float orc_f32_from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round an fp32 value to the nearer of its two bf16 neighbours; on a tie take
 * the one whose last significand bit is 0.  Past the largest finite bf16 the
 * upper neighbour is 2^128, i.e. infinity.  NaN becomes the quiet NaN with the
 * input's sign. */
uint16_t orc_bf16_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16 & 0x8000u) | 0x7FC0u);
  if (isinf(f)) return (uint16_t)(u >> 16);
  uint16_t lo = (uint16_t)(u >> 16); /* truncation toward zero */
  if ((u & 0xFFFFu) == 0) return lo; /* already a bf16 value */
  uint16_t hi = (uint16_t)(lo + 1);  /* next bf16 magnitude away from zero */
  double vlo = (double)orc_f32_from_bf16(lo);
  double vhi;
  if ((hi & 0x7FFFu) == 0x7F80u)
    vhi = copysign(ldexp(1.0, 128), (double)f);
  else
    vhi = (double)orc_f32_from_bf16(hi);
  double dlo = fabs((double)f - vlo);
  double dhi = fabs(vhi - (double)f);
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1u) ? hi : lo;
}

void orc_bf16_round_array(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(in[i]);
}

/* ---------------------------------------------------------------- quantiser */

/* Round a magnitude a >= 0 to the E2M1 grid: the grid step is 0.5 below 1 and
 * 2^(floor(log2 a) - 1) above (one mantissa bit), round to the nearest multiple
 * of the step with ties to the even multiple (the even code), then saturate at
 * 6.  Returns the 3-bit magnitude code. */
static int e2m1_round_magnitude(double a) {
  double step;
  if (a < 1.0) {
    step = 0.5;
  } else {
    int E;
    frexp(a, &E); /* a = f * 2^E, f in [0.5, 1): floor(log2 a) = E - 1 */
    step = ldexp(1.0, (E - 1) - 1);
  }
  double q = rint(a / step) * step; /* a / step is exact: step is a power of two */
  if (q > 6.0) q = 6.0;
  for (int c = 0; c < 8; ++c)
    if (orc_e2m1_value(c) == q) return c;
  return -1; /* unreachable */
}

/* One 32-element block, OCP rule: shared exponent floor(log2 amax) - 2 (2 is the
 * largest E2M1 exponent), biased by 127 and clamped to [0, 254]; each element is
 * divided by the shared power of two and rounded to E2M1.  A block holding NaN
 * or infinity gets the NaN scale 0xFF and zero codes; an all-zero block gets
 * scale 0 and keeps each element's sign bit. */
static void quantize_block(const double* v, uint8_t* codes4, uint8_t* scale) {
  int nonfinite = 0;
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) {
    if (!isfinite(v[i]))
      nonfinite = 1;
    else if (fabs(v[i]) > amax)
      amax = fabs(v[i]);
  }
  if (nonfinite) {
    *scale = 255;
    for (int i = 0; i < 32; ++i) codes4[i] = 0;
    return;
  }
  if (amax == 0.0) {
    *scale = 0;
    for (int i = 0; i < 32; ++i) codes4[i] = signbit(v[i]) ? 8 : 0;
    return;
  }
  int E;
  frexp(amax, &E);
  int s = (E - 1) - 2 + 127;
  if (s < 0) s = 0;
  if (s > 254) s = 254;
  *scale = (uint8_t)s;
  for (int i = 0; i < 32; ++i) {
    double r = ldexp(v[i], 127 - s); /* exact in fp64 */
    int mag = e2m1_round_magnitude(fabs(r));
    codes4[i] = (uint8_t)((signbit(v[i]) ? 8 : 0) | mag);
  }
}

/* The quantisers below treat every row on its own; with many rows they are
 * spread over OpenMP threads (the same arithmetic on each row). */
void orc_quantize_f64(const double* v, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static) if (rows > 64)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < K / 32; ++b) {
      uint8_t c4[32];
      quantize_block(v + r * K + b * 32, c4, scales + r * (K / 32) + b);
      for (int i = 0; i < 32; i += 2)
        codes[r * (K / 2) + b * 16 + i / 2] = (uint8_t)(c4[i] | (c4[i + 1] << 4));
    }
  }
}

void orc_quantize_f32(const float* v, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static) if (rows > 64)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[32];
    for (int64_t b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i) blk[i] = (double)v[r * K + b * 32 + i];
      uint8_t c4[32];
      quantize_block(blk, c4, scales + r * (K / 32) + b);
      for (int i = 0; i < 32; i += 2)
        codes[r * (K / 2) + b * 16 + i / 2] = (uint8_t)(c4[i] | (c4[i + 1] << 4));
    }
  }
}

void orc_quantize_bf16(const uint16_t* v, int64_t rows, int64_t K, uint8_t* codes,
                       uint8_t* scales) {
#pragma omp parallel for schedule(static) if (rows > 64)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[32];
    for (int64_t b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i) blk[i] = (double)orc_f32_from_bf16(v[r * K + b * 32 + i]);
      uint8_t c4[32];
      quantize_block(blk, c4, scales + r * (K / 32) + b);
      for (int i = 0; i < 32; i += 2)
        codes[r * (K / 2) + b * 16 + i / 2] = (uint8_t)(c4[i] | (c4[i + 1] << 4));
    }
  }
}

/* ---------------------------------------------------------------- router */

/* Per token: softmax over all E_global logits in fp64, take the k largest
 * probabilities (equal probabilities: lower expert id first), then divide each
 * pick by the sum of the k picks and round once to fp32.  Returns -1 if a logit
 * is NaN (the routing of such a token is not defined). */
int orc_route(const float* logits, int64_t T, int64_t E, int32_t k, int32_t* ids, float* w) {
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  int status = 0;
  for (int64_t t = 0; t < T && status == 0; ++t) {
    const float* l = logits + t * E;
    double m = -INFINITY;
    for (int64_t e = 0; e < E; ++e) {
      if (isnan(l[e])) status = -1;
      if ((double)l[e] > m) m = (double)l[e];
    }
    if (status) break;
    double z = 0.0;
    for (int64_t e = 0; e < E; ++e) {
      p[e] = exp((double)l[e] - m);
      z += p[e];
    }
    for (int64_t e = 0; e < E; ++e) p[e] = p[e] / z;
    memset(taken, 0, (size_t)E);
    double sel_sum = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || p[e] > p[best]) best = e; /* strict '>' keeps the lower id on ties */
      }
      taken[best] = 1;
      ids[t * k + j] = (int32_t)best;
      sel_sum += p[best];
    }
    for (int32_t j = 0; j < k; ++j) w[t * k + j] = (float)(p[ids[t * k + j]] / sel_sum);
  }
  free(p);
  free(taken);
  return status;
}

/* ---------------------------------------------------------------- permutation */

/* Assignment slot s = t*k + j.  A slot is local when first_local <= id <
 * first_local + E_local; local expert e = id - first_local.  With shared_id >= 0
 * a slot whose id equals shared_id belongs to the shared expert, table entry
 * E_local (the tables then have E_local + 1 experts).  Counting sort that keeps
 * slot order within each expert. */
static int64_t local_expert(int32_t id, int64_t first_local, int64_t E_local, int64_t shared_id) {
  if (shared_id >= 0 && id == shared_id) return E_local;
  int64_t e = (int64_t)id - first_local;
  return (e >= 0 && e < E_local) ? e : -1;
}

int64_t orc_permute(const int32_t* ids, int64_t T, int32_t k, int64_t first_local, int64_t E_local,
                    int64_t shared_id, int32_t* counts, int32_t* offsets, int32_t* sorted,
                    int32_t* inv) {
  const int64_t n_slots = T * k;
  const int64_t n_exp = E_local + (shared_id >= 0 ? 1 : 0);
  for (int64_t e = 0; e < n_exp; ++e) counts[e] = 0;
  for (int64_t s = 0; s < n_slots; ++s) {
    int64_t e = local_expert(ids[s], first_local, E_local, shared_id);
    if (e >= 0) counts[e] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < n_exp; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)calloc((size_t)(n_exp > 0 ? n_exp : 1), sizeof(int32_t));
  for (int64_t s = 0; s < n_slots; ++s) {
    int64_t e = local_expert(ids[s], first_local, E_local, shared_id);
    if (e >= 0) {
      int32_t pos = offsets[e] + cursor[e];
      cursor[e] += 1;
      sorted[pos] = (int32_t)s;
      inv[s] = pos;
    } else {
      inv[s] = -1;
    }
  }
  free(cursor);
  return offsets[n_exp];
}

/* ---------------------------------------------------------------- SwiGLU */

/* gate clamped from above at L, up clamped to [-L, L]; a comparison with NaN is
 * false, so NaN passes through.  silu(g) = g * sigmoid(g), all in fp32. */
float orc_swiglu(float g, float u, float limit) {
  float gc = (g > limit) ? limit : g;
  float uc = (u > limit) ? limit : ((u < -limit) ? -limit : u);
  float sig = 1.0f / (1.0f + expf(-gc));
  return (gc * sig) * uc;
}

/* ---------------------------------------------------------------- MXFP8 */

/* E4M3 value of an 8-bit code: bit 7 sign, bits 6..3 exponent (bias 7), bits
 * 2..0 mantissa.  e = 0 holds the subnormals m/8 * 2^-6; exponent 15 with
 * mantissa 7 is NaN and there is no infinity, so the largest magnitude is
 * 1.75 * 2^8 = 448 (the OCP 8-bit floating-point format that the MX
 * specification pairs with the same UE8M0 block scale). */
double orc_e4m3_value(int32_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp(m / 8.0, -6);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Round a magnitude a >= 0 to the E4M3 grid: the step is 2^-9 below 2^-6 (the
 * subnormals) and 2^(floor(log2 a) - 3) above (three mantissa bits); nearest
 * multiple of the step, ties to the even multiple (the even code), saturating
 * at 448.  Returns the 7-bit magnitude code, read off the rounded value. */
static int e4m3_round_magnitude(double a) {
  double step;
  if (a < ldexp(1.0, -6)) {
    step = ldexp(1.0, -9);
  } else {
    int E;
    frexp(a, &E);
    step = ldexp(1.0, (E - 1) - 3);
  }
  double q = rint(a / step) * step;
  if (q > 448.0) q = 448.0;
  if (q < ldexp(1.0, -6)) return (int)(q / ldexp(1.0, -9)); /* 0..7: the mantissa */
  int E;
  double f = frexp(q, &E); /* q = f * 2^E, f in [0.5, 1): exponent E - 1 */
  int m = (int)((2.0 * f - 1.0) * 8.0);
  return ((E - 1 + 7) << 3) | m;
}

/* One 32-element block, OCP rule for FP8 elements: shared exponent
 * floor(log2 amax) - 8 (8 is the largest E4M3 exponent), biased by 127 and
 * clamped to [0, 254]; each element is divided by the shared power of two and
 * rounded to E4M3.  NaN/infinity and all-zero blocks as for MXFP4. */
static void quantize8_block(const double* v, uint8_t* codes, uint8_t* scale) {
  int nonfinite = 0;
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) {
    if (!isfinite(v[i]))
      nonfinite = 1;
    else if (fabs(v[i]) > amax)
      amax = fabs(v[i]);
  }
  if (nonfinite) {
    *scale = 255;
    for (int i = 0; i < 32; ++i) codes[i] = 0;
    return;
  }
  if (amax == 0.0) {
    *scale = 0;
    for (int i = 0; i < 32; ++i) codes[i] = signbit(v[i]) ? 0x80 : 0;
    return;
  }
  int E;
  frexp(amax, &E);
  int s = (E - 1) - 8 + 127;
  if (s < 0) s = 0;
  if (s > 254) s = 254;
  *scale = (uint8_t)s;
  for (int i = 0; i < 32; ++i) {
    double r = ldexp(v[i], 127 - s); /* exact in fp64 */
    codes[i] = (uint8_t)((signbit(v[i]) ? 0x80 : 0) | e4m3_round_magnitude(fabs(r)));
  }
}

void orc_quantize8_bf16(const uint16_t* v, int64_t rows, int64_t K, uint8_t* codes,
                        uint8_t* scales) {
#pragma omp parallel for schedule(static) if (rows > 64)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[32];
    for (int64_t b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i) blk[i] = (double)orc_f32_from_bf16(v[r * K + b * 32 + i]);
      quantize8_block(blk, codes + r * K + b * 32, scales + r * (K / 32) + b);
    }
  }
}

void orc_quantize8_f64(const double* v, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static) if (rows > 64)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < K / 32; ++b)
      quantize8_block(v + r * K + b * 32, codes + r * K + b * 32, scales + r * (K / 32) + b);
}

void orc_dequant8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                  float* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k)
      out[r * K + k] = (float)(orc_e4m3_value(codes[r * K + k]) * orc_ue8m0_value(scales[r * (K / 32) + k / 32]));
}

/* ---------------------------------------------------------------- layer */

int64_t orc_moe_forward(const orc_dims* d, const uint16_t* x, const float* logits,
                        const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2,
                        const uint8_t* w2s, const uint8_t* token_mask, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* inv,
                        uint16_t* act, uint8_t* xq, uint8_t* xs, uint8_t* actq, uint8_t* acts,
                        float* out32, uint16_t* out, int32_t nthreads) {
  const int64_t T = d->T, H = d->H, I = d->I, Eg = d->E_global, El = d->E_local;
  const int64_t f = d->first_local;
  const int32_t kr = d->top_k;               /* routed picks per token */
  const int32_t sh = d->shared ? 1 : 0;      /* shared expert present */
  const int32_t k = kr + sh;                 /* slots per token */
  const int64_t Ew = El + sh;                /* experts in the weight buffers and tables */
  if (T < 0 || H <= 0 || I <= 0 || H % 32 || I % 32 || El <= 0 || Eg <= 0 || f < 0 ||
      f + El > Eg || kr < 1 || kr > Eg || (d->a4 && d->a8) ||
      (d->given_actq && (!(d->a4 || d->a8) || !actq || !acts)))
    return -2;
  /* bf16 slot of each excluded expert (j-th excluded in expert order), else -1 */
  int64_t* xslot = (int64_t*)malloc(sizeof(int64_t) * (size_t)Ew);
  int64_t n_bf16 = 0;
  for (int64_t e = 0; e < Ew; ++e) xslot[e] = (d->bf16_expert && d->bf16_expert[e]) ? n_bf16++ : -1;
  if (n_bf16 > 0 && (!d->w13_bf16 || !d->w2_bf16)) {
    free(xslot);
    return -2;
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t S = T * k;
  int32_t* ids_ = ids ? ids : (int32_t*)malloc(sizeof(int32_t) * (size_t)(S ? S : 1));
  float* w_ = w ? w : (float*)malloc(sizeof(float) * (size_t)(S ? S : 1));
  int32_t* cnt_ = counts ? counts : (int32_t*)malloc(sizeof(int32_t) * (size_t)Ew);
  int32_t* off_ = offsets ? offsets : (int32_t*)malloc(sizeof(int32_t) * (size_t)(Ew + 1));
  int32_t* sor_ = sorted ? sorted : (int32_t*)malloc(sizeof(int32_t) * (size_t)(S ? S : 1));
  int32_t* inv_ = inv ? inv : (int32_t*)malloc(sizeof(int32_t) * (size_t)(S ? S : 1));

  /* the k routed picks of token t go to slots t*k + j, j < kr; the shared
   * expert (id E_global, outside the router's range) takes slot t*k + kr with
   * weight 1 */
  int32_t* rids = (int32_t*)malloc(sizeof(int32_t) * nz(T * kr));
  float* rw = (float*)malloc(sizeof(float) * nz(T * kr));
  int64_t status = orc_route(logits, T, Eg, kr, rids, rw);
  for (int64_t t = 0; t < T && status == 0; ++t) {
    for (int32_t j = 0; j < kr; ++j) {
      ids_[t * k + j] = rids[t * kr + j];
      w_[t * k + j] = rw[t * kr + j];
    }
    if (sh) {
      ids_[t * k + kr] = (int32_t)Eg;
      w_[t * k + kr] = 1.0f;
    }
  }
  free(rids);
  free(rw);
  int64_t N = 0;
  if (status == 0) N = orc_permute(ids_, T, k, f, El, sh ? Eg : -1, cnt_, off_, sor_, inv_);

  /* activations as fp32 values: x itself, or (A4) x quantised along H and
   * decoded again */
  float* xf = NULL;
  if (status == 0) {
    xf = (float*)malloc(sizeof(float) * nz(T * H));
    if (d->a4) {
      uint8_t* q = xq ? xq : (uint8_t*)malloc((size_t)(T * H / 2 ? T * H / 2 : 1));
      uint8_t* s = xs ? xs : (uint8_t*)malloc((size_t)(T * H / 32 ? T * H / 32 : 1));
      orc_quantize_bf16(x, T, H, q, s);
      orc_dequant(q, s, T, H, xf);
      if (!xq) free(q);
      if (!xs) free(s);
    } else if (d->a8) {
      uint8_t* q = xq ? xq : (uint8_t*)malloc(nz(T * H));
      uint8_t* s = xs ? xs : (uint8_t*)malloc(nz(T * H / 32));
      orc_quantize8_bf16(x, T, H, q, s);
      orc_dequant8(q, s, T, H, xf);
      if (!xq) free(q);
      if (!xs) free(s);
    } else {
      for (int64_t i = 0; i < T * H; ++i) xf[i] = orc_f32_from_bf16(x[i]);
    }
  }
  /* x as bf16 values, for the excluded experts of a quantised-activation layer */
  float* xb = xf;
  if (status == 0 && n_bf16 > 0 && (d->a4 || d->a8)) {
    xb = (float*)malloc(sizeof(float) * nz(T * H));
    for (int64_t i = 0; i < T * H; ++i) xb[i] = orc_f32_from_bf16(x[i]);
  }

  /* which sorted positions need expert work */
  int64_t* yrow = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N ? N : 1));
  int64_t n_work = 0;
  for (int64_t p = 0; p < N; ++p) {
    int64_t t = sor_[p] / k;
    yrow[p] = (!token_mask || token_mask[t]) ? n_work++ : -1;
  }
  float* y = (float*)malloc(sizeof(float) * nz(n_work * H));

  /* dequantised expert weights, K-major so each output keeps its K order */
  float* w13t = (float*)malloc(sizeof(float) * (size_t)(H * 2 * I));
  float* w2t = (float*)malloc(sizeof(float) * (size_t)(I * H));
  float* rowbuf = (float*)malloc(sizeof(float) * (size_t)(H > 2 * I ? H : 2 * I));

  for (int64_t e = 0; e < Ew && status == 0; ++e) {
    int any = 0;
    for (int64_t p = off_[e]; p < off_[e + 1]; ++p) any |= (yrow[p] >= 0);
    if (!any) continue;
    const int64_t xs_e = xslot[e];   /* >= 0: bf16 weights */
    const float* xin = xs_e >= 0 ? xb : xf;
    if (xs_e >= 0) {
      const uint16_t* b13 = d->w13_bf16 + xs_e * (2 * I) * H;
      const uint16_t* b2 = d->w2_bf16 + xs_e * H * I;
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < 2 * I; ++n)
        for (int64_t kk = 0; kk < H; ++kk) w13t[kk * (2 * I) + n] = orc_f32_from_bf16(b13[n * H + kk]);
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < H; ++n)
        for (int64_t i = 0; i < I; ++i) w2t[i * H + n] = orc_f32_from_bf16(b2[n * I + i]);
    } else {
      const uint8_t* c13 = w13 + e * (2 * I) * (H / 2);
      const uint8_t* s13 = w13s + e * (2 * I) * (H / 32);
      const uint8_t* c2 = w2 + e * H * (I / 2);
      const uint8_t* s2 = w2s + e * H * (I / 32);
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < 2 * I; ++n) {
        float tmp[32];
        for (int64_t b = 0; b < H / 32; ++b) {
          orc_dequant(c13 + n * (H / 2) + b * 16, s13 + n * (H / 32) + b, 1, 32, tmp);
          for (int i = 0; i < 32; ++i) w13t[(b * 32 + i) * (2 * I) + n] = tmp[i];
        }
      }
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < H; ++n) {
        float tmp[32];
        for (int64_t b = 0; b < I / 32; ++b) {
          orc_dequant(c2 + n * (I / 2) + b * 16, s2 + n * (I / 32) + b, 1, 32, tmp);
          for (int i = 0; i < 32; ++i) w2t[(b * 32 + i) * H + n] = tmp[i];
        }
      }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = off_[e]; p < off_[e + 1]; ++p) {
      if (yrow[p] < 0) continue;
      int64_t t = sor_[p] / k;
      float* h = (float*)malloc(sizeof(float) * (size_t)(2 * I));
      float* a = (float*)malloc(sizeof(float) * (size_t)I);
      uint16_t* ab = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
      /* gate_up: h[n] = sum_k x[k] * W13[n][k], fp32, k ascending */
      for (int64_t n = 0; n < 2 * I; ++n) h[n] = 0.0f;
      for (int64_t kk = 0; kk < H; ++kk) {
        float xv = xin[t * H + kk];
        const float* wr = w13t + kk * (2 * I);
        for (int64_t n = 0; n < 2 * I; ++n) h[n] = h[n] + xv * wr[n];
      }
      /* clamped SwiGLU, rounded to bf16 */
      for (int64_t i = 0; i < I; ++i) ab[i] = orc_bf16_from_f32(orc_swiglu(h[i], h[I + i], d->clamp_limit));
      if (act)
        for (int64_t i = 0; i < I; ++i) act[p * I + i] = ab[i];
      if (xs_e >= 0) {
        for (int64_t i = 0; i < I; ++i) a[i] = orc_f32_from_bf16(ab[i]);
      } else if (d->a4 && d->given_actq) {
        orc_dequant(actq + p * (I / 2), acts + p * (I / 32), 1, I, a);
      } else if (d->a8 && d->given_actq) {
        orc_dequant8(actq + p * I, acts + p * (I / 32), 1, I, a);
      } else if (d->a8) {
        uint8_t* q = (uint8_t*)malloc((size_t)I);
        uint8_t* s = (uint8_t*)malloc((size_t)(I / 32));
        orc_quantize8_bf16(ab, 1, I, q, s);
        orc_dequant8(q, s, 1, I, a);
        if (actq) memcpy(actq + p * I, q, (size_t)I);
        if (acts) memcpy(acts + p * (I / 32), s, (size_t)(I / 32));
        free(q);
        free(s);
      } else if (d->a4) {
        uint8_t* q = (uint8_t*)malloc((size_t)(I / 2));
        uint8_t* s = (uint8_t*)malloc((size_t)(I / 32));
        orc_quantize_bf16(ab, 1, I, q, s);
        orc_dequant(q, s, 1, I, a);
        if (actq) memcpy(actq + p * (I / 2), q, (size_t)(I / 2));
        if (acts) memcpy(acts + p * (I / 32), s, (size_t)(I / 32));
        free(q);
        free(s);
      } else {
        for (int64_t i = 0; i < I; ++i) a[i] = orc_f32_from_bf16(ab[i]);
      }
      /* down: y[n] = sum_i a[i] * W2[n][i], fp32, i ascending */
      float* yr = y + yrow[p] * H;
      for (int64_t n = 0; n < H; ++n) yr[n] = 0.0f;
      for (int64_t i = 0; i < I; ++i) {
        float av = a[i];
        const float* wr = w2t + i * H;
        for (int64_t n = 0; n < H; ++n) yr[n] = yr[n] + av * wr[n];
      }
      free(h);
      free(a);
      free(ab);
    }
  }

  /* combine: out32[t][n] = sum over local slots j (ascending) of w[t][j] * y */
  if (status == 0) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      if (token_mask && !token_mask[t]) continue;
      for (int64_t n = 0; n < H; ++n) {
        float acc = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
          int32_t pos = inv_[t * k + j];
          if (pos < 0) continue;
          float prod = w_[t * k + j] * y[yrow[pos] * H + n];
          acc = acc + prod;
        }
        if (out32) out32[t * H + n] = acc;
        if (out) out[t * H + n] = orc_bf16_from_f32(acc);
      }
    }
  }

  free(rowbuf);
  free(w13t);
  free(w2t);
  free(y);
  free(yrow);
  if (xb != xf) free(xb);
  free(xf);
  free(xslot);
  if (!ids) free(ids_);
  if (!w) free(w_);
  if (!counts) free(cnt_);
  if (!offsets) free(off_);
  if (!sorted) free(sor_);
  if (!inv) free(inv_);
  return status == 0 ? N : status;
}
