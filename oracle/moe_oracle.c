/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle for the routed-experts
 * MoE decode step (MXFP8 activations x FP4 weights).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or call
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (vLLM API documentation pages):
 *   [experts]  "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.experts"
 *   [runtime]  "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.experts_runtime"
 * Element formats: OCP Microscaling (MX) v1.0 -- e2m1 (FP4), e4m3 (FP8, "fn": no
 * infinities, 0x7F/0xFF are NaN, max 448) and E8M0 block scales over 32 elements.
 *
 * Everything is computed in double precision and rounded once where the method
 * rounds (FP32 accumulator, FP32 hidden, BF16 output).  Readings of points the pages
 * leave open are listed in the repository's design notes and restated next to the
 * function that takes them.
 *
 * Parity pins: every function here is pinned by a `-m "not gpu"` test (decode against
 * torch's own float8/float4 decoders, encode against a brute-force nearest search,
 * block exponents against closed forms, FC1/FC2 against dense FP64 matmuls of
 * independently decoded operands, the gated activation against closed-form values
 * g*u/(1+e^-g) of hand-set asymmetric gate/up pairs and against torch's SiLU,
 * routing invariants).  No function is unpinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------------
 * Element decoders (OCP MX v1.0 element tables).
 * ------------------------------------------------------------------------------ */

/* FP4 e2m1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
ORACLE_API double oracle_e2m1_value(unsigned nibble) {
  unsigned s = (nibble >> 3) & 1u, e = (nibble >> 1) & 3u, m = nibble & 1u;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
  return s ? -mag : mag;
}

/* FP8 e4m3fn: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
 * Exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; max finite 448. */
ORACLE_API double oracle_e4m3_value(unsigned code) {
  unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* E8M0 scale: 2^(code - 127); 0xFF is NaN. */
ORACLE_API double oracle_e8m0_value(unsigned code) {
  if (code == 255) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* BF16 is the upper half of an IEEE binary32. */
static float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* binary32 -> BF16, round to nearest, ties to even (finite inputs). */
ORACLE_API uint16_t oracle_float_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  /* Exact RNE: compare the discarded 16 bits against half an ulp. */
  uint32_t hi = u >> 16, lo = u & 0xFFFFu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* ------------------------------------------------------------------------------
 * e4m3 encoder: round to nearest representable value, ties to the even code
 * (even mantissa), saturating to +-448 instead of producing NaN ("satfinite").
 * The experts page's pack_fp8 / fp8_bits helpers have no body on the page; this is
 * the reading taken: RNE + satfinite, never NaN for finite input, sign of zero kept.
 * ------------------------------------------------------------------------------ */
ORACLE_API unsigned oracle_e4m3_encode(float v) {
  unsigned sign = signbit(v) ? 0x80u : 0u;
  double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7Eu;
  /* The spacing of e4m3 values around a: 2^-9 below 2^-6 (subnormals), otherwise
   * 2^(floor(log2 a) - 3) (three mantissa bits). */
  double quantum;
  if (a < ldexp(1.0, -6)) {
    quantum = ldexp(1.0, -9);
  } else {
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) -> floor(log2 a) = ex - 1 */
    quantum = ldexp(1.0, ex - 1 - 3);
  }
  double q = a / quantum;     /* exact: division by a power of two */
  double r = nearbyint(q);    /* default rounding mode: ties to even */
  double val = r * quantum;   /* a representable e4m3 magnitude (<= 448) */
  if (val > 448.0) val = 448.0;
  /* Encode the magnitude: find the code whose value equals val. */
  if (val == 0.0) return sign;
  if (val < ldexp(1.0, -6)) return sign | (unsigned)(val / ldexp(1.0, -9));
  int ex;
  double f = frexp(val, &ex);  /* val = (2f) * 2^(ex-1), 2f in [1, 2) */
  unsigned e = (unsigned)(ex - 1 + 7);
  unsigned m = (unsigned)((2.0 * f - 1.0) * 8.0);
  return sign | (e << 3) | m;
}

/* ------------------------------------------------------------------------------
 * E8M0 block exponent of an MX block with absolute maximum amax (experts page,
 * mx_block / plan_chunk and store_hidden call mx_exponent(amax) and
 * mx_exponent(amax, floor=...); the helper's body is not on the page).
 *   amax == 0            -> e = -127 (scale byte 0x00)
 *   amax = M * 2^E, M in [1, 2):
 *     floor rule (OCP MX v1.0):      e = E - 8   (8 = e4m3's largest exponent)
 *     ceil rule (no saturation):     the smallest e with amax * 2^-e <= 448,
 *                                    i.e. e = E - 8 + (M > 1.75)
 *   e is clamped to [-127, 127]; the scale byte is e + 127.
 * ------------------------------------------------------------------------------ */
ORACLE_API int oracle_block_exponent(float amax, int floor_rule) {
  double a = fabs((double)amax);
  if (a == 0.0) return -127;
  int ex;
  double f = frexp(a, &ex); /* a = (2f) * 2^(ex-1) */
  int E = ex - 1;
  double M = 2.0 * f;
  int e = E - 8;
  if (!floor_rule && M > 1.75) e += 1;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* MXFP8 quantization of one block of 32 FP32 values: exact amax, E8M0 exponent,
 * exact scaling by 2^-e, e4m3 RNE-satfinite per element (experts page, mx_block). */
ORACLE_API void oracle_quantize_block(const float* v, int floor_rule, uint8_t* codes,
                                      uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  int e = oracle_block_exponent(amax, floor_rule);
  for (int i = 0; i < 32; ++i) {
    /* v * 2^-e is exact in double; it is then a binary32 value's multiple as well
     * (the scaled magnitudes of interest are far inside binary32's range). */
    double scaled = ldexp((double)v[i], -e);
    codes[i] = (uint8_t)oracle_e4m3_encode((float)scaled);
  }
  *scale = (uint8_t)(e + 127);
}

/* ------------------------------------------------------------------------------
 * Plan: MXFP8 of every token row (experts page, ExpertsPlanKernel / plan_chunk),
 * with the default (ceil) exponent rule.  x: BF16 [B, D] row-major.
 * codes: [B, D] e4m3, scales: [B, D/32] E8M0.
 * ------------------------------------------------------------------------------ */
ORACLE_API int oracle_plan(const uint16_t* x, int B, int D, uint8_t* codes, uint8_t* scales) {
  if (B < 0 || D <= 0 || D % 32) return -1;
  float block[32];
  for (int t = 0; t < B; ++t)
    for (int b = 0; b < D / 32; ++b) {
      for (int i = 0; i < 32; ++i) block[i] = bf16_to_float(x[(size_t)t * D + b * 32 + i]);
      oracle_quantize_block(block, 0, codes + (size_t)t * D + b * 32,
                            scales + (size_t)t * (D / 32) + b);
    }
  return 0;
}

/* ------------------------------------------------------------------------------
 * Unit table (experts page, ExpertsKernel.group): expert e's routes, in token order,
 * fill ceil(n_e / 8) units; units are numbered in ascending expert order; a unit row
 * holds the route's pair index t*K + s, -1 where padded.
 * Returns the number of units, or -1 on invalid ids (out of range, or one token
 * naming an expert twice: the pages require distinct top-k ids per token).
 * unit_expert: [B*K], unit_rows: [B*K, 8] (capacity: every route in its own unit).
 * ------------------------------------------------------------------------------ */
ORACLE_API int oracle_group(const int32_t* ids, int B, int K, int E, int32_t* unit_expert,
                            int32_t* unit_rows) {
  for (int t = 0; t < B; ++t)
    for (int s = 0; s < K; ++s) {
      int32_t e = ids[t * K + s];
      if (e < 0 || e >= E) return -1;
      for (int s2 = 0; s2 < s; ++s2)
        if (ids[t * K + s2] == e) return -1;
    }
  int n = 0;
  for (int e = 0; e < E; ++e) {
    int count = 0;
    for (int t = 0; t < B; ++t)
      for (int s = 0; s < K; ++s) {
        if (ids[t * K + s] != e) continue;
        if (count % 8 == 0) {
          unit_expert[n] = e;
          for (int j = 0; j < 8; ++j) unit_rows[n * 8 + j] = -1;
          ++n;
        }
        unit_rows[(n - 1) * 8 + count % 8] = t * K + s;
        ++count;
      }
  }
  return n;
}

/* ------------------------------------------------------------------------------
 * One route through the expert (experts page: stage / consume for FC1,
 * store_hidden for the gated activation and the hidden's MXFP8 requantization,
 * fc2 for the second matmul and the BF16 output row).
 *
 * Canonical layouts:
 *   w13 [E, 2I, D/2] bytes: two e2m1 per byte, low nibble = even k;
 *        rows 0..I-1 are the gate projection, rows I..2I-1 the up projection.
 *   s13 [E, 2I, D/32] E8M0, one per 32 consecutive k of a row.
 *   w2  [E, D, I/2], s2 [E, D, I/32] likewise (rows = output features d).
 *
 *   FC1:   a[r] = fp32( sum_k dq(W13[e,r,k]) * dq(X[t,k]) )          (FP64 sum)
 *   act:   h[i] = fp32( silu(g) * u ), g = a[i], u = a[I+i]  (SwiGLU; the pages'
 *          SiTU activation has no formula on the page)
 *   requant: MXFP8 per 32 hidden values, exponent rule `hidden_floor`
 *   FC2:   y[d] = bf16( fp32( sum_i dq(W2[e,d,i]) * dq(Hq[i]) ) )      (FP64 sum)
 * Output rows carry no routing weight (the weights are used by the combine only).
 * ------------------------------------------------------------------------------ */
typedef struct {
  int E, D, I, hidden_floor;
  const uint8_t *w13, *s13, *w2, *s2;
  const uint8_t *xcodes, *xscales;
  const int32_t* ids;
  int B, K;
  const int32_t* routes;
  int n_routes;
  uint16_t* out;
  float* out_f32;
  float* fc1;
  float* hidden; /* optional: the FP32 hidden before its requantization */
  double* fc1_abs; /* optional: sum over k of |w * x| per FC1 row (the sum's condition) */
  uint8_t *hcodes, *hscales;
  double *e2m1, *e4m3, *e8m0; /* decode tables (plain lookups of the decoders above) */
} oracle_job;

static inline double fp4_at(const oracle_job* j, const uint8_t* row, int k) {
  uint8_t byte = row[k >> 1];
  return j->e2m1[(k & 1) ? (byte >> 4) : (byte & 15)];
}

/* TwoSum (Knuth): returns s = a + b and whether the addition rounded. */
static inline double two_sum(double a, double b, int64_t* inexact) {
  double s = a + b;
  double bb = s - a;
  double err = (a - (s - bb)) + (b - bb);
  if (err != 0.0) ++*inexact;
  return s;
}

static int64_t oracle_route(const oracle_job* j, int out_row, int route) {
  const int D = j->D, I = j->I;
  const int t = route / j->K, e = j->ids[route];
  int64_t inexact = 0;
  float* a = (float*)malloc(sizeof(float) * 2 * I);
  float* h = (float*)malloc(sizeof(float) * I);
  uint8_t* hq = (uint8_t*)malloc(I);
  uint8_t* hs = (uint8_t*)malloc(I / 32);
  const uint8_t* xc = j->xcodes + (size_t)t * D;
  const uint8_t* xs = j->xscales + (size_t)t * (D / 32);
  /* FC1 */
  for (int r = 0; r < 2 * I; ++r) {
    const uint8_t* wrow = j->w13 + ((size_t)e * 2 * I + r) * (D / 2);
    const uint8_t* srow = j->s13 + ((size_t)e * 2 * I + r) * (D / 32);
    double acc = 0.0, mag = 0.0;
    for (int k = 0; k < D; ++k) {
      double w = fp4_at(j, wrow, k) * j->e8m0[srow[k / 32]];
      double x = j->e4m3[xc[k]] * j->e8m0[xs[k / 32]];
      acc = two_sum(acc, w * x, &inexact);
      mag += fabs(w * x);
    }
    a[r] = (float)acc;
    if (j->fc1_abs) j->fc1_abs[(size_t)out_row * 2 * I + r] = mag;
  }
  /* SwiGLU, FP32 hidden (no BF16 rounding before the requantization) */
  for (int i = 0; i < I; ++i) {
    double g = a[i], u = a[I + i];
    h[i] = (float)(g / (1.0 + exp(-g)) * u);
  }
  for (int b = 0; b < I / 32; ++b) oracle_quantize_block(h + 32 * b, j->hidden_floor, hq + 32 * b, hs + b);
  /* FC2 */
  uint16_t* y = j->out + (size_t)out_row * D;
  for (int d = 0; d < D; ++d) {
    const uint8_t* wrow = j->w2 + ((size_t)e * D + d) * (I / 2);
    const uint8_t* srow = j->s2 + ((size_t)e * D + d) * (I / 32);
    double acc = 0.0;
    for (int i = 0; i < I; ++i) {
      double w = fp4_at(j, wrow, i) * j->e8m0[srow[i / 32]];
      double x = j->e4m3[hq[i]] * j->e8m0[hs[i / 32]];
      acc = two_sum(acc, w * x, &inexact);
    }
    y[d] = oracle_float_to_bf16((float)acc);
    if (j->out_f32) j->out_f32[(size_t)out_row * D + d] = (float)acc;
  }
  if (j->fc1) memcpy(j->fc1 + (size_t)out_row * 2 * I, a, sizeof(float) * 2 * I);
  if (j->hidden) memcpy(j->hidden + (size_t)out_row * I, h, sizeof(float) * I);
  if (j->hcodes) memcpy(j->hcodes + (size_t)out_row * I, hq, I);
  if (j->hscales) memcpy(j->hscales + (size_t)out_row * (I / 32), hs, I / 32);
  free(a);
  free(h);
  free(hq);
  free(hs);
  return inexact;
}

typedef struct {
  const oracle_job* job;
  int first, step;
  int64_t inexact;
} oracle_worker;

static void* oracle_worker_main(void* arg) {
  oracle_worker* w = (oracle_worker*)arg;
  const oracle_job* j = w->job;
  for (int i = w->first; i < j->n_routes; i += w->step)
    w->inexact += oracle_route(j, i, j->routes ? j->routes[i] : i);
  return NULL;
}

/* Runs the routes listed in `routes` (NULL: all B*K routes, in pair order) and writes
 * output row i for the i-th listed route (`out_f32`, optional: the same rows before
 * their BF16 rounding, i.e. the exact FC2 sums rounded once to FP32; `fc1`, `fc1_abs`,
 * `hidden`, `hcodes`, `hscales`, optional: the route's FC1 values [2I], the sums of
 * their terms' magnitudes [2I] (in FP64: they bound how far an FP32 summation in any
 * order can land from the exact value), FP32 hidden [I] and its MXFP8 codes [I] and
 * scales [I/32]).  Routes are independent of each other, so
 * they are spread over `nthreads` threads.  `inexact` (optional) receives the number
 * of FP64 additions that rounded (0 certifies the FC1/FC2 sums as exact).
 * Returns 0, or -1 on invalid arguments / ids. */
ORACLE_API int oracle_experts(int E, int D, int I, const uint8_t* w13, const uint8_t* s13,
                              const uint8_t* w2, const uint8_t* s2, const uint8_t* xcodes,
                              const uint8_t* xscales, const int32_t* ids, int B, int K,
                              const int32_t* routes, int n_routes, int hidden_floor,
                              uint16_t* out, float* out_f32, float* fc1, double* fc1_abs, float* hidden,
                              uint8_t* hcodes, uint8_t* hscales, int nthreads, int64_t* inexact) {
  if (E <= 0 || D <= 0 || I <= 0 || D % 32 || I % 32 || B < 0 || K <= 0) return -1;
  for (int r = 0; r < B * K; ++r)
    if (ids[r] < 0 || ids[r] >= E) return -1;
  if (!routes) n_routes = B * K;
  for (int i = 0; routes && i < n_routes; ++i)
    if (routes[i] < 0 || routes[i] >= B * K) return -1;
  double e2m1[16], e4m3[256], e8m0[256];
  for (int c = 0; c < 16; ++c) e2m1[c] = oracle_e2m1_value((unsigned)c);
  for (int c = 0; c < 256; ++c) e4m3[c] = oracle_e4m3_value((unsigned)c);
  for (int c = 0; c < 256; ++c) e8m0[c] = oracle_e8m0_value((unsigned)c);
  oracle_job job = {E, D, I, hidden_floor, w13, s13, w2, s2, xcodes, xscales, ids, B, K,
                    routes, n_routes, out, out_f32, fc1, hidden, fc1_abs, hcodes, hscales, e2m1, e4m3, e8m0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  oracle_worker workers[256];
  pthread_t threads[256];
  for (int i = 0; i < nthreads; ++i) {
    workers[i].job = &job;
    workers[i].first = i;
    workers[i].step = nthreads;
    workers[i].inexact = 0;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&threads[i], NULL, oracle_worker_main, &workers[i]);
  oracle_worker_main(&workers[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(threads[i], NULL);
  int64_t total = 0;
  for (int i = 0; i < nthreads; ++i) total += workers[i].inexact;
  if (inexact) *inexact = total;
  return 0;
}

/* ------------------------------------------------------------------------------
 * Weighted top-k combine (experts page, ExpertsKernel.finalize: each token's staged
 * slot rows are summed with the routing weights in FP32).  The local part only:
 *   out[t, d] = bf16( sum_s w[t, s] * y[t*K + s, d] ), summed in FP64, rounded to
 *   FP32 then BF16.
 * ------------------------------------------------------------------------------ */
ORACLE_API int oracle_combine(const uint16_t* rows, const float* weights, int B, int K, int D,
                              uint16_t* out) {
  if (B < 0 || K <= 0 || D <= 0) return -1;
  for (int t = 0; t < B; ++t)
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int s = 0; s < K; ++s)
        acc += (double)weights[t * K + s] * (double)bf16_to_float(rows[((size_t)t * K + s) * D + d]);
      out[(size_t)t * D + d] = oracle_float_to_bf16((float)acc);
    }
  return 0;
}

/* Array conveniences for the test harness (loops over the scalar definitions). */
ORACLE_API void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e4m3_encode(v[i]);
}
ORACLE_API void oracle_block_exponent_array(const float* amax, int64_t n, int floor_rule, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_block_exponent(amax[i], floor_rule);
}
ORACLE_API void oracle_quantize_blocks(const float* v, int64_t nblocks, int floor_rule, uint8_t* codes,
                                       uint8_t* scales) {
  for (int64_t b = 0; b < nblocks; ++b) oracle_quantize_block(v + 32 * b, floor_rule, codes + 32 * b, scales + b);
}
