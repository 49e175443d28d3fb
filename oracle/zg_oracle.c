/*
 * zg_oracle.c -- plain, slow, fp64 CPU oracle of the ZGCM-1 hybrid attention core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py may load this library.  It shares no code, header, table or constant with the HIP path
 * (global_attention_gated_amd/) and never calls it.
 *
 * What it computes (every step in float64, inputs decoded exactly from bf16):
 *   zo_rmsnorm  -- QK normalisation with RMSNorm, per (token, head) row of D values:
 *                  y_d = x_d * w_d / sqrt(mean_d' x_d'^2 + eps).
 *                  (ZGCM-1 paper summaries: onedev.kr "How it works" names RMSNorm QK-normalisation;
 *                   jaehun.me "How Gated SWA Behaves" applies RMS normalisation to the query and key.)
 *   zo_rope     -- partial rotary position embedding on the leading R dims (R = 42 of 128 for the
 *                  rotary fraction 0.33 both pages give): each pair (2i, 2i+1), i < R/2, of a row at
 *                  absolute position p is rotated by the angle p * base^(-2i/R), in the RoFormer
 *                  convention (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).  Dims >= R are
 *                  left alone.  Applied after RMSNorm (the order in which jaehun.me lists them).
 *   zo_attend   -- softmax attention of query rows over key rows selected by position:
 *                  key j is visible to query i iff 0 <= kpos_j <= qpos_i and, for a sliding window W,
 *                  qpos_i - kpos_j < W (the window counts the query itself: jaehun.me's worked example,
 *                  window 4, the 4th token sees 4 tokens including itself).  Global causal layers
 *                  pass window <= 0.  Scores q.k / sqrt(D), explicit max-subtracted softmax.
 *                  If gate logits are given (gated SWA, onedev.kr "How it works" and jaehun.me
 *                  "How Gated SWA Behaves": output = A_SWA(q,k,v) (.) sigmoid(g_proj(h))), each output
 *                  element is multiplied by 1 / (1 + exp(-g)); global layers pass no gate.
 *   zo_round_bf16 -- round-to-nearest-even to bf16 (the stored form of outputs and cached keys).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

double zo_bf16_to_f64(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void zo_decode_bf16(const uint16_t* in, int64_t n, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = zo_bf16_to_f64(in[i]);
}

/* Single rounding of a double to bf16 (8 significant bits), ties to even.  NaN/inf pass through. */
uint16_t zo_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  int e;
  double m = frexp(x, &e);                   /* x = m * 2^e, 0.5 <= |m| < 1 */
  double r = ldexp(nearbyint(ldexp(m, 8)), e - 8); /* default rounding mode: nearest, ties to even */
  float f = (float)r;                        /* exact: r has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

void zo_round_bf16(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = zo_f64_to_bf16(in[i]);
}

void zo_rmsnorm(const double* x, int64_t rows, int32_t D, const double* w, double eps, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const double* xr = x + r * D;
    double ss = 0.0;
    for (int32_t d = 0; d < D; d++) ss += xr[d] * xr[d];
    double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (int32_t d = 0; d < D; d++) y[r * D + d] = xr[d] * inv * w[d];
  }
}

void zo_rope(double* x, int64_t rows, int32_t D, const int64_t* pos, int32_t R, double base) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    double* xr = x + r * D;
    for (int32_t i = 0; 2 * i + 1 < R && 2 * i + 1 < D; i++) {
      double theta = pow(base, -2.0 * (double)i / (double)R);
      double a = (double)pos[r] * theta;
      double c = cos(a), s = sin(a);
      double x0 = xr[2 * i], x1 = xr[2 * i + 1];
      xr[2 * i] = x0 * c - x1 * s;
      xr[2 * i + 1] = x0 * s + x1 * c;
    }
  }
}

static int visible(int64_t qp, int64_t kp, int64_t window) {
  if (kp < 0 || kp > qp) return 0;
  if (window > 0 && qp - kp >= window) return 0;
  return 1;
}

void zo_attend(int64_t nq, int32_t D, const double* qhat, const int64_t* qpos, int64_t nk, const double* khat,
               const double* v, const int64_t* kpos, int64_t window, const double* gate_logits, double* out) {
  const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t i = 0; i < nq; i++) {
      const double* q = qhat + i * D;
      double* o = out + i * D;
      double m = -INFINITY;
      int64_t nvis = 0;
      for (int64_t j = 0; j < nk; j++) {
        if (!visible(qpos[i], kpos[j], window)) { s[j] = -INFINITY; continue; }
        double acc = 0.0;
        for (int32_t d = 0; d < D; d++) acc += q[d] * khat[j * D + d];
        s[j] = acc * scale;
        if (s[j] > m) m = s[j];
        nvis++;
      }
      for (int32_t d = 0; d < D; d++) o[d] = 0.0;
      if (nvis == 0) {
        for (int32_t d = 0; d < D; d++) o[d] = NAN;
        continue;
      }
      double denom = 0.0;
      for (int64_t j = 0; j < nk; j++) {
        if (s[j] == -INFINITY) continue;
        double p = exp(s[j] - m);
        denom += p;
        for (int32_t d = 0; d < D; d++) o[d] += p * v[j * D + d];
      }
      for (int32_t d = 0; d < D; d++) o[d] /= denom;
      if (gate_logits) {
        const double* g = gate_logits + i * D;
        for (int32_t d = 0; d < D; d++) o[d] *= 1.0 / (1.0 + exp(-g[d]));
      }
    }
    free(s);
  }
}

int zo_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
