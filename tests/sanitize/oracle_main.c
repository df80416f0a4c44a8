/* Drives every routine of oracle/laoracle.c on small inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py):
 * masks, initial states, both feature maps, the normaliser on and off,
 * Dk != Dv, T = 0 and T = 1, every update rule with per-head and per-dim
 * decays, shared and per-head beta, GQA groups of 3, and the backward pass.
 * It checks only that every result is finite and every call accepted; the
 * values are pinned by tests/test_oracle_pins.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_causal(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, const double* q, const double* k,
                  const double* v, const uint8_t* mask, const double* S0, const double* Z0, int fm, int use_norm,
                  double eps, double* y, double* S_out, double* Z_out);
int oracle_noncausal(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, const double* q, const double* k,
                     const double* v, const uint8_t* mask, int fm, int use_norm, double eps, double* y, double* S,
                     double* Z);
int oracle_la_op(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv, const double* q,
                 const double* k, const double* v, const double* past, const double* decay, int decay_per_dim,
                 const double* beta, int beta_per_head, int rule, double scale, double* out, double* present);
int oracle_causal_backward(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, const double* q,
                           const double* k, const double* v, const uint8_t* mask, const double* S0,
                           const double* Z0, const double* dy, const double* dS_T, const double* dZ_T, int fm,
                           int use_norm, double eps, double* dq, double* dk, double* dv, double* dS0, double* dZ0);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double urand(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double* arr(int64_t n) {
  double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int64_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}
static int finite(const double* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}
static int fails = 0;
static void check(int ok, const char* what) {
  if (!ok) {
    printf("FAILED: %s\n", what);
    fails++;
  }
}

int main(void) {
  const int64_t B = 2, H = 3;
  const int64_t Ts[] = {0, 1, 37};
  const int64_t dims[][2] = {{8, 8}, {4, 12}, {12, 4}};
  for (int ti = 0; ti < 3; ++ti)
    for (int di = 0; di < 3; ++di)
      for (int fm = 0; fm < 2; ++fm)
        for (int norm = 0; norm < 2; ++norm)
          for (int masked = 0; masked < 2; ++masked)
            for (int with_state = 0; with_state < 2; ++with_state) {
              const int64_t T = Ts[ti], Dk = dims[di][0], Dv = dims[di][1];
              double *q = arr(B * T * H * Dk), *k = arr(B * T * H * Dk), *v = arr(B * T * H * Dv);
              double *S0 = arr(B * H * Dk * Dv), *Z0 = arr(B * H * Dk), *dy = arr(B * T * H * Dv);
              double *dS = arr(B * H * Dk * Dv), *dZ = arr(B * H * Dk);
              for (int64_t i = 0; i < B * H * Dk; ++i) Z0[i] = fabs(Z0[i]) + 1.0;
              uint8_t* m = (uint8_t*)malloc((size_t)(B * T > 0 ? B * T : 1));
              for (int64_t i = 0; i < B * T; ++i) m[i] = (uint8_t)(urand() > -0.6);
              double *y = arr(B * T * H * Dv), *S = arr(B * H * Dk * Dv), *Z = arr(B * H * Dk);
              const uint8_t* mp = masked ? m : NULL;
              check(oracle_causal(B, T, H, Dk, Dv, q, k, v, mp, with_state ? S0 : NULL,
                                  with_state && norm ? Z0 : NULL, fm, norm, 1e-6, y, S, Z) == 0, "causal");
              check(finite(y, B * T * H * Dv) && finite(S, B * H * Dk * Dv), "causal finite");
              check(oracle_noncausal(B, T, H, Dk, Dv, q, k, v, mp, fm, norm, 1e-6, y, S, Z) == 0, "noncausal");
              check(finite(y, B * T * H * Dv), "noncausal finite");
              double *dq = arr(B * T * H * Dk), *dk = arr(B * T * H * Dk), *dv = arr(B * T * H * Dv);
              check(oracle_causal_backward(B, T, H, Dk, Dv, q, k, v, mp, with_state ? S0 : NULL,
                                           with_state && norm ? Z0 : NULL, dy, with_state ? dS : NULL,
                                           with_state && norm ? dZ : NULL, fm, norm, 1e-6, dq, dk, dv, S, Z) == 0,
                    "backward");
              check(finite(dq, B * T * H * Dk) && finite(dk, B * T * H * Dk) && finite(dv, B * T * H * Dv) &&
                        finite(S, B * H * Dk * Dv),
                    "backward finite");
              free(q); free(k); free(v); free(S0); free(Z0); free(dy); free(dS); free(dZ); free(m);
              free(y); free(S); free(Z); free(dq); free(dk); free(dv);
            }
  /* the operator form: every rule, GQA group of 3, per-head and per-dim decays,
     per-head and shared beta, with and without a past state */
  const int64_t Hkv = 2, Hq = 6;
  for (int ti = 0; ti < 3; ++ti)
    for (int di = 0; di < 3; ++di)
      for (int rule = 0; rule < 4; ++rule)
        for (int pd = 0; pd < 2; ++pd)
          for (int bph = 0; bph < 2; ++bph)
            for (int with_past = 0; with_past < 2; ++with_past) {
              const int64_t T = Ts[ti], Dk = dims[di][0], Dv = dims[di][1];
              double *q = arr(B * T * Hq * Dk), *k = arr(B * T * Hkv * Dk), *v = arr(B * T * Hkv * Dv);
              double *g = arr(B * T * Hkv * (pd ? Dk : 1)), *be = arr(B * T * (bph ? Hkv : 1));
              for (int64_t i = 0; i < B * T * Hkv * (pd ? Dk : 1); ++i) g[i] = -fabs(g[i]);
              for (int64_t i = 0; i < B * T * (bph ? Hkv : 1); ++i) be[i] = 0.5 * (be[i] + 1.0);
              double *past = arr(B * Hkv * Dk * Dv), *out = arr(B * T * Hq * Dv), *pres = arr(B * Hkv * Dk * Dv);
              const int gated = rule == 1 || rule == 3, delta = rule >= 2;
              check(oracle_la_op(B, T, Hq, Hkv, Dk, Dv, q, k, v, with_past ? past : NULL, gated ? g : NULL, pd,
                                 delta ? be : NULL, bph, rule, 0.5, out, pres) == 0,
                    "la_op");
              check(finite(out, B * T * Hq * Dv) && finite(pres, B * Hkv * Dk * Dv), "la_op finite");
              free(q); free(k); free(v); free(g); free(be); free(past); free(out); free(pres);
            }
  /* argument errors are reported, not acted on */
  check(oracle_causal(-1, 4, 1, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1, 1e-6, NULL, NULL, NULL) != 0,
        "causal rejects B < 0");
  check(oracle_la_op(1, 4, 3, 2, 4, 4, NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, 0, 1.0, NULL, NULL) != 0,
        "la_op rejects Hq % Hkv");
  printf("%s (%d failures)\n", fails ? "FAIL" : "OK", fails);
  return fails ? 1 : 0;
}
