/*
 * laoracle.c -- plain, slow, fp64 CPU oracle for kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
 * leg use it.  It shares no code, header or constant with the HIP library.
 *
 * Every routine is the per-token recurrence written out in the order the pages
 * state it, in double precision.  Inputs arrive already widened to double (the
 * exact values of whatever bf16 / fp32 tensor the GPU sees).  Loops are
 * parallelised over independent (batch, head) units only; inside a unit the
 * order of operations is the plain sequential one.
 *
 * Layouts (row-major, innermost last):
 *   q, k : (B, T, H, Dk)      v, y : (B, T, H, Dv)       mask : (B, T), 0 = invalid
 *   S    : (B, H, Dk, Dv)     Z    : (B, H, Dk)
 * For the operator form (oracle_la_op) q, k, v, out are packed (B, T, heads*dim),
 * which is byte-identical to the 4-D layout above.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Feature maps ("[Feature] LinearAttention layer for Keras", section
 * "Feature maps"): elu_plus_one is elu(x)+1 with the standard elu slope 1,
 * i.e. x+1 for x>0 and exp(x) otherwise; relu is relu(x) plus the layer's
 * normalization epsilon. */
enum { ORACLE_FM_ELU_PLUS_ONE = 0, ORACLE_FM_RELU_EPS = 1 };

static double phi(double x, int fm, double eps) {
  if (fm == ORACLE_FM_ELU_PLUS_ONE) return x > 0.0 ? x + 1.0 : exp(x);
  return (x > 0.0 ? x : 0.0) + eps;
}

/* Causal recurrence with 2-D validity mask ("[Feature] LinearAttention layer for
 * Keras", sections "Mathematical definition / Causal", "Masking / Causal",
 * "Streaming State").  Per unit (b,h) and token t:
 *   if mask[b,t]:  S += phi(k_t) v_t^T ; Z += phi(k_t) ;
 *                  y_t = phi(q_t)^T S / (phi(q_t)^T Z + eps)   (or phi(q_t)^T S)
 *   else:          S, Z unchanged ; y_t = 0
 * The current token is part of its own context (update before readout).
 * S0/Z0 NULL means a zero initial state; S_out/Z_out NULL means "not wanted". */
int oracle_causal(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                  const double* q, const double* k, const double* v,
                  const uint8_t* mask, const double* S0, const double* Z0,
                  int fm, int use_norm, double eps,
                  double* y, double* S_out, double* Z_out) {
  if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      double* S = (double*)calloc((size_t)(Dk * Dv), sizeof(double));
      double* Z = (double*)calloc((size_t)Dk, sizeof(double));
      double* fk = (double*)malloc((size_t)Dk * sizeof(double));
      double* fq = (double*)malloc((size_t)Dk * sizeof(double));
      const int64_t u = b * H + h;
      if (S0) memcpy(S, S0 + u * Dk * Dv, (size_t)(Dk * Dv) * sizeof(double));
      if (Z0) memcpy(Z, Z0 + u * Dk, (size_t)Dk * sizeof(double));
      for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        double* yt = y + row * Dv;
        if (mask && !mask[b * T + t]) {
          for (int64_t c = 0; c < Dv; ++c) yt[c] = 0.0;
          continue;
        }
        const double* kt = k + row * Dk;
        const double* vt = v + row * Dv;
        const double* qt = q + row * Dk;
        for (int64_t d = 0; d < Dk; ++d) fk[d] = phi(kt[d], fm, eps);
        for (int64_t d = 0; d < Dk; ++d) fq[d] = phi(qt[d], fm, eps);
        for (int64_t d = 0; d < Dk; ++d) {
          for (int64_t c = 0; c < Dv; ++c) S[d * Dv + c] += fk[d] * vt[c];
          Z[d] += fk[d];
        }
        double den = 0.0;
        for (int64_t d = 0; d < Dk; ++d) den += fq[d] * Z[d];
        den += eps;
        for (int64_t c = 0; c < Dv; ++c) {
          double num = 0.0;
          for (int64_t d = 0; d < Dk; ++d) num += fq[d] * S[d * Dv + c];
          yt[c] = use_norm ? num / den : num;
        }
      }
      if (S_out) memcpy(S_out + u * Dk * Dv, S, (size_t)(Dk * Dv) * sizeof(double));
      if (Z_out) memcpy(Z_out + u * Dk, Z, (size_t)Dk * sizeof(double));
      free(S); free(Z); free(fk); free(fq);
    }
  }
  return 0;
}

/* Non-causal form ("[Feature] LinearAttention layer for Keras", sections
 * "Mathematical definition / Non-causal" and "Masking / Non-causal"):
 *   S = sum over valid j of phi(k_j) v_j^T,  Z = sum over valid j of phi(k_j)
 *   y_i = phi(q_i)^T S / (phi(q_i)^T Z + eps)  (or phi(q_i)^T S), 0 at invalid i.
 * S_out/Z_out (optional) receive the reduced statistics. */
int oracle_noncausal(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                     const double* q, const double* k, const double* v,
                     const uint8_t* mask, int fm, int use_norm, double eps,
                     double* y, double* S_out, double* Z_out) {
  if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      double* S = (double*)calloc((size_t)(Dk * Dv), sizeof(double));
      double* Z = (double*)calloc((size_t)Dk, sizeof(double));
      double* f = (double*)malloc((size_t)Dk * sizeof(double));
      const int64_t u = b * H + h;
      for (int64_t t = 0; t < T; ++t) {
        if (mask && !mask[b * T + t]) continue;
        const int64_t row = (b * T + t) * H + h;
        for (int64_t d = 0; d < Dk; ++d) f[d] = phi(k[row * Dk + d], fm, eps);
        for (int64_t d = 0; d < Dk; ++d) {
          for (int64_t c = 0; c < Dv; ++c) S[d * Dv + c] += f[d] * v[row * Dv + c];
          Z[d] += f[d];
        }
      }
      for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        double* yt = y + row * Dv;
        if (mask && !mask[b * T + t]) {
          for (int64_t c = 0; c < Dv; ++c) yt[c] = 0.0;
          continue;
        }
        for (int64_t d = 0; d < Dk; ++d) f[d] = phi(q[row * Dk + d], fm, eps);
        double den = eps;
        for (int64_t d = 0; d < Dk; ++d) den += f[d] * Z[d];
        for (int64_t c = 0; c < Dv; ++c) {
          double num = 0.0;
          for (int64_t d = 0; d < Dk; ++d) num += f[d] * S[d * Dv + c];
          yt[c] = use_norm ? num / den : num;
        }
      }
      if (S_out) memcpy(S_out + u * Dk * Dv, S, (size_t)(Dk * Dv) * sizeof(double));
      if (Z_out) memcpy(Z_out + u * Dk, Z, (size_t)Dk * sizeof(double));
      free(S); free(Z); free(f);
    }
  }
  return 0;
}

/* The operator form ("LinearAttention" operator page, sections "Description",
 * "Inputs", "Attributes"), for one of four update rules, run token by token:
 *   linear      : S = S + k v^T
 *   gated       : S = exp(g) * S + k v^T
 *   delta       : S = S + beta * k (v - S^T k)^T
 *   gated_delta : S = exp(g) * S + beta * k (v - exp(g) * S^T k)^T
 * and for every query head h served by kv head j:  o = scale * q^T S  (S after
 * this token's update).  Query head h reads kv head h / (Hq/Hkv) (contiguous
 * groups).  decay is (B,T,Hkv) (one scalar per kv head; decay_per_dim = 0) or
 * (B,T,Hkv*Dk) (one factor per key row of S; decay_per_dim = 1).  beta is
 * (B,T,Hkv) (beta_per_head = 1) or (B,T,1) (beta_per_head = 0). */
enum { ORACLE_RULE_LINEAR = 0, ORACLE_RULE_GATED = 1, ORACLE_RULE_DELTA = 2,
       ORACLE_RULE_GATED_DELTA = 3 };

int oracle_la_op(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv,
                 const double* q, const double* k, const double* v,
                 const double* past, const double* decay, int decay_per_dim,
                 const double* beta, int beta_per_head, int rule, double scale,
                 double* out, double* present) {
  if (B < 0 || T < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Dk < 1 || Dv < 1) return 1;
  const int gated = (rule == ORACLE_RULE_GATED || rule == ORACLE_RULE_GATED_DELTA);
  const int delta = (rule == ORACLE_RULE_DELTA || rule == ORACLE_RULE_GATED_DELTA);
  if (gated && !decay) return 2;
  if (delta && !beta) return 3;
  const int64_t G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t j = 0; j < Hkv; ++j) {
      double* S = (double*)calloc((size_t)(Dk * Dv), sizeof(double));
      double* a = (double*)malloc((size_t)Dk * sizeof(double));
      double* r = (double*)malloc((size_t)Dv * sizeof(double));
      const int64_t u = b * Hkv + j;
      if (past) memcpy(S, past + u * Dk * Dv, (size_t)(Dk * Dv) * sizeof(double));
      for (int64_t t = 0; t < T; ++t) {
        const double* kt = k + ((b * T + t) * Hkv + j) * Dk;
        const double* vt = v + ((b * T + t) * Hkv + j) * Dv;
        /* decay factor per key row of S */
        for (int64_t d = 0; d < Dk; ++d) {
          double g = 0.0;
          if (gated) g = decay_per_dim ? decay[((b * T + t) * Hkv + j) * Dk + d]
                                       : decay[(b * T + t) * Hkv + j];
          a[d] = exp(g);
        }
        for (int64_t d = 0; d < Dk; ++d)
          for (int64_t c = 0; c < Dv; ++c) S[d * Dv + c] *= a[d];
        if (delta) {
          const double bt = beta_per_head ? beta[(b * T + t) * Hkv + j] : beta[b * T + t];
          /* r = v - S^T k, with S already decayed */
          for (int64_t c = 0; c < Dv; ++c) {
            double sk = 0.0;
            for (int64_t d = 0; d < Dk; ++d) sk += S[d * Dv + c] * kt[d];
            r[c] = vt[c] - sk;
          }
          for (int64_t d = 0; d < Dk; ++d)
            for (int64_t c = 0; c < Dv; ++c) S[d * Dv + c] += bt * kt[d] * r[c];
        } else {
          for (int64_t d = 0; d < Dk; ++d)
            for (int64_t c = 0; c < Dv; ++c) S[d * Dv + c] += kt[d] * vt[c];
        }
        for (int64_t h = j * G; h < (j + 1) * G; ++h) {
          const double* qt = q + ((b * T + t) * Hq + h) * Dk;
          double* ot = out + ((b * T + t) * Hq + h) * Dv;
          for (int64_t c = 0; c < Dv; ++c) {
            double acc = 0.0;
            for (int64_t d = 0; d < Dk; ++d) acc += qt[d] * S[d * Dv + c];
            ot[c] = scale * acc;
          }
        }
      }
      if (present) memcpy(present + u * Dk * Dv, S, (size_t)(Dk * Dv) * sizeof(double));
      free(S); free(a); free(r);
    }
  }
  return 0;
}

/* Derivative of phi (the Keras proposal's feature maps): elu(x)+1 has slope 1
 * for x > 0 and exp(x) otherwise; relu(x)+eps has slope 1 for x > 0 and 0
 * otherwise (0 taken at x = 0). */
static double dphi(double x, int fm) {
  if (fm == 0) return x > 0.0 ? 1.0 : exp(x);
  return x > 0.0 ? 1.0 : 0.0;
}

/* Gradients of oracle_causal by reverse-mode differentiation of the same
 * per-token recurrence (the Keras proposal asks for recurrent/parallel gradient
 * parity and float64 numerical-gradient checks, "Stability" and "Acceptance").
 * Given dy (B,T,H,Dv) and optional gradients dS_T, dZ_T of the final state:
 * a forward sweep records S_t, Z_t after each token; a reverse sweep, with
 * G = dL/dS_t and g = dL/dZ_t accumulated from the later tokens,
 *   valid t:  num = S_t^T phi(q_t),  den = phi(q_t)^T Z_t + eps
 *             dnum = dy_t / den (or dy_t),  dden = -(dy_t . num) / den^2 (or 0)
 *             dphi(q_t) = S_t dnum + Z_t dden,   G += phi(q_t) dnum^T,  g += phi(q_t) dden
 *             dphi(k_t) = G v_t + g,   dv_t = G^T phi(k_t)
 *   invalid t: no gradient to q_t, k_t, v_t; G, g pass through,
 * then dq = dphi(q) * phi'(q), dk = dphi(k) * phi'(k), dS_0 = G, dZ_0 = g. */
int oracle_causal_backward(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                           const double* q, const double* k, const double* v,
                           const uint8_t* mask, const double* S0, const double* Z0,
                           const double* dy, const double* dS_T, const double* dZ_T,
                           int fm, int use_norm, double eps,
                           double* dq, double* dk, double* dv, double* dS0, double* dZ0) {
  if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      const int64_t u = b * H + h;
      double* Ss = (double*)calloc((size_t)((T + 1) * Dk * Dv), sizeof(double));  /* S after token t-1 at t */
      double* Zs = (double*)calloc((size_t)((T + 1) * Dk), sizeof(double));
      double* G = (double*)calloc((size_t)(Dk * Dv), sizeof(double));
      double* g = (double*)calloc((size_t)Dk, sizeof(double));
      double* fq = (double*)malloc((size_t)Dk * sizeof(double));
      double* fk = (double*)malloc((size_t)Dk * sizeof(double));
      double* dnum = (double*)malloc((size_t)Dv * sizeof(double));
      if (S0) memcpy(Ss, S0 + u * Dk * Dv, (size_t)(Dk * Dv) * sizeof(double));
      if (Z0) memcpy(Zs, Z0 + u * Dk, (size_t)Dk * sizeof(double));
      /* forward sweep: Ss[t+1] = state after token t */
      for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        double* S1 = Ss + (t + 1) * Dk * Dv;
        double* Z1 = Zs + (t + 1) * Dk;
        memcpy(S1, Ss + t * Dk * Dv, (size_t)(Dk * Dv) * sizeof(double));
        memcpy(Z1, Zs + t * Dk, (size_t)Dk * sizeof(double));
        if (mask && !mask[b * T + t]) continue;
        for (int64_t d = 0; d < Dk; ++d) {
          const double f = phi(k[row * Dk + d], fm, eps);
          for (int64_t c = 0; c < Dv; ++c) S1[d * Dv + c] += f * v[row * Dv + c];
          Z1[d] += f;
        }
      }
      if (dS_T) memcpy(G, dS_T + u * Dk * Dv, (size_t)(Dk * Dv) * sizeof(double));
      if (dZ_T) memcpy(g, dZ_T + u * Dk, (size_t)Dk * sizeof(double));
      /* reverse sweep */
      for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t row = (b * T + t) * H + h;
        double* dqt = dq + row * Dk;
        double* dkt = dk + row * Dk;
        double* dvt = dv + row * Dv;
        if (mask && !mask[b * T + t]) {
          for (int64_t d = 0; d < Dk; ++d) dqt[d] = dkt[d] = 0.0;
          for (int64_t c = 0; c < Dv; ++c) dvt[c] = 0.0;
          continue;
        }
        const double* S = Ss + (t + 1) * Dk * Dv;
        const double* Z = Zs + (t + 1) * Dk;
        const double* dyt = dy + row * Dv;
        for (int64_t d = 0; d < Dk; ++d) {
          fq[d] = phi(q[row * Dk + d], fm, eps);
          fk[d] = phi(k[row * Dk + d], fm, eps);
        }
        double den = eps, dden = 0.0;
        for (int64_t d = 0; d < Dk; ++d) den += fq[d] * Z[d];
        double dy_num = 0.0;
        for (int64_t c = 0; c < Dv; ++c) {
          double num = 0.0;
          for (int64_t d = 0; d < Dk; ++d) num += fq[d] * S[d * Dv + c];
          dy_num += dyt[c] * num;
          dnum[c] = use_norm ? dyt[c] / den : dyt[c];
        }
        if (use_norm) dden = -dy_num / (den * den);
        for (int64_t d = 0; d < Dk; ++d) {
          double a = Z[d] * dden;
          for (int64_t c = 0; c < Dv; ++c) a += S[d * Dv + c] * dnum[c];
          dqt[d] = a * dphi(q[row * Dk + d], fm);
        }
        for (int64_t d = 0; d < Dk; ++d) {
          for (int64_t c = 0; c < Dv; ++c) G[d * Dv + c] += fq[d] * dnum[c];
          g[d] += fq[d] * dden;
        }
        for (int64_t d = 0; d < Dk; ++d) {
          double a = g[d];
          for (int64_t c = 0; c < Dv; ++c) a += G[d * Dv + c] * v[row * Dv + c];
          dkt[d] = a * dphi(k[row * Dk + d], fm);
        }
        for (int64_t c = 0; c < Dv; ++c) {
          double a = 0.0;
          for (int64_t d = 0; d < Dk; ++d) a += G[d * Dv + c] * fk[d];
          dvt[c] = a;
        }
      }
      if (dS0) memcpy(dS0 + u * Dk * Dv, G, (size_t)(Dk * Dv) * sizeof(double));
      if (dZ0) memcpy(dZ0 + u * Dk, g, (size_t)Dk * sizeof(double));
      free(Ss); free(Zs); free(G); free(g); free(fq); free(fk); free(dnum);
    }
  }
  return 0;
}

/* Number of OpenMP threads a parallel loop above will use (for reporting). */
int oracle_max_threads(void) { return omp_get_max_threads(); }
