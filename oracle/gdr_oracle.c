/*
 * gdr_oracle.c -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the HIP library, and nothing in the product
 * path may call it.
 *
 * What it computes
 * ----------------
 * The method is named on the FlashQLA pages ("[GDN] Add FlashQLA backend
 * dispatch", Summary: a fused forward/backward kernel for the Gated Delta
 * Rule; "flashqla-linear-attention", Core API: q,k [B,T,Hq,K], v [B,T,Hv,V],
 * g and beta [B,T,Hv], optional initial_state [B,Hv,K,V]).  The recurrence
 * itself is the gated delta rule of Gated Delta Networks (Yang, Kautz,
 * Hatamizadeh, 2024), written for a K x V state S:
 *
 *     a_t = exp(g_t)                     (g is a natural-log decay)
 *     e_t = v_t - (a_t S_{t-1})^T k_t    (prediction error, a V-vector)
 *     S_t = a_t S_{t-1} + beta_t k_t e_t^T
 *     o_t = scale * S_t^T q_t            (the updated state is read)
 *
 * Value head h reads q/k head h / (Hv/Hq) (grouped value attention, GVA).
 *
 * Four entry points:
 *   oracle_fwd          token recurrence, forward
 *   oracle_bwd          reverse-mode derivative of the token recurrence,
 *                       derived by hand (states re-computed from a
 *                       checkpoint every CKPT tokens)
 *   oracle_chunked_fwd  the chunked rearrangement (WY form), done naively in
 *                       fp64 for any chunk size; also returns the per-chunk
 *                       stage tensors (chunk-local cumsum of g, the inverse
 *                       A, chunk-start states h)
 *   oracle_chunked_bwd  reverse-mode derivative of the chunked form
 *
 * Layouts (all row-major, fp64, tokens flattened over the batch):
 *   q, k      [Ttot, Hq, K]      v, o, do, dv   [Ttot, Hv, V]
 *   g, beta   [Ttot, Hv]         states          [N, Hv, K, V]
 *   cu        [N+1] int64 token offsets of the N sequences (a dense batch of
 *             B rows of length T is cu = 0, T, 2T, ..., BT)
 *   mask      optional [N*Hv] bytes: compute only the (sequence, head) units
 *             whose byte is non-zero (others are left untouched).
 * Return value: 0 on success, -1 on a bad argument, -2 on allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 64

static int bad_args(int64_t N, const int64_t* cu, int64_t Hq, int64_t Hv, int64_t K, int64_t V) {
  if (N < 0 || !cu || Hq <= 0 || Hv <= 0 || K <= 0 || V <= 0) return 1;
  if (Hv % Hq != 0) return 1;
  if (cu[0] != 0) return 1;
  for (int64_t n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return 1;
  return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* ------------------------------------------------------------------------ */
/* Token recurrence, forward.                                               */
/* ------------------------------------------------------------------------ */
int oracle_fwd(int64_t N, const int64_t* cu, int64_t Hq, int64_t Hv, int64_t K, int64_t V,
               const double* q, const double* k, const double* v, const double* g,
               const double* beta, double scale, const double* h0, double* o, double* ht,
               const uint8_t* mask, int nthreads) {
  if (bad_args(N, cu, Hq, Hv, K, V)) return -1;
  set_threads(nthreads);
  const int64_t G = Hv / Hq;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < N * Hv; ++u) {
    if (mask && !mask[u]) continue;
    const int64_t n = u / Hv, h = u % Hv, hq = h / G;
    double* S = (double*)malloc(sizeof(double) * K * V);
    double* e = (double*)malloc(sizeof(double) * V);
    if (!S || !e) {
      err = -2;
      free(S);
      free(e);
      continue;
    }
    if (h0) memcpy(S, h0 + u * K * V, sizeof(double) * K * V);
    else memset(S, 0, sizeof(double) * K * V);
    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      const double* kt = k + (t * Hq + hq) * K;
      const double* qt = q + (t * Hq + hq) * K;
      const double* vt = v + (t * Hv + h) * V;
      const double a = exp(g[t * Hv + h]);
      const double b = beta[t * Hv + h];
      for (int64_t i = 0; i < K * V; ++i) S[i] *= a; /* S <- a S_{t-1} */
      for (int64_t j = 0; j < V; ++j) {
        double p = 0.0;
        for (int64_t i = 0; i < K; ++i) p += S[i * V + j] * kt[i];
        e[j] = vt[j] - p;
      }
      for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < V; ++j) S[i * V + j] += b * kt[i] * e[j];
      double* ot = o + (t * Hv + h) * V;
      for (int64_t j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * qt[i];
        ot[j] = scale * acc;
      }
    }
    if (ht) memcpy(ht + u * K * V, S, sizeof(double) * K * V);
    free(S);
    free(e);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Token recurrence, backward.                                              */
/*                                                                          */
/* Loss L = sum(do * o) + sum(dht * S_T).  Walking the tokens backwards     */
/* with dS = dL/dS_t (output term of token t included):                     */
/*   dS  += scale q_t do_t^T          dq_t = scale S_t do_t                 */
/*   dbeta_t = k_t^T dS e_t           de = beta_t dS^T k_t,  dv_t = de      */
/*   dk_t = beta_t dS e_t - P_t de    (P_t = a_t S_{t-1})                   */
/*   dP = dS - k_t de^T               dg_t = sum(dP * P_t)                  */
/*   dS <- a_t dP                     (gradient into S_{t-1})               */
/* dq and dk are summed over the Hv/Hq value heads of a group, in head      */
/* order, after the per-unit loop.                                          */
/* ------------------------------------------------------------------------ */
int oracle_bwd(int64_t N, const int64_t* cu, int64_t Hq, int64_t Hv, int64_t K, int64_t V,
               const double* q, const double* k, const double* v, const double* g,
               const double* beta, double scale, const double* h0, const double* dO,
               const double* dht, double* dq, double* dk, double* dv, double* dbeta, double* dg,
               double* dh0, const uint8_t* mask, int nthreads) {
  if (bad_args(N, cu, Hq, Hv, K, V)) return -1;
  set_threads(nthreads);
  const int64_t G = Hv / Hq;
  const int64_t Ttot = cu[N];
  /* per value head partials of dq and dk: [Ttot, Hv, K] */
  double* dqh = (double*)calloc((size_t)(Ttot * Hv * K + 1), sizeof(double));
  double* dkh = (double*)calloc((size_t)(Ttot * Hv * K + 1), sizeof(double));
  if (!dqh || !dkh) {
    free(dqh);
    free(dkh);
    return -2;
  }
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < N * Hv; ++u) {
    if (mask && !mask[u]) continue;
    const int64_t n = u / Hv, h = u % Hv, hq = h / G;
    const int64_t t0 = cu[n], t1 = cu[n + 1], L = t1 - t0;
    const int64_t nck = (L + CKPT - 1) / CKPT;
    const size_t KV = (size_t)(K * V);
    double* ck = (double*)malloc(sizeof(double) * KV * (size_t)(nck + 1));
    double* seg = (double*)malloc(sizeof(double) * KV * (CKPT + 1));
    double* dS = (double*)malloc(sizeof(double) * KV);
    double* dP = (double*)malloc(sizeof(double) * KV);
    double* e = (double*)malloc(sizeof(double) * V);
    double* de = (double*)malloc(sizeof(double) * V);
    if (!ck || !seg || !dS || !dP || !e || !de) {
      err = -2;
      free(ck); free(seg); free(dS); free(dP); free(e); free(de);
      continue;
    }
    /* forward pass, keeping the state before every CKPT-th token */
    double* S = ck; /* ck[0] = initial state */
    if (h0) memcpy(S, h0 + u * KV, sizeof(double) * KV);
    else memset(S, 0, sizeof(double) * KV);
    for (int64_t c = 0; c < nck; ++c) {
      double* Sn = ck + (size_t)(c + 1) * KV;
      memcpy(Sn, ck + (size_t)c * KV, sizeof(double) * KV);
      for (int64_t t = t0 + c * CKPT; t < t0 + (c + 1) * CKPT && t < t1; ++t) {
        const double* kt = k + (t * Hq + hq) * K;
        const double* vt = v + (t * Hv + h) * V;
        const double a = exp(g[t * Hv + h]), b = beta[t * Hv + h];
        for (size_t i = 0; i < KV; ++i) Sn[i] *= a;
        for (int64_t j = 0; j < V; ++j) {
          double p = 0.0;
          for (int64_t i = 0; i < K; ++i) p += Sn[i * V + j] * kt[i];
          e[j] = vt[j] - p;
        }
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) Sn[i * V + j] += b * kt[i] * e[j];
      }
    }
    if (dht) memcpy(dS, dht + u * KV, sizeof(double) * KV);
    else memset(dS, 0, sizeof(double) * KV);
    for (int64_t c = nck - 1; c >= 0; --c) {
      const int64_t ts = t0 + c * CKPT;
      const int64_t te = (ts + CKPT < t1) ? ts + CKPT : t1;
      /* seg[m] = state before token ts+m, seg[te-ts] = state after the segment */
      memcpy(seg, ck + (size_t)c * KV, sizeof(double) * KV);
      for (int64_t t = ts; t < te; ++t) {
        double* Sp = seg + (size_t)(t - ts) * KV;
        double* Sn = seg + (size_t)(t - ts + 1) * KV;
        const double* kt = k + (t * Hq + hq) * K;
        const double* vt = v + (t * Hv + h) * V;
        const double a = exp(g[t * Hv + h]), b = beta[t * Hv + h];
        for (size_t i = 0; i < KV; ++i) Sn[i] = a * Sp[i];
        for (int64_t j = 0; j < V; ++j) {
          double p = 0.0;
          for (int64_t i = 0; i < K; ++i) p += Sn[i * V + j] * kt[i];
          e[j] = vt[j] - p;
        }
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) Sn[i * V + j] += b * kt[i] * e[j];
      }
      for (int64_t t = te - 1; t >= ts; --t) {
        const double* Sprev = seg + (size_t)(t - ts) * KV;
        const double* Scur = seg + (size_t)(t - ts + 1) * KV;
        const double* kt = k + (t * Hq + hq) * K;
        const double* qt = q + (t * Hq + hq) * K;
        const double* vt = v + (t * Hv + h) * V;
        const double* dot = dO + (t * Hv + h) * V;
        const double a = exp(g[t * Hv + h]), b = beta[t * Hv + h];
        /* prediction error of token t, from P_t = a S_{t-1} */
        for (int64_t j = 0; j < V; ++j) {
          double p = 0.0;
          for (int64_t i = 0; i < K; ++i) p += a * Sprev[i * V + j] * kt[i];
          e[j] = vt[j] - p;
        }
        /* output term */
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) dS[i * V + j] += scale * qt[i] * dot[j];
        double* dqt = dqh + (t * Hv + h) * K;
        for (int64_t i = 0; i < K; ++i) {
          double acc = 0.0;
          for (int64_t j = 0; j < V; ++j) acc += Scur[i * V + j] * dot[j];
          dqt[i] = scale * acc;
        }
        /* S_t = P + beta k e^T */
        double db = 0.0;
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) db += kt[i] * dS[i * V + j] * e[j];
        dbeta[t * Hv + h] = db;
        for (int64_t j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int64_t i = 0; i < K; ++i) acc += dS[i * V + j] * kt[i];
          de[j] = b * acc;
          dv[(t * Hv + h) * V + j] = de[j];
        }
        double* dkt = dkh + (t * Hv + h) * K;
        for (int64_t i = 0; i < K; ++i) {
          double acc1 = 0.0, acc2 = 0.0;
          for (int64_t j = 0; j < V; ++j) {
            acc1 += dS[i * V + j] * e[j];
            acc2 += a * Sprev[i * V + j] * de[j];
          }
          dkt[i] = b * acc1 - acc2;
        }
        double dgt = 0.0;
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) {
            const double d = dS[i * V + j] - kt[i] * de[j];
            dP[i * V + j] = d;
            dgt += d * a * Sprev[i * V + j];
          }
        dg[t * Hv + h] = dgt;
        for (size_t i = 0; i < KV; ++i) dS[i] = a * dP[i];
      }
    }
    if (dh0) memcpy(dh0 + u * KV, dS, sizeof(double) * KV);
    free(ck); free(seg); free(dS); free(dP); free(e); free(de);
  }
  /* group sums for q/k heads */
  for (int64_t n = 0; n < N; ++n)
    for (int64_t hq = 0; hq < Hq; ++hq) {
      int any = 0;
      for (int64_t r = 0; r < G; ++r)
        if (!mask || mask[n * Hv + hq * G + r]) any = 1;
      if (!any) continue;
      for (int64_t t = cu[n]; t < cu[n + 1]; ++t)
        for (int64_t i = 0; i < K; ++i) {
          double sq = 0.0, sk = 0.0;
          for (int64_t r = 0; r < G; ++r) {
            const int64_t h = hq * G + r;
            sq += dqh[(t * Hv + h) * K + i];
            sk += dkh[(t * Hv + h) * K + i];
          }
          dq[(t * Hq + hq) * K + i] = sq;
          dk[(t * Hq + hq) * K + i] = sk;
        }
    }
  free(dqh);
  free(dkh);
  return err;
}

/* ------------------------------------------------------------------------ */
/* Chunked form, naive fp64.                                                */
/*                                                                          */
/* Inside a chunk of Cc tokens with start state S (gamma = cumsum of g from */
/* the chunk start, Gam_ri = exp(gamma_r - gamma_i) for i <= r):            */
/*   M = strict lower part of diag(beta) (K K^T) o Gam                      */
/*   A = (I + M)^{-1}                (forward substitution)                 */
/*   X = diag(beta e^gamma) K,  Y = diag(beta) V,   R = Y - X S             */
/*   Delta = A R                      (= U - W S with W = A X, U = A Y)     */
/*   O = scale (diag(e^gamma) Q S + lower_incl(Q K^T o Gam) Delta)          */
/*   S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma}) Delta               */
/* Unrolling the token recurrence inside the chunk gives exactly this, so   */
/* the chunked form equals the recurrence up to rounding.                   */
/* ------------------------------------------------------------------------ */

/* per-chunk scratch, sized for chunk C */
typedef struct {
  double *gam, *M, *A, *R, *D, *P, *X;
} chunk_ws;

static int ws_alloc(chunk_ws* w, int64_t C, int64_t K, int64_t V) {
  w->gam = (double*)malloc(sizeof(double) * C);
  w->M = (double*)malloc(sizeof(double) * C * C);
  w->A = (double*)malloc(sizeof(double) * C * C);
  w->R = (double*)malloc(sizeof(double) * C * V);
  w->D = (double*)malloc(sizeof(double) * C * V);
  w->P = (double*)malloc(sizeof(double) * C * C);
  w->X = (double*)malloc(sizeof(double) * C * K);
  return (w->gam && w->M && w->A && w->R && w->D && w->P && w->X) ? 0 : -2;
}
static void ws_free(chunk_ws* w) {
  free(w->gam); free(w->M); free(w->A); free(w->R); free(w->D); free(w->P); free(w->X);
}

/* Forward quantities of one chunk: gam, M, A, X, R, Delta(D), P.
   Rows of the chunk are tokens ts .. ts+Cc-1. */
static void chunk_forward_terms(chunk_ws* w, int64_t Cc, int64_t ts, int64_t h, int64_t hq,
                                int64_t Hq, int64_t Hv, int64_t K, int64_t V, const double* q,
                                const double* k, const double* v, const double* g,
                                const double* beta, const double* S) {
  double acc = 0.0;
  for (int64_t r = 0; r < Cc; ++r) {
    acc += g[(ts + r) * Hv + h];
    w->gam[r] = acc;
  }
  for (int64_t r = 0; r < Cc; ++r) {
    const double* kr = k + ((ts + r) * Hq + hq) * K;
    const double* qr = q + ((ts + r) * Hq + hq) * K;
    const double br = beta[(ts + r) * Hv + h];
    for (int64_t i = 0; i < Cc; ++i) {
      const double* ki = k + ((ts + i) * Hq + hq) * K;
      double kk = 0.0, qk = 0.0;
      for (int64_t c = 0; c < K; ++c) {
        kk += kr[c] * ki[c];
        qk += qr[c] * ki[c];
      }
      const double gm = (i <= r) ? exp(w->gam[r] - w->gam[i]) : 0.0;
      w->M[r * Cc + i] = (i < r) ? br * kk * gm : 0.0;
      w->P[r * Cc + i] = (i <= r) ? qk * gm : 0.0;
    }
  }
  /* A = (I + M)^{-1}: row r of (I+M) A = I gives
     A[r][j] = [r==j] - sum_{j <= i < r} M[r][i] A[i][j]                     */
  for (int64_t r = 0; r < Cc; ++r)
    for (int64_t j = 0; j < Cc; ++j) {
      if (j > r) {
        w->A[r * Cc + j] = 0.0;
        continue;
      }
      double s = (r == j) ? 1.0 : 0.0;
      for (int64_t i = j; i < r; ++i) s -= w->M[r * Cc + i] * w->A[i * Cc + j];
      w->A[r * Cc + j] = s;
    }
  for (int64_t r = 0; r < Cc; ++r) {
    const double* kr = k + ((ts + r) * Hq + hq) * K;
    const double* vr = v + ((ts + r) * Hv + h) * V;
    const double br = beta[(ts + r) * Hv + h];
    const double xs = br * exp(w->gam[r]);
    for (int64_t c = 0; c < K; ++c) w->X[r * K + c] = xs * kr[c];
    for (int64_t j = 0; j < V; ++j) {
      double xsum = 0.0;
      for (int64_t c = 0; c < K; ++c) xsum += w->X[r * K + c] * S[c * V + j];
      w->R[r * V + j] = br * vr[j] - xsum;
    }
  }
  for (int64_t r = 0; r < Cc; ++r)
    for (int64_t j = 0; j < V; ++j) {
      double s = 0.0;
      for (int64_t i = 0; i <= r; ++i) s += w->A[r * Cc + i] * w->R[i * V + j];
      w->D[r * V + j] = s;
    }
}

/* S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma}) Delta */
static void chunk_state_update(chunk_ws* w, int64_t Cc, int64_t ts, int64_t hq, int64_t Hq,
                               int64_t K, int64_t V, const double* k, double* S) {
  const double gL = w->gam[Cc - 1];
  const double aL = exp(gL);
  for (int64_t c = 0; c < K; ++c)
    for (int64_t j = 0; j < V; ++j) {
      double s = aL * S[c * V + j];
      for (int64_t i = 0; i < Cc; ++i)
        s += exp(gL - w->gam[i]) * k[((ts + i) * Hq + hq) * K + c] * w->D[i * V + j];
      S[c * V + j] = s;
    }
}

int oracle_chunked_fwd(int64_t N, const int64_t* cu, int64_t Hq, int64_t Hv, int64_t K, int64_t V,
                       int64_t C, const double* q, const double* k, const double* v,
                       const double* g, const double* beta, double scale, const double* h0,
                       double* gcum, double* Aout, double* o, double* hout, double* ht,
                       const uint8_t* mask, int nthreads) {
  if (bad_args(N, cu, Hq, Hv, K, V) || C <= 0) return -1;
  set_threads(nthreads);
  const int64_t G = Hv / Hq;
  /* chunk offsets for the h output: off[n] = sum_{m<n} ceil(len_m / C) */
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
  if (!off) return -2;
  off[0] = 0;
  for (int64_t n = 0; n < N; ++n) off[n + 1] = off[n] + (cu[n + 1] - cu[n] + C - 1) / C;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < N * Hv; ++u) {
    if (mask && !mask[u]) continue;
    const int64_t n = u / Hv, h = u % Hv, hq = h / G;
    const size_t KV = (size_t)(K * V);
    chunk_ws w;
    double* S = (double*)malloc(sizeof(double) * KV);
    if (ws_alloc(&w, C, K, V) || !S) {
      err = -2;
      ws_free(&w);
      free(S);
      continue;
    }
    if (h0) memcpy(S, h0 + u * KV, sizeof(double) * KV);
    else memset(S, 0, sizeof(double) * KV);
    int64_t c = 0;
    for (int64_t ts = cu[n]; ts < cu[n + 1]; ts += C, ++c) {
      const int64_t Cc = (cu[n + 1] - ts < C) ? cu[n + 1] - ts : C;
      if (hout) memcpy(hout + ((off[n] + c) * Hv + h) * KV, S, sizeof(double) * KV);
      chunk_forward_terms(&w, Cc, ts, h, hq, Hq, Hv, K, V, q, k, v, g, beta, S);
      for (int64_t r = 0; r < Cc; ++r) {
        if (gcum) gcum[(ts + r) * Hv + h] = w.gam[r];
        if (Aout)
          for (int64_t i = 0; i < C; ++i)
            Aout[((ts + r) * Hv + h) * C + i] = (i < Cc) ? w.A[r * Cc + i] : 0.0;
        const double* qr = q + ((ts + r) * Hq + hq) * K;
        const double er = exp(w.gam[r]);
        for (int64_t j = 0; j < V; ++j) {
          double qs = 0.0, pd = 0.0;
          for (int64_t cc = 0; cc < K; ++cc) qs += qr[cc] * S[cc * V + j];
          for (int64_t i = 0; i <= r; ++i) pd += w.P[r * Cc + i] * w.D[i * V + j];
          o[((ts + r) * Hv + h) * V + j] = scale * (er * qs + pd);
        }
      }
      chunk_state_update(&w, Cc, ts, hq, Hq, K, V, k, S);
    }
    if (ht) memcpy(ht + u * KV, S, sizeof(double) * KV);
    ws_free(&w);
    free(S);
  }
  free(off);
  return err;
}

/* ------------------------------------------------------------------------ */
/* Chunked form, backward (reverse over chunks).  dSn is the gradient with  */
/* respect to the chunk's end state; per chunk, with dP_ri = scale do_r .   */
/* Delta_i (i <= r) and E_ri the elementwise products named below:          */
/*   dDelta = diag(e^{gL-gamma}) K dSn + scale lower_incl(P)^T dO           */
/*   dR = A^T dDelta                                                        */
/*   dS = e^{gL} dSn + scale (diag(e^gamma) Q)^T dO - X^T dR                */
/*   dq_r = scale e^{g_r} S do_r + sum_i dP_ri Gam_ri k_i                   */
/*   dk_i += sum_r dP_ri Gam_ri q_r + e^{gL-g_i} dSn Delta_i                */
/*   dA = dDelta R^T ; dM = strict_lower(-A^T dA A^T)                       */
/*   dv_r = beta_r dR_r ; dX = -dR S^T ; dk_r += beta_r e^{g_r} dX_r        */
/*   dbeta_r = v_r.dR_r + e^{g_r} k_r.dX_r + sum_{i<r} dM_ri (k_r.k_i) Gam_ri*/
/*   dk += (dM o beta Gam) K + (dM o beta Gam)^T K                          */
/*   dgamma_r: + scale e^{g_r} q_r^T S do_r + rowsum(dP o P) - colsum(dP o P)*/
/*             + rowsum(dM o M) - colsum(dM o M) + beta_r e^{g_r} k_r.dX_r   */
/*             - F_r, and the last row adds sum_i F_i + e^{gL} <S, dSn>,     */
/*             F_i = e^{gL-g_i} k_i^T dSn Delta_i                            */
/*   dg = reverse cumsum of dgamma inside the chunk                         */
/* ------------------------------------------------------------------------ */
int oracle_chunked_bwd(int64_t N, const int64_t* cu, int64_t Hq, int64_t Hv, int64_t K, int64_t V,
                       int64_t C, const double* q, const double* k, const double* v,
                       const double* g, const double* beta, double scale, const double* h0,
                       const double* dO, const double* dht, double* dq, double* dk, double* dv,
                       double* dbeta, double* dg, double* dh0, const uint8_t* mask, int nthreads) {
  if (bad_args(N, cu, Hq, Hv, K, V) || C <= 0) return -1;
  set_threads(nthreads);
  const int64_t G = Hv / Hq;
  const int64_t Ttot = cu[N];
  double* dqh = (double*)calloc((size_t)(Ttot * Hv * K + 1), sizeof(double));
  double* dkh = (double*)calloc((size_t)(Ttot * Hv * K + 1), sizeof(double));
  if (!dqh || !dkh) {
    free(dqh);
    free(dkh);
    return -2;
  }
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < N * Hv; ++u) {
    if (mask && !mask[u]) continue;
    const int64_t n = u / Hv, h = u % Hv, hq = h / G;
    const size_t KV = (size_t)(K * V);
    const int64_t L = cu[n + 1] - cu[n];
    const int64_t nch = (L + C - 1) / C;
    chunk_ws w;
    double* Ss = (double*)malloc(sizeof(double) * KV * (size_t)(nch + 1));
    double* dS = (double*)malloc(sizeof(double) * KV);
    double* dSprev = (double*)malloc(sizeof(double) * KV);
    double* dD = (double*)malloc(sizeof(double) * C * V);
    double* dR = (double*)malloc(sizeof(double) * C * V);
    double* dA = (double*)malloc(sizeof(double) * C * C);
    double* T1 = (double*)malloc(sizeof(double) * C * C);
    double* dM = (double*)malloc(sizeof(double) * C * C);
    double* dX = (double*)malloc(sizeof(double) * C * K);
    double* dgam = (double*)malloc(sizeof(double) * C);
    if (ws_alloc(&w, C, K, V) || !Ss || !dS || !dSprev || !dD || !dR || !dA || !T1 || !dM ||
        !dX || !dgam) {
      err = -2;
      ws_free(&w);
      free(Ss); free(dS); free(dSprev); free(dD); free(dR); free(dA); free(T1); free(dM);
      free(dX); free(dgam);
      continue;
    }
    /* forward: chunk-start states */
    if (h0) memcpy(Ss, h0 + u * KV, sizeof(double) * KV);
    else memset(Ss, 0, sizeof(double) * KV);
    for (int64_t c = 0; c < nch; ++c) {
      const int64_t ts = cu[n] + c * C;
      const int64_t Cc = (cu[n + 1] - ts < C) ? cu[n + 1] - ts : C;
      memcpy(Ss + (size_t)(c + 1) * KV, Ss + (size_t)c * KV, sizeof(double) * KV);
      chunk_forward_terms(&w, Cc, ts, h, hq, Hq, Hv, K, V, q, k, v, g, beta, Ss + (size_t)c * KV);
      chunk_state_update(&w, Cc, ts, hq, Hq, K, V, k, Ss + (size_t)(c + 1) * KV);
    }
    if (dht) memcpy(dS, dht + u * KV, sizeof(double) * KV);
    else memset(dS, 0, sizeof(double) * KV);
    for (int64_t c = nch - 1; c >= 0; --c) {
      const int64_t ts = cu[n] + c * C;
      const int64_t Cc = (cu[n + 1] - ts < C) ? cu[n + 1] - ts : C;
      const double* S = Ss + (size_t)c * KV;
      chunk_forward_terms(&w, Cc, ts, h, hq, Hq, Hv, K, V, q, k, v, g, beta, S);
      const double gL = w.gam[Cc - 1], aL = exp(gL);
      for (int64_t r = 0; r < Cc; ++r) dgam[r] = 0.0;
      /* dDelta */
      for (int64_t i = 0; i < Cc; ++i) {
        const double* ki = k + ((ts + i) * Hq + hq) * K;
        const double di = exp(gL - w.gam[i]);
        for (int64_t j = 0; j < V; ++j) {
          double s1 = 0.0, s2 = 0.0;
          for (int64_t c2 = 0; c2 < K; ++c2) s1 += ki[c2] * dS[c2 * V + j];
          for (int64_t r = i; r < Cc; ++r) s2 += w.P[r * Cc + i] * dO[((ts + r) * Hv + h) * V + j];
          dD[i * V + j] = di * s1 + scale * s2;
        }
      }
      /* dR = A^T dDelta */
      for (int64_t i = 0; i < Cc; ++i)
        for (int64_t j = 0; j < V; ++j) {
          double s = 0.0;
          for (int64_t r = i; r < Cc; ++r) s += w.A[r * Cc + i] * dD[r * V + j];
          dR[i * V + j] = s;
        }
      /* dS for the previous chunk */
      for (int64_t c2 = 0; c2 < K; ++c2)
        for (int64_t j = 0; j < V; ++j) {
          double s = aL * dS[c2 * V + j];
          for (int64_t r = 0; r < Cc; ++r) {
            const double qrc = q[((ts + r) * Hq + hq) * K + c2];
            s += scale * exp(w.gam[r]) * qrc * dO[((ts + r) * Hv + h) * V + j];
            s -= w.X[r * K + c2] * dR[r * V + j];
          }
          dSprev[c2 * V + j] = s;
        }
      /* output path: dq, dk from P, dgamma from P and from Q~ */
      for (int64_t r = 0; r < Cc; ++r) {
        const double* qr = q + ((ts + r) * Hq + hq) * K;
        const double* dor = dO + ((ts + r) * Hv + h) * V;
        const double er = exp(w.gam[r]);
        double* dqr = dqh + ((ts + r) * Hv + h) * K;
        for (int64_t c2 = 0; c2 < K; ++c2) {
          double s = 0.0;
          for (int64_t j = 0; j < V; ++j) s += S[c2 * V + j] * dor[j];
          dqr[c2] += scale * er * s;
        }
        double qsd = 0.0;
        for (int64_t c2 = 0; c2 < K; ++c2)
          for (int64_t j = 0; j < V; ++j) qsd += qr[c2] * S[c2 * V + j] * dor[j];
        dgam[r] += scale * er * qsd;
        for (int64_t i = 0; i <= r; ++i) {
          double dp = 0.0;
          for (int64_t j = 0; j < V; ++j) dp += dor[j] * w.D[i * V + j];
          dp *= scale;
          const double gm = exp(w.gam[r] - w.gam[i]);
          const double* ki = k + ((ts + i) * Hq + hq) * K;
          double* dki = dkh + ((ts + i) * Hv + h) * K;
          for (int64_t c2 = 0; c2 < K; ++c2) {
            dqr[c2] += dp * gm * ki[c2];
            dki[c2] += dp * gm * qr[c2];
          }
          const double E = dp * w.P[r * Cc + i];
          dgam[r] += E;
          dgam[i] -= E;
        }
      }
      /* state path: dk and dgamma from S_end */
      {
        double Fsum = 0.0;
        for (int64_t i = 0; i < Cc; ++i) {
          const double di = exp(gL - w.gam[i]);
          const double* ki = k + ((ts + i) * Hq + hq) * K;
          double* dki = dkh + ((ts + i) * Hv + h) * K;
          double F = 0.0;
          for (int64_t c2 = 0; c2 < K; ++c2) {
            double s = 0.0;
            for (int64_t j = 0; j < V; ++j) s += dS[c2 * V + j] * w.D[i * V + j];
            dki[c2] += di * s;
            F += ki[c2] * s;
          }
          F *= di;
          dgam[i] -= F;
          Fsum += F;
        }
        double sds = 0.0;
        for (size_t x = 0; x < KV; ++x) sds += S[x] * dS[x];
        dgam[Cc - 1] += Fsum + aL * sds;
      }
      /* WY path: dA, dX, dY */
      for (int64_t r = 0; r < Cc; ++r)
        for (int64_t i = 0; i < Cc; ++i) {
          double s = 0.0;
          for (int64_t j = 0; j < V; ++j) s += dD[r * V + j] * w.R[i * V + j];
          dA[r * Cc + i] = s;
        }
      for (int64_t r = 0; r < Cc; ++r) {
        const double* kr = k + ((ts + r) * Hq + hq) * K;
        const double* vr = v + ((ts + r) * Hv + h) * V;
        const double br = beta[(ts + r) * Hv + h];
        const double er = exp(w.gam[r]);
        double dbv = 0.0;
        for (int64_t j = 0; j < V; ++j) {
          dv[((ts + r) * Hv + h) * V + j] = br * dR[r * V + j];
          dbv += vr[j] * dR[r * V + j];
        }
        double kdx = 0.0;
        double* dkr = dkh + ((ts + r) * Hv + h) * K;
        for (int64_t c2 = 0; c2 < K; ++c2) {
          double s = 0.0;
          for (int64_t j = 0; j < V; ++j) s += dR[r * V + j] * S[c2 * V + j];
          dX[r * K + c2] = -s;
          dkr[c2] += br * er * dX[r * K + c2];
          kdx += kr[c2] * dX[r * K + c2];
        }
        dbeta[(ts + r) * Hv + h] = dbv + er * kdx;
        dgam[r] += br * er * kdx;
      }
      /* dM = strict_lower(-A^T dA A^T) */
      for (int64_t r = 0; r < Cc; ++r)
        for (int64_t i = 0; i < Cc; ++i) {
          double s = 0.0;
          for (int64_t m = 0; m < Cc; ++m) s += w.A[m * Cc + r] * dA[m * Cc + i];
          T1[r * Cc + i] = s; /* A^T dA */
        }
      for (int64_t r = 0; r < Cc; ++r)
        for (int64_t i = 0; i < Cc; ++i) {
          if (i >= r) {
            dM[r * Cc + i] = 0.0;
            continue;
          }
          double s = 0.0;
          for (int64_t m = 0; m < Cc; ++m) s += T1[r * Cc + m] * w.A[i * Cc + m];
          dM[r * Cc + i] = -s;
        }
      for (int64_t r = 0; r < Cc; ++r) {
        const double* kr = k + ((ts + r) * Hq + hq) * K;
        const double br = beta[(ts + r) * Hv + h];
        double* dkr = dkh + ((ts + r) * Hv + h) * K;
        for (int64_t i = 0; i < r; ++i) {
          const double* ki = k + ((ts + i) * Hq + hq) * K;
          double* dki = dkh + ((ts + i) * Hv + h) * K;
          const double gm = exp(w.gam[r] - w.gam[i]);
          double kk = 0.0;
          for (int64_t c2 = 0; c2 < K; ++c2) kk += kr[c2] * ki[c2];
          dbeta[(ts + r) * Hv + h] += dM[r * Cc + i] * kk * gm;
          const double coef = dM[r * Cc + i] * br * gm;
          for (int64_t c2 = 0; c2 < K; ++c2) {
            dkr[c2] += coef * ki[c2];
            dki[c2] += coef * kr[c2];
          }
          const double E2 = dM[r * Cc + i] * w.M[r * Cc + i];
          dgam[r] += E2;
          dgam[i] -= E2;
        }
      }
      /* dg = reverse cumsum of dgamma */
      {
        double s = 0.0;
        for (int64_t r = Cc - 1; r >= 0; --r) {
          s += dgam[r];
          dg[(ts + r) * Hv + h] = s;
        }
      }
      memcpy(dS, dSprev, sizeof(double) * KV);
    }
    if (dh0) memcpy(dh0 + u * KV, dS, sizeof(double) * KV);
    ws_free(&w);
    free(Ss); free(dS); free(dSprev); free(dD); free(dR); free(dA); free(T1); free(dM);
    free(dX); free(dgam);
  }
  for (int64_t n = 0; n < N; ++n)
    for (int64_t hq = 0; hq < Hq; ++hq) {
      int any = 0;
      for (int64_t r = 0; r < G; ++r)
        if (!mask || mask[n * Hv + hq * G + r]) any = 1;
      if (!any) continue;
      for (int64_t t = cu[n]; t < cu[n + 1]; ++t)
        for (int64_t i = 0; i < K; ++i) {
          double sq = 0.0, sk = 0.0;
          for (int64_t r = 0; r < G; ++r) {
            const int64_t hh = hq * G + r;
            sq += dqh[(t * Hv + hh) * K + i];
            sk += dkh[(t * Hv + hh) * K + i];
          }
          dq[(t * Hq + hq) * K + i] = sq;
          dk[(t * Hq + hq) * K + i] = sk;
        }
    }
  free(dqh);
  free(dkh);
  return err;
}
