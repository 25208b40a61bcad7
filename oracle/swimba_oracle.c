/*
 * swimba_oracle.c -- plain, slow, fp64 CPU oracle for the Swimba
 * (Switch Mamba) parameter-space mixture-of-experts selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * Pages cited (by title and section):
 *   [SW] "Swimba: Switch Mamba Model Scales State Space Models"
 *        (gist.science summaries in Spanish, Dutch and French).  The Dutch
 *        technical summary, section "Kernmechanisme van Swimba", writes the
 *        mixed recurrence; the French summary, "Fondements Théoriques", states
 *        Theorems 1-4.
 *   [MB] "Mamba y las SSMs: el retorno del estado persistente", sections
 *        "SSMs - Modelos de espacios de estados" (the linear state/output
 *        equations with the D feed-through) and "Mamba" (selective B_t, C_t,
 *        the zero-order-hold transition exp(Delta_t A), Figure 2: Delta as the
 *        forgetting factor).
 *
 * What is computed (one channel d of one sequence b; N state entries):
 *   router     l_e = sum_d x_d Wr[d,e]; the k largest (ties: lower e first);
 *              gates = softmax over the k selected logits (convex weights).
 *   mixing     Abar[n] = sum_j g_j A[e_j,d,n], beta = sum_j g_j bias[e_j,d],
 *              delta = sum_j g_j Dskip[e_j,d]      (parameters mixed, [SW])
 *   discretise Delta = softplus(dt_raw + beta); a[n] = exp(Delta Abar[n])
 *              ([MB] "Mamba": transition exp(Delta A)); injection
 *              Delta * B[t,n] * x (Euler form of the input term), or with
 *              zoh = 1 the zero-order hold (exp(Delta Abar) - 1)/Abar * B x
 *              ([MB] "Mamba": B_bar = A^{-1}(exp(Delta A) - I) B)
 *   recurrence h[n] <- a[n] h[n] + Delta B[t,n] x      ([MB], [SW])
 *   readout    y = sum_n C[t,n] h[n] + delta x          (after the update)
 * The separate design keeps one state per expert and advances only the
 * selected ones ([SW] the two MoE-SSM designs; Theorem 4).  The stream-mixed
 * form (ref_scan_streams) shares A and mixes the experts' B X injections and
 * C readouts instead ([SW] "Kernmechanisme van Swimba").
 *
 * Readings where the pages are silent are listed in the design document:
 * Euler injection, bias mixed before softplus, gates = softmax over the top
 * k, equal logits broken towards the lower expert index, zero initial state.
 *
 * Every loop is the definition written out, in fp64, in the order the
 * definition states it.  OpenMP runs independent (b,d) channels (and
 * independent tokens in the router) in parallel; that changes no result.
 */
#include <math.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>

/* Stable softplus, log(1 + exp(z)) = max(z,0) + log1p(exp(-|z|)). */
static double softplus(double z) {
  return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
}

/*
 * Coefficient of B_t x in the discretised input term of one state entry with
 * transition Abar:
 *   zoh == 0: Euler, Delta (the form the scans use by default);
 *   zoh == 1: zero-order hold, B_bar = A^{-1}(exp(Delta A) - I) B ([MB]
 *             "Mamba", the discretised state equations), i.e. the coefficient
 *             (exp(Delta Abar) - 1) / Abar, which tends to Delta as Abar -> 0.
 */
static double input_coeff(double Dt, double Abar, int zoh) {
  if (!zoh) return Dt;
  double z = Dt * Abar;
  return z == 0.0 ? Dt : expm1(z) / Abar;
}

/* ---------------------------------------------------------------- router */
/*
 * ref_route: per token t of T, logits over E experts, the top k and their
 * gates ([SW] Dutch summary "Kernmechanisme": a router computes per-token
 * weights pi_t over the active experts, e.g. top-1 or top-k).
 *   x      [T, D]   token features (the scanned input)
 *   Wr     [D, E]   router weights
 *   idx    [T, k]   out: selected experts, largest logit first
 *   gate   [T, k]   out: softmax over the selected logits
 *   logits [T, E]   out (may be NULL): the fp64 logits
 *   absdot [T, E]   out (may be NULL): sum_d |x_d Wr[d,e]|, the magnitude
 *                   that bounds the rounding error of any float summation
 */
void ref_route(int64_t T, int D, int E, int k, const double* x,
               const double* Wr, int32_t* idx, double* gate, double* logits,
               double* absdot) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* l = (double*)malloc(sizeof(double) * (size_t)E);
    int* taken = (int*)calloc((size_t)E, sizeof(int));
    for (int e = 0; e < E; ++e) {
      double s = 0.0, sa = 0.0;
      for (int d = 0; d < D; ++d) {
        double p = x[t * D + d] * Wr[(int64_t)d * E + e];
        s += p;
        sa += fabs(p);
      }
      l[e] = s;
      if (logits) logits[t * E + e] = s;
      if (absdot) absdot[t * E + e] = sa;
    }
    /* top-k by (logit descending, index ascending) */
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      idx[t * k + j] = best;
    }
    /* softmax restricted to the selected experts */
    double m = l[idx[t * k + 0]];
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp(l[idx[t * k + j]] - m);
    for (int j = 0; j < k; ++j) gate[t * k + j] = exp(l[idx[t * k + j]] - m) / z;
    free(l);
    free(taken);
  }
}

/* ----------------------------------------------------------- mixed scan */
/*
 * ref_scan: the parameter-space-mixed selective scan, one state trajectory
 * per (b,d) ([SW] "Kernmechanisme van Swimba"; Theorem 1: one selective SSM).
 *   x, dt_raw [B, L, D]     inputs and pre-activation step sizes
 *   Bm, Cm    [B, L, N]     selective input / output vectors B_t, C_t
 *   idx, gate [B, L, k]     routing (from ref_route or forced)
 *   A         [E, D, N]     per-expert diagonal transitions (negative)
 *   dt_bias   [E, D]        per-expert step-size bias
 *   Dskip     [E, D]        per-expert feed-through D
 *   h0        [B, D, N]     initial state, or NULL for zeros
 *   y         [B, L, D]     out
 *   h_final   [B, D, N]     out, or NULL
 *   zoh       0: Euler input term Delta B x; 1: zero-order hold (input_coeff)
 */
void ref_scan(int B, int L, int D, int N, int E, int k, const double* x,
              const double* dt_raw, const double* Bm, const double* Cm,
              const int32_t* idx, const double* gate, const double* A,
              const double* dt_bias, const double* Dskip, const double* h0,
              double* y, double* h_final, int zoh) {
  (void)E;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int d = 0; d < D; ++d) {
      double* h = (double*)malloc(sizeof(double) * (size_t)N);
      for (int n = 0; n < N; ++n)
        h[n] = h0 ? h0[((int64_t)b * D + d) * N + n] : 0.0;
      for (int t = 0; t < L; ++t) {
        int64_t bt = (int64_t)b * L + t;
        const int32_t* e = idx + bt * k;
        const double* g = gate + bt * k;
        double xv = x[bt * D + d];
        /* mixed per-token parameters */
        double beta = 0.0, delta = 0.0;
        for (int j = 0; j < k; ++j) {
          beta += g[j] * dt_bias[(int64_t)e[j] * D + d];
          delta += g[j] * Dskip[(int64_t)e[j] * D + d];
        }
        double Dt = softplus(dt_raw[bt * D + d] + beta);
        double yv = 0.0;
        for (int n = 0; n < N; ++n) {
          double Abar = 0.0;
          for (int j = 0; j < k; ++j)
            Abar += g[j] * A[((int64_t)e[j] * D + d) * N + n];
          double a = exp(Dt * Abar);
          double bb = input_coeff(Dt, Abar, zoh) * Bm[bt * N + n] * xv;
          h[n] = a * h[n] + bb;
          yv += Cm[bt * N + n] * h[n];
        }
        y[bt * D + d] = yv + delta * xv;
      }
      if (h_final)
        for (int n = 0; n < N; ++n) h_final[((int64_t)b * D + d) * N + n] = h[n];
      free(h);
    }
  }
}

/* -------------------------------------------------------- separate scan */
/*
 * ref_scan_separate: the "MoE of separate SSMs" design: one state trajectory
 * per expert.  At token t, for each slot j (in slot order) the selected
 * expert e = idx[t,j] advances its own state with its own (unmixed)
 * parameters and emits y_e; the token's output is sum_j g_j y_e.  Experts
 * not selected at t keep their state unchanged ([SW] Spanish summary
 * "Distinción de Diseños", French "Distinction des deux designs";
 * Theorem 4: the two designs differ once routing varies over time).
 *   h0, h_final [B, E, D, N] (NULL allowed); other arrays as ref_scan.
 */
void ref_scan_separate(int B, int L, int D, int N, int E, int k,
                       const double* x, const double* dt_raw,
                       const double* Bm, const double* Cm, const int32_t* idx,
                       const double* gate, const double* A,
                       const double* dt_bias, const double* Dskip,
                       const double* h0, double* y, double* h_final, int zoh) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int d = 0; d < D; ++d) {
      double* H = (double*)malloc(sizeof(double) * (size_t)E * N);
      for (int e = 0; e < E; ++e)
        for (int n = 0; n < N; ++n)
          H[e * N + n] = h0 ? h0[(((int64_t)b * E + e) * D + d) * N + n] : 0.0;
      for (int t = 0; t < L; ++t) {
        int64_t bt = (int64_t)b * L + t;
        double xv = x[bt * D + d];
        double yv = 0.0;
        for (int j = 0; j < k; ++j) {
          int e = idx[bt * k + j];
          double Dt = softplus(dt_raw[bt * D + d] + dt_bias[(int64_t)e * D + d]);
          double ye = 0.0;
          for (int n = 0; n < N; ++n) {
            double Ae = A[((int64_t)e * D + d) * N + n];
            double a = exp(Dt * Ae);
            H[e * N + n] = a * H[e * N + n] + input_coeff(Dt, Ae, zoh) * Bm[bt * N + n] * xv;
            ye += Cm[bt * N + n] * H[e * N + n];
          }
          ye += Dskip[(int64_t)e * D + d] * xv;
          yv += gate[bt * k + j] * ye;
        }
        y[bt * D + d] = yv;
      }
      if (h_final)
        for (int e = 0; e < E; ++e)
          for (int n = 0; n < N; ++n)
            h_final[(((int64_t)b * E + e) * D + d) * N + n] = H[e * N + n];
      free(H);
    }
  }
}

/*
 * ref_scan_slots: the other reading of separate trajectories: one state per
 * routing slot instead of per expert.  Slot j's state advances at every token
 * with the parameters of the expert selected in that slot, e = idx[t,j]
 * (its own A, dt_bias and Dskip, unmixed), and keeps its value across a change
 * of expert; y = sum_j g_j (C_t . h_j + Dskip[e,d] x).  The gates weight the
 * outputs only, never the states.  Where a slot keeps its expert for the whole
 * sequence this equals the per-expert trajectories of ref_scan_separate
 * ([SW] Spanish summary "Distinción de Diseños", French "Distinction des deux
 * designs": the designs differ in which state a selected expert advances).
 *   h0, h_final [B, k, D, N] (NULL allowed); other arrays as ref_scan.
 */
void ref_scan_slots(int B, int L, int D, int N, int E, int k,
                    const double* x, const double* dt_raw,
                    const double* Bm, const double* Cm, const int32_t* idx,
                    const double* gate, const double* A,
                    const double* dt_bias, const double* Dskip,
                    const double* h0, double* y, double* h_final, int zoh) {
  (void)E;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int d = 0; d < D; ++d) {
      double* H = (double*)malloc(sizeof(double) * (size_t)k * N);
      for (int j = 0; j < k; ++j)
        for (int n = 0; n < N; ++n)
          H[j * N + n] = h0 ? h0[(((int64_t)b * k + j) * D + d) * N + n] : 0.0;
      for (int t = 0; t < L; ++t) {
        int64_t bt = (int64_t)b * L + t;
        double xv = x[bt * D + d];
        double yv = 0.0;
        for (int j = 0; j < k; ++j) {
          const int64_t ed = (int64_t)idx[bt * k + j] * D + d;  /* (expert, channel) */
          double Dt = softplus(dt_raw[bt * D + d] + dt_bias[ed]);
          double yj = 0.0;
          for (int n = 0; n < N; ++n) {
            double Aj = A[ed * N + n];
            H[j * N + n] = exp(Dt * Aj) * H[j * N + n] +
                           input_coeff(Dt, Aj, zoh) * Bm[bt * N + n] * xv;
            yj += Cm[bt * N + n] * H[j * N + n];
          }
          yv += gate[bt * k + j] * (yj + Dskip[ed] * xv);
        }
        y[bt * D + d] = yv;
      }
      if (h_final)
        for (int j = 0; j < k; ++j)
          for (int n = 0; n < N; ++n)
            h_final[(((int64_t)b * k + j) * D + d) * N + n] = H[j * N + n];
      free(H);
    }
  }
}

/*
 * ref_scan_all_experts: the third reading of separate trajectories: every
 * expert keeps a state per channel and advances it at every token with its
 * own parameters, whether or not the router selected it; the router only
 * chooses whose outputs the token mixes, y = sum_j g_j y_{idx[t,j]} with
 * y_e = C_t . h_e + Dskip[e,d] x.  Each expert's trajectory is therefore a
 * plain selective scan with that expert's parameters, independent of the
 * routing, and the cost is E state updates per token instead of k
 * ([SW] Spanish summary "Distinción de Diseños", French "Distinction des
 * deux designs": separate SSMs, one per expert).
 *   h0, h_final [B, E, D, N] (NULL allowed); other arrays as ref_scan.
 */
void ref_scan_all_experts(int B, int L, int D, int N, int E, int k,
                          const double* x, const double* dt_raw,
                          const double* Bm, const double* Cm, const int32_t* idx,
                          const double* gate, const double* A,
                          const double* dt_bias, const double* Dskip,
                          const double* h0, double* y, double* h_final, int zoh) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int d = 0; d < D; ++d) {
      double* S = (double*)malloc(sizeof(double) * (size_t)E * N);  /* states [E][N] */
      double* out = (double*)malloc(sizeof(double) * (size_t)E);     /* y_e of token t */
      for (int e = 0; e < E; ++e)
        for (int n = 0; n < N; ++n)
          S[e * N + n] = h0 ? h0[(((int64_t)b * E + e) * D + d) * N + n] : 0.0;
      for (int t = 0; t < L; ++t) {
        const int64_t bt = (int64_t)b * L + t;
        const double u = x[bt * D + d];
        /* every expert advances */
        for (int e = 0; e < E; ++e) {
          const int64_t ed = (int64_t)e * D + d;
          const double step = softplus(dt_raw[bt * D + d] + dt_bias[ed]);
          double acc = Dskip[ed] * u;
          for (int n = 0; n < N; ++n) {
            const double an = A[ed * N + n];
            S[e * N + n] = exp(step * an) * S[e * N + n] +
                           input_coeff(step, an, zoh) * Bm[bt * N + n] * u;
            acc += Cm[bt * N + n] * S[e * N + n];
          }
          out[e] = acc;
        }
        /* the selected outputs, gate-weighted, in slot order */
        double yv = 0.0;
        for (int j = 0; j < k; ++j) yv += gate[bt * k + j] * out[idx[bt * k + j]];
        y[bt * D + d] = yv;
      }
      if (h_final)
        for (int e = 0; e < E; ++e)
          for (int n = 0; n < N; ++n)
            h_final[(((int64_t)b * E + e) * D + d) * N + n] = S[e * N + n];
      free(out);
      free(S);
    }
  }
}

/* ------------------------------------------------- stream-mixed scan */
/*
 * ref_scan_streams: the pages' own form of the mixed layer ([SW] Dutch
 * summary "Kernmechanisme van Swimba", French "Architecture de Swimba"):
 * every expert emits candidate streams B_t, C_t and an input X_t; the
 * transition A is shared by all experts; the state update mixes the
 * injections, h_t = A h_{t-1} + sum_e pi_{t,e} B^(e)_t X^(e)_t, and the
 * readout mixes the output vectors, y_t = (sum_e pi_{t,e} C^(e)_t)^T h_t.
 * The streams arrive per routing slot: slot j of token t holds the streams
 * of the j-th selected expert and pi_{t,e_j} = gate[t,j].
 * The shared transition is discretised as in the selective scan ([MB]
 * "Mamba"; [SW] Theorem 1, one selective SSM): the step size is not an
 * expert stream, so Delta = softplus(dt_raw + dt_bias) is shared, the
 * transition is exp(Delta A[d,n]) and the mixed injection enters as
 * Delta * sum_j g_j B_j[n] X_j[d].  The printed readout has no
 * feed-through term, so none is added.
 *   X        [B, L, k, D]   per-slot input streams
 *   dt_raw   [B, L, D]
 *   Bs, Cs   [B, L, k, N]   per-slot B and C streams
 *   gate     [B, L, k]
 *   A        [D, N]         shared diagonal transition (negative)
 *   dt_bias  [D]
 *   h0, h_final [B, D, N] (NULL allowed); y [B, L, D] out
 */
void ref_scan_streams(int B, int L, int D, int N, int k, const double* X,
                      const double* dt_raw, const double* Bs,
                      const double* Cs, const double* gate, const double* A,
                      const double* dt_bias, const double* h0, double* y,
                      double* h_final) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int d = 0; d < D; ++d) {
      double* h = (double*)malloc(sizeof(double) * (size_t)N);
      for (int n = 0; n < N; ++n)
        h[n] = h0 ? h0[((int64_t)b * D + d) * N + n] : 0.0;
      for (int t = 0; t < L; ++t) {
        int64_t bt = (int64_t)b * L + t;
        const double* g = gate + bt * k;
        double Dt = softplus(dt_raw[bt * D + d] + dt_bias[d]);
        double yv = 0.0;
        for (int n = 0; n < N; ++n) {
          double inj = 0.0, c = 0.0;
          for (int j = 0; j < k; ++j) {
            inj += g[j] * Bs[(bt * k + j) * N + n] * X[(bt * k + j) * D + d];
            c += g[j] * Cs[(bt * k + j) * N + n];
          }
          h[n] = exp(Dt * A[(int64_t)d * N + n]) * h[n] + Dt * inj;
          yv += c * h[n];
        }
        y[bt * D + d] = yv;
      }
      if (h_final)
        for (int n = 0; n < N; ++n) h_final[((int64_t)b * D + d) * N + n] = h[n];
      free(h);
    }
  }
}

/* ------------------------------------------------------ plain Mamba scan */
/*
 * ref_mamba_scan: the single-expert selective scan ([MB] "Mamba": state
 * update with exp(Delta_t A) and selective B_t, C_t; "SSMs": D feed-through).
 * Written independently of ref_scan so that the E = 1 and identical-expert
 * reductions (Theorem 1) compare two different pieces of code.
 *   A [D, N], dt_bias [D], Dskip [D]; h0, h_final [B, D, N] (NULL allowed).
 */
void ref_mamba_scan(int B, int L, int D, int N, const double* x,
                    const double* dt_raw, const double* Bm, const double* Cm,
                    const double* A, const double* dt_bias,
                    const double* Dskip, const double* h0, double* y,
                    double* h_final, int zoh) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int d = 0; d < D; ++d) {
      double* h = (double*)malloc(sizeof(double) * (size_t)N);
      for (int n = 0; n < N; ++n)
        h[n] = h0 ? h0[((int64_t)b * D + d) * N + n] : 0.0;
      for (int t = 0; t < L; ++t) {
        int64_t bt = (int64_t)b * L + t;
        double u = x[bt * D + d];
        double Dt = softplus(dt_raw[bt * D + d] + dt_bias[d]);
        double out = Dskip[d] * u;
        for (int n = 0; n < N; ++n) {
          double An = A[(int64_t)d * N + n];
          h[n] = exp(Dt * An) * h[n] + input_coeff(Dt, An, zoh) * Bm[bt * N + n] * u;
          out += Cm[bt * N + n] * h[n];
        }
        y[bt * D + d] = out;
      }
      if (h_final)
        for (int n = 0; n < N; ++n) h_final[((int64_t)b * D + d) * N + n] = h[n];
      free(h);
    }
  }
}

/* ------------------------------------------------------- mixed backward */
/*
 * ref_scan_backward: gradients of the mixed scan (ref_scan) for training
 * ([SW] French summary, "Résultats Expérimentaux": the Swimba layers are
 * trained).  Given dL/dy [B,L,D] and dL/dh_final [B,D,N] (NULL = 0), returns
 * dL/d of every input: dx, ddt_raw [B,L,D]; dBm, dCm [B,L,N] (summed over
 * channels); dgate [B,L,k] (summed over channels; the gates are taken as
 * free inputs); dA [E,D,N], dbias, dDskip [E,D] (summed over batch and
 * tokens); dh0 [B,D,N].
 * The adjoint of the state, lam_t = dL/dh_t, obeys the reverse recurrence
 *   lam_t = C_t dy_t + a_{t+1} lam_{t+1},   lam_{L-1} starts from dh_final,
 * and each forward quantity receives the chain rule of its one use:
 *   h_t = a_t h_{t-1} + Delta B_t x   ->  dx += lam Delta B, dB += lam Delta x,
 *                                          dDelta += lam (a Abar h_{t-1} + B x),
 *                                          dAbar += lam a Delta h_{t-1}
 *   y_t = C_t . h_t + delta x        ->  dC += dy h_t, dx += delta dy,
 *                                          ddelta = dy x
 *   Delta = softplus(z), z = dt_raw + beta  ->  dz = dDelta sigmoid(z)
 *   beta, delta, Abar = sum_j g_j (bias, Dskip, A)[e_j]  ->  per slot j:
 *     dbias[e_j] += g_j dz, dDskip[e_j] += g_j ddelta, dA[e_j] += g_j dAbar,
 *     dgate_j += bias[e_j] dz + Dskip[e_j] ddelta + A[e_j] . dAbar.
 * OpenMP splits the channels d (each thread owns the parameter gradients of
 * its channels, summed over b in order); the sums over channels are added
 * per thread and then in thread order.
 */
void ref_scan_backward(int B, int L, int D, int N, int E, int k,
                       const double* x, const double* dt_raw, const double* Bm,
                       const double* Cm, const int32_t* idx, const double* gate,
                       const double* A, const double* dt_bias,
                       const double* Dskip, const double* h0, const double* dy,
                       const double* dh_final, double* dx, double* ddt_raw,
                       double* dBm, double* dCm, double* dgate, double* dA,
                       double* dbias, double* dDskip, double* dh0) {
  const int64_t BL = (int64_t)B * L;
  const int64_t red = BL * (2 * N + k); /* per-thread sums over channels */
#ifdef _OPENMP
  const int nth = omp_get_max_threads();
#else
  const int nth = 1;
#endif
  double* part = (double*)calloc((size_t)nth * (size_t)red, sizeof(double));
  for (int64_t i = 0; i < (int64_t)E * D * N; ++i) dA[i] = 0.0;
  for (int64_t i = 0; i < (int64_t)E * D; ++i) dbias[i] = dDskip[i] = 0.0;
#pragma omp parallel
  {
#ifdef _OPENMP
    double* my = part + (size_t)omp_get_thread_num() * (size_t)red;
#else
    double* my = part;
#endif
    double* Dt = (double*)malloc(sizeof(double) * (size_t)L);
    double* zz = (double*)malloc(sizeof(double) * (size_t)L);
    double* Ab = (double*)malloc(sizeof(double) * (size_t)L * N);
    double* aa = (double*)malloc(sizeof(double) * (size_t)L * N);
    double* hh = (double*)malloc(sizeof(double) * (size_t)(L + 1) * N);
    double* lam = (double*)malloc(sizeof(double) * (size_t)N);
    double* dAbar = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(static)
    for (int d = 0; d < D; ++d) {
      for (int b = 0; b < B; ++b) {
        /* forward, keeping every state: hh[(t+1)N + n] = h_t, hh[n] = h_{-1} */
        for (int n = 0; n < N; ++n)
          hh[n] = h0 ? h0[((int64_t)b * D + d) * N + n] : 0.0;
        for (int t = 0; t < L; ++t) {
          int64_t bt = (int64_t)b * L + t;
          double beta = 0.0;
          for (int j = 0; j < k; ++j)
            beta += gate[bt * k + j] * dt_bias[(int64_t)idx[bt * k + j] * D + d];
          zz[t] = dt_raw[bt * D + d] + beta;
          Dt[t] = softplus(zz[t]);
          for (int n = 0; n < N; ++n) {
            double s = 0.0;
            for (int j = 0; j < k; ++j)
              s += gate[bt * k + j] * A[((int64_t)idx[bt * k + j] * D + d) * N + n];
            Ab[(int64_t)t * N + n] = s;
            aa[(int64_t)t * N + n] = exp(Dt[t] * s);
            hh[(int64_t)(t + 1) * N + n] = aa[(int64_t)t * N + n] * hh[(int64_t)t * N + n] +
                                           Dt[t] * Bm[bt * N + n] * x[bt * D + d];
          }
        }
        /* reverse */
        for (int n = 0; n < N; ++n)
          lam[n] = dh_final ? dh_final[((int64_t)b * D + d) * N + n] : 0.0;
        for (int t = L - 1; t >= 0; --t) {
          int64_t bt = (int64_t)b * L + t;
          double xv = x[bt * D + d], g_dy = dy[bt * D + d];
          double delta = 0.0;
          for (int j = 0; j < k; ++j)
            delta += gate[bt * k + j] * Dskip[(int64_t)idx[bt * k + j] * D + d];
          double dxv = delta * g_dy, dDt = 0.0;
          for (int n = 0; n < N; ++n) {
            const double ht = hh[(int64_t)(t + 1) * N + n], hp = hh[(int64_t)t * N + n];
            const double a = aa[(int64_t)t * N + n];
            lam[n] += Cm[bt * N + n] * g_dy;
            my[bt * (2 * N + k) + N + n] += g_dy * ht;                  /* dC */
            my[bt * (2 * N + k) + n] += lam[n] * Dt[t] * xv;            /* dB */
            dxv += lam[n] * Dt[t] * Bm[bt * N + n];
            dDt += lam[n] * (a * Ab[(int64_t)t * N + n] * hp + Bm[bt * N + n] * xv);
            dAbar[n] = lam[n] * a * Dt[t] * hp;
          }
          double sig = 1.0 / (1.0 + exp(-zz[t]));
          double dz = dDt * sig, ddelta = g_dy * xv;
          dx[bt * D + d] = dxv;
          ddt_raw[bt * D + d] = dz;
          for (int j = 0; j < k; ++j) {
            int e = idx[bt * k + j];
            double gj = gate[bt * k + j], s = 0.0;
            dbias[(int64_t)e * D + d] += gj * dz;
            dDskip[(int64_t)e * D + d] += gj * ddelta;
            for (int n = 0; n < N; ++n) {
              dA[((int64_t)e * D + d) * N + n] += gj * dAbar[n];
              s += A[((int64_t)e * D + d) * N + n] * dAbar[n];
            }
            my[bt * (2 * N + k) + 2 * N + j] +=
                dt_bias[(int64_t)e * D + d] * dz + Dskip[(int64_t)e * D + d] * ddelta + s;
          }
          for (int n = 0; n < N; ++n) lam[n] *= aa[(int64_t)t * N + n];
        }
        for (int n = 0; n < N; ++n) dh0[((int64_t)b * D + d) * N + n] = lam[n];
      }
    }
    free(Dt);
    free(zz);
    free(Ab);
    free(aa);
    free(hh);
    free(lam);
    free(dAbar);
  }
  for (int64_t i = 0; i < BL * N; ++i) dBm[i] = dCm[i] = 0.0;
  for (int64_t i = 0; i < BL * k; ++i) dgate[i] = 0.0;
  for (int th = 0; th < nth; ++th) {
    const double* p = part + (size_t)th * (size_t)red;
    for (int64_t bt = 0; bt < BL; ++bt) {
      for (int n = 0; n < N; ++n) {
        dBm[bt * N + n] += p[bt * (2 * N + k) + n];
        dCm[bt * N + n] += p[bt * (2 * N + k) + N + n];
      }
      for (int j = 0; j < k; ++j) dgate[bt * k + j] += p[bt * (2 * N + k) + 2 * N + j];
    }
  }
  free(part);
}

/* ------------------------------------------------------------ decode step */
/*
 * ref_step: one decoding step on a persistent state ([MB] Figure 2: the
 * state lives on and is updated once per token).  Routing comes from the
 * router on this token's x (when idx_in is NULL) or is forced.
 *   x, dt_raw [B, D]; Bm, Cm [B, N]; Wr [D, E]; idx_in, gate_in [B, k] or NULL
 *   state [B, D, N] in/out; y [B, D] out; idx_out, gate_out [B, k] out
 *   (may be NULL).
 */
void ref_step(int B, int D, int N, int E, int k, const double* x,
              const double* dt_raw, const double* Bm, const double* Cm,
              const double* Wr, const int32_t* idx_in, const double* gate_in,
              const double* A, const double* dt_bias, const double* Dskip,
              double* state, double* y, int32_t* idx_out, double* gate_out,
              int zoh) {
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * k);
  double* gate = (double*)malloc(sizeof(double) * (size_t)B * k);
  if (idx_in) {
    for (int64_t i = 0; i < (int64_t)B * k; ++i) {
      idx[i] = idx_in[i];
      gate[i] = gate_in[i];
    }
  } else {
    ref_route(B, D, E, k, x, Wr, idx, gate, NULL, NULL);
  }
  /* a step is the scan over a sequence of length one, state carried */
  ref_scan(B, 1, D, N, E, k, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip,
           state, y, state, zoh);
  if (idx_out)
    for (int64_t i = 0; i < (int64_t)B * k; ++i) idx_out[i] = idx[i];
  if (gate_out)
    for (int64_t i = 0; i < (int64_t)B * k; ++i) gate_out[i] = gate[i];
  free(idx);
  free(gate);
}

/* Threads the parallel loops above use (for reporting the CPU baseline). */
#ifdef _OPENMP
int ref_num_threads(void) { return omp_get_max_threads(); }
#else
int ref_num_threads(void) { return 1; }
#endif
