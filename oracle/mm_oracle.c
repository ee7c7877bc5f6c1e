/*
 * mm_oracle.c -- plain, slow, fp64 CPU oracle for the Matryoshka-sliced
 * conv1d+SiLU and selective scan (SSD).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; it is written from the pages, not from the kernels.
 *
 * Sources (pages as titled):
 *  - "MatMamba: A Matryoshka State Space Model" (arXiv 2410.06718), the
 *    paragraph that decomposes the Mamba2 block into input projection, a
 *    causal 1-D convolution of kernel size 4 whose weights concatenate the
 *    x, B and C filters, a chunk + selective scan (SSM) with learnable A and D,
 *    and the SiLU nonlinearity sigma that follows the convolution.
 *  - same page, the nesting paragraph: a sub-block M_i uses W[0:d_i] along
 *    d_inner and A[0:h_i] along heads, h_i = d_i / d_head, d_i = e * m_i.
 *  - "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 *    (digest page), Proposed Method / Sampling Rule: the selective SSM updates
 *    the hidden state with input-dependent discretised parameters; Ablations:
 *    real-valued parameters, Delta (dt), B and C selective.
 *
 * The display equations of the block did not survive on the MatMamba page.
 * The recurrence taken here is the plain Mamba2 (SSD) reading, one real
 * scalar A_h and D_h per head, Euler-discretised input:
 *     H_t = exp(dt_t * A_h) * H_{t-1} + dt_t * x_t (outer) B_t      (P x N)
 *     y_t = H_t . C_t + D_h * x_t                                     (P)
 * computed token by token in fp64, with no chunking, blocking or reordering.
 *
 * Layouts (all dense, row-major, fp64):
 *   x  (batch, seqlen, n_heads, P)      dt (batch, seqlen, n_heads)
 *   B, C (batch, seqlen, ngroups, N)    A, D (n_heads)
 *   state (batch, n_heads, P, N)        y  (batch, seqlen, n_heads, P)
 *   conv input/output (batch, seqlen, conv_dim), conv_dim = d_inner + 2*ngroups*N,
 *   channel order [x | B | C];  conv weights (conv_dim, 4), tap 3 = current token;
 *   conv state (batch, conv_dim, 3), oldest input first.
 * Head h belongs to group h / (n_heads / ngroups).
 * Per-sequence activity: heads_active[b] heads are active in sequence b; the
 * conv's active channels are c < heads_active[b]*P (x part) and c >= d_inner
 * (B and C are shared by all heads and never sliced).  Inactive outputs and
 * states are left untouched.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* SiLU(v) = v * sigmoid(v), the nonlinearity the MatMamba block paragraph
 * names after the convolution. */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/*
 * Causal depthwise convolution with 4 taps followed by SiLU, per channel:
 *   pre[t,c] = bias[c] + sum_{k=0..3} w[c,k] * u[t-3+k, c]
 *   out[t,c] = SiLU(pre[t,c])
 * where u[tau<0, c] is conv_state[c, tau+3] when a state is given, else 0.
 * The new state is the last three inputs u[l-3..l-1] (from the old state when
 * l < 3).  "Applied in groups" on the MatMamba page is read as depthwise: one
 * 4-tap filter per channel of the concatenated [x | B | C] stream.
 */
void oracle_conv1d_silu(const double* u, double* out, const double* w,
                        const double* bias, double* conv_state, int64_t batch,
                        int64_t seqlen, int64_t conv_dim, int64_t d_inner,
                        int64_t d_head, const int64_t* heads_active) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t c = 0; c < conv_dim; ++c) {
      const int64_t d_b = heads_active[b] * d_head;
      if (c < d_inner && c >= d_b) continue; /* outside the slice */
      double hist[3] = {0.0, 0.0, 0.0};    /* u[-3], u[-2], u[-1] */
      if (conv_state) {
        for (int k = 0; k < 3; ++k) hist[k] = conv_state[(b * conv_dim + c) * 3 + k];
      }
      double win[4];
      for (int64_t t = 0; t < seqlen; ++t) {
        for (int k = 0; k < 4; ++k) {
          int64_t tau = t - 3 + k;
          win[k] = tau >= 0 ? u[(b * seqlen + tau) * conv_dim + c] : hist[tau + 3];
        }
        double pre = bias ? bias[c] : 0.0;
        for (int k = 0; k < 4; ++k) pre += w[c * 4 + k] * win[k];
        out[(b * seqlen + t) * conv_dim + c] = silu(pre);
      }
      if (conv_state) {
        double nh[3];
        for (int k = 0; k < 3; ++k) {
          int64_t tau = seqlen - 3 + k;
          nh[k] = tau >= 0 ? u[(b * seqlen + tau) * conv_dim + c] : hist[tau + 3];
        }
        for (int k = 0; k < 3; ++k) conv_state[(b * conv_dim + c) * 3 + k] = nh[k];
      }
    }
  }
}

/* One token of the recurrence for one (sequence, head):
 *   H <- exp(dt*A) * H + dt * x (outer) B ;  y = H . C + D * x */
static void recur_token(double* H, const double* x, double dt, double A,
                        const double* Bv, const double* Cv, double Dh,
                        double* y, int64_t P, int64_t N) {
  const double alpha = exp(dt * A);
  for (int64_t p = 0; p < P; ++p) {
    double* row = H + p * N;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      row[n] = alpha * row[n] + dt * x[p] * Bv[n];
      acc += row[n] * Cv[n];
    }
    y[p] = acc + Dh * x[p];
  }
}

/*
 * Selective scan over the first heads_active[b] heads of every sequence,
 * token by token.  h0 (nullable) is the state before the first token;
 * h_final (nullable) receives the state after the last token.  D nullable
 * means D = 0.  Only active heads of y / h_final are written.
 */
void oracle_ssd_forward(const double* x, const double* dt, const double* A,
                        const double* B, const double* C, const double* D,
                        const double* h0, double* y, double* h_final,
                        int64_t batch, int64_t seqlen, int64_t n_heads,
                        int64_t P, int64_t N, int64_t ngroups,
                        const int64_t* heads_active, double* scratch) {
  /* scratch: batch * n_heads * P * N doubles, one running state per unit */
  const int64_t heads_per_group = n_heads / ngroups;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < n_heads; ++h) {
      if (h >= heads_active[b]) continue;
      const int64_t g = h / heads_per_group;
      double* H = scratch + (b * n_heads + h) * P * N;
      for (int64_t i = 0; i < P * N; ++i)
        H[i] = h0 ? h0[(b * n_heads + h) * P * N + i] : 0.0;
      const double Dh = D ? D[h] : 0.0;
      for (int64_t t = 0; t < seqlen; ++t) {
        const int64_t row = b * seqlen + t;
        recur_token(H, x + (row * n_heads + h) * P, dt[row * n_heads + h], A[h],
                    B + (row * ngroups + g) * N, C + (row * ngroups + g) * N, Dh,
                    y + (row * n_heads + h) * P, P, N);
      }
      if (h_final) {
        for (int64_t i = 0; i < P * N; ++i)
          h_final[(b * n_heads + h) * P * N + i] = H[i];
      }
    }
  }
}

/*
 * Single-token recurrent decode step (the linear-time recurrent inference of
 * the Mamba page, Strengths): one token of the recurrence above applied in
 * place to `state` for the active heads of every sequence.
 *   x_t (batch, n_heads, P), dt_t (batch, n_heads), B_t, C_t (batch, ngroups, N)
 */
void oracle_ssd_step(double* state, const double* x_t, const double* dt_t,
                     const double* A, const double* B_t, const double* C_t,
                     const double* D, double* y_t, int64_t batch,
                     int64_t n_heads, int64_t P, int64_t N, int64_t ngroups,
                     const int64_t* heads_active) {
  const int64_t heads_per_group = n_heads / ngroups;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < n_heads; ++h) {
      if (h >= heads_active[b]) continue;
      const int64_t g = h / heads_per_group;
      recur_token(state + (b * n_heads + h) * P * N, x_t + (b * n_heads + h) * P,
                  dt_t[b * n_heads + h], A[h], B_t + (b * ngroups + g) * N,
                  C_t + (b * ngroups + g) * N, D ? D[h] : 0.0,
                  y_t + (b * n_heads + h) * P, P, N);
    }
  }
}

/*
 * Gated RMSNorm over the first d channels of each token row (the output side
 * of the MatMamba block paragraph: sigma = SiLU gates the scan output with z,
 * Norm = RMSNorm; the display equation is lost, and the gate is read as
 * applied before the norm, as in the Mamba2 block):
 *   g_c   = y_c * SiLU(z_c),              c < d
 *   out_c = g_c * w_c / sqrt(mean_{c<d} g_c^2 + eps)
 * y, z, out: rows x d (row-major, unit stride); w: d.
 */
void oracle_gated_rmsnorm(const double* y, const double* z, const double* w, double eps,
                          double* out, int64_t rows, int64_t d) {
  #pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* yr = y + r * d;
    const double* zr = z + r * d;
    double* o = out + r * d;
    double ss = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      const double g = yr[c] * silu(zr[c]);
      o[c] = g;
      ss += g * g;
    }
    const double inv = 1.0 / sqrt(ss / (double)d + eps);
    for (int64_t c = 0; c < d; ++c) o[c] = o[c] * inv * w[c];
  }
}

/*
 * Reverse-mode gradient of oracle_ssd_forward (the recurrence above, for
 * training the nested sub-blocks jointly: MatMamba page, training paragraph,
 * where the loss sums the outputs of every granularity and the gradients of
 * the shared weights add up).  Given the cotangents dy of y and dhT of the
 * final state (nullable = 0), with L = sum dy.y + sum dhT.h_final, the chain
 * rule taken token by token backwards gives, with Gs = dL/dH_t accumulated:
 *     Gs      += dy_t (outer) C_t                   (H_t feeds y_t)
 *     dC_t    += H_t^T dy_t                         (summed over the group's heads)
 *     dx_t     = dt_t Gs B_t + D_h dy_t
 *     dB_t    += dt_t Gs^T x_t                      (summed over the group's heads)
 *     ddt_t    = <Gs, A_h a_t H_{t-1} + x_t (outer) B_t>,   a_t = exp(dt_t A_h)
 *     dA_h    += <Gs, dt_t a_t H_{t-1}>             (summed over sequences)
 *     dD_h    += dy_t . x_t                         (summed over sequences)
 *     Gs       = a_t Gs                             (now dL/dH_{t-1})
 * and dh0 = Gs after the first token.  The forward states H_t of a unit are
 * kept (seqlen + 1 of them) and walked backwards.
 *
 * Only active heads are read or written in dx, ddt, dh0; dA, dD (n_heads) are
 * written for the heads active in at least one sequence; dB, dC (batch,
 * seqlen, ngroups, N) are overwritten everywhere (0 where no head of the
 * group is active).  dD, dh0 nullable.
 */
void oracle_ssd_backward(const double* x, const double* dt, const double* A,
                         const double* B, const double* C, const double* D,
                         const double* h0, const double* dy, const double* dhT,
                         double* dx, double* ddt, double* dA, double* dB, double* dC,
                         double* dD, double* dh0, int64_t batch, int64_t seqlen,
                         int64_t n_heads, int64_t P, int64_t N, int64_t ngroups,
                         const int64_t* heads_active) {
  const int64_t heads_per_group = n_heads / ngroups;
  const int64_t PN = P * N;
  double* dA_bh = (double*)calloc((size_t)(batch * n_heads), sizeof(double));
  double* dD_bh = (double*)calloc((size_t)(batch * n_heads), sizeof(double));
  for (int64_t i = 0; i < batch * seqlen * ngroups * N; ++i) {
    dB[i] = 0.0;
    dC[i] = 0.0;
  }
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < n_heads; ++h) {
      if (h >= heads_active[b]) continue;
      const int64_t g = h / heads_per_group;
      const int64_t unit = b * n_heads + h;
      /* Hs[t+1] = state after token t; Hs[0] = initial state */
      double* Hs = (double*)malloc((size_t)((seqlen + 1) * PN) * sizeof(double));
      double* Gs = (double*)malloc((size_t)PN * sizeof(double));
      for (int64_t i = 0; i < PN; ++i) Hs[i] = h0 ? h0[unit * PN + i] : 0.0;
      for (int64_t t = 0; t < seqlen; ++t) {
        const int64_t row = b * seqlen + t;
        const double* xt = x + (row * n_heads + h) * P;
        const double* Bt = B + (row * ngroups + g) * N;
        const double d = dt[row * n_heads + h];
        const double a = exp(d * A[h]);
        const double* Hp = Hs + t * PN;
        double* Hn = Hs + (t + 1) * PN;
        for (int64_t p = 0; p < P; ++p)
          for (int64_t n = 0; n < N; ++n)
            Hn[p * N + n] = a * Hp[p * N + n] + d * xt[p] * Bt[n];
      }
      for (int64_t i = 0; i < PN; ++i) Gs[i] = dhT ? dhT[unit * PN + i] : 0.0;
      const double Dh = D ? D[h] : 0.0;
      double dA_acc = 0.0, dD_acc = 0.0;
      for (int64_t t = seqlen - 1; t >= 0; --t) {
        const int64_t row = b * seqlen + t;
        const double* xt = x + (row * n_heads + h) * P;
        const double* dyt = dy + (row * n_heads + h) * P;
        const double* Bt = B + (row * ngroups + g) * N;
        const double* Ct = C + (row * ngroups + g) * N;
        double* dBt = dB + (row * ngroups + g) * N;
        double* dCt = dC + (row * ngroups + g) * N;
        const double d = dt[row * n_heads + h];
        const double a = exp(d * A[h]);
        const double* Hcur = Hs + (t + 1) * PN;
        const double* Hprev = Hs + t * PN;
        for (int64_t p = 0; p < P; ++p)
          for (int64_t n = 0; n < N; ++n) Gs[p * N + n] += dyt[p] * Ct[n];
        for (int64_t n = 0; n < N; ++n) {
          double sc = 0.0, sb = 0.0;
          for (int64_t p = 0; p < P; ++p) {
            sc += Hcur[p * N + n] * dyt[p];
            sb += Gs[p * N + n] * xt[p];
          }
#pragma omp atomic
          dCt[n] += sc;
#pragma omp atomic
          dBt[n] += d * sb;
        }
        double sdt = 0.0, sda = 0.0;
        for (int64_t p = 0; p < P; ++p) {
          double gb = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            const double gv = Gs[p * N + n];
            gb += gv * Bt[n];
            sda += gv * Hprev[p * N + n];
            sdt += gv * xt[p] * Bt[n];
          }
          dx[(row * n_heads + h) * P + p] = d * gb + Dh * dyt[p];
          dD_acc += dyt[p] * xt[p];
        }
        /* d/d(dt) of a*Hprev + dt*x(outer)B, and d/dA of a = exp(dt*A) */
        ddt[row * n_heads + h] = A[h] * a * sda + sdt;
        dA_acc += d * a * sda;
        for (int64_t i = 0; i < PN; ++i) Gs[i] *= a;
      }
      dA_bh[unit] = dA_acc;
      dD_bh[unit] = dD_acc;
      if (dh0)
        for (int64_t i = 0; i < PN; ++i) dh0[unit * PN + i] = Gs[i];
      free(Hs);
      free(Gs);
    }
  }
  for (int64_t h = 0; h < n_heads; ++h) {
    int any = 0;
    double sa = 0.0, sd = 0.0;
    for (int64_t b = 0; b < batch; ++b) {
      if (h >= heads_active[b]) continue;
      any = 1;
      sa += dA_bh[b * n_heads + h];
      sd += dD_bh[b * n_heads + h];
    }
    if (!any) continue;
    dA[h] = sa;
    if (dD) dD[h] = sd;
  }
  free(dA_bh);
  free(dD_bh);
}

/*
 * Reverse-mode gradient of oracle_conv1d_silu for the cotangent dout of its
 * output (the new conv state it returns is not differentiated).  With
 * pre[t,c] as above and SiLU'(v) = s (1 + v (1 - s)), s = 1 / (1 + exp(-v)):
 *     dpre[t,c]   = dout[t,c] SiLU'(pre[t,c])
 *     du[tau,c]   = sum_k w[c,k] dpre[tau+3-k, c]     (0 <= tau+3-k < seqlen)
 *     dw[c,k]    += sum_t dpre[t,c] u[t-3+k, c]        (u[<0] from the state or 0)
 *     dbias[c]   += sum_t dpre[t,c]
 *     dstate[c,j] = sum_k w[c,k] dpre[j-k, c]           (input u[j-3], j = 0..2)
 * summed over the sequences in which channel c is active.  du and dstate are
 * written for the active channels only; dw, dbias for channels active in at
 * least one sequence.  bias, conv_state, dbias, dstate nullable (dstate
 * needs conv_state's layout (batch, conv_dim, 3)).
 */
void oracle_conv1d_silu_backward(const double* u, const double* w, const double* bias,
                                 const double* conv_state, const double* dout, double* du,
                                 double* dw, double* dbias, double* dstate, int64_t batch,
                                 int64_t seqlen, int64_t conv_dim, int64_t d_inner,
                                 int64_t d_head, const int64_t* heads_active) {
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < conv_dim; ++c) {
    double* dpre = (double*)malloc((size_t)(seqlen > 0 ? seqlen : 1) * sizeof(double));
    double sw[4] = {0.0, 0.0, 0.0, 0.0}, sbias = 0.0;
    int any = 0;
    for (int64_t b = 0; b < batch; ++b) {
      if (c < d_inner && c >= heads_active[b] * d_head) continue;
      any = 1;
      double hist[3] = {0.0, 0.0, 0.0};
      if (conv_state)
        for (int k = 0; k < 3; ++k) hist[k] = conv_state[(b * conv_dim + c) * 3 + k];
      for (int64_t t = 0; t < seqlen; ++t) {
        double win[4];
        for (int k = 0; k < 4; ++k) {
          const int64_t tau = t - 3 + k;
          win[k] = tau >= 0 ? u[(b * seqlen + tau) * conv_dim + c] : hist[tau + 3];
        }
        double pre = bias ? bias[c] : 0.0;
        for (int k = 0; k < 4; ++k) pre += w[c * 4 + k] * win[k];
        const double s = 1.0 / (1.0 + exp(-pre));
        const double dp = dout[(b * seqlen + t) * conv_dim + c] * s * (1.0 + pre * (1.0 - s));
        dpre[t] = dp;
        for (int k = 0; k < 4; ++k) sw[k] += dp * win[k];
        sbias += dp;
      }
      for (int64_t tau = 0; tau < seqlen; ++tau) {
        double acc = 0.0;
        for (int k = 0; k < 4; ++k) {
          const int64_t t = tau + 3 - k;
          if (t < seqlen) acc += w[c * 4 + k] * dpre[t];
        }
        du[(b * seqlen + tau) * conv_dim + c] = acc;
      }
      if (dstate) {
        for (int j = 0; j < 3; ++j) {
          double acc = 0.0;
          for (int k = 0; k < 4; ++k) {
            const int64_t t = j - k;
            if (t >= 0 && t < seqlen) acc += w[c * 4 + k] * dpre[t];
          }
          dstate[(b * conv_dim + c) * 3 + j] = acc;
        }
      }
    }
    if (any) {
      for (int k = 0; k < 4; ++k) dw[c * 4 + k] = sw[k];
      if (dbias) dbias[c] = sbias;
    }
    free(dpre);
  }
}
