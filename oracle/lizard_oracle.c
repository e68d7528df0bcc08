/*
 * Plain fp64 CPU oracle for Lizard attention (forward and one decode step).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes, and where the pages define it:
 *
 *   Feature map        fmap 0: phi(x) = softmax over features of (x . W_phi)
 *                      (the softmax-over-features map of the synthetic
 *                      workloads), W_phi [d, df].
 *                      fmap 1: the Lizard paper's own "Hedgehog" map,
 *                      phi(x) = exp(x . W_phi) (+) exp(-x . W_phi), the two
 *                      halves concatenated, W_phi [d, df/2], df even
 *                      (arXiv page, Method section, hardware-efficient
 *                      reparameterization paragraph).  No normalisation.
 *   Global branch      h_i = gamma_i (.) h_{i-1} + phi(k_i) v_i^T,
 *                      y_i = phi(q_i)^T h_i, with a per-key-dimension gate
 *                      gamma_i = exp(log_gamma_i) that scales every row of h
 *                      (papernotes.org summary of the Lizard paper, section
 *                      "key designs", Gated Linear Attention item).
 *   Local branch       softmax over [q_i.T_k ; q_i.k_j for the W most recent
 *                      keys j, i included] applied to [T_v ; v_j]
 *                      (same summary, "key designs", Anchor Window Attention
 *                      item; the meta-memory tokens T are always visible).
 *   Merge              y = mix * y_gla + (1 - mix) * y_win
 *                      (same summary, "overall framework": the two branch
 *                      outputs are combined with weights).
 *
 * It is deliberately the literal token-by-token recurrence and a brute-force
 * window softmax, in double precision, with no blocking, chunking or
 * reordering.  OpenMP runs independent (batch, query head) pairs in parallel.
 *
 * The backward pass (oracle_lizard_bwd) is the chain rule taken through those
 * same steps in reverse order: the states S_i of the forward recurrence are
 * kept, the recurrence is walked from the last token to the first carrying
 * dL/dS, each window softmax is differentiated on its own, and the feature
 * maps last.  The gradients are those the pages' training needs (arXiv page,
 * Experiments: the first stage trains the feature maps and the gate; the
 * Introduction's throughput claim is a training number).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* fmap 0: phi = softmax_f( sum_i x[i] * w[i*df + f] ), max subtracted first.
 * fmap 1: z_j = sum_i x[i] * w[i*(df/2) + j]; phi_j = exp(z_j) and
 *         phi_{df/2 + j} = exp(-z_j) for j < df/2. */
static void feature_map(const double *x, const double *w, int d, int df,
                        int fmap, double *z, double *phi) {
  if (fmap == 1) {
    const int h = df / 2;
    for (int j = 0; j < h; ++j) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += x[i] * w[(int64_t)i * h + j];
      phi[j] = exp(acc);
      phi[h + j] = exp(-acc);
    }
    return;
  }
  double zmax = -INFINITY;
  for (int f = 0; f < df; ++f) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += x[i] * w[(int64_t)i * df + f];
    z[f] = acc;
    if (acc > zmax) zmax = acc;
  }
  double sum = 0.0;
  for (int f = 0; f < df; ++f) {
    phi[f] = exp(z[f] - zmax);
    sum += phi[f];
  }
  for (int f = 0; f < df; ++f) phi[f] /= sum;
}

static double dot(const double *a, const double *b, int n) {
  double acc = 0.0;
  for (int i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

/*
 * Forward over whole sequences.
 *   q [B,Hq,L,d]; k, v [B,Hkv,L,d]; lg (log gamma) [B,Hkv,L,df]
 *   wq, wk: W_phi for query / key side, [.,d,df] (fmap 0) or [.,d,df/2]
 *           (fmap 1); head h uses w + h*w_stride (w_stride = 0: one matrix
 *           shared by all heads)
 *   fmap    feature map: 0 softmax over features, 1 Hedgehog (see above)
 *   tk, tv  [Hkv,M,d] meta-memory keys / values
 *   y, y_gla, y_win [B,Hq,L,d] (y_gla / y_win may be NULL)
 *   state_out [B,Hkv,df,d] final h (may be NULL)
 * Query head hq reads key/value head hq / (Hq/Hkv).
 * Returns 0, or -1 on a shape it cannot take.
 */
int oracle_lizard_fwd(const double *q, const double *k, const double *v,
                      const double *lg, const double *wq, const double *wk,
                      int64_t w_stride, const double *tk, const double *tv,
                      int B, int Hq, int Hkv, int L, int d, int df, int W,
                      int M, double mix, double scale, int fmap, double *y,
                      double *y_gla, double *y_win, double *state_out) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 0 || d < 1 || df < 1 || W < 1 ||
      M < 0 || Hq % Hkv != 0 || fmap < 0 || fmap > 1 || (fmap == 1 && df % 2))
    return -1;
  const int G = Hq / Hkv;
  const int nb = B * Hq;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < nb; ++bh) {
    const int b = bh / Hq, hq = bh % Hq, hk = hq / G;
    const double *qh = q + ((int64_t)b * Hq + hq) * L * d;
    const double *kh = k + ((int64_t)b * Hkv + hk) * L * d;
    const double *vh = v + ((int64_t)b * Hkv + hk) * L * d;
    const double *gh = lg + ((int64_t)b * Hkv + hk) * L * df;
    const double *wqh = wq + (int64_t)hq * w_stride;
    const double *wkh = wk + (int64_t)hk * w_stride;
    const double *tkh = tk + (int64_t)hk * M * d;
    const double *tvh = tv + (int64_t)hk * M * d;
    double *S = calloc((size_t)df * d, sizeof(double));
    double *phq = malloc(sizeof(double) * df);
    double *phk = malloc(sizeof(double) * df);
    double *z = malloc(sizeof(double) * df);
    double *logit = malloc(sizeof(double) * (M + (W < L ? W : L) + 1));
    double *yg = malloc(sizeof(double) * d);
    double *yw = malloc(sizeof(double) * d);
    for (int i = 0; i < L; ++i) {
      const double *qi = qh + (int64_t)i * d;
      const double *ki = kh + (int64_t)i * d;
      const double *vi = vh + (int64_t)i * d;
      const double *gi = gh + (int64_t)i * df;
      /* global branch: decay every key-dimension row, then add phi(k) v^T */
      feature_map(ki, wkh, d, df, fmap, z, phk);
      feature_map(qi, wqh, d, df, fmap, z, phq);
      for (int f = 0; f < df; ++f) {
        const double gam = exp(gi[f]);
        double *row = S + (int64_t)f * d;
        for (int e = 0; e < d; ++e) row[e] = gam * row[e] + phk[f] * vi[e];
      }
      for (int e = 0; e < d; ++e) yg[e] = 0.0;
      for (int f = 0; f < df; ++f) {
        const double *row = S + (int64_t)f * d;
        for (int e = 0; e < d; ++e) yg[e] += phq[f] * row[e];
      }
      /* local branch: M meta keys plus keys j in [i-W+1, i] */
      const int lo = i - W + 1 > 0 ? i - W + 1 : 0;
      int n = 0;
      double mx = -INFINITY;
      for (int m = 0; m < M; ++m) {
        logit[n] = scale * dot(qi, tkh + (int64_t)m * d, d);
        if (logit[n] > mx) mx = logit[n];
        ++n;
      }
      for (int j = lo; j <= i; ++j) {
        logit[n] = scale * dot(qi, kh + (int64_t)j * d, d);
        if (logit[n] > mx) mx = logit[n];
        ++n;
      }
      double zsum = 0.0;
      for (int a = 0; a < n; ++a) {
        logit[a] = exp(logit[a] - mx);
        zsum += logit[a];
      }
      for (int e = 0; e < d; ++e) yw[e] = 0.0;
      n = 0;
      for (int m = 0; m < M; ++m, ++n)
        for (int e = 0; e < d; ++e) yw[e] += logit[n] * tvh[(int64_t)m * d + e];
      for (int j = lo; j <= i; ++j, ++n)
        for (int e = 0; e < d; ++e) yw[e] += logit[n] * vh[(int64_t)j * d + e];
      for (int e = 0; e < d; ++e) yw[e] /= zsum;
      const int64_t o = (((int64_t)b * Hq + hq) * L + i) * d;
      for (int e = 0; e < d; ++e) {
        y[o + e] = mix * yg[e] + (1.0 - mix) * yw[e];
        if (y_gla) y_gla[o + e] = yg[e];
        if (y_win) y_win[o + e] = yw[e];
      }
    }
    if (state_out && hq % G == 0)
      memcpy(state_out + ((int64_t)b * Hkv + hk) * df * d, S,
             sizeof(double) * df * d);
    free(S); free(phq); free(phk); free(z); free(logit); free(yg); free(yw);
  }
  return 0;
}

/*
 * One decode step: every sequence n takes one new token.
 *   state [N,Hkv,df,d]           h, updated in place
 *   ring_k, ring_v [N,Hkv,W,d]   the last W keys / values; token t sits in
 *                                slot t % W; updated in place
 *   pos [N]                      tokens already seen (index of the new token);
 *                                incremented
 *   q [N,Hq,d]; k, v [N,Hkv,d]; lg [N,Hkv,df]; out, y_gla, y_win [N,Hq,d]
 *   wq, wk, w_stride, fmap: as in the forward
 * The per-token arithmetic is the forward's: decay then add, read out, and a
 * softmax over the M meta keys and the min(pos+1, W) newest keys.
 */
int oracle_lizard_decode(double *state, double *ring_k, double *ring_v,
                         int32_t *pos, const double *q, const double *k,
                         const double *v, const double *lg, const double *wq,
                         const double *wk, int64_t w_stride, const double *tk,
                         const double *tv, int N, int Hq, int Hkv, int d,
                         int df, int W, int M, double mix, double scale,
                         int fmap, double *out, double *y_gla, double *y_win) {
  if (N < 1 || Hq < 1 || Hkv < 1 || d < 1 || df < 1 || W < 1 || M < 0 ||
      Hq % Hkv != 0 || fmap < 0 || fmap > 1 || (fmap == 1 && df % 2))
    return -1;
  for (int n = 0; n < N; ++n)
    if (pos[n] < 0) return -1;
  const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int n = 0; n < N; ++n) {
    const int p = pos[n];
    const int slot = p % W;
    const int nvalid = p + 1 < W ? p + 1 : W;
    double *phi = malloc(sizeof(double) * df);
    double *z = malloc(sizeof(double) * df);
    double *logit = malloc(sizeof(double) * (M + W));
    double *yg = malloc(sizeof(double) * d);
    double *yw = malloc(sizeof(double) * d);
    for (int hk = 0; hk < Hkv; ++hk) {
      const int64_t nh = (int64_t)n * Hkv + hk;
      const double *kt = k + nh * d, *vt = v + nh * d, *gt = lg + nh * df;
      double *S = state + nh * df * d;
      feature_map(kt, wk + (int64_t)hk * w_stride, d, df, fmap, z, phi);
      for (int f = 0; f < df; ++f) {
        const double gam = exp(gt[f]);
        for (int e = 0; e < d; ++e)
          S[(int64_t)f * d + e] = gam * S[(int64_t)f * d + e] + phi[f] * vt[e];
      }
      memcpy(ring_k + (nh * W + slot) * d, kt, sizeof(double) * d);
      memcpy(ring_v + (nh * W + slot) * d, vt, sizeof(double) * d);
    }
    for (int hq = 0; hq < Hq; ++hq) {
      const int hk = hq / G;
      const int64_t nh = (int64_t)n * Hkv + hk;
      const double *qt = q + ((int64_t)n * Hq + hq) * d;
      const double *S = state + nh * df * d;
      feature_map(qt, wq + (int64_t)hq * w_stride, d, df, fmap, z, phi);
      for (int e = 0; e < d; ++e) yg[e] = 0.0;
      for (int f = 0; f < df; ++f)
        for (int e = 0; e < d; ++e) yg[e] += phi[f] * S[(int64_t)f * d + e];
      int cnt = 0;
      double mx = -INFINITY;
      for (int m = 0; m < M; ++m, ++cnt) {
        logit[cnt] = scale * dot(qt, tk + ((int64_t)hk * M + m) * d, d);
        if (logit[cnt] > mx) mx = logit[cnt];
      }
      for (int a = 0; a < nvalid; ++a, ++cnt) {
        const int s = (p - a) % W;
        logit[cnt] = scale * dot(qt, ring_k + (nh * W + s) * d, d);
        if (logit[cnt] > mx) mx = logit[cnt];
      }
      double zsum = 0.0;
      for (int a = 0; a < cnt; ++a) {
        logit[a] = exp(logit[a] - mx);
        zsum += logit[a];
      }
      for (int e = 0; e < d; ++e) yw[e] = 0.0;
      cnt = 0;
      for (int m = 0; m < M; ++m, ++cnt)
        for (int e = 0; e < d; ++e)
          yw[e] += logit[cnt] * tv[((int64_t)hk * M + m) * d + e];
      for (int a = 0; a < nvalid; ++a, ++cnt) {
        const int s = (p - a) % W;
        for (int e = 0; e < d; ++e)
          yw[e] += logit[cnt] * ring_v[(nh * W + s) * d + e];
      }
      const int64_t o = ((int64_t)n * Hq + hq) * d;
      for (int e = 0; e < d; ++e) {
        yw[e] /= zsum;
        out[o + e] = mix * yg[e] + (1.0 - mix) * yw[e];
        if (y_gla) y_gla[o + e] = yg[e];
        if (y_win) y_win[o + e] = yw[e];
      }
    }
    pos[n] = p + 1;
    free(phi); free(z); free(logit); free(yg); free(yw);
  }
  return 0;
}

/* Backward of feature_map: given x, phi(x) and dL/dphi, add dL/dx to dx and
 * dL/dW to dw (same layout as w).  fmap 0: dz_f = phi_f (dphi_f - sum_g
 * phi_g dphi_g); fmap 1: dz_j = phi_j dphi_j - phi_{h+j} dphi_{h+j}.  Then
 * dx_i = sum_f W[i][f] dz_f and dW[i][f] += x_i dz_f. */
static void feature_map_bwd(const double *x, const double *w, int d, int df,
                            int fmap, const double *phi, const double *dphi,
                            double *dz, double *dx, double *dw) {
  int cols = df;
  if (fmap == 1) {
    cols = df / 2;
    for (int j = 0; j < cols; ++j)
      dz[j] = phi[j] * dphi[j] - phi[cols + j] * dphi[cols + j];
  } else {
    double inner = 0.0;
    for (int f = 0; f < df; ++f) inner += phi[f] * dphi[f];
    for (int f = 0; f < df; ++f) dz[f] = phi[f] * (dphi[f] - inner);
  }
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int c = 0; c < cols; ++c) {
      acc += w[(int64_t)i * cols + c] * dz[c];
      dw[(int64_t)i * cols + c] += x[i] * dz[c];
    }
    dx[i] += acc;
  }
}

/*
 * Gradients of a scalar loss through oracle_lizard_fwd, given dy = dL/dy
 * [B,Hq,L,d].  Outputs (overwritten): dq [B,Hq,L,d]; dk, dv [B,Hkv,L,d];
 * dlg [B,Hkv,L,df]; dwq and dwk shaped like wq and wk (one matrix when
 * w_stride = 0, else one per query / key-value head; w_stride must then be
 * d * cols); dtk, dtv [Hkv,M,d].  dwq and dwk are kept apart even when the
 * caller passes one matrix as both: its gradient is then their sum.
 *
 * For each (b, query head) the forward recurrence is run first, keeping every
 * S_i (L * df * d doubles).  Then, from i = L-1 down to 0, with G = dL/dS_i:
 *   G += phi_q(q_i) (mix dy_i)^T            (y_gla_i = phi_q^T S_i)
 *   dphi_q(q_i) = S_i (mix dy_i)
 *   dphi_k(k_i) = G v_i,  dv_i += G^T phi_k(k_i)   (S_i gets phi_k v_i^T)
 *   dlg_i[f] = gamma_i[f] sum_e G[f][e] S_{i-1}[f][e]
 *   G = diag(gamma_i) G                       (S_i = diag(gamma_i) S_{i-1} ...)
 * and the window softmax of token i is differentiated with (1 - mix) dy_i:
 *   dp_a = dy_w . value_a, ds_a = p_a (dp_a - sum_b p_b dp_b),
 *   dq_i += scale sum_a ds_a key_a, dkey_a += scale ds_a q_i,
 *   dvalue_a += p_a dy_w  (keys / values: meta tokens or k_j, v_j).
 * Returns 0, or -1 on a shape it cannot take.
 */
int oracle_lizard_bwd(const double *q, const double *k, const double *v,
                      const double *lg, const double *wq, const double *wk,
                      int64_t w_stride, const double *tk, const double *tv,
                      const double *dy, int B, int Hq, int Hkv, int L, int d,
                      int df, int W, int M, double mix, double scale, int fmap,
                      double *dq, double *dk, double *dv, double *dlg,
                      double *dwq, double *dwk, double *dtk, double *dtv) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 0 || d < 1 || df < 1 || W < 1 ||
      M < 0 || Hq % Hkv != 0 || fmap < 0 || fmap > 1 || (fmap == 1 && df % 2))
    return -1;
  const int cols = fmap == 1 ? df / 2 : df;
  const int64_t wsz = (int64_t)d * cols;
  if (w_stride != 0 && w_stride != wsz) return -1;
  const int G = Hq / Hkv;
  const int nwq = w_stride ? Hq : 1, nwk = w_stride ? Hkv : 1;
  memset(dq, 0, sizeof(double) * (size_t)B * Hq * L * d);
  memset(dk, 0, sizeof(double) * (size_t)B * Hkv * L * d);
  memset(dv, 0, sizeof(double) * (size_t)B * Hkv * L * d);
  memset(dlg, 0, sizeof(double) * (size_t)B * Hkv * L * df);
  memset(dwq, 0, sizeof(double) * (size_t)nwq * wsz);
  memset(dwk, 0, sizeof(double) * (size_t)nwk * wsz);
  if (M > 0) {
    memset(dtk, 0, sizeof(double) * (size_t)Hkv * M * d);
    memset(dtv, 0, sizeof(double) * (size_t)Hkv * M * d);
  }
  const int ntask = B * Hkv;
  /* per task (b, kv head): private sums of the gradients shared between tasks */
  double *pwq = calloc((size_t)ntask * nwq * wsz, sizeof(double));
  double *pwk = calloc((size_t)ntask * nwk * wsz, sizeof(double));
  double *ptk = calloc((size_t)ntask * (M > 0 ? M : 1) * d, sizeof(double));
  double *ptv = calloc((size_t)ntask * (M > 0 ? M : 1) * d, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
  for (int task = 0; task < ntask; ++task) {
    const int b = task / Hkv, hk = task % Hkv;
    const int64_t kvo = ((int64_t)b * Hkv + hk) * L;
    const double *kh = k + kvo * d, *vh = v + kvo * d, *gh = lg + kvo * df;
    double *dkh = dk + kvo * d, *dvh = dv + kvo * d, *dgh = dlg + kvo * df;
    const double *wkh = wk + (int64_t)hk * w_stride;
    double *dwkh = pwk + (int64_t)task * nwk * wsz + (w_stride ? (int64_t)hk * wsz : 0);
    const double *tkh = tk + (int64_t)hk * M * d, *tvh = tv + (int64_t)hk * M * d;
    double *dtkh = ptk + (int64_t)task * (M > 0 ? M : 1) * d;
    double *dtvh = ptv + (int64_t)task * (M > 0 ? M : 1) * d;
    double *S = malloc(sizeof(double) * (size_t)(L + 1) * df * d); /* S[i+1] = S_i */
    double *Gr = malloc(sizeof(double) * (size_t)df * d);
    double *phq = malloc(sizeof(double) * (size_t)L * df);
    double *phk = malloc(sizeof(double) * (size_t)L * df);
    double *dphq = malloc(sizeof(double) * df);
    double *dphk = malloc(sizeof(double) * df);
    double *z = malloc(sizeof(double) * df);
    double *dz = malloc(sizeof(double) * df);
    double *p = malloc(sizeof(double) * (M + (W < L ? W : L) + 1));
    double *dp = malloc(sizeof(double) * (M + (W < L ? W : L) + 1));
    double *ydg = malloc(sizeof(double) * d);
    for (int i = 0; i < L; ++i) feature_map(kh + (int64_t)i * d, wkh, d, df, fmap, z, phk + (int64_t)i * df);
    for (int g = 0; g < G; ++g) {
      const int hq = hk * G + g;
      const int64_t qo = ((int64_t)b * Hq + hq) * L;
      const double *qh = q + qo * d, *dyh = dy + qo * d;
      double *dqh = dq + qo * d;
      const double *wqh = wq + (int64_t)hq * w_stride;
      double *dwqh = pwq + (int64_t)task * nwq * wsz + (w_stride ? (int64_t)hq * wsz : 0);
      for (int i = 0; i < L; ++i) feature_map(qh + (int64_t)i * d, wqh, d, df, fmap, z, phq + (int64_t)i * df);
      /* forward recurrence, every state kept */
      memset(S, 0, sizeof(double) * (size_t)df * d);
      for (int i = 0; i < L; ++i) {
        const double *prev = S + (int64_t)i * df * d;
        double *cur = S + (int64_t)(i + 1) * df * d;
        for (int f = 0; f < df; ++f) {
          const double gam = exp(gh[(int64_t)i * df + f]);
          for (int e = 0; e < d; ++e)
            cur[(int64_t)f * d + e] = gam * prev[(int64_t)f * d + e] +
                                      phk[(int64_t)i * df + f] * vh[(int64_t)i * d + e];
        }
      }
      /* reverse sweep of the global branch */
      memset(Gr, 0, sizeof(double) * (size_t)df * d);
      for (int i = L - 1; i >= 0; --i) {
        const double *Si = S + (int64_t)(i + 1) * df * d, *Sp = S + (int64_t)i * df * d;
        const double *vi = vh + (int64_t)i * d, *pq = phq + (int64_t)i * df, *pk = phk + (int64_t)i * df;
        for (int e = 0; e < d; ++e) ydg[e] = mix * dyh[(int64_t)i * d + e];
        for (int f = 0; f < df; ++f) {
          double a = 0.0;
          for (int e = 0; e < d; ++e) {
            Gr[(int64_t)f * d + e] += pq[f] * ydg[e];
            a += Si[(int64_t)f * d + e] * ydg[e];
          }
          dphq[f] = a;
        }
        for (int f = 0; f < df; ++f) {
          double a = 0.0, c = 0.0;
          for (int e = 0; e < d; ++e) {
            a += Gr[(int64_t)f * d + e] * vi[e];
            c += Gr[(int64_t)f * d + e] * Sp[(int64_t)f * d + e];
          }
          dphk[f] = a;
          const double gam = exp(gh[(int64_t)i * df + f]);
          dgh[(int64_t)i * df + f] += gam * c;
        }
        for (int e = 0; e < d; ++e) {
          double a = 0.0;
          for (int f = 0; f < df; ++f) a += Gr[(int64_t)f * d + e] * pk[f];
          dvh[(int64_t)i * d + e] += a;
        }
        for (int f = 0; f < df; ++f) {
          const double gam = exp(gh[(int64_t)i * df + f]);
          for (int e = 0; e < d; ++e) Gr[(int64_t)f * d + e] *= gam;
        }
        feature_map_bwd(qh + (int64_t)i * d, wqh, d, df, fmap, pq, dphq, dz, dqh + (int64_t)i * d, dwqh);
        feature_map_bwd(kh + (int64_t)i * d, wkh, d, df, fmap, pk, dphk, dz, dkh + (int64_t)i * d, dwkh);
      }
      /* window branch, token by token */
      for (int i = 0; i < L; ++i) {
        const double *qi = qh + (int64_t)i * d;
        const double *dyi = dyh + (int64_t)i * d;
        const int lo = i - W + 1 > 0 ? i - W + 1 : 0;
        int n = 0;
        double mx = -INFINITY;
        for (int m = 0; m < M; ++m, ++n) {
          p[n] = scale * dot(qi, tkh + (int64_t)m * d, d);
          if (p[n] > mx) mx = p[n];
        }
        for (int j = lo; j <= i; ++j, ++n) {
          p[n] = scale * dot(qi, kh + (int64_t)j * d, d);
          if (p[n] > mx) mx = p[n];
        }
        double zsum = 0.0;
        for (int a = 0; a < n; ++a) {
          p[a] = exp(p[a] - mx);
          zsum += p[a];
        }
        double inner = 0.0;
        n = 0;
        for (int m = 0; m < M; ++m, ++n) {
          p[n] /= zsum;
          dp[n] = (1.0 - mix) * dot(dyi, tvh + (int64_t)m * d, d);
          inner += p[n] * dp[n];
        }
        for (int j = lo; j <= i; ++j, ++n) {
          p[n] /= zsum;
          dp[n] = (1.0 - mix) * dot(dyi, vh + (int64_t)j * d, d);
          inner += p[n] * dp[n];
        }
        n = 0;
        for (int m = 0; m < M; ++m, ++n) {
          const double ds = p[n] * (dp[n] - inner);
          for (int e = 0; e < d; ++e) {
            dqh[(int64_t)i * d + e] += scale * ds * tkh[(int64_t)m * d + e];
            dtkh[(int64_t)m * d + e] += scale * ds * qi[e];
            dtvh[(int64_t)m * d + e] += p[n] * (1.0 - mix) * dyi[e];
          }
        }
        for (int j = lo; j <= i; ++j, ++n) {
          const double ds = p[n] * (dp[n] - inner);
          for (int e = 0; e < d; ++e) {
            dqh[(int64_t)i * d + e] += scale * ds * kh[(int64_t)j * d + e];
            dkh[(int64_t)j * d + e] += scale * ds * qi[e];
            dvh[(int64_t)j * d + e] += p[n] * (1.0 - mix) * dyi[e];
          }
        }
      }
    }
    free(S); free(Gr); free(phq); free(phk); free(dphq); free(dphk); free(z); free(dz);
    free(p); free(dp); free(ydg);
  }
  for (int task = 0; task < ntask; ++task) {
    for (int64_t x = 0; x < (int64_t)nwq * wsz; ++x) dwq[x] += pwq[(int64_t)task * nwq * wsz + x];
    for (int64_t x = 0; x < (int64_t)nwk * wsz; ++x) dwk[x] += pwk[(int64_t)task * nwk * wsz + x];
    if (M > 0) {
      const int hk = task % Hkv;
      for (int64_t x = 0; x < (int64_t)M * d; ++x) {
        dtk[(int64_t)hk * M * d + x] += ptk[(int64_t)task * M * d + x];
        dtv[(int64_t)hk * M * d + x] += ptv[(int64_t)task * M * d + x];
      }
    }
  }
  free(pwq); free(pwk); free(ptk); free(ptv);
  return 0;
}

/* Threads the OpenMP runtime will use (reported by the CPU baseline). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
