/*
 * RAT+ hot-path oracle: a plain, slow, obviously-correct CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library) never calls it and shares no code with it.
 *
 * All arithmetic is IEEE double.  Each function follows the definition it
 * cites, with no blocking, fusion or reordering beyond that definition.
 *
 * Sources (titles and sections of the pages this method is described on):
 *  [ABS]  "RAT+: Train Dense, Infer Sparse -- Recurrence Augmented Attention
 *         for Dilated Inference", abstract (arXiv 2602.18196): dilated
 *         attention cuts attention FLOPs and the KV cache by the dilation D;
 *         the pretrained model is switched at inference time to dilated
 *         attention, optionally with local windows, or to hybrid layer/head
 *         compositions; the recurrence runs over the full sequence.
 *  [Z21]  zhichai.net deep dive "RAT+ 深度拆解", section 2.1 (Full-Sequence
 *         Recurrence): an input-dependent forget-gate recurrence whose state
 *         at each token has accumulated everything since the start of the
 *         sequence (recurrence length = T); computed in prefill by an
 *         associative scan.  The original RAT recurred only inside chunks of
 *         size D.
 *  [Z1]   same page, section 一: dilated attention skips tokens at a fixed
 *         interval D.
 *  [Z22]  same page, section 2.2: D = 1 is dense attention.
 *  [Z6]   same page, section 六 (head-wise hybrid): some heads dense, the
 *         rest dilated, in one layer.
 *
 * Readings taken where the pages are silent (the recurrence formula itself
 * was lost from the page text):
 *  - recurrence h_t = g_t*h_{t-1} + (1-g_t)*x_t per channel, h_{-1} = 0,
 *    the same gate g for keys and values;
 *  - anchors are the chunk ends j = D-1 (mod D), i.e. the last position of
 *    every RAT chunk of size D;
 *  - query t attends to {t} U {j < t : j = D-1 mod D} U {max(0,t-W) .. t-1}
 *    (set union; W = 0 means no window);
 *  - scale defaults to 1/sqrt(hd) (chosen by the caller);
 *  - stored states are rounded to the storage type (bf16: round to nearest
 *    even) when the storage type is bf16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define IDX4(b, h, t, c, H, T, HD) \
  ((((int64_t)(b) * (H) + (h)) * (int64_t)(T) + (t)) * (int64_t)(HD) + (c))

/* ------------------------------------------------------------------ */
/* bf16 storage rounding: keep 8 significant bits, round half to even.  */
/* Finite inputs only (the method has no non-finite values).            */
/* ------------------------------------------------------------------ */
double rat_oracle_round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e); /* |x| = f * 2^e, f in [0.5, 1) */
  /* spacing of bf16 numbers near x is 2^(e-8); below the smallest normal
     (2^-126) the spacing is fixed at 2^-133 */
  int shift = 8 - e;
  if (e - 1 < -126) shift = 133;
  double scaled = ldexp(x, shift);
  double r = nearbyint(scaled); /* default rounding mode: half to even */
  return ldexp(r, -shift);
}

void rat_oracle_round_bf16_array(int64_t n, double* x) {
  for (int64_t i = 0; i < n; ++i) x[i] = rat_oracle_round_bf16(x[i]);
}

/* ------------------------------------------------------------------ */
/* [Z21] gated recurrence over the full sequence, as a sequential loop.  */
/*   h_t = g_t * h_{t-1} + (1 - g_t) * x_t,  h_{-1} = 0.                 */
/* g, x, h_out: [B,H,T,hd]; state_out: [B,H,hd] (h_{T-1}).               */
/* h_out and state_out may be NULL.                                      */
/* ------------------------------------------------------------------ */
void rat_oracle_scan(int B, int H, int T, int hd, const double* g,
                     const double* x, double* h_out, double* state_out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int c = 0; c < hd; ++c) {
        double s = 0.0;
        for (int t = 0; t < T; ++t) {
          int64_t i = IDX4(b, h, t, c, H, T, hd);
          s = g[i] * s + (1.0 - g[i]) * x[i];
          if (h_out) h_out[i] = s;
        }
        if (state_out) state_out[((int64_t)b * H + h) * hd + c] = s;
      }
}

/* ------------------------------------------------------------------ */
/* [ABS][Z1][Z22] membership of key position j in query t's key set.    */
/* ------------------------------------------------------------------ */
int rat_oracle_in_keyset(int64_t t, int64_t j, int D, int W) {
  if (j < 0 || j > t) return 0;
  if (j == t) return 1;                        /* own position            */
  if (j % D == D - 1) return 1;                /* stride-D anchor, j < t  */
  if (W > 0 && j >= t - W) return 1;           /* local window            */
  return 0;
}

/* |S(t)| by enumeration (used by tests to check the closed form). */
int64_t rat_oracle_keyset_size(int64_t t, int D, int W) {
  int64_t n = 0;
  for (int64_t j = 0; j <= t; ++j) n += rat_oracle_in_keyset(t, j, D, W);
  return n;
}

/* softmax attention of one query row over its key set (definition).
   q: [hd]; hk, hv: the head's [T,hd] states; o: [hd]; returns lse. */
static double attend_row(int64_t t, int hd, int D, int W, double scale,
                         const double* q, const double* hk, const double* hv,
                         double* o) {
  double m = -INFINITY;
  for (int64_t j = 0; j <= t; ++j) {
    if (!rat_oracle_in_keyset(t, j, D, W)) continue;
    double e = 0.0;
    for (int c = 0; c < hd; ++c) e += q[c] * hk[j * hd + c];
    e *= scale;
    if (e > m) m = e;
  }
  double l = 0.0;
  for (int c = 0; c < hd; ++c) o[c] = 0.0;
  for (int64_t j = 0; j <= t; ++j) {
    if (!rat_oracle_in_keyset(t, j, D, W)) continue;
    double e = 0.0;
    for (int c = 0; c < hd; ++c) e += q[c] * hk[j * hd + c];
    e *= scale;
    double w = exp(e - m);
    l += w;
    for (int c = 0; c < hd; ++c) o[c] += w * hv[j * hd + c];
  }
  for (int c = 0; c < hd; ++c) o[c] /= l;
  return m + log(l);
}

/* ------------------------------------------------------------------ */
/* Dilated causal softmax attention for every query (definition).        */
/* q, hk, hv, o: [B,H,T,hd]; lse: [B,H,T] (nullable); D, W: [H].         */
/* ------------------------------------------------------------------ */
void rat_oracle_attention(int B, int H, int T, int hd, const int32_t* D,
                          const int32_t* W, double scale, const double* q,
                          const double* hk, const double* hv, double* o,
                          double* lse) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const double* hkh = hk + IDX4(b, h, 0, 0, H, T, hd);
      const double* hvh = hv + IDX4(b, h, 0, 0, H, T, hd);
      for (int t = 0; t < T; ++t) {
        int64_t i = IDX4(b, h, t, 0, H, T, hd);
        double l = attend_row(t, hd, D[h], W[h], scale, q + i, hkh, hvh, o + i);
        if (lse) lse[((int64_t)b * H + h) * T + t] = l;
      }
    }
}

/* Same, for a list of (b, h, t) triples only.  rows: [n][3];            */
/* o_rows: [n][hd]; lse_rows: [n] (nullable).                            */
void rat_oracle_attention_rows(int B, int H, int T, int hd, const int32_t* D,
                               const int32_t* W, double scale, const double* q,
                               const double* hk, const double* hv, int64_t n,
                               const int64_t* rows, double* o_rows,
                               double* lse_rows) {
  (void)B;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < n; ++r) {
    int64_t b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
    double l = attend_row(t, hd, D[h], W[h], scale,
                          q + IDX4(b, h, t, 0, H, T, hd),
                          hk + IDX4(b, h, 0, 0, H, T, hd),
                          hv + IDX4(b, h, 0, 0, H, T, hd), o_rows + r * hd);
    if (lse_rows) lse_rows[r] = l;
  }
}

/* ------------------------------------------------------------------ */
/* [ABS] KV cache of the anchors only: per head floor(T_cap / D_h) rows,  */
/* heads packed one after another.  Returns R = total rows per batch     */
/* row; fills off[0..H] (off[H] = R).                                    */
/* ------------------------------------------------------------------ */
int64_t rat_oracle_anchor_offsets(int H, int64_t T_cap, const int32_t* D,
                                  int64_t* off) {
  int64_t r = 0;
  for (int h = 0; h < H; ++h) {
    if (off) off[h] = r;
    r += T_cap / D[h];
  }
  if (off) off[H] = r;
  return r;
}

/* Cache contents after a prefill of T positions (definition of layout):  */
/*  Kc[b, off[h] + a] = hk[b, h, a*D_h + D_h - 1] for a < floor(T/D_h);    */
/*  ring[b, roff[h] + (p mod W_h)] = hk[b, h, p] for max(0,T-W_h) <= p < T */
/* Rows not named above are left untouched.  Kc: [B,R,hd];               */
/* ring: [B, sum W, hd] (nullable when every W is 0).                    */
void rat_oracle_build_cache(int B, int H, int T, int hd, const int32_t* D,
                            const int32_t* W, int64_t T_cap, const double* hs,
                            double* Kc, double* ring) {
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (H + 1));
  int64_t R = rat_oracle_anchor_offsets(H, T_cap, D, off);
  int64_t WS = 0;
  int64_t* roff = (int64_t*)malloc(sizeof(int64_t) * (H + 1));
  for (int h = 0; h < H; ++h) { roff[h] = WS; WS += W[h]; }
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      for (int64_t a = 0; a < (int64_t)T / D[h]; ++a) {
        int64_t p = a * D[h] + D[h] - 1;
        memcpy(Kc + ((int64_t)b * R + off[h] + a) * hd,
               hs + IDX4(b, h, p, 0, H, T, hd), sizeof(double) * hd);
      }
      if (ring && W[h] > 0) {
        int64_t p0 = T - W[h] > 0 ? T - W[h] : 0;
        for (int64_t p = p0; p < T; ++p)
          memcpy(ring + ((int64_t)b * WS + roff[h] + p % W[h]) * hd,
                 hs + IDX4(b, h, p, 0, H, T, hd), sizeof(double) * hd);
      }
    }
  free(off);
  free(roff);
}

/* ------------------------------------------------------------------ */
/* One decode step at position pos (definition, not the cache):          */
/*   s <- g*s + (1-g)*x for x in {k, v} (state in/out, [B,H,hd]);         */
/*   hat_t = s, rounded to the storage type when st_bf16;                */
/*   o = softmax attention of q over S(pos), using the stored history     */
/*       hk_hist/hv_hist [B,H,pos,hd] for j < pos and hat_t for j = pos.  */
/* q, k, v, g: [B,H,hd]; o, hk_new, hv_new: [B,H,hd] (new ones nullable).  */
/* ------------------------------------------------------------------ */
void rat_oracle_decode_step(int B, int H, int hd, const int32_t* D,
                            const int32_t* W, double scale, int64_t pos,
                            const double* q, const double* k, const double* v,
                            const double* g, double* state_k, double* state_v,
                            const double* hk_hist, const double* hv_hist,
                            int st_bf16, double* o, double* hk_new,
                            double* hv_new) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      int64_t bh = (int64_t)b * H + h;
      const double* qq = q + bh * hd;
      double* hatk = (double*)malloc(sizeof(double) * hd);
      double* hatv = (double*)malloc(sizeof(double) * hd);
      for (int c = 0; c < hd; ++c) {
        int64_t i = bh * hd + c;
        state_k[i] = g[i] * state_k[i] + (1.0 - g[i]) * k[i];
        state_v[i] = g[i] * state_v[i] + (1.0 - g[i]) * v[i];
        hatk[c] = st_bf16 ? rat_oracle_round_bf16(state_k[i]) : state_k[i];
        hatv[c] = st_bf16 ? rat_oracle_round_bf16(state_v[i]) : state_v[i];
        if (hk_new) hk_new[i] = hatk[c];
        if (hv_new) hv_new[i] = hatv[c];
      }
      const double* hkh = hk_hist + bh * pos * hd;
      const double* hvh = hv_hist + bh * pos * hd;
      double m = -INFINITY;
      for (int64_t j = 0; j <= pos; ++j) {
        if (!rat_oracle_in_keyset(pos, j, D[h], W[h])) continue;
        const double* kr = (j == pos) ? hatk : hkh + j * hd;
        double e = 0.0;
        for (int c = 0; c < hd; ++c) e += qq[c] * kr[c];
        e *= scale;
        if (e > m) m = e;
      }
      double l = 0.0;
      double* oo = o + bh * hd;
      for (int c = 0; c < hd; ++c) oo[c] = 0.0;
      for (int64_t j = 0; j <= pos; ++j) {
        if (!rat_oracle_in_keyset(pos, j, D[h], W[h])) continue;
        const double* kr = (j == pos) ? hatk : hkh + j * hd;
        const double* vr = (j == pos) ? hatv : hvh + j * hd;
        double e = 0.0;
        for (int c = 0; c < hd; ++c) e += qq[c] * kr[c];
        e *= scale;
        double w = exp(e - m);
        l += w;
        for (int c = 0; c < hd; ++c) oo[c] += w * vr[c];
      }
      for (int c = 0; c < hd; ++c) oo[c] /= l;
      free(hatk);
      free(hatv);
    }
}

int rat_oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads used by the parallel loops over (b, h) from here on (timing of the
   baseline on one core; the results do not depend on it). */
void rat_oracle_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* Backward of the prefill (reverse-mode derivative of the definitions  */
/* above), for a loss L whose gradient with respect to o is dO.  The    */
/* pages train RAT+ densely with active recurrence learning and adapt   */
/* it to a dilation ([Z22], [Z23]); this is the gradient that training  */
/* path needs.  Steps, per (b, h):                                     */
/*  1. the forward recurrence of keys and values ([Z21]); the attention */
/*     reads the states rounded to the storage type when st_bf16, and   */
/*     the rounding is taken as the identity in the derivative;         */
/*  2. per query t, over its key set S(t): p_j = softmax_j(scale q.hk_j),*/
/*     dP_j = dO_t . hv_j, delta = sum_j p_j dP_j, dS_j = p_j (dP_j -    */
/*     delta); dq_t = scale sum_j dS_j hk_j; dhk_j += scale dS_j q_t;    */
/*     dhv_j += p_j dO_t;                                               */
/*  3. the recurrence in reverse: lambda_t = dh_t + g_{t+1} lambda_{t+1} */
/*     (lambda_T = 0); dx_t = (1 - g_t) lambda_t; dg_t accumulates      */
/*     lambda_t (h_{t-1} - x_t) over keys and values (h_{-1} = 0).      */
/* q, k, v, g, dO, dq, dk, dv, dg: [B,H,T,hd].                           */
/* ------------------------------------------------------------------ */
void rat_oracle_backward(int B, int H, int T, int hd, const int32_t* D,
                         const int32_t* W, double scale, const double* q,
                         const double* k, const double* v, const double* g,
                         const double* dO, int st_bf16, double* dq, double* dk,
                         double* dv, double* dg) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int64_t base = IDX4(b, h, 0, 0, H, T, hd);
      const int64_t n = (int64_t)T * hd;
      double* hk = (double*)malloc(sizeof(double) * n);
      double* hv = (double*)malloc(sizeof(double) * n);
      double* hkr = (double*)malloc(sizeof(double) * n);
      double* hvr = (double*)malloc(sizeof(double) * n);
      double* dhk = (double*)calloc(n, sizeof(double));
      double* dhv = (double*)calloc(n, sizeof(double));
      double* p = (double*)malloc(sizeof(double) * T);
      double* dp = (double*)malloc(sizeof(double) * T);
      /* 1. forward recurrence */
      for (int c = 0; c < hd; ++c) {
        double sk = 0.0, sv = 0.0;
        for (int t = 0; t < T; ++t) {
          const int64_t i = base + (int64_t)t * hd + c;
          sk = g[i] * sk + (1.0 - g[i]) * k[i];
          sv = g[i] * sv + (1.0 - g[i]) * v[i];
          hk[(int64_t)t * hd + c] = sk;
          hv[(int64_t)t * hd + c] = sv;
        }
      }
      for (int64_t i = 0; i < n; ++i) {
        hkr[i] = st_bf16 ? rat_oracle_round_bf16(hk[i]) : hk[i];
        hvr[i] = st_bf16 ? rat_oracle_round_bf16(hv[i]) : hv[i];
      }
      /* 2. attention backward, query by query */
      for (int t = 0; t < T; ++t) {
        const double* qt = q + base + (int64_t)t * hd;
        const double* dot = dO + base + (int64_t)t * hd;
        double m = -INFINITY;
        for (int j = 0; j <= t; ++j) {
          p[j] = -INFINITY;
          if (!rat_oracle_in_keyset(t, j, D[h], W[h])) continue;
          double e = 0.0;
          for (int c = 0; c < hd; ++c) e += qt[c] * hkr[(int64_t)j * hd + c];
          p[j] = scale * e;
          if (p[j] > m) m = p[j];
        }
        double l = 0.0;
        for (int j = 0; j <= t; ++j) {
          p[j] = (p[j] == -INFINITY) ? 0.0 : exp(p[j] - m);
          l += p[j];
        }
        double delta = 0.0;
        for (int j = 0; j <= t; ++j) {
          p[j] /= l;
          dp[j] = 0.0;
          if (p[j] == 0.0) continue;
          for (int c = 0; c < hd; ++c) dp[j] += dot[c] * hvr[(int64_t)j * hd + c];
          delta += p[j] * dp[j];
        }
        double* dqt = dq + base + (int64_t)t * hd;
        for (int c = 0; c < hd; ++c) dqt[c] = 0.0;
        for (int j = 0; j <= t; ++j) {
          if (p[j] == 0.0) continue;
          const double ds = p[j] * (dp[j] - delta);
          for (int c = 0; c < hd; ++c) {
            dqt[c] += scale * ds * hkr[(int64_t)j * hd + c];
            dhk[(int64_t)j * hd + c] += scale * ds * qt[c];
            dhv[(int64_t)j * hd + c] += p[j] * dot[c];
          }
        }
      }
      /* 3. the recurrence in reverse */
      for (int c = 0; c < hd; ++c) {
        double lk = 0.0, lv = 0.0;
        for (int t = T - 1; t >= 0; --t) {
          const int64_t i = base + (int64_t)t * hd + c;
          const double gn = (t + 1 < T) ? g[i + hd] : 0.0;
          lk = dhk[(int64_t)t * hd + c] + gn * lk;
          lv = dhv[(int64_t)t * hd + c] + gn * lv;
          dk[i] = (1.0 - g[i]) * lk;
          dv[i] = (1.0 - g[i]) * lv;
          const double pk = t > 0 ? hk[(int64_t)(t - 1) * hd + c] : 0.0;
          const double pv = t > 0 ? hv[(int64_t)(t - 1) * hd + c] : 0.0;
          dg[i] = lk * (pk - k[i]) + lv * (pv - v[i]);
        }
      }
      free(hk); free(hv); free(hkr); free(hvr); free(dhk); free(dhv); free(p); free(dp);
    }
}
