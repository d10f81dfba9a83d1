/* Runs every oracle entry point once on a tiny case, for the AddressSanitizer
   and UndefinedBehaviorSanitizer build of rat_oracle.c (test infrastructure:
   out-of-bounds accesses, leaks and undefined arithmetic in the oracle make
   this program fail).  Exit status 0 when every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void rat_oracle_scan(int B, int H, int T, int hd, const double* g, const double* x,
                     double* h_out, double* state_out);
int64_t rat_oracle_keyset_size(int64_t t, int D, int W);
void rat_oracle_attention(int B, int H, int T, int hd, const int32_t* D, const int32_t* W,
                          double scale, const double* q, const double* hk, const double* hv,
                          double* o, double* lse);
void rat_oracle_attention_rows(int B, int H, int T, int hd, const int32_t* D, const int32_t* W,
                               double scale, const double* q, const double* hk,
                               const double* hv, int64_t n, const int64_t* rows, double* o_rows,
                               double* lse_rows);
int64_t rat_oracle_anchor_offsets(int H, int64_t T_cap, const int32_t* D, int64_t* off);
void rat_oracle_build_cache(int B, int H, int T, int hd, const int32_t* D, const int32_t* W,
                            int64_t T_cap, const double* hs, double* Kc, double* ring);
void rat_oracle_decode_step(int B, int H, int hd, const int32_t* D, const int32_t* W,
                            double scale, int64_t pos, const double* q, const double* k,
                            const double* v, const double* g, double* state_k, double* state_v,
                            const double* hk_hist, const double* hv_hist, int st_bf16, double* o,
                            double* hk_new, double* hv_new);
void rat_oracle_backward(int B, int H, int T, int hd, const int32_t* D, const int32_t* W,
                         double scale, const double* q, const double* k, const double* v,
                         const double* g, const double* dO, int st_bf16, double* dq, double* dk,
                         double* dv, double* dg);
void rat_oracle_round_bf16_array(int64_t n, double* x);

static double* arr(int64_t n, unsigned* s, double lo, double hi) {
  double* a = (double*)malloc(sizeof(double) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    *s = *s * 1664525u + 1013904223u;
    a[i] = lo + (hi - lo) * (double)(*s >> 8) / 16777216.0;
  }
  return a;
}

static int finite(const double* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

int main(void) {
  enum { B = 2, H = 3, T = 37, HD = 8 };
  const int32_t D[H] = {3, 1, 40};
  const int32_t W[H] = {0, 5, 2};
  const int64_t n = (int64_t)B * H * T * HD;
  unsigned s = 12345u;
  double* q = arr(n, &s, -1, 1);
  double* k = arr(n, &s, -1, 1);
  double* v = arr(n, &s, -1, 1);
  double* g = arr(n, &s, 0.05, 0.95);
  double* dO = arr(n, &s, -1, 1);
  double* hk = malloc(sizeof(double) * n);
  double* hv = malloc(sizeof(double) * n);
  double* sk = malloc(sizeof(double) * B * H * HD);
  double* sv = malloc(sizeof(double) * B * H * HD);
  double* o = malloc(sizeof(double) * n);
  double* lse = malloc(sizeof(double) * B * H * T);
  int ok = 1;
  rat_oracle_scan(B, H, T, HD, g, k, hk, sk);
  rat_oracle_scan(B, H, T, HD, g, v, hv, sv);
  rat_oracle_round_bf16_array(n, hk);
  rat_oracle_round_bf16_array(n, hv);
  rat_oracle_attention(B, H, T, HD, D, W, 0.35, q, hk, hv, o, lse);
  ok = ok && finite(o, n) && finite(lse, B * H * T);
  for (int64_t t = 0; t < T; ++t) ok = ok && rat_oracle_keyset_size(t, 3, 5) >= 1;

  int64_t rows[3 * 3] = {0, 0, 0, 1, 2, T - 1, 1, 1, 17};
  double orow[3 * HD], lrow[3];
  rat_oracle_attention_rows(B, H, T, HD, D, W, 0.35, q, hk, hv, 3, rows, orow, lrow);
  ok = ok && finite(orow, 3 * HD) && finite(lrow, 3);

  const int64_t T_cap = T + 4;
  int64_t off[H + 1];
  const int64_t R = rat_oracle_anchor_offsets(H, T_cap, D, off);
  int64_t WS = 0;
  for (int h = 0; h < H; ++h) WS += W[h];
  double* Kc = malloc(sizeof(double) * B * R * HD);
  double* ring = malloc(sizeof(double) * B * WS * HD);
  for (int64_t i = 0; i < B * R * HD; ++i) Kc[i] = 0.0;
  for (int64_t i = 0; i < B * WS * HD; ++i) ring[i] = 0.0;
  rat_oracle_build_cache(B, H, T, HD, D, W, T_cap, hk, Kc, ring);
  ok = ok && finite(Kc, B * R * HD) && finite(ring, B * WS * HD);

  /* one decode step at position T from the prefill's state and history */
  double* q1 = arr(B * H * HD, &s, -1, 1);
  double* k1 = arr(B * H * HD, &s, -1, 1);
  double* v1 = arr(B * H * HD, &s, -1, 1);
  double* g1 = arr(B * H * HD, &s, 0.05, 0.95);
  double o1[B * H * HD], hk1[B * H * HD], hv1[B * H * HD];
  rat_oracle_decode_step(B, H, HD, D, W, 0.35, T, q1, k1, v1, g1, sk, sv, hk, hv, 1, o1, hk1, hv1);
  ok = ok && finite(o1, B * H * HD) && finite(sk, B * H * HD);

  double* dq = malloc(sizeof(double) * n);
  double* dk = malloc(sizeof(double) * n);
  double* dv = malloc(sizeof(double) * n);
  double* dg = malloc(sizeof(double) * n);
  rat_oracle_backward(B, H, T, HD, D, W, 0.35, q, k, v, g, dO, 1, dq, dk, dv, dg);
  ok = ok && finite(dq, n) && finite(dk, n) && finite(dv, n) && finite(dg, n);

  double* all[] = {q, k, v, g, dO, hk, hv, sk, sv, o, lse, Kc, ring, q1, k1, v1, g1, dq, dk, dv, dg};
  for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
  printf("oracle driver: %s\n", ok ? "ok" : "non-finite output");
  return ok ? 0 : 1;
}
