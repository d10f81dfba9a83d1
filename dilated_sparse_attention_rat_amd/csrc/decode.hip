// One decode step of a RAT+ layer at position pos for every (b, h).
//
// Method: zhichai.net deep dive "RAT+ 深度拆解", section 2.1 -- the
// recurrence state accumulates the whole sequence, so decode needs one state
// update per token; RAT+ abstract -- attention reads a KV cache that is D
// times smaller (anchors only), plus the optional local window.
//   s <- g*s + (1-g)*x (fp32);  hat = ST(s)
//   o = softmax attention of q over: anchors a < floor(max(0,pos-W)/D)
//       (compact rows of Kc/Vc), the window slots of positions
//       max(0,pos-W) .. pos-1 (ring), and hat (own position).
//   Then state <- s, ring slot pos mod W <- hat, and anchor row pos / D <- hat
//   when pos = D-1 (mod D).  The ring slot being replaced holds position
//   pos-W, which is still inside this step's window, so every write happens
//   after every read of the step.
//
// Design: the step is a pure HBM stream of the cache rows (about 1 FLOP per
// byte).  Each workgroup streams a contiguous range of cache rows of one
// (b, h) with 16-byte loads (16 lanes per 256-byte row, 16 rows per pass, 4
// passes in flight), keeps an online softmax per row group, and merges the
// row groups in LDS.  With one split per (b, h) (enough (b, h) to fill the
// chip) the same workgroup also updates the state and writes o, the ring
// slot and the anchor row after a barrier; with several splits the partial
// (max, sum, acc) go to a workspace and a combine kernel merges them and
// does the writes.
#include "rat_device.h"

namespace rat {

namespace {

constexpr int kU = 4;  // rows per lane-group per iteration

// Own position + writes, executed by threads c < HD of the block after all
// reads of this (b, h) are complete.  M, L, A: merged softmax state of the
// cache keys (log2 domain).
template <typename ST, int HD>
__device__ __forceinline__ void finish_step(const DecodeParams& p, int b, int h, float M,
                                            float L, float A, float* s_red) {
  const int c = threadIdx.x;
  const int64_t bh = (int64_t)b * p.H + h;
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  const int pos = p.pos;
  float hatk = 0.f, hatv = 0.f, sk = 0.f, sv = 0.f, part = 0.f;
  if (c < HD) {
    const int64_t i = bh * HD + c;
    const ST* qp = reinterpret_cast<const ST*>(p.q);
    const ST* kp = reinterpret_cast<const ST*>(p.k);
    const ST* vp = reinterpret_cast<const ST*>(p.v);
    const ST* gp = reinterpret_cast<const ST*>(p.g);
    const float gg = (float)gp[i];
    sk = gg * p.sk[i] + (1.f - gg) * (float)kp[i];
    sv = gg * p.sv[i] + (1.f - gg) * (float)vp[i];
    hatk = st_round(sk, (ST*)nullptr);
    hatv = st_round(sv, (ST*)nullptr);
    part = (float)qp[i] * p.scale_log2 * hatk;
  }
  // block reduction of q . hat_k over the HD channels
  for (int m = 32; m >= 1; m >>= 1) part += shfl_xor_f(part, m);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = part;
  __syncthreads();
  float sown = 0.f;
#pragma unroll
  for (int w = 0; w < (HD + 63) / 64; ++w) sown += s_red[w];
  if (c < HD) {
    const float Mn = fmaxf(M, sown);
    const float a = exp2f(M - Mn);
    const float e = exp2f(sown - Mn);
    const float out = (A * a + e * hatv) / (L * a + e);
    ST* op = reinterpret_cast<ST*>(p.o);
    op[bh * HD + c] = (ST)out;
    p.sk[bh * HD + c] = sk;
    p.sv[bh * HD + c] = sv;
    if (W > 0) {
      const int64_t off = ((int64_t)b * p.WS + p.ht.roff[h] + pos % W) * HD + c;
      reinterpret_cast<ST*>(p.kr)[off] = (ST)hatk;
      reinterpret_cast<ST*>(p.vr)[off] = (ST)hatv;
    }
    if (pos % D == D - 1) {
      const int64_t off = ((int64_t)b * p.R + p.ht.aoff[h] + pos / D) * HD + c;
      reinterpret_cast<ST*>(p.Kc)[off] = (ST)hatk;
      reinterpret_cast<ST*>(p.Vc)[off] = (ST)hatv;
    }
  }
}

template <typename ST, int HD, bool FUSED>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const DecodeParams p) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;            // lanes per row
  constexpr int RPP = kDecodeThreads / LPR;  // rows per pass
  __shared__ float s_m[RPP], s_l[RPP];
  __shared__ float s_acc[RPP][HD];
  __shared__ float s_red[4];

  // block -> (head, batch row, split): classes of heads by keys read, most
  // first (a head-wise hybrid's long dense splits start in the first wave of
  // workgroups, the short ones fill in beside them); within a class, batch
  // row by batch row, then head, then split
  const int blk = blockIdx.x;
  int r0 = 0, base = 0, r1 = p.class_end[0];
  while (blk >= base + (r1 - r0) * p.B * p.splits) {
    base += (r1 - r0) * p.B * p.splits;
    r0 = r1;
    r1 = p.class_end[r0];
  }
  const int per_b = (r1 - r0) * p.splits;
  const int local = blk - base;
  const int b = local / per_b;
  const int rem = local - b * per_b;
  const int rank = r0 + rem / p.splits;
  const int split = rem - (rem / p.splits) * p.splits;
  const int h = p.perm[rank];
  const int64_t bh = (int64_t)b * p.H + h;
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  const int pos = p.pos;
  const int na = max(0, pos - W) / D;  // anchors read from the cache
  const int nw = min(W, pos);          // window slots read from the ring
  const int nk = na + nw;
  const int chunk = (nk + p.splits - 1) / p.splits;
  const int kbeg = split * chunk;
  const int kend = min(nk, kbeg + chunk);

  const int tid = threadIdx.x;
  const int rg = tid / LPR;
  const int cl = tid - rg * LPR;
  const int c0 = cl * VEC;

  float q[VEC];
  {
    const u32x4 u = ld_raw16(reinterpret_cast<const ST*>(p.q) + bh * HD + c0);
    unpack16(u, q, (ST*)nullptr);
#pragma unroll
    for (int i = 0; i < VEC; ++i) q[i] *= p.scale_log2;
  }
  const ST* kc = reinterpret_cast<const ST*>(p.Kc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
  const ST* vc = reinterpret_cast<const ST*>(p.Vc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
  const ST* kr = reinterpret_cast<const ST*>(p.kr) + ((int64_t)b * p.WS + p.ht.roff[h]) * HD;
  const ST* vr = reinterpret_cast<const ST*>(p.vr) + ((int64_t)b * p.WS + p.ht.roff[h]) * HD;

  float m = -1e30f, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;

  // Rows kb + u*RPP (u < kU) per iteration, the next iteration's loads
  // issued before this one's rows are consumed (two register sets, the loop
  // unrolled by two).  Loads past kend re-read row kend-1 (always masked),
  // so every load is unconditional and waits cover only the rows in use.
  constexpr int STEP = RPP * kU;
  auto load = [&](int k0, u32x4 (&ku)[kU], u32x4 (&vu)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int key = min(k0 + u * RPP, kend - 1);
      const ST* ks = key < na ? kc + (int64_t)key * HD : kr + (int64_t)(key - na) * HD;
      const ST* vs = key < na ? vc + (int64_t)key * HD : vr + (int64_t)(key - na) * HD;
      ku[u] = ld_raw16_nt(ks + c0);
      vu[u] = ld_raw16_nt(vs + c0);
    }
  };
  auto consume = [&](int k0, const u32x4 (&ku)[kU], const u32x4 (&vu)[kU]) {
    float sc[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float kf[VEC];
      unpack16(ku[u], kf, (ST*)nullptr);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) d += q[i] * kf[i];
#pragma unroll
      for (int msk = LPR / 2; msk >= 1; msk >>= 1) d += shfl_xor_f(d, msk);
      sc[u] = k0 + u * RPP < kend ? d : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int u = 1; u < kU; ++u) mx = fmaxf(mx, sc[u]);
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float pu = exp2f(sc[u] - mn);
      l += pu;
      float vf[VEC];
      unpack16(vu[u], vf, (ST*)nullptr);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += pu * vf[i];
    }
  };
  {
    u32x4 ka[kU], va[kU], kn[kU], vn[kU];
    int kb = kbeg + rg;
    if (kb < kend) load(kb, ka, va);
    for (; kb < kend; kb += 2 * STEP) {
      if (kb + STEP < kend) load(kb + STEP, kn, vn);
      consume(kb, ka, va);
      if (kb + STEP >= kend) break;
      if (kb + 2 * STEP < kend) load(kb + 2 * STEP, ka, va);
      consume(kb + STEP, kn, vn);
    }
  }

  // merge the row groups
  if (cl == 0) {
    s_m[rg] = m;
    s_l[rg] = l;
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_acc[rg][c0 + i] = acc[i];
  __syncthreads();

  float M = -1e30f, L = 0.f, A = 0.f;
  if (tid < HD) {
#pragma unroll 4
    for (int r = 0; r < RPP; ++r) M = fmaxf(M, s_m[r]);
#pragma unroll 4
    for (int r = 0; r < RPP; ++r) {
      const float w = exp2f(s_m[r] - M);
      L += s_l[r] * w;
      A += s_acc[r][tid] * w;
    }
  }
  if constexpr (FUSED) {
    finish_step<ST, HD>(p, b, h, M, L, A, s_red);
  } else {
    if (tid < HD) {
      float* part = p.part + (bh * p.splits + split) * (HD + 2);
      if (tid == 0) {
        part[0] = M;
        part[1] = L;
      }
      part[2 + tid] = A;
    }
  }
}

// Merge of the splits' partials by log-sum-exp.  The splits' maxima and row
// sums are read by one lane per split and reduced over the workgroup; each
// channel's accumulators are then summed in split order with the loads of
// eight splits in flight at a time (a loop with one dependent load per
// split costs a memory round trip per split).
template <int HD>
__device__ __forceinline__ float block_reduce(float v, bool is_max, float* s_tmp) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float w = shfl_xor_f(v, o);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  if ((threadIdx.x & 63) == 0) s_tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s_tmp[0];
#pragma unroll
  for (int w = 1; w < HD / 64; ++w) r = is_max ? fmaxf(r, s_tmp[w]) : r + s_tmp[w];
  __syncthreads();  // s_tmp is reused
  return r;
}

template <typename ST, int HD>
__global__ __launch_bounds__(HD) void decode_combine_kernel(const DecodeParams p) {
  __shared__ float s_red[4];
  __shared__ float s_tmp[HD / 64];
  const int bhi = blockIdx.x;
  const int b = bhi / p.H;
  const int h = bhi - b * p.H;
  const int c = threadIdx.x;
  const int S = p.splits;
  const float* part = p.part + (int64_t)bhi * S * (HD + 2);
  float m = -1e30f;
  for (int s = c; s < S; s += HD) m = fmaxf(m, part[s * (HD + 2)]);
  const float M = block_reduce<HD>(m, true, s_tmp);
  float l = 0.f;
  for (int s = c; s < S; s += HD) l += part[s * (HD + 2) + 1] * exp2f(part[s * (HD + 2)] - M);
  const float L = block_reduce<HD>(l, false, s_tmp);
  float A = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float mv[8], av[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, S - 1);
      mv[u] = part[s * (HD + 2)];
      av[u] = part[s * (HD + 2) + 2 + c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) A += av[u] * exp2f(mv[u] - M);
  }
  finish_step<ST, HD>(p, b, h, M, L, A, s_red);
}

template <typename ST, int HD>
int launch_t(const DecodeParams& p, hipStream_t st) {
  const int nbh = p.B * p.H;
  if (nbh == 0) return 0;
  if (p.splits == 1) {
    hipLaunchKernelGGL((decode_kernel<ST, HD, true>), dim3(nbh), dim3(kDecodeThreads), 0, st, p);
    return (int)hipGetLastError();
  }
  hipLaunchKernelGGL((decode_kernel<ST, HD, false>), dim3(nbh * p.splits), dim3(kDecodeThreads),
                     0, st, p);
  int e = (int)hipGetLastError();
  if (e) return e;
  hipLaunchKernelGGL((decode_combine_kernel<ST, HD>), dim3(nbh), dim3(HD), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_decode(int dtype, int hd, const DecodeParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) return hd == 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
  return hd == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace rat
