// Prefill dilated causal attention over the anchor-only cache.
//
// Method: RAT+ abstract -- attention dilated by D (FLOPs and KV cache cut by
// D), optional local window, head-wise hybrids; zhichai.net deep dive
// "RAT+ 深度拆解", section 一 (stride-D token skipping), section 2.2 (D = 1
// is dense attention), section 六 (some heads dense, the rest dilated).
// Query t attends to anchors j = D-1 (mod D), j < max(0, t-W) (compact rows
// a < floor(max(0,t-W)/D) of Kc/Vc), to the window max(0,t-W) .. t-1 and to
// itself (rows of hk/hv).
//
// Design (flash-style, one pass over q/hk/hv, o written once):
//  * workgroup = 4 waves = 128 queries of one (b, h); a workgroup takes a
//    pair of query tiles (i, nq-1-i) so all workgroups of a head cost about
//    the same; heads are ordered by per-workgroup cost (heaviest first) so a
//    head-wise hybrid launch is scheduled longest-job-first;
//  * K/V tiles of 64 keys are staged in LDS once per workgroup: K row-major,
//    V transposed (keys contiguous) so both MFMA operands are plain
//    ds_read_b128 / ds_read_b64;
//  * scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16),
//    so each lane owns one query column: the row max needs two cross-lane
//    steps, the running sum stays per lane, and P^T is already the B operand
//    of O^T += V^T P^T (keys permuted identically on both operands);
//  * the staircase mask of the anchors (a < floor(max(0,t-W)/D)) and the band
//    mask of the window are applied only on the tiles that need them;
//  * with no window the own position is a per-query dot product folded into
//    the initial softmax state (no 1-of-64 wasted MFMA band tile);
//  * online softmax in the log2 domain (exp2), fp32 accumulation, bf16 P.
#include "rat_device.h"

namespace rat {

namespace {

template <typename ST, int HD>
struct AttnCfg {
  static constexpr int BM = kAttnBM;
  static constexpr int BN = (sizeof(ST) == 4 && HD == 128) ? 32 : kAttnBN;
  static constexpr int NS = HD / 32;    // K=32 slabs of the QK^T product
  static constexpr int NDB = HD / 16;   // 16-row d-blocks of O^T
  static constexpr int NMB = BN / 16;   // 16-key blocks of S^T
  static constexpr int NKK = BN / 32;   // K=32 key slabs of the PV product
  static constexpr int PAD = 16 / (int)sizeof(ST);
  static constexpr int KSTR = HD + PAD;  // K tile row stride (elements)
  static constexpr int VSTR = BN + PAD;  // V^T tile row stride (elements)
  static constexpr int VEC = StTraits<ST>::VEC;
};

// Stage rows [row0, row0 + BN) of a [*, HD] matrix into LDS: K row-major,
// V transposed.  Rows at or beyond nvalid are zero-filled (never read).
template <typename ST, int HD>
__device__ __forceinline__ void stage_kv(const ST* __restrict__ ksrc, const ST* __restrict__ vsrc,
                                         int nvalid, ST* sK, ST* sVt) {
  using C = AttnCfg<ST, HD>;
  constexpr int VEC = C::VEC;
  constexpr int CPR = HD / VEC;  // 16-byte chunks per row
  const int tid = threadIdx.x;
#pragma unroll
  for (int idx = tid; idx < C::BN * CPR; idx += 256) {
    const int row = idx / CPR;
    const int c16 = idx - row * CPR;
    u32x4 u = {0u, 0u, 0u, 0u};
    if (row < nvalid) u = ld_raw16(ksrc + (int64_t)row * HD + c16 * VEC);
    st_raw16(sK + row * C::KSTR + c16 * VEC, u);
  }
#pragma unroll
  for (int idx = tid; idx < (C::BN / 4) * CPR; idx += 256) {
    const int kg = idx / CPR;
    const int dg = idx - kg * CPR;
    u32x4 u[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = 4 * kg + rr;
      u[rr] = u32x4{0u, 0u, 0u, 0u};
      if (row < nvalid) u[rr] = ld_raw16(vsrc + (int64_t)row * HD + dg * VEC);
    }
    ST* dst = sVt + (dg * VEC) * C::VSTR + 4 * kg;
    if constexpr (sizeof(ST) == 2) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int w = e >> 1;
        const int sh = (e & 1) * 16;
        const uint32_t x0 = (u[0][w] >> sh) & 0xffffu, x1 = (u[1][w] >> sh) & 0xffffu;
        const uint32_t x2 = (u[2][w] >> sh) & 0xffffu, x3 = (u[3][w] >> sh) & 0xffffu;
        u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
        *reinterpret_cast<u32x2*>(dst + e * C::VSTR) = pk;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        u32x4 pk = {u[0][e], u[1][e], u[2][e], u[3][e]};
        *reinterpret_cast<u32x4*>(dst + e * C::VSTR) = pk;
      }
    }
  }
}

template <typename ST, int HD>
struct WaveState {
  using C = AttnCfg<ST, HD>;
  Frag<ST> qf[2][C::NS];   // Q^T B-operand fragments of the wave's 2 query blocks
  f32x4 acc[2][C::NDB];    // O^T accumulators
  float m[2], l[2];        // running max (log2 domain) and per-lane partial sum
  int tq[2];               // query positions
  int nlo[2];              // anchors visible to each query
};

// One staged tile against one wave's 32 queries.
//  kind 0: anchors, key index = anchor index a, visible iff a < nlo(t)
//  kind 1: band,    key index = position j,     visible iff t-W <= j <= t
template <typename ST, int HD>
__device__ __forceinline__ void tile_update(WaveState<ST, HD>& ws, const ST* sK, const ST* sVt,
                                            int key0, int kind, bool need_mask, int W,
                                            float scale_log2) {
  using C = AttnCfg<ST, HD>;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;

  f32x4 S[C::NMB][2];
#pragma unroll
  for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) S[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) {
      const Frag<ST> a = frag_ld8(sK + (16 * mb + col) * C::KSTR + 32 * s + 8 * g);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) mma16(S[mb][nb], a, ws.qf[nb][s]);
    }
  }

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = S[mb][nb][i] * scale_log2;
        if (need_mask) {
          const int key = key0 + 16 * mb + 4 * g + i;
          const bool vis = (kind == 0) ? (key < ws.nlo[nb])
                                       : (key <= ws.tq[nb] && key >= ws.tq[nb] - W);
          v = vis ? v : -INFINITY;
        }
        S[mb][nb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float mnew = fmaxf(ws.m[nb], tmax);
    const float alpha = exp2f(ws.m[nb] - mnew);
    ws.m[nb] = mnew;
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2f(S[mb][nb][i] - mnew);
        S[mb][nb][i] = pv;
        lsum += pv;
      }
    ws.l[nb] = ws.l[nb] * alpha + lsum;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) ws.acc[nb][db] *= alpha;
  }

#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
    Frag<ST> pb[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) pb[nb] = frag_from(S[2 * kk][nb], S[2 * kk + 1][nb], (ST*)nullptr);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const ST* vrow = sVt + (16 * db + col) * C::VSTR + 32 * kk + 4 * g;
      const Frag<ST> va = frag_ld4x2(vrow, vrow + 16);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) mma16(ws.acc[nb][db], va, pb[nb]);
    }
  }
}

template <typename ST, int HD>
__device__ __forceinline__ void process_tile(const AttnParams& p, int b, int h, int t0, ST* sK,
                                             ST* sVt) {
  using C = AttnCfg<ST, HD>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int T = p.T;
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  const int64_t bh = (int64_t)b * p.H + h;
  const ST* qp = reinterpret_cast<const ST*>(p.q) + bh * T * HD;
  const ST* hkp = reinterpret_cast<const ST*>(p.hk) + bh * T * HD;
  const ST* hvp = reinterpret_cast<const ST*>(p.hv) + bh * T * HD;
  const ST* kcp = reinterpret_cast<const ST*>(p.Kc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
  const ST* vcp = reinterpret_cast<const ST*>(p.Vc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;

  const int tw0 = t0 + 32 * wave;              // first query of this wave
  const bool wave_active = tw0 < T;
  const int tlast_blk = min(t0 + C::BM - 1, T - 1);
  const int tlast_w = min(tw0 + 31, T - 1);

  WaveState<ST, HD> ws;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    ws.tq[nb] = tw0 + 16 * nb + col;
    const int tcl = min(ws.tq[nb], T - 1);
    ws.nlo[nb] = max(0, tcl - W) / D;
    const ST* qrow = qp + (int64_t)tcl * HD;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) ws.qf[nb][s] = frag_ld8(qrow + 32 * s + 8 * g);
    if (W == 0) {
      // own position only: fold it into the initial state
      const ST* krow = hkp + (int64_t)tcl * HD;
      float d = 0.f;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) d += frag_dot(ws.qf[nb][s], frag_ld8(krow + 32 * s + 8 * g));
      d += shfl_xor_f(d, 16);
      d += shfl_xor_f(d, 32);
      ws.m[nb] = d * p.scale_log2;
      ws.l[nb] = (g == 0) ? 1.f : 0.f;
      const ST* vrow = hvp + (int64_t)tcl * HD;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) ws.acc[nb][db] = ld4_f32(vrow + 16 * db + 4 * g);
    } else {
      ws.m[nb] = -1e30f;
      ws.l[nb] = 0.f;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) ws.acc[nb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // ---- anchors from the compact cache --------------------------------------
  const int n_end = max(0, tlast_blk - W) / D;
  const int w_end = wave_active ? max(0, tlast_w - W) / D : 0;
  const int w_full = wave_active ? max(0, tw0 - W) / D : 0;
  for (int a0 = 0; a0 < n_end; a0 += C::BN) {
    stage_kv<ST, HD>(kcp + (int64_t)a0 * HD, vcp + (int64_t)a0 * HD, n_end - a0, sK, sVt);
    __syncthreads();
    if (a0 < w_end)
      tile_update<ST, HD>(ws, sK, sVt, a0, 0, a0 + C::BN > w_full, W, p.scale_log2);
    __syncthreads();
  }

  // ---- window band (own position included) from hk/hv -----------------------
  if (W > 0) {
    const int jb0 = max(0, t0 - W);
    const int wj0 = max(0, tw0 - W);
    for (int j0 = jb0; j0 <= tlast_blk; j0 += C::BN) {
      stage_kv<ST, HD>(hkp + (int64_t)j0 * HD, hvp + (int64_t)j0 * HD, tlast_blk + 1 - j0, sK,
                       sVt);
      __syncthreads();
      if (wave_active && j0 <= tlast_w && j0 + C::BN > wj0) {
        // the tile is fully visible to all 32 queries iff
        // tw0+31 - W <= j0 and j0 + BN - 1 <= tw0 (and no clamped rows)
        const bool full = (tw0 + 31 - W <= j0) && (j0 + C::BN - 1 <= tw0) && (tw0 + 31 < T);
        tile_update<ST, HD>(ws, sK, sVt, j0, 1, !full, W, p.scale_log2);
      }
      __syncthreads();
    }
  }

  // ---- normalise and store --------------------------------------------------
  ST* op = reinterpret_cast<ST*>(p.o) + bh * T * HD;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float lt = ws.l[nb];
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    const int t = ws.tq[nb];
    if (t < T) {
      const float inv = 1.f / lt;
      ST* orow = op + (int64_t)t * HD;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) st4(orow + 16 * db + 4 * g, ws.acc[nb][db] * inv);
      if (p.lse != nullptr && g == 0) p.lse[bh * T + t] = (ws.m[nb] + __log2f(lt)) * kLn2;
    }
  }
}

template <typename ST, int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const AttnParams p) {
  using C = AttnCfg<ST, HD>;
  __shared__ __attribute__((aligned(16))) ST sK[C::BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) ST sVt[HD * C::VSTR];

  const int L = blockIdx.x;
  const int per_rank = p.B * p.np;
  const int rank = L / per_rank;
  const int rem = L - rank * per_rank;
  const int b = rem / p.np;
  const int pr = rem - b * p.np;
  const int h = p.perm[rank];

  const int qa = p.nq - 1 - pr;  // heavy tile first
  process_tile<ST, HD>(p, b, h, qa * C::BM, sK, sVt);
  if (pr < qa) {
    __syncthreads();
    process_tile<ST, HD>(p, b, h, pr * C::BM, sK, sVt);
  }
}

template <typename ST, int HD>
int launch_t(const AttnParams& p, hipStream_t st) {
  const int64_t nblk = (int64_t)p.H * p.B * p.np;
  if (nblk == 0) return 0;
  hipLaunchKernelGGL((attn_prefill_kernel<ST, HD>), dim3((unsigned)nblk), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_attn_prefill(int dtype, int hd, const AttnParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) return hd == 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
  return hd == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace rat
