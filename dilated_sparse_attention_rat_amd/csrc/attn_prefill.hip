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
//  * workgroup = 4 waves = 64*QB queries of one (b, h), QB = 16-query blocks
//    per wave (1 for streaming-bound calls: fewer registers, more waves in
//    flight; 2 for MFMA-bound calls: twice the reuse of every LDS operand);
//    a workgroup takes a pair of query tiles (i, nq-1-i) so all workgroups of
//    a head cost about the same; heads are ordered by per-workgroup cost
//    (heaviest first) so a head-wise hybrid launch is longest-job-first;
//  * K/V tiles of 64 keys are staged in LDS once per workgroup: K row-major,
//    V transposed (keys contiguous) so both MFMA operands are plain
//    ds_read_b128 / ds_read_b64; the global loads of tile i+1 are issued
//    into registers before tile i's MFMAs, so their latency is hidden;
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

constexpr float kRescaleSlack = 8.0f;  // log2 units

template <typename ST, int HD, int QB>
struct AttnCfg {
  static constexpr int BM = 64 * QB;    // queries per tile: 4 waves x 16*QB
  static constexpr int BN = (sizeof(ST) == 4 && HD == 128) ? 32 : kAttnBN;
  static constexpr int NS = HD / 32;    // K=32 slabs of the QK^T product
  static constexpr int NDB = HD / 16;   // 16-row d-blocks of O^T
  static constexpr int NMB = BN / 16;   // 16-key blocks of S^T
  static constexpr int NKK = BN / 32;   // K=32 key slabs of the PV product
  // Row strides padded so that the fragment reads of 16 (K, 16 B each) or 16
  // (V^T, 8 B each) consecutive lanes hit distinct LDS banks: K rows are
  // 68 dwords apart (bf16) and V^T rows 34 dwords apart.
  static constexpr int KSTR = HD + 16 / (int)sizeof(ST);  // K tile row stride
  static constexpr int VSTR = BN + 4;                     // V^T tile row stride
  static constexpr int VEC = StTraits<ST>::VEC;
  static constexpr int CPR = HD / VEC;   // 16-byte chunks per row
  static constexpr int KITEMS = BN * CPR;          // K chunks per tile
  static constexpr int VITEMS = (BN / 4) * CPR;    // V work items (4 rows x VEC)
  static constexpr int KPT = (KITEMS + 255) / 256;  // per thread
  static constexpr int VPT = (VITEMS + 255) / 256;
};

// One K/V tile held in registers between its global load and its LDS store
// (the load of tile i+1 is in flight while tile i is being computed).  V work
// items run key-group fastest so that the transposed LDS stores of
// consecutive lanes land in consecutive 8-byte slots (no bank conflicts).
template <typename ST, int HD, int QB>
struct Prefetch {
  using C = AttnCfg<ST, HD, QB>;
  u32x4 k[C::KPT];
  u32x4 v[C::VPT][4];

  // Rows [0, BN) of ksrc/vsrc (nvalid >= 1).  Rows at or beyond nvalid
  // re-read row nvalid-1: such keys are always masked (weight exactly 0) and
  // the duplicated V row is finite, so they contribute nothing, and the
  // loads need no branches.
  __device__ __forceinline__ void load(const ST* __restrict__ ksrc, const ST* __restrict__ vsrc,
                                       int nvalid) {
    const int tid = threadIdx.x;
    const int last = nvalid - 1;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int idx = min(tid + 256 * i, C::KITEMS - 1);
      const int row = idx / C::CPR;
      const int c16 = idx - row * C::CPR;
      k[i] = ld_raw16(ksrc + (int64_t)min(row, last) * HD + c16 * C::VEC);
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int idx = min(tid + 256 * i, C::VITEMS - 1);
      const int dg = idx / (C::BN / 4);
      const int kg = idx - dg * (C::BN / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        v[i][rr] = ld_raw16(vsrc + (int64_t)min(4 * kg + rr, last) * HD + dg * C::VEC);
    }
  }

  // K row-major, V transposed (keys contiguous)
  __device__ __forceinline__ void store(ST* sK, ST* sVt) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / C::CPR;
      const int c16 = idx - row * C::CPR;
      if (idx < C::KITEMS) st_raw16(sK + row * C::KSTR + c16 * C::VEC, k[i]);
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int idx = tid + 256 * i;
      const int dg = idx / (C::BN / 4);
      const int kg = idx - dg * (C::BN / 4);
      if (idx >= C::VITEMS) continue;
      ST* dst = sVt + (dg * C::VEC) * C::VSTR + 4 * kg;
      if constexpr (sizeof(ST) == 2) {
#pragma unroll
        for (int e = 0; e < C::VEC; ++e) {
          const int w = e >> 1;
          const int sh = (e & 1) * 16;
          const uint32_t x0 = (v[i][0][w] >> sh) & 0xffffu, x1 = (v[i][1][w] >> sh) & 0xffffu;
          const uint32_t x2 = (v[i][2][w] >> sh) & 0xffffu, x3 = (v[i][3][w] >> sh) & 0xffffu;
          u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
          *reinterpret_cast<u32x2*>(dst + e * C::VSTR) = pk;
        }
      } else {
#pragma unroll
        for (int e = 0; e < C::VEC; ++e) {
          u32x4 pk = {v[i][0][e], v[i][1][e], v[i][2][e], v[i][3][e]};
          *reinterpret_cast<u32x4*>(dst + e * C::VSTR) = pk;
        }
      }
    }
  }
};

template <typename ST, int HD, int QB>
struct WaveState {
  using C = AttnCfg<ST, HD, QB>;
  Frag<ST> qf[QB][C::NS];  // Q^T B-operand fragments of the wave's query blocks
  f32x4 acc[QB][C::NDB];   // O^T accumulators
  float m[QB], l[QB];      // running max (log2 domain) and per-lane partial sum
  int tq[QB];              // query positions
  int nlo[QB];             // anchors visible to each query
};

// One staged tile against one wave's 16*QB queries.
//  kind 0: anchors, key index = anchor index a, visible iff a < nlo(t)
//  kind 1: band,    key index = position j,     visible iff t-W <= j <= t
template <typename ST, int HD, int QB>
__device__ __forceinline__ void tile_update(WaveState<ST, HD, QB>& ws, const ST* sK,
                                            const ST* sVt, int key0, int kind, bool need_mask,
                                            int W, float scale_log2) {
  using C = AttnCfg<ST, HD, QB>;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;

  f32x4 S[C::NMB][QB];
#pragma unroll
  for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) S[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) {
      const Frag<ST> a = frag_ld8(sK + (16 * mb + col) * C::KSTR + 32 * s + 8 * g);
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) mma16(S[mb][nb], a, ws.qf[nb][s]);
    }
  }

  // Online softmax in the log2 domain, scores scaled by c = scale*log2(e).
  // The running max m is raised only when a tile's max exceeds it by more
  // than kRescaleSlack: every weight is then exp2(c*s - m) <= 2^kRescaleSlack
  // (no overflow in fp32 or bf16), the result is the same softmax, and the
  // accumulators are rescaled on few tiles (wave-uniform skip otherwise).
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    // visible keys of this lane's query: lo <= key <= hi
    //   anchors: a < nlo(t);  band: t - W <= j <= t
    const int lo = kind == 0 ? 0 : ws.tq[nb] - W;
    const int hi = kind == 0 ? ws.nlo[nb] - 1 : ws.tq[nb];
    const int base = key0 + 4 * g - lo;
    const uint32_t span = (uint32_t)(hi - lo);
    float tmax = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = (uint32_t)(base + 16 * mb + i) <= span && hi >= lo;
          S[mb][nb][i] = vis ? S[mb][nb][i] : -INFINITY;
        }
    }
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, S[mb][nb][i]);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float mcand = tmax * scale_log2;
    const bool grow = mcand > ws.m[nb] + kRescaleSlack;
    if (__any(grow)) {
      const float mnew = grow ? mcand : ws.m[nb];
      const float alpha = __builtin_amdgcn_exp2f(ws.m[nb] - mnew);
      ws.m[nb] = mnew;
      ws.l[nb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) ws.acc[nb][db] *= alpha;
    }
    const float mneg = -ws.m[nb];
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][nb][i], scale_log2, mneg));
        S[mb][nb][i] = pv;
        lsum += pv;
      }
    ws.l[nb] += lsum;
  }

#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
    Frag<ST> pb[QB];
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) pb[nb] = frag_from(S[2 * kk][nb], S[2 * kk + 1][nb], (ST*)nullptr);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const ST* vrow = sVt + (16 * db + col) * C::VSTR + 32 * kk + 4 * g;
      const Frag<ST> va = frag_ld4x2(vrow, vrow + 16);
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) mma16(ws.acc[nb][db], va, pb[nb]);
    }
  }
}

template <typename ST, int HD, int QB>
__device__ __forceinline__ void process_tile(const AttnParams& p, int b, int h, int t0, ST* sK,
                                             ST* sVt) {
  using C = AttnCfg<ST, HD, QB>;
  constexpr int QW = 16 * QB;  // queries per wave
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

  const int tw0 = t0 + QW * wave;              // first query of this wave
  const bool wave_active = tw0 < T;
  const int tlast_blk = min(t0 + C::BM - 1, T - 1);
  const int tlast_w = min(tw0 + QW - 1, T - 1);

  // the tile's key tiles: anchors [0, n_end) then the band [jb0, tlast_blk]
  const int n_end = max(0, tlast_blk - W) / D;
  const int jb0 = max(0, t0 - W);
  const int na_t = (n_end + C::BN - 1) / C::BN;
  const int nb_t = W > 0 ? (tlast_blk - jb0 + C::BN) / C::BN : 0;
  const int n_items = na_t + nb_t;
  auto item_src = [&](int i, const ST*& ks, const ST*& vs, int& nvalid, int& key0) {
    if (i < na_t) {
      key0 = i * C::BN;
      ks = kcp + (int64_t)key0 * HD;
      vs = vcp + (int64_t)key0 * HD;
      nvalid = n_end - key0;
    } else {
      key0 = jb0 + (i - na_t) * C::BN;
      ks = hkp + (int64_t)key0 * HD;
      vs = hvp + (int64_t)key0 * HD;
      nvalid = tlast_blk + 1 - key0;
    }
  };

  Prefetch<ST, HD, QB> pf;
  if (n_items > 0) {
    const ST *ks, *vs;
    int nv, k0;
    item_src(0, ks, vs, nv, k0);
    pf.load(ks, vs, nv);
  }

  WaveState<ST, HD, QB> ws;
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
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

  const int w_end = wave_active ? max(0, tlast_w - W) / D : 0;
  const int w_full = wave_active ? max(0, tw0 - W) / D : 0;
  const int wj0 = max(0, tw0 - W);
  for (int i = 0; i < n_items; ++i) {
    __syncthreads();  // every wave is done reading the previous tile
    pf.store(sK, sVt);
    __syncthreads();
    const ST *ks, *vs;
    int nv, key0;
    if (i + 1 < n_items) {  // next tile's loads overlap this tile's MFMAs
      item_src(i + 1, ks, vs, nv, key0);
      pf.load(ks, vs, nv);
    }
    item_src(i, ks, vs, nv, key0);
    const int kind = i < na_t ? 0 : 1;
    bool part, need_mask;
    if (kind == 0) {
      part = key0 < w_end;
      need_mask = key0 + C::BN > w_full;
    } else {
      part = wave_active && key0 <= tlast_w && key0 + C::BN > wj0;
      // fully visible to all of the wave's queries iff
      // tw0+QW-1 - W <= key0 and key0 + BN - 1 <= tw0 (and no clamped rows)
      need_mask = !((tw0 + QW - 1 - W <= key0) && (key0 + C::BN - 1 <= tw0) && (tw0 + QW - 1 < T));
    }
    if (part) tile_update<ST, HD, QB>(ws, sK, sVt, key0, kind, need_mask, W, p.scale_log2);
  }

  // ---- normalise and store --------------------------------------------------
  ST* op = reinterpret_cast<ST*>(p.o) + bh * T * HD;
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
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

// Occupancy target: 2 waves per SIMD (two workgroups per CU) for both QB, so
// one workgroup's MFMAs overlap the other's staging and softmax (QB = 2 fits
// the resulting 256-register budget without spills).
template <typename ST, int HD, int QB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_kernel(const AttnParams p) {
  using C = AttnCfg<ST, HD, QB>;
  __shared__ __attribute__((aligned(16))) ST sK[C::BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) ST sVt[HD * C::VSTR];

  const int L = blockIdx.x;
  const int per_rank = p.B * p.np;
  const int rank = L / per_rank;
  const int rem = L - rank * per_rank;
  const int b = rem / p.np;
  const int pr = rem - b * p.np;
  const int h = p.perm[rank];

  const int qa = p.nq - 1 - pr;  // heavy tile first, then its partner
  const int ntiles = pr < qa ? 2 : 1;
  for (int it = 0; it < ntiles; ++it)
    process_tile<ST, HD, QB>(p, b, h, (it == 0 ? qa : pr) * C::BM, sK, sVt);
}

template <typename ST, int HD>
int launch_t(const AttnParams& p, hipStream_t st) {
  const int64_t nblk = (int64_t)p.H * p.B * p.np;
  if (nblk == 0) return 0;
  if (p.qb == 2)
    hipLaunchKernelGGL((attn_prefill_kernel<ST, HD, 2>), dim3((unsigned)nblk), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<ST, HD, 1>), dim3((unsigned)nblk), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_attn_prefill(int dtype, int hd, const AttnParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) return hd == 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
  return hd == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace rat
