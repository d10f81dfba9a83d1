// Decode step of dilated attention combined with top-k block selection, and
// the history cache it reads.
//
// Method: RAT+ abstract (v1) -- a RAT+ model sparsified to top-k block
// attention; zhichai.net deep dive "RAT+ 深度拆解", section 四 -- dilation
// and top-k block selection combine: the dilated anchors cover the whole
// past, the selected blocks add density where the query needs it.  The
// pages fix neither the block size nor the scoring; the reading here:
//  * blocks are the aligned runs of kTopkBlock positions, eligible when
//    they lie wholly before the window start max(0, pos - W);
//  * a block's score is q . (mean stored key state of the block), kept per
//    block in fp32 beside the history; the k highest are selected (equal
//    scores: the lower block first);
//  * the query attends to its dilated key set (anchors, window, itself) and
//    to the selected blocks' positions that are not anchor positions (an
//    anchor position in an eligible block is always an included anchor, so
//    the union counts it once).
//
// Design: one workgroup per (b, h).  The block scores go to LDS, sized to
// the block table (one fp32 mean row per 8-32 lanes, reduced by cross-lane
// adds), k rounds of a workgroup arg-max select the blocks, then the
// anchors, ring slots and the selected blocks' rows are streamed with an
// online softmax as in the plain decode step (16-byte loads, one row per
// 8-32 lanes, 4 rows in flight per lane group); after every read the step
// writes o, the state, the ring slot, the anchor row, the history row pos
// and, when pos ends a block, that block's mean.
#include "rat_device.h"

namespace rat {

namespace {

constexpr int kTU = 4;  // rows per lane group per iteration
constexpr int kSU = 4;  // block-mean rows per lane group per scoring pass

// History rows t0 .. t0+T-1 that fall in one block of kTopkBlock rows of
// one (b, h), and the block's mean once the block is complete.  Rows of the
// block before t0 were written by an earlier call and are read back from the
// history for the mean.
template <typename ST, int HD>
__global__ __launch_bounds__(256) void topk_cache_build_kernel(const ST* __restrict__ hk,
                                                               const ST* __restrict__ hv, ST* Hk,
                                                               ST* Hv, float* means, int T,
                                                               int t0, int64_t T_cap, int64_t NB) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;  // lanes per row
  constexpr int RG = 256 / LPR;  // row groups
  __shared__ float s_sum[RG][HD];
  const int m = t0 / kTopkBlock + (int)blockIdx.x;
  const int64_t bh = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int tid = threadIdx.x;
  const int rg = tid / LPR;
  const int c0 = (tid - rg * LPR) * VEC;
  const int b0 = m * kTopkBlock;
  const int r0 = max(b0, t0);
  const int r1 = min(t0 + T, b0 + kTopkBlock);
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  for (int r = r0 + rg; r < r1; r += RG) {
    const u32x4 ku = ld_raw16(hk + (bh * T + (r - t0)) * HD + c0);
    const u32x4 vu = ld_raw16(hv + (bh * T + (r - t0)) * HD + c0);
    st_raw16(Hk + (bh * T_cap + r) * HD + c0, ku);
    st_raw16(Hv + (bh * T_cap + r) * HD + c0, vu);
    float kf[VEC];
    unpack16(ku, kf, (ST*)nullptr);
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] += kf[i];
  }
  if (r1 - b0 < kTopkBlock) return;  // block not complete yet (uniform): no mean
  for (int r = b0 + rg; r < r0; r += RG) {  // rows of an earlier call
    float kf[VEC];
    unpack16(ld_raw16(Hk + (bh * T_cap + r) * HD + c0), kf, (ST*)nullptr);
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] += kf[i];
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_sum[rg][c0 + i] = acc[i];
  __syncthreads();
  if (tid < HD) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += s_sum[g][tid];
    means[(bh * NB + m) * HD + tid] = s * (1.0f / kTopkBlock);
  }
}

template <typename ST, int HD>
__global__ __launch_bounds__(256) void decode_topk_kernel(const TopkParams p) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;    // lanes per row
  constexpr int RPP = 256 / LPR;   // rows per pass
  extern __shared__ float s_sc[];  // [NB] block scores (dynamic LDS)
  __shared__ int s_sel[kTopkMaxK];
  __shared__ float s_m[RPP], s_l[RPP];
  __shared__ float s_acc[RPP][HD];
  __shared__ float s_redf[4];
  __shared__ int s_redi[4];

  const int bhi = blockIdx.x;
  const int b = bhi / p.H;
  const int h = bhi - b * p.H;
  const int64_t bh = bhi;
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  const int pos = p.pos;
  const int lo = max(0, pos - W);
  const int na = lo / D;               // anchors
  const int nw = pos - lo;             // window positions (ring slots)
  const int ne = lo / kTopkBlock;      // eligible blocks
  const int ks = min(p.k, ne);         // blocks selected
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // ---- scores of the eligible blocks (q . mean key state) ----------------
  // kSU rows per lane group per pass: every load of a pass is issued before
  // the first is used (rows past the last eligible block re-read it)
  const float* mp = p.means + bh * p.NB * HD;
  for (int m0 = 0; m0 < ne; m0 += RPP * kSU) {
    f32x4 f[kSU][VEC / 4];
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      const float* row = mp + (int64_t)min(m0 + u * RPP + rg, ne - 1) * HD + c0;
#pragma unroll
      for (int i = 0; i < VEC / 4; ++i) f[u][i] = *reinterpret_cast<const f32x4*>(row + 4 * i);
    }
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < VEC / 4; ++i)
        d += q[4 * i] * f[u][i][0] + q[4 * i + 1] * f[u][i][1] + q[4 * i + 2] * f[u][i][2] +
             q[4 * i + 3] * f[u][i][3];
#pragma unroll
      for (int msk = LPR / 2; msk >= 1; msk >>= 1) d += shfl_xor_f(d, msk);
      const int m = m0 + u * RPP + rg;
      if (cl == 0 && m < ne) s_sc[m] = d;
    }
  }
  __syncthreads();

  // ---- top-k: ks rounds of a workgroup arg-max (ties: lower block) --------
  for (int r = 0; r < ks; ++r) {
    float best = -INFINITY;
    int bi = INT32_MAX;
    for (int m = tid; m < ne; m += 256) {
      const float s = s_sc[m];
      if (s > best || (s == best && m < bi)) {
        best = s;
        bi = m;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ob = __shfl_xor(best, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (lane == 0) {
      s_redf[wave] = best;
      s_redi[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float bb = s_redf[0];
      int ii = s_redi[0];
      for (int w = 1; w < 4; ++w)
        if (s_redf[w] > bb || (s_redf[w] == bb && s_redi[w] < ii)) {
          bb = s_redf[w];
          ii = s_redi[w];
        }
      // no comparable score left (NaN input): the slot selects nothing
      if (ii >= ne) ii = -1;
      s_sel[r] = ii;
      // a taken block becomes NaN, which no comparison selects again
      if (ii >= 0) s_sc[ii] = __builtin_nanf("");
    }
    __syncthreads();
  }

  // ---- attention: anchors, window slots, selected blocks' rows ------------
  const ST* kc = reinterpret_cast<const ST*>(p.Kc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
  const ST* vc = reinterpret_cast<const ST*>(p.Vc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
  const ST* kr = reinterpret_cast<const ST*>(p.kr) + ((int64_t)b * p.WS + p.ht.roff[h]) * HD;
  const ST* vr = reinterpret_cast<const ST*>(p.vr) + ((int64_t)b * p.WS + p.ht.roff[h]) * HD;
  const ST* hkh = reinterpret_cast<const ST*>(p.hk) + bh * p.T_cap * HD;
  const ST* hvh = reinterpret_cast<const ST*>(p.hv) + bh * p.T_cap * HD;
  const int nk = na + nw + ks * kTopkBlock;

  float m = -1e30f, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  for (int kb = rg; kb < nk; kb += RPP * kTU) {
    u32x4 ku[kTU], vu[kTU];
    bool ok[kTU];
#pragma unroll
    for (int u = 0; u < kTU; ++u) {
      const int key0 = kb + u * RPP;
      const int key = min(key0, nk - 1);
      // key index -> row: anchors [0, na), ring slots [na, na+nw), then the
      // selected blocks' rows (an anchor position among them is skipped)
      const int rb = key - na - nw;
      const int blk = rb >= 0 ? s_sel[rb / kTopkBlock] : 0;
      const int bp = max(blk, 0) * kTopkBlock + (rb >= 0 ? rb % kTopkBlock : 0);
      bool valid = key0 < nk;
      if (rb >= 0) valid = valid && blk >= 0 && bp % D != D - 1;
      const ST* ks_ = key < na ? kc + (int64_t)key * HD
                               : (rb < 0 ? kr + (int64_t)(key - na) * HD : hkh + (int64_t)bp * HD);
      const ST* vs_ = key < na ? vc + (int64_t)key * HD
                               : (rb < 0 ? vr + (int64_t)(key - na) * HD : hvh + (int64_t)bp * HD);
      ku[u] = ld_raw16_nt(ks_ + c0);
      vu[u] = ld_raw16_nt(vs_ + c0);
      ok[u] = valid;
    }
    float sc[kTU];
#pragma unroll
    for (int u = 0; u < kTU; ++u) {
      float kf[VEC];
      unpack16(ku[u], kf, (ST*)nullptr);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) d += q[i] * kf[i];
#pragma unroll
      for (int msk = LPR / 2; msk >= 1; msk >>= 1) d += shfl_xor_f(d, msk);
      sc[u] = ok[u] ? d : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int u = 1; u < kTU; ++u) mx = fmaxf(mx, sc[u]);
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < kTU; ++u) {
      const float pu = exp2f(sc[u] - mn);
      l += pu;
      float vf[VEC];
      unpack16(vu[u], vf, (ST*)nullptr);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += pu * vf[i];
    }
  }

  // merge the row groups
  if (cl == 0) {
    s_m[rg] = m;
    s_l[rg] = l;
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_acc[rg][c0 + i] = acc[i];
  __syncthreads();  // every read of the step is complete from here on

  float M = -1e30f, L = 0.f, A = 0.f;
  if (tid < HD) {
    for (int r = 0; r < RPP; ++r) M = fmaxf(M, s_m[r]);
    for (int r = 0; r < RPP; ++r) {
      const float w = exp2f(s_m[r] - M);
      L += s_l[r] * w;
      A += s_acc[r][tid] * w;
    }
  }

  // ---- own position, state update and the step's writes -------------------
  const int c = tid;
  float hatk = 0.f, hatv = 0.f, nsk = 0.f, nsv = 0.f, part = 0.f;
  if (c < HD) {
    const int64_t i = bh * HD + c;
    const float gg = (float)reinterpret_cast<const ST*>(p.g)[i];
    nsk = gg * p.sk[i] + (1.f - gg) * (float)reinterpret_cast<const ST*>(p.k_in)[i];
    nsv = gg * p.sv[i] + (1.f - gg) * (float)reinterpret_cast<const ST*>(p.v_in)[i];
    hatk = st_round(nsk, (ST*)nullptr);
    hatv = st_round(nsv, (ST*)nullptr);
    part = (float)reinterpret_cast<const ST*>(p.q)[i] * p.scale_log2 * hatk;
  }
  for (int msk = 32; msk >= 1; msk >>= 1) part += shfl_xor_f(part, msk);
  if (lane == 0) s_redf[wave] = part;
  __syncthreads();
  float sown = 0.f;
#pragma unroll
  for (int w = 0; w < (HD + 63) / 64; ++w) sown += s_redf[w];
  if (c < HD) {
    const float Mn = fmaxf(M, sown);
    const float a = exp2f(M - Mn);
    const float e = exp2f(sown - Mn);
    reinterpret_cast<ST*>(p.o)[bh * HD + c] = (ST)((A * a + e * hatv) / (L * a + e));
    p.sk[bh * HD + c] = nsk;
    p.sv[bh * HD + c] = nsv;
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
    // the history row of pos, and the mean of the block pos completes
    reinterpret_cast<ST*>(p.hk)[(bh * p.T_cap + pos) * HD + c] = (ST)hatk;
    reinterpret_cast<ST*>(p.hv)[(bh * p.T_cap + pos) * HD + c] = (ST)hatv;
    const int mb = pos / kTopkBlock;
    if (pos % kTopkBlock == kTopkBlock - 1 && mb < p.NB) {
      float s = 0.f;
      for (int r = pos - kTopkBlock + 1; r < pos; ++r) s += (float)hkh[(int64_t)r * HD + c];
      p.means[(bh * p.NB + mb) * HD + c] = (s + hatk) * (1.0f / kTopkBlock);
    }
  }
  if (p.sel != nullptr && tid < p.k) p.sel[bh * p.k + tid] = tid < ks ? s_sel[tid] : -1;
}

template <typename ST, int HD>
int launch_t(const TopkParams& p, hipStream_t st) {
  const int64_t nbh = (int64_t)p.B * p.H;
  if (nbh == 0) return 0;
  const size_t lds = sizeof(float) * (size_t)(p.NB > 0 ? p.NB : 1);
  hipLaunchKernelGGL((decode_topk_kernel<ST, HD>), dim3((unsigned)nbh), dim3(256), lds, st, p);
  return (int)hipGetLastError();
}

template <typename ST, int HD>
int launch_build_t(int B, int H, int64_t T, int64_t T_cap, int64_t t0, const void* hk,
                   const void* hv, void* Hk, void* Hv, float* means, hipStream_t st) {
  if (B == 0 || H == 0 || T == 0) return 0;
  // the blocks that rows t0 .. t0+T-1 touch
  const int64_t nblk = (t0 + T - 1) / kTopkBlock - t0 / kTopkBlock + 1;
  const dim3 grid((unsigned)nblk, (unsigned)H, (unsigned)B);
  hipLaunchKernelGGL((topk_cache_build_kernel<ST, HD>), grid, dim3(256), 0, st,
                     reinterpret_cast<const ST*>(hk), reinterpret_cast<const ST*>(hv),
                     reinterpret_cast<ST*>(Hk), reinterpret_cast<ST*>(Hv), means, (int)T, (int)t0,
                     T_cap, T_cap / kTopkBlock);
  return (int)hipGetLastError();
}

}  // namespace

int launch_decode_topk(int dtype, int hd, const TopkParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) return hd == 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
  return hd == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

int launch_topk_cache_build(int dtype, int hd, int B, int H, int64_t T, int64_t T_cap,
                            int64_t t0, const void* hk, const void* hv, void* Hk, void* Hv,
                            float* means, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16)
    return hd == 128 ? launch_build_t<bf16, 128>(B, H, T, T_cap, t0, hk, hv, Hk, Hv, means, st)
                     : launch_build_t<bf16, 64>(B, H, T, T_cap, t0, hk, hv, Hk, Hv, means, st);
  return hd == 128 ? launch_build_t<float, 128>(B, H, T, T_cap, t0, hk, hv, Hk, Hv, means, st)
                   : launch_build_t<float, 64>(B, H, T, T_cap, t0, hk, hv, Hk, Hv, means, st);
}

}  // namespace rat
