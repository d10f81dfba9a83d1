// Prefill backward: gradients of q, k, v and g for a loss whose gradient
// with respect to the attention output o is dO (the training path of RAT+:
// dense pretraining with active recurrence learning and a short adaptation
// to a dilation, zhichai.net deep dive, sections 2.2 and 2.3).  The
// recurrence (section 2.1) and the dilated attention (abstract; section 一)
// are the forward of csrc/scan.hip and csrc/attn_prefill.hip.
//
// Kernels, in stream order:
//  1. bwd_dq_kernel (query-parallel, MFMA): per query t over its key set
//     (anchors j = D-1 mod D before the window, the window t-W..t-1, t):
//     P = exp2(c*q.hk - lse*log2 e) from the forward's lse, dP = dO.hv,
//     delta = dO.o, dS = P (dP - delta); dq = scale sum dS hk.  The own
//     position is handled per lane: its dq term, and the two scalars of its
//     state-gradient terms (scale dS_own and P_own; the terms are those
//     times q_t and dO_t) kept for kernel 3; delta is kept for kernel 2.
//  2. bwd_dkv_kernel (key-parallel, MFMA): for each tile of 64 keys -- a
//     tile of anchors (rows of hk/hv at positions aD+D-1) or a tile of
//     window positions -- over the query tiles that see them:
//     dhv += P^T dO, dhk += scale dS^T q.  An anchor tile's queries are split
//     over several workgroups, each writing a partial sum of the anchor
//     gradients; window tiles write the window gradients of their positions.
//  3. bwd_rscan_kernel: the recurrence in reverse,
//     lambda_t = dh_t + g_{t+1} lambda_{t+1} (lambda_T = 0), where dh_t is the
//     own term, the window gradient and, at anchor positions, the anchor
//     gradient's partial sums; dk = (1-g) lambda_k,
//     dv = (1-g) lambda_v, dg = lambda_k (h^k_{t-1} - k) + lambda_v
//     (h^v_{t-1} - v) with the stored states (h_{-1} = 0).  One persistent
//     pass over chunks from the end of the sequence, linked by the forward
//     scan's chunk-aggregate tree, so every row is read once.  With several
//     partial anchor gradients, a small kernel first sums them into the
//     first buffer.
// The storage rounding of the states enters the derivative as the identity.
#include <algorithm>

#include "scan_tree.h"

// fp32 tiles at hd = 128 need more LDS than two workgroups per CU allow, so
// those instantiations run at one wave per SIMD (the bf16 ones at two)
#pragma clang diagnostic ignored "-Wpass-failed"

namespace rat {

namespace {

// XCD-aware block order: workgroups are dealt round-robin over the 8 XCDs,
// each with its own L2.  Block L is the (L / 8)-th block of XCD L % 8; the
// per-XCD sequence runs over whole (b, h) groups of n blocks, so all blocks
// of one (b, h) -- which share that head's Q, dO and anchor rows -- run on
// one XCD.  Returns false for the padding blocks past B*H.
constexpr int kXcds = 8;
__device__ __forceinline__ bool xcd_group(int nbh, int n, int& bh, int& x) {
  const int L = blockIdx.x;
  const int xcd = L % kXcds;
  const int s = L / kXcds;
  bh = (s / n) * kXcds + xcd;
  x = s % n;
  return bh < nbh;
}

template <typename ST, int HD>
struct BwdCfg {
  static constexpr int BN = 64;          // keys (or queries) per staged tile
  static constexpr int NS = HD / 32;     // K=32 slabs over channels
  static constexpr int NDB = HD / 16;    // 16-channel blocks of the transposed accumulators
  static constexpr int NMB = BN / 16;    // 16-row blocks of a score tile
  static constexpr int NKK = BN / 32;    // K=32 slabs over the tile's rows
  static constexpr int VEC = StTraits<ST>::VEC;
  static constexpr int CPR = HD / VEC;   // 16-byte chunks per row
  // padded strides (as in the forward): row-major rows 68 dwords apart
  // (bf16), transposed rows 34 dwords apart
  static constexpr int RSTR = HD + 16 / (int)sizeof(ST);
  static constexpr int TSTR = BN + 4;
  static constexpr int G4 = (BN / 4) * CPR;       // items of 4 rows x VEC channels
  static constexpr int G4PT = (G4 + 255) / 256;   // per thread
  // bf16 reads the transposed operands straight out of the row-major tile
  // (ds_read_b64_tr_b16); fp32 stages a transposed copy
  static constexpr bool TR = sizeof(ST) == 2;
  static constexpr int TLDS = TR ? 8 : HD * TSTR;  // transposed copy (elements)
};

// A operand whose K dimension runs over a staged tile's rows: channels
// 16db + col, rows 32kk + 4g + j (slots j < 4) and 32kk + 16 + 4g + j (slots
// j >= 4), from the row-major tile (bf16) or its transposed copy (fp32).
template <typename ST, int HD>
__device__ __forceinline__ Frag<ST> frag_rows(const ST* sRow, const ST* sT, int kk, int db,
                                              int col, int g) {
  using C = BwdCfg<ST, HD>;
  if constexpr (C::TR) {
    return frag_ld_tr(sRow + (32 * kk + 4 * g + (col >> 2)) * C::RSTR + 16 * db + 4 * (col & 3),
                      16 * C::RSTR);
  } else {
    const ST* r = sT + (16 * db + col) * C::TSTR + 32 * kk + 4 * g;
    return frag_ld4x2(r, r + 16);
  }
}

// A tile of BN rows staged through registers into LDS: items of 4
// consecutive rows x VEC channels, stored row-major and, with TRANS, also
// transposed (rows contiguous per channel, the layout of an A operand whose
// K dimension runs over the tile's rows).  Rows at or beyond nvalid re-read
// row nvalid-1 (finite; every use of them is masked).
template <typename ST, int HD, bool TRANS>
struct Stage4 {
  using C = BwdCfg<ST, HD>;
  u32x4 r[C::G4PT][4];

  template <typename RowPtr>
  __device__ __forceinline__ void load(RowPtr row, int nvalid) {
    const int tid = threadIdx.x;
    const int last = nvalid - 1;
#pragma unroll
    for (int i = 0; i < C::G4PT; ++i) {
      const int idx = min(tid + 256 * i, C::G4 - 1);
      const int dg = idx / (C::BN / 4);
      const int kg = idx - dg * (C::BN / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) r[i][rr] = ld_raw16(row(min(4 * kg + rr, last)) + dg * C::VEC);
    }
  }

  __device__ __forceinline__ void store(ST* sRow, ST* sT) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::G4PT; ++i) {
      const int idx = tid + 256 * i;
      if (idx >= C::G4) continue;
      const int dg = idx / (C::BN / 4);
      const int kg = idx - dg * (C::BN / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) st_raw16(sRow + (4 * kg + rr) * C::RSTR + dg * C::VEC, r[i][rr]);
      if constexpr (TRANS) {
        ST* dst = sT + (dg * C::VEC) * C::TSTR + 4 * kg;
        if constexpr (sizeof(ST) == 2) {
#pragma unroll
          for (int e = 0; e < C::VEC; ++e) {
            const int w = e >> 1;
            const int sh = (e & 1) * 16;
            const uint32_t x0 = (r[i][0][w] >> sh) & 0xffffu, x1 = (r[i][1][w] >> sh) & 0xffffu;
            const uint32_t x2 = (r[i][2][w] >> sh) & 0xffffu, x3 = (r[i][3][w] >> sh) & 0xffffu;
            u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
            *reinterpret_cast<u32x2*>(dst + e * C::TSTR) = pk;
          }
        } else {
#pragma unroll
          for (int e = 0; e < C::VEC; ++e) {
            u32x4 pk = {r[i][0][e], r[i][1][e], r[i][2][e], r[i][3][e]};
            *reinterpret_cast<u32x4*>(dst + e * C::TSTR) = pk;
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// 1. dq, delta and the own-position state gradients
// ---------------------------------------------------------------------------
// Workgroup: 4 waves x 16 queries of one (b, h), query tile qt (heaviest
// first).  Key tiles as in the forward: anchors [0, n_end) then the window
// positions [jb0, last query].  K and V are staged row-major; the dq product
// reads K's transposed fragments from the same tile (bf16: transposing LDS
// reads; fp32: a transposed copy).
template <typename ST, int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const BwdParams p) {
  using C = BwdCfg<ST, HD>;
  __shared__ __attribute__((aligned(16))) ST sK[C::BN * C::RSTR];
  __shared__ __attribute__((aligned(16))) ST sV[C::BN * C::RSTR];
  __shared__ __attribute__((aligned(16))) ST sKt[C::TLDS];

  const int nq = (p.T + C::BN - 1) / C::BN;
  int bhi, xi;
  if (!xcd_group(p.B * p.H, nq, bhi, xi)) return;
  const int qt = nq - 1 - xi;
  const int h = bhi % p.H;
  const int b = bhi / p.H;
  const int T = p.T;
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t base = bh * T * HD;
  const ST* qp = reinterpret_cast<const ST*>(p.q) + base;
  const ST* hkp = reinterpret_cast<const ST*>(p.hk) + base;
  const ST* hvp = reinterpret_cast<const ST*>(p.hv) + base;
  const ST* op = reinterpret_cast<const ST*>(p.o) + base;
  const ST* dop = reinterpret_cast<const ST*>(p.dO) + base;

  const int tq0 = qt * C::BN;
  const int tw0 = tq0 + 16 * wave;
  const int tq = tw0 + col;
  const bool valid = tq < T;
  const int64_t row = (int64_t)min(tq, T - 1) * HD;

  // ---- the lane's query: fragments, own position, delta ------------------
  Frag<ST> qf[C::NS], dof[C::NS];
  float s_own = 0.f, dp_own = 0.f, delta = 0.f;
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    qf[s] = frag_ld8(qp + row + 32 * s + 8 * g);
    dof[s] = frag_ld8(dop + row + 32 * s + 8 * g);
    s_own += frag_dot(qf[s], frag_ld8(hkp + row + 32 * s + 8 * g));
    dp_own += frag_dot(dof[s], frag_ld8(hvp + row + 32 * s + 8 * g));
    delta += frag_dot(dof[s], frag_ld8(op + row + 32 * s + 8 * g));
  }
  s_own = xor16_32_sum(s_own);
  dp_own = xor16_32_sum(dp_own);
  delta = xor16_32_sum(delta);
  const float lse2 = p.lse[bh * T + min(tq, T - 1)] * kLog2e;
  const float p_own = __builtin_amdgcn_exp2f(s_own * p.scale_log2 - lse2);
  const float ds_own = p_own * (dp_own - delta);
  if (valid && g == 0) {
    p.delta[bh * T + tq] = delta;
    *reinterpret_cast<f32x2*>(p.own + 2 * (bh * T + tq)) = f32x2{p.scale * ds_own, p_own};
  }
  // dq^T accumulators start at the own term ds_own * hk_t (unscaled)
  f32x4 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = ds_own * ld4_f32(hkp + row + 16 * db + 4 * g);
  Frag<ST> qs[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) qs[s] = frag_scale(qf[s], p.scale_log2);

  // ---- key tiles ----------------------------------------------------------
  const int tlast = min(tq0 + C::BN - 1, T - 1);   // last query of the tile
  const int wlast = min(tw0 + 15, T - 1);          // last query of the wave
  const int n_end = max(0, tlast - W) / D;
  const int jb0 = max(0, tq0 - W);
  const int na_t = (n_end + C::BN - 1) / C::BN;
  const int nb_t = W > 0 ? (tlast - jb0 + C::BN) / C::BN : 0;
  const int n_items = na_t + nb_t;
  const int nlo = max(0, min(tq, T - 1) - W) / D;  // anchors visible to the lane's query
  const int w_end = tw0 < T ? max(0, wlast - W) / D : 0;
  const int w_full = tw0 < T ? max(0, tw0 - W) / D : 0;
  const int wj0 = max(0, tw0 - W);
  const ST* kcp = hkp;  // anchor a is the state at position a*D + D - 1
  const ST* vcp = hvp;
  auto item = [&](int i, int& key0, int& nvalid, bool& anchor) {
    anchor = i < na_t;
    if (anchor) {
      key0 = i * C::BN;
      nvalid = n_end - key0;
    } else {
      key0 = jb0 + (i - na_t) * C::BN;
      nvalid = tlast + 1 - key0;
    }
  };
  Stage4<ST, HD, !C::TR> pk;
  Stage4<ST, HD, false> pv;
  auto load = [&](int i) {
    int key0, nv;
    bool anchor;
    item(i, key0, nv, anchor);
    // one load path for both kinds (a branch between two would make the
    // compiler wait for the loads at the join)
    const int stride = anchor ? D : 1;
    const int first = anchor ? key0 * D + D - 1 : key0;
    pk.load([&](int r) { return kcp + ((int64_t)first + (int64_t)r * stride) * HD; }, nv);
    pv.load([&](int r) { return vcp + ((int64_t)first + (int64_t)r * stride) * HD; }, nv);
  };
  if (n_items > 0) load(0);
  for (int i = 0; i < n_items; ++i) {
    __syncthreads();
    pk.store(sK, sKt);
    pv.store(sV, nullptr);
    __syncthreads();
    if (i + 1 < n_items) load(i + 1);
    int key0, nv;
    bool anchor;
    item(i, key0, nv, anchor);
    bool part, need_mask;
    if (anchor) {
      part = key0 < w_end;
      need_mask = key0 + C::BN > w_full;
    } else {
      part = tw0 < T && key0 <= wlast && key0 + C::BN > wj0;
      need_mask = !((tw0 + 15 - W <= key0) && (key0 + C::BN <= tw0) && (tw0 + 15 < T));
    }
    if (!part) continue;
    f32x4 S[C::NMB], dP[C::NMB];
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) {
      S[mb] = f32x4{-lse2, -lse2, -lse2, -lse2};
      dP[mb] = f32x4{-delta, -delta, -delta, -delta};
    }
#pragma unroll
    for (int s = 0; s < C::NS; ++s)
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) {
        mma16(S[mb], frag_ld8(sK + (16 * mb + col) * C::RSTR + 32 * s + 8 * g), qs[s]);
        mma16(dP[mb], frag_ld8(sV + (16 * mb + col) * C::RSTR + 32 * s + 8 * g), dof[s]);
      }
    // visible keys of the lane's query: anchors a < nlo; window t-W..t-1
    const int lo = anchor ? 0 : tq - W;
    const int hi = anchor ? nlo - 1 : tq - 1;
    const int kb = key0 + 4 * g - lo;
    const uint32_t span = (uint32_t)(hi - lo);
    f32x4 dS[C::NMB];
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool vis = !need_mask || (valid && (uint32_t)(kb + 16 * mb + e) <= span && hi >= lo);
        const float pe = vis ? __builtin_amdgcn_exp2f(S[mb][e]) : 0.f;
        dS[mb][e] = pe * dP[mb][e];
      }
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      const Frag<ST> bfr = frag_from(dS[2 * kk], dS[2 * kk + 1], (ST*)nullptr);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        mma16(acc[db], frag_rows<ST, HD>(sK, sKt, kk, db, col, g), bfr);
    }
  }

  if (valid) {
    ST* dqp = reinterpret_cast<ST*>(p.dq) + base + (int64_t)tq * HD;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) st4(dqp + 16 * db + 4 * g, p.scale * acc[db]);
  }
}

// dq with the anchors resident (no head has a window and every head's
// anchors fit in LDS, bf16): a workgroup stages all of its head's anchors
// (rows aD+D-1 of hk and hv) once, then its NW waves take 16-query blocks
// r + nra*(wave + NW*j) independently -- no barrier after the staging.  Per
// block the arithmetic is that of bwd_dq_kernel over the anchor tiles.
template <typename ST, int HD, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void bwd_dq_resident_kernel(const BwdParams p) {
  using C = BwdCfg<ST, HD>;
  constexpr int NT = 64 * NW;
  static_assert(C::TR, "bf16 only: the dq product reads K^T with transposing LDS reads");
  __shared__ __attribute__((aligned(16))) ST sK[kResidentAnchors * C::RSTR];
  __shared__ __attribute__((aligned(16))) ST sV[kResidentAnchors * C::RSTR];

  const int nbh = p.B * p.H;
  const int bhi = blockIdx.x % nbh;  // the nra workgroups of a head are nbh apart
  const int r = blockIdx.x / nbh;
  const int h = bhi % p.H;
  const int T = p.T;
  const int D = p.ht.D[h];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t bh = bhi;
  const int64_t base = bh * T * HD;
  const ST* qp = reinterpret_cast<const ST*>(p.q) + base;
  const ST* hkp = reinterpret_cast<const ST*>(p.hk) + base;
  const ST* hvp = reinterpret_cast<const ST*>(p.hv) + base;
  const ST* op = reinterpret_cast<const ST*>(p.o) + base;
  const ST* dop = reinterpret_cast<const ST*>(p.dO) + base;

  // ---- stage anchors a < (T-1)/D, padded to whole tiles with row nan-1 ----
  const int nan = (T - 1) / D;
  if (nan > 0) {
    const int rows = (nan + C::BN - 1) / C::BN * C::BN;
    for (int idx = tid; idx < rows * C::CPR; idx += NT) {
      const int row = idx / C::CPR;
      const int c = idx - row * C::CPR;
      const int64_t src = ((int64_t)min(row, nan - 1) * D + D - 1) * HD + c * C::VEC;
      st_raw16(sK + row * C::RSTR + c * C::VEC, ld_raw16(hkp + src));
      st_raw16(sV + row * C::RSTR + c * C::VEC, ld_raw16(hvp + src));
    }
  }
  __syncthreads();  // the only barrier: the anchors are read-only from here on

  const int nblk = (T + 15) / 16;
  for (int bi = r + p.nra * wave; bi < nblk; bi += p.nra * NW) {
    const int tw0 = 16 * bi;
    const int tq = tw0 + col;
    const bool valid = tq < T;
    const int64_t row = (int64_t)min(tq, T - 1) * HD;

    // the lane's query: fragments, own position, delta
    Frag<ST> qf[C::NS], dof[C::NS];
    float s_own = 0.f, dp_own = 0.f, delta = 0.f;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      qf[s] = frag_ld8(qp + row + 32 * s + 8 * g);
      dof[s] = frag_ld8(dop + row + 32 * s + 8 * g);
      s_own += frag_dot(qf[s], frag_ld8(hkp + row + 32 * s + 8 * g));
      dp_own += frag_dot(dof[s], frag_ld8(hvp + row + 32 * s + 8 * g));
      delta += frag_dot(dof[s], frag_ld8(op + row + 32 * s + 8 * g));
    }
    s_own = xor16_32_sum(s_own);
    dp_own = xor16_32_sum(dp_own);
    delta = xor16_32_sum(delta);
    const float lse2 = p.lse[bh * T + min(tq, T - 1)] * kLog2e;
    const float p_own = __builtin_amdgcn_exp2f(s_own * p.scale_log2 - lse2);
    const float ds_own = p_own * (dp_own - delta);
    if (valid && g == 0) {
      p.delta[bh * T + tq] = delta;
      *reinterpret_cast<f32x2*>(p.own + 2 * (bh * T + tq)) = f32x2{p.scale * ds_own, p_own};
    }
    f32x4 acc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] = ds_own * ld4_f32(hkp + row + 16 * db + 4 * g);
    Frag<ST> qs[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) qs[s] = frag_scale(qf[s], p.scale_log2);

    // anchors a < nlo are visible to the lane's query (no window)
    const int nlo = min(tq, T - 1) / D;
    const int w_end = min(tw0 + 15, T - 1) / D;  // anchors any query of the block sees
    const int w_full = tw0 / D;                  // anchors every query of the block sees
    for (int key0 = 0; key0 < w_end; key0 += C::BN) {
      const bool need_mask = key0 + C::BN > w_full;
      const ST* tk = sK + key0 * C::RSTR;
      const ST* tv = sV + key0 * C::RSTR;
      f32x4 S[C::NMB], dP[C::NMB];
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) {
        S[mb] = f32x4{-lse2, -lse2, -lse2, -lse2};
        dP[mb] = f32x4{-delta, -delta, -delta, -delta};
      }
#pragma unroll
      for (int s = 0; s < C::NS; ++s)
#pragma unroll
        for (int mb = 0; mb < C::NMB; ++mb) {
          mma16(S[mb], frag_ld8(tk + (16 * mb + col) * C::RSTR + 32 * s + 8 * g), qs[s]);
          mma16(dP[mb], frag_ld8(tv + (16 * mb + col) * C::RSTR + 32 * s + 8 * g), dof[s]);
        }
      f32x4 dS[C::NMB];
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = !need_mask || (valid && key0 + 16 * mb + 4 * g + e < nlo);
          const float pe = vis ? __builtin_amdgcn_exp2f(S[mb][e]) : 0.f;
          dS[mb][e] = pe * dP[mb][e];
        }
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) {
        const Frag<ST> bfr = frag_from(dS[2 * kk], dS[2 * kk + 1], (ST*)nullptr);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          mma16(acc[db], frag_rows<ST, HD>(tk, nullptr, kk, db, col, g), bfr);
      }
    }
    if (valid) {
      ST* dqp = reinterpret_cast<ST*>(p.dq) + base + (int64_t)tq * HD;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) st4(dqp + 16 * db + 4 * g, p.scale * acc[db]);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. state gradients from the keys' side
// ---------------------------------------------------------------------------
// Workgroup: one tile of 64 keys of one (b, h), 16 per wave (the wave's keys
// are the B operand, held in registers).  Tile x < na_t: anchors
// [64x, 64x+64), seen by queries t >= (a+1)D + W; next nb_t tiles: window
// positions [64y, 64y+64), seen by queries j+1 .. j+W.  Per query tile of 64:
// Q and dO staged row-major (their transposed fragments read from the same
// tiles, as in the dq kernel), lse and delta beside them.
template <typename ST, int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_kernel(const BwdParams p) {
  using C = BwdCfg<ST, HD>;
  __shared__ __attribute__((aligned(16))) ST sQ[C::BN * C::RSTR];
  __shared__ __attribute__((aligned(16))) ST sO[C::BN * C::RSTR];
  __shared__ __attribute__((aligned(16))) ST sQt[C::TLDS];
  __shared__ __attribute__((aligned(16))) ST sOt[C::TLDS];
  __shared__ __attribute__((aligned(16))) float sL[C::BN];
  __shared__ __attribute__((aligned(16))) float sDl[C::BN];

  int bhi, x;
  if (!xcd_group(p.B * p.H, p.nkt, bhi, x)) return;
  const int h = bhi % p.H;
  const int b = bhi / p.H;
  const int T = p.T;
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  const int na = T / D;                              // anchors of the head
  const int na_t = (na + C::BN - 1) / C::BN;
  const int nb_t = W > 0 ? (T + C::BN - 1) / C::BN : 0;
  if (x >= na_t * p.nsplit + nb_t) return;
  const bool anchor = x < na_t * p.nsplit;
  const int split = anchor ? x % p.nsplit : 0;
  const int key0 = anchor ? (x / p.nsplit) * C::BN : (x - na_t * p.nsplit) * C::BN;
  const int nkeys = anchor ? na : T;                 // valid key indices < nkeys

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t base = bh * T * HD;
  const ST* qp = reinterpret_cast<const ST*>(p.q) + base;
  const ST* hkp = reinterpret_cast<const ST*>(p.hk) + base;
  const ST* hvp = reinterpret_cast<const ST*>(p.hv) + base;
  const ST* dop = reinterpret_cast<const ST*>(p.dO) + base;
  const float* lsep = p.lse + bh * T;
  const float* dlp = p.delta + bh * T;

  // the lane's key (B-operand column): index key and its state row
  const int key = key0 + 16 * wave + col;
  const int keyc = min(key, nkeys - 1);
  const int kpos = anchor ? keyc * D + D - 1 : keyc;  // position of its state
  Frag<ST> kf[C::NS], vf[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    kf[s] = frag_scale(frag_ld8(hkp + (int64_t)kpos * HD + 32 * s + 8 * g), p.scale_log2);
    vf[s] = frag_ld8(hvp + (int64_t)kpos * HD + 32 * s + 8 * g);
  }
  f32x4 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[db] = dk[db];
  }

  // queries that see the tile: anchors from (key0+1)D + W on; window
  // positions from key0+1 to the tile's last key + W
  int t_lo, t_hi;
  if (anchor) {
    t_lo = (int)min<int64_t>((int64_t)(key0 + 1) * D + W, T);
    t_hi = T - 1;
  } else {
    t_lo = key0 + 1;
    t_hi = (int)min<int64_t>(T - 1, (int64_t)min(key0 + C::BN, nkeys) - 1 + W);
  }
  int qt0 = t_lo / C::BN;
  int qt1 = t_lo <= t_hi ? t_hi / C::BN : qt0 - 1;
  if (anchor && p.nsplit > 1) {  // this workgroup's share of the query tiles
    const int len = (qt1 - qt0 + p.nsplit) / p.nsplit;
    const int a0 = qt0 + split * len;
    qt1 = min(qt1, a0 + len - 1);
    qt0 = a0;
  }

  // queries that see the lane's key: an interval [vlo, vhi] (anchor: from
  // (key+1)D + W on; window: key+1 .. key+W; both below T), tested per
  // element with one unsigned compare (no per-element branch); an empty
  // interval (a key past the last valid one, or one no query sees) is moved
  // to 2^30, which no query position reaches
  int vlo = anchor ? (int)min<int64_t>((int64_t)(key + 1) * D + W, T) : key + 1;
  int vhi = anchor ? T - 1 : min(T - 1, key + W);
  if (key >= nkeys || vhi < vlo) vlo = vhi = 0x40000000;
  const uint32_t vspan = (uint32_t)(vhi - vlo);

  Stage4<ST, HD, !C::TR> pq, po;
  float lpre = 0.f, dpre = 0.f;
  auto load = [&](int qt) {
    const int tq0 = qt * C::BN;
    const int nv = min(C::BN, T - tq0);
    pq.load([&](int r) { return qp + (int64_t)(tq0 + r) * HD; }, nv);
    po.load([&](int r) { return dop + (int64_t)(tq0 + r) * HD; }, nv);
    if (tid < C::BN) {
      const int t = min(tq0 + tid, T - 1);
      lpre = lsep[t] * kLog2e;
      dpre = dlp[t];
    }
  };
  if (qt0 <= qt1) load(qt0);
  for (int qt = qt0; qt <= qt1; ++qt) {
    __syncthreads();
    pq.store(sQ, sQt);
    po.store(sO, sOt);
    if (tid < C::BN) {
      sL[tid] = lpre;
      sDl[tid] = dpre;
    }
    __syncthreads();
    if (qt < qt1) load(qt + 1);
    const int tq0 = qt * C::BN;
    f32x4 S[C::NMB], dP[C::NMB];
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL + 16 * mb + 4 * g);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(sDl + 16 * mb + 4 * g);
      S[mb] = -l4;
      dP[mb] = -d4;
    }
#pragma unroll
    for (int s = 0; s < C::NS; ++s)
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) {
        mma16(S[mb], frag_ld8(sQ + (16 * mb + col) * C::RSTR + 32 * s + 8 * g), kf[s]);
        mma16(dP[mb], frag_ld8(sO + (16 * mb + col) * C::RSTR + 32 * s + 8 * g), vf[s]);
      }
    // element (query t = tq0 + 16mb + 4g + e, the lane's key)
    f32x4 P[C::NMB], dS[C::NMB];
    const int tb = tq0 + 4 * g - vlo;  // query t = tq0 + 16mb + 4g + e, relative to vlo
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool vis = (uint32_t)(tb + 16 * mb + e) <= vspan;
        const float ex = __builtin_amdgcn_exp2f(S[mb][e]);
        const float pe = vis ? ex : 0.f;
        P[mb][e] = pe;
        dS[mb][e] = pe * dP[mb][e];
      }
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      const Frag<ST> bp = frag_from(P[2 * kk], P[2 * kk + 1], (ST*)nullptr);
      const Frag<ST> bs = frag_from(dS[2 * kk], dS[2 * kk + 1], (ST*)nullptr);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        mma16(dv[db], frag_rows<ST, HD>(sO, sOt, kk, db, col, g), bp);
        mma16(dk[db], frag_rows<ST, HD>(sQ, sQt, kk, db, col, g), bs);
      }
    }
  }

  if (key < nkeys) {
    // anchors: this split's partial sums; window: the position's gradient
    float* dkp = anchor ? p.dKc + split * p.kc_split + ((int64_t)b * p.R + p.ht.aoff[h] + key) * HD
                        : p.dhk + base + (int64_t)key * HD;
    float* dvp = anchor ? p.dVc + split * p.kc_split + ((int64_t)b * p.R + p.ht.aoff[h] + key) * HD
                        : p.dhv + base + (int64_t)key * HD;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      *reinterpret_cast<f32x4*>(dkp + 16 * db + 4 * g) = p.scale * dk[db];
      *reinterpret_cast<f32x4*>(dvp + 16 * db + 4 * g) = dv[db];
    }
  }
}

// ---------------------------------------------------------------------------
// 3. the recurrence in reverse: one persistent kernel over chunks, linked by
//    the chunk-aggregate tree of the forward scan (csrc/scan_tree.h)
// ---------------------------------------------------------------------------
// Partial anchor gradients summed into split 0 (splits in a fixed order, so
// the result is deterministic); the reverse scan then reads one buffer.
__global__ __launch_bounds__(256) void bwd_anchor_sum_kernel(float* dKc, float* dVc, int64_t n4,
                                                             int nsplit) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4* k = reinterpret_cast<f32x4*>(dKc);
  f32x4* v = reinterpret_cast<f32x4*>(dVc);
  f32x4 sk = k[i], sv = v[i];
  for (int s = 1; s < nsplit; ++s) {
    sk += k[i + s * n4];
    sv += v[i + s * n4];
  }
  k[i] = sk;
  v[i] = sv;
}

// lambda_t = dh_t + a_t lambda_{t+1} with a_t = g_{t+1} (0 at t = T-1) is a
// chain of affine maps, composed like the forward's h_t = g_t h_{t-1} +
// (1-g_t) x_t but from the end of the sequence: ticket i is the i-th chunk
// from the end (reversed chunk rc = i / nseq of sequence i % nseq), and the
// tree links the reversed chunks exactly as the forward links its chunks.
// Layout as in the forward: LPR lanes cover a row with 16-byte accesses, a
// lane holds S consecutive rows, RG row-groups make a chunk of RG*S rows.
//  * loads: g of rows tbase .. tbase+S (a_t and 1-g_t), q, dO and the two
//    own-position scalars (the own term), the window gradients (W > 0) and
//    the anchor gradients at anchor rows;
//  * pass 1 reduces the rows to the lane's map (last row first); the
//    row-groups are composed in LDS (from the last);
//  * waves 0..NH-1 publish the chunk's map and the parents it completes,
//    waves 2..2+NH-1 compose the carry: lambda after the chunk (0 after the
//    last one);
//  * then k, v and the stored states of rows tbase-1 .. tbase+S-2 are
//    loaded (issued before the tree round trip they would keep 64 more
//    registers live across it and spill: the backward of the 1.5B-like
//    prefill took 8% longer), and pass 2 recomputes
//    dh_t from the kept q, dO and scalars (the window and anchor gradients
//    again, from L2), runs the rows from the carry, last row first, and
//    writes
//    dk = (1-g) lambda_k, dv = (1-g) lambda_v and
//    dg = lambda_k (h^k_{t-1} - k_t) + lambda_v (h^v_{t-1} - v_t).
// Every input row is read once (the window and anchor gradients twice, the
// second time normally from L2).
template <typename ST, int HD, int S>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_rscan_kernel(const BwdParams p) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;  // lanes per row
  constexpr int RG = 256 / LPR;  // row-groups per chunk
  constexpr int LC = RG * S;     // rows per chunk
  constexpr int NH = HD / 64;    // channel halves of the tree waves
  static_assert(HD % 64 == 0 && LPR <= 64, "layout");
  __shared__ float s_A[RG][HD];
  __shared__ float s_Bk[RG][HD];
  __shared__ float s_Bv[RG][HD];
  __shared__ float s_lk[HD];
  __shared__ float s_lv[HD];
  __shared__ uint32_t s_epoch;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  if (tid == 0) s_epoch = ld_acquire_u32(p.rhdr + kEpochWord);
  __syncthreads();
  const uint32_t epoch = s_epoch;
  const uint32_t tag = tree_tag(epoch);
  const int T = p.T;
  const int nseq = p.B * p.H;
  const uint32_t n = (uint32_t)nseq * (uint32_t)p.nchunk;
  const int r = tid / LPR;
  const int c0 = (tid - r * LPR) * VEC;

  for (uint32_t ticket = blockIdx.x; ticket < n; ticket += gridDim.x) {
    const int rc = (int)(ticket / (uint32_t)nseq);
    const int seq = (int)(ticket - (uint32_t)rc * (uint32_t)nseq);
    const int chunk = p.nchunk - 1 - rc;
    const int b = seq / p.H;
    const int h = seq - b * p.H;
    const int D = p.ht.D[h];
    const int W = p.ht.W[h];
    const int64_t bh = (int64_t)seq;
    const int64_t off = bh * T * HD + c0;
    const int tbase = chunk * LC + r * S;
    const int64_t arow0 = (int64_t)b * p.R + p.ht.aoff[h];

    // ---- loads (unconditional, rows clamped to the sequence) ---------------
    u32x4 gr[S + 1], qr[S], orow[S];
    f32x2 own[S];
#pragma unroll
    for (int s = 0; s <= S; ++s)
      gr[s] = ld_raw16(reinterpret_cast<const ST*>(p.g) + off + (int64_t)min(tbase + s, T - 1) * HD);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = min(tbase + s, T - 1);
      qr[s] = ld_raw16(reinterpret_cast<const ST*>(p.q) + off + (int64_t)t * HD);
      orow[s] = ld_raw16(reinterpret_cast<const ST*>(p.dO) + off + (int64_t)t * HD);
      own[s] = *reinterpret_cast<const f32x2*>(p.own + 2 * (bh * T + t));
    }
    // dh of row s (t = tbase + s): the own term from the kept q, dO and
    // scalars, plus the window and anchor gradients (read where they exist;
    // pass 2 reads them again, from L2)
    auto dh_row = [&](int s, float (&dk)[VEC], float (&dv)[VEC]) {
      const int t = min(tbase + s, T - 1);
      float qv[VEC], ov[VEC];
      unpack16(qr[s], qv, (ST*)nullptr);
      unpack16(orow[s], ov, (ST*)nullptr);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        dk[e] = own[s][0] * qv[e];
        dv[e] = own[s][1] * ov[e];
      }
      if (W > 0) {
        const int64_t i = off + (int64_t)t * HD;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(p.dhk + i + e);
          const f32x4 y = *reinterpret_cast<const f32x4*>(p.dhv + i + e);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dk[e + j] += x[j];
            dv[e + j] += y[j];
          }
        }
      }
      if (t % D == D - 1) {
        const int64_t i = (arow0 + t / D) * HD + c0;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(p.dKc + i + e);
          const f32x4 y = *reinterpret_cast<const f32x4*>(p.dVc + i + e);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dk[e + j] += x[j];
            dv[e + j] += y[j];
          }
        }
      }
    };
    // ---- pass 1: the lane's map (last row first) -----------------------------
    {
      float A[VEC], Bk[VEC], Bv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        A[e] = 1.f;
        Bk[e] = 0.f;
        Bv[e] = 0.f;
      }
#pragma unroll
      for (int s = S - 1; s >= 0; --s) {
        const int t = tbase + s;
        if (t < T) {
          float an[VEC], dk[VEC], dv[VEC];
          unpack16(gr[s + 1], an, (ST*)nullptr);
          dh_row(s, dk, dv);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float a = t + 1 < T ? an[e] : 0.f;
            A[e] *= a;
            Bk[e] = a * Bk[e] + dk[e];
            Bv[e] = a * Bv[e] + dv[e];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        s_A[r][c0 + e] = A[e];
        s_Bk[r][c0 + e] = Bk[e];
        s_Bv[r][c0 + e] = Bv[e];
      }
    }
    __syncthreads();

    // ---- the row-groups (from the last), the tree, the carry ----------------
    if (wave < NH) {
      const int half = wave;
      const int c = 64 * half + lane;
      float ra = 1.f, rbk = 0.f, rbv = 0.f;
      for (int rr = RG - 1; rr >= 0; --rr) {
        const float a = s_A[rr][c], bk = s_Bk[rr][c], bv = s_Bv[rr][c];
        s_A[rr][c] = ra;  // map of the row-groups after rr
        s_Bk[rr][c] = rbk;
        s_Bv[rr][c] = rbv;
        rbk = a * rbk + bk;
        rbv = a * rbv + bv;
        ra = ra * a;
      }
      tree_publish<HD>(p.ragg, p.rhdr, p.rnlevels, p.rlbase, p.rnodes, seq, rc, half, ra, rbk,
                       rbv, tag, lane);
    } else if (wave >= 2 && wave < 2 + NH) {
      const int half = wave - 2;
      float one = 1.f, lk = 0.f, lv = 0.f;  // lambda after the last position is 0
      tree_carry<HD>(p.ragg, p.rhdr, p.rnlevels, p.rlbase, p.rnodes, seq, rc, half, one, lk, lv,
                     tag, lane);
      s_lk[64 * half + lane] = lk;
      s_lv[64 * half + lane] = lv;
    }
    __syncthreads();
    // pass-2 rows: k, v of the lane's rows, the stored states of the rows
    // before them (after the carry)
    u32x4 kr[S], vr[S], pk[S], pv[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t rt = (int64_t)min(tbase + s, T - 1) * HD;
      const int64_t rp = (int64_t)max(min(tbase + s, T - 1) - 1, 0) * HD;
      kr[s] = ld_raw16(reinterpret_cast<const ST*>(p.k) + off + rt);
      vr[s] = ld_raw16(reinterpret_cast<const ST*>(p.v) + off + rt);
      pk[s] = ld_raw16(reinterpret_cast<const ST*>(p.hk) + off + rp);
      pv[s] = ld_raw16(reinterpret_cast<const ST*>(p.hv) + off + rp);
    }

    // ---- pass 2: the rows from the carry, last row first --------------------
    {
      float lk[VEC], lv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int c = c0 + e;
        lk[e] = s_A[r][c] * s_lk[c] + s_Bk[r][c];
        lv[e] = s_A[r][c] * s_lv[c] + s_Bv[r][c];
      }
      ST* dkp = reinterpret_cast<ST*>(p.dk) + off;
      ST* dvp = reinterpret_cast<ST*>(p.dv) + off;
      ST* dgp = reinterpret_cast<ST*>(p.dg) + off;
#pragma unroll
      for (int s = S - 1; s >= 0; --s) {
        const int t = tbase + s;
        if (t < T) {
          float an[VEC], gt[VEC], kv[VEC], vv[VEC], hkp[VEC], hvp[VEC], dk[VEC], dv[VEC];
          dh_row(s, dk, dv);
          unpack16(gr[s + 1], an, (ST*)nullptr);
          unpack16(gr[s], gt, (ST*)nullptr);
          unpack16(kr[s], kv, (ST*)nullptr);
          unpack16(vr[s], vv, (ST*)nullptr);
          unpack16(pk[s], hkp, (ST*)nullptr);
          unpack16(pv[s], hvp, (ST*)nullptr);
          float ok[VEC], ov[VEC], og[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float a = t + 1 < T ? an[e] : 0.f;
            lk[e] = dk[e] + a * lk[e];
            lv[e] = dv[e] + a * lv[e];
            const float hk_prev = t > 0 ? hkp[e] : 0.f;
            const float hv_prev = t > 0 ? hvp[e] : 0.f;
            ok[e] = (1.f - gt[e]) * lk[e];
            ov[e] = (1.f - gt[e]) * lv[e];
            og[e] = lk[e] * (hk_prev - kv[e]) + lv[e] * (hv_prev - vv[e]);
          }
          const int64_t rt = (int64_t)t * HD;
          st_raw16(dkp + rt, pack16(ok, (ST*)nullptr));
          st_raw16(dvp + rt, pack16(ov, (ST*)nullptr));
          st_raw16(dgp + rt, pack16(og, (ST*)nullptr));
        }
      }
    }
    __syncthreads();  // LDS is reused by the next chunk
  }

  // retire: the last workgroup advances the epoch
  if (tid == 0) tree_retire(p.rhdr, epoch);
}

template <typename ST, int HD>
int launch_t(const BwdParams& p, hipStream_t st) {
  const int nq = (p.T + 63) / 64;
  const int ngrp = (p.B * p.H + kXcds - 1) / kXcds * kXcds;  // (b, h) groups, padded
  if constexpr (sizeof(ST) == 2) {
    if (p.nra > 0)
      hipLaunchKernelGGL((bwd_dq_resident_kernel<ST, HD, kBwdResidentWaves>),
                         dim3(p.B * p.H * p.nra), dim3(64 * kBwdResidentWaves), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<ST, HD>), dim3(ngrp * nq), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<ST, HD>), dim3(ngrp * nq), dim3(256), 0, st, p);
  }
  if (p.nkt > 0)
    hipLaunchKernelGGL((bwd_dkv_kernel<ST, HD>), dim3(ngrp * p.nkt), dim3(256), 0, st, p);
  if (p.nsplit > 1 && p.kc_split > 0) {
    const int64_t n4 = p.kc_split / 4;
    hipLaunchKernelGGL(bwd_anchor_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                       p.dKc, p.dVc, n4, p.nsplit);
  }
  // the reverse scan: persistent, at most as many workgroups as the device
  // holds at once (every wait is on a smaller ticket of a resident one)
  const void* kern = reinterpret_cast<const void*>(&bwd_rscan_kernel<ST, HD, kScanRowsPerThread>);
  const int lim = coop_grid_limit(kern, 256);
  if (lim <= 0) return (int)hipErrorInvalidValue;
  const int64_t nticket = (int64_t)p.B * p.H * p.nchunk;
  const unsigned grid = (unsigned)std::min<int64_t>(nticket, lim);
  hipLaunchKernelGGL((bwd_rscan_kernel<ST, HD, kScanRowsPerThread>), dim3(grid), dim3(256), 0, st,
                     p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_backward(int dtype, int hd, const BwdParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) return hd == 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
  return hd == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace rat
