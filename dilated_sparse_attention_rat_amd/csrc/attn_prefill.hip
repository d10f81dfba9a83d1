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
//    a head cost about the same (single tiles, heaviest first, when pairs
//    would leave too few workgroups, or when every head's window outweighs
//    its anchors so that tile costs hardly grow along the sequence); heads are ordered by per-workgroup
//    cost (heaviest first) so a head-wise hybrid launch is longest-job-first;
//  * K/V tiles of 64 keys are staged in LDS once per workgroup, both
//    row-major for bf16: K fragments are plain ds_read_b128 and the V^T
//    fragments of the PV product come out of ds_read_b64_tr_b16, the gfx950
//    transposing read, so staging is a plain copy (fp32 stages V transposed,
//    keys contiguous); the global loads of tile i+1 are issued into
//    registers before tile i's MFMAs, so their latency is hidden (for
//    windowless heads, bf16, hd 128, two blocks per wave, the tiles go
//    straight into two LDS stages with global_load_lds_dwordx4 instead, with
//    one barrier per tile);
//  * scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16),
//    so each lane owns one query column: the row max needs two cross-lane
//    steps, and P^T is already the B operand of O^T += V^T P^T (keys
//    permuted identically on both operands); the row sums come out of the
//    same product through one all-ones V^T block (an MFMA per key slab
//    instead of a VALU add per score);
//  * the staircase mask of the anchors (a < floor(max(0,t-W)/D)) and the band
//    mask of the window are applied only on the tiles that need them;
//  * the own position is a per-query dot product folded into the initial
//    softmax state (with no window this saves a 1-of-64 MFMA band tile; with
//    a window the band mask covers t-W .. t-1);
//  * online softmax in the log2 domain: Q is pre-scaled by scale*log2(e) and
//    the score accumulators start at -m, so the MFMA output is directly the
//    exp2 argument (no per-score multiply-add); fp32 accumulation, bf16 P.
#include "rat_device.h"

namespace rat {

namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 units

// c0 + a*b into a fresh accumulator (c0 is left as it is)
__device__ __forceinline__ f32x4 mma16_from(const f32x4& c0, const Frag<bf16>& a, const Frag<bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16_from(const f32x4& c0, const Frag<float>& a, const Frag<float>& b) {
  f32x4 c = c0;
  mma16(c, a, b);
  return c;
}

__device__ __forceinline__ Frag<bf16> frag_ones(bf16*) {
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  return f;
}
__device__ __forceinline__ Frag<float> frag_ones(float*) {
  return Frag<float>{f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f}};
}


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
  // row-major V tile (bf16): the transposing reads of a 16-lane group cover
  // 4 rows x 32 bytes; rows 72 dwords apart put the 8 rows read by each half
  // wave on disjoint banks
  static constexpr int VRSTR = HD + 32 / (int)sizeof(ST);
  static constexpr int VEC = StTraits<ST>::VEC;
  static constexpr int CPR = HD / VEC;   // 16-byte chunks per row
  // bf16: V is staged row-major like K and its transposed MFMA fragments are
  // read with ds_read_b64_tr_b16; fp32: V is staged transposed (keys
  // contiguous)
  static constexpr bool VROW = sizeof(ST) == 2;
  static constexpr int KITEMS = BN * CPR;          // K chunks per tile
  static constexpr int VTITEMS = (BN / 4) * CPR;  // transposed staging: 4 rows x VEC items
  static constexpr int VITEMS = VROW ? KITEMS : VTITEMS;  // V items of the streamed tile
  static constexpr int KPT = (KITEMS + 255) / 256;  // per thread
  static constexpr int VPT = (VITEMS + 255) / 256;
  static constexpr int VROWS = VROW ? 1 : 4;       // rows per V item
  static constexpr int VLDS = VROW ? BN * VRSTR : HD * VSTR;  // V tile elements in LDS
};

// One K/V tile held in registers between its global load and its LDS store
// (the load of tile i+1 is in flight while tile i is being computed).  V work
// items run key-group fastest so that the transposed LDS stores of
// consecutive lanes land in consecutive 8-byte slots (no bank conflicts).
template <typename ST, int HD, int QB>
struct Prefetch {
  using C = AttnCfg<ST, HD, QB>;
  u32x4 k[C::KPT];
  u32x4 v[C::VPT][C::VROWS];

  // Rows [0, BN) of the tile (nvalid >= 1); rows.k(r) / rows.v(r) give the
  // K and V row pointers of tile row r.  Rows at or beyond nvalid re-read row
  // nvalid-1: such keys are always masked (weight exactly 0) and the
  // duplicated V row is finite, so they contribute nothing, and the loads
  // need no branches.
  template <typename Rows>
  __device__ __forceinline__ void load(const Rows& rows, int nvalid) {
    const int tid = threadIdx.x;
    const int last = nvalid - 1;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int idx = min(tid + 256 * i, C::KITEMS - 1);
      const int row = idx / C::CPR;
      const int c16 = idx - row * C::CPR;
      k[i] = ld_raw16(rows.k(min(row, last)) + c16 * C::VEC);
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int idx = min(tid + 256 * i, C::VITEMS - 1);
      if constexpr (C::VROW) {
        const int row = idx / C::CPR;
        const int c16 = idx - row * C::CPR;
        v[i][0] = ld_raw16(rows.v(min(row, last)) + c16 * C::VEC);
      } else {
        const int dg = idx / (C::BN / 4);
        const int kg = idx - dg * (C::BN / 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          v[i][rr] = ld_raw16(rows.v(min(4 * kg + rr, last)) + dg * C::VEC);
      }
    }
  }

  // Linear rows (row r of K at kh + r*HD, of V at vh + r*HD), bf16: buffer
  // loads with 32-bit offsets shared by K and V, one address per chunk.
  __device__ __forceinline__ void load_linear(const ST* kh, const ST* vh, int nvalid) {
    static_assert(C::VROW && C::VPT == C::KPT, "row-major V");
    const auto kr = buffer_region(kh);
    const auto vr = buffer_region(vh);
    const int tid = threadIdx.x;
    const int last = nvalid - 1;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int idx = min(tid + 256 * i, C::KITEMS - 1);
      const int row = idx / C::CPR;
      const int c16 = idx - row * C::CPR;
      const uint32_t off = (uint32_t)((min(row, last) * HD + c16 * C::VEC) * (int)sizeof(ST));
      k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
      v[i][0] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
    }
  }

  // K row-major; V row-major (bf16) or transposed (fp32, keys contiguous)
  __device__ __forceinline__ void store(ST* sK, ST* sV) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / C::CPR;
      const int c16 = idx - row * C::CPR;
      if (C::KITEMS % 256 == 0 || idx < C::KITEMS) st_raw16(sK + row * C::KSTR + c16 * C::VEC, k[i]);
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int idx = tid + 256 * i;
      if (C::VITEMS % 256 != 0 && idx >= C::VITEMS) continue;
      if constexpr (C::VROW) {
        const int row = idx / C::CPR;
        const int c16 = idx - row * C::CPR;
        st_raw16(sV + row * C::VRSTR + c16 * C::VEC, v[i][0]);
      } else {
        const int dg = idx / (C::BN / 4);
        const int kg = idx - dg * (C::BN / 4);
        ST* dst = sV + (dg * C::VEC) * C::VSTR + 4 * kg;
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
  float m[QB];             // running max (log2 domain)
  f32x4 l[QB];             // running sum, in every element and every lane (an
                           // all-ones V^T block through the PV MFMA)
  int tq[QB];              // query positions
  int nlo[QB];             // anchors visible to each query
};

// Raw per-lane query inputs of a wave's 16*QB queries: q fragments, the own
// key fragments and the own value row slice (4 elements per 16-row d-block).
template <typename ST>
struct Raw4;
template <>
struct Raw4<bf16> {
  u32x2 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ f32x4 f32() const {
    return f32x4{bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1])};
  }
};
template <>
struct Raw4<float> {
  f32x4 u;
  __device__ __forceinline__ void load(const float* p) { u = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ f32x4 f32() const { return u; }
};

template <typename ST, int HD, int QB>
struct QueryIn {
  using C = AttnCfg<ST, HD, QB>;
  Frag<ST> q[QB][C::NS];
  Frag<ST> k[QB][C::NS];
  Raw4<ST> v[QB][C::NDB];

  // rows of the wave's queries tw0 + 16*nb + (lane % 16), clamped to T-1
  // (q rows q_st elements apart, state rows HD apart)
  __device__ __forceinline__ void load(const ST* qp, const ST* hkp, const ST* hvp, int tw0, int T,
                                       int64_t q_st) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int g = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      const int tr = min(tw0 + 16 * nb + col, T - 1);
      const int64_t row = (int64_t)tr * HD;
      const int64_t qrow = (int64_t)tr * q_st;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        q[nb][s] = frag_ld8(qp + qrow + 32 * s + 8 * g);
        k[nb][s] = frag_ld8(hkp + row + 32 * s + 8 * g);
      }
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) v[nb][db].load(hvp + row + 16 * db + 4 * g);
    }
  }
};

// One staged tile against one wave's 16*QB queries, in three phases:
// scores (MFMA), softmax (VALU), PV (MFMA).  VR: V tile row-major (row
// stride VS), else transposed (keys contiguous, row stride VS).
//  kind 0: anchors, key index = anchor index a, visible iff a < nlo(t)
//  kind 1: band,    key index = position j,     visible iff t-W <= j <= t
template <typename ST, int HD, int QB>
struct TileRegs {
  using C = AttnCfg<ST, HD, QB>;
  f32x4 S[C::NMB][QB];     // scores S^T, then exp2 arguments
  Frag<ST> P[C::NKK][QB];  // P^T as the B operand of the PV product
};

// S = c*K Q^T - m.  With Q pre-scaled by c = scale*log2(e) the MFMA result
// is directly the exp2 argument of the running softmax (the first slab's
// MFMAs read one {-m} tuple per query block as their C operand).
// SW: the tile is unpadded (rows HD elements apart) with K row r holding its
// 16-byte chunk c at c ^ (r % 16) and V row r at c ^ 2 (r % 8), the layout
// the direct-to-LDS staging writes (else K rows KSTR and V rows VRSTR apart).
// SCHED >= 0: the compiler's instruction-group scheduling strategy of that
// number for the block (LDS reads interleaved with the MFMAs it feeds);
// measured per kernel, none where it does not pay.
template <typename ST, int HD, int QB, bool SW = false, int SCHED = -1>
__device__ __forceinline__ void tile_scores(const WaveState<ST, HD, QB>& ws, const ST* sK,
                                            TileRegs<ST, HD, QB>& tr) {
  using C = AttnCfg<ST, HD, QB>;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  if constexpr (SCHED >= 0) __builtin_amdgcn_iglp_opt(SCHED);
  f32x4 minit[QB];
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    const float mneg = -ws.m[nb];
    minit[nb] = f32x4{mneg, mneg, mneg, mneg};
  }
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) {
      // 16 lanes read 16 rows at one chunk: distinct banks in either layout
      const Frag<ST> a = SW ? frag_ld8(sK + (16 * mb + col) * HD + 8 * ((4 * s + g) ^ col))
                            : frag_ld8(sK + (16 * mb + col) * C::KSTR + 32 * s + 8 * g);
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) {
        if (s == 0)
          tr.S[mb][nb] = mma16_from(minit[nb], a, ws.qf[nb][s]);
        else
          mma16(tr.S[mb][nb], a, ws.qf[nb][s]);
      }
    }
  }
}

// Online softmax in the log2 domain.  The running max m is raised only when
// a tile's max exceeds it by more than kRescaleSlack: every weight is then
// exp2(c*s - m) <= 2^kRescaleSlack (no overflow in fp32 or bf16), the result
// is the same softmax, and the accumulators are rescaled on few tiles
// (wave-uniform skip otherwise).  One basic block per phase for all query
// blocks (masks, maxima, the rare rescale, the exponentials), so the
// exponentials of one block can be scheduled among MFMAs.
template <typename ST, int HD, int QB>
__device__ __forceinline__ void tile_softmax(WaveState<ST, HD, QB>& ws, TileRegs<ST, HD, QB>& tr,
                                             int key0, int kind, bool need_mask, int W) {
  using C = AttnCfg<ST, HD, QB>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  if (need_mask) {
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      // visible keys of this lane's query: lo <= key <= hi
      //   anchors: a < nlo(t);  band: t - W <= j <= t - 1 (own position folded)
      const int lo = kind == 0 ? 0 : ws.tq[nb] - W;
      const int hi = kind == 0 ? ws.nlo[nb] - 1 : ws.tq[nb] - 1;
      const int base = key0 + 4 * g - lo;
      const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = (uint32_t)(base + 16 * mb + i) <= span && hi >= lo;
          tr.S[mb][nb][i] = vis ? tr.S[mb][nb][i] : -INFINITY;
        }
    }
  }
  float tmax[QB];
  bool grow_any = false;
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    float t = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) t = fmaxf(t, tr.S[mb][nb][i]);
    tmax[nb] = xor16_32_max(t);
    grow_any = grow_any || tmax[nb] > kRescaleSlack;
  }
  if (__any(grow_any)) {
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      const float delta = tmax[nb] > kRescaleSlack ? tmax[nb] : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      ws.m[nb] += delta;
      ws.l[nb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) ws.acc[nb][db] *= alpha;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) tr.S[mb][nb] -= delta;
    }
  }
#pragma unroll
  for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < QB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tr.S[mb][nb][i] = __builtin_amdgcn_exp2f(tr.S[mb][nb][i]);
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
    for (int nb = 0; nb < QB; ++nb)
      tr.P[kk][nb] = frag_from(tr.S[2 * kk][nb], tr.S[2 * kk + 1][nb], (ST*)nullptr);
}

// O^T += V^T P^T, and the row sums through one all-ones V^T block (sum_k
// P[k][query] in every element: the same bf16-rounded weights as the
// numerator).
template <typename ST, int HD, int QB, bool VR = AttnCfg<ST, HD, QB>::VROW,
          int VS = (VR ? AttnCfg<ST, HD, QB>::VRSTR : AttnCfg<ST, HD, QB>::VSTR), bool SW = false,
          int SCHED = -1>
__device__ __forceinline__ void tile_pv(WaveState<ST, HD, QB>& ws, const TileRegs<ST, HD, QB>& tr,
                                        const ST* sV) {
  using C = AttnCfg<ST, HD, QB>;
  static_assert(!VR || sizeof(ST) == 2, "transposing reads are 16-bit");
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  if constexpr (SCHED >= 0) __builtin_amdgcn_iglp_opt(SCHED);
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      Frag<ST> va;
      if constexpr (VR && SW) {
        // as below; the 8-byte piece of row r sits in chunk c ^ 2 (r % 8)
        // (rows r and r + 16 share the swizzle)
        const int r = 32 * kk + 4 * g + (col >> 2);
        const int c = 2 * db + ((col >> 1) & 1);
        va = frag_ld_tr(sV + r * HD + 8 * (c ^ (2 * (r & 7))) + 4 * (col & 1), 16 * HD);
      } else if constexpr (VR) {
        // keys 32kk + 4g + j (slots j < 4) and 32kk + 16 + 4g + j (slots
        // j >= 4) of channel 16db + col, transposed out of the row-major tile
        va = frag_ld_tr(sV + (32 * kk + 4 * g + (col >> 2)) * VS + 16 * db + 4 * (col & 3), 16 * VS);
      } else {
        const ST* vrow = sV + (16 * db + col) * VS + 32 * kk + 4 * g;
        va = frag_ld4x2(vrow, vrow + 16);
      }
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) mma16(ws.acc[nb][db], va, tr.P[kk][nb]);
    }
    const Frag<ST> ones = frag_ones((ST*)nullptr);
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) mma16(ws.l[nb], ones, tr.P[kk][nb]);
  }
}

template <typename ST, int HD, int QB, bool VR = AttnCfg<ST, HD, QB>::VROW,
          int VS = (VR ? AttnCfg<ST, HD, QB>::VRSTR : AttnCfg<ST, HD, QB>::VSTR), bool SW = false,
          int SCHED = -1>
__device__ __forceinline__ void tile_update(WaveState<ST, HD, QB>& ws, const ST* sK,
                                            const ST* sV, int key0, int kind, bool need_mask,
                                            int W) {
  TileRegs<ST, HD, QB> tr;
  tile_scores<ST, HD, QB, SW, SCHED>(ws, sK, tr);
  tile_softmax<ST, HD, QB>(ws, tr, key0, kind, need_mask, W);
  tile_pv<ST, HD, QB, VR, VS, SW, SCHED>(ws, tr, sV);
}

// Key rows of one staged tile.  Anchor tiles, and band tiles at positions
// >= t0, are linear: row r at kh + r*HD (n2 = 0).  A band tile that starts
// before t0 (a continuation's window reaching into the previous call) reads
// its first n2 = t0 - key0 rows (at most W) from the previous call's ring,
// slot = position mod W: row r < n2 at kr + r*HD, where kr points at the
// slot of key0, minus W rows once the slot wraps (r >= n1); rows r >= n2 at
// kh + r*HD (kh = this call's row 0 minus n2 rows).  The selection is
// branch-free on scalars, so every tile issues the same global loads.
template <typename ST, int HD>
struct RowMap {
  const ST* kh;
  const ST* vh;
  const ST* kr;
  const ST* vr;
  int n1, n2, W;
  __device__ __forceinline__ int64_t row(int r) const {
    return (int64_t)(r >= n1 && r < n2 ? r - W : r) * HD;
  }
  __device__ __forceinline__ const ST* k(int r) const { return (r < n2 ? kr : kh) + row(r); }
  __device__ __forceinline__ const ST* v(int r) const { return (r < n2 ? vr : vh) + row(r); }
};

// One query tile of 64*QB queries at local row lt0 (absolute position
// p.t0 + lt0).  `qin` holds this tile's query inputs (already loaded).
// Positions (queries, band keys, anchors) are absolute; rows of q, hk, hv,
// o and lse are local to this call.
// DMA (bf16, HD 128, QB 2, no ring): sK and sV hold two stages of BN x HD
// each, filled straight from global memory (global_load_lds_dwordx4) in the
// swizzled layout of tile_scores / tile_pv: the loads of key tile i+1 fly
// while tile i is computed, no staging registers, one barrier per tile.
template <typename ST, int HD, int QB, bool RING, bool DMA = false>
__device__ __forceinline__ void process_tile(const AttnParams& p, int b, int h, int lt0, ST* sK,
                                             ST* sV, const QueryIn<ST, HD, QB>& qin) {
  using C = AttnCfg<ST, HD, QB>;
  constexpr int QW = 16 * QB;  // queries per wave
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int T = p.T;
  const int a0 = p.t0;  // absolute position of local row 0
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  const int64_t bh = (int64_t)b * p.H + h;
  const ST* hkp = reinterpret_cast<const ST*>(p.hk) + bh * T * HD;
  const ST* hvp = reinterpret_cast<const ST*>(p.hv) + bh * T * HD;
  const ST* kcp = reinterpret_cast<const ST*>(p.Kc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
  const ST* vcp = reinterpret_cast<const ST*>(p.Vc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
  const int64_t rofs = ((int64_t)b * p.WS + p.ht.roff[h]) * HD;
  // previous call's ring (only read when t0 > 0 and W > 0, where it is set)
  const ST* rkp = reinterpret_cast<const ST*>(p.kr) + rofs;
  const ST* rvp = reinterpret_cast<const ST*>(p.vr) + rofs;

  const int tw0 = lt0 + QW * wave;             // first query of this wave (local)
  const bool wave_active = tw0 < T;
  const int alast_blk = a0 + min(lt0 + C::BM - 1, T - 1);  // last query (absolute)
  const int aw0 = a0 + tw0;                                // absolute
  const int awlast = a0 + min(tw0 + QW - 1, T - 1);

  // the tile's key tiles: anchors [0, n_end) then the band [jb0, alast_blk]
  const int n_end = max(0, alast_blk - W) / D;
  const int jb0 = max(0, a0 + lt0 - W);
  const int na_t = (n_end + C::BN - 1) / C::BN;
  const int nb_t = W > 0 ? (alast_blk - jb0 + C::BN) / C::BN : 0;
  const int n_items = na_t + nb_t;
  // key tile i: its rows, first key position and number of valid rows
  auto item_src = [&](int i, RowMap<ST, HD>& rows, int& nvalid, int& key0) {
    rows.n1 = rows.n2 = 0;
    rows.W = W;
    if (i < na_t) {
      key0 = i * C::BN;
      rows.kh = kcp + (int64_t)key0 * HD;
      rows.vh = vcp + (int64_t)key0 * HD;
      nvalid = n_end - key0;
    } else {
      key0 = jb0 + (i - na_t) * C::BN;
      rows.kh = hkp + (int64_t)(key0 - a0) * HD;  // rows before t0: ring
      rows.vh = hvp + (int64_t)(key0 - a0) * HD;
      nvalid = alast_blk + 1 - key0;
    }
    rows.kr = rows.kh;
    rows.vr = rows.vh;
    if (RING && i >= na_t && key0 < a0) {
      const int s0 = key0 % W;
      rows.n2 = a0 - key0;
      rows.n1 = min(rows.n2, W - s0);
      rows.kr = rkp + (int64_t)s0 * HD;
      rows.vr = rvp + (int64_t)s0 * HD;
    }
  };
  auto load_item = [&](Prefetch<ST, HD, QB>& pf, int i) {
    RowMap<ST, HD> rows;
    int nv, k0;
    item_src(i, rows, nv, k0);
    if constexpr (!RING && C::VROW)
      pf.load_linear(rows.kh, rows.vh, nv);
    else
      pf.load(rows, nv);
  };

  // Stage st of the direct-to-LDS path: instruction j (of BN/4 per tensor,
  // BN/16 per wave) fills rows 4j .. 4j+3; lane l lands 16 bytes at chunk
  // l % 16 of row 4j + l / 16, so it loads the global chunk whose swizzled
  // place that is.  Rows at or past nvalid re-read row nvalid-1 (masked).
  auto dma_item = [&](int i, int st) {
    static_assert(!DMA || (sizeof(ST) == 2 && HD == 128 && !RING && C::BN % 16 == 0), "DMA");
    if constexpr (DMA) {
      RowMap<ST, HD> rows;
      int nv, k0;
      item_src(i, rows, nv, k0);
      ST* dK = sK + st * (C::BN * HD);
      ST* dV = sV + st * (C::BN * HD);
      const int pc = lane & 15;
#pragma unroll
      for (int j = 0; j < C::BN / 16; ++j) {
        const int ins = (C::BN / 16) * wave + j;
        const int r = 4 * ins + (lane >> 4);
        const int64_t rs = (int64_t)min(r, nv - 1) * HD;
        dma16(rows.kh + rs + 8 * (pc ^ (r & 15)), dK + ins * 4 * HD);
        dma16(rows.vh + rs + 8 * (pc ^ (2 * (r & 7))), dV + ins * 4 * HD);
      }
    }
  };
  Prefetch<ST, HD, QB> pf;
  if constexpr (DMA) {
    __syncthreads();  // the workgroup's previous tile loop is done with both stages
    if (n_items > 0) dma_item(0, 0);
  } else {
    if (n_items > 0) load_item(pf, 0);
  }

  // own position folded into the initial state (m = its score, from the
  // unscaled q in fp32; l = 1; acc = its value row).  The MFMA operand is Q
  // pre-scaled by c = scale*log2(e), so tile scores come out in log2 units
  // (bf16: q*c is rounded once, a relative 2^-9 per element, the same order
  // as the bf16 rounding of P).
  WaveState<ST, HD, QB> ws;
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    ws.tq[nb] = aw0 + 16 * nb + col;
    ws.nlo[nb] = max(0, min(ws.tq[nb], a0 + T - 1) - W) / D;
    float d = 0.f;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      d += frag_dot(qin.q[nb][s], qin.k[nb][s]);
      ws.qf[nb][s] = frag_scale(qin.q[nb][s], p.scale_log2);
    }
    d = xor16_32_sum(d);
    ws.m[nb] = d * p.scale_log2;
    ws.l[nb] = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) ws.acc[nb][db] = qin.v[nb][db].f32();
  }

  const int w_end = wave_active ? max(0, awlast - W) / D : 0;
  const int w_full = wave_active ? max(0, aw0 - W) / D : 0;
  const int wj0 = max(0, aw0 - W);
  for (int i = 0; i < n_items; ++i) {
    const ST* tK = sK;
    const ST* tV = sV;
    if constexpr (DMA) {
      // this wave's loads of tile i have landed (and every earlier memory
      // operation); after the barrier every wave's have, and every wave is
      // done with tile i-1, whose stage the loads of tile i+1 then refill
      RAT_WAIT_VM_LGKM(0);
      lds_barrier();
      if (i + 1 < n_items) dma_item(i + 1, (i + 1) & 1);
      tK = sK + (i & 1) * (C::BN * HD);
      tV = sV + (i & 1) * (C::BN * HD);
    } else {
      __syncthreads();  // every wave is done reading the previous tile
      pf.store(sK, sV);
      __syncthreads();
      if (i + 1 < n_items) load_item(pf, i + 1);  // overlaps this tile's MFMAs
    }
    RowMap<ST, HD> rows;
    int nv, key0;
    item_src(i, rows, nv, key0);
    const int kind = i < na_t ? 0 : 1;
    bool part, need_mask;
    if (kind == 0) {
      part = key0 < w_end;
      need_mask = key0 + C::BN > w_full;
    } else {
      part = wave_active && key0 <= awlast && key0 + C::BN > wj0;
      // fully visible to all of the wave's queries iff
      // aw0+QW-1 - W <= key0 and key0 + BN - 1 <= aw0 - 1 (and no clamped rows)
      need_mask = !((aw0 + QW - 1 - W <= key0) && (key0 + C::BN <= aw0) && (tw0 + QW - 1 < T));
    }
    if (part) {
      if constexpr (DMA)
        tile_update<ST, HD, QB, C::VROW, C::VRSTR, true, 0>(ws, tK, tV, key0, kind, need_mask, W);
      else
        tile_update<ST, HD, QB, C::VROW, (C::VROW ? C::VRSTR : C::VSTR), false,
                    (QB == 2 && HD == 128 && sizeof(ST) == 2) ? 1 : -1>(ws, tK, tV, key0, kind,
                                                                    need_mask, W);
    }
  }

  // ---- normalise and store --------------------------------------------------
  ST* op = reinterpret_cast<ST*>(p.o) + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    const float lt = ws.l[nb][0];
    const int t = ws.tq[nb] - a0;  // local row
    if (t < T) {
      const float inv = 1.f / lt;
      ST* orow = op + (int64_t)t * p.o_st;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) st4(orow + 16 * db + 4 * g, ws.acc[nb][db] * inv);
      if (p.lse != nullptr && g == 0) p.lse[bh * T + t] = (ws.m[nb] + __log2f(lt)) * kLn2;
    }
  }
}

// Occupancy: one workgroup's MFMAs overlap the others' staging and softmax.
// QB = 2 runs 2 waves per SIMD (fits the 256-register budget without
// spills); QB = 1 runs 3 (168 registers; its tiles are short and wait on
// memory, so more waves in flight beat prefetching the partner tile's
// queries, which would need 48 more registers).  RING: a continuation whose
// window reaches before t0 (band rows from the previous call's ring);
// without it the band tiles are plain linear reads.
template <typename ST, int HD, int QB, bool RING, bool DMA = false>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(QB == 1 ? 3 : 2, QB == 1 ? 3 : 2)))
void attn_prefill_kernel(const AttnParams p) {
  using C = AttnCfg<ST, HD, QB>;
  // two stages of unpadded tiles for the direct-to-LDS path, one padded
  // stage otherwise
  __shared__ __attribute__((aligned(1024))) ST sK[DMA ? 2 * C::BN * HD : C::BN * C::KSTR];
  __shared__ __attribute__((aligned(1024))) ST sV[DMA ? 2 * C::BN * HD : C::VLDS];

  // block -> (unit, pair), a unit being one (head rank, batch row), units in
  // descending cost.  Workgroup i runs on XCD i % 8, and each XCD has its own
  // L2, so the pairs of a unit are kept on few XCDs: in every group of eight
  // consecutive units, XCD x runs the first half of unit x's pairs and the
  // second half of unit 7-x's.  A unit's anchor rows and band tiles are then
  // fetched into two L2s rather than all eight, and the cost per XCD stays
  // level even where a group mixes heavy and light heads.  The units past
  // the last full group are dealt round-robin.
  const int L = blockIdx.x;
  const int grouped = (p.B * p.H) / 8 * 8 * p.np;
  int u, pr;
  if (L < grouped) {
    const int x = L & 7;
    const int s = L >> 3;
    const int grp = s / p.np;
    pr = s - grp * p.np;
    u = 8 * grp + (pr < (p.np + 1) / 2 ? x : 7 - x);
  } else {
    const int r = L - grouped;
    u = grouped / p.np + r / p.np;
    pr = r - (r / p.np) * p.np;
  }
  const int rank = u / p.B;
  const int b = u - rank * p.B;
  const int h = p.perm[rank];

  const int qa = p.nq - 1 - pr;  // heavy tile first, then its partner
  const int ntiles = p.paired && pr < qa ? 2 : 1;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t off = bh * p.T * HD;
  const ST* qp = reinterpret_cast<const ST*>(p.q) + (bh / p.H) * p.q_sb + (bh % p.H) * p.q_sh;
  const ST* hkp = reinterpret_cast<const ST*>(p.hk) + off;
  const ST* hvp = reinterpret_cast<const ST*>(p.hv) + off;
  const int wave = threadIdx.x >> 6;
  QueryIn<ST, HD, QB> qin;
  qin.load(qp, hkp, hvp, qa * C::BM + 16 * QB * wave, p.T, p.q_st);
  process_tile<ST, HD, QB, RING, DMA>(p, b, h, qa * C::BM, sK, sV, qin);
  if (ntiles == 2) {
    qin.load(qp, hkp, hvp, pr * C::BM + 16 * QB * wave, p.T, p.q_st);
    process_tile<ST, HD, QB, RING, DMA>(p, b, h, pr * C::BM, sK, sV, qin);
  }
}

// ---------------------------------------------------------------------------
// Resident-anchor kernel: no window and at most kResidentAnchors anchors per
// head (e.g. T = 4096 at D = 16), bf16.  A workgroup loads its head's anchor
// rows into LDS once (K and V row-major: 140 KB at hd = 128; V's transposed
// MFMA fragments come from ds_read_b64_tr_b16) and its
// 16 waves then stream 16-query blocks independently -- no barrier and no
// global K/V traffic per block; with four waves per SIMD, the waves waiting
// for their next block's query rows (q, own key, own value) overlap the
// others' MFMAs.  Blocks of a head are dealt round-robin over its workgroups
// and waves, so every wave sees the same mix of short (early) and long
// (late) query rows.
// ---------------------------------------------------------------------------
template <typename ST, int HD, int QB>
__device__ __forceinline__ void resident_block(const AttnParams& p, int64_t bh, int D, int tb,
                                               const ST* sK, const ST* sV,
                                               const QueryIn<ST, HD, QB>& qin) {
  using C = AttnCfg<ST, HD, QB>;
  constexpr int QW = 16 * QB;  // queries of the block
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int T = p.T;

  const int a0 = p.t0;  // absolute position of local row 0
  WaveState<ST, HD, QB> ws;
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    ws.tq[nb] = a0 + tb + 16 * nb + col;
    ws.nlo[nb] = min(ws.tq[nb], a0 + T - 1) / D;
    float d = 0.f;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      d += frag_dot(qin.q[nb][s], qin.k[nb][s]);
      ws.qf[nb][s] = frag_scale(qin.q[nb][s], p.scale_log2);
    }
    d = xor16_32_sum(d);
    ws.m[nb] = d * p.scale_log2;
    ws.l[nb] = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) ws.acc[nb][db] = qin.v[nb][db].f32();
  }
  const int n_end = (a0 + min(tb + QW - 1, T - 1)) / D;  // anchors any query of the block sees
  const int w_full = (a0 + tb) / D;                      // anchors every query of the block sees
  for (int key0 = 0; key0 < n_end; key0 += C::BN)
    tile_update<ST, HD, QB, true, C::VRSTR>(ws, sK + key0 * C::KSTR, sV + key0 * C::VRSTR, key0, 0,
                                       key0 + C::BN > w_full, 0);

  // buffer stores: lanes of rows past T (and the lse of lanes g > 0, or a
  // null lse) use an offset outside the region, which the hardware drops
  const auto orsrc = buffer_region(reinterpret_cast<ST*>(p.o) + (int64_t)(bh / p.H) * p.o_sb +
                                   (int64_t)(bh % p.H) * p.o_sh);
  const auto lrsrc = buffer_region(p.lse != nullptr ? p.lse + bh * T : nullptr);
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    const float lt = ws.l[nb][0];
    const int t = ws.tq[nb] - a0;  // local row
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const uint32_t ob =
          t < T ? (uint32_t)(((int64_t)t * p.o_st + 16 * db + 4 * g) * sizeof(ST)) : kDropOffset;
      buffer_st4(orsrc, ob, ws.acc[nb][db] * inv);
    }
    const uint32_t lb = (t < T && g == 0 && p.lse != nullptr) ? (uint32_t)t * 4u : kDropOffset;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((ws.m[nb] + __log2f(lt)) * kLn2), lrsrc,
                                          lb, 0, 0);
  }
}

template <typename ST, int HD, int QB, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void attn_resident_kernel(const AttnParams p) {
  using C = AttnCfg<ST, HD, QB>;
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) ST sK[kResidentAnchors * C::KSTR];
  __shared__ __attribute__((aligned(16))) ST sV[kResidentAnchors * C::VRSTR];

  const int L = blockIdx.x;
  const int per_rank = p.B * p.nra;
  const int rank = L / per_rank;
  const int rem = L - rank * per_rank;
  const int b = rem / p.nra;
  const int r = rem - b * p.nra;
  const int h = p.perm[rank];
  const int T = p.T;
  const int D = p.ht.D[h];
  const int64_t bh = (int64_t)b * p.H + h;
  const int tid = threadIdx.x;

  // ---- stage the anchors a < floor((t0+T-1)/D) (<= kResidentAnchors) -----
  const int nan = (p.t0 + T - 1) / D;
  if (nan > 0) {
    const ST* kcp = reinterpret_cast<const ST*>(p.Kc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
    const ST* vcp = reinterpret_cast<const ST*>(p.Vc) + ((int64_t)b * p.R + p.ht.aoff[h]) * HD;
    const int nt = (nan + C::BN - 1) / C::BN;
    for (int j = 0; j < nt; ++j) {
      // K: BN rows x CPR 16-byte chunks; rows at or past nan re-read row
      // nan-1 (finite, always masked)
#pragma unroll
      for (int i = 0; i < (C::KITEMS + NT - 1) / NT; ++i) {
        const int idx = tid + NT * i;
        if (idx < C::KITEMS) {
          const int row = idx / C::CPR;
          const int c16 = idx - row * C::CPR;
          const int a = min(C::BN * j + row, nan - 1);
          st_raw16(sK + (C::BN * j + row) * C::KSTR + c16 * C::VEC,
                   ld_raw16(kcp + (int64_t)a * HD + c16 * C::VEC));
        }
      }
      // V row-major like K (its transposed fragments are read with
      // ds_read_b64_tr_b16)
#pragma unroll
      for (int i = 0; i < (C::KITEMS + NT - 1) / NT; ++i) {
        const int idx = tid + NT * i;
        if (idx < C::KITEMS) {
          const int row = idx / C::CPR;
          const int c16 = idx - row * C::CPR;
          const int a = min(C::BN * j + row, nan - 1);
          st_raw16(sV + (C::BN * j + row) * C::VRSTR + c16 * C::VEC,
                   ld_raw16(vcp + (int64_t)a * HD + c16 * C::VEC));
        }
      }
    }
  }
  __syncthreads();  // the only barrier: anchors are read-only from here on

  // ---- 16*QB-query blocks: block r + nra*(wave + NW*k) ------------------
  constexpr int QW = 16 * QB;
  const int wave = tid >> 6;
  const int nblk = (T + QW - 1) / QW;
  const int stride = p.nra * NW;
  const int first = r + p.nra * wave;
  const int64_t off = bh * T * HD;
  const ST* qp = reinterpret_cast<const ST*>(p.q) + (bh / p.H) * p.q_sb + (bh % p.H) * p.q_sh;
  const ST* hkp = reinterpret_cast<const ST*>(p.hk) + off;
  const ST* hvp = reinterpret_cast<const ST*>(p.hv) + off;
  // the wave's blocks first + j*stride; the NW waves of the CU hide the load
  // latency of each block's query inputs
  for (int bi = first; bi < nblk; bi += stride) {
    QueryIn<ST, HD, QB> qa;
    qa.load(qp, hkp, hvp, QW * bi, T, p.q_st);
    resident_block<ST, HD, QB>(p, bh, D, QW * bi, sK, sV, qa);
  }
}

template <typename ST, int HD>
int launch_t(const AttnParams& p, hipStream_t st) {
  if (p.mode == 1) {
    if constexpr (sizeof(ST) == 2) {
      const int64_t nwg = (int64_t)p.H * p.B * p.nra;
      if (nwg == 0) return 0;
      hipLaunchKernelGGL((attn_resident_kernel<ST, HD, kResidentQB, kResidentWaves>),
                         dim3((unsigned)nwg), dim3(64 * kResidentWaves), 0, st, p);
      return (int)hipGetLastError();
    }
    return (int)hipErrorInvalidValue;
  }
  const int64_t nblk = (int64_t)p.H * p.B * p.np;
  if (nblk == 0) return 0;
  // the ring-reading variant only where a window reaches before t0
  const bool ring = p.t0 > 0 && p.WS > 0;
  const dim3 grid((unsigned)nblk), block(256);
  if (p.qb == 2) {
    if (ring)
      hipLaunchKernelGGL((attn_prefill_kernel<ST, HD, 2, true>), grid, block, 0, st, p);
    else if (sizeof(ST) == 2 && HD == 128 && p.dma)
      hipLaunchKernelGGL((attn_prefill_kernel<ST, HD, 2, false, sizeof(ST) == 2 && HD == 128>), grid,
                         block, 0, st, p);
    else
      hipLaunchKernelGGL((attn_prefill_kernel<ST, HD, 2, false>), grid, block, 0, st, p);
  } else {
    if (ring)
      hipLaunchKernelGGL((attn_prefill_kernel<ST, HD, 1, true>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((attn_prefill_kernel<ST, HD, 1, false>), grid, block, 0, st, p);
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_attn_prefill(int dtype, int hd, const AttnParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) return hd == 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
  return hd == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace rat
