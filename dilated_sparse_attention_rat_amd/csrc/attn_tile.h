// Building blocks of the prefill attention kernels (csrc/attn_prefill.hip,
// csrc/attn_resident.hip): the launch configuration, the wave's online
// softmax state, the query inputs, and one staged key tile against a wave's
// queries (scores, softmax, PV product).  The method and the design are
// described at the top of csrc/attn_prefill.hip.
#pragma once

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

}  // namespace

}  // namespace rat
