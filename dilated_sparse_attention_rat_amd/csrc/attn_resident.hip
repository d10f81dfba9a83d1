// Prefill dilated causal attention, resident-anchor kernel (windowless bf16
// heads with at most kResidentAnchors anchors each).  Method and design: the
// top of csrc/attn_prefill.hip; the tile building blocks: csrc/attn_tile.h.
// This file is compiled with the compiler's memory-clause scheduling
// strategy (the build's per-file flags), which measured faster for this
// kernel only.
#include "attn_tile.h"

namespace rat {

namespace {

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

}  // namespace

// the resident-anchor launch (bf16 only; the host selects it)
int launch_attn_resident(int dtype, int hd, const AttnParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype != RAT_DTYPE_BF16) return (int)hipErrorInvalidValue;
  const int64_t nwg = (int64_t)p.H * p.B * p.nra;
  if (nwg == 0) return 0;
  if (hd == 128)
    hipLaunchKernelGGL((attn_resident_kernel<bf16, 128, kResidentQB, kResidentWaves>),
                       dim3((unsigned)nwg), dim3(64 * kResidentWaves), 0, st, p);
  else
    hipLaunchKernelGGL((attn_resident_kernel<bf16, 64, kResidentQB, kResidentWaves>),
                       dim3((unsigned)nwg), dim3(64 * kResidentWaves), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace rat
