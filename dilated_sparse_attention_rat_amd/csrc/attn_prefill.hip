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
#include "attn_tile.h"

namespace rat {

namespace {

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
      // wave-uniform LDS bases and tile rows in SGPRs; per lane only a
      // 32-bit byte offset (row clamp, row, swizzled chunk)
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const uint32_t lK = lds_addr(sK + st * (C::BN * HD));
      const uint32_t lV = lds_addr(sV + st * (C::BN * HD));
      const int pc = lane & 15;
#pragma unroll
      for (int j = 0; j < C::BN / 16; ++j) {
        const int ins = (C::BN / 16) * wv + j;
        const int r = 4 * ins + (lane >> 4);
        const uint32_t ro = (uint32_t)min(r, nv - 1) * (uint32_t)(HD * sizeof(ST));
        const uint32_t lo = (uint32_t)(ins * 4 * HD * sizeof(ST));
        dma16s(rows.kh, ro + 16u * (uint32_t)(pc ^ (r & 15)), lK + lo);
        dma16s(rows.vh, ro + 16u * (uint32_t)(pc ^ (2 * (r & 7))), lV + lo);
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
  // In a paired launch the groups from gsingle on take single tiles instead
  // (nq per unit): they run last, tile by tile across all of those groups,
  // heaviest first, and the hardware hands them out in decreasing cost as
  // slots free up, which shortens the tail.
  const int L = blockIdx.x;
  const int nfull = (p.B * p.H) / 8;
  const int gs = min(p.gsingle, nfull);
  const int paired_blocks = gs * 8 * p.np;
  const int single_blocks = (nfull - gs) * 8 * p.nq;
  int u, pr;
  bool tail = false;
  if (L < paired_blocks) {
    const int x = L & 7;
    const int s = L >> 3;
    const int g = s / p.np;
    pr = s - g * p.np;
    u = 8 * g + (pr < (p.np + 1) / 2 ? x : 7 - x);
  } else if (L < paired_blocks + single_blocks) {
    tail = true;
    const int r = L - paired_blocks;
    const int x = r & 7;
    const int s = r >> 3;
    const int ntg = nfull - gs;  // tail groups
    pr = s / ntg;
    const int g = gs + (s - pr * ntg);
    u = 8 * g + (pr < (p.nq + 1) / 2 ? x : 7 - x);
  } else {
    const int r = L - paired_blocks - single_blocks;
    u = 8 * nfull + r / p.np;
    pr = r - (r / p.np) * p.np;
  }
  const int rank = u / p.B;
  const int b = u - rank * p.B;
  const int h = p.perm[rank];

  const int qa = p.nq - 1 - pr;  // heavy tile first, then its partner
  const int ntiles = p.paired && !tail && pr < qa ? 2 : 1;
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

template <typename ST, int HD>
int launch_t(const AttnParams& p, hipStream_t st) {
  const int64_t nblk = p.nblk;
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
  if (p.mode == 1) return launch_attn_resident(dtype, hd, p, stream);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) return hd == 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
  return hd == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace rat
