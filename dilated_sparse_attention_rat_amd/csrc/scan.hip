// Prefill recurrence h_t = g_t*h_{t-1} + (1-g_t)*x_t over keys and values,
// with the anchor-cache compaction, the window-ring tail and the final
// state fused into the same pass.
//
// Method: zhichai.net deep dive "RAT+ 深度拆解", section 2.1 -- the gated
// recurrence runs over the whole sequence and prefill evaluates it as an
// associative scan; RAT+ abstract -- the KV cache keeps only the stride-D
// anchors.  The scan combines the affine maps h -> A*h + B of consecutive
// segments: (A1,B1) then (A2,B2) = (A1*A2, A2*B1 + B2).
//
// Design (one pass over HBM, every input read once):
//  * one workgroup (256 lanes) owns one chunk of LC consecutive positions of
//    one (b, h) sequence across all hd channels; lanes are laid out as
//    row-groups x channel-vectors so each row of hd values is read and
//    written with 16-byte accesses by consecutive lanes (coalesced);
//  * each lane keeps its S rows of k, v, g in registers, reduces them to a
//    local affine map, and the row-groups are scanned in LDS;
//  * chunks are linked through a radix-8 tree of chunk aggregates in a small
//    fp32 workspace (entries tagged with a launch epoch): each chunk
//    publishes its aggregate, the chunk owning the last child of a node
//    publishes the node, and a chunk's carry-in is the in-order composition
//    of at most 7 nodes per level that precede it.  No chunk waits on a
//    serial chain, and the composition order is fixed, so the scan is
//    bitwise deterministic run to run;
//  * the kernel is persistent: its grid is at most the number of workgroups
//    the device holds at once, so all of them are resident together;
//    chunks are assigned statically in chunk-major order, so every node a
//    workgroup waits on belongs to a smaller ticket of a resident workgroup
//    (no deadlock) and no atomic ticket counter is needed (same-address
//    device-scope atomics serialise at about 10 ns each); every wait is
//    bounded;
//  * the second pass re-runs the sequential recurrence from the chunk's
//    carry-in on the registers and streams hk/hv, anchor rows, ring slots
//    and the final fp32 state out with 16-byte stores.
#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "rat_device.h"

namespace rat {

namespace {

constexpr uint32_t kSpinLimit = 1u << 16;

__device__ __forceinline__ uint32_t ld_acquire_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent_f32(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_coherent_f32(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Workspace header words (uint32): the launch epoch, the error flag, and the
// done counters that let the last block advance the epoch.  Counters sit
// 256 bytes apart so their atomics do not queue on one address.
constexpr int kEpochWord = 0;
constexpr int kErrorWord = 2;
constexpr int kTopWord = 32;
constexpr int kDoneBase = 64;
constexpr int kDoneStride = 64;
constexpr int kDoneSlots = 64;
static_assert(kDoneBase + kDoneSlots * kDoneStride <= kScanHeaderBytes / 4, "header");

constexpr int kScanRadixLog2 = 3;
static_assert((1 << kScanRadixLog2) == kScanRadix, "radix");

// Wait until this wave's earlier global accesses have completed.  Every
// workspace access below is a coherent (agent-scope, sc1) atomic access, so
// completion order is all the publication protocol needs: data stores
// complete before the tag store is issued, and data loads are issued only
// after the tag load has returned.  No cache write-back or invalidation is
// required (an agent-scope fence would write back / invalidate the whole L2
// of the XCD on every call).
__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The hd channels are independent; the tree works on 64-channel halves, one
// wave per half with one channel per lane.  Every published value is a 64-bit
// word (launch tag << 32 | fp32 bits) written and read with single-copy
// atomic 64-bit accesses, so a reader that sees the current tag in a word
// also sees its value: no separate flag, no store drain, one round trip.
__device__ __forceinline__ void st_tagged(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish one half of a tree node (A, Bk, Bv of this lane's channel).
template <int HD>
__device__ __forceinline__ void publish_node(const ScanParams& p, int64_t e, int half, float A,
                                             float Bk, float Bv, uint32_t tag, int lane) {
  uint64_t* d = p.agg + e * 3 * HD + 64 * half + lane;
  st_tagged(d, tag, A);
  st_tagged(d + HD, tag, Bk);
  st_tagged(d + 2 * HD, tag, Bv);
}

// Compose the n (< radix) consecutive nodes [e0, e0 + n), in order, after
// the running map (A, Bk, Bv) of one channel.  All 3n words are loaded at
// once and re-loaded until every tag in the wave is current; every wait is
// bounded.
template <int HD>
__device__ __forceinline__ void fold_nodes(const ScanParams& p, int64_t e0, int n, int half,
                                           float& A, float& Bk, float& Bv, uint32_t tag,
                                           int lane) {
  if (n <= 0) return;
  uint64_t w[kScanRadix - 1][3];
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < kScanRadix - 1; ++i) {
      if (i < n) {
        const uint64_t* d = p.agg + (e0 + i) * 3 * HD + 64 * half + lane;
        w[i][0] = ld_tagged(d);
        w[i][1] = ld_tagged(d + HD);
        w[i][2] = ld_tagged(d + 2 * HD);
      }
    }
#pragma unroll
    for (int i = 0; i < kScanRadix - 1; ++i)
      if (i < n)
        ok = ok && (uint32_t)(w[i][0] >> 32) == tag && (uint32_t)(w[i][1] >> 32) == tag &&
             (uint32_t)(w[i][2] >> 32) == tag;
    if (__all(ok)) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) st_relaxed_u32(p.hdr + kErrorWord, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int i = 0; i < kScanRadix - 1; ++i) {
    if (i < n) {
      const float a = __uint_as_float((uint32_t)w[i][0]);
      Bk = a * Bk + __uint_as_float((uint32_t)w[i][1]);
      Bv = a * Bv + __uint_as_float((uint32_t)w[i][2]);
      A = A * a;
    }
  }
}

// The carry-in of a chunk: the state st (2*HD tagged words, the k and v
// states after the previous block; nullptr: keep the running state) and
// then the n (< radix) consecutive nodes [e0, e0 + n) composed onto the
// running state (Bk, Bv) of one channel, all loaded in one batch and
// re-loaded until every tag in the wave is current; every wait is bounded.
template <int HD>
__device__ __forceinline__ void fold_state_nodes(const ScanParams& p, const uint64_t* st,
                                                 int64_t e0, int n, int half, float& Bk,
                                                 float& Bv, uint32_t tag, int lane) {
  if (n <= 0 && st == nullptr) return;
  uint64_t w[kScanRadix - 1][3];
  uint64_t sw[2] = {0, 0};
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
    if (st != nullptr) {
      sw[0] = ld_tagged(st + 64 * half + lane);
      sw[1] = ld_tagged(st + HD + 64 * half + lane);
    }
#pragma unroll
    for (int i = 0; i < kScanRadix - 1; ++i) {
      if (i < n) {
        const uint64_t* d = p.agg + (e0 + i) * 3 * HD + 64 * half + lane;
        w[i][0] = ld_tagged(d);
        w[i][1] = ld_tagged(d + HD);
        w[i][2] = ld_tagged(d + 2 * HD);
      }
    }
    if (st != nullptr) ok = (uint32_t)(sw[0] >> 32) == tag && (uint32_t)(sw[1] >> 32) == tag;
#pragma unroll
    for (int i = 0; i < kScanRadix - 1; ++i)
      if (i < n)
        ok = ok && (uint32_t)(w[i][0] >> 32) == tag && (uint32_t)(w[i][1] >> 32) == tag &&
             (uint32_t)(w[i][2] >> 32) == tag;
    if (__all(ok)) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) st_relaxed_u32(p.hdr + kErrorWord, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (st != nullptr) {
    Bk = __uint_as_float((uint32_t)sw[0]);
    Bv = __uint_as_float((uint32_t)sw[1]);
  }
#pragma unroll
  for (int i = 0; i < kScanRadix - 1; ++i) {
    if (i < n) {
      const float a = __uint_as_float((uint32_t)w[i][0]);
      Bk = a * Bk + __uint_as_float((uint32_t)w[i][1]);
      Bv = a * Bv + __uint_as_float((uint32_t)w[i][2]);
    }
  }
}

template <typename ST, int HD, int S>
struct ChunkRows {
  u32x4 k[S], v[S], g[S];
};

// Issue the loads of this lane's S rows of chunk `ticket` (kept in registers
// for both passes).  The loads are unconditional (rows at or past T re-read
// row T-1 and are ignored) so the compiler can count outstanding loads
// exactly and wait only for the ones it needs.
template <typename ST, int HD, int S>
__device__ __forceinline__ void load_rows(const ScanParams& p, uint32_t ticket,
                                          ChunkRows<ST, HD, S>& rw) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;
  constexpr int RG = kScanThreads / LPR;
  constexpr int LC = RG * S;
  const int tid = threadIdx.x;
  const int chunk = (int)(ticket / (uint32_t)p.nseq);
  const int seq = (int)(ticket % (uint32_t)p.nseq);
  const int r = tid / LPR;
  const int c0 = (tid - r * LPR) * VEC;
  const int tbase = chunk * LC + r * S;
  const int b = seq / p.H;
  const int64_t in_base = (int64_t)b * p.in_sb + (int64_t)(seq - b * p.H) * p.in_sh + c0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = min(tbase + s, p.T - 1);
    const int64_t off = in_base + (int64_t)t * p.in_st;
    rw.k[s] = ld_raw16_nt(reinterpret_cast<const ST*>(p.k) + off);
    rw.v[s] = ld_raw16_nt(reinterpret_cast<const ST*>(p.v) + off);
    rw.g[s] = ld_raw16_nt(reinterpret_cast<const ST*>(p.g) + off);
  }
}

// The gate of one row: g itself, or (GATE) sigmoid(g + bias) with g the
// gate's pre-activation and the head's per-channel bias.
template <int VEC, bool GATE>
__device__ __forceinline__ void apply_gate(float (&gf)[VEC], const float (&gbias)[VEC]) {
  if constexpr (GATE) {
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      gf[i] = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-(gf[i] + gbias[i]) * kLog2e));
  }
}

template <typename ST, int HD, bool GATE>
__device__ __forceinline__ void load_gate_bias(const ScanParams& p, int h, int c0,
                                               float (&gbias)[StTraits<ST>::VEC]) {
  if constexpr (GATE) {
#pragma unroll
    for (int i = 0; i < StTraits<ST>::VEC; ++i) gbias[i] = p.gate_bias[h * HD + c0 + i];
  }
}

// Row-group maps of one chunk in LDS: one set per chunk in flight.
template <int RG, int HD>
struct PrefixSet {
  float A[RG][HD];
  float Bk[RG][HD];
  float Bv[RG][HD];
  float tot[3][HD];  // the whole chunk's map (A, Bk, Bv)
};

// Phase A of the pipeline.  Pass 1 of ticket tn (rows rn): each lane reduces
// its rows to an affine map, the row-groups' maps go to LDS set `sn`, then
//  * waves 0..NH-1 scan the row-groups of set sn (exclusive prefix, kept for
//    pass 2) and publish the chunk's aggregate and, for the owner of a node's
//    last child, the node;
//  * waves 2..2+NH-1 compose, concurrently, the carry-in of ticket tc (the
//    chunk whose pass 2 follows) into s_hk / s_hv.
// Publication never waits on a carry, so no chain forms along the sequence:
// every tree node depends on input data only.  The carry is the in-order
// composition, top tree level first, of the complete nodes that precede the
// chunk (at most radix-1 per level): a fixed order, so the result is bitwise
// deterministic.  Ticket tc was published one pipeline step earlier than its
// carry is composed, and so were the chunks of its round before it, so the
// carry's loads normally find every node already there.
template <typename ST, int HD, int S, bool GATE>
__device__ __forceinline__ void scan_phase_a(const ScanParams& p, uint32_t tag, bool pub,
                                             uint32_t tn, const ChunkRows<ST, HD, S>& rn,
                                             PrefixSet<kScanThreads / (HD / StTraits<ST>::VEC), HD>& sn,
                                             bool carry, uint32_t tc,
                                             const PrefixSet<kScanThreads / (HD / StTraits<ST>::VEC), HD>& sc,
                                             float* s_hk, float* s_hv) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;           // lanes per row
  constexpr int RG = kScanThreads / LPR;  // row-groups per chunk
  constexpr int LC = RG * S;              // rows per chunk
  constexpr int NH = HD / 64;             // channel halves
  const int tid = threadIdx.x;
  const int r = tid / LPR;
  const int c0 = (tid - r * LPR) * VEC;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  if (pub) {
    const int chunk = (int)(tn / (uint32_t)p.nseq);
    const int seq = (int)(tn % (uint32_t)p.nseq);
    const int h = seq % p.H;
    const int tbase = chunk * LC + r * S;
    float gbias[VEC];
    load_gate_bias<ST, HD, GATE>(p, h, c0, gbias);
    float A[VEC], Bk[VEC], Bv[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      A[i] = 1.f;
      Bk[i] = 0.f;
      Bv[i] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (tbase + s < p.T) {
        float gf[VEC], kf[VEC], vf[VEC];
        unpack16(rn.g[s], gf, (ST*)nullptr);
        apply_gate<VEC, GATE>(gf, gbias);
        unpack16(rn.k[s], kf, (ST*)nullptr);
        unpack16(rn.v[s], vf, (ST*)nullptr);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          A[i] *= gf[i];
          Bk[i] = gf[i] * Bk[i] + (1.f - gf[i]) * kf[i];
          Bv[i] = gf[i] * Bv[i] + (1.f - gf[i]) * vf[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      sn.A[r][c0 + i] = A[i];
      sn.Bk[r][c0 + i] = Bk[i];
      sn.Bv[r][c0 + i] = Bv[i];
    }
  }
  __syncthreads();

  if (wave < NH) {
    if (pub) {
      const int chunk = (int)(tn / (uint32_t)p.nseq);
      const int seq = (int)(tn % (uint32_t)p.nseq);
      const int half = wave;
      const int c = 64 * half + lane;
      float ra = 1.f, rbk = 0.f, rbv = 0.f;
      for (int rr = 0; rr < RG; ++rr) {
        const float a = sn.A[rr][c], bk = sn.Bk[rr][c], bv = sn.Bv[rr][c];
        sn.A[rr][c] = ra;  // exclusive prefix of the row-groups
        sn.Bk[rr][c] = rbk;
        sn.Bv[rr][c] = rbv;
        rbk = a * rbk + bk;
        rbv = a * rbv + bv;
        ra = ra * a;
      }
      sn.tot[0][c] = ra;
      sn.tot[1][c] = rbk;
      sn.tot[2][c] = rbv;
      // A node of level l+1 is the in-order composition of its radix
      // children; the chunk that owns the last child computes and publishes
      // it.  Only the levels a carry inside a block folds are published.
      int64_t node = chunk;
      for (int lv = 0; lv < p.blk_levels; ++lv) {
        const int64_t lvl0 = p.lbase[lv] + (int64_t)seq * p.nodes[lv];
        publish_node<HD>(p, lvl0 + node, half, ra, rbk, rbv, tag, lane);
        if (lv + 1 >= p.blk_levels || (node % kScanRadix) != kScanRadix - 1) break;
        float fA = 1.f, fBk = 0.f, fBv = 0.f;
        fold_nodes<HD>(p, lvl0 + node - (kScanRadix - 1), kScanRadix - 1, half, fA, fBk, fBv,
                       tag, lane);
        rbk = ra * fBk + rbk;  // then this node itself
        rbv = ra * fBv + rbv;
        ra = fA * ra;
        node /= kScanRadix;
      }
    }
  } else if (wave >= 2 && wave < 2 + NH) {
    if (carry) {
      const int chunk = (int)(tc / (uint32_t)p.nseq);
      const int seq = (int)(tc % (uint32_t)p.nseq);
      const int half = wave - 2;
      const int c = 64 * half + lane;
      // The carry-in of chunk `chunk` of block kb: the state after block
      // kb-1 (for kb = 0 the state before row 0: zero for a prefill, the
      // given state for a continuation), then the tree nodes that cover
      // the block's chunks before this one, top level first.
      const int kb = chunk / p.mblk;
      const int bs = kb * p.mblk;
      float hin_k = 0.f, hin_v = 0.f;
      const uint64_t* st = nullptr;
      if (kb > 0) {
        st = p.incl + ((int64_t)seq * p.nchunk + (kb - 1)) * 2 * HD;
      } else if (p.sk_in != nullptr) {
        hin_k = p.sk_in[(int64_t)seq * HD + c];
        hin_v = p.sv_in[(int64_t)seq * HD + c];
      }
      for (int lv = p.blk_levels - 1; lv >= 0; --lv) {
        const int64_t nd = (int64_t)chunk >> (kScanRadixLog2 * lv);
        const int64_t first = max(nd & ~(int64_t)(kScanRadix - 1), (int64_t)bs >> (kScanRadixLog2 * lv));
        const int64_t lvl0 = p.lbase[lv] + (int64_t)seq * p.nodes[lv];
        fold_state_nodes<HD>(p, st, lvl0 + first, (int)(nd - first), half, hin_k, hin_v, tag, lane);
        st = nullptr;  // the block state is taken with the top level's nodes
      }
      if (st != nullptr)  // no level inside the block (one chunk per block)
        fold_state_nodes<HD>(p, st, 0, 0, half, hin_k, hin_v, tag, lane);
      s_hk[c] = hin_k;
      s_hv[c] = hin_v;
      // the last chunk of a block publishes the state after it (its carry-in
      // through the chunk's whole map) for the next block's carries
      if (chunk % p.mblk == p.mblk - 1 && chunk + 1 < p.nchunk) {
        const float a = sc.tot[0][c];
        uint64_t* d = p.incl + ((int64_t)seq * p.nchunk + kb) * 2 * HD + c;
        st_tagged(d, tag, a * hin_k + sc.tot[1][c]);
        st_tagged(d + HD, tag, a * hin_v + sc.tot[2][c]);
      }
    }
  }
  __syncthreads();
}

// Phase B: pass 2 of ticket tc (rows rc, its row-group prefix in set sc, its
// carry-in in s_hk / s_hv): the sequential recurrence from the carry-in, with
// hk/hv, anchor rows, ring slots and the final fp32 state streamed out.
template <typename ST, int HD, int S, bool GATE>
__device__ __forceinline__ void scan_phase_b(const ScanParams& p, uint32_t tc,
                                             const ChunkRows<ST, HD, S>& rc,
                                             const PrefixSet<kScanThreads / (HD / StTraits<ST>::VEC), HD>& sc,
                                             const float* s_hk, const float* s_hv) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;
  constexpr int RG = kScanThreads / LPR;
  constexpr int LC = RG * S;
  const int tid = threadIdx.x;
  const int chunk = (int)(tc / (uint32_t)p.nseq);
  const int seq = (int)(tc % (uint32_t)p.nseq);
  const int b = seq / p.H;
  const int h = seq - b * p.H;
  const int T = p.T;
  const int r = tid / LPR;
  const int c0 = (tid - r * LPR) * VEC;
  const int tbase = chunk * LC + r * S;
  const int64_t seq_base = (int64_t)seq * T * HD;
  float gbias[VEC];
  load_gate_bias<ST, HD, GATE>(p, h, c0, gbias);
  float sk[VEC], sv[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const int c = c0 + i;
    sk[i] = sc.A[r][c] * s_hk[c] + sc.Bk[r][c];
    sv[i] = sc.A[r][c] * s_hv[c] + sc.Bv[r][c];
  }
  const int D = p.ht.D[h];
  const int W = p.ht.W[h];
  ST* hkp = reinterpret_cast<ST*>(p.hk);
  ST* hvp = reinterpret_cast<ST*>(p.hv);
  ST* Kcp = reinterpret_cast<ST*>(p.Kc);
  ST* Vcp = reinterpret_cast<ST*>(p.Vc);
  ST* krp = reinterpret_cast<ST*>(p.kr);
  ST* vrp = reinterpret_cast<ST*>(p.vr);
  const int64_t arow0 = (int64_t)b * p.R + p.ht.aoff[h];
  const int64_t rrow0 = (int64_t)b * p.WS + p.ht.roff[h];
  const int tabs = p.t0 + tbase;  // absolute position of row tbase
  int aq = tabs / D;              // anchor index candidate of row tbase
  int ar = tabs - aq * D;         // phase of row tbase
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = tbase + s;
    if (t < T) {
      float gf[VEC], kf[VEC], vf[VEC];
      unpack16(rc.g[s], gf, (ST*)nullptr);
      apply_gate<VEC, GATE>(gf, gbias);
      unpack16(rc.k[s], kf, (ST*)nullptr);
      unpack16(rc.v[s], vf, (ST*)nullptr);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        sk[i] = gf[i] * sk[i] + (1.f - gf[i]) * kf[i];
        sv[i] = gf[i] * sv[i] + (1.f - gf[i]) * vf[i];
      }
      const u32x4 ok = pack16(sk, (ST*)nullptr);
      const u32x4 ov = pack16(sv, (ST*)nullptr);
      if (hkp != nullptr) {
        const int64_t off = seq_base + (int64_t)t * HD + c0;
        st_raw16(hkp + off, ok);
        st_raw16(hvp + off, ov);
      }
      if (ar == D - 1) {
        const int64_t off = (arow0 + aq) * HD + c0;
        st_raw16(Kcp + off, ok);
        st_raw16(Vcp + off, ov);
      }
      if (W > 0 && t >= T - W) {
        const int64_t off = (rrow0 + ((p.t0 + t) % W)) * HD + c0;
        st_raw16(krp + off, ok);
        st_raw16(vrp + off, ov);
      }
      if (t == T - 1) {
        const int64_t off = (int64_t)seq * HD + c0;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          p.sk[off + i] = sk[i];
          p.sv[off + i] = sv[i];
        }
      }
    }
    if (++ar == D) {
      ar = 0;
      ++aq;
    }
  }
}

// Persistent kernel: the grid is sized to the number of workgroups that can
// be resident at once, so every workgroup runs concurrently.  Workgroup w
// processes tickets w, w + G, w + 2G, ... in order; ticket t is chunk t / nseq
// of sequence t % nseq.  A chunk waits only on nodes of earlier chunks of its
// own sequence, i.e. on smaller tickets, so the smallest unfinished ticket
// can always proceed (no deadlock), and no ticket counter (atomic) is needed.
// Every workgroup reads the epoch first; the last one to finish advances it,
// so the epoch is this launch's tag.
//
// Pipeline, per step (tickets t, t+G, t+2G in three register buffers):
//   phase A: pass 1 of t+G and its publication || the carry-in of t;
//   then the loads of t+2G (into the buffer pass 2 of t-G freed);
//   phase B: pass 2 of t.
// So a ticket is published one step before its carry is composed, and the
// tree round trip of a chunk overlaps the next chunk's pass 1.
template <typename ST, int HD, int S, bool GATE>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void scan_kernel(const ScanParams p) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;
  constexpr int RG = kScanThreads / LPR;
  static_assert(HD % 64 == 0 && LPR <= 64, "layout");
  __shared__ PrefixSet<RG, HD> s_set[2];
  __shared__ float s_hk[HD];
  __shared__ float s_hv[HD];
  __shared__ uint32_t s_epoch;

  const int tid = threadIdx.x;
  const uint32_t G = gridDim.x;
  const uint32_t n = (uint32_t)p.nticket;
  uint32_t t = blockIdx.x;
  // (loads are unconditional -- past the end they re-load the last ticket
  // and are ignored -- so the compiler counts outstanding loads exactly)
  ChunkRows<ST, HD, S> r0, r1, r2;
  load_rows<ST, HD, S>(p, min(t, n - 1), r0);
  load_rows<ST, HD, S>(p, min(t + G, n - 1), r1);
  // the epoch after the first rows' loads: its round trip (every workgroup
  // reads the same word) overlaps their arrival
  if (tid == 0) s_epoch = ld_acquire_u32(p.hdr + kEpochWord);
  __syncthreads();
  const uint32_t epoch = s_epoch;
  const uint32_t tag = (epoch % 0x3FFFFFFFu) + 1u;

  if (t < n) {
    scan_phase_a<ST, HD, S, GATE>(p, tag, true, t, r0, s_set[0], false, t, s_set[1], s_hk, s_hv);
    // one pipeline step: ticket t in `cur` (set sc), t+G in `nxt`; the loads
    // of t+2G go to `far` after the carry is known (vector memory operations
    // complete in order, so a carry load issued after them would wait for
    // them) and before pass 2, whose time covers their latency
    auto step = [&](const ChunkRows<ST, HD, S>& cur, const ChunkRows<ST, HD, S>& nxt,
                    ChunkRows<ST, HD, S>& far, int sc) {
      const uint32_t t1 = t + G;
      scan_phase_a<ST, HD, S, GATE>(p, tag, t1 < n, t1, nxt, s_set[sc ^ 1], true, t, s_set[sc],
                                    s_hk, s_hv);
      load_rows<ST, HD, S>(p, min(t + 2 * G, n - 1), far);
      scan_phase_b<ST, HD, S, GATE>(p, t, cur, s_set[sc], s_hk, s_hv);
      __syncthreads();  // set sc and the carry are reused by the next step
      t = t1;
    };
    int sc = 0;
    while (true) {
      step(r0, r1, r2, sc);
      sc ^= 1;
      if (t >= n) break;
      step(r1, r2, r0, sc);
      sc ^= 1;
      if (t >= n) break;
      step(r2, r0, r1, sc);
      sc ^= 1;
      if (t >= n) break;
    }
  }

  // retire: two-level done count; the last workgroup advances the epoch
  if (tid == 0) {
    const uint32_t slot = blockIdx.x % kDoneSlots;
    const uint32_t in_slot = (G - 1 - slot) / kDoneSlots + 1;
    const uint32_t used = G < (uint32_t)kDoneSlots ? G : (uint32_t)kDoneSlots;
    vm_drain();
    uint32_t* ctr = p.hdr + kDoneBase + slot * kDoneStride;
    if (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == in_slot - 1) {
      st_relaxed_u32(ctr, 0u);
      uint32_t* top = p.hdr + kTopWord;
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == used - 1) {
        st_relaxed_u32(top, 0u);
        st_relaxed_u32(p.hdr + kEpochWord, epoch + 1u);
      }
    }
  }
}

// T = 0: the state is the state before row 0 (zero for a prefill)
__global__ void state_init_kernel(float* sk, float* sv, const float* sk_in, const float* sv_in,
                                  int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    sk[i] = sk_in != nullptr ? sk_in[i] : 0.f;
    sv[i] = sv_in != nullptr ? sv_in[i] : 0.f;
  }
}

// Continuation ring carry: the slot of each position p in
// [max(0, t0 + T - W), t0) -- still inside the window after the continuation
// and not rewritten by it -- is copied from the previous ring to the new
// one.  Grid: (chunks of one head's slots, H, B); one 16-byte chunk each.
template <typename ST, int HD>
__global__ void ring_carry_kernel(const ST* __restrict__ kin, const ST* __restrict__ vin, ST* kout,
                                  ST* vout, HeadTables ht, int64_t WS, int64_t t0, int64_t T) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int CPR = HD / VEC;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t W = ht.W[h];
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= W * CPR) return;
  const int64_t slot = idx / CPR;
  const int c16 = (int)(idx - slot * CPR);
  // the position held by this slot before the continuation: the last p < t0
  // with p = slot (mod W)
  const int64_t p = t0 - 1 - (((t0 - 1 - slot) % W) + W) % W;
  if (p < 0 || p < t0 + T - W) return;
  const int64_t off = ((int64_t)b * WS + ht.roff[h] + slot) * HD + c16 * VEC;
  st_raw16(kout + off, ld_raw16(kin + off));
  st_raw16(vout + off, ld_raw16(vin + off));
}

// Largest grid whose workgroups can all be resident at once (cached per
// device and kernel; the cache is the library's only mutable state, written
// once under a lock).
int coop_grid_limit(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, kernel});
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const int lim = per_cu * cus;
  cache[{dev, kernel}] = lim;
  return lim;
}

template <typename ST, int HD>
int launch_scan_t(const ScanParams& p, hipStream_t st) {
  if (p.T == 0) {
    const int64_t n = (int64_t)p.nseq * HD;
    if (n == 0) return 0;
    hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       p.sk, p.sv, p.sk_in, p.sv_in, n);
    return (int)hipGetLastError();
  }
  // the gated variant has its own register use, hence its own residency limit
  const bool gated = p.gate_bias != nullptr;
  const void* kern = gated
      ? reinterpret_cast<const void*>(&scan_kernel<ST, HD, kScanRowsPerThread, true>)
      : reinterpret_cast<const void*>(&scan_kernel<ST, HD, kScanRowsPerThread, false>);
  const int lim = coop_grid_limit(kern, kScanThreads);
  if (lim <= 0) return (int)hipErrorInvalidValue;
  // A plain launch: with the grid within the device's capacity every
  // workgroup is placed as soon as the stream reaches the kernel.  (A
  // cooperative launch gives the same residency as a formal guarantee but
  // costs about 20 us of queue drain per launch.)  If other streams hold
  // CUs, the late workgroups start when those finish; a wait that outlasts
  // the spin bound is reported in the workspace error word, never a hang.
  // Rounds of G tickets hold whole blocks: G = nseq * mblk with mblk the
  // largest power of two that fits the device (one chunk per block when the
  // sequences outnumber the resident workgroups).
  ScanParams q = p;
  int64_t g = lim;
  q.mblk = 1;
  if (p.nseq <= lim) {
    while ((int64_t)p.nseq * q.mblk * 2 <= lim) q.mblk *= 2;
    g = (int64_t)p.nseq * q.mblk;
  }
  q.blk_levels = 0;
  for (int64_t span = 1; span < q.mblk && q.blk_levels < p.nlevels; span *= kScanRadix)
    ++q.blk_levels;
  const unsigned grid = (unsigned)std::min<int64_t>(p.nticket, g);
  if (gated)
    hipLaunchKernelGGL((scan_kernel<ST, HD, kScanRowsPerThread, true>), dim3(grid),
                       dim3(kScanThreads), 0, st, q);
  else
    hipLaunchKernelGGL((scan_kernel<ST, HD, kScanRowsPerThread, false>), dim3(grid),
                       dim3(kScanThreads), 0, st, q);
  return (int)hipGetLastError();
}

}  // namespace

int scan_rows_per_chunk(int dtype, int hd) {
  const int vec = dtype == RAT_DTYPE_BF16 ? 8 : 4;
  const int lpr = hd / vec;
  return (kScanThreads / lpr) * kScanRowsPerThread;
}

template <typename ST, int HD>
int launch_ring_carry_t(int B, int H, int64_t WS, const HeadTables& ht, int64_t t0, int64_t T,
                        const void* kin, const void* vin, void* kout, void* vout, hipStream_t st) {
  constexpr int CPR = HD / StTraits<ST>::VEC;
  int64_t wmax = 0;
  for (int h = 0; h < H; ++h) wmax = std::max<int64_t>(wmax, ht.W[h]);
  if (wmax == 0 || t0 == 0 || B == 0 || H == 0) return 0;
  const dim3 grid((unsigned)((wmax * CPR + 255) / 256), (unsigned)H, (unsigned)B);
  hipLaunchKernelGGL((ring_carry_kernel<ST, HD>), grid, dim3(256), 0, st,
                     reinterpret_cast<const ST*>(kin), reinterpret_cast<const ST*>(vin),
                     reinterpret_cast<ST*>(kout), reinterpret_cast<ST*>(vout), ht, WS, t0, T);
  return (int)hipGetLastError();
}

int launch_ring_carry(int dtype, int hd, int B, int H, int64_t WS, const HeadTables& ht,
                      int64_t t0, int64_t T, const void* kr_in, const void* vr_in, void* kr_out,
                      void* vr_out, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16)
    return hd == 128 ? launch_ring_carry_t<bf16, 128>(B, H, WS, ht, t0, T, kr_in, vr_in, kr_out, vr_out, st)
                     : launch_ring_carry_t<bf16, 64>(B, H, WS, ht, t0, T, kr_in, vr_in, kr_out, vr_out, st);
  return hd == 128 ? launch_ring_carry_t<float, 128>(B, H, WS, ht, t0, T, kr_in, vr_in, kr_out, vr_out, st)
                   : launch_ring_carry_t<float, 64>(B, H, WS, ht, t0, T, kr_in, vr_in, kr_out, vr_out, st);
}

int launch_scan(int dtype, int hd, const ScanParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) {
    return hd == 128 ? launch_scan_t<bf16, 128>(p, st) : launch_scan_t<bf16, 64>(p, st);
  }
  return hd == 128 ? launch_scan_t<float, 128>(p, st) : launch_scan_t<float, 64>(p, st);
}

}  // namespace rat
