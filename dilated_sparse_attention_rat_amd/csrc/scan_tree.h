// The chunk-aggregate tree that links the chunks of a persistent scan (the
// forward recurrence in csrc/scan.hip, the reverse one of the backward in
// csrc/backward.hip).
//
// Method: zhichai.net deep dive "RAT+ 深度拆解", section 2.1 -- the gated
// recurrence is a chain of affine maps x -> A*x + B per channel, so any run
// of consecutive positions composes into one such map and a prefix over
// chunks is a composition of chunk maps.
//
// Protocol (workspace: a header of kScanHeaderBytes, then 3*hd 64-bit words
// per tree entry):
//  * a chunk publishes its map as level-0 node; the chunk that owns the last
//    of 8 children composes and publishes their parent (level l+1);
//  * a chunk's carry is the in-order composition of at most 7 complete nodes
//    per level that precede it, top level first (a fixed order: bitwise
//    deterministic results);
//  * every value is a 64-bit word (launch tag << 32 | fp32 bits) written and
//    read with single-copy atomic accesses at agent scope, so a reader that
//    sees the current tag also sees the value: no flag, no fence;
//  * the tag is derived from the launch epoch in the header, which the last
//    workgroup to retire advances, so entries of earlier launches (and a
//    zero-filled workspace) never look current;
//  * every wait is bounded; a wait that runs out sets the header's error
//    word instead of hanging.
#pragma once

#include "rat_device.h"

namespace rat {

constexpr uint32_t kSpinLimit = 1u << 16;

// Header words (uint32): the launch epoch, the error flag, and the done
// counters that let the last block advance the epoch.  Counters sit 256
// bytes apart so their atomics do not queue on one address.
constexpr int kEpochWord = 0;
constexpr int kErrorWord = 2;
constexpr int kTopWord = 32;
constexpr int kDoneBase = 64;
constexpr int kDoneStride = 64;
constexpr int kDoneSlots = 64;
static_assert(kDoneBase + kDoneSlots * kDoneStride <= kScanHeaderBytes / 4, "header");

constexpr int kScanRadixLog2 = 3;
static_assert((1 << kScanRadixLog2) == kScanRadix, "radix");

__device__ __forceinline__ uint32_t ld_acquire_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's earlier global accesses have completed.  Every
// workspace access of the tree is a coherent (agent-scope) atomic access, so
// completion order is all the publication protocol needs: data stores
// complete before the tag store is issued, and data loads are issued only
// after the tag load has returned.  No cache write-back or invalidation is
// required (an agent-scope fence would write back / invalidate the whole L2
// of the XCD on every call).
__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void st_tagged(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The launch tag of an epoch (never 0, the value of a zero-filled entry).
__device__ __forceinline__ uint32_t tree_tag(uint32_t epoch) { return (epoch % 0x3FFFFFFFu) + 1u; }

// The hd channels are independent; the tree works on 64-channel halves, one
// wave per half with one channel per lane.  Publish one half of node e (A,
// Bk, Bv of this lane's channel).
template <int HD>
__device__ __forceinline__ void publish_node(uint64_t* agg, int64_t e, int half, float A,
                                             float Bk, float Bv, uint32_t tag, int lane) {
  uint64_t* d = agg + e * 3 * HD + 64 * half + lane;
  st_tagged(d, tag, A);
  st_tagged(d + HD, tag, Bk);
  st_tagged(d + 2 * HD, tag, Bv);
}

// Compose the n (< radix) consecutive nodes [e0, e0 + n), in order, after
// the running map (A, Bk, Bv) of one channel.  All 3n words are loaded at
// once and re-loaded until every tag in the wave is current; every wait is
// bounded.
template <int HD>
__device__ __forceinline__ void fold_nodes(const uint64_t* agg, uint32_t* hdr, int64_t e0, int n,
                                           int half, float& A, float& Bk, float& Bv, uint32_t tag,
                                           int lane) {
  if (n <= 0) return;
  uint64_t w[kScanRadix - 1][3];
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < kScanRadix - 1; ++i) {
      if (i < n) {
        const uint64_t* d = agg + (e0 + i) * 3 * HD + 64 * half + lane;
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
      if (lane == 0) st_relaxed_u32(hdr + kErrorWord, 1u);
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

// Publish a chunk's map (ra, rbk, rbv) as node `node` of level 0 and, while
// it owns the last child, the parents above it.  lbase/nodes: first entry
// and nodes per sequence of each level.
template <int HD>
__device__ __forceinline__ void tree_publish(uint64_t* agg, uint32_t* hdr, int nlevels,
                                             const int64_t* lbase, const int* nodes, int seq,
                                             int64_t node, int half, float ra, float rbk,
                                             float rbv, uint32_t tag, int lane) {
  for (int lv = 0; lv < nlevels; ++lv) {
    const int64_t lvl0 = lbase[lv] + (int64_t)seq * nodes[lv];
    publish_node<HD>(agg, lvl0 + node, half, ra, rbk, rbv, tag, lane);
    if (lv + 1 >= nlevels || (node % kScanRadix) != kScanRadix - 1) break;
    float fA = 1.f, fBk = 0.f, fBv = 0.f;
    fold_nodes<HD>(agg, hdr, lvl0 + node - (kScanRadix - 1), kScanRadix - 1, half, fA, fBk, fBv,
                   tag, lane);
    rbk = ra * fBk + rbk;  // then this node itself
    rbv = ra * fBv + rbv;
    ra = fA * ra;
    node /= kScanRadix;
  }
}

// Compose the complete nodes that precede chunk `chunk`, top level first,
// onto (A, Bk, Bv).
template <int HD>
__device__ __forceinline__ void tree_carry(const uint64_t* agg, uint32_t* hdr, int nlevels,
                                           const int64_t* lbase, const int* nodes, int seq,
                                           int64_t chunk, int half, float& A, float& Bk,
                                           float& Bv, uint32_t tag, int lane) {
  for (int lv = nlevels - 1; lv >= 0; --lv) {
    const int64_t nd = chunk >> (kScanRadixLog2 * lv);
    const int64_t first = nd & ~(int64_t)(kScanRadix - 1);
    const int64_t lvl0 = lbase[lv] + (int64_t)seq * nodes[lv];
    fold_nodes<HD>(agg, hdr, lvl0 + first, (int)(nd - first), half, A, Bk, Bv, tag, lane);
  }
}

// Retire a workgroup (thread 0 only): two-level done count; the last
// workgroup of the launch advances the epoch.
__device__ __forceinline__ void tree_retire(uint32_t* hdr, uint32_t epoch) {
  const uint32_t G = gridDim.x;
  const uint32_t slot = blockIdx.x % kDoneSlots;
  const uint32_t in_slot = (G - 1 - slot) / kDoneSlots + 1;
  const uint32_t used = G < (uint32_t)kDoneSlots ? G : (uint32_t)kDoneSlots;
  vm_drain();
  uint32_t* ctr = hdr + kDoneBase + slot * kDoneStride;
  if (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == in_slot - 1) {
    st_relaxed_u32(ctr, 0u);
    uint32_t* top = hdr + kTopWord;
    if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == used - 1) {
      st_relaxed_u32(top, 0u);
      st_relaxed_u32(hdr + kEpochWord, epoch + 1u);
    }
  }
}

}  // namespace rat
