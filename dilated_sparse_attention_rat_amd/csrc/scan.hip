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
//  * chunks are handed out by an atomic ticket in sequence-interleaved
//    order, so every node a block waits on belongs to a block already
//    running (no deadlock); every wait is bounded;
//  * the second pass re-runs the sequential recurrence from the chunk's
//    carry-in on the registers and streams hk/hv, anchor rows, ring slots
//    and the final fp32 state out with 16-byte stores.
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

// Publish one aggregate-tree node: data with coherent stores, then the tag.
template <int HD, int CPL>
__device__ __forceinline__ void publish_node(const ScanParams& p, int64_t e, const float* A,
                                             const float* Bk, const float* Bv, uint32_t tag,
                                             int lane) {
  float* d = p.agg + e * 3 * HD;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    st_coherent_f32(d + c, A[j]);
    st_coherent_f32(d + HD + c, Bk[j]);
    st_coherent_f32(d + 2 * HD + c, Bv[j]);
  }
  vm_drain();
  if (lane == 0) st_relaxed_u32(p.flags + e, tag);
}

// Compose the n (< radix) consecutive nodes [e0, e0 + n), in order, after
// the running map (A, Bk, Bv).  Lane j polls node e0 + j; every wait is
// bounded.  All n aggregates are then loaded at once.
template <int HD, int CPL>
__device__ __forceinline__ void fold_nodes(const ScanParams& p, int64_t e0, int n, float* A,
                                           float* Bk, float* Bv, uint32_t tag, int lane) {
  if (n <= 0) return;
  bool ready = lane >= n;
  uint32_t spins = 0;
  while (true) {
    if (!ready) ready = ld_acquire_u32(p.flags + e0 + lane) == tag;
    if (__all(ready)) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) st_relaxed_u32(p.hdr + 2, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  vm_drain();
  float a[kScanRadix - 1][CPL], bk[kScanRadix - 1][CPL], bv[kScanRadix - 1][CPL];
#pragma unroll
  for (int i = 0; i < kScanRadix - 1; ++i) {
    if (i < n) {
      const float* d = p.agg + (e0 + i) * 3 * HD;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        a[i][j] = ld_coherent_f32(d + c);
        bk[i][j] = ld_coherent_f32(d + HD + c);
        bv[i][j] = ld_coherent_f32(d + 2 * HD + c);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kScanRadix - 1; ++i) {
    if (i < n) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        Bk[j] = a[i][j] * Bk[j] + bk[i][j];
        Bv[j] = a[i][j] * Bv[j] + bv[i][j];
        A[j] = A[j] * a[i][j];
      }
    }
  }
}

template <typename ST, int HD, int S>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const ScanParams p) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;           // lanes per row
  constexpr int RG = kScanThreads / LPR;  // row-groups per chunk
  constexpr int LC = RG * S;              // rows per chunk
  constexpr int CPL = HD / 64;            // channels per lane in the carry wave
  static_assert(HD % 64 == 0 && LPR <= 64, "layout");

  __shared__ float s_A[RG][HD];
  __shared__ float s_Bk[RG][HD];
  __shared__ float s_Bv[RG][HD];
  __shared__ float s_hk[HD];
  __shared__ float s_hv[HD];
  __shared__ uint32_t s_ticket, s_tag;

  // Tickets: blocks are split into nclass classes by blockIdx; class x owns
  // the sequences s = x (mod nclass) and hands out their chunks in
  // chunk-major order through its own counter.  A chunk only waits on
  // earlier chunks of its own sequence, i.e. on smaller tickets of its own
  // class, which blocks already running hold: no deadlock.  Every block reads
  // the class epoch before taking its ticket, so the block that takes the
  // class's last ticket can reset the counter and advance the epoch (the
  // next launch's tag) without any further atomic.
  const int tid = threadIdx.x;
  const int cls = (int)(blockIdx.x % (unsigned)p.nclass);
  uint32_t* slot = p.hdr + cls * kScanClassStride;
  const uint32_t per_class = (uint32_t)(p.nticket / p.nclass);
  if (tid == 0) {
    const uint32_t ep = ld_acquire_u32(slot + 1);
    vm_drain();
    const uint32_t tk = __hip_atomic_fetch_add(slot, 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    if (tk == per_class - 1) {
      st_relaxed_u32(slot, 0u);
      st_relaxed_u32(slot + 1, ep + 1u);
    }
    s_ticket = tk;
    s_tag = (ep % 0x3FFFFFFFu) + 1u;
  }
  __syncthreads();
  const uint32_t ticket = s_ticket;
  const uint32_t tag = s_tag;
  const bool valid_ticket = ticket < per_class;
  const int nseq_c = p.nseq / p.nclass;  // sequences of this class

  const int chunk = valid_ticket ? (int)(ticket / (uint32_t)nseq_c) : 0;
  const int seq = valid_ticket ? cls + p.nclass * (int)(ticket % (uint32_t)nseq_c) : 0;
  const int b = seq / p.H;
  const int h = seq - b * p.H;
  const int T = p.T;
  const int r = tid / LPR;
  const int cl = tid - r * LPR;
  const int c0 = cl * VEC;
  const int tbase = chunk * LC + r * S;
  const int64_t seq_base = (int64_t)seq * T * HD;

  const ST* __restrict__ kp = reinterpret_cast<const ST*>(p.k);
  const ST* __restrict__ vp = reinterpret_cast<const ST*>(p.v);
  const ST* __restrict__ gp = reinterpret_cast<const ST*>(p.g);

  // ---- issue the loads of this lane's S rows (kept for both passes) ------
  u32x4 rk[S], rv[S], rg[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = tbase + s;
    if (valid_ticket && t < T) {
      const int64_t off = seq_base + (int64_t)t * HD + c0;
      rk[s] = ld_raw16_nt(kp + off);
      rv[s] = ld_raw16_nt(vp + off);
      rg[s] = ld_raw16_nt(gp + off);
    }
  }

  // ---- pass 1: affine map of this lane's rows ----------------------------
  float A[VEC], Bk[VEC], Bv[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    A[i] = 1.f;
    Bk[i] = 0.f;
    Bv[i] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = tbase + s;
    if (valid_ticket && t < T) {
      float gf[VEC], kf[VEC], vf[VEC];
      unpack16(rg[s], gf, (ST*)nullptr);
      unpack16(rk[s], kf, (ST*)nullptr);
      unpack16(rv[s], vf, (ST*)nullptr);
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
    s_A[r][c0 + i] = A[i];
    s_Bk[r][c0 + i] = Bk[i];
    s_Bv[r][c0 + i] = Bv[i];
  }
  __syncthreads();

  // ---- wave 0: row-group scan, publish the chunk and completed parents ---
  if (tid < 64) {
    const int lane = tid;
    float cA[CPL], cBk[CPL], cBv[CPL];  // chunk aggregate per channel
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      float ra = 1.f, rbk = 0.f, rbv = 0.f;
      for (int rr = 0; rr < RG; ++rr) {
        const float a = s_A[rr][c], bk = s_Bk[rr][c], bv = s_Bv[rr][c];
        s_A[rr][c] = ra;  // exclusive prefix of the row-groups
        s_Bk[rr][c] = rbk;
        s_Bv[rr][c] = rbv;
        rbk = a * rbk + bk;
        rbv = a * rbv + bv;
        ra = ra * a;
      }
      cA[j] = ra;
      cBk[j] = rbk;
      cBv[j] = rbv;
    }
    if (valid_ticket) {
      // A node of level l+1 is the in-order composition of its radix
      // children; the chunk that owns the last child computes and publishes
      // it.
      int64_t node = chunk;
      for (int lv = 0; lv < p.nlevels; ++lv) {
        const int64_t lvl0 = p.lbase[lv] + (int64_t)seq * p.nodes[lv];
        publish_node<HD, CPL>(p, lvl0 + node, cA, cBk, cBv, tag, lane);
        if (lv + 1 >= p.nlevels || (node % kScanRadix) != kScanRadix - 1) break;
        float fA[CPL], fBk[CPL], fBv[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          fA[j] = 1.f;
          fBk[j] = 0.f;
          fBv[j] = 0.f;
        }
        fold_nodes<HD, CPL>(p, lvl0 + node - (kScanRadix - 1), kScanRadix - 1, fA, fBk, fBv, tag,
                            lane);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {  // then this node itself
          fBk[j] = cA[j] * fBk[j] + cBk[j];
          fBv[j] = cA[j] * fBv[j] + cBv[j];
          fA[j] = fA[j] * cA[j];
          cA[j] = fA[j];
          cBk[j] = fBk[j];
          cBv[j] = fBv[j];
        }
        node /= kScanRadix;
      }
    }
  }

  // ---- wave 1, concurrently: carry-in of this chunk ------------------------
  // Compose, top tree level first, the complete nodes that precede this
  // chunk (at most radix-1 per level).  The order is fixed, so the result is
  // bitwise deterministic.  Publication (wave 0) never waits on a carry, so
  // no chain forms along the sequence: every node depends on input data only.
  if (tid >= 64 && tid < 128) {
    const int lane = tid - 64;
    float one[CPL], hin_k[CPL], hin_v[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      one[j] = 1.f;
      hin_k[j] = 0.f;
      hin_v[j] = 0.f;
    }
    if (valid_ticket) {
      for (int lv = p.nlevels - 1; lv >= 0; --lv) {
        const int64_t nd = (int64_t)chunk >> (kScanRadixLog2 * lv);
        const int64_t first = nd & ~(int64_t)(kScanRadix - 1);
        const int64_t lvl0 = p.lbase[lv] + (int64_t)seq * p.nodes[lv];
        fold_nodes<HD, CPL>(p, lvl0 + first, (int)(nd - first), one, hin_k, hin_v, tag, lane);
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      s_hk[lane + 64 * j] = hin_k[j];
      s_hv[lane + 64 * j] = hin_v[j];
    }
  }
  __syncthreads();

  // ---- pass 2: sequential recurrence from the carry-in, stream outputs ---
  if (valid_ticket) {
    float sk[VEC], sv[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int c = c0 + i;
      sk[i] = s_A[r][c] * s_hk[c] + s_Bk[r][c];
      sv[i] = s_A[r][c] * s_hv[c] + s_Bv[r][c];
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
    int aq = tbase / D;             // anchor index candidate of row tbase
    int ar = tbase - aq * D;        // phase of row tbase
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = tbase + s;
      if (t < T) {
        float gf[VEC], kf[VEC], vf[VEC];
        unpack16(rg[s], gf, (ST*)nullptr);
        unpack16(rk[s], kf, (ST*)nullptr);
        unpack16(rv[s], vf, (ST*)nullptr);
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
          const int64_t off = (rrow0 + (t % W)) * HD + c0;
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

}

// T = 0: the state is h_{-1} = 0
__global__ void zero_state_kernel(float* sk, float* sv, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    sk[i] = 0.f;
    sv[i] = 0.f;
  }
}

template <typename ST, int HD>
int launch_scan_t(const ScanParams& p, hipStream_t st) {
  if (p.T == 0) {
    const int64_t n = (int64_t)p.nseq * HD;
    if (n == 0) return 0;
    hipLaunchKernelGGL(zero_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       p.sk, p.sv, n);
    return (int)hipGetLastError();
  }
  hipLaunchKernelGGL((scan_kernel<ST, HD, kScanRowsPerThread>), dim3(p.nticket),
                     dim3(kScanThreads), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace

int scan_rows_per_chunk(int dtype, int hd) {
  const int vec = dtype == RAT_DTYPE_BF16 ? 8 : 4;
  const int lpr = hd / vec;
  return (kScanThreads / lpr) * kScanRowsPerThread;
}

int launch_scan(int dtype, int hd, const ScanParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RAT_DTYPE_BF16) {
    return hd == 128 ? launch_scan_t<bf16, 128>(p, st) : launch_scan_t<bf16, 64>(p, st);
  }
  return hd == 128 ? launch_scan_t<float, 128>(p, st) : launch_scan_t<float, 64>(p, st);
}

}  // namespace rat
