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

#include "scan_tree.h"

namespace rat {

namespace {

template <typename ST, int HD, int S>
struct ChunkRows {
  u32x4 k[S], v[S], g[S];
  f32x4 gb[StTraits<ST>::VEC / 4];  // gate bias of the lane's channels (gated variant)
};

// Issue the loads of this lane's S rows of chunk `ticket` (kept in registers
// for both passes).  The loads are unconditional (rows at or past T re-read
// row T-1 and are ignored) so the compiler can count outstanding loads
// exactly and wait only for the ones it needs.
template <typename ST, int HD, int S, bool GATE>
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
  // the gate bias rides with the rows: loaded at the chunk's start instead,
  // it would be ordered behind the previous chunk's output stores (vector
  // memory completes in order) and hold up pass 1 until they drain
  if constexpr (GATE) {
    const float* gbp = p.gate_bias + (int64_t)(seq - b * p.H) * HD + c0;
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) rw.gb[j] = *reinterpret_cast<const f32x4*>(gbp + 4 * j);
  }
}

// One chunk: pass 1, tree publication and carry, then pass 2.  `between`
// runs after the carry is known and before pass 2: the caller issues the
// next chunk's loads there, so that no tree load waits behind them (vector
// memory counters complete in order) while pass 2 still overlaps them.
template <typename ST, int HD, int S, bool GATE, typename F>
__device__ __forceinline__ void scan_chunk(const ScanParams& p, uint32_t ticket, uint32_t tag,
                                           const ChunkRows<ST, HD, S>& rw, float (*s_A)[HD],
                                           float (*s_Bk)[HD], float (*s_Bv)[HD], float* s_hk,
                                           float* s_hv, F&& between) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;           // lanes per row
  constexpr int RG = kScanThreads / LPR;  // row-groups per chunk
  constexpr int LC = RG * S;              // rows per chunk
  const int tid = threadIdx.x;
  const int chunk = (int)(ticket / (uint32_t)p.nseq);
  const int seq = (int)(ticket % (uint32_t)p.nseq);
  const int b = seq / p.H;
  const int h = seq - b * p.H;
  const int T = p.T;
  const int r = tid / LPR;
  const int cl = tid - r * LPR;
  const int c0 = cl * VEC;
  const int tbase = chunk * LC + r * S;
  const int64_t seq_base = (int64_t)seq * T * HD;
  const u32x4* rk = rw.k;
  const u32x4* rv = rw.v;
  const u32x4* rg = rw.g;
  // GATE: g holds the gate's pre-activation; the gate is sigmoid(g + bias)
  // with the head's per-channel bias (fused here instead of a separate pass)
  auto gate = [&](float (&gf)[VEC]) {
    if constexpr (GATE) {
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        gf[i] = __builtin_amdgcn_rcpf(
            1.f + __builtin_amdgcn_exp2f(-(gf[i] + rw.gb[i / 4][i % 4]) * kLog2e));
    }
  };

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
    if (t < T) {
      float gf[VEC], kf[VEC], vf[VEC];
      unpack16(rg[s], gf, (ST*)nullptr);
      gate(gf);
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

  // ---- waves 0..NH-1: row-group scan of half j, publish chunk and parents -
  // ---- waves 2..2+NH-1, concurrently: carry-in of half j -------------------
  // Publication never waits on a carry, so no chain forms along the
  // sequence: every tree node depends on input data only.  The carry is the
  // in-order composition, top tree level first, of the complete nodes that
  // precede this chunk (at most radix-1 per level): a fixed order, so the
  // result is bitwise deterministic.
  {
    constexpr int NH = HD / 64;  // channel halves
    const int wave = tid >> 6;
    const int lane = tid & 63;
    if (wave < NH) {
      const int half = wave;
      const int c = 64 * half + lane;
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
      // A node of level l+1 is the in-order composition of its radix
      // children; the chunk that owns the last child computes and publishes
      // it.
      tree_publish<HD>(p.agg, p.hdr, p.nlevels, p.lbase, p.nodes, seq, chunk, half, ra, rbk, rbv,
                       tag, lane);
    } else if (wave >= 2 && wave < 2 + NH) {
      const int half = wave - 2;
      // the state before row 0: zero for a prefill, the given state for a
      // continuation; the nodes before this chunk are composed onto it
      float one = 1.f;
      float hin_k = p.sk_in != nullptr ? p.sk_in[(int64_t)seq * HD + 64 * half + lane] : 0.f;
      float hin_v = p.sv_in != nullptr ? p.sv_in[(int64_t)seq * HD + 64 * half + lane] : 0.f;
      tree_carry<HD>(p.agg, p.hdr, p.nlevels, p.lbase, p.nodes, seq, chunk, half, one, hin_k,
                     hin_v, tag, lane);
      s_hk[64 * half + lane] = hin_k;
      s_hv[64 * half + lane] = hin_v;
    }
  }
  __syncthreads();
  between();

  // ---- pass 2: sequential recurrence from the carry-in, stream outputs ---
  {
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
    const int tabs = p.t0 + tbase;  // absolute position of row tbase
    int aq = tabs / D;              // anchor index candidate of row tbase
    int ar = tabs - aq * D;         // phase of row tbase
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = tbase + s;
      if (t < T) {
        float gf[VEC], kf[VEC], vf[VEC];
        unpack16(rg[s], gf, (ST*)nullptr);
        gate(gf);
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

}

// Persistent kernel: the grid is sized to the number of workgroups that can
// be resident at once, so every workgroup runs concurrently.  Workgroup w processes tickets w, w + G, w + 2G, ... in
// order; ticket t is chunk t / nseq of sequence t % nseq.  A chunk waits only
// on nodes of earlier chunks of its own sequence, i.e. on smaller tickets, so
// the smallest unfinished ticket can always proceed (no deadlock), and no
// ticket counter (atomic) is needed.  Every workgroup reads the epoch first;
// the last one to finish advances it, so the epoch is this launch's tag.
template <typename ST, int HD, int S, bool GATE>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void scan_kernel(const ScanParams p) {
  constexpr int VEC = StTraits<ST>::VEC;
  constexpr int LPR = HD / VEC;
  constexpr int RG = kScanThreads / LPR;
  static_assert(HD % 64 == 0 && LPR <= 64, "layout");
  __shared__ float s_A[RG][HD];
  __shared__ float s_Bk[RG][HD];
  __shared__ float s_Bv[RG][HD];
  __shared__ float s_hk[HD];
  __shared__ float s_hv[HD];
  __shared__ uint32_t s_epoch;

  const int tid = threadIdx.x;
  if (tid == 0) s_epoch = ld_acquire_u32(p.hdr + kEpochWord);
  __syncthreads();
  const uint32_t epoch = s_epoch;
  const uint32_t tag = tree_tag(epoch);
  const uint32_t G = gridDim.x;

  // Two register buffers: the rows of the next chunk are loaded while the
  // current chunk streams its outputs.
  const uint32_t n = (uint32_t)p.nticket;
  ChunkRows<ST, HD, S> ra, rb;
  uint32_t ticket = blockIdx.x;
  if (ticket < n) load_rows<ST, HD, S, GATE>(p, ticket, ra);
  while (ticket < n) {
    const uint32_t t1 = ticket + G;
    // (prefetches are unconditional -- past the end they re-load the last
    // ticket and are ignored -- so outstanding loads are counted exactly)
    scan_chunk<ST, HD, S, GATE>(p, ticket, tag, ra, s_A, s_Bk, s_Bv, s_hk, s_hv,
                          [&] { load_rows<ST, HD, S, GATE>(p, min(t1, n - 1), rb); });
    __syncthreads();  // LDS is reused by the next chunk
    if (t1 >= n) break;
    const uint32_t t2 = t1 + G;
    scan_chunk<ST, HD, S, GATE>(p, t1, tag, rb, s_A, s_Bk, s_Bv, s_hk, s_hv,
                          [&] { load_rows<ST, HD, S, GATE>(p, min(t2, n - 1), ra); });
    __syncthreads();
    ticket = t2;
  }

  // retire: the last workgroup advances the epoch
  if (tid == 0) tree_retire(p.hdr, epoch);
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
  const unsigned grid = (unsigned)std::min<int64_t>(p.nticket, lim);
  if (gated)
    hipLaunchKernelGGL((scan_kernel<ST, HD, kScanRowsPerThread, true>), dim3(grid),
                       dim3(kScanThreads), 0, st, p);
  else
    hipLaunchKernelGGL((scan_kernel<ST, HD, kScanRowsPerThread, false>), dim3(grid),
                       dim3(kScanThreads), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace

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
  // a chunk at least as long as every window rewrites every live slot itself
  if (wmax == 0 || t0 == 0 || B == 0 || H == 0 || T >= wmax) return 0;
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
