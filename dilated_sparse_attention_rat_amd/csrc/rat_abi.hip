// C-ABI layer of the RAT+ hot path: host-side validation, per-head offset
// tables (anchor cache and window ring), launch configuration, and the
// launches on the caller's stream.  No allocation, no synchronisation, no
// global mutable state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include <mutex>

#include "rat.h"
#include "rat_params.h"

using namespace rat;

namespace {

constexpr int64_t kMaxT = (int64_t)1 << 30;  // positions are int32 in kernels

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int dtype, int B, int H, int hd, const int32_t* D, const int32_t* W) {
  if (B < 0 || H < 0 || D == nullptr || W == nullptr) return RAT_ERR_INVALID_ARG;
  if (H > RAT_MAX_HEADS) return RAT_ERR_UNSUPPORTED;
  if (dtype != RAT_DTYPE_BF16 && dtype != RAT_DTYPE_F32) return RAT_ERR_UNSUPPORTED;
  if (hd != 64 && hd != 128) return RAT_ERR_UNSUPPORTED;
  for (int h = 0; h < H; ++h) {
    if (D[h] < 1 || W[h] < 0) return RAT_ERR_INVALID_ARG;
    if ((int64_t)W[h] > kMaxT) return RAT_ERR_INVALID_ARG;
  }
  return RAT_OK;
}

// Fills the per-head tables; returns RAT_OK or an error if an offset does
// not fit the kernels' 32-bit row indices.
int fill_tables(int H, int64_t T_cap, const int32_t* D, const int32_t* W, HeadTables& ht,
                int64_t& R, int64_t& WS) {
  std::memset(&ht, 0, sizeof(ht));
  R = 0;
  WS = 0;
  for (int h = 0; h < H; ++h) {
    ht.D[h] = D[h];
    ht.W[h] = W[h];
    ht.aoff[h] = (int32_t)R;
    ht.roff[h] = (int32_t)WS;
    R += T_cap / D[h];
    WS += W[h];
    if (R > INT32_MAX || WS > INT32_MAX) return RAT_ERR_UNSUPPORTED;
  }
  return RAT_OK;
}

int map_hip(int e) { return e == 0 ? RAT_OK : RAT_ERR_HIP; }

// Workspace of the scan: header, then per tree node an aggregate (A, Bk, Bv:
// 3*hd values, each a 64-bit tagged word).  Level l has ceil(nchunk / 8^l) nodes per
// sequence; levels are added until the top one has at most 8 nodes.
struct ScanLayout {
  int64_t nchunk = 0, nticket = 0, entries = 0;
  int nlevels = 0;
  int nodes[kScanMaxLevels] = {};
  int64_t lbase[kScanMaxLevels] = {};
  int64_t agg_off = 0, bytes = 0;
};

bool scan_layout(int B, int H, int64_t T, int hd, int dtype, ScanLayout& L) {
  const int lc = scan_rows_per_chunk(dtype, hd);
  L.nchunk = (T + lc - 1) / lc;
  L.nticket = (int64_t)B * H * L.nchunk;
  int64_t n = std::max<int64_t>(L.nchunk, 1);
  L.nlevels = 0;
  L.entries = 0;
  while (true) {
    if (L.nlevels >= kScanMaxLevels) return false;
    L.nodes[L.nlevels] = (int)n;
    L.lbase[L.nlevels] = L.entries;
    L.entries += (int64_t)B * H * n;
    ++L.nlevels;
    if (n <= kScanRadix) break;
    n = (n + kScanRadix - 1) / kScanRadix;
  }
  auto up = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  L.agg_off = kScanHeaderBytes;
  L.bytes = up(L.agg_off + L.entries * 3 * hd * 8);
  return true;
}

}  // namespace

extern "C" {

const char* rat_version(void) { return "rat-mi355x 0.1.0 (gfx950)"; }

const char* rat_status_string(int status) {
  switch (status) {
    case RAT_OK: return "ok";
    case RAT_ERR_INVALID_ARG: return "invalid argument";
    case RAT_ERR_UNSUPPORTED: return "unsupported configuration (dtype, head dim or size)";
    case RAT_ERR_CAPACITY: return "position beyond the cache capacity T_cap";
    case RAT_ERR_WORKSPACE: return "workspace missing or too small";
    case RAT_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int64_t rat_anchor_rows(int H, int64_t T_cap, const int32_t* D, int64_t* offsets_out) {
  if (H < 0 || T_cap < 0 || (H > 0 && D == nullptr)) return RAT_ERR_INVALID_ARG;
  int64_t r = 0;
  for (int h = 0; h < H; ++h) {
    if (D[h] < 1) return RAT_ERR_INVALID_ARG;
    if (offsets_out) offsets_out[h] = r;
    r += T_cap / D[h];
  }
  if (offsets_out) offsets_out[H] = r;
  return r;
}

int64_t rat_ring_rows(int H, const int32_t* W, int64_t* offsets_out) {
  if (H < 0 || (H > 0 && W == nullptr)) return RAT_ERR_INVALID_ARG;
  int64_t r = 0;
  for (int h = 0; h < H; ++h) {
    if (W[h] < 0) return RAT_ERR_INVALID_ARG;
    if (offsets_out) offsets_out[h] = r;
    r += W[h];
  }
  if (offsets_out) offsets_out[H] = r;
  return r;
}

int64_t rat_scan_workspace_bytes(int B, int H, int64_t T, int hd) {
  if (B < 0 || H < 0 || T < 0 || T > kMaxT) return RAT_ERR_INVALID_ARG;
  if (hd != 64 && hd != 128) return RAT_ERR_UNSUPPORTED;
  // the chunk length depends on the storage type; size for the larger of the
  // two layouts so one workspace serves both
  ScanLayout a, b;
  if (!scan_layout(B, H, T, hd, RAT_DTYPE_BF16, a) || !scan_layout(B, H, T, hd, RAT_DTYPE_F32, b))
    return RAT_ERR_UNSUPPORTED;
  return std::max(a.bytes, b.bytes);
}

namespace {
// Scan of rows [0, T) at absolute positions t0 .. t0+T-1, from the state
// (sk_in, sv_in) before row 0 (null: zero).  kr_in/vr_in: the ring before the
// call (continuation; null or equal to the output ring: no carry copy).
int scan_impl(int dtype, int B, int H, int64_t T, int hd, const int32_t* D, const int32_t* W,
              int64_t T_cap, int64_t t0, const void* k, const void* v, const void* g,
              const float* sk_in, const float* sv_in, void* hk, void* hv, void* Kc, void* Vc,
              const void* kr_in, const void* vr_in, void* k_ring, void* v_ring, float* state_k,
              float* state_v, void* workspace, size_t workspace_bytes, void* stream,
              const float* gate_bias = nullptr, bool in_tok = false) {
  int st = check_common(dtype, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  if (T < 0 || t0 < 0 || T_cap > kMaxT) return RAT_ERR_INVALID_ARG;
  if (t0 + T > T_cap) return RAT_ERR_CAPACITY;
  if (B == 0 || H == 0) return RAT_OK;
  ScanParams p;
  std::memset(&p, 0, sizeof(p));
  st = fill_tables(H, T_cap, D, W, p.ht, p.R, p.WS);
  if (st != RAT_OK) return st;
  if (state_k == nullptr || state_v == nullptr || !aligned16(state_k) || !aligned16(state_v))
    return RAT_ERR_INVALID_ARG;
  if ((sk_in == nullptr) != (sv_in == nullptr)) return RAT_ERR_INVALID_ARG;
  if (sk_in && (!aligned16(sk_in) || !aligned16(sv_in) || sk_in == state_k || sv_in == state_v ||
                sk_in == state_v || sv_in == state_k))
    return RAT_ERR_INVALID_ARG;  // the input state is read while the output is written
  if (p.WS > 0 && (!k_ring || !v_ring || !aligned16(k_ring) || !aligned16(v_ring)))
    return RAT_ERR_INVALID_ARG;
  if ((kr_in == nullptr) != (vr_in == nullptr)) return RAT_ERR_INVALID_ARG;
  if (kr_in && (!aligned16(kr_in) || !aligned16(vr_in))) return RAT_ERR_INVALID_ARG;
  if (T > 0) {
    if (!k || !v || !g || !aligned16(k) || !aligned16(v) || !aligned16(g)) return RAT_ERR_INVALID_ARG;
    if ((hk == nullptr) != (hv == nullptr)) return RAT_ERR_INVALID_ARG;
    if (hk && (!aligned16(hk) || !aligned16(hv))) return RAT_ERR_INVALID_ARG;
    if (p.R > 0 && (!Kc || !Vc || !aligned16(Kc) || !aligned16(Vc))) return RAT_ERR_INVALID_ARG;
    ScanLayout L;
    if (!scan_layout(B, H, T, hd, dtype, L)) return RAT_ERR_UNSUPPORTED;
    if (workspace == nullptr || !aligned16(workspace) || (int64_t)workspace_bytes < L.bytes)
      return RAT_ERR_WORKSPACE;
    if (L.nticket > INT32_MAX) return RAT_ERR_UNSUPPORTED;
    char* ws = static_cast<char*>(workspace);
    p.hdr = reinterpret_cast<uint32_t*>(ws);
    p.agg = reinterpret_cast<uint64_t*>(ws + L.agg_off);
    p.nticket = (int)L.nticket;
    p.nchunk = (int)L.nchunk;
    p.nlevels = L.nlevels;
    for (int l = 0; l < L.nlevels; ++l) {
      p.nodes[l] = L.nodes[l];
      p.lbase[l] = L.lbase[l];
    }
  }
  p.B = B;
  p.H = H;
  p.T = (int)T;
  p.t0 = (int)t0;
  p.nseq = B * H;
  p.k = k;
  p.v = v;
  p.g = g;
  p.hk = hk;
  p.hv = hv;
  p.Kc = Kc;
  p.Vc = Vc;
  p.kr = k_ring;
  p.vr = v_ring;
  p.sk = state_k;
  p.sv = state_v;
  p.sk_in = sk_in;
  p.sv_in = sv_in;
  p.gate_bias = gate_bias;
  // k, v, g: [B,H,T,hd], or token-major [B,T,H,hd] (in_tok)
  p.in_sb = (int64_t)H * T * hd;
  p.in_sh = in_tok ? hd : T * hd;
  p.in_st = in_tok ? (int64_t)H * hd : hd;
  if (p.WS > 0 && t0 > 0 && kr_in != nullptr && kr_in != k_ring) {
    // window positions before t0 that stay in the window: previous ring ->
    // new ring (disjoint from the slots the scan writes)
    st = map_hip(launch_ring_carry(dtype, hd, B, H, p.WS, p.ht, t0, T, kr_in, vr_in, k_ring,
                                   v_ring, stream));
    if (st != RAT_OK) return st;
  }
  return map_hip(launch_scan(dtype, hd, p, stream));
}
}  // namespace

int rat_scan_prefill(int dtype, int B, int H, int64_t T, int hd, const int32_t* D,
                     const int32_t* W, int64_t T_cap, const void* k, const void* v, const void* g,
                     void* hk, void* hv, void* Kc, void* Vc, void* k_ring, void* v_ring,
                     float* state_k, float* state_v, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return scan_impl(dtype, B, H, T, hd, D, W, T_cap, 0, k, v, g, nullptr, nullptr, hk, hv, Kc, Vc,
                   nullptr, nullptr, k_ring, v_ring, state_k, state_v, workspace, workspace_bytes,
                   stream);
}

int rat_scan_prefill_continue(int dtype, int B, int H, int64_t T, int hd, const int32_t* D,
                              const int32_t* W, int64_t T_cap, int64_t t0, const void* k,
                              const void* v, const void* g, const float* state_k_in,
                              const float* state_v_in, void* hk, void* hv, void* Kc, void* Vc,
                              const void* k_ring_in, const void* v_ring_in, void* k_ring,
                              void* v_ring, float* state_k, float* state_v, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (state_k_in == nullptr || state_v_in == nullptr) return RAT_ERR_INVALID_ARG;
  return scan_impl(dtype, B, H, T, hd, D, W, T_cap, t0, k, v, g, state_k_in, state_v_in, hk, hv,
                   Kc, Vc, k_ring_in, v_ring_in, k_ring, v_ring, state_k, state_v, workspace,
                   workspace_bytes, stream);
}

namespace {
// Attention of queries [0, T) at absolute positions t0 .. t0+T-1.  Window
// keys before t0 come from (kr_prev, vr_prev), the ring as it was before the
// continuation's scan.
int attn_impl(int dtype, int B, int H, int64_t T, int hd, const int32_t* D, const int32_t* W,
              float scale, int64_t T_cap, int64_t t0, const void* q, const void* hk,
              const void* hv, const void* Kc, const void* Vc, const void* kr_prev,
              const void* vr_prev, void* o, float* lse, void* stream, bool o_tok = false,
              bool q_tok = false) {
  int st = check_common(dtype, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  if (T < 0 || t0 < 0 || T_cap > kMaxT) return RAT_ERR_INVALID_ARG;
  if (t0 + T > T_cap) return RAT_ERR_CAPACITY;
  if (!(scale <= 0.f) && !std::isfinite(scale)) return RAT_ERR_INVALID_ARG;
  if (B == 0 || H == 0 || T == 0) return RAT_OK;
  AttnParams p;
  std::memset(&p, 0, sizeof(p));
  int64_t WS;
  st = fill_tables(H, T_cap, D, W, p.ht, p.R, WS);
  if (st != RAT_OK) return st;
  if (!q || !hk || !hv || !o || !aligned16(q) || !aligned16(hk) || !aligned16(hv) || !aligned16(o))
    return RAT_ERR_INVALID_ARG;
  if (p.R > 0 && (!Kc || !Vc || !aligned16(Kc) || !aligned16(Vc))) return RAT_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return RAT_ERR_INVALID_ARG;
  if (t0 > 0 && WS > 0 && (!kr_prev || !vr_prev || !aligned16(kr_prev) || !aligned16(vr_prev)))
    return RAT_ERR_INVALID_ARG;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)hd);
  p.B = B;
  p.H = H;
  p.T = (int)T;
  p.t0 = (int)t0;
  // 16-query blocks per wave: 2 when the average query attends to 256 keys
  // or more (every staged K/V element then serves 32 queries of a wave, half
  // the LDS bytes per FLOP), else 1 (short key sets: fewer registers, more
  // waves in flight)
  const int64_t tmid = t0 + T / 2;
  double avg_keys = 0.0;
  for (int h = 0; h < H; ++h)
    avg_keys += (double)std::max<int64_t>(0, tmid - W[h]) / D[h] + std::min<int64_t>(W[h], tmid);
  avg_keys /= H;
  p.qb = avg_keys >= 256.0 ? 2 : 1;
  // resident-anchor kernel: bf16, no window, every head's anchors fit in LDS
  // (per-(b,h) output rows are addressed with 32-bit byte offsets there)
  bool resident = dtype == RAT_DTYPE_BF16 && T * (o_tok ? H : 1) * hd * 2 <= INT32_MAX;
  for (int h = 0; h < H && resident; ++h)
    resident = W[h] == 0 && (t0 + T - 1) / D[h] <= kResidentAnchors;
  if (resident) {
    // about one workgroup per CU, at least one query block per wave
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return RAT_ERR_HIP;
    const int64_t nbh = (int64_t)B * H;
    const int64_t nblk = (T + 16 * kResidentQB - 1) / (16 * kResidentQB);
    int64_t nra = (std::max(cus, 1) + nbh - 1) / nbh;
    nra = std::max<int64_t>(1, std::min<int64_t>(nra, (nblk + kResidentWaves - 1) / kResidentWaves));
    if (nbh * nra > INT32_MAX) return RAT_ERR_UNSUPPORTED;
    p.mode = 1;
    p.nra = (int)nra;
  }
  const int bm = 64 * p.qb;
  p.nq = (int)((T + bm - 1) / bm);
  p.np = (p.nq + 1) / 2;
  p.paired = 1;
  if (!resident) {
    // Pairs (i, nq-1-i) even out the causal staircase; when pairing would
    // leave fewer than two rounds of resident workgroups (a short chunk),
    // single tiles give twice the parallelism instead.
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return RAT_ERR_HIP;
    const int64_t slots = (int64_t)cus * (p.qb == 1 ? 3 : 2);  // resident workgroups
    // Where every head's window holds at least as many keys as its anchors
    // ever do, a tile's cost hardly grows along the sequence: single tiles,
    // so that neighbouring query tiles, which share band rows, run at the
    // same time and find them in L2.
    bool band_bound = true;
    for (int h = 0; h < H; ++h) band_bound = band_bound && (t0 + T) / D[h] <= W[h];
    if ((int64_t)B * H * p.np < 2 * slots || band_bound) {
      p.np = p.nq;
      p.paired = 0;
    }
  }
  // A paired launch dispatches the last quarter of its groups of 8 units as
  // single tiles, heaviest first, so that the last workgroups to start are
  // short ones (workload 4: 2 of 8 groups, 3% faster than none; 1 or 3
  // groups gained less).
  {
    const int64_t units = (int64_t)B * H;
    const int64_t nfull = units / 8;
    const int64_t gs = p.paired ? nfull - nfull / kAttnTailDiv : nfull;
    p.gsingle = (int)gs;
    p.nblk = gs * 8 * p.np + (nfull - gs) * 8 * p.nq + (units - 8 * nfull) * p.np;
  }
  if (p.nblk > INT32_MAX) return RAT_ERR_UNSUPPORTED;
  // K/V tiles straight into LDS (two stages, no staging registers) for the
  // streamed two-block kernel (a continuation whose window reaches into the
  // previous ring keeps register staging)
  p.dma = p.mode == 0 && dtype == RAT_DTYPE_BF16 && hd == 128 && p.qb == 2;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.q = q;
  p.q_sb = (int64_t)H * T * hd;
  p.q_sh = q_tok ? hd : T * hd;
  p.q_st = q_tok ? (int64_t)H * hd : hd;
  p.hk = hk;
  p.hv = hv;
  p.Kc = Kc;
  p.Vc = Vc;
  p.kr = kr_prev;
  p.vr = vr_prev;
  p.WS = WS;
  p.o = o;
  p.o_sb = o_tok ? T * H * hd : (int64_t)H * T * hd;
  p.o_sh = o_tok ? hd : T * hd;
  p.o_st = o_tok ? (int64_t)H * hd : hd;
  p.lse = lse;
  // heads in descending cost of one pair-block (anchor tiles + band tiles of
  // the heaviest and the lightest query tile), so heavy heads start first
  const int bn = kAttnBN;
  auto tiles = [&](int h, int qt) -> int64_t {
    const int64_t a0 = t0 + (int64_t)qt * bm;
    const int64_t tl = t0 + std::min<int64_t>((int64_t)qt * bm + bm - 1, T - 1);
    const int64_t na = std::max<int64_t>(0, tl - W[h]) / D[h];
    int64_t n = (na + bn - 1) / bn + 1;
    if (W[h] > 0) n += (tl - std::max<int64_t>(0, a0 - W[h]) + bn) / bn;
    return n;
  };
  int64_t cost[RAT_MAX_HEADS];
  for (int h = 0; h < H; ++h) {
    cost[h] = tiles(h, p.nq - 1) + (p.nq > 1 ? tiles(h, 0) : 0);
    p.perm[h] = h;
  }
  std::stable_sort(p.perm, p.perm + H, [&](int a, int b) { return cost[a] > cost[b]; });
  return map_hip(launch_attn_prefill(dtype, hd, p, stream));
}
}  // namespace

int rat_dilated_attn_prefill(int dtype, int B, int H, int64_t T, int hd, const int32_t* D,
                             const int32_t* W, float scale, int64_t T_cap, const void* q,
                             const void* hk, const void* hv, const void* Kc, const void* Vc,
                             void* o, float* lse, void* stream) {
  return attn_impl(dtype, B, H, T, hd, D, W, scale, T_cap, 0, q, hk, hv, Kc, Vc, nullptr, nullptr,
                   o, lse, stream);
}

int rat_dilated_attn_prefill_continue(int dtype, int B, int H, int64_t T, int hd,
                                      const int32_t* D, const int32_t* W, float scale,
                                      int64_t T_cap, int64_t t0, const void* q, const void* hk,
                                      const void* hv, const void* Kc, const void* Vc,
                                      const void* k_ring_prev, const void* v_ring_prev, void* o,
                                      float* lse, void* stream) {
  return attn_impl(dtype, B, H, T, hd, D, W, scale, T_cap, t0, q, hk, hv, Kc, Vc, k_ring_prev,
                   v_ring_prev, o, lse, stream);
}

namespace {
int decode_splits(int B, int H, int64_t T_cap, const int32_t* D, const int32_t* W, int requested) {
  if (requested > 0) return requested;
  int64_t maxk = 0;
  for (int h = 0; h < H; ++h) maxk = std::max<int64_t>(maxk, T_cap / D[h] + W[h]);
  const int64_t nbh = std::max<int64_t>(1, (int64_t)B * H);
  // aim for >= 2048 workgroups (8 per CU), but keep >= 256 rows per split
  int64_t s = (2048 + nbh - 1) / nbh;
  s = std::min<int64_t>(s, std::max<int64_t>(1, maxk / 256));
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, 64));
}
}  // namespace

int64_t rat_decode_workspace_bytes(int B, int H, int hd, int64_t T_cap, const int32_t* D,
                                   const int32_t* W, int num_splits) {
  int st = check_common(RAT_DTYPE_BF16, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  if (T_cap < 0 || T_cap > kMaxT || num_splits < 0) return RAT_ERR_INVALID_ARG;
  const int s = decode_splits(B, H, T_cap, D, W, num_splits);
  if (s <= 1) return 0;
  return (int64_t)B * H * s * (hd + 2) * 4;
}

}  // extern "C"

namespace {
// The decode step of rat_decode_step and rat_decode_step_noalloc.  With
// scratch set, the split-K partials go to the library's own device array
// (workspace, workspace_bytes: its address on this device and its size).
int decode_impl(int dtype, int B, int H, int hd, const int32_t* D, const int32_t* W, float scale,
                int64_t pos, int64_t T_cap, const void* q, const void* k, const void* v,
                const void* g, float* state_k, float* state_v, void* Kc, void* Vc, void* k_ring,
                void* v_ring, void* o, int num_splits, void* workspace, size_t workspace_bytes,
                void* stream, bool scratch);
}  // namespace

extern "C" {

int rat_decode_step(int dtype, int B, int H, int hd, const int32_t* D, const int32_t* W,
                    float scale, int64_t pos, int64_t T_cap, const void* q, const void* k,
                    const void* v, const void* g, float* state_k, float* state_v, void* Kc,
                    void* Vc, void* k_ring, void* v_ring, void* o, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(dtype, B, H, hd, D, W, scale, pos, T_cap, q, k, v, g, state_k, state_v, Kc,
                     Vc, k_ring, v_ring, o, num_splits, workspace, workspace_bytes, stream, false);
}

int rat_decode_step_noalloc(int dtype, int B, int H, int hd, const int32_t* D, const int32_t* W,
                            float scale, int64_t pos, int64_t T_cap, const void* q,
                            const void* k, const void* v, const void* g, float* state_k,
                            float* state_v, void* Kc, void* Vc, void* k_ring, void* v_ring,
                            void* o, int num_splits, void* stream) {
  return decode_impl(dtype, B, H, hd, D, W, scale, pos, T_cap, q, k, v, g, state_k, state_v, Kc,
                     Vc, k_ring, v_ring, o, num_splits, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {

// Split-K partials of rat_decode_step_noalloc: one array per device, kept
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a handle); its device address comes from
// hipGetSymbolAddress, once per device.
__device__ __align__(256) float scratch[RAT_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RAT_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RAT_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return RAT_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return RAT_OK;
}

int decode_impl(int dtype, int B, int H, int hd, const int32_t* D, const int32_t* W, float scale,
                int64_t pos, int64_t T_cap, const void* q, const void* k, const void* v,
                const void* g, float* state_k, float* state_v, void* Kc, void* Vc, void* k_ring,
                void* v_ring, void* o, int num_splits, void* workspace, size_t workspace_bytes,
                void* stream, bool scratch) {
  int st = check_common(dtype, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  if (T_cap < 0 || T_cap > kMaxT || pos < 0 || num_splits < 0 || num_splits > 1024)
    return RAT_ERR_INVALID_ARG;
  if (pos >= T_cap) return RAT_ERR_CAPACITY;
  if (!(scale <= 0.f) && !std::isfinite(scale)) return RAT_ERR_INVALID_ARG;
  if (B == 0 || H == 0) return RAT_OK;
  DecodeParams p;
  std::memset(&p, 0, sizeof(p));
  st = fill_tables(H, T_cap, D, W, p.ht, p.R, p.WS);
  if (st != RAT_OK) return st;
  for (const void* ptr : {q, k, v, g, (const void*)o})
    if (!ptr || !aligned16(ptr)) return RAT_ERR_INVALID_ARG;
  if (!state_k || !state_v || !aligned16(state_k) || !aligned16(state_v)) return RAT_ERR_INVALID_ARG;
  if (p.R > 0 && (!Kc || !Vc || !aligned16(Kc) || !aligned16(Vc))) return RAT_ERR_INVALID_ARG;
  if (p.WS > 0 && (!k_ring || !v_ring || !aligned16(k_ring) || !aligned16(v_ring)))
    return RAT_ERR_INVALID_ARG;
  const int s = decode_splits(B, H, T_cap, D, W, num_splits);
  if (s > 1) {
    const int64_t need = (int64_t)B * H * s * (hd + 2) * 4;
    if (scratch) {
      if (need > (int64_t)RAT_NOALLOC_SCRATCH_BYTES) return RAT_ERR_WORKSPACE;
      st = scratch_address(&workspace);
      if (st != RAT_OK) return st;
      workspace_bytes = RAT_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || !aligned16(workspace) || (int64_t)workspace_bytes < need)
      return RAT_ERR_WORKSPACE;
  }
  if ((int64_t)B * H > INT32_MAX / 2 || (int64_t)B * H * s > INT32_MAX) return RAT_ERR_UNSUPPORTED;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)hd);
  // heads in the grid by the keys they read, most first: a head-wise hybrid's
  // long (dense) splits then start in the first wave of workgroups and the
  // short ones fill in beside them
  {
    int64_t keys[kMaxHeads];
    for (int h = 0; h < H; ++h) {
      keys[h] = std::max<int64_t>(0, pos - W[h]) / D[h] + std::min<int64_t>(W[h], pos);
      p.perm[h] = h;
    }
    std::stable_sort(p.perm, p.perm + H, [&](int a, int b) { return keys[a] > keys[b]; });
    for (int r = 0; r < H;) {
      int e = r + 1;
      while (e < H && keys[p.perm[e]] == keys[p.perm[r]]) ++e;
      for (int i = r; i < e; ++i) p.class_end[i] = e;
      r = e;
    }
  }
  p.B = B;
  p.H = H;
  p.splits = s;
  p.pos = (int)pos;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.sk = state_k;
  p.sv = state_v;
  p.Kc = Kc;
  p.Vc = Vc;
  p.kr = k_ring;
  p.vr = v_ring;
  p.o = o;
  p.part = static_cast<float*>(workspace);
  return map_hip(launch_decode(dtype, hd, p, stream));
}

}  // namespace

extern "C" {

int rat_topk_cache_build(int dtype, int B, int H, int64_t T, int hd, int64_t T_cap,
                         int64_t t0, const void* hk, const void* hv, void* hk_hist,
                         void* hv_hist, float* block_means, void* stream) {
  if (dtype != RAT_DTYPE_BF16 && dtype != RAT_DTYPE_F32) return RAT_ERR_UNSUPPORTED;
  if (hd != 64 && hd != 128) return RAT_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || T < 0 || t0 < 0 || T_cap < 0 || T_cap > kMaxT)
    return RAT_ERR_INVALID_ARG;
  if (t0 + T > T_cap) return RAT_ERR_CAPACITY;
  if (B > 65535 || H > 65535) return RAT_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || T == 0) return RAT_OK;
  for (const void* ptr : {hk, hv, (const void*)hk_hist, (const void*)hv_hist})
    if (!ptr || !aligned16(ptr)) return RAT_ERR_INVALID_ARG;
  // a block completes in this call when it ends inside t0 .. t0+T-1
  const bool completes = (t0 + T) / kTopkBlock > t0 / kTopkBlock;
  if (completes && (!block_means || !aligned16(block_means))) return RAT_ERR_INVALID_ARG;
  return map_hip(launch_topk_cache_build(dtype, hd, B, H, T, T_cap, t0, hk, hv, hk_hist, hv_hist,
                                         block_means, stream));
}

int rat_decode_step_topk(int dtype, int B, int H, int hd, const int32_t* D, const int32_t* W,
                         float scale, int64_t pos, int64_t T_cap, int k_blocks, const void* q,
                         const void* k, const void* v, const void* g, float* state_k,
                         float* state_v, void* Kc, void* Vc, void* k_ring, void* v_ring,
                         void* hk_hist, void* hv_hist, float* block_means, void* o,
                         int32_t* sel_out, void* stream) {
  int st = check_common(dtype, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  if (T_cap < 0 || T_cap > kMaxT || pos < 0 || k_blocks < 0) return RAT_ERR_INVALID_ARG;
  if (k_blocks > kTopkMaxK || T_cap / kTopkBlock > kTopkMaxBlocks) return RAT_ERR_UNSUPPORTED;
  if (pos >= T_cap) return RAT_ERR_CAPACITY;
  if (!(scale <= 0.f) && !std::isfinite(scale)) return RAT_ERR_INVALID_ARG;
  if (B == 0 || H == 0) return RAT_OK;
  if ((int64_t)B * H > INT32_MAX / 2) return RAT_ERR_UNSUPPORTED;
  TopkParams p;
  std::memset(&p, 0, sizeof(p));
  st = fill_tables(H, T_cap, D, W, p.ht, p.R, p.WS);
  if (st != RAT_OK) return st;
  for (const void* ptr : {q, k, v, g, (const void*)o, (const void*)hk_hist, (const void*)hv_hist})
    if (!ptr || !aligned16(ptr)) return RAT_ERR_INVALID_ARG;
  if (!state_k || !state_v || !aligned16(state_k) || !aligned16(state_v)) return RAT_ERR_INVALID_ARG;
  if (p.R > 0 && (!Kc || !Vc || !aligned16(Kc) || !aligned16(Vc))) return RAT_ERR_INVALID_ARG;
  if (p.WS > 0 && (!k_ring || !v_ring || !aligned16(k_ring) || !aligned16(v_ring)))
    return RAT_ERR_INVALID_ARG;
  if (T_cap >= kTopkBlock && (!block_means || !aligned16(block_means))) return RAT_ERR_INVALID_ARG;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)hd);
  p.B = B;
  p.H = H;
  p.pos = (int)pos;
  p.k = k_blocks;
  p.T_cap = T_cap;
  p.NB = T_cap / kTopkBlock;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.q = q;
  p.k_in = k;
  p.v_in = v;
  p.g = g;
  p.sk = state_k;
  p.sv = state_v;
  p.Kc = Kc;
  p.Vc = Vc;
  p.kr = k_ring;
  p.vr = v_ring;
  p.hk = hk_hist;
  p.hv = hv_hist;
  p.means = block_means;
  p.o = o;
  p.sel = sel_out;
  return map_hip(launch_decode_topk(dtype, hd, p, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// prefill backward
// ---------------------------------------------------------------------------
namespace {

// Backward workspace (fp32 throughout), each part 256-byte aligned:
// delta [B,H,T], own-position scalars [B,H,T][2], window gradients dhk and
// dhv [B,H,T,hd] (only when some head has a window), partial anchor
// gradients dKc and dVc [kBwdMaxSplit][B,R,hd], chunk maps
// [B*H][nchunk][3][hd], carries [B*H][nchunk][2][hd].
constexpr int kBwdMaxSplit = 8;

// Backward workspace: the reverse scan's tree first (the forward scan's
// layout: header, then the tagged tree entries; sized for either storage
// type, so the header sits at offset 0 and a buffer zero-filled once serves
// calls of any size that fits), then the per-call intermediates.
struct BwdLayout {
  int64_t R = 0;
  int64_t tree_bytes = 0;
  int64_t off_delta = 0, off_own = 0, off_dhk = 0, off_dhv = 0, off_dkc = 0, off_dvc = 0,
          bytes = 0;
};

bool bwd_layout(int B, int H, int64_t T, int hd, const int32_t* D, const int32_t* W,
                BwdLayout& L) {
  L.R = 0;
  bool window = false;
  for (int h = 0; h < H; ++h) {
    L.R += T / D[h];
    window = window || (W != nullptr && W[h] > 0);
  }
  ScanLayout tb, tf;
  if (!scan_layout(B, H, T, hd, RAT_DTYPE_BF16, tb) || !scan_layout(B, H, T, hd, RAT_DTYPE_F32, tf))
    return false;
  L.tree_bytes = std::max(tb.bytes, tf.bytes);
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t bh = (int64_t)B * H;
  const int64_t dh = window ? bh * T * hd * 4 : 0;
  int64_t o = up(L.tree_bytes);
  L.off_delta = o; o = up(o + bh * T * 4);
  L.off_own = o; o = up(o + bh * T * 8);
  L.off_dhk = o; o = up(o + dh);
  L.off_dhv = o; o = up(o + dh);
  L.off_dkc = o; o = up(o + kBwdMaxSplit * (int64_t)B * L.R * hd * 4);
  L.off_dvc = o; o = up(o + kBwdMaxSplit * (int64_t)B * L.R * hd * 4);
  L.bytes = o;
  return L.R <= INT32_MAX && bh * T * hd < ((int64_t)1 << 62);
}

}  // namespace

extern "C" {

int64_t rat_prefill_backward_workspace_bytes(int B, int H, int64_t T, int hd, const int32_t* D,
                                             const int32_t* W) {
  if (T < 0 || T > kMaxT) return RAT_ERR_INVALID_ARG;
  const int st = check_common(RAT_DTYPE_BF16, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  BwdLayout L;
  if (!bwd_layout(B, H, T, hd, D, W, L)) return RAT_ERR_UNSUPPORTED;
  return L.bytes;
}

int rat_prefill_backward(int dtype, int B, int H, int64_t T, int hd, const int32_t* D,
                         const int32_t* W, float scale, const void* q, const void* k,
                         const void* v, const void* g, const void* hk, const void* hv,
                         const void* o, const float* lse, const void* dO, void* dq, void* dk,
                         void* dv, void* dg, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int st = check_common(dtype, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  if (T < 0 || T > kMaxT) return RAT_ERR_INVALID_ARG;
  if (!(scale <= 0.f) && !std::isfinite(scale)) return RAT_ERR_INVALID_ARG;
  if (B == 0 || H == 0 || T == 0) return RAT_OK;
  const void* in[] = {q, k, v, g, hk, hv, o, lse, dO};
  void* out[] = {dq, dk, dv, dg};
  for (const void* ptr : in)
    if (ptr == nullptr || !aligned16(ptr)) return RAT_ERR_INVALID_ARG;
  for (void* ptr : out)
    if (ptr == nullptr || !aligned16(ptr)) return RAT_ERR_INVALID_ARG;
  BwdLayout L;
  if (!bwd_layout(B, H, T, hd, D, W, L)) return RAT_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace) || (int64_t)workspace_bytes < L.bytes)
    return RAT_ERR_WORKSPACE;
  BwdParams p;
  std::memset(&p, 0, sizeof(p));
  int64_t R, WS;
  st = fill_tables(H, T, D, W, p.ht, R, WS);
  if (st != RAT_OK) return st;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)hd);
  p.B = B;
  p.H = H;
  p.T = (int)T;
  p.scale = sc;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.R = R;
  ScanLayout tl;
  if (!scan_layout(B, H, T, hd, dtype, tl)) return RAT_ERR_UNSUPPORTED;
  if (tl.nticket > INT32_MAX) return RAT_ERR_UNSUPPORTED;
  p.nchunk = (int)tl.nchunk;
  p.rnlevels = tl.nlevels;
  for (int l = 0; l < tl.nlevels; ++l) {
    p.rnodes[l] = tl.nodes[l];
    p.rlbase[l] = tl.lbase[l];
  }
  // the queries of an anchor tile are shared by nsplit workgroups (partial
  // sums) so that the key-side grid holds about two workgroups per CU
  int64_t max_na_t = 0;
  for (int h = 0; h < H; ++h) max_na_t = std::max<int64_t>(max_na_t, (T / D[h] + 63) / 64);
  int nsplit = 1;
  if (max_na_t > 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return RAT_ERR_HIP;
    const int64_t wgs = (int64_t)B * H * max_na_t;
    nsplit = (int)std::min<int64_t>(kBwdMaxSplit, std::max<int64_t>(1, (2 * cus + wgs - 1) / wgs));
    nsplit = (int)std::min<int64_t>(nsplit, (T + 63) / 64);
  }
  int64_t nkt = 0;
  for (int h = 0; h < H; ++h) {
    const int64_t na_t = (T / D[h] + 63) / 64;
    const int64_t nb_t = W[h] > 0 ? (T + 63) / 64 : 0;
    nkt = std::max(nkt, na_t * nsplit + nb_t);
  }
  if (nkt > INT32_MAX) return RAT_ERR_UNSUPPORTED;
  p.nkt = (int)nkt;
  p.nsplit = nsplit;
  // dq with the anchors resident in LDS: bf16, no window, every head's
  // anchors fit; about one workgroup per CU, at least one block per wave
  bool resident = dtype == RAT_DTYPE_BF16;
  for (int h = 0; h < H && resident; ++h)
    resident = W[h] == 0 && (T - 1) / D[h] <= kResidentAnchors;
  if (resident) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return RAT_ERR_HIP;
    const int64_t nbh = (int64_t)B * H;
    const int64_t nblk = (T + 15) / 16;
    int64_t nra = (std::max(cus, 1) + nbh - 1) / nbh;
    nra = std::max<int64_t>(
        1, std::min<int64_t>(nra, (nblk + kBwdResidentWaves - 1) / kBwdResidentWaves));
    if (nbh * nra <= INT32_MAX) p.nra = (int)nra;
  }
  p.kc_split = (int64_t)B * R * hd;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.hk = hk;
  p.hv = hv;
  p.o = o;
  p.lse = lse;
  p.dO = dO;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dg = dg;
  char* ws = static_cast<char*>(workspace);
  p.delta = reinterpret_cast<float*>(ws + L.off_delta);
  p.own = reinterpret_cast<float*>(ws + L.off_own);
  p.dhk = reinterpret_cast<float*>(ws + L.off_dhk);
  p.dhv = reinterpret_cast<float*>(ws + L.off_dhv);
  p.dKc = reinterpret_cast<float*>(ws + L.off_dkc);
  p.dVc = reinterpret_cast<float*>(ws + L.off_dvc);
  p.rhdr = reinterpret_cast<uint32_t*>(ws);
  p.ragg = reinterpret_cast<uint64_t*>(ws + tl.agg_off);
  return map_hip(launch_backward(dtype, hd, p, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// layer prefill: projections (the library's own MFMA GEMM) around the scan
// and attention
// ---------------------------------------------------------------------------
namespace {

// layer workspace: the scan workspace first (its header, with the launch
// epoch and the error word, then sits at offset 0 whatever the call's size,
// so a buffer zeroed once serves calls of any size that fits), then q, k, v
// and the gate pre-activation token-major [B,T,H,hd] (the projections'
// output), hk, hv [B,H,T,hd] and o token-major (all ST)
struct LayerLayout {
  int64_t act = 0, off_act = 0, scan_bytes = 0, bytes = 0;
};

bool layer_layout(int dtype, int B, int H, int64_t T, int hd, LayerLayout& L) {
  const int64_t es = dtype == RAT_DTYPE_BF16 ? 2 : 4;
  L.act = ((int64_t)B * H * T * hd * es + 255) / 256 * 256;
  L.scan_bytes = rat_scan_workspace_bytes(B, H, T, hd);
  if (L.scan_bytes < 0) return false;
  L.off_act = (L.scan_bytes + 255) / 256 * 256;
  L.bytes = L.off_act + 7 * L.act;
  return true;
}

}  // namespace

extern "C" {

int64_t rat_layer_workspace_bytes(int dtype, int B, int H, int64_t T, int hd) {
  if (B < 0 || H < 0 || T < 0 || T > kMaxT) return RAT_ERR_INVALID_ARG;
  if (dtype != RAT_DTYPE_BF16 && dtype != RAT_DTYPE_F32) return RAT_ERR_UNSUPPORTED;
  if (hd != 64 && hd != 128) return RAT_ERR_UNSUPPORTED;
  LayerLayout L;
  if (!layer_layout(dtype, B, H, T, hd, L)) return RAT_ERR_UNSUPPORTED;
  return L.bytes;
}

}  // extern "C"

namespace {
// Every check rat_layer_prefill (and the scan and attention it runs) makes
// before launching anything.  RAT_OK with nothing to do when B, H or T is 0.
int layer_check(int dtype, int B, int H, int64_t T, int hd, int dm, const int32_t* D,
                const int32_t* W, float scale, int64_t T_cap, const void* x, const void* w_q,
                const void* w_k, const void* w_v, const void* w_g, const float* b_g,
                const void* w_o, const void* out, const float* lse, const void* Kc,
                const void* Vc, const void* k_ring, const void* v_ring, const float* state_k,
                const float* state_v, const void* workspace, size_t workspace_bytes) {
  int st = check_common(dtype, B, H, hd, D, W);
  if (st != RAT_OK) return st;
  if (T < 0 || T_cap > kMaxT || dm <= 0) return RAT_ERR_INVALID_ARG;
  if (T > T_cap) return RAT_ERR_CAPACITY;
  if (!(scale <= 0.f) && !std::isfinite(scale)) return RAT_ERR_INVALID_ARG;
  if (B == 0 || H == 0 || T == 0) return RAT_OK;
  const void* ptrs[] = {x, w_q, w_k, w_v, w_g, b_g, w_o, out};
  for (const void* ptr : ptrs)
    if (ptr == nullptr || !aligned16(ptr)) return RAT_ERR_INVALID_ARG;
  const int64_t HD = (int64_t)H * hd;
  if ((int64_t)B * T > INT32_MAX || HD > INT32_MAX || T * HD > INT32_MAX)
    return RAT_ERR_UNSUPPORTED;
  // the bf16 GEMM moves 16-byte pieces of rows (8 elements) and has at most
  // 65535 row tiles of 256
  if (dtype == RAT_DTYPE_BF16 && (dm % 8 != 0 || (int64_t)B * T > 65535LL * 256))
    return RAT_ERR_UNSUPPORTED;
  LayerLayout L;
  if (!layer_layout(dtype, B, H, T, hd, L)) return RAT_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace) || (int64_t)workspace_bytes < L.bytes)
    return RAT_ERR_WORKSPACE;
  // the cache the scan and attention write and read
  HeadTables ht;
  int64_t R, WS;
  st = fill_tables(H, T_cap, D, W, ht, R, WS);
  if (st != RAT_OK) return st;
  if (state_k == nullptr || state_v == nullptr || !aligned16(state_k) || !aligned16(state_v))
    return RAT_ERR_INVALID_ARG;
  if (WS > 0 && (!k_ring || !v_ring || !aligned16(k_ring) || !aligned16(v_ring)))
    return RAT_ERR_INVALID_ARG;
  if (R > 0 && (!Kc || !Vc || !aligned16(Kc) || !aligned16(Vc))) return RAT_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return RAT_ERR_INVALID_ARG;
  return RAT_OK;
}

// The launches of one layer (arguments already checked by layer_check).
int layer_run(int dtype, int B, int H, int64_t T, int hd, int dm, const int32_t* D,
              const int32_t* W, float scale, int64_t T_cap, const void* x, const void* w_q,
              const void* w_k, const void* w_v, const void* w_g, const float* b_g,
              const void* w_o, void* out, float* lse, void* Kc, void* Vc, void* k_ring,
              void* v_ring, float* state_k, float* state_v, void* workspace, size_t workspace_bytes,
              void* stream) {
  if (B == 0 || H == 0 || T == 0) return RAT_OK;
  const int64_t HD = (int64_t)H * hd;
  LayerLayout L;
  layer_layout(dtype, B, H, T, hd, L);
  int st = RAT_OK;
  char* ws = static_cast<char*>(workspace);
  char* act = ws + L.off_act;
  void* q = act;
  void* k = act + L.act;
  void* v = act + 2 * L.act;
  void* g = act + 3 * L.act;
  void* hk = act + 4 * L.act;
  void* hv = act + 5 * L.act;
  void* o = act + 6 * L.act;
  // projections token-major, [B*T, H*hd] = x [B*T, dm] W [dm, H*hd]: one
  // grouped GEMM for q, k, v and the gate pre-activation
  GemmParams gp;
  std::memset(&gp, 0, sizeof(gp));
  gp.M = (int)(B * T);
  gp.K = dm;
  gp.Ng = (int)HD;
  gp.ngroups = 4;
  gp.A = x;
  gp.lda = dm;
  gp.B[0] = w_q;
  gp.B[1] = w_k;
  gp.B[2] = w_v;
  gp.B[3] = w_g;
  gp.ldb = HD;
  gp.C[0] = q;
  gp.C[1] = k;
  gp.C[2] = v;
  gp.C[3] = g;
  gp.ldc = HD;
  st = map_hip(launch_gemm(dtype, gp, stream));
  if (st != RAT_OK) return st;
  // recurrence with the gate sigmoid(g + b_g) fused into its loads
  st = scan_impl(dtype, B, H, T, hd, D, W, T_cap, 0, k, v, g, nullptr, nullptr, hk, hv, Kc, Vc,
                 nullptr, nullptr, k_ring, v_ring, state_k, state_v, ws,
                 (size_t)L.scan_bytes, stream, b_g, true);
  if (st != RAT_OK) return st;
  // dilated attention; o written token-major for the output projection
  st = attn_impl(dtype, B, H, T, hd, D, W, scale, T_cap, 0, q, hk, hv, Kc, Vc, nullptr, nullptr,
                 o, lse, stream, true, true);
  if (st != RAT_OK) return st;
  // out [B*T, dm] = o [B*T, H*hd] W_o [H*hd, dm]
  std::memset(&gp, 0, sizeof(gp));
  gp.M = (int)(B * T);
  gp.K = (int)HD;
  gp.Ng = dm;
  gp.ngroups = 1;
  gp.A = o;
  gp.lda = HD;
  gp.B[0] = w_o;
  gp.ldb = dm;
  gp.C[0] = out;
  gp.ldc = dm;
  st = map_hip(launch_gemm(dtype, gp, stream));
  if (st != RAT_OK) return st;
  return RAT_OK;
}


// Stack workspace: one layer workspace (reused layer after layer), then the
// activations between layers [B, T, dm].
int64_t stack_tmp_offset(int dtype, int B, int H, int64_t T, int hd) {
  LayerLayout L;
  if (!layer_layout(dtype, B, H, T, hd, L)) return -1;
  return (L.bytes + 255) / 256 * 256;
}
}  // namespace

extern "C" {

int rat_layer_prefill(int dtype, int B, int H, int64_t T, int hd, int dm, const int32_t* D,
                      const int32_t* W, float scale, int64_t T_cap, const void* x,
                      const void* w_q, const void* w_k, const void* w_v, const void* w_g,
                      const float* b_g, const void* w_o, void* out, float* lse, void* Kc,
                      void* Vc, void* k_ring, void* v_ring, float* state_k, float* state_v,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const int st = layer_check(dtype, B, H, T, hd, dm, D, W, scale, T_cap, x, w_q, w_k, w_v, w_g,
                             b_g, w_o, out, lse, Kc, Vc, k_ring, v_ring, state_k, state_v,
                             workspace, workspace_bytes);
  if (st != RAT_OK) return st;
  return layer_run(dtype, B, H, T, hd, dm, D, W, scale, T_cap, x, w_q, w_k, w_v, w_g, b_g, w_o,
                   out, lse, Kc, Vc, k_ring, v_ring, state_k, state_v, workspace, workspace_bytes,
                   stream);
}

int64_t rat_stack_workspace_bytes(int dtype, int B, int H, int64_t T, int hd, int dm) {
  const int64_t lw = rat_layer_workspace_bytes(dtype, B, H, T, hd);
  if (lw < 0) return lw;
  if (dm <= 0 || B < 0 || T < 0) return RAT_ERR_INVALID_ARG;
  const int64_t es = dtype == RAT_DTYPE_BF16 ? 2 : 4;
  return stack_tmp_offset(dtype, B, H, T, hd) + (int64_t)B * T * dm * es;
}

int rat_stack_prefill(int dtype, int nlayers, int B, int H, int64_t T, int hd, int dm,
                      const int32_t* D, const int32_t* W, float scale, int64_t T_cap,
                      const void* x, const void* const* w_q, const void* const* w_k,
                      const void* const* w_v, const void* const* w_g, const float* const* b_g,
                      const void* const* w_o, void* out, void* const* Kc, void* const* Vc,
                      void* const* k_ring, void* const* v_ring, float* const* state_k,
                      float* const* state_v, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (nlayers < 1 || !D || !W || !w_q || !w_k || !w_v || !w_g || !b_g || !w_o || !Kc || !Vc ||
      !k_ring || !v_ring || !state_k || !state_v)
    return RAT_ERR_INVALID_ARG;
  const int64_t need = rat_stack_workspace_bytes(dtype, B, H, T, hd, dm);
  if (need < 0) return (int)need;
  if (B == 0 || H == 0 || T == 0) {
    for (int l = 0; l < nlayers; ++l) {
      const int st = check_common(dtype, B, H, hd, D + (int64_t)l * H, W + (int64_t)l * H);
      if (st != RAT_OK) return st;
    }
    return T > T_cap ? RAT_ERR_CAPACITY : RAT_OK;
  }
  if (workspace == nullptr || !aligned16(workspace) || (int64_t)workspace_bytes < need)
    return RAT_ERR_WORKSPACE;
  char* tmp = static_cast<char*>(workspace) + stack_tmp_offset(dtype, B, H, T, hd);
  const size_t lw = (size_t)stack_tmp_offset(dtype, B, H, T, hd);
  // layer l reads x (l = 0) or the activations between layers, and writes
  // them (out for the last layer); a layer reads its input only in its first
  // launch and writes its output in its last, so one buffer serves both
  auto in_of = [&](int l) -> const void* { return l == 0 ? x : tmp; };
  auto out_of = [&](int l) -> void* { return l == nlayers - 1 ? out : tmp; };
  for (int l = 0; l < nlayers; ++l) {
    const int st = layer_check(dtype, B, H, T, hd, dm, D + (int64_t)l * H, W + (int64_t)l * H,
                               scale, T_cap, in_of(l), w_q[l], w_k[l], w_v[l], w_g[l], b_g[l],
                               w_o[l], out_of(l), nullptr, Kc[l], Vc[l], k_ring[l], v_ring[l],
                               state_k[l], state_v[l], workspace, lw);
    if (st != RAT_OK) return st;
  }
  for (int l = 0; l < nlayers; ++l) {
    const int st = layer_run(dtype, B, H, T, hd, dm, D + (int64_t)l * H, W + (int64_t)l * H,
                             scale, T_cap, in_of(l), w_q[l], w_k[l], w_v[l], w_g[l], b_g[l],
                             w_o[l], out_of(l), nullptr, Kc[l], Vc[l], k_ring[l], v_ring[l],
                             state_k[l], state_v[l], workspace, lw, stream);
    if (st != RAT_OK) return st;
  }
  return RAT_OK;
}

}  // extern "C"
