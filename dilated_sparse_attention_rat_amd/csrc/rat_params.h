// Kernel parameter blocks, filled on the host by the C-ABI layer and passed
// by value as kernel arguments (per-head tables included, so a head-wise
// hybrid needs no device-side table and no extra copy).
#pragma once

#include <stdint.h>

#include "rat.h"

namespace rat {

constexpr int kMaxHeads = RAT_MAX_HEADS;

struct HeadTables {
  int32_t D[kMaxHeads];     // dilation per head
  int32_t W[kMaxHeads];     // window per head
  int32_t aoff[kMaxHeads];  // first anchor-cache row of the head
  int32_t roff[kMaxHeads];  // first ring slot of the head
};

// Scan workspace header (32 KB): uint32 word 0 is the launch epoch, word 2
// the error flag (a wait for an aggregate timed out), and 64 done counters
// 256 bytes apart follow (see scan.hip).
constexpr int64_t kScanHeaderBytes = 32 * 1024;

constexpr int kScanRadix = 8;      // fan-in of the chunk-aggregate tree
constexpr int kScanMaxLevels = 10;

struct ScanParams {
  int B, H, T;
  int t0;          // absolute position of row 0 (continuation; 0 for a prefill)
  int nseq;        // B * H
  int nchunk;      // chunks per sequence
  int nticket;     // nseq * nchunk (= grid size)
  int nlevels;     // levels of the aggregate tree (top level has <= radix nodes)
  int nodes[kScanMaxLevels];     // nodes per sequence at each level
  int64_t lbase[kScanMaxLevels]; // first entry of each level in flags/agg
  int64_t R;       // anchor rows per batch row
  int64_t WS;      // ring slots per batch row
  const void* k;
  const void* v;
  const void* g;
  void* hk;        // nullable (cache-only mode)
  void* hv;
  void* Kc;
  void* Vc;
  void* kr;        // nullable iff all W == 0
  void* vr;
  float* sk;
  float* sv;
  const float* sk_in;  // state before row 0 (nullable: zero)
  const float* sv_in;
  const float* gate_bias;  // nullable; else g is the gate's pre-activation and
                           // the gate is sigmoid(g + gate_bias[h*hd + c])
  int64_t in_sb, in_sh, in_st;  // element strides of k, v, g over b, h, t
                                // ([B,H,T,hd]: H*T*hd, T*hd, hd)
  uint32_t* hdr;    // workspace header (kScanHeaderBytes)
  uint64_t* agg;    // [entries][3][hd]: (tag << 32 | fp32) of A, Bk, Bv
  HeadTables ht;
};

// Resident-anchor attention applies when no head has a window and every
// head's anchors fit in LDS (bf16).
constexpr int kResidentAnchors = 256;
constexpr int kResidentWaves = 16;  // waves per resident-anchor workgroup
constexpr int kResidentQB = 1;      // 16-query blocks per wave and block
constexpr int kBwdResidentWaves = 12;  // waves per workgroup of the resident-anchor dq kernel

struct AttnParams {
  int B, H, T;
  int t0;            // absolute position of query / state row 0
  int mode;          // 0: streamed K/V tiles; 1: resident anchors
  int nra;           // mode 1: workgroups per (b, h)
  int qb;            // 16-query blocks per wave (1 or 2): tile = 64*qb queries
  int nq;            // query tiles per (b, h)
  int np;            // workgroups per (b, h): pairs of query tiles, or single tiles
  int paired;        // 1: workgroup pr takes tiles nq-1-pr and pr; 0: tile nq-1-pr only
  int gsingle;       // paired launches: groups of 8 units from gsingle on take single tiles
  int64_t nblk;      // workgroups of the streamed launch
  int dma;           // K/V tiles loaded straight into LDS (bf16, hd 128, qb 2, no ring)
  float scale_log2;  // scale * log2(e)
  int64_t R;
  const void* q;
  int64_t q_sb, q_sh, q_st;  // element strides of q over b, h, t
  const void* hk;
  const void* hv;
  const void* Kc;
  const void* Vc;
  const void* kr;    // ring of the positions before t0 (window keys < t0)
  const void* vr;
  int64_t WS;        // ring slots per batch row
  void* o;
  int64_t o_sb, o_sh, o_st;  // element strides of o over b, h, t ([B,H,T,hd]:
                             // H*T*hd, T*hd, hd; token-major [B,T,H,hd]:
                             // T*H*hd, hd, H*hd)
  float* lse;        // nullable
  int32_t perm[kMaxHeads];  // heads in descending per-block cost
  HeadTables ht;
};

struct DecodeParams {
  int B, H;
  int splits;
  int pos;
  float scale_log2;
  int64_t R;
  int64_t WS;
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  float* sk;
  float* sv;
  void* Kc;
  void* Vc;
  void* kr;
  void* vr;
  void* o;
  float* part;       // [B*H][splits][2 + hd] (m, l, acc) when splits > 1
  HeadTables ht;
  // grid order: heads by keys read, most first (perm[rank] = head); heads
  // reading as many keys form a class, ranks [r, class_end[r]) for the first
  // rank r of a class, and a class's blocks run batch row by batch row
  int32_t perm[kMaxHeads];
  int32_t class_end[kMaxHeads];
};

// Decode with top-k block selection: the decode step's fields plus the
// state history and its block means.
struct TopkParams {
  int B, H;
  int pos;
  int k;             // blocks selected per (b, h)
  int64_t T_cap;     // rows of the history per (b, h)
  int64_t NB;        // block-mean rows per (b, h): T_cap / kTopkBlock
  float scale_log2;
  int64_t R;
  int64_t WS;
  const void* q;
  const void* k_in;
  const void* v_in;
  const void* g;
  float* sk;
  float* sv;
  void* Kc;
  void* Vc;
  void* kr;
  void* vr;
  void* hk;          // [B, H, T_cap, hd] stored states (history)
  void* hv;
  float* means;      // [B, H, NB, hd] fp32 mean key state of each complete block
  void* o;
  int32_t* sel;      // nullable: [B, H, k] selected blocks, -1 past the count
  HeadTables ht;
};

struct BwdParams {
  int B, H, T;
  float scale;       // score scale
  float scale_log2;  // scale * log2(e)
  int64_t R;         // anchor rows per batch row (floor(T / D_h) summed over heads)
  int nchunk;        // reverse-scan chunks per sequence (scan_rows_per_chunk rows each)
  int nkt;           // workgroups per head in the key-side grid (max over heads)
  int nsplit;        // workgroups sharing the queries of one anchor tile
  int nra;           // > 0: dq with the anchors resident in LDS, nra workgroups per (b, h)
  int64_t kc_split;  // elements of one partial anchor-gradient buffer (B*R*hd)
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* hk;    // forward states (stored)
  const void* hv;
  const void* o;     // forward output
  const float* lse;  // forward lse (natural log)
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  void* dg;
  float* delta;      // workspace: [B,H,T] dO . o
  float* own;        // workspace: [B,H,T][2] scale*dS and P of the own position
  float* dhk;        // workspace: [B,H,T,hd] window gradients (heads with W > 0)
  float* dhv;
  float* dKc;        // workspace: [nsplit][B,R,hd] partial anchor gradients
  float* dVc;
  // the reverse scan's chunk-aggregate tree (the forward scan's protocol):
  // header words, then [entries][3][hd] tagged words; level l holds
  // rnodes[l] nodes per sequence from entry rlbase[l]
  uint32_t* rhdr;
  uint64_t* ragg;
  int rnlevels;
  int rnodes[kScanMaxLevels];
  int64_t rlbase[kScanMaxLevels];
  HeadTables ht;
};

// Projection GEMM: C_g = A B_g for groups g < ngroups, B_g [K, Ng] and
// C_g [M, Ng] row-major; column n of the grouped product is column n % Ng
// of group n / Ng.
struct GemmParams {
  int M, K, Ng, ngroups;
  const void* A;     // [M, K], row stride lda
  int64_t lda;
  const void* B[4];  // [K, Ng] each, row stride ldb
  int64_t ldb;
  void* C[4];        // [M, Ng] each, row stride ldc
  int64_t ldc;
};

// launchers (one per kernel family); return hipError_t as int
int launch_gemm(int dtype, const GemmParams& p, void* stream);
int launch_scan(int dtype, int hd, const ScanParams& p, void* stream);
// Continuation: copy the ring slots of positions [max(0, t0+T-W), t0) that
// stay in the window from ring_in to ring_out (the scan writes the rest).
int launch_ring_carry(int dtype, int hd, int B, int H, int64_t WS, const HeadTables& ht,
                      int64_t t0, int64_t T, const void* kr_in, const void* vr_in, void* kr_out,
                      void* vr_out, void* stream);
int launch_attn_prefill(int dtype, int hd, const AttnParams& p, void* stream);
int launch_attn_resident(int dtype, int hd, const AttnParams& p, void* stream);
int launch_decode(int dtype, int hd, const DecodeParams& p, void* stream);
int launch_backward(int dtype, int hd, const BwdParams& p, void* stream);
int launch_decode_topk(int dtype, int hd, const TopkParams& p, void* stream);
// history cache: rows [0, T) of hk/hv ([B,H,T,hd]) into Hk/Hv ([B,H,T_cap,hd])
// and the mean of every complete block into means ([B,H,T_cap/64,hd] fp32)
int launch_topk_cache_build(int dtype, int hd, int B, int H, int64_t T, int64_t T_cap,
                            int64_t t0, const void* hk, const void* hv, void* Hk, void* Hv,
                            float* means, void* stream);

// sizes shared by the host layer and the kernels
constexpr int kScanThreads = 256;
constexpr int kScanRowsPerThread = 4;
int scan_rows_per_chunk(int dtype, int hd);
// Largest grid of `kernel` (at `threads` per workgroup) whose workgroups can
// all be resident at once on the current device; <= 0 on error.
int coop_grid_limit(const void* kernel, int threads);

constexpr int kAttnBN = 64;    // keys per LDS tile
constexpr int kAttnTailDiv = 4;  // a paired launch runs its last 1/kAttnTailDiv of full groups as single tiles
constexpr int kDecodeThreads = 256;
constexpr int kTopkBlock = RAT_TOPK_BLOCK;   // positions per selectable block
constexpr int kTopkMaxK = RAT_TOPK_MAX_K;    // blocks selected per (b, h), at most
constexpr int kTopkMaxBlocks = 8192;    // eligible blocks per (b, h), at most (scores in LDS)

}  // namespace rat
