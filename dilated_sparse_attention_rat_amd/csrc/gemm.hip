// Dense projections of the layer (the steps on either side of the hot path):
// C = A B with A [M, K] (the layer input x, or o) and B [K, N] (a projection
// matrix), both row-major, fp32 accumulation, output in the storage type.
// One launch may cover several B/C pairs side by side along N (the q, k, v
// and gate projections of x: one grouped GEMM over N = 4*H*hd columns).
//
// Method: RAT+ abstract -- RAT+ augments the attention of a transformer
// layer, whose q, k, v come from linear projections of the input and whose
// output is projected back; zhichai.net deep dive "RAT+ 深度拆解", section
// 2.1 -- the forget gate is input dependent (a projection of x).
//
// Design (bf16, gfx950): the main kernel is gemm_bf16_dma_kernel below
// (K % 32 == 0): 256 x 256 tiles on 32x32x16 MFMAs at two waves per SIMD,
// direct-to-LDS loads, output regrouped through LDS.  gemm_bf16_kernel
// covers any K % 8 == 0:
//  * it computes C^T = B^T A^T on v_mfma_f32_16x16x32_bf16, so an
//    accumulator lane holds four consecutive columns n of one row m of C
//    (one 8-byte store) -- the same orientation as O^T = V^T P^T in the
//    attention kernels;
//  * B^T fragments come out of row-major B tiles [32 k][128 n] through
//    ds_read_b64_tr_b16 (the gfx950 transposing LDS read), A^T fragments
//    out of row-major A tiles [256 m][32 k] with two 8-byte reads each, in
//    the k order of the transposing read;
//  * workgroup tile 128 (n) x 256 (m), 4 waves of 64 x 128, K steps of 32;
//    one register staging buffer, LDS double-buffered (one barrier per K
//    step), the global loads of step s+1 in flight while step s is
//    computed; two workgroups per CU;
//  * rows past M and columns past N re-read the last valid one (their
//    outputs are not stored); K is zero-padded to the step (K % 8 == 0).
// fp32 storage runs a plain FMA kernel (no MFMA), for correctness checks.
#include "rat_device.h"

namespace rat {

namespace {

constexpr int kGemmBN = 128;   // n per workgroup (rows of C^T)
constexpr int kGemmBM = 256;   // m per workgroup
constexpr int kGemmBK = 32;    // k per step
constexpr int kGemmWS = kGemmBN + 16;  // B tile row stride (elements): 72 dwords
constexpr int kGemmXS = kGemmBK + 8;   // A tile row stride (elements): 20 dwords

struct GemmTileLoads {
  u32x4 b[2];  // B tile: 32 rows x 16 chunks = 512 chunks, 2 per thread
  u32x4 a[4];  // A tile: 256 rows x 4 chunks = 1024 chunks, 4 per thread
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16 sB[2][kGemmBK * kGemmWS];
  __shared__ __attribute__((aligned(16))) bf16 sA[2][kGemmBM * kGemmXS];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * kGemmBN;
  const int m0 = blockIdx.y * kGemmBM;
  const int wn = wave & 1;   // wave's n offset 64*wn
  const int wm = wave >> 1;  // wave's m offset 128*wm
  const int N = p.ngroups * p.Ng;

  // per-thread global sources (fixed over the K loop)
  const bf16* bsrc[2];
  int brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    brow[i] = idx >> 4;  // k row of the tile
    const int n = min(n0 + (idx & 15) * 8, N - 8);
    const int grp = n / p.Ng;
    bsrc[i] = reinterpret_cast<const bf16*>(p.B[grp]) + (n - grp * p.Ng);
  }
  const bf16* asrc[4];
  int akc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i;
    const int m = min(m0 + (idx >> 2), p.M - 1);
    akc[i] = (idx & 3) * 8;  // k offset of the chunk within the step
    asrc[i] = reinterpret_cast<const bf16*>(p.A) + (int64_t)m * p.lda + akc[i];
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load = [&](GemmTileLoads& t, int ks) {
    const int k0 = ks * kGemmBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = k0 + brow[i];
      t.b[i] = k < p.K ? ld_raw16(bsrc[i] + (int64_t)k * p.ldb) : zero;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) t.a[i] = k0 + akc[i] < p.K ? ld_raw16(asrc[i] + k0) : zero;
  };
  auto store = [&](const GemmTileLoads& t, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      st_raw16(&sB[buf][(idx >> 4) * kGemmWS + (idx & 15) * 8], t.b[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      st_raw16(&sA[buf][(idx >> 2) * kGemmXS + (idx & 3) * 8], t.a[i]);
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = (p.K + kGemmBK - 1) / kGemmBK;
  GemmTileLoads t;
  load(t, 0);
  store(t, 0);
  __syncthreads();
  auto compute = [&](int buf) {
    const bf16* sb = sB[buf];
    const bf16* sa = sA[buf];
    Frag<bf16> af[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const bf16* r = sa + (128 * wm + 16 * mb + col) * kGemmXS + 4 * g;
      af[mb] = frag_ld4x2(r, r + 16);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // B^T rows n = 64 wn + 16 nb + col, k slots (g, j) -> k = 4g + j and
      // 16 + 4g + j, the order frag_ld4x2 reads A in
      const Frag<bf16> bfr = frag_ld_tr(
          sb + (4 * g + (col >> 2)) * kGemmWS + 64 * wn + 16 * nb + 4 * (col & 3), 16 * kGemmWS);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) mma16(acc[nb][mb], bfr, af[mb]);
    }
  };
  // step s computes buffer s % 2 while the loads of step s + 1 are in
  // flight; they are stored into the other buffer after the compute
  for (int s = 0; s < nks; ++s) {
    load(t, min(s + 1, nks - 1));
    compute(s & 1);
    store(t, (s & 1) ^ 1);
    __syncthreads();
  }

  // epilogue: lane (col, g) of block (nb, mb) holds C[m][n .. n+3] with
  // m = m0 + 128 wm + 16 mb + col, n = n0 + 64 wn + 16 nb + 4 g
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 64 * wn + 16 * nb + 4 * g;
    if (n >= N) continue;
    const int grp = n / p.Ng;
    bf16* cbase = reinterpret_cast<bf16*>(p.C[grp]) + (n - grp * p.Ng);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = m0 + 128 * wm + 16 * mb + col;
      if (m < p.M) st4(cbase + (int64_t)m * p.ldc, acc[nb][mb]);
    }
  }
}

// Direct-to-LDS variant (bf16, K % 32 == 0): workgroup tile 256 (n) x 256
// (m), 8 waves of 64 (n) x 128 (m), two per SIMD, one workgroup per CU, on
// v_mfma_f32_32x32x16_bf16 (the 32 x 32 form keeps the matrix pipe busier
// from few waves than the 16 x 16 form, which reaches about 57% of the bf16
// rate from one wave per SIMD, measured).  A wave's 64 x 128 fp32
// accumulators take 128 registers, so two waves fit a SIMD: one wave's LDS
// reads and waits run beside the other's MFMAs (6% faster than four waves
// of 128 x 128 at one per SIMD, measured).  Per FLOP the workgroup tile
// reads half the global bytes of a 128-wide tile.  Every K step's tiles are fetched with
// global_load_lds_dwordx4 (lane l's 16 bytes land at the instruction's LDS
// base + 16 l, checked on the device), so no register staging: a ring of
// four LDS stages (32 KB each) holds the step being computed and the three
// whose loads are in flight.
//  * Fragments: MFMA lane l covers row l % 32 of its operand and k slots
//    8 (l / 32) + s.  A^T fragments are single 16-byte reads of the
//    row-major A tile [256 m][32 k]; B^T fragments come out of two
//    transposing reads of the B tile (two halves of [32 k][128 n]; wave
//    column wn reads columns 64 (wn % 2) .. +63 of half wn / 2), 16-lane
//    group G reading k rows 8 (G / 2) + 0..3 (then 4 on) of columns
//    16 (G % 2) + 0..15 of a 32-column block.
//  * Swizzles (tiles unpadded): A row r holds 16-byte chunk c at
//    c ^ ((r >> 2) & 3), so 16 lanes reading 16 rows cover all banks; B row
//    r holds chunk c at c ^ 4 (r & 3), so the 4 rows x 64 bytes of one
//    32-lane transposing pass fall on distinct banks.
//  * Accumulator element i of lane l is C^T row n = 8 (i / 4) + 4 (l / 32)
//    + i % 4, column m = l % 32; the epilogue regroups them through LDS into
//    whole 16-byte row pieces (A, B and C rows 16-byte aligned: pointers
//    16-byte aligned, ld* and Ng multiples of 8).
constexpr int kWideBN = 256;
constexpr int kWideBM = 256;
constexpr int kWideHalf = kGemmBK * 128;          // elements of one B half
constexpr int kWideAStage = kWideBM * kGemmBK;  // elements
constexpr int kWideBStage = 2 * kWideHalf;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_dma_kernel(const GemmParams p) {
  // one array per stage, indexed statically
  __shared__ __attribute__((aligned(1024))) bf16 sA0[kWideAStage];
  __shared__ __attribute__((aligned(1024))) bf16 sA1[kWideAStage];
  __shared__ __attribute__((aligned(1024))) bf16 sA2[kWideAStage];
  __shared__ __attribute__((aligned(1024))) bf16 sA3[kWideAStage];
  __shared__ __attribute__((aligned(1024))) bf16 sB0[kWideBStage];
  __shared__ __attribute__((aligned(1024))) bf16 sB1[kWideBStage];
  __shared__ __attribute__((aligned(1024))) bf16 sB2[kWideBStage];
  __shared__ __attribute__((aligned(1024))) bf16 sB3[kWideBStage];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  // Tile order.  Workgroup i runs on XCD i % 8 (each XCD has its own L2).
  // With the plain raster, a grid of 8 n-tiles gives each XCD one n-tile and
  // every m-tile, so every XCD streams all of A.  When both tile counts are
  // multiples of 8, XCD x takes m-tiles [x Mt/8, (x+1) Mt/8) and walks the
  // n-tiles in blocks of 8: at any time its workgroups cover a few m-tiles
  // by 8 n-tiles, and no A tile is fetched by more than one XCD.
  int tm = blockIdx.y, tn = blockIdx.x;
  if ((gridDim.x & 7) == 0 && (gridDim.y & 7) == 0) {
    const int pid = blockIdx.x + blockIdx.y * gridDim.x;
    const int x = pid & 7;
    const int s = pid >> 3;
    const int mx = gridDim.y >> 3;  // m-tiles per XCD
    const int r = s % (mx * 8);
    tm = x * mx + r / 8;
    tn = (s / (mx * 8)) * 8 + (r & 7);
  }
  const int n0 = tn * kWideBN;
  const int m0 = tm * kWideBM;
  const int wn = wave & 3;   // wave's n offset 64*wn (B half wn / 2)
  const int wm = wave >> 2;  // wave's m offset 128*wm
  const int N = p.ngroups * p.Ng;

  // this lane's sources: A instruction j < 2 covers rows 16 (2 wave + j) ..
  // +15 of the tile; B instruction j < 2 is number q = 2 wave + j of the
  // sixteen, rows 4 (q % 8) .. +3 of half q / 8
  const bf16* asrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int m = min(m0 + row, p.M - 1);
    asrc[j] = reinterpret_cast<const bf16*>(p.A) + (int64_t)m * p.lda + 8 * c;
  }
  const bf16* bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = 2 * wave + j;
    const int row = 4 * (q & 7) + (lane >> 4);
    const int c = (lane & 15) ^ (4 * (row & 3));
    const int n = min(n0 + 128 * (q >> 3) + 8 * c, N - 8);
    const int grp = n / p.Ng;
    bsrc[j] = reinterpret_cast<const bf16*>(p.B[grp]) + (int64_t)row * p.ldb + (n - grp * p.Ng);
  }
  auto issue = [&](bf16* __restrict__ sa, bf16* __restrict__ sb, int ks) {
    const int64_t k0 = (int64_t)ks * kGemmBK;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(asrc[j] + k0, sa + (2 * wave + j) * 16 * kGemmBK);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = 2 * wave + j;
      dma16(bsrc[j] + k0 * p.ldb, sb + (q >> 3) * kWideHalf + (q & 7) * 4 * 128);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[nb][mb][e] = 0.f;

  // fragments of k half kh (k 16 kh .. +15 of the step): A^T of 32-row
  // block mb, B^T of 32-column block nb
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int G = lane >> 4;
  const int tj = (lane >> 2) & 3;
  const int tq = lane & 3;
  const int bofs = (wn >> 1) * kWideHalf + (8 * (G >> 1) + tj) * 128 + 4 * (tq & 1);
  auto read_a = [&](const bf16* __restrict__ sa, int kh, Frag<bf16>* af) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = 128 * wm + 32 * mb + l32;
      af[mb] = frag_ld8(sa + r * kGemmBK + 8 * ((2 * kh + lh) ^ ((r >> 2) & 3)));
    }
  };
  auto read_b = [&](const bf16* __restrict__ sb, int kh, Frag<bf16>* bf) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int c = 8 * (wn & 1) + 4 * nb + 2 * (G & 1) + (tq >> 1);
      bf[nb] = frag_ld_tr(sb + bofs + kh * 16 * 128 + 8 * (c ^ (4 * tj)), 4 * 128);
    }
  };
  auto mma_half = [&](const Frag<bf16>* bf, const Frag<bf16>* af) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[nb].v, af[mb].v, acc[nb][mb], 0, 0, 0);
  };

  const int nks = p.K / kGemmBK;
  // Step s computes stage s % 4: its first k half from fragments read ahead,
  // its second from fragments read at the step's start.  Between the two,
  // once this thread's loads of step s + 1 are done (those of step s + 2,
  // four, may still be in flight), the barrier makes every wave's part of
  // step s + 1 visible and frees stage (s + 3) % 4, last read at step s - 1,
  // for the loads of step s + 3; the first half's fragments of step s + 1
  // are then read under the second half's MFMAs, and the barrier wait sits
  // under the first half's.
  Frag<bf16> af0[4], bf0[2];
  auto step = [&](int s, const bf16* __restrict__ sa, const bf16* __restrict__ sb,
                  const bf16* __restrict__ sa1, const bf16* __restrict__ sb1,
                  bf16* __restrict__ na, bf16* __restrict__ nb2) {
    if (s >= nks) return;
    Frag<bf16> af1[4], bf1[2];
    read_a(sa, 1, af1);
    read_b(sb, 1, bf1);
    mma_half(bf0, af0);
    if (s + 1 < nks) {
      if (s + 2 < nks)
        RAT_WAIT_VM_LGKM(4);
      else
        RAT_WAIT_VM_LGKM(0);
      lds_barrier();
      if (s + 3 < nks) issue(na, nb2, s + 3);
      read_a(sa1, 0, af0);
      read_b(sb1, 0, bf0);
    }
    mma_half(bf1, af1);
  };
  issue(sA0, sB0, 0);
  if (nks > 1) issue(sA1, sB1, 1);
  if (nks > 2) issue(sA2, sB2, 2);
  if (nks > 2)
    RAT_WAIT_VM_LGKM(8);
  else if (nks > 1)
    RAT_WAIT_VM_LGKM(4);
  else
    RAT_WAIT_VM_LGKM(0);
  lds_barrier();
  read_a(sA0, 0, af0);
  read_b(sB0, 0, bf0);
  for (int s0 = 0; s0 < nks; s0 += 4) {
    step(s0, sA0, sB0, sA1, sB1, sA3, sB3);
    step(s0 + 1, sA1, sB1, sA2, sB2, sA0, sB0);
    step(s0 + 2, sA2, sB2, sA3, sB3, sA1, sB1);
    step(s0 + 3, sA3, sB3, sA0, sB0, sA2, sB2);
  }

  // Epilogue through LDS: element 4 e + i of lane l in block (nb, mb) is
  // C[m][n + i] with m = 128 wm + 32 mb + l % 32, n = 64 wn + 32 nb + 8 e +
  // 4 (l / 32) (tile coordinates), i.e. 8-byte pieces of 32 different rows
  // per store instruction.  Each wave instead writes one 32-row block at a
  // time into its own LDS region (one of the eight stage arrays; rows 72
  // elements apart, so the 32 rows of one write pass spread over the banks
  // and every row starts 16-byte aligned), then reads it back as 16-byte row
  // pieces and stores 8 whole 128-byte row segments per instruction.  Every
  // stage's loads were waited for in the loop; the barrier frees the stage
  // buffers of all waves.
  __syncthreads();
  constexpr int kCS = 72;  // staging row stride (elements)
  bf16* sC = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sA2 : wave == 3 ? sA3
           : wave == 4 ? sB0 : wave == 5 ? sB1 : wave == 6 ? sB2 : sB3;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4 v = {acc[nb][mb][4 * e], acc[nb][mb][4 * e + 1], acc[nb][mb][4 * e + 2],
                         acc[nb][mb][4 * e + 3]};
        st4(sC + l32 * kCS + 32 * nb + 8 * e + 4 * lh, v);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int c8 = 8 * (lane & 7);
      const u32x4 v = *reinterpret_cast<const u32x4*>(sC + row * kCS + c8);
      const int m = m0 + 128 * wm + 32 * mb + row;
      const int n = n0 + 64 * wn + c8;
      if (m < p.M && n < N) {
        const int grp = n / p.Ng;
        bf16* dst = reinterpret_cast<bf16*>(p.C[grp]) + (int64_t)m * p.ldc + (n - grp * p.Ng);
        *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
  }
}

// fp32 storage: one thread per output element, fp32 FMA in k order
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams p) {
  const int N = p.ngroups * p.Ng;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.M * N) return;
  const int m = (int)(i / N);
  const int n = (int)(i - (int64_t)m * N);
  const int grp = n / p.Ng;
  const int c = n - grp * p.Ng;
  const float* a = reinterpret_cast<const float*>(p.A) + (int64_t)m * p.lda;
  const float* b = reinterpret_cast<const float*>(p.B[grp]) + c;
  float s = 0.f;
  for (int k = 0; k < p.K; ++k) s = fmaf(a[k], b[(int64_t)k * p.ldb], s);
  reinterpret_cast<float*>(p.C[grp])[(int64_t)m * p.ldc + c] = s;
}

}  // namespace

int launch_gemm(int dtype, const GemmParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t N = (int64_t)p.ngroups * p.Ng;
  if (p.M == 0 || N == 0) return 0;
  if (dtype == RAT_DTYPE_BF16) {
    if (p.K % kGemmBK == 0 && p.K > 0) {
      const dim3 grid((unsigned)((N + kWideBN - 1) / kWideBN),
                      (unsigned)((p.M + kWideBM - 1) / kWideBM));
      hipLaunchKernelGGL(gemm_bf16_dma_kernel, grid, dim3(512), 0, st, p);
    } else {
      const dim3 grid((unsigned)((N + kGemmBN - 1) / kGemmBN),
                      (unsigned)((p.M + kGemmBM - 1) / kGemmBM));
      hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, st, p);
    }
  } else {
    const int64_t n = (int64_t)p.M * N;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  }
  return (int)hipGetLastError();
}

}  // namespace rat
