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
// Design (bf16, gfx950):
//  * the kernel computes C^T = B^T A^T on v_mfma_f32_16x16x32_bf16, so an
//    accumulator lane holds four consecutive columns n of one row m of C
//    (one 8-byte store) -- the same orientation as O^T = V^T P^T in the
//    attention kernels;
//  * B^T fragments come out of row-major B tiles [32 k][128 n] through
//    ds_read_b64_tr_b16 (the gfx950 transposing LDS read), A^T fragments
//    out of row-major A tiles [256 m][32 k] with two 8-byte reads each, in
//    the k order of the transposing read;
//  * workgroup tile 128 (n) x 256 (m), 4 waves of 64 x 128, K steps of 32;
//    LDS double-buffered (one barrier per K step), the global loads of step
//    s+1 in flight while step s is computed; two workgroups per CU;
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

// Direct-to-LDS variant (bf16, K % 32 == 0): every K step's tiles are
// fetched with global_load_lds_dwordx4 (lane l's 16 bytes land at the
// instruction's LDS base + 16 l, checked on the device), so no register
// staging: a ring of three LDS stages holds the step being computed and the
// two whose loads are in flight.  Here k slot (g, j) of a fragment is
// k = 8g + j: A^T fragments are single 16-byte reads and the transposing B^T
// reads take rows 8g .. 8g+7.  The tiles are unpadded and XOR-swizzled so
// that the reads stay conflict-free: in the A tile (64 bytes per row)
// 16-byte chunk c of row r sits at c ^ ((r >> 2) & 3); in the B tile (256
// bytes per row) at c ^ 2 f(r), f(r) = (r & 3) | ((r >> 1) & 4), which is
// distinct over the eight rows one 32-lane pass of a transposing read
// touches.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kGemmStages = 3;
constexpr int kGemmAStage = kGemmBM * kGemmBK;  // elements
constexpr int kGemmBStage = kGemmBK * kGemmBN;

// s_waitcnt vmcnt(n) lgkmcnt(0) (expcnt at its maximum), and a workgroup
// barrier that is a compiler-level fence only: the direct-to-LDS loads are
// waited for explicitly, and a __syncthreads() would also wait for the
// loads still in flight for later steps.
#define RAT_WAIT_VM_LGKM(n) __builtin_amdgcn_s_waitcnt(0x0070 | (n))
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_dma_kernel(const GemmParams p) {
  // one array per stage, indexed statically: the compiler then sees that a
  // fragment read of stage s does not alias the loads in flight into the
  // other two (it would otherwise wait for all of them before every read)
  __shared__ __attribute__((aligned(1024))) bf16 sA0[kGemmAStage];
  __shared__ __attribute__((aligned(1024))) bf16 sA1[kGemmAStage];
  __shared__ __attribute__((aligned(1024))) bf16 sA2[kGemmAStage];
  __shared__ __attribute__((aligned(1024))) bf16 sB0[kGemmBStage];
  __shared__ __attribute__((aligned(1024))) bf16 sB1[kGemmBStage];
  __shared__ __attribute__((aligned(1024))) bf16 sB2[kGemmBStage];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * kGemmBN;
  const int m0 = blockIdx.y * kGemmBM;
  const int wn = wave & 1;
  const int wm = wave >> 1;
  const int N = p.ngroups * p.Ng;

  // this lane's sources: A instructions j < 4 cover rows 16 (4 wave + j) ..
  // +15 of the tile, B instructions j < 2 rows 4 (2 wave + j) .. +3
  const bf16* asrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * (4 * wave + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int m = min(m0 + row, p.M - 1);
    asrc[j] = reinterpret_cast<const bf16*>(p.A) + (int64_t)m * p.lda + 8 * c;
  }
  const bf16* bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 4 * (2 * wave + j) + (lane >> 4);
    const int c = (lane & 15) ^ (2 * ((row & 3) | ((row >> 1) & 4)));
    const int n = min(n0 + 8 * c, N - 8);
    const int grp = n / p.Ng;
    bsrc[j] = reinterpret_cast<const bf16*>(p.B[grp]) + (int64_t)row * p.ldb + (n - grp * p.Ng);
  }
  auto issue = [&](bf16* sa, bf16* sb, int ks) {
    const int64_t k0 = (int64_t)ks * kGemmBK;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(asrc[j] + k0),
                                       (lds_void_t*)(sa + (4 * wave + j) * 16 * kGemmBK), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[j] + k0 * p.ldb),
                                       (lds_void_t*)(sb + (2 * wave + j) * 4 * kGemmBN), 16, 0, 0);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const bf16* sa, const bf16* sb) {
    Frag<bf16> af[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int r = 128 * wm + 16 * mb + col;
      af[mb] = frag_ld8(sa + r * kGemmBK + 8 * (g ^ ((r >> 2) & 3)));
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // rows 8g + (col >> 2) and, one read later, 4 rows on (same swizzle)
      const int kr = 8 * g + (col >> 2);
      const int c = 8 * wn + 2 * nb + ((col & 3) >> 1);
      const int f = (kr & 3) | ((kr >> 1) & 4);
      const Frag<bf16> bfr =
          frag_ld_tr(sb + kr * kGemmBN + 8 * (c ^ (2 * f)) + 4 * (col & 1), 4 * kGemmBN);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) mma16(acc[nb][mb], bfr, af[mb]);
    }
  };

  const int nks = p.K / kGemmBK;
  // step s computes stage s % 3: once this wave's loads of step s are done
  // (at most the next step's six outstanding) the barrier makes every wave's
  // part visible and frees stage (s + 2) % 3, read at step s - 1, for the
  // loads of step s + 2
  auto step = [&](int s, const bf16* sa, const bf16* sb, bf16* na, bf16* nb2) {
    if (s + 1 < nks)
      RAT_WAIT_VM_LGKM(6);
    else
      RAT_WAIT_VM_LGKM(0);
    lds_barrier();
    if (s + 2 < nks) issue(na, nb2, s + 2);
    if (s < nks) compute(sa, sb);
  };
  issue(sA0, sB0, 0);
  if (nks > 1) issue(sA1, sB1, 1);
  for (int s0 = 0; s0 < nks; s0 += 3) {
    step(s0, sA0, sB0, sA2, sB2);
    step(s0 + 1, sA1, sB1, sA0, sB0);
    step(s0 + 2, sA2, sB2, sA1, sB1);
  }

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
    const dim3 grid((unsigned)((N + kGemmBN - 1) / kGemmBN),
                    (unsigned)((p.M + kGemmBM - 1) / kGemmBM));
    if (p.K % kGemmBK == 0 && p.K > 0)
      hipLaunchKernelGGL(gemm_bf16_dma_kernel, grid, dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, st, p);
  } else {
    const int64_t n = (int64_t)p.M * N;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  }
  return (int)hipGetLastError();
}

}  // namespace rat
