// Device-side building blocks shared by the RAT+ kernels (gfx950 only).
//
// Storage types: bf16 (8 per 16-byte vector) and fp32 (4 per vector).  All
// arithmetic is fp32; bf16 stores round to nearest even (gfx950 has a
// hardware pack-convert for this).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rat_params.h"

namespace rat {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename ST>
struct StTraits;
template <>
struct StTraits<bf16> {
  static constexpr int VEC = 8;  // elements per 16-byte vector
};
template <>
struct StTraits<float> {
  static constexpr int VEC = 4;
};

// ---------------------------------------------------------------------------
// 16-byte vector load / store with conversion to / from fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ u32x4 ld_raw16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld_raw16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_raw16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// raw 16 bytes -> fp32 values
__device__ __forceinline__ void unpack16(const u32x4& u, float (&f)[8], bf16*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(u[i]);
    f[2 * i + 1] = bf16_hi(u[i]);
  }
}
__device__ __forceinline__ void unpack16(const u32x4& u, float (&f)[4], float*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
}
// fp32 values -> raw 16 bytes
__device__ __forceinline__ u32x4 pack16(const float (&f)[8], bf16*) {
  u32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return u;
}
__device__ __forceinline__ u32x4 pack16(const float (&f)[4], float*) {
  u32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __float_as_uint(f[i]);
  return u;
}

// round one fp32 value to the storage type and back (what a store + load
// of that value would give)
__device__ __forceinline__ float st_round(float x, bf16*) {
  return bf16_lo(pack_bf16x2(x, 0.0f));
}
__device__ __forceinline__ float st_round(float x, float*) { return x; }

// ---------------------------------------------------------------------------
// MFMA fragments: 8 k-values per lane for one 16x16 tile step of K = 32.
//   A operand: lane l holds row (l % 16), k-slot (l / 16, j), j = 0..7
//   B operand: lane l holds col (l % 16), k-slot (l / 16, j)
//   C (16x16 fp32): lane l holds col (l % 16), rows 4*(l/16) + i, i = 0..3
// The k-slot -> k mapping is free as long as A and B agree on it.
// bf16 uses one v_mfma_f32_16x16x32_bf16; fp32 uses eight
// v_mfma_f32_16x16x4_f32, the j-th on slot (l / 16, j).
// ---------------------------------------------------------------------------
template <typename ST>
struct Frag;
template <>
struct Frag<bf16> {
  bf16x8 v;
};
template <>
struct Frag<float> {
  f32x4 lo, hi;
};

__device__ __forceinline__ void mma16(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], c, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loads (global_load_lds_dwordx4) and their waits
// ---------------------------------------------------------------------------
// s_waitcnt vmcnt(n) lgkmcnt(0) (expcnt at its maximum; n < 64), and a
// workgroup barrier that is a compiler-level fence only: the direct-to-LDS
// loads are waited for explicitly, and a __syncthreads() would also wait for
// the loads still in flight for later steps.
#define RAT_WAIT_VM_LGKM(n) \
  __builtin_amdgcn_s_waitcnt(0x0070 | ((n) & 15) | (((n) >> 4) << 14))
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// global_load_lds_dwordx4 from this lane's src to LDS base dst (+ 16 bytes
// per lane; dst is the same for every lane of the wave).  Written out rather
// than through the builtin: the compiler cannot tell which LDS stage a
// builtin load writes, and waits for every one in flight before each LDS
// read.  Nothing is returned in registers (the
// address is read at issue); completion is waited for with vmcnt before the
// barrier that publishes a stage.  M0 (the LDS base) is saved and restored
// around the load, so the compiler's own use of M0 is undisturbed; one wait
// state separates the M0 write from its use.
__device__ __forceinline__ void dma16(const void* src, const bf16* dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}

// dma16 with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (the scalar-base form of the same load): no 64-bit address
// arithmetic per lane.  lds_base is the wave-uniform LDS byte address.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const bf16* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

// 8 consecutive storage elements -> fragment
__device__ __forceinline__ Frag<bf16> frag_ld8(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> frag_ld8(const float* p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}
// two groups of 4 consecutive elements -> fragment (slots j<4 from p0, j>=4 from p1)
__device__ __forceinline__ Frag<bf16> frag_ld4x2(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> frag_ld4x2(const float* p0, const float* p1) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p0);
  f.hi = *reinterpret_cast<const f32x4*>(p1);
  return f;
}
// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// 4j + i / 4 of its group, j = 0..3 (the gfx950 lane layout, checked on the
// device).  With lanes 4j..4j+3 addressing row j of a 4-row x 16-column
// block (4 columns each), lane i gets column i of the 4 rows: two reads,
// the second `step` elements further on, fill the 8 slots of an MFMA
// fragment.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ Frag<bf16> frag_ld_tr(const bf16* p, int step) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + step));
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}

// fp32 values -> fragment (slots j<4 from a, j>=4 from b)
__device__ __forceinline__ Frag<bf16> frag_from(const f32x4& a, const f32x4& b, bf16*) {
  f32x4 x = a, y = b;
  bf16x4 ha = __builtin_convertvector(x, bf16x4);
  bf16x4 hb = __builtin_convertvector(y, bf16x4);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> frag_from(const f32x4& a, const f32x4& b, float*) {
  Frag<float> f;
  f.lo = a;
  f.hi = b;
  return f;
}
// fragment scaled by c (bf16: rounded back to nearest even)
__device__ __forceinline__ Frag<bf16> frag_scale(const Frag<bf16>& f, float c) {
  f32x4 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = (float)f.v[j] * c;
    b[j] = (float)f.v[4 + j] * c;
  }
  return frag_from(a, b, (bf16*)nullptr);
}
__device__ __forceinline__ Frag<float> frag_scale(const Frag<float>& f, float c) {
  Frag<float> r;
  r.lo = f.lo * c;
  r.hi = f.hi * c;
  return r;
}
// fragment -> its 8 values in k-slot order (j = 0..7)
__device__ __forceinline__ void frag_to_f32(const Frag<bf16>& f, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)f.v[j];
}
__device__ __forceinline__ void frag_to_f32(const Frag<float>& f, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = f.lo[j];
    x[4 + j] = f.hi[j];
  }
}
// dot product of two fragments (fp32 accumulate)
__device__ __forceinline__ float frag_dot(const Frag<bf16>& a, const Frag<bf16>& b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (float)a.v[j] * (float)b.v[j];
  return s;
}
__device__ __forceinline__ float frag_dot(const Frag<float>& a, const Frag<float>& b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += a.lo[j] * b.lo[j];
#pragma unroll
  for (int j = 0; j < 4; ++j) s += a.hi[j] * b.hi[j];
  return s;
}

__device__ __forceinline__ Frag<bf16> frag_zero(bf16*) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = (bf16)0.0f;
  return f;
}
__device__ __forceinline__ Frag<float> frag_zero(float*) {
  Frag<float> f;
  f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  f.hi = f.lo;
  return f;
}

// 4 consecutive storage elements -> fp32
__device__ __forceinline__ f32x4 ld4_f32(const bf16* p) {
  u32x2 u = *reinterpret_cast<const u32x2*>(p);
  return f32x4{bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1])};
}
__device__ __forceinline__ f32x4 ld4_f32(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
// fp32 x4 -> 4 consecutive storage elements
__device__ __forceinline__ void st4(bf16* p, const f32x4& v) {
  u32x2 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *reinterpret_cast<u32x2*>(p) = u;
}
__device__ __forceinline__ void st4(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// Buffer resource over one region of < 2^31 bytes.  A buffer access at byte
// offset kDropOffset lies outside every such region: loads return 0 and
// stores are discarded by the hardware, which lets masked accesses be issued
// unconditionally (straight-line code, exact counts of outstanding memory
// operations).  dword 3 = 0x00020000: raw 32-bit data format, the gfx9
// buffer default.
constexpr uint32_t kDropOffset = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_region(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)kDropOffset, 0x00020000);
}
// fp32 x4 -> 4 consecutive bf16 at byte offset `off` of a region
__device__ __forceinline__ void buffer_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, const f32x4& v) {
  u32x2 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
}

// cross-lane helpers (wave64)
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Max / sum of v over lanes {i, i^16, i^32, i^48} on the VALU, no LDS round
// trip: with both operands equal to x, v_permlane16_swap returns x at lanes
// i and i^16 in its two outputs, and v_permlane32_swap x at i and i^32.
__device__ __forceinline__ float xor16_32_max(float v) {
  const uint32_t a = __float_as_uint(v);
  const u32x2 r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const uint32_t b = __float_as_uint(v);
  const u32x2 t = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float xor16_32_sum(float v) {
  const uint32_t a = __float_as_uint(v);
  const u32x2 r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const uint32_t b = __float_as_uint(v);
  const u32x2 t = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

}  // namespace rat
