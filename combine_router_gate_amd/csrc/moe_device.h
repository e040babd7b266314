// Device helpers for the gfx950 (CDNA4) MoE kernels: 16-byte vector types,
// bf16 / OCP-E4M3 conversions, order-preserving keys and 16-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kTileT = 64;         // tokens per histogram tile (one bit each)
constexpr int kFp8Block = 128;     // hidden elements per fp8 scale
constexpr float kFp8Max = 448.0f;  // largest finite E4M3FN magnitude

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));   // 8 bytes

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming load: data read once, kept out of the caches' retained set.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// Streaming store: output not re-read by this kernel; skips cache allocation.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t packed) {
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xffff0000u);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 bf16 (one 16-byte vector) <-> 8 fp32
__device__ __forceinline__ void unpack8_bf16(const u32x4& v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
__device__ __forceinline__ u32x4 pack8_bf16(const float f[8]) {
  u32x4 v;
  v.x = pack_bf16x2(f[0], f[1]);
  v.y = pack_bf16x2(f[2], f[3]);
  v.z = pack_bf16x2(f[4], f[5]);
  v.w = pack_bf16x2(f[6], f[7]);
  return v;
}

// ------------------------------------------------------------------ E4M3
// OCP 8-bit floating point, E4M3 ("FN") variant: bias 7, 3 mantissa bits,
// exponent field 0 subnormal (m * 2^-9), S.1111.111 NaN, no infinities.

// Four fp32 -> four E4M3 codes (byte i = value i) with the gfx950 converter
// v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even, sign of zero kept).
// Inputs are clamped to +-448 first, which makes the result saturating.  The
// fp8 dispatch parity tests pin this path against an independent encoder on
// every E4M3 value, every rounding midpoint and their fp32 neighbours.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c,
                                                 float d) {
  a = fmaxf(fminf(a, kFp8Max), -kFp8Max);
  b = fmaxf(fminf(b, kFp8Max), -kFp8Max);
  c = fmaxf(fminf(c, kFp8Max), -kFp8Max);
  d = fmaxf(fminf(d, kFp8Max), -kFp8Max);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t ef = (c >> 3) & 0xfu, mf = c & 7u;
  float mag;
  if (ef == 0) {
    mag = (float)mf * 0.001953125f;                   // m * 2^-9
  } else {
    mag = __uint_as_float(((ef + 120u) << 23) | (mf << 20));
  }
  if (ef == 15 && mf == 7) mag = __builtin_nanf("");
  return (c & 0x80u) ? -mag : mag;
}

// ------------------------------------------------------------------ barrier

// Workgroup barrier for LDS traffic only: this wave's LDS operations
// complete, then s_barrier.  __syncthreads() also waits for every
// outstanding global load of the wave (its fence semantics), which would
// drain a software-pipelined prefetch at each step; this one keeps them in
// flight.  Only valid where the barrier orders LDS accesses alone.
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------------------ LDS copies

// Direct global->LDS copy of 16 (or 4) bytes per lane from base + off: lane
// l's data lands at lds + 16 l (+ 4 l).  Issued from inline assembly so the
// compiler, which would otherwise wait for every copy in flight before any
// LDS read, leaves the waiting to the caller's pipeline (s_waitcnt vmcnt(n)
// counts these copies in issue order).  The copy takes its LDS address from
// M0, which is saved and restored around it; one wait state separates the
// write of M0 from the copy that reads it.  The copy has no register result.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void copy_to_lds16(const void* base, uint32_t off,
                                              uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(uniform_ptr(base)),
        "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}
__device__ __forceinline__ void copy_to_lds4(const void* base, uint32_t off,
                                             uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(uniform_ptr(base)),
        "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Wait for this wave's copies and LDS operations, then meet the other waves:
// every copy the workgroup issued before the barrier has landed.
__device__ __forceinline__ void copies_barrier() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
               ::: "memory");
}

// ------------------------------------------------------------------ keys

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ------------------------------------------------------------------ reductions

// 64-bit DPP move within each row of 16 lanes (CTRL: a DPP control word).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf,
                                             0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(
      0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Maximum over each aligned group of 16 lanes (all lanes get the result):
// rotations by 8, 4, 2, 1 within the DPP row (row_ror = 0x120 + n), so the
// reduction stays in the ALU instead of round-tripping through LDS.
__device__ __forceinline__ unsigned long long max16_u64(unsigned long long v) {
  unsigned long long o;
  o = dpp_u64<0x128>(v); v = o > v ? o : v;
  o = dpp_u64<0x124>(v); v = o > v ? o : v;
  o = dpp_u64<0x122>(v); v = o > v ? o : v;
  o = dpp_u64<0x121>(v); v = o > v ? o : v;
  return v;
}

}  // namespace moe
