// Device-side helpers shared by the indexer kernels (gfx950).
//
// Number formats follow the C ABI header: bf16 round-to-nearest-even, OCP E4M3FN with
// round-to-nearest-even, UE8M0 scale exponents chosen so that payloads never saturate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bit helpers

__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __uint_as_float(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

// fp32 -> bf16 bits, nearest even; NaN stays a (quiet) NaN of the same sign.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = f2u(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16_rne(x)); }

// Smallest e with amax <= 448 * 2^e, 0 for amax == 0, clamped to [-127, 127].
// amax = 1.f * 2^(E-127): e = (E - 135) + (f > 0.75), since 448 = 1.75 * 2^8.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
  uint32_t u = f2u(amax) & 0x7FFFFFFFu;
  if (u == 0) return 0;
  int bias_fix = 0;
  if (u < 0x00800000u) {                       // subnormal: scale up exactly by 2^64
    u = f2u(u2f(u) * 18446744073709551616.0f);
    bias_fix = 64;
  }
  int E = (int)(u >> 23);
  uint32_t man = u & 0x7FFFFFu;
  int e = E - 135 + (man > 0x600000u ? 1 : 0) - bias_fix;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E4M3FN code of x with |x| <= 448, round to nearest even (x is exactly representable
// as the scaled fp32 value; the caller guarantees no saturation).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t u = f2u(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {                       // below 2^-6: quantum 2^-9 (subnormal codes)
    code = (uint32_t)__builtin_rintf(u2f(a) * 512.0f);   // 0..8; 8 is the code of 2^-6
  } else {
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // exponent(8) | mantissa(3)
    code = r - (120u << 3);
  }
  return sign | code;
}

// ---------------------------------------------------------------- buffers

constexpr int kBufferFlags = 0x00020000;   // buffer descriptor word 3: raw 32-bit data format

// Buffer descriptor over `bytes` bytes at `base` (both wave-uniform; read from lane 0 so the
// descriptor lives in scalar registers). Loads past `bytes` return zeros, stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t plo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t phi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* q = reinterpret_cast<void*>(((uint64_t)phi << 32) | plo);
  return __builtin_amdgcn_make_buffer_rsrc(q, 0, __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// ---------------------------------------------------------------- documents

// Document of token t: the b in [0, B) with cu[b] <= t < cu[b+1] (last such b for empty
// documents). cu is read on the device; values are clamped by the caller.
__device__ __forceinline__ int find_doc(const int32_t* __restrict__ cu, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (__ldg(cu + mid) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Order-preserving uint32 key of an fp32 score (-0 is folded onto +0).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = f2u(s);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return u2f(u);
}

}  // namespace dsa
