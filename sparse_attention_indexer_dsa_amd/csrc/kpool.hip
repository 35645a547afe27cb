// KPool key compression (Megatron-LM PR 7522, "Changes"): per document, every complete
// group of kpool tokens becomes one pooled key, a softmax-weighted sum of its tokens
// with weights from a bf16 per-token gate plus an fp32 per-slot bias. Pooling restarts
// at every document; an incomplete last group is not pooled.
//
// Arithmetic is pinned so that any correct implementation agrees bit for bit: fp32,
// one rounding per operation (this file is built without contraction), the softmax sum
// and the weighted sum accumulated left to right, and the exponential `pexp` below.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

// exp(z) for z <= 0: Cody-Waite reduction with ln2 = LN2_HI + LN2_LO, degree-7 Taylor
// polynomial (coefficients fp32(1/k!)) by Horner's rule with fused multiply-adds, and
// an exact scaling by 2^n. Returns 0 below -104.
__device__ __forceinline__ float pexp(float z) {
  if (z < -104.0f) return 0.0f;
  const float n = __builtin_rintf(z * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e4p-1f, z);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float p = 0x1.a01a02p-13f;                 // 1/7!
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
  p = __builtin_fmaf(p, r, 0x1p-1f);          // 1/2!
  p = __builtin_fmaf(p, r, 0x1p+0f);          // 1/1!
  p = __builtin_fmaf(p, r, 0x1p+0f);          // 1/0!
  return ldexpf(p, (int)n);
}

// cu_pools[b] = sum over documents before b of floor(len/kpool). One block.
__global__ __launch_bounds__(256) void pool_offsets_kernel(const int32_t* __restrict__ cu, int B, int S, int kp,
                                                            int32_t* __restrict__ cu_pools) {
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int per = (B + 255) / 256;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int sum = 0;
  for (int b = b0; b < b1; ++b) {
    const int lo = clampi(cu[b], 0, S), hi = clampi(cu[b + 1], lo, S);
    sum += (hi - lo) / kp;
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {      // inclusive scan
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? part[tid - 1] : 0;
  for (int b = b0; b < b1; ++b) {
    cu_pools[b] = run;
    const int lo = clampi(cu[b], 0, S), hi = clampi(cu[b + 1], lo, S);
    run += (hi - lo) / kp;
  }
  if (tid == 255) cu_pools[B] = part[255];
}

// The pooled key of pool gp (lane holds elements lane + 64 i) in the scoring precision.
template <int D, int PREC>
__device__ __forceinline__ void store_pooled(const KpoolLaunch& a, int gp, int lane, const float (&acc)[D / 64]) {
  constexpr int E = D / 64;
  const long long orow = (long long)gp * D;
  if (PREC == kPrecBF16) {
#pragma unroll
    for (int i = 0; i < E; ++i)
      reinterpret_cast<uint16_t*>(a.pooled)[orow + lane + 64 * i] = f32_to_bf16_rne(acc[i]);
  } else if (PREC == kPrecFP8) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(acc[i]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const int e = ue8m0_exponent(amax);
#pragma unroll
    for (int i = 0; i < E; ++i)
      reinterpret_cast<uint8_t*>(a.pooled)[orow + lane + 64 * i] = (uint8_t)e4m3_encode(ldexpf(acc[i], -e));
    if (lane == 0) a.pooled_scale[gp] = (uint8_t)(e + 127);
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {               // element lane + 64 i lies in block 2i + lane/32
      float amax = fabsf(acc[i]);
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const int e = ue8m0_exponent(amax);
      reinterpret_cast<uint8_t*>(a.pooled)[orow + lane + 64 * i] = (uint8_t)e4m3_encode(ldexpf(acc[i], -e));
      if ((lane & 31) == 0) a.pooled_scale[(long long)gp * (D / 32) + 2 * i + lane / 32] = (uint8_t)(e + 127);
    }
  }
}

template <int D, bool K_BF16, int PREC>
__global__ __launch_bounds__(256) void kpool_kernel(KpoolLaunch a) {
  constexpr int E = D / 64;                      // elements per lane
  const int lane = threadIdx.x & 63;
  const int gp = blockIdx.x * 4 + threadIdx.x / 64;
  const int P = a.cu_pools[a.B];
  if (gp >= P) return;
  // document of pool gp: last b with cu_pools[b] <= gp
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_pools[mid] <= gp) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int start = clampi(a.cu[b], 0, a.S) + (gp - a.cu_pools[b]) * a.kpool;
  const int kp = a.kpool;

  // softmax weights over the pool's slots (every lane computes them redundantly)
  float m = -INFINITY;
  for (int j = 0; j < kp; ++j) m = fmaxf(m, bf16_to_f32(a.gate[start + j]) + a.bias[j]);
  float sigma = 0.f;
  for (int j = 0; j < kp; ++j) {
    const float z = bf16_to_f32(a.gate[start + j]) + a.bias[j];
    sigma = j == 0 ? pexp(z - m) : sigma + pexp(z - m);
  }

  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  for (int j = 0; j < kp; ++j) {
    const float z = bf16_to_f32(a.gate[start + j]) + a.bias[j];
    const float aj = pexp(z - m) / sigma;
    const long long row = (long long)(start + j) * D;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = lane + 64 * i;
      const float kv = K_BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.k)[row + e])
                              : reinterpret_cast<const float*>(a.k)[row + e];
      const float prod = aj * kv;
      acc[i] = j == 0 ? prod : acc[i] + prod;
    }
  }

  store_pooled<D, PREC>(a, gp, lane, acc);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the row
// broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_prefix_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// The same pooled keys with fewer than 64 documents and a compile-time pool size: every
// wave finds its pool's document itself (lane b holds document b's boundaries and pool
// count; a prefix sum gives cu_pools, which the first wave also writes, so no separate
// launch precedes this one), and all gate, bias and key loads of the pool are issued
// before any is used. The arithmetic is the generic kernel's, operation for operation.
template <int D, bool K_BF16, int PREC, int KP>
__global__ __launch_bounds__(256) void kpool_fast_kernel(KpoolLaunch a) {
  constexpr int E = D / 64;                      // elements per lane
  const int lane = threadIdx.x & 63;
  const int gp = blockIdx.x * 4 + threadIdx.x / 64;
  int lo = 0, np = 0;
  if (lane < a.B) {
    lo = clampi(a.cu[lane], 0, a.S);
    const int hi = clampi(a.cu[lane + 1], lo, a.S);
    np = (hi - lo) / KP;
  }
  const int incl = wave_prefix_sum(np);
  const int excl = incl - np;                    // cu_pools[lane] for lane < B
  const int P = __builtin_amdgcn_readlane(incl, 63);
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    if (lane < a.B) a.cu_pools[lane] = excl;
    if (lane == a.B) a.cu_pools[a.B] = P;
  }
  if (gp >= P) return;
  // document of pool gp: the last b with cu_pools[b] <= gp (lane 0 always qualifies)
  const unsigned long long m64 = __ballot(lane < a.B && excl <= gp);
  const int b = 63 - __clzll((long long)m64);
  const int start = __builtin_amdgcn_readlane(lo, b) + (gp - __builtin_amdgcn_readlane(excl, b)) * KP;

  float z[KP], kv[KP][E];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    z[j] = bf16_to_f32(a.gate[start + j]) + a.bias[j];
    const long long row = (long long)(start + j) * D;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = lane + 64 * i;
      kv[j][i] = K_BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.k)[row + e])
                        : reinterpret_cast<const float*>(a.k)[row + e];
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < KP; ++j) m = fmaxf(m, z[j]);
  float sigma = 0.f;
#pragma unroll
  for (int j = 0; j < KP; ++j) sigma = j == 0 ? pexp(z[j] - m) : sigma + pexp(z[j] - m);
  float acc[E];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const float aj = pexp(z[j] - m) / sigma;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float prod = aj * kv[j][i];
      acc[i] = j == 0 ? prod : acc[i] + prod;
    }
  }
  store_pooled<D, PREC>(a, gp, lane, acc);
}

template <int D, bool K_BF16, int PREC, int KP>
void launch_fast(const KpoolLaunch& a, int blocks, hipStream_t st) {
  hipLaunchKernelGGL((kpool_fast_kernel<D, K_BF16, PREC, KP>), dim3(blocks), dim3(256), 0, st, a);
}

template <int D, bool K_BF16, int PREC>
void launch_fast_kp(const KpoolLaunch& a, int blocks, hipStream_t st) {
  switch (a.kpool) {
    case 2: launch_fast<D, K_BF16, PREC, 2>(a, blocks, st); break;
    case 3: launch_fast<D, K_BF16, PREC, 3>(a, blocks, st); break;
    default: launch_fast<D, K_BF16, PREC, 4>(a, blocks, st); break;
  }
}

// One launch when every document fits a lane and kpool is 2, 3 or 4 (at least one
// workgroup, which writes cu_pools even when there is no pool).
template <int D, bool K_BF16>
hipError_t launch_kp_fast(const KpoolLaunch& a, hipStream_t st) {
  const int pmax = a.S / a.kpool;
  const int blocks = pmax > 0 ? (pmax + 3) / 4 : 1;
  switch (a.precision) {
    case kPrecBF16: launch_fast_kp<D, K_BF16, kPrecBF16>(a, blocks, st); break;
    case kPrecFP8: launch_fast_kp<D, K_BF16, kPrecFP8>(a, blocks, st); break;
    default: launch_fast_kp<D, K_BF16, kPrecMXFP8>(a, blocks, st); break;
  }
  return hipGetLastError();
}

template <int D, bool K_BF16>
hipError_t launch_kp(const KpoolLaunch& a, hipStream_t st) {
  const int pmax = a.S / a.kpool;
  if (pmax == 0) return hipSuccess;
  const int blocks = (pmax + 3) / 4;
  switch (a.precision) {
    case kPrecBF16: hipLaunchKernelGGL((kpool_kernel<D, K_BF16, kPrecBF16>), dim3(blocks), dim3(256), 0, st, a); break;
    case kPrecFP8: hipLaunchKernelGGL((kpool_kernel<D, K_BF16, kPrecFP8>), dim3(blocks), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((kpool_kernel<D, K_BF16, kPrecMXFP8>), dim3(blocks), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kpool(const KpoolLaunch& a, hipStream_t st) {
  if (a.B < 64 && a.kpool >= 2 && a.kpool <= 4) {
    if (a.D == 128) return a.k_bf16 ? launch_kp_fast<128, true>(a, st) : launch_kp_fast<128, false>(a, st);
    return a.k_bf16 ? launch_kp_fast<64, true>(a, st) : launch_kp_fast<64, false>(a, st);
  }
  hipLaunchKernelGGL(pool_offsets_kernel, dim3(1), dim3(256), 0, st, a.cu, a.B, a.S, a.kpool, a.cu_pools);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.D == 128) return a.k_bf16 ? launch_kp<128, true>(a, st) : launch_kp<128, false>(a, st);
  return a.k_bf16 ? launch_kp<64, true>(a, st) : launch_kp<64, false>(a, st);
}

}  // namespace dsa
