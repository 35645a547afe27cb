// Fused indexer preprocessing and quantisation (gfx950).
//
// Keys: LayerNorm over D (pinned pairwise halving sums), then RoPE, then quantisation.
// Queries: RoPE, then quantisation. Everything runs in fp32 with one rounding per
// operation (this file is built without floating-point contraction); with rope_fp32 off
// the input and the output of RoPE are rounded to bf16 (the default path's materialised
// BF16, Megatron-LM PR 8403, "What does this PR do?" and "Motivation").
//
// Layouts. Queries: one vector (t,h) of D elements per group of D/16 lanes, lane g holding
// the 16 contiguous elements 16g .. 16g+15. Keys: one token per
// group of 16 lanes, lane g holding elements g, g+16, g+32, ... so that the halving sum
// a[i] += a[i+n] is in-lane for n >= 16 and a single shuffle for n = 8, 4, 2, 1.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

struct PreArgs {
  const void* q_in; const void* k_in;
  int T, S, H, D;
  const int32_t* cu; int B;
  const float* gamma; const float* beta; float eps;
  const float* cos_t; const float* sin_t;
  int R, max_pos, interleaved, rope_fp32;
  void* q_op; uint8_t* q_scale; void* k_op; uint8_t* k_scale;
  float* q_f32; float* k_f32;
  // query thread split (see preprocess_q): parts per vector with rotated elements, and
  // ceil(2^16 / n) for n = nr and n = D/16 - nr (0 when n = 0): x / n = (x * m) >> 16 for x < 256
  int q_nr, q_mul_r, q_mul_p;
};

__device__ __forceinline__ int token_position(const int32_t* cu, int B, int T, int t) {
  int b = find_doc(cu, B, t);
  int start = clampi(__ldg(cu + b), 0, T);
  return max(0, t - start);
}

// ------------------------------------------------------------------ queries

// Max over lane groups of fp32 magnitudes (non-negative floats order like their bits):
// 16 lanes = one DPP row, 8 lanes = half a row, 4 lanes = a quad, 2 lanes = a pair.
template <int N>
__device__ __forceinline__ float group_amax(float a) {
  uint32_t m = f2u(a);
  if (N == 1) return a;
  if (N == 16) {
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x121, 0xf, 0xf, false));   // row_ror:1
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x122, 0xf, 0xf, false));   // row_ror:2
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x124, 0xf, 0xf, false));   // row_ror:4
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xf, 0xf, false));   // row_ror:8
  } else {
    if (N == 8) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xf, 0xf, false));  // row_half_mirror
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    if (N >= 4) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xf, 0xf, false));  // quad_perm [2,3,0,1]
  }
  return u2f(m);
}

// E4M3 codes of x * 2^-e, four per word (exact scaling; the codes are the
// round-to-nearest-even ones, which the gfx950 conversion produces bit for bit for
// |values| <= 448).
template <int N>
__device__ __forceinline__ void e4m3_pack(const float (&x)[N], int e, uint32_t (&w)[N / 4]) {
#pragma unroll
  for (int h = 0; h < N / 4; ++h) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * h], -e), ldexpf(x[4 * h + 1], -e), 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * h + 2], -e), ldexpf(x[4 * h + 3], -e), v, true);
    w[h] = (uint32_t)v;
  }
}

// N contiguous input elements (bf16 bits or fp32) at element offset `off`, widened to fp32.
template <bool IN_BF16, int N>
__device__ __forceinline__ void load_in(const void* base, long long off, float (&x)[N]) {
  if (IN_BF16) {
#pragma unroll
    for (int c = 0; c < N / 8; ++c) {
      const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off + 8 * c);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * c + 2 * j] = u2f(w[j] << 16);
        x[8 * c + 2 * j + 1] = u2f(w[j] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off + 4 * c);
      x[4 * c] = f.x; x[4 * c + 1] = f.y; x[4 * c + 2] = f.z; x[4 * c + 3] = f.w;
    }
  }
}

// The same loads as load_in, kept as raw words (converted later by convert_in), so that
// loads issued before a branch stay in flight across it.
template <bool IN_BF16, int N>
using RawIn = uint4[IN_BF16 ? N / 8 : N / 4];

template <bool IN_BF16, int N>
__device__ __forceinline__ void load_raw(const void* base, long long off, RawIn<IN_BF16, N>& r) {
  constexpr int NR = IN_BF16 ? N / 8 : N / 4;
#pragma unroll
  for (int c = 0; c < NR; ++c)
    r[c] = IN_BF16 ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off + 8 * c)
                   : *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + off + 4 * c);
}

template <bool IN_BF16, int N>
__device__ __forceinline__ void convert_in(const RawIn<IN_BF16, N>& r, float (&x)[N]) {
  constexpr int NR = IN_BF16 ? N / 8 : N / 4;
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    const uint32_t w[4] = {r[c].x, r[c].y, r[c].z, r[c].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (IN_BF16) {
        x[8 * c + 2 * j] = u2f(w[j] << 16);
        x[8 * c + 2 * j + 1] = u2f(w[j] & 0xFFFF0000u);
      } else {
        x[4 * c + j] = u2f(w[j]);
      }
    }
  }
}

template <int N>
__device__ __forceinline__ void load_f32(const float* p, float (&x)[N]) {
#pragma unroll
  for (int c = 0; c < N / 4; ++c) {
    const float4 f = reinterpret_cast<const float4*>(p)[c];
    x[4 * c] = f.x; x[4 * c + 1] = f.y; x[4 * c + 2] = f.z; x[4 * c + 3] = f.w;
  }
}

// One (t, h) query vector per D/NE lanes; the lane of part g owns elements NE*g .. NE*g+NE-1.
// With rotate-half RoPE a lane's elements must rotate together: NE divides rope_dim/2.
// A block's VPB vectors are split by part: the threads first hold the parts that RoPE
// touches (the last nr parts of every vector), then the others, so that whole waves either
// rotate or not (a wave with both kinds would run both code paths). The scale's magnitude
// maximum then spans waves: each part writes its maximum to its own LDS slot and, after one
// barrier, every lane takes the maximum over the slots of its scale block.
template <int D, bool IN_BF16, int PREC, int NE>
__device__ __forceinline__ void preprocess_q(const PreArgs& a, int block) {
  constexpr int G = D / NE;                      // lanes per vector
  constexpr int VPB = 256 / G;                   // vectors per block
  constexpr int NS = PREC == kPrecFP8 ? 1 : D / 32;   // scales per vector
  __shared__ __attribute__((aligned(16))) uint32_t amax_s[PREC == kPrecBF16 ? 1 : VPB * G];   // [vector][part]
  static_assert(NE == 16, "the split factors are computed for 16 elements per lane");
  const int nr = a.q_nr;                         // parts per vector with rotated elements
  const int tau = threadIdx.x;
  int vb, g;                                     // vector within the block, part
  if (tau < VPB * nr) {
    vb = (tau * a.q_mul_r) >> 16;
    g = G - nr + (tau - vb * nr);
  } else {
    const int x = tau - VPB * nr;
    vb = (x * a.q_mul_p) >> 16;
    g = x - vb * (G - nr);
  }
  const long long nvec = (long long)a.T * a.H;
  const long long v_raw = (long long)block * VPB + vb;
  const bool valid = v_raw < nvec;
  const long long v = valid ? v_raw : 0;         // past the end: vector 0 is read, nothing stored
  const int t = (int)(v / a.H);
  const long long base = v * D + NE * g;
  const int e0 = NE * g;                         // first element of this lane

  // Every load that does not need the token's position is issued first (the vector part, and
  // for rotate-half RoPE its partner half a rotation away in the same vector, read from memory
  // — the partner lane's cache lines — rather than exchanged between lanes); the position
  // lookup follows while they are in flight, then the angle table.
  const bool rot_half = a.R > 0 && !a.interleaved && e0 >= D - a.R;   // uniform per wave
  const bool first = e0 < D - a.R / 2;           // first half of the rotated dims
  // document boundaries for the position lookup, one per lane (fewer than 64 documents)
  const int lane = threadIdx.x & 63;
  const bool wave_cu = a.R > 0 && a.B < 64;
  const int cb = wave_cu && lane < a.B ? __ldg(a.cu + lane) : 0;
  RawIn<IN_BF16, NE> rx, rp;
  load_raw<IN_BF16, NE>(a.q_in, base, rx);
  if (rot_half) load_raw<IN_BF16, NE>(a.q_in, base + (first ? a.R / 2 : -(a.R / 2)), rp);
  int pos = 0;
  if (a.R > 0) {
    // a wave's vectors normally belong to one token: its document is then the last b with
    // cu[b] <= t, found by a ballot over the boundaries loaded above (else a binary search)
    const int t0 = __builtin_amdgcn_readfirstlane(t);
    int tpos;
    if (wave_cu && __all(t == t0)) {
      const unsigned long long m = __ballot(lane < a.B && cb <= t0);
      const int b = m ? 63 - __clzll((long long)m) : 0;
      tpos = max(0, t0 - clampi(__builtin_amdgcn_readlane(cb, b), 0, a.T));
    } else {
      tpos = token_position(a.cu, a.B, a.T, t);
    }
    pos = min(tpos, a.max_pos - 1);
  }
  float x[NE];
  convert_in<IN_BF16, NE>(rx, x);
  if (!IN_BF16 && !a.rope_fp32) {
#pragma unroll
    for (int j = 0; j < NE; ++j) x[j] = bf16_round(x[j]);
  }

  if (a.R > 0) {
    const int rs = D - a.R;
    const int half = a.R / 2;
    const float* crow = a.cos_t + (long long)pos * half;
    const float* srow = a.sin_t + (long long)pos * half;
    if (a.interleaved) {
#pragma unroll
      for (int j = 0; j < NE; j += 2) {
        const int e = e0 + j;
        if (e >= rs) {
          const int col = (e - rs) / 2;
          const float c = crow[col], s = srow[col];
          const float x1 = x[j], x2 = x[j + 1];
          x[j] = x1 * c - x2 * s;
          x[j + 1] = x2 * c + x1 * s;
        }
      }
    } else if (rot_half) {
      // rotate-half (NE divides rope_dim / 2, so a lane's elements rotate together)
      float p[NE];
      convert_in<IN_BF16, NE>(rp, p);
      if (!IN_BF16 && !a.rope_fp32) {
#pragma unroll
        for (int j = 0; j < NE; ++j) p[j] = bf16_round(p[j]);
      }
      const int col = e0 - rs - (first ? 0 : half);
      float c[NE], sn[NE];
      load_f32<NE>(crow + col, c);
      load_f32<NE>(srow + col, sn);
#pragma unroll
      for (int j = 0; j < NE; ++j) x[j] = first ? (x[j] * c[j] - p[j] * sn[j]) : (x[j] * c[j] + p[j] * sn[j]);
    }
    if (!a.rope_fp32) {
#pragma unroll
      for (int j = 0; j < NE; ++j) x[j] = bf16_round(x[j]);
    }
  }

  if (a.q_f32 && valid) {
    float4* o = reinterpret_cast<float4*>(a.q_f32 + base);
#pragma unroll
    for (int c = 0; c < NE / 4; ++c) o[c] = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
  }

  if (PREC == kPrecBF16) {
    uint32_t w[NE / 2];
#pragma unroll
    for (int j = 0; j < NE / 2; ++j)
      w[j] = (uint32_t)f32_to_bf16_rne(x[2 * j]) | ((uint32_t)f32_to_bf16_rne(x[2 * j + 1]) << 16);
    uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.q_op) + base);
    if (valid) {
#pragma unroll
      for (int c = 0; c < NE / 8; ++c) o[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
    }
  } else {
    // magnitude maximum per scale block (the vector for FP8, 32 elements for MXFP8): each
    // part's maximum to its own LDS slot, then the maximum over the block's parts
    // (non-negative floats order like their bits)
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < NE; ++j) amax = fmaxf(amax, fabsf(x[j]));
    amax_s[vb * G + g] = f2u(amax);
    __syncthreads();
    constexpr int PB = NS == 1 ? G : 32 / NE;    // parts per scale block
    const int p0 = NS == 1 ? 0 : (g / PB) * PB;
    uint32_t mb = 0u;
#pragma unroll
    for (int q = 0; q < PB; ++q) mb = max(mb, amax_s[vb * G + p0 + q]);
    const int e = ue8m0_exponent(u2f(mb));
    uint32_t w[NE / 4];
    e4m3_pack<NE>(x, e, w);
    if (valid) {
      if (e0 % (NS == 1 ? D : 32) == 0) a.q_scale[v * NS + (NS == 1 ? 0 : e0 / 32)] = (uint8_t)(e + 127);
      uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(a.q_op) + base);
#pragma unroll
      for (int c = 0; c < NE / 16; ++c) o[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
    }
  }
}

// ------------------------------------------------------------------ keys

template <int D, bool IN_BF16, int PREC>
__device__ __forceinline__ void preprocess_k(const PreArgs& a, int block) {
  constexpr int V = D / 16;                      // elements per lane
  const int g = threadIdx.x & 15;
  const int lane = threadIdx.x & 63;
  const int gbase = lane - g;
  const int s_raw = block * 16 + threadIdx.x / 16;
  const bool live = s_raw < a.S;
  const int s = live ? s_raw : 0;

  float x[V];
#pragma unroll
  for (int m = 0; m < V; ++m) {
    const long long off = (long long)s * D + g + 16 * m;
    x[m] = IN_BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.k_in)[off])
                   : reinterpret_cast<const float*>(a.k_in)[off];
  }

  if (a.gamma) {
    // pinned halving sum: for n = D/2 .. 1: a[i] += a[i+n], i < n
    auto tree = [&](const float* val) -> float {
      float v[V];
#pragma unroll
      for (int m = 0; m < V; ++m) v[m] = val[m];
#pragma unroll
      for (int n = V / 2; n >= 1; n >>= 1) {
#pragma unroll
        for (int m = 0; m < n; ++m) v[m] = v[m] + v[m + n];
      }
      float r = v[0];
#pragma unroll
      for (int n = 8; n >= 1; n >>= 1) {
        const float o = __shfl(r, gbase + ((g + n) & 15), 64);
        if (g < n) r = r + o;
      }
      return __shfl(r, gbase, 64);
    };
    const float inv_d = 1.0f / (float)D;
    const float mean = tree(x) * inv_d;
    float d[V], dd[V];
#pragma unroll
    for (int m = 0; m < V; ++m) { d[m] = x[m] - mean; dd[m] = d[m] * d[m]; }
    const float var = tree(dd) * inv_d;
    // correctly rounded sqrt and divide (the library is built with
    // -fhip-fp32-correctly-rounded-divide-sqrt and without denormal flushing)
    const float rstd = 1.0f / sqrtf(var + a.eps);
#pragma unroll
    for (int m = 0; m < V; ++m) {
      const int e = g + 16 * m;
      const float y = (d[m] * rstd) * a.gamma[e];
      x[m] = y + (a.beta ? a.beta[e] : 0.0f);
    }
  }
  if (!a.rope_fp32) {
#pragma unroll
    for (int m = 0; m < V; ++m) x[m] = bf16_round(x[m]);
  }

  if (a.R > 0) {
    const int rs = D - a.R;
    const int pos = min(token_position(a.cu, a.B, a.S, s), a.max_pos - 1);
    const int half = a.R / 2;
    const float* crow = a.cos_t + (long long)pos * half;
    const float* srow = a.sin_t + (long long)pos * half;
    if (a.interleaved) {
#pragma unroll
      for (int m = 0; m < V; ++m) {
        const int e = g + 16 * m;
        const float p = __shfl_xor(x[m], 1, 64);
        if (e >= rs) {
          const int col = (e - rs) / 2;
          const float c = crow[col], sn = srow[col];
          x[m] = (e & 1) ? (x[m] * c + p * sn) : (x[m] * c - p * sn);
        }
      }
    } else {
      const int mh = half / 16;                  // partner is m +- mh, in-lane
      float y[V];
#pragma unroll
      for (int m = 0; m < V; ++m) {
        const int e = g + 16 * m;
        y[m] = x[m];
        if (e >= rs) {
          const bool first = e < rs + half;
          const int col = e - rs - (first ? 0 : half);
          const float c = crow[col], sn = srow[col];
          float p = 0.f;
#pragma unroll
          for (int mm = 0; mm < V; ++mm)
            if (mm == (first ? m + mh : m - mh)) p = x[mm];
          y[m] = first ? (x[m] * c - p * sn) : (x[m] * c + p * sn);
        }
      }
#pragma unroll
      for (int m = 0; m < V; ++m) x[m] = y[m];
    }
    if (!a.rope_fp32) {
#pragma unroll
      for (int m = 0; m < V; ++m) x[m] = bf16_round(x[m]);
    }
  }

  if (a.k_f32 && live) {
#pragma unroll
    for (int m = 0; m < V; ++m) a.k_f32[(long long)s * D + g + 16 * m] = x[m];
  }

  if (PREC == kPrecBF16) {
    if (live) {
#pragma unroll
      for (int m = 0; m < V; ++m)
        reinterpret_cast<uint16_t*>(a.k_op)[(long long)s * D + g + 16 * m] = f32_to_bf16_rne(x[m]);
    }
  } else if (PREC == kPrecFP8) {
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < V; ++m) amax = fmaxf(amax, fabsf(x[m]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const int e = ue8m0_exponent(amax);
    if (live) {
#pragma unroll
      for (int m = 0; m < V; ++m)
        reinterpret_cast<uint8_t*>(a.k_op)[(long long)s * D + g + 16 * m] = (uint8_t)e4m3_encode(ldexpf(x[m], -e));
      if (g == 0) a.k_scale[s] = (uint8_t)(e + 127);
    }
  } else {
#pragma unroll
    for (int b = 0; b < V / 2; ++b) {            // 32-element block b = slots m = 2b, 2b+1
      float amax = fmaxf(fabsf(x[2 * b]), fabsf(x[2 * b + 1]));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const int e = ue8m0_exponent(amax);
      if (live) {
        uint8_t* o = reinterpret_cast<uint8_t*>(a.k_op) + (long long)s * D;
        o[g + 32 * b] = (uint8_t)e4m3_encode(ldexpf(x[2 * b], -e));
        o[g + 32 * b + 16] = (uint8_t)e4m3_encode(ldexpf(x[2 * b + 1], -e));
        if (g == 0) a.k_scale[(long long)s * (D / 32) + b] = (uint8_t)(e + 127);
      }
    }
  }
}

// One launch: the first blocks preprocess keys (16 tokens each), the rest queries.
template <int D, bool IN_BF16, int PREC, int NE>
__global__ __launch_bounds__(256) void preprocess_kernel(PreArgs a, int k_blocks) {
  if ((int)blockIdx.x < k_blocks) preprocess_k<D, IN_BF16, PREC>(a, blockIdx.x);
  else preprocess_q<D, IN_BF16, PREC, NE>(a, blockIdx.x - k_blocks);
}

template <int D, bool IN_BF16, int PREC, int NE>
hipError_t launch_pre_ne(const PreArgs& a, hipStream_t st) {
  constexpr int qvpb = 256 / (D / NE);           // query vectors per block
  const long long q_blocks = (a.q_in && a.T > 0) ? ((long long)a.T * a.H + qvpb - 1) / qvpb : 0;
  const long long k_blocks = (a.k_in && a.S > 0) ? (a.S + 15) / 16 : 0;
  if (q_blocks + k_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((preprocess_kernel<D, IN_BF16, PREC, NE>), dim3((unsigned)(q_blocks + k_blocks)), dim3(256), 0,
                     st, a, (int)k_blocks);
  return hipGetLastError();
}

template <int D, bool IN_BF16, int PREC>
hipError_t launch_pre(const PreArgs& a, hipStream_t st) {
  return launch_pre_ne<D, IN_BF16, PREC, 16>(a, st);
}

template <int D, bool IN_BF16>
hipError_t launch_pre_p(const PreArgs& a, int prec, hipStream_t st) {
  switch (prec) {
    case kPrecBF16: return launch_pre<D, IN_BF16, kPrecBF16>(a, st);
    case kPrecFP8: return launch_pre<D, IN_BF16, kPrecFP8>(a, st);
    default: return launch_pre<D, IN_BF16, kPrecMXFP8>(a, st);
  }
}

}  // namespace

hipError_t launch_preprocess(const PreprocessLaunch& p, hipStream_t st) {
  PreArgs a;
  a.q_in = p.q_in; a.k_in = p.k_in;
  a.T = p.T; a.S = p.S; a.H = p.H; a.D = p.D;
  a.cu = p.cu; a.B = p.B;
  a.gamma = p.gamma; a.beta = p.beta; a.eps = p.eps;
  a.cos_t = p.cos_t; a.sin_t = p.sin_t;
  a.R = p.rope_dim; a.max_pos = p.max_pos; a.interleaved = p.interleaved; a.rope_fp32 = p.rope_fp32;
  a.q_op = p.q_op; a.q_scale = p.q_scale; a.k_op = p.k_op; a.k_scale = p.k_scale;
  a.q_f32 = p.q_f32; a.k_f32 = p.k_f32;
  {
    const int G = p.D / 16;
    a.q_nr = p.rope_dim > 0 ? G - (p.D - p.rope_dim) / 16 : 0;
    a.q_mul_r = a.q_nr > 0 ? (65536 + a.q_nr - 1) / a.q_nr : 0;
    a.q_mul_p = G - a.q_nr > 0 ? (65536 + (G - a.q_nr) - 1) / (G - a.q_nr) : 0;
  }
  if (p.D == 128) return p.in_bf16 ? launch_pre_p<128, true>(a, p.precision, st) : launch_pre_p<128, false>(a, p.precision, st);
  return p.in_bf16 ? launch_pre_p<64, true>(a, p.precision, st) : launch_pre_p<64, false>(a, p.precision, st);
}

}  // namespace dsa
