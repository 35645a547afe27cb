// Indexer scoring on gfx950 matrix cores.
//
// For query t and candidate c (a key, or a pooled key when kpool > 1):
//     I[t,c] = sm_scale * sum_h w[t,h] * ReLU(q[t,h,:] . k[c,:])
// (Megatron-LM PR 8403: per-head weights passed to the scoring call, codex review
// finding 3; ReLU scoring, finding 1.) The q.k contraction over D runs on MFMA with fp32
// accumulation; ReLU, the weights, the head sum and the causal mask are applied to the
// MFMA result in registers, so per-head logits never leave the chip. Only the per-query
// scores of causal candidates are written, to the score workspace (row stride fixed).
//
// Work decomposition. A workgroup of 4 waves owns 256/H consecutive query tokens of one
// document; each wave owns 64 MFMA rows = 64/H tokens x H heads, whose q operands stay in
// registers for the whole sweep. The workgroup sweeps the document's causal keys in LDS
// tiles of 64 keys (two 32-key MFMA column blocks). Workgroups are numbered from the end
// of the documents so the longest causal rows start first. FP8 and MXFP8 tiles go from HBM
// straight into LDS (no staging registers), which lets those kernels run 3 waves per SIMD;
// bf16 tiles pass through registers at 2 waves per SIMD.
//
// MFMA shapes (lane l, h = l/32):
//   bf16  v_mfma_f32_32x32x16_bf16: A lane holds row l%32, k = 8h .. 8h+7.
//   fp8   v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3): A lane holds row l%32,
//         bytes 0-15 = k 16h..16h+15, bytes 16-31 = k 32+16h..32+16h+15; the scale of
//         32-element block j of row m is supplied by lane m + 32j. B mirrors A.
//   C (32x32 fp32): lane l holds column l%32, rows 8(i/4) + 4h + (i%4), i = 0..15.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kNK = 64;          // keys per LDS tile
constexpr int kThreads = 256;

struct ScoreArgs {
  const void* q_op; const uint8_t* q_scale;
  const void* k_op; const uint8_t* k_scale;
  const void* w; int w_bf16;
  // raw queries when the query preprocessing is done in this kernel (FUSE)
  const void* q_in; int in_bf16;
  const float* cos_t; const float* sin_t;
  int R, max_pos, interleaved, rope_fp32;
  void* q_op_out; uint8_t* q_scale_out;    // optional copies of the operands built (FUSE)
  int T, S, B, max_seqlen, kpool;
  const int32_t* cu; const int32_t* cu_pools;
  float sm_scale;
  float* scores; int stride; int max_cand;
  int ntiles;                    // query tiles per document (ceil(max_seqlen / tokens per workgroup))
};

__device__ __forceinline__ float relu(float x) {
  // max(x, 0) on the bit pattern: negative values (sign bit set, -0 included) become +0;
  // one integer max, without the quieting step a float max needs in IEEE mode
  return u2f((uint32_t)max((int)f2u(x), 0));
}

__device__ __forceinline__ float pair_sum(float x) {
  // lanes l and l^32 hold the two halves of the rows of one column: add them
  auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f(r[0]) + u2f(r[1]);
}

// Sum over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ int wave_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

// Query tile of block j. Tiles of all documents are taken in one order: tile index p
// descending (longest causal rows first), documents ascending within a level, empty tiles
// skipped. The hardware deals consecutive blocks to the XCDs in turn, so every XCD gets an
// equal share of every length class (a block-to-document map by block index modulo the
// document count would tie documents to XCDs). Up to 64 documents are handled this way (one
// per lane; the search is a binary search on the number of tiles at level >= p); with more,
// documents interleave by block index. Returns false for blocks past the last tile.
__device__ __forceinline__ bool tile_of_block(const ScoreArgs& a, int tq, int j, int& b_out, int& p_out) {
  if (a.B > 64) {
    b_out = j % a.B;
    p_out = a.ntiles - 1 - j / a.B;
    return true;
  }
  const int lane = threadIdx.x & 63;
  int nt = 0;                                    // tiles of document `lane`
  if (lane < a.B) {
    const int lo = clampi(a.cu[lane], 0, a.T), hi = clampi(a.cu[lane + 1], lo, a.T);
    nt = (min(hi - lo, a.max_seqlen) + tq - 1) / tq;
  }
  auto count_ge = [&](int p) { return wave_sum(max(0, nt - p)); };   // tiles with index >= p
  if (count_ge(0) <= j) return false;
  int plo = 0, phi = a.ntiles - 1;               // invariant: count_ge(plo) > j
  while (plo < phi) {
    const int mid = (plo + phi + 1) >> 1;
    if (count_ge(mid) > j) plo = mid; else phi = mid - 1;
  }
  const int r = j - count_ge(plo + 1);           // rank among the documents with tile plo
  const unsigned long long has = __ballot(nt > plo);
  const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(has >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)has, 0));
  const unsigned long long hit = __ballot(nt > plo && before == r);
  b_out = __ffsll((long long)hit) - 1;
  p_out = plo;
  return true;
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): the wave's
// 64 lanes fill 1 KB at `lds` in lane order.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

template <int PREC>
using AOperand = typename std::conditional<PREC != kPrecBF16, i32x8, bf16x8>::type;

// Query operands of one operand row built in registers from the raw query vector (fused
// preprocessing): the same steps, in the same fp32 arithmetic, as the preprocessing kernel
// (bf16 carrier rounding when rope_fp32 is off, RoPE, then bf16 RNE, or UE8M0 scale + E4M3
// codes), but on the elements this lane holds in the MFMA A layout. The lane holds NG groups
// of GS contiguous elements of the vector: fp8 group g = (kk, s) starts at 32 g + 16 hl
// (GS = 16), bf16 group kk at 16 kk + 8 hl (GS = 8); the other half of the vector is in lane
// l ^ 32. Rotate-half partners are in-lane (group g + half / GSTEP): the host takes the
// fused path only when half is a multiple of GSTEP.
template <int D, int PREC>
__device__ __forceinline__ void build_q_row(const ScoreArgs& a, long long vec, bool ok, int pos, int hl,
                                            AOperand<PREC> (&aop)[(PREC != kPrecBF16) ? D / 64 : D / 16],
                                            int (&asc)[(PREC != kPrecBF16) ? D / 64 : D / 16]) {
  constexpr bool kFP8 = PREC != kPrecBF16;
  constexpr int GS = kFP8 ? 16 : 8;              // elements per group
  constexpr int GSTEP = kFP8 ? 32 : 16;          // vector offset between consecutive groups
  constexpr int NG = D / GSTEP;                  // groups per lane
  constexpr int KSTEPS = kFP8 ? D / 64 : D / 16;
  float x[NG][GS];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const long long off = vec * D + GSTEP * g + (GS)*hl;
#pragma unroll
    for (int c = 0; c < GS / 8; ++c) {
      if (a.in_bf16) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (ok) raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q_in) + off + 8 * c);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[g][8 * c + 2 * j] = u2f(w4[j] << 16);
          x[g][8 * c + 2 * j + 1] = u2f(w4[j] & 0xFFFF0000u);
        }
      } else {
        float4 f0 = make_float4(0, 0, 0, 0), f1 = make_float4(0, 0, 0, 0);
        if (ok) {
          const float4* pf = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q_in) + off + 8 * c);
          f0 = pf[0];
          f1 = pf[1];
        }
        x[g][8 * c] = f0.x; x[g][8 * c + 1] = f0.y; x[g][8 * c + 2] = f0.z; x[g][8 * c + 3] = f0.w;
        x[g][8 * c + 4] = f1.x; x[g][8 * c + 5] = f1.y; x[g][8 * c + 6] = f1.z; x[g][8 * c + 7] = f1.w;
      }
    }
  }
  if (!a.in_bf16 && !a.rope_fp32) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int j = 0; j < GS; ++j) x[g][j] = bf16_round(x[g][j]);
  }
  if (a.R > 0) {
    const int rs = D - a.R, half = a.R / 2;
    const float* crow = a.cos_t + (long long)min(pos, a.max_pos - 1) * half;
    const float* srow = a.sin_t + (long long)min(pos, a.max_pos - 1) * half;
    if (a.interleaved) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < GS; j += 2) {
          const int e = GSTEP * g + GS * hl + j;
          if (e >= rs) {
            const int cidx = (e - rs) / 2;
            const float c = crow[cidx], sn = srow[cidx];
            const float x1 = x[g][j], x2 = x[g][j + 1];
            x[g][j] = x1 * c - x2 * sn;
            x[g][j + 1] = x2 * c + x1 * sn;
          }
        }
    } else {
      const int dg = half / GSTEP;               // partner group distance
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int g2 = g + 1; g2 < NG; ++g2) {
          const int e0 = GSTEP * g + GS * hl;    // first element of group g
          if (g2 - g == dg && e0 >= rs && e0 < rs + half) {
            const int cidx = e0 - rs;
            float c[GS], sn[GS];
#pragma unroll
            for (int j = 0; j < GS; j += 4) {
              const float4 cv = *reinterpret_cast<const float4*>(crow + cidx + j);
              const float4 sv = *reinterpret_cast<const float4*>(srow + cidx + j);
              c[j] = cv.x; c[j + 1] = cv.y; c[j + 2] = cv.z; c[j + 3] = cv.w;
              sn[j] = sv.x; sn[j + 1] = sv.y; sn[j + 2] = sv.z; sn[j + 3] = sv.w;
            }
#pragma unroll
            for (int j = 0; j < GS; ++j) {
              const float x1 = x[g][j], x2 = x[g2][j];
              x[g][j] = x1 * c[j] - x2 * sn[j];
              x[g2][j] = x2 * c[j] + x1 * sn[j];
            }
          }
        }
    }
    if (!a.rope_fp32) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < GS; ++j) x[g][j] = bf16_round(x[g][j]);
    }
  }

  if constexpr (!kFP8) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      uint32_t w4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w4[j] = (uint32_t)f32_to_bf16_rne(x[kk][2 * j]) | ((uint32_t)f32_to_bf16_rne(x[kk][2 * j + 1]) << 16);
      const uint4 v = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      aop[kk] = *reinterpret_cast<const AOperand<PREC>*>(&v);
      asc[kk] = 0;
      if (a.q_op_out && ok)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.q_op_out) + vec * D + GSTEP * kk + GS * hl) = v;
    }
  } else {

  // E4M3 codes of a group at exponent e (x * 2^-e exact; the conversion rounds to nearest
  // even, which matches the format definition for |values| <= 448)
  auto encode = [&](int g, int e, uint32_t (&wd)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[g][4 * q], -e), ldexpf(x[g][4 * q + 1], -e), 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[g][4 * q + 2], -e), ldexpf(x[g][4 * q + 3], -e), v, true);
      wd[q] = (uint32_t)v;
    }
  };
  auto lane_pair_max = [](float m) {            // max over lanes l and l ^ 32 (non-negative)
    auto r = __builtin_amdgcn_permlane32_swap(f2u(m), f2u(m), false, false);
    return fmaxf(u2f(r[0]), u2f(r[1]));
  };
  uint32_t wd[NG][4];
  if (PREC == kPrecFP8) {
    float amax = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int j = 0; j < GS; ++j) amax = fmaxf(amax, fabsf(x[g][j]));
    const int e = ue8m0_exponent(lane_pair_max(amax));
#pragma unroll
    for (int g = 0; g < NG; ++g) encode(g, e, wd[g]);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) asc[kk] = e + 127;
    if (a.q_scale_out && ok && hl == 0) a.q_scale_out[vec] = (uint8_t)(e + 127);
  } else {
    // group g = (kk, s) is half of 32-block 2 kk + s; lane hl supplies block 2 kk + hl's scale
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < GS; ++j) amax = fmaxf(amax, fabsf(x[g][j]));
      const int e = ue8m0_exponent(lane_pair_max(amax));
      encode(g, e, wd[g]);
      if ((g & 1) == hl) {
        asc[g / 2] = e + 127;
        if (a.q_scale_out && ok) a.q_scale_out[vec * (D / 32) + g] = (uint8_t)(e + 127);
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    i32x8 t8;
#pragma unroll
    for (int q = 0; q < 4; ++q) { t8[q] = (int)wd[2 * kk][q]; t8[4 + q] = (int)wd[2 * kk + 1][q]; }
    aop[kk] = t8;
  }
  if (a.q_op_out && ok) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(a.q_op_out) + vec * D + GSTEP * g + GS * hl) =
          make_uint4(wd[g][0], wd[g][1], wd[g][2], wd[g][3]);
  }
  }
}

// FP8 / MXFP8 operands (without the fused query preprocessing) stage key tiles by direct
// buffer-to-LDS loads, which need no staging registers: with 32 or 64 heads the kernel then
// fits 3 waves per SIMD.
template <int H, int D, int PREC, bool FUSE>
__global__ __launch_bounds__(kThreads, (PREC != kPrecBF16 && !FUSE && H >= 32) ? 3 : 2)
void score_kernel(ScoreArgs a) {
  constexpr bool kFP8 = PREC != kPrecBF16;
  constexpr bool kDMA = kFP8 && !FUSE;
  constexpr int ES = kFP8 ? 1 : 2;               // operand bytes per element
  constexpr int RB = D * ES;                     // operand bytes per key row
  // LDS key rows: padded by 16 bytes (register staging), or unpadded with the 16-byte chunks
  // of row r permuted by c -> c ^ swz(r) (direct loads), both so that the 16 lanes that LDS
  // serves together (16 consecutive rows, one chunk each: 256 bytes over the 64 banks) hit
  // distinct banks: rows 256 / RB apart share a bank window, swz(r) = (r / (256 / RB)) mod
  // (RB / 16) tells them apart
  constexpr int ROWB = kDMA ? RB : RB + 16;
  constexpr int CHR = RB / 16;                   // 16-byte chunks per row
  constexpr int RPW = 256 / RB > 0 ? 256 / RB : 1;   // rows per 256-byte bank window
  auto swz = [](int r) { return (r / RPW) & (CHR - 1); };
  constexpr int KSTEPS = kFP8 ? D / 64 : D / 16; // MFMAs per 32x32 output block
  constexpr int TPW = 64 / H;                    // tokens per wave
  constexpr int TQ = 4 * TPW;                    // tokens per workgroup
  constexpr int NSB = D / 32;                    // 32-element scale blocks per row

  constexpr int NSBL = PREC == kPrecMXFP8 ? NSB : 1;   // key scales per LDS row
  // the two tile buffers are separate arrays: with direct loads into one while the other is
  // read, the compiler can then tell that the reads need not wait for those loads
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[kNK * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds1[kNK * ROWB];
  auto k_lds = [&](int b) -> uint8_t* { return b ? k_lds1 : k_lds0; };
  __shared__ uint8_t ks_lds[2][kFP8 ? kNK * NSBL : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int hl = lane >> 5;
  const int col = lane & 31;

  // ---- which document and query tile
  int b, p;
  if (!tile_of_block(a, TQ, blockIdx.x, b, p)) return;
  const int lo = clampi(a.cu[b], 0, a.T);
  const int hi = clampi(a.cu[b + 1], lo, a.T);
  const int L = min(hi - lo, a.max_seqlen);
  const int u0 = p * TQ;
  if (u0 >= L) return;
  const int kp = a.kpool;
  const int u_last = min(u0 + TQ, L) - 1;
  const int n_keys = min((u_last + 1) / kp, a.max_cand);
  const int kbase = kp == 1 ? lo : a.cu_pools[b];

  // ---- q operands, scales and weights of this wave's 64 rows (resident)
  const int ut0 = u0 + wv * TPW;                 // first token position of the wave
  typedef AOperand<PREC> AType;
  AType aop[2][KSTEPS];
  int asc[2][KSTEPS];
  // The per-row weights: in registers, or (bf16 operands with 64 heads, where the resident
  // q operands already take 64 registers) in LDS, read as four broadcast 16-byte loads per
  // 32-row block in the epilogue, which keeps the kernel within 256 registers without spills
  // (the fused variant keeps them in registers: its prologue needs the LDS reads' registers).
  constexpr bool kWLds = !kFP8 && H == 64 && !FUSE;
  float wl[2][16];
  __shared__ __attribute__((aligned(16))) float w_lds[kWLds ? 4 * 64 : 1];
  if (FUSE) {
    // one operand row at a time (each holds 64 fp32 values while it is being built)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = rb * 32 + col;
      const int tl = r / H, h = r % H;
      __builtin_amdgcn_sched_barrier(0);
      build_q_row<D, PREC>(a, (long long)(lo + ut0 + tl) * H + h, ut0 + tl < L, ut0 + tl, hl, aop[rb], asc[rb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = rb * 32 + col;                 // operand row held by this lane
    const int tl = r / H, h = r % H;
    const bool ok = ut0 + tl < L;
    const long long vec = (long long)(lo + ut0 + tl) * H + h;
#pragma unroll
    for (int kk = 0; kk < (FUSE ? 0 : KSTEPS); ++kk) {
      if (kFP8) {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(a.q_op) + vec * D + kk * 64 + 16 * hl;
        uint4 v0 = ok ? *reinterpret_cast<const uint4*>(base) : make_uint4(0, 0, 0, 0);
        uint4 v1 = ok ? *reinterpret_cast<const uint4*>(base + 32) : make_uint4(0, 0, 0, 0);
        i32x8 t8;
        t8[0] = v0.x; t8[1] = v0.y; t8[2] = v0.z; t8[3] = v0.w;
        t8[4] = v1.x; t8[5] = v1.y; t8[6] = v1.z; t8[7] = v1.w;
        aop[rb][kk] = *reinterpret_cast<AType*>(&t8);
        int s = 127;
        if (ok) s = PREC == kPrecFP8 ? a.q_scale[vec] : a.q_scale[vec * NSB + 2 * kk + hl];
        asc[rb][kk] = s;
      } else {
        const uint16_t* base = reinterpret_cast<const uint16_t*>(a.q_op) + vec * D + kk * 16 + 8 * hl;
        uint4 v = ok ? *reinterpret_cast<const uint4*>(base) : make_uint4(0, 0, 0, 0);
        aop[rb][kk] = *reinterpret_cast<AType*>(&v);
        asc[rb][kk] = 0;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // unconditional loads (rows past the document read its last token and are zeroed
      // below) under one uniform dtype branch, so the 16 loads are in flight together
      const int rr = rb * 32 + (i / 4) * 8 + hl * 4 + (i % 4);
      const long long wi = (long long)(lo + min(ut0 + rr / H, L - 1)) * H + rr % H;
      wl[rb][i] = a.w_bf16 ? 0.f : reinterpret_cast<const float*>(a.w)[wi];
    }
    if (a.w_bf16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = rb * 32 + (i / 4) * 8 + hl * 4 + (i % 4);
        const long long wi = (long long)(lo + min(ut0 + rr / H, L - 1)) * H + rr % H;
        wl[rb][i] = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.w)[wi]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = rb * 32 + (i / 4) * 8 + hl * 4 + (i % 4);
      const float wv_ = ut0 + rr / H < L ? wl[rb][i] : 0.f;
      wl[rb][i] = wv_;
      if (kWLds && col < 4 && (i % 4) == col) w_lds[wv * 64 + rr] = wv_;   // each row once
    }
  }
  if (kWLds) __syncthreads();

  // candidates of the tokens this lane writes (see the epilogue)
  int cand_tok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = ut0 + j;
    cand_tok[j] = (j < TPW && u < L) ? min((u + 1) / kp, a.max_cand) : 0;
  }
  // score rows of this wave's tokens, as a buffer: lanes that write nothing (masked
  // candidates, duplicate lanes) store to an offset past its end, which the hardware drops
  const __amdgpu_buffer_rsrc_t out_r =
      make_rsrc(a.scores + (long long)(lo + ut0) * a.stride, TPW * a.stride * 4);
  constexpr uint32_t kDrop = 0xFFFFFFF0u;

  // ---- key-tile staging through buffer loads: the buffer covers the stageable rows of this
  //      document (candidates that exist in the key array), so rows past them read as zeros
  //      without branches. Each thread moves NCH fixed 16-byte chunks of every tile; only
  //      the descriptor's base (a scalar) advances from tile to tile.
  constexpr int CH = RB / 16;                    // 16-byte chunks per key row
  static_assert((kNK * CH) % kThreads == 0, "tile chunks must divide over the workgroup");
  constexpr int NCH = kNK * CH / kThreads;
  constexpr int NSC = kNK * NSBL;                // scale bytes per tile
  const int lim = (int)max(0LL, min((long long)n_keys, (long long)a.S - kbase));   // stageable rows
  const uint8_t* kdoc = reinterpret_cast<const uint8_t*>(a.k_op) + (long long)kbase * RB;
  const uint8_t* sdoc = kFP8 ? a.k_scale + (long long)kbase * NSBL : nullptr;
  // Direct loads: instruction it of wave w fills the tile's 16-byte slots
  // (w NCH + it) * 64 + lane, slot s holding chunk (s % CH) ^ swz(row) of row s / CH.
  int goff[NCH], lds_off[NCH];
#pragma unroll
  for (int it = 0; it < NCH; ++it) {
    if (kDMA) {
      const int sl = (wv * NCH + it) * 64 + lane;
      const int row = sl / CH, p = sl % CH;
      goff[it] = row * RB + (p ^ swz(row)) * 16;
      lds_off[it] = 0;                         // unused: the destination is wave-uniform
    } else {
      const int ch = it * kThreads + tid;
      const int row = ch / CH, cc = ch % CH;
      goff[it] = row * RB + cc * 16;
      lds_off[it] = row * ROWB + cc * 16;
    }
  }
  const int sc_i = tid % NSC;                    // scale byte this thread stages (duplicates agree)

  struct Stage { uint4 v[kDMA ? 1 : NCH]; uint32_t s; };
  // key tile c0 to registers, or (direct loads) to LDS buffer `dbuf`; its scales to registers
  auto fetch = [&](Stage& st, int c0, int dbuf) {
    const int rem = max(0, lim - c0);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kdoc + (long long)c0 * RB, rem * RB);
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      if (kDMA) {
        lds_dma16(kr, k_lds(dbuf) + (__builtin_amdgcn_readfirstlane(wv) * NCH + it) * 1024, goff[it]);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(kr, goff[it], 0, 0);
        st.v[kDMA ? 0 : it] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
    st.s = 0;
    if (kFP8) {
      const __amdgpu_buffer_rsrc_t sr = make_rsrc(sdoc + (long long)c0 * NSBL, rem * NSBL);
      st.s = __builtin_amdgcn_raw_buffer_load_b8(sr, sc_i, 0, 0);
    }
  };
  auto put = [&](const Stage& st, int buf) {
#pragma unroll
    for (int it = 0; it < (kDMA ? 0 : NCH); ++it) *reinterpret_cast<uint4*>(k_lds(buf) + lds_off[it]) = st.v[it];
    if (kFP8) ks_lds[buf][sc_i] = (uint8_t)st.s;
  };
  // LDS byte offsets of this lane's B-operand chunks in its row of column block 0 (rows
  // nb * 32 + col of block nb add the constant nb * 32 * ROWB): chunks 4 kk + hl and
  // 4 kk + 2 + hl (fp8), swizzled by the row's low bits with direct loads
  int boff[kFP8 ? KSTEPS : 1][2];
#pragma unroll
  for (int kk = 0; kk < (kFP8 ? KSTEPS : 0); ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 4 * kk + 2 * h + hl;
      boff[kk][h] = col * ROWB + ((kDMA ? (c ^ swz(col)) : c) << 4);   // swz(nb * 32 + col) = swz(col)
    }

  // ---- one 32-key column block: q.k on MFMA into acc
  typedef f32x16 Acc[2];
  auto mma = [&](int buf, int nb, Acc& acc) {
    const uint8_t* kl = k_lds(buf);
    const int krow_l = nb * 32 + col;            // key (LDS row) of this lane's B operand / C column
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (kFP8) {
        uint4 v0 = *reinterpret_cast<const uint4*>(kl + nb * 32 * ROWB + boff[kk][0]);
        uint4 v1 = *reinterpret_cast<const uint4*>(kl + nb * 32 * ROWB + boff[kk][1]);
        i32x8 bop;
        bop[0] = v0.x; bop[1] = v0.y; bop[2] = v0.z; bop[3] = v0.w;
        bop[4] = v1.x; bop[5] = v1.y; bop[6] = v1.z; bop[7] = v1.w;
        const int bsc = PREC == kPrecFP8 ? ks_lds[buf][krow_l] : ks_lds[buf][krow_l * NSBL + 2 * kk + hl];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              *reinterpret_cast<const i32x8*>(&aop[rb][kk]), bop, acc[rb], 0, 0, 0, asc[rb][kk], 0, bsc);
      } else {
        uint4 v = *reinterpret_cast<const uint4*>(kl + krow_l * ROWB + kk * 32 + 16 * hl);
        bf16x8 bop = *reinterpret_cast<bf16x8*>(&v);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(&aop[rb][kk]), bop, acc[rb], 0, 0, 0);
      }
    }
  };

  // ---- ReLU, weights and head sum of one column block (first candidate cb) in registers
  auto epilogue = [&](const Acc& acc, int cb) {
    const int c = cb + col;                      // candidate index (document-local)
    if (H == 64) {
      float s = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float w4[4];
          if (kWLds) {
            const float4 q = *reinterpret_cast<const float4*>(w_lds + wv * 64 + rb * 32 + g * 8 + hl * 4);
            w4[0] = q.x; w4[1] = q.y; w4[2] = q.z; w4[3] = q.w;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) w4[k] = wl[rb][4 * g + k];
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) s = __builtin_fmaf(w4[k], relu(acc[rb][4 * g + k]), s);
        }
      s = pair_sum(s) * a.sm_scale;
      const uint32_t off = (hl == 0 && (uint32_t)c < (uint32_t)cand_tok[0]) ? (uint32_t)c * 4u : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(f2u(s), out_r, off, 0, 0);
    } else if (H == 32) {
      float s[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) v = __builtin_fmaf(wl[rb][i], relu(acc[rb][i]), v);
        s[rb] = pair_sum(v) * a.sm_scale;
      }
      // lanes 0-31 write token 0, lanes 32-63 token 1
      const int ct = hl ? cand_tok[1] : cand_tok[0];
      const uint32_t off = (uint32_t)c < (uint32_t)ct ? (uint32_t)(hl * a.stride + c) * 4u : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(f2u(hl ? s[1] : s[0]), out_r, off, 0, 0);
    } else {                                     // H == 16: rows 0-15 / 16-31 of a block are two tokens
      float s[4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v0 = __builtin_fmaf(wl[rb][i], relu(acc[rb][i]), v0);
#pragma unroll
        for (int i = 8; i < 16; ++i) v1 = __builtin_fmaf(wl[rb][i], relu(acc[rb][i]), v1);
        s[2 * rb] = pair_sum(v0) * a.sm_scale;
        s[2 * rb + 1] = pair_sum(v1) * a.sm_scale;
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int j = 2 * rb + hl;
        const float v = hl ? s[2 * rb + 1] : s[2 * rb];
        const int ct = hl ? cand_tok[2 * rb + 1] : cand_tok[2 * rb];
        const uint32_t off = (uint32_t)c < (uint32_t)ct ? (uint32_t)(j * a.stride + c) * 4u : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(f2u(v), out_r, off, 0, 0);
      }
    }
  };

  // ---- sweep. Tiles alternate between two LDS buffers. Register staging (bf16): while
  //      tile kt is multiplied out of one buffer, tile kt + 1 waits in registers for the other
  //      buffer and tile kt + 2 is in flight, so a load has two tiles of work to land. Direct
  //      loads (fp8, MXFP8): tile kt + 1 streams into the other buffer. Each column block's
  //      epilogue runs while the next block's MFMAs execute (the first call of a workgroup
  //      stores nothing: its candidates are negative). One barrier per tile.
  const int n_tiles = (n_keys + kNK - 1) / kNK;
  if (n_tiles == 0) return;
  Acc acc0, acc1;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc1[rb][i] = 0.f;
  auto compute = [&](int buf, int c0) {
    mma(buf, 0, acc0);
    epilogue(acc1, c0 - 32);
    mma(buf, 1, acc1);
    epilogue(acc0, c0);
  };
  int kt = 0;
  if constexpr (kDMA) {
    // Direct loads, one tile ahead: tile kt + 1 streams into the other LDS buffer while tile
    // kt is multiplied out; the barrier that ends each tile first waits for this wave's loads
    // (vmcnt 0), so the next tile is in LDS for every wave after it.
    Stage st;
    fetch(st, 0, 0);
    put(st, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): the direct loads have landed
    __syncthreads();
    for (; kt + 1 < n_tiles; kt += 2) {          // buffer 0 holds tile kt
      fetch(st, (kt + 1) * kNK, 1);
      compute(0, kt * kNK);
      put(st, 1);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      fetch(st, (kt + 2) * kNK, 0);
      compute(1, (kt + 1) * kNK);
      put(st, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
  } else {
    Stage sa, sb;
    fetch(sa, 0, 0);
    fetch(sb, kNK, 0);
    put(sa, 0);
    __syncthreads();
    fetch(sa, 2 * kNK, 0);
    for (; kt + 1 < n_tiles; kt += 2) {          // buffer 0 holds tile kt, sb tile kt+1, sa tile kt+2
      compute(0, kt * kNK);
      put(sb, 1);
      __syncthreads();
      fetch(sb, (kt + 3) * kNK, 0);
      compute(1, (kt + 1) * kNK);
      put(sa, 0);
      __syncthreads();
      fetch(sa, (kt + 4) * kNK, 0);
    }
  }
  if (kt < n_tiles) compute(0, kt * kNK);        // odd tile count: the last tile is in buffer 0
  epilogue(acc1, n_tiles * kNK - 32);
}

template <int H, int D, int PREC>
hipError_t launch_h(const ScoreArgs& a, bool fuse, hipStream_t st) {
  const long long blocks = (long long)a.ntiles * a.B;
  if (blocks == 0) return hipSuccess;
  if (fuse)
    hipLaunchKernelGGL((score_kernel<H, D, PREC, true>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((score_kernel<H, D, PREC, false>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, int PREC>
hipError_t launch_d(const ScoreArgs& a, int H, bool fuse, hipStream_t st) {
  switch (H) {
    case 16: return launch_h<16, D, PREC>(a, fuse, st);
    case 32: return launch_h<32, D, PREC>(a, fuse, st);
    default: return launch_h<64, D, PREC>(a, fuse, st);
  }
}

template <int PREC>
hipError_t launch_p(const ScoreArgs& a, int H, int D, bool fuse, hipStream_t st) {
  return D == 128 ? launch_d<128, PREC>(a, H, fuse, st) : launch_d<64, PREC>(a, H, fuse, st);
}

}  // namespace

bool score_can_fuse_rope(int precision, int rope_dim, int interleaved) {
  if (rope_dim == 0 || interleaved) return true;
  return (rope_dim / 2) % (precision == kPrecBF16 ? 16 : 32) == 0;
}

hipError_t launch_score(const ScoreTopkLaunch& p, hipStream_t st) {
  ScoreArgs a;
  a.q_op = p.q_op; a.q_scale = p.q_scale; a.k_op = p.k_op; a.k_scale = p.k_scale;
  a.w = p.w; a.w_bf16 = p.w_bf16;
  a.q_in = p.q_in; a.in_bf16 = p.in_bf16;
  a.cos_t = p.cos_t; a.sin_t = p.sin_t;
  a.R = p.rope_dim; a.max_pos = p.max_pos; a.interleaved = p.interleaved; a.rope_fp32 = p.rope_fp32;
  a.q_op_out = p.q_op_out; a.q_scale_out = p.q_scale_out;
  a.T = p.T; a.S = p.S; a.B = p.B; a.max_seqlen = p.max_seqlen; a.kpool = p.kpool;
  a.cu = p.cu; a.cu_pools = p.cu_pools;
  a.sm_scale = p.sm_scale;
  a.scores = p.scores; a.stride = p.stride; a.max_cand = p.max_cand;
  const int tq = 256 / p.H;
  a.ntiles = (p.max_seqlen + tq - 1) / tq;
  const bool fuse = p.q_in != nullptr;
  switch (p.precision) {
    case kPrecBF16: return launch_p<kPrecBF16>(a, p.H, p.D, fuse, st);
    case kPrecFP8: return launch_p<kPrecFP8>(a, p.H, p.D, fuse, st);
    default: return launch_p<kPrecMXFP8>(a, p.H, p.D, fuse, st);
  }
}

}  // namespace dsa
