// Per-row top-k selection over the score workspace, with KPool expansion (gfx950).
//
// One workgroup per query row. Each thread holds 4-candidate chunks of the row, interleaved
// across the workgroup, in registers; chunk groups past the row's last candidate are skipped
// by every pass. A 2048-bin histogram linear in the score (LDS integer atomics) gives the bin
// holding the topk-th largest score, and its suffix sums give every bin its range of output
// slots. Every candidate of that bin and of the bins above it is placed in its bin's range
// with its score and index; its exact rank inside the bin (score descending, index
// ascending) then gives its output position, and the threshold bin keeps only as many as the
// selection still needs. Candidates equal to the last score taken are thus taken lowest
// indices first (deterministic tie breaking, Megatron-LM PR 5992, "Key changes"). A row
// whose bins do not separate the scores (a few outliers stretching the range) is binned
// again over its selected region; rows neither level separates (clustered or tied scores,
// no finite range) are finished by a second kernel: an 11 + 11 + 10-bit radix select, a
// compaction by block prefix sums and a bitonic network.
// Rows longer than
// 4096 candidates run in launch shapes sized to them. No floating-point atomics; the result
// does not depend on scheduling. Outputs are padded with -1 / -inf. For KPool (PR 7522,
// "Changes") selected pools are expanded to their tokens and the query's incomplete causal
// pool is appended when requested.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

struct TopkArgs {
  const float* scores; int stride; int max_cand;
  int T, B, max_seqlen, kpool, kpool_tail, topk, p2max;
  int hist_off;   // byte offset of the histogram in dynamic LDS
  // Rows handled by this launch: those with a candidate count in [cls_lo, cls_hi], in
  // document order; cls_map == 0: every row, block b = row b (see map_row).
  int cls_lo, cls_hi, cls_map;
  const int32_t* cu; const int32_t* cu_pools;
  int32_t* out_indices; float* out_scores; int32_t* out_lengths; int32_t* out_pool_indices;
};

typedef unsigned long long u64;

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((u64)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts (within rows of 16
// lanes) and the row broadcasts of lanes 15 and 31 (across rows).
__device__ __forceinline__ int wave_prefix_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// Inclusive suffix sum over the 64 lanes of a wave (lane l gets the sum over lanes >= l).
__device__ __forceinline__ int wave_suffix_sum(int v) {
  const int incl = wave_prefix_sum(v);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  return total - incl + v;
}

// Bitonic stages with distance j < 64*V inside one register-resident segment of 64*V
// elements: x[v] holds element seg_base + 64 v + lane. Direction of position i: up when
// (i & k) == 0. Runs stages j = j0, j0/2, ..., 1.
template <int V, int JV>
__device__ __forceinline__ void inlane_stage(u64 (&x)[V], int seg_base, int k) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if ((v & JV) == 0) {
      const int i = seg_base + 64 * v + lane;
      const bool up = (i & k) == 0;
      const u64 a = x[v], b = x[v + JV];
      const bool sw = (a > b) == up;
      x[v] = sw ? b : a;
      x[v + JV] = sw ? a : b;
    }
  }
}

template <int V>
__device__ __forceinline__ void segment_stages(u64 (&x)[V], int seg_base, int k, int j0) {
  const int lane = threadIdx.x & 63;
  for (int j = j0; j >= 1; j >>= 1) {
    if (j >= 64) {
      // in-lane exchanges between slots v and v + j/64 (register indices fixed at compile time)
      if (V >= 4 && j == 128) inlane_stage<V, (V >= 4 ? 2 : 0)>(x, seg_base, k);
      else if (V >= 2) inlane_stage<V, (V >= 2 ? 1 : 0)>(x, seg_base, k);
    } else {
      const bool lower = (lane & j) == 0;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int i = seg_base + 64 * v + lane;
        const bool up = (i & k) == 0;
        const u64 y = shfl_xor_u64(x[v], j);
        const u64 mn = x[v] < y ? x[v] : y, mx = x[v] < y ? y : x[v];
        x[v] = (lower == up) ? mn : mx;
      }
    }
  }
}

// Ascending bitonic sort of sel[0, n2) (n2 a power of two >= 64) by the whole workgroup.
template <int V, int NT>
__device__ __forceinline__ void bitonic_sort(u64* sel, int n2) {
  constexpr int NW = NT / 64;
  constexpr int SEG = 64 * V;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nseg = n2 / SEG;
  // 1) every segment sorted on its own (k = 2 .. SEG), alternating directions as the
  //    bitonic network requires (direction comes from the global position)
  for (int s = wv; s < nseg; s += NW) {
    u64 x[V];
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = sel[s * SEG + 64 * v + lane];
    for (int k = 2; k <= SEG; k <<= 1) segment_stages<V>(x, s * SEG, k, k >> 1);
#pragma unroll
    for (int v = 0; v < V; ++v) sel[s * SEG + 64 * v + lane] = x[v];
  }
  // 2) merges wider than a segment: the stages j >= SEG in LDS, the rest in registers
  for (int k = 2 * SEG; k <= n2; k <<= 1) {
    for (int j = k >> 1; j >= SEG; j >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < n2; i += NT) {
        const int p = i ^ j;
        if (p > i) {
          const bool up = (i & k) == 0;
          const u64 a = sel[i], b = sel[p];
          if ((a > b) == up) { sel[i] = b; sel[p] = a; }
        }
      }
    }
    __syncthreads();
    for (int s = wv; s < nseg; s += NW) {
      u64 x[V];
#pragma unroll
      for (int v = 0; v < V; ++v) x[v] = sel[s * SEG + 64 * v + lane];
      segment_stages<V>(x, s * SEG, k, SEG >> 1);
#pragma unroll
      for (int v = 0; v < V; ++v) sel[s * SEG + 64 * v + lane] = x[v];
    }
  }
  __syncthreads();
}

// Wave-wide max (MAX) or min of a uint32 with DPP steps; the result is valid in every lane.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extreme(uint32_t x) {
  const int id = MAX ? 0 : -1;
  int v = (int)x;
#define DSA_STEP(ctrl, rm)                                                        \
  {                                                                               \
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(id, v, ctrl, rm, 0xf, false); \
    const uint32_t c = (uint32_t)v;                                               \
    v = (int)(MAX ? (o > c ? o : c) : (o < c ? o : c));                           \
  }
  DSA_STEP(0x111, 0xf) DSA_STEP(0x112, 0xf) DSA_STEP(0x114, 0xf) DSA_STEP(0x118, 0xf)
  DSA_STEP(0x142, 0xa) DSA_STEP(0x143, 0xc)
#undef DSA_STEP
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// Block-wide min and max of one uint32 pair per thread (results valid in every thread).
// Uses buf[2*NW].
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, int* buf) {
  constexpr int NW = NT / 64;
  mn = wave_extreme<false>(mn);
  mx = wave_extreme<true>(mx);
  if (NW == 1) return;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { buf[threadIdx.x >> 6] = (int)mn; buf[NW + (threadIdx.x >> 6)] = (int)mx; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t a = (uint32_t)buf[w], b = (uint32_t)buf[NW + w];
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
}

// Exclusive prefix sum of one int per thread over the block (in thread order); `tot` gets
// the block total. Uses wsum[NW] (NW <= 16, 16-byte aligned).
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int* wsum, int& tot) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_prefix_sum(v);
  __syncthreads();
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = incl - v;
  tot = 0;
  if (NW == 1) {
    tot = wsum[0];
  } else {
#pragma unroll
    for (int w4 = 0; w4 < (NW + 3) / 4; ++w4) {
      const int4 q = reinterpret_cast<const int4*>(wsum)[w4];
      const int qa[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w = 4 * w4 + j;
        if (w < NW) { if (w < wv) before += qa[j]; tot += qa[j]; }
      }
    }
  }
  return before;
}

// Finds the bin of a descending rank inside a histogram of NB bins (NB % NT == 0): the bin
// d with above(d) < krem <= above(d) + hist[d], above(d) = count in bins > d. Thread tid
// owns bins [tid*PER, tid*PER + PER), so higher bins live in higher threads. Returns d in
// misc[0], above(d) in misc[1] and hist[d] in misc[2] (valid in every thread afterwards).
template <int NT, int NB>
__device__ __forceinline__ void find_rank_bin(const uint32_t* hist, int krem, int* wsum, int* misc) {
  constexpr int NW = NT / 64;
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t h[PER];
  if (PER >= 4) {
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(hist + tid * PER + j);
      h[j] = q.x; h[j + 1] = q.y; h[j + 2] = q.z; h[j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) h[j] = hist[tid * PER + j];
  }
  int mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) mine += (int)h[j];
  const int suf = wave_suffix_sum(mine);
  if (lane == 0) wsum[wv] = suf;
  __syncthreads();
  int above = suf - mine;
  if (NW > 1) {
#pragma unroll
    for (int w4 = 0; w4 < (NW + 3) / 4; ++w4) {
      const int4 q = reinterpret_cast<const int4*>(wsum)[w4];
      const int qa[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w = 4 * w4 + j;
        if (w < NW && w > wv) above += qa[j];
      }
    }
  }
#pragma unroll
  for (int j = PER - 1; j >= 0; --j) {
    const int hc = (int)h[j];
    if (above < krem && krem <= above + hc) { misc[0] = tid * PER + j; misc[1] = above; misc[2] = hc; }
    above += hc;
  }
  __syncthreads();
}

// The same search over the 2048 pass-1 bins, which then replaces every bin's count c by
// (above(d) << 16) | c: above(d) is the first output slot of bin d (counts and slots are at
// most 32768, so both fields fit). Sets misc[6] (zeroed by the caller) when a thread owning
// a bin at or above the found one has a bin of more than `heavy` keys, and misc[8] (set to
// 2047 by the caller) to the bin holding the rank2-th largest key when there is one. Only
// the thread whose bins hold a rank scans them one by one.
template <int NT>
__device__ __forceinline__ void scan_pass1_bins(uint32_t* hist, int krem, int* wsum, int* misc, int heavy,
                                                int rank2) {
  constexpr int NW = NT / 64;
  constexpr int PER = 2048 / NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t h[PER];
  if (PER >= 4) {
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(hist + tid * PER + j);
      h[j] = q.x; h[j + 1] = q.y; h[j + 2] = q.z; h[j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) h[j] = hist[tid * PER + j];
  }
  int mine = 0;
  uint32_t hmax = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { mine += (int)h[j]; hmax = max(hmax, h[j]); }
  const int suf = wave_suffix_sum(mine);
  if (lane == 0) wsum[wv] = suf;
  __syncthreads();
  int above = suf - mine;   // count in the bins of higher threads
  if (NW > 1) {
#pragma unroll
    for (int w4 = 0; w4 < (NW + 3) / 4; ++w4) {
      const int4 q = reinterpret_cast<const int4*>(wsum)[w4];
      const int qa[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w = 4 * w4 + j;
        if (w < NW && w > wv) above += qa[j];
      }
    }
  }
  uint32_t st[PER];
  st[PER - 1] = (uint32_t)above;
#pragma unroll
  for (int j = PER - 2; j >= 0; --j) st[j] = st[j + 1] + h[j + 1];
  if (PER >= 4) {
#pragma unroll
    for (int j = 0; j < PER; j += 4)
      *reinterpret_cast<uint4*>(hist + tid * PER + j) =
          make_uint4(st[j] << 16 | h[j], st[j + 1] << 16 | h[j + 1], st[j + 2] << 16 | h[j + 2], st[j + 3] << 16 | h[j + 3]);
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) hist[tid * PER + j] = st[j] << 16 | h[j];
  }
  if (above < krem && hmax > (uint32_t)heavy) misc[6] = 1;
  if (above < krem && krem <= above + mine) {
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      const int a0 = (int)st[j], hc = (int)h[j];
      if (a0 < krem && krem <= a0 + hc) { misc[0] = tid * PER + j; misc[1] = a0; misc[2] = hc; }
    }
  }
  if (above < rank2 && rank2 <= above + mine) {
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      const int a0 = (int)st[j], hc = (int)h[j];
      if (a0 < rank2 && rank2 <= a0 + hc) misc[8] = tid * PER + j;
    }
  }
  __syncthreads();
}

constexpr int kBucketMax = 64;   // a bin larger than this at or above the threshold: binned again, else the fallback
constexpr int kHistSlots = 2048 + 16;   // pass-1 bins, then a slot that counts non-candidates
constexpr int kFallbackGrid = 1024;     // workgroups of the fallback launch

struct RowInfo {
  int t, b, lo, u, cand, nsel;
};

__device__ __forceinline__ RowInfo row_info(const TopkArgs& a, int t) {
  RowInfo r;
  r.t = t;
  r.b = find_doc(a.cu, a.B, t);
  r.lo = clampi(a.cu[r.b], 0, a.T);
  r.u = max(0, min(t - r.lo, a.max_seqlen - 1));
  r.cand = min((r.u + 1) / a.kpool, a.max_cand);
  r.nsel = min(a.topk, r.cand);
  return r;
}

// Output rows of query t: entries in selection order at positions dest < nsel (score bits and
// the candidate's document-local index), then padding (-inf / -1, KPool tail tokens) and the
// length. Buffer stores take 32-bit offsets.
struct RowOut {
  float* os; int32_t* oi; int32_t* op;
  __amdgpu_buffer_rsrc_t rs, ri;
  int topk, kp, width, lo, pbase;
  __device__ __forceinline__ RowOut(const TopkArgs& a, int t, int lo_, int b)
      : RowOut(a, t, lo_, a.kpool > 1 ? a.cu_pools[b] : 0, 0) {}
  // with the document's first pool index given
  __device__ __forceinline__ RowOut(const TopkArgs& a, int t, int lo_, int pbase_, int) {
    topk = a.topk; kp = a.kpool; lo = lo_;
    width = kp == 1 ? topk : topk * kp + kp - 1;
    os = a.out_scores + (long long)t * topk;
    oi = a.out_indices + (long long)t * width;
    op = (kp > 1 && a.out_pool_indices) ? a.out_pool_indices + (long long)t * topk : nullptr;
    pbase = pbase_;
    rs = make_rsrc(os, topk * 4);
    ri = make_rsrc(oi, width * 4);
  }
  __device__ __forceinline__ void store(int dest, uint32_t score_bits, int ix) const {
    __builtin_amdgcn_raw_buffer_store_b32(score_bits, rs, dest * 4, 0, 0);
    if (kp == 1) {
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(lo + ix), ri, dest * 4, 0, 0);
    } else {
      if (op) op[dest] = pbase + ix;
      for (int j = 0; j < kp; ++j)
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(lo + ix * kp + j), ri, (dest * kp + j) * 4, 0, 0);
    }
  }
  // padding after the first nsel entries, the KPool tail, the length (thread 0)
  template <int NT>
  __device__ __forceinline__ void finish(const TopkArgs& a, int t, int nsel, int u) const {
    const int tid = threadIdx.x;
    for (int j = nsel + tid; j < topk; j += NT) os[j] = -INFINITY;
    if (kp == 1) {
      for (int j = nsel + tid; j < topk; j += NT) oi[j] = -1;
      if (tid == 0) a.out_lengths[t] = nsel;
    } else {
      if (op)
        for (int j = nsel + tid; j < topk; j += NT) op[j] = -1;
      const int tail = a.kpool_tail ? (u + 1) % kp : 0;
      const int npool_tok = nsel * kp;
      const int tail_start = lo + (u / kp) * kp;
      for (int s2 = npool_tok + tid; s2 < width; s2 += NT)
        oi[s2] = s2 < npool_tok + tail ? tail_start + (s2 - npool_tok) : -1;
      if (tid == 0) a.out_lengths[t] = npool_tok + tail;
    }
  }
};

// The row of block j. A launch over every row takes row j. A size-class launch (CLS) takes
// the rows whose candidate count lies in [cls_lo, cls_hi]: candidate counts grow with the
// position u in a document, so each document contributes the positions [ulo, uhi] (the class
// holding max_cand also every position past it), in document order and positions ascending.
// Returns false when j is past the launch's rows.
//
// A launch over every row finds the row's document by a binary search over cu (scalar
// loads: one or two steps for a few documents). A size-class launch with at most 64
// documents reads one document's bounds per lane (both loads in flight together) and takes
// the row and its document from a prefix sum, a ballot and readlane: one memory round trip
// instead of a pass over the documents followed by the search (measured 4 % faster on the
// 32768-token, 12-document workload). More documents take a pass per 64 documents and the
// search. The two are separate kernels: the table's code alone, not taken, cost the launch
// over every row 2 % (registers, and later score loads).
__device__ __forceinline__ int class_rows_of(const TopkArgs& a, int b, int ulo, int uhi, int& lo) {
  int n = 0;
  lo = 0;
  if (b < a.B) {
    lo = clampi(a.cu[b], 0, a.T);
    const int hi = clampi(a.cu[b + 1], lo, a.T);
    n = max(0, min(hi - lo - 1, uhi) - ulo + 1);
  }
  return n;
}

template <bool CLS>
__device__ __forceinline__ bool map_row(const TopkArgs& a, int j, int& t, int& b, int& lo, int& pbase) {
  const int lane = threadIdx.x & 63;
  const int kp = a.kpool;
  if (CLS && a.B <= 64) {
    int dlo = 0, dpb = 0;
    if (kp > 1 && lane < a.B) dpb = a.cu_pools[lane];
    const int ulo = a.cls_lo <= 0 ? 0 : a.cls_lo * kp - 1;
    const int uhi = a.cls_hi >= a.max_cand ? 0x7FFFFFFF : a.cls_hi * kp + kp - 2;
    const int n = class_rows_of(a, lane, ulo, uhi, dlo);
    const int incl = wave_prefix_sum(n);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (j >= total) return false;
    const int r = j;
    b = __ffsll((long long)__ballot(incl - n <= r && r < incl)) - 1;
    t = __builtin_amdgcn_readlane(dlo, b) + ulo + (r - __builtin_amdgcn_readlane(incl - n, b));
    b = __builtin_amdgcn_readfirstlane(b);
    t = __builtin_amdgcn_readfirstlane(t);
    lo = __builtin_amdgcn_readlane(dlo, b);
    pbase = __builtin_amdgcn_readlane(dpb, b);
    return true;
  }
  if (!CLS) {
    if (j >= a.T) return false;
    t = j;
  } else {
    const int ulo = a.cls_lo <= 0 ? 0 : a.cls_lo * kp - 1;
    const int uhi = a.cls_hi >= a.max_cand ? 0x7FFFFFFF : a.cls_hi * kp + kp - 2;
    int total = 0, dl;
    for (int b0 = 0; b0 < a.B; b0 += 64)
      total += __builtin_amdgcn_readlane(wave_prefix_sum(class_rows_of(a, b0 + lane, ulo, uhi, dl)), 63);
    if (j >= total) return false;
    const int r = j;
    int base = 0;
    t = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int n = class_rows_of(a, b0 + lane, ulo, uhi, dl);
      const int incl = wave_prefix_sum(n);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (r - base < tot) {
        const int src = __ffsll((long long)__ballot(incl - n <= r - base && r - base < incl)) - 1;
        t = __shfl(dl, src, 64) + ulo + (r - base - __shfl(incl - n, src, 64));
        break;
      }
      base += tot;
    }
  }
  t = __builtin_amdgcn_readfirstlane(t);
  b = find_doc(a.cu, a.B, t);
  lo = clampi(a.cu[b], 0, a.T);
  pbase = kp > 1 ? a.cu_pools[b] : 0;
  return true;
}

// At most 82 SGPRs (74 allocated besides VCC and the like): measured on the device, a wave
// of more than about 90 keeps a SIMD at 7 waves or fewer, while the VGPRs here allow 8; the
// few values that no longer fit move to VGPR lanes.
template <int NT, int EPT, bool CLS>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_num_sgpr(82))) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  u64* selA = reinterpret_cast<u64*>(smem);                                  // [p2max + kBucketMax]
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + a.hist_off);           // [kHistSlots]
  int* wsum = reinterpret_cast<int*>(hist + kHistSlots);                     // [32]
  int* misc = wsum + 32;                                                     // [16]

  const int tid = threadIdx.x;
  // the row (uniform: its values stay in scalar registers)
  int t, b, lo, pbase;
  if (!map_row<CLS>(a, blockIdx.x, t, b, lo, pbase)) return;
  const int u = max(0, min(t - lo, a.max_seqlen - 1));
  const int cand = min((u + 1) / a.kpool, a.max_cand);
  const int nsel = min(a.topk, cand);

  // ---- the row's scores in registers. Thread tid holds the 4-candidate chunks
  //      c = e*NT + tid (candidates 4c .. 4c+3), so one load instruction covers 16*NT
  //      consecutive bytes, and a chunk group e lies entirely past the row once 4*e*NT >= cand:
  //      such groups are skipped by every per-candidate pass (uniform branch). Only the last
  //      live group can hold slots past the row (`in` below). All loads are issued before any
  //      is used; the buffer descriptor ends at the row's last candidate, so loads of groups
  //      past it return zeros without touching memory. Up to 16 candidates per thread the
  //      order-preserving keys (0 past the row) and the pass-1 bins are kept in registers;
  //      with 32 only the scores are (-0 folded onto +0) and keys and bins are recomputed
  //      where needed: a few more instructions, but 64 fewer registers, which keeps 8 waves
  //      per SIMD (more rows in flight).
  static_assert(EPT % 4 == 0, "candidates are held in chunks of 4");
  static_assert(EPT <= 32, "one bit per candidate in a 32-bit mask");
  constexpr int NCH = EPT / 4;
  auto live = [&](int e) { return 4 * e * NT < cand; };
  auto full = [&](int e) { return 4 * (e + 1) * NT <= cand; };
  auto idx = [&](int e, int j) { return 4 * (e * NT + tid) + j; };
  auto in = [&](int e, int j) { return full(e) || idx(e, j) < cand; };
  // order-preserving key of a score: negative scores invert all bits, others set the sign bit
  auto keyof = [](float x) {
    const uint32_t v = f2u(x);
    return v ^ ((uint32_t)((int)v >> 31) | 0x80000000u);
  };
  constexpr bool KEEP = EPT <= 16;
  float val[EPT];
  int binA[KEEP ? EPT : 1];
  // Range of the candidates, branch-free: slots past the row enter the minimum and maximum
  // as a quiet NaN, which fminf / fmaxf ignore, and the product-sum `fin` (v * 0 summed;
  // slots past the row load as +0 and add nothing) turns NaN as soon as one candidate is NaN
  // or infinite.
  float vlo = NAN, vhi = NAN, fin = 0.f;
  {
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.scores + (long long)t * a.stride, cand * 4);
    __attribute__((ext_vector_type(4))) uint32_t raw[NCH];
#pragma unroll
    for (int e = 0; e < NCH; ++e) raw[e] = __builtin_amdgcn_raw_buffer_load_b128(rr, (e * NT + tid) * 16, 0, 0);
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
      if (!live(e)) continue;
      if (full(e)) {                             // (uniform) no slot past the row
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = u2f(raw[e][j]) + 0.0f;   // -0 + 0 = +0
          val[4 * e + j] = v;
          vlo = fminf(vlo, v);
          vhi = fmaxf(vhi, v);
          fin = __builtin_fmaf(v, 0.f, fin);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = u2f(raw[e][j]) + 0.0f;
          val[4 * e + j] = v;
          const float m = idx(e, j) < cand ? v : NAN;
          vlo = fminf(vlo, m);
          vhi = fmaxf(vhi, m);
          fin = __builtin_fmaf(v, 0.f, fin);
        }
      }
    }
  }

  // ---- range of the row's candidates as keys (max and min in one reduction; a thread with
  //      no candidate contributes the neutral keys); a NaN or infinite score makes the
  //      maximum key the largest one, so the row has no finite range
  uint32_t kmin = vlo == vlo ? keyof(vlo) : 0xFFFFFFFFu;
  uint32_t kmax = fin != fin ? 0xFFFFFFFFu : (vhi == vhi ? keyof(vhi) : 0u);
  block_minmax<NT>(kmin, kmax, wsum);
  const RowOut out(a, t, lo, pbase, 0);
  if (cand == 0 || kmin == kmax) {
    // no candidate, or all scores equal: the lowest indices, in index order
    for (int j = tid; j < nsel; j += NT) out.store(j, f2u(key_score(kmin)), j);
    out.finish<NT>(a, t, nsel, u);
    return;
  }

  bool fast = false;     // order through the bins (below)
  int d1 = 0, a1 = 0, c1 = 0;   // the bin of the nsel-th largest score, candidates above it, in it
  const float vmin = key_score(kmin), vmax = key_score(kmax);
  const float span = vmax - vmin;
  const bool finite = span > 0.f && span < INFINITY;   // every candidate score finite, not all equal
  const float vscale = finite ? 2048.f / span : 0.f;
  const float voff = -vmin * vscale;
  // First-level bin: (v - vmin) * 2048 / span as one fma (any rounding keeps the bins
  // monotone in v). Second level (rows the first does not separate): the candidates of
  // first-level bins >= dex, over [lo2, hi2], those above hi2 clamped into the top bin; the
  // others get a spare slot.
  int lvl = 0, dex = 0;
  float vscale2 = 0.f, voff2 = 0.f;
  auto bin1 = [&](float x) { return min(2047, max(0, (int)__builtin_fmaf(x, vscale, voff))); };
  auto bin2 = [&](float x) { return min(2047, max(0, (int)__builtin_fmaf(x, vscale2, voff2))); };
  auto binof = [&](float x) {
    if (lvl == 0) return bin1(x);
    return bin1(x) >= dex ? bin2(x) : 2048 + (int)(threadIdx.x & 15);
  };
  // Bins over the two register layouts. With KEEP, slots past the row carry a bin of 2048 or
  // more (a spare slot), so no bin test below selects them; without it the `in` test does.
  auto binat = [&](int e, int j) {
    if constexpr (KEEP) return binA[4 * e + j]; else return binof(val[4 * e + j]);
  };
  auto cand_at = [&](int e, int j) {
    if constexpr (KEEP) return true; else return in(e, j);
  };
  auto run_pass = [&](int pass) {
    // ---- pass: 2048 bins linear in the score over [vmin, vmax]. Bins are monotone in the
    //      score, and a smooth score distribution spreads evenly over them, so the LDS
    //      atomics rarely collide and the threshold bin holds few candidates. The same bins
    //      then order the selection: bins at and above the threshold bin, taken from the
    //      top, are the selection in descending order up to the order inside each bin.
    //      Slots past the row count in 2048..2063 (spread over banks so that their atomics
    //      do not serialise on one address). A row the first level does not separate (a
    //      crowded threshold bin or selected bin, typically because a few outlying scores
    //      stretch [vmin, vmax]) is binned again, its candidates in first-level bins below
    //      the threshold bin left out, over the exact range from the smallest remaining
    //      score to the largest score in bins up to the 17th largest's; the at most 16
    //      scores above that go to the top bin.
    if (pass == 1) {
      // the second range: the smallest score in first-level bins >= d1 and the largest in
      // bins <= the 17th largest's
      const int dstar = misc[8];
      uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
      for (int e = 0; e < NCH; ++e)
        if (live(e)) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (in(e, j)) {
              int b1;
              if constexpr (KEEP) b1 = binA[4 * e + j]; else b1 = bin1(val[4 * e + j]);
              const uint32_t k = keyof(val[4 * e + j]);
              if (b1 >= d1) kmn = min(kmn, k);
              if (b1 <= dstar) kmx = max(kmx, k);
            }
        }
      block_minmax<NT>(kmn, kmx, wsum);
      if (kmn == 0xFFFFFFFFu || kmx == 0u) return;
      const float lo2 = key_score(kmn), hi2 = key_score(kmx);
      const float span2 = hi2 - lo2;
      if (!(span2 > 0.f && span2 < INFINITY)) return;
      dex = d1;
      vscale2 = 2048.f / span2;
      voff2 = -lo2 * vscale2;
      if (!(vscale2 < INFINITY) || !(fabsf(voff2) < INFINITY)) return;
      lvl = 1;
      __syncthreads();   // every thread has read misc and wsum above
    }
    for (int i = tid; i < kHistSlots / 4; i += NT) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) { misc[6] = 0; misc[8] = 2047; }
    __syncthreads();
    // (a group with no slot past the row skips the per-slot test: uniform branch)
    auto bin_slot = [&](int e, int j, bool inside) {
      int d = 2048 + (tid & 15);
      if (inside) {
        if constexpr (KEEP) d = lvl == 0 ? bin1(val[4 * e + j])
                                         : (binA[4 * e + j] >= dex ? bin2(val[4 * e + j]) : d);
        else d = binof(val[4 * e + j]);
      }
      if constexpr (KEEP) binA[4 * e + j] = d;
      atomicAdd(&hist[d], 1u);
    };
#pragma unroll
    for (int e = 0; e < NCH; ++e)
      if (live(e)) {
        if (full(e)) {
#pragma unroll
          for (int j = 0; j < 4; ++j) bin_slot(e, j, true);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) bin_slot(e, j, idx(e, j) < cand);
        }
      }
    __syncthreads();
    scan_pass1_bins<NT>(hist, nsel, wsum, misc, kBucketMax, 17);
    d1 = misc[0];
    a1 = misc[1];
    c1 = misc[2];
    // a bin at or above d1 of more than kBucketMax candidates (d1 itself included) is too
    // crowded to rank inside
    fast = misc[6] == 0;
  };
  if (finite) run_pass(0);
  if (finite && !fast) run_pass(1);

  if (fast) {
    // ---- every candidate of bins d1 .. 2047 (the selection, plus the rest of bin d1) takes
    //      the next slot of its bin's range as (~key, bin, index): ascending order inside a
    //      bin is score descending, then index ascending. The bin's word holds its first
    //      slot (count in higher bins) in its high half since the scan. Every score here is
    //      finite.
    u64* ord = selA;
#pragma unroll
    for (int e = 0; e < NCH; ++e)
      if (live(e)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = binat(e, j);
          if (cand_at(e, j) && d >= d1 && d < 2048) {
            const uint32_t slot = atomicAdd(&hist[d], 0x10000u) >> 16;
            ord[slot] = ((u64)(~keyof(val[4 * e + j])) << 32) | ((uint32_t)d << 16) | (uint32_t)idx(e, j);
          }
        }
      }
    __syncthreads();
    // ---- each entry's rank inside its bin gives its output position. After the scatter the
    //      high half of a bin's word is the end of its range (every entry of bins >= d1 was
    //      placed); bin d1 keeps its first nsel - a1 entries, which takes the lowest indices
    //      among scores equal to the last one taken. Two entries per thread at a time, so
    //      that their LDS reads overlap; a bin is read four entries at a time (reads past its
    //      end stay inside the workgroup's LDS and are masked out).
    const int krem1 = nsel - a1;
    const int n_ent = a1 + c1;
    auto store = [&](u64 v, int dest) {
      out.store(dest, f2u(key_score(~(uint32_t)(v >> 32))), (int)((uint32_t)v & 0xFFFFu));
    };
    for (int i0 = tid; i0 < n_ent; i0 += 2 * NT) {
      const bool two = i0 + NT < n_ent;
      const u64 v0 = ord[i0];
      const u64 v1 = two ? ord[i0 + NT] : 0ull;
      const int e0 = (int)(((uint32_t)v0 >> 16) & 2047u), e1 = (int)(((uint32_t)v1 >> 16) & 2047u);
      const uint32_t w0 = hist[e0], w1 = hist[e1];
      const int end0 = (int)(w0 >> 16), end1 = two ? (int)(w1 >> 16) : 0;
      const int b0 = end0 - (int)(w0 & 0xFFFFu);
      const int b1 = two ? end1 - (int)(w1 & 0xFFFFu) : 0;
      int r0 = 0, r1 = 0;
      for (int q = 0; b0 + q < end0 || b1 + q < end1; q += 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u64 x0 = ord[b0 + q + j], x1 = ord[b1 + q + j];
          r0 += b0 + q + j < end0 && x0 < v0;
          r1 += b1 + q + j < end1 && x1 < v1;
        }
      }
      if (e0 != d1 || r0 < krem1) store(v0, b0 + r0);
      if (two && (e1 != d1 || r1 < krem1)) store(v1, b1 + r1);
    }
    out.finish<NT>(a, t, nsel, u);
    return;
  }

  // Rows the bins do not separate (a selected bin of more than kBucketMax keys, the threshold
  // bin's included, or no finite score range) are left to topk_fallback_kernel, which finds
  // them by this negative length. Finishing them here would double this kernel's registers
  // (fewer rows in flight for every row) to save one launch.
  if (tid == 0) a.out_lengths[t] = -1;
}

// One row the bin ordering does not handle (a clustered threshold bin, a selected bin of more
// than kBucketMax keys, no finite score range), by the whole workgroup, from its keys in
// registers (0: no candidate, candidate c in key[4e+j] with c = 4(e*NT + tid) + j): the
// topk-th largest key by an 11 + 11 + 10-bit radix select; compaction by block prefix sums
// (keys above the threshold in any order, then the krem lowest-index keys equal to it);
// ordering by the bitonic network.
template <int NT, int EPT>
__device__ __forceinline__ void fallback_keys(const TopkArgs& a, const RowInfo& cur, const uint32_t (&key)[EPT],
                                              u64* sel, uint32_t* hist, int* wsum, int* misc) {
  static_assert(EPT % 4 == 0, "candidates are held in chunks of 4");
  constexpr int NCH = EPT / 4;
  const int tid = threadIdx.x;
  const int topk = a.topk;
  const int t = cur.t;
  const int cand = cur.cand, nsel = cur.nsel;
  auto live = [&](int e) { return 4 * e * NT < cand; };
  auto idx = [&](int e, int j) { return 4 * (e * NT + tid) + j; };
  uint32_t thr = 1u;    // every selected key is >= thr (all candidates when cand <= topk)
  int krem = cand;      // keys equal to thr that are taken, lowest indices first
  if (cand > topk) {
    uint32_t prefix = 0, pmask = 0;
    krem = topk;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nbins = pass == 2 ? 1024 : 2048;
      __syncthreads();
      for (int q = tid; q < 2048; q += NT) hist[q] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < NCH; ++e)
        if (live(e)) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t k = key[4 * e + j];
            if (k != 0u && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nbins - 1)], 1u);
          }
        }
      __syncthreads();
      find_rank_bin<NT, 2048>(hist, krem, wsum, misc);
      krem -= misc[1];
      prefix |= (uint32_t)misc[0] << shift;
      pmask |= (uint32_t)(nbins - 1) << shift;
    }
    thr = prefix;
  }

  // ---- compaction into sel[0, nsel): one block prefix sum of (above << 16 | equal)
  //      counts gives every thread its slots; only when fewer equal keys are taken than
  //      exist is their index order needed, from a second prefix sum with one count field
  //      per chunk group (index order is group-major)
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < NCH; ++e)
    if (live(e)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t k = key[4 * e + j];
        n_gt += k > thr;
        n_eq += k == thr && k != 0u;
      }
    }
  int tot;
  const int before = block_exclusive_sum<NT>((n_gt << 16) | n_eq, wsum, tot);
  const int ngt = tot >> 16, neq = tot & 0xFFFF;
  int pos_gt = before >> 16;
  if (neq <= krem) {
    int pos_eq = ngt + (before & 0xFFFF);
#pragma unroll
    for (int e = 0; e < NCH; ++e)
      if (live(e)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t k = key[4 * e + j];
          const u64 v = ((u64)(~k) << 32) | (uint32_t)idx(e, j);
          if (k > thr) sel[pos_gt++] = v;
          else if (k == thr && k != 0u) sel[pos_eq++] = v;
        }
      }
  } else {
    // group e's equal keys come after all equal keys of groups < e; inside group e,
    // thread order then position in the chunk. Fields of 16 bits, two groups per sum.
    int eq_before_group = 0;
#pragma unroll
    for (int e2 = 0; e2 < NCH; e2 += 2) {
      int c0 = 0, c1 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t k0 = key[4 * e2 + j];
        c0 += k0 == thr && k0 != 0u;
        if (e2 + 1 < NCH) {
          const uint32_t k1 = key[4 * (e2 + 1) + j];
          c1 += k1 == thr && k1 != 0u;
        }
      }
      int gtot;
      const int gb = block_exclusive_sum<NT>((c1 << 16) | c0, wsum, gtot);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = e2 + h;
        if (e < NCH) {
          int rank = eq_before_group + (h ? gb >> 16 : gb & 0xFFFF);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t k = key[4 * e + j];
            if (k == thr && k != 0u) {
              if (rank < krem) sel[ngt + rank] = ((u64)(~k) << 32) | (uint32_t)idx(e, j);
              ++rank;
            }
          }
          eq_before_group += h ? gtot >> 16 : gtot & 0xFFFF;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < NCH; ++e)
      if (live(e)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t k = key[4 * e + j];
          if (k > thr) sel[pos_gt++] = ((u64)(~k) << 32) | (uint32_t)idx(e, j);
        }
      }
  }

  // ---- ordering by the bitonic network, then the outputs
  int n2 = 64;
  while (n2 < nsel) n2 <<= 1;
  for (int q = nsel + tid; q < n2; q += NT) sel[q] = ~0ull;
  __syncthreads();
  if (n2 <= 128) bitonic_sort<1, NT>(sel, n2);
  else bitonic_sort<4, NT>(sel, n2);
  const RowOut out(a, t, cur.lo, cur.b);
  for (int j = tid; j < nsel; j += NT)
    out.store(j, f2u(key_score(~(uint32_t)(sel[j] >> 32))), (int)(uint32_t)sel[j]);
  out.finish<NT>(a, t, nsel, cur.u);
  __syncthreads();   // the row's LDS is reused by the next flagged row
}

template <int NT, int EPT>
__device__ __forceinline__ void fallback_row(const TopkArgs& a, int t, u64* sel, uint32_t* hist, int* wsum,
                                             int* misc) {
  constexpr int NCH = EPT / 4;
  const int tid = threadIdx.x;
  const RowInfo cur = row_info(a, t);
  const int cand = cur.cand;
  uint32_t key[EPT];   // 0: no candidate
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.scores + (long long)t * a.stride, cand * 4);
#pragma unroll
  for (int e = 0; e < NCH; ++e) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rr, (e * NT + tid) * 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = f2u(u2f(v[j]) + 0.0f);   // -0 + 0 = +0
      const uint32_t k = x ^ ((uint32_t)((int)x >> 31) | 0x80000000u);
      key[4 * e + j] = 4 * (e * NT + tid) + j < cand ? k : 0u;
    }
  }
  __syncthreads();   // the previous row's LDS contents are dead
  fallback_keys<NT, EPT>(a, cur, key, sel, hist, wsum, misc);
}

// Rows the fast kernel left (negative length): a fixed grid of workgroups, each reading the
// flags of 64 of its rows at a time (rows blockIdx.x + i*gridDim.x) and processing flagged
// rows one after the other.
template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_fallback_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  u64* sel = reinterpret_cast<u64*>(smem);                                   // [p2max]
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + a.hist_off);           // [kHistSlots]
  int* wsum = reinterpret_cast<int*>(hist + kHistSlots);                     // [32]
  int* misc = wsum + 32;                                                     // [16]
  const int lane = threadIdx.x & 63;
  const int G = gridDim.x;
  for (int r0 = blockIdx.x; r0 < a.T; r0 += 64 * G) {
    const int row = r0 + lane * G;
    const bool flagged = row < a.T && a.out_lengths[row] < 0;
    u64 m = __ballot(flagged);
    __syncthreads();   // every wave has read the flags before any row's length is rewritten
    while (m) {
      const int i = __ffsll((long long)m) - 1;
      m &= m - 1;
      fallback_row<NT, EPT>(a, __builtin_amdgcn_readfirstlane(r0 + i * G), sel, hist, wsum, misc);
    }
  }
}

// Launches kernel k (one of the two kernels at one shape) with `lds` bytes of dynamic LDS.
// A launch above the default 64 KB of dynamic LDS needs the kernel's limit raised first.
// The limit of a kernel only ever grows, to the largest size a launch of it has needed on
// that device: a launch captured into a graph earlier keeps a limit at least as large as
// its own when it is replayed after calls of smaller sizes. The check, the raise and the
// launch happen under one lock, so another host thread cannot change the limit in between.
template <int NT, void (*K)(TopkArgs)>
hipError_t launch_kernel(const TopkArgs& a, size_t lds, int grid, hipStream_t st) {
  if (lds <= 64 * 1024) {
    hipLaunchKernelGGL(K, dim3(grid), dim3(NT), lds, st, a);
    return hipGetLastError();
  }
  constexpr int kDevices = 64;
  static std::mutex mu;
  static size_t raised[kDevices] = {0};
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  // devices past the table get the largest limit any launch can need, once per call
  const size_t want = device < kDevices ? lds : kTopkMaxLds;
  if (device >= kDevices || raised[device] < want) {
    e = hipFuncSetAttribute((const void*)K, hipFuncAttributeMaxDynamicSharedMemorySize, (int)want);
    if (e != hipSuccess) return e;
    if (device < kDevices) raised[device] = want;
  }
  hipLaunchKernelGGL(K, dim3(grid), dim3(NT), lds, st, a);
  return hipGetLastError();
}

// A launch over every row only happens when no row has more than 4096 candidates (at most
// 16 per thread); wider shapes only run size classes.
template <int NT, int EPT>
hipError_t launch_cfg(const TopkArgs& a, size_t lds, int grid, hipStream_t st) {
  if (a.cls_map) return launch_kernel<NT, topk_kernel<NT, EPT, true>>(a, lds, grid, st);
  if constexpr (EPT <= 16) return launch_kernel<NT, topk_kernel<NT, EPT, false>>(a, lds, grid, st);
  return hipErrorInvalidValue;
}

template <int NT, int EPT>
hipError_t launch_fallback(const TopkArgs& a, size_t lds, int grid, hipStream_t st) {
  return launch_kernel<NT, topk_fallback_kernel<NT, EPT>>(a, lds, grid, st);
}

int p2_of(int topk, int max_cand) {
  int p2 = 64;
  while (p2 < topk && p2 < max_cand) p2 <<= 1;
  return p2;
}

}  // namespace

// Dynamic LDS layout: selA [p2max + kBucketMax] u64 (the selection and the rest of the
// threshold bin) | hist [kHistSlots] u32 | wsum [32] | misc [16].
int topk_hist_offset(int max_cand, int topk) { return (p2_of(topk, max_cand) + kBucketMax) * 8; }

size_t topk_lds_bytes(int max_cand, int topk) {
  return (size_t)topk_hist_offset(max_cand, topk) + kHistSlots * 4 + 32 * 4 + 16 * 4;
}

hipError_t launch_topk(const ScoreTopkLaunch& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  TopkArgs a;
  a.scores = p.scores; a.stride = p.stride; a.max_cand = p.max_cand;
  a.T = p.T; a.B = p.B; a.max_seqlen = p.max_seqlen; a.kpool = p.kpool; a.kpool_tail = p.kpool_tail;
  a.topk = p.topk;
  a.cu = p.cu; a.cu_pools = p.cu_pools;
  a.out_indices = p.out_indices; a.out_scores = p.out_scores; a.out_lengths = p.out_lengths;
  a.out_pool_indices = p.out_pool_indices;
  // Rows longer than 4096 candidates go to the smallest launch shape that holds them, one
  // launch per size class, longest rows first: a document's early positions have few
  // candidates and would otherwise run in the shape its longest row needs (fewer rows in
  // flight, more waiting waves per row). Shorter rows share one launch: below 4096 the
  // shapes differ little and an extra launch costs more than it saves.
  const int mc = p.max_cand;
  static const int kClassMax[] = {4096, 8192, 16384, kTopkMaxCand};
  int nclass = 0;
  while (kClassMax[nclass] < mc) ++nclass;
  for (int c = nclass; c >= 0; --c) {
    const int lo = c == 0 ? 0 : kClassMax[c - 1] + 1;
    const int hi = std::min(kClassMax[c], mc);
    a.cls_lo = lo; a.cls_hi = hi; a.cls_map = nclass > 0;
    a.p2max = p2_of(p.topk, hi);
    a.hist_off = topk_hist_offset(hi, p.topk);
    const size_t lds = topk_lds_bytes(hi, p.topk);
    long long grid = p.T;
    if (c < nclass) {   // positions [lo*kp - 1, hi*kp + kp - 2] of each document
      const long long ulo = lo == 0 ? 0 : (long long)lo * p.kpool - 1;
      const long long uhi = (long long)hi * p.kpool + p.kpool - 2;
      grid = std::min(grid, (long long)p.B * (uhi - ulo + 1));
    }
    if (grid <= 0) continue;
    hipError_t e;
    if (hi <= 1024) e = launch_cfg<256, 4>(a, lds, (int)grid, st);   // chunks of 4: at least 4 per thread
    // up to 2048 candidates: two waves of 16 per thread (each wave repeats the row's fixed
    // steps, and the kernel is bound by VALU issue: measured 3 % faster than four waves of 8;
    // at 4096 candidates two waves of 32 are 20 % slower, at 109 VGPRs)
    else if (hi <= 2048) e = launch_cfg<128, 16>(a, lds, (int)grid, st);
    else if (hi <= 4096) e = launch_cfg<256, 16>(a, lds, (int)grid, st);
    // Longer rows take more candidates per thread rather than wider workgroups: a
    // workgroup's serial steps (block reductions, the histogram scan) then cost
    // fewer waiting waves, and more rows are in flight per CU (measured: 8193-candidate rows
    // 1.5x faster as 256 x 32 than as 1024 x 16).
    else if (hi <= 8192) e = launch_cfg<256, 32>(a, lds, (int)grid, st);
    else if (hi <= 16384) e = launch_cfg<512, 32>(a, lds, (int)grid, st);
    else e = launch_cfg<1024, 32>(a, lds, (int)grid, st);
    if (e != hipSuccess) return e;
  }
  // Rows the bin kernels left (clustered or tied scores, no finite score range), found by
  // their negative length: one launch over a fixed grid in the shape of the longest row.
  a.cls_lo = 0; a.cls_hi = mc; a.cls_map = 0;
  a.p2max = p2_of(p.topk, mc);
  a.hist_off = topk_hist_offset(mc, p.topk);
  const size_t lds = topk_lds_bytes(mc, p.topk);
  const int grid = std::min(p.T, kFallbackGrid);
  if (mc <= 1024) return launch_fallback<256, 4>(a, lds, grid, st);
  if (mc <= 2048) return launch_fallback<256, 8>(a, lds, grid, st);
  if (mc <= 4096) return launch_fallback<256, 16>(a, lds, grid, st);
  if (mc <= 8192) return launch_fallback<256, 32>(a, lds, grid, st);
  if (mc <= 16384) return launch_fallback<512, 32>(a, lds, grid, st);
  return launch_fallback<1024, 32>(a, lds, grid, st);
}

}  // namespace dsa
