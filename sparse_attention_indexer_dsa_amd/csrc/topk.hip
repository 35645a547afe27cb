// Per-row top-k selection over the score workspace, with KPool expansion (gfx950).
//
// Each workgroup owns one query row. The row's candidate scores are loaded into LDS as
// order-preserving uint32 keys; a three-pass radix select (11 + 11 + 10 bits, LDS
// histograms with integer atomics) finds the k-th largest key; candidates above it are
// taken, and among candidates equal to it the lowest indices are taken (deterministic
// tie breaking, Megatron-LM PR 5992, "Key changes"). The selection is then sorted by
// (score descending, index ascending) with a bitonic sort in LDS and written with -1 /
// -inf padding. For KPool (PR 7522, "Changes") the selected pools are expanded to their
// tokens and the query's incomplete causal pool is appended when requested.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kNT = 256;

struct TopkArgs {
  const float* scores; int stride; int max_cand;
  int T, B, max_seqlen, kpool, kpool_tail, topk, p2;
  const int32_t* cu; const int32_t* cu_pools;
  int32_t* out_indices; float* out_scores; int32_t* out_lengths; int32_t* out_pool_indices;
};

// Inclusive suffix sum over kNT per-thread values (result: sum of values of threads >= tid).
__device__ __forceinline__ int block_suffix_sum(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kNT; off <<= 1) {
    const int o = tid + off < kNT ? buf[tid + off] : 0;
    __syncthreads();
    buf[tid] += o;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kNT) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  unsigned long long* sel = reinterpret_cast<unsigned long long*>(smem);          // [p2]
  uint32_t* hist = reinterpret_cast<uint32_t*>(sel + a.p2);                        // [2048]
  int* scan = reinterpret_cast<int*>(hist + 2048);                                 // [kNT]
  int* misc = scan + kNT;                                                          // [4]
  uint32_t* keys = reinterpret_cast<uint32_t*>(misc + 4);                          // [max_cand]

  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int b = find_doc(a.cu, a.B, t);
  const int lo = clampi(a.cu[b], 0, a.T);
  const int u = max(0, min(t - lo, a.max_seqlen - 1));
  const int kp = a.kpool;
  const int cand = min((u + 1) / kp, a.max_cand);
  const int topk = a.topk;
  const int nsel = min(topk, cand);
  const float* row = a.scores + (long long)t * a.stride;

  for (int i = tid; i < cand; i += kNT) keys[i] = score_key(row[i]);
  __syncthreads();

  if (cand <= topk) {
    for (int i = tid; i < cand; i += kNT)
      sel[i] = ((unsigned long long)(~keys[i]) << 32) | (uint32_t)i;
  } else {
    // ---- radix select of the topk-th largest key
    uint32_t prefix = 0, pmask = 0;
    int krem = topk;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nbins = pass == 2 ? 1024 : 2048;
      for (int i = tid; i < nbins; i += kNT) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < cand; i += kNT) {
        const uint32_t k = keys[i];
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (nbins - 1)], 1u);
      }
      __syncthreads();
      const int per = nbins / kNT;
      int mine = 0;
      for (int j = 0; j < per; ++j) mine += hist[tid * per + j];
      const int incl = block_suffix_sum(mine, scan);
      int above = incl - mine;                   // count in bins above this thread's range
      for (int j = per - 1; j >= 0; --j) {
        const int bin = tid * per + j;
        const int hcount = hist[bin];
        if (above < krem && krem <= above + hcount) { misc[0] = bin; misc[1] = above; }
        above += hcount;
      }
      __syncthreads();
      const int digit = misc[0];
      krem -= misc[1];
      prefix |= (uint32_t)digit << shift;
      pmask |= (uint32_t)(nbins - 1) << shift;
      __syncthreads();
    }
    const uint32_t thr = prefix;                 // the topk-th largest key; krem copies of it are taken
    // ---- compaction: keys above thr anywhere in [0, topk-krem); ties in index order after them
    const int chunk = (cand + kNT - 1) / kNT;
    const int i0 = min(cand, tid * chunk), i1 = min(cand, i0 + chunk);
    int ties = 0;
    for (int i = i0; i < i1; ++i) ties += keys[i] == thr;
    const int incl = block_suffix_sum(ties, scan);
    // ties of threads before this one = total - inclusive suffix
    if (tid == 0) { misc[2] = incl; misc[3] = 0; }
    __syncthreads();
    int rank = misc[2] - incl;
    const int ngt = topk - krem;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = keys[i];
      const unsigned long long v = ((unsigned long long)(~k) << 32) | (uint32_t)i;
      if (k > thr) {
        const int pos = atomicAdd(&misc[3], 1);
        sel[pos] = v;
      } else if (k == thr) {
        if (rank < krem) sel[ngt + rank] = v;
        ++rank;
      }
    }
  }
  for (int i = nsel + tid; i < a.p2; i += kNT) sel[i] = ~0ull;
  __syncthreads();

  // ---- bitonic sort (ascending on ~key:index = score descending, index ascending)
  int n2 = 1;
  while (n2 < nsel) n2 <<= 1;
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += kNT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = sel[i], y = sel[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) { sel[i] = y; sel[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }

  // ---- outputs
  float* os = a.out_scores + (long long)t * topk;
  for (int j = tid; j < topk; j += kNT)
    os[j] = j < nsel ? key_score(~(uint32_t)(sel[j] >> 32)) : -INFINITY;
  if (kp == 1) {
    int32_t* oi = a.out_indices + (long long)t * topk;
    for (int j = tid; j < topk; j += kNT) oi[j] = j < nsel ? lo + (int)(uint32_t)sel[j] : -1;
    if (tid == 0) a.out_lengths[t] = nsel;
  } else {
    const int pbase = a.cu_pools[b];
    if (a.out_pool_indices) {
      int32_t* op = a.out_pool_indices + (long long)t * topk;
      for (int j = tid; j < topk; j += kNT) op[j] = j < nsel ? pbase + (int)(uint32_t)sel[j] : -1;
    }
    const int tail = a.kpool_tail ? (u + 1) % kp : 0;
    const int width = topk * kp + kp - 1;
    const int npool_tok = nsel * kp;
    const int tail_start = lo + (u / kp) * kp;
    int32_t* oi = a.out_indices + (long long)t * width;
    for (int s = tid; s < width; s += kNT) {
      int v = -1;
      if (s < npool_tok) v = lo + (int)(uint32_t)sel[s / kp] * kp + s % kp;
      else if (s < npool_tok + tail) v = tail_start + (s - npool_tok);
      oi[s] = v;
    }
    if (tid == 0) a.out_lengths[t] = npool_tok + tail;
  }
}

}  // namespace

size_t topk_lds_bytes(int max_cand, int p2) {
  return (size_t)p2 * 8 + 2048 * 4 + kNT * 4 + 16 + (size_t)max_cand * 4;
}

hipError_t launch_topk(const ScoreTopkLaunch& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  TopkArgs a;
  a.scores = p.scores; a.stride = p.stride; a.max_cand = p.max_cand;
  a.T = p.T; a.B = p.B; a.max_seqlen = p.max_seqlen; a.kpool = p.kpool; a.kpool_tail = p.kpool_tail;
  a.topk = p.topk;
  int p2 = 1;
  while (p2 < p.topk && p2 < p.max_cand) p2 <<= 1;
  a.p2 = p2;
  a.cu = p.cu; a.cu_pools = p.cu_pools;
  a.out_indices = p.out_indices; a.out_scores = p.out_scores; a.out_lengths = p.out_lengths;
  a.out_pool_indices = p.out_pool_indices;
  const size_t lds = topk_lds_bytes(p.max_cand, p2);
  // Raise the dynamic LDS limit to the full 160 KB once per device (not a stream
  // operation, so it is done before any graph capture reaches here).
  static std::mutex mu;
  static uint64_t done_mask = 0;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (device >= 64 || !(done_mask >> device & 1)) {
      e = hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
      if (device < 64) done_mask |= 1ull << device;
    }
  }
  hipLaunchKernelGGL(topk_kernel, dim3(p.T), dim3(kNT), lds, st, a);
  return hipGetLastError();
}

}  // namespace dsa
