// Softmax over each row's selected scores (gfx950).
//
// The optional third output of the indexer's top-k, the predicted distribution its loss
// reuses (Megatron-LM PR 5992 reviews: "What was verified", the return arity with
// return_softmax; "Areas checked and found clean", the loss reusing the compact softmax):
// p_j = exp(s_j - m) / sum_i exp(s_i - m) over the row's selected scores, m their maximum;
// padding (-inf) gets 0 and a row with nothing selected is all zeros.
//
// One wave per row, four rows per workgroup, every lane summing its own entries in a fixed
// order and the wave reductions fixed DPP trees, so the result does not depend on
// scheduling. Rows of up to 2048 entries (a multiple of 4, 16-byte aligned) are held in
// registers: 16-byte loads, one read and one write of the row. Other rows take lane l's
// entries l, l+64, ... and read the row three times (maximum, sum, output; the later reads
// hit the cache). Every lane reads only the entries it writes, so the output may overwrite
// the scores.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

// Wave-wide max and sum of fp32 values by fixed DPP trees (row shifts, then the row
// broadcasts of lanes 15 and 31), result read from lane 63.
__device__ __forceinline__ float wave_max_f32(float x) {
  const int id = (int)0xFF800000u;   // -inf
#define DSA_STEP(ctrl, rm) x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(x), ctrl, rm, 0xf, false)));
  DSA_STEP(0x111, 0xf) DSA_STEP(0x112, 0xf) DSA_STEP(0x114, 0xf) DSA_STEP(0x118, 0xf)
  DSA_STEP(0x142, 0xa) DSA_STEP(0x143, 0xc)
#undef DSA_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ float wave_sum_f32(float x) {
#define DSA_STEP(ctrl, rm) x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rm, 0xf, false));
  DSA_STEP(0x111, 0xf) DSA_STEP(0x112, 0xf) DSA_STEP(0x114, 0xf) DSA_STEP(0x118, 0xf)
  DSA_STEP(0x142, 0xa) DSA_STEP(0x143, 0xc)
#undef DSA_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__global__ __launch_bounds__(256) void selection_softmax_kernel(const float* scores, int T, int topk, float* out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                            // whole waves: no cross-wave work
  const float* s = scores + (long long)t * topk;
  float* o = out + (long long)t * topk;
  float m = -INFINITY;
  for (int j = lane; j < topk; j += 64) m = fmaxf(m, s[j]);
  m = wave_max_f32(m);
  if (m == -INFINITY) {                          // nothing selected
    for (int j = lane; j < topk; j += 64) o[j] = 0.f;
    return;
  }
  float sum = 0.f;
  for (int j = lane; j < topk; j += 64) sum += expf(s[j] - m);   // exp(-inf) = 0 for padding
  sum = wave_sum_f32(sum);
  for (int j = lane; j < topk; j += 64) o[j] = expf(s[j] - m) / sum;
}

// Rows of at most 256*V entries in registers: lane l holds the 4-entry chunks c*64 + l.
template <int V>
__global__ __launch_bounds__(256) void selection_softmax_reg_kernel(const float* scores, int T, int topk, float* out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                            // whole waves: no cross-wave work
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(scores + (long long)t * topk, topk * 4);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + (long long)t * topk, topk * 4);
  float x[4 * V];
#pragma unroll
  for (int c = 0; c < V; ++c) {
    const auto r = __builtin_amdgcn_raw_buffer_load_b128(rin, (c * 64 + lane) * 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[4 * c + j] = 4 * (c * 64 + lane) + j < topk ? u2f(r[j]) : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4 * V; ++k) m = fmaxf(m, x[k]);
  m = wave_max_f32(m);
  float sum = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int k = 0; k < 4 * V; ++k) {
      x[k] = expf(x[k] - m);                     // exp(-inf) = 0 for padding
      sum += x[k];
    }
    sum = wave_sum_f32(sum);
  }
#pragma unroll
  for (int c = 0; c < V; ++c) {
    __attribute__((ext_vector_type(4))) uint32_t w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = f2u(m == -INFINITY ? 0.f : x[4 * c + j] / sum);
    __builtin_amdgcn_raw_buffer_store_b128(w, rout, (c * 64 + lane) * 16, 0, 0);   // past the row: dropped
  }
}

}  // namespace

hipError_t launch_selection_softmax(const float* scores, int T, int topk, float* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  const bool vec = topk % 4 == 0 && reinterpret_cast<uintptr_t>(scores) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(out) % 16 == 0;
  if (vec && topk <= 256) hipLaunchKernelGGL(selection_softmax_reg_kernel<1>, grid, block, 0, st, scores, T, topk, out);
  else if (vec && topk <= 512) hipLaunchKernelGGL(selection_softmax_reg_kernel<2>, grid, block, 0, st, scores, T, topk, out);
  else if (vec && topk <= 1024) hipLaunchKernelGGL(selection_softmax_reg_kernel<4>, grid, block, 0, st, scores, T, topk, out);
  else if (vec && topk <= 2048) hipLaunchKernelGGL(selection_softmax_reg_kernel<8>, grid, block, 0, st, scores, T, topk, out);
  else hipLaunchKernelGGL(selection_softmax_kernel, grid, block, 0, st, scores, T, topk, out);
  return hipGetLastError();
}

}  // namespace dsa
