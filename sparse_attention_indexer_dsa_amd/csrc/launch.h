// Internal launcher interface between the C ABI layer (api.cpp) and the kernels.
// Arguments here are already validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

enum { kPrecBF16 = 0, kPrecFP8 = 1, kPrecMXFP8 = 2 };

struct PreprocessLaunch {
  const void* q_in; const void* k_in; bool in_bf16;
  int T, S, H, D;
  const int32_t* cu; int B;
  const float* gamma; const float* beta; float eps;
  const float* cos_t; const float* sin_t;
  int rope_dim, max_pos, interleaved, rope_fp32;
  int precision;
  void* q_op; uint8_t* q_scale; void* k_op; uint8_t* k_scale;
  float* q_f32; float* k_f32;
};
hipError_t launch_preprocess(const PreprocessLaunch& p, hipStream_t st);

struct KpoolLaunch {
  const void* k; bool k_bf16; int S, D;
  const int32_t* cu; int B;
  const uint16_t* gate; const float* bias; int kpool;
  int precision;
  void* pooled; uint8_t* pooled_scale; int32_t* cu_pools;
};
hipError_t launch_kpool(const KpoolLaunch& p, hipStream_t st);

struct ScoreTopkLaunch {
  const void* q_op; const uint8_t* q_scale;
  const void* k_op; const uint8_t* k_scale;
  const void* w; bool w_bf16;
  int T, S, H, D;
  const int32_t* cu; int B; int max_seqlen;
  int kpool; const int32_t* cu_pools; int kpool_tail;
  int topk; float sm_scale; int precision;
  int32_t* out_indices; float* out_scores; int32_t* out_lengths; int32_t* out_pool_indices;
  float* scores;          // workspace: [T, stride] fp32
  int stride;             // row stride of the score workspace (floats)
  int max_cand;           // candidates per row upper bound
  // Fused query preprocessing (q_in != nullptr): the scoring kernel builds its q operands
  // from the raw queries (RoPE, carrier rounding, quantisation); q_op / q_scale unused.
  const void* q_in = nullptr; bool in_bf16 = true;
  const float* cos_t = nullptr; const float* sin_t = nullptr;
  int rope_dim = 0, max_pos = 0, interleaved = 0, rope_fp32 = 0;
  void* q_op_out = nullptr; uint8_t* q_scale_out = nullptr;   // optional copies of those operands
};
// Whether the fused query preprocessing supports this RoPE layout (rotate-half partners must
// sit in the same lane of the MFMA operand layout).
bool score_can_fuse_rope(int precision, int rope_dim, int interleaved);
hipError_t launch_score(const ScoreTopkLaunch& p, hipStream_t st);
hipError_t launch_topk(const ScoreTopkLaunch& p, hipStream_t st);

// Fixed device scratch of the entry point that allocates nothing (noalloc.hip): the size of
// the array on every GPU, and its address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t(128) << 20) + 4096;
hipError_t noalloc_scratch(void** out);

hipError_t launch_selection_softmax(const float* scores, int T, int topk, float* out, hipStream_t st);

// Sparse absorbed-MLA attention: latent entry width (key) and value width, in elements.
constexpr int kMlaKeyWidth = 576;
constexpr int kMlaValueWidth = 512;
hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const int32_t* lengths,
                             int T, int H, int S, int topk, float sm_scale, uint16_t* out, float* lse,
                             hipStream_t st);

// Largest row (candidates) the LDS top-k supports, and the most LDS a workgroup can hold
// (gfx950: 160 KB per CU).
constexpr int kTopkMaxCand = 32768;
constexpr size_t kTopkMaxLds = 160 * 1024;

// On-device peak measurements (peak.hip)
double mfma_peak_flops(int precision, int blocks, int iters);
int mfma_peak_threads();
hipError_t launch_mfma_peak(int precision, int blocks, int iters, float* out, hipStream_t st);
hipError_t launch_stream(const void* src, void* dst, size_t bytes, int copy, hipStream_t st);

}  // namespace dsa
