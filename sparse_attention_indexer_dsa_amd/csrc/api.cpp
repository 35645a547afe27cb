// C ABI of the indexer library: host-side validation, workspace sizing and dispatch.
// Nothing here allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/dsa_bench.h"
#include "../../include/dsa_index.h"
#include "launch.h"

namespace dsa {
size_t topk_lds_bytes(int max_cand, int topk);
}

namespace {

thread_local std::string g_last_error;

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status_t device_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_precision(int p) { return p == DSA_PREC_BF16 || p == DSA_PREC_FP8 || p == DSA_PREC_MXFP8; }

dsa_status_t check_precision(int p) {
  if (!valid_precision(p))
    return fail(DSA_ERR_UNSUPPORTED,
                "unsupported DSA indexer scoring precision %d; expected bf16 (0), fp8 (1) or mxfp8 (2)", p);
  return DSA_OK;
}

dsa_status_t check_hd(int H, int D, bool need_h) {
  if (D <= 0 || (need_h && H <= 0)) return fail(DSA_ERR_INVALID_ARGUMENT, "H and D must be positive (H=%d, D=%d)", H, D);
  if (need_h && H != 16 && H != 32 && H != 64)
    return fail(DSA_ERR_UNSUPPORTED, "indexer heads H=%d unsupported; expected 16, 32 or 64", H);
  if (D != 64 && D != 128) return fail(DSA_ERR_UNSUPPORTED, "head dim D=%d unsupported; expected 64 or 128", D);
  return DSA_OK;
}

int max_candidates(int max_seqlen, int kpool) { return kpool == 1 ? max_seqlen : max_seqlen / kpool; }

int row_stride(int max_cand) {
  const int c = max_cand < 1 ? 1 : max_cand;
  return (c + 63) / 64 * 64;
}

constexpr size_t kMaxLds = dsa::kTopkMaxLds;

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status_t dsa_index_preprocess(
    const void* q_in, const void* k_in, dsa_dtype_t in_dtype,
    int32_t T, int32_t S, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs,
    const float* ln_gamma, const float* ln_beta, float ln_eps,
    const float* rope_cos, const float* rope_sin,
    int32_t rope_dim, int32_t rope_max_pos, int32_t rope_interleaved,
    int32_t rope_fp32, dsa_precision_t precision,
    void* q_op, uint8_t* q_scale, void* k_op, uint8_t* k_scale,
    float* q_f32_out, float* k_f32_out,
    hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_precision((int)precision)) != DSA_OK) return st;
  if (in_dtype != DSA_DTYPE_BF16 && in_dtype != DSA_DTYPE_FP32)
    return fail(DSA_ERR_INVALID_ARGUMENT, "in_dtype %d must be bf16 (0) or fp32 (1)", (int)in_dtype);
  if (!q_in && !k_in) return fail(DSA_ERR_INVALID_ARGUMENT, "q_in and k_in are both NULL");
  if (T < 0 || S < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "T=%d and S=%d must be non-negative", T, S);
  if (q_in && k_in && T != S) return fail(DSA_ERR_INVALID_ARGUMENT, "T=%d != S=%d: queries and keys share cu_seqlens", T, S);
  if ((st = check_hd(H, D, q_in != nullptr)) != DSA_OK) return st;
  if (!cu_seqlens || num_seqs < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "cu_seqlens must be given with num_seqs >= 1");
  if (rope_dim < 0 || rope_dim > D || (rope_dim % 2) != 0)
    return fail(DSA_ERR_UNSUPPORTED, "rope_dim=%d must be even and within [0, D=%d]", rope_dim, D);
  if (rope_dim > 0 && !rope_interleaved && rope_dim % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "rotate-half RoPE needs rope_dim %% 32 == 0 (got %d)", rope_dim);
  if (rope_dim > 0 && (!rope_cos || !rope_sin || rope_max_pos < 1))
    return fail(DSA_ERR_INVALID_ARGUMENT, "rope tables and rope_max_pos >= 1 required when rope_dim > 0");
  if (rope_dim > 0 && (!aligned(rope_cos, 16) || !aligned(rope_sin, 16)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "rope tables must be 16-byte aligned");
  const bool fp8 = precision != DSA_PREC_BF16;
  if (q_in) {
    if (!q_op) return fail(DSA_ERR_INVALID_ARGUMENT, "q_op is NULL");
    if (fp8 && !q_scale) return fail(DSA_ERR_INVALID_ARGUMENT, "q_scale is NULL for an fp8 precision");
    if (!aligned(q_in, 16) || !aligned(q_op, 16) || (q_f32_out && !aligned(q_f32_out, 16)))
      return fail(DSA_ERR_INVALID_ARGUMENT, "query buffers must be 16-byte aligned");
  }
  if (k_in) {
    if (!k_op) return fail(DSA_ERR_INVALID_ARGUMENT, "k_op is NULL");
    if (fp8 && !k_scale) return fail(DSA_ERR_INVALID_ARGUMENT, "k_scale is NULL for an fp8 precision");
    if (!aligned(k_in, 16) || !aligned(k_op, 16) || (k_f32_out && !aligned(k_f32_out, 16)))
      return fail(DSA_ERR_INVALID_ARGUMENT, "key buffers must be 16-byte aligned");
  }
  dsa::PreprocessLaunch p;
  p.q_in = q_in; p.k_in = k_in; p.in_bf16 = in_dtype == DSA_DTYPE_BF16;
  p.T = q_in ? T : 0; p.S = k_in ? S : 0; p.H = H; p.D = D;
  p.cu = cu_seqlens; p.B = num_seqs;
  p.gamma = ln_gamma; p.beta = ln_beta; p.eps = ln_eps;
  p.cos_t = rope_cos; p.sin_t = rope_sin;
  p.rope_dim = rope_dim; p.max_pos = rope_max_pos; p.interleaved = rope_interleaved ? 1 : 0;
  p.rope_fp32 = rope_fp32 ? 1 : 0; p.precision = (int)precision;
  p.q_op = q_op; p.q_scale = q_scale; p.k_op = k_op; p.k_scale = k_scale;
  p.q_f32 = q_f32_out; p.k_f32 = k_f32_out;
  hipError_t e = dsa::launch_preprocess(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_preprocess");
  return DSA_OK;
}

dsa_status_t dsa_index_kpool(
    const void* k, dsa_dtype_t k_dtype, int32_t S, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs,
    const uint16_t* gate_bf16, const float* slot_bias, int32_t kpool,
    dsa_precision_t precision,
    void* pooled_op, uint8_t* pooled_scale, int32_t* cu_pools,
    hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_precision((int)precision)) != DSA_OK) return st;
  if (k_dtype != DSA_DTYPE_BF16 && k_dtype != DSA_DTYPE_FP32)
    return fail(DSA_ERR_INVALID_ARGUMENT, "k_dtype %d must be bf16 (0) or fp32 (1)", (int)k_dtype);
  if ((st = check_hd(0, D, false)) != DSA_OK) return st;
  if (S < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "S=%d must be non-negative", S);
  if (kpool < 1 || kpool > 64) return fail(DSA_ERR_UNSUPPORTED, "kpool=%d must be within [1, 64]", kpool);
  if (!cu_seqlens || num_seqs < 1 || !cu_pools)
    return fail(DSA_ERR_INVALID_ARGUMENT, "cu_seqlens, num_seqs >= 1 and cu_pools are required");
  if (S > 0 && (!k || !gate_bf16 || !slot_bias || !pooled_op))
    return fail(DSA_ERR_INVALID_ARGUMENT, "k, gate_bf16, slot_bias and pooled_op are required");
  if (precision != DSA_PREC_BF16 && S / kpool > 0 && !pooled_scale)
    return fail(DSA_ERR_INVALID_ARGUMENT, "pooled_scale is NULL for an fp8 precision");
  dsa::KpoolLaunch p;
  p.k = k; p.k_bf16 = k_dtype == DSA_DTYPE_BF16; p.S = S; p.D = D;
  p.cu = cu_seqlens; p.B = num_seqs;
  p.gate = gate_bf16; p.bias = slot_bias; p.kpool = kpool;
  p.precision = (int)precision;
  p.pooled = pooled_op; p.pooled_scale = pooled_scale; p.cu_pools = cu_pools;
  hipError_t e = dsa::launch_kpool(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_kpool");
  return DSA_OK;
}

size_t dsa_index_workspace_size(int32_t T, int32_t H, int32_t D, int32_t num_seqs,
                                int32_t max_seqlen, int32_t topk, int32_t kpool,
                                dsa_precision_t precision) {
  (void)H; (void)D; (void)num_seqs; (void)topk; (void)precision;
  if (T < 0 || max_seqlen < 0 || kpool < 1) return 0;
  const int stride = row_stride(max_candidates(max_seqlen, kpool));
  return (size_t)T * (size_t)stride * sizeof(float) + 256;
}

namespace {

// Per-document byte offsets into keys and score rows are 32-bit in the kernels.
constexpr int kMaxCandidates = 1 << 22;

// Validation shared by the scoring and selection entry points. Fills `p` on success.
dsa_status_t check_geometry(int T, const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int kpool,
                            const int32_t* cu_pools, int topk, bool need_topk) {
  if (T < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "T=%d must be non-negative", T);
  if (need_topk && topk < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "topk=%d must be >= 1", topk);
  if (kpool < 1 || kpool > 64) return fail(DSA_ERR_UNSUPPORTED, "kpool=%d must be within [1, 64]", kpool);
  if (kpool > 1 && !cu_pools) return fail(DSA_ERR_INVALID_ARGUMENT, "cu_pools is required when kpool > 1");
  if (!cu_seqlens || num_seqs < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "cu_seqlens must be given with num_seqs >= 1");
  if (max_seqlen < 0 || (T > 0 && max_seqlen < 1))
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_seqlen=%d must be >= 1", max_seqlen);
  const int max_cand = max_candidates(max_seqlen, kpool);
  if (max_cand > kMaxCandidates)
    return fail(DSA_ERR_UNSUPPORTED, "%d candidates per row exceed the supported %d", max_cand, kMaxCandidates);
  if (need_topk) {
    if (max_cand > dsa::kTopkMaxCand)
      return fail(DSA_ERR_UNSUPPORTED, "%d candidates per row exceed the supported %d", max_cand, dsa::kTopkMaxCand);
    if (dsa::topk_lds_bytes(max_cand, topk) > kMaxLds)
      return fail(DSA_ERR_UNSUPPORTED, "topk=%d with %d candidates per row exceeds the on-chip selection buffer",
                  topk, max_cand);
    if ((long long)topk * kpool + kpool - 1 > 0x7FFFFFFFLL)
      return fail(DSA_ERR_INVALID_ARGUMENT, "topk*kpool overflows");
  }
  return DSA_OK;
}

dsa_status_t check_score_args(const void* q_op, const uint8_t* q_scale, const void* k_op, const uint8_t* k_scale,
                              const void* w, dsa_dtype_t w_dtype, int T, int S, int H, int D, int precision,
                              const void* workspace, bool need_ws = true) {
  dsa_status_t st;
  if ((st = check_precision(precision)) != DSA_OK) return st;
  if (w_dtype != DSA_DTYPE_BF16 && w_dtype != DSA_DTYPE_FP32)
    return fail(DSA_ERR_INVALID_ARGUMENT, "w_dtype %d must be bf16 (0) or fp32 (1)", (int)w_dtype);
  if (T < 0 || S < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "T=%d and S=%d must be non-negative", T, S);
  if ((st = check_hd(H, D, true)) != DSA_OK) return st;
  if (T == 0) return DSA_OK;
  const bool fp8 = precision != DSA_PREC_BF16;
  if (!q_op || !w || (need_ws && !workspace)) return fail(DSA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (S > 0 && !k_op) return fail(DSA_ERR_INVALID_ARGUMENT, "k_op is NULL");
  if (fp8 && (!q_scale || (S > 0 && !k_scale)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q_scale/k_scale are required for an fp8 precision");
  if (!aligned(q_op, 16) || (k_op && !aligned(k_op, 16)) || (need_ws && !aligned(workspace, 256)) ||
      !aligned(w, w_dtype == DSA_DTYPE_FP32 ? 4 : 2))
    return fail(DSA_ERR_INVALID_ARGUMENT, "misaligned buffer (operands 16 B, workspace 256 B, weights 4 B)");
  return DSA_OK;
}

dsa_status_t check_outputs(const int32_t* oi, const float* os, const int32_t* ol, const int32_t* op,
                           const void* workspace, bool need_ws = true) {
  if (!oi || !os || !ol || (need_ws && !workspace))
    return fail(DSA_ERR_INVALID_ARGUMENT, "a required output pointer is NULL");
  if (!aligned(oi, 4) || !aligned(os, 4) || !aligned(ol, 4) || (op && !aligned(op, 4)) ||
      (need_ws && !aligned(workspace, 256)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "misaligned output (4 B) or workspace (256 B)");
  return DSA_OK;
}

dsa::ScoreTopkLaunch make_launch(const void* q_op, const uint8_t* q_scale, const void* k_op, const uint8_t* k_scale,
                                 const void* w, dsa_dtype_t w_dtype, int T, int S, int H, int D,
                                 const int32_t* cu, int B, int max_seqlen, int kpool, const int32_t* cu_pools,
                                 int kpool_tail, int topk, float sm_scale, int precision, int32_t* oi, float* os,
                                 int32_t* ol, int32_t* op, const void* workspace) {
  dsa::ScoreTopkLaunch p;
  p.q_op = q_op; p.q_scale = q_scale; p.k_op = k_op; p.k_scale = k_scale;
  p.w = w; p.w_bf16 = w_dtype == DSA_DTYPE_BF16;
  p.T = T; p.S = S; p.H = H; p.D = D;
  p.cu = cu; p.B = B; p.max_seqlen = max_seqlen;
  p.kpool = kpool; p.cu_pools = cu_pools; p.kpool_tail = kpool_tail ? 1 : 0;
  p.topk = topk; p.sm_scale = sm_scale; p.precision = precision;
  p.out_indices = oi; p.out_scores = os; p.out_lengths = ol;
  p.out_pool_indices = kpool > 1 ? op : nullptr;
  p.scores = static_cast<float*>(const_cast<void*>(workspace));
  const int max_cand = max_candidates(max_seqlen, kpool);
  p.stride = row_stride(max_cand);
  p.max_cand = max_cand;
  return p;
}

}  // namespace

dsa_status_t dsa_index_score(
    const void* q_op, const uint8_t* q_scale,
    const void* k_op, const uint8_t* k_scale,
    const void* w, dsa_dtype_t w_dtype,
    int32_t T, int32_t S, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    int32_t kpool, const int32_t* cu_pools,
    float sm_scale, dsa_precision_t precision,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_score_args(q_op, q_scale, k_op, k_scale, w, w_dtype, T, S, H, D, (int)precision, workspace)) != DSA_OK)
    return st;
  if ((st = check_geometry(T, cu_seqlens, num_seqs, max_seqlen, kpool, cu_pools, 1, false)) != DSA_OK) return st;
  if (T == 0) return DSA_OK;
  const size_t need = dsa_index_workspace_size(T, H, D, num_seqs, max_seqlen, 1, kpool, precision);
  if (workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  dsa::ScoreTopkLaunch p = make_launch(q_op, q_scale, k_op, k_scale, w, w_dtype, T, S, H, D, cu_seqlens, num_seqs,
                                       max_seqlen, kpool, cu_pools, 0, 1, sm_scale, (int)precision, nullptr, nullptr,
                                       nullptr, nullptr, workspace);
  hipError_t e = dsa::launch_score(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_score");
  return DSA_OK;
}

dsa_status_t dsa_index_topk(
    const void* workspace, size_t workspace_bytes,
    int32_t T, const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    int32_t kpool, const int32_t* cu_pools, int32_t kpool_tail, int32_t topk,
    int32_t* out_indices, float* out_scores, int32_t* out_lengths, int32_t* out_pool_indices,
    hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_geometry(T, cu_seqlens, num_seqs, max_seqlen, kpool, cu_pools, topk, true)) != DSA_OK) return st;
  if (T == 0) return DSA_OK;
  if ((st = check_outputs(out_indices, out_scores, out_lengths, out_pool_indices, workspace)) != DSA_OK) return st;
  const size_t need = dsa_index_workspace_size(T, 0, 0, num_seqs, max_seqlen, topk, kpool, DSA_PREC_BF16);
  if (workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  dsa::ScoreTopkLaunch p = make_launch(nullptr, nullptr, nullptr, nullptr, nullptr, DSA_DTYPE_FP32, T, 0, 0, 0,
                                       cu_seqlens, num_seqs, max_seqlen, kpool, cu_pools, kpool_tail, topk, 1.0f,
                                       0, out_indices, out_scores, out_lengths, out_pool_indices, workspace);
  hipError_t e = dsa::launch_topk(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_topk");
  return DSA_OK;
}

dsa_status_t dsa_index_score_topk(
    const void* q_op, const uint8_t* q_scale,
    const void* k_op, const uint8_t* k_scale,
    const void* w, dsa_dtype_t w_dtype,
    int32_t T, int32_t S, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    int32_t kpool, const int32_t* cu_pools, int32_t kpool_tail,
    int32_t topk, float sm_scale, dsa_precision_t precision,
    int32_t* out_indices, float* out_scores, int32_t* out_lengths,
    int32_t* out_pool_indices,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_score_args(q_op, q_scale, k_op, k_scale, w, w_dtype, T, S, H, D, (int)precision, workspace)) != DSA_OK)
    return st;
  if ((st = check_geometry(T, cu_seqlens, num_seqs, max_seqlen, kpool, cu_pools, topk, true)) != DSA_OK) return st;
  if (T == 0) return DSA_OK;
  if ((st = check_outputs(out_indices, out_scores, out_lengths, out_pool_indices, workspace)) != DSA_OK) return st;
  const size_t need = dsa_index_workspace_size(T, H, D, num_seqs, max_seqlen, topk, kpool, precision);
  if (workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  dsa::ScoreTopkLaunch p = make_launch(q_op, q_scale, k_op, k_scale, w, w_dtype, T, S, H, D, cu_seqlens, num_seqs,
                                       max_seqlen, kpool, cu_pools, kpool_tail, topk, sm_scale, (int)precision,
                                       out_indices, out_scores, out_lengths, out_pool_indices, workspace);
  hipError_t e = dsa::launch_score(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_score_topk (score)");
  e = dsa::launch_topk(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_score_topk (top-k)");
  return DSA_OK;
}

dsa_status_t dsa_index_score_topk_noalloc(
    const void* q_op, const uint8_t* q_scale,
    const void* k_op, const uint8_t* k_scale,
    const void* w, dsa_dtype_t w_dtype,
    int32_t T, int32_t S, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    int32_t kpool, const int32_t* cu_pools, int32_t kpool_tail,
    int32_t topk, float sm_scale, dsa_precision_t precision,
    int32_t* out_indices, float* out_scores, int32_t* out_lengths,
    int32_t* out_pool_indices, hipStream_t stream) {
  static_assert(DSA_NOALLOC_SCRATCH_BYTES == dsa::kNoAllocScratchBytes, "scratch size of the header and the library");
  dsa_status_t st;
  if ((st = check_score_args(q_op, q_scale, k_op, k_scale, w, w_dtype, T, S, H, D, (int)precision, nullptr,
                             false)) != DSA_OK)
    return st;
  if ((st = check_geometry(T, cu_seqlens, num_seqs, max_seqlen, kpool, cu_pools, topk, true)) != DSA_OK) return st;
  if (T == 0) return DSA_OK;
  if ((st = check_outputs(out_indices, out_scores, out_lengths, out_pool_indices, nullptr, false)) != DSA_OK)
    return st;
  const size_t need = dsa_index_workspace_size(T, H, D, num_seqs, max_seqlen, topk, kpool, precision);
  if (need > dsa::kNoAllocScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED,
                "dsa_index_score_topk_noalloc: T=%d rows of max_seqlen=%d (kpool %d) need %zu bytes of scratch; "
                "the fixed scratch holds %zu (use dsa_index_score_topk with a workspace)",
                T, max_seqlen, kpool, need, dsa::kNoAllocScratchBytes);
  void* scratch = nullptr;
  hipError_t e = dsa::noalloc_scratch(&scratch);
  if (e != hipSuccess) return device_fail(e, "dsa_index_score_topk_noalloc (scratch address)");
  dsa::ScoreTopkLaunch p = make_launch(q_op, q_scale, k_op, k_scale, w, w_dtype, T, S, H, D, cu_seqlens, num_seqs,
                                       max_seqlen, kpool, cu_pools, kpool_tail, topk, sm_scale, (int)precision,
                                       out_indices, out_scores, out_lengths, out_pool_indices, scratch);
  e = dsa::launch_score(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_score_topk_noalloc (score)");
  e = dsa::launch_topk(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_score_topk_noalloc (top-k)");
  return DSA_OK;
}

namespace {

dsa_status_t check_fused_rope(int precision, int D, const float* rope_cos, const float* rope_sin, int rope_dim,
                              int rope_max_pos, int rope_interleaved) {
  if (rope_dim < 0 || rope_dim > D || (rope_dim % 2) != 0)
    return fail(DSA_ERR_UNSUPPORTED, "rope_dim=%d must be even and within [0, D=%d]", rope_dim, D);
  if (rope_dim > 0 && !rope_interleaved && rope_dim % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "rotate-half RoPE needs rope_dim %% 32 == 0 (got %d)", rope_dim);
  if (!dsa::score_can_fuse_rope(precision, rope_dim, rope_interleaved ? 1 : 0))
    return fail(DSA_ERR_UNSUPPORTED,
                "rotate-half RoPE over %d dims with an fp8 precision needs rope_dim %% 64 == 0 here; use "
                "dsa_index_preprocess + dsa_index_score_topk", rope_dim);
  if (rope_dim > 0 && (!rope_cos || !rope_sin || rope_max_pos < 1))
    return fail(DSA_ERR_INVALID_ARGUMENT, "rope tables and rope_max_pos >= 1 required when rope_dim > 0");
  if (rope_dim > 0 && (!aligned(rope_cos, 16) || !aligned(rope_sin, 16)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "rope tables must be 16-byte aligned");
  return DSA_OK;
}

void set_fused_q(dsa::ScoreTopkLaunch& p, const void* q_in, dsa_dtype_t in_dtype, const float* rope_cos,
                 const float* rope_sin, int rope_dim, int rope_max_pos, int rope_interleaved, int rope_fp32,
                 void* q_op_out, uint8_t* q_scale_out) {
  p.q_in = q_in; p.in_bf16 = in_dtype == DSA_DTYPE_BF16;
  p.cos_t = rope_cos; p.sin_t = rope_sin;
  p.rope_dim = rope_dim; p.max_pos = rope_max_pos; p.interleaved = rope_interleaved ? 1 : 0;
  p.rope_fp32 = rope_fp32 ? 1 : 0;
  p.q_op_out = q_op_out; p.q_scale_out = q_scale_out;
}

}  // namespace

dsa_status_t dsa_index_score_fused(
    const void* q_in, dsa_dtype_t in_dtype,
    const void* k_op, const uint8_t* k_scale,
    const void* w, dsa_dtype_t w_dtype,
    int32_t T, int32_t S, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    const float* rope_cos, const float* rope_sin,
    int32_t rope_dim, int32_t rope_max_pos, int32_t rope_interleaved, int32_t rope_fp32,
    float sm_scale, dsa_precision_t precision,
    void* q_op_out, uint8_t* q_scale_out,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_precision((int)precision)) != DSA_OK) return st;
  if (in_dtype != DSA_DTYPE_BF16 && in_dtype != DSA_DTYPE_FP32)
    return fail(DSA_ERR_INVALID_ARGUMENT, "in_dtype %d must be bf16 (0) or fp32 (1)", (int)in_dtype);
  // the operand checks of dsa_index_score, with q_in standing for the (absent) q operands
  if ((st = check_score_args(q_in, static_cast<const uint8_t*>(q_in), k_op, k_scale, w, w_dtype, T, S, H, D,
                             (int)precision, workspace)) != DSA_OK)
    return st;
  if ((st = check_fused_rope((int)precision, D, rope_cos, rope_sin, rope_dim, rope_max_pos, rope_interleaved)) != DSA_OK)
    return st;
  if ((st = check_geometry(T, cu_seqlens, num_seqs, max_seqlen, 1, nullptr, 1, false)) != DSA_OK) return st;
  if (T == 0) return DSA_OK;
  if (q_op_out && !aligned(q_op_out, 16)) return fail(DSA_ERR_INVALID_ARGUMENT, "q_op_out must be 16-byte aligned");
  const size_t need = dsa_index_workspace_size(T, H, D, num_seqs, max_seqlen, 1, 1, precision);
  if (workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  dsa::ScoreTopkLaunch p = make_launch(nullptr, nullptr, k_op, k_scale, w, w_dtype, T, S, H, D, cu_seqlens,
                                       num_seqs, max_seqlen, 1, nullptr, 0, 1, sm_scale, (int)precision, nullptr,
                                       nullptr, nullptr, nullptr, workspace);
  set_fused_q(p, q_in, in_dtype, rope_cos, rope_sin, rope_dim, rope_max_pos, rope_interleaved, rope_fp32,
              q_op_out, q_scale_out);
  hipError_t e = dsa::launch_score(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_score_fused");
  return DSA_OK;
}

size_t dsa_index_forward_workspace_size(int32_t T, int32_t D, int32_t max_seqlen, dsa_precision_t precision) {
  if (T < 0 || max_seqlen < 0 || (D != 64 && D != 128)) return 0;
  const size_t es = precision == DSA_PREC_BF16 ? 2 : 1;
  const size_t nsb = precision == DSA_PREC_BF16 ? 0 : (precision == DSA_PREC_FP8 ? 1 : (size_t)D / 32);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t scores = (size_t)T * (size_t)row_stride(max_seqlen) * sizeof(float);
  return up(scores) + up((size_t)T * D * es) + up((size_t)T * nsb) + 256;
}

dsa_status_t dsa_index_forward(
    const void* q_in, const void* k_in, dsa_dtype_t in_dtype,
    const void* w, dsa_dtype_t w_dtype,
    int32_t T, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    const float* ln_gamma, const float* ln_beta, float ln_eps,
    const float* rope_cos, const float* rope_sin,
    int32_t rope_dim, int32_t rope_max_pos, int32_t rope_interleaved, int32_t rope_fp32,
    int32_t topk, float sm_scale, dsa_precision_t precision,
    int32_t* out_indices, float* out_scores, int32_t* out_lengths,
    void* q_op_out, uint8_t* q_scale_out,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_precision((int)precision)) != DSA_OK) return st;
  if (in_dtype != DSA_DTYPE_BF16 && in_dtype != DSA_DTYPE_FP32)
    return fail(DSA_ERR_INVALID_ARGUMENT, "in_dtype %d must be bf16 (0) or fp32 (1)", (int)in_dtype);
  if (w_dtype != DSA_DTYPE_BF16 && w_dtype != DSA_DTYPE_FP32)
    return fail(DSA_ERR_INVALID_ARGUMENT, "w_dtype %d must be bf16 (0) or fp32 (1)", (int)w_dtype);
  if ((st = check_hd(H, D, true)) != DSA_OK) return st;
  if ((st = check_fused_rope((int)precision, D, rope_cos, rope_sin, rope_dim, rope_max_pos, rope_interleaved)) != DSA_OK)
    return st;
  if ((st = check_geometry(T, cu_seqlens, num_seqs, max_seqlen, 1, nullptr, topk, true)) != DSA_OK) return st;
  if (T == 0) return DSA_OK;
  if (!q_in || !k_in || !w) return fail(DSA_ERR_INVALID_ARGUMENT, "q_in, k_in and w are required");
  if (!aligned(q_in, 16) || !aligned(k_in, 16) || !aligned(w, w_dtype == DSA_DTYPE_FP32 ? 4 : 2) ||
      (q_op_out && !aligned(q_op_out, 16)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "misaligned input (q, k, q_op_out 16 B; weights 4 B)");
  if ((st = check_outputs(out_indices, out_scores, out_lengths, nullptr, workspace)) != DSA_OK) return st;
  const size_t need = dsa_index_forward_workspace_size(T, D, max_seqlen, precision);
  if (workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  // workspace: score rows, then the quantised keys and their scales
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t es = precision == DSA_PREC_BF16 ? 2 : 1;
  uint8_t* k_op = ws + up((size_t)T * (size_t)row_stride(max_seqlen) * sizeof(float));
  uint8_t* k_scale = precision == DSA_PREC_BF16 ? nullptr : k_op + up((size_t)T * D * es);
  // keys: LayerNorm, RoPE, quantisation
  dsa::PreprocessLaunch pp;
  pp.q_in = nullptr; pp.k_in = k_in; pp.in_bf16 = in_dtype == DSA_DTYPE_BF16;
  pp.T = 0; pp.S = T; pp.H = H; pp.D = D;
  pp.cu = cu_seqlens; pp.B = num_seqs;
  pp.gamma = ln_gamma; pp.beta = ln_beta; pp.eps = ln_eps;
  pp.cos_t = rope_cos; pp.sin_t = rope_sin;
  pp.rope_dim = rope_dim; pp.max_pos = rope_max_pos; pp.interleaved = rope_interleaved ? 1 : 0;
  pp.rope_fp32 = rope_fp32 ? 1 : 0; pp.precision = (int)precision;
  pp.q_op = nullptr; pp.q_scale = nullptr; pp.k_op = k_op; pp.k_scale = k_scale;
  pp.q_f32 = nullptr; pp.k_f32 = nullptr;
  hipError_t e = dsa::launch_preprocess(pp, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_forward (keys)");
  // scores with the query preprocessing fused into the scoring kernel, then top-k
  dsa::ScoreTopkLaunch p = make_launch(nullptr, nullptr, k_op, k_scale, w, w_dtype, T, T, H, D, cu_seqlens,
                                       num_seqs, max_seqlen, 1, nullptr, 0, topk, sm_scale, (int)precision,
                                       out_indices, out_scores, out_lengths, nullptr, workspace);
  set_fused_q(p, q_in, in_dtype, rope_cos, rope_sin, rope_dim, rope_max_pos, rope_interleaved, rope_fp32,
              q_op_out, q_scale_out);
  e = dsa::launch_score(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_forward (score)");
  e = dsa::launch_topk(p, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_forward (top-k)");
  return DSA_OK;
}

dsa_status_t dsa_index_selection_softmax(const float* scores, int32_t T, int32_t topk, float* out,
                                         hipStream_t stream) {
  if (T < 0 || topk < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "need T >= 0 and topk >= 1 (T=%d, topk=%d)", T, topk);
  if (T == 0) return DSA_OK;
  if (!scores || !out) return fail(DSA_ERR_INVALID_ARGUMENT, "scores and out must not be NULL");
  if (!aligned(scores, 4) || !aligned(out, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "scores and out must be 4-byte aligned");
  hipError_t e = dsa::launch_selection_softmax(scores, T, topk, out, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_selection_softmax");
  return DSA_OK;
}

dsa_status_t dsa_index_sparse_attention(const void* q, const void* kv, const int32_t* indices,
                                        const int32_t* lengths, int32_t T, int32_t H, int32_t S, int32_t topk,
                                        int32_t dk, int32_t dv, float sm_scale, void* out, float* out_lse,
                                        hipStream_t stream) {
  if (T < 0 || S < 0 || H < 1 || topk < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "need T >= 0, S >= 0, H >= 1 and topk >= 1 (T=%d, S=%d, H=%d, topk=%d)", T,
                S, H, topk);
  if (dk != dsa::kMlaKeyWidth || dv != dsa::kMlaValueWidth)
    return fail(DSA_ERR_UNSUPPORTED, "entry width %d / value width %d: only %d / %d is supported", dk, dv,
                dsa::kMlaKeyWidth, dsa::kMlaValueWidth);
  if (H % 16 != 0) return fail(DSA_ERR_UNSUPPORTED, "H must be a multiple of 16 (H=%d)", H);
  if ((long long)S * dk * 2 > 0x7FFFFFFFll)
    return fail(DSA_ERR_UNSUPPORTED, "the latent tensor must stay below 2 GiB (S=%d)", S);
  if (!std::isfinite(sm_scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  if (T == 0) return DSA_OK;
  if (!q || !indices || !out || (S > 0 && !kv))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q, indices, out (and kv when S > 0) must not be NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(indices, 4) ||
      (lengths && !aligned(lengths, 4)) || (out_lse && !aligned(out_lse, 4)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q, kv, out must be 16-byte aligned; indices, lengths, out_lse 4-byte");
  hipError_t e = dsa::launch_sparse_mla(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), indices,
                                        lengths, T, H, S, topk, sm_scale, static_cast<uint16_t*>(out), out_lse, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_index_sparse_attention");
  return DSA_OK;
}

dsa_status_t dsa_bench_mfma(dsa_precision_t precision, int32_t blocks, int32_t iters, float* out,
                            hipStream_t stream) {
  dsa_status_t st;
  if ((st = check_precision((int)precision)) != DSA_OK) return st;
  if (blocks < 1 || blocks > 65536 || iters < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "need 1 <= blocks <= 65536 and iters >= 1 (blocks=%d, iters=%d)", blocks, iters);
  if (!out || !aligned(out, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "out must be a 4-byte aligned device pointer");
  hipError_t e = dsa::launch_mfma_peak(precision == DSA_PREC_BF16 ? 0 : 1, blocks, iters, out, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_bench_mfma");
  return DSA_OK;
}

double dsa_bench_mfma_flops(dsa_precision_t precision, int32_t blocks, int32_t iters) {
  if (!valid_precision((int)precision) || blocks < 1 || iters < 1) return 0.0;
  return dsa::mfma_peak_flops(precision == DSA_PREC_BF16 ? 0 : 1, blocks, iters);
}

dsa_status_t dsa_bench_stream(const void* src, void* dst, size_t bytes, int32_t copy, hipStream_t stream) {
  if (bytes == 0 || bytes % 16 != 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "bytes=%zu must be a positive multiple of 16", bytes);
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16))
    return fail(DSA_ERR_INVALID_ARGUMENT, "src and dst must be 16-byte aligned device pointers");
  if (copy != 0 && copy != 1) return fail(DSA_ERR_INVALID_ARGUMENT, "copy=%d must be 0 or 1", copy);
  hipError_t e = dsa::launch_stream(src, dst, bytes, copy, stream);
  if (e != hipSuccess) return device_fail(e, "dsa_bench_stream");
  return DSA_OK;
}

}  // extern "C"
