/*
 * dsa_index.h - C ABI of the DSA lightning-indexer hot path on AMD Instinct MI355X (gfx950).
 *
 * The indexer of DeepSeek Sparse Attention scores, for every query token t and
 * every causal key c of t's document,
 *
 *     I[t,c] = sm_scale * sum_h w[t,h] * ReLU(q[t,h,:] . k[c,:])
 *
 * and keeps the `topk` best keys per query. Sources (Megatron-LM pull requests):
 *   - PR 8403 ("What does this PR do?", "Implementation", codex review findings 1-3):
 *     the single scoring call taking q, k, per-head weights w, ratio and sm_scale; ReLU
 *     scoring; key LayerNorm then RoPE kept in FP32 (`dsa_indexer_rope_fp32`); BF16
 *     or FP8 (E4M3 with UE8M0 per-vector scales) scoring precision; an unknown
 *     precision is a ValueError; the (indices, lengths, scores) outputs.
 *   - PR 5992 ("[dev] [DeepSeek-V4] Add compact BF16 and MXFP8 DSA indexer support",
 *     "Key changes" and review summaries): MXFP8 scoring, caller-owned workspaces that
 *     are safe under graph capture, live cu_seqlens read on every call, deterministic
 *     top-k tie breaking.
 *   - PR 7522 ("Changes"): KPool pooled keys (BF16 per-token gate, FP32 per-slot bias),
 *     selection over pools expanded back to token indices, the incomplete causal tail
 *     pool, pooling restarting at document boundaries, the NoPE indexer.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; all arrays are dense and
 *     row-major with the last dimension contiguous. Scalars are host values.
 *   - Queries and keys are packed (THD): documents b = 0..num_seqs-1 occupy rows
 *     cu_seqlens[b] .. cu_seqlens[b+1]-1. cu_seqlens is int32 [num_seqs+1] in device
 *     memory with cu_seqlens[0] = 0, non-decreasing, last entry = T. It is read on the
 *     device on every call, so it may change between graph capture and replay.
 *     Positions (for RoPE) restart at 0 in every document. Query t's causal keys are
 *     the keys of its own document at positions 0..u (u = t's position), that is
 *     global key rows cu_seqlens[b] .. t.
 *   - The library never allocates, frees or synchronises the host inside a call. All
 *     work is enqueued on `stream` (asynchronous); results are ready when the stream is.
 *     Calls may be captured into a HIP graph on one stream (tested: a captured step
 *     replayed with new document boundaries matches eager calls). Capture that spreads the
 *     calls of one step over several streams joined by events is not covered by tests.
 *   - Device-side data is trusted but never read out of bounds: a malformed cu_seqlens
 *     is clamped to [0, T] and documents longer than `max_seqlen` are truncated to it
 *     (their later rows see at most max_seqlen candidates); results are then unspecified.
 *   - Every entry point returns a status. Host-side validation runs before anything is
 *     enqueued; on a non-OK status nothing was enqueued unless the status is
 *     DSA_ERR_DEVICE. dsa_last_error() describes the last non-OK status of the calling
 *     thread.
 *   - Results are deterministic: identical inputs give byte-identical outputs on every
 *     call and stream (no floating-point atomics, fixed reduction orders).
 */
#ifndef DSA_INDEX_H
#define DSA_INDEX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,   /* NULL/misaligned pointer, bad size, bad enum value */
  DSA_ERR_UNSUPPORTED = 2,        /* valid but outside the supported matrix (precision, H, D, rope_dim, sizes) */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_DEVICE = 4              /* a HIP launch failed; dsa_last_error() carries the HIP message */
} dsa_status_t;

typedef enum {
  DSA_PREC_BF16 = 0,   /* bf16 operands, round to nearest even from the fp32 carrier */
  DSA_PREC_FP8 = 1,    /* OCP E4M3FN payload + one UE8M0 scale per D-vector */
  DSA_PREC_MXFP8 = 2   /* OCP E4M3FN payload + one UE8M0 scale per 32 elements */
} dsa_precision_t;

typedef enum { DSA_DTYPE_BF16 = 0, DSA_DTYPE_FP32 = 1 } dsa_dtype_t;

/*
 * Scoring operand formats (the `q_op/k_op` and `*_scale` arrays below):
 *   bf16 : uint16 bf16 bit patterns [.., D]; no scale array (pass NULL).
 *   fp8  : uint8 E4M3FN codes [.., D]; scale = uint8 UE8M0 code per vector, value
 *          2^(code-127); the exponent e is the smallest integer with amax <= 448 * 2^e
 *          (e = 0 for an all-zero vector, clamped to [-127,127]), payload =
 *          round-to-nearest-even E4M3FN of x * 2^-e (never saturates).
 *   mxfp8: as fp8 but one scale per 32 consecutive elements: scale array [.., D/32].
 */

/*
 * dsa_index_preprocess - key LayerNorm then RoPE in fp32, fused with quantisation to the
 * scoring operands (PR 8403, "What does this PR do?", "Motivation", "Implementation";
 * PR 5992, "Key changes" for MXFP8; PR 7522, "Changes" for NoPE).
 *
 *   q_in      [T,H,D] in_dtype, or NULL to skip queries (then q_op/q_scale/q_f32_out unused)
 *   k_in      [S,D]   in_dtype, or NULL to skip keys. T == S when both are given; with one
 *             of them NULL the other's row count must match cu_seqlens[num_seqs].
 *   ln_gamma, ln_beta  fp32 [D] key LayerNorm affine (the effective gamma); gamma NULL =>
 *             no LayerNorm; beta NULL => zero. LayerNorm: mean and biased variance over D
 *             with a pinned pairwise halving sum, rstd = 1/sqrt(var + ln_eps), each fp32
 *             operation rounded separately. Queries get no LayerNorm.
 *   rope_cos, rope_sin fp32 [rope_max_pos, rope_dim/2]: angle table, row = position inside
 *             the document, 16-byte aligned. rope_dim = 0 => NoPE (tables unused, may be NULL).
 *             RoPE rotates the last rope_dim dims: rotate-half pairs (j, j+rope_dim/2) when
 *             rope_interleaved = 0 (rope_dim % 32 == 0 required), adjacent pairs (2j, 2j+1)
 *             when 1 (rope_dim even). y1 = x1*c - x2*s, y2 = x2*c + x1*s, no fused
 *             multiply-add. Positions >= rope_max_pos read the last table row.
 *   rope_fp32 0 => default path: the input of RoPE and its output are rounded to bf16
 *             (the "materialised BF16" round-trip); 1 => the fp32 carrier is kept up to
 *             quantisation.
 *   precision output operand format (see above).
 *   q_op [T,H,D], q_scale ([T,H] fp8, [T,H,D/32] mxfp8, NULL for bf16),
 *   k_op [S,D],   k_scale ([S] fp8, [S,D/32] mxfp8, NULL for bf16).
 *   q_f32_out [T,H,D], k_f32_out [S,D]: optional fp32 carriers just before quantisation.
 * Supported: H in {16,32,64}, D in {64,128}. Pointers: q_in/k_in/q_op/k_op and the fp32
 * outputs 16-byte aligned.
 */
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
    hipStream_t stream);

/*
 * dsa_index_kpool - KPool key compression (PR 7522, "Changes").
 *
 * Within each document, pool p holds tokens cu_seqlens[b] + p*kpool + j, j < kpool; only
 * complete pools exist and pooling restarts at every document. With
 * z_j = gate[token_j] + slot_bias[j] (fp32), m = max z, e_j = pexp(z_j - m),
 * sigma = e_0 + e_1 + ... (left to right), a_j = e_j / sigma, the pooled key is
 * a_0*k_0 + a_1*k_1 + ... accumulated left to right in fp32 (no fused multiply-add),
 * then quantised to `precision`. pexp is a pinned exponential: 0 below -104, otherwise
 * n = rint(z*log2e), r = fma(-n, ln2_lo, fma(-n, ln2_hi, z)) with ln2_hi = 0x3F317200,
 * ln2_lo = 0x35BFBE8E, a degree-7 Taylor polynomial in r by Horner's rule with fused
 * multiply-adds, scaled by 2^n.
 *
 *   k          [S,D] keys (raw or preprocessed carriers), k_dtype bf16 or fp32
 *   gate_bf16  [S]   bf16 bit patterns, one compression logit per token
 *   slot_bias  [kpool] fp32
 *   kpool      2..64 (1 is accepted and copies the keys)
 *   pooled_op  [floor(S/kpool), D] operand rows, pooled_scale as for keys (NULL for bf16);
 *              only the first cu_pools[num_seqs] rows are written.
 *   cu_pools   int32 [num_seqs+1] output: cu_pools[b] = complete pools in documents < b.
 */
dsa_status_t dsa_index_kpool(
    const void* k, dsa_dtype_t k_dtype, int32_t S, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs,
    const uint16_t* gate_bf16, const float* slot_bias, int32_t kpool,
    dsa_precision_t precision,
    void* pooled_op, uint8_t* pooled_scale, int32_t* cu_pools,
    hipStream_t stream);

/*
 * dsa_index_workspace_size - bytes of caller-owned workspace dsa_index_score_topk needs.
 * It holds the fp32 scores of every row's candidates at a fixed row stride (a multiple of
 * 64 not below the largest candidate count, max_seqlen or max_seqlen/kpool) plus 256
 * bytes. Pure host computation; returns 0 for invalid arguments.
 */
size_t dsa_index_workspace_size(int32_t T, int32_t H, int32_t D, int32_t num_seqs,
                                int32_t max_seqlen, int32_t topk, int32_t kpool,
                                dsa_precision_t precision);

/*
 * dsa_index_score_topk - scores of every causal candidate, then per-row top-k
 * (PR 8403 codex review findings 1-3; PR 5992 "Key changes"; PR 7522 "Changes").
 * Equivalent to dsa_index_score followed by dsa_index_topk on the same stream.
 *
 *   q_op, q_scale  [T,H,D] scoring operands (+ scales) as produced by dsa_index_preprocess
 *   k_op, k_scale  [S,D] token keys (kpool == 1), or [S,D] pooled keys (kpool > 1, S = rows
 *                  of pooled_op)
 *   w              [T,H] per-head weights, fp32 or bf16 (w_dtype)
 *   cu_seqlens     as above; max_seqlen is a static host upper bound of the document
 *                  lengths (sizes the grid and the workspace)
 *   kpool, cu_pools, kpool_tail: kpool > 1 scores pools: query t at position u sees the
 *                  floor((u+1)/kpool) complete pools of its document (pooled row
 *                  cu_pools[b] + p); kpool_tail != 0 appends its incomplete causal pool.
 *   topk >= 1, sm_scale multiplies every score.
 *   Outputs (all written in full, padding -1 / -inf):
 *     out_scores [T,topk] fp32 - selected scores (pool scores when kpool > 1), ordered by
 *                score descending then index ascending; ties go to the lower index.
 *     out_indices: kpool == 1: [T,topk] int32 global key rows (cu_seqlens[b] + c).
 *                  kpool  > 1: [T, topk*kpool + kpool - 1] int32 token indices: every
 *                  selected pool's kpool tokens in ascending order, pools in selection
 *                  order, then the tail tokens (pool start .. t).
 *     out_lengths [T] int32: valid entries of out_indices (tokens when kpool > 1).
 *     out_pool_indices [T,topk] int32 global pooled rows (kpool > 1), may be NULL.
 *   workspace, workspace_bytes: device buffer of at least dsa_index_workspace_size(...)
 *   bytes, 256-byte aligned. Its contents on entry do not matter.
 * Supported: H in {16,32,64}, D in {64,128}; max_seqlen/kpool <= 32768 candidates per row.
 */
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
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_index_score - the scoring half of dsa_index_score_topk: writes the fp32 score of every
 * causal candidate of every query row into `workspace` and nothing else. Row t occupies
 * floats [t*stride, t*stride + cand(t)) with stride = the smallest multiple of 64 that is
 * >= max(1, max_seqlen) (kpool == 1) or max(1, max_seqlen/kpool) (kpool > 1), and
 * cand(t) = u+1 or floor((u+1)/kpool) for t at position u of its document; entry c is the
 * score of document-local candidate c. Other workspace bytes are left untouched. Arguments
 * and errors are as for dsa_index_score_topk, except that topk is not used and the bound on
 * candidates per row is 4194304 (2^22) instead of 32768 (DSA_ERR_UNSUPPORTED above it).
 */
dsa_status_t dsa_index_score(
    const void* q_op, const uint8_t* q_scale,
    const void* k_op, const uint8_t* k_scale,
    const void* w, dsa_dtype_t w_dtype,
    int32_t T, int32_t S, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    int32_t kpool, const int32_t* cu_pools,
    float sm_scale, dsa_precision_t precision,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_index_topk - the selection half of dsa_index_score_topk: reads the score rows that
 * dsa_index_score wrote into `workspace` (same T, cu_seqlens, max_seqlen and kpool) and
 * writes out_indices / out_scores / out_lengths / out_pool_indices exactly as
 * dsa_index_score_topk does.
 */
dsa_status_t dsa_index_topk(
    const void* workspace, size_t workspace_bytes,
    int32_t T, const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    int32_t kpool, const int32_t* cu_pools, int32_t kpool_tail, int32_t topk,
    int32_t* out_indices, float* out_scores, int32_t* out_lengths, int32_t* out_pool_indices,
    hipStream_t stream);

/*
 * dsa_index_score_topk_noalloc - dsa_index_score_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, outputs and errors without `workspace` /
 * `workspace_bytes`. The score rows go to a fixed scratch array the library holds on every
 * GPU it runs on, DSA_NOALLOC_SCRATCH_BYTES bytes, from the time its code is loaded on the
 * device until the process ends. The call allocates and frees nothing.
 *   - Sizes: the call needs dsa_index_workspace_size(T, H, D, num_seqs, max_seqlen, topk,
 *     kpool, precision) bytes of scratch (T rows times the row stride times 4, plus 256):
 *     e.g. 8192 rows of 4096 candidates. A larger problem returns DSA_ERR_UNSUPPORTED
 *     before anything is enqueued; use dsa_index_score_topk with a workspace instead.
 *   - Sharing: every call on one GPU uses that GPU's one array, which keeps the last call's
 *     contents (nothing in it needs to start at zero). Calls that overlap on one GPU (on
 *     different streams, or from several host threads without ordering) race on it and
 *     give undefined results: order them on one stream.
 *   - The array's device address is looked up once per device, on the first call made
 *     with that device current.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)134221824) /* 128 MiB + 4 KiB */
dsa_status_t dsa_index_score_topk_noalloc(
    const void* q_op, const uint8_t* q_scale,
    const void* k_op, const uint8_t* k_scale,
    const void* w, dsa_dtype_t w_dtype,
    int32_t T, int32_t S, int32_t H, int32_t D,
    const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
    int32_t kpool, const int32_t* cu_pools, int32_t kpool_tail,
    int32_t topk, float sm_scale, dsa_precision_t precision,
    int32_t* out_indices, float* out_scores, int32_t* out_lengths,
    int32_t* out_pool_indices, hipStream_t stream);

/* Message of the last non-OK status returned on the calling thread ("" if none). */
const char* dsa_last_error(void);

/*
 * dsa_index_score_fused - dsa_index_score with the query preprocessing fused into the
 * scoring kernel: it takes the raw queries q_in [T,H,D] (bf16 or fp32, in_dtype, 16-byte
 * aligned) and the RoPE arguments of dsa_index_preprocess instead of q_op / q_scale, and
 * builds each query's operands (RoPE, carrier rounding, quantisation) in registers, byte-
 * identical to those dsa_index_preprocess writes. The keys (k_op, k_scale) come
 * preprocessed as for dsa_index_score (kpool 1). Writes the same workspace rows as
 * dsa_index_score. q_op_out / q_scale_out: optional copies of the query operands built
 * (as for dsa_index_forward; NULL: not written). Errors as for dsa_index_score, plus the
 * RoPE restriction of dsa_index_forward.
 */
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
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_index_forward - the whole indexer hot path in one call, for kpool == 1: the keys are
 * preprocessed (LayerNorm, RoPE, quantisation, as dsa_index_preprocess) into the workspace,
 * the scoring kernel preprocesses each query vector itself (RoPE, quantisation) straight
 * into its MFMA operands, so quantised queries never go through memory, and the top-k
 * follows (the steps the pages describe for the indexer forward: preprocessing, scoring,
 * top-k; Megatron-LM PR 8403 "What does this PR do?", PR 5992 "Key changes"). Results are
 * those of dsa_index_preprocess + dsa_index_score_topk with the same arguments (operands
 * byte-identical, hence identical scores and selections).
 *
 *   q_in [T,H,D], k_in [T,D]  bf16 or fp32 (in_dtype), 16-byte aligned; queries and keys
 *             share cu_seqlens (S = T).
 *   w, cu_seqlens, num_seqs, max_seqlen, topk, sm_scale, precision: as for
 *             dsa_index_score_topk; ln_*, rope_*: as for dsa_index_preprocess.
 *   out_indices [T,topk], out_scores [T,topk], out_lengths [T]: as for dsa_index_score_topk.
 *   q_op_out, q_scale_out: optional (NULL: not written). When given, the quantised query
 *             operands the scoring kernel built ([T,H,D] bf16 or E4M3 bytes, 16-byte
 *             aligned; scales [T,H] or [T,H,D/32]) for rows of tokens at positions
 *             < max_seqlen; other rows are not written.
 *   workspace  >= dsa_index_forward_workspace_size(T, D, max_seqlen, precision) bytes,
 *             256-byte aligned (score rows, then quantised keys and scales).
 * Errors as for dsa_index_score_topk; DSA_ERR_UNSUPPORTED also for rotate-half RoPE with
 * an fp8 precision when rope_dim % 64 != 0 (the two halves of a rotated pair then sit in
 * different lanes of the MFMA operand layout; the two-call path supports it).
 */
size_t dsa_index_forward_workspace_size(int32_t T, int32_t D, int32_t max_seqlen,
                                        dsa_precision_t precision);

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
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_index_selection_softmax - softmax over each row's selected scores: the optional third
 * output of the indexer's top-k, the predicted distribution that the indexer loss reuses
 * (Megatron-LM PR 5992 reviews: "What was verified", the top-k call's return arity with
 * return_softmax; "Areas checked and found clean", the loss reusing the compact softmax).
 * For row t: out[t,j] = exp(s_j - m) / sum_i exp(s_i - m) with s = scores[t, 0..topk) and m
 * the row's maximum; -inf entries (the padding of the top-k outputs) get 0, and a row with
 * no finite entry is all zeros. With KPool it runs over the selected pools' scores.
 *   scores   [T, topk] fp32, DEVICE, 4-byte aligned: out_scores of a top-k call.
 *   out      [T, topk] fp32, DEVICE, 4-byte aligned, caller-owned; may be `scores` itself.
 * Arithmetic: fp32, expf, one division per entry; per-row sums in a fixed order (results do
 * not depend on scheduling). Errors: DSA_ERR_INVALID_ARGUMENT for T < 0, topk < 1, NULL or
 * misaligned pointers (T > 0); DSA_ERR_DEVICE if the launch fails.
 */
dsa_status_t dsa_index_selection_softmax(const float* scores, int32_t T, int32_t topk, float* out,
                                         hipStream_t stream);

/*
 * dsa_index_sparse_attention - absorbed-MLA attention of every query head over the latent
 * entries its row selected: the consumer of the indexer's top-k (Megatron-LM PR 8403,
 * "Fused Path": FlashMLA sparse attention after the indexer, compressed KV width 576 =
 * kv_lora_rank 512 + 64; codex review finding 1: value width 512, invalid slots and
 * supplied lengths). One latent entry per token serves every head; the key is the whole
 * entry, the value its first dv elements. For query t the selected entries are the slots
 * j < lengths[t] (all topk slots when lengths is NULL) whose index lies in [0, S); -1 marks an
 * empty slot. With s_j = sm_scale * q[t,h,:] . kv[j,:]:
 *     out[t,h,:]   = sum_j exp(s_j - m) kv[j, 0..dv) / sum_j exp(s_j - m),  m = max_j s_j
 *     out_lse[t,h] = m + log(sum_j exp(s_j - m))   (natural log)
 * A row with nothing selected gives zeros and out_lse -inf. A slot listed twice counts twice.
 *   q        [T, H, dk] bf16, DEVICE, 16-byte aligned.
 *   kv       [S, dk] bf16, DEVICE, 16-byte aligned (may be NULL when S == 0).
 *   indices  [T, topk] int32, DEVICE: token indices into kv (the out_indices of a top-k call,
 *            which hold document offsets already; KPool rows hold expanded token indices).
 *   lengths  [T] int32, DEVICE, or NULL: slots used per row (out_lengths of a top-k call),
 *            clamped to [0, topk].
 *   dk, dv   576 and 512 (DSA_ERR_UNSUPPORTED otherwise); H a multiple of 16.
 *   out      [T, H, dv] bf16, DEVICE, 16-byte aligned, caller-owned.
 *   out_lse  [T, H] fp32, DEVICE, or NULL (not written).
 * Arithmetic: q.k products in fp32 on MFMA (bf16 operands); softmax in fp32, base 2, with the
 * weights rounded to bf16 (nearest even) for the value product and summed in fp32 for the
 * normaliser; output rounded to bf16 (nearest even). Results do not depend on scheduling.
 * Errors: DSA_ERR_INVALID_ARGUMENT for T < 0, S < 0, H < 1, topk < 1, a non-finite sm_scale,
 * NULL or misaligned pointers (T > 0); DSA_ERR_UNSUPPORTED for other widths, H % 16 != 0 or
 * S * dk * 2 >= 2^31; DSA_ERR_DEVICE if the launch fails. Index values are not an error:
 * anything outside [0, S) is an empty slot.
 */
dsa_status_t dsa_index_sparse_attention(const void* q, const void* kv, const int32_t* indices,
                                        const int32_t* lengths, int32_t T, int32_t H, int32_t S, int32_t topk,
                                        int32_t dk, int32_t dv, float sm_scale, void* out, float* out_lse,
                                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEX_H */
