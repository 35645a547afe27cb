// Sparse absorbed-MLA attention over the indexer's selection (gfx950).
//
// The consumer of the top-k: every query head attends only to the latent entries its row
// selected (Megatron-LM PR 8403, "Fused Path": FlashMLA sparse attention after the indexer,
// compressed KV width 576 = kv_lora_rank 512 + 64; codex review finding 1: value width 512,
// invalid slots and supplied lengths). One 576-wide bf16 entry per token serves every head:
// the key is the whole entry, the value its first 512 elements. For query t, head h and the
// selected entries j (slots j < length[t] holding a valid token index):
//     out[t,h,:] = sum_j softmax_j(sm_scale * q[t,h,:] . kv[j,:]) kv[j,:512]
//     lse[t,h]   = log sum_j exp(sm_scale * q[t,h,:] . kv[j,:])
//
// Work decomposition. A workgroup of 4 waves owns one query token and 64 of its heads, one
// wave per 16 heads; the wave's q operands (16 heads x 576) stay in registers. The row's
// slots are swept in tiles of 32, each gathered key-major into one of two LDS buffers by
// direct buffer-to-LDS loads: tile j+1 streams in while tile j is multiplied out, so the
// gather's memory latency hides behind a tile of work (the entries' indices are read a tile
// earlier still). An entry's value part (its first 512 elements, 1024 bytes: one load of 64
// lanes x 16 bytes) lands in a row of its own, rows 32 bytes apart modulo 256; the other 64
// elements of 8 keys form one load, their 16-byte chunks XOR-swizzled by the key. The scores
// (contraction over the 576 elements) are formed transposed, S^T = K q^T, with the keys as
// MFMA rows read by 16-byte loads and the wave's 16 heads as columns, so that a lane ends
// with one head and 8 of the tile's keys. Those 8 weights are, as they stand, the lane's
// operand of the weighted sum, also formed transposed (O^T = V^T P^T), whose value operands
// come from transposing loads (ds_read_b64_tr_b16: within each group of 16 lanes, lane 4a + b
// gets element b of the 8-byte pieces addressed by lanes a, a + 4, a + 8 and a + 12, so lanes
// addressing 4 keys x 4 column pieces receive 4 keys of one column each). The weighted sum is
// shared by waves 2p and 2p + 1: each hands its weights (and its heads' rescale factor) to the
// other through LDS, and each then multiplies its half of the 512 value columns by the weights
// of the pair's 32 heads, so that every value operand it loads serves two MFMAs (one read of
// the values per pair instead of per wave; the key operands of the scores, by contrast, are
// read by every wave for its own heads). Entries are read through a buffer descriptor over
// the latent tensor: an empty slot or an index outside [0, S) reads zeros without touching
// memory and its score is masked.
//
// Softmax: online, in base 2 (scores pre-multiplied by sm_scale * log2 e). A head's running
// maximum (kept by each of its 4 lanes) is raised only when a score exceeds it by more than 8
// (then the 128 accumulator registers are rescaled); otherwise weights up to 2^8 accumulate
// against the older maximum, which is exact in real arithmetic and keeps the rescale, and
// every cross-lane reduction, off the common path. Weights enter the value product as bf16
// (nearest even); the normaliser sums them in fp32. Workgroups are numbered so that groups of
// kTokGroup consecutive tokens, whose selections overlap, go to the XCDs in turn (block b runs
// on XCD b % 8): the workgroups in flight on an XCD share entries through its L2, and every XCD
// gets tokens from all positions of the documents (a causal row's slot count grows with its
// position, so contiguous eighths of the tokens would give the XCDs unequal work).
//
// MFMA v_mfma_f32_16x16x32_bf16 (lane l): A holds row l%16, 8 consecutive k from 8(l/16);
// B holds column l%16, the same k; the 16x16 fp32 result gives lane l column l%16, rows
// 4(l/16) .. 4(l/16)+3. Below r16 = l % 16 and g4 = l / 16.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

constexpr int kDK = kMlaKeyWidth, kDV = kMlaValueWidth;
constexpr int kRowB = kDK * 2;                 // bytes per latent entry
constexpr int kVB = kDV * 2;                   // its value part
constexpr int kRB = kRowB - kVB;               // the rest (the 64 positional elements)
constexpr int kNK = 32;                        // slots per tile
constexpr int kTokGroup = 64;                  // consecutive tokens per XCD turn
constexpr int kVPitch = kVB + 32;              // value-part LDS row (32-byte skew between keys)
constexpr int kLdsV = kNK * kVPitch;
constexpr int kLdsTile = kLdsV + kNK * kRB;    // one tile buffer: value parts, then the rest
constexpr int kOPitch = kDV + 16;              // output staging row (one head, half the value columns)
constexpr int kLdsOut = 4 * 32 * kOPitch;      // the output staging after the sweep
constexpr int kLdsMain = 2 * kLdsTile > kLdsOut ? 2 * kLdsTile : kLdsOut;
constexpr int kXch = 64 * 16 + 64 * 4 + 64 * 4;   // per wave: weights (B operand), rescale factor, 1 / sum
constexpr int kLdsBytes = kLdsMain + 4 * kXch;
constexpr int kSteps = kDK / 32;               // MFMA k-steps of the score product
constexpr int kVSteps = kDV / 32;              // ... of them within the value part
constexpr int kVBlocks = kDV / 32;             // 16-column blocks of a wave's half of the value product
static_assert(kDK % 32 == 0 && kDV % 128 == 0 && kDV < kDK, "entry layout");
static_assert(kVB == 64 * 16 && kRB == 8 * 16 && kNK == 32, "one direct load per value part; one per 8 keys' rest");
static_assert(kLdsOut <= kLdsMain && 2 * kLdsBytes <= 160 * 1024, "two workgroups per CU; output staging reuses the tiles");

// LDS banks (measured on the device with one access pattern per kernel and the bank-conflict
// counter). A ds_read_b128 serves a wave in 4 cycles of 16 lanes, each cycle the 8-lane blocks
// b and b ^ 3 (lanes 0-7 with 24-31, 8-15 with 16-23, 32-39 with 56-63, 40-47 with 48-55;
// every other pairing of blocks was seen not to collide). A b64 access (the transposing read
// included) serves 32 lanes a cycle. 64 banks of 4 bytes.
// - Key operands (b128), lane (r16, g4) reading element chunk 4 ks + g4 of key r16: with
//   value rows 1056 bytes apart a cycle's 16 lanes take the 16-byte slots 2 r + c (r = 0..7)
//   and 2 r + c + 1 (the block of the next g4), all distinct modulo 256 bytes.
// - The rest of the entry (chunk c of 8 at c ^ rsw(r), rows 128 bytes apart): distinct too.
// - Value operands (transposing b64): the 32 lanes of groups g4 = 0, 1 (or 2, 3) read 32-byte
//   pieces of 8 consecutive keys, 32 bytes apart modulo 256: distinct.
// - Weights handed within a pair (b128, 16 bytes per lane in lane order): distinct.
// - Output staging (b64 writes, rows 528 bytes apart): lane (r16, g4) writes dwords
//   4 r16 + 8 c + 2 g4 + {0, 1} modulo 64: distinct over 32 lanes. Its reads (b128, lanes
//   0-31 one row, 32-63 the next, 16 bytes apart within a row): the paired blocks fall on
//   distinct banks.
__device__ __forceinline__ int rsw(int r) { return (r >> 1) & 7; }

// 16 bytes per lane from buffer offset voffset to LDS at lds + 16 * lane (lds wave-uniform).
// Written as assembly so that the compiler does not see an LDS store in flight: it would
// otherwise wait for these loads before every LDS read it cannot tell apart from them (the
// transposing loads among them), which would serialise the gather with the tile before it.
// The kernel waits for them itself (vmcnt(0) before the barrier that publishes a tile); the
// compiler's own vmcnt waits only grow stricter from loads it does not count, since loads
// complete in issue order. M0 (the LDS address of the load) is saved and restored; one wait
// state separates its write from the load that reads it.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, const uint8_t* lds, uint32_t voffset) {
  const uint32_t la = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(r), "s"(la)
      : "memory");
}

struct AttnArgs {
  const uint16_t* q; const uint16_t* kv; const int32_t* indices; const int32_t* lengths;
  int T, H, S, topk;
  float scale_log2;      // sm_scale * log2(e)
  int tper;              // tokens per XCD (whole groups)
  uint16_t* out; float* lse;
};

// bf16 bits of x, nearest even (one v_cvt_pk_bf16_f32 on gfx950; the values here are finite).
__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__global__ __launch_bounds__(256, 2) void sparse_mla_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int nhb = (a.H + 63) / 64;
  const int xcd = blockIdx.x & 7, seq = blockIdx.x >> 3;
  const int loc = seq / nhb;                   // the XCD's loc-th token
  const int t = ((loc / kTokGroup) * 8 + xcd) * kTokGroup + loc % kTokGroup;
  if (t >= a.T) return;                        // whole workgroup
  const int h0 = (seq % nhb) * 64 + 16 * wv;   // this wave's heads (scores, softmax)
  const int e = wv & 1;                        // its half of the value columns
  const int hp = h0 - 16 * e;                  // the pair's 32 heads (value product)
  const bool active = h0 < a.H;                // wave-uniform
  const bool pair_active = hp < a.H;           // a pair past the heads only gathers
  const int n = a.lengths ? clampi(__ldg(a.lengths + t), 0, a.topk) : a.topk;
  const int32_t* irow = a.indices + (long long)t * a.topk;
  const uint32_t kvend = (uint32_t)a.S * kRowB; // the descriptor's end; offsets from there read zeros
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(a.kv, (int)kvend);

  const int r16 = lane & 15, g4 = lane >> 4;
  // q operands: head h0 + r16, elements 32*ks + 8*g4 .. +7
  bf16x8 qa[kSteps];
  if (active) {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((long long)t * a.H + h0 + r16) * kDK + 8 * g4);
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const uint4 v = qp[4 * ks];
      qa[ks] = *reinterpret_cast<const bf16x8*>(&v);
    }
  }
  // O^T: heads h0 + r16 (b = 0) and h0 ^ 16 + r16 (b = 1, the other wave's), value columns
  // 256 e + 16 c + 4 g4 + i
  f32x4 o[kVBlocks][2];
#pragma unroll
  for (int c = 0; c < kVBlocks; ++c) o[c][0] = o[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;             // head h0 + r16: running maximum, this lane's weight sum
  uint8_t* const xme = smem + kLdsMain + wv * kXch;          // what this wave hands to the other
  const uint8_t* const xot = smem + kLdsMain + (wv ^ 1) * kXch;

  // Gather (nothing passes through registers). Lanes l and 32 + l of every wave hold offm, the
  // byte offset of slot j0 + l's entry in the latent tensor, or the descriptor's end for an
  // empty slot or an index outside [0, S) (a byte offset below 2^32 even past the end). Wave
  // wv loads the value parts of keys 8 wv .. 8 wv + 7 (lane l: chunk l) and the rest of
  // those 8 keys (lane l: key 8 wv + l / 8, LDS chunk l % 8).
  const int rkey = 8 * wv + (lane >> 3);
  const uint32_t rchunk = kVB + 16 * ((lane & 7) ^ rsw(rkey));
  auto slot_ix = [&](int j0) {                // every lane loads (clamped address) ...
    return __ldg(irow + min(j0 + (lane & 31), a.topk - 1));
  };
  auto slot_off = [&](int ix, int j0) -> uint32_t {   // ... then masks
    return (j0 + (lane & 31) < n && ix >= 0 && ix < a.S) ? (uint32_t)ix * kRowB : kvend;
  };
  auto gather = [&](uint32_t offm, int buf) {
    uint8_t* dst = smem + buf * kLdsTile;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int key = 8 * wv + k;
      lds_dma16(rkv, dst + key * kVPitch, (uint32_t)__builtin_amdgcn_readlane((int)offm, key) + 16 * lane);
    }
    const uint32_t ro = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * rkey, (int)offm);
    lds_dma16(rkv, dst + kLdsV + wv * 8 * kRB, ro + rchunk);
  };
  // prologue: tile 0 in flight, the indices of tile 1 requested (first used after the wait
  // for tile 0, so that no wait for them holds up the gather)
  uint32_t vm_next = 0;
  int ixn = 0;
  if (n > 0) {
    const uint32_t off0 = slot_off(slot_ix(0), 0);
    gather(off0, 0);
    vm_next = (uint32_t)__ballot(lane < 32 && off0 != kvend);
    ixn = slot_ix(kNK);
  }

  for (int j0 = 0, buf = 0; j0 < n; j0 += kNK, buf ^= 1) {
    const uint32_t vmask = vm_next;            // valid slots of this tile (bit j - j0)
    __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): this wave's loads of the tile have landed
    __syncthreads();                           // ... every wave's; the other buffer is no longer read
    if (j0 + kNK < n) {                        // the next tile streams in during this one
      const uint32_t offm = slot_off(ixn, j0 + kNK);
      gather(offm, buf ^ 1);
      vm_next = (uint32_t)__ballot(lane < 32 && offm != kvend);
      ixn = slot_ix(j0 + 2 * kNK);             // past the row: a clamped read, unused
    }
    const uint8_t* kvt = smem + buf * kLdsTile;   // value parts [32][kVPitch]
    const uint8_t* krt = kvt + kLdsV;             // the rest [32][128], chunks swizzled
    bf16x8 pb = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};   // this wave's weights (zero for heads past H)
    float alpha = 1.f;                            // ... and their heads' rescale factor
    if (active) {
      // ---- scores, transposed: A = keys (row r16 of each 16-key half: elements 32 ks + 8 g4 ..
      //      +7), B = q (column = head r16). Lane (r16, g4) gets head r16 with keys 4 g4 + i
      //      (s0) and 16 + 4 g4 + i (s1), i = 0..3.
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
      auto key_op = [&](int ks, int half) -> u32x4 {
        // (rsw(16 + r16) = rsw(r16))
        const uint8_t* p = ks < kVSteps ? kvt + (16 * half + r16) * kVPitch + 64 * ks + 16 * g4
                                        : krt + (16 * half + r16) * kRB + 16 * ((4 * (ks - kVSteps) + g4) ^ rsw(r16));
        return *reinterpret_cast<const u32x4*>(p);
      };
      // loads kSAhead steps ahead of their products, the order pinned step by step (the
      // scheduler would otherwise keep only about two loads in flight)
      constexpr int kSAhead = 2;
      u32x4 kb0[kSteps], kb1[kSteps];
#pragma unroll
      for (int ks = 0; ks < kSAhead; ++ks) { kb0[ks] = key_op(ks, 0); kb1[ks] = key_op(ks, 1); }
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        if (ks + kSAhead < kSteps) { kb0[ks + kSAhead] = key_op(ks + kSAhead, 0); kb1[ks + kSAhead] = key_op(ks + kSAhead, 1); }
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(&kb0[ks]), qa[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(&kb1[ks]), qa[ks], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint32_t vb = vmask >> (4 * g4);      // bit i: key 4 g4 + i; bit 16 + i: key 16 + 4 g4 + i
      float x0[4], x1[4];
      bool raise = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x0[i] = (vb >> i) & 1u ? s0[i] * a.scale_log2 : -INFINITY;
        x1[i] = (vb >> (16 + i)) & 1u ? s1[i] * a.scale_log2 : -INFINITY;
        raise |= fmaxf(x0[i], x1[i]) > m + 8.f;   // m is the same in the head's 4 lanes
      }
      if (__ballot(raise) != 0ull) {
        // new maxima (every head of the wave, so the decision stays uniform): over the lane's
        // 8 keys, then the head's 4 lanes r16 + 16 g4
        float mt = fmaxf(fmaxf(fmaxf(x0[0], x0[1]), fmaxf(x0[2], x0[3])), fmaxf(fmaxf(x1[0], x1[1]), fmaxf(x1[2], x1[3])));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);   // exp2(-inf) = 0 at the start
        m = mn;
        lsum *= alpha;
#pragma unroll
        for (int c = 0; c < kVBlocks; ++c) o[c][0] *= alpha;
      }
      // weights (valid slots have finite scores and a finite maximum), as bf16: the B operand of
      // the weighted sum, contraction positions 8 g4 + i (key 4 g4 + i) and 8 g4 + 4 + i (key
      // 16 + 4 g4 + i)
      f32x8 pf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[i] = (vb >> i) & 1u ? __builtin_amdgcn_exp2f(x0[i] - m) : 0.f;
        pf[4 + i] = (vb >> (16 + i)) & 1u ? __builtin_amdgcn_exp2f(x1[i] - m) : 0.f;
        lsum += pf[i] + pf[4 + i];
      }
      pb = __builtin_bit_cast(bf16x8, __builtin_convertvector(pf, bf16x8v));
    }
    // ---- the pair's weights: each wave hands its heads' weights and rescale factor to the other
    //      (LDS only: the barrier does not wait for the next tile's loads). The slots are written
    //      again only after the next loop-top barrier, which the other wave reaches after its read.
    *reinterpret_cast<bf16x8*>(xme + 16 * lane) = pb;
    *reinterpret_cast<float*>(xme + 1024 + 4 * lane) = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (!pair_active) continue;
    const bf16x8 pbo = *reinterpret_cast<const bf16x8*>(xot + 16 * lane);
    const float alo = *reinterpret_cast<const float*>(xot + 1024 + 4 * lane);
    if (__ballot(alo != 1.f) != 0ull) {       // (a factor of 1 would leave them as they are)
#pragma unroll
      for (int c = 0; c < kVBlocks; ++c) o[c][1] *= alo;
    }
    // ---- weighted values of the pair's 32 heads over this wave's 256 value columns, transposed:
    //      A = values (row = column 256 e + 16 c + r16; contraction positions 8 g4 .. +7) by two
    //      transposing loads, lanes a + 4j of group g4 addressing key 4 g4 + j (first) or
    //      16 + 4 g4 + j (second), columns 256 e + 16 c + 4 a .. +3; each A serves both heads' blocks
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const uint8_t* vlo = kvt + (4 * g4 + (r16 >> 2)) * kVPitch + 8 * (r16 & 3) + kVB / 2 * e;
    const uint8_t* vhi = vlo + 16 * kVPitch;
    // loads run kPVAhead column blocks ahead of the products (written in that order: the
    // scheduler keeps source order where it cannot afford the registers to reorder)
    constexpr int kPVAhead = 2;
    v4i16 lo4[kPVAhead], hi4[kPVAhead];
#pragma unroll
    for (int c = 0; c < kPVAhead; ++c) {
      lo4[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vlo + 32 * c));
      hi4[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vhi + 32 * c));
    }
#pragma unroll
    for (int c = 0; c < kVBlocks; ++c) {
      const bf16x8 av = __builtin_shufflevector(lo4[c % kPVAhead], hi4[c % kPVAhead], 0, 1, 2, 3, 4, 5, 6, 7);
      if (c + kPVAhead < kVBlocks) {
        lo4[c % kPVAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vlo + 32 * (c + kPVAhead)));
        hi4[c % kPVAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vhi + 32 * (c + kPVAhead)));
      }
      o[c][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[c][0], 0, 0, 0);
      o[c][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pbo, o[c][1], 0, 0, 0);
    }
  }

  // ---- normalise: the head's weight sum over its 4 lanes (the pair swaps 1 / sum); stage the
  //      wave's 32 heads x 256 bf16 columns in LDS, store them as 512-byte row pieces
  float l = lsum;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse && active && g4 == 0)
    a.lse[(long long)t * a.H + h0 + r16] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
  *reinterpret_cast<float*>(xme + 1280 + 4 * lane) = inv;
  __syncthreads();                             // every wave is done with the tile buffers
  if (!pair_active) return;
  const float invo = *reinterpret_cast<const float*>(xot + 1280 + 4 * lane);
  uint8_t* ost = smem + wv * 32 * kOPitch;     // rows: heads hp .. hp + 31
#pragma unroll
  for (int c = 0; c < kVBlocks; ++c)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x4 v = o[c][b] * (b ? invo : inv);
      const uint64_t pk = (uint64_t)bf16_bits(v[0]) | (uint64_t)bf16_bits(v[1]) << 16 |
                          (uint64_t)bf16_bits(v[2]) << 32 | (uint64_t)bf16_bits(v[3]) << 48;
      *reinterpret_cast<uint64_t*>(ost + (16 * (e ^ b) + r16) * kOPitch + 2 * (16 * c + 4 * g4)) = pk;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint4* dst = reinterpret_cast<uint4*>(a.out + ((long long)t * a.H + hp) * kDV + kDV / 2 * e);
#pragma unroll
  for (int i = 0; i < 16; ++i) {               // rows 2i, 2i + 1: 32 lanes x 16 bytes each
    const int row = 2 * i + (lane >> 5);
    if (hp + row < a.H)
      dst[row * (kDV / 8) + (lane & 31)] = *reinterpret_cast<const uint4*>(ost + row * kOPitch + 16 * (lane & 31));
  }
}

}  // namespace

hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const int32_t* lengths,
                             int T, int H, int S, int topk, float sm_scale, uint16_t* out, float* lse,
                             hipStream_t st) {
  if (T == 0) return hipSuccess;
  {
    // more than 64 KB of dynamic LDS: allowed once per device
    static std::mutex mu;
    static bool done[64] = {false};
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (device >= 64 || !done[device]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_mla_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) return e;
      if (device < 64) done[device] = true;
    }
  }
  AttnArgs a;
  a.q = q; a.kv = kv; a.indices = indices; a.lengths = lengths;
  a.T = T; a.H = H; a.S = S; a.topk = topk;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.tper = (((T + kTokGroup - 1) / kTokGroup + 7) / 8) * kTokGroup;
  a.out = out; a.lse = lse;
  const int nhb = (H + 63) / 64;
  const long long blocks = 8ll * a.tper * nhb;
  hipLaunchKernelGGL(sparse_mla_kernel, dim3((unsigned)blocks), dim3(256), kLdsBytes, st, a);
  return hipGetLastError();
}

}  // namespace dsa
