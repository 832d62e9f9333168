// Internal helpers shared by the HIP translation units of liboscar.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

constexpr int kPage = OSCAR_PAGE_TOKENS;
constexpr int kMaxBf16 = OSCAR_MAX_BF16_TOKENS;
constexpr int kBf16PagesPerSplit = 4;                              // one wave per page
constexpr int kMaxSplits = 1024;        // history chunks per (sequence, KV head)
constexpr int kMfmaTargetBlocks = 256;          // matrix-core INT2 kernel: default grid, one block per CU
// Waves per block of the matrix-core INT2 kernel: 16 (four per SIMD, at most
// 128 registers each), or 8 (two per SIMD, 256 registers) for the instances
// whose page loop needs more than 128 registers: with D = 128 and G = 32
// (four groups per token) at 8 q heads per KV head or with a codebook, and
// with a codebook at 8 q heads per KV head and G = 32 or (D = 128) G = 64.
// Spilled registers would be reloaded from scratch inside the page loop, and
// each reload waits for every page load issued before it.  gq: 4 or 8, the q
// heads of a wave (fewer than 4 per KV head use 4).
__host__ __device__ constexpr int mfma_waves(int d, int g, int gq, bool cb) {
  return ((d == 128 && g == 32 && (gq == 8 || cb)) || (cb && gq == 8 && (g == 32 || (d == 128 && g == 64))))
             ? 8 : 16;
}
// Query A operand sets per QK step of the matrix-core INT2 kernel (gq: its
// q-head slots, 4 or 8): with a codebook one per code plane (the query
// pieces times the plane's weight, all planes contracted into one
// accumulator), except at D = 128 with 8 q heads per KV head and G = 32 or
// 128, where the three sets would not fit the registers of the instance's
// waves (G = 128 at 8 waves per block instead of 16 measured slower than
// the unfolded planes) and the planes keep separate accumulators; without a
// codebook one
__host__ __device__ constexpr int mfma_a_planes(int d, int g, int gq, bool cb) {
  return cb && !(d == 128 && gq == 8 && (g == 32 || g == 128)) ? 3 : 1;
}
// sequences the kernel balances its blocks across (one per thread of a block)
__host__ __device__ constexpr int mfma_max_balanced(int waves) { return 64 * waves; }
// KV heads per block of the matrix-core INT2 kernel: 2 (1 for a single KV
// head); the block's waves are split evenly over them.  Two heads per block
// keep the partial results per (sequence, q head) few when a batch has only a
// few sequences (each block still fills one compute unit), and measured at
// least as fast as 4 or 8 heads per block on long batches.
__host__ __device__ constexpr int mfma_heads_per_block(int hkv) { return hkv >= 2 ? 2 : 1; }
// QK matrix instructions per page and head quad of the matrix-core INT2 kernel
// (int8 K = 64 channels each, one per group inside a 64-channel block)
__host__ __device__ constexpr int mfma_qk_steps(int d, int g) { return (d / 64) * (g < 64 ? 64 / g : 1); }
constexpr int kBf16Splits = kMaxBf16 / (kPage * kBf16PagesPerSplit); // 5 BF16 partials
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
#ifndef OSCAR_ROT_PARTS
#define OSCAR_ROT_PARTS 2
#endif
#ifndef OSCAR_STEP_PRE_WAVES
#define OSCAR_STEP_PRE_WAVES 6
#endif
constexpr int kRotParts = OSCAR_ROT_PARTS;         // R rows of a rotation thread, requested in parts
constexpr int kStepPreWaves = OSCAR_STEP_PRE_WAVES; // decode-step prologue: waves per SIMD it must fit

// Byte offsets of the four sections of one INT2 page record (16 tokens, one KV
// head): K codes [16][D/4] | V codes [D][4] | K (s,z) [16][D/G] dwords | V (s,z).
struct RecLayout {
  // One (page, KV head) record: a code region of 64 lane slots of D/32 words
  // (slot l = 16*kb + t: the D/64 K words of token t, part kb, then the D/64 V
  // words of channels l, l + 64, ...) and a scale/zero region of 16 token
  // slots of 2*D/G words (K groups, then V groups; scale | zero << 16).
  int D, G;
  __host__ __device__ constexpr RecLayout(int d, int g) : D(d), G(g) {}
  __host__ __device__ constexpr int slot_words() const { return D / 32; }
  __host__ __device__ constexpr int codes_bytes() const { return 64 * (D / 32) * 4; }
  __host__ __device__ constexpr int tok_words() const { return 2 * (D / G); }
  // byte offsets
  __host__ __device__ constexpr int kword(int slot, int blk) const { return (slot * (D / 32) + blk) * 4; }
  __host__ __device__ constexpr int vword(int slot, int h2) const { return (slot * (D / 32) + D / 64 + h2) * 4; }
  __host__ __device__ constexpr int tok_sz(int t) const { return codes_bytes() + t * tok_words() * 4; }
  __host__ __device__ constexpr int ksz(int t, int g) const { return tok_sz(t) + g * 4; }
  __host__ __device__ constexpr int vsz(int t, int g) const { return tok_sz(t) + (D / G + g) * 4; }
  __host__ __device__ constexpr int bytes() const { return codes_bytes() + kPage * tok_words() * 4; }
};

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Shared history pages as the kernels see them (one oscar_shared_pages entry
// plus its launch plan): `parts` equal page ranges, each one block per KV
// head and group of up to kCasRowsPerBlock query rows; the segment's blocks
// start at block_base of the cascade grid.
constexpr int kMaxShared = OSCAR_MAX_SHARED;
constexpr int kCasWaves = 4;                 // waves per cascade block
constexpr int kCasRowsPerWave = 32;          // two 16-row MFMA tiles
constexpr int kCasRowsPerBlock = kCasWaves * kCasRowsPerWave;
struct SharedSeg {
  int first, num;        // logical history pages [first, first + num)
  int seq0, nseq;        // member sequences [seq0, seq0 + nseq)
  int parts, rgroups;    // page ranges, row groups
  int block_base;        // first block of the segment in the cascade grid
};

// Debug build (OSCAR_DEBUG): report an index that a kernel clamps or skips
// (it goes on as in the release build) through the status word.
#ifdef OSCAR_DEBUG
#define OSCAR_DCHECK(ok, status)                                                   \
  do {                                                                            \
    if (!(ok) && (status) != nullptr) atomicOr((status), (uint32_t)OSCAR_STATUS_DEBUG_BOUNDS); \
  } while (0)
#else
#define OSCAR_DCHECK(ok, status) \
  do {                           \
  } while (0)
#endif

// Workspace partition used by decode_attn and merge.
struct WsLayout {
  size_t qrot;      // fp32 [B][Hq][D]     q . R_k (unscaled)
  size_t qpk;       // matrix-core kernel only: int32 [B][Hkv][g/4][planes][mfma_qk_steps][64][4]
                    //   its QK A operands (the rotated query in 7-bit pieces;
                    //   planes: mfma_a_planes)
  size_t nslots;    // matrix-core kernel only: int32 [B] partial slots each sequence used
  size_t qhd;       // matrix-core kernel only: [B][Hq][8] per q head: int exponent
                    //   (bits), then sum of q_rot over each group * sm_scale * log2(e)
  size_t vgrid;     // matrix-core kernel with a codebook only: uint32 [Hkv][4] the
                    //   V levels as Lmin + beta * h[c]: h[c] in f16 (low bytes,
                    //   high bytes), Lmin and beta (fp32 bits)
  size_t qcas;      // shared pages only: int8 [B][Hq][3][D] the 7-bit pieces of the
                    //   rotated query (piece-major), each 16-channel block stored
                    //   4x4-transposed (byte 4i + j = channel 4j + i) for the MFMA
  size_t part_o;    // fp32 [B][Hq][S][D]  history chunk partial outputs (rotated basis)
  size_t part_ml;   // fp32 [B][Hq][S][2]  (max logit in log2 units, sum of exponentials)
  size_t bf_o;      // fp32 [B][Hq][kBf16Splits][D]  BF16 segment partial outputs
  size_t bf_ml;     // fp32 [B][Hq][kBf16Splits][2]
  size_t total;
  int splits;       // S
  int pages_per_split;
};

// Kernel-side description of a decode call (passed by value).
struct DecodeParams {
  int B, Hq, Hkv, g, D, G;
  const uint8_t *int2_pool;
  int64_t num_int2_pages;
  const uint16_t *bf16_k, *bf16_v;
  int64_t num_bf16_pages;
  const int32_t *hist_pages;
  int hist_stride;
  const int32_t *hist_len;
  const int32_t *bf16_pages;
  int bf16_stride;
  const int32_t *bf16_len;
  int max_hist_len;
  float sm_log2;       // softmax scale * log2(e)
  int int2_kind;       // resolved history kernel: OSCAR_INT2_VALU, _MFMA or OSCAR_HISTORY_BF16
  int splits, pages_per_split;   // partial slots per (sequence, q head); nominal pages
  int mfma_parts;      // matrix-core kernel: blocks per head group = B * mfma_parts
  int mfma_balanced;   // matrix-core kernel: may balance blocks across sequences
  const float *codebook;   // [Hkv][2][4] code levels (K, V) or nullptr = 0, 1, 2, 3
  uint32_t *status;        // the cache's sticky status word (debug-build checks) or nullptr
  // shared history pages (cascade): the partial slots of a sequence are first
  // its cascade slots (sum of `parts` over its segments, in page order), then
  // those of the matrix-core kernel, which skips the shared pages
  int n_shared;
  int cas_slots;           // max over sequences of their cascade slots
  int cas_blocks;          // cascade grid size
  SharedSeg shared[kMaxShared];
  uint8_t *ws;
  WsLayout L;
  int16_t q_of_kv[OSCAR_MAX_Q_HEADS];  // [Hkv][g] q heads of each KV head
  int16_t kv_of_q[OSCAR_MAX_Q_HEADS];  // [Hq] KV head of each q head
};

// Wave-local ordering of LDS traffic between lanes of one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Launchers (defined next to their kernels).
hipError_t launch_write_bf16(const oscar_cache &c, int n, const int32_t *dst, const uint16_t *k,
                             const uint16_t *v, hipStream_t s);
hipError_t launch_demote(const oscar_cache &c, int n, const int32_t *src, const int32_t *dst,
                         const float *Rk, const float *Rv, const float *ck, const float *cv,
                         hipStream_t s);
hipError_t launch_qrot(const DecodeParams &p, const uint16_t *q, const float *Rk, hipStream_t s);
hipError_t launch_bf16_seg(const DecodeParams &p, const uint16_t *q, hipStream_t s);
hipError_t launch_int2_valu(const DecodeParams &p, hipStream_t s);
hipError_t launch_int2_mfma(const DecodeParams &p, hipStream_t s);
hipError_t launch_int2_cascade(const DecodeParams &p, hipStream_t s);

// Cascade slots of sequence b (the partial slots its shared segments fill)
// and the history pages they cover from page 0.
__host__ __device__ inline int cascade_slots(const DecodeParams &p, int b, int *skip_pages) {
  int n = 0, skip = 0;
  for (int i = 0; i < p.n_shared; ++i) {
    const SharedSeg &s = p.shared[i];
    if (b >= s.seq0 && b < s.seq0 + s.nseq) {
      n += s.parts;
      skip = s.first + s.num > skip ? s.first + s.num : skip;
    }
  }
  if (skip_pages) *skip_pages = skip;
  return n;
}
hipError_t launch_bf16_hist(const DecodeParams &p, const uint16_t *q, hipStream_t s);
hipError_t launch_merge(const DecodeParams &p, const float *Rv, float *out, float *lse,
                        hipStream_t s);
hipError_t launch_step_pre(const DecodeParams &p, const oscar_cache &c, const uint16_t *q,
                           const float *Rk, const float *Rv, const float *ck, const float *cv,
                           const int32_t *dsrc, const int32_t *ddst, const int32_t *new_slot,
                           const uint16_t *k_new, const uint16_t *v_new, hipStream_t s);

}  // namespace oscar
