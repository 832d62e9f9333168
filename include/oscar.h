/*
 * oscar.h - C ABI of the OSCAR split-cache INT2 decode path on MI355X (gfx950).
 *
 * The method (pages: the m.th-motor.com repost of the OSCAR authors' article,
 * the arddev.tech summary "OSCAR 2bit KV cache", and the snilld.dk post on
 * OSCAR making 2-bit KV cache practical):
 *   - the first 64 tokens (attention sinks) and the last 256 tokens (recent
 *     window) of each sequence stay in BF16 (thmotor: split-cache paragraph;
 *     arddev: analytics section and the launch flags in "how to apply today");
 *   - the long middle history is stored rotated by R = U . Hadamard .
 *     bit-reversal and quantised to INT2 per group of channels with a bf16
 *     scale and zero point and a clipping ratio, four 2-bit codes per byte
 *     (thmotor: rotation formula after Fig. 1; split-cache paragraph);
 *   - each decode step the oldest recent token is rotated, clipped, quantised,
 *     packed and demoted into the history (thmotor: split-cache paragraph);
 *   - decode attends the BF16 segment and the INT2 segment separately and merges
 *     them with an online-softmax merge (thmotor: decode-stage sentence of the
 *     split-cache paragraph).
 *
 * Conventions
 *   - Pointers are DEVICE pointers unless marked [host].  bf16 values are passed
 *     as their uint16_t bit patterns.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream).  Buffers must stay valid until the stream
 *     has executed the work.
 *   - Every call validates its arguments on the host before any HIP call.  On
 *     failure it returns a negative oscar_status, enqueues nothing, leaves all
 *     outputs untouched and records a message readable by oscar_last_error().
 *     A failed kernel launch returns OSCAR_EHIP.  Device-side faults surface at
 *     the caller's next synchronisation (HIP semantics).
 *   - Calls are re-entrant; the only library state is a thread-local error
 *     string and, for oscar_decode_step_noalloc, its per-device workspace
 *     array and that array's device addresses.  Calls that write the same
 *     cache records from several streams concurrently race.
 *
 * Cache layout (HBM)
 *   INT2 history pool: uint8 [num_int2_pages][Hkv][oscar_record_bytes(D, G)].
 *   One record holds 16 tokens of one KV head, as little-endian 32-bit words:
 *     code region   64 lane slots of D/32 words.  Slot l = 16*kb + t holds
 *                   the D/64 K words of token t, part kb (word blk: channels
 *                   64*blk + 16*kb + i in bits 2i, i = 0..15), then the D/64
 *                   V words of channels l, l+64, ... (token t in bits 2t)
 *     (s, z) region 16 token slots of 2*D/G words: the K words of groups
 *                   0..D/G-1, then the V words; each word is bf16 scale in
 *                   bits 0..15 and bf16 zero in bits 16..31
 *   A reader lane l takes slot l and token slot l % 16 with one 16-byte load
 *   each (D = 128, G = 64).
 *   Codes are in {0,1,2,3}; the dequantised rotated value is code*scale + zero
 *   (zero + scale*level[code] with a codebook, see oscar_cache.codebook).
 *   BF16 pools: uint16 [num_bf16_pages][Hkv][16][D], one for K and one for V.
 *   A token slot is page*16 + offset within the page.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OSCAR_OK = 0,
  OSCAR_EINVAL = -1,        /* bad pointer, size, range or combination        */
  OSCAR_EUNSUPPORTED = -2,  /* valid but not built (head_dim, group size, ...) */
  OSCAR_EWORKSPACE = -3,    /* workspace smaller than required                 */
  OSCAR_EHIP = -4           /* a HIP runtime call or kernel launch failed      */
} oscar_status;

enum {
  OSCAR_PAGE_TOKENS = 16,
  OSCAR_SINK_TOKENS = 64,
  OSCAR_RECENT_TOKENS = 256,
  OSCAR_MAX_BF16_TOKENS = 320,   /* sink + recent                              */
  OSCAR_MAX_Q_HEADS = 256,
  OSCAR_MAX_SHARED = 16          /* shared page segments per call              */
};

/* Parts of oscar_decode_attn (bit mask). */
enum {
  OSCAR_PHASE_QROT = 1,     /* q . R_k into the workspace (with the matrix-core
                               kernel also its query operands and, with a
                               codebook, each KV head's V grid)              */
  OSCAR_PHASE_BF16 = 2,     /* BF16 sink/recent segment partial                  */
  OSCAR_PHASE_INT2 = 4,     /* INT2 history chunk partials                       */
  OSCAR_PHASE_ALL = 7
};

/* Options of oscar_decode_attn / oscar_decode_step (bit mask). */
enum {
  OSCAR_FLAG_DETERMINISTIC = 1  /* accepted and without effect: every kernel
                                   assigns its work statically, so a call's
                                   outputs are bitwise the same on every run
                                   (and the fused step equals the separate
                                   calls bit for bit)                          */
};

/* Which kernel computes the INT2 segment.  AUTO picks MFMA, which serves 1,
 * 2, 4 or 8 q heads per KV head (with 1 or 2 the head quads are partly empty;
 * it still reads the cache about 2.3 to 2.9 times faster than VALU there).
 * The MFMA kernel carries its PV operands in f16.  Without a codebook the
 * weights are p * scale_v * 2^(8-b) (p <= 4, 2^(8-b) <= 16), so every V group
 * scale must stay below OSCAR_MFMA_V_SCALE_LIMIT.  With a codebook the
 * weights are p * scale_v and the other operand is each V level written as
 * base + beta * h with an integer |h| <= 2048 (exact in f16); the check
 * keeps every
 * V group scale times c = max(1, largest |V level|) / 16 below the limit,
 * and every |V level| below 16 times it.  The demotion paths check this for
 * every group they write and set OSCAR_STATUS_MFMA_V_RANGE in
 * oscar_cache.status when it fails; the caller must then ask for VALU, which
 * has no such limit (its outputs over such a cache are correct, the MFMA
 * kernel's may be inf or NaN). */
enum {
  OSCAR_INT2_AUTO = 0,
  OSCAR_INT2_VALU = 1,      /* vector-ALU dot products                         */
  OSCAR_INT2_MFMA = 2,      /* matrix-core contraction                         */
  OSCAR_HISTORY_BF16 = 3    /* comparison layout, no INT2: the history pages are
                               BF16 pages of the BF16 pool (unrotated,
                               unquantised); oscar_decode_attn skips the query
                               rotation and oscar_merge ignores R_v            */
};

/* Largest V group scale (times c with a codebook, see above) that the MFMA
 * kernel's f16 PV weights hold: 16 * 4 * 1023 = 65472 < 65504. */
#define OSCAR_MFMA_V_SCALE_LIMIT 1023.0f

/* Bits of the sticky device status word oscar_cache.status.  The demotion
 * paths (oscar_demote_pack and the demotion inside oscar_decode_step) OR
 * them in; nothing clears them but the caller (e.g. a hipMemsetAsync of 0).
 * They report problems in device-resident inputs, which the host-side
 * validation cannot see without a device-to-host read. */
enum {
  OSCAR_STATUS_CLIP_RANGE = 1,    /* a clip ratio outside (0, 1] (or NaN) was
                                     met: the groups quantised with it were
                                     written with scale 0, zero 0 and codes 0
                                     (the token reads back as 0) instead of
                                     from a clipped range                      */
  OSCAR_STATUS_MFMA_V_RANGE = 2,  /* a V group scale (times c with a
                                     codebook) reached OSCAR_MFMA_V_SCALE_LIMIT,
                                     or a V level its 16-fold: use
                                     OSCAR_INT2_VALU for this cache            */
  OSCAR_STATUS_NONFINITE = 4,     /* a rotated value, scale or zero point was
                                     inf or NaN (an inf/NaN input token, or
                                     values near the fp32 range): its codes,
                                     scale and zero are unspecified            */
  OSCAR_STATUS_DEBUG_BOUNDS = 8   /* debug build only (liboscar_debug.so,
                                     compiled with OSCAR_DEBUG): a kernel met
                                     an index it otherwise clamps or skips
                                     without a word - a page id outside the
                                     pool, a history or BF16 length beyond its
                                     bound, a demotion slot outside its pool -
                                     a merge row with more partial slots than
                                     the workspace holds, or a member of a
                                     shared segment whose history ends inside
                                     the segment's pages                       */
};

typedef struct {
  int32_t num_kv_heads;      /* Hkv >= 1                                        */
  int32_t head_dim;          /* D in {64, 128}                                  */
  int32_t group_size;        /* G in {32, 64, 128}, G divides D                 */
  int32_t page_size;         /* must be 16                                      */
  uint8_t *int2_pool;        /* [num_int2_pages][Hkv][record]                   */
  int64_t num_int2_pages;
  uint16_t *bf16_k_pool;     /* [num_bf16_pages][Hkv][16][D]                    */
  uint16_t *bf16_v_pool;
  int64_t num_bf16_pages;
  const float *codebook;     /* [Hkv][2][4] fp32 or NULL.  Lloyd-Max codebook
                                variant (thmotor, closing paragraph): per KV
                                head the 4 levels of the K codes, then of the V
                                codes, ascending and finite, in units of the
                                group scale above the zero point; a code then
                                stands for zero + scale * level and is chosen
                                as the nearest level (thresholds at the
                                midpoints, a tie to the lower level).  NULL =
                                the uniform levels 0, 1, 2, 3.  Both INT2
                                kernels read it.  The matrix-core one runs QK
                                on the codes and two more bit planes (one when
                                the K b0&b1 coefficient ((L3 - L2) - L1) + L0,
                                evaluated in fp32 in that order, is 0, as for
                                levels symmetric about their middle) and PV
                                on the V levels written per KV head as
                                base + beta * h[c] with integers
                                -2048 <= h[c] <= 2048, beta = span / H, H in
                                [2048, 4095], chosen for the closest fit
                                (typically within 2e-6 of the level span,
                                1e-5 at the 99th percentile of random level
                                sets; non-finite levels are taken in f16).
                                Level order and finiteness are not checked
                                (device memory); the quantiser counts the
                                level midpoints below a value, whatever the
                                order                                        */
  uint32_t *status;          /* device word (4-byte aligned) or NULL: sticky
                                OSCAR_STATUS_* bits set by the demotion paths
                                (the calls that write records); NULL = not
                                reported                                     */
} oscar_cache;

/* History pages that several sequences share (a common prompt prefix held
 * once in a paged, prefix-aware cache: thmotor, split-cache paragraph - the
 * method works with paged KV and radix prefix caching; Fig. 6 - throughput
 * grows with the prefix-cache hit ratio).  Sequences seq_begin ..
 * seq_begin + num_seqs - 1 list the same physical INT2 pages at logical
 * history pages first_page .. first_page + num_pages - 1 (the pages are read
 * from sequence seq_begin's table), and each of those pages holds 16 tokens
 * for every one of them.  With the matrix-core INT2 kernel (AUTO or MFMA),
 * one group per token (G == D) and uniform codes (no codebook), the pages are
 * attended once for all the sequences' q heads
 * (up to num_seqs x Hq/Hkv query rows per KV head) and the result is merged
 * with each sequence's own pages; otherwise every sequence reads them as its
 * own.  The segments of one sequence must tile its first history pages:
 * ordered by first_page, the first starts at page 0 and each next one where
 * the previous ends.  Every member's hist_len must cover its segments' pages
 * whole (hist_len >= 16 * (first_page + num_pages)): they are attended whole
 * for each member (device memory, not checked; the debug build reports a
 * shorter history through OSCAR_STATUS_DEBUG_BOUNDS). */
typedef struct {
  int32_t first_page;
  int32_t num_pages;         /* >= 1                                            */
  int32_t seq_begin;
  int32_t num_seqs;          /* >= 2                                            */
} oscar_shared_pages;

typedef struct {
  int32_t batch;             /* B >= 1                                          */
  int32_t num_q_heads;       /* Hq, a multiple of Hkv, <= OSCAR_MAX_Q_HEADS     */
  const int32_t *kv_head_of_q; /* [host][Hq] KV head of each q head, every KV
                                  head used by exactly Hq/Hkv q heads; NULL means
                                  h -> h / (Hq/Hkv)                             */
  const int32_t *hist_pages; /* [B][hist_stride] physical INT2 page ids in token
                                order; entries past ceil(hist_len/16) unread     */
  int32_t hist_stride;
  const int32_t *hist_len;   /* [B] INT2 history tokens, 0 <= len <= max_hist_len */
  const int32_t *bf16_pages; /* [B][bf16_stride] physical BF16 page ids         */
  int32_t bf16_stride;
  const int32_t *bf16_len;   /* [B] BF16 tokens (sink + recent), 0..320; slots
                                0..len-1 of the listed pages are attended (their
                                order does not matter)                          */
  int32_t max_hist_len;      /* [host] upper bound on every hist_len; sizes the
                                grid without a device-to-host read               */
  float sm_scale;            /* softmax scale; 0 means 1/sqrt(D)                */
  int32_t num_splits;        /* history chunks per (sequence, KV head); 0 = auto;
                                at most min(1024, history pages) are used       */
  int32_t int2_kernel;       /* OSCAR_INT2_AUTO / _VALU / _MFMA, or
                                OSCAR_HISTORY_BF16                              */
  uint32_t phases;           /* oscar_decode_attn work: OR of OSCAR_PHASE_*; 0 means
                                all.  Phases may be issued in separate calls (e.g.
                                on two streams or between timing events); the
                                INT2 phase reads the rotated query that the QROT
                                phase writes into the workspace                 */
  uint32_t flags;            /* OR of OSCAR_FLAG_*; 0 = defaults                  */
  int32_t num_shared;        /* [host] entries of `shared`, 0..OSCAR_MAX_SHARED  */
  const oscar_shared_pages *shared;  /* [host] shared history pages, or NULL    */
} oscar_decode_args;

/* Bytes of one INT2 page record: 2*16*(D/4) + 2*16*(D/G)*4. */
size_t oscar_record_bytes(int32_t head_dim, int32_t group_size);

/* Text for the last non-OK status returned on this thread ("" if none). */
const char *oscar_last_error(void);

/*
 * oscar_write_bf16 - store n new tokens' K and V into BF16 slots (the new
 * decode token goes into the recent window; thmotor split-cache paragraph).
 *   dst_slot [n]       BF16 slot page*16+off, or -1 to skip the entry
 *   k_new, v_new       [n][Hkv][D] bf16
 * Errors: EINVAL for NULL pointers with n > 0, n < 0, bad cache descriptor.
 */
int oscar_write_bf16(const oscar_cache *cache, int32_t n, const int32_t *dst_slot,
                     const uint16_t *k_new, const uint16_t *v_new, void *stream);

/*
 * oscar_demote_pack - rotate, clip, quantise and pack n tokens from BF16 slots
 * into INT2 history slots (thmotor: split-cache paragraph, rotate/clip/
 * quantize/pack at demotion, four 2-bit values per byte; the clipping
 * threshold is per layer and head, calibration paragraph).
 *   src_slot [n]   BF16 slot (page*16+off) read for every KV head, or -1 to skip
 *   dst_slot [n]   INT2 slot (page*16+off) written for every KV head
 *   R_k, R_v       [Hkv][D][D] fp32, row-vector convention x = k . R;
 *                  R_v == NULL means identity (value rotation folded upstream)
 *   clip_k, clip_v [Hkv] fp32 clipping ratios in (0, 1], per KV head
 * Per (token, KV head, K|V): x = k . R in fp64; per group of G consecutive
 * channels mx, mn = max, min; scale = (c*mx - c*mn)/3 and zero = c*mn rounded
 * to bf16 (nearest even, from fp64); code = clamp(rint((x - zero)/scale), 0, 3)
 * (0 when scale == 0).  The other tokens' bits in a shared record are
 * preserved, so any set of distinct destination slots may be demoted in one
 * call; two entries with the same destination race.
 * Device-side checks (reported through cache->status, see OSCAR_STATUS_*):
 * a clip ratio outside (0, 1] is rejected (that head's K or V groups are
 * written as scale 0, zero 0, codes 0), a V scale at the matrix-core limit
 * and non-finite values are flagged.
 * Errors: EINVAL (NULL pointers with n > 0, misaligned pointers), EUNSUPPORTED
 * (D, G), EHIP.
 */
int oscar_demote_pack(const oscar_cache *cache, int32_t n, const int32_t *src_slot,
                      const int32_t *dst_slot, const float *R_k, const float *R_v,
                      const float *clip_k, const float *clip_v, void *stream);

/* Workspace bytes oscar_decode_attn, oscar_merge and oscar_decode_step need
 * for these arguments (host only).  0 when the arguments are invalid (the
 * reason is in oscar_last_error()); never 0 for valid arguments. */
size_t oscar_decode_workspace_bytes(const oscar_cache *cache, const oscar_decode_args *args);

/*
 * oscar_decode_plan - the history chunking oscar_decode_attn will use for these
 * arguments (host only): num_splits chunks of pages_per_split pages per
 * (sequence, KV head), the workspace size, and the INT2 kernel that runs
 * (OSCAR_INT2_VALU, OSCAR_INT2_MFMA or OSCAR_HISTORY_BF16, AUTO resolved).
 * Any output may be NULL.
 * VALU kernel and BF16 history: automatic chunking (num_splits == 0) aims at
 * 2048 (sequence, KV head, chunk) units while keeping every chunk at least 8x
 * the bytes of its partial result and 16 pages long; chunk c covers pages
 * [c*pages_per_split, (c+1)*pages_per_split) and empty chunks are dropped.
 * MFMA kernel: a chunk is one of num_splits equal parts of each sequence's
 * history.  One block of 16 waves serves one part for a pair of KV heads
 * (8 waves per head); the waves of a head take fixed, interleaved batches of
 * its pages and their results are combined in wave order into one partial per
 * (q head, part).
 * Automatic chunking aims at 256 blocks (one per compute unit) while keeping
 * every part at least 2x its partial bytes and 8 pages per head;
 * pages_per_split is nominal.  An explicit num_splits is capped at the page
 * count and at 1024.
 */
int oscar_decode_plan(const oscar_cache *cache, const oscar_decode_args *args,
                      int32_t *num_splits, int32_t *pages_per_split, size_t *workspace_bytes,
                      int32_t *int2_kernel);

/*
 * oscar_decode_attn - attend every q head over both segments, producing partial
 * results in `workspace` (thmotor: decode stage of the split-cache paragraph).
 *   q          [B][Hq][D] bf16
 *   R_k        [Hkv][D][D] fp32: the history is attended with q . R_k (unused,
 *              may be NULL, with OSCAR_HISTORY_BF16)
 *   workspace  >= oscar_decode_workspace_bytes; contents valid for a following
 *              oscar_merge with the same cache/args on the same stream
 * Partials per (sequence, q head): one for the BF16 segment (unrotated q and
 * K/V) and one per history chunk (rotated basis), each (max logit, sum of
 * exponentials, unnormalised output), fp32.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP.
 */
int oscar_decode_attn(const oscar_cache *cache, const oscar_decode_args *args,
                      const uint16_t *q, const float *R_k, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * oscar_merge - log-sum-exp merge of the history chunks, un-rotation of the
 * history output by R_v^T, and online-softmax merge with the BF16 segment
 * (thmotor: online softmax merge of the two segments).
 *   R_v  [Hkv][D][D] fp32 or NULL (identity)
 *   out  [B][Hq][D] fp32 attention output
 *   lse  [B][Hq] fp32 natural-log softmax denominator, or NULL
 * A (sequence, head) with no tokens at all gets out = 0 and lse = -inf.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP.
 */
int oscar_merge(const oscar_cache *cache, const oscar_decode_args *args,
                const void *workspace, size_t workspace_bytes, const float *R_v,
                float *out, float *lse, void *stream);

/*
 * oscar_decode_step - one whole decode step of a batch in three launches
 * (m.th-motor.com repost of the OSCAR article, split-cache paragraph: the new
 * token enters the recent window, the oldest recent token is rotated,
 * clipped, quantised, packed and demoted, and decode attends the BF16 and
 * INT2 segments and merges them).  Same result, bit for bit, as
 *   oscar_demote_pack(cache, B, demote_src, demote_dst, R_k, R_v, clip_k, clip_v)
 *   oscar_write_bf16(cache, B, new_slot, k_new, v_new)
 *   oscar_decode_attn(cache, args, q, R_k, workspace)
 *   oscar_merge(cache, args, workspace, R_v, out, lse)
 * with the first launch doing the demotion, the token store, the query
 * rotation and the BF16 segment side by side (the BF16 segment reads the new
 * token from k_new/v_new), then the INT2 history chunks, then the merge.
 *   demote_src, demote_dst [B] slots (page*16 + offset) of sequence b's
 *              demoted token, -1 = no demotion for b
 *   new_slot   [B] BF16 slot of sequence b's new token, -1 = none; it may be
 *              demote_src[b] (the freed slot) but no other sequence's
 *              demote_src, and must be one of the slots args lists for b
 *   k_new, v_new [B][Hkv][D] bf16, 16-byte aligned
 *   args       describes the cache after the step (lengths include the new
 *              token and the demoted one); phases must be 0 (or
 *              OSCAR_PHASE_ALL); the history kind must be an INT2 one
 * Errors: as the four calls, plus EINVAL for phases != 0 and EUNSUPPORTED for
 * OSCAR_HISTORY_BF16.  Nothing is launched on an error.
 */
int oscar_decode_step(const oscar_cache *cache, const oscar_decode_args *args,
                      const int32_t *demote_src, const int32_t *demote_dst, const float *clip_k,
                      const float *clip_v, const int32_t *new_slot, const uint16_t *k_new,
                      const uint16_t *v_new, const uint16_t *q, const float *R_k, const float *R_v,
                      void *workspace, size_t workspace_bytes, float *out, float *lse,
                      void *stream);

/* Bytes of the device workspace that oscar_decode_step_noalloc uses: one
 * copy per device, part of the library's device code, held until the process
 * ends (16 MiB: enough for a Qwen3-8B-shaped batch of 64 sequences at 100K
 * context, or a Qwen3-32B-shaped batch of 16 at 128K). */
#define OSCAR_NOALLOC_WORKSPACE_BYTES (16u << 20)

/*
 * oscar_decode_step_noalloc - oscar_decode_step with no workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): the step's
 * workspace is the library's own static device array.  It calls no
 * hipMalloc, hipFree or allocating library routine.  Arguments, results and
 * errors are those of oscar_decode_step, plus:
 *   - OSCAR_EWORKSPACE when oscar_decode_workspace_bytes(cache, args) exceeds
 *     OSCAR_NOALLOC_WORKSPACE_BYTES (nothing is launched);
 *   - the work is enqueued for the current device, which must be the stream's
 *     (EINVAL otherwise); the first call on a device looks up that device's
 *     copy of the array (hipGetSymbolAddress), so make it outside a capture.
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (nothing in it needs clearing: each step writes what it
 * reads).  Calls that overlap on one device - on two streams, or from two
 * threads without ordering - race on it.
 */
int oscar_decode_step_noalloc(const oscar_cache *cache, const oscar_decode_args *args,
                              const int32_t *demote_src, const int32_t *demote_dst,
                              const float *clip_k, const float *clip_v, const int32_t *new_slot,
                              const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                              const float *R_k, const float *R_v, float *out, float *lse,
                              void *stream);

#ifdef __cplusplus
}
#endif
#endif /* OSCAR_H */
