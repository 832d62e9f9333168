// Host side of liboscar: argument validation, workspace layout, launches.
// Validation never calls the HIP runtime, so every argument error is reported
// the same way with or without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "common.hpp"

// Workspace of oscar_decode_step_noalloc: one copy per device, held until
// the process ends.  In host code this name is only a stand-in for the
// symbol; its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_WORKSPACE_BYTES];

namespace oscar {
namespace {

thread_local std::string g_err;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_dev[kMaxDevices];   // device address of `scratch` on each device

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(OSCAR_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_cache(const oscar_cache *c) {
  if (c == nullptr) return fail(OSCAR_EINVAL, "cache is NULL");
  if (c->page_size != OSCAR_PAGE_TOKENS)
    return fail(OSCAR_EINVAL, "page_size must be %d (got %d)", OSCAR_PAGE_TOKENS, c->page_size);
  if (c->num_kv_heads < 1 || c->num_kv_heads > OSCAR_MAX_Q_HEADS)
    return fail(OSCAR_EINVAL, "num_kv_heads out of range (got %d)", c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(OSCAR_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  const int G = c->group_size;
  if (G != 32 && G != 64 && G != 128)
    return fail(OSCAR_EUNSUPPORTED, "group_size must be 32, 64 or 128 (got %d)", G);
  if (G > c->head_dim || c->head_dim % G != 0)
    return fail(OSCAR_EUNSUPPORTED, "group_size %d does not divide head_dim %d", G, c->head_dim);
  if (c->num_int2_pages < 0 || c->num_bf16_pages < 0)
    return fail(OSCAR_EINVAL, "negative page count");
  if (c->num_int2_pages > 0 && (c->int2_pool == nullptr || !aligned(c->int2_pool, 16)))
    return fail(OSCAR_EINVAL, "int2_pool is NULL or not 16-byte aligned");
  if (c->num_bf16_pages > 0 &&
      (c->bf16_k_pool == nullptr || c->bf16_v_pool == nullptr || !aligned(c->bf16_k_pool, 16) ||
       !aligned(c->bf16_v_pool, 16)))
    return fail(OSCAR_EINVAL, "bf16 pools are NULL or not 16-byte aligned");
  if (c->status != nullptr && !aligned(c->status, 4))
    return fail(OSCAR_EINVAL, "status word is not 4-byte aligned");
  return OSCAR_OK;
}

// Fills kv_of_q / q_of_kv; checks every KV head is used by exactly g q heads.
int build_head_map(const oscar_cache *c, const oscar_decode_args *a, DecodeParams *p) {
  const int Hq = a->num_q_heads, Hkv = c->num_kv_heads;
  if (Hq < 1 || Hq > OSCAR_MAX_Q_HEADS)
    return fail(OSCAR_EINVAL, "num_q_heads out of range (got %d)", Hq);
  if (Hq % Hkv != 0)
    return fail(OSCAR_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", Hq, Hkv);
  const int g = Hq / Hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(OSCAR_EUNSUPPORTED, "q heads per KV head must be 1, 2, 4 or 8 (got %d)", g);
  int cnt[OSCAR_MAX_Q_HEADS] = {0};
  for (int h = 0; h < Hq; ++h) {
    const int j = a->kv_head_of_q ? a->kv_head_of_q[h] : h / g;
    if (j < 0 || j >= Hkv)
      return fail(OSCAR_EINVAL, "kv_head_of_q[%d] = %d outside [0, %d)", h, j, Hkv);
    if (cnt[j] >= g)
      return fail(OSCAR_EINVAL, "KV head %d is used by more than %d q heads", j, g);
    p->kv_of_q[h] = (int16_t)j;
    p->q_of_kv[j * g + cnt[j]] = (int16_t)h;
    ++cnt[j];
  }
  p->g = g;
  return OSCAR_OK;
}

int check_args(const oscar_cache *c, const oscar_decode_args *a, DecodeParams *p) {
  int st = check_cache(c);
  if (st) return st;
  if (a == nullptr) return fail(OSCAR_EINVAL, "args is NULL");
  if (a->batch < 1) return fail(OSCAR_EINVAL, "batch must be >= 1 (got %d)", a->batch);
  st = build_head_map(c, a, p);
  if (st) return st;
  if (a->max_hist_len < 0) return fail(OSCAR_EINVAL, "max_hist_len < 0");
  if (a->hist_len == nullptr || a->bf16_len == nullptr)
    return fail(OSCAR_EINVAL, "hist_len / bf16_len must not be NULL");
  const int need_hist = (a->max_hist_len + OSCAR_PAGE_TOKENS - 1) / OSCAR_PAGE_TOKENS;
  if (need_hist > 0) {
    if (a->hist_pages == nullptr) return fail(OSCAR_EINVAL, "hist_pages is NULL");
    if (a->hist_stride < need_hist)
      return fail(OSCAR_EINVAL, "hist_stride %d < ceil(max_hist_len/16) = %d", a->hist_stride,
                  need_hist);
    if (a->int2_kernel == OSCAR_HISTORY_BF16) {
      if (c->num_bf16_pages <= 0) return fail(OSCAR_EINVAL, "max_hist_len > 0 but no BF16 pages");
    } else if (c->num_int2_pages <= 0) {
      return fail(OSCAR_EINVAL, "max_hist_len > 0 but no INT2 pages");
    }
  }
  if (a->bf16_pages == nullptr || a->bf16_stride < 1)
    return fail(OSCAR_EINVAL, "bf16_pages is NULL or bf16_stride < 1");
  if (!(a->sm_scale >= 0.f) || !std::isfinite(a->sm_scale))
    return fail(OSCAR_EINVAL, "sm_scale must be finite and >= 0");
  if (a->num_splits < 0) return fail(OSCAR_EINVAL, "num_splits < 0");
  if (a->int2_kernel < OSCAR_INT2_AUTO || a->int2_kernel > OSCAR_HISTORY_BF16)
    return fail(OSCAR_EINVAL, "int2_kernel must be 0, 1, 2 or 3");
  if (a->phases & ~(uint32_t)OSCAR_PHASE_ALL) return fail(OSCAR_EINVAL, "unknown phase bits");
  if (a->flags & ~(uint32_t)OSCAR_FLAG_DETERMINISTIC) return fail(OSCAR_EINVAL, "unknown flag bits");

  p->B = a->batch;
  p->Hq = a->num_q_heads;
  p->Hkv = c->num_kv_heads;
  p->D = c->head_dim;
  p->G = c->group_size;
  p->int2_pool = c->int2_pool;
  p->num_int2_pages = c->num_int2_pages;
  p->bf16_k = c->bf16_k_pool;
  p->bf16_v = c->bf16_v_pool;
  p->num_bf16_pages = c->num_bf16_pages;
  p->hist_pages = a->hist_pages;
  p->hist_stride = a->hist_stride;
  p->hist_len = a->hist_len;
  p->bf16_pages = a->bf16_pages;
  p->bf16_stride = a->bf16_stride;
  p->bf16_len = a->bf16_len;
  p->max_hist_len = a->max_hist_len;
  const float sm = a->sm_scale > 0.f ? a->sm_scale : 1.0f / std::sqrt((float)c->head_dim);
  p->sm_log2 = sm * kLog2e;

  // INT2 kernel: the matrix-core one serves every supported ratio and reads
  // the cache faster than the vector-ALU one at each of them
  p->codebook = c->codebook;
  p->status = c->status;
  int kind = a->int2_kernel;
  if (kind == OSCAR_INT2_AUTO) kind = OSCAR_INT2_MFMA;
  p->int2_kind = kind;

  // shared history pages: validated whatever kernel runs; attended once for
  // all their sequences (cascade) with the matrix-core kernel when a token's
  // channels form one group (G == D) and the codes are uniform (the cascade
  // has no codebook path: with one, every sequence reads its pages itself)
  if (a->num_shared < 0 || a->num_shared > OSCAR_MAX_SHARED)
    return fail(OSCAR_EINVAL, "num_shared must be in [0, %d] (got %d)", OSCAR_MAX_SHARED,
                a->num_shared);
  if (a->num_shared > 0 && a->shared == nullptr) return fail(OSCAR_EINVAL, "shared is NULL");
  for (int i = 0; i < a->num_shared; ++i) {
    const oscar_shared_pages &e = a->shared[i];
    if (e.first_page < 0 || e.num_pages < 1 || e.num_seqs < 2 || e.seq_begin < 0 ||
        (long long)e.seq_begin + e.num_seqs > a->batch)
      return fail(OSCAR_EINVAL, "shared[%d]: pages [%d, +%d) of sequences [%d, +%d) out of range",
                  i, e.first_page, e.num_pages, e.seq_begin, e.num_seqs);
    if ((long long)(e.first_page + (long long)e.num_pages) * OSCAR_PAGE_TOKENS > a->max_hist_len)
      return fail(OSCAR_EINVAL, "shared[%d] ends beyond max_hist_len", i);
  }
  if (a->num_shared > 0) {
    // the segments of every sequence tile its first pages, in page order
    for (int b = 0; b < a->batch; ++b) {
      int next = 0, left = 0;
      for (int i = 0; i < a->num_shared; ++i)
        left += (b >= a->shared[i].seq_begin && b < a->shared[i].seq_begin + a->shared[i].num_seqs);
      while (left > 0) {
        int found = -1;
        for (int i = 0; i < a->num_shared; ++i) {
          const oscar_shared_pages &e = a->shared[i];
          if (b >= e.seq_begin && b < e.seq_begin + e.num_seqs && e.first_page == next) {
            if (found >= 0) return fail(OSCAR_EINVAL, "sequence %d: two shared segments at page %d", b, next);
            found = i;
          }
        }
        if (found < 0)
          return fail(OSCAR_EINVAL, "sequence %d: its shared segments do not tile pages from 0 (gap at %d)",
                      b, next);
        next += a->shared[found].num_pages;
        --left;
      }
    }
  }
  p->n_shared = 0;
  p->cas_slots = 0;
  p->cas_blocks = 0;
  if (a->num_shared > 0 && kind == OSCAR_INT2_MFMA && c->group_size == c->head_dim &&
      c->codebook == nullptr) {
    // page ranges of about equal size so that the grid holds ~2 blocks per
    // compute unit (as many as fit at once), each at least kCasMinPages pages
    // (its partials, written and read back, stay well below the pages' bytes)
    constexpr int kCasMinPages = 32, kCasTargetBlocks = 512;
    long long work = 0;
    const int g = p->g;
    for (int i = 0; i < a->num_shared; ++i) {
      const int rg = (a->shared[i].num_seqs * g + kCasRowsPerBlock - 1) / kCasRowsPerBlock;
      work += (long long)a->shared[i].num_pages * rg * c->num_kv_heads;
    }
    long long pc = (work + kCasTargetBlocks - 1) / kCasTargetBlocks;
    pc = pc < kCasMinPages ? kCasMinPages : pc;
    int base = 0;
    for (int i = 0; i < a->num_shared; ++i) {
      const oscar_shared_pages &e = a->shared[i];
      SharedSeg &sg = p->shared[i];
      sg.first = e.first_page;
      sg.num = e.num_pages;
      sg.seq0 = e.seq_begin;
      sg.nseq = e.num_seqs;
      sg.parts = (int)((e.num_pages + pc - 1) / pc);
      sg.rgroups = (e.num_seqs * g + kCasRowsPerBlock - 1) / kCasRowsPerBlock;
      sg.block_base = base;
      base += sg.parts * c->num_kv_heads * sg.rgroups;
    }
    p->n_shared = a->num_shared;
    p->cas_blocks = base;
    for (int b = 0; b < a->batch; ++b) {
      const int n = cascade_slots(*p, b, nullptr);
      p->cas_slots = n > p->cas_slots ? n : p->cas_slots;
    }
  }

  // history split.  Vector-ALU kernel: enough waves to fill the chip once (4
  // waves per (sequence, KV head, chunk)), each chunk streaming at least 8x
  // the bytes of its partial result (read and written once more by the merge)
  // and 16 pages.  Matrix-core kernel: one block of 16 (or 8) waves per
  // (sequence, pair of KV heads, part), the pair's waves combining
  // their results into one partial per (q head, part); enough parts for one
  // block per compute unit, each part at least 2x its partial bytes and 8
  // pages per head; its pages_per_split is nominal.
  const int npages = need_hist;
  int S = 1;
  if (npages > 0) {
    if (a->num_splits > 0) {
      S = a->num_splits > npages ? npages : a->num_splits;
    } else {
      const bool mf = kind == OSCAR_INT2_MFMA;
      const int hg = mfma_heads_per_block(c->num_kv_heads);
      const int units = mf ? a->batch * ((c->num_kv_heads + hg - 1) / hg) : a->batch * c->num_kv_heads;
      const int target = mf ? kMfmaTargetBlocks : 2048;
      // bytes of one history page of one KV head
      const double rec = kind == OSCAR_HISTORY_BF16 ? 2.0 * kPage * p->D * 2
                                                    : (double)RecLayout(p->D, p->G).bytes();
      const double part_bytes = 2.0 * p->g * (p->D + 2) * 4.0;   // write + read back
      int min_pages = (int)std::ceil((mf ? 2.0 : 8.0) * part_bytes / rec);
      const int floor_pages = mf ? 8 : 16;
      min_pages = min_pages < floor_pages ? floor_pages : min_pages;
      int s_fill = (target + units - 1) / units;
      int s_cap = npages / min_pages;
      S = s_fill < s_cap ? s_fill : s_cap;
      S = S < 1 ? 1 : S;
    }
  }
  S = S > kMaxSplits ? kMaxSplits : S;
  const int pps = npages > 0 ? (npages + S - 1) / S : 0;
  if (npages > 0 && kind != OSCAR_INT2_MFMA) S = (npages + pps - 1) / pps;
  p->pages_per_split = pps;
  p->mfma_parts = S;
  p->mfma_balanced = 0;
  if (kind == OSCAR_INT2_MFMA) {
    // S parts per sequence on average; with the blocks balanced across
    // sequences one sequence may use up to 2S + 2 partial slots
    const int waves = mfma_waves(p->D, p->G, p->g == 8 ? 8 : 4, c->codebook != nullptr);
    p->mfma_balanced = a->batch > 1 && a->batch <= mfma_max_balanced(waves) &&
                       (long long)a->batch * npages < (1LL << 31);
    int cap = 2 * S + 2;
    if (p->n_shared > 0 && npages > 0) {
      // the shared pages are skipped, so the pages left can sit in a few
      // sequences (those with their own continuation): with every history at
      // the length bound, the sequence with the most pages left is covered by
      // about blocks * its pages / all pages left blocks, plus the ends
      long long left = 0, most = 0;
      for (int b = 0; b < a->batch; ++b) {
        int skip = 0;
        cascade_slots(*p, b, &skip);
        const long long own = npages - skip > 0 ? npages - skip : 0;
        left += own;
        most = own > most ? own : most;
      }
      const long long blocks = (long long)a->batch * S;
      const long long need = left > 0 ? (blocks * most + left - 1) / left + 2 : 2;
      cap = need > cap ? (int)(need < kMaxSplits ? need : kMaxSplits) : cap;
    }
    S = cap;
  }
  S += p->cas_slots;                 // the cascade's slots come first in each row
  p->splits = S;

  WsLayout &L = p->L;
  const size_t BH = (size_t)a->batch * a->num_q_heads;
  size_t off = 0;
  L.qrot = off; off = align256(off + BH * p->D * 4);
  const bool mf = p->int2_kind == OSCAR_INT2_MFMA;
  L.qpk = off;
  off = align256(off + (mf ? (size_t)a->batch * c->num_kv_heads * ((p->g + 3) / 4) *
                                 mfma_a_planes(p->D, p->G, p->g == 8 ? 8 : 4, c->codebook != nullptr) *
                                 mfma_qk_steps(p->D, p->G) *
                                 64 * 4 * 4 : 0));
  L.qhd = off; off = align256(off + (mf ? BH * 8 * 4 : 0));
  L.vgrid = off; off = align256(off + (mf && c->codebook != nullptr ? (size_t)c->num_kv_heads * 16 : 0));
  L.qcas = off; off = align256(off + (p->n_shared > 0 ? BH * 3 * p->D : 0));
  L.nslots = off; off = align256(off + (mf ? (size_t)a->batch * 4 : 0));
  L.part_o = off; off = align256(off + BH * S * p->D * 4);
  L.part_ml = off; off = align256(off + BH * S * 2 * 4);
  L.bf_o = off; off = align256(off + BH * kBf16Splits * p->D * 4);
  L.bf_ml = off; off = align256(off + BH * kBf16Splits * 2 * 4);
  L.total = off;
  L.splits = S;
  L.pages_per_split = pps;
  return OSCAR_OK;
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" {

size_t oscar_record_bytes(int32_t head_dim, int32_t group_size) {
  if (head_dim <= 0 || group_size <= 0 || head_dim % 4 || head_dim % group_size) return 0;
  return (size_t)RecLayout(head_dim, group_size).bytes();
}

const char *oscar_last_error(void) { return g_err.c_str(); }

int oscar_write_bf16(const oscar_cache *cache, int32_t n, const int32_t *dst_slot,
                     const uint16_t *k_new, const uint16_t *v_new, void *stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (n < 0) return fail(OSCAR_EINVAL, "n < 0");
  if (n == 0) return OSCAR_OK;
  if (!dst_slot || !k_new || !v_new) return fail(OSCAR_EINVAL, "NULL slot or token pointer");
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(OSCAR_EINVAL, "k_new / v_new must be 16-byte aligned");
  if (cache->num_bf16_pages <= 0) return fail(OSCAR_EINVAL, "cache has no BF16 pages");
  hipError_t e = launch_write_bf16(*cache, n, dst_slot, k_new, v_new, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "oscar_write_bf16 launch");
  return OSCAR_OK;
}

int oscar_demote_pack(const oscar_cache *cache, int32_t n, const int32_t *src_slot,
                      const int32_t *dst_slot, const float *R_k, const float *R_v,
                      const float *clip_k, const float *clip_v, void *stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (n < 0) return fail(OSCAR_EINVAL, "n < 0");
  if (n == 0) return OSCAR_OK;
  if (!src_slot || !dst_slot) return fail(OSCAR_EINVAL, "NULL slot list");
  if (!R_k || !aligned(R_k, 16)) return fail(OSCAR_EINVAL, "R_k is NULL or not 16-byte aligned");
  if (R_v && !aligned(R_v, 16)) return fail(OSCAR_EINVAL, "R_v is not 16-byte aligned");
  if (!clip_k || !clip_v) return fail(OSCAR_EINVAL, "NULL clip ratios");
  if (cache->num_bf16_pages <= 0 || cache->num_int2_pages <= 0)
    return fail(OSCAR_EINVAL, "cache needs BF16 and INT2 pages");
  hipError_t e = launch_demote(*cache, n, src_slot, dst_slot, R_k, R_v, clip_k, clip_v,
                               (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "oscar_demote_pack launch");
  return OSCAR_OK;
}

size_t oscar_decode_workspace_bytes(const oscar_cache *cache, const oscar_decode_args *args) {
  DecodeParams p{};
  if (check_args(cache, args, &p) != OSCAR_OK) return 0;
  return p.L.total;
}

int oscar_decode_plan(const oscar_cache *cache, const oscar_decode_args *args,
                      int32_t *num_splits, int32_t *pages_per_split, size_t *workspace_bytes,
                      int32_t *int2_kernel) {
  DecodeParams p{};
  int st = check_args(cache, args, &p);
  if (st) return st;
  if (num_splits) *num_splits = p.int2_kind == OSCAR_INT2_MFMA ? p.mfma_parts : p.splits;
  if (pages_per_split) *pages_per_split = p.pages_per_split;
  if (workspace_bytes) *workspace_bytes = p.L.total;
  if (int2_kernel) *int2_kernel = p.int2_kind;
  return OSCAR_OK;
}

int oscar_decode_attn(const oscar_cache *cache, const oscar_decode_args *args, const uint16_t *q,
                      const float *R_k, void *workspace, size_t workspace_bytes, void *stream) {
  DecodeParams p{};
  int st = check_args(cache, args, &p);
  if (st) return st;
  if (!q || !aligned(q, 16)) return fail(OSCAR_EINVAL, "q is NULL or not 16-byte aligned");
  if (p.int2_kind != OSCAR_HISTORY_BF16 && (!R_k || !aligned(R_k, 16)))
    return fail(OSCAR_EINVAL, "R_k is NULL or not 16-byte aligned");
  if (!workspace || !aligned(workspace, 256))
    return fail(OSCAR_EINVAL, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < p.L.total)
    return fail(OSCAR_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                p.L.total);
  p.ws = static_cast<uint8_t *>(workspace);
  hipStream_t s = (hipStream_t)stream;
  const uint32_t ph = args->phases ? args->phases : (uint32_t)OSCAR_PHASE_ALL;
  hipError_t e = hipSuccess;
  const bool bf16_hist = p.int2_kind == OSCAR_HISTORY_BF16;
  if ((ph & OSCAR_PHASE_QROT) && !bf16_hist) {
    e = launch_qrot(p, q, R_k, s);
    if (e != hipSuccess) return hip_fail(e, "q rotation launch");
  }
  if (ph & OSCAR_PHASE_BF16) {
    e = launch_bf16_seg(p, q, s);
    if (e != hipSuccess) return hip_fail(e, "BF16 segment launch");
  }
  if ((ph & OSCAR_PHASE_INT2) && args->max_hist_len > 0) {
    if (p.n_shared > 0) {
      e = launch_int2_cascade(p, s);
      if (e != hipSuccess) return hip_fail(e, "shared history pages launch");
    }
    e = bf16_hist ? launch_bf16_hist(p, q, s)
        : p.int2_kind == OSCAR_INT2_MFMA ? launch_int2_mfma(p, s) : launch_int2_valu(p, s);
    if (e != hipSuccess) return hip_fail(e, "history segment launch");
  }
  return OSCAR_OK;
}

int oscar_merge(const oscar_cache *cache, const oscar_decode_args *args, const void *workspace,
                size_t workspace_bytes, const float *R_v, float *out, float *lse, void *stream) {
  DecodeParams p{};
  int st = check_args(cache, args, &p);
  if (st) return st;
  if (!out) return fail(OSCAR_EINVAL, "out is NULL");
  if (R_v && !aligned(R_v, 16)) return fail(OSCAR_EINVAL, "R_v is not 16-byte aligned");
  if (!workspace || !aligned(workspace, 256))
    return fail(OSCAR_EINVAL, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < p.L.total)
    return fail(OSCAR_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                p.L.total);
  p.ws = static_cast<uint8_t *>(const_cast<void *>(workspace));
  if (args->max_hist_len == 0) p.splits = 0;   // no history chunk was produced
  if (p.int2_kind == OSCAR_HISTORY_BF16) R_v = nullptr;   // unrotated history
  hipError_t e = launch_merge(p, R_v, out, lse, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return OSCAR_OK;
}

}  // extern "C"

namespace oscar {
namespace {

// Host checks of a decode step's arguments other than the workspace.
int check_step(const oscar_cache *cache, const oscar_decode_args *args, DecodeParams &p,
               const int32_t *demote_src, const int32_t *demote_dst, const float *clip_k,
               const float *clip_v, const int32_t *new_slot, const uint16_t *k_new,
               const uint16_t *v_new, const uint16_t *q, const float *R_k, const float *R_v,
               float *out) {
  int st = check_args(cache, args, &p);
  if (st) return st;
  if (args->phases != 0 && args->phases != (uint32_t)OSCAR_PHASE_ALL)
    return fail(OSCAR_EINVAL, "oscar_decode_step runs every phase (phases must be 0 or ALL)");
  if (p.int2_kind == OSCAR_HISTORY_BF16)
    return fail(OSCAR_EUNSUPPORTED, "oscar_decode_step needs an INT2 history");
  if (!demote_src || !demote_dst || !new_slot) return fail(OSCAR_EINVAL, "NULL slot list");
  if (!clip_k || !clip_v) return fail(OSCAR_EINVAL, "NULL clip ratios");
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(OSCAR_EINVAL, "k_new / v_new are NULL or not 16-byte aligned");
  if (!q || !aligned(q, 16)) return fail(OSCAR_EINVAL, "q is NULL or not 16-byte aligned");
  if (!R_k || !aligned(R_k, 16)) return fail(OSCAR_EINVAL, "R_k is NULL or not 16-byte aligned");
  if (R_v && !aligned(R_v, 16)) return fail(OSCAR_EINVAL, "R_v is not 16-byte aligned");
  if (!out) return fail(OSCAR_EINVAL, "out is NULL");
  if (cache->num_bf16_pages <= 0) return fail(OSCAR_EINVAL, "cache has no BF16 pages");
  return OSCAR_OK;
}

// The three launches of a decode step (arguments checked, p.ws set).
int launch_step(DecodeParams &p, const oscar_cache *cache, const oscar_decode_args *args,
                const int32_t *demote_src, const int32_t *demote_dst, const float *clip_k,
                const float *clip_v, const int32_t *new_slot, const uint16_t *k_new,
                const uint16_t *v_new, const uint16_t *q, const float *R_k, const float *R_v,
                float *out, float *lse, hipStream_t s) {
  hipError_t e = launch_step_pre(p, *cache, q, R_k, R_v, clip_k, clip_v, demote_src, demote_dst,
                                 new_slot, k_new, v_new, s);
  if (e != hipSuccess) return hip_fail(e, "decode-step prologue launch");
  if (args->max_hist_len > 0) {
    if (p.n_shared > 0) {
      e = launch_int2_cascade(p, s);
      if (e != hipSuccess) return hip_fail(e, "shared history pages launch");
    }
    e = p.int2_kind == OSCAR_INT2_MFMA ? launch_int2_mfma(p, s) : launch_int2_valu(p, s);
    if (e != hipSuccess) return hip_fail(e, "history segment launch");
  } else {
    p.splits = 0;                               // no history chunk was produced
  }
  e = launch_merge(p, R_v, out, lse, s);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return OSCAR_OK;
}

// Device address of `scratch` on the device the work is enqueued on (the
// current device, which must be the stream's).  Looked up once per device,
// with that device current.
int scratch_address(hipStream_t s, uint8_t **out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (s != nullptr) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sd != cur)
      return fail(OSCAR_EINVAL, "stream belongs to device %d but device %d is current", (int)sd, cur);
  }
  if (cur < 0 || cur >= kMaxDevices) return fail(OSCAR_EUNSUPPORTED, "device %d out of range", cur);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[cur] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_dev[cur] = static_cast<uint8_t *>(ptr);
  }
  *out = g_scratch_dev[cur];
  return OSCAR_OK;
}

}  // namespace
}  // namespace oscar

extern "C" {

int oscar_decode_step(const oscar_cache *cache, const oscar_decode_args *args,
                      const int32_t *demote_src, const int32_t *demote_dst, const float *clip_k,
                      const float *clip_v, const int32_t *new_slot, const uint16_t *k_new,
                      const uint16_t *v_new, const uint16_t *q, const float *R_k, const float *R_v,
                      void *workspace, size_t workspace_bytes, float *out, float *lse,
                      void *stream) {
  DecodeParams p{};
  int st = check_step(cache, args, p, demote_src, demote_dst, clip_k, clip_v, new_slot, k_new,
                      v_new, q, R_k, R_v, out);
  if (st) return st;
  if (!workspace || !aligned(workspace, 256))
    return fail(OSCAR_EINVAL, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < p.L.total)
    return fail(OSCAR_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                p.L.total);
  p.ws = static_cast<uint8_t *>(workspace);
  return launch_step(p, cache, args, demote_src, demote_dst, clip_k, clip_v, new_slot, k_new,
                     v_new, q, R_k, R_v, out, lse, (hipStream_t)stream);
}

int oscar_decode_step_noalloc(const oscar_cache *cache, const oscar_decode_args *args,
                              const int32_t *demote_src, const int32_t *demote_dst,
                              const float *clip_k, const float *clip_v, const int32_t *new_slot,
                              const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                              const float *R_k, const float *R_v, float *out, float *lse,
                              void *stream) {
  DecodeParams p{};
  int st = check_step(cache, args, p, demote_src, demote_dst, clip_k, clip_v, new_slot, k_new,
                      v_new, q, R_k, R_v, out);
  if (st) return st;
  if (p.L.total > (size_t)OSCAR_NOALLOC_WORKSPACE_BYTES)
    return fail(OSCAR_EWORKSPACE, "workspace of %zu bytes exceeds the %zu-byte static workspace",
                p.L.total, (size_t)OSCAR_NOALLOC_WORKSPACE_BYTES);
  hipStream_t s = (hipStream_t)stream;
  uint8_t *ws = nullptr;
  st = scratch_address(s, &ws);
  if (st) return st;
  p.ws = ws;
  return launch_step(p, cache, args, demote_src, demote_dst, clip_k, clip_v, new_slot, k_new,
                     v_new, q, R_k, R_v, out, lse, s);
}

}  // extern "C"
