// INT2 history pages shared by several sequences, attended once for all of
// them.  In a paged cache with prefix caching, sequences that share a prompt
// prefix list the same physical pages (m.th-motor.com repost of the OSCAR
// article: the split cache works with paged KV and radix prefix caching, and
// Fig. 6 shows throughput growing with the prefix-cache hit ratio).  Reading
// such a page once per sequence repeats its unpacking and contractions for
// every sequence; here one pass over the page serves every query row of every
// sequence that shares it (rows = member sequences x q heads of the KV head).
//
// Each wave owns 32 query rows (two 16-row tiles) and walks the part's pages:
//   QK on v_mfma_i32_16x16x64_i8 with the roles of the per-sequence kernel
//     swapped: A = the page's 2-bit codes (16 tokens x 64 channels, exact
//     int8), B = one 7-bit piece of the rotated query per column (16 rows);
//     three pieces into three accumulators, recombined per value as
//     (p0 << 14) + (p1 << 7) + p2 (exact), then scale and zero point per
//     (token, group).  Output lane l holds rows 4(l/16)+v (tokens) of column
//     l % 16 (its query row).
//   PV on v_mfma_f32_16x16x16_f16 as O^T = V^T P: B = the softmax weights in
//     exactly the layout the QK result has (so no LDS transpose), A = the V
//     codes of 16 channels as the exact f16 values 1 + code/16 or 1 + code/4:
//     one rotate places tokens t and t + 8 (16 bits apart in a V word) at
//     mantissa bits 6 and 22 or 8 and 24, one AND-OR per register.  The
//     weights carry the factor 16 or 4; the "+1" part is removed with one
//     more MFMA per page against an all-ones A; the zero point adds
//     sum_t p * zero per group.
// The running max per row is lazy (raised only when a logit exceeds it by
// more than 2 in log2 units), as in the per-sequence kernel, so the f16
// weights stay below 64 * scale_v and the same V-scale limit applies.
//
// Row order inside a tile: output row r of the QK product (and k slot r of
// PV) is token 2(r/4) + {0, 8, 1, 9}[r % 4], so that the low and high halves
// of each PV register are tokens t and t + 8.
#include "common.hpp"

namespace oscar {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ v4h as_v4h2(uint32_t a, uint32_t b) {
  v4h r;
  __builtin_memcpy(&r, &a, 4);
  __builtin_memcpy(reinterpret_cast<char *>(&r) + 4, &b, 4);
  return r;
}

__device__ __forceinline__ v8h as_v8h(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v8h r;
  __builtin_memcpy(&r, &a, 4);
  __builtin_memcpy(reinterpret_cast<char *>(&r) + 4, &b, 4);
  __builtin_memcpy(reinterpret_cast<char *>(&r) + 8, &c, 4);
  __builtin_memcpy(reinterpret_cast<char *>(&r) + 12, &d, 4);
  return r;
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// NW consecutive words at byte offset `off` of a buffer resource
template <int NW>
__device__ __forceinline__ void rsrc_words(uint32_t *dst, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  if constexpr (NW == 1) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
  } else if constexpr (NW == 2) {
    const u2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    dst[0] = v.x; dst[1] = v.y;
  } else {
    static_assert(NW % 4 == 0, "1, 2 or a multiple of 4 words");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0);
      dst[4 * i] = v.x; dst[4 * i + 1] = v.y; dst[4 * i + 2] = v.z; dst[4 * i + 3] = v.w;
    }
  }
}

// token of QK output row (PV k slot) r
__device__ __forceinline__ int cas_token(int r) { return 2 * (r >> 2) + ((r & 1) ? 8 : 0) + ((r >> 1) & 1); }

}  // namespace

#ifndef OSCAR_CAS_STAGES
#define OSCAR_CAS_STAGES 2   // ring of pairs of pages: one pair in flight
#endif
#ifndef OSCAR_CAS_WAVES_PER_SIMD
#define OSCAR_CAS_WAVES_PER_SIMD 2
#endif
template <int D, int G>
__global__ __launch_bounds__(64 * kCasWaves)
__attribute__((amdgpu_waves_per_eu(OSCAR_CAS_WAVES_PER_SIMD, OSCAR_CAS_WAVES_PER_SIMD)))
void k_int2_cascade(DecodeParams p) {
  constexpr RecLayout RL(D, G);
  constexpr int NG = D / G;                  // groups per token (1 or 2)
  constexpr int NBLK = D / 64;               // 64-channel blocks (K words per token slot)
  constexpr int NSL = D / 16;                // 16-channel PV slices
  constexpr int NT = kCasRowsPerWave / 16;   // 16-row tiles per wave
  constexpr float kLazy = 2.f;               // log2 headroom of the running max
  constexpr float kOver = 2.f;               // a raised max sits this far above the logits
  // one group per token: with two (D = 128, G = 64) the doubled scale/zero
  // words and per-group accumulators no longer fit the register budget
  static_assert(G == D, "one group per token");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;

  // ---- the block's segment, page range, KV head and row group ----
  int si = 0;
  while (si + 1 < p.n_shared && (int)blockIdx.x >= p.shared[si + 1].block_base) ++si;
  const SharedSeg sg = p.shared[si];
  const int local = (int)blockIdx.x - sg.block_base;
  const int part = local % sg.parts;
  const int j = (local / sg.parts) % p.Hkv;
  const int rgi = local / (sg.parts * p.Hkv);
  const int pb = sg.first + (int)((long long)sg.num * part / sg.parts);
  const int pe = sg.first + (int)((long long)sg.num * (part + 1) / sg.parts);
  const int rows = sg.nseq * p.g;
  const int row0 = rgi * kCasRowsPerBlock + w * kCasRowsPerWave;
  if (row0 >= rows) return;                  // a wave with no rows (no barriers below)
  const int S = p.splits;

  // ---- per tile: this lane's query row (column l % 16) ----
  // B operands (16 piece bytes of the row per piece and 64-channel block) are
  // kept in LDS, each lane reading back only its own 16 bytes: registers go to
  // the page ring and the PV accumulators
  __shared__ v4i qlds[kCasWaves][NT][3][NBLK][64];
  float qsc[NT], qz[NT][NG];                 // 2^-qe * sm_scale * log2(e); group sums
  // the (sequence, q head) of tile t's row of this lane, and whether it exists
  auto row_of = [&](int t, int &b, size_t &bh) {
    const int row = row0 + 16 * t + r16;
    const bool ok = row < rows;
    const int m = ok ? row / p.g : 0, hh = ok ? row % p.g : 0;
    b = sg.seq0 + m;
    int h = p.q_of_kv[j * p.g];
    for (int k = 1; k < p.g; ++k) h = hh == k ? p.q_of_kv[j * p.g + k] : h;
    bh = (size_t)b * p.Hq + h;
    return ok;
  };
  bool rv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int b;
    size_t bh;
    rv[t] = row_of(t, b, bh);
    const int8_t *qc = reinterpret_cast<const int8_t *>(p.ws + p.L.qcas) + bh * 3 * D;
#pragma unroll
    for (int pc = 0; pc < 3; ++pc)
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
        qlds[w][t][pc][blk][lane] = rv[t] ? *reinterpret_cast<const v4i *>(qc + pc * D + 64 * blk + 16 * g4)
                                          : v4i{0, 0, 0, 0};
    const float *hd = reinterpret_cast<const float *>(p.ws + p.L.qhd) + bh * 8;
    qsc[t] = rv[t] ? ldexpf(1.f, -__float_as_int(hd[0])) * p.sm_log2 : 0.f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) qz[t][gg] = rv[t] ? hd[1 + gg] : 0.f;
  }

  // ---- page ring ----
  struct Stage {
    uint32_t kw[NBLK];                       // K words of token cas_token(r16), part g4
    uint32_t vw[NSL];                        // V words of channels r16 + 16 * sl
    uint32_t sz[8 * NG];                     // (scale, zero) words of tokens 2g4, 2g4+1, 2g4+8, 2g4+9
    int ok;
  };
  using cint32 = const __attribute__((address_space(4))) int32_t;
  cint32 *ptab = (cint32 *)(p.hist_pages + (size_t)sg.seq0 * p.hist_stride);
  const size_t rec_stride = (size_t)p.Hkv * RL.bytes();
  const uint8_t *pool_j = p.int2_pool + (size_t)j * RL.bytes();
  const int npool = p.num_int2_pages < 0x7fffffff ? (int)p.num_int2_pages : 0x7fffffff;
  const uint32_t off_k = (uint32_t)RL.kword(16 * g4 + cas_token(r16), 0);
  const uint32_t off_sz0 = (uint32_t)RL.tok_sz(2 * g4), off_sz1 = (uint32_t)RL.tok_sz(2 * g4 + 8);

  // The waves of a block read the same pages; each starts a quarter of the
  // range further on (the softmax does not depend on the order), so that
  // every wave leads the HBM reads of its own quarter and the others find
  // those pages in the L2 or the last-level cache: four times the distinct
  // pages in flight per block.
  const int npg = pe - pb;
  const int shift = npg > 0 ? (int)((long long)npg * w / kCasWaves) : 0;
  // page table entries in this wave's order, 64 positions per register:
  // lane l of chunk c holds the physical page of position 64 c + l (a
  // position past the range: the wave's first page).  The next chunk is
  // loaded while the current one is used; pages are picked by readlane
  auto ptab_chunk = [&](int c) -> int {
    const int i = 64 * c + lane;
    int k = (i < npg ? i : 0) + shift;
    k = pb + (k >= npg ? k - npg : k);
    return ptab[k];
  };
  int pt_cur = 0, pt_next = 0;
  if (npg > 0) {
    pt_cur = ptab_chunk(0);
    pt_next = npg > 64 ? ptab_chunk(1) : 0;
  }
  auto issue = [&](Stage &sgi, int i) {      // i: position in this wave's order (uniform)
    // a position past the range (the second page of a last, odd pair) loads
    // the wave's first page again and is marked empty: its weights are 0,
    // and the values they multiply are those of a written record
    if ((i & 63) == 0 && i > 0) {            // uniform: the next chunk of the table
      pt_cur = pt_next;
      if (i + 64 < npg) pt_next = ptab_chunk((i >> 6) + 1);
    }
    const bool inr = i < npg;
    const int phys = __builtin_amdgcn_readlane(pt_cur, i & 63);
    const bool valid = phys >= 0 && phys < npool;
    OSCAR_DCHECK(valid, p.status);
    sgi.ok = inr && valid;
    const uint8_t *rec = pool_j + (valid ? (size_t)phys : 0) * rec_stride;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(rec), (short)0, RL.bytes(), 0x00020000);
    rsrc_words<NBLK>(sgi.kw, rs, off_k);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint32_t tmp[NBLK];
      rsrc_words<NBLK>(tmp, rs, (uint32_t)RL.vword(r16 + 16 * q4, 0));
#pragma unroll
      for (int h2 = 0; h2 < NBLK; ++h2) sgi.vw[q4 + 4 * h2] = tmp[h2];
    }
    rsrc_words<4 * NG>(sgi.sz, rs, off_sz0);
    rsrc_words<4 * NG>(sgi.sz + 4 * NG, rs, off_sz1);
  };

  // running state per tile (the lane's row): m_run the row's running max,
  // set exactly by the first pair of pages and raised lazily after that;
  // lsum and zacc the lane's partial sums of p and p * zero_v; acc the PV
  // accumulators (channels 16 sl + 4 g4 + i), corr the sum of the PV weights
  float m_run[NT], lsum[NT], zacc[NT];
  v4f acc[NT][NSL], corr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = 0.f;
    lsum[t] = 0.f;
    zacc[t] = 0.f;
    corr[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) acc[t][sl] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  bool started = false;                      // m_run holds a row maximum (uniform)
  const uint32_t rot = (uint32_t)(4 * g4 - 6) & 31u;   // token 2g4 of a V word to bit 6
  uint32_t f16one, mlo, mhi;
  asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(f16one));
  asm volatile("s_mov_b32 %0, 0xc000c0" : "=s"(mlo));
  asm volatile("s_mov_b32 %0, 0x3000300" : "=s"(mhi));
  const v8h ones = as_v8h(f16one, f16one, f16one, f16one);
  // sz word of value v (tokens 2g4, 2g4+8, 2g4+1, 2g4+9): K (scale, zero),
  // then V; the PV factor of value v (mantissa bit 6 or 8 of its code)
  constexpr int kSzBase[4] = {0, 4, 2, 6};
  constexpr float kPvf[4] = {16.f, 16.f, 4.f, 4.f};

  // A pair of pages per step: the PV contraction takes the 32 tokens of both
  // in one v_mfma_f32_16x16x32_f16 (k slots 8 g4 .. 8 g4 + 3: the lane's 4
  // tokens of page a, 8 g4 + 4 .. 8 g4 + 7: of page b; the A and B operands
  // of a lane list the same tokens in the same order).  Logits are kept
  // relative to the running max: s' = dot * (k_scale * qsc) + (k_zero * qz - m).
  auto process = [&](Stage &sa, Stage &sb) {
    if (!sa.ok && !sb.ok) return;
    float sv[2][NT][4];                      // relative logits, -inf for an empty page
    float vsf[2][4], vz[2][4];               // V scale * PV factor, V zero per value
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      Stage &sgi = pg ? sb : sa;
      const float empty = sgi.ok ? 0.f : -INFINITY;   // uniform
      float ks[4], kz[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t kw = sgi.sz[kSzBase[v]], vw = sgi.sz[kSzBase[v] + 1];
        ks[v] = bf16_lo(kw);
        kz[v] = bf16_hi(kw);
        vsf[pg][v] = bf16_lo(vw) * kPvf[v];
        vz[pg][v] = bf16_hi(vw);
      }
      // QK A operands: the codes as bytes (byte j of dword i = channel
      // 4j + i of the lane's 16 channels)
      v4i kb[NBLK];
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        const uint32_t e = sgi.kw[blk];
        kb[blk] = v4i{(int)(e & 0x03030303u), (int)((e >> 2) & 0x03030303u),
                      (int)((e >> 4) & 0x03030303u), (int)((e >> 6) & 0x03030303u)};
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        v4i qa[3];
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
          qa[pc] = v4i{0, 0, 0, 0};
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk)
            qa[pc] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb[blk], qlds[w][t][pc][blk][lane], qa[pc], 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          int dhi = (qa[0][v] << 7) + qa[1][v];
          asm volatile("" : "+v"(dhi));
          const float dot = (float)((dhi << 7) + qa[2][v]);
          sv[pg][t][v] = fmaf(dot, ks[v] * qsc[t], fmaf(kz[v], qz[t][0], empty - m_run[t]));
        }
      }
    }

    // ---- lazy running max, per tile: raised when a logit of the tile's
    // rows exceeds it by more than kLazy (log2 units), and set on the first
    // pair; a raised row max is placed kOver above the new maximum, so that
    // the next raise needs a rise of more than kLazy + kOver ----
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float mx = fmaxf(fmaxf(fmaxf(sv[0][t][0], sv[0][t][1]), fmaxf(sv[0][t][2], sv[0][t][3])),
                       fmaxf(fmaxf(sv[1][t][0], sv[1][t][1]), fmaxf(sv[1][t][2], sv[1][t][3])));
      if (__builtin_expect(!started || __any(mx > kLazy), 0)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // the rise of the row max (the first pair: the max itself)
        const float delta = !started ? mx + kOver : (mx > kLazy ? mx + kOver : 0.f);
        const float alpha = started ? __builtin_amdgcn_exp2f(-delta) : 0.f;
        m_run[t] += delta;
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int v = 0; v < 4; ++v) sv[pg][t][v] -= delta;
        lsum[t] *= alpha;
        zacc[t] *= alpha;
        corr[t] *= alpha;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) acc[t][sl] *= alpha;
      }
    }
    started = true;
    // weights (<= 4; 0 for a missing page) and the PV B operands
    // p * scale_v * (16 or 4) in f16, page a then page b
    v8h pbv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float pr[2][4];
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pr[pg][v] = __builtin_amdgcn_exp2f(sv[pg][t][v]);
          lsum[t] += pr[pg][v];
          zacc[t] = fmaf(pr[pg][v], vz[pg][v], zacc[t]);
        }
      pbv[t] = as_v8h(pack_f16(pr[0][0] * vsf[0][0], pr[0][1] * vsf[0][1]),
                      pack_f16(pr[0][2] * vsf[0][2], pr[0][3] * vsf[0][3]),
                      pack_f16(pr[1][0] * vsf[1][0], pr[1][1] * vsf[1][1]),
                      pack_f16(pr[1][2] * vsf[1][2], pr[1][3] * vsf[1][3]));
      corr[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pbv[t], corr[t], 0, 0, 0);
    }
    // ---- PV: A = V codes of channel r16 + 16 sl, tokens (2g4, 2g4+8 | 2g4+1,
    // 2g4+9) of page a, then of page b ----
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const uint32_t xa = __builtin_amdgcn_alignbit(sa.vw[sl], sa.vw[sl], rot);
      const uint32_t xb = __builtin_amdgcn_alignbit(sb.vw[sl], sb.vw[sl], rot);
      const v8h av = as_v8h((xa & mlo) | f16one, (xa & mhi) | f16one, (xb & mlo) | f16one,
                            (xb & mhi) | f16one);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t][sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbv[t], acc[t][sl], 0, 0, 0);
    }
  };

  // ring of NSP pairs of pages (NSP - 1 pairs in flight)
  constexpr int NSP = OSCAR_CAS_STAGES;
  Stage st[NSP][2];
  const int npair = (npg + 1) / 2;
  if (npair > 0) {
#pragma unroll
    for (int i = 0; i < NSP - 1; ++i) {
      issue(st[i][0], 2 * i);
      issue(st[i][1], 2 * i + 1);
    }
    for (int i0 = 0; i0 < npair; i0 += NSP) {
#pragma unroll
      for (int s2 = 0; s2 < NSP; ++s2) {
        const int nx = i0 + s2 + NSP - 1;
        issue(st[(s2 + NSP - 1) % NSP][0], 2 * nx);
        issue(st[(s2 + NSP - 1) % NSP][1], 2 * nx + 1);
        if (i0 + s2 < npair) process(st[s2][0], st[s2][1]);
      }
    }
  }

  // ---- partials: (max, sum, output) per (row, part) ----
  float *po = reinterpret_cast<float *>(p.ws + p.L.part_o);
  float *pml = reinterpret_cast<float *>(p.ws + p.L.part_ml);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float L = lsum[t];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    float Z = zacc[t];
    Z += __shfl_xor(Z, 16);
    Z += __shfl_xor(Z, 32);
    int b;
    size_t bh;
    if (!row_of(t, b, bh)) continue;
    // this part's slot: after the parts of the sequence's earlier segments
    int slot = part;
    for (int i = 0; i < p.n_shared; ++i) {
      const SharedSeg &o = p.shared[i];
      if (b >= o.seq0 && b < o.seq0 + o.nseq && o.first < sg.first) slot += o.parts;
    }
    const size_t prow = bh * S + slot;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const v4f o = acc[t][sl] - corr[t] + Z;
      *reinterpret_cast<v4f *>(po + prow * D + 16 * sl + 4 * g4) = o;
    }
    if (g4 == 0) {
      pml[prow * 2 + 0] = m_run[t];
      pml[prow * 2 + 1] = L;
    }
  }
}

hipError_t launch_int2_cascade(const DecodeParams &p, hipStream_t s) {
  if (p.n_shared <= 0 || p.cas_blocks <= 0) return hipSuccess;
  const dim3 grid(p.cas_blocks), blk(64 * kCasWaves);
  if (p.D == 64 && p.G == 64) hipLaunchKernelGGL((k_int2_cascade<64, 64>), grid, blk, 0, s, p);
  else if (p.D == 128 && p.G == 128) hipLaunchKernelGGL((k_int2_cascade<128, 128>), grid, blk, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace oscar
