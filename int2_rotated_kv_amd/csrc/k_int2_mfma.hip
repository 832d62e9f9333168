// INT2 history segment on the matrix cores (m.th-motor.com repost of the OSCAR
// article, decode stage: the INT2 kernel unpacks the 2-bit codes, restores
// scale/zero point and accumulates in floating point).
//
// The history is stored as per-token, per-group asymmetric codes:
//   x_hat[t, c] = code[t, c] * scale[t, g(c)] + zero[t, g(c)],  code in {0..3}.
// Both contractions of decode attention are split so that the 2-bit codes
// enter a matrix instruction unchanged and the per-(token, group) scale/zero
// are applied to its small outputs:
//
//   logits  s[h, t] = sum_g scale[t,g] * (q_h . code_t)_g + sum_g zero[t,g] * Q[h,g]
//     (q_h . code_t)_g on v_mfma_i32_16x16x64_i8: B = codes (exact int8), A = the
//     rotated query as a 21-bit integer split into three 7-bit pieces, one per
//     A row; the three int32 results recombine exactly as p0*2^14 + p1*2^7 + p2.
//   values  o[h, c] = sum_t w[h,t,g(c)] * code[t,c] + sum_t p[h,t] * zero[t,g(c)],
//           w = p * scale_v
//     sum_t w * code on v_mfma_f32_4x4x4_16b_f16 (16 blocks of 4 heads x 4
//     channels x 4 tokens, so lane l owns channels l, l+64): B = codes as the
//     exact f16 values 1 + code * 2^(b-10), the code masked into mantissa bit
//     b in {4, 6, 8} of its half straight from the packed word or one of two
//     shifted copies; A = w * 2^(8-b) in f16, so A * B = A + w * code / 4;
//     fp32 accumulation; the A part is removed with sum_t A (same f16 values).
//
// One block of 16 waves (8 for the instances that need more than 128
// registers per wave, see mfma_waves) covers 2 KV heads (half the waves per
// head each) and an equal share of the batch's history pages (one or more segments, see the
// schedule below); the waves of a head take fixed, interleaved batches of 4
// consecutive pages of a segment (a wave that falls behind its head's others
// raises its issue priority, since the SIMD arbiter favours older waves), and
// the block combines them in wave order into one partial per (q head,
// segment): outputs are bitwise the same on every run.  Each wave keeps 3
// pages in flight in a register ring.  The query operands (A words,
// exponents, group sums) come from the workspace, written by the q rotation.  The running max
// per head is lazy: it is raised (16-lane DPP reductions, rescale of the
// partial sums) only when a logit exceeds it by more than 2 (log2 units), so
// unnormalised weights stay below 4.  Serves 1, 2, 4 or 8 q heads per KV head
// (with fewer than 4 a head quad is partly empty: zero A rows, unused
// accumulator heads) and needs V group scales below 1024 (A = w * 16 must stay
// in f16 range).
#include "common.hpp"

namespace oscar {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

// 16-lane (DPP row) reductions; every lane of the row receives the result.
// Operands are finite or -inf, so no NaN canonicalisation is needed; the
// s_nop covers the VALU-write -> DPP-read hazard.
__device__ __forceinline__ float row_max(float x) {
  asm volatile(
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf"
      : "+v"(x));
  return x;
}
// max of two floats that are finite or -inf (no NaN handling needed)
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float row_sum(float x) {
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf"
      : "+v"(x));
  return x;
}

__device__ __forceinline__ v4h as_v4h(uint32_t a, uint32_t b) {
  v4h r;
  __builtin_memcpy(&r, &a, 4);
  __builtin_memcpy(reinterpret_cast<char *>(&r) + 4, &b, 4);
  return r;
}

// k-slot order shared by the PV operands: token pair u = 0..7 is (u, u + 8),
// held by the two f16 halves of one B register; MFMA ti takes pairs 2ti and
// 2ti + 1, so token t sits in A slot 2 * (t % 8) + t / 8.
__device__ __forceinline__ int pv_slot(int t) { return 2 * (t & 7) + (t >> 3); }
// mantissa bit b of token pair u in its B register (x1 = v << 4, x0 = v,
// x2 = v >> 6): u = 0, 1, 2 from x1 at 4, 6, 8; u = 3, 4 from x0 at 6, 8;
// u = 5, 6, 7 from x2 at 4, 6, 8.  A carries the factor 2^(8 - b).
__device__ __forceinline__ float pv_factor(int t) {
  const int u = t & 7;
  return (u == 0 || u == 5) ? 16.f : (u == 1 || u == 3 || u == 6) ? 4.f : 1.f;
}

template <int NW>
__device__ __forceinline__ void load_words(uint32_t (&dst)[NW], const uint32_t *src) {
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4 *>(src)[i];
      dst[4 * i] = v.x; dst[4 * i + 1] = v.y; dst[4 * i + 2] = v.z; dst[4 * i + 3] = v.w;
    }
  } else if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(src);
    dst[0] = v.x; dst[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) dst[i] = src[i];
  }
}

// NW consecutive words at byte offset `off` of a buffer resource (16- or
// 8-byte loads); the resource's base and bounds live in scalar registers, so
// a wave-uniform base costs no vector instructions
template <int NW>
__device__ __forceinline__ void buf_words(uint32_t (&dst)[NW], __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0);
      dst[4 * i] = v.x; dst[4 * i + 1] = v.y; dst[4 * i + 2] = v.z; dst[4 * i + 3] = v.w;
    }
  } else {
    static_assert(NW == 2, "2 or a multiple of 4 words");
    const u2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    dst[0] = v.x; dst[1] = v.y;
  }
}

}  // namespace


constexpr int kPidCap = 1024;                   // page ids of a segment staged in LDS

// LDS of the matrix-core kernel (HB waves per block)
template <int D, int G, int GQ, int HB>
struct Int2Shared {
  int cum[64 * HB + 1];                           // work units before sequence b
  int pst[64 * HB];                               // unit where sequence b's pages start
  int wsum[HB];
  int batch_ctr[8];                               // per head: batches its waves started
  int pid_lds[kPidCap];
  float qf_all[HB][GQ][D];                        // per wave: its partial outputs at the end
  // per wave: the PV weights w[grp][head][slot]
  __align__(16) _Float16 wbuf_all[HB][D / G][GQ][16];
  float mlw[HB][GQ][2];
};
template <int D, int G, int GQ, bool CB, int HB>
__global__ __launch_bounds__(64 * HB) void k_int2_mfma(DecodeParams p) {
  constexpr RecLayout RL(D, G);
  constexpr int NG = D / G;            // groups per token
  constexpr int NBLK = D / 64;         // 64-channel blocks (one int8 MFMA K each)
  constexpr int GPB = G < 64 ? 64 / G : 1;   // groups inside one 64-channel block
  constexpr int NQK = NBLK * GPB;      // QK MFMAs per head quad per page
  constexpr int NH = D / 64;           // 64-channel halves of PV (lane owns l + 64*h2)
  constexpr int NQ = GQ / 4;           // head quads
  static_assert(GQ == 4 || GQ == 8, "one or two head quads (1, 2 or 4 q heads use one)");

  constexpr int NP = CB ? 3 : 1;       // QK code planes: the codes; with a codebook also b0, b0&b1
  constexpr bool kPermPlanes = CB;    // the b0 and b0&b1 planes looked up from the code bytes
  constexpr int NPA = mfma_a_planes(D, G, GQ, CB);   // query A operand sets
  constexpr bool kSepAcc = NP > NPA;  // planes in accumulators of their own, weighted here
  __shared__ Int2Shared<D, G, GQ, HB> lds;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave (uniform)
  // block = (group of HG KV heads, block index within the group); WH waves
  // per head share the block's pages and their results are combined into one
  // partial per (q head, segment)
  const int HG = mfma_heads_per_block(p.Hkv);
  const int WH = HB / HG;
  const int S = p.splits;                         // partial slots per (sequence, q head)
  const int S_reg = S - p.cas_slots;              // of them this kernel's (after the cascade's)
  const int ngrp = (p.Hkv + HG - 1) / HG;
  const int NBT = gridDim.x / ngrp;               // blocks per head group
  const int hg = blockIdx.x / NBT;
  const int ib = blockIdx.x % NBT;
  const int P = NBT / p.B;                        // parts per sequence when not balanced
  // waves 4k .. 4k+3 sit in issue slot k of the CU's four SIMDs, and the
  // arbiter favours lower slots; with at most 4 heads per block, wave w
  // serving head w % HG puts every head's waves in every issue slot
  const int jl = w % HG;                          // head within the group
  const bool live = hg * HG + jl < p.Hkv;         // a last group may be short
  const int j = live ? hg * HG + jl : 0;          // this wave's KV head
  const int r16 = lane & 15, kb = lane >> 4;      // row-in-16 and lane group

  // Lloyd-Max codebook.  QK: the level of code c = b0 + 2*b1 is
  //   L[c] = L0 + cA*c + cB*b0 + cC*b0*b1,
  //   cA = (L2 - L0)/2, cB = (L1 - L0) - cA, cC = L3 - L2 - L1 + L0,
  // so the int8 contraction runs on the codes (as without a codebook) and on
  // the b0 and b0&b1 bit planes, and the L0 part joins the zero point.  The
  // planes go into one accumulator, the A operand of each holding the pieces
  // of the query times the plane's weight (formed with the q rotation);
  // where three A sets would not fit the registers (mfma_a_planes) each
  // plane has its own accumulator, weighted by cA, cB, cC here.  PV: the V
  // levels are written as
  //   L[c] = vL0 + vbeta * h[c],  h[c] integers in [-2048, 2048] (exact in
  // f16), vbeta = (Lmax - Lmin) / H with H in [2048, 4095] and vL0 = Lmin +
  // (2048 - phi) * vbeta with phi in [0, 1), Lmin and Lmax the smallest and
  // largest level: the common shift phi brings the four values
  // H (L[c] - Lmin) / (Lmax - Lmin) + phi as close to integers as it can,
  // and H is the one of its 2048 values with the smallest resulting error
  // (formed once per KV head with the q rotation and read from the
  // workspace; see v_grid_words).  Then |L[c] - vL0 - vbeta h[c]| is
  // typically ~2e-6 of Lmax - Lmin (over random level sets: 99th percentile
  // 1e-5, worst seen 6e-5), where rounding the levels to f16 errs by up to
  // 2^-11 of |L[c]|.  Each code's h is looked up
  // by byte permutes from a table of the 4 (low bytes in one word, high
  // bytes in another), PV runs once on them with the weights p * scale_v,
  // and the vL0 part joins the zero point.  Four equal levels take h = 0
  // (exact); non-finite levels take h = the levels rounded to f16, vL0 = 0,
  // vbeta = 1.  Without a codebook no plane is formed.
  float kcA = 1.f, kcB = 0.f, kcC = 0.f, kL0 = 0.f;   // K levels
  uint32_t vtab_lo = 0, vtab_hi = 0;                 // h[c] in f16: low, high bytes
  float vL0 = 0.f, vbeta = 1.f;                      // V levels = vL0 + vbeta * h[c]
  if constexpr (CB) {
    const float *lk = p.codebook + j * 8;
    kL0 = lk[0];
    kcA = 0.5f * (lk[2] - lk[0]);
    kcB = (lk[1] - lk[0]) - kcA;
    kcC = ((lk[3] - lk[2]) - lk[1]) + lk[0];
    // the V grid of this KV head, formed with the q rotation (scalar loads)
    using cu32 = const __attribute__((address_space(4))) uint32_t;
    cu32 *vg = (cu32 *)(p.ws + p.L.vgrid) + j * 4;
    vtab_lo = vg[0];
    vtab_hi = vg[1];
    vL0 = __uint_as_float(vg[2]);
    vbeta = __uint_as_float(vg[3]);
  }
  // a symmetric K codebook (L3 - L2 = L1 - L0, as a Lloyd-Max fit of a
  // symmetric distribution gives) has no b0&b1 term: its QK plane is
  // skipped, which leaves every result bitwise the same (its coefficient is
  // 0); the test is uniform over the wave (one KV head)
  const bool plane2 = CB && kcC != 0.f;

  // ---------------- schedule: this block's segments ----------------
  // The histories of the batch laid end to end, each sequence counted as its
  // pages plus kSegCost units for the fixed cost of a segment (query operands,
  // page ids, the combine and the partial's stores), hold T units; block ib
  // of its head group covers units [T*ib/NB, T*(ib+1)/NB) with
  // NB = min(NBT, T/16) blocks at work, so blocks get about equal work
  // whatever the sequence lengths (a block does not collect the fixed costs
  // of many short sequences).  A range that crosses a sequence boundary is
  // handled as one segment per sequence, each writing its own partial slot:
  // the index of the block among the blocks that cover that sequence's pages.
  // If some sequence would need more than S slots (lengths far from equal),
  // or the batch is larger than the block, every block instead takes one of P
  // equal parts of one sequence (slot = part).
  auto clamp_len = [&](int v) {
    OSCAR_DCHECK(v >= 0 && v <= p.max_hist_len && v <= kPage * p.hist_stride, p.status);
    v = v < 0 ? 0 : v;
    v = v > p.max_hist_len ? p.max_hist_len : v;
    return v > kPage * p.hist_stride ? kPage * p.hist_stride : v;
  };
  // pages of sequence b this kernel reads: those after its shared pages,
  // which the cascade kernel attends (with none shared: all of them)
  auto own_pages = [&](int b, int *skip) {
    const int hlb = clamp_len(p.hist_len[b]);
    const int npg = (hlb + kPage - 1) / kPage;
    int sk = 0;
    if (p.n_shared > 0) cascade_slots(p, b, &sk);
    // the cascade attends every shared page whole for each member, so a
    // member's history must cover them
    OSCAR_DCHECK(sk * kPage <= hlb, p.status);
    sk = sk < npg ? sk : npg;
    *skip = sk;
    return npg - sk;
  };
  constexpr int kSegCost = 128;                   // units of a segment's fixed cost
  auto &cum = lds.cum;                            // units before sequence b
  auto &pst = lds.pst;                            // unit of sequence b's first page
  auto &wsum = lds.wsum;
  const bool scan = p.mfma_balanced != 0;         // B <= 64 * HB and no overflow
  int T = 0, NB = 1;
  bool balanced = false;
  if (scan) {
    const int t = threadIdx.x;
    int skip_t = 0;
    const int v = t < p.B ? own_pages(t, &skip_t) : 0;
    const int wv = v > 0 ? v + kSegCost : 0;      // work units of sequence t
    int x = wv;                                   // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int before = 0;
    for (int k = 0; k < w; ++k) before += wsum[k];
    if (t < p.B) {
      cum[t] = before + x - wv;
      pst[t] = before + x - v;                    // the pages are the sequence's last units
    }
    if (t == p.B - 1) cum[p.B] = before + x;
    __syncthreads();
    T = cum[p.B];
    NB = T / 16 < NBT ? T / 16 : NBT;
    NB = NB < 1 ? 1 : NB;
    // the block holding unit u: the largest i with T*i/NB <= u; the blocks
    // covering sequence t's pages: those holding units pst .. pst + v - 1
    bool bad = false;
    int first = 0, last = -1;
    if (t < p.B && v > 0 && T > 0) {
      first = (int)(((long long)(pst[t] + 1) * NB - 1) / T);
      last = (int)(((long long)(pst[t] + v) * NB - 1) / T);
      bad = last - first + 1 > S_reg;
    }
    balanced = T > 0 && !__syncthreads_or(bad);
    // the merge reads each sequence's slot count
    if (hg == 0 && ib == 0 && t < p.B) reinterpret_cast<int *>(p.ws + p.L.nslots)[t] = balanced ? last - first + 1 : P;
  }
  const long long g0 = balanced && ib < NB ? (long long)T * ib / NB : 0;
  const long long g1 = balanced && ib < NB ? (long long)T * (ib + 1) / NB : 0;
  int bseg = 0;                                   // next sequence to look at
  if (balanced) {
    int lo = 0, hi = p.B - 1;                     // last b with cum[b] <= g0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    bseg = lo;
  } else {
    bseg = ib / (P > 0 ? P : 1);
  }
  bool fallback_done = false;

  // page ids (the first kPidCap of a segment) are staged in LDS, so a batch's
  // ids are an LDS read away rather than a scalar-cache miss
  auto &batch_ctr = lds.batch_ctr;             // per head: batches its waves started
  auto &pid_lds = lds.pid_lds;
  auto &qf_all = lds.qf_all;                   // per wave: its partial outputs at the end
  auto &wbuf_all = lds.wbuf_all;               // per wave: w[grp][head][slot]
  auto &mlw = lds.mlw;

  // the query operands (prepared with the q rotation), requested as soon as
  // a segment's sequence is known, before its length and page ids: A words of
  // the wave's head quads, and per q head its exponent and group sums
  // (wave-uniform scalar loads)
  v4i aq[NQ][NPA][NQK];
  int qe_h[GQ];
  float qz_h[GQ][NG];
  auto load_query = [&](int b) {
    const v4i *qpk = reinterpret_cast<const v4i *>(p.ws + p.L.qpk) +
                     ((size_t)b * p.Hkv + j) * NQ * NPA * NQK * 64 + lane;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
      for (int pl = 0; pl < NPA; ++pl)
#pragma unroll
        for (int m = 0; m < NQK; ++m) aq[qd][pl][m] = qpk[((qd * NPA + pl) * NQK + m) * 64];
    using cf32 = const __attribute__((address_space(4))) float;
    cf32 *qhd = (cf32 *)(p.ws + p.L.qhd);
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      // with fewer than GQ q heads per KV head the missing heads' A rows are
      // zero; their per-head constants are taken from head 0 and never used
      cf32 *hd = qhd + ((size_t)b * p.Hq + p.q_of_kv[j * p.g + (h < p.g ? h : 0)]) * 8;
      qe_h[h] = __float_as_int(hd[0]);
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) qz_h[h][g2] = hd[1 + g2];
    }
  };

  for (;;) {
  // ---------------- next segment: sequence b, its pages [pbeg, pend) ----------------
  int b, pbeg, pend_all, slot;
  if (balanced) {
    // skip sequences whose pages [pst, cum[b + 1]) miss [g0, g1)
    while (bseg < p.B && cum[bseg] < g1 &&
           (cum[bseg + 1] < g1 ? cum[bseg + 1] : g1) <= (pst[bseg] > g0 ? pst[bseg] : g0))
      ++bseg;
    if (bseg >= p.B || ib >= NB || cum[bseg] >= g1) break;
    b = bseg++;
    load_query(b);
    const long long lo = pst[b] > g0 ? pst[b] : g0;
    const long long hi = cum[b + 1] < g1 ? cum[b + 1] : g1;
    pbeg = (int)(lo - pst[b]);
    pend_all = (int)(hi - pst[b]);
    slot = ib - (int)(((long long)(pst[b] + 1) * NB - 1) / T);
  } else {
    if (fallback_done || bseg >= p.B || P == 0) break;
    fallback_done = true;
    b = bseg;
    load_query(b);
    const int part = ib % P;
    int sk;
    const int npg = own_pages(b, &sk);
    pbeg = (int)((long long)npg * part / P);
    pend_all = (int)((long long)npg * (part + 1) / P);
    slot = part;
  }
  {
    // past the sequence's shared pages; its cascade slots come first
    int sk = 0;
    const int ncas = p.n_shared > 0 ? cascade_slots(p, b, &sk) : 0;
    if (ncas > 0) {
      const int npg = (clamp_len(p.hist_len[b]) + kPage - 1) / kPage;
      sk = sk < npg ? sk : npg;
      pbeg += sk;
      pend_all += sk;
      slot += ncas;
    }
  }
  const int hl = clamp_len(p.hist_len[b]);
  const int pend = live ? pend_all : pbeg;        // no pages for a wave without a head
  {
    const int n = pend_all - pbeg < kPidCap ? pend_all - pbeg : kPidCap;
    const int32_t *tab = p.hist_pages + (size_t)b * p.hist_stride + pbeg;
    for (int i = threadIdx.x; i < n; i += 64 * HB) pid_lds[i] = tab[i];
  }

  // ---------------- page loop: register ring of NS pages ----------------
  // stage data of one page for this lane: K words of token r16 / lane group kb,
  // K and V (scale, zero) words of token r16, and the V words of channels
  // lane + 64*h2 (adjacent in the record).
#ifndef OSCAR_INT2_STAGES
#define OSCAR_INT2_STAGES 4
#endif
#ifndef OSCAR_INT2_BATCH
#define OSCAR_INT2_BATCH 4
#endif
  constexpr int NS = OSCAR_INT2_STAGES;   // pages in the register ring (NS-1 in flight)
  constexpr int NB = OSCAR_INT2_BATCH;    // pages per batch of a wave
  static_assert(NS % NB == 0, "the ring holds whole batches");
  constexpr int SW = D / 32;             // words of a lane slot: NBLK K words, NH V words
  struct Stage {
    uint32_t c[SW];                      // K words of (token r16, part kb), V words of channels lane + 64*h2
    uint32_t sz[2 * NG];                 // token r16: K (scale, zero) per group, then V
    int ok;
  };
  Stage st[NS];
  // page ids past the staged ones through the constant address space:
  // wave-uniform scalar loads, counted apart from the vector loads so reading
  // one never drains the ring
  using cint32 = const __attribute__((address_space(4))) int32_t;
  cint32 *ptab = (cint32 *)(p.hist_pages + (size_t)b * p.hist_stride);
  const uint32_t rec_stride = (uint32_t)p.Hkv * (uint32_t)RL.bytes();   // bytes per page
  const uint8_t *pool_j = p.int2_pool + (size_t)j * RL.bytes();

  // per-lane byte offsets inside a record: lane slot `lane` (= 16*kb + r16)
  // and token slot r16
  const uint32_t off_c = (uint32_t)RL.kword(lane, 0);
  const uint32_t off_sz = (uint32_t)RL.tok_sz(r16);
  const int npool = p.num_int2_pages < 0x7fffffff ? (int)p.num_int2_pages : 0x7fffffff;

  // page id of history page k in [pbeg, pend) (wave-uniform; the callers
  // ask only for the pages of a wave's positions)
  auto page_id = [&](int k) -> int {
    const int i = k - pbeg;
    const int id = i < kPidCap ? __builtin_amdgcn_readfirstlane(pid_lds[i]) : ptab[k];
    OSCAR_DCHECK(id >= 0 && id < npool, p.status);
    return id;
  };
  // the same from the table itself (before the ids are staged)
  auto table_id = [&](int k) -> int {
    const int id = ptab[k];
    OSCAR_DCHECK(id >= 0 && id < npool, p.status);
    return id;
  };

  // Work distribution: the n pages of the segment are dealt out as whole
  // rounds of batches of NB consecutive pages (the k-th batch of the i-th
  // wave of a head is batch i + WH*k), then the pages left after the last
  // whole round (fewer than WH*NB) one at a time (page i, i + WH, ... of the
  // rest), so that no wave of a short segment has a whole batch more than
  // another.  Which pages a wave sums, and so every rounding, is the same on
  // every run.  The SIMD arbiter favours older waves, which would leave the
  // younger ones finishing last; so every NB pages a wave counts the pages
  // its head's waves have started, in batches (an LDS counter, used for
  // nothing else), and raises its issue priority while it is more than
  // kPrioLag / WH batches behind their mean.  Priorities change only the
  // timing.
  constexpr int kPrioLag = 2;
  int ngrab = 0;                                  // batches this wave started (uniform)
  const int wih = w / HG;                         // this wave's index among its head's
  auto prio_tick = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&batch_ctr[jl], 1);
    v = __builtin_amdgcn_readfirstlane(v);
    if (v > WH * ngrab + kPrioLag) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(0);
    ++ngrab;
  };
  const int nseg = pend - pbeg;                   // this head's pages (0 for a wave without one)
  const int full = nseg / (WH * NB) * (WH * NB);  // pages in whole rounds of batches
  const int rpos = full / WH;                     // this wave's positions in them (a multiple of NB)
  const int ntail = nseg - full;
  const int npos = rpos + (ntail > wih ? (ntail - wih + WH - 1) / WH : 0);   // positions of this wave
  // pages of successive positions (uniform): +1 inside a batch, to the
  // wave's next batch at a batch start, then the single pages WH apart
  const int jump = (WH - 1) * NB + 1;
  const int tail0 = pbeg + full + wih;            // page of position rpos
  auto next_page = [&](int t, int pg, bool batch_start) -> int {   // page of position t after pg
    return t < rpos ? (batch_start ? pg + jump : pg + 1) : (t == rpos ? tail0 : pg + WH);
  };

  auto issue = [&](Stage &sg, int phys) {      // wave-uniform phys
    // a negative id is a large unsigned one: one compare checks both ends
    sg.ok = (uint32_t)phys < (uint32_t)npool;
    // out-of-range stages still load (from page 0) so every lane issues the
    // same load sequence; their data is never used
    const uint8_t *rec = pool_j + (uint64_t)(sg.ok ? (uint32_t)phys : 0u) * rec_stride;
    // one record as a buffer resource (word 3: 32-bit data format, required
    // non-zero for buffer loads on this family); reads past it return 0
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(rec), (short)0, RL.bytes(), 0x00020000);
    buf_words<SW>(sg.c, rs, off_c);
    buf_words<2 * NG>(sg.sz, rs, off_sz);
  };

  // the wave's positions go to ring slots in order, NS - 1 requests ahead of
  // processing; a position past npos loads nothing that is used.  ipg is the
  // page of the next position to request, pgr[slot] the page a stage holds.
  // The first NS - 1 requests take their page ids from the table itself, so
  // they leave before the staging barrier.
  int ipg = rpos > 0 ? pbeg + wih * NB : tail0;
  int pgr[NS];
  static_assert(NS - 1 <= NB, "the first requests lie in the first batch");
  if (npos > 0) {
#pragma unroll
    for (int idx = 0; idx < NS - 1; ++idx) {
      pgr[idx] = ipg;
      issue(st[idx], idx < npos ? table_id(ipg) : -1);
      ipg = next_page(idx + 1, ipg, (idx + 1) % NB == 0);
    }
  }
  if (threadIdx.x < 8) batch_ctr[threadIdx.x] = 0;
  __syncthreads();
  if (npos > 0) prio_tick();                      // the first batch

  float (*qf)[D] = qf_all[w];
  _Float16 (*wbuf)[GQ][16] = wbuf_all[w];            // [grp][head][slot]

  // per-lane constants of the (head, token) layout of the QK result:
  // lane (kb, r16) holds head 4*qd + kb, token r16
  float qscale[NQ], qzl[NQ][NG];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    int qe_l = qe_h[0];
    float z_l[NG];
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) z_l[g2] = qz_h[0][g2];
#pragma unroll
    for (int h = 1; h < GQ; ++h) {
      const bool mine = h == qd * 4 + kb;
      qe_l = mine ? qe_h[h] : qe_l;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) z_l[g2] = mine ? qz_h[h][g2] : z_l[g2];
    }
    qscale[qd] = ldexpf(1.f, -qe_l) * p.sm_log2;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) qzl[qd][g2] = z_l[g2];
  }

  // running state; QK layout: lane = (head 4*qd + kb, token r16)
  float m_run[NQ], lsum[NQ], zacc[NQ][NG];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    m_run[qd] = -INFINITY;
    lsum[qd] = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) zacc[qd][g2] = 0.f;
  }
  // PV accumulators: acc[qd][h2][i] = o[head 4*qd + i][channel lane + 64*h2]
  v4f acc[NQ][NH];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int h2 = 0; h2 < NH; ++h2) acc[qd][h2] = v4f{0.f, 0.f, 0.f, 0.f};

  // code -> f16 (1 + code/4) masks, held in registers (opaque to the compiler)
  // so that (x & m) | c selects one v_and_or_b32
  uint32_t m4, m6, m8, f16one;
  asm volatile("s_mov_b32 %0, 0x300030" : "=s"(m4));
  asm volatile("s_mov_b32 %0, 0xc000c0" : "=s"(m6));
  asm volatile("s_mov_b32 %0, 0x3000300" : "=s"(m8));
  asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(f16one));
  // k slot of this lane's token in the PV A operands, and the A factor
  // 2^(8-b) of its mantissa bit; with a codebook the slots of the level
  // lookup (token t in slot 4 * (t % 4) + t / 4, no factor)
  const int pvs = CB ? 4 * (r16 & 3) + (r16 >> 2) : pv_slot(r16);
  const float pvf = CB ? 1.f : pv_factor(r16);
  constexpr float kLazy = 2.f;                 // log2 headroom of the running max
  float m_thr[NQ];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) m_thr[qd] = -INFINITY;

  // the sequence's last page when it is partial (else -1), and its tokens
  const int tail_pg = (hl & (kPage - 1)) ? hl / kPage : -1;
  const int tail_n = hl & (kPage - 1);
  auto process = [&](Stage &sg, int pg) {          // pg: history page index (< ceil(hl / 16))
    if (!sg.ok) return;
    const int ntok = pg == tail_pg ? tail_n : kPage;
    // tokens past the history length (only on a sequence's last, partial page):
    // logit -inf and (scale, zero) read as 0, since unwritten record bytes may
    // hold any bit pattern
    if (ntok < kPage) {
      const uint32_t vmask = r16 < ntok ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int g2 = 0; g2 < 2 * NG; ++g2) sg.sz[g2] &= vmask;
    }

    // ---------------- QK on int8 MFMA ----------------
    // per group: the dot products of the query pieces with the codes (with a
    // codebook also with the b0 and b0&b1 planes), recombined from the three
    // pieces as p0*2^14 + p1*2^7 + p2 (two shift-adds; the empty asm keeps
    // the compiler from re-associating them into two shifts and an add3).
    // The planes share one accumulator when their A operands carry the plane
    // weights (kSepAcc false), else each plane is recombined as soon as it is
    // done.  With kPermPlanes the code bytes of the first plane are kept, and
    // each byte of the other planes is looked up from them by one byte
    // permute (tables b0 = c & 1 and b0&b1 = (c == 3)) instead of being
    // extracted from the packed word again
    auto recombine = [](const v4i &a) -> float {
      int dhi = (a[0] << 7) + a[1];
      asm volatile("" : "+v"(dhi));
      return (float)((dhi << 7) + a[2]);
    };
    constexpr int NACC = kSepAcc ? NP : 1;
    float dv[NACC][NQ][NG];
    v4i qacc[NQ][NG];
    v4i cbytes[NBLK];
#pragma unroll
    for (int pl = 0; pl < NP; ++pl) {
      const int ap = kSepAcc ? 0 : pl;           // A operand set of this plane
      if constexpr (NP == 3) {
        if (pl == 2 && !plane2) {
          if constexpr (kSepAcc) {
#pragma unroll
            for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
              for (int g2 = 0; g2 < NG; ++g2) dv[NACC - 1][qd][g2] = 0.f;
          }
          continue;
        }
      }
      if (kSepAcc || pl == 0) {
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
          for (int g2 = 0; g2 < NG; ++g2) qacc[qd][g2] = v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        v4i bq;
        if (kPermPlanes && pl > 0) {
          const uint32_t tab = pl == 1 ? 0x01000100u : 0x01000000u;   // byte c: plane value of code c
#pragma unroll
          for (int r = 0; r < 4; ++r) bq[r] = (int)__builtin_amdgcn_perm(tab, tab, (uint32_t)cbytes[blk][r]);
        } else {
          const uint32_t d = sg.c[blk];
          const uint32_t e = pl == 2 ? d & (d >> 1) : d;   // bit 2i of e: b0 & b1 of channel i
          const uint32_t mk = pl == 0 ? 0x03030303u : 0x01010101u;
          bq = v4i{(int)(e & mk), (int)((e >> 2) & mk), (int)((e >> 4) & mk), (int)((e >> 6) & mk)};
          if constexpr (kPermPlanes) cbytes[blk] = bq;
        }
#pragma unroll
        for (int gs = 0; gs < GPB; ++gs) {
          const int m = blk * GPB + gs;
          const int g2 = (64 * blk) / G + gs;
#pragma unroll
          for (int qd = 0; qd < NQ; ++qd)
            qacc[qd][g2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[qd][ap][m], bq, qacc[qd][g2], 0, 0, 0);
        }
      }
      if (kSepAcc || pl == NP - 1 || (NP == 3 && pl == 1 && !plane2)) {
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
          for (int g2 = 0; g2 < NG; ++g2) dv[kSepAcc ? pl : 0][qd][g2] = recombine(qacc[qd][g2]);
      }
    }
    float s_[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      float sc = 0.f, zt = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) {
        float dot = dv[0][qd][g2];
        if constexpr (kSepAcc) dot = fmaf(kcC, dv[NACC - 1][qd][g2], fmaf(kcB, dv[1 % NACC][qd][g2], kcA * dot));
        const float ks = bf16_lo(sg.sz[g2]);
        sc = fmaf(ks, dot, sc);
        // the zero point, and the codebook's L0 part of every level
        zt = fmaf(CB ? fmaf(ks, kL0, bf16_hi(sg.sz[g2])) : bf16_hi(sg.sz[g2]), qzl[qd][g2], zt);
      }
      s_[qd] = fmaf(sc, qscale[qd], zt);
    }
    if (__builtin_expect(ntok < kPage, 0)) {
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) s_[qd] = r16 < ntok ? s_[qd] : -INFINITY;
    }

    // ---------------- online softmax (lazy running max per head) ----------------
    bool grow = false;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) grow |= s_[qd] > m_thr[qd];
    if (__builtin_expect(__any(grow), 0)) {
      float alpha[NQ];
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        const float mnew = max_raw(m_run[qd], row_max(s_[qd]));
        alpha[qd] = m_run[qd] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qd] - mnew);
        m_run[qd] = mnew;
        m_thr[qd] = mnew + kLazy;
        lsum[qd] *= alpha[qd];
#pragma unroll
        for (int g2 = 0; g2 < NG; ++g2) zacc[qd][g2] *= alpha[qd];
      }
      // accumulator element i of head quad qd is head 4*qd + i, whose alpha is
      // uniform over the 16 lanes 16*i .. of quad qd
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[qd]), 16 * i));
#pragma unroll
          for (int h2 = 0; h2 < NH; ++h2) acc[qd][h2][i] *= a;
        }
    }
    float pr[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      pr[qd] = __builtin_amdgcn_exp2f(s_[qd] - m_run[qd]);   // < 4; 0 for masked tokens
      lsum[qd] += pr[qd];
    }
    float pa[NQ];                                 // A weights carry the factor 2^(8-b)
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) pa[qd] = pr[qd] * pvf;

    // ---------------- PV weights to LDS ----------------
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) {
      const float vs = bf16_lo(sg.sz[NG + g2]), vz = bf16_hi(sg.sz[NG + g2]);
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        zacc[qd][g2] = fmaf(pr[qd], vz, zacc[qd][g2]);
        const _Float16 wh = (_Float16)(pa[qd] * vs);
        // uniform codes: remove the implicit one of the f16 code values;
        // codebook: the vL0 part of the levels
        if constexpr (!CB) zacc[qd][g2] = fmaf(-4.f, (float)wh, zacc[qd][g2]);
        else zacc[qd][g2] = fmaf(vL0, (float)wh, zacc[qd][g2]);
        wbuf[g2][qd * 4 + kb][pvs] = wh;
      }
    }
    wave_lds_sync();

    // ---------------- PV on f16 MFMA, 4 token quads ----------------
    if constexpr (CB) {
      // codebook: MFMA ti takes tokens ti, ti + 4, ti + 8, ti + 12 (token t
      // of a V word sits in bits 2t); byte i of the selector is the code of
      // token 4i + ti, the permutes give the low and the high bytes of the
      // four tokens' f16 levels, and two more interleave them into f16 pairs
#pragma unroll
      for (int h2 = 0; h2 < NH; ++h2) {
        const uint32_t x0 = sg.c[NBLK + h2];
        const int g2 = (lane + 64 * h2) / G;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const uint32_t sel = (x0 >> (2 * ti)) & 0x03030303u;
          const uint32_t lo = __builtin_amdgcn_perm(vtab_hi, vtab_lo, sel);
          const uint32_t hi = __builtin_amdgcn_perm(vtab_lo, vtab_hi, sel);
          const v4h bv = as_v4h(__builtin_amdgcn_perm(hi, lo, 0x05010400u),
                                __builtin_amdgcn_perm(hi, lo, 0x07030602u));
#pragma unroll
          for (int qd = 0; qd < NQ; ++qd) {
            const uint2 u = *reinterpret_cast<const uint2 *>(&wbuf[g2][qd * 4 + (lane & 3)][4 * ti]);
            acc[qd][h2] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_v4h(u.x, u.y), bv, acc[qd][h2], 0, 0, 0);
          }
        }
      }
    } else {
      // token t of a V word sits in bits 2t; B register u holds tokens (u, u+8)
      // in its two halves at the mantissa bit given by pv_factor
      uint32_t xs[NH][3];                         // the word and two shifted copies
#pragma unroll
      for (int h2 = 0; h2 < NH; ++h2) {
        const uint32_t x0 = sg.c[NBLK + h2];
        xs[h2][0] = x0;
        xs[h2][1] = x0 << 4;
        xs[h2][2] = x0 >> 6;
      }
      // B register u (tokens u, u+8): copy (x1 x1 x1 x0 x0 x2 x2 x2)[u], mask
      // at mantissa bit (4 6 8 6 8 4 6 8)[u]
      auto breg = [&](int h2, int u) -> uint32_t {
        const uint32_t x = u < 3 ? xs[h2][1] : u < 5 ? xs[h2][0] : xs[h2][2];
        const int b = (u == 0 || u == 5) ? 4 : (u == 1 || u == 3 || u == 6) ? 6 : 8;
        return (x & (b == 4 ? m4 : b == 6 ? m6 : m8)) | f16one;
      };
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
        for (int h2 = 0; h2 < NH; ++h2) {
          const int g2 = (lane + 64 * h2) / G;
          const v4h bv = as_v4h(breg(h2, 2 * ti), breg(h2, 2 * ti + 1));
#pragma unroll
          for (int qd = 0; qd < NQ; ++qd) {
            const uint2 u = *reinterpret_cast<const uint2 *>(&wbuf[g2][qd * 4 + (lane & 3)][4 * ti]);
            acc[qd][h2] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_v4h(u.x, u.y), bv, acc[qd][h2], 0, 0, 0);
          }
        }
      }
    }
    wave_lds_sync();
  };

  // each step requests the position NS - 1 ahead and processes one
  for (int t0 = 0; t0 < npos; t0 += NS) {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int idx = t0 + s2 + NS - 1;           // request position (t0 is a multiple of NB)
      const int slot = (s2 + NS - 1) % NS;
      if ((s2 + NS - 1) % NB == 0) prio_tick();
      pgr[slot] = ipg;
      issue(st[slot], idx < npos ? page_id(ipg) : -1);
      ipg = next_page(idx + 1, ipg, (s2 + NS) % NB == 0);
      if (t0 + s2 < npos) process(st[s2], pgr[s2]);
    }
  }

  __builtin_amdgcn_s_setprio(0);

  // ---------------- epilogue: one partial per (q head, segment) ----------------
  // each wave leaves its unnormalised output and (max, sum) per head in LDS
  // (its own query slot, no longer read), then the block combines the WH waves
  // of every head:  M = max m_w, L = sum L_w 2^(m_w - M), O = sum O_w 2^(m_w - M)
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    // head 4*qd + kb's sums over its 16 token lanes
    const float L = row_sum(lsum[qd]);
    float Z[NG];
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) Z[g2] = row_sum(zacc[qd][g2]);
    if (r16 == 0) {
      mlw[w][qd * 4 + kb][0] = m_run[qd];
      mlw[w][qd * 4 + kb][1] = L;
    }
    // accumulator element i: head 4*qd + i, channel lane + 64*h2; the zero-point
    // and offset part of head 4*qd + i is uniform over lanes 16*i ..
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int h2 = 0; h2 < NH; ++h2) {
        const int c = lane + 64 * h2;
        float zz = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < NG; ++g2) {
          const float zg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Z[g2]), 16 * i));
          zz = (c / G == g2) ? zg : zz;
        }
        // uniform codes: the f16 code values carry a factor 1/4; codebook:
        // PV ran on h[c], the levels' integer part
        qf[qd * 4 + i][c] = (CB ? vbeta : 4.f) * acc[qd][h2][i] + zz;
      }
    }
  }
  __syncthreads();
  float *po = reinterpret_cast<float *>(p.ws + p.L.part_o);
  float *pml = reinterpret_cast<float *>(p.ws + p.L.part_ml);
  for (int idx = threadIdx.x; idx < HG * GQ * D; idx += 64 * HB) {
    const int c = idx % D, hh = (idx / D) % GQ, jl2 = idx / (D * GQ);
    const int j2 = hg * HG + jl2;
    if (j2 >= p.Hkv) break;                       // the rest of idx is past the group too
    auto wave_of = [&](int k) { return jl2 + HG * k; };   // the waves of head jl2
    float M = -INFINITY;
    for (int k = 0; k < WH; ++k) M = fmaxf(M, mlw[wave_of(k)][hh][0]);
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
      for (int k = 0; k < WH; ++k) {
        const int wk = wave_of(k);
        const float m = mlw[wk][hh][0];
        if (m == -INFINITY) continue;
        const float a = exp2f(m - M);
        O = fmaf(a, qf_all[wk][hh][c], O);
        L = fmaf(a, mlw[wk][hh][1], L);
      }
    }
    if (hh >= p.g) continue;                      // a head the KV head does not have
    const size_t row = ((size_t)b * p.Hq + p.q_of_kv[j2 * p.g + hh]) * S + slot;
    po[row * D + c] = O;
    if (c == 0) {
      pml[row * 2 + 0] = M;
      pml[row * 2 + 1] = L;
    }
  }
  __syncthreads();                                // LDS is reused by the next segment
  }  // segments
}

template <int D, int G, int GQ, bool CB>
static void launch_mfma_inst(const DecodeParams &p, hipStream_t s) {
  // B * mfma_parts blocks per group of KV heads (balanced across sequences
  // inside the kernel)
  constexpr int HB = mfma_waves(D, G, GQ, CB);
  const int hg = mfma_heads_per_block(p.Hkv);
  const int ngrp = (p.Hkv + hg - 1) / hg;
  const dim3 grid(p.B * ngrp * p.mfma_parts), blk(64 * HB);
  hipLaunchKernelGGL((k_int2_mfma<D, G, GQ, CB, HB>), grid, blk, 0, s, p);
}

template <int D, int G>
static void launch_mfma_dg(const DecodeParams &p, hipStream_t s) {
  const bool cb = p.codebook != nullptr;
  if (p.g == 8 && cb) launch_mfma_inst<D, G, 8, true>(p, s);
  else if (p.g == 8) launch_mfma_inst<D, G, 8, false>(p, s);
  else if (cb) launch_mfma_inst<D, G, 4, true>(p, s);
  else launch_mfma_inst<D, G, 4, false>(p, s);
}

hipError_t launch_int2_mfma(const DecodeParams &p, hipStream_t s) {
  if (p.g != 1 && p.g != 2 && p.g != 4 && p.g != 8) return hipErrorInvalidValue;
  if (p.D == 64 && p.G == 32) launch_mfma_dg<64, 32>(p, s);
  else if (p.D == 64 && p.G == 64) launch_mfma_dg<64, 64>(p, s);
  else if (p.D == 128 && p.G == 32) launch_mfma_dg<128, 32>(p, s);
  else if (p.D == 128 && p.G == 64) launch_mfma_dg<128, 64>(p, s);
  else if (p.D == 128 && p.G == 128) launch_mfma_dg<128, 128>(p, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace oscar
