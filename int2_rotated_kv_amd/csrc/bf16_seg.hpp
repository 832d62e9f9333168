// BF16 (sink + recent) segment as a block-level device routine, shared by the
// BF16 segment kernel and the fused decode-step kernel (m.th-motor.com repost
// of the OSCAR article, decode stage: the BF16 kernel handles sink/recent).
#pragma once
#include "common.hpp"

namespace oscar {

typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// BF16 segment: up to 320 unrotated tokens per sequence in BF16 pages.  Grid
// (sequence x KV head, 5 chunks of 4 pages); one wave per page, the g q heads
// of the KV head share every load.  Per page (16 tokens):
//   QK on v_mfma_f32_16x16x32_bf16: A = 16 K rows (lane (kb, t) holds channels
//      32m + 8kb .. +7 of token t: one 16-byte load), B = the q heads (bf16,
//      exact products, fp32 accumulation); lane (kb, h) receives tokens
//      4kb .. 4kb+3 of head h.
//   softmax per head over the 16 tokens (4 in-lane, 4 lane groups).
//   PV on the vector ALU: lane owns channels D/64*lane .. +D/64-1 and
//      accumulates p * v over the 16 tokens, p from LDS.
// Every load of the page is issued before any of it is used.  Each chunk
// writes one partial per q head.
// ---------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int D, int GQ>
struct SegShared {
  __align__(16) float pb[4][kPage][GQ];   // per wave: p[token][head]
  float wm[4][GQ], wl[4][GQ];
  float wo[4][GQ][D];
};

// The token of this step, not yet in the pool: slot[b] (page * 16 + offset,
// negative = none) of sequence b reads k[b][j][:], v[b][j][:] instead.
struct NewTok {
  const int32_t *slot;
  const uint16_t *k, *v;               // [B][Hkv][D] bf16
};

template <int D, int GQ>
__device__ __forceinline__ void bf16_seg_body(const DecodeParams &p, const uint16_t *__restrict__ q,
                                              int b, int j, int split, int tid, const NewTok &nt,
                                              SegShared<D, GQ> &sh) {
  constexpr int NM = D / 32;           // QK matrix instructions (32 channels each)
  constexpr int NCH = D / 64;          // PV channels per lane
  static_assert(GQ <= 16, "q heads are the 16 columns of the QK product");
  const int lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, kb = lane >> 4;
  auto &pb = sh.pb;
  auto &wm = sh.wm;
  auto &wl = sh.wl;
  auto &wo = sh.wo;

  // segment length, this wave's page id and the new token's slot (one round
  // trip), then every load of the page (a second one)
  const int pgi = split * kBf16PagesPerSplit + w;     // page index in the table
  int T = p.bf16_len[b];
  const int64_t page = pgi < p.bf16_stride ? p.bf16_pages[(size_t)b * p.bf16_stride + pgi] : -1;
  OSCAR_DCHECK(T >= 0 && T <= kMaxBf16, p.status);
  OSCAR_DCHECK(pgi * kPage >= T || pgi >= p.bf16_stride || (page >= 0 && page < p.num_bf16_pages), p.status);
  const int ns = nt.slot != nullptr ? nt.slot[b] : -1;
  T = T < 0 ? 0 : T;
  T = T > kMaxBf16 ? kMaxBf16 : T;
  T = T > kPage * p.bf16_stride ? kPage * p.bf16_stride : T;
  const int ntok = T - pgi * kPage;
  const bool live = ntok > 0 && page >= 0 && page < p.num_bf16_pages;

  // q operands: lane (kb, h) holds channels 32m + 8kb .. +7 of q head h
  v8bf qb[NM];
  {
    const int hq = r16 < GQ ? p.q_of_kv[j * GQ + r16] : 0;
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + ((size_t)b * p.Hq + hq) * D + 8 * kb);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 v = r16 < GQ ? qp[4 * m] : make_uint4(0u, 0u, 0u, 0u);
      __builtin_memcpy(&qb[m], &v, 16);
    }
  }
  // this step's token sits at offset noff of this wave's page (noff = -1: not here)
  const int noff = (live && ns >= 0 && (ns >> 4) == page) ? (ns & 15) : -1;
  v8bf ka[NM];
  uint32_t vraw[kPage];
  if (live) {
    // the pool rows are read whatever the new token's slot holds (in bounds:
    // the page is live); that token's K row then replaces the pool's one
    const size_t base = ((page * p.Hkv + j) * kPage) * D;
    const uint4 *kp = reinterpret_cast<const uint4 *>(p.bf16_k + base + (size_t)r16 * D + 8 * kb);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 v = kp[4 * m];
      __builtin_memcpy(&ka[m], &v, 16);
    }
    if (r16 == noff) {
      const uint4 *kn = reinterpret_cast<const uint4 *>(nt.k + ((size_t)b * p.Hkv + j) * D + 8 * kb);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 v = kn[4 * m];
        __builtin_memcpy(&ka[m], &v, 16);
      }
    }
    const uint16_t *vp = p.bf16_v + base;
#pragma unroll
    for (int tt = 0; tt < kPage; ++tt) {
      if constexpr (NCH == 2) vraw[tt] = reinterpret_cast<const uint32_t *>(vp)[(size_t)tt * (D / 2) + lane];
      else vraw[tt] = vp[(size_t)tt * D + lane];
    }
    if (noff >= 0) {
      const uint16_t *vn = nt.v + ((size_t)b * p.Hkv + j) * D;
      uint32_t x;
      if constexpr (NCH == 2) x = reinterpret_cast<const uint32_t *>(vn)[lane];
      else x = vn[lane];
#pragma unroll
      for (int tt = 0; tt < kPage; ++tt) vraw[tt] = tt == noff ? x : vraw[tt];
    }
  }

  float m_h = -INFINITY, l_h = 0.f;
  float o[GQ][NCH];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int k = 0; k < NCH; ++k) o[h][k] = 0.f;
  if (live) {
    // ---- QK ----
    v4f sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[m], qb[m], sacc, 0, 0, 0);
    // lane (kb, h): tokens 4kb + i of head h; slots past the segment length
    // (any bits) get logit -inf
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (4 * kb + i < ntok) ? sacc[i] * p.sm_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));           // >= one valid token: finite
    float pr[4], l = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = exp2f(sv[i] - mx);                    // 0 for masked slots
      l += pr[i];
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    m_h = mx;
    l_h = l;
    if (r16 < GQ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[w][4 * kb + i][r16] = pr[i];
    }
    wave_lds_sync();
    // ---- PV ----  (slots past the segment length may hold any bits: 0)
#pragma unroll
    for (int tt = 0; tt < kPage; ++tt) {
      float v[NCH];
      if constexpr (NCH == 2) {
        v[0] = tt < ntok ? bf16_lo(vraw[tt]) : 0.f;
        v[1] = tt < ntok ? bf16_hi(vraw[tt]) : 0.f;
      } else {
        v[0] = tt < ntok ? bf16_to_f32((uint16_t)vraw[tt]) : 0.f;
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float ph = pb[w][tt][h];
#pragma unroll
        for (int k = 0; k < NCH; ++k) o[h][k] = fmaf(ph, v[k], o[h][k]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) wo[w][h][lane * NCH + k] = o[h][k];
  }
  if (kb == 0 && r16 < GQ) { wm[w][r16] = m_h; wl[w][r16] = l_h; }
  __syncthreads();
  float *bo = reinterpret_cast<float *>(p.ws + p.L.bf_o);
  float *bml = reinterpret_cast<float *>(p.ws + p.L.bf_ml);
  for (int i = tid; i < GQ * D; i += 256) {
    const int h = i / D, c = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) M = fmaxf(M, wm[k][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (wm[k][h] == -INFINITY) continue;
        const float a = exp2f(wm[k][h] - M);
        L = fmaf(wl[k][h], a, L);
        O = fmaf(wo[k][h][c], a, O);
      }
    }
    const size_t row = ((size_t)b * p.Hq + p.q_of_kv[j * GQ + h]) * kBf16Splits + split;
    bo[row * D + c] = O;
    if (c == 0) {
      bml[row * 2 + 0] = M;
      bml[row * 2 + 1] = L;
    }
  }
}

}  // namespace oscar
