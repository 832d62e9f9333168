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
//     exact f16 values 1 + code/4, A = w in f16, fp32 accumulation; the "+1"
//     part is removed with sum_t w (of the same f16 values).
//
// One block (4 waves) per (sequence, KV head, chunk of pages); each wave walks
// every 4th page of the chunk with the next page's loads in flight, keeping an
// exact running max per head (16-lane DPP reductions).  Requires 4 or 8 q heads
// per KV head and V group scales below the f16 range (65504).
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

// k-slot order shared by the PV operands: lane group kb, element i <-> token
// kb + {0, 8, 4, 12}[i]; token t sits in slot 4*(t%4) + e(t/4), e = {0,2,1,3}.
__device__ __forceinline__ int pv_slot(int t) {
  const int i = t >> 2;
  return 4 * (t & 3) + (((i & 1) << 1) | (i >> 1));
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

}  // namespace

template <int D, int G, int GQ>
__global__ __launch_bounds__(256) void k_int2_mfma(DecodeParams p) {
  constexpr RecLayout RL(D, G);
  constexpr int NG = D / G;            // groups per token
  constexpr int NBLK = D / 64;         // 64-channel blocks (one int8 MFMA K each)
  constexpr int GPB = G < 64 ? 64 / G : 1;   // groups inside one 64-channel block
  constexpr int NQK = NBLK * GPB;      // QK MFMAs per head quad per page
  constexpr int NH = D / 64;           // 64-channel halves of PV (lane owns l + 64*h2)
  constexpr int NQ = GQ / 4;           // head quads
  static_assert(GQ == 4 || GQ == 8, "4 or 8 q heads per KV head");

  const int S = p.splits;
  const int unit = blockIdx.x / S;
  const int split = blockIdx.x % S;
  const int b = unit / p.Hkv;
  const int j = unit % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int r16 = lane & 15, kb = lane >> 4;     // row-in-16 and lane group

  __shared__ float qf[GQ][D];                    // q_rot (unscaled)
  __shared__ int qexp[GQ];                       // q_int = rint(q * 2^qexp)
  __shared__ float qz[GQ][NG];                   // sm_log2 * sum of q over the group
  __shared__ __align__(16) _Float16 wbuf[4][NG][GQ][16];       // per wave: w[grp][head][slot]
  __shared__ float wm[4][GQ], wl[4][GQ];
  __shared__ float wo[4][GQ][D];

  // ---------------- prologue: query as integer pieces ----------------
  const float *qrot = reinterpret_cast<const float *>(p.ws + p.L.qrot);
  for (int i = tid; i < GQ * D; i += 256) {
    const int h = i / D, c = i % D;
    qf[h][c] = qrot[((size_t)b * p.Hq + p.q_of_kv[j * GQ + h]) * D + c];
  }
  __syncthreads();
  if (tid < GQ) {
    float mx = 0.f;
    for (int c = 0; c < D; ++c) mx = fmaxf(mx, fabsf(qf[tid][c]));
    int e = 0;
    if (mx > 0.f) (void)frexpf(mx, &e);          // mx < 2^e
    int qe = mx > 0.f ? 20 - e : 0;              // |q| * 2^qexp < 2^20
    qexp[tid] = qe > 126 ? 126 : (qe < -100 ? -100 : qe);
  }
  if (tid >= 64 && tid < 64 + GQ * NG) {
    const int h = (tid - 64) / NG, g2 = (tid - 64) % NG;
    float s = 0.f;
    for (int c = g2 * G; c < (g2 + 1) * G; ++c) s += qf[h][c];
    qz[h][g2] = s * p.sm_log2;
  }
  __syncthreads();

  // A operands: row = 4*h + piece (piece 3 is zero), lane group kb, VGPR e,
  // byte bb <-> channel 64*blk + 16*kb + 4*bb + e (the B unpack order).
  v4i aq[NQ][NQK];
  {
    const int hrow = r16 >> 2, pc = r16 & 3;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const int h = qd * 4 + hrow;
      const float sc = ldexpf(1.f, qexp[h]);
#pragma unroll
      for (int m = 0; m < NQK; ++m) {
        const int blk = m / GPB, gsub = m % GPB;
        const int g2 = (64 * blk) / G + gsub;
        int vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t word = 0;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int c = 64 * blk + 16 * kb + 4 * bb + e;
            int piece = 0;
            if (pc < 3 && c / G == g2) {
              const int qi = (int)rintf(qf[h][c] * sc);
              piece = pc == 0 ? (qi >> 14) : pc == 1 ? ((qi >> 7) & 127) : (qi & 127);
            }
            word |= ((uint32_t)piece & 0xFFu) << (8 * bb);
          }
          vv[e] = (int)word;
        }
        aq[qd][m] = v4i{vv[0], vv[1], vv[2], vv[3]};
      }
    }
  }
  // per-lane constants of the (head, token) layout of the QK result
  float qscale[NQ], qzl[NQ][NG];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    const int h = qd * 4 + kb;
    qscale[qd] = ldexpf(1.f, -qexp[h]) * p.sm_log2;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) qzl[qd][g2] = qz[h][g2];
  }

  int hl = p.hist_len[b];
  hl = hl < 0 ? 0 : hl;
  hl = hl > p.max_hist_len ? p.max_hist_len : hl;
  hl = hl > kPage * p.hist_stride ? kPage * p.hist_stride : hl;
  const int npages = (hl + kPage - 1) / kPage;
  const int p0 = split * p.pages_per_split;
  int p1 = p0 + p.pages_per_split;
  p1 = p1 > npages ? npages : p1;

  // running state; QK layout: lane = (head kb [+4 qd], token r16)
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

  // ---------------- page loop: 4-stage register ring ----------------
  // stage data of one page for this lane: K words of token r16 / lane group kb,
  // K and V (scale, zero) words of token r16, and the V words of channels
  // lane + 64*h2 (adjacent in the record).
  constexpr int NS = 4;
  constexpr int VPL = D / 64;
  struct Stage {
    uint32_t k[NBLK], ks[NG], vs[NG], v[VPL];
    int ok;
  };
  Stage st[NS];
  const int nk = p1 - p0 - w > 0 ? (p1 - p0 - w + 3) / 4 : 0;   // pages of this wave
  const int32_t *ptab = p.hist_pages + (size_t)b * p.hist_stride;
  const size_t rec_stride = (size_t)p.Hkv * RL.bytes();
  const uint8_t *pool_j = p.int2_pool + (size_t)j * RL.bytes();
  int pid_vec = 0, pid_base = -64;

  auto page_id = [&](int k) -> int {           // wave-uniform k
    if (k - pid_base >= 64) {
      pid_base = k;
      const int kk = k + lane;
      pid_vec = kk < nk ? ptab[p0 + w + 4 * kk] : -1;
    }
    return __builtin_amdgcn_readlane(pid_vec, k - pid_base);
  };
  auto issue = [&](Stage &sg, int k) {
    int phys = k < nk ? page_id(k) : -1;
    sg.ok = phys >= 0 && phys < p.num_int2_pages;
    // out-of-range stages still load (from page 0) so every lane issues the
    // same load sequence; their data is never used
    const uint8_t *rec = pool_j + (sg.ok ? (size_t)phys : 0) * rec_stride;
    load_words<NBLK>(sg.k, reinterpret_cast<const uint32_t *>(rec + RL.kcodes()) + r16 * (D / 16) + kb * NBLK);
    load_words<NG>(sg.ks, reinterpret_cast<const uint32_t *>(rec + RL.ksz()) + r16 * NG);
    load_words<NG>(sg.vs, reinterpret_cast<const uint32_t *>(rec + RL.vsz()) + r16 * NG);
    load_words<VPL>(sg.v, reinterpret_cast<const uint32_t *>(rec + RL.vcodes()) + lane * VPL);
  };
  // code -> f16 (1 + code/4) masks, held in registers (opaque to the compiler)
  // so that (x & m) | c selects one v_and_or_b32
  uint32_t m_code, f16one;
  asm volatile("s_mov_b32 %0, 0x3000300" : "=s"(m_code));
  asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(f16one));
  const int pvs = pv_slot(r16);

  auto process = [&](Stage &sg, int k) {
    if (!sg.ok) return;
    const int pg = p0 + w + 4 * k;
    const int ntok = hl - pg * kPage < kPage ? hl - pg * kPage : kPage;
    // tokens past the history length (only on a sequence's last, partial page):
    // logit -inf and (scale, zero) read as 0, since unwritten record bytes may
    // hold any bit pattern
    const bool partial = ntok < kPage;           // wave-uniform
    if (partial) {
      const uint32_t vmask = r16 < ntok ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) { sg.ks[g2] &= vmask; sg.vs[g2] &= vmask; }
    }
    const float sinv = r16 < ntok ? 0.f : -INFINITY;

    // ---------------- QK on int8 MFMA ----------------
    v4i qacc[NQ][NG];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) qacc[qd][g2] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const uint32_t d = sg.k[blk];
      const v4i bq = v4i{(int)(d & 0x03030303u), (int)((d >> 2) & 0x03030303u),
                         (int)((d >> 4) & 0x03030303u), (int)((d >> 6) & 0x03030303u)};
#pragma unroll
      for (int gs = 0; gs < GPB; ++gs) {
        const int m = blk * GPB + gs;
        const int g2 = (64 * blk) / G + gs;
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd)
          qacc[qd][g2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[qd][m], bq, qacc[qd][g2], 0, 0, 0);
      }
    }
    float s_[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      float sc = 0.f, zt = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) {
        const int dint = ((qacc[qd][g2][0] << 7) + qacc[qd][g2][1]) * 128 + qacc[qd][g2][2];
        sc = fmaf(bf16_lo(sg.ks[g2]), (float)dint, sc);
        zt = fmaf(bf16_hi(sg.ks[g2]), qzl[qd][g2], zt);
      }
      s_[qd] = fmaf(sc, qscale[qd], zt) + sinv;
    }

    // ---------------- online softmax (exact running max per head) ----------------
    bool grow = false;
    float mnew[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      mnew[qd] = max_raw(m_run[qd], row_max(s_[qd]));
      grow |= mnew[qd] > m_run[qd];
    }
    if (__builtin_expect(__any(grow), 0)) {
      float alpha[NQ];
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        alpha[qd] = m_run[qd] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qd] - mnew[qd]);
        m_run[qd] = mnew[qd];
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
      pr[qd] = __builtin_amdgcn_exp2f(s_[qd] - m_run[qd]);   // 0 for masked tokens
      lsum[qd] += pr[qd];
    }

    // ---------------- PV weights to LDS ----------------
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) {
      const float vs = bf16_lo(sg.vs[g2]), vz = bf16_hi(sg.vs[g2]);
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        const _Float16 wh = (_Float16)(pr[qd] * vs);
        zacc[qd][g2] = fmaf(pr[qd], vz, zacc[qd][g2]);
        zacc[qd][g2] = fmaf(-4.f, (float)wh, zacc[qd][g2]);
        wbuf[w][g2][qd * 4 + kb][pvs] = wh;
      }
    }
    wave_lds_sync();

    // ---------------- PV on f16 MFMA, 4 token quads ----------------
    // quad ti: tokens (ti, ti+8, ti+4, ti+12) as k = 0..3; token t of a V word
    // sits in bits 2t, so v << (8 - 2ti) and v >> 2ti put each pair at f16
    // mantissa bits 8..9 / 24..25
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int h2 = 0; h2 < NH; ++h2) {
        const uint32_t v = sg.v[h2];
        const v4h bv = as_v4h(((v << (8 - 2 * ti)) & m_code) | f16one, ((v >> (2 * ti)) & m_code) | f16one);
        const int g2 = (lane + 64 * h2) / G;
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd) {
          const uint2 u = *reinterpret_cast<const uint2 *>(&wbuf[w][g2][qd * 4 + (lane & 3)][4 * ti]);
          acc[qd][h2] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_v4h(u.x, u.y), bv, acc[qd][h2], 0, 0, 0);
        }
      }
    }
    wave_lds_sync();
  };

  if (nk > 0) {
#pragma unroll
    for (int s2 = 0; s2 < NS - 1; ++s2) issue(st[s2], s2);
    for (int k = 0; k < nk; k += NS) {
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        issue(st[(s2 + NS - 1) % NS], k + s2 + NS - 1);
        if (k + s2 < nk) process(st[s2], k + s2);
      }
    }
  }

  // ---------------- wave epilogue ----------------
  // head h's sums: row sums over the 16 token lanes of quad h/4, lane group h%4
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    const float L = row_sum(lsum[qd]);
    float Z[NG];
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) Z[g2] = row_sum(zacc[qd][g2]);
    const int h = qd * 4 + kb;
    if (r16 == 0) {
      wm[w][h] = m_run[qd];
      wl[w][h] = L;
    }
    // the zero-point / offset part is added to every channel of its group
    if (r16 < NG) {
      float zz = Z[0];
#pragma unroll
      for (int g2 = 1; g2 < NG; ++g2) zz = r16 == g2 ? Z[g2] : zz;
      wo[w][h][0 + r16] = zz;          // staged in the first NG channels, moved below
    }
  }
  wave_lds_sync();
  float zst[GQ][NG];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) zst[h][g2] = wo[w][h][g2];
  wave_lds_sync();
  // accumulator element i of quad qd, half h2: head 4*qd + i, channel lane + 64*h2
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int h2 = 0; h2 < NH; ++h2) {
      const int c = lane + 64 * h2;
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[w][4 * qd + i][c] = 4.f * acc[qd][h2][i] + zst[4 * qd + i][c / G];
    }
  __syncthreads();

  // ---------------- combine the 4 waves, write the chunk partial ----------------
  float *po = reinterpret_cast<float *>(p.ws + p.L.part_o);
  float *pml = reinterpret_cast<float *>(p.ws + p.L.part_ml);
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
    const int hq = p.q_of_kv[j * GQ + h];
    const size_t row = ((size_t)b * p.Hq + hq) * S + split;
    po[row * D + c] = O;
    if (c == 0) {
      pml[row * 2 + 0] = M;
      pml[row * 2 + 1] = L;
    }
  }
}

template <int D, int G>
static void launch_mfma_dg(const DecodeParams &p, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv * p.splits), blk(256);
  if (p.g == 8) hipLaunchKernelGGL((k_int2_mfma<D, G, 8>), grid, blk, 0, s, p);
  else hipLaunchKernelGGL((k_int2_mfma<D, G, 4>), grid, blk, 0, s, p);
}

hipError_t launch_int2_mfma(const DecodeParams &p, hipStream_t s) {
  if (p.g != 4 && p.g != 8) return hipErrorInvalidValue;
  if (p.D == 64 && p.G == 32) launch_mfma_dg<64, 32>(p, s);
  else if (p.D == 64 && p.G == 64) launch_mfma_dg<64, 64>(p, s);
  else if (p.D == 128 && p.G == 32) launch_mfma_dg<128, 32>(p, s);
  else if (p.D == 128 && p.G == 64) launch_mfma_dg<128, 64>(p, s);
  else if (p.D == 128 && p.G == 128) launch_mfma_dg<128, 128>(p, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace oscar
