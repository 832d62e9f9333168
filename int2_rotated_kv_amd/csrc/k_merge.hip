// Online-softmax merge of the split cache's partial results (m.th-motor.com
// repost of the OSCAR article, decode stage: the BF16 and INT2 segment results
// are combined by an online-softmax merge).  Per q head:
//   history chunks:  M = max m_s, L = sum l_s 2^(m_s - M), O = sum o_s 2^(m_s - M)
//   un-rotation:     O_hist = O . R_v^T   (the history values are stored as v . R_v)
//   BF16 splits:     (m_b, l_b, o_b) merged the same way (unrotated)
//   final:           M' = max(M, m_b); out = (O_hist 2^(M-M') + o_b 2^(m_b-M'))
//                                            / (L 2^(M-M') + l_b 2^(m_b-M'))
//   lse = M' ln2 + ln(denominator)  (natural-log units)
#include "common.hpp"

namespace oscar {

constexpr int kMergeThreads = 256;
constexpr int kMergeRegChunks = 8;       // chunk outputs per thread loaded up front

// One block (4 waves) per (sequence, q head).  Every load the block needs is
// issued first (chunk maxima and sums, the first chunk outputs of each thread,
// its slice of the R_v row, the BF16 partials), so the block waits for memory
// about once; the rest is LDS exchanges.  Thread (group gi, channel c) sums
// chunks gi, gi + NGR, ... for channel c and multiplies the slice gi of the
// R_v row c.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void k_merge(DecodeParams p, const float *__restrict__ Rv,
                                                         float *__restrict__ out, float *__restrict__ lse) {
  constexpr int NGR = kMergeThreads / D;         // thread groups (2 or 4)
  constexpr int KPG = D / NGR / 4;               // float4 of an R_v row per group
  const size_t bh = blockIdx.x;
  const int j = p.kv_of_q[bh % p.Hq];
  const int tid = threadIdx.x, lane = tid & 63;
  const int c = tid % D, gi = tid / D;
  const int S = p.splits;
  extern __shared__ float a_s[];                 // [S] chunk weights 2^(m_s - M)
  __shared__ __align__(16) float Os[D];          // merged history output (rotated basis)
  __shared__ float red[NGR][D];
  __shared__ float ML[2];

  const float *ml = reinterpret_cast<const float *>(p.ws + p.L.part_ml) + bh * S * 2;
  const float *po = reinterpret_cast<const float *>(p.ws + p.L.part_o) + bh * S * D;
  const float *bml = reinterpret_cast<const float *>(p.ws + p.L.bf_ml) + bh * kBf16Splits * 2;
  const float *bo = reinterpret_cast<const float *>(p.ws + p.L.bf_o) + bh * kBf16Splits * D + c;

  // ---- every load up front ----
  float ov[kMergeRegChunks];                     // chunk outputs gi + NGR*k, channel c
#pragma unroll
  for (int k = 0; k < kMergeRegChunks; ++k) {
    const int s2 = gi + NGR * k;
    ov[k] = s2 < S ? po[(size_t)s2 * D + c] : 0.f;
  }
  float4 r[KPG];
  if (Rv != nullptr) {
    const float4 *row = reinterpret_cast<const float4 *>(Rv + ((size_t)j * D + c) * D) + gi * KPG;
#pragma unroll
    for (int k = 0; k < KPG; ++k) r[k] = row[k];
  }
  float bm[kBf16Splits], bl[kBf16Splits], bov[kBf16Splits];
#pragma unroll
  for (int s2 = 0; s2 < kBf16Splits; ++s2) {
    bm[s2] = bml[2 * s2];
    bl[s2] = bml[2 * s2 + 1];
    bov[s2] = gi == 0 ? bo[(size_t)s2 * D] : 0.f;
  }
  float mv = -INFINITY, lv = 0.f;                // wave 0: chunk lane
  if (tid < 64 && lane < S) {
    mv = ml[2 * lane];
    lv = ml[2 * lane + 1];
  }

  // ---- chunk weights (wave 0): M = max m_s, L = sum l_s 2^(m_s - M) ----
  if (tid < 64) {
    float M = mv;
    for (int s2 = lane + 64; s2 < S; s2 += 64) M = fmaxf(M, ml[2 * s2]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f;
    for (int s2 = lane; s2 < S; s2 += 64) {
      const float m = s2 == lane ? mv : ml[2 * s2];
      const float l = s2 == lane ? lv : ml[2 * s2 + 1];
      const float a = (m == -INFINITY) ? 0.f : exp2f(m - M);
      a_s[s2] = a;
      L = fmaf(l, a, L);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    if (lane == 0) { ML[0] = M; ML[1] = L; }
  }
  __syncthreads();

  // ---- O[c] = sum_s a_s o_s[c]; a chunk with weight 0 (no tokens) adds 0
  // whatever its stored output holds ----
  {
    float O0 = 0.f, O1 = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeRegChunks; ++k) {
      const int s2 = gi + NGR * k;
      const float wgt = s2 < S ? a_s[s2] : 0.f;
      float &O = (k & 1) ? O1 : O0;
      O = fmaf(wgt, wgt != 0.f ? ov[k] : 0.f, O);
    }
    for (int s2 = gi + NGR * kMergeRegChunks; s2 < S; s2 += NGR) {
      const float v = po[(size_t)s2 * D + c], wgt = a_s[s2];
      O0 = fmaf(wgt, wgt != 0.f ? v : 0.f, O0);
    }
    red[gi][c] = O0 + O1;
  }
  __syncthreads();
  if (tid < D) {
    float O = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NGR; ++g2) O += red[g2][tid];
    Os[tid] = O;
  }
  __syncthreads();

  // ---- un-rotation O_hist[c] = sum_k O[k] R_v[j][c][k] ----
  float oh;
  if (Rv != nullptr) {
    const float4 *o4 = reinterpret_cast<const float4 *>(Os) + gi * KPG;
    float x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int k = 0; k < KPG; ++k) {
      const float4 o = o4[k];
      float &x = (k & 1) ? x1 : x0;
      x = fmaf(o.x, r[k].x, fmaf(o.y, r[k].y, fmaf(o.z, r[k].z, fmaf(o.w, r[k].w, x))));
    }
    red[gi][c] = x0 + x1;
    __syncthreads();
    oh = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NGR; ++g2) oh += red[g2][c];
  } else {
    oh = Os[c];
  }
  if (gi != 0) return;

  // ---- merge with the BF16 segment ----
  float mb = -INFINITY;
#pragma unroll
  for (int s2 = 0; s2 < kBf16Splits; ++s2) mb = fmaxf(mb, bm[s2]);
  float lb = 0.f, obv = 0.f;
  if (mb != -INFINITY) {
#pragma unroll
    for (int s2 = 0; s2 < kBf16Splits; ++s2) {
      if (bm[s2] == -INFINITY) continue;
      const float a = exp2f(bm[s2] - mb);
      lb = fmaf(bl[s2], a, lb);
      obv = fmaf(bov[s2], a, obv);
    }
  }
  const float M = ML[0], L = ML[1];
  const float M2 = fmaxf(M, mb);
  if (M2 == -INFINITY) {
    out[bh * D + c] = 0.f;
    if (c == 0 && lse != nullptr) lse[bh] = -INFINITY;
    return;
  }
  const float ea = (M == -INFINITY) ? 0.f : exp2f(M - M2);
  const float eb = (mb == -INFINITY) ? 0.f : exp2f(mb - M2);
  const float den = fmaf(L, ea, lb * eb);
  out[bh * D + c] = fmaf(oh, ea, obv * eb) / den;
  if (c == 0 && lse != nullptr) lse[bh] = M2 * kLn2 + logf(den);
}

hipError_t launch_merge(const DecodeParams &p, const float *Rv, float *out, float *lse,
                        hipStream_t s) {
  const dim3 grid(p.B * p.Hq), blk(kMergeThreads);
  const size_t lds = (size_t)(p.splits > 0 ? p.splits : 1) * sizeof(float);
  if (p.D == 64) hipLaunchKernelGGL(k_merge<64>, grid, blk, lds, s, p, Rv, out, lse);
  else hipLaunchKernelGGL(k_merge<128>, grid, blk, lds, s, p, Rv, out, lse);
  return hipGetLastError();
}

}  // namespace oscar
