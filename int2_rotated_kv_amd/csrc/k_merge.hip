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

// One block (4 waves) per (sequence, q head).  Phase 1 (wave 0) reduces the
// chunk maxima and sums and stages the chunk weights in LDS; phase 2 splits
// the chunks over 256 / D thread groups that sum weighted chunk outputs with
// independent loads; phase 3 un-rotates (the same groups split the R_v row)
// and merges the BF16 segment.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void k_merge(DecodeParams p, const float *__restrict__ Rv,
                                                         float *__restrict__ out, float *__restrict__ lse) {
  constexpr int NGR = kMergeThreads / D;         // thread groups (2 or 4)
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

  // phase 1: M = max_s m_s, L = sum_s l_s 2^(m_s - M)
  if (tid < 64) {
    float M = -INFINITY;
    for (int s2 = lane; s2 < S; s2 += 64) M = fmaxf(M, ml[2 * s2]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f;
    for (int s2 = lane; s2 < S; s2 += 64) {
      const float m = ml[2 * s2];
      const float a = (m == -INFINITY) ? 0.f : exp2f(m - M);
      a_s[s2] = a;
      L = fmaf(ml[2 * s2 + 1], a, L);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    if (lane == 0) { ML[0] = M; ML[1] = L; }
  }
  __syncthreads();

  // phase 2: O[c] = sum_s a_s o_s[c]; chunks gi, gi + NGR, ...  A chunk with
  // weight 0 (no tokens) contributes 0 whatever its stored output holds.
  {
    float O0 = 0.f, O1 = 0.f, O2 = 0.f, O3 = 0.f;
    int s2 = gi;
    for (; s2 + 3 * NGR < S; s2 += 4 * NGR) {
      const float v0 = po[(size_t)s2 * D + c], v1 = po[(size_t)(s2 + NGR) * D + c];
      const float v2 = po[(size_t)(s2 + 2 * NGR) * D + c], v3 = po[(size_t)(s2 + 3 * NGR) * D + c];
      const float w0 = a_s[s2], w1 = a_s[s2 + NGR], w2 = a_s[s2 + 2 * NGR], w3 = a_s[s2 + 3 * NGR];
      O0 = fmaf(w0, w0 != 0.f ? v0 : 0.f, O0);
      O1 = fmaf(w1, w1 != 0.f ? v1 : 0.f, O1);
      O2 = fmaf(w2, w2 != 0.f ? v2 : 0.f, O2);
      O3 = fmaf(w3, w3 != 0.f ? v3 : 0.f, O3);
    }
    for (; s2 < S; s2 += NGR) {
      const float v0 = po[(size_t)s2 * D + c], w0 = a_s[s2];
      O0 = fmaf(w0, w0 != 0.f ? v0 : 0.f, O0);
    }
    red[gi][c] = (O0 + O1) + (O2 + O3);
  }
  __syncthreads();
  if (tid < D) {
    float O = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NGR; ++g2) O += red[g2][tid];
    Os[tid] = O;
  }
  __syncthreads();

  // phase 3: un-rotation O_hist[c] = sum_k O[k] R_v[j][c][k], group gi taking
  // k in [gi*D/NGR, (gi+1)*D/NGR)
  float oh;
  if (Rv != nullptr) {
    constexpr int KPG = D / NGR / 4;             // float4 per group
    const float4 *row = reinterpret_cast<const float4 *>(Rv + ((size_t)j * D + c) * D) + gi * KPG;
    const float4 *o4 = reinterpret_cast<const float4 *>(Os) + gi * KPG;
    float4 r[KPG];
#pragma unroll
    for (int k = 0; k < KPG; ++k) r[k] = row[k];
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

  // BF16 segment partials of this head, then the final merge
  const float *bml = reinterpret_cast<const float *>(p.ws + p.L.bf_ml) + bh * kBf16Splits * 2;
  const float *bo = reinterpret_cast<const float *>(p.ws + p.L.bf_o) + bh * kBf16Splits * D + c;
  float mb = -INFINITY;
#pragma unroll
  for (int s2 = 0; s2 < kBf16Splits; ++s2) mb = fmaxf(mb, bml[2 * s2]);
  float lb = 0.f, obv = 0.f;
  if (mb != -INFINITY) {
#pragma unroll
    for (int s2 = 0; s2 < kBf16Splits; ++s2) {
      const float ms = bml[2 * s2];
      if (ms == -INFINITY) continue;
      const float a = exp2f(ms - mb);
      lb = fmaf(bml[2 * s2 + 1], a, lb);
      obv = fmaf(bo[(size_t)s2 * D], a, obv);
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
