// Online-softmax merge of the split cache's partial results (m.th-motor.com
// repost of the OSCAR article, decode stage: the BF16 and INT2 segment results
// are combined by an online-softmax merge).  Per q head:
//   history chunks:  M = max m_s, L = sum l_s 2^(m_s - M), O = sum o_s 2^(m_s - M)
//   un-rotation:     O_hist = O . R_v^T   (the history values are stored as v . R_v)
//   BF16 splits:     (m_b, l_b, o_b) merged the same way (unrotated)
//   final:           M' = max(M, m_b); out = (O_hist 2^(M-M') + o_b 2^(m_b-M'))
//                                            / (L 2^(M-M') + l_b 2^(m_b-M'))
//   lse = M' ln2 + ln(denominator)  (natural-log units)
// One block per (sequence, KV head): its g q heads share every R_v row load.
#include "common.hpp"

namespace oscar {

namespace {
__device__ __forceinline__ void lse_merge(const float *ml, const float *o, int n, int stride_o,
                                          int c, float &M, float &L, float &O) {
  M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, ml[2 * s]);
  L = 0.f;
  O = 0.f;
  if (M == -INFINITY) return;
  for (int s = 0; s < n; ++s) {
    const float ms = ml[2 * s];
    if (ms == -INFINITY) continue;
    const float a = exp2f(ms - M);
    L = fmaf(ml[2 * s + 1], a, L);
    O = fmaf(o[(size_t)s * stride_o + c], a, O);
  }
}
}  // namespace

template <int D, int GQ>
__global__ __launch_bounds__(D) void k_merge(DecodeParams p, const float *__restrict__ Rv,
                                             float *__restrict__ out, float *__restrict__ lse) {
  const int b = blockIdx.x / p.Hkv;
  const int j = blockIdx.x % p.Hkv;
  const int c = threadIdx.x;
  const int S = p.splits;
  __shared__ __align__(16) float Os[GQ][D];
  __shared__ float Ms[GQ], Ls[GQ];

  const float *pml = reinterpret_cast<const float *>(p.ws + p.L.part_ml);
  const float *po = reinterpret_cast<const float *>(p.ws + p.L.part_o);
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const size_t bh = (size_t)b * p.Hq + p.q_of_kv[j * GQ + h];
    float M, L, O;
    lse_merge(pml + bh * S * 2, po + bh * S * D, S, D, c, M, L, O);
    Os[h][c] = O;
    if (c == 0) { Ms[h] = M; Ls[h] = L; }
  }
  __syncthreads();

  float oh[GQ];
  if (Rv != nullptr) {
    // O_hist[h][c] = sum_i O[h][i] * R_v[j][c][i]: thread c streams row c of R_v
    const float4 *row = reinterpret_cast<const float4 *>(Rv + ((size_t)j * D + c) * D);
#pragma unroll
    for (int h = 0; h < GQ; ++h) oh[h] = 0.f;
#pragma unroll 4
    for (int i4 = 0; i4 < D / 4; ++i4) {
      const float4 r = row[i4];
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float4 o4 = *reinterpret_cast<const float4 *>(&Os[h][4 * i4]);
        oh[h] = fmaf(o4.x, r.x, fmaf(o4.y, r.y, fmaf(o4.z, r.z, fmaf(o4.w, r.w, oh[h]))));
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < GQ; ++h) oh[h] = Os[h][c];
  }

  const float *bml = reinterpret_cast<const float *>(p.ws + p.L.bf_ml);
  const float *bo = reinterpret_cast<const float *>(p.ws + p.L.bf_o);
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const size_t bh = (size_t)b * p.Hq + p.q_of_kv[j * GQ + h];
    float mb, lb, ob;
    lse_merge(bml + bh * kBf16Splits * 2, bo + bh * kBf16Splits * D, kBf16Splits, D, c, mb, lb, ob);
    const float M = Ms[h], L = Ls[h];
    const float M2 = fmaxf(M, mb);
    if (M2 == -INFINITY) {
      out[bh * D + c] = 0.f;
      if (c == 0 && lse != nullptr) lse[bh] = -INFINITY;
      continue;
    }
    const float a = (M == -INFINITY) ? 0.f : exp2f(M - M2);
    const float bb = (mb == -INFINITY) ? 0.f : exp2f(mb - M2);
    const float den = fmaf(L, a, lb * bb);
    out[bh * D + c] = fmaf(oh[h], a, ob * bb) / den;
    if (c == 0 && lse != nullptr) lse[bh] = M2 * kLn2 + logf(den);
  }
}

template <int D>
static void launch_merge_d(const DecodeParams &p, const float *Rv, float *out, float *lse,
                           hipStream_t s) {
  const dim3 grid(p.B * p.Hkv), blk(D);
  switch (p.g) {
    case 1: hipLaunchKernelGGL((k_merge<D, 1>), grid, blk, 0, s, p, Rv, out, lse); break;
    case 2: hipLaunchKernelGGL((k_merge<D, 2>), grid, blk, 0, s, p, Rv, out, lse); break;
    case 4: hipLaunchKernelGGL((k_merge<D, 4>), grid, blk, 0, s, p, Rv, out, lse); break;
    default: hipLaunchKernelGGL((k_merge<D, 8>), grid, blk, 0, s, p, Rv, out, lse); break;
  }
}

hipError_t launch_merge(const DecodeParams &p, const float *Rv, float *out, float *lse,
                        hipStream_t s) {
  if (p.D == 64) launch_merge_d<64>(p, Rv, out, lse, s);
  else launch_merge_d<128>(p, Rv, out, lse, s);
  return hipGetLastError();
}

}  // namespace oscar
