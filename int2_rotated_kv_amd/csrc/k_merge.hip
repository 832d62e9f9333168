// Online-softmax merge of the split cache's partial results (m.th-motor.com
// repost of the OSCAR article, decode stage: the BF16 and INT2 segment results
// are combined by an online-softmax merge).
//   history chunks:  M = max m_s, L = sum l_s 2^(m_s - M), O = sum o_s 2^(m_s - M)
//   un-rotation:     O_hist = O . R_v^T   (the history values are stored as v . R_v)
//   with BF16 part:  M' = max(M, m_b); out = (O_hist 2^(M-M') + o_b 2^(m_b-M'))
//                                            / (L 2^(M-M') + l_b 2^(m_b-M'))
//   lse = M' ln2 + ln(denominator)  (natural-log units)
#include "common.hpp"

namespace oscar {

template <int D>
__global__ __launch_bounds__(D) void k_merge(DecodeParams p, const float *__restrict__ Rv,
                                             float *__restrict__ out, float *__restrict__ lse) {
  const int bh = blockIdx.x;
  const int h = bh % p.Hq;
  const int j = p.kv_of_q[h];
  const int c = threadIdx.x;
  const int lane = c & 63, w = c >> 6;
  const int S = p.splits;
  __shared__ float Os[D], Oh[D];

  const float *pml = reinterpret_cast<const float *>(p.ws + p.L.part_ml) + (size_t)bh * S * 2;
  const float *po = reinterpret_cast<const float *>(p.ws + p.L.part_o) + (size_t)bh * S * D;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pml[2 * s]);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ms = pml[2 * s];
      if (ms == -INFINITY) continue;
      const float a = exp2f(ms - M);
      L = fmaf(pml[2 * s + 1], a, L);
      O = fmaf(po[(size_t)s * D + c], a, O);
    }
  }
  Os[c] = O;
  __syncthreads();
  if (Rv != nullptr) {
    // row r of R_v dotted with O, one wave per row, rows split over the waves
    const float *R = Rv + (size_t)j * D * D;
    for (int r = w; r < D; r += D / 64) {
      float acc = 0.f;
#pragma unroll
      for (int i = lane; i < D; i += 64) acc = fmaf(R[(size_t)r * D + i], Os[i], acc);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
      if (lane == 0) Oh[r] = acc;
    }
  } else {
    Oh[c] = Os[c];
  }
  __syncthreads();

  const float mb = reinterpret_cast<const float *>(p.ws + p.L.bf_ml)[(size_t)bh * 2 + 0];
  const float lb = reinterpret_cast<const float *>(p.ws + p.L.bf_ml)[(size_t)bh * 2 + 1];
  const float ob = reinterpret_cast<const float *>(p.ws + p.L.bf_o)[(size_t)bh * D + c];
  const float M2 = fmaxf(M, mb);
  if (M2 == -INFINITY) {
    out[(size_t)bh * D + c] = 0.f;
    if (c == 0 && lse != nullptr) lse[bh] = -INFINITY;
    return;
  }
  const float a = (M == -INFINITY) ? 0.f : exp2f(M - M2);
  const float bb = (mb == -INFINITY) ? 0.f : exp2f(mb - M2);
  const float den = fmaf(L, a, lb * bb);
  out[(size_t)bh * D + c] = fmaf(Oh[c], a, ob * bb) / den;
  if (c == 0 && lse != nullptr) lse[bh] = M2 * kLn2 + logf(den);
}

hipError_t launch_merge(const DecodeParams &p, const float *Rv, float *out, float *lse,
                        hipStream_t s) {
  const int nb = p.B * p.Hq;
  if (p.D == 64) hipLaunchKernelGGL(k_merge<64>, dim3(nb), dim3(64), 0, s, p, Rv, out, lse);
  else hipLaunchKernelGGL(k_merge<128>, dim3(nb), dim3(128), 0, s, p, Rv, out, lse);
  return hipGetLastError();
}

}  // namespace oscar
