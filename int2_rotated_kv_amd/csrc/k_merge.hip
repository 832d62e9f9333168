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

constexpr int kMergeRegChunks = 8;       // chunk rows per thread loaded up front
constexpr int kMergeWideRows = 512;      // 1024-thread blocks below this many rows

// Sum of RPT values per lane across the LPR lanes of a row group, folded so
// that every exchange also halves the number of values: after log2(LPR) steps
// lane l holds the full sum of value number `base`, with RPT <= LPR.
template <int CNT, int O>
__device__ __forceinline__ void fold_sum(float *v, int lane, int &base) {
  if constexpr (O >= 1) {
    if constexpr (CNT > 1) {
      constexpr int H = CNT / 2;
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, O);
      }
      if (up) base += H;
      fold_sum<H, O / 2>(v, lane, base);
    } else {
      v[0] += __shfl_xor(v[0], O);
      fold_sum<1, O / 2>(v, lane, base);
    }
  }
}

// One block of NT threads per (sequence, q head).  A row of D floats (a chunk
// output, a row of R_v) is read by D/4 consecutive lanes, 16 bytes each, so
// every load is a contiguous row segment.  Every load the block needs is
// issued first: the chunk (m, l) pairs (thread s holds chunk s), the first
// kMergeRegChunks chunk rows of each row group, the thread's float4 of RPT
// rows of R_v and the BF16 partials; the rest is shuffles and LDS exchanges.
// NT = 1024 serves long chunk lists of a few (sequence, q head) rows (a
// small batch split many ways), 256 the rest: with many rows, a longer list
// is walked by the 256 threads in turn (a 1024-thread block per row costs
// more in block turnover than the longer walk).
template <int D, int NT>
__global__ __launch_bounds__(NT) void k_merge(DecodeParams p, const float *__restrict__ Rv,
                                              float *__restrict__ out, float *__restrict__ lse) {
  constexpr int LPR = D / 4;                   // lanes per row (float4 each)
  constexpr int RG = NT / LPR;                 // row groups
  constexpr int NW = NT / 64;                  // waves
  constexpr int RPT = D / RG;                  // R_v rows per thread
  static_assert(RPT >= 1 && RPT <= LPR && (RPT & (RPT - 1)) == 0, "R_v row split");
  const size_t bh = blockIdx.x;
  const int j = p.kv_of_q[bh % p.Hq];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cq = tid % LPR, rg = tid / LPR;
  const int S = p.splits;                      // row stride of the partials
  // chunks of this sequence: all S, or the slots the matrix-core kernel used
  int n = S;
  if (S > 0 && p.int2_kind == OSCAR_INT2_MFMA) {
    // the cascade slots of shared pages, then the matrix-core kernel's
    const int b = (int)(bh / p.Hq);
    n = p.mfma_balanced ? reinterpret_cast<const int *>(p.ws + p.L.nslots)[b] : p.mfma_parts;
    if (p.n_shared > 0) n += cascade_slots(p, b, nullptr);
    OSCAR_DCHECK(n <= S, p.status);
    n = n < S ? n : S;
  }
  extern __shared__ float a_s[];               // [S] chunk weights 2^(m_s - M)
  __shared__ float4 red[NW][LPR];              // per-wave channel sums
  __shared__ __align__(16) float Os[D];        // merged history output (rotated basis)
  __shared__ float OH[D];                      // un-rotated history output
  __shared__ float wred[2][NW];

  const float2 *ml = reinterpret_cast<const float2 *>(p.ws + p.L.part_ml) + bh * S;
  const float4 *po = reinterpret_cast<const float4 *>(p.ws + p.L.part_o) + bh * S * LPR + cq;
  const float *bml = reinterpret_cast<const float *>(p.ws + p.L.bf_ml) + bh * kBf16Splits * 2;
  const float *bo = reinterpret_cast<const float *>(p.ws + p.L.bf_o) + bh * kBf16Splits * D + tid;

  // ---- every load up front ----
  float2 mlv = make_float2(-INFINITY, 0.f);
  if (tid < n) mlv = ml[tid];
  float4 ov[kMergeRegChunks];                  // chunk rows rg + RG*k, channels 4cq..4cq+3
#pragma unroll
  for (int k = 0; k < kMergeRegChunks; ++k) {
    const int s2 = rg + RG * k;
    ov[k] = s2 < n ? po[(size_t)s2 * LPR] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 r[RPT];                               // R_v[j] rows rg + RG*i, columns 4cq..4cq+3
  if (Rv != nullptr) {
    const float4 *rrow = reinterpret_cast<const float4 *>(Rv + (size_t)j * D * D) + cq;
#pragma unroll
    for (int i = 0; i < RPT; ++i) r[i] = rrow[(size_t)(rg + RG * i) * LPR];
  }
  float bm[kBf16Splits], bl[kBf16Splits], bov[kBf16Splits];
#pragma unroll
  for (int s2 = 0; s2 < kBf16Splits; ++s2) {
    bm[s2] = bml[2 * s2];
    bl[s2] = bml[2 * s2 + 1];
    bov[s2] = tid < D ? bo[(size_t)s2 * D] : 0.f;
  }

  // ---- chunk weights: M = max m_s, L = sum l_s 2^(m_s - M) ----
  float M = mlv.x;
  for (int s2 = tid + NT; s2 < n; s2 += NT) M = fmaxf(M, ml[s2].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) wred[0][wv] = M;
  __syncthreads();
  M = wred[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, wred[0][w]);
  float L = 0.f;
  for (int s2 = tid; s2 < n; s2 += NT) {
    const float2 t = s2 == tid ? mlv : ml[s2];
    const float a = (t.x == -INFINITY) ? 0.f : exp2f(t.x - M);
    a_s[s2] = a;
    L = fmaf(t.y, a, L);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  if (lane == 0) wred[1][wv] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += wred[1][w];

  // ---- O = sum_s a_s o_s; a chunk with weight 0 (no tokens) adds 0 whatever
  // its stored output holds ----
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kMergeRegChunks; ++k) {
    const int s2 = rg + RG * k;
    const float wgt = s2 < n ? a_s[s2] : 0.f;
    if (wgt != 0.f) {
      acc.x = fmaf(wgt, ov[k].x, acc.x);
      acc.y = fmaf(wgt, ov[k].y, acc.y);
      acc.z = fmaf(wgt, ov[k].z, acc.z);
      acc.w = fmaf(wgt, ov[k].w, acc.w);
    }
  }
  for (int s2 = rg + RG * kMergeRegChunks; s2 < n; s2 += RG) {
    const float wgt = a_s[s2];
    if (wgt != 0.f) {
      const float4 v = po[(size_t)s2 * LPR];
      acc.x = fmaf(wgt, v.x, acc.x);
      acc.y = fmaf(wgt, v.y, acc.y);
      acc.z = fmaf(wgt, v.z, acc.z);
      acc.w = fmaf(wgt, v.w, acc.w);
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {         // row groups inside the wave
    acc.x += __shfl_xor(acc.x, o);
    acc.y += __shfl_xor(acc.y, o);
    acc.z += __shfl_xor(acc.z, o);
    acc.w += __shfl_xor(acc.w, o);
  }
  if (lane < LPR) red[wv][lane] = acc;
  __syncthreads();
  if (tid < D) {
    const float *rf = reinterpret_cast<const float *>(&red[0][0]);
    float O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) O += rf[w * D + tid];
    Os[tid] = O;
  }
  __syncthreads();

  // ---- un-rotation O_hist[c] = sum_k O[k] R_v[j][c][k] ----
  float oh = 0.f;
  if (Rv != nullptr) {
    const float4 o4 = reinterpret_cast<const float4 *>(Os)[cq];
    float v[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      v[i] = fmaf(o4.x, r[i].x, fmaf(o4.y, r[i].y, fmaf(o4.z, r[i].z, o4.w * r[i].w)));
    int base = 0;
    fold_sum<RPT, LPR / 2>(v, lane, base);
    OH[rg + RG * base] = v[0];                 // the lanes of one row agree
    __syncthreads();
    if (tid < D) oh = OH[tid];
  } else if (tid < D) {
    oh = Os[tid];
  }
  if (tid >= D) return;

  // ---- merge with the BF16 segment ----
  const int c = tid;
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

template <int D>
static void launch_merge_d(const DecodeParams &p, const float *Rv, float *out, float *lse,
                           size_t lds, hipStream_t s) {
  const dim3 grid(p.B * p.Hq);
  if (p.splits > 64 && p.B * p.Hq < kMergeWideRows)
    hipLaunchKernelGGL((k_merge<D, 1024>), grid, dim3(1024), lds, s, p, Rv, out, lse);
  else hipLaunchKernelGGL((k_merge<D, 256>), grid, dim3(256), lds, s, p, Rv, out, lse);
}

hipError_t launch_merge(const DecodeParams &p, const float *Rv, float *out, float *lse,
                        hipStream_t s) {
  const size_t lds = (size_t)(p.splits > 0 ? p.splits : 1) * sizeof(float);
  if (p.D == 64) launch_merge_d<64>(p, Rv, out, lse, lds, s);
  else launch_merge_d<128>(p, Rv, out, lse, lds, s);
  return hipGetLastError();
}

}  // namespace oscar
