// BF16-history comparison: decode attention over a cache that keeps the whole
// history in BF16 pages (no rotation, no quantisation), the uncompressed
// storage the OSCAR decode speed-ups are stated against (m.th-motor.com repost
// of the OSCAR article, system-gains paragraph and Fig. 5: 100K context,
// batch 1 and large batch, relative to BF16 history storage).  Same paged
// layout as the sink/recent pages: [page][Hkv][16][D] bf16 for K and for V;
// the history page table lists pages of the BF16 pool.
//
// Grid (sequence x KV head x chunk), 4 waves per block; chunk c covers history
// pages [c * pages_per_split, (c + 1) * pages_per_split).  Each wave walks
// every 4th page of the chunk with one page in flight while it processes the
// previous one.  Per page (16 tokens), as in the BF16 segment kernel:
//   QK on v_mfma_f32_16x16x32_bf16 (A = the 16 K rows, B = the g q heads),
//   online softmax per head (running max, rescale of the partial sums),
//   PV on the vector ALU (lane owns channels D/64*lane .. +D/64-1).
// The 4 waves combine in LDS and write one partial per (q head, chunk) in the
// history-chunk slots of the workspace, unrotated (merge with R_v = identity).
#include "common.hpp"

namespace oscar {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int D, int GQ>
__global__ __launch_bounds__(256) void k_bf16_hist(DecodeParams p, const uint16_t *__restrict__ q) {
  constexpr int NM = D / 32;           // QK matrix instructions (32 channels each)
  constexpr int NCH = D / 64;          // PV channels per lane
  static_assert(GQ <= 16, "q heads are the 16 columns of the QK product");
  const int S = p.splits;
  const int unit = blockIdx.x / S, chunk = blockIdx.x % S;
  const int b = unit / p.Hkv, j = unit % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, kb = lane >> 4;

  __shared__ __align__(16) float pb[4][kPage][GQ];   // per wave: p[token][head]
  __shared__ float al[4][GQ];                        // per wave: rescale of each head
  __shared__ float wm[4][GQ], wl[4][GQ];
  __shared__ float wo[4][GQ][D];

  int hl = p.hist_len[b];
  hl = hl < 0 ? 0 : hl;
  hl = hl > p.max_hist_len ? p.max_hist_len : hl;
  hl = hl > kPage * p.hist_stride ? kPage * p.hist_stride : hl;
  const int npages = (hl + kPage - 1) / kPage;
  const int pbeg = chunk * p.pages_per_split;
  const int pend = pbeg + p.pages_per_split < npages ? pbeg + p.pages_per_split : npages;
  const int32_t *ptab = p.hist_pages + (size_t)b * p.hist_stride;

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

  struct Stage {
    v8bf ka[NM];                       // K rows: token r16, channels 32m + 8kb ..
    uint32_t vr[kPage];                // V of the lane's channels, every token
    int ntok;                          // valid tokens (0: no page)
  };
  auto issue = [&](Stage &sg, int k) {            // wave-uniform k
    sg.ntok = 0;
    if (k >= pend) return;
    const int64_t page = ptab[k];
    if (page < 0 || page >= p.num_bf16_pages) return;
    const int nt = hl - k * kPage;
    sg.ntok = nt < kPage ? nt : kPage;
    const size_t base = ((page * p.Hkv + j) * kPage) * D;
    const uint4 *kp = reinterpret_cast<const uint4 *>(p.bf16_k + base + (size_t)r16 * D + 8 * kb);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 v = kp[4 * m];
      __builtin_memcpy(&sg.ka[m], &v, 16);
    }
    const uint16_t *vp = p.bf16_v + base;
#pragma unroll
    for (int tt = 0; tt < kPage; ++tt) {
      if constexpr (NCH == 2) sg.vr[tt] = reinterpret_cast<const uint32_t *>(vp)[(size_t)tt * (D / 2) + lane];
      else sg.vr[tt] = vp[(size_t)tt * D + lane];
    }
  };

  // running state: m_run / l_run of head r16 (replicated over the 4 lane
  // groups), o[h][k] of channel NCH*lane + k for every head
  float m_run = -INFINITY, l_run = 0.f;
  float o[GQ][NCH];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int k = 0; k < NCH; ++k) o[h][k] = 0.f;

  auto process = [&](const Stage &sg) {
    const int ntok = sg.ntok;
    if (ntok == 0) return;
    v4f sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sg.ka[m], qb[m], sacc, 0, 0, 0);
    // lane (kb, h): tokens 4kb + i of head h; slots past the length get -inf
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (4 * kb + i < ntok) ? sacc[i] * p.sm_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));           // >= one valid token: finite
    const float mnew = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - mnew);
    float pr[4], l = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = exp2f(sv[i] - mnew);                  // 0 for masked slots
      l += pr[i];
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_run = fmaf(l_run, alpha, l);
    m_run = mnew;
    if (r16 < GQ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[w][4 * kb + i][r16] = pr[i];
      if (kb == 0) al[w][r16] = alpha;
    }
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float a = al[w][h];
#pragma unroll
      for (int k = 0; k < NCH; ++k) o[h][k] *= a;
    }
    // slots past the length may hold any bits: their V reads as 0
#pragma unroll
    for (int tt = 0; tt < kPage; ++tt) {
      float v[NCH];
      if constexpr (NCH == 2) {
        v[0] = tt < ntok ? bf16_lo(sg.vr[tt]) : 0.f;
        v[1] = tt < ntok ? bf16_hi(sg.vr[tt]) : 0.f;
      } else {
        v[0] = tt < ntok ? bf16_to_f32((uint16_t)sg.vr[tt]) : 0.f;
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float ph = pb[w][tt][h];
#pragma unroll
        for (int k = 0; k < NCH; ++k) o[h][k] = fmaf(ph, v[k], o[h][k]);
      }
    }
    wave_lds_sync();
  };

  // pages pbeg + w, + 4, ...: two stages, one load in flight
  Stage st0, st1;
  int k = pbeg + w;
  issue(st0, k);
  while (k < pend) {
    issue(st1, k + 4);
    process(st0);
    if (k + 4 >= pend) break;
    issue(st0, k + 8);
    process(st1);
    k += 8;
  }

#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) wo[w][h][lane * NCH + kk] = o[h][kk];
  if (kb == 0 && r16 < GQ) { wm[w][r16] = m_run; wl[w][r16] = l_run; }
  __syncthreads();
  float *po = reinterpret_cast<float *>(p.ws + p.L.part_o);
  float *pml = reinterpret_cast<float *>(p.ws + p.L.part_ml);
  for (int i = tid; i < GQ * D; i += 256) {
    const int h = i / D, c = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) M = fmaxf(M, wm[k2][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        if (wm[k2][h] == -INFINITY) continue;
        const float a = exp2f(wm[k2][h] - M);
        L = fmaf(wl[k2][h], a, L);
        O = fmaf(wo[k2][h][c], a, O);
      }
    }
    const size_t row = ((size_t)b * p.Hq + p.q_of_kv[j * GQ + h]) * S + chunk;
    po[row * D + c] = O;
    if (c == 0) {
      pml[row * 2 + 0] = M;
      pml[row * 2 + 1] = L;
    }
  }
}

template <int D>
static void launch_bf16_hist_d(const DecodeParams &p, const uint16_t *q, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv * p.splits), blk(256);
  switch (p.g) {
    case 1: hipLaunchKernelGGL((k_bf16_hist<D, 1>), grid, blk, 0, s, p, q); break;
    case 2: hipLaunchKernelGGL((k_bf16_hist<D, 2>), grid, blk, 0, s, p, q); break;
    case 4: hipLaunchKernelGGL((k_bf16_hist<D, 4>), grid, blk, 0, s, p, q); break;
    default: hipLaunchKernelGGL((k_bf16_hist<D, 8>), grid, blk, 0, s, p, q); break;
  }
}

hipError_t launch_bf16_hist(const DecodeParams &p, const uint16_t *q, hipStream_t s) {
  if (p.D == 64) launch_bf16_hist_d<64>(p, q, s);
  else launch_bf16_hist_d<128>(p, q, s);
  return hipGetLastError();
}

}  // namespace oscar
