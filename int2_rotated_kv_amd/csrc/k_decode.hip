// Decode-attention kernels over the split cache: query rotation, the BF16
// (sink + recent) segment, and the vector-ALU variant of the INT2 history
// segment (m.th-motor.com repost of the OSCAR article, decode stage of the
// split-cache paragraph: the INT2 kernel unpacks, restores scale/zero point
// and accumulates in floating point; the BF16 kernel handles sink/recent; an
// online-softmax merge combines them).
//
// Logits are carried in log2 units: s = (q . k) * sm_scale * log2(e), so every
// exponential is exp2.  Partials per (sequence, q head, chunk) are
// (m = max s, l = sum 2^(s - m), o = sum 2^(s - m) v) in fp32.
#include "common.hpp"
#include "bf16_seg.hpp"
#include "demote.hpp"

namespace oscar {

typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// q . R_k for every (sequence, q head): the history keys are stored as k . R_k,
// so (q . R_k) . (k . R_k) = q . k for an orthogonal R_k.  fp64 accumulation,
// one rounding to fp32.
// ---------------------------------------------------------------------------
// 256 threads per (sequence, q head): thread (group gi, column quad c4) sums
// rows gi*RPG .. +RPG-1 of R for columns 4*c4 .. +3 (one 16-byte load per row,
// all issued together); the row groups are added in LDS.
template <int D>
struct QrotShared {
  double qs[D];
  double part[256 / (D / 4)][D];
  float qf[D];                           // q . R_k rounded to fp32
  int qe;
};

// Largest circular gap among the fractional parts f[0..3] (in [0, 1)) and
// the point that follows it: the four lie on an arc of length 1 - gap that
// starts at that point.
template <typename T>
__device__ inline void arc_of(const T f[4], T &gap, T &start) {
  T a[4] = {f[0], f[1], f[2], f[3]};
  // sorting network for 4 values
  auto cs = [](T &x, T &y) {
    const T lo = x < y ? x : y, hi = x < y ? y : x;
    x = lo;
    y = hi;
  };
  cs(a[0], a[1]);
  cs(a[2], a[3]);
  cs(a[0], a[2]);
  cs(a[1], a[3]);
  cs(a[1], a[2]);
  gap = a[0] + T(1) - a[3];        // the wrap-around gap, then the inner ones
  start = a[0];
  for (int k = 0; k < 3; ++k) {
    const T g = a[k + 1] - a[k];
    if (g > gap) {
      gap = g;
      start = a[k + 1];
    }
  }
}

// The V grid of a Lloyd-Max codebook for the matrix-core kernel's PV, by one
// wave (64 lanes, all active): the four V levels lv as base + beta * h[c]
// with integers -2048 <= h[c] <= 2048 (exact in f16).  With Lmin, Lmax the
// smallest and largest level, r[c] = (L[c] - Lmin) / (Lmax - Lmin) and H in
// [2048, 4095]: beta = (Lmax - Lmin) / H, base = Lmin + (2048 - phi) * beta
// with phi in [0, 1) placing the four values H r[c] + phi as close to
// integers as a common shift can (the centre of the shortest arc that holds
// their fractional parts goes to an integer: error (1 - largest gap) / 2),
// and H the one with the smallest error / H: lane l compares
// H = 2048 + 32 l + i (i < 32) in fp32 on the two inner ratios (those of
// the extremes are 0 and 1, fractional part 0), the wave keeps the smallest
// (the smallest H on a tie).  The chosen grid is formed in fp64: phi, then
// base and beta rounded to fp32 (as the kernel uses them), then
// h[c] = rint((L[c] - base) / beta).  Four equal levels give h = 0 and
// base = Lmin; non-finite levels give h = the levels rounded to f16,
// base = 0 and beta = 1.  out: h[c] in f16 as two words (byte c of out[0]
// the low byte, of out[1] the high byte), base and beta as fp32 bits.
__device__ void v_grid_words(const float *lv4, int lane, uint32_t out[4]) {
  const double lv[4] = {lv4[0], lv4[1], lv4[2], lv4[3]};
  const double lmin = fmin(fmin(lv[0], lv[1]), fmin(lv[2], lv[3]));
  const double lmax = fmax(fmax(lv[0], lv[1]), fmax(lv[2], lv[3]));
  const double sp = lmax - lmin;
  float hv[4] = {(float)lv[0], (float)lv[1], (float)lv[2], (float)lv[3]};
  float base = 0.f, beta = 1.f;
  if (isfinite(lv[0] + lv[1] + lv[2] + lv[3])) {
    base = (float)lmin;
    if (sp == 0.0) {
      hv[0] = hv[1] = hv[2] = hv[3] = 0.f;
    } else {
      double r[4];
      for (int k = 0; k < 4; ++k) r[k] = (lv[k] - lmin) / sp;   // in [0, 1]
      // the two inner ratios: the middle two of the sorted four
      double s4[4] = {r[0], r[1], r[2], r[3]};
      for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 3 - a; ++b) {
          const double x = fmin(s4[b], s4[b + 1]), y = fmax(s4[b], s4[b + 1]);
          s4[b] = x;
          s4[b + 1] = y;
        }
      const float r1 = (float)s4[1], r2 = (float)s4[2];
      float best = INFINITY;
      int bh = 4095;
      for (int i = 0; i < 32; ++i) {
        const int H = 2048 + 32 * lane + i;
        const float hf = (float)H;
        const float t1 = hf * r1, t2 = hf * r2;
        const float f1 = t1 - floorf(t1), f2 = t2 - floorf(t2);
        const float lo = fminf(f1, f2), hi = fmaxf(f1, f2);
        const float gap = fmaxf(fmaxf(lo, hi - lo), 1.f - hi);   // points 0, lo, hi
        const float e = 0.5f * (1.f - gap) * __builtin_amdgcn_rcpf(hf);
        if (e < best) {
          best = e;
          bh = H;
        }
      }
      float bw = best;
      for (int o = 32; o >= 1; o >>= 1) bw = fminf(bw, __shfl_xor(bw, o));
      int hw = best == bw ? bh : 4096;
      for (int o = 32; o >= 1; o >>= 1) hw = min(hw, __shfl_xor(hw, o));
      const int H = __builtin_amdgcn_readfirstlane(hw);
      double f[4];
      for (int k = 0; k < 4; ++k) {
        const double t = H * r[k];
        f[k] = t - floor(t);
      }
      double gap, start;
      arc_of(f, gap, start);
      double phi = -(start + 0.5 * (1.0 - gap));   // the arc's centre onto an integer
      phi -= floor(phi);
      beta = (float)(sp / H);
      base = (float)(lmin + (2048.0 - phi) * (sp / H));
      for (int k = 0; k < 4; ++k) {
        const double h = rint((lv[k] - (double)base) / (double)beta);
        hv[k] = (float)fmin(fmax(h, -2048.0), 2048.0);
      }
    }
  }
  uint32_t lo = 0, hi = 0;
  for (int k = 0; k < 4; ++k) {
    const _Float16 h = (_Float16)hv[k];
    uint16_t hb;
    __builtin_memcpy(&hb, &h, 2);
    lo |= (uint32_t)(hb & 0xFF) << (8 * k);
    hi |= (uint32_t)(hb >> 8) << (8 * k);
  }
  out[0] = lo;
  out[1] = hi;
  out[2] = __float_as_uint(base);
  out[3] = __float_as_uint(beta);
}

template <int D>
__device__ __forceinline__ void qrot_body(const DecodeParams &p, const uint16_t *__restrict__ q,
                                          const float *__restrict__ Rk, int bh, int tid,
                                          QrotShared<D> &sh) {
  constexpr int NC4 = D / 4;             // column quads
  constexpr int NGR = 256 / NC4;         // row groups
  constexpr int RPG = D / NGR;           // rows per group
  const int h = bh % p.Hq;
  const int j = p.kv_of_q[h];
  const int c4 = tid % NC4, gi = tid / NC4;
  if (tid < D) sh.qs[tid] = (double)bf16_to_f32(q[(size_t)bh * D + tid]);
  __syncthreads();
  // the R rows in two halves (the second requested once the first is used),
  // so that these blocks need fewer registers than the other block kinds of
  // the decode-step prologue allow
  const float4 *R = reinterpret_cast<const float4 *>(Rk + (size_t)j * D * D) + c4;
  constexpr int RH = RPG / kRotParts;
  float4 r[RH];
#pragma unroll
  for (int i = 0; i < RH; ++i) r[i] = R[(size_t)(gi * RPG + i) * NC4];
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
  for (int hf = 0; hf < kRotParts; ++hf) {
    if (hf > 0) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < RH; ++i) r[i] = R[(size_t)(gi * RPG + hf * RH + i) * NC4];
    }
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      const double qi = sh.qs[gi * RPG + hf * RH + i];
      a0 = fma(qi, (double)r[i].x, a0);
      a1 = fma(qi, (double)r[i].y, a1);
      a2 = fma(qi, (double)r[i].z, a2);
      a3 = fma(qi, (double)r[i].w, a3);
    }
  }
  sh.part[gi][4 * c4 + 0] = a0;
  sh.part[gi][4 * c4 + 1] = a1;
  sh.part[gi][4 * c4 + 2] = a2;
  sh.part[gi][4 * c4 + 3] = a3;
  __syncthreads();
  if (tid < D) {
    double acc = 0.0;
#pragma unroll
    for (int g2 = 0; g2 < NGR; ++g2) acc += sh.part[g2][tid];
    reinterpret_cast<float *>(p.ws + p.L.qrot)[(size_t)bh * D + tid] = (float)acc;
    sh.qf[tid] = (float)acc;
  }
  if (p.int2_kind != OSCAR_INT2_MFMA) return;

  // Operands of the matrix-core INT2 kernel for this q head (h_in-th of its
  // KV head's g): q_rot as a 21-bit integer qi = rint(q * 2^qe) with
  // |q| * 2^qe < 2^20, split into 7-bit pieces qi >> 14, (qi >> 7) & 127,
  // qi & 127 that fill A rows 4*(h_in % 4) + piece of head quad h_in / 4 (row
  // 4*(h_in % 4) + 3 is zero); per QK step m (64 channels of one group) lane
  // (kb, row) holds in dword e, byte bb the piece of channel
  // 64*blk + 16*kb + 4*bb + e.  Also the exponent and the group sums of q_rot
  // (their zero-point term) times sm_scale*log2(e).
  // With a codebook the K level of code c = b0 + 2*b1 is
  // L0 + cA*c + cB*b0 + cC*b0*b1 (cA = (L2 - L0)/2, cB = L1 - L0 - cA,
  // cC = L3 - L2 - L1 + L0); the kernel contracts the three planes c, b0,
  // b0&b1 into one accumulator (mfma_a_planes): plane pl gets the pieces of
  // rint(fl(q * c_pl) * 2^qe), with |q| * max|c_pl| * 2^qe < 2^20.
  __syncthreads();
  const int G = p.G, NG = D / G;
  const int NPc = mfma_a_planes(D, G, p.g == 8 ? 8 : 4, p.codebook != nullptr);   // A operand sets
  float kc[3] = {1.f, 0.f, 0.f};
  if (NPc == 3) {
    const float *lk = p.codebook + (size_t)j * 8;
    kc[0] = 0.5f * (lk[2] - lk[0]);
    kc[1] = (lk[1] - lk[0]) - kc[0];
    kc[2] = ((lk[3] - lk[2]) - lk[1]) + lk[0];
  }
  if (tid < 64) {
    float mx = 0.f;
    float gs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const float v = sh.qf[tid + 64 * k];
      mx = fmaxf(mx, fabsf(v));
      gs[(tid + 64 * k) / G] += v;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
#pragma unroll
    for (int g2 = 0; g2 < 4; ++g2)
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) gs[g2] += __shfl_xor(gs[g2], o);
    if (NPc == 3) mx *= fmaxf(fmaxf(fabsf(kc[0]), fabsf(kc[1])), fabsf(kc[2]));
    int e = 0;
    if (mx > 0.f) (void)frexpf(mx, &e);          // mx < 2^e
    int qe = mx > 0.f ? 20 - e : 0;              // |q| * 2^qe < 2^20
    qe = qe > 126 ? 126 : (qe < -100 ? -100 : qe);
    if (tid == 0) {
      sh.qe = qe;
      float *hd = reinterpret_cast<float *>(p.ws + p.L.qhd) + (size_t)bh * 8;
      hd[0] = __int_as_float(qe);
      for (int g2 = 0; g2 < NG; ++g2) hd[1 + g2] = gs[g2] * p.sm_log2;
    }
  }
  __syncthreads();
  const int j2 = p.kv_of_q[h];
  int h_in = 0;
  for (int k = 0; k < p.g; ++k) h_in = p.q_of_kv[j2 * p.g + k] == h ? k : h_in;
  const int gpb = G < 64 ? 64 / G : 1;
  const int nqk = mfma_qk_steps(D, G);
  const int nq = (p.g + 3) / 4;          // head quads (the last one partly empty if g < 4)
  const float sc = ldexpf(1.f, sh.qe);
  const int b = bh / p.Hq;
  // the V grid of the codebook, once per KV head (its first q head in
  // sequence 0)
  if (p.codebook != nullptr && b == 0 && h_in == 0 && tid < 64) {
    uint32_t words[4];
    v_grid_words(p.codebook + (size_t)j2 * 8 + 4, tid, words);
    if (tid < 4) reinterpret_cast<uint32_t *>(p.ws + p.L.vgrid)[(size_t)j2 * 4 + tid] = words[tid];
  }
  if (p.n_shared > 0) {
    // the same pieces for the shared-page kernel, whose B operands hold one
    // q row per column: [b][h][piece][D], channel 16k + 4j + i at byte
    // 16k + 4i + j so that dword i of a 16-byte load is the MFMA's k-slot
    // order (byte j of dword i = channel 4j + i, as the unpacked codes)
    int8_t *dst = reinterpret_cast<int8_t *>(p.ws + p.L.qcas) + (size_t)bh * 3 * D;
    for (int t = tid; t < 3 * D; t += 256) {
      const int pc = t / D, c = t % D;
      const int qi = (int)rintf(sh.qf[c] * sc);
      const int piece = pc == 0 ? (qi >> 14) : pc == 1 ? ((qi >> 7) & 127) : (qi & 127);
      dst[pc * D + (c & ~15) + 4 * (c & 3) + ((c >> 2) & 3)] = (int8_t)piece;
    }
  }
  // layout [b][Hkv][head quad][plane][m][lane][dword]
  for (int t = tid; t < NPc * nqk * 64; t += 256) {
    const int pl = t / (nqk * 64), u = t % (nqk * 64);
    const int m = u >> 6, pc = (u >> 4) & 3, kb = (u >> 2) & 3, e = u & 3;
    const int blk = m / gpb, g2 = (64 * blk) / G + m % gpb;
    const float kp = kc[pl];
    uint32_t word = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int c = 64 * blk + 16 * kb + 4 * bb + e;
      int piece = 0;
      if (pc < 3 && c / G == g2) {
        const int qi = (int)rintf((NPc == 1 ? sh.qf[c] : sh.qf[c] * kp) * sc);
        piece = pc == 0 ? (qi >> 14) : pc == 1 ? ((qi >> 7) & 127) : (qi & 127);
      }
      word |= ((uint32_t)piece & 0xFFu) << (8 * bb);
    }
    const int lane = 16 * kb + 4 * (h_in & 3) + pc;
    int32_t *dst = reinterpret_cast<int32_t *>(p.ws + p.L.qpk);
    dst[(((((size_t)b * p.Hkv + j2) * nq + (h_in >> 2)) * NPc + pl) * nqk + m) * 256 + lane * 4 + e] =
        (int32_t)word;
  }
  // with fewer than 4 q heads per KV head the rows of the quad's missing heads
  // are zero (written by the last present head; nq == 1)
  if (p.g < 4 && h_in == p.g - 1) {
    int32_t *dst = reinterpret_cast<int32_t *>(p.ws + p.L.qpk);
    for (int t = tid; t < NPc * nqk * 64 * (4 - p.g); t += 256) {
      const int hh = p.g + t / (NPc * nqk * 64), u = t % (NPc * nqk * 64);
      const int pl = u / (nqk * 64), v = u % (nqk * 64);
      const int m = v >> 6, pc = (v >> 4) & 3, kb = (v >> 2) & 3, e = v & 3;
      const int lane = 16 * kb + 4 * hh + pc;
      dst[((((size_t)b * p.Hkv + j2) * NPc + pl) * nqk + m) * 256 + lane * 4 + e] = 0;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_qrot(DecodeParams p, const uint16_t *__restrict__ q,
                                              const float *__restrict__ Rk) {
  __shared__ QrotShared<D> sh;
  qrot_body<D>(p, q, Rk, blockIdx.x, threadIdx.x, sh);
}

hipError_t launch_qrot(const DecodeParams &p, const uint16_t *q, const float *Rk, hipStream_t s) {
  const int nb = p.B * p.Hq;
  if (p.D == 64) hipLaunchKernelGGL(k_qrot<64>, dim3(nb), dim3(256), 0, s, p, q, Rk);
  else hipLaunchKernelGGL(k_qrot<128>, dim3(nb), dim3(256), 0, s, p, q, Rk);
  return hipGetLastError();
}

template <int D, int GQ>
__global__ __launch_bounds__(256) void k_bf16_seg(DecodeParams p, const uint16_t *__restrict__ q) {
  __shared__ SegShared<D, GQ> sh;
  bf16_seg_body<D, GQ>(p, q, blockIdx.x / p.Hkv, blockIdx.x % p.Hkv, blockIdx.y, threadIdx.x,
                       NewTok{nullptr, nullptr, nullptr}, sh);
}

template <int D>
static void launch_bf16_d(const DecodeParams &p, const uint16_t *q, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv, kBf16Splits), blk(256);
  switch (p.g) {
    case 1: hipLaunchKernelGGL((k_bf16_seg<D, 1>), grid, blk, 0, s, p, q); break;
    case 2: hipLaunchKernelGGL((k_bf16_seg<D, 2>), grid, blk, 0, s, p, q); break;
    case 4: hipLaunchKernelGGL((k_bf16_seg<D, 4>), grid, blk, 0, s, p, q); break;
    default: hipLaunchKernelGGL((k_bf16_seg<D, 8>), grid, blk, 0, s, p, q); break;
  }
}

hipError_t launch_bf16_seg(const DecodeParams &p, const uint16_t *q, hipStream_t s) {
  if (p.D == 64) launch_bf16_d<64>(p, q, s);
  else launch_bf16_d<128>(p, q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-step prologue in one launch: every block is one of
//   [B*Hkv*5]  BF16 segment chunk (b, j, split), reading this step's token
//              from the k_new/v_new inputs at its slot,
//   [B*Hkv*2]  demotion of sequence b's oldest recent token for KV head j, K
//              or V, then the store of that half of head j of b's new token
//              into its BF16 slot (after every read of the demoted slot),
//   [B*Hq]     q . R_k of one (sequence, q head).
// The three kinds are independent, so they run side by side instead of in four
// dependent launches.
// ---------------------------------------------------------------------------
// The three block kinds share one LDS area (about 9.7 KB at D = 128 rather
// than their 28 KB sum), so that LDS does not limit how many blocks a CU
// holds: every kind is bound by the latency of a few dependent memory round
// trips, so the number of blocks in flight sets the launch time.
template <int D, int GQ>
union StepPreShared {
  SegShared<D, GQ> seg;
  DemoteOneShared<D> dem;
  QrotShared<D> qr;
};

template <int D, int G, int GQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kStepPreWaves)))
void k_step_pre(DecodeParams p, const uint16_t *__restrict__ q,
                                                  const float *__restrict__ Rk, DemoteArgs da,
                                                  NewTok nt) {
  __shared__ StepPreShared<D, GQ> sh;
  const int tid = threadIdx.x;
  int bid = blockIdx.x;
  const int nseg = p.B * p.Hkv * kBf16Splits;
  if (bid < nseg) {
    const int bj = bid / kBf16Splits;
    bf16_seg_body<D, GQ>(p, q, bj / p.Hkv, bj % p.Hkv, bid % kBf16Splits, tid, nt, sh.seg);
    return;
  }
  bid -= nseg;
  const int ndem = p.B * p.Hkv * 2;
  if (bid < ndem) {
    const int b = bid / (2 * p.Hkv), j = (bid / 2) % p.Hkv, half = bid % 2;
    demote_one_body<D, G>(da, b, j, half, tid, sh.dem);
    __syncthreads();
    // every read of the demoted slot (this half of head j) is done; b's new
    // token may reuse it
    const int ns = nt.slot[b];
    if (ns >= 0 && (ns >> 4) < p.num_bf16_pages && tid < D / 8) {
      const bool isv = half != 0;
      const int c8 = tid;
      const int64_t page = ns >> 4, off = ns & 15;
      const uint4 *src = reinterpret_cast<const uint4 *>((isv ? nt.v : nt.k) + ((size_t)b * p.Hkv + j) * D);
      uint4 *dst = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(isv ? p.bf16_v : p.bf16_k) +
                                             ((page * p.Hkv + j) * kPage + off) * D);
      dst[c8] = src[c8];
    }
    return;
  }
  bid -= ndem;
  qrot_body<D>(p, q, Rk, bid, tid, sh.qr);
}

template <int D, int G>
static void launch_step_pre_dg(const DecodeParams &p, const uint16_t *q, const float *Rk,
                               const DemoteArgs &da, const NewTok &nt, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv * kBf16Splits + p.B * p.Hkv * 2 + p.B * p.Hq), blk(256);
  switch (p.g) {
    case 1: hipLaunchKernelGGL((k_step_pre<D, G, 1>), grid, blk, 0, s, p, q, Rk, da, nt); break;
    case 2: hipLaunchKernelGGL((k_step_pre<D, G, 2>), grid, blk, 0, s, p, q, Rk, da, nt); break;
    case 4: hipLaunchKernelGGL((k_step_pre<D, G, 4>), grid, blk, 0, s, p, q, Rk, da, nt); break;
    default: hipLaunchKernelGGL((k_step_pre<D, G, 8>), grid, blk, 0, s, p, q, Rk, da, nt); break;
  }
}

hipError_t launch_step_pre(const DecodeParams &p, const oscar_cache &c, const uint16_t *q,
                           const float *Rk, const float *Rv, const float *ck, const float *cv,
                           const int32_t *dsrc, const int32_t *ddst, const int32_t *new_slot,
                           const uint16_t *k_new, const uint16_t *v_new, hipStream_t s) {
  const DemoteArgs da = demote_args(c, p.B, dsrc, ddst, Rk, Rv, ck, cv);
  const NewTok nt{new_slot, k_new, v_new};
  const int D = p.D, G = p.G;
  if (D == 64 && G == 32) launch_step_pre_dg<64, 32>(p, q, Rk, da, nt, s);
  else if (D == 64 && G == 64) launch_step_pre_dg<64, 64>(p, q, Rk, da, nt, s);
  else if (D == 128 && G == 32) launch_step_pre_dg<128, 32>(p, q, Rk, da, nt, s);
  else if (D == 128 && G == 64) launch_step_pre_dg<128, 64>(p, q, Rk, da, nt, s);
  else if (D == 128 && G == 128) launch_step_pre_dg<128, 128>(p, q, Rk, da, nt, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// INT2 history segment, vector-ALU variant.  One block (4 waves) per
// (sequence, KV head, chunk of pages); each wave walks every 4th page of the
// chunk.  Per page (16 tokens):
//   QK:  lane (t = lane%16, part = lane/16) takes the KW K words of token t,
//        part `part` (16 channels each), dots them with q_rot and applies each
//        word's group scale/zero: s = scale * sum(q*code) + zero * sum(q); the
//        four parts are summed across lanes.
//   softmax: running max per head over the 16 token lanes; p = 2^(s - m).
//   PV:  lane owns channels lane + 64k and accumulates
//        sum_t (p*scale_v) * code_v; the zero-point part sum_t p*zero_v depends
//        only on (head, group) and is accumulated on the token lanes.
// With a Lloyd-Max codebook (CB) every code stands for its level L[code]
// (x_hat = zero + scale * L[code]) and the same sums run over L[code].
// ---------------------------------------------------------------------------
// level of a 2-bit code from 4 levels held in registers
__device__ __forceinline__ float code_level(const float (&L)[4], uint32_t cd) {
  const float lo = (cd & 1u) ? L[1] : L[0];
  const float hi = (cd & 1u) ? L[3] : L[2];
  return (cd & 2u) ? hi : lo;
}

template <int D, int G, int GQ, bool CB>
__global__ __launch_bounds__(256) void k_int2_valu(DecodeParams p) {
  constexpr RecLayout RL(D, G);
  constexpr int NG = D / G;       // groups per token (<= 4)
  constexpr int NBLK = D / 64;    // 64-channel blocks per token
  constexpr int KW = D / 64;      // K words per QK lane (D/16 words over 4 parts)
  constexpr int CPL = D / 64;     // PV channels per lane
  static_assert(NG <= 4, "one QK part per group publishes its V scale");

  const int S = p.splits;
  const int unit = blockIdx.x / S;
  const int split = blockIdx.x % S;
  const int b = unit / p.Hkv;
  const int j = unit % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = lane & 15, part = lane >> 4;
  float lk[4] = {0.f, 1.f, 2.f, 3.f}, lvv[4] = {0.f, 1.f, 2.f, 3.f};   // K and V code levels
  if constexpr (CB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lk[i] = p.codebook[j * 8 + i];
      lvv[i] = p.codebook[j * 8 + 4 + i];
    }
  }

  __shared__ float qs[D][GQ];                 // q_rot * sm_log2, heads innermost
  __shared__ float qword[D / 16][GQ];         // sum of q over each K word's 16 channels
  __shared__ float pw[4][NG][16][GQ];         // per wave: p * scale_v per (group, token, head)
  __shared__ float zred[4][NG][GQ];           // per wave: sum_t p * zero_v
  __shared__ float wm[4][GQ], wl[4][GQ];
  __shared__ float wo[4][GQ][D];

  const float *qrot = reinterpret_cast<const float *>(p.ws + p.L.qrot);
  for (int i = tid; i < GQ * D; i += 256) {
    const int h = i / D, c = i % D;
    const int hq = p.q_of_kv[j * GQ + h];
    qs[c][h] = qrot[((size_t)b * p.Hq + hq) * D + c] * p.sm_log2;
  }
  __syncthreads();
  if (tid < (D / 16) * GQ) {
    const int q = tid / GQ, h = tid % GQ;
    const int c0 = 64 * (q % NBLK) + 16 * (q / NBLK);
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += qs[c0 + i][h];
    qword[q][h] = s;
  }
  __syncthreads();

  int hl = p.hist_len[b];
  OSCAR_DCHECK(hl >= 0 && hl <= p.max_hist_len && hl <= kPage * p.hist_stride, p.status);
  hl = hl < 0 ? 0 : hl;
  hl = hl > p.max_hist_len ? p.max_hist_len : hl;
  hl = hl > kPage * p.hist_stride ? kPage * p.hist_stride : hl;
  const int npages = (hl + kPage - 1) / kPage;
  const int p0 = split * p.pages_per_split;
  int p1 = p0 + p.pages_per_split;
  p1 = p1 > npages ? npages : p1;

  float m[GQ], lsum[GQ], zacc[GQ], o[GQ][CPL];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
    zacc[h] = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[h][k] = 0.f;
  }

  for (int pg = p0 + w; pg < p1; pg += 4) {
    const int phys = p.hist_pages[(size_t)b * p.hist_stride + pg];
    OSCAR_DCHECK(phys >= 0 && phys < p.num_int2_pages, p.status);
    if (phys < 0 || phys >= p.num_int2_pages) continue;
    const uint8_t *rec = p.int2_pool + ((size_t)phys * p.Hkv + j) * RL.bytes();
    const int ntok = hl - pg * kPage < kPage ? hl - pg * kPage : kPage;

    // ---- loads ----
    // lane slot `lane` (= 16*part + t) holds this lane's K and V words
    uint32_t kw[KW];
#pragma unroll
    for (int i = 0; i < KW; ++i) kw[i] = *reinterpret_cast<const uint32_t *>(rec + RL.kword(lane, i));
    uint32_t ksz[NG];
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) ksz[g2] = *reinterpret_cast<const uint32_t *>(rec + RL.ksz(t, g2));
    const uint32_t vszw = part < NG ? *reinterpret_cast<const uint32_t *>(rec + RL.vsz(t, part)) : 0u;
    uint32_t vcw[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k)   // channel lane + 64k
      vcw[k] = *reinterpret_cast<const uint32_t *>(rec + RL.vword(lane, k));

    // ---- QK ----
    float sv[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) sv[h] = 0.f;
#pragma unroll
    for (int i = 0; i < KW; ++i) {
      const int q = part * KW + i;
      const int c0 = 64 * (q % NBLK) + 16 * (q / NBLK);
      const int gq = c0 / G;
      float dot[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) dot[h] = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t cd = (kw[i] >> (2 * k)) & 3u;
        const float cf = CB ? code_level(lk, cd) : (float)cd;
#pragma unroll
        for (int h = 0; h < GQ; ++h) dot[h] = fmaf(qs[c0 + k][h], cf, dot[h]);
      }
      const float ksc = bf16_lo(ksz[gq]), kze = bf16_hi(ksz[gq]);
#pragma unroll
      for (int h = 0; h < GQ; ++h) sv[h] += fmaf(ksc, dot[h], kze * qword[q][h]);
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float v = sv[h];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      sv[h] = t < ntok ? v : -INFINITY;
    }

    // ---- online softmax ----
    // (scale, zero) of tokens not yet written are never used: unwritten record
    // bytes may hold any bit pattern
    const float vsc = t < ntok ? bf16_lo(vszw) : 0.f;
    const float vze = t < ntok ? bf16_hi(vszw) : 0.f;
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float pm = sv[h];
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) pm = fmaxf(pm, __shfl_xor(pm, o2));
      const float mn = fmaxf(m[h], pm);
      const float alpha = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - mn);
      const float pr = (sv[h] == -INFINITY) ? 0.f : exp2f(sv[h] - mn);
      m[h] = mn;
      lsum[h] = fmaf(lsum[h], alpha, pr);
      zacc[h] = fmaf(zacc[h], alpha, pr * vze);
#pragma unroll
      for (int k = 0; k < CPL; ++k) o[h][k] *= alpha;
      // lane (t, part < NG) publishes p * scale_v of group `part`
      if (part < NG) pw[w][part][t][h] = pr * vsc;
    }
    wave_lds_sync();

    // ---- PV ----
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      const int gc = c / G;
#pragma unroll 4
      for (int tt = 0; tt < 16; ++tt) {
        const uint32_t cd = (vcw[k] >> (2 * tt)) & 3u;
        const float cf = CB ? code_level(lvv, cd) : (float)cd;
#pragma unroll
        for (int h = 0; h < GQ; ++h) o[h][k] = fmaf(pw[w][gc][tt][h], cf, o[h][k]);
      }
    }
    wave_lds_sync();
  }

  // ---- wave epilogue: sum the per-token-lane partial sums ----
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float l = lsum[h], z = zacc[h];
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1) {
      l += __shfl_xor(l, o2);
      z += __shfl_xor(z, o2);
    }
    lsum[h] = l;
    if (t == 0 && part < NG) zred[w][part][h] = z;
  }
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) wo[w][h][lane + 64 * k] = o[h][k] + zred[w][(lane + 64 * k) / G][h];
    if (lane == 0) { wm[w][h] = m[h]; wl[w][h] = lsum[h]; }
  }
  __syncthreads();

  // ---- combine the 4 waves, write the chunk partial ----
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

template <int D, int G, bool CB>
static void launch_int2_valu_cb(const DecodeParams &p, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv * p.splits), blk(256);
  switch (p.g) {
    case 1: hipLaunchKernelGGL((k_int2_valu<D, G, 1, CB>), grid, blk, 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_int2_valu<D, G, 2, CB>), grid, blk, 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_int2_valu<D, G, 4, CB>), grid, blk, 0, s, p); break;
    default: hipLaunchKernelGGL((k_int2_valu<D, G, 8, CB>), grid, blk, 0, s, p); break;
  }
}

template <int D, int G>
static void launch_int2_valu_dg(const DecodeParams &p, hipStream_t s) {
  if (p.codebook != nullptr) launch_int2_valu_cb<D, G, true>(p, s);
  else launch_int2_valu_cb<D, G, false>(p, s);
}

hipError_t launch_int2_valu(const DecodeParams &p, hipStream_t s) {
  if (p.D == 64 && p.G == 32) launch_int2_valu_dg<64, 32>(p, s);
  else if (p.D == 64 && p.G == 64) launch_int2_valu_dg<64, 64>(p, s);
  else if (p.D == 128 && p.G == 32) launch_int2_valu_dg<128, 32>(p, s);
  else if (p.D == 128 && p.G == 64) launch_int2_valu_dg<128, 64>(p, s);
  else if (p.D == 128 && p.G == 128) launch_int2_valu_dg<128, 128>(p, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace oscar
