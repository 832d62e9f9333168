// Demotion of BF16 tokens into the rotated INT2 history as a block-level
// device routine, shared by the demotion kernel and the fused decode-step
// kernel.  It rotates, clips, quantises and packs (m.th-motor.com repost of the
// OSCAR article, split-cache paragraph: the oldest recent token is
// rotated/clipped/quantised/packed and moved to the INT2 history, four 2-bit
// values per byte).
//
// Arithmetic (all fp64 so that codes are reproducible bit for bit):
//   x = k . R                      k bf16, R fp32: every product is exact in fp64
//   mx, mn = max, min over the G consecutive channels of a group
//   scale = (c*mx - c*mn) / 3      zero = c*mn      (c = clipping ratio)
//   s_b, z_b = bf16 round-to-nearest-even of scale, zero (directly from fp64)
//   code = clamp(rint((x - z_b) / s_b), 0, 3), or 0 when s_b == 0; with a
//          Lloyd-Max codebook the nearest level (quant_code)
#pragma once
#include "common.hpp"

namespace oscar {

// fp64 -> bf16 bit pattern, round to nearest, ties to even, in one step.
__device__ inline uint16_t f64_to_bf16_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((u >> 63) << 15);
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a == 0) return sign;
  const int bexp = (int)(a >> 52);
  if (bexp == 0x7FF) return (uint16_t)(sign | 0x7F80u | ((a << 12) ? 0x40u : 0u));
  if (bexp == 0) return sign;               // below 2^-1022: rounds to zero in bf16
  int E = bexp - 1023;                      // |x| = 1.f * 2^E
  const uint64_t m = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int shift = 45 + (E < -126 ? (-126 - E) : 0);  // keep 8 bits, fewer when subnormal
  if (shift >= 64) return sign;
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (E < -126) return (uint16_t)(sign | (uint16_t)q);   // q == 128 encodes 2^-126
  if (q == 256) { q = 128; ++E; }
  if (E > 127) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(q & 127));
}

// Arguments of a demotion (one list of n entries).
struct DemoteArgs {
  const uint16_t *bf_k, *bf_v;     // BF16 pools [pages][Hkv][16][D]
  uint8_t *pool;                   // INT2 pool [pages][Hkv][record]
  int Hkv, n;
  int64_t n_bf16_pages, n_int2_pages;
  const int32_t *src, *dst;        // [n] slots page*16 + offset; negative = skip
  const float *Rk, *Rv;            // [Hkv][D][D]; Rv may be NULL (identity)
  const float *clip_k, *clip_v;    // [Hkv]
  const float *codebook;           // [Hkv][2][4] code levels (K, V) or nullptr
  uint32_t *status;                // sticky OSCAR_STATUS_* word or nullptr
};

// The clipped range [c*mn, c*mx] of a group (one fp64 product each) when the
// ratio c is in (0, 1]; a ratio outside it (or NaN) is rejected: the range is
// [+0, +0], so the group gets scale 0, zero 0 and codes 0, and the
// OSCAR_STATUS_CLIP_RANGE bit is set.
__device__ inline void clipped_range(float c, double mx, double mn, uint32_t &flags, double &hi,
                                     double &lo) {
#pragma clang fp contract(off)
  if (c > 0.f && c <= 1.f) {
    hi = (double)c * mx;
    lo = (double)c * mn;
  } else {
    flags |= OSCAR_STATUS_CLIP_RANGE;
    hi = 0.0;
    lo = 0.0;
  }
}

// Factor c of the matrix-core kernel's f16 PV range check on a V scale:
// scale * c must stay below OSCAR_MFMA_V_SCALE_LIMIT.  Uniform levels: the
// weights are p * scale * 2^(8-b) <= 64 * scale, c = 1.  Codebook: the
// weights are p * scale <= 4 * scale and the V levels are f16 operands, c =
// max(1, largest |level|) / 16; a level of magnitude 16 * limit or more (or
// not finite) fails at any scale.
__device__ inline float v_coef_max(const float *lv) {
  if (lv == nullptr) return 1.f;
  float m = 1.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (!(fabsf(lv[k]) < 16.f * OSCAR_MFMA_V_SCALE_LIMIT)) return INFINITY;
    m = fmaxf(m, fabsf(lv[k]));
  }
  return m * (1.f / 16.f);
}

// Status bits of one group's bf16 scale and zero (and, for V, the f16 range
// of the matrix-core kernel's weights).
__device__ inline uint32_t group_flags(double scale, double lo, uint16_t sb, bool isv, const float *lv) {
  uint32_t f = 0;
  if (!isfinite(scale) || !isfinite(lo)) f |= OSCAR_STATUS_NONFINITE;
  if (isv && !(bf16_to_f32(sb) * v_coef_max(lv) < OSCAR_MFMA_V_SCALE_LIMIT))
    f |= OSCAR_STATUS_MFMA_V_RANGE;
  return f;
}

// Code of rotated value x in a group with bf16 scale sd and zero zd (both as
// fp64): with the uniform levels clamp(rint((x - zd) / sd), 0, 3); with a
// codebook lv (4 ascending levels) the nearest level: the count of the
// thresholds (lv[k] + lv[k+1]) / 2 strictly below u = (x - zd) / sd, every
// step one fp64 operation.  0 when sd == 0.
__device__ inline uint32_t quant_code(double x, double zd, double sd, const float *lv) {
  if (sd == 0.0) return 0;
  const double u = (x - zd) / sd;
  if (lv == nullptr) {
    const double qv = fmin(fmax(rint(u), 0.0), 3.0);
    return (uint32_t)qv;
  }
  const double l0 = lv[0], l1 = lv[1], l2 = lv[2], l3 = lv[3];
  return (uint32_t)(u > 0.5 * (l0 + l1)) + (uint32_t)(u > 0.5 * (l1 + l2)) +
         (uint32_t)(u > 0.5 * (l2 + l3));
}

template <int D>
struct DemoteOneShared {
  double ks[D];                        // the token's source values
  double part[256 / (D / 4)][D];       // row-group partial sums of k . R
  double red_mx[2], red_mn[2];         // per wave, groups wider than a wave
  int src, dst;
};

// Demotion of one entry e of the slot lists for KV head j, K (half 0) or V
// (half 1), by a block of 256 threads.  The rotation x = k . R is split like
// the query rotation: thread (row group gi, column quad c4) sums rows
// gi*RPG .. +RPG-1 for columns 4*c4 .. +3 (fp64 fma chain, its R loads issued
// before the token is read), the row groups are added in order in LDS; then
// threads c < D own channel c.  Every thread must call it (it has block
// barriers); it returns once the entry's bytes are written, after every read
// of the source slot.
template <int D, int G>
__device__ __forceinline__ void demote_one_body(const DemoteArgs &a, int e, int j, int half, int tid,
                                                DemoteOneShared<D> &sh) {
#pragma clang fp contract(off)
  constexpr RecLayout RL(D, G);
  constexpr int NC4 = D / 4;           // column quads
  constexpr int NGR = 256 / NC4;       // row groups
  constexpr int RPG = D / NGR;         // rows per group
  constexpr int GW = G < 64 ? G : 64;  // lanes of a group inside one wave
  const bool isv = half != 0;
  const float *R = isv ? a.Rv : a.Rk;
  const int c4 = tid % NC4, gi = tid / NC4;
  // the R rows in two halves (the second requested once the first is used),
  // so that these blocks need fewer registers than the other block kinds of
  // the decode-step prologue allow
  constexpr int RH = RPG / kRotParts;
  float4 r[RH];
  const float4 *Rp = reinterpret_cast<const float4 *>(R + (size_t)j * D * D) + c4;
  if (R != nullptr) {
#pragma unroll
    for (int i = 0; i < RH; ++i) r[i] = Rp[(size_t)(gi * RPG + i) * NC4];
  }
  if (tid == 0) {
    int sv = -1, dv = -1;
    if (e < a.n) { sv = a.src[e]; dv = a.dst[e]; }
    // entries with a negative or out-of-range slot are skipped
    // an entry is skipped by -1 in both lists
    OSCAR_DCHECK((sv < 0 && dv < 0) || (sv >= 0 && dv >= 0 && (sv >> 4) < a.n_bf16_pages &&
                                        (dv >> 4) < a.n_int2_pages), a.status);
    if (sv < 0 || dv < 0 || (sv >> 4) >= a.n_bf16_pages || (dv >> 4) >= a.n_int2_pages) {
      sv = -1;
      dv = -1;
    }
    sh.src = sv;
    sh.dst = dv;
  }
  __syncthreads();
  const int s = sh.src, d = sh.dst;
  if (d < 0) return;                   // uniform over the block
  if (tid < D) {
    const uint16_t *bf = isv ? a.bf_v : a.bf_k;
    const int64_t page = s >> 4, off = s & 15;
    sh.ks[tid] = (double)bf16_to_f32(bf[((page * a.Hkv + j) * kPage + off) * D + tid]);
  }
  __syncthreads();

  double x = 0.0;
  if (R != nullptr) {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    // the R values are widened one row at a time, next to their use (the
    // ordered conversions keep 4 doubles live instead of RPG*4)
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      if (i > 0 && i % RH == 0) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i2 = 0; i2 < RH; ++i2) r[i2] = Rp[(size_t)(gi * RPG + i + i2) * NC4];
      }
      const double ki = sh.ks[gi * RPG + i];
      double rx, ry, rz, rw;
      asm volatile("v_cvt_f64_f32 %0, %1" : "=v"(rx) : "v"(r[i % RH].x));
      asm volatile("v_cvt_f64_f32 %0, %1" : "=v"(ry) : "v"(r[i % RH].y));
      asm volatile("v_cvt_f64_f32 %0, %1" : "=v"(rz) : "v"(r[i % RH].z));
      asm volatile("v_cvt_f64_f32 %0, %1" : "=v"(rw) : "v"(r[i % RH].w));
      a0 = fma(ki, rx, a0);
      a1 = fma(ki, ry, a1);
      a2 = fma(ki, rz, a2);
      a3 = fma(ki, rw, a3);
    }
    sh.part[gi][4 * c4 + 0] = a0;
    sh.part[gi][4 * c4 + 1] = a1;
    sh.part[gi][4 * c4 + 2] = a2;
    sh.part[gi][4 * c4 + 3] = a3;
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int g2 = 0; g2 < NGR; ++g2) x += sh.part[g2][tid];
    }
  } else if (tid < D) {
    x = sh.ks[tid];
  }

  // group max / min (threads c < D: whole waves)
  const int c = tid;
  double mx = x, mn = x;
  if (c < D) {
#pragma unroll
    for (int o = 1; o < GW; o <<= 1) {
      mx = fmax(mx, __shfl_xor(mx, o));
      mn = fmin(mn, __shfl_xor(mn, o));
    }
  }
  if constexpr (G > 64) {
    if (c < D && (c & 63) == 0) { sh.red_mx[c >> 6] = mx; sh.red_mn[c >> 6] = mn; }
    __syncthreads();
    mx = fmax(sh.red_mx[0], sh.red_mx[1]);
    mn = fmin(sh.red_mn[0], sh.red_mn[1]);
  }
  if (c >= D) return;

  uint32_t flags = isfinite(x) ? 0u : (uint32_t)OSCAR_STATUS_NONFINITE;
  double hi, lo;
  clipped_range(isv ? a.clip_v[j] : a.clip_k[j], mx, mn, flags, hi, lo);
  const double scale = (hi - lo) / 3.0;
  const uint16_t sb = f64_to_bf16_rne(scale);
  const uint16_t zb = f64_to_bf16_rne(lo);
  const double sd = (double)bf16_to_f32(sb);
  const double zd = (double)bf16_to_f32(zb);
  const float *lv = a.codebook ? a.codebook + (j * 2 + (isv ? 1 : 0)) * 4 : nullptr;
  const uint32_t code = quant_code(x, zd, sd, lv);
  const int64_t page = d >> 4, off = d & 15;
  uint8_t *rec = a.pool + ((size_t)page * a.Hkv + j) * RL.bytes();
  if ((c % G) == 0) {
    const int o = isv ? RL.vsz((int)off, c / G) : RL.ksz((int)off, c / G);
    *reinterpret_cast<uint32_t *>(rec + o) = (uint32_t)sb | ((uint32_t)zb << 16);
    flags |= group_flags(scale, lo, sb, isv, lv);
  }
  if (flags != 0 && a.status != nullptr) atomicOr(a.status, flags);
  if (!isv) {
    // K: word blk of lane slot 16*kb + t holds channels 64*blk + 16*kb + i of
    // token t at bits 2i
    const int kb = (c & 63) >> 4, blk = c >> 6;
    uint32_t w = code << (2 * (c & 15));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) w |= __shfl_xor(w, o);
    if ((c & 15) == 0) *reinterpret_cast<uint32_t *>(rec + RL.kword(16 * kb + (int)off, blk)) = w;
  } else {
    // V: channel-major, one dword per channel holds the 16 tokens of a page;
    // this token's two bits only
    uint32_t *wp = reinterpret_cast<uint32_t *>(rec + RL.vword(c & 63, c >> 6));
    const int shf = 2 * (int)off;
    atomicAnd(wp, ~(3u << shf));
    atomicOr(wp, code << shf);
  }
}

DemoteArgs demote_args(const oscar_cache &c, int n, const int32_t *src, const int32_t *dst,
                       const float *Rk, const float *Rv, const float *ck, const float *cv);

}  // namespace oscar
