// Demotion of BF16 tokens into the rotated INT2 history, and the BF16 token
// write.  The demotion rotates, clips, quantises and packs (m.th-motor.com
// repost of the OSCAR article, split-cache paragraph: the oldest recent token
// is rotated/clipped/quantised/packed and moved to the INT2 history, four
// 2-bit values per byte).
//
// Arithmetic (all fp64 so that codes are reproducible bit for bit):
//   x = k . R                      k bf16, R fp32: every product is exact in fp64
//   mx, mn = max, min over the G consecutive channels of a group
//   scale = (c*mx - c*mn) / 3      zero = c*mn      (c = clipping ratio)
//   s_b, z_b = bf16 round-to-nearest-even of scale, zero (directly from fp64)
//   code = clamp(rint((x - z_b) / s_b), 0, 3), or 0 when s_b == 0
#include "common.hpp"

namespace oscar {

// fp64 -> bf16 bit pattern, round to nearest, ties to even, in one step.
__device__ uint16_t f64_to_bf16_rne(double x) {
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

// One block: up to T entries of the slot lists (16 for bulk fills, 1 for the
// few tokens of a decode step), one KV head (blockIdx.y), K or V (blockIdx.z).
// Thread c owns rotated channel c of the block's tokens.
template <int D, int G, int T>
__global__ __launch_bounds__(D) void k_demote(const uint16_t *__restrict__ bf_k,
                                             const uint16_t *__restrict__ bf_v,
                                             uint8_t *__restrict__ pool, int Hkv, int n,
                                             int64_t n_bf16_pages, int64_t n_int2_pages,
                                             const int32_t *__restrict__ src,
                                             const int32_t *__restrict__ dst,
                                             const float *__restrict__ Rk,
                                             const float *__restrict__ Rv,
                                             const float *__restrict__ clip_k,
                                             const float *__restrict__ clip_v) {
  // every fp64 operation below is rounded on its own, as specified: no fusion
  // of the clip products into the subtraction
#pragma clang fp contract(off)
  constexpr RecLayout RL(D, G);
  constexpr int GW = G < 64 ? G : 64;       // lanes of a group inside one wave
  const int c = threadIdx.x;
  const int j = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const int e0 = blockIdx.x * T;

  __shared__ __align__(16) double xs[T][D];
  __shared__ int s_src[T], s_dst[T];
  __shared__ double red_mx[2][T], red_mn[2][T];

  // one token: the D loads of this thread's R column do not depend on the
  // token, so they are issued first
  const float *R = isv ? Rv : Rk;
  float rcol[T == 1 ? D : 1];
  if constexpr (T == 1) {
    if (R != nullptr) {
      const float *Rj = R + (size_t)j * D * D;
#pragma unroll
      for (int i = 0; i < D; ++i) rcol[i] = Rj[(size_t)i * D + c];
    }
  }

  if (c < T) {
    const int e = e0 + c;
    int sv = -1, dv = -1;
    if (e < n) { sv = src[e]; dv = dst[e]; }
    // entries with a negative or out-of-range slot are skipped
    if (sv < 0 || dv < 0 || (sv >> 4) >= n_bf16_pages || (dv >> 4) >= n_int2_pages) {
      sv = -1;
      dv = -1;
    }
    s_src[c] = sv;
    s_dst[c] = dv;
  }
  __syncthreads();

  const uint16_t *bf = isv ? bf_v : bf_k;
  for (int t = 0; t < T; ++t) {
    const int s = s_src[t];
    double v = 0.0;
    if (s >= 0) {
      const int64_t page = s >> 4, off = s & 15;
      v = (double)bf16_to_f32(bf[((page * Hkv + j) * kPage + off) * D + c]);
    }
    xs[t][c] = v;
  }
  __syncthreads();

  double x[T];
  if (R != nullptr && T == 1) {
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int i = 0; i < D; i += 2) {
      const double2 kk = *reinterpret_cast<const double2 *>(&xs[0][i]);
      a0 = fma(kk.x, (double)rcol[i], a0);
      a1 = fma(kk.y, (double)rcol[i + 1], a1);
    }
    x[0] = a0 + a1;
  } else if (R != nullptr) {
    R += (size_t)j * D * D;
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = 0.0;
#pragma unroll 4
    for (int i = 0; i < D; i += 2) {
      const double r0 = (double)R[(size_t)i * D + c];
      const double r1 = (double)R[(size_t)(i + 1) * D + c];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const double2 kk = *reinterpret_cast<const double2 *>(&xs[t][i]);
        x[t] = fma(kk.y, r1, fma(kk.x, r0, x[t]));
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = xs[t][c];
  }

  // group max / min
  double mx[T], mn[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    double a = x[t], b = x[t];
#pragma unroll
    for (int o = 1; o < GW; o <<= 1) {
      a = fmax(a, __shfl_xor(a, o));
      b = fmin(b, __shfl_xor(b, o));
    }
    mx[t] = a;
    mn[t] = b;
  }
  if constexpr (G > 64) {
    const int w = c >> 6;
    if ((c & 63) == 0) {
      for (int t = 0; t < T; ++t) { red_mx[w][t] = mx[t]; red_mn[w][t] = mn[t]; }
    }
    __syncthreads();
    for (int t = 0; t < T; ++t) {
      mx[t] = fmax(red_mx[0][t], red_mx[1][t]);
      mn[t] = fmin(red_mn[0][t], red_mn[1][t]);
    }
  }

  const double clip = (double)(isv ? clip_v[j] : clip_k[j]);
  uint32_t codes[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const double hi = clip * mx[t];
    const double lo = clip * mn[t];
    const double scale = (hi - lo) / 3.0;
    const uint16_t sb = f64_to_bf16_rne(scale);
    const uint16_t zb = f64_to_bf16_rne(lo);
    const double sd = (double)bf16_to_f32(sb);
    const double zd = (double)bf16_to_f32(zb);
    uint32_t code = 0;
    if (sd != 0.0) {
      double qv = rint((x[t] - zd) / sd);
      qv = fmin(fmax(qv, 0.0), 3.0);
      code = (uint32_t)qv;
    }
    codes[t] = code;
    const int d = s_dst[t];
    if (d >= 0 && (c % G) == 0) {
      const int64_t page = d >> 4, off = d & 15;
      uint8_t *rec = pool + ((size_t)page * Hkv + j) * RL.bytes();
      const int o = isv ? RL.vsz((int)off, c / G) : RL.ksz((int)off, c / G);
      *reinterpret_cast<uint32_t *>(rec + o) = (uint32_t)sb | ((uint32_t)zb << 16);
    }
  }

  if (!isv) {
    // K: word blk of lane slot 16*kb + t holds channels 64*blk + 16*kb + i of
    // token t at bits 2i
    const int kb = (c & 63) >> 4, blk = c >> 6;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint32_t w = codes[t] << (2 * (c & 15));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) w |= __shfl_xor(w, o);
      const int d = s_dst[t];
      if (d >= 0 && (c & 15) == 0) {
        const int64_t page = d >> 4, off = d & 15;
        uint8_t *rec = pool + ((size_t)page * Hkv + j) * RL.bytes();
        *reinterpret_cast<uint32_t *>(rec + RL.kword(16 * kb + (int)off, blk)) = w;
      }
    }
  } else {
    // V: channel-major, one dword per channel holds the 16 tokens of a page;
    // entries of this block that share a page are combined first.
    for (int t = 0; t < T; ++t) {
      const int d = s_dst[t];
      if (d < 0) continue;
      const int page = d >> 4;
      bool leader = true;
      for (int u = 0; u < t; ++u)
        if (s_dst[u] >= 0 && (s_dst[u] >> 4) == page) leader = false;
      if (!leader) continue;
      uint32_t mask = 0, bits = 0;
      for (int u = t; u < T; ++u) {
        const int du = s_dst[u];
        if (du >= 0 && (du >> 4) == page) {
          const int sh = 2 * (du & 15);
          mask |= 3u << sh;
          bits = (bits & ~(3u << sh)) | (codes[u] << sh);
        }
      }
      uint8_t *rec = pool + ((size_t)page * Hkv + j) * RL.bytes();
      // V word of channel c: lane slot c % 64, V word c / 64
      uint32_t *wp = reinterpret_cast<uint32_t *>(rec + RL.vword(c & 63, c >> 6));
      if (mask == 0xFFFFFFFFu) {
        *wp = bits;
      } else {
        atomicAnd(wp, ~mask);
        atomicOr(wp, bits);
      }
    }
  }
}

__global__ void k_write_bf16(uint16_t *__restrict__ pk, uint16_t *__restrict__ pv, int Hkv, int D,
                             int64_t n_pages, const int32_t *__restrict__ dst,
                             const uint16_t *__restrict__ kn, const uint16_t *__restrict__ vn) {
  const int e = blockIdx.x;
  const int d = dst[e];
  if (d < 0 || (d >> 4) >= n_pages) return;   // skipped entry
  const int64_t page = d >> 4, off = d & 15;
  const int per8 = Hkv * D / 8;               // 16-byte chunks per token
  for (int i = threadIdx.x; i < per8; i += blockDim.x) {
    const int j = i / (D / 8), c8 = i - j * (D / 8);
    const size_t o = ((page * Hkv + j) * kPage + off) * D / 8 + c8;
    reinterpret_cast<uint4 *>(pk)[o] = reinterpret_cast<const uint4 *>(kn)[(size_t)e * per8 + i];
    reinterpret_cast<uint4 *>(pv)[o] = reinterpret_cast<const uint4 *>(vn)[(size_t)e * per8 + i];
  }
}

hipError_t launch_write_bf16(const oscar_cache &c, int n, const int32_t *dst, const uint16_t *k,
                             const uint16_t *v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_write_bf16, dim3(n), dim3(128), 0, s, c.bf16_k_pool, c.bf16_v_pool,
                     c.num_kv_heads, c.head_dim, c.num_bf16_pages, dst, k, v);
  return hipGetLastError();
}

template <int D, int G>
static void launch_demote_t(const oscar_cache &c, int n, const int32_t *src, const int32_t *dst,
                            const float *Rk, const float *Rv, const float *ck, const float *cv,
                            hipStream_t s) {
  // few tokens (a decode step): one token per block for parallelism; bulk
  // fills: 16 tokens per block so every R load serves 16 dot products
  if ((n + 15) / 16 * c.num_kv_heads * 2 < 1024) {
    dim3 grid(n, c.num_kv_heads, 2);
    hipLaunchKernelGGL((k_demote<D, G, 1>), grid, dim3(D), 0, s, c.bf16_k_pool, c.bf16_v_pool,
                       c.int2_pool, c.num_kv_heads, n, c.num_bf16_pages, c.num_int2_pages, src, dst,
                       Rk, Rv, ck, cv);
  } else {
    dim3 grid((n + 15) / 16, c.num_kv_heads, 2);
    hipLaunchKernelGGL((k_demote<D, G, 16>), grid, dim3(D), 0, s, c.bf16_k_pool, c.bf16_v_pool,
                       c.int2_pool, c.num_kv_heads, n, c.num_bf16_pages, c.num_int2_pages, src, dst,
                       Rk, Rv, ck, cv);
  }
}

hipError_t launch_demote(const oscar_cache &c, int n, const int32_t *src, const int32_t *dst,
                         const float *Rk, const float *Rv, const float *ck, const float *cv,
                         hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int D = c.head_dim, G = c.group_size;
  if (D == 64 && G == 32) launch_demote_t<64, 32>(c, n, src, dst, Rk, Rv, ck, cv, s);
  else if (D == 64 && G == 64) launch_demote_t<64, 64>(c, n, src, dst, Rk, Rv, ck, cv, s);
  else if (D == 128 && G == 32) launch_demote_t<128, 32>(c, n, src, dst, Rk, Rv, ck, cv, s);
  else if (D == 128 && G == 64) launch_demote_t<128, 64>(c, n, src, dst, Rk, Rv, ck, cv, s);
  else if (D == 128 && G == 128) launch_demote_t<128, 128>(c, n, src, dst, Rk, Rv, ck, cv, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace oscar
