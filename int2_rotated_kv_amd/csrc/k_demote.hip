// Demotion of BF16 tokens into the rotated INT2 history (the block routine is
// in demote.hpp), and the BF16 token write.
#include "demote.hpp"

namespace oscar {

// Bulk fills (prompt histories): one block = 16 consecutive entries of the
// slot lists, one KV head (blockIdx.y), K or V (blockIdx.z).  The rotation of
// the 16 tokens, X[16][D] = K[16][D] . R, runs on the fp64 matrix cores
// (v_mfma_f64_16x16x4f64: every product of a bf16 value and an fp32 R entry is
// exact in fp64, the sums are fp64): wave w computes the channels 64w..64w+63
// as four 16-column tiles, tile ct holding channels 64w + 4j + ct (j = 0..15)
// so that one 16-byte R load per lane and k-step feeds all four tiles.  The
// token values come from LDS (rows padded to D + 4 doubles: at most 2-way
// bank conflicts), the results go back to LDS.  The group statistics (max,
// min, clipped range, bf16 scale and zero) are computed once per (token,
// group) by a few threads each, and thread c then quantises channel c of the
// 16 tokens one by one; a token's V bits are gathered per page word and a word
// is written once all tokens of its page in this block are in (whole-page
// words with one store, others with AND/OR atomics).
template <int D, int G>
__global__ __launch_bounds__(D) void k_demote_bulk(DemoteArgs a) {
#pragma clang fp contract(off)
  typedef double v4d __attribute__((ext_vector_type(4)));
  constexpr int T = 16;
  constexpr int XS = D + 4;                    // padded row stride of xs (doubles)
  constexpr RecLayout RL(D, G);
  constexpr int NG = D / G;                    // groups per token
  constexpr int RT = D / (T * NG);             // threads per (token, group): 2, 4 or 8
  constexpr int PG = G / RT;                   // channels each of them scans (16)
  const int c = threadIdx.x;
  const int j = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const int e0 = blockIdx.x * T;
  __shared__ __align__(16) double xs[T][XS];   // token values, then rotated values
  __shared__ int s_src[T], s_dst[T];
  __shared__ double s_sd[T][NG], s_zd[T][NG];  // bf16 scale and zero as fp64

  const float *R = isv ? a.Rv : a.Rk;
  const float *Rj = R != nullptr ? R + (size_t)j * D * D : nullptr;
  if (c < T) {
    const int e = e0 + c;
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
    s_src[c] = sv;
    s_dst[c] = dv;
  }
  __syncthreads();
  const uint16_t *bf = isv ? a.bf_v : a.bf_k;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int s = s_src[t];
    double v = 0.0;
    if (s >= 0) {
      const int64_t page = s >> 4, off = s & 15;
      v = (double)bf16_to_f32(bf[((page * a.Hkv + j) * kPage + off) * D + c]);
    }
    xs[t][c] = v;
  }
  __syncthreads();

  double x[T];
  if (Rj != nullptr) {
    // lane (ti, kq) = (l % 16, l / 16): A = token ti's value at k = 4s + kq,
    // B = R[4s + kq][64w + 4ti + ct] for tile ct; the result of tile ct,
    // element r, is X[token kq + 4r][channel 64w + 4ti + ct]
    const int l = c & 63, w = c >> 6;
    const int ti = l & 15, kq = l >> 4;
    const float4 *R4 = reinterpret_cast<const float4 *>(Rj) + 16 * w + ti;
    v4d acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int s = 0; s < D / 4; ++s) {
      const int k = 4 * s + kq;
      const double av = xs[ti][k];
      const float4 rv = R4[(size_t)k * (D / 4)];
      acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.x, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.y, acc[1], 0, 0, 0);
      acc[2] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.z, acc[2], 0, 0, 0);
      acc[3] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.w, acc[3], 0, 0, 0);
    }
    __syncthreads();                           // every wave has read the token values
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) xs[kq + 4 * r][64 * w + 4 * ti + ct] = acc[ct][r];
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < T; ++t) x[t] = xs[t][c];

  uint32_t flags = 0;
  const float clip = isv ? a.clip_v[j] : a.clip_k[j];
  const float *lv = a.codebook ? a.codebook + (j * 2 + (isv ? 1 : 0)) * 4 : nullptr;
  // Per (token, group), once: max and min (RT consecutive threads scan PG
  // channels each, then combine by shuffles), the clipped range, and the bf16
  // scale and zero, which the first of them also stores in the record.
  {
    const int pr = c / RT, sub = c % RT;
    const int t = pr / NG, g2 = pr % NG;
    const double *row = &xs[t][g2 * G + sub * PG];
    double mx = row[0], mn = row[0];
#pragma unroll
    for (int i = 1; i < PG; ++i) {
      mx = fmax(mx, row[i]);
      mn = fmin(mn, row[i]);
    }
#pragma unroll
    for (int o = 1; o < RT; o <<= 1) {
      mx = fmax(mx, __shfl_xor(mx, o));
      mn = fmin(mn, __shfl_xor(mn, o));
    }
    if (sub == 0) {
      double hi, lo;
      clipped_range(clip, mx, mn, flags, hi, lo);
      const double scale = (hi - lo) / 3.0;
      const uint16_t sb = f64_to_bf16_rne(scale);
      const uint16_t zb = f64_to_bf16_rne(lo);
      s_sd[t][g2] = (double)bf16_to_f32(sb);
      s_zd[t][g2] = (double)bf16_to_f32(zb);
      const int d = s_dst[t];
      if (d >= 0) {
        const int64_t page = d >> 4, off = d & 15;
        uint8_t *rec = a.pool + ((size_t)page * a.Hkv + j) * RL.bytes();
        const int o = isv ? RL.vsz((int)off, g2) : RL.ksz((int)off, g2);
        *reinterpret_cast<uint32_t *>(rec + o) = (uint32_t)sb | ((uint32_t)zb << 16);
        flags |= group_flags(scale, lo, sb, isv, lv);
      }
    }
  }
  __syncthreads();

  int vpage = -1;                              // V word being gathered (uniform)
  uint32_t vmask = 0, vbits = 0;
  auto flush_v = [&]() {
    if (vpage < 0) return;
    uint8_t *rec = a.pool + ((size_t)vpage * a.Hkv + j) * RL.bytes();
    // V word of channel c: lane slot c % 64, V word c / 64
    uint32_t *wp = reinterpret_cast<uint32_t *>(rec + RL.vword(c & 63, c >> 6));
    if (vmask == 0xFFFFFFFFu) {
      *wp = vbits;
    } else {
      atomicAnd(wp, ~vmask);
      atomicOr(wp, vbits);
    }
  };
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int d = s_dst[t];
    if (d < 0) continue;                       // uniform
    if (!isfinite(x[t])) flags |= OSCAR_STATUS_NONFINITE;
    const uint32_t code = quant_code(x[t], s_zd[t][c / G], s_sd[t][c / G], lv);
    const int64_t page = d >> 4, off = d & 15;
    uint8_t *rec = a.pool + ((size_t)page * a.Hkv + j) * RL.bytes();
    if (!isv) {
      // K: word blk of lane slot 16*kb + t holds channels 64*blk + 16*kb + i of
      // token t at bits 2i
      const int kb = (c & 63) >> 4, blk = c >> 6;
      uint32_t w = code << (2 * (c & 15));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) w |= __shfl_xor(w, o);
      if ((c & 15) == 0) *reinterpret_cast<uint32_t *>(rec + RL.kword(16 * kb + (int)off, blk)) = w;
    } else {
      if ((int)page != vpage) {
        flush_v();
        vpage = (int)page;
        vmask = 0;
        vbits = 0;
      }
      const int shf = 2 * (int)off;
      vmask |= 3u << shf;
      vbits = (vbits & ~(3u << shf)) | (code << shf);
    }
  }
  if (isv) flush_v();
  if (flags != 0 && a.status != nullptr) atomicOr(a.status, flags);
}

// The few tokens of a decode step: one (entry, KV head, K|V) per block of 256
// threads (the body the fused decode-step kernel uses as well).
template <int D, int G>
__global__ __launch_bounds__(256) void k_demote_one(DemoteArgs a) {
  __shared__ DemoteOneShared<D> sh;
  demote_one_body<D, G>(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, sh);
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
static void launch_demote_t(const DemoteArgs &a, hipStream_t s) {
  // few tokens (a decode step): one token per block for parallelism; bulk
  // fills: 16 tokens per block so every R load serves 16 dot products
  if ((a.n + 15) / 16 * a.Hkv * 2 < 1024) {
    hipLaunchKernelGGL((k_demote_one<D, G>), dim3(a.n, a.Hkv, 2), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_demote_bulk<D, G>), dim3((a.n + 15) / 16, a.Hkv, 2), dim3(D), 0, s, a);
  }
}

DemoteArgs demote_args(const oscar_cache &c, int n, const int32_t *src, const int32_t *dst,
                       const float *Rk, const float *Rv, const float *ck, const float *cv) {
  DemoteArgs a;
  a.bf_k = c.bf16_k_pool;
  a.bf_v = c.bf16_v_pool;
  a.pool = c.int2_pool;
  a.Hkv = c.num_kv_heads;
  a.n = n;
  a.n_bf16_pages = c.num_bf16_pages;
  a.n_int2_pages = c.num_int2_pages;
  a.src = src;
  a.dst = dst;
  a.Rk = Rk;
  a.Rv = Rv;
  a.clip_k = ck;
  a.clip_v = cv;
  a.codebook = c.codebook;
  a.status = c.status;
  return a;
}

hipError_t launch_demote(const oscar_cache &c, int n, const int32_t *src, const int32_t *dst,
                         const float *Rk, const float *Rv, const float *ck, const float *cv,
                         hipStream_t s) {
  if (n == 0) return hipSuccess;
  const DemoteArgs a = demote_args(c, n, src, dst, Rk, Rv, ck, cv);
  const int D = c.head_dim, G = c.group_size;
  if (D == 64 && G == 32) launch_demote_t<64, 32>(a, s);
  else if (D == 64 && G == 64) launch_demote_t<64, 64>(a, s);
  else if (D == 128 && G == 32) launch_demote_t<128, 32>(a, s);
  else if (D == 128 && G == 64) launch_demote_t<128, 64>(a, s);
  else if (D == 128 && G == 128) launch_demote_t<128, 128>(a, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace oscar
