// Demotion of BF16 tokens into the rotated INT2 history (the block routine is
// in demote.hpp), and the BF16 token write.
#include "demote.hpp"

namespace oscar {

// Bulk fills (prompt histories): one wave = 16 consecutive entries of the
// slot lists, one KV head (blockIdx.y), K or V (blockIdx.z), all D channels.
// The rotation of the 16 tokens, X[16][D] = K[16][D] . R, runs on the fp64
// matrix cores (v_mfma_f64_16x16x4f64: A[i][k] from lane i + 16k, B[k][j]
// from lane j + 16k, D[i][j] in lane j + 16 (i mod 4), element i / 4; every
// product of a bf16 value and an fp32 R entry is exact in fp64, the sums are
// fp64) as 4 * D/64 tiles of 16 columns: tile (h, ct) holds channels
// 64h + 4j + ct, so that one 16-byte R load per lane, k-step and half feeds
// four tiles, and lane (ti, kq) = (l % 16, l / 16) ends up with token
// kq + 4r (r = 0..3) at channels 64h + 4ti + ct.  Everything after the
// rotation stays in registers: a group's max and min by reductions over the
// 8 or 16 lanes of a row that hold it; its clipped range and bf16 scale and
// zero computed once, by one of those lanes (which stores the record word),
// and shuffled to the others; the codes; the K words by an OR over the 4
// lanes of a quad, and the V words of a page by an OR over the 4 lanes that
// hold a channel's tokens (whole-page words with one store, others with
// AND/OR atomics).  No barrier after the token load, so the waves of a
// compute unit drift out of phase and one wave's vector work runs under
// another's matrix instructions.
template <int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void k_demote_bulk(DemoteArgs a) {
#pragma clang fp contract(off)
  typedef double v4d __attribute__((ext_vector_type(4)));
  constexpr int T = 16;
  constexpr int XS = D + 4;                    // padded row stride of xs (floats)
  constexpr RecLayout RL(D, G);
  constexpr int NH = D / 64;                   // 64-channel halves (tiles 4h .. 4h + 3)
  constexpr int GL = G >= 64 ? 16 : G / 4;     // lanes of a row that share a group
  constexpr int NGV = G > 64 ? 1 : NH;         // groups a lane holds per token (one per half, or one)
  const int l = threadIdx.x;
  const int ti = l & 15, kq = l >> 4;
  const int j = blockIdx.y;
  const bool isv = blockIdx.z != 0;
  const int e0 = blockIdx.x * T;
  __shared__ __align__(16) float xs[T][XS];    // the 16 tokens' values

  // entry e0 + t in lane t (t < 16); an entry with a negative or out-of-range
  // slot is skipped (-1 in both lists)
  int sv = -1, dv = -1;
  if (l < T) {
    const int e = e0 + l;
    if (e < a.n) { sv = a.src[e]; dv = a.dst[e]; }
    OSCAR_DCHECK((sv < 0 && dv < 0) || (sv >= 0 && dv >= 0 && (sv >> 4) < a.n_bf16_pages &&
                                        (dv >> 4) < a.n_int2_pages), a.status);
    if (sv < 0 || dv < 0 || (sv >> 4) >= a.n_bf16_pages || (dv >> 4) >= a.n_int2_pages) {
      sv = -1;
      dv = -1;
    }
  }
  // the token values into LDS, 16 bytes (8 channels) per load; a skipped
  // entry's token reads as 0
  const uint16_t *bf = isv ? a.bf_v : a.bf_k;
  constexpr int CPT = D / 8;                   // 16-byte chunks per token
#pragma unroll
  for (int i = 0; i < T * CPT / 64; ++i) {
    const int c = l + 64 * i;
    const int t = c / CPT, pp = c % CPT;
    const int s = __shfl(sv, t);
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (s >= 0) {
      const int64_t page = s >> 4, off = s & 15;
      u = *reinterpret_cast<const uint4 *>(bf + ((page * a.Hkv + j) * kPage + off) * D + 8 * pp);
    }
    float4 *dst = reinterpret_cast<float4 *>(&xs[t][8 * pp]);
    dst[0] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    dst[1] = make_float4(bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w));
  }
  __syncthreads();

  // x = k . R: acc[h][ct][r] = X[kq + 4r][64h + 4ti + ct]
  const float *R = isv ? a.Rv : a.Rk;
  const float *Rj = R != nullptr ? R + (size_t)j * D * D : nullptr;
  v4d acc[NH][4];
  if (Rj != nullptr) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[h][ct] = v4d{0.0, 0.0, 0.0, 0.0};
    const float4 *R4 = reinterpret_cast<const float4 *>(Rj) + ti;
#pragma unroll 1
    for (int st = 0; st < D / 4; ++st) {
      const int k = 4 * st + kq;
      const double av = (double)xs[ti][k];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float4 rv = R4[(size_t)k * (D / 4) + 16 * h];
        acc[h][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.x, acc[h][0], 0, 0, 0);
        acc[h][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.y, acc[h][1], 0, 0, 0);
        acc[h][2] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.z, acc[h][2], 0, 0, 0);
        acc[h][3] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)rv.w, acc[h][3], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[h][ct][r] = (double)xs[kq + 4 * r][64 * h + 4 * ti + ct];
  }

  uint32_t flags = 0;
  const float clip = isv ? a.clip_v[j] : a.clip_k[j];
  const float *lv = a.codebook ? a.codebook + (j * 2 + (isv ? 1 : 0)) * 4 : nullptr;
  // this lane's tokens kq + 4r: destination slot (-1 = skipped)
  int dr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) dr[r] = __shfl(dv, kq + 4 * r);
  // the codes of the lane's tokens, 2 bits per token r, per tile
  uint32_t cp[NH][4];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) cp[h][ct] = 0;

  // The bf16 scale and zero of (token r, group v of the lane) are computed
  // once, by lane 4v + r of each GL-lane part of a row (the lanes holding
  // that group), which also stores the record word; the other lanes of the
  // part take them from there.  Group max and min by reductions over the
  // part; each lane keeps those of its own (r, v).
  const int li = ti % GL;
  const int part0 = l - li;                    // first lane of this lane's GL-lane part
  double mxs = 0.0, mns = 0.0;
  int ds = -1;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int v = 0; v < NGV; ++v) {
      double mx = acc[v][0][r], mn = acc[v][0][r];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          if (NGV > 1 && h != v) continue;
          mx = fmax(mx, acc[h][ct][r]);
          mn = fmin(mn, acc[h][ct][r]);
        }
#pragma unroll
      for (int o = 1; o < GL; o <<= 1) {
        mx = fmax(mx, __shfl_xor(mx, o));
        mn = fmin(mn, __shfl_xor(mn, o));
      }
      if (li == 4 * v + r) { mxs = mx; mns = mn; ds = dr[r]; }
    }
  double sd1 = 0.0, zd1 = 0.0;
  if (li < 4 * NGV) {
    double hi, lo;
    clipped_range(clip, mxs, mns, flags, hi, lo);
    const double scale = (hi - lo) / 3.0;
    const uint16_t sb = f64_to_bf16_rne(scale);
    const uint16_t zb = f64_to_bf16_rne(lo);
    sd1 = (double)bf16_to_f32(sb);
    zd1 = (double)bf16_to_f32(zb);
    if (ds >= 0) {
      flags |= group_flags(scale, lo, sb, isv, lv);
      const int g2 = (64 * (li >> 2) + 4 * ti) / G;
      const int off = ds & 15;
      uint8_t *rec = a.pool + ((size_t)(ds >> 4) * a.Hkv + j) * RL.bytes();
      const int o = isv ? RL.vsz(off, g2) : RL.ksz(off, g2);
      *reinterpret_cast<uint32_t *>(rec + o) = (uint32_t)sb | ((uint32_t)zb << 16);
    }
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int d = dr[r];
    const int off = d & 15;
    uint8_t *rec = a.pool + ((size_t)(d >= 0 ? (d >> 4) : 0) * a.Hkv + j) * RL.bytes();
    double sd[NGV], zd[NGV];                   // scale and zero of token kq + 4r's groups
#pragma unroll
    for (int v = 0; v < NGV; ++v) {
      sd[v] = __shfl(sd1, part0 + 4 * v + r);
      zd[v] = __shfl(zd1, part0 + 4 * v + r);
    }
    // codes of token kq + 4r at the lane's channels
    uint32_t code[NH][4];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const double x = acc[h][ct][r];
        if (d >= 0 && !isfinite(x)) flags |= OSCAR_STATUS_NONFINITE;
        const int v = NGV > 1 ? h : 0;
        code[h][ct] = quant_code(x, zd[v], sd[v], lv);
        cp[h][ct] |= code[h][ct] << (2 * r);
      }
    if (!isv) {
      // K word h of lane slot 16 kb + off holds channels 64h + 16kb + i at
      // bits 2i: the 4 lanes of a quad (ti = 4kb .. 4kb + 3) hold 4 channels each
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        uint32_t w = (code[h][0] | (code[h][1] << 2) | (code[h][2] << 4) | (code[h][3] << 6)) << (8 * (ti & 3));
        w |= __shfl_xor(w, 1);
        w |= __shfl_xor(w, 2);
        if (d >= 0 && (ti & 3) == 0)
          *reinterpret_cast<uint32_t *>(rec + RL.kword(16 * (ti >> 2) + off, h)) = w;
      }
    }
  }

  if (isv) {
    // V word of channel c (lane slot c % 64, word c / 64) holds token slot o
    // of the page at bits 2o.  Per page named by the entries (in entry
    // order): the lanes' bits of its tokens, ORed over the 4 lanes that hold
    // a channel (kq = 0..3), stored by the kq = 0 lane.
    uint32_t todo = (uint32_t)__ballot(l < T && dv >= 0);   // tokens not yet stored (uniform)
    while (todo != 0) {
      const int t0 = __builtin_ctz(todo);
      const int P = __shfl(dv, t0) >> 4;                    // uniform
      const uint32_t inp = (uint32_t)__ballot(l < T && dv >= 0 && (dv >> 4) == P);
      todo &= ~inp;
      uint32_t cov = 0;                                     // token slots of P written here
      for (uint32_t m = inp; m != 0; m &= m - 1) cov |= 3u << (2 * (__shfl(dv, __builtin_ctz(m)) & 15));
      uint8_t *rec = a.pool + ((size_t)P * a.Hkv + j) * RL.bytes();
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          uint32_t b = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (dr[r] >= 0 && (dr[r] >> 4) == P) b |= ((cp[h][ct] >> (2 * r)) & 3u) << (2 * (dr[r] & 15));
          b |= __shfl_xor(b, 16);
          b |= __shfl_xor(b, 32);
          if (kq == 0) {
            uint32_t *wp = reinterpret_cast<uint32_t *>(rec + RL.vword(4 * ti + ct, h));
            if (cov == 0xFFFFFFFFu) {
              *wp = b;
            } else {
              atomicAnd(wp, ~cov);
              atomicOr(wp, b);
            }
          }
        }
    }
  }
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
    hipLaunchKernelGGL((k_demote_bulk<D, G>), dim3((a.n + 15) / 16, a.Hkv, 2), dim3(64), 0, s, a);
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
