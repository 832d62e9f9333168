// Demotion of BF16 tokens into the rotated INT2 history (the block routine is
// in demote.hpp), and the BF16 token write.
#include "demote.hpp"

namespace oscar {

// One block: up to T entries of the slot lists (16 for bulk fills, 1 for the
// few tokens of a decode step), one KV head (blockIdx.y), K or V (blockIdx.z).
// Thread c owns rotated channel c of the block's tokens.
template <int D, int G, int T>
__global__ __launch_bounds__(D) void k_demote(DemoteArgs a) {
  __shared__ DemoteShared<D, T> sh;
  demote_body<D, G, T>(a, blockIdx.x * T, blockIdx.y, blockIdx.z, threadIdx.x, true, sh);
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
    hipLaunchKernelGGL((k_demote<D, G, 16>), dim3((a.n + 15) / 16, a.Hkv, 2), dim3(D), 0, s, a);
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
