// Latent-cache append: only (c^KV, RoPE_t(k^R)) is cached per token (the
// "DeepSeek-V3" notes, ekkoxiao.github.io, §KeyValue).  k^R is rotated at
// the token's position on the way in; c^KV is copied, or quantised to OCP
// E4M3 with one fp32 scale per token per 128 channels (the 1x128 tile rule of
// "DeepSeek-V3 Technical Report", process-cxr.github.io, §Fine-grained
// quantization; E4M3 max 448 from "DeepSeek-V3 技术报告精读", §FP8 混合精度训练).
#include "common.h"
#include "kernels.h"

namespace mla {

// One wave per token: lane l handles c^KV channels 8l..8l+7 and, for l < 32,
// RoPE pair l of k^R.
template <typename T>
__global__ void __launch_bounds__(256) cache_write_rows_kernel(CacheWriteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int pos = a.pos ? a.pos[t] : a.pos0 + t;
  const int slot = a.slot ? a.slot[t] : a.bt[pos / kPage] * kPage + pos % kPage;
  T* row = (T*)a.rows + (size_t)slot * kRow;
  const T* c = (const T*)a.c_kv + (size_t)t * kDc;
#pragma unroll
  for (int i = 0; i < 8; ++i) row[8 * lane + i] = c[8 * lane + i];
  if (lane < 32) {
    const T* k = (const T*)a.k_r + (size_t)t * kDr;
    const float x0 = (float)k[2 * lane], x1 = (float)k[2 * lane + 1];
    float cs, sn;
    rope_cs(pos, a.rope.theta[lane], cs, sn);
    row[kDc + 2 * lane] = (T)(x0 * cs - x1 * sn);
    row[kDc + 2 * lane + 1] = (T)(x0 * sn + x1 * cs);
  }
}

// Round a finite fp32 value with |x| <= 448 to the nearest E4M3 code (ties to
// even).  E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals are
// m * 2^-9; the largest finite value is 1.75 * 2^8 = 448.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (ax < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9 (rounding may reach 2^-6 = code 8)
    return sign | (uint32_t)rintf(ax * 512.0f);
  }
  const uint32_t ab = __float_as_uint(ax);
  int e = (int)(ab >> 23) - 127;
  uint32_t m = (ab >> 20) & 7u;
  const uint32_t rem = ab & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) {
    if (++m == 8u) { m = 0; ++e; }
  }
  return sign | ((uint32_t)(e + 7) << 3) | m;
}

__global__ void __launch_bounds__(256) cache_write_fp8_kernel(CacheWriteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int pos = a.pos ? a.pos[t] : a.pos0 + t;
  const int slot = a.slot ? a.slot[t] : a.bt[pos / kPage] * kPage + pos % kPage;
  const bf16* c = (const bf16*)a.c_kv + (size_t)t * kDc + 8 * lane;
  float v[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = bf2f(c[i]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  // 16 lanes cover one 128-channel tile
#pragma unroll
  for (int d = 8; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = __fdiv_rn(v[i], scale);
    q = fminf(fmaxf(q, -448.0f), 448.0f);
    const uint32_t code = e4m3_rne(q);
    if (i < 4) lo |= code << (8 * i); else hi |= code << (8 * (i - 4));
  }
  uint8_t* dst = a.ckv8 + (size_t)slot * kDc + 8 * lane;
  *(uint2*)dst = make_uint2(lo, hi);
  if ((lane & 15) == 0) a.scale8[(size_t)slot * 4 + (lane >> 4)] = scale;
  if (lane < 32) {
    const bf16* k = (const bf16*)a.k_r + (size_t)t * kDr;
    const float x0 = bf2f(k[2 * lane]), x1 = bf2f(k[2 * lane + 1]);
    float cs, sn;
    rope_cs(pos, a.rope.theta[lane], cs, sn);
    bf16* kr = (bf16*)a.kr8 + (size_t)slot * kDr;
    kr[2 * lane] = f2bf(x0 * cs - x1 * sn);
    kr[2 * lane + 1] = f2bf(x0 * sn + x1 * cs);
  }
}

hipError_t launch_cache_write(const CacheWriteArgs& a, int kind, hipStream_t s) {
  const dim3 grid((a.T + 3) / 4), blk(256);
  if (kind == kKindF32) {
    hipLaunchKernelGGL(cache_write_rows_kernel<float>, grid, blk, 0, s, a);
  } else if (kind == kKindBf16) {
    hipLaunchKernelGGL(cache_write_rows_kernel<bf16>, grid, blk, 0, s, a);
  } else {
    hipLaunchKernelGGL(cache_write_fp8_kernel, grid, blk, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
