// Latent-cache append: only (c^KV, RoPE_t(k^R)) is cached per token (the
// "DeepSeek-V3" notes, ekkoxiao.github.io, §KeyValue).  k^R is rotated at
// the token's position on the way in; c^KV is copied, or quantised to OCP
// E4M3 with one fp32 scale per token per 128 channels (the 1x128 tile rule of
// "DeepSeek-V3 Technical Report", process-cxr.github.io, §Fine-grained
// quantization; E4M3 max 448 from "DeepSeek-V3 技术报告精读", §FP8 混合精度训练).
#include <type_traits>

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

// The same stores from fp32 partial sums (plane row stride part_ld, c^KV at
// column part_col): one workgroup per token, wave w
// owning c^KV channels 128w .. 128w+127 (one fp8 tile; two channels per lane)
// and k^R pairs 8w .. 8w+7 (lanes 0..7).  Each channel's partials are loaded
// in batches of 8 and added in plane order, then rounded once to the input
// precision T (what the unsplit product would have written).
// Plane columns col and col+1 (a float2) summed over the planes in plane order,
// 0 + p_0 + p_1 + ...: batches of 16 planes, every load issued before the
// adds (indices past the last plane re-read it and add zero).
template <typename T>
__device__ __forceinline__ float2 sum_planes2(const CacheWriteArgs& a, int t, int col) {
  const size_t plane = (size_t)a.T * a.part_ld;
  const float* p = a.part + (size_t)t * a.part_ld + col;
  float2 s = make_float2(0.f, 0.f);
  for (int i0 = 0; i0 < a.splits; i0 += 16) {
    float2 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = *(const float2*)(p + (size_t)min(i0 + j, a.splits - 1) * plane);
    // planes past the last add zero (exact), so no load waits on a branch
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool in = i0 + j < a.splits;
      s.x += in ? v[j].x : 0.f;
      s.y += in ? v[j].y : 0.f;
    }
  }
  return make_float2((float)(T)s.x, (float)(T)s.y);
}

template <int KIND>
__global__ void __launch_bounds__(256) cache_write_partials_kernel(CacheWriteArgs a) {
  using T = typename std::conditional<KIND == kKindF32, float, bf16>::type;
  const int t = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pos = a.pos[t];
  const int slot = a.slot[t];
  const int ch = 128 * wave + 2 * lane;
  const float2 vv = sum_planes2<T>(a, t, a.part_col + ch);
  const float v0 = vv.x, v1 = vv.y;
  if constexpr (KIND == kKindFp8) {
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
    const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    const float q0 = fminf(fmaxf(__fdiv_rn(v0, scale), -448.0f), 448.0f);
    const float q1 = fminf(fmaxf(__fdiv_rn(v1, scale), -448.0f), 448.0f);
    const uint16_t codes = (uint16_t)(e4m3_rne(q0) | (e4m3_rne(q1) << 8));
    *(uint16_t*)(a.ckv8 + (size_t)slot * kDc + ch) = codes;
    if (lane == 0) a.scale8[(size_t)slot * 4 + wave] = scale;
  } else {
    T* row = (T*)a.rows + (size_t)slot * kRow;
    row[ch] = (T)v0;
    row[ch + 1] = (T)v1;
  }
  if (lane < 8) {
    const int m = 8 * wave + lane;   // RoPE pair
    const float2 xx = sum_planes2<T>(a, t, a.part_col + kDc + 2 * m);
    const float x0 = xx.x, x1 = xx.y;
    float cs, sn;
    rope_cs(pos, a.rope.theta[m], cs, sn);
    T* kr = KIND == kKindFp8 ? (T*)a.kr8 + (size_t)slot * kDr : (T*)a.rows + (size_t)slot * kRow + kDc;
    kr[2 * m] = (T)(x0 * cs - x1 * sn);
    kr[2 * m + 1] = (T)(x0 * sn + x1 * cs);
  }
  // the query's latent c^Q, when it shares the planes (columns 0 .. cq_width-1)
  if (a.cq) {
    for (int c2 = threadIdx.x; 2 * c2 < a.cq_width; c2 += 256) {
      const float2 q = sum_planes2<bf16>(a, t, 2 * c2);
      bf16x2 o;
      o[0] = f2bf(q.x);
      o[1] = f2bf(q.y);
      *(bf16x2*)(a.cq + (size_t)t * a.cq_width + 2 * c2) = o;
    }
  }
}

hipError_t launch_cache_write(const CacheWriteArgs& a, int kind, hipStream_t s) {
  if (a.part) {
    if (kind == kKindF32) hipLaunchKernelGGL(cache_write_partials_kernel<kKindF32>, dim3(a.T), dim3(256), 0, s, a);
    else if (kind == kKindBf16) hipLaunchKernelGGL(cache_write_partials_kernel<kKindBf16>, dim3(a.T), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(cache_write_partials_kernel<kKindFp8>, dim3(a.T), dim3(256), 0, s, a);
    return hipGetLastError();
  }
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
