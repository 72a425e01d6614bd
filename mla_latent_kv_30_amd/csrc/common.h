// Shared device helpers for the gfx950 MLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kDc = 512;      // latent width d_c
constexpr int kDr = 64;       // RoPE key width
constexpr int kDn = 128;      // nope (content) head width
constexpr int kDv = 128;      // value head width
constexpr int kRow = 576;     // cached elements per token: d_c + rope
constexpr int kPage = 64;     // tokens per cache page
constexpr int kMaxHeads = 128;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

// ---- matrix cores ---------------------------------------------------------
// Operand layouts (checked on gfx950):
//   32x32x16: A lane l holds row l%32, k = 8*(l/32)+j; B lane l holds column l%32,
//             k = 8*(l/32)+j; C lane l holds column l%32, rows 8*(r/4)+4*(l/32)+r%4.
//   16x16x32: A row l%16, k = 8*(l/16)+j; B column l%16, same k; C column l%16,
//             rows 4*(l/16)+r.
//   16x16x16: as 16x16x32 with k = 4*(l/16)+j, j < 4.
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16k16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*(short4v*)&a, *(short4v*)&b, c, 0, 0, 0);
}

// ---- LDS ------------------------------------------------------------------
// Transposing LDS read of four 16-bit elements.  Within each group of 16
// lanes, lane 4a+b receives element b of the 8-byte chunks addressed by lanes
// a, a+4, a+8, a+12 (in that order).  So if lane s of the group points at
// row (s/4) and columns 4*(s%4)..4*(s%4)+3 of a row-major tile, lane n of the
// group receives column n of rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* lds_byte_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(lds_byte_ptr));
}
__device__ __forceinline__ int4v lds_read_b128(const void* lds_byte_ptr) {
  return *(const MLA_LDS int4v*)(lds_byte_ptr);
}
// The same reads at a 32-bit LDS byte address (keeps address arithmetic in
// single registers instead of 64-bit generic pointers).
__device__ __forceinline__ bf16x4 lds_read_tr16_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(uintptr_t)addr);
}
__device__ __forceinline__ int4v lds_read_b128_at(uint32_t addr) {
  return *(const MLA_LDS int4v*)(uintptr_t)addr;
}

// This lane's index in its wave, computed afresh at every call: the asm is
// volatile, so a loop recomputes it instead of keeping it live (or spilled).
__device__ __forceinline__ int lane_id_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Value that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS uint8_t*)p;
}

// Asynchronous copy HBM -> LDS of 4 bytes per lane: lane i writes LDS bytes
// [lds_base + 4 i, +4) from buffer offset soff + voff (voff = 4 i); reads past
// the buffer's record count land as zeros.  Issued as inline assembly so the
// compiler does not serialise it against every later LDS read; completion is
// tracked by the caller with wait_vmcnt<>() followed by a workgroup barrier.
// The instruction has no register results and reads its address operands at
// issue; it writes M0, which no compiler-generated code in these kernels
// relies on.  One wait state separates the M0 write from the LDS-DMA that
// reads it.
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base, uint32_t voff,
                                         uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rs), "s"(soff)
               : "memory");
}

// As lds_dma4 with 16 bytes per lane: lane i writes LDS bytes
// [lds_base + 16 i, +16) from buffer offset soff + voff.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base, uint32_t voff,
                                          uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rs), "s"(soff)
               : "memory");
}

// The same copies with the non-temporal hint (nt) when NT: for rows that are
// read once, so that they do not displace reused data from the caches.
template <bool NT>
__device__ __forceinline__ void lds_dma4_hint(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base, uint32_t voff,
                                              uint32_t soff) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen nt lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rs), "s"(soff)
                 : "memory");
  } else {
    lds_dma4(rs, lds_base, voff, soff);
  }
}
template <bool NT>
__device__ __forceinline__ void lds_dma16_hint(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base, uint32_t voff,
                                               uint32_t soff) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rs), "s"(soff)
                 : "memory");
  } else {
    lds_dma16(rs, lds_base, voff, soff);
  }
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// ---- cross-lane -----------------------------------------------------------
// Reductions over the lane pair (l, l^32) and over (l, l^16) inside each
// half-wave, via the gfx950 lane-swap instructions.
__device__ __forceinline__ float pair32_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- RoPE -----------------------------------------------------------------
// Frequencies theta_m = base^(-2m/64), m = 0..31, computed on the host in
// double and passed by value.
struct RopeTable {
  double theta[32];
};

// cos/sin of pos*theta: the angle is formed and reduced modulo 2*pi in double
// (positions reach 2^17 radians), then evaluated in fp32.
__device__ __forceinline__ void rope_cs(int pos, double theta, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)pos * theta;
  a -= two_pi * rint(a * (1.0 / two_pi));
  sincosf((float)a, &s, &c);
}


// ---- split merge and value up-projection ----------------------------------
// Shared by the merge + up-projection kernel and the merge that the decode
// launch runs itself, so that both give the same bits.  A split sequence's
// pieces c (each normalised over its own keys, log-sum-exp lse_c) combine
// as lse = log sum_c e^{lse_c}, z = sum_c e^{lse_c - lse} z_c (the
// "DeepSeek-V3" notes, ekkoxiao.github.io, §潜在向量的作用: o = W^UV z).
// One batch of NB pieces folded into the running maximum mx, the weight sum
// wsum and NCH channel accumulators; padding entries carry lv = -inf.
template <int NB, int NCH>
__device__ __forceinline__ void merge_batch(const float (&lv)[NB], const float (&zv)[NB][NCH], float& mx,
                                            float& wsum, float (&acc)[NCH]) {
  float mb = mx;
#pragma unroll
  for (int u = 0; u < NB; ++u) mb = fmaxf(mb, lv[u]);
  const float alpha = __expf(mx - mb);  // mx = -inf on the first batch: alpha = 0
  wsum *= alpha;
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] *= alpha;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const float w = __expf(lv[u] - mb);
    wsum += w;
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = fmaf(w, zv[u][c], acc[c]);
  }
  mx = mb;
}

// Eight bf16 weights (one 16-byte load) times channels z0 (first four) and
// z1 (last four), accumulated in order.
__device__ __forceinline__ float dot8_bf16(int4v w, float4 z0, float4 z1) {
  const uint32_t w0 = (uint32_t)w[0], w1 = (uint32_t)w[1], w2 = (uint32_t)w[2], w3 = (uint32_t)w[3];
  float t = __uint_as_float(w0 << 16) * z0.x;
  t = fmaf(__uint_as_float(w0 & 0xffff0000u), z0.y, t);
  t = fmaf(__uint_as_float(w1 << 16), z0.z, t);
  t = fmaf(__uint_as_float(w1 & 0xffff0000u), z0.w, t);
  t = fmaf(__uint_as_float(w2 << 16), z1.x, t);
  t = fmaf(__uint_as_float(w2 & 0xffff0000u), z1.y, t);
  t = fmaf(__uint_as_float(w3 << 16), z1.z, t);
  t = fmaf(__uint_as_float(w3 & 0xffff0000u), z1.w, t);
  return t;
}

// Sums of NR row partials over the 64 lanes of a wave (v[r]: this lane's
// partial of row r).  At distance 2^k, k = 5 .. 6 - log2(NR), each lane
// keeps the half of its rows selected by lane bit k and adds its partner's
// copy of that half; the remaining distances add plainly.  Lane l ends with
// row l >> (6 - log2 NR).  Every row is summed over the same pairing
// (distances 32, 16, 8, 4, 2, 1) whatever NR is.
template <int NR>
__device__ __forceinline__ float wave_rows_sum(float (&v)[NR], int lane) {
  constexpr int n = NR == 32 ? 5 : NR == 16 ? 4 : NR == 8 ? 3 : -1;
  static_assert(n > 0, "8, 16 or 32 rows");
#pragma unroll
  for (int k = 5; k >= 6 - n; --k) {
    const int half = 1 << (k - (6 - n));
    const bool upper = (lane >> k) & 1;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      // opaque copies: a select between two array elements would otherwise be
      // folded into a run-time array index, lowered as a compare chain
      float lo = v[i], hi = v[i + half];
      asm volatile("" : "+v"(lo), "+v"(hi));
      const float keep = upper ? hi : lo;
      const float send = upper ? lo : hi;
      v[i] = keep + __shfl_xor(send, 1 << k);
    }
  }
  float r = v[0];
#pragma unroll
  for (int d = (1 << (6 - n)) >> 1; d >= 1; d >>= 1) r += __shfl_xor(r, d);
  return r;
}

}  // namespace mla
