// Value up-projection o_i = W_i^UV z_i (the "DeepSeek-V3" notes,
// ekkoxiao.github.io, §潜在向量的作用: values are summed in latent space and
// up-projected afterwards).  W_i^UV is stored [128 d][512 c], so the
// contraction index c is contiguous in both operands: no transposition needed.
#include "common.h"
#include "kernels.h"

namespace mla {

// bf16 weights: o^T[d, n] = sum_c W[d, c] z^T[c, n] on 32x32x16 matrix cores.
// Workgroup = (head, 256 query rows); wave = 64 rows (2 column tiles) x all
// 128 d (4 row tiles).  z is rounded to bf16 on load; accumulation is fp32.
// The contraction runs in chunks of two 16-wide steps whose 16 operand loads
// are issued one chunk ahead, so memory latency overlaps the products.
struct UpChunk {
  int4v w[2][4];     // [step][row tile]: W[32mt + l%32][c0 .. c0+7]
  float4 z[2][2][2]; // [step][column tile][half]: z[row][c0 .. c0+7]
};

// A query row past N reads the workgroup's first row instead: it only feeds
// its own output column, which is not stored.
__device__ __forceinline__ void up_load(UpChunk& ch, const bf16* __restrict__ w, const float* const (&zr)[2], int k0,
                                        int lane) {
  const int g = lane >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c0 = 16 * (k0 + s) + 8 * g;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ch.w[s][mt] = *(const int4v*)(w + (size_t)(32 * mt + (lane & 31)) * kDc + c0);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float4* zp = (const float4*)(zr[nt] + c0);
      ch.z[s][nt][0] = zp[0];
      ch.z[s][nt][1] = zp[1];
    }
  }
}

__global__ void __launch_bounds__(256) upproj_bf16_kernel(UpprojArgs a) {
  const int h = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.y * 256 + wave * 64;
  if (n0 >= a.N) return;
  const int g = lane >> 5;
  const bf16* __restrict__ w = (const bf16*)a.w_uv + (size_t)h * kDv * kDc;
  int nrow[2];
  bool nok[2];
  const float* zr[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    nrow[nt] = n0 + 32 * nt + (lane & 31);
    nok[nt] = nrow[nt] < a.N;
    zr[nt] = a.z + ((size_t)(nok[nt] ? nrow[nt] : n0) * a.H + h) * kDc;
  }
  floatx16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = floatx16{};
  auto compute = [&](const UpChunk& ch) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 bz[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float4 u0 = ch.z[s][nt][0], u1 = ch.z[s][nt][1];
        bz[nt] = bf16x8{f2bf(u0.x), f2bf(u0.y), f2bf(u0.z), f2bf(u0.w),
                        f2bf(u1.x), f2bf(u1.y), f2bf(u1.z), f2bf(u1.w)};
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 aw = __builtin_bit_cast(bf16x8, ch.w[s][mt]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32(aw, bz[nt], acc[mt][nt]);
      }
    }
  };
  // two chunk buffers used in turn (no copy between them, so a chunk's loads
  // are only waited for when that chunk is consumed)
  UpChunk ca, cb;
  up_load(ca, w, zr, 0, lane);
  for (int k0 = 0; k0 < kDc / 16; k0 += 4) {
    up_load(cb, w, zr, k0 + 2, lane);
    compute(ca);
    if (k0 + 4 < kDc / 16) up_load(ca, w, zr, k0 + 4, lane);
    compute(cb);
  }
  // C layout: column = query row, rows d = 32mt + 8(r/4) + 4g + r%4
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!nok[nt]) continue;
    const size_t base = ((size_t)nrow[nt] * a.H + h) * kDv;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * mt + 8 * q4 + 4 * g;
        const floatx16& v = acc[mt][nt];
        if (a.o_bf16) {
          bf16x4 ov = {f2bf(v[4 * q4]), f2bf(v[4 * q4 + 1]), f2bf(v[4 * q4 + 2]), f2bf(v[4 * q4 + 3])};
          *(bf16x4*)((bf16*)a.o + base + d) = ov;
        } else {
          *(float4*)((float*)a.o + base + d) = make_float4(v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]);
        }
      }
  }
}

// Few query rows (decode, N <= 32): workgroup = (head, 16-row tile of d), so
// a launch has H * 8 workgroups.  The 4 waves split the contraction over c
// (128 each); every operand load of a lane is issued before the first
// product (one memory round trip), and the partial sums meet in LDS.
// 16x16x32 matrix cores: A = W (16 d x 32 c), B = z^T (32 c x 16 rows).
constexpr int kUpSmallMaxN = 32;

__global__ void __launch_bounds__(256) upproj_bf16_small_kernel(UpprojArgs a) {
  __shared__ floatx4 red[3][2][64];
  const int h = blockIdx.x, dt = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = lane >> 4, s = lane & 15;
  const bf16* w = (const bf16*)a.w_uv + ((size_t)h * kDv + 16 * dt + s) * kDc + 128 * wave + 8 * G;
  bf16x8 aw[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) aw[kk] = __builtin_bit_cast(bf16x8, *(const int4v*)(w + 32 * kk));
  float4 zr[2][4][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = 16 * nt + s;
    const bool ok = n < a.N;
    const float* zp = a.z + ((size_t)(ok ? n : 0) * a.H + h) * kDc + 128 * wave + 8 * G;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float4 u0 = make_float4(0, 0, 0, 0), u1 = u0;
      if (ok && 16 * nt < a.N) {
        u0 = *(const float4*)(zp + 32 * kk);
        u1 = *(const float4*)(zp + 32 * kk + 4);
      }
      zr[nt][kk][0] = u0;
      zr[nt][kk][1] = u1;
    }
  }
  floatx4 acc[2] = {floatx4{}, floatx4{}};
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float4 u0 = zr[nt][kk][0], u1 = zr[nt][kk][1];
      const bf16x8 bz = {f2bf(u0.x), f2bf(u0.y), f2bf(u0.z), f2bf(u0.w),
                         f2bf(u1.x), f2bf(u1.y), f2bf(u1.z), f2bf(u1.w)};
      acc[nt] = mfma16(aw[kk], bz, acc[nt]);
    }
  }
  if (wave > 0) {
    red[wave - 1][0][lane] = acc[0];
    red[wave - 1][1][lane] = acc[1];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int o = 0; o < 3; ++o) {
    acc[0] += red[o][0][lane];
    acc[1] += red[o][1][lane];
  }
  // C layout: column = query row 16nt + s, rows d = 16 dt + 4G + r
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = 16 * nt + s;
    if (n >= a.N) continue;
    const size_t base = ((size_t)n * a.H + h) * kDv + 16 * dt + 4 * G;
    const floatx4& v = acc[nt];
    if (a.o_bf16) {
      *(bf16x4*)((bf16*)a.o + base) = bf16x4{f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
    } else {
      *(float4*)((float*)a.o + base) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// fp32 weights: one workgroup per (row, head), z in LDS, one thread per d
// with 2 threads sharing a row of W (halves of c), exact fp32 FMA chains.
__global__ void __launch_bounds__(256) upproj_f32_kernel(UpprojArgs a) {
  const int nh = blockIdx.x;
  const int h = nh % a.H;
  __shared__ float zs[kDc];
  __shared__ float part[256];
  const float* zr = a.z + (size_t)nh * kDc;
  for (int i = threadIdx.x; i < kDc; i += 256) zs[i] = zr[i];
  __syncthreads();
  const int d = threadIdx.x >> 1, half = threadIdx.x & 1;
  const float* w = (const float*)a.w_uv + ((size_t)h * kDv + d) * kDc + half * 256;
  float acc = 0.f;
  for (int c = 0; c < 256; ++c) acc = fmaf(w[c], zs[half * 256 + c], acc);
  part[threadIdx.x] = acc;
  __syncthreads();
  if (half == 0) {
    const float v = part[threadIdx.x] + part[threadIdx.x + 1];
    if (a.o_bf16) ((bf16*)a.o)[(size_t)nh * kDv + d] = f2bf(v);
    else ((float*)a.o)[(size_t)nh * kDv + d] = v;
  }
}

hipError_t launch_upproj(const UpprojArgs& a, int w_kind, hipStream_t s) {
  if (w_kind == kKindF32) {
    hipLaunchKernelGGL(upproj_f32_kernel, dim3(a.N * a.H), dim3(256), 0, s, a);
  } else if (a.N <= kUpSmallMaxN) {
    hipLaunchKernelGGL(upproj_bf16_small_kernel, dim3(a.H, kDv / 16), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(upproj_bf16_kernel, dim3(a.H, (a.N + 255) / 256), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
