// Measured ceilings of the units the attention kernels are bound by: HBM
// streaming reads, dense bf16 matrix-core issue (the two MFMA shapes the
// kernels use) and LDS reads per compute unit (plain 16-byte reads and the
// transposing 8-byte reads of the value product).  Each kernel does nothing
// but the operation it measures, on in-register or in-LDS data where it can,
// and folds what it read into one value per workgroup so that no load or
// product can be removed.  The caller times the launch; the work per launch
// is returned by the entry point (mla_ceilings.h).
#include "mla_ceilings.h"
#include "common.h"

namespace mla {
namespace {

constexpr int kHbmThreads = 256;
constexpr int kHbmUnroll = 8;  // 16-byte loads in flight per thread

// Grid-stride streaming read: each thread keeps kHbmUnroll 16-byte loads in
// flight, consecutive lanes on consecutive 16-byte chunks.
__global__ void __launch_bounds__(kHbmThreads) hbm_read_kernel(const int4v* __restrict__ p, long long n16,
                                                               float* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * kHbmThreads;
  long long i = (long long)blockIdx.x * kHbmThreads + threadIdx.x;
  int4v acc = {0, 0, 0, 0};
  for (; i + (kHbmUnroll - 1) * stride < n16; i += kHbmUnroll * stride) {
    int4v v[kHbmUnroll];
#pragma unroll
    for (int k = 0; k < kHbmUnroll; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kHbmUnroll; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  // every lane ran the loads; one value per workgroup keeps them alive
  if (threadIdx.x == 0) sink[blockIdx.x] = __int_as_float(x);
}

// Dense matrix-core issue: every wave runs `iters` rounds of NCHAIN
// independent accumulation chains (so no product waits for the one before).
// Two waves per SIMD, as in the attention kernels; under that register
// budget the products accumulate in ordinary VGPRs in place (with the
// accumulation registers free, 16x16 accumulators were copied between them
// every round).
template <int SHAPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = f2bf(1.0f + 0.001f * (float)((tid + j) & 7));
    b[j] = f2bf(0.5f - 0.001f * (float)((tid * 3 + j) & 7));
  }
  float out = 0.f;
  if constexpr (SHAPE == MLA_CEILING_MFMA_32X32X16) {
    constexpr int NCHAIN = 4;
    floatx16 c[NCHAIN];
#pragma unroll
    for (int k = 0; k < NCHAIN; ++k) c[k] = floatx16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < NCHAIN; ++k) c[k] = mfma32(a, b, c[k]);
    }
#pragma unroll
    for (int k = 0; k < NCHAIN; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) out += c[k][r];
  } else {
    constexpr int NCHAIN = 8;
    floatx4 c[NCHAIN];
#pragma unroll
    for (int k = 0; k < NCHAIN; ++k) c[k] = floatx4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < NCHAIN; ++k) c[k] = mfma16(a, b, c[k]);
    }
#pragma unroll
    for (int k = 0; k < NCHAIN; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) out += c[k][r];
  }
  if (tid == 0) sink[blockIdx.x] = out;
}

constexpr int kLdsThreads = 512;
constexpr int kLdsBytes = 128 * 1024;
constexpr int kLdsUnroll = 8;

// LDS reads: one 512-thread workgroup per compute unit fills 128 KB of LDS,
// then every wave reads it back `iters` times kLdsUnroll reads per round,
// each at a different offset.  Plain reads: lane l reads the 16 bytes at
// 16 l of a 1 KB span (conflict-free).  Transposing reads: lane l reads the
// 8 bytes at 8 l of a 512-byte span.
template <int KIND>
__global__ void __launch_bounds__(kLdsThreads) lds_read_kernel(int iters, float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) int4v buf[kLdsBytes / 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsBytes / 16; i += kLdsThreads) buf[i] = int4v{i, i ^ 0x55, i * 3, ~i};
  __syncthreads();
  const uint32_t base = lds_addr(buf);
  int4v acc = {0, 0, 0, 0};
  if constexpr (KIND == MLA_CEILING_LDS_B128) {
    const uint32_t l0 = 16 * lane + 1024 * wave;
    for (int it = 0; it < iters; ++it) {
      int4v v[kLdsUnroll];
#pragma unroll
      for (int k = 0; k < kLdsUnroll; ++k)
        v[k] = lds_read_b128_at(base + ((l0 + (uint32_t)(it * kLdsUnroll + k) * 8192u) & (kLdsBytes - 1)));
#pragma unroll
      for (int k = 0; k < kLdsUnroll; ++k) acc ^= v[k];
    }
  } else {
    const uint32_t l0 = 8 * lane + 512 * wave;
    for (int it = 0; it < iters; ++it) {
      bf16x4 v[kLdsUnroll];
#pragma unroll
      for (int k = 0; k < kLdsUnroll; ++k)
        v[k] = lds_read_tr16_at(base + ((l0 + (uint32_t)(it * kLdsUnroll + k) * 4096u) & (kLdsBytes - 1)));
#pragma unroll
      for (int k = 0; k < kLdsUnroll; ++k) {
        const int2v w = __builtin_bit_cast(int2v, v[k]);
        acc[0] ^= w[0];
        acc[1] ^= w[1];
      }
    }
  }
  const int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (tid == 0) sink[blockIdx.x] = __int_as_float(x);
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  return n;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

int32_t mla_ceiling_sink_floats(void) { return MLA_CEILING_SINK_FLOATS; }

mla_status mla_ceiling_hbm_read(const void* buf, size_t bytes, float* sink, double* work, void* stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15)) return MLA_ERR_INVALID_ARG;
  const int cus = device_cus();
  if (cus < 0) return MLA_ERR_HIP;
  const int grid = cus * 16 <= MLA_CEILING_SINK_FLOATS ? cus * 16 : MLA_CEILING_SINK_FLOATS;
  (void)hipGetLastError();
  hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(kHbmThreads), 0, (hipStream_t)stream, (const int4v*)buf,
                     (long long)(bytes / 16), sink);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  if (work) *work = (double)bytes;
  return MLA_OK;
}

mla_status mla_ceiling_mfma_bf16(int32_t shape, int32_t iters, float* sink, double* work, void* stream) {
  if (!sink || iters < 1 || (shape != MLA_CEILING_MFMA_32X32X16 && shape != MLA_CEILING_MFMA_16X16X32))
    return MLA_ERR_INVALID_ARG;
  const int cus = device_cus();
  if (cus < 0) return MLA_ERR_HIP;
  // two 256-thread workgroups per compute unit: two waves on every SIMD
  const int grid = 2 * cus <= MLA_CEILING_SINK_FLOATS ? 2 * cus : MLA_CEILING_SINK_FLOATS;
  (void)hipGetLastError();
  if (shape == MLA_CEILING_MFMA_32X32X16) {
    hipLaunchKernelGGL(mfma_loop_kernel<MLA_CEILING_MFMA_32X32X16>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       iters, sink);
  } else {
    hipLaunchKernelGGL(mfma_loop_kernel<MLA_CEILING_MFMA_16X16X32>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       iters, sink);
  }
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  // 4 waves per workgroup; per product 2*M*N*K = 32768 (32x32x16) or 16384
  // (16x16x32) FLOPs, 4 or 8 products per round
  const double per_round = shape == MLA_CEILING_MFMA_32X32X16 ? 4.0 * 32768.0 : 8.0 * 16384.0;
  if (work) *work = (double)grid * 4.0 * (double)iters * per_round;
  return MLA_OK;
}

mla_status mla_ceiling_lds_read(int32_t kind, int32_t iters, float* sink, double* work, void* stream) {
  if (!sink || iters < 1 || (kind != MLA_CEILING_LDS_B128 && kind != MLA_CEILING_LDS_TR_B64))
    return MLA_ERR_INVALID_ARG;
  const int cus = device_cus();
  if (cus < 0) return MLA_ERR_HIP;
  const int grid = cus <= MLA_CEILING_SINK_FLOATS ? cus : MLA_CEILING_SINK_FLOATS;
  (void)hipGetLastError();
  if (kind == MLA_CEILING_LDS_B128) {
    hipLaunchKernelGGL(lds_read_kernel<MLA_CEILING_LDS_B128>, dim3(grid), dim3(kLdsThreads), 0, (hipStream_t)stream,
                       iters, sink);
  } else {
    hipLaunchKernelGGL(lds_read_kernel<MLA_CEILING_LDS_TR_B64>, dim3(grid), dim3(kLdsThreads), 0,
                       (hipStream_t)stream, iters, sink);
  }
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  const double per_lane = kind == MLA_CEILING_LDS_B128 ? 16.0 : 8.0;
  if (work) *work = (double)grid * kLdsThreads * (double)iters * kLdsUnroll * per_lane;
  return MLA_OK;
}

}  // extern "C"
