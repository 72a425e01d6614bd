// Value up-projection o_i = W_i^UV z_i (the "DeepSeek-V3" notes,
// ekkoxiao.github.io, §潜在向量的作用: values are summed in latent space and
// up-projected afterwards).  W_i^UV is stored [128 d][512 c], so the
// contraction index c is contiguous in both operands: no transposition needed.
#include "common.h"
#include "kernels.h"

namespace mla {

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

// Mid-sized row counts (33 .. 256 rows, the 64 tokens of a 64-sequence
// decode step): workgroup = (head, 32 query rows), wave w = output rows
// d = 32w .. 32w+31, one 32x32 tile over the 512 channels on 32x32x16 matrix
// cores.  A launch has H * ceil(N / 32) workgroups of four busy waves (a
// 64-row wave tile would leave three of four waves idle at such N).  The contraction runs in four chunks of 128 channels: the
// chunk's W^UV block (128 rows x 256 B) and z rows (32 x 512 B, rounded to
// bf16) are loaded with whole rows per instruction (16 bytes per lane,
// consecutive lanes along a row) and staged in LDS, from which the matrix
// cores read their operands; the next chunk's loads are in flight while a
// chunk is multiplied.  (Loading the operands straight in the matrix-core
// layout touched 32 rows, so 32 cache lines, per load instruction, and ran
// at 2.2 TB/s.)
constexpr int kUpMidMaxN = 256;
constexpr int kUpMidChunk = 128;                     // channels per chunk
constexpr int kUpMidWStride = kUpMidChunk * 2 + 16;  // LDS row stride (bytes) of the W block
constexpr int kUpMidZStride = kUpMidChunk * 2 + 16;  // and of the z rows (bf16)

struct UpMidRegs {
  int4v w[8];    // W rows (t + 256 i) / 16, 16 bytes at (t % 16)
  float4 z[4];   // z rows (t + 256 i) / 32, 4 channels at 4 (t % 32)
};

__global__ void __launch_bounds__(256) upproj_bf16_mid_kernel(UpprojArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[kDv * kUpMidWStride];   // 34,816 B
  __shared__ __attribute__((aligned(16))) uint8_t z_lds[32 * kUpMidZStride];    // 8,704 B
  const int h = blockIdx.x, n0 = 32 * blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5;
  const bf16* wh = (const bf16*)a.w_uv + (size_t)h * kDv * kDc;
  auto load = [&](UpMidRegs& r, int c0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, ch = idx & 15;
      r.w[i] = *(const int4v*)(wh + (size_t)row * kDc + c0 + 8 * ch);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 5, q = idx & 31;
      const int n = min(n0 + row, a.N - 1);  // a row past N repeats the last one; its column is not stored
      r.z[i] = *(const float4*)(a.z + ((size_t)n * a.H + h) * kDc + c0 + 4 * q);
    }
  };
  auto stage = [&](const UpMidRegs& r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, ch = idx & 15;
      *(int4v*)(w_lds + row * kUpMidWStride + 16 * ch) = r.w[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 5, q = idx & 31;
      const float4 u = r.z[i];
      *(bf16x4*)(z_lds + row * kUpMidZStride + 8 * q) = bf16x4{f2bf(u.x), f2bf(u.y), f2bf(u.z), f2bf(u.w)};
    }
  };
  // operands of step j (16 channels) of a chunk: A lane l = W row 32w + l%32,
  // channels 16j + 8g .. +7; B lane l = z row l%32, the same channels
  const uint8_t* wa = w_lds + (32 * wave + (lane & 31)) * kUpMidWStride + 16 * g;
  const uint8_t* zb = z_lds + (lane & 31) * kUpMidZStride + 16 * g;
  floatx16 acc = floatx16{};
  UpMidRegs ra, rb;
  load(ra, 0);
#pragma unroll
  for (int k = 0; k < kDc / kUpMidChunk; ++k) {
    UpMidRegs& cur = (k & 1) ? rb : ra;
    UpMidRegs& nxt = (k & 1) ? ra : rb;
    if (k > 0) __syncthreads();  // every wave is done with the previous chunk's LDS
    stage(cur);
    if (k + 1 < kDc / kUpMidChunk) load(nxt, kUpMidChunk * (k + 1));
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kUpMidChunk / 16; ++j) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, *(const int4v*)(wa + 32 * j));
      const bf16x8 bv = __builtin_bit_cast(bf16x8, *(const int4v*)(zb + 32 * j));
      acc = mfma32(av, bv, acc);
    }
  }
  // C layout: column = query row n0 + l%32, rows d = 32w + 8(r/4) + 4g + r%4
  const int n = n0 + (lane & 31);
  if (n >= a.N) return;
  const size_t base = ((size_t)n * a.H + h) * kDv + 32 * wave;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int d = 8 * q4 + 4 * g;
    if (a.o_bf16) {
      *(bf16x4*)((bf16*)a.o + base + d) =
          bf16x4{f2bf(acc[4 * q4]), f2bf(acc[4 * q4 + 1]), f2bf(acc[4 * q4 + 2]), f2bf(acc[4 * q4 + 3])};
    } else {
      *(float4*)((float*)a.o + base + d) = make_float4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
    }
  }
}

// Many rows (prefill): workgroup = (head, 128 query rows), wave w = rows
// 32w .. 32w+31 against all 128 outputs (four 32x32 tiles), so W^UV_h is
// read once per 128 rows.  As in the mid-sized kernel, each chunk of 64
// channels of W^UV_h (128 rows x 128 B) and of the z rows (128 x 256 B,
// rounded to bf16) is loaded along whole rows, 16 bytes per lane, and
// staged in LDS (two buffers: the next chunk is stored while the current
// one is multiplied, one barrier per chunk; loads run two chunks ahead).
constexpr int kUpBigChunk = 64;                      // channels per chunk
constexpr int kUpBigStride = kUpBigChunk * 2 + 16;   // LDS row stride (bytes), W and z alike
constexpr int kUpBigBuf = 2 * 128 * kUpBigStride;    // one chunk: W block + z rows

struct UpBigRegs {
  int4v w[4];    // W rows (t + 256 i) / 8, 16 bytes at (t % 8)
  float4 z[8];   // z rows (t + 256 i) / 16, 4 channels at 4 (t % 16)
};

__global__ void __launch_bounds__(256) upproj_bf16_rows_kernel(UpprojArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kUpBigBuf];  // 73,728 B
  const int h = blockIdx.x, n0 = 128 * blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5;
  const bf16* wh = (const bf16*)a.w_uv + (size_t)h * kDv * kDc;
  auto load = [&](UpBigRegs& r, int c0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, ch = idx & 7;
      r.w[i] = *(const int4v*)(wh + (size_t)row * kDc + c0 + 8 * ch);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, q = idx & 15;
      const int n = min(n0 + row, a.N - 1);  // a row past N repeats the last one; its column is not stored
      r.z[i] = *(const float4*)(a.z + ((size_t)n * a.H + h) * kDc + c0 + 4 * q);
    }
  };
  auto stage = [&](const UpBigRegs& r, uint8_t* buf) {
    uint8_t* wl = buf;
    uint8_t* zl = buf + 128 * kUpBigStride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, ch = idx & 7;
      *(int4v*)(wl + row * kUpBigStride + 16 * ch) = r.w[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, q = idx & 15;
      const float4 u = r.z[i];
      *(bf16x4*)(zl + row * kUpBigStride + 8 * q) = bf16x4{f2bf(u.x), f2bf(u.y), f2bf(u.z), f2bf(u.w)};
    }
  };
  floatx16 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = floatx16{};
  // chunk c is loaded into r[c & 1] two chunks before it is staged
  UpBigRegs r[2];
  load(r[0], 0);
  load(r[1], kUpBigChunk);
  stage(r[0], lds);
  load(r[0], 2 * kUpBigChunk);
  __syncthreads();
  constexpr int kChunks = kDc / kUpBigChunk;  // 8
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const uint8_t* buf = lds + (k & 1) * kUpBigBuf;
    // operands of step j (16 channels): A lane l = W row 32mt + l%32, B lane
    // l = z row 32w + l%32, channels 16j + 8g .. +7
    const uint8_t* wa = buf + (lane & 31) * kUpBigStride + 16 * g;
    const uint8_t* zb = buf + 128 * kUpBigStride + (32 * wave + (lane & 31)) * kUpBigStride + 16 * g;
#pragma unroll
    for (int j = 0; j < kUpBigChunk / 16; ++j) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, *(const int4v*)(zb + 32 * j));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, *(const int4v*)(wa + 32 * mt * kUpBigStride + 32 * j));
        acc[mt] = mfma32(av, bv, acc[mt]);
      }
    }
    if (k + 1 < kChunks) {
      // chunk k+1 goes into the other buffer, last read in chunk k-1 (done
      // by every wave before the previous barrier); its registers then take
      // the loads of chunk k+3
      stage(r[(k + 1) & 1], lds + ((k + 1) & 1) * kUpBigBuf);
      if (k + 3 < kChunks) load(r[(k + 1) & 1], kUpBigChunk * (k + 3));
      __syncthreads();
    }
  }
  // C layout: column = query row n0 + 32w + l%32, rows d = 32mt + 8(r/4) + 4g + r%4
  const int n = n0 + 32 * wave + (lane & 31);
  if (n >= a.N) return;
  const size_t base = ((size_t)n * a.H + h) * kDv;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * mt + 8 * q4 + 4 * g;
      const floatx16& v = acc[mt];
      if (a.o_bf16) {
        *(bf16x4*)((bf16*)a.o + base + d) = bf16x4{f2bf(v[4 * q4]), f2bf(v[4 * q4 + 1]), f2bf(v[4 * q4 + 2]),
                                                   f2bf(v[4 * q4 + 3])};
      } else {
        *(float4*)((float*)a.o + base + d) = make_float4(v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]);
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
  } else if (a.N <= kUpMidMaxN) {
    hipLaunchKernelGGL(upproj_bf16_mid_kernel, dim3(a.H, (a.N + 31) / 32), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(upproj_bf16_rows_kernel, dim3(a.H, (a.N + 127) / 128), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
