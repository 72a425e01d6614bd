// Absorbed query: q~_i = (W_i^UK)^T q_i^C and the rotated position query
// RoPE_pos(q_i^R) (the "DeepSeek-V3" notes, ekkoxiao.github.io,
// §潜在向量的作用 and §Query).  Output row per (token, head): [q~ (512) | q^R' (64)].
//
// bf16 path: per head the product is [N x 128] x [128 x 512].  W_i^UK is
// stored [128 d][512 c] (row block of the up-projection), so the contraction
// index d is the slow one; a 128 x 128 slice of it is staged in LDS and the
// gfx950 transposing LDS read hands the matrix cores d-packed operands.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kAbsRowsPerWave = 32;
constexpr int kAbsRowsPerBlock = 4 * kAbsRowsPerWave;   // 128 query tokens per workgroup
constexpr int kAbsCols = 128;                           // c-slice of W per workgroup
constexpr int kAbsLdsStride = kAbsCols * 2 + 32;        // padded row stride (bytes): rows 8 banks apart
constexpr int kAbsOutStride = kAbsCols * 2 + 8;         // output staging row stride (bytes)

// Many query rows.  A workgroup owns one 128-channel quarter cq of q~ for
// one head h and a stripe of row blocks (128 query rows each): row blocks
// s, s + RS, s + 2 RS, ... of RB = ceil(N / 128).  Its W slice (128 d x 128
// c) is loaded into LDS once and stays there; the q_c operand of the next
// row block is loaded while the current one is multiplied and stored.
// 4 waves, each 32 query rows x 128 c per row block.
// Grid: 32 * ceil(H * RS / 8) workgroups in one dimension; job = s * H + h.
// Workgroups go to the eight XCDs in turn, so workgroup L takes quarter
// (L >> 3) & 3 of job (L & 7) + 8 (L >> 5): the four quarters of a job run on
// one XCD, and the q_c rows they share come from HBM once into that XCD's
// L2 instead of once into each of four.  Jobs that run at the same time are
// neighbouring heads of the same rows, whose q_c and q~ rows are neighbours
// in memory.  RS is chosen so that there are about two workgroups per CU.
// The rotation of a row block's 128 rows is shared by the four quarters.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
absorb_bf16_kernel(AbsorbArgs a, int RB, int RS) {
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[kDn * kAbsLdsStride];  // W[d][c-slice]
  // each wave's 32 rows x 128 channels of output (rows 264 bytes apart: a
  // store instruction's 32 rows land 2 banks apart)
  __shared__ __attribute__((aligned(16))) uint8_t stage_lds[4 * kAbsRowsPerWave * kAbsOutStride];
  const int L = blockIdx.x;
  const int job = (L & 7) + 8 * (L >> 5), cq = (L >> 3) & 3;
  if (job >= a.H * RS) return;
  const int stripe = job / a.H, h = job - stripe * a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5;
  const bf16* __restrict__ w = (const bf16*)a.w_uk + (size_t)h * kDn * kDc + cq * kAbsCols;
  // W[0:128][cq*128 : cq*128+128]: 128 rows of 16 chunks of 16 bytes
  int4v wv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + 256 * i, d = idx >> 4, ch = idx & 15;
    wv[i] = *(const int4v*)(w + (size_t)d * kDc + ch * 8);
  }
  // Per row block: the B operand q_c^T (k = d, n = query row; lane holds row
  // n0 + lane%32, d = 16kk + 8g + j), and this quarter's 32 rows of the
  // rotation, n_blk + 32cq .. +31, one pair (2m, 2m+1) per item.
  struct Operands {
    int4v qv[8];
    uint32_t rx[4];
    int rpos[4];
    double rth[4];
  };
  auto load_operands = [&](int rb, Operands& o) {
    const int nrow = rb * kAbsRowsPerBlock + wave * kAbsRowsPerWave + (lane & 31);
    const bf16* __restrict__ qc = (const bf16*)a.q_c + ((size_t)(nrow < a.N ? nrow : 0) * a.H + h) * kDn;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) o.qv[kk] = *(const int4v*)(qc + 16 * kk + 8 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int item = tid + 256 * j, n = rb * kAbsRowsPerBlock + 32 * cq + (item >> 5), m = item & 31;
      const int nc = n < a.N ? n : 0;
      o.rx[j] = *(const uint32_t*)((const bf16*)a.q_r + ((size_t)nc * a.H + h) * kDr + 2 * m);
      o.rpos[j] = a.pos[nc];
      o.rth[j] = a.rope.theta[m];
    }
  };
  Operands op;
  load_operands(stripe, op);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + 256 * i, d = idx >> 4, ch = idx & 15;
    *(int4v*)(w_lds + d * kAbsLdsStride + ch * 16) = wv[i];
  }
  __syncthreads();  // the W slice stays in place for every row block
  // A operand: W^T (m = c, k = d) by transposing reads: 16-lane group G owns
  // columns 16*(G%2) .. +15 of the 32-wide tile and rows d0 + 4*(lane%16 / 4)
  const int dsub = (lane & 15) >> 2;
  const int cl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint8_t* const stage = stage_lds + wave * (kAbsRowsPerWave * kAbsOutStride);
  for (int rb = stripe; rb < RB; rb += RS) {
    const int n_blk = rb * kAbsRowsPerBlock;
    const int n0 = n_blk + wave * kAbsRowsPerWave;
    const bool nok = n0 + (lane & 31) < a.N;
    bf16x8 qb[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[kk] = __builtin_bit_cast(bf16x8, nok ? op.qv[kk] : int4v{0, 0, 0, 0});
    uint32_t rx[4];
    int rpos[4];
    double rth[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rx[j] = op.rx[j];
      rpos[j] = op.rpos[j];
      rth[j] = op.rth[j];
    }
    // the next row block's operands load under this one's products and stores
    if (rb + RS < RB) load_operands(rb + RS, op);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int item = tid + 256 * j, n = n_blk + 32 * cq + (item >> 5), m = item & 31;
      if (n < a.N) {
        float c, sn;
        rope_cs(rpos[j], rth[j], c, sn);
        const float x0 = __uint_as_float(rx[j] << 16), x1 = __uint_as_float(rx[j] & 0xffff0000u);
        bf16* out = (bf16*)a.q_abs + ((size_t)n * a.H + h) * kRow + kDc + 2 * m;
        *(bf16x2*)out = bf16x2{f2bf(x0 * c - x1 * sn), f2bf(x0 * sn + x1 * c)};
      }
    }
    if (n0 >= a.N) continue;  // this wave has no rows in the block (uniform per wave)
    floatx16 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc[mt] = floatx16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int d0 = 16 * kk + 8 * g + dsub;
        const uint8_t* p0 = w_lds + d0 * kAbsLdsStride + (32 * mt + cl) * 2;
        bf16x4 lo = lds_read_tr16(p0);
        bf16x4 hi = lds_read_tr16(p0 + 4 * kAbsLdsStride);
        bf16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[mt] = mfma32(av, qb[kk], acc[mt]);
      }
    }
    // C layout: column = query row n0 + lane%32, rows c = 32mt + 8(r/4) + 4g + r%4.
    // The rows go through the wave's own staging area and leave as 256-byte
    // row slices, 16 bytes per lane and 4 rows per instruction, instead of
    // 16-byte pieces of 32 rows per instruction.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v = {f2bf(acc[mt][4 * q4]), f2bf(acc[mt][4 * q4 + 1]), f2bf(acc[mt][4 * q4 + 2]),
                    f2bf(acc[mt][4 * q4 + 3])};
        *(bf16x4*)(stage + (lane & 31) * kAbsOutStride + (32 * mt + 8 * q4 + 4 * g) * 2) = v;
      }
#pragma unroll
    for (int i = 0; i < kAbsRowsPerWave / 4; ++i) {
      const int r = 4 * i + (lane >> 4);
      const int4v v = *(const int4v*)(stage + r * kAbsOutStride + 16 * (lane & 15));
      if (n0 + r < a.N)
        *(int4v*)((bf16*)a.q_abs + ((size_t)(n0 + r) * a.H + h) * kRow + cq * kAbsCols + 8 * (lane & 15)) = v;
    }
  }
}

// Few query rows (decode, N <= 32): workgroup = (head, 64-channel slice of
// q~), so a launch has H * 8 workgroups and each reads only its 16 KB of W.
// All W loads of a thread are issued before any of them is stored to LDS
// (one memory round trip).  Wave w computes channels 16w .. 16w+15 of the
// slice for every row on 16x16x32 matrix cores: A = W^T (16 c x 32 d) by
// transposing LDS reads, B = q_c^T straight from memory.
constexpr int kAbsSmallCols = 64;
constexpr int kAbsSmallStride = kAbsSmallCols * 2 + 16;  // 144 B: transposing reads hit distinct banks
constexpr int kAbsSmallMaxN = 32;

__global__ void __launch_bounds__(256) absorb_small_kernel(AbsorbArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[kDn * kAbsSmallStride];  // W[d][64-channel slice]
  const int h = blockIdx.x, cs = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = lane >> 4, s = lane & 15;
  const bf16* w = (const bf16*)a.w_uk + (size_t)h * kDn * kDc + cs * kAbsSmallCols;
  int4v wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // 128 rows x 8 chunks of 16 bytes
    const int idx = tid + 256 * i, d = idx >> 3, ch = idx & 7;
    wv[i] = *(const int4v*)(w + (size_t)d * kDc + ch * 8);
  }
  // B operand q_c^T: lane holds query row 16nt + s, d = 32kk + 8G + j
  bf16x8 qb[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = 16 * nt + s;
    const bool ok = n < a.N;
    const bf16* qc = (const bf16*)a.q_c + ((size_t)(ok ? n : 0) * a.H + h) * kDn;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      int4v v = *(const int4v*)(qc + 32 * kk + 8 * G);
      if (!ok) v = int4v{0, 0, 0, 0};
      qb[nt][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // rotation: the N x 32 pairs of this head are shared by the 8 workgroups
  // of the head (4N pairs each, one per thread); loads issued with the rest
  const int ritem = cs * 4 * a.N + tid;
  const bool rot = tid < 4 * a.N;
  const int rn = rot ? ritem >> 5 : 0, rm = ritem & 31;
  uint32_t rx = 0;
  int rpos = 0;
  double rth = 0.0;
  if (rot) {
    rx = *(const uint32_t*)((const bf16*)a.q_r + ((size_t)rn * a.H + h) * kDr + 2 * rm);
    rpos = a.pos[rn];
    rth = a.rope.theta[rm];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i, d = idx >> 3, ch = idx & 7;
    *(int4v*)(w_lds + d * kAbsSmallStride + ch * 16) = wv[i];
  }
  __syncthreads();
  if (rot) {  // after the barrier: its operands arrived with the W slice
    asm volatile("" : "+v"(rpos));  // converted here, not where it was loaded
    float c, sn;
    rope_cs(rpos, rth, c, sn);
    const float x0 = __uint_as_float(rx << 16), x1 = __uint_as_float(rx & 0xffff0000u);
    bf16* out = (bf16*)a.q_abs + ((size_t)rn * a.H + h) * kRow + kDc + 2 * rm;
    *(bf16x2*)out = bf16x2{f2bf(x0 * c - x1 * sn), f2bf(x0 * sn + x1 * c)};
  }
  // A operand by transposing reads: source lane s of group G points at row
  // d = 32kk + 8G + s/4 (+4), columns c0 + 4(s%4) .. +3; lane s receives
  // column c0 + s of four consecutive rows.
  const int c0 = 16 * wave;
  const uint8_t* ap = w_lds + (8 * G + (s >> 2)) * kAbsSmallStride + 2 * (c0 + 4 * (s & 3));
  bf16x8 av[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x4 lo = lds_read_tr16(ap + 32 * kk * kAbsSmallStride);
    bf16x4 hi = lds_read_tr16(ap + (32 * kk + 4) * kAbsSmallStride);
    av[kk] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (16 * nt >= a.N) break;
    floatx4 acc = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mfma16(av[kk], qb[nt][kk], acc);
    // C layout: column = query row 16nt + s, rows c = c0 + 4G + r
    const int n = 16 * nt + s;
    if (n < a.N) {
      bf16* out = (bf16*)a.q_abs + ((size_t)n * a.H + h) * kRow + cs * kAbsSmallCols + c0 + 4 * G;
      *(bf16x4*)out = bf16x4{f2bf(acc[0]), f2bf(acc[1]), f2bf(acc[2]), f2bf(acc[3])};
    }
  }
}

// fp32: one thread per (row, head, c); W reads coalesce along c.
__global__ void __launch_bounds__(256) absorb_f32_kernel(AbsorbArgs a) {
  const int nh = blockIdx.x;  // n * H + h
  const int n = nh / a.H, h = nh % a.H;
  __shared__ float qs[kDn];
  const float* qc = (const float*)a.q_c + (size_t)nh * kDn;
  if (threadIdx.x < kDn) qs[threadIdx.x] = qc[threadIdx.x];
  __syncthreads();
  const float* w = (const float*)a.w_uk + (size_t)h * kDn * kDc;
  float* out = (float*)a.q_abs + (size_t)nh * kRow;
  for (int c = threadIdx.x; c < kDc; c += 256) {
    float acc = 0.f;
    for (int d = 0; d < kDn; ++d) acc = fmaf(w[(size_t)d * kDc + c], qs[d], acc);
    out[c] = acc;
  }
  if (threadIdx.x < 32) {
    const int m = threadIdx.x;
    const float* qr = (const float*)a.q_r + (size_t)nh * kDr;
    float c, s;
    rope_cs(a.pos[n], a.rope.theta[m], c, s);
    const float x0 = qr[2 * m], x1 = qr[2 * m + 1];
    out[kDc + 2 * m] = x0 * c - x1 * s;
    out[kDc + 2 * m + 1] = x0 * s + x1 * c;
  }
}

hipError_t launch_absorb(const AbsorbArgs& a, int kind, hipStream_t s) {
  if (kind == kKindF32) {
    hipLaunchKernelGGL(absorb_f32_kernel, dim3(a.N * a.H), dim3(256), 0, s, a);
  } else if (a.N <= kAbsSmallMaxN) {
    hipLaunchKernelGGL(absorb_small_kernel, dim3(a.H, kDc / kAbsSmallCols), dim3(256), 0, s, a);
  } else {
    // row-block stripes: about two workgroups per CU, each stripe at least one row block
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    const int RB = (a.N + kAbsRowsPerBlock - 1) / kAbsRowsPerBlock;
    const int RS = std::max(1, std::min(RB, (2 * cus + 4 * a.H - 1) / (4 * a.H)));
    hipLaunchKernelGGL(absorb_bf16_kernel, dim3(32 * ((a.H * RS + 7) / 8)), dim3(256), 0, s, a, RB, RS);
  }
  return hipGetLastError();
}

}  // namespace mla
