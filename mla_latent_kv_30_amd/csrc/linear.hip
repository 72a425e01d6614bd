// Projections around the attention, Y = X W^T with bf16 operands and fp32
// accumulation on the 32x32x16 matrix cores:
//   cache append   [c^KV | k^R] = h [W^DKV; W^KR]^T       (§KeyValue)
//   query path     c^Q = h W^DQ^T, [q^C | q^R] = c^Q [W^UQ; W^QR]^T  (§Query)
//   output         u = [o_1 .. o_H] W^O^T                   (§注意力计算)
// Both operands are K-major (each row of X and of W is contiguous along the
// contraction), which is the order the matrix-core operands want: a lane's
// eight consecutive k values are one 16-byte LDS read.
//
// Tiles: TM rows of W (output features) x TN rows of X (tokens), k in steps
// of 64 (one 128-byte row slice per operand row).  Tiles are staged in LDS by
// LDS-DMA in a ring of STAGES buffers; one workgroup barrier per k step.
// Within each 32-row group of a staged tile the even rows come first, then
// the odd rows, and chunk c of LDS row p sits at chunk position
// c ^ 2((p >> 2) & 3): gfx950 serves a 16-byte LDS read per half-wave (even
// lanes, then odd lanes) over 128 four-byte banks, and with this placement
// the 32 reads of a half-wave (16 rows x 2 chunks) fall on 32 distinct bank
// groups.
//
// Long contractions with few output tiles are split over k (grid z); each
// split writes fp32 partials and a second kernel sums them in split order.

#include "kernels.h"

namespace mla {
namespace {

constexpr int kTK = 64;              // k per stage
constexpr int kSlice = kTK * 2;      // bytes of one row per stage
constexpr int kRsrc3 = 0x00020000;   // raw untyped buffer access

// Tile row held at LDS row p: in each 32-row group LDS rows 0..15 hold the
// even tile rows and 16..31 the odd ones.
__device__ __forceinline__ int tile_row(int p) {
  const int q = p & 31;
  return (p & ~31) + (q < 16 ? 2 * q : 2 * (q - 16) + 1);
}
__device__ __forceinline__ int chunk_perm(int p) { return 2 * ((p >> 2) & 3); }

// Wait until at most the copies of this wave's `later` (0..4) most recently
// issued steps are in flight (P copies per step).
template <int P, int MAXL>
__device__ __forceinline__ void wait_steps(int later) {
  if constexpr (MAXL >= 4) {
    if (later >= 4) { wait_vmcnt<4 * P>(); return; }
  }
  if constexpr (MAXL >= 3) {
    if (later == 3) { wait_vmcnt<3 * P>(); return; }
  }
  if constexpr (MAXL >= 2) {
    if (later == 2) { wait_vmcnt<2 * P>(); return; }
  }
  if constexpr (MAXL >= 1) {
    if (later == 1) { wait_vmcnt<P>(); return; }
  }
  wait_vmcnt<0>();
}

template <int WM, int WN, int FM, int FN, int STAGES>
struct Tile {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = WM * FM * 32;
  static constexpr int TN = WN * FN * 32;
  static constexpr int kCopies = (TM + TN) / 8;          // 1 KB LDS-DMA copies per stage
  static constexpr int kPerWave = kCopies / kWaves;
  static constexpr int kStageBytes = (TM + TN) * kSlice;
  static constexpr int kLdsBytes = STAGES * kStageBytes;
  static_assert(kWaves == 4 || kWaves == 8, "the copy plan takes 4 or 8 waves");
  static_assert(kCopies % kWaves == 0, "copies must split evenly over the waves");
  static_assert(STAGES >= 2 && STAGES <= 6 && (STAGES - 2) * kPerWave < 64, "vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// Output tile of workgroup b: consecutive tiles go to one XCD (the hardware
// deals workgroups to the 8 XCDs in turn), and inside that range tiles run
// in column groups of 4 M-tiles so that the workgroups live at one time on
// an XCD share their X and W rows in its L2.
__device__ __forceinline__ void tile_of(int b, int mt, int nt, int& m, int& n) {
  const int T = mt * nt;
  int t = b;
  if ((T & 7) == 0) t = (b & 7) * (T >> 3) + (b >> 3);
  const int gm = 4;
  const int span = gm * nt;
  const int g = t / span, r = t - g * span;
  const int width = min(gm, mt - g * gm);
  n = r / width;
  m = g * gm + (r - n * width);
}

// Y[n][m .. m+3] (m % 4 == 0; the four features lie in one block of Y).
__device__ __forceinline__ void store_out(const LinearArgs& a, int n, int m, float4 v) {
  const int e1 = a.Mb[0], e2 = a.Mb[0] + a.Mb[1];
  const int b = m < e1 ? 0 : (m < e2 ? 1 : 2);
  const int mm = m - (b == 0 ? 0 : (b == 1 ? e1 : e2));
  const size_t at = (size_t)n * a.Mb[b] + mm;
  void* y = a.y[b];
  if ((a.out_bf16 >> b) & 1) {
    bf16x4 h;
    h[0] = f2bf(v.x); h[1] = f2bf(v.y); h[2] = f2bf(v.z); h[3] = f2bf(v.w);
    *(bf16x4*)((bf16*)y + at) = h;
  } else {
    *(float4*)((float*)y + at) = v;
  }
}

template <int WM, int WN, int FM, int FN, int STAGES>
__global__ __launch_bounds__(64 * WM * WN) void linear_kernel(LinearArgs a) {
  using T = Tile<WM, WN, FM, FN, STAGES>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[T::kLdsBytes];
  const int wave = uniform((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int mtile, ntile;
  tile_of(blockIdx.x, a.mt, a.nt, mtile, ntile);
  mtile = uniform(mtile);
  ntile = uniform(ntile);
  const int m0 = mtile * T::TM, n0 = ntile * T::TN;
  const int s = blockIdx.y;
  const int nk = (a.K / kTK);
  const int kt0 = s * a.kt_split;
  const int kt1 = min(nk, kt0 + a.kt_split);
  const int steps = kt1 - kt0;

  // ---- copy plan ----
  // Copy q of a stage (q = wave + W c, W waves) fills LDS bytes
  // [q KB, q KB + 1 KB): LDS rows 8q .. 8q+7, i.e. rows 8 (wave % 4) + l/8
  // of the stage's 32-row group q / 4 = (W/4) c + wave / 4.  The lane part
  // of the offset is the same for every copy of a wave; the group's first
  // row is a scalar.  W groups come first (features), then X groups
  // (tokens); the 32 rows of a W group sit in one block of W (rows past the
  // last block read as zeros).
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t rowb = (uint32_t)a.K * 2;
  const int pr = 8 * (wave & 3) + (lane >> 3);
  const uint32_t lane_vo = (uint32_t)tile_row(pr) * rowb + 16u * (uint32_t)((lane & 7) ^ chunk_perm(pr));
  const int e1 = a.Mb[0], e2 = a.Mb[0] + a.Mb[1];
  auto issue = [&](int step) {
    const uint32_t stage = lds0 + (uint32_t)((step % STAGES) * T::kStageBytes);
    const uint32_t koff = (uint32_t)((kt0 + step) * kSlice);
#pragma unroll
    for (int c = 0; c < T::kPerWave; ++c) {
      const uint32_t ldsq = stage + 1024u * (uint32_t)(wave + c * T::kWaves);
      const int gq = (T::kWaves / 4) * c + (wave >> 2);   // row group of this copy
      // W group (block chosen by selects) or X group, no branches
      const bool is_w = 32 * gq < T::TM;
      const int row0 = m0 + 32 * gq;
      const bool b0 = row0 < e1, b1 = row0 < e2;
      const bf16* base = uniform_ptr(is_w ? (b0 ? a.w[0] : (b1 ? a.w[1] : a.w[2])) : a.x);
      const int rows = uniform(is_w ? (b0 ? a.Mb[0] : (b1 ? a.Mb[1] : a.Mb[2])) : a.N);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)((uint32_t)rows * rowb), kRsrc3);
      const int r = uniform(is_w ? row0 - (b0 ? 0 : (b1 ? e1 : e2)) : n0 + 32 * gq - T::TM);
      lds_dma16(rs, uniform((int)ldsq), lane_vo + (uint32_t)r * rowb, koff);
    }
  };

  // ---- fragment addresses: lane reads row (l % 32) of each 32-row group ----
  const int wm = wave % WM, wn = wave / WM;
  const int prow = ((lane & 31) >> 1) + 16 * (lane & 1);
  const int cp = chunk_perm(prow);
  const int hf = lane >> 5;
  const uint32_t a_off = (uint32_t)(((wm * FM) * 32 + prow) * kSlice);
  const uint32_t b_off = (uint32_t)((T::TM + (wn * FN) * 32 + prow) * kSlice);

  floatx16 acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;

#pragma unroll
  for (int i = 0; i < STAGES - 1; ++i)
    if (i < steps) issue(i);

  for (int i = 0; i < steps; ++i) {
    // copies of step i are done once at most those of the later issued steps remain
    wait_steps<T::kPerWave, STAGES - 2>(min(STAGES - 2, steps - 1 - i));
    __syncthreads();
    if (i + STAGES - 1 < steps) issue(i + STAGES - 1);
    const uint32_t stage = lds0 + (uint32_t)((i % STAGES) * T::kStageBytes);
    // Fragments of the four 16-k substeps, double-buffered: the reads of
    // substep j+1 are issued before the products of substep j (the fence
    // keeps them there; the pins keep the products after it), so each wait
    // covers only reads issued one substep earlier.
    bf16x8 af[2][FM], bfr[2][FN];
    auto read = [&](int j, int buf) {
      const uint32_t co = 16u * (uint32_t)((2 * j + hf) ^ cp);
#pragma unroll
      for (int f = 0; f < FM; ++f)
        af[buf][f] = __builtin_bit_cast(bf16x8, lds_read_b128_at(stage + a_off + f * 32 * kSlice + co));
#pragma unroll
      for (int g = 0; g < FN; ++g)
        bfr[buf][g] = __builtin_bit_cast(bf16x8, lds_read_b128_at(stage + b_off + g * 32 * kSlice + co));
    };
    read(0, 0);
#pragma unroll
    for (int j = 0; j < kTK / 16; ++j) {
      const int cur = j & 1;
      if (j + 1 < kTK / 16) read(j + 1, cur ^ 1);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int f = 0; f < FM; ++f) asm volatile("" : "+v"(af[cur][f]));
#pragma unroll
      for (int g = 0; g < FN; ++g) asm volatile("" : "+v"(bfr[cur][g]));
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int g = 0; g < FN; ++g) acc[f][g] = mfma32(af[cur][f], bfr[cur][g], acc[f][g]);
    }
  }

  // ---- epilogue: lane holds token (l % 32) and features 8q + 4hf + e ----
  const int M = a.Mb[0] + a.Mb[1] + a.Mb[2];
#pragma unroll
  for (int g = 0; g < FN; ++g) {
    const int n = n0 + (wn * FN + g) * 32 + (lane & 31);
    if (n >= a.N) continue;
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int mg = m0 + (wm * FM + f) * 32;   // uniform: a 32-feature group
      if (mg >= M) continue;
      // one tile at a time in VGPRs (else all accumulators are moved out at once)
      floatx16 t = acc[f][g];
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = mg + 8 * q + 4 * hf;
        const float4 v = make_float4(t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]);
        if (a.splits > 1) {
          *(float4*)(a.part + ((size_t)s * a.N + n) * M + m) = v;
          continue;
        }
        store_out(a, n, m, v);
      }
    }
  }
}

// Sum of the split partials (in split order) for 4 consecutive features.
__global__ __launch_bounds__(256) void linear_reduce_kernel(LinearArgs a) {
  const int M = a.Mb[0] + a.Mb[1] + a.Mb[2];
  const int M4 = M / 4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)a.N * M4) return;
  const int n = (int)(idx / M4);
  const int m = 4 * (int)(idx - (size_t)n * M4);
  const size_t plane = (size_t)a.N * M;
  const float* p = a.part + (size_t)n * M + m;
  // 0 + p_0 + p_1 + ... in plane order: batches of 16 planes, all loads
  // issued before the adds (indices past the last plane re-read it)
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < a.splits; s0 += 16) {
    float4 w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = *(const float4*)(p + (size_t)min(s0 + j, a.splits - 1) * plane);
#pragma unroll
    for (int j = 0; j < 16; ++j) {   // past the last plane: add zero (exact)
      const bool in = s0 + j < a.splits;
      v.x += in ? w[j].x : 0.f;
      v.y += in ? w[j].y : 0.f;
      v.z += in ? w[j].z : 0.f;
      v.w += in ? w[j].w : 0.f;
    }
  }
  store_out(a, n, m, v);
}

// W'[r][512 i + c] = sum_j W^O[r][128 i + j] W_i^UV[j][c]: a one-time weight
// transform.  Block: head i, 256 consecutive c, 64 rows r; the 64 x 128
// slice of W^O is staged in LDS, W^UV is read down its columns (coalesced
// across the block).
constexpr int kFoldRows = 64;
__global__ __launch_bounds__(256) void fold_kernel(const bf16* __restrict__ w_uv, const bf16* __restrict__ w_o,
                                                   bf16* __restrict__ w_fold, int H, int d) {
  __shared__ float wo[kFoldRows][kDv];
  const int c = blockIdx.x * 256 + threadIdx.x;   // 0..511
  const int i = blockIdx.y;
  const int r0 = blockIdx.z * kFoldRows;
  for (int e = threadIdx.x; e < kFoldRows * kDv; e += 256) {
    const int rr = e / kDv, j = e - rr * kDv;
    wo[rr][j] = r0 + rr < d ? bf2f(w_o[(size_t)(r0 + rr) * H * kDv + i * kDv + j]) : 0.f;
  }
  __syncthreads();
  float acc[kFoldRows];
#pragma unroll
  for (int rr = 0; rr < kFoldRows; ++rr) acc[rr] = 0.f;
  const bf16* col = w_uv + (size_t)i * kDv * kDc + c;
  for (int j = 0; j < kDv; ++j) {
    const float w = bf2f(col[(size_t)j * kDc]);
#pragma unroll
    for (int rr = 0; rr < kFoldRows; ++rr) acc[rr] = fmaf(wo[rr][j], w, acc[rr]);
  }
#pragma unroll
  for (int rr = 0; rr < kFoldRows; ++rr)
    if (r0 + rr < d) w_fold[(size_t)(r0 + rr) * H * kDc + (size_t)i * kDc + c] = f2bf(acc[rr]);
}

template <int WM, int WN, int FM, int FN, int STAGES>
hipError_t run(LinearArgs a, hipStream_t st) {
  using T = Tile<WM, WN, FM, FN, STAGES>;
  hipLaunchKernelGGL((linear_kernel<WM, WN, FM, FN, STAGES>), dim3(a.mt * a.nt, a.splits), dim3(T::kThreads), 0, st,
                     a);
  hipError_t e = hipGetLastError();
  // no outputs named: the caller consumes the partials itself
  if (e != hipSuccess || a.splits == 1 || a.y[0] == nullptr) return e;
  const size_t n4 = (size_t)a.N * ((a.Mb[0] + a.Mb[1] + a.Mb[2]) / 4);
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Tile shape by token count: decode-sized products (N <= 64) stream W
// through 128-row tiles with 5-6 stages (one workgroup per compute unit keeps
// 64-80 KB of W in flight); larger N use square tiles.  A product with at
// most half as many output tiles as compute units is split over k, about one
// workgroup per compute unit, with S N / K <= 1/16 so that the fp32 partials
// (written once, read once) stay within a quarter of the weight bytes, and
// at least 8 k steps per split so that the copy ring fills.
namespace {

void plan_splits(LinearPlan& p, int N, int M, int K, int cus) {
  p.mt = (M + p.tm - 1) / p.tm;
  p.nt = (N + p.tn - 1) / p.tn;
  const int nk = K / kTK;
  const int tiles = p.mt * p.nt;
  int splits = 1;
  if (tiles * 2 <= cus) {
    splits = cus / tiles;                                  // one workgroup per compute unit
    splits = min(splits, max(1, K / (16 * N)));            // partial bytes <= weight bytes / 4
    splits = min(splits, max(1, nk / 8));                  // at least 8 k steps (a full ring) per split
  }
  p.kt_split = (nk + splits - 1) / splits;
  p.splits = (nk + p.kt_split - 1) / p.kt_split;
  p.part_bytes = p.splits > 1 ? (size_t)p.splits * N * M * sizeof(float) : 0;
}

}  // namespace

LinearPlan plan_linear(int N, int M, int K, int cus) {
  LinearPlan p;
  if (N <= 32) {
    p.cfg = kLinSkinny32; p.tm = 128; p.tn = 32;
  } else if (N <= 64) {
    p.cfg = kLinSkinny64; p.tm = 128; p.tn = 64;
  } else if (N <= 512) {
    p.cfg = kLinMid; p.tm = 128; p.tn = 128;
  } else {
    p.cfg = kLinLarge; p.tm = 256; p.tn = 256;
  }
  plan_splits(p, N, M, K, cus);
  // a decode-sized product that 128-row tiles cannot spread over half of
  // the compute units (few output rows, short contraction) takes 64-row tiles
  if (N <= 64 && p.mt * p.nt * p.splits * 2 < cus) {
    LinearPlan q;
    q.cfg = kLinNarrow; q.tm = 64; q.tn = 64;
    plan_splits(q, N, M, K, cus);
    if (q.mt * q.nt * q.splits > p.mt * p.nt * p.splits) p = q;
  }
  return p;
}

hipError_t launch_linear(LinearArgs a, const LinearPlan& p, hipStream_t st) {
  a.mt = p.mt;
  a.nt = p.nt;
  a.splits = p.splits;
  a.kt_split = p.kt_split;
  switch (p.cfg) {
    case kLinSkinny32: return run<4, 1, 1, 1, 6>(a, st);
    case kLinSkinny64: return run<4, 1, 1, 2, 5>(a, st);
    case kLinMid: return run<2, 2, 2, 2, 3>(a, st);
    case kLinNarrow: return run<2, 2, 1, 1, 6>(a, st);
    default: return run<2, 4, 4, 2, 2>(a, st);
  }
}

hipError_t launch_fold_wuv_wo(const bf16* w_uv, const bf16* w_o, bf16* w_fold, int H, int d, hipStream_t st) {
  hipLaunchKernelGGL(fold_kernel, dim3(kDc / 256, H, (d + kFoldRows - 1) / kFoldRows), dim3(256), 0, st, w_uv, w_o,
                     w_fold, H, d);
  return hipGetLastError();
}

}  // namespace mla
