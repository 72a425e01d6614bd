// Device-side pieces of the decode kernels (decode.hip): the work schedule
// (shared by the matrix-core and fp32 kernels), the LDS row layout, the
// page-block copies and the fp8 expansion.
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kRowBytes = kRow * 2;                 // 1152
constexpr int kPageBytes = kPage * kRowBytes;       // 73728
constexpr int kBlock = 32;                          // scheduling granule (tokens)

// ---------------------------------------------------------------------------
// Work schedule shared by the decode and merge kernels.
// ---------------------------------------------------------------------------
//
// Three modes:
//   prefill  unit w = query row T-1-w of one sequence (longest rows first);
//   uniform  S chunks per sequence, chunk = ceil(ceil(L/64)/S) pages,
//            unit w = (b = w/S, chunk w%S), partial slot w;
//   balanced the 32-token blocks of all sequences, concatenated, are cut into
//            G nearly equal ranges (G = min(units, blocks)); a unit walks the
//            sequences its range touches.  Each sequence is preceded by
//            kStartCost blocks that hold no tokens: they stand for the cost of
//            starting a sequence (query load, first copies, final store), so a
//            unit that switches sequences gets correspondingly fewer tokens.
//            Unit w's piece of sequence b goes to partial slot w + b (unique:
//            the pieces of unit w have increasing b, and unit w+1 starts at or
//            after unit w's last b).
constexpr int kStartCost = 4;

// Exclusive prefix sums of kStartCost + the 32-token block count of every
// sequence into pfx[0..B], and the lengths into lens[0..B); returns the
// total.  Called by all threads; B <= kMaxSchedB.  If bt is given, its
// nbt <= 4 * blockDim.x entries (the whole block table) are copied into
// bt_lds as well: the loads go out together with the length loads, so the
// page lookups of the copy issue need no further round trip to memory.
// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// inside each row of 16 lanes (lanes shifted in from outside the row add 0),
// then the total of row 0 is added to row 1 and that of row 2 to row 3
// (row_bcast:15), and the total of rows 0-1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

static __device__ int block_prefix(const int32_t* __restrict__ seq_lens, int B, int* pfx, int* lens,
                                   const int32_t* __restrict__ bt = nullptr, int nbt = 0, int* bt_lds = nullptr) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;
  int btv[4];
  if (bt != nullptr) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + k * nthreads;
      btv[k] = i < nbt ? bt[i] : 0;
    }
  }
  if (B <= 64) {
    // one sequence per lane of wave 0, and a single barrier for the prefix
    // and the block-table copy
    if (wave == 0) {
      const int L = seq_lens[min(lane, B - 1)];
      const int v = lane < B ? kStartCost + (L + kBlock - 1) / kBlock : 0;
      const int x = wave_incl_scan(v);
      if (lane < B) {
        pfx[lane] = x - v;
        lens[lane] = L;
      }
      if (lane == B - 1) pfx[B] = x;
    }
    if (bt != nullptr) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = tid + k * nthreads;
        if (i < nbt) bt_lds[i] = btv[k];
      }
    }
    __syncthreads();
    return uniform(pfx[B]);
  }
  const int per = (B + nthreads - 1) / nthreads;  // <= 4
  const int base = tid * per;
  int loc[4];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = min(base + k, B - 1);
    const int L = seq_lens[i];  // loaded unconditionally so the loads overlap
    const int v = (k < per && base + k < B) ? kStartCost + (L + kBlock - 1) / kBlock : 0;
    if (k < per && base + k < B) lens[base + k] = L;
    loc[k] = v;
    sum += v;
  }
  int x = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  if (bt != nullptr) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + k * nthreads;
      if (i < nbt) bt_lds[i] = btv[k];
    }
  }
  __syncthreads();
  int excl = x - sum;
  for (int w = 0; w < wave; ++w) excl += wsum[w];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < per && base + k < B) pfx[base + k] = excl;
    excl += loc[k];
  }
  if (tid == nthreads - 1) pfx[B] = excl;
  __syncthreads();
  return uniform(pfx[B]);
}

// floor(x / d) for 0 <= x and 0 < d, in 32-bit arithmetic when x fits (the
// operands are wave-uniform, so the branch is too).
__device__ __forceinline__ long long udiv_fast(long long x, long long d) {
  if (x < (1ll << 32) && d < (1ll << 32)) return (long long)((uint32_t)x / (uint32_t)d);
  return x / d;
}

// Unit of the balanced split that owns block g (G units over P blocks).
__device__ __forceinline__ int unit_of_block(long long g, long long G, long long P) {
  return (int)udiv_fast((g + 1) * G - 1, P);
}

// One piece of work: tokens [t0, t1) of sequence b, whose length is L.
struct Segment {
  int b, t0, t1, L;
  int slot;   // partial slot of this piece
  int slot0;  // partial slot of the sequence's first piece
  int parts;  // pieces the sequence was cut into (1: this one is whole)
};

struct Schedule {
  int mode;          // 0 prefill, 1 uniform, 2 balanced
  int w;             // this unit
  long long G, P;    // balanced: units in use, total blocks
  long long g0, g1;  // balanced: this unit's block range
  int b;             // balanced: next sequence to look at
  int done;
  const int* pfx;    // balanced: block prefix and lengths in LDS
  const int* lens;
};

__device__ __forceinline__ Schedule schedule_begin(const DecodeArgs& a, const int* pfx, const int* lens, int P) {
  Schedule s{};
  s.w = blockIdx.x;
  s.pfx = pfx;
  s.lens = lens;
  if (a.prefill_T > 0) {
    s.mode = 0;
  } else if (a.splits > 0) {
    s.mode = 1;
  } else {
    s.mode = 2;
    s.P = P;
    s.G = min((long long)a.units, (long long)P);
    s.done = s.w >= s.G;
    if (!s.done) {
      s.g0 = udiv_fast((long long)s.w * s.P, s.G);
      s.g1 = udiv_fast((long long)(s.w + 1) * s.P, s.G);
      if (a.B <= 64) {
        // pfx rises strictly, so the b with pfx[b] <= g0 are 0 .. lo
        const int lane = threadIdx.x & 63;
        const bool le = lane < a.B && pfx[min(lane, a.B - 1)] <= s.g0;
        s.b = __popcll(__builtin_amdgcn_ballot_w64(le)) - 1;
      } else {
        int lo = 0, hi = a.B;  // last b with pfx[b] <= g0
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pfx[mid] <= s.g0) lo = mid; else hi = mid;
        }
        s.b = uniform(lo);
      }
    }
  }
  return s;
}

// Next piece of this unit's work; every thread of the workgroup gets the
// same answer.
__device__ __forceinline__ bool schedule_next(const DecodeArgs& a, Schedule& s, Segment& seg) {
  if (s.done) return false;
  if (s.mode == 0) {
    s.done = 1;
    const int t = a.prefill_T - 1 - s.w;
    const int L = a.prefill_pos0 + t + 1;
    seg = Segment{t, 0, L, L, 0, 0, 1};
    return true;
  }
  if (s.mode == 1) {
    s.done = 1;
    const int S = a.splits;
    const int b = s.w / S, k = s.w % S;
    const int L = a.seq_lens[b];
    const int np = (L + kPage - 1) / kPage;
    const int chunk = (np + S - 1) / S;
    const int pb = k * chunk, pe = min(pb + chunk, np);
    if (pb >= pe) return false;
    seg = Segment{b, pb * kPage, min(pe * kPage, L), L, s.w, b * S, (np + chunk - 1) / chunk};
    return true;
  }
  while (s.b < a.B) {
    const int b = s.b;
    const int r0 = uniform(s.pfx[b]) + kStartCost, r1 = uniform(s.pfx[b + 1]);  // token blocks of b
    if (r0 >= s.g1) break;
    s.b = b + 1;
    const int k0 = (int)(max(s.g0, (long long)r0) - r0);
    const int k1 = (int)(min(s.g1, (long long)r1) - r0);
    if (k0 < k1) {
      const int L = uniform(s.lens[b]);
      const int first = unit_of_block(r0, s.G, s.P);
      const int last = unit_of_block(r1 - 1, s.G, s.P);
      seg = Segment{b, k0 * kBlock, min(k1 * kBlock, L), L, s.w + b, first + b, last - first + 1};
      return true;
    }
  }
  s.done = 1;
  return false;
}

// ---------------------------------------------------------------------------
// LDS page layout
// ---------------------------------------------------------------------------
//
// Pages are streamed in blocks of 32 rows (half a page).  A block buffer in
// LDS holds 32 rows of 1152 bytes, unpadded: row r at r * 1152.  The 16-byte
// chunks of a row are permuted inside each aligned group of eight: chunk c
// of row r sits at chunk position c ^ swz(r).  gfx950 serves a 16-byte LDS
// read per half-wave (even lanes, then odd lanes) over 128 banks of 4 bytes,
// and the transposing 8-byte read per quarter-wave; without the permutation
// the rows of an operand tile (1152 = 9 * 128) would pile onto a quarter of
// the banks.  With it, the score operand reads, the transposing value reads
// and the dequantising writes below are all conflict-free.  Rows 2k and 2k+1
// Copies move 16 bytes per lane: 8 rows (576 16-byte chunks) are nine 1 KB
// copies, lane i of copy j fetching the chunk that belongs at LDS chunk
// 64 j + i of the 8 rows, i.e. chunk ((64 j + i) % 72) ^ swz of row
// (64 j + i) / 72 in HBM.
constexpr int kBlockRows = kBlock;                     // 32
constexpr int kBlockBytes = kBlockRows * kRowBytes;    // 36864
constexpr int kNBuf = 4;                               // block buffers: 3 in flight + 1 in use
constexpr int kWaves = 8;                              // every decode workgroup has 8 waves
constexpr int kCopyBytes = 1024;                       // one LDS-DMA copy: 64 lanes x 16 bytes
constexpr int kGroupRows = 8;                          // rows moved by nine copies
constexpr int kGroupBytes = kGroupRows * kRowBytes;    // 9216
constexpr int kCopiesPerGroup = kGroupBytes / kCopyBytes;  // 9
// A block is 4 groups; wave w moves copies 0..4 (w < 4) or 5..8 (w >= 4) of
// group w % 4.
constexpr int kCopiesLo = 5, kCopiesHi = kCopiesPerGroup - kCopiesLo;
constexpr int kRsrcWord3 = 0x00020000;                 // raw untyped buffer access

__device__ __forceinline__ int swz(int r) { return 2 * ((r >> 2) & 3) + ((r >> 4) & 1); }
// LDS byte offset of byte x (x < 1152) of row r.
__device__ __forceinline__ int lds_off(int r, int x) { return r * kRowBytes + (x ^ (swz(r) << 4)); }

// Copy the first `hi` rows of a 32-row block (rows 32*half .. of a bf16
// page) into an LDS block buffer.  The buffer resource covers exactly those
// rows, so rows at or past hi (past the sequence end, or owned by the next
// unit) arrive as zeros and stale or non-finite pool contents never reach
// the matrix cores.
__device__ __forceinline__ void issue_block_bf16(const uint8_t* page, int half, uint8_t* buf, int hi, int wave,
                                                 int lane) {
  asm volatile("" : "+s"(wave));  // re-derived per copy, not kept live across the loop
  lane = lane_id_fresh();
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(page + half * kBlockBytes), (short)0, uniform(hi * kRowBytes), kRsrcWord3);
  const int g = wave & 3;
  const uint32_t lb = lds_addr(buf) + g * kGroupBytes;
  auto copy = [&](int j) {
    const int q = 64 * j + lane;
    const int r = q / 72, c = q - 72 * r;
    const uint32_t vo = (uint32_t)(r * kRowBytes + 16 * (c ^ swz(kGroupRows * g + r)));
    lds_dma16(rs, lb + kCopyBytes * j, vo, g * kGroupBytes);
  };
  if (wave < 4) {
#pragma unroll
    for (int j = 0; j < kCopiesLo; ++j) copy(j);
  } else {
#pragma unroll
    for (int j = kCopiesLo; j < kCopiesPerGroup; ++j) copy(j);
  }
}

// The same copies prepared for issue one at a time, so that a computing wave
// can spread them over its score products (copies issued back to back by all
// waves at once queue at the address unit).  n = 0: nothing to copy.
struct BlockCopies {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t lb;  // LDS address of this wave's 8-row group
  int g;        // the group
  int j0, n;    // this wave's first copy of the group and how many
};

__device__ __forceinline__ BlockCopies plan_block_bf16(const uint8_t* page, int half, uint8_t* buf, int hi, int wave) {
  BlockCopies c;
  c.g = wave & 3;
  c.rs = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(page + half * kBlockBytes), (short)0,
                                           uniform(hi * kRowBytes), kRsrcWord3);
  c.lb = lds_addr(buf) + c.g * kGroupBytes;
  c.j0 = wave < 4 ? 0 : kCopiesLo;
  c.n = wave < 4 ? kCopiesLo : kCopiesHi;
  return c;
}

// Copy t (< c.n) of this wave.
__device__ __forceinline__ void issue_copy(const BlockCopies& c, int t) {
  const int lane = lane_id_fresh();
  const int j = c.j0 + t;
  const int q = 64 * j + lane;
  const int r = q / 72, cc = q - 72 * r;
  const uint32_t vo = (uint32_t)(r * kRowBytes + 16 * (cc ^ swz(kGroupRows * c.g + r)));
  lds_dma16(c.rs, c.lb + kCopyBytes * j, vo, c.g * kGroupBytes);
}

// Wait until at most the copies of this wave's `n` (0..3) most recently
// issued blocks are in flight (waves 0..3 issue C_LO copies per block,
// waves 4..7 C_HI).
template <int C>
__device__ __forceinline__ void wait_blocks_c(int n) {
  if (n >= 3) wait_vmcnt<3 * C>(); else if (n == 2) wait_vmcnt<2 * C>(); else if (n == 1) wait_vmcnt<C>();
  else wait_vmcnt<0>();
}
template <int C_LO, int C_HI>
__device__ __forceinline__ void wait_blocks(int n, int wave) {
  if (wave < 4) wait_blocks_c<C_LO>(n); else wait_blocks_c<C_HI>(n);
}

// fp8 staging buffer of one block: codes [32][512], scales [32][4] fp32,
// rotated k^R [32][64] bf16.
constexpr int kStCkv = 0;
constexpr int kStScale = kBlockRows * kDc;                  // 16384
constexpr int kStKr = kStScale + kBlockRows * 4 * 4;        // 16896
constexpr int kStageBytes = kStKr + kBlockRows * kDr * 2;   // 20992
constexpr int kFp8Copies = 3;                               // per wave and block

// Wave w copies codes 2w, 2w+1 (1 KB each), and either 128 bytes of scales
// (w < 4, 8 lanes) or 1 KB of k^R (w >= 4).
__device__ __forceinline__ void issue_block_fp8(const uint8_t* ckv8, const float* scale8, const uint8_t* kr8,
                                                int page, int half, uint8_t* stage, int hi, int wave, int lane) {
  asm volatile("" : "+s"(wave));
  const size_t row0 = (size_t)page * kPage + half * kBlockRows;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(ckv8 + row0 * kDc), (short)0, uniform(hi * kDc), kRsrcWord3);
  const uint32_t lb = lds_addr(stage);
  const uint32_t vo = lane * 16;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int off = (2 * wave + k) * kCopyBytes;
    lds_dma16(rc, lb + kStCkv + off, vo, off);
  }
  if (wave < 4) {
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(scale8 + row0 * 4), (short)0, uniform(hi * 16), kRsrcWord3);
    if (lane < 8) {
      const int off = wave * 128;
      lds_dma16(rsc, lb + kStScale + off, vo, off);
    }
  } else {
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(kr8 + row0 * (kDr * 2)), (short)0, uniform(hi * kDr * 2), kRsrcWord3);
    const int off = (wave - 4) * kCopyBytes;
    lds_dma16(rk, lb + kStKr + off, vo, off);
  }
}

// Copy the absorbed queries of HG head groups (rows h0 .. h0+15 of each,
// 1152 bytes per head) into LDS at `dst` ([HG][16][1152]); heads at or past
// H arrive as zeros.  All 8 waves share the copies: HG * 9 per wave.
template <int HG>
__device__ __forceinline__ void issue_query_copy(const uint8_t* qrow, int H, uint8_t* dst, int wave, int lane) {
  constexpr int kDmaBytes = 256;                          // 64 lanes x 4 bytes
  constexpr int kPerGroup = 16 * kRowBytes / kDmaBytes;  // 72
  const uint32_t lb = lds_addr(dst);
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const int rows = uniform(min(16, H - 16 * hg));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(qrow + (size_t)16 * hg * kRowBytes), (short)0, uniform(max(rows, 0) * kRowBytes),
        kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kPerGroup / kWaves; ++i) {
      const int off = (i * kWaves + wave) * kDmaBytes;
      lds_dma4(rs, lb + hg * 16 * kRowBytes + off, lane * 4, off);
    }
  }
}

// Expand a staged fp8 block into the bf16 row layout with NTHREADS threads.
// Item t: row t/16, channels 32(t%16) .. +31 (a quarter of a 128-channel
// tile, one scale); items t < 256 of the second loop copy one 16-byte chunk
// of a row's k^R.  Rows past the valid range are zeros in the staging
// buffer (codes and scales), so they expand to zeros.
template <int NTHREADS>
__device__ __forceinline__ void dequant_block(const uint8_t* stage, uint8_t* buf, int wave) {
  // offsets recomputed per block, not held across the loop
  const int t0 = 64 * wave + lane_id_fresh();
  constexpr int kItems = kBlockRows * 16, kKrItems = kBlockRows * 8;
#pragma unroll
  for (int it = 0; it < (kItems + NTHREADS - 1) / NTHREADS; ++it) {
    const int t = t0 + it * NTHREADS;
    if (t >= kItems) break;
    const int r = t >> 4, sub = t & 15;
    const float sc = *(const float*)(stage + kStScale + (r * 4 + (sub >> 2)) * 4);
    const uint8_t* src = stage + kStCkv + r * kDc + sub * 32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int4v raw = lds_read_b128(src + 16 * j);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int word = raw[2 * h + e];
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
          v[4 * e + 0] = f2bf(lo[0] * sc);
          v[4 * e + 1] = f2bf(lo[1] * sc);
          v[4 * e + 2] = f2bf(hi[0] * sc);
          v[4 * e + 3] = f2bf(hi[1] * sc);
        }
        const int chunk = sub * 4 + 2 * j + h;  // 8 channels = one 16-byte chunk
        *(MLA_LDS bf16x8*)(buf + lds_off(r, chunk * 16)) = v;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < (kKrItems + NTHREADS - 1) / NTHREADS; ++it) {
    const int t = t0 + it * NTHREADS;
    if (t >= kKrItems) break;
    const int kr_row = t >> 3, kc = t & 7;
    const int4v kr = lds_read_b128(stage + kStKr + kr_row * (kDr * 2) + kc * 16);
    *(MLA_LDS int4v*)(buf + lds_off(kr_row, kDc * 2 + kc * 16)) = kr;
  }
}

// ---------------------------------------------------------------------------
// Block cursor
// ---------------------------------------------------------------------------

// Position in a unit's stream of 32-token blocks: block k of a piece.
struct Cursor {
  Schedule sch;
  Segment seg;
  int k;
  int valid;
};

__device__ __forceinline__ void cursor_next(const DecodeArgs& a, Cursor& c) {
  if (c.k < (c.seg.t1 - 1) / kBlock) {
    ++c.k;
    return;
  }
  c.valid = schedule_next(a, c.sch, c.seg);
  c.k = c.valid ? c.seg.t0 / kBlock : 0;
}

constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is refreshed

// q[j] = channels 32(k0 + j) + 8g .. +7 of the lane's head row (zeros for a
// head at or past H).
template <int NQ>
__device__ __forceinline__ void load_query(bf16x8 (&q)[NQ], const bf16* __restrict__ src_rows, int H, int head,
                                           int g, int k0 = 0) {
  const int hc = head < H ? head : H - 1;
  const int keep = head < H ? -1 : 0;
  const int4v* src = (const int4v*)(src_rows + (size_t)hc * kRow) + 4 * k0;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    int4v v = src[4 * j + g];
    v &= keep;
    q[j] = __builtin_bit_cast(bf16x8, v);
  }
}

// Use the query registers, so the compiler's own wait for their loads is
// placed here and not at the first score product, where later page copies
// (which its counter does not see) would be waited for as well.
template <int NQ>
__device__ __forceinline__ void consume_query(bf16x8 (&q)[NQ]) {
#pragma unroll
  for (int j = 0; j < NQ; ++j) asm volatile("" : "+v"(q[j]));
}

}  // namespace mla
