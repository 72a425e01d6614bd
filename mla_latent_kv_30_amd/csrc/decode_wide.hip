// Absorbed-MLA decode for 65 to 128 heads (and multi-token decode with that
// many query heads): the wide kernel.
//
// What it computes is the decode of decode.hip (the "DeepSeek-V3" notes,
// ekkoxiao.github.io, §注意力计算 and §潜在向量的作用): per head i and
// cached token j, s_j = (q~_i . c_j + q^R_i . k^R_j) * scale, an online
// softmax over the tokens, and z_i = sum_j a_j c_j.
//
// Why a second kernel: at 128 heads every 32-token block of cached rows
// (36 KB) is multiplied by the absorbed queries of all heads (147 KB of
// bf16) and accumulated into all heads' latent sums (256 KB of fp32).  Both
// live in registers, and with 16 heads per wave every block is read out of
// LDS by eight waves twice (rows for the scores, transposed for the value
// product): 557 KB of LDS reads per block.  Here a workgroup has four
// waves, one per SIMD, each with the whole 512-entry register file:
//   * wave w owns heads 32w .. 32w+31: its absorbed queries (144 VGPRs) and
//     its latent accumulators Z^T (512 channels x 32 heads, 256 registers,
//     held in the accumulation registers);
//   * each block is read by four waves instead of eight: 147 KB of 16-byte
//     row reads for the scores and 131 KB of transposing reads for the value
//     product, 278 KB per block;
//   * the products are bf16 32x32x16 matrix-core operations (32 tokens x 32
//     heads of scores in one accumulation chain; 32 channels x 32 heads per
//     value tile);
//   * the value product of block i-1 runs after the scores of block i, so
//     the softmax of block i can issue while the matrix cores work through
//     the value products; that keeps block i-1 readable for one more step,
//     so two blocks (not three) are in flight while one is scored and one is
//     accumulated (four 36 KB buffers);
//   * with one wave per SIMD nothing hides a stall, so a step is one fixed
//     sequence of products with their operand reads issued a few products
//     ahead and the softmax and copy instructions placed between them
//     (wide_step).
// The work schedule, the paged copies (LDS-DMA), the row layout in LDS and
// the split-KV partials are those of decode.hip (decode_common.h).
#include "decode_common.h"

namespace mla {
namespace {

constexpr int kWWaves = 4;                  // one wave per SIMD
constexpr int kWThreads = kWWaves * 64;
constexpr int kWNBuf = 4;                   // value(i-1), scores(i), blocks i+1 and i+2 in flight
constexpr int kWNBuf8 = 3;                  // fp8: value(i-1), scores(i), expansion of i+1
constexpr int kWAhead = 2;                  // blocks copied ahead of the one being scored
constexpr int kWCopies = kCopiesPerGroup;   // 9 copies per wave and block: wave w moves 8-row group w
// Operand reads in flight, in products, and value products led with
// operands read before the loop's barrier (wide_step): bf16 4 and 4; fp8 3
// and none (its registers are full).
constexpr int kWDepth = 4, kWLead = 4;
constexpr int kWDepth8 = 3, kWLead8 = 0;

static_assert(kWWaves * kGroupRows == kBlockRows, "four waves move the four 8-row groups of a block");

// LDS row layout of this kernel: rows of 1152 bytes, the 16-byte chunks of
// row r permuted inside each aligned group of eight as c -> c ^ swzw(r),
//     swzw(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3).
// Bank model (measured on gfx950 with the bank-conflict counter over lane
// patterns): a 16-byte read is served a quarter-wave (16 consecutive lanes)
// at a time and a transposing 8-byte read a half-wave at a time, each pass
// over 64 banks of 4 bytes; a pass is conflict-free when its lanes touch
// distinct 16-byte (resp. 8-byte) units modulo 256 bytes.  A row is 4.5 such
// windows long, so rows r and r + 2 start at the same bank and only the
// permutation tells them apart:
//   * score operand: a quarter-wave reads the same chunk of 16 consecutive
//     rows; for each row parity, swzw takes eight distinct values over the
//     eight rows (it is a bijection of (r >> 1) & 7), so the 16 reads land
//     on 16 distinct units;
//   * value operand: a half-wave reads rows b .. b+3 (b a multiple of 4) at
//     the four chunks 4(ct & 1) + 0..3 of a group of eight; bit 2 of swzw is
//     (r >> 1) & 1, so rows r and r + 2 (same parity) take opposite halves of
//     the group, and the 32 eight-byte reads land on 32 distinct units.
__device__ __forceinline__ int swzw(int r) { return 4 * ((r >> 1) & 1) + ((r >> 2) & 3); }
__device__ __forceinline__ int lds_off_w(int r, int x) { return r * kRowBytes + (x ^ (swzw(r) << 4)); }

// The absorbed query of a wave for 32x32x16 products: K-step kk holds
// channels 16kk + 8h .. +7 (h = lane / 32) of head h0 + lane % 32.
struct WideQuery {
  bf16x8 q[36];
};

// Latent accumulators Z^T: tile ct holds channels 32ct + 8(r / 4) + 4h + r % 4
// (register r) of head h0 + lane % 32.
struct WideAcc {
  floatx16 z[16];
};

// Running softmax state of the lane's head: maximum in log2 units and this
// lane's partial denominator (its 16 tokens of each block).
struct WideSoftmax {
  float m, l;
};

__device__ __forceinline__ void load_query_wide(WideQuery& Q, const bf16* __restrict__ rows, int H, int h0) {
  const int lane = lane_id_fresh();
  const int head = h0 + (lane & 31);
  const int hc = head < H ? head : H - 1;
  const int keep = head < H ? -1 : 0;
  const int4v* src = (const int4v*)(rows + (size_t)hc * kRow) + (lane >> 5);
#pragma unroll
  for (int kk = 0; kk < 36; ++kk) {
    int4v x = src[2 * kk];
    x &= keep;
    Q.q[kk] = __builtin_bit_cast(bf16x8, x);
  }
}

// Place the compiler's wait for the query loads here.
__device__ __forceinline__ void consume_query_wide(WideQuery& Q) {
#pragma unroll
  for (int kk = 0; kk < 36; ++kk) asm volatile("" : "+v"(Q.q[kk]));
}

// The copies of one 32-row block for 4 waves: wave w moves all nine 1 KB
// copies of 8-row group w, in this kernel's row layout.
struct WideCopies {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t lb;  // LDS address of this wave's 8-row group
  int g;        // the group
  int n;        // copies to issue (0: no block)
};

__device__ __forceinline__ WideCopies plan_block_wide(const uint8_t* page, int half, uint8_t* buf, int hi,
                                                      int wave) {
  WideCopies c;
  c.g = wave;
  c.rs = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(page + half * kBlockBytes), (short)0,
                                           uniform(hi * kRowBytes), kRsrcWord3);
  c.lb = lds_addr(buf) + c.g * kGroupBytes;
  c.n = kWCopies;
  return c;
}

// Wait until at most the copies of this wave's n (0 or 1) most recently
// issued blocks are in flight.
__device__ __forceinline__ void wait_blocks_wide(int n) {
  if (n >= 1) wait_vmcnt<kWCopies>(); else wait_vmcnt<0>();
}

// Z^T tile += A B on the matrix cores with the accumulator in the
// accumulation registers.  Written as one instruction so that the register
// allocator keeps every accumulator tile in place there (left to itself it
// moved tiles between register files and spilled); the compiler cannot see
// this instruction's latency, so the code below waits explicitly before any
// other instruction touches an accumulator (acc_settle()).
__device__ __forceinline__ void mfma32_acc(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last accumulation and an ordinary instruction that
// reads or writes an accumulator tile (more than the 18 a 16-pass product
// needs), and between such a write and the next accumulation.
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Outside the matrix cores the accumulators are only read, one register at
// a time through explicit accumulation-register reads: arithmetic written on
// the tiles themselves would let the register allocator move whole tiles
// between register files (and spill), which the single-instruction
// accumulations above avoid.  They are reset on the matrix cores, and a
// moved running maximum is handled without scaling them in place (below).
__device__ __forceinline__ float acc_get(const floatx16& t, int r) {
  float x;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(t[r]));
  return x;
}

// Every tile to zero, on the matrix cores: 0 x 0 + 0, in one statement.
// The compiler materialises `zero` with ordinary vector moves just before
// it and cannot see that a matrix-core instruction reads it, so the leading
// s_nop supplies the wait states between that write and the first read.
// "+a": the zeros go to the tiles' own registers (an output-only operand
// would let the allocator pick others and copy at every join).
__device__ __forceinline__ void reset_acc_mfma(WideAcc& Z) {
  const bf16x8 zero = {};
  asm volatile(
      "s_nop 7\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %1, %16, %16, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %3, %16, %16, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %5, %16, %16, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %7, %16, %16, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %8, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %9, %16, %16, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %10, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %11, %16, %16, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %12, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %13, %16, %16, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %14, %16, %16, 0\n\tv_mfma_f32_32x32x16_bf16 %15, %16, %16, 0"
      : "+a"(Z.z[0]), "+a"(Z.z[1]), "+a"(Z.z[2]), "+a"(Z.z[3]), "+a"(Z.z[4]), "+a"(Z.z[5]), "+a"(Z.z[6]),
        "+a"(Z.z[7]), "+a"(Z.z[8]), "+a"(Z.z[9]), "+a"(Z.z[10]), "+a"(Z.z[11]), "+a"(Z.z[12]), "+a"(Z.z[13]),
        "+a"(Z.z[14]), "+a"(Z.z[15])
      : "v"(zero));
}

// A running maximum moved by more than the lazy threshold: the sums so far
// (Z, and what earlier moves left in the piece's output rows) are relative
// to the old maximum and must be scaled by alpha = 2^(m_old - m_new).  The
// accumulators are not scaled in place, nor reset: the difference goes to
// the piece's own output rows (z or its partial slot, [head][512] fp32),
//     out <- alpha out + (alpha - 1) Z      (out = 0 before the first move),
// and the accumulation simply continues, so that at the end
//     out + Z = alpha (out_old + Z_old) + (Z - Z_old),
// the old sums scaled and the new ones as they are.  The final store adds
// `out` back.  The cancellation against Z_old costs a few fp32 roundings of
// the accumulator's own size.
__device__ __forceinline__ void flush_wide(const WideAcc& Z, float alpha, bool has_stored, float* zdst, int h0,
                                           int H) {
  const int lane = lane_id_fresh();
  const int head = h0 + (lane & 31), h = lane >> 5;
  if (head >= H) return;
  const float am1 = alpha - 1.0f;
  float* row = zdst + (size_t)head * kDc + 4 * h;
#pragma unroll
  for (int ct = 0; ct < 16; ++ct) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx16& t = Z.z[ct];
      float4* dst = (float4*)(row + 32 * ct + 8 * q);
      float4 o = make_float4(acc_get(t, 4 * q) * am1, acc_get(t, 4 * q + 1) * am1, acc_get(t, 4 * q + 2) * am1,
                             acc_get(t, 4 * q + 3) * am1);
      if (has_stored) {
        const float4 prev = *dst;
        o.x = fmaf(alpha, prev.x, o.x);
        o.y = fmaf(alpha, prev.y, o.y);
        o.z = fmaf(alpha, prev.z, o.z);
        o.w = fmaf(alpha, prev.w, o.w);
      }
      *dst = o;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Normalise and store a finished piece: z rows [head][512] (plus what an
// earlier flush left there) and lse[head].
__device__ __forceinline__ void store_wide(const WideAcc& Z, float l_tot, float m, bool has_stored, float* zdst,
                                           float* ldst, int h0, int H) {
  constexpr float kLn2 = 0.69314718055994530942f;
  const int lane = lane_id_fresh();
  const int head = h0 + (lane & 31), h = lane >> 5;
  if (head >= H) return;
  // l = 0: every key of the piece lies after this query token (multi-token
  // decode): z = 0 and lse = -inf, which the merge weighs 0
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  float* row = zdst + (size_t)head * kDc + 4 * h;
#pragma unroll
  for (int ct = 0; ct < 16; ++ct) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx16& t = Z.z[ct];
      float4* dst = (float4*)(row + 32 * ct + 8 * q);
      float4 o = make_float4(acc_get(t, 4 * q), acc_get(t, 4 * q + 1), acc_get(t, 4 * q + 2), acc_get(t, 4 * q + 3));
      if (has_stored) {
        const float4 prev = *dst;
        o.x += prev.x;
        o.y += prev.y;
        o.z += prev.z;
        o.w += prev.w;
      }
      *dst = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (ldst != nullptr && h == 0) ldst[head] = (m + __log2f(l_tot)) * kLn2;
}

// Per-lane LDS offsets of the operand reads within a block buffer, advanced
// by one buffer per step (all reads then take immediate offsets on top).
//   sa[k4]          score operand of K-step kk (kk % 4 == k4): row lane % 32,
//                   bytes 32 kk + 16 (lane / 32); kk / 4 adds 128 bytes;
//   va[t][hh][c2]   value operand of K-step t, tile ct (ct % 2 == c2): the
//                   rows 16 t + 8 hh + 4 h + s / 4 of value_wide's pattern;
//                   ct / 2 adds 128 bytes.
struct WideAddr {
  uint32_t sa[4];
  uint32_t va[2][2][2];
};

__device__ __forceinline__ WideAddr wide_addr(uint32_t score_buf, uint32_t value_buf) {
  const int lane = lane_id_fresh();
  WideAddr A;
  const int row = lane & 31, h = lane >> 5;
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) A.sa[k4] = score_buf + lds_off_w(row, 32 * k4 + 16 * h);
  const int G = lane >> 4, s = lane & 15;
  const int hv = G >> 1, hf = G & 1;
  const int x = 32 * hf + 8 * (s & 3);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
        A.va[t][hh][c2] = value_buf + lds_off_w(16 * t + 8 * hh + 4 * hv + (s >> 2), 64 * c2 + x);
  return A;
}

// From step i to step i+1 in a ring of NB buffers: the score reads move
// from buffer i % NB to the next one, the value reads from buffer
// (i - 1) % NB to the next one.
template <int NB>
__device__ __forceinline__ void advance_addr(WideAddr& A, int i) {
  constexpr uint32_t kNext = kBlockBytes, kWrap = (uint32_t)(-(NB - 1) * kBlockBytes);
  const uint32_t ds = i % NB == NB - 1 ? kWrap : kNext;
  const uint32_t dv = i % NB == 0 ? kWrap : kNext;
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) A.sa[k4] += ds;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) A.va[t][hh][c2] += dv;
}

__device__ __forceinline__ bf16x8 score_operand(const WideAddr& A, int kk) {
  return __builtin_bit_cast(bf16x8, lds_read_b128_at(A.sa[kk & 3] + 128 * (kk >> 2)));
}

// Value operand n: K-step n / 16, channel tile n % 16 (a tile's two
// products are 16 products apart).
__device__ __forceinline__ bf16x8 value_operand(const WideAddr& A, int n) {
  const int ct = n & 15, t = n >> 4;
  const bf16x4 lo = lds_read_tr16_at(A.va[t][0][ct & 1] + 128 * (ct >> 1));
  const bf16x4 hi = lds_read_tr16_at(A.va[t][1][ct & 1] + 128 * (ct >> 1));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Per-lane source offsets of this wave's nine copies of an 8-row group (they
// depend only on the lane and the group): copy j, lane i fills LDS chunk
// 64 j + i of the group, i.e. chunk cc of row r = (64 j + i) / 72, which holds
// source chunk cc ^ swzw(8 g + r).
struct WideCopyOffsets {
  uint32_t vo[kWCopies];
};

__device__ __forceinline__ WideCopyOffsets copy_offsets(int g) {
  const int lane = lane_id_fresh();
  WideCopyOffsets o;
#pragma unroll
  for (int j = 0; j < kWCopies; ++j) {
    const int q = 64 * j + lane;
    const int r = q / 72, cc = q - 72 * r;
    o.vo[j] = (uint32_t)(r * kRowBytes + 16 * (cc ^ swzw(kGroupRows * g + r)));
  }
#pragma unroll
  for (int j = 0; j < kWCopies; ++j) asm volatile("" : "+v"(o.vo[j]));
  return o;
}

// ---------------------------------------------------------------------------
// fp8 cache (E4M3 latent codes, one fp32 scale per token and 128 channels,
// bf16 k^R): each block's codes, scales and k^R land in a staging buffer and
// are expanded into a bf16 block buffer (code * scale rounded to bf16, the
// 8-wave kernel's arithmetic) during the step before the block is scored,
// between that step's score products.  The products are the bf16 path's.
// ---------------------------------------------------------------------------
// Staging layout: codes [32 rows][512], the 16-byte chunk c of row r at
// chunk position c ^ 8 (r & 1); scales [32][4] fp32, then 128 bytes that the
// scale copies may overrun with zeros; k^R [32][64] bf16.
constexpr int kW8Codes = 0;
constexpr int kW8Scales = kBlockRows * kDc;                   // 16384
constexpr int kW8Kr = kW8Scales + kBlockRows * 16 + 128;      // 17024
constexpr int kW8Stage = kW8Kr + kBlockRows * kDr * 2;        // 21120
static_assert(kW8Stage % 16 == 0, "staging buffers stay 16-byte aligned");

struct WideFp8Copies {
  __amdgpu_buffer_rsrc_t rc, rk, rs;  // codes, k^R, scales of the block's rows (zeros past the valid ones)
  uint32_t lb;                        // the staging buffer
};

__device__ __forceinline__ WideFp8Copies plan_block_fp8w(const DecodeArgs& a, int page, int half, int hi,
                                                         uint32_t stage) {
  const size_t row0 = (size_t)page * kPage + half * kBlockRows;
  WideFp8Copies c;
  c.rc = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(a.ckv8 + row0 * kDc), (short)0, uniform(hi * kDc),
                                           kRsrcWord3);
  c.rk = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(a.kr8 + row0 * (kDr * 2)), (short)0,
                                           uniform(hi * kDr * 2), kRsrcWord3);
  c.rs = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(a.scale8 + row0 * 4), (short)0, uniform(hi * 16),
                                           kRsrcWord3);
  c.lb = stage;
  return c;
}

// Copy t (0..5) of wave w for one block: t < 4 moves codes of rows
// 2(4w+t), 2(4w+t)+1 (1 KB, in the staging permutation: lane l fills chunk
// position l & 31 of row 2(4w+t) + (l >> 5), which holds chunk
// (l & 31) ^ 8 (l >> 5)); t = 4 the k^R of rows 8w .. 8w+7; t = 5 the scales
// of rows 8w .. 8w+15 with 4-byte copies (the last 8 of them also land, with
// the same values, in the next wave's; wave 3's extra rows are past the
// block and arrive as zeros in the pad).
template <bool NT>
__device__ __forceinline__ void issue_copy_fp8w(const WideFp8Copies& c, int t, int w, uint32_t code_voff) {
  const int lane = lane_id_fresh();
  if (t < 4) {
    const uint32_t off = (uint32_t)(4 * w + t) * kCopyBytes;
    lds_dma16_hint<NT>(c.rc, c.lb + kW8Codes + off, code_voff, off);
  } else if (t == 4) {
    lds_dma16_hint<NT>(c.rk, c.lb + kW8Kr + w * kCopyBytes, (uint32_t)(16 * lane), w * kCopyBytes);
  } else if (t == 5) {
    lds_dma4_hint<NT>(c.rs, c.lb + kW8Scales + w * 128, (uint32_t)(4 * lane), w * 128);
  }
}
constexpr int kW8Copies = 6;

// The expansion of one block by the 256 threads.  Thread t takes row r and
// the four 16-code chunks g + 8j' (one per 128-channel tile) of it: with
// q = t >> 4, e = (t >> 3) & 1, g = t & 7, r = b(q) or b(q) ^ 5 for
// b(q) = (q & 3) + 8 (q >> 2).  Rows r and r ^ 5 share a quarter-wave and
// differ in parity and in bit 2, which makes both the staging reads (slot j
// at chunk position g + 8j, i.e. chunk g + 8 (j ^ (r & 1))) and the writes
// into the bf16 layout free of bank conflicts.  Slices by score product kk:
// scales at 0, k^R read at 2 and written at 12, per-block setup at 4, slot
// j read at 8j + 1 and converted in two halves at 8j + 5/6 (written at
// 8j + 7) and 8j + 8/9 (written at 8j + 10).
struct WideExpand {
  int r, g;        // the thread's row and chunk (fixed)
  floatx4 sc;      // the row's four scales, in slot order
  int4v kr;        // a 16-byte piece of k^R
  int4v code[2];   // slot codes in flight (two slots overlap)
  bf16x8 out;      // half a slot, converted
  uint32_t w0, w1; // write bases of the two halves (slot 0 position)
  int p;           // r & 1
};

__device__ __forceinline__ int expand_row(int t) {
  const int q = t >> 4, e = (t >> 3) & 1;
  const int b = (q & 3) + 8 * (q >> 2);
  return e ? (b ^ 5) : b;
}

__device__ __forceinline__ void expand_init(WideExpand& X) {
  const int t = threadIdx.x;
  X.r = expand_row(t);
  X.g = t & 7;
}

__device__ __forceinline__ void expand_slice(WideExpand& X, int kk, uint32_t stage, uint32_t buf) {
  const int r = X.r, g = X.g;
  if (kk == 0) {
    X.sc = *(const MLA_LDS floatx4*)(uintptr_t)(stage + kW8Scales + 16 * r);
  } else if (kk == 2) {
    // k^R piece of row thread / 8, chunk thread % 8
    const int t = (int)threadIdx.x;
    X.kr = lds_read_b128_at(stage + kW8Kr + (t >> 3) * (kDr * 2) + 16 * (t & 7));
  } else if (kk == 4) {
    // slot j holds tile j ^ p: swap the scales into slot order
    X.p = r & 1;
    const floatx4 s0 = X.sc;
    const bool sw1 = X.p != 0;
    X.sc[0] = sw1 ? s0[1] : s0[0];
    X.sc[1] = sw1 ? s0[0] : s0[1];
    X.sc[2] = sw1 ? s0[3] : s0[2];
    X.sc[3] = sw1 ? s0[2] : s0[3];
    const int sw = swzw(r) << 4;
    X.w0 = buf + r * kRowBytes + 128 * (g >> 2) + ((32 * (g & 3)) ^ sw);
    X.w1 = buf + r * kRowBytes + 128 * (g >> 2) + ((32 * (g & 3) + 16) ^ sw);
  } else if (kk == 12) {
    const int t = (int)threadIdx.x;
    const int rk = t >> 3, kc = t & 7;
    *(MLA_LDS int4v*)(uintptr_t)(buf + lds_off_w(rk, kDc * 2 + 16 * kc)) = X.kr;
  }
  if (kk >= 1 && kk <= 25 && (kk - 1) % 8 == 0) {
    const int j = (kk - 1) / 8;
    X.code[j & 1] = lds_read_b128_at(stage + kW8Codes + r * kDc + 16 * g + 128 * j);
  }
  if (kk >= 5 && kk <= 34) {
    const int j = (kk - 5) / 8, ph = (kk - 5) % 8;  // phases 0,1: words 0,1; 2: write; 3,4: words 2,3; 5: write
    if (j < 4 && ph != 2 && ph != 5 && ph < 5) {
      const int wd = ph < 2 ? ph : ph - 1;           // word 0..3
      const float scj = X.sc[j];
      const int word = X.code[j & 1][wd];
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      const int o = 4 * (wd & 1);
      X.out[o + 0] = f2bf(lo[0] * scj);
      X.out[o + 1] = f2bf(lo[1] * scj);
      X.out[o + 2] = f2bf(hi[0] * scj);
      X.out[o + 3] = f2bf(hi[1] * scj);
      asm volatile("" : "+v"(X.out));
    } else if (j < 4 && (ph == 2 || ph == 5)) {
      const uint32_t dst = (ph == 2 ? X.w0 : X.w1) + ((uint32_t)(j ^ X.p) << 8);
      *(MLA_LDS bf16x8*)(uintptr_t)dst = X.out;
    }
  }
}

// Keep a value computed at this point of the instruction sequence.
__device__ __forceinline__ void anchor(float& x) { asm volatile("" : "+v"(x)); }

// Maxima that need no quieting of their inputs (the operands are scores or
// -inf, never NaN): gfx950's three-input maximum.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float pair32_maximum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One step of the unit's block stream: the scores of block i (buffer
// `A.sa`), the online softmax of block i, and the value product of block
// i-1 (buffer `A.va`) with its probabilities Pp.  Written as one straight
// sequence of 68 matrix-core products, each with the operand read it needs
// D products ahead (the ring rb), the page copies of block i+2 after every
// fourth score product and the softmax arithmetic spread over the value
// products; the scheduling barriers keep that order (left to itself the
// compiler gathered the reads next to their products and the softmax ahead
// of them, and the one wave on each SIMD then waited on every LDS round
// trip).
// Order of the products: value products 0 .. V0-1, the 36 score products,
// value products V0 .. 31.  With V0 > 0 the operands of the first V0 come
// from reads issued at the end of the previous step, before the loop's
// barrier: they read block i-1, which has been in place since the step
// before and is not overwritten before the next barrier, so right after the
// barrier the matrix cores have work whose operands are already in
// registers while the first score reads of the newly landed block are in
// flight.  With V0 = 0 a step reads its first D operands itself.  Every
// value tile still accumulates its products in the same order.
// advance() moves A to the next step's buffers; it is called once the last
// read of this step's operands is issued.
// mask (uniform): tokens at or past hi (per lane) are excluded.  The
// callbacks place the rest of a step's work between score products, where
// it issues in their shadow instead of after them: copy(t) issues copy t of
// a later block after score products 3, 7, .., 35 (t = 0..8); book(t), t =
// 0, 1, 2, the scalar bookkeeping (the next copy plan, the block cursors)
// after score products 1, 5 and 9; expand(kk) a slice of the fp8 expansion
// of the next block after every score product kk.
template <int D, int V0, class Copy, class Book, class Expand, class Advance>
__device__ __forceinline__ void wide_step(const WideQuery& Q, WideAcc& Z, WideAddr& A, bf16x8 (&rb)[D],
                                          const bf16x8 (&Pp)[2], bf16x8 (&Pc)[2], WideSoftmax& st,
                                          float scale_log2, bool mask, int hi, bool& rescale, float& alpha,
                                          Copy&& copy, Book&& book, Expand&& expand, Advance&& advance) {
  constexpr int kP = 68;  // 36 score + 32 value products
  static_assert(V0 == 0 || (V0 >= D && V0 <= 16 && kP % D == 0),
                "lead value products: their reads fill the ring in order and never read the new block");
  // the operand of product p of this step
  auto operand = [&](int p) {
    return p < V0 ? value_operand(A, p) : p < V0 + 36 ? score_operand(A, p - V0) : value_operand(A, p - 36);
  };
  if constexpr (V0 == 0) {
#pragma unroll
    for (int j = 0; j < D; ++j) rb[j] = operand(j);
  }
  // issue the read for product p + D into the slot product p frees
  auto refill = [&](int p) {
    if (p + D < kP) {
      rb[p % D] = operand(p + D);
    } else if constexpr (V0 > 0) {
      rb[p % D] = value_operand(A, p + D - kP);  // the next step's lead products (A advanced)
    }
    if (p + D == kP - 1) advance();
  };
  // lead value products 0 .. V0-1, each issued before the read that
  // refills its slot: the first waits only for operands read before the
  // barrier (and the page load), not for a read of the new block
#pragma unroll
  for (int p = 0; p < V0; ++p) {
    mfma32_acc(Z.z[p & 15], rb[p % D], Pp[0]);
    refill(p);
    __builtin_amdgcn_sched_barrier(0);
  }
  // scores
  floatx16 S = floatx16{};
#pragma unroll
  for (int kk = 0; kk < 36; ++kk) {
    const int p = V0 + kk;
    const bf16x8 a = rb[p % D];
    refill(p);
    S = mfma32(a, Q.q[kk], S);
    if ((kk & 3) == 3) copy(kk >> 2);
    if ((kk & 3) == 1 && kk < 12) book(kk >> 2);
    expand(kk);
    __builtin_amdgcn_sched_barrier(0);
  }
  // value products V0 .. 31 with the softmax of S woven in
  const int h = lane_id_fresh() >> 5;
  float mx = -INFINITY, sum = 0.f, nm = 0.f;
  bool need = false;
#pragma unroll
  for (int m = 0; m < 32 - V0; ++m) {
    const int n = V0 + m, p = 36 + n;
    const bf16x8 a = rb[p % D];
    refill(p);
    mfma32_acc(Z.z[n & 15], a, Pp[n >> 4]);
    // each piece of the softmax is pinned to its step (anchor()): its
    // results are used only in the next step, and the compiler would
    // otherwise move the arithmetic out of this sequence
    if (m == 2) {
      if (__builtin_expect(mask, 0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * h + (r & 3) >= hi) S[r] = -INFINITY;
      }
      mx = max3f(max3f(max3f(S[0], S[1], S[2]), max3f(S[3], S[4], S[5]), max3f(S[6], S[7], S[8])),
                 max3f(S[9], S[10], S[11]), max3f(max3f(S[12], S[13], S[14]), S[15], -INFINITY));
      anchor(mx);
    } else if (m == 3) {
      mx = pair32_maximum(mx) * scale_log2;  // scale > 0: the maximum commutes with it
      anchor(mx);
    } else if (m == 4) {
      // the first scores of a piece set the maximum (the accumulators are
      // zero); later ones move it only when it grows by more than 2^8
      const float mnew = __builtin_elementwise_maximum(st.m, mx);
      const bool first = st.m == -INFINITY;
      need = !first && mnew > st.m + kLazyRescale;
      alpha = need ? fast_exp2(st.m - mnew) : 1.0f;
      st.l *= alpha;
      st.m = (need || first) ? mnew : st.m;
      // a head that has seen only masked scores keeps m = -inf: probabilities 0
      nm = st.m == -INFINITY ? 0.f : -st.m;
      anchor(nm);
      anchor(alpha);
      anchor(st.l);
      anchor(st.m);
    } else if (m == 5) {
      rescale = __builtin_amdgcn_ballot_w64(need) != 0;
    } else if (m >= 6 && m < 22) {
      const int r = m - 6;
      float pr = fast_exp2(fmaf(S[r], scale_log2, nm));
      anchor(pr);
      sum += pr;
      anchor(sum);
      Pc[r >> 3][r & 7] = f2bf(pr);
      if (r & 1) asm volatile("" : "+v"(Pc[r >> 3]));
    } else if (m == 22) {
      st.l += sum;
      anchor(st.l);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// NT: the copies carry the non-temporal hint (decode streams every row
// once; prefill re-reads the same keys for every query row and keeps them
// cached).
template <bool FP8, bool NT>
__global__ void __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_wide_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  // bf16: four block buffers.  fp8: three bf16 block buffers and two
  // staging buffers (the copies of block i+2 land in one while block i+1 is
  // expanded from the other).
  constexpr int NB = FP8 ? kWNBuf8 : kWNBuf;
  constexpr int D = FP8 ? kWDepth8 : kWDepth, V0 = FP8 ? kWLead8 : kWLead;
  constexpr int kBufBytes = NB * kBlockBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBufBytes + (FP8 ? 2 * kW8Stage : 0)];
  __shared__ int pfx[kMaxSchedB + 1];
  __shared__ int lens[kMaxSchedB];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h0 = 32 * wave;

  int P = 0;
  if (a.splits == 0 && a.prefill_T == 0) P = block_prefix(a.seq_lens, a.B, pfx, lens, nullptr, 0, nullptr);
  Cursor cp;
  cp.sch = schedule_begin(a, pfx, lens, P);
  cp.valid = schedule_next(a, cp.sch, cp.seg);
  if (!cp.valid) return;
  cp.k = cp.seg.t0 / kBlock;

  auto qrow = [&](const Segment& s) { return (const bf16*)a.q + (size_t)s.b * a.H * kRow; };
  auto block_hi = [&](const Cursor& c) { return min(c.seg.t1 - c.k * kBlock, kBlock); };
  // The page of the block at cursor c, a block-table entry read with a
  // scalar load.
  auto page_fetch = [&](const Cursor& c) {
    if (!c.valid) return 0;
    const int32_t* bt = a.prefill_T > 0 ? block_table : block_table + (size_t)c.seg.b * a.max_pages;
    return bt[uniform(c.k >> 1)];
  };
  auto note_pieces = [&](const Segment& s) {
    if (a.meta != nullptr && s.slot == s.slot0 && tid == 0) *(int2*)(a.meta + 2 * s.b) = make_int2(s.slot0, s.parts);
  };
  // copies of block j (at cursor c, on page pg) into its buffer (bf16) or
  // staging buffer (fp8); no rows when c is past the unit's work
  const uint32_t stage0 = lds_addr(smem + kBufBytes);
  auto plan_wide = [&](const Cursor& c, int pg, int j) {
    const int half = c.valid ? c.k & 1 : 0, rows = c.valid ? block_hi(c) : 0;
    if constexpr (FP8) {
      return plan_block_fp8w(a, uniform(pg), half, rows, stage0 + (uint32_t)(j & 1) * kW8Stage);
    } else {
      const uint8_t* page = a.rows + (size_t)uniform(pg) * kPageBytes;
      return plan_block_wide(page, half, smem + (j % NB) * kBlockBytes, rows, wave);
    }
  };
  // where a piece's normalised sums go: z and lse for a whole sequence, a
  // partial slot otherwise
  auto piece_out = [&](const Segment& sg, float*& zo, float*& lo) {
    const bool whole = sg.parts == 1;
    zo = whole ? a.z + (size_t)sg.b * a.H * kDc : a.zp + (size_t)sg.slot * a.H * kDc;
    lo = whole ? (a.lse ? a.lse + (size_t)sg.b * a.H : nullptr) : a.lsep + (size_t)sg.slot * a.H;
  };

  // The value product of step 0 reads buffer NB - 1 with zero
  // probabilities: its rows must be finite, so it starts as zeros.
  for (int j = tid; j < kBlockBytes / 16; j += kWThreads)
    *(int4v*)(smem + (NB - 1) * kBlockBytes + 16 * j) = int4v{0, 0, 0, 0};

  WideQuery Q;
  WideAcc Z;
  WideSoftmax st;
  WideCopyOffsets co;      // bf16: source offsets of the nine copies
  uint32_t code_voff = 0;  // fp8: source offset of the lane in a code copy
  WideExpand X;
  if constexpr (FP8) {
    const int lane = lane_id_fresh();
    code_voff = (uint32_t)((lane >> 5) * kDc + 16 * ((lane & 31) ^ (8 * (lane >> 5))));
    asm volatile("" : "+v"(code_voff));
    expand_init(X);
  } else {
    co = copy_offsets(wave);
  }
  auto issue_block = [&](const auto& nbk, int t) {
    if constexpr (FP8) {
      if (t < kW8Copies) issue_copy_fp8w<NT>(nbk, t, wave, code_voff);
    } else {
      lds_dma16_hint<NT>(nbk.rs, nbk.lb + kCopyBytes * t, co.vo[t], nbk.g * kGroupBytes);
    }
  };
  load_query_wide(Q, qrow(cp.seg), a.H, h0);
  Cursor ld = cp;
#pragma unroll
  for (int j = 0; j < kWAhead; ++j) {
    // the first two blocks (a piece shorter than that leaves a copy of no
    // rows: it moves nothing and keeps the count of copies per block fixed)
    const auto nbj = plan_wide(ld, page_fetch(ld), j);
#pragma unroll
    for (int t = 0; t < kWCopies; ++t) issue_block(nbj, t);
    if (ld.valid) cursor_next(a, ld);
  }
  if constexpr (FP8) {
    // block 0 is expanded before the loop (its copies are the older half of
    // the two blocks in flight); block 1 is expanded in step 0
    wait_vmcnt<kW8Copies>();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 36; ++kk) expand_slice(X, kk, stage0, lds_addr(smem));
  }
  auto nb = plan_wide(ld, page_fetch(ld), kWAhead);
  if (ld.valid) cursor_next(a, ld);
  int ld_klast = (ld.seg.t1 - 1) / kBlock;  // the copy cursor's last block in its piece
  consume_query_wide(Q);
  reset_acc_mfma(Z);
  st.m = -INFINITY;
  st.l = 0.f;
  note_pieces(cp.seg);
  const uint32_t base = lds_addr(smem);
  WideAddr A = wide_addr(base, base + (NB - 1) * kBlockBytes);
  __syncthreads();  // the zeroed buffer (and fp8: block 0) is visible to every wave
  bf16x8 rb[D];     // operand reads in flight (wide_step)
  if constexpr (V0 > 0) {
#pragma unroll
    for (int j = 0; j < D; ++j) rb[j] = value_operand(A, j);  // step 0's lead products (zero rows)
  }

  // The block scored in the previous step, whose value product is still to
  // be done: its probabilities, where its piece goes and, if it ended the
  // piece, the piece's softmax totals.
  bf16x8 Pp[2] = {bf16x8{}, bf16x8{}};
  bool prev_last = false;
  float* zdst = nullptr;    // its piece's output rows
  float* ldst = nullptr;
  float *zcur, *lcur;       // those of the piece being scored
  piece_out(cp.seg, zcur, lcur);
  int klast = (cp.seg.t1 - 1) / kBlock;  // its last block
  bool has_stored = false;  // a flush left part of its piece's sums there
  float l_end = 0.f, m_end = 0.f;

  for (int i = 0;; ++i) {
    const bool cur = cp.valid;  // block i exists (else only block i-1's value product is left)
    // the page of block i+3 for the copy plan in this step: a scalar load.
    // bf16: issued before the barrier, so that it arrives under the wait
    // there (the first product waits for every LDS read and scalar load in
    // flight); fp8: after it, under the first score reads.
    int pg = 0;
    if constexpr (!FP8) pg = page_fetch(ld);
    if constexpr (FP8) {
      // the staged copies of block i+1 (the only ones in flight) and this
      // wave's expansion of block i (LDS stores) are complete
      wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
      // every wave issues nine copies per block, so the copies of the block
      // after this one are the last nine issued
      wait_blocks_wide(1);
    }
    // block i has landed; every wave is done with step i-1.  A bare barrier:
    // the copies are complete by the wait above, every LDS read of step i-1
    // was consumed by its product except the lead reads of this step (of
    // block i-1, whose buffer the copies of this step do not touch), and no
    // ordinary LDS store is in flight, so no fence (and no wait for the page
    // read in flight) is needed; the empty asm keeps the compiler from moving
    // LDS reads across it.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (FP8) pg = page_fetch(ld);
    // multi-token decode: query token t of the sequence sees keys up to
    // L - q_len + t, so the last q_len - 1 - t keys are masked for it
    int hi = cur ? block_hi(cp) : kBlock;
    const bool mask = hi < kBlock || a.q_len > 1;
    if (a.q_len > 1 && cur) {
      const int head = min(h0 + (lane_id_fresh() & 31), a.H - 1);
      hi = min(hi, cp.seg.L - (a.q_len - 1 - head / a.hs) - kBlock * cp.k);
    }
    bf16x8 Pc[2];
    bool rescale_c = false;
    float alpha_c = 1.f;
    // Bookkeeping inside the step (the common case of each cursor move; a
    // move to another piece is finished after the step): the copy plan of
    // block i+3, then the copy cursor and the scoring cursor one block on.
    decltype(nb) nb_next;
    bool ld_switch = false;
    const bool last_now = cur && cp.k == klast;  // block i ends its piece
    auto book = [&](int t) {
      if (t == 0) {
        nb_next = plan_wide(ld, pg, i + kWAhead + 1);
      } else if (t == 1) {
        ld_switch = ld.valid && ld.k == ld_klast;
        ld.k += (ld.valid && !ld_switch) ? 1 : 0;
      } else {
        cp.k += (cur && !last_now) ? 1 : 0;
      }
    };
    // scores and softmax of block i (of stale rows when there is no block i:
    // unused), value product of block i-1 (zero probabilities at i = 0), and
    // the copies of block i+2 into the buffer of block i-2
    auto copy = [&](int t) { issue_block(nb, t); };
    // fp8: block i+1 from its staging buffer into the buffer of block i-2
    const uint32_t xs = stage0 + (uint32_t)((i + 1) & 1) * kW8Stage;
    const uint32_t xb = base + (uint32_t)((i + 1) % NB) * kBlockBytes;
    auto expand = [&](int kk) {
      if constexpr (FP8) expand_slice(X, kk, xs, xb);
    };
    auto advance = [&]() { advance_addr<NB>(A, i); };
    wide_step<D, V0>(Q, Z, A, rb, Pp, Pc, st, a.scale_log2, mask, hi, rescale_c, alpha_c, copy, book, expand,
                     advance);
    // Everything that does not happen at every block (a moved maximum, the
    // end of a piece, a cursor moving to another piece, the end of the
    // unit's work) behind one branch.
    const bool rare = !cur || rescale_c || prev_last || ld_switch || last_now;
    if (__builtin_expect(rare, 0)) {
      if (i > 0 && cur && rescale_c) {
        // block i moved a running maximum: the sums up to block i-1 are
        // relative to the old one (block i's value product comes next)
        acc_settle();
        flush_wide(Z, alpha_c, has_stored, zdst, h0, a.H);
        has_stored = true;
      }
      if (i > 0 && prev_last) {
        // block i-1 ended its piece: its sums are complete
        acc_settle();
        store_wide(Z, l_end, m_end, has_stored, zdst, ldst, h0, a.H);
        has_stored = false;
        reset_acc_mfma(Z);
      }
      if (!cur) {
        wait_vmcnt<0>();  // no copy into this workgroup's LDS outlives it
        break;
      }
      if (ld_switch) {
        cursor_next(a, ld);  // to the copy cursor's next piece
        ld_klast = (ld.seg.t1 - 1) / kBlock;
      }
      zdst = zcur;
      ldst = lcur;
      if (last_now) {
        // block i ends its piece: keep its totals for the store after the
        // next value product, and move to the next piece
        l_end = pair32_sum(st.l);
        m_end = st.m;
        cursor_next(a, cp);
        if (cp.valid) {
          // its query replaces this one (only the value product of the
          // finished piece remains, and it does not use the query)
          load_query_wide(Q, qrow(cp.seg), a.H, h0);
          consume_query_wide(Q);
          st.m = -INFINITY;
          st.l = 0.f;
          note_pieces(cp.seg);
          piece_out(cp.seg, zcur, lcur);
          klast = (cp.seg.t1 - 1) / kBlock;
        }
      }
    } else {
      zdst = zcur;
      ldst = lcur;
    }
    nb = nb_next;  // the copies of block i+3, issued in the next step
    Pp[0] = Pc[0];
    Pp[1] = Pc[1];
    prev_last = last_now;
  }
}

}  // namespace

hipError_t launch_decode_wide(const DecodeArgs& a, bool fp8, hipStream_t s) {
  const dim3 grid(a.units), blk(kWThreads);
  const bool nt = a.prefill_T == 0;
  if (fp8 && nt) hipLaunchKernelGGL((decode_wide_kernel<true, true>), grid, blk, 0, s, a, a.block_table);
  else if (fp8) hipLaunchKernelGGL((decode_wide_kernel<true, false>), grid, blk, 0, s, a, a.block_table);
  else if (nt) hipLaunchKernelGGL((decode_wide_kernel<false, true>), grid, blk, 0, s, a, a.block_table);
  else hipLaunchKernelGGL((decode_wide_kernel<false, false>), grid, blk, 0, s, a, a.block_table);
  return hipGetLastError();
}

}  // namespace mla
