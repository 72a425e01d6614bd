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
//     heads of scores in two chains; 32 channels x 32 heads per value tile);
//   * the value product of block i-1 runs after the scores of block i, so
//     the softmax of block i can issue while the matrix cores work through
//     the value products; that keeps block i-1 readable for one more step,
//     so two blocks (not three) are in flight while one is scored and one is
//     accumulated (four 36 KB buffers).
// The work schedule, the paged copies (LDS-DMA), the row layout in LDS and
// the split-KV partials are those of decode.hip (decode_common.h).
#include "decode_common.h"

namespace mla {
namespace {

constexpr int kWWaves = 4;                  // one wave per SIMD
constexpr int kWThreads = kWWaves * 64;
constexpr int kWNBuf = 4;                   // value(i-1), scores(i), blocks i+1 and i+2 in flight
constexpr int kWAhead = 2;                  // blocks copied ahead of the one being scored
constexpr int kWCopies = kCopiesPerGroup;   // 9 copies per wave and block: wave w moves 8-row group w
constexpr int kWBt = 4 * kWThreads;         // block-table entries block_prefix can copy with 256 threads
constexpr int kWScoreDepth = 6;             // score operand reads in flight
constexpr int kWValueDepth = 3;             // value operand tiles (two transposing reads each) in flight

static_assert(kWWaves * kGroupRows == kBlockRows, "four waves move the four 8-row groups of a block");

// LDS row layout of this kernel: rows of 1152 bytes, the 16-byte chunks of
// row r permuted inside each aligned group of eight as c -> c ^ swzw(r).
// swzw(r) = 4 ((r >> 2) & 1) + ((r >> 3) & 3) is a different permutation from
// decode.hip's, chosen for the 32x32 operand patterns (gfx950 serves a 16-byte
// read per half-wave and a transposing 8-byte read per wave from 128 banks of
// 4 bytes):
//   * score operand: a half-wave reads one chunk of all 32 rows; rows of equal
//     r % 4 sit in the same 128-byte bank window, and swzw takes eight
//     distinct values over r >> 2, so the 32 reads fill 512 distinct bytes;
//   * value operand: a wave reads 8 rows base + 4h + k (h, k < 4; base a
//     multiple of 8) at four chunks 4(ct & 1) + 2hf + e; bit 2 of swzw is h,
//     so the two row halves land in disjoint halves of each chunk group, and
//     the 64 eight-byte reads again fill 512 distinct bytes.
__device__ __forceinline__ int swzw(int r) { return 4 * ((r >> 2) & 1) + ((r >> 3) & 3); }
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

// Copy j of this wave: lane i fills LDS chunk 64j + i of the 8-row group,
// i.e. chunk cc of row r = (64j + i) / 72, which holds source chunk
// cc ^ swzw(8g + r).
__device__ __forceinline__ void issue_copy_wide(const WideCopies& c, int j) {
  const int lane = lane_id_fresh();
  const int q = 64 * j + lane;
  const int r = q / 72, cc = q - 72 * r;
  const uint32_t vo = (uint32_t)(r * kRowBytes + 16 * (cc ^ swzw(kGroupRows * c.g + r)));
  lds_dma16(c.rs, c.lb + kCopyBytes * j, vo, c.g * kGroupBytes);
}

// Wait until at most the copies of this wave's n (0 or 1) most recently
// issued blocks are in flight.
__device__ __forceinline__ void wait_blocks_wide(int n) {
  if (n >= 1) wait_vmcnt<kWCopies>(); else wait_vmcnt<0>();
}

// Scores of the 32 rows of a block buffer: S^T = R Q^T (32 tokens x 32
// heads), K = 576 in 36 steps of 16, accumulated in two chains (even and odd
// steps) so that consecutive products do not wait on each other.  Lane l of
// the result holds head h0 + l % 32 and tokens 8(r / 4) + 4h + r % 4.
// dma(t) (t = 0..8) is called after every fourth K-step.
template <class Dma>
__device__ __forceinline__ floatx16 scores_wide(const WideQuery& Q, uint32_t buf, Dma&& dma) {
  const int lane = lane_id_fresh();
  const int row = lane & 31, h = lane >> 5;
  // A operand at K-step kk: row `row`, bytes 32kk + 16h; the permutation
  // touches bits 4..6, so kk % 4 picks one of four bases and kk / 4 adds 128
  uint32_t ap[4];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) ap[k4] = buf + lds_off_w(row, 32 * k4 + 16 * h);
  asm volatile("" : "+v"(ap[0]), "+v"(ap[1]), "+v"(ap[2]), "+v"(ap[3]));
  auto rd = [&](int kk) { return lds_read_b128_at(ap[kk & 3] + 128 * (kk >> 2)); };
  floatx16 S0 = floatx16{}, S1 = floatx16{};
  constexpr int D = kWScoreDepth;
  int4v a[D];
#pragma unroll
  for (int i = 0; i < D; ++i) a[i] = rd(i);
#pragma unroll
  for (int kk = 0; kk < 36; ++kk) {
    const bf16x8 c = __builtin_bit_cast(bf16x8, a[kk % D]);
    if (kk + D < 36) a[kk % D] = rd(kk + D);
    if (kk & 1) S1 = mfma32(c, Q.q[kk], S1); else S0 = mfma32(c, Q.q[kk], S0);
    if ((kk & 3) == 3) dma(kk >> 2);
  }
  return S0 + S1;
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

// Value product of one block buffer: Z^T_ct += C^T_ct P^T over the two
// K-steps t of 16 tokens.  Slot 8h + j of step t is token 16t + 4h + j
// (j < 4) or 16t + 8 + 4h + (j - 4): P[t] is then score registers 8t .. 8t+7
// of the lane as they are, and the A operand (32 channels x 16 tokens) comes
// from two transposing reads: in 16-lane group G (h = G / 2, hf = G % 2)
// lane s points at row 16t + 4h + s / 4 (resp. + 8), bytes
// 64ct + 32hf + 8(s % 4) .. +7, and receives channel 32ct + 16hf + s.
__device__ __forceinline__ void value_wide(WideAcc& Z, const bf16x8 (&P)[2], uint32_t buf) {
  const int lane = lane_id_fresh();
  const int G = lane >> 4, s = lane & 15;
  const int h = G >> 1, hf = G & 1;
  const int x = 32 * hf + 8 * (s & 3);
  uint32_t vb[2][2][2];  // [t][lo / hi rows][ct % 2]; ct / 2 adds 128 bytes
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) vb[t][hh][c2] = buf + lds_off_w(16 * t + 8 * hh + 4 * h + (s >> 2), 64 * c2 + x);
  asm volatile("" : "+v"(vb[0][0][0]), "+v"(vb[0][0][1]), "+v"(vb[0][1][0]), "+v"(vb[0][1][1]));
  asm volatile("" : "+v"(vb[1][0][0]), "+v"(vb[1][0][1]), "+v"(vb[1][1][0]), "+v"(vb[1][1][1]));
  // operand n: K-step n / 16, channel tile n % 16 (a tile's two products
  // are 16 products apart, so none waits for the one before)
  auto vread = [&](int n) {
    const int ct = n & 15, t = n >> 4;
    const bf16x4 lo = lds_read_tr16_at(vb[t][0][ct & 1] + 128 * (ct >> 1));
    const bf16x4 hi = lds_read_tr16_at(vb[t][1][ct & 1] + 128 * (ct >> 1));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  constexpr int D = 2 * kWValueDepth;
  bf16x8 va[D];
#pragma unroll
  for (int i = 0; i < D; ++i) va[i] = vread(i);
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    const bf16x8 cur = va[n % D];
    if (n + D < 32) va[n % D] = vread(n + D);
    mfma32_acc(Z.z[n & 15], cur, P[n >> 4]);
  }
}

// Online softmax of a block's scores for the lane's head.  Tokens at or past
// hi are masked (it may differ per head in multi-token decode).  Returns the
// block's probabilities as the value product's B operands and, when the
// running maximum moved, the factor the accumulators must be scaled by
// before this block's value product (rescale set, alpha).
__device__ __forceinline__ void softmax_wide(WideSoftmax& st, const floatx16& S, int hi, float scale_log2,
                                             bf16x8 (&P)[2], bool& rescale, float& alpha) {
  const int h = lane_id_fresh() >> 5;
  float x[16];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float y = 8 * (r >> 2) + 4 * h + (r & 3) < hi ? S[r] * scale_log2 : -INFINITY;
    x[r] = y;
    mx = fmaxf(mx, y);
  }
  mx = pair32_max(mx);
  const float mnew = fmaxf(st.m, mx);
  // the first scores of a piece set the maximum (the accumulators are
  // zero); later ones move it only when it grows by more than 2^8
  const bool need = st.m != -INFINITY && mnew > st.m + kLazyRescale;
  if (st.m == -INFINITY) st.m = mnew;
  rescale = __builtin_amdgcn_ballot_w64(need) != 0;
  if (__builtin_expect(rescale, 0)) {
    alpha = need ? fast_exp2(st.m - mnew) : 1.0f;
    if (need) st.m = mnew;
    st.l *= alpha;
  }
  // a head that has seen only masked scores keeps m = -inf: probabilities 0
  const float mref = st.m == -INFINITY ? 0.f : st.m;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = fast_exp2(x[r] - mref);
    sum += p;
    P[r >> 3][r & 7] = f2bf(p);
  }
  st.l += sum;
}

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

template <bool FP8>
__global__ void __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_wide_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  static_assert(!FP8, "the fp8 cache takes the 16-head kernel");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWNBuf * kBlockBytes];
  __shared__ int pfx[kMaxSchedB + 1];
  __shared__ int lens[kMaxSchedB];
  __shared__ int bt_lds[kWBt];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h0 = 32 * wave;

  const bool bt_local = a.splits == 0 && a.prefill_T == 0 && a.B * a.max_pages <= kWBt;
  int P = 0;
  if (a.splits == 0 && a.prefill_T == 0)
    P = block_prefix(a.seq_lens, a.B, pfx, lens, bt_local ? block_table : nullptr, a.B * a.max_pages, bt_lds);
  Cursor cp;
  cp.sch = schedule_begin(a, pfx, lens, P);
  cp.valid = schedule_next(a, cp.sch, cp.seg);
  if (!cp.valid) return;
  cp.k = cp.seg.t0 / kBlock;

  auto qrow = [&](const Segment& s) { return (const bf16*)a.q + (size_t)s.b * a.H * kRow; };
  auto block_hi = [&](const Cursor& c) { return min(c.seg.t1 - c.k * kBlock, kBlock); };
  auto page_of = [&](const Cursor& c) {
    if (bt_local) return uniform(bt_lds[c.seg.b * a.max_pages + (c.k >> 1)]);
    const int32_t* bt = a.prefill_T > 0 ? block_table : block_table + (size_t)c.seg.b * a.max_pages;
    return bt[uniform(c.k >> 1)];
  };
  auto note_pieces = [&](const Segment& s) {
    if (a.meta != nullptr && s.slot == s.slot0 && tid == 0) *(int2*)(a.meta + 2 * s.b) = make_int2(s.slot0, s.parts);
  };
  // copies of the block at cursor c into buffer `slot`; no rows when c is
  // past the unit's work
  auto plan_wide = [&](const Cursor& c, int slot) {
    const uint8_t* page = c.valid ? a.rows + (size_t)page_of(c) * kPageBytes : a.rows;
    return plan_block_wide(page, c.valid ? c.k & 1 : 0, smem + slot * kBlockBytes, c.valid ? block_hi(c) : 0, wave);
  };

  WideQuery Q;
  WideAcc Z;
  WideSoftmax st;
  load_query_wide(Q, qrow(cp.seg), a.H, h0);
  Cursor ld = cp;
#pragma unroll
  for (int j = 0; j < kWAhead; ++j) {
    // the first two blocks (a piece shorter than that leaves a copy of no
    // rows: it moves nothing and keeps the count of copies per block fixed)
    const WideCopies nb = plan_wide(ld, j);
#pragma unroll
    for (int t = 0; t < kWCopies; ++t) issue_copy_wide(nb, t);
    if (ld.valid) cursor_next(a, ld);
  }
  consume_query_wide(Q);
  reset_acc_mfma(Z);
  st.m = -INFINITY;
  st.l = 0.f;
  note_pieces(cp.seg);

  // The block scored in the previous step, whose value product is still to
  // be done: its probabilities, where its piece goes and, if it ended the
  // piece, the piece's softmax totals.
  bf16x8 Pp[2];
  bool prev_last = false;
  float* zdst = nullptr;    // its piece's output rows
  float* ldst = nullptr;
  bool has_stored = false;  // a flush left part of its piece's sums there
  float l_end = 0.f, m_end = 0.f;

  for (int i = 0;; ++i) {
    const bool cur = cp.valid;  // block i exists (else only block i-1's value product is left)
    // every wave issues nine copies per block, so the copies of the block
    // after this one are the last nine issued
    wait_blocks_wide(1);
    __syncthreads();  // block i has landed; every wave is done with step i-1
    // the copies of block i + 2 go into the buffer of block i - 2
    const WideCopies nb = plan_wide(ld, (i + kWAhead) % kWNBuf);
    if (ld.valid) cursor_next(a, ld);
    // scores of block i (of stale rows when there is no block i: unused)
    const floatx16 S = scores_wide(Q, lds_addr(smem + (i % kWNBuf) * kBlockBytes),
                                   [&](int t) { issue_copy_wide(nb, t); });
    // softmax of block i: its probabilities go to the next step's value
    // product, after block i-1's (which still needs Pp)
    bf16x8 Pc[2];
    bool rescale_c = false;
    float alpha_c = 1.f;
    if (cur) {
      // multi-token decode: query token t of the sequence sees keys up to
      // L - q_len + t, so the last q_len - 1 - t keys are masked for it
      int hi = block_hi(cp);
      if (a.q_len > 1) {
        const int head = min(h0 + (lane_id_fresh() & 31), a.H - 1);
        hi = min(hi, cp.seg.L - (a.q_len - 1 - head / a.hs) - kBlock * cp.k);
      }
      softmax_wide(st, S, hi, a.scale_log2, Pc, rescale_c, alpha_c);
    }
    if (i > 0) {
      value_wide(Z, Pp, lds_addr(smem + ((i + kWNBuf - 1) % kWNBuf) * kBlockBytes));
      if (__builtin_expect(rescale_c, 0)) {
        // block i moved a running maximum: the sums up to block i-1 are
        // relative to the old one (block i's value product comes next)
        acc_settle();
        flush_wide(Z, alpha_c, has_stored, zdst, h0, a.H);
        has_stored = true;
      }
      if (prev_last) {
        acc_settle();
        store_wide(Z, l_end, m_end, has_stored, zdst, ldst, h0, a.H);
        has_stored = false;
        reset_acc_mfma(Z);
      }
    }
    if (!cur) break;
    Pp[0] = Pc[0];
    Pp[1] = Pc[1];
    prev_last = cp.k == (cp.seg.t1 - 1) / kBlock;
    {
      const Segment& sg = cp.seg;
      const bool whole = sg.parts == 1;
      zdst = whole ? a.z + (size_t)sg.b * a.H * kDc : a.zp + (size_t)sg.slot * a.H * kDc;
      ldst = whole ? (a.lse ? a.lse + (size_t)sg.b * a.H : nullptr) : a.lsep + (size_t)sg.slot * a.H;
    }
    if (prev_last) {
      l_end = pair32_sum(st.l);
      m_end = st.m;
    }
    cursor_next(a, cp);
    if (prev_last && cp.valid) {
      // next piece: its query replaces this one (only the value product of
      // the finished piece remains, and it does not use the query)
      load_query_wide(Q, qrow(cp.seg), a.H, h0);
      consume_query_wide(Q);
      st.m = -INFINITY;
      st.l = 0.f;
      note_pieces(cp.seg);
    }
  }
}

}  // namespace

hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_wide_kernel<false>), dim3(a.units), dim3(kWThreads), 0, s, a, a.block_table);
  return hipGetLastError();
}

}  // namespace mla
