// Absorbed-MLA decode over the paged latent cache, and the split-KV merge.
//
// Per query token and head i (the "DeepSeek-V3" notes, ekkoxiao.github.io):
//   s_j = (q~_i . c_j + q^R_i . k^R_j) * scale     (§注意力计算 + §潜在向量的作用)
//   a_j = softmax_j(s),  z_i = sum_j a_j c_j        (§潜在向量的作用)
// All heads of a sequence read the same cached rows, so for a 64-token page
// the scores of a wave's heads are one dense product S^T = R Q^T
// (R: 64 x 576 rows, Q: heads x 576), and the latent accumulation is a second
// one, Z^T += C^T P^T (C: the 512-wide c^KV part of the rows).  Both run on
// bf16 matrix cores with fp32 accumulation.
//
// Work decomposition (one 512-thread workgroup per unit of work):
//   * Pages stream HBM -> LDS with asynchronous LDS-DMA loads into one
//     buffer while the previous page is consumed; every row is read from HBM
//     once and shared by all heads.  The stream runs on across the sequence
//     boundaries inside a unit, so a unit never waits for a cold first page.
//   * Wave w owns 16 heads (hg = w % HG) and a token slice of each page
//     (tg = w / HG).  Its absorbed query stays in VGPRs, its accumulator Z^T
//     (16 heads x 512 fp32) in accumulation registers, and every value a lane
//     holds belongs to one head, so the online softmax never leaves the lane.
//   * Score operand: 16-byte LDS reads of rows.  Value operand: gfx950's
//     transposing LDS read (ds_read_b64_tr_b16) turns row-major c^KV into
//     token-packed matrix-core operands without a transposed copy.
//   * fp8 cache: the e4m3 codes, their per-(token, 128-channel) scales and
//     the bf16 k^R of a page land in a staging buffer and are expanded once
//     into the same bf16 row layout (code * scale rounded to bf16), so the
//     matrix-core part is shared with the bf16 cache ("DeepSeek-V3 Technical
//     Report", process-cxr.github.io, §Fine-grained quantization: scaling per
//     1 x 128 tile of a token, applied when the tile is consumed).
//   * Long sequences are cut into chunks; each chunk leaves a normalised
//     partial (z_c, lse_c) that is combined exactly:
//     lse = log sum_c e^{lse_c}, z = sum_c e^{lse_c - lse} z_c.  Either a
//     separate merge kernel does it, or the last unit to finish a chunk of a
//     sequence (found with a per-sequence arrival counter) merges it in place.
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
//            sequences its range touches.  Unit w's piece of sequence b goes
//            to partial slot w + b (unique: the pieces of unit w have
//            increasing b, and unit w+1 starts at or after unit w's last b).

// Exclusive prefix sums of the 32-token block counts into pfx[0..B];
// returns the total.  Called by all threads; B <= kMaxSchedB.
__device__ int block_prefix(const int32_t* __restrict__ seq_lens, int B, int* pfx) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int per = (B + nthreads - 1) / nthreads;  // <= 4
  const int base = tid * per;
  int loc[4];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = min(base + k, B - 1);
    const int L = seq_lens[i];  // loaded unconditionally so the loads overlap
    const int v = (k < per && base + k < B) ? (L + kBlock - 1) / kBlock : 0;
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

// Unit of the balanced split that owns block g (G units over P blocks).
__device__ __forceinline__ int unit_of_block(long long g, long long G, long long P) {
  return (int)(((g + 1) * G - 1) / P);
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
};

__device__ __forceinline__ Schedule schedule_begin(const DecodeArgs& a, const int* pfx, int P) {
  Schedule s{};
  s.w = blockIdx.x;
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
      s.g0 = (long long)s.w * s.P / s.G;
      s.g1 = (long long)(s.w + 1) * s.P / s.G;
      int lo = 0, hi = a.B;  // last b with pfx[b] <= g0
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pfx[mid] <= s.g0) lo = mid; else hi = mid;
      }
      s.b = uniform(lo);
    }
  }
  return s;
}

// Next piece of this unit's work; every thread of the workgroup gets the
// same answer.
__device__ __forceinline__ bool schedule_next(const DecodeArgs& a, const int* pfx, Schedule& s, Segment& seg) {
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
    const int p0 = uniform(pfx[b]), p1 = uniform(pfx[b + 1]);
    if (p0 >= s.g1) break;
    s.b = b + 1;
    const int k0 = (int)(max(s.g0, (long long)p0) - p0);
    const int k1 = (int)(min(s.g1, (long long)p1) - p0);
    if (k0 < k1) {
      const int L = a.seq_lens[b];
      const int first = unit_of_block(p0, s.G, s.P);
      const int last = unit_of_block(p1 - 1, s.G, s.P);
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
// A page is 64 rows of 1152 bytes, stored unpadded: row r at r * 1152.  The
// 16-byte chunks of a row are permuted inside each aligned group of eight:
// chunk c of row r sits at chunk position c ^ swz(r).  gfx950 serves a
// 16-byte LDS read per half-wave (even lanes, then odd lanes) over 128 banks
// of 4 bytes, and the transposing 8-byte read per quarter-wave; without the
// permutation the rows of an operand tile (1152 = 9 * 128) would pile onto a
// quarter of the banks.  With it, the score operand reads, the transposing
// value reads and the dequantising writes below are all conflict-free.
// Rows 2k and 2k+1 share swz, so a row pair (2304 contiguous bytes in HBM)
// is still moved by nine 256-byte LDS-DMA instructions: lane i fetches the
// 4 bytes that belong at pair offset (256 k + 4 i), i.e. HBM pair offset
// 256 k + ((4 i) ^ (swz << 4)).
constexpr int kBufBytes = kPageBytes;                  // one bf16 page
constexpr int kDmaBytes = 256;                         // 64 lanes x 4 bytes
constexpr int kPairBytes = 2 * kRowBytes;              // 2304
constexpr int kDmaPerPair = kPairBytes / kDmaBytes;    // 9
constexpr int kWaves = 8;                              // every decode workgroup has 8 waves
constexpr int kRowsPerWave = kPage / kWaves;           // 8
constexpr int kDmaPerWave = kRowsPerWave / 2 * kDmaPerPair;  // 36 (< 64 outstanding)
constexpr int kRsrcWord3 = 0x00020000;                 // raw untyped buffer access

__device__ __forceinline__ int swz(int r) { return 2 * ((r >> 2) & 3) + ((r >> 4) & 1); }
// LDS byte offset of byte x (x < 1152) of row r.
__device__ __forceinline__ int lds_off(int r, int x) { return r * kRowBytes + (x ^ (swz(r) << 4)); }

// Copy rows [lo, hi) of a bf16 page into an LDS buffer; wave w moves rows
// 8w .. 8w+7.  The buffer resource covers exactly the first `hi` rows, so
// rows at or past hi (past the sequence end, or owned by the next unit)
// arrive as zeros and stale or non-finite pool contents never reach the
// matrix cores.  Rows below lo (only ever 0 or 32) belong to the previous
// unit: waves whose rows all lie there issue nothing, and the compute skips
// those rows.
__device__ __forceinline__ void issue_page_bf16(const uint8_t* page, uint8_t* buf, int lo, int hi, int wave,
                                                int lane) {
  asm volatile("" : "+s"(wave));  // re-derived per copy, not kept live across the loop
  if (wave * kRowsPerWave + kRowsPerWave <= lo) return;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(page), (short)0,
                                                                      uniform(hi * kRowBytes), kRsrcWord3);
  const uint32_t lb = lds_addr(buf);
#pragma unroll
  for (int j = 0; j < kRowsPerWave / 2; ++j) {
    const int pair = wave * (kRowsPerWave / 2) + j;
    const uint32_t vo = (uint32_t)((lane * 4) ^ (swz(2 * pair) << 4));
#pragma unroll
    for (int k = 0; k < kDmaPerPair; ++k) {
      const int off = pair * kPairBytes + k * kDmaBytes;
      lds_dma4(rs, lb + off, vo, off);
    }
  }
}

// fp8 staging buffer of one page: codes [64][512], scales [64][4] fp32,
// rotated k^R [64][64] bf16.
constexpr int kStCkv = 0;
constexpr int kStScale = kPage * kDc;                  // 32768
constexpr int kStKr = kStScale + kPage * 4 * 4;        // 33792
constexpr int kStageBytes = kStKr + kPage * kDr * 2;   // 41984
constexpr int kFp8DmaPerWave = 16 + 1 + 4;             // codes, scales (half wave), k^R

__device__ __forceinline__ void issue_page_fp8(const uint8_t* ckv8, const float* scale8, const uint8_t* kr8,
                                               int page, uint8_t* stage, int lo, int hi, int wave, int lane) {
  asm volatile("" : "+s"(wave));
  if (wave * kRowsPerWave + kRowsPerWave <= lo) return;
  const size_t pg = (size_t)page;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(ckv8 + pg * (kPage * kDc)), (short)0, uniform(hi * kDc), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(scale8 + pg * (kPage * 4)), (short)0, uniform(hi * 16), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(kr8 + pg * (kPage * kDr * 2)), (short)0, uniform(hi * kDr * 2), kRsrcWord3);
  const uint32_t lb = lds_addr(stage);
  const uint32_t vo = lane * 4;
#pragma unroll
  for (int k = 0; k < 16; ++k) {  // codes: rows 8w .. 8w+7 are 4096 contiguous bytes
    const int off = wave * (kRowsPerWave * kDc) + k * kDmaBytes;
    lds_dma4(rc, lb + kStCkv + off, vo, off);
  }
  if (lane < 32) {  // scales: 8 rows x 16 bytes
    const int off = wave * (kRowsPerWave * 16);
    lds_dma4(rsc, lb + kStScale + off, vo, off);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // k^R: 8 rows x 128 bytes
    const int off = wave * (kRowsPerWave * kDr * 2) + k * kDmaBytes;
    lds_dma4(rk, lb + kStKr + off, vo, off);
  }
}

// Expand a staged fp8 page into the bf16 row layout.  Thread t: row t/8,
// channels 64(t%8) .. +63 (one 128-channel tile's half, one scale), plus one
// 16-byte chunk of the row's k^R.  Rows past the valid range are zeros in
// the staging buffer (codes and scales), so they expand to zeros.
__device__ __forceinline__ void dequant_page(const uint8_t* stage, uint8_t* buf) {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));  // offsets recomputed per page, not held across the loop
  const int r = t >> 3, sub = t & 7;
  const float sc = *(const float*)(stage + kStScale + (r * 4 + (sub >> 1)) * 4);
  const uint8_t* src = stage + kStCkv + r * kDc + sub * 64;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
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
      const int chunk = sub * 8 + 2 * j + h;  // 8 channels = one 16-byte chunk
      *(MLA_LDS bf16x8*)(buf + lds_off(r, chunk * 16)) = v;
    }
    asm volatile("" ::: "memory");  // one 16-code read in flight at a time
  }
  const int kc = t & 7;
  const int4v kr = lds_read_b128(stage + kStKr + r * (kDr * 2) + kc * 16);
  *(MLA_LDS int4v*)(buf + lds_off(r, kDc * 2 + kc * 16)) = kr;
}

// ---------------------------------------------------------------------------
// Matrix-core compute on one page buffer
// ---------------------------------------------------------------------------

// Per-wave state: 16 heads.  Lane l serves head h0 + l%16; its lane group
// g = l/16 picks which channels / tokens of each matrix-core operand it holds.
struct WaveState {
  bf16x8 q[18];      // absorbed query, B operand of S^T = R Q^T: channels 32kk + 8g + j
  floatx4 zacc[32];  // Z^T channel tile mt: channels 16mt + 4g + r, column = head
  float m, l;        // running max (log2 units) and this lane's partial sum
};

constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is refreshed

__device__ __forceinline__ void load_query(WaveState& st, const bf16* __restrict__ q, int H, int head, int g) {
  const int hc = head < H ? head : H - 1;
  const int keep = head < H ? -1 : 0;
  const int4v* src = (const int4v*)(q + (size_t)hc * kRow);
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    int4v v = src[4 * kk + g];
    v &= keep;
    st.q[kk] = __builtin_bit_cast(bf16x8, v);
  }
}

// Use the query registers, so the compiler's own wait for their loads is
// placed here and not at the first score product, where later page copies
// (which its counter does not see) would be waited for as well.
__device__ __forceinline__ void consume_query(WaveState& st) {
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) asm volatile("" : "+v"(st.q[kk]));
}

__device__ __forceinline__ void reset_state(WaveState& st) {
#pragma unroll
  for (int t = 0; t < 32; ++t) st.zacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Online softmax over NV scores per lane.  x: scaled (log2 units) scores,
// -inf where masked; p: probabilities relative to the running maximum.  The
// maximum is only moved when it grows by more than kLazyRescale, so the
// accumulator is rescaled rarely; p stays <= 2^kLazyRescale.
template <int NV>
__device__ __forceinline__ void softmax_update(WaveState& st, float (&x)[NV], float (&p)[NV]) {
  float mx = x[0];
#pragma unroll
  for (int r = 1; r < NV; ++r) mx = fmaxf(mx, x[r]);
  mx = pair32_max(pair16_max(mx));
  const float mnew = fmaxf(st.m, mx);
  const bool need = mnew > st.m + kLazyRescale;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
    const float alpha = need ? fast_exp2(st.m - mnew) : 1.0f;
    if (need) st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < 32; ++t) st.zacc[t] *= alpha;
  }
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < NV; ++r) {
    p[r] = fast_exp2(x[r] - st.m);
    sum += p[r];
  }
  st.l += sum;
}

// Score of one 16-token subtile (rows t0 .. t0+15, t0 a multiple of 16):
// S^T (16 tokens x 16 heads), K = 576 in 18 steps of 32 channels.  Row index
// m of the product maps to token t0 + 4(m%4) + m/4, so score register r of
// lane group g is token t0 + 4r + g.
__device__ __forceinline__ floatx4 score16(const WaveState& st, uint32_t buf, int t0, int lane) {
  const int g = lane >> 4, m = lane & 15;
  const int r = t0 + 4 * (m & 3) + (m >> 2);
  // byte 64kk + 16g of the row: the permutation only touches bits 4..6, so
  // even and odd kk each have one base and a constant stride of 128 bytes
  const uint32_t ap0 = buf + lds_off(r, 16 * g);
  const uint32_t ap1 = buf + lds_off(r, 64 + 16 * g);
  auto rd = [&](int kk) { return lds_read_b128_at((kk & 1 ? ap1 : ap0) + 128 * (kk >> 1)); };
  floatx4 S = {};
  constexpr int D = 3;  // operand reads in flight
  int4v a[D];
#pragma unroll
  for (int i = 0; i < D; ++i) a[i] = rd(i);
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    const int4v cur = a[kk % D];
    if (kk + D < 18) a[kk % D] = rd(kk + D);
    S = mfma16(__builtin_bit_cast(bf16x8, cur), st.q[kk], S);
  }
  return S;
}

// One tile of TT (16 or 32) tokens starting at row t0 of the page buffer;
// rows at or past `hi` are masked.  Value product Z^T += C^T P^T: A = C^T
// (16 channels x TT tokens) through transposing LDS reads, B = P^T.  For
// TT = 32 the K = 32 slots of lane group g are tokens t0 + 4j + g (j < 4,
// first subtile) and t0 + 16 + 4(j-4) + g.
template <int TT>
__device__ __forceinline__ void tile(WaveState& st, uint32_t buf, int t0, int hi, int lane, float scale_log2) {
  // Recompute the lane's operand offsets in every tile rather than let the
  // compiler keep one set per tile position and buffer live across the loop.
  asm volatile("" : "+v"(lane));
  constexpr int NS = TT / 16;
  const int g = lane >> 4;
  float x[4 * NS], p[4 * NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const floatx4 S = score16(st, buf, t0 + 16 * u, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = S[r] * scale_log2;
      x[4 * u + r] = t0 + 16 * u + 4 * r + g < hi ? v : -INFINITY;
    }
  }
  softmax_update<4 * NS>(st, x, p);
  // Source lane s' of each 16-lane group points at row t0 + 4(s'/4) + g,
  // channels 16mt + 4(s'%4) .. +3, i.e. row byte 32mt + 8(s'%4); as above,
  // the permutation leaves a base per mt%4 and a stride of 128 bytes.
  const int vr = t0 + g + 4 * ((lane & 15) >> 2);
  const int vx = 8 * (lane & 3);
  uint32_t vb[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) vb[q4] = buf + lds_off(vr, 32 * q4 + vx);
  constexpr int D = 3;
  if constexpr (TT == 32) {
    // rows + 16 differ only in bit 0 of swz, i.e. by 16 * 1152 +- 16 bytes
    const uint32_t dh = lds_off(vr + 16, vx) - lds_off(vr, vx);
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = f2bf(p[j]);
    auto vread = [&](int mt) {
      bf16x4 lo = lds_read_tr16_at(vb[mt & 3] + 128 * (mt >> 2));
      bf16x4 hi = lds_read_tr16_at(vb[mt & 3] + dh + 128 * (mt >> 2));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8 va[D];
#pragma unroll
    for (int i = 0; i < D; ++i) va[i] = vread(i);
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const bf16x8 cur = va[mt % D];
      if (mt + D < 32) va[mt % D] = vread(mt + D);
      st.zacc[mt] = mfma16(cur, pb, st.zacc[mt]);
    }
  } else {
    const bf16x4 pb = {f2bf(p[0]), f2bf(p[1]), f2bf(p[2]), f2bf(p[3])};
    auto vread = [&](int mt) { return lds_read_tr16_at(vb[mt & 3] + 128 * (mt >> 2)); };
    bf16x4 va[D];
#pragma unroll
    for (int i = 0; i < D; ++i) va[i] = vread(i);
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const bf16x4 cur = va[mt % D];
      if (mt + D < 32) va[mt % D] = vread(mt + D);
      st.zacc[mt] = mfma16k16(cur, pb, st.zacc[mt]);
    }
  }
}

// Normalise and write one wave's 16 heads: z rows [head][512], lse[head].
__device__ __forceinline__ void store_state(const WaveState& st, float l_tot, float* zdst, float* ldst, int h0, int H,
                                            int lane) {
  constexpr float kLn2 = 0.69314718055994530942f;
  const int head = h0 + (lane & 15);
  const int g = lane >> 4;
  if (head >= H) return;
  const float inv = 1.0f / l_tot;
  float* row = zdst + (size_t)head * kDc;
#pragma unroll
  for (int mt = 0; mt < 32; ++mt) {
    *(float4*)(row + 16 * mt + 4 * g) = make_float4(st.zacc[mt][0] * inv, st.zacc[mt][1] * inv,
                                                    st.zacc[mt][2] * inv, st.zacc[mt][3] * inv);
  }
  if (ldst != nullptr && g == 0) ldst[head] = (st.m + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// Merge of one sequence's partials (shared by the merge kernel and the
// in-kernel merge of the last-arriving unit)
// ---------------------------------------------------------------------------
// One wave per head: the chunks' log-sum-exps are read one per lane and
// reduced across the wave; then each lane folds its 8 channels of every
// chunk, 8 chunk loads in flight.
__device__ __forceinline__ void merge_head(const DecodeArgs& a, int b, int head, int slot0, int n, int lane) {
  // pass 1: maximum log-sum-exp over the chunks
  float mmax = -INFINITY;
  for (int c0 = 0; c0 < n; c0 += 64)
    if (c0 + lane < n) mmax = fmaxf(mmax, a.lsep[(size_t)(slot0 + c0 + lane) * a.H + head]);
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, d));
  // pass 2: weights (one chunk per lane) and the weighted sum of the chunks' z
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float wsum = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    float w = 0.f;
    if (c0 + lane < n) w = __expf(a.lsep[(size_t)(slot0 + c0 + lane) * a.H + head] - mmax);
    wsum += w;
    const int m = min(64, n - c0);
    for (int i0 = 0; i0 < m; i0 += 8) {
      float wv[8];
      float4 v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = min(i0 + u, m - 1);  // every slot loaded holds a partial of this sequence
        wv[u] = i0 + u < m ? __shfl(w, i) : 0.f;
        const size_t sl = (size_t)(slot0 + c0 + i) * a.H + head;
        const float4* zp = (const float4*)(a.zp + sl * kDc) + lane * 2;
        v0[u] = zp[0];
        v1[u] = zp[1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wi = wv[u];
        acc[0] += wi * v0[u].x; acc[1] += wi * v0[u].y; acc[2] += wi * v0[u].z; acc[3] += wi * v0[u].w;
        acc[4] += wi * v1[u].x; acc[5] += wi * v1[u].y; acc[6] += wi * v1[u].z; acc[7] += wi * v1[u].w;
      }
    }
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) wsum += __shfl_xor(wsum, d);
  const float inv = 1.0f / wsum;
  float4* zo = (float4*)(a.z + ((size_t)b * a.H + head) * kDc) + lane * 2;
  zo[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  zo[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (a.lse != nullptr && lane == 0) a.lse[(size_t)b * a.H + head] = mmax + __logf(wsum);
}

// After this workgroup stored its partial of `seg`: count the arrival and
// report whether this was the sequence's last piece (the counter is left at
// zero for the next call).  Called by all threads.
__device__ __forceinline__ bool arrive(const DecodeArgs& a, const Segment& seg, int expected, int* flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this thread's partial stores
  __syncthreads();
  if (threadIdx.x == 0) {
    // system scope: performed past every XCD's L2, so all units count on one copy
    const int old = __hip_atomic_fetch_add(a.counters + seg.b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int last = old == expected - 1;
    if (last) __hip_atomic_exchange(a.counters + seg.b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    *flag = last;
  }
  __syncthreads();
  const bool last = uniform(*flag) != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other pieces' stores
  return last;
}

// ---------------------------------------------------------------------------
// bf16 / fp8-cache matrix-core decode
// ---------------------------------------------------------------------------
//
// 8 waves: all of them copy pages; the first HG*TG compute.  HG head groups
// of 16 heads, TG token slices of each page.  FP8 selects the fp8 pool: two
// staging buffers (the next page's copy lands in one while the other is
// expanded) and one bf16 page buffer.
template <int HG, int TG, bool FP8>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mfma_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  static_assert(HG * TG <= kWaves, "too many compute waves");
  constexpr int TPW = kPage / TG;           // tokens of each page a wave scores
  constexpr int TT = TPW >= 32 ? 32 : 16;   // tokens per tile
  static_assert(TPW % TT == 0, "tile must divide the wave's slice");
  constexpr int kSmem = FP8 ? 2 * kStageBytes + kBufBytes : 2 * kBufBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  __shared__ int pfx[kMaxSchedB + 1];
  __shared__ int flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const bool computes = wave < HG * TG;
  const int hg = wave % HG, tg = wave / HG;
  const int h0 = hg * 16;
  const bool fused = a.counters != nullptr;

  int P = 0;
  if (a.splits == 0 && a.prefill_T == 0) P = block_prefix(a.seq_lens, a.B, pfx);
  Schedule sch = schedule_begin(a, pfx, P);
  Segment seg;
  if (!schedule_next(a, pfx, sch, seg)) return;

  // page buffers: bf16 -> smem + (i&1) * kBufBytes; fp8 -> stage (i&1), one bf16 buffer
  uint8_t* const bfbuf = FP8 ? smem + 2 * kStageBytes : smem;
  auto bt_row = [&](const Segment& s) {
    return a.prefill_T > 0 ? block_table : block_table + (size_t)s.b * a.max_pages;
  };
  auto qrow = [&](const Segment& s) { return (const bf16*)a.q + (size_t)s.b * a.H * kRow; };
  auto page_lo = [&](const Segment& s, int p) { return max(s.t0 - p * kPage, 0); };
  auto page_hi = [&](const Segment& s, int p) { return min(s.t1 - p * kPage, kPage); };
  // block-table reads use a uniform index, so they are scalar loads that do
  // not wait behind the page copies in flight
  auto issue = [&](const Segment& s, int p, int i) {
    const int page = bt_row(s)[uniform(p)];
    if constexpr (FP8) {
      issue_page_fp8(a.ckv8, a.scale8, a.kr8, page, smem + (i & 1) * kStageBytes, page_lo(s, p), page_hi(s, p),
                     wave, lane);
    } else {
      issue_page_bf16(a.rows + (size_t)page * kPageBytes, smem + (i & 1) * kBufBytes, page_lo(s, p), page_hi(s, p),
                      wave, lane);
    }
  };

  // Pieces of sequences whose merge falls to this unit: at most the first
  // and the last piece of a unit can be partial, so two at most.
  int pend_n = 0, pb0 = 0, ps0 = 0, pc0 = 0, pb1 = 0, ps1 = 0, pc1 = 0;

  // The query loads and the first page copy travel together; consuming the
  // query right after waits for both (the compiler's counter only knows the
  // query loads), before the second page's copy is issued.
  WaveState st;
  int p = seg.t0 / kPage;
  load_query(st, qrow(seg), a.H, h0 + (lane & 15), lane >> 4);
  issue(seg, p, 0);
  consume_query(st);
  reset_state(st);
  for (int i = 0;; ++i) {
    const bool seg_last = p == (seg.t1 - 1) / kPage;
    Segment nseg = seg;
    int np = p + 1;
    bool more = true;
    if (seg_last) {
      more = schedule_next(a, pfx, sch, nseg);
      np = nseg.t0 / kPage;
    }
    if (more) {
      issue(nseg, np, i + 1);
      if constexpr (FP8) wait_vmcnt<kFp8DmaPerWave>(); else wait_vmcnt<kDmaPerWave>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    uint8_t* buf;
    if constexpr (FP8) {
      dequant_page(smem + (i & 1) * kStageBytes, bfbuf);
      __syncthreads();
      buf = bfbuf;
    } else {
      buf = smem + (i & 1) * kBufBytes;
    }
    const uint32_t bufa = lds_addr(buf);
    const int lo = page_lo(seg, p), hi = page_hi(seg, p);
    if (computes) {
#pragma unroll
      for (int t = 0; t < TPW / TT; ++t) {
        const int t0 = tg * TPW + t * TT;
        if (t0 + TT > lo && t0 < hi) tile<TT>(st, bufa, t0, hi, lane, a.scale_log2);
      }
    }
    __syncthreads();  // the buffer is free: refilled next round, or merge scratch below

    if (seg_last) {
      // combine the token slices of the TG waves that share a head group: a
      // tree over LDS in the free page buffer, at most two slots per pass
      float l_tot = pair32_sum(pair16_sum(st.l));
      if constexpr (TG > 1) {
        uint8_t* scratch = buf;
        floatx4* zx = (floatx4*)scratch;                   // [2][32 tiles][64 lanes]
        float* ml = (float*)(scratch + 2 * 32 * 64 * 16);  // [2][2][64]
        static_assert(2 * 32 * 64 * 16 + 2 * 2 * 64 * 4 <= kBufBytes, "merge scratch");
        // Runtime loops on purpose: unrolled, the conditional accumulator
        // update would be duplicated per pass and cost register copies.
#pragma unroll 1
        for (int half = TG / 2; half >= 1; half /= 2) {
#pragma unroll 1
          for (int s0 = 0; s0 < half * HG; s0 += 2) {
            const int slw = (tg - half) * HG + hg - s0;  // slot this wave hands over
            if (computes && tg >= half && tg < 2 * half && slw >= 0 && slw < 2) {
              floatx4* dst = zx + (size_t)slw * 32 * 64;
#pragma unroll
              for (int t = 0; t < 32; ++t) dst[t * 64 + lane] = st.zacc[t];
              ml[(slw * 2) * 64 + lane] = st.m;
              ml[(slw * 2 + 1) * 64 + lane] = l_tot;
            }
            __syncthreads();
            const int slr = tg * HG + hg - s0;  // slot this wave takes over
            if (computes && tg < half && slr >= 0 && slr < 2) {
              const float mo = ml[(slr * 2) * 64 + lane];
              const float lo2 = ml[(slr * 2 + 1) * 64 + lane];
              const float mstar = fmaxf(st.m, mo);
              const float a0 = st.m == -INFINITY ? 0.f : fast_exp2(st.m - mstar);
              const float ao = mo == -INFINITY ? 0.f : fast_exp2(mo - mstar);
              l_tot = l_tot * a0 + lo2 * ao;
              const floatx4* src = zx + (size_t)slr * 32 * 64;
#pragma unroll
              for (int t = 0; t < 32; ++t) {
                st.zacc[t] = st.zacc[t] * a0 + src[t * 64 + lane] * ao;
                if (t % 8 == 7) asm volatile("" ::: "memory");  // 8 tiles' loads in flight, not 32
              }
              st.m = mstar;
            }
            __syncthreads();
          }
        }
      }
      const bool whole = seg.parts == 1;
      if (computes && tg == 0) {
        float* zdst;
        float* ldst;
        if (whole) {
          zdst = a.z + (size_t)seg.b * a.H * kDc;
          ldst = a.lse ? a.lse + (size_t)seg.b * a.H : nullptr;
        } else {
          zdst = a.zp + (size_t)seg.slot * a.H * kDc;
          ldst = a.lsep + (size_t)seg.slot * a.H;
        }
        store_state(st, l_tot, zdst, ldst, h0, a.H, lane);
      }
      if (!whole && fused && arrive(a, seg, seg.parts, &flag)) {
        if (pend_n == 0) {
          pb0 = seg.b, ps0 = seg.slot0, pc0 = seg.parts;
        } else {
          pb1 = seg.b, ps1 = seg.slot0, pc1 = seg.parts;
        }
        ++pend_n;
      }
      if (more) {
        load_query(st, qrow(nseg), a.H, h0 + (lane & 15), lane >> 4);
        consume_query(st);
        reset_state(st);
      }
      seg = nseg;
    }
    if (!more) break;
    p = np;
  }

  for (int k = 0; k < pend_n; ++k) {
    const int b = uniform(k ? pb1 : pb0), s0 = uniform(k ? ps1 : ps0), n = uniform(k ? pc1 : pc0);
    for (int h = wave; h < a.H; h += kWaves) merge_head(a, b, h, s0, n, lane);
  }
}

// ---------------------------------------------------------------------------
// fp32 decode (VALU; small and exact-arithmetic cases)
// ---------------------------------------------------------------------------
// One workgroup per (unit, head).  Tokens are scored 256 at a time (one per
// thread), then every thread folds them into its two channels of z.  Partials
// are always merged by the merge kernel.
__global__ void __launch_bounds__(256) decode_f32_kernel(DecodeArgs a) {
  __shared__ float qs[kRow];
  __shared__ float ps[256];
  __shared__ float red[8];
  __shared__ int pfx[kMaxSchedB + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  int P = 0;
  if (a.splits == 0 && a.prefill_T == 0) P = block_prefix(a.seq_lens, a.B, pfx);
  Schedule sch = schedule_begin(a, pfx, P);
  Segment seg;
  while (schedule_next(a, pfx, sch, seg)) {
    const int32_t* bt = a.prefill_T > 0 ? a.block_table : a.block_table + (size_t)seg.b * a.max_pages;
    const float* q = (const float*)a.q + ((size_t)seg.b * a.H + head) * kRow;
    const float* pool = (const float*)a.rows;
    __syncthreads();
    for (int i = tid; i < kRow; i += 256) qs[i] = q[i];
    __syncthreads();
    float m = -INFINITY, l = 0.f, z0 = 0.f, z1 = 0.f;
    const int j0 = seg.t0, j1 = seg.t1;
    for (int jb = j0; jb < j1; jb += 256) {
      const int j = jb + tid;
      float s = -INFINITY;
      if (j < j1) {
        const float* row = pool + ((size_t)bt[j / kPage] * kPage + (j % kPage)) * kRow;
        float acc = 0.f;
        for (int k = 0; k < kRow; ++k) acc = fmaf(qs[k], row[k], acc);
        s = acc * a.scale_log2;
      }
      // block max
      float v = s;
      for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
      if (lane == 0) red[wave] = v;
      __syncthreads();
      const float bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      const float mnew = fmaxf(m, bm);
      const float alpha = exp2f(m - mnew);
      const float pj = exp2f(s - mnew);
      ps[tid] = pj;
      float ssum = pj;
      for (int d = 32; d > 0; d >>= 1) ssum += __shfl_xor(ssum, d);
      __syncthreads();
      if (lane == 0) red[4 + wave] = ssum;
      __syncthreads();
      l = l * alpha + (red[4] + red[5] + red[6] + red[7]);
      z0 *= alpha;
      z1 *= alpha;
      m = mnew;
      const int n = min(256, j1 - jb);
      for (int t = 0; t < n; ++t) {
        const int jj = jb + t;
        const float* row = pool + ((size_t)bt[jj / kPage] * kPage + (jj % kPage)) * kRow;
        z0 = fmaf(ps[t], row[tid], z0);
        z1 = fmaf(ps[t], row[tid + 256], z1);
      }
      __syncthreads();
    }
    float* zdst;
    float* ldst;
    if (seg.parts == 1) {
      zdst = a.z + ((size_t)seg.b * a.H + head) * kDc;
      ldst = a.lse ? a.lse + (size_t)seg.b * a.H + head : nullptr;
    } else {
      zdst = a.zp + ((size_t)seg.slot * a.H + head) * kDc;
      ldst = a.lsep + (size_t)seg.slot * a.H + head;
    }
    zdst[tid] = z0 / l;
    zdst[tid + 256] = z1 / l;
    if (ldst != nullptr && tid == 0) *ldst = (m + log2f(l)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// Split merge kernel: one workgroup per (sequence, 8 heads), one wave per head
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512) merge_kernel(DecodeArgs a) {
  __shared__ int pfx[kMaxSchedB + 1];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.y * 8 + wave;
  int slot0, n;
  if (a.splits > 0) {
    const int S = a.splits;
    const int np = (a.seq_lens[b] + kPage - 1) / kPage;
    const int chunk = (np + S - 1) / S;
    n = (np + chunk - 1) / chunk;
    slot0 = b * S;
  } else {
    const int P = block_prefix(a.seq_lens, a.B, pfx);
    const long long G = min((long long)a.units, (long long)P);
    const int first = unit_of_block(pfx[b], G, P);
    const int last = unit_of_block(pfx[b + 1] - 1, G, P);
    n = last - first + 1;
    slot0 = first + b;
  }
  if (n <= 1 || head >= a.H) return;
  merge_head(a, b, head, slot0, n, lane);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <bool FP8>
static void launch_mfma(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.units), blk(kWaves * 64);
  if (a.H <= 16) {
    hipLaunchKernelGGL((decode_mfma_kernel<1, 4, FP8>), grid, blk, 0, s, a, a.block_table);
  } else if (a.H <= 32) {
    hipLaunchKernelGGL((decode_mfma_kernel<2, 4, FP8>), grid, blk, 0, s, a, a.block_table);
  } else if (a.H <= 64) {
    hipLaunchKernelGGL((decode_mfma_kernel<4, 2, FP8>), grid, blk, 0, s, a, a.block_table);
  } else {
    hipLaunchKernelGGL((decode_mfma_kernel<8, 1, FP8>), grid, blk, 0, s, a, a.block_table);
  }
}

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t s) {
  if (kind == kKindF32) {
    hipLaunchKernelGGL(decode_f32_kernel, dim3(a.units, a.H), dim3(256), 0, s, a);
  } else if (kind == kKindFp8) {
    launch_mfma<true>(a, s);
  } else {
    launch_mfma<false>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.B, (a.H + 7) / 8), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
