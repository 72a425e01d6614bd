// Absorbed-MLA decode over the paged latent cache, and the split-KV merge.
//
// Per query token and head i (the "DeepSeek-V3" notes, ekkoxiao.github.io):
//   s_j = (q~_i . c_j + q^R_i . k^R_j) * scale     (§注意力计算 + §潜在向量的作用)
//   a_j = softmax_j(s),  z_i = sum_j a_j c_j        (§潜在向量的作用)
// All heads of a sequence read the same cached rows, so for a 64-token page
// the scores of the wave's heads are one dense product S^T = R Q^T
// (R: 64 x 576 rows, Q: heads x 576), and the latent accumulation is a second
// one, Z^T += C^T P^T (C: the 512-wide c^KV part of the rows).  Both run on
// bf16 matrix cores with fp32 accumulation.
//
// Work decomposition (one 256-thread workgroup per chunk of pages):
//   * The page's 64 rows (72 KB bf16) are copied HBM -> LDS with
//     asynchronous 16-byte LDS-DMA loads into one of two buffers while the
//     other buffer is being consumed, so every row is read from HBM once and
//     shared by all heads.
//   * Wave w owns HPW heads (hg = w % HG) and a token slice of each page
//     (tg = w / HG).  Its absorbed query stays in VGPRs for the whole chunk,
//     its accumulator Z^T (HPW x 512 fp32) in accumulation registers, and
//     every value a lane holds belongs to one head, so the online softmax
//     rescale never leaves the lane.
//   * Score operand: 16-byte LDS reads of rows.  Value operand: gfx950's
//     transposing LDS read (ds_read_b64_tr_b16) turns row-major c^KV into
//     token-packed matrix-core operands without a transposed copy.
//   * Row pairs are padded in LDS so the operand reads of consecutive rows,
//     and of the rows the transposing reads fetch together, hit distinct banks.
//   * Long sequences are cut into chunks; each chunk leaves a normalised
//     partial (z_c, lse_c) that the merge kernel combines exactly:
//     lse = log sum_c e^{lse_c}, z = sum_c e^{lse_c - lse} z_c.
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kRowBytes = kRow * 2;                 // 1152
constexpr int kPageBytes = kPage * kRowBytes;       // 73728

// ---------------------------------------------------------------------------
// Chunk schedule shared by the decode and merge kernels.
// ---------------------------------------------------------------------------

// Exclusive prefix sums of pages per sequence into pfx[0..B] and the
// lengths into lens[0..B); returns the total page count.  Called by all
// threads of the workgroup; B <= kMaxSchedB.
__device__ int block_page_prefix(const int32_t* __restrict__ seq_lens, int B, int* pfx, int* lens) {
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
    const int v = (k < per && base + k < B) ? (L + kPage - 1) / kPage : 0;
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
  return pfx[B];
}

// Unit that owns global page g in the balanced split of `total` pages over G units.
__device__ __forceinline__ int unit_of_page(long long g, long long G, long long total) {
  return (int)(((g + 1) * G - 1) / total);
}

struct Segment {
  int b, pb, pe, slot, whole;
};

// Walks the segments (sequence, page range) of this workgroup's unit in order.
// Every thread of the workgroup sees the same sequence of segments.
struct SegmentIter {
  int mode;             // 0 prefill, 1 uniform splits, 2 balanced
  int b, b_end;         // balanced: next sequence to look at
  long long g0, g1;     // balanced: global page range of this unit
  int done;
};

__device__ __forceinline__ SegmentIter segments_begin(const DecodeArgs& a, const int* pfx, int total) {
  SegmentIter it{};
  const int w = blockIdx.x;
  if (a.prefill_T > 0) {
    it.mode = 0;
  } else if (a.splits > 0) {
    it.mode = 1;
  } else {
    it.mode = 2;
    const long long G = a.units;
    it.g0 = (long long)w * total / G;
    it.g1 = (long long)(w + 1) * total / G;
    int lo = 0, hi = a.B;  // last b with pfx[b] <= g0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pfx[mid] <= it.g0) lo = mid; else hi = mid;
    }
    it.b = lo;
    it.done = it.g0 >= it.g1;
  }
  return it;
}

__device__ __forceinline__ bool segments_next(const DecodeArgs& a, const int* pfx, SegmentIter& it, Segment& seg) {
  if (it.done) return false;
  const int w = blockIdx.x;
  if (it.mode == 0) {  // one query row per unit, longest rows first
    it.done = 1;
    const int t = a.prefill_T - 1 - w;
    const int L = a.prefill_pos0 + t + 1;
    seg = Segment{t, 0, (L + kPage - 1) / kPage, 0, 1};
    return true;
  }
  if (it.mode == 1) {
    it.done = 1;
    const int S = a.splits;
    const int b = w / S, s = w % S;
    const int np = (a.seq_lens[b] + kPage - 1) / kPage;
    const int chunk = (np + S - 1) / S;
    const int pb = s * chunk, pe = min(pb + chunk, np);
    seg = Segment{b, pb, pe, w, (pb == 0 && pe == np) ? 1 : 0};
    return pb < pe;
  }
  while (it.b < a.B && pfx[it.b] < it.g1) {
    const int b = it.b++;
    const int np = pfx[b + 1] - pfx[b];
    const int pb = (int)(max(it.g0, (long long)pfx[b]) - pfx[b]);
    const int pe = (int)(min(it.g1, (long long)pfx[b + 1]) - pfx[b]);
    if (pb < pe) {
      seg = Segment{b, pb, pe, w + b, (pb == 0 && pe == np) ? 1 : 0};
      return true;
    }
  }
  it.done = 1;
  return false;
}

// ---------------------------------------------------------------------------
// bf16 matrix-core decode
// ---------------------------------------------------------------------------
//
// LDS page layout.  A page is 64 rows of 1152 bytes.  Rows are kept in
// pairs: rows 2k and 2k+1 are 2304 contiguous bytes in HBM and land in LDS at
// k * kGroupStride, copied by nine 256-byte LDS-DMA instructions (4 bytes per
// lane, fully coalesced).  The 16 extra bytes per pair put 16 consecutive rows
// on 16 distinct 16-byte bank slots (row 2k+1 sits 128 bytes after row 2k
// mod 256), and rows i, i+4, i+8, i+12 on one contiguous 128-byte span, which
// is what the value-operand transposing reads below fetch together.
constexpr int kGroupBytes = 2 * kRowBytes;             // 2304
constexpr int kGroupStride = kGroupBytes + 16;         // 2320
constexpr int kBufBytes = (kPage / 2) * kGroupStride;  // 74240
constexpr int kDmaBytes = 256;                         // 64 lanes x 4 bytes
constexpr int kDmaPerGroup = kGroupBytes / kDmaBytes;  // 9
constexpr int kWaves = 8;                              // every decode workgroup has 8 waves
constexpr int kDmaPerWave = (kPage / 2) / kWaves * kDmaPerGroup;  // 36 (< 64 outstanding)
constexpr int kRsrcWord3 = 0x00020000;                 // raw untyped buffer access

__device__ __forceinline__ int lds_row(int t) { return (t >> 1) * kGroupStride + (t & 1) * kRowBytes; }

// Copy one cache page into an LDS buffer: wave w moves row pairs 4w .. 4w+3.
// The buffer resource covers exactly the `valid` rows of the page: the copy
// cannot leave them, and rows past the end of the sequence arrive as zeros,
// so stale or non-finite pool contents never reach the matrix cores.
__device__ __forceinline__ void issue_page_copy(const uint8_t* page, uint8_t* buf, int valid, int wave, int lane) {
  // Re-derive the wave's offsets at every copy instead of keeping dozens of
  // loop-invariant scalars alive across the page loop.
  asm volatile("" : "+s"(wave));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(page), (short)0,
                                                                      uniform(valid * kRowBytes), kRsrcWord3);
  const uint32_t vo = lane * 4;
  const uint32_t lb = lds_addr(buf);
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int grp = wave * (kDmaPerWave / kDmaPerGroup) + i / kDmaPerGroup, part = i % kDmaPerGroup;
    lds_dma4(rs, lb + grp * kGroupStride + part * kDmaBytes, vo, grp * kGroupBytes + part * kDmaBytes);
  }
}

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

// Score of one 16-token subtile (rows t0 .. t0+15): S^T (16 tokens x 16 heads),
// K = 576 in 18 steps of 32 channels.  Row index m of the product maps to
// token t0 + 4(m%4) + m/4, so score register r of lane group g is token
// t0 + 4r + g.
__device__ __forceinline__ floatx4 score16(const WaveState& st, const uint8_t* buf, int t0, int lane) {
  const int g = lane >> 4, m = lane & 15;
  const uint8_t* ap = buf + lds_row(t0 + 4 * (m & 3) + (m >> 2)) + g * 16;
  floatx4 S = {};
  constexpr int D = 3;  // operand reads in flight
  int4v a[D];
#pragma unroll
  for (int i = 0; i < D; ++i) a[i] = lds_read_b128(ap + 64 * i);
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    const int4v cur = a[kk % D];
    if (kk + D < 18) a[kk % D] = lds_read_b128(ap + 64 * (kk + D));
    S = mfma16(__builtin_bit_cast(bf16x8, cur), st.q[kk], S);
  }
  return S;
}

// One tile of TT (16 or 32) tokens starting at row t0 of the page buffer.
// Value product Z^T += C^T P^T: A = C^T (16 channels x TT tokens) through
// transposing LDS reads, B = P^T.  For TT = 32 the K = 32 slots of lane group
// g are tokens t0 + 4j + g (j < 4, subtile 0) and t0 + 16 + 4(j-4) + g.
template <int TT>
__device__ __forceinline__ void tile(WaveState& st, const uint8_t* buf, int t0, int valid, int lane,
                                     float scale_log2) {
  constexpr int NS = TT / 16;
  const int g = lane >> 4;
  float x[4 * NS], p[4 * NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const floatx4 S = score16(st, buf, t0 + 16 * u, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = S[r] * scale_log2;
      x[4 * u + r] = t0 + 16 * u + 4 * r + g < valid ? v : -INFINITY;
    }
  }
  softmax_update<4 * NS>(st, x, p);
  // source lane s' of each 16-lane group points at row t0 + 16u + 4(s'/4) + g,
  // channels 16mt + 4(s'%4) .. +3
  const uint8_t* vp = buf + lds_row(t0 + g + 4 * ((lane & 15) >> 2)) + 8 * (lane & 3);
  constexpr int D = 3;
  if constexpr (TT == 32) {
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = f2bf(p[j]);
    auto vread = [&](int mt) {
      bf16x4 lo = lds_read_tr16(vp + mt * 32);
      bf16x4 hi = lds_read_tr16(vp + 8 * kGroupStride + mt * 32);  // rows + 16
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
    auto vread = [&](int mt) { return lds_read_tr16(vp + mt * 32); };
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

// 8 waves: all of them copy pages; the first HG*TG compute.  HG head groups
// of 16 heads, TG token slices of each page.
template <int HG, int TG>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_bf16_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  static_assert(HG * TG <= kWaves, "too many compute waves");
  constexpr int TPW = kPage / TG;           // tokens of each page a wave scores
  constexpr int TT = TPW >= 32 ? 32 : 16;   // tokens per tile
  static_assert(TPW % TT == 0, "tile must divide the wave's slice");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kBufBytes];
  __shared__ int pfx[kMaxSchedB + 1];
  __shared__ int lens[kMaxSchedB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const bool computes = wave < HG * TG;
  const int hg = wave % HG, tg = wave / HG;
  const int h0 = hg * 16;

  int total = 0;
  if (a.splits == 0 && a.prefill_T == 0) total = block_page_prefix(a.seq_lens, a.B, pfx, lens);

  SegmentIter it = segments_begin(a, pfx, total);
  Segment seg;
  while (segments_next(a, pfx, it, seg)) {
    seg.b = uniform(seg.b);
    seg.pb = uniform(seg.pb);
    seg.pe = uniform(seg.pe);
    seg.slot = uniform(seg.slot);
    seg.whole = uniform(seg.whole);
    const int L = uniform(a.prefill_T > 0 ? a.prefill_pos0 + seg.b + 1
                                          : (a.splits == 0 ? lens[seg.b] : a.seq_lens[seg.b]));
    const int32_t* bt = a.prefill_T > 0 ? block_table : block_table + (size_t)seg.b * a.max_pages;
    const bf16* qrow = (const bf16*)a.q + (size_t)seg.b * a.H * kRow;

    const int npg = seg.pe - seg.pb;
    // block-table reads use a uniform index, so they are scalar loads that do
    // not wait behind the page copies in flight
    auto page_ptr = [&](int pi) { return a.rows + (size_t)bt[uniform(pi)] * kPageBytes; };
    auto page_valid = [&](int pi) { return min(kPage, L - pi * kPage); };

    // The query loads and the first page copy travel together; consuming the
    // query right after waits for both (the compiler's counter only knows the
    // query loads), before the second page's copy is issued.
    WaveState st;
    load_query(st, qrow, a.H, h0 + (lane & 15), lane >> 4);
    issue_page_copy(page_ptr(seg.pb), smem, page_valid(seg.pb), wave, lane);
    consume_query(st);
#pragma unroll
    for (int t = 0; t < 32; ++t) st.zacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
    for (int i = 0; i < npg; ++i) {
      const int pi = seg.pb + i;
      const uint8_t* buf = smem + (i & 1) * kBufBytes;
      if (i + 1 < npg) {
        issue_page_copy(page_ptr(pi + 1), smem + ((i + 1) & 1) * kBufBytes, page_valid(pi + 1), wave, lane);
        wait_vmcnt<kDmaPerWave>();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();
      const int valid = page_valid(pi);
      if (computes) {
#pragma unroll
        for (int t = 0; t < TPW / TT; ++t) {
          const int t0 = tg * TPW + t * TT;
          if (t0 < valid) tile<TT>(st, buf, t0, valid, lane, a.scale_log2);
        }
      }
      __syncthreads();
    }

    // combine the token slices of the TG waves that share a head group:
    // a tree over LDS, half of the remaining slices handing over per round
    float l_tot = pair32_sum(pair16_sum(st.l));
    if constexpr (TG > 1) {
      // slot (tg - half, hg) carries slice tg over to slice tg - half
      floatx4* zx = (floatx4*)smem;  // [(TG/2) * HG][32 tiles][64 lanes]
      float* ml = (float*)(smem + 2 * kBufBytes) - 2 * (TG / 2) * HG * 64;
      static_assert((TG / 2) * HG * 32 * 64 * 16 + 2 * (TG / 2) * HG * 64 * 4 <= 2 * kBufBytes, "merge space");
#pragma unroll
      for (int half = TG / 2; half >= 1; half /= 2) {
        if (computes && tg >= half && tg < 2 * half) {
          const int slot = (tg - half) * HG + hg;
          floatx4* dst = zx + (size_t)slot * 32 * 64;
#pragma unroll
          for (int t = 0; t < 32; ++t) dst[t * 64 + lane] = st.zacc[t];
          ml[(slot * 2) * 64 + lane] = st.m;
          ml[(slot * 2 + 1) * 64 + lane] = l_tot;
        }
        __syncthreads();
        if (computes && tg < half) {
          const int slot = tg * HG + hg;
          const float mo = ml[(slot * 2) * 64 + lane];
          const float lo = ml[(slot * 2 + 1) * 64 + lane];
          const float mstar = fmaxf(st.m, mo);
          const float a0 = st.m == -INFINITY ? 0.f : fast_exp2(st.m - mstar);
          const float ao = mo == -INFINITY ? 0.f : fast_exp2(mo - mstar);
          l_tot = l_tot * a0 + lo * ao;
          const floatx4* src = zx + (size_t)slot * 32 * 64;
#pragma unroll
          for (int t = 0; t < 32; ++t) st.zacc[t] = st.zacc[t] * a0 + src[t * 64 + lane] * ao;
          st.m = mstar;
        }
        __syncthreads();
      }
    }
    if (computes && tg == 0) {
      float* zdst;
      float* ldst;
      if (seg.whole) {
        zdst = a.z + (size_t)seg.b * a.H * kDc;
        ldst = a.lse ? a.lse + (size_t)seg.b * a.H : nullptr;
      } else {
        zdst = a.zp + (size_t)seg.slot * a.H * kDc;
        ldst = a.lsep + (size_t)seg.slot * a.H;
      }
      store_state(st, l_tot, zdst, ldst, h0, a.H, lane);
    }
    __syncthreads();  // LDS is reused by the next segment
  }
}

// ---------------------------------------------------------------------------
// fp32 decode (VALU; small and exact-arithmetic cases)
// ---------------------------------------------------------------------------
// One workgroup per (unit, head).  Tokens are scored 256 at a time (one per
// thread), then every thread folds them into its two channels of z.
__global__ void __launch_bounds__(256) decode_f32_kernel(DecodeArgs a) {
  __shared__ float qs[kRow];
  __shared__ float ps[256];
  __shared__ float red[8];
  __shared__ int pfx[kMaxSchedB + 1];
  __shared__ int lens[kMaxSchedB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  int total = 0;
  if (a.splits == 0 && a.prefill_T == 0) total = block_page_prefix(a.seq_lens, a.B, pfx, lens);
  SegmentIter it = segments_begin(a, pfx, total);
  Segment seg;
  while (segments_next(a, pfx, it, seg)) {
    const int L = a.prefill_T > 0 ? a.prefill_pos0 + seg.b + 1 : a.seq_lens[seg.b];
    const int32_t* bt = a.prefill_T > 0 ? a.block_table : a.block_table + (size_t)seg.b * a.max_pages;
    const float* q = (const float*)a.q + ((size_t)seg.b * a.H + head) * kRow;
    const float* pool = (const float*)a.rows;
    __syncthreads();
    for (int i = tid; i < kRow; i += 256) qs[i] = q[i];
    __syncthreads();
    float m = -INFINITY, l = 0.f, z0 = 0.f, z1 = 0.f;
    const int j0 = seg.pb * kPage, j1 = min(seg.pe * kPage, L);
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
    if (seg.whole) {
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
// Split merge: lse = log sum_c e^{lse_c};  z = sum_c e^{lse_c - lse} z_c
// ---------------------------------------------------------------------------
// One workgroup per (sequence, 4 heads); one wave per head.  The chunks'
// log-sum-exps are read one per lane and reduced across the wave; then each
// lane folds its 8 channels of every chunk, several chunk loads in flight.
__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs a) {
  __shared__ int pfx[kMaxSchedB + 1];
  __shared__ int lens[kMaxSchedB];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.y * 4 + wave;
  int first = 0, last = 0, slot0 = 0;
  long long G = 0, total = 0;  // balanced split: units with no pages wrote no partial
  const int np = (a.seq_lens[b] + kPage - 1) / kPage;
  if (a.splits > 0) {
    const int S = a.splits;
    const int chunk = (np + S - 1) / S;
    const int used = (np + chunk - 1) / chunk;
    if (used <= 1) return;
    first = 0;
    last = used - 1;
    slot0 = b * S;
  } else {
    total = block_page_prefix(a.seq_lens, a.B, pfx, lens);
    G = a.units;
    first = unit_of_page(pfx[b], G, total);
    last = unit_of_page(pfx[b + 1] - 1, G, total);
    if (first == last) return;
    slot0 = b;  // slot of unit w for sequence b is w + b
  }
  if (head >= a.H) return;
  const int n = last - first + 1;
  auto owns_pages = [&](int c) { return G == 0 || c * total / G < (c + 1) * total / G; };
  // pass 1: maximum log-sum-exp over the chunks
  float mmax = -INFINITY;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int c = first + c0 + lane;
    if (c0 + lane < n && owns_pages(c)) mmax = fmaxf(mmax, a.lsep[(size_t)(slot0 + c) * a.H + head]);
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, d));
  // pass 2: weights (one chunk per lane) and the weighted sum of the chunks' z
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float wsum = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int c = first + c0 + lane;
    float w = 0.f;
    if (c0 + lane < n && owns_pages(c)) w = __expf(a.lsep[(size_t)(slot0 + c) * a.H + head] - mmax);
    wsum += w;
    const int m = min(64, n - c0);
    // Chunks go in batches of 8 whose loads are all in flight together.
    // Every slot loaded lies inside the workspace; slots of units without
    // pages hold no partial and are dropped by the select, not by a multiply.
    for (int i0 = 0; i0 < m; i0 += 8) {
      float wv[8];
      float4 v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = min(i0 + u, m - 1);
        wv[u] = i0 + u < m ? __shfl(w, i) : 0.f;
        const size_t sl = (size_t)(slot0 + first + c0 + i) * a.H + head;
        const float4* zp = (const float4*)(a.zp + sl * kDc) + lane * 2;
        v0[u] = zp[0];
        v1[u] = zp[1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wi = wv[u];
        const bool use = wi != 0.f;
        acc[0] += use ? wi * v0[u].x : 0.f; acc[1] += use ? wi * v0[u].y : 0.f;
        acc[2] += use ? wi * v0[u].z : 0.f; acc[3] += use ? wi * v0[u].w : 0.f;
        acc[4] += use ? wi * v1[u].x : 0.f; acc[5] += use ? wi * v1[u].y : 0.f;
        acc[6] += use ? wi * v1[u].z : 0.f; acc[7] += use ? wi * v1[u].w : 0.f;
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t s) {
  const dim3 blk(256);
  if (kind == kKindF32) {
    hipLaunchKernelGGL(decode_f32_kernel, dim3(a.units, a.H), blk, 0, s, a);
  } else if (a.H <= 16) {
    hipLaunchKernelGGL((decode_bf16_kernel<1, 4>), dim3(a.units), dim3(kWaves * 64), 0, s, a, a.block_table);
  } else if (a.H <= 32) {
    hipLaunchKernelGGL((decode_bf16_kernel<2, 4>), dim3(a.units), dim3(kWaves * 64), 0, s, a, a.block_table);
  } else if (a.H <= 64) {
    hipLaunchKernelGGL((decode_bf16_kernel<4, 2>), dim3(a.units), dim3(kWaves * 64), 0, s, a, a.block_table);
  } else {
    hipLaunchKernelGGL((decode_bf16_kernel<8, 1>), dim3(a.units), dim3(kWaves * 64), 0, s, a, a.block_table);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.B, (a.H + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
