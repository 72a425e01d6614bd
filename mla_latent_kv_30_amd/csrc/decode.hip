// Absorbed-MLA decode over the paged latent cache (the split-KV merge of its
// partials is in merge.hip).
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
//   * Wave w owns 16 heads (hg = w % HG) and a slice of the 512 latent
//     channels (cg = w / HG).  Its absorbed query and its accumulator Z^T
//     stay in registers, and every value a lane holds belongs to one head, so
//     the online softmax never leaves the lane.  With a single head group the
//     four computing waves would all compute the same scores; they split the
//     score product instead (a 16-token subtile times half of the 576
//     channels each) and add the partial products exchanged through LDS.
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
//     partial (z_c, lse_c) that the merge kernel combines exactly:
//     lse = log sum_c e^{lse_c}, z = sum_c e^{lse_c - lse} z_c.
#include <type_traits>

#include "decode_common.h"

namespace mla {

// ---------------------------------------------------------------------------
// Matrix-core compute on one block buffer
// ---------------------------------------------------------------------------

// Per-wave state: 16 heads and NT tiles of 16 latent channels.  Lane l serves
// head h0 + l%16; its lane group g = l/16 picks which channels / tokens of
// each matrix-core operand it holds.
template <int NT, int NQ = 18>
struct WaveState {
  bf16x8 q[NQ];      // absorbed query, B operand of S^T = R Q^T: channels 32(k0 + kk) + 8g + j
  floatx4 zacc[NT];  // Z^T tile j: channels c0 + 16j + 4g + r, column = head
  float m, l;        // running max (log2 units) and this lane's partial sum
};

template <int NT, int NQ>
__device__ __forceinline__ void reset_state(WaveState<NT, NQ>& st) {
#pragma unroll
  for (int t = 0; t < NT; ++t) st.zacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Online softmax over NV scores per lane.  x: scaled (log2 units) scores,
// -inf where masked; p: probabilities relative to the running maximum.  The
// maximum is only moved when it grows by more than kLazyRescale, so the
// accumulator is rescaled rarely; p stays <= 2^kLazyRescale.
template <int NT, int NQ, int NV>
__device__ __forceinline__ void softmax_update(WaveState<NT, NQ>& st, float (&x)[NV], float (&p)[NV]) {
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
    for (int t = 0; t < NT; ++t) st.zacc[t] *= alpha;
  }
  // a head that has seen only masked scores so far keeps m = -inf: its
  // probabilities are 0 (exp2(-inf - 0)), not exp2(-inf + inf)
  const float mref = st.m == -INFINITY ? 0.f : st.m;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < NV; ++r) {
    p[r] = fast_exp2(x[r] - mref);
    sum += p[r];
  }
  st.l += sum;
}

// Scores of the 32 rows of a block buffer as two 16-token subtiles, S^T
// (16 tokens x 16 heads) each, K = 576 in 18 steps of 32 channels; the two
// accumulation chains are interleaved so that back-to-back matrix-core ops
// never wait on each other.  Row index m of a subtile's product maps to
// token 16u + 4(m%4) + m/4, so score register r of lane group g in subtile u
// is token 16u + 4r + g.
// dma(t) is called after K-steps 2, 5, 8, 11, 14 and 17 (t = 0..5): it issues
// the wave's t-th copy of a later block, if there is one.
template <int D, class Dma>  // operand reads in flight per chain
__device__ __forceinline__ void score32(const bf16x8 (&q)[18], uint32_t buf, int lane, floatx4& S0, floatx4& S1,
                                        Dma&& dma) {
  const int g = lane >> 4, m = lane & 15;
  const int r = 4 * (m & 3) + (m >> 2);
  // byte 64kk + 16g of the row: the permutation only touches bits 4..6, so
  // even and odd kk each have one base per subtile and a constant stride of
  // 128 bytes
  uint32_t ap[2][2];  // [subtile][kk parity]
  ap[0][0] = buf + lds_off(r, 16 * g);
  ap[0][1] = buf + lds_off(r, 64 + 16 * g);
  ap[1][0] = buf + lds_off(r + 16, 16 * g);
  ap[1][1] = buf + lds_off(r + 16, 64 + 16 * g);
  // opaque bases: every read is then one base register plus an immediate offset
  asm volatile("" : "+v"(ap[0][0]), "+v"(ap[0][1]), "+v"(ap[1][0]), "+v"(ap[1][1]));
  auto rd = [&](int u, int kk) { return lds_read_b128_at(ap[u][kk & 1] + 128 * (kk >> 1)); };
  S0 = floatx4{};
  S1 = floatx4{};
  int4v a0[D], a1[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    a0[i] = rd(0, i);
    a1[i] = rd(1, i);
  }
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    const int4v c0 = a0[kk % D], c1 = a1[kk % D];
    if (kk + D < 18) {
      a0[kk % D] = rd(0, kk + D);
      a1[kk % D] = rd(1, kk + D);
    }
    S0 = mfma16(__builtin_bit_cast(bf16x8, c0), q[kk], S0);
    S1 = mfma16(__builtin_bit_cast(bf16x8, c1), q[kk], S1);
    if (kk % 3 == 2) dma(kk / 3);
  }
}

// One 16-token subtile u of a block buffer over the nine K-steps k0 .. k0+8
// (k0 = 0 or 9): the partial product S^T of those 288 channels, in the
// register layout of score32.  dma(t) is called after steps 1, 3, 5, 7 and 8.
template <int D, class Dma>
__device__ __forceinline__ floatx4 score_half(const bf16x8 (&q)[9], uint32_t buf, int lane, int u, int k0,
                                              Dma&& dma) {
  const int g = lane >> 4, m = lane & 15;
  const int r = 4 * (m & 3) + (m >> 2) + 16 * u;
  // step j reads bf[j & 1] + 128 (j >> 1): steps of equal parity differ by
  // whole 128-byte strides, which the permutation (bits 4..6) leaves alone
  uint32_t bf[2];
  bf[0] = buf + lds_off(r, 64 * k0 + 16 * g);
  bf[1] = buf + lds_off(r, 64 * (k0 + 1) + 16 * g);
  asm volatile("" : "+v"(bf[0]), "+v"(bf[1]));
  auto rd = [&](int j) { return lds_read_b128_at(bf[j & 1] + 128 * (j >> 1)); };
  floatx4 S = floatx4{};
  int4v a[D];
#pragma unroll
  for (int i = 0; i < D; ++i) a[i] = rd(i);
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const int4v c = a[j % D];
    if (j + D < 9) a[j % D] = rd(j + D);
    S = mfma16(__builtin_bit_cast(bf16x8, c), q[j], S);
    if (j % 2 == 1) dma(j / 2);
  }
  dma(4);
  return S;
}

// One block buffer (32 rows); rows at or past `hi` (per lane: it may differ
// between the query tokens of multi-token decode) are masked.  Scores for
// the wave's 16 heads over the 32 tokens, then the value product
// Z^T += C^T P^T for the wave's NT channel tiles, starting at tile mt0 (a
// multiple of 4): A = C^T (16 channels x 32 tokens) through transposing LDS
// reads, B = P^T.  The K = 32 slots of lane group g are tokens 4j + g
// (j < 4) and 16 + 4(j-4) + g.
template <int NT, int NQ>
__device__ __forceinline__ void softmax_value(WaveState<NT, NQ>& st, const floatx4 (&S)[2], uint32_t buf, int hi,
                                              int lane, int mt0, float scale_log2);

template <int NT, class Dma>
__device__ __forceinline__ void block_compute(WaveState<NT>& st, uint32_t buf, int hi, int lane, int mt0,
                                              float scale_log2, Dma&& dma) {
  // Recompute the lane's operand offsets in every call rather than let the
  // compiler keep one set per buffer live across the block loop.
  lane = lane_id_fresh();
  floatx4 S[2];
  // deeper operand prefetch where the accumulator leaves registers for it
  score32<NT <= 16 ? 4 : 1>(st.q, buf, lane, S[0], S[1], dma);
  softmax_value(st, S, buf, hi, lane, mt0, scale_log2);
}

// The scores of one 16-head group split over its four computing waves
// (channel groups): wave w multiplies subtile w & 1 over K-steps
// 9 (w >> 1) .. +8, the four partial products meet in LDS (`exch`, 4 KB:
// [wave][lane] x 16 bytes) across one barrier, and every wave adds the two
// halves of each subtile in the same order, so all four hold the same
// scores and the same softmax state.  The barrier is reached by every wave
// of the workgroup exactly once per call; the waves that do not compute
// meet it from the block loop.
template <int NT, class Dma>
__device__ __forceinline__ void block_compute_ksplit(WaveState<NT, 9>& st, uint32_t buf, uint32_t exch, int wave,
                                                     int hi, int lane, int mt0, float scale_log2, Dma&& dma) {
  lane = lane_id_fresh();
  const floatx4 part = score_half<4>(st.q, buf, lane, wave & 1, 9 * (wave >> 1), dma);
  *(MLA_LDS floatx4*)(uintptr_t)(exch + (64 * wave + lane) * 16) = part;
  __syncthreads();
  floatx4 S[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const floatx4 lo = *(const MLA_LDS floatx4*)(uintptr_t)(exch + (64 * u + lane) * 16);
    const floatx4 hi2 = *(const MLA_LDS floatx4*)(uintptr_t)(exch + (64 * (u + 2) + lane) * 16);
    S[u] = lo + hi2;
  }
  softmax_value(st, S, buf, hi, lane, mt0, scale_log2);
}

// Softmax of the block's scores S (the two subtiles of score32's layout) and
// the value product Z^T += C^T P^T for the wave's NT channel tiles.
template <int NT, int NQ>
__device__ __forceinline__ void softmax_value(WaveState<NT, NQ>& st, const floatx4 (&S)[2], uint32_t buf, int hi,
                                              int lane, int mt0, float scale_log2) {
  const int g = lane >> 4;
  float x[8], p[8];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = S[u][r] * scale_log2;
      x[4 * u + r] = 16 * u + 4 * r + g < hi ? v : -INFINITY;
    }
  }
  softmax_update(st, x, p);
  // Source lane s' of each 16-lane group points at row 4(s'/4) + g,
  // channels 16mt + 4(s'%4) .. +3, i.e. row byte 32mt + 8(s'%4); the
  // permutation leaves a base per mt%4 (and per row half) and a stride of
  // 128 bytes.
  const int vr = g + 4 * ((lane & 15) >> 2);
  const int vx = 8 * (lane & 3);
  uint32_t vb[2][4];  // [rows +0 / +16][mt % 4]
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    vb[0][q4] = buf + lds_off(vr, 32 * q4 + vx) + 32 * mt0;
    vb[1][q4] = buf + lds_off(vr + 16, 32 * q4 + vx) + 32 * mt0;
  }
  asm volatile("" : "+v"(vb[0][0]), "+v"(vb[0][1]), "+v"(vb[0][2]), "+v"(vb[0][3]));
  asm volatile("" : "+v"(vb[1][0]), "+v"(vb[1][1]), "+v"(vb[1][2]), "+v"(vb[1][3]));
  bf16x8 pb;
#pragma unroll
  for (int j = 0; j < 8; ++j) pb[j] = f2bf(p[j]);
  auto vread = [&](int j) {
    bf16x4 lo = lds_read_tr16_at(vb[0][j & 3] + 128 * (j >> 2));
    bf16x4 hi = lds_read_tr16_at(vb[1][j & 3] + 128 * (j >> 2));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  constexpr int D = NT < 3 ? NT : 3;
  bf16x8 va[D];
#pragma unroll
  for (int i = 0; i < D; ++i) va[i] = vread(i);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const bf16x8 cur = va[j % D];
    if (j + D < NT) va[j % D] = vread(j + D);
    st.zacc[j] = mfma16(cur, pb, st.zacc[j]);
  }
}

// Cache policy of a buffer access at device scope (sc1): it is coherent
// across the XCDs' separate L2 caches without any cache maintenance.
constexpr int kDeviceScope = 16;

// Normalise and write one wave's part: z rows [head][512] at channels
// c0 .. c0 + 16 NT, and lse[head] if with_lse.  DEV: the stores are made at
// device scope, for a reader in the same launch on another CU.
template <bool DEV = false, int NT, int NQ>
__device__ __forceinline__ void store_state(const WaveState<NT, NQ>& st, float l_tot, float* zdst, float* ldst, int h0,
                                            int H, int lane, int c0, bool with_lse) {
  constexpr float kLn2 = 0.69314718055994530942f;
  const int head = h0 + (lane & 15);
  const int g = lane >> 4;
  if (head >= H) return;
  // l_tot = 0: a piece all of whose keys lie after this query token (multi-
  // token decode); it leaves z = 0 and lse = -inf, which the merge weighs 0
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse = (st.m + __log2f(l_tot)) * kLn2;
  if constexpr (DEV) {
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(zdst), (short)0, 0x7fffffff, kRsrcWord3);
    const uint32_t off = (uint32_t)(head * kDc + c0 + 4 * g) * 4u;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int4v v = int4v{__float_as_int(st.zacc[j][0] * inv), __float_as_int(st.zacc[j][1] * inv),
                            __float_as_int(st.zacc[j][2] * inv), __float_as_int(st.zacc[j][3] * inv)};
      __builtin_amdgcn_raw_buffer_store_b128(v, rz, off + 64u * j, 0, kDeviceScope);
    }
    if (with_lse && ldst != nullptr && g == 0) {
      const __amdgpu_buffer_rsrc_t rl =
          __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(ldst), (short)0, 0x7fffffff, kRsrcWord3);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(lse), rl, 4u * head, 0, kDeviceScope);
    }
  } else {
    float* row = zdst + (size_t)head * kDc + c0;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      *(float4*)(row + 16 * j + 4 * g) = make_float4(st.zacc[j][0] * inv, st.zacc[j][1] * inv,
                                                     st.zacc[j][2] * inv, st.zacc[j][3] * inv);
    }
    if (with_lse && ldst != nullptr && g == 0) ldst[head] = lse;
  }
}

// ---------------------------------------------------------------------------
// Merge and value up-projection inside the decode launch
// ---------------------------------------------------------------------------
// With a.tickets set, the launch also does the work of merge_upproj_kernel
// (o_i = W_i^UV z_i, the "DeepSeek-V3" notes, ekkoxiao.github.io,
// §潜在向量的作用; the exact log-sum-exp merge of the pieces first):
//   * the pieces are stored at device scope (sc1: coherent across the XCDs'
//     L2 caches); when a unit has finished all its pieces, every wave waits
//     for its stores to complete and one thread adds 1 to ticket[b].piece
//     for every sequence b the unit stored a piece of;
//   * then workgroup u takes the (sequence, head) jobs u, u + U, ...: it
//     loads its W^UV rows, waits until ticket[b].piece counts every piece of
//     b, reads the pieces at device scope, merges them in slot order exactly
//     as merge_upproj_kernel does (same helpers, same bits) and multiplies;
//   * the job that brings ticket[b].job to H clears both counters, so the
//     next launch starts from zero without a memset.
// A release / acquire fence pair at agent scope instead writes back and
// invalidates whole L2 caches; on the 16-head decode that made the launch
// several times slower than the two-launch form.
// The launch has at most one workgroup per CU, so every producer is
// resident while a job waits.  The wait is bounded all the same: a job whose
// pieces have not all arrived within 0.2 s writes NaN.

// Pieces of sequence b: first partial slot and count (the producer side's
// Segment::slot0 and Segment::parts).
struct PieceRange {
  int slot0, parts;
};

__device__ __forceinline__ PieceRange piece_range(const DecodeArgs& a, const int* pfx, int P, int b) {
  if (a.splits == 0) {
    const long long G = min((long long)a.units, (long long)P);
    const int r0 = uniform(pfx[b]) + kStartCost, r1 = uniform(pfx[b + 1]);
    const int first = unit_of_block(r0, G, P), last = unit_of_block(r1 - 1, G, P);
    return PieceRange{first + b, last - first + 1};
  }
  const int S = a.splits;
  const int L = a.seq_lens[b];
  const int np = (L + kPage - 1) / kPage;
  const int chunk = (np + S - 1) / S;
  return PieceRange{b * S, (np + chunk - 1) / chunk};
}

// A device-scope load of one float at byte offset off from base (uniform).
__device__ __forceinline__ float load_dev(const float* base, uint32_t off) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(base), (short)0, 0x7fffffff, kRsrcWord3);
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kDeviceScope));
}

// Longest wait for the pieces of a job: 0.2 s of the 100 MHz real-time counter.
constexpr uint64_t kWaitTicks = 20000000;

// One (sequence, head) job by the whole 512-thread workgroup; zs is 2 KB of
// LDS and flag one int of it.
__device__ __forceinline__ void merge_job(const DecodeArgs& a, const int* pfx, int P, int job, float* zs,
                                          int* flag) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = job / a.H, head = job - b * a.H;
  const PieceRange pr = piece_range(a, pfx, P, b);
  int32_t* const ticket = a.tickets + kTicketInts * b;
  // the first poll goes out before the weight rows, so that its answer does
  // not wait for them (vector loads complete in order)
  int seen = 0;
  if (tid == 0) seen = __hip_atomic_load(ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // wave w: rows 16w .. 16w+15 of W^UV_head, lane l: channels 8l .. 8l+7
  const int4v* wrow = (const int4v*)((const bf16*)a.w_uv + ((size_t)(head % a.hs) * kDv + 16 * wave) * kDc) + lane;
  int4v wv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wv[r] = wrow[r * (kDc / 8)];
  if (tid == 0) {
    int ok = seen >= pr.parts;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (!ok) {
      __builtin_amdgcn_s_sleep(1);
      ok = __hip_atomic_load(ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= pr.parts;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) break;
    }
    *flag = ok;
  }
  __syncthreads();
  const bool ok = *(volatile int*)flag != 0;
  float* zrow = a.z + ((size_t)b * a.H + head) * kDc;
  float zval;
  if (!ok) {
    zval = __builtin_nanf("");
    zrow[tid] = zval;
    if (a.lse != nullptr && tid == 0) a.lse[(size_t)b * a.H + head] = zval;
  } else if (pr.parts == 1) {  // finished in one piece: z is final
    zval = load_dev(zrow, 4u * tid);
  } else {
    float mx = -INFINITY, wsum = 0.f;
    float acc[1] = {0.f};
    const int n = pr.parts;
    const float* zp0 = a.zp + (size_t)pr.slot0 * a.H * kDc;
    const float* lp0 = a.lsep + (size_t)pr.slot0 * a.H;
    // batches as merge_upproj_kernel takes them
    auto batches = [&](auto nb) {
      constexpr int kNB = decltype(nb)::value;
      for (int c0 = 0; c0 < n; c0 += kNB) {
        float lv[kNB];
        float zv[kNB][1];
#pragma unroll
        for (int u = 0; u < kNB; ++u) {
          // past the last piece: weight e^{-inf} = 0 times 0 (merge_upproj_kernel
          // re-loads the last piece there; 0 times it adds the same zero)
          const uint32_t sl = (uint32_t)((c0 + u) * a.H + head);
          const bool in = c0 + u < n;
          lv[u] = in ? load_dev(lp0, 4u * sl) : -INFINITY;
          zv[u][0] = in ? load_dev(zp0, 4u * (sl * kDc + tid)) : 0.f;
        }
        merge_batch(lv, zv, mx, wsum, acc);
      }
    };
    if (n <= 16) batches(std::integral_constant<int, 16>{});
    else batches(std::integral_constant<int, 32>{});
    const float inv = 1.0f / wsum;
    zval = acc[0] * inv;
    zrow[tid] = zval;
    if (a.lse != nullptr && tid == 0) a.lse[(size_t)b * a.H + head] = mx + __logf(wsum);
  }
  zs[tid] = zval;
  __syncthreads();
  // every piece of this job has been read: count the job (its answer is
  // needed only after the product below)
  int prev = 0;
  if (tid == 0) prev = __hip_atomic_fetch_add(ticket + kTicketInts / 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float4 z0 = *(const float4*)(zs + 8 * lane), z1 = *(const float4*)(zs + 8 * lane + 4);
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = dot8_bf16(wv[r], z0, z1);
  const float o_val = wave_rows_sum(v, lane);  // row lane >> 2 of the wave's 16
  if ((lane & 3) == 0) {
    const size_t oi = ((size_t)b * a.H + head) * kDv + 16 * wave + (lane >> 2);
    if (a.o_bf16) ((bf16*)a.o)[oi] = f2bf(o_val);
    else ((float*)a.o)[oi] = o_val;
  }
  if (tid == 0 && prev == a.H - 1) {  // the sequence's last job clears its counters
    __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ticket + kTicketInts / 2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // zs and flag are reused by the next job
}

// ---------------------------------------------------------------------------
// bf16 / fp8-cache matrix-core decode
// ---------------------------------------------------------------------------

// 8 waves: all of them copy blocks; the first HG*CG compute.  HG head groups
// of 16 heads times CG groups of 512/CG latent channels: every computing wave
// scores all tokens of a block for its heads (the CG waves of a head group
// compute the same scores) and accumulates only its channels, so the waves
// never combine partial softmax states.
//
// Pipeline (bf16): block i sits in buffer i % 4.  Each step waits for its
// own copy of block i, meets the other waves at one barrier (after which
// block i is complete and buffer (i+3) % 4 = (i-1) % 4 is no longer read),
// computes block i and then issues the copy of block i+3, so up to three
// blocks are in flight while one is consumed.  fp8: the copies land in four
// staging buffers and every block is expanded into one bf16 buffer between
// two barriers.
template <int HG, int CG, bool FP8>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mfma_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  static_assert(HG * CG <= kWaves, "too many compute waves");
  constexpr int NT = 32 / CG;  // channel tiles per wave
  static_assert(NT % 4 == 0, "channel groups start on a multiple of 4 tiles");
  constexpr int kSmem = FP8 ? kNBuf * kStageBytes + kBlockBytes : kNBuf * kBlockBytes;
  constexpr int kCopyLo = FP8 ? kFp8Copies : kCopiesLo;  // copies per block of waves 0..3
  constexpr int kCopyHi = FP8 ? kFp8Copies : kCopiesHi;  // and of waves 4..7
  // one head group: its four computing waves split the scores (K halves x
  // subtiles) and exchange the partial products
  constexpr bool kKSplit = HG == 1 && CG == 4;
  constexpr int NQ = kKSplit ? 9 : 18;
  // the exchange area comes out of the block-table copy, so that the
  // workgroup still fits the 160 KB of LDS
  constexpr int kBt = kKSplit ? kBtLds - 64 : kBtLds;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  __shared__ int pfx[kMaxSchedB + 1];
  __shared__ int lens[kMaxSchedB];
  __shared__ int bt_lds[kBt];
  __shared__ __attribute__((aligned(16))) float exch[kKSplit ? 4 * 64 * 4 : 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const bool computes = wave < HG * CG;
  const int hg = wave % HG, cg = wave / HG;
  const int h0 = hg * 16;
  const int mt0 = cg * NT;

  // a small block table (the balanced split over a few sequences, where
  // start-up latency matters most) is kept in LDS
  const bool bt_local = a.splits == 0 && a.prefill_T == 0 && a.B * a.max_pages <= kBt;
  int P = 0;
  if (a.splits == 0 && a.prefill_T == 0)
    P = block_prefix(a.seq_lens, a.B, pfx, lens, bt_local ? block_table : nullptr, a.B * a.max_pages, bt_lds);
  // the launch's own merge and up-projection jobs, after the unit's pieces
  // (of sequences pub0 .. pub1), which are published first
  int pub0 = 0, pub1 = -1;
  auto merge_jobs = [&]() {
    if (a.tickets == nullptr) return;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's piece stores are complete
    __syncthreads();  // ... and every other wave's; the block buffers are free
    if (tid == 0) {
      for (int b = pub0; b <= pub1; ++b)
        __hip_atomic_fetch_add(a.tickets + kTicketInts * b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float* zs = (float*)smem;
    int* flag = (int*)(smem + kDc * sizeof(float));
    for (int job = blockIdx.x; job < a.B * a.H; job += gridDim.x) merge_job(a, pfx, P, job, zs, flag);
  };
  // the unit's own pieces (a unit with none returns at once)
  [&]() {
    Cursor cp;
    cp.sch = schedule_begin(a, pfx, lens, P);
    cp.valid = schedule_next(a, cp.sch, cp.seg);
    if (!cp.valid) return;
    cp.k = cp.seg.t0 / kBlock;

    auto qrow = [&](const Segment& s) { return (const bf16*)a.q + (size_t)s.b * a.H * kRow; };
    auto block_hi = [&](const Cursor& c) { return min(c.seg.t1 - c.k * kBlock, kBlock); };
    // block-table reads use a uniform index, so they are scalar loads that do
    // not wait behind the copies in flight
    auto page_of = [&](const Cursor& c) {
      if (bt_local) return uniform(bt_lds[c.seg.b * a.max_pages + (c.k >> 1)]);
      const int32_t* bt = a.prefill_T > 0 ? block_table : block_table + (size_t)c.seg.b * a.max_pages;
      return bt[uniform(c.k >> 1)];
    };
    auto issue = [&](const Cursor& c, int slot) {
      const int page = page_of(c);
      if constexpr (FP8) {
        issue_block_fp8(a.ckv8, a.scale8, a.kr8, page, c.k & 1, smem + slot * kStageBytes, block_hi(c), wave, lane);
      } else {
        issue_block_bf16(a.rows + (size_t)page * kPageBytes, c.k & 1, smem + slot * kBlockBytes, block_hi(c), wave,
                         lane);
      }
    };
    // The first piece of every sequence records where its partials start and
    // how many pieces there are (1: finished here), for the merge kernel.
    auto note_pieces = [&](const Segment& s) {
      if (a.meta != nullptr && s.slot == s.slot0 && tid == 0) *(int2*)(a.meta + 2 * s.b) = make_int2(s.slot0, s.parts);
    };

    // First query: for up to two head groups it is copied into LDS like the
    // blocks (into the one buffer the first three blocks leave free), so that
    // waiting for it does not also wait for the blocks issued after it; with
    // more head groups it is loaded into registers directly.  Either way the
    // first three blocks are in flight meanwhile.
    WaveState<NT, NQ> st;
    // first K-step of the wave's query registers: 0 or 9 for the four waves
    // that split the scores, 0 for a wave that only copies (it loads a query
    // it never uses, and must not read past the head's 576 elements)
    const int k0 = kKSplit && computes ? 9 * (wave >> 1) : 0;
    static_assert(32 * (9 + NQ) <= kRow || !kKSplit, "split query registers stay inside the head's row");
    static_assert(32 * NQ <= kRow, "query registers stay inside the head's row");
    constexpr bool kQueryViaLds = HG <= 2;
    uint8_t* const qlds = FP8 ? smem + kNBuf * kStageBytes : smem + (kNBuf - 1) * kBlockBytes;
    static_assert(HG > 2 || 2 * 16 * kRowBytes <= kBlockBytes, "query staging space");
    if constexpr (kQueryViaLds) {
      issue_query_copy<HG>((const uint8_t*)qrow(cp.seg), a.H, qlds, wave, lane);
    } else {
      load_query(st.q, qrow(cp.seg), a.H, h0 + (lane & 15), lane >> 4, k0);
    }
    Cursor ld = cp;
    int issued = 0;
    // With the query staged through LDS, block 0 goes out with it and blocks
    // 1 and 2 only once it has landed: all workgroups start at once, and the
    // query and first block would otherwise queue behind 27 MB of later blocks.
    constexpr int kFirst = kQueryViaLds ? 1 : kNBuf - 1;
  #pragma unroll
    for (int j = 0; j < kFirst; ++j) {
      if (ld.valid) {
        issue(ld, j);
        ++issued;
        cursor_next(a, ld);
      }
    }
    if constexpr (kQueryViaLds) {
      wait_blocks<kCopyLo, kCopyHi>(issued, wave);  // the query copies, issued before the blocks, are done
      __syncthreads();
      // lane: head h0 + l%16, channels 32kk + 8g .. +7 of its row
      const uint32_t qa = lds_addr(qlds) + (16 * hg + (lane & 15)) * kRowBytes + 16 * (lane >> 4);
  #pragma unroll
      for (int kk = 0; kk < NQ; ++kk) st.q[kk] = __builtin_bit_cast(bf16x8, lds_read_b128_at(qa + 64 * (k0 + kk)));
    } else {
      consume_query(st.q);
    }
  #pragma unroll
    for (int j = kFirst; j < kNBuf - 1; ++j) {
      if (ld.valid) {
        issue(ld, j);
        ++issued;
        cursor_next(a, ld);
      }
    }
    reset_state(st);
    note_pieces(cp.seg);
    for (int i = 0;; ++i) {
      // wait for this wave's part of block i: the copies issued after it may stay in flight
      wait_blocks<kCopyLo, kCopyHi>(issued - i - 1, wave);
      __syncthreads();
      uint8_t* buf;
      if constexpr (FP8) {
        dequant_block<kWaves * 64>(smem + (i % kNBuf) * kStageBytes, smem + kNBuf * kStageBytes, wave);
        __syncthreads();
        buf = smem + kNBuf * kStageBytes;
      } else {
        buf = smem + (i % kNBuf) * kBlockBytes;
      }
      // The copy of block i+3 goes into the buffer of block i-1, which every
      // wave finished before the barrier.  bf16: a computing wave issues its
      // copies one by one between its score products.
      BlockCopies nb;
      nb.n = 0;
      if constexpr (!FP8) {
        if (ld.valid)
          nb = plan_block_bf16(a.rows + (size_t)page_of(ld) * kPageBytes, ld.k & 1,
                               smem + ((i + kNBuf - 1) % kNBuf) * kBlockBytes, block_hi(ld), wave);
      }
      auto dma = [&](int t) {
        if constexpr (!FP8) {
          if (t < nb.n) issue_copy(nb, t);
        }
      };
      if (computes) {
        // multi-token decode: query token t of the sequence sees keys up to
        // L - q_len + t, so the last q_len - 1 - t keys are masked for it
        int hi = block_hi(cp);
        if (a.q_len > 1) {
          const int head = min(h0 + (lane_id_fresh() & 15), a.H - 1);
          hi = min(hi, cp.seg.L - (a.q_len - 1 - head / a.hs) - kBlock * cp.k);
        }
        if constexpr (kKSplit) {
          block_compute_ksplit<NT>(st, lds_addr(buf), lds_addr(exch), wave, hi, lane, mt0, a.scale_log2, dma);
        } else {
          block_compute<NT>(st, lds_addr(buf), hi, lane, mt0, a.scale_log2, dma);
        }
      } else {
  #pragma unroll
        for (int t = 0; t < kCopiesLo; ++t) dma(t);
        if constexpr (kKSplit) __syncthreads();  // the score exchange of the computing waves
      }
      if (ld.valid) {
        if constexpr (FP8) issue(ld, (i + kNBuf - 1) % kNBuf);
        ++issued;
        cursor_next(a, ld);
      }

      if (cp.k == (cp.seg.t1 - 1) / kBlock) {  // last block of this piece
        const float l_tot = pair32_sum(pair16_sum(st.l));
        if (computes) {
          const Segment& sg = cp.seg;
          const bool whole = sg.parts == 1;
          float* zdst = whole ? a.z + (size_t)sg.b * a.H * kDc : a.zp + (size_t)sg.slot * a.H * kDc;
          float* ldst = whole ? (a.lse ? a.lse + (size_t)sg.b * a.H : nullptr) : a.lsep + (size_t)sg.slot * a.H;
          if (a.tickets != nullptr) store_state<true>(st, l_tot, zdst, ldst, h0, a.H, lane, mt0 * 16, cg == 0);
          else store_state(st, l_tot, zdst, ldst, h0, a.H, lane, mt0 * 16, cg == 0);
        }
        if (pub1 < pub0) pub0 = cp.seg.b;
        pub1 = cp.seg.b;
        cursor_next(a, cp);
        if (!cp.valid) break;
        load_query(st.q, qrow(cp.seg), a.H, h0 + (lane & 15), lane >> 4, k0);
        consume_query(st.q);
        reset_state(st);
        note_pieces(cp.seg);
      } else {
        cursor_next(a, cp);
      }
    }
  }();
  merge_jobs();
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
  int P = 0;
  if (a.splits == 0 && a.prefill_T == 0) P = block_prefix(a.seq_lens, a.B, pfx, lens);
  Schedule sch = schedule_begin(a, pfx, lens, P);
  Segment seg;
  while (schedule_next(a, sch, seg)) {
    if (a.meta != nullptr && head == 0 && seg.slot == seg.slot0 && tid == 0)
      *(int2*)(a.meta + 2 * seg.b) = make_int2(seg.slot0, seg.parts);
    const int32_t* bt = a.prefill_T > 0 ? a.block_table : a.block_table + (size_t)seg.b * a.max_pages;
    const float* q = (const float*)a.q + ((size_t)seg.b * a.H + head) * kRow;
    const float* pool = (const float*)a.rows;
    __syncthreads();
    for (int i = tid; i < kRow; i += 256) qs[i] = q[i];
    __syncthreads();
    float m = -INFINITY, l = 0.f, z0 = 0.f, z1 = 0.f;
    // multi-token decode: query token head / hs sees keys up to L - q_len + token
    const int j0 = seg.t0, j1 = a.q_len > 1 ? min(seg.t1, seg.L - (a.q_len - 1 - head / a.hs)) : seg.t1;
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
    const float inv = l > 0.f ? 1.0f / l : 0.f;  // l = 0: every key of the piece is masked
    zdst[tid] = z0 * inv;
    zdst[tid + 256] = z1 * inv;
    if (ldst != nullptr && tid == 0) *ldst = l > 0.f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
  }
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
    (void)launch_decode_wide(a, FP8, s);  // 65..128 heads: decode_wide.hip (error read by the caller)
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

}  // namespace mla
