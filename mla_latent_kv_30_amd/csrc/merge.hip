// Split-KV merge of the decode pass's partials, alone and fused with the
// value up-projection.  A sequence cut into pieces c, each normalised over
// its own keys with log-sum-exp lse_c, is recombined exactly:
//   lse = log sum_c e^{lse_c},  z = sum_c e^{lse_c - lse} z_c
// and then, fused for few sequences, o_i = W_i^UV z_i (the "DeepSeek-V3"
// notes, ekkoxiao.github.io, §潜在向量的作用).  The decode pass records for
// every sequence its first partial slot and its piece count.
#include "common.h"
#include "kernels.h"

namespace mla {

// ---------------------------------------------------------------------------
// Split merge: lse = log sum_c e^{lse_c};  z = sum_c e^{lse_c - lse} z_c
// ---------------------------------------------------------------------------
// One workgroup per (head, sequence), 128 threads of 4 channels each.  The
// sequence's first slot and piece count come from the decode pass's record;
// the pieces' log-sum-exps and z slices are loaded a batch at a time (one
// round trip per batch) and folded with a running maximum.  A batch is 8
// pieces when the sequence has at most 8 and 32 otherwise: past the last
// piece a batch re-loads that piece, so a wide batch over few pieces would
// mostly fetch repeats.
template <int NB>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int slot0, int n, int head, int tid, float& m,
                                             float& wsum, float4& acc) {
  for (int c0 = 0; c0 < n; c0 += NB) {
    float lv[NB];
    float4 zv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = min(c0 + u, n - 1);  // every slot loaded holds a piece of this sequence
      const size_t sl = (size_t)(slot0 + c) * a.H + head;
      lv[u] = c0 + u < n ? a.lsep[sl] : -INFINITY;
      zv[u] = *(const float4*)(a.zp + sl * kDc + 4 * tid);
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < NB; ++u) mb = fmaxf(mb, lv[u]);
    const float alpha = __expf(m - mb);  // m = -inf on the first batch: alpha = 0
    wsum *= alpha;
    acc.x *= alpha; acc.y *= alpha; acc.z *= alpha; acc.w *= alpha;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float w = __expf(lv[u] - mb);  // 0 for the padding entries
      wsum += w;
      acc.x += w * zv[u].x; acc.y += w * zv[u].y; acc.z += w * zv[u].z; acc.w += w * zv[u].w;
    }
    m = mb;
  }
}

__global__ void __launch_bounds__(128) merge_kernel(DecodeArgs a) {
  const int head = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int2 mt = *(const int2*)(a.meta + 2 * b);
  const int slot0 = mt.x, n = mt.y;
  if (n <= 1) return;  // finished in one piece by the decode pass
  float m = -INFINITY, wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (n <= 8) merge_pieces<8>(a, slot0, n, head, tid, m, wsum, acc);
  else merge_pieces<32>(a, slot0, n, head, tid, m, wsum, acc);
  const float inv = 1.0f / wsum;
  *(float4*)(a.z + ((size_t)b * a.H + head) * kDc + 4 * tid) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse != nullptr && tid == 0) a.lse[(size_t)b * a.H + head] = m + __logf(wsum);
}

// ---------------------------------------------------------------------------
// Split merge fused with the value up-projection o_i = W_i^UV z_i (the
// "DeepSeek-V3" notes, ekkoxiao.github.io, §潜在向量的作用), for few sequences
// ---------------------------------------------------------------------------
// One workgroup per (head, sequence), 256 threads.  The sequence's pieces are
// merged as merge_kernel does (2 channels per thread), into LDS and into z;
// then o = W^UV_h z is a matrix-vector product on the vector units.  Wave w
// owns output rows 32w .. 32w+31; one load instruction brings a whole 1 KB
// row, lane l holding channels 8l .. 8l+7, so every lane keeps 32 partial
// dot products that a butterfly over the wave finally sums.  The 32 row
// loads go out before the merge, so the weight and partial latencies
// overlap.  Every sequence re-reads W^UV_h (from L2), so this form is only
// used for up to kFusedMaxB sequences.
// The pieces of one sequence, NB per batch (one round trip each), folded
// into a running maximum, weight sum and this thread's two channels of z
// (merge_batch).
// The batch is 16 pieces for sequences of at most 16 and 32 otherwise, so
// that up to 32 pieces cost one round trip; past the last piece a batch
// re-loads that piece.
template <int NB>
__device__ __forceinline__ void fused_merge_pieces(const DecodeArgs& a, int slot0, int n, int head, int tid,
                                                   float& mx, float& wsum, float (&acc)[2]) {
  for (int c0 = 0; c0 < n; c0 += NB) {
    float lv[NB];
    float zv[NB][2];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = min(c0 + u, n - 1);  // every slot loaded holds a piece of this sequence
      const size_t sl = (size_t)(slot0 + c) * a.H + head;
      lv[u] = c0 + u < n ? a.lsep[sl] : -INFINITY;
      const float2 v = *(const float2*)(a.zp + sl * kDc + 2 * tid);
      zv[u][0] = v.x;
      zv[u][1] = v.y;
    }
    merge_batch(lv, zv, mx, wsum, acc);
  }
}

__global__ void __launch_bounds__(256) merge_upproj_kernel(MergeUpArgs m) {
  const DecodeArgs& a = m.d;
  const int head = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ __attribute__((aligned(16))) float zs[kDc];
  // multi-token decode: head h' of the merge is head h' % hs of token h' / hs
  const int4v* wrow = (const int4v*)((const bf16*)m.w_uv + ((size_t)(head % a.hs) * kDv + 32 * wave) * kDc) + lane;
  int4v wv[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) wv[r] = wrow[r * (kDc / 8)];

  float* zrow = a.z + ((size_t)b * a.H + head) * kDc;
  int slot0 = 0, n = 1;
  if (a.meta != nullptr) {
    const int2 mt = *(const int2*)(a.meta + 2 * b);
    slot0 = mt.x;
    n = mt.y;
  }
  if (n <= 1) {  // finished in one piece: the decode pass wrote z
    const float2 v = *(const float2*)(zrow + 2 * tid);
    zs[2 * tid] = v.x;
    zs[2 * tid + 1] = v.y;
  } else {
    float mx = -INFINITY, wsum = 0.f;
    float acc[2] = {0.f, 0.f};
    if (n <= 16) fused_merge_pieces<16>(a, slot0, n, head, tid, mx, wsum, acc);
    else fused_merge_pieces<32>(a, slot0, n, head, tid, mx, wsum, acc);
    const float inv = 1.0f / wsum;
    const float2 z2 = make_float2(acc[0] * inv, acc[1] * inv);
    zs[2 * tid] = z2.x;
    zs[2 * tid + 1] = z2.y;
    *(float2*)(zrow + 2 * tid) = z2;
    if (a.lse != nullptr && tid == 0) a.lse[(size_t)b * a.H + head] = mx + __logf(wsum);
  }
  __syncthreads();

  const float4 z0 = *(const float4*)(zs + 8 * lane), z1 = *(const float4*)(zs + 8 * lane + 4);
  float v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = dot8_bf16(wv[r], z0, z1);
  const float o_val = wave_rows_sum(v, lane);  // row lane >> 1 of the wave's 32
  if ((lane & 1) == 0) {
    const size_t oi = ((size_t)b * a.H + head) * kDv + 32 * wave + (lane >> 1);
    if (m.o_bf16) ((bf16*)m.o)[oi] = f2bf(o_val);
    else ((float*)m.o)[oi] = o_val;
  }
}

hipError_t launch_merge_upproj(const MergeUpArgs& m, hipStream_t s) {
  hipLaunchKernelGGL(merge_upproj_kernel, dim3(m.d.H, m.d.B), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.H, a.B), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
