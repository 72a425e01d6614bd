// Internal launch interface between the C entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace mla {

constexpr int kMaxSchedB = 512;  // sequences a balanced (auto) split can schedule
constexpr int kTicketInts = 64;  // 256 bytes of counters per sequence (decode + merge in one launch)
constexpr int kBtLds = 2048;     // block-table entries a decode workgroup keeps in LDS
constexpr int kKindF32 = 0;
constexpr int kKindBf16 = 1;
constexpr int kKindFp8 = 2;

struct DecodeArgs {
  const void* q;               // [NQ][H][576] fp32 or bf16
  const uint8_t* rows;         // fp32/bf16 pool [pages][64][576]
  const uint8_t* ckv8;         // fp8 pool parts
  const float* scale8;
  const uint8_t* kr8;
  const int32_t* block_table;  // [B][max_pages] (prefill: one row)
  const int32_t* seq_lens;     // [B] (prefill: unused)
  int32_t B, H, max_pages;
  int32_t splits;              // > 0: S chunks per sequence; 0: balanced over `units`
                               // (32-token blocks of all sequences in equal ranges)
  int32_t units;               // workgroups along x
  int32_t prefill_T;           // > 0: causal prefill of T rows (unit w -> row T-1-w)
  int32_t prefill_pos0;
  float scale_log2;            // softmax_scale * log2(e)
  int32_t q_len;               // query tokens per sequence (multi-token decode), 1 otherwise
  int32_t hs;                  // heads of one query token (H / q_len): head h' is token h' / hs
  float* z;
  float* lse;
  float* zp;                   // partials [slots][H][512]
  float* lsep;                 // partials [slots][H]
  int32_t* meta;               // [B][2] first partial slot and piece count of each
                               // split sequence (written by decode, read by merge)
  // Merge and value up-projection inside the decode launch (tickets != NULL;
  // one workgroup per CU at most, so that every unit is resident at once):
  int32_t* tickets;            // [B][kTicketInts]: piece counter at 0, job counter at
                               // kTicketInts / 2 (separate 128-byte lines); zero
                               // before the launch and left zero by it
  const void* w_uv;            // [hs][128][512] bf16
  void* o;                     // [B][H][128] out
  int32_t o_bf16;
};

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t s);
// 65..128 heads over a bf16 cache (four waves of 32 heads)
hipError_t launch_decode_wide(const DecodeArgs& a, bool fp8, hipStream_t s);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s);

// merge + value up-projection in one launch (bf16 W^UV, B <= kFusedMaxB)
constexpr int kFusedMaxB = 32;
struct MergeUpArgs {
  DecodeArgs d;      // B, H, z, lse and the workspace parts (meta == NULL: no partials)
  const void* w_uv;  // [H][128][512] bf16
  void* o;           // [B][H][128]
  int32_t o_bf16;
};
hipError_t launch_merge_upproj(const MergeUpArgs& m, hipStream_t s);

struct AbsorbArgs {
  const void* q_c;
  const void* q_r;
  const int32_t* pos;
  const void* w_uk;
  void* q_abs;
  int32_t N, H;
  RopeTable rope;
};
hipError_t launch_absorb(const AbsorbArgs& a, int kind, hipStream_t s);

struct CacheWriteArgs {
  const void* c_kv;
  const void* k_r;
  const int32_t* pos;   // [T], or NULL: token t is at position pos0 + t
  const int32_t* slot;  // [T], or NULL: slot from block table `bt` at that position
  const int32_t* bt;
  int32_t pos0;
  int32_t T;
  void* rows;
  uint8_t* ckv8;
  float* scale8;
  void* kr8;
  RopeTable rope;
  const float* part;    // non-NULL: inputs are the sums of `splits` fp32 partial
  int32_t splits;       // planes [splits][T][part_ld], c^KV | k^R at columns
  int32_t part_ld;      // part_col .. part_col+575, rounded once to the input
  int32_t part_col;     // precision (c_kv, k_r unused)
  bf16* cq;             // optional: columns 0 .. cq_width-1 of the planes,
  int32_t cq_width;     // summed and stored as bf16 [T][cq_width]
};
hipError_t launch_cache_write(const CacheWriteArgs& a, int kind, hipStream_t s);

struct UpprojArgs {
  const float* z;
  const void* w_uv;
  void* o;
  int32_t N, H;
  int32_t o_bf16;
};
hipError_t launch_upproj(const UpprojArgs& a, int w_kind, hipStream_t s);

// Y = X W^T (bf16 operands, fp32 accumulate); W is the row concatenation of
// up to three blocks [w[0]; w[1]; w[2]] (Mb[b] rows each, multiples of 32)
// and Y the matching column concatenation [y[0] | y[1] | y[2]].
constexpr int kLinBlocks = 3;
struct LinearArgs {
  const bf16* x;                 // [N][K]
  const bf16* w[kLinBlocks];     // [Mb[b]][K]
  void* y[kLinBlocks];           // [N][Mb[b]]
  int32_t Mb[kLinBlocks];        // 0: block absent
  float* part;                   // [splits][N][M] fp32 partials (splits > 1)
  int32_t N, K;
  int32_t out_bf16;              // bit b: y[b] in bf16 (else fp32)
  int32_t mt, nt, splits, kt_split;   // filled from the plan
};
constexpr int kLinSkinny32 = 0;  // 128 W rows x 32 tokens (N <= 32)
constexpr int kLinSkinny64 = 1;  // 128 x 64 (N <= 64)
constexpr int kLinMid = 2;       // 128 x 128
constexpr int kLinLarge = 3;     // 256 x 256
constexpr int kLinNarrow = 4;    // 64 x 64 (N <= 64, few output rows)
struct LinearPlan {
  int cfg, tm, tn, mt, nt, splits, kt_split;
  size_t part_bytes;
};
LinearPlan plan_linear(int N, int M, int K, int cus);
hipError_t launch_linear(LinearArgs a, const LinearPlan& p, hipStream_t s);

// W' = W^O blockdiag(W_1^UV .. W_H^UV): [d][H*512] bf16 from W^O [d][H*128]
// and W^UV [H][128][512], both bf16.
hipError_t launch_fold_wuv_wo(const bf16* w_uv, const bf16* w_o, bf16* w_fold, int H, int d, hipStream_t s);

}  // namespace mla
