/*
 * mla.h — C interface of libmla: absorbed Multi-head Latent Attention (MLA)
 * over a paged latent KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (the "DeepSeek-V3" equation notes, ekkoxiao.github.io):
 *   - each cached token keeps only (c^KV, k^R): a 512-element joint latent
 *     and a 64-element RoPE key shared by all heads (§KeyValue);
 *   - per head i the content key is k^C = W_i^UK c^KV; absorbing W_i^UK into
 *     the query gives q~_i = (W_i^UK)^T q_i^C, so the content score is
 *     q~_i . c^KV (§潜在向量的作用);
 *   - s = (q~_i . c_j + q_i^R . k_j^R) * scale, softmax over the visible
 *     tokens j, and the values are summed in latent space,
 *     z_i = sum_j a_{ij} c_j, before the up-projection o_i = W_i^UV z_i
 *     (§注意力计算 and §潜在向量的作用).
 *
 * Dimensions are fixed by the model ("DeepSeek-V3 技术报告精读",
 * oopvo.github.io, §维度分解详解): d_c = 512, rope 64, nope 128, v 128.
 * A cached row is 576 elements: c^KV (512) followed by the *rotated* k^R (64).
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are device pointers owned by the caller, dense and
 *     row-major in the shapes given.  The library allocates no memory and
 *     keeps no state except a per-device property cache.
 *   - Every tensor pointer (and every workspace) must be 16-byte aligned:
 *     the kernels move 16-byte vectors.  A misaligned pointer is rejected
 *     with MLA_ERR_INVALID_ARG (int32 index arrays are exempt).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Arguments are validated on the host before any HIP call; a
 *     rejected call launches nothing and returns its status synchronously.
 *   - A kernel launch failure returns MLA_ERR_HIP.  Faults during execution
 *     surface at the caller's next synchronisation.  No C++ exception
 *     crosses this interface.
 *   - RoPE rotates interleaved pairs (x[2m], x[2m+1]) counter-clockwise by
 *     pos * theta_m with theta_m = rope_base^(-2m/64), m = 0..31 (per-pair
 *     angle of §YaRN 扩展; frequency formula of "企业官网建设流程全解析",
 *     discosf.com, §4.3).  rope_base is 10000 for DeepSeek-V3.
 *   - softmax_scale is 1/sqrt(128 + 64) for the model (§注意力计算); it
 *     multiplies the raw dot product before the exponential.
 *   - Entry points are reentrant; concurrent calls on different streams are
 *     safe as long as their output and workspace buffers do not overlap.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad dtype combination */
  MLA_ERR_UNSUPPORTED = 2, /* valid request the library does not implement   */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  MLA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed      */
} mla_status;

typedef enum {
  MLA_F32 = 0,      /* IEEE fp32                                             */
  MLA_BF16 = 1,     /* bfloat16                                              */
  MLA_FP8_E4M3 = 2  /* OCP E4M3 (max 448), only for the cached latent c^KV  */
} mla_dtype;

#define MLA_D_C 512
#define MLA_D_R 64
#define MLA_D_NOPE 128
#define MLA_D_V 128
#define MLA_ROW 576
#define MLA_PAGE 64
#define MLA_MAX_HEADS 128

/*
 * Paged latent cache.  A pool of `num_pages` pages of 64 token slots; a
 * sequence's block-table row lists the pool page of each of its 64-token
 * blocks.  Layout by dtype:
 *   MLA_F32, MLA_BF16: rows      [num_pages][64][576]  (c^KV | rotated k^R)
 *   MLA_FP8_E4M3:      ckv_fp8   [num_pages][64][512]  e4m3 codes of c^KV
 *                      ckv_scale [num_pages][64][4]    fp32, one per 128
 *                                                      channels of a token
 *                      kr        [num_pages][64][64]   bf16 rotated k^R
 * The fp8 form follows the 1x128 per-token tile rule ("DeepSeek-V3 Technical
 * Report", process-cxr.github.io, §Fine-grained quantization): for each token
 * and 128-channel tile, scale = amax/448 in fp32 (1 for an all-zero tile) and
 * code = e4m3(round-to-nearest-even(clamp(c/scale, -448, 448))).
 * Unused pointers for a dtype must be NULL.  page_size must be 64.
 */
typedef struct {
  int32_t dtype;
  int32_t num_pages;
  int32_t page_size;
  int32_t reserved;
  void* rows;
  void* ckv_fp8;
  float* ckv_scale;
  void* kr;
} mla_cache;

/*
 * Rotary frequencies of the decoupled RoPE path (q^R, k^R).  Plain RoPE:
 * theta_j = base^(-2j/64).  YaRN ("DeepSeek-V3" notes, §YaRN 扩展; the
 * Technical Report, §Long Context Extension: s = 40, alpha = 1, beta = 32):
 *   theta'_j = (1 - gamma_j) theta_j / s + gamma_j theta_j,
 * gamma_j = clamp((r_j - alpha) / (beta - alpha), 0, 1) with r_j =
 * orig_len * theta_j / (2 pi) the turns group j makes over the context the
 * model was trained on before the extension (4096).  yarn_factor = 1 is plain
 * RoPE.  The same frequencies must rotate q^R (mla_absorb_q_rope) and k^R
 * (mla_cache_write_rope / mla_prefill_causal_rope).  YaRN's attention factor
 * (mla_yarn_attention_factor) multiplies the softmax scale the caller passes.
 */
typedef struct {
  float base;         /* 10000 */
  float yarn_factor;  /* s >= 1 */
  float yarn_alpha;   /* > 0 */
  float yarn_beta;    /* > yarn_alpha */
  int32_t orig_len;   /* >= 1 */
} mla_rope;

/* 0.1 ln s + 1 (the Technical Report, §Long Context Extension): the factor
 * YaRN applies to the attention scores; s <= 1 gives 1. */
double mla_yarn_attention_factor(double s);

/*
 * Checks of what the decode entry points take on trust (device data the
 * host does not read): every seq_lens[b] in [q_len, 64*max_pages] (q_len = 1
 * for one query token per sequence) and, when block_table is not NULL, every
 * page a sequence uses (entries 0 .. ceil(L_b/64)-1 of its row) in
 * [0, num_pages).
 * mla_validate_decode_inputs checks host copies:
 *   seq_lens [B], block_table [B][max_pages] or NULL (host memory)
 *   returns MLA_OK or MLA_ERR_INVALID_ARG.
 * mla_set_debug(1) (or MLA_DEBUG=1 in the environment) makes mla_decode,
 * mla_decode_partial, mla_decode_multi and mla_decode_multi_upproj copy the
 * lengths and the block table to the host in stream order, synchronise the
 * stream and apply the same check before launching (MLA_ERR_INVALID_ARG,
 * nothing launched).  A debugging aid: it blocks the caller and cannot run
 * under stream capture.
 */
mla_status mla_validate_decode_inputs(const int32_t* seq_lens, const int32_t* block_table, int32_t B,
                                      int32_t max_pages, int32_t num_pages, int32_t q_len);
void mla_set_debug(int32_t on);

/* Human-readable name of a status code (static storage). */
const char* mla_status_string(int32_t status);

/*
 * mla_absorb_q — the absorbed query (§潜在向量的作用: q~_i = (W_i^UK)^T q_i^C)
 * and the rotated position query (§Query: q^R = RoPE_t(...)).
 *   q_c   [N][H][128]   content query (dtype)
 *   q_r   [N][H][64]    position query before rotation (dtype)
 *   pos   [N] int32     position of each query token (>= 0)
 *   w_uk  [H][128][512] head i's row block of the key up-projection (dtype)
 *   q_abs [N][H][576]   out: q~ (512) followed by RoPE_pos(q_r) (64) (dtype)
 *   dtype MLA_F32 (fp32 throughout) or MLA_BF16 (bf16 in/out, fp32 accumulate)
 * Errors: MLA_ERR_INVALID_ARG for N < 1, H not in [1,128], a NULL pointer or
 * another dtype.
 */
mla_status mla_absorb_q(const void* q_c, const void* q_r, const int32_t* pos, const void* w_uk,
                        void* q_abs, int32_t N, int32_t H, int32_t dtype, float rope_base,
                        void* stream);

/* mla_absorb_q with the rotary frequencies of `rope` (NULL: base 10000,
 * no YaRN).  Errors: as mla_absorb_q, and MLA_ERR_INVALID_ARG for a rope
 * outside the ranges stated at mla_rope. */
mla_status mla_absorb_q_rope(const void* q_c, const void* q_r, const int32_t* pos, const void* w_uk, void* q_abs,
                             int32_t N, int32_t H, int32_t dtype, const mla_rope* rope, void* stream);

/*
 * mla_cache_write — store T tokens' (c^KV, RoPE_pos(k^R)) into the pool
 * (§KeyValue: only c^KV and the rotated k^R are cached).
 *   c_kv [T][512], k_r [T][64] (before rotation), in `in_dtype`
 *   pos  [T] int32   position of each token (the k^R rotation angle)
 *   slot [T] int32   pool row = page*64 + offset, in [0, num_pages*64)
 * Combinations: in MLA_F32 -> cache MLA_F32; in MLA_BF16 -> cache MLA_BF16
 * or MLA_FP8_E4M3 (quantised as described at mla_cache).  Slots must be
 * distinct; rows not named by `slot` are left untouched.
 */
mla_status mla_cache_write(const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* slot,
                           int32_t T, int32_t in_dtype, const mla_cache* cache, float rope_base,
                           void* stream);

/* mla_cache_write with the rotary frequencies of `rope` (as mla_absorb_q_rope). */
mla_status mla_cache_write_rope(const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* slot,
                                int32_t T, int32_t in_dtype, const mla_cache* cache, const mla_rope* rope,
                                void* stream);

/*
 * Workspace bytes mla_decode needs for B sequences, H heads and
 * `num_splits` (0 = automatic).  Depends only on its arguments and the
 * current device's compute-unit count.
 */
size_t mla_decode_workspace_size(int32_t B, int32_t H, int32_t num_splits);

/*
 * mla_decode — one new query token per sequence attends to all of its
 * cached tokens: scores (§注意力计算 with the absorbed content term of
 * §潜在向量的作用), softmax over the sequence, latent-space accumulation
 * z_i = sum_j a_{ij} c_j.  Long sequences are split into chunks whose
 * partial (z, log-sum-exp) pairs are merged exactly by log-sum-exp weights.
 *   q_abs        [B][H][576]  from mla_absorb_q (fp32 for an fp32 cache,
 *                             bf16 for a bf16 or fp8 cache)
 *   cache        the pool (see mla_cache)
 *   block_table  [B][max_pages] int32 pool page of each 64-token block
 *   seq_lens     [B] int32 cached tokens per sequence, 1 <= L <= 64*max_pages
 *                (the query is the newest of them)
 *   num_splits   0: the library cuts the 32-token blocks of all sequences
 *                into one nearly equal range per compute unit (a range may
 *                span sequences; for B > 512 every sequence is one chunk);
 *                S > 0: sequence b is cut into S chunks of
 *                ceil(ceil(L_b/64)/S) pages (trailing chunks may be empty).
 *   workspace    device scratch of at least mla_decode_workspace_size bytes
 *                (no initialisation needed); calls that share a workspace
 *                must not run concurrently.
 *   z            [B][H][512] fp32 out: normalised latent aggregate
 *   lse          [B][H] fp32 out (may be NULL): natural-log log-sum-exp of
 *                the scaled scores
 * seq_lens is device memory and is not inspected on the host: lengths of 0
 * or beyond 64*max_pages are undefined behaviour.
 * Errors: MLA_ERR_INVALID_ARG (NULL, B < 1, H not in [1,128], max_pages < 1,
 * page_size != 64, softmax_scale not finite and > 0, num_splits < 0 or
 * > 256, a pointer missing for the cache dtype); MLA_ERR_WORKSPACE.
 */
mla_status mla_decode(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                      const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages,
                      float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes,
                      float* z, float* lse, void* stream);

/*
 * The two halves of mla_decode, for callers that schedule the merge
 * themselves (overlapping it with other work, or combining chunk partials
 * produced by several calls).  mla_decode(...) is exactly
 * mla_decode_partial(...) followed by mla_decode_merge(...) on the same
 * stream with the same arguments.
 *
 * mla_decode_partial: the split pass.  Sequences that fall into a single
 * chunk get their final z / lse; every other chunk leaves its normalised
 * partial (z_c, lse_c) in the workspace.  Same arguments and errors as
 * mla_decode.
 */
mla_status mla_decode_partial(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages, float softmax_scale,
                              int32_t num_splits, void* workspace, size_t ws_bytes, float* z, float* lse,
                              void* stream);

/*
 * mla_decode_merge: lse = log sum_c e^{lse_c}, z = sum_c e^{lse_c - lse} z_c
 * over the chunks of each sequence that mla_decode_partial split (sequences
 * it finished in one chunk are left untouched).  B, H, num_splits,
 * seq_lens and the workspace must be those of the preceding partial pass.
 * Errors: MLA_ERR_INVALID_ARG (NULL seq_lens or z, B < 1, H not in [1,128],
 * num_splits < 0 or > 256); MLA_ERR_WORKSPACE.
 */
mla_status mla_decode_merge(const int32_t* seq_lens, int32_t B, int32_t H, int32_t num_splits, void* workspace,
                            size_t ws_bytes, float* z, float* lse, void* stream);

/* Bytes of device memory mla_decode_noalloc holds on every device it runs on. */
#define MLA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/*
 * mla_decode_noalloc — mla_decode for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): it takes no workspace and calls no allocator.  Its
 * split partials go to a device array of MLA_DECODE_NOALLOC_SCRATCH_BYTES
 * inside the library, one per device, held from the first use of the
 * library's code on that device until the process ends.  Arguments, outputs
 * and results are those of mla_decode (same kernels, same launch shapes,
 * bit-identical z and lse); the caller still provides q_abs, the cache, the
 * block table, the lengths, z and lse.  The debug mode's host-side checks
 * are not run.
 * Every call on one device shares that device's array and leaves its
 * contents behind (no call needs them cleared): calls that overlap in time on
 * one device race and must be ordered by the caller (one stream, or events).
 * Errors: as mla_decode; MLA_ERR_WORKSPACE when the call needs more than
 * MLA_DECODE_NOALLOC_SCRATCH_BYTES (mla_decode_workspace_size(B, H,
 * num_splits) bytes: with the automatic split, (CUs + B) * H * 2 KiB plus a
 * little, so B = 64, H = 128 fits); MLA_ERR_HIP if the array's device
 * address cannot be obtained.
 */
mla_status mla_decode_noalloc(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages,
                              float softmax_scale, int32_t num_splits, float* z, float* lse, void* stream);

/*
 * mla_decode_multi — q_len new tokens per sequence attend at once (the
 * multi-token decode of speculative verification, "DeepSeek-V3" notes
 * §Multi-Token Prediction): query token t of sequence b is at position
 * L_b - q_len + t and attends to cached tokens 0 .. L_b - q_len + t, i.e.
 * causally among the new tokens, which are already in the cache.
 *   q_abs      [B][q_len][H][576] (mla_absorb_q with N = B*q_len rows at those
 *              positions)
 *   seq_lens   [B] cached tokens including the q_len new ones; L_b >= q_len
 *   z          [B][q_len][H][512] fp32 out; lse [B][q_len][H] or NULL
 *   workspace  mla_decode_workspace_size(B, q_len*H, num_splits) bytes
 * Otherwise as mla_decode, with q_len*H heads: q_len*H <= 128.  The value
 * up-projection is mla_upproj_v with N = B*q_len.  (mla_decode_merge_upproj
 * is for one query token per sequence.)  Errors: as mla_decode, and
 * MLA_ERR_INVALID_ARG for q_len < 1 or q_len*H > 128.
 */
mla_status mla_decode_multi(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t H, int32_t max_pages,
                            float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes, float* z,
                            float* lse, void* stream);

/*
 * mla_decode_multi_upproj: mla_decode_multi followed by the value
 * up-projection o = W_i^UV z (§潜在向量的作用) of every query token's heads:
 * o [B][q_len][H][128] in o_dtype.  With a bf16 weight, B <= 32 and
 * q_len*H <= 64 the split merge and the up-projection run as one launch (as
 * in mla_decode_merge_upproj; z stays fp32 in that product), otherwise as
 * the merge and mla_upproj_v with N = B*q_len.  z and lse are written as
 * mla_decode_multi writes them.  Errors: those of mla_decode_multi, plus
 * MLA_ERR_INVALID_ARG for a NULL w_uv or o, or a dtype outside
 * {MLA_F32, MLA_BF16}.
 */
mla_status mla_decode_multi_upproj(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t H, int32_t max_pages,
                                   float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes, float* z,
                                   float* lse, const void* w_uv, int32_t w_dtype, void* o, int32_t o_dtype,
                                   void* stream);

/*
 * mla_decode_merge_upproj: mla_decode_merge followed by mla_upproj_v on its z
 * (o_i = W_i^UV z_i, §潜在向量的作用), with N = B.  Arguments as for those
 * two calls; z and lse are written as mla_decode_merge writes them.  With a
 * bf16 weight, B <= 32 and H <= 64 both run in one launch, whose product
 * keeps z in fp32 (bf16 weight values, fp32 accumulation); otherwise it is
 * the two calls (each of that launch's workgroups reads a head's whole
 * W^UV, which costs more than it saves with many heads).  Errors: those of mla_decode_merge, plus MLA_ERR_INVALID_ARG for a
 * NULL w_uv or o, or a dtype outside {MLA_F32, MLA_BF16}.
 */
mla_status mla_decode_merge_upproj(const int32_t* seq_lens, int32_t B, int32_t H, int32_t num_splits,
                                   void* workspace, size_t ws_bytes, float* z, float* lse, const void* w_uv,
                                   int32_t w_dtype, void* o, int32_t o_dtype, void* stream);

/*
 * mla_decode_upproj — one new token per sequence from the absorbed query to
 * the head outputs: mla_decode followed by o_i = W_i^UV z_i (the "DeepSeek-V3"
 * notes, ekkoxiao.github.io, §潜在向量的作用), i.e. mla_decode_partial then
 * mla_decode_merge_upproj, with the same arguments and the same results
 * (z, lse and o bit for bit).
 * Where it can, the whole step is one launch: with a bf16 or fp8 cache,
 * H <= 64, a bf16 W^UV, B <= 32 and no more work units than compute units,
 * the decode kernel merges and up-projects itself.  A finished piece of a
 * sequence increments a counter in the workspace; a (sequence, head) job
 * waits, inside the kernel, until the counter shows every piece, and the
 * last job of the sequence sets the counters back to zero.
 *   w_uv       [H][128][512] in w_dtype (MLA_BF16 or MLA_F32)
 *   o          [B][H][128] out in o_dtype (MLA_BF16 or MLA_F32)
 *   workspace  at least mla_decode_upproj_workspace_size(B, H, num_splits)
 *              bytes.  Its last 256*B bytes (from byte
 *              mla_decode_workspace_size(B, H, num_splits): two counters per
 *              sequence, on separate cache lines) must be zero before the
 *              first call; every call leaves them zero.  Calls
 *              that share a workspace must not run concurrently, and the
 *              one-launch form needs the GPU's compute units to itself
 *              (every unit resident at once).  A job whose pieces have not
 *              arrived within 0.2 s writes NaN to its z, lse and o rows; the
 *              counters must then be zeroed again.
 * Errors: those of mla_decode and mla_decode_merge_upproj.
 */
mla_status mla_decode_upproj(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages, float softmax_scale,
                             int32_t num_splits, void* workspace, size_t ws_bytes, float* z, float* lse,
                             const void* w_uv, int32_t w_dtype, void* o, int32_t o_dtype, void* stream);
/* Workspace bytes of mla_decode_upproj (0 for invalid arguments). */
size_t mla_decode_upproj_workspace_size(int32_t B, int32_t H, int32_t num_splits);
/* Launches mla_decode_upproj makes for these arguments on the current
 * device: 1 (the one-launch form), 2, or 0 for invalid arguments
 * (cache_dtype and w_dtype are MLA_* dtype codes). */
int32_t mla_decode_upproj_launches(int32_t B, int32_t H, int32_t num_splits, int32_t cache_dtype,
                                   int32_t w_dtype);

/*
 * mla_prefill_causal — T new tokens of one sequence, at positions
 * pos0 .. pos0+T-1, are written into the cache and attend causally: query t
 * sees cached tokens 0 .. pos0+t inclusive (§注意力计算 sums up to the
 * current position).  pos0 tokens must already be in the cache.
 *   q_abs           [T][H][576] from mla_absorb_q with pos = pos0 + t
 *   c_kv, k_r       [T][512], [T][64] the new tokens (k_r before rotation)
 *   cache           the pool (fp32 or bf16 rows, or the fp8 form, into which
 *                   the new tokens are quantised as mla_cache_write does)
 *   block_table_row [ceil((pos0+T)/64)] int32 pool pages of the sequence
 *   z               [T][H][512] fp32 out; lse [T][H] fp32 out or NULL
 * dtype of q_abs, c_kv, k_r: fp32 for an fp32 cache, bf16 otherwise.
 * Errors: MLA_ERR_INVALID_ARG as for mla_decode.
 */
mla_status mla_prefill_causal(const void* q_abs, const void* c_kv, const void* k_r, int32_t pos0,
                              const mla_cache* cache, const int32_t* block_table_row, int32_t T,
                              int32_t H, float softmax_scale, float rope_base, float* z, float* lse,
                              void* stream);

/* mla_prefill_causal with the rotary frequencies of `rope` (as mla_absorb_q_rope). */
mla_status mla_prefill_causal_rope(const void* q_abs, const void* c_kv, const void* k_r, int32_t pos0,
                                   const mla_cache* cache, const int32_t* block_table_row, int32_t T, int32_t H,
                                   float softmax_scale, const mla_rope* rope, float* z, float* lse, void* stream);

/*
 * mla_upproj_v — o_i = W_i^UV z_i (§潜在向量的作用, value up-projection).
 *   z    [N][H][512] fp32
 *   w_uv [H][128][512] head i's row block of the value up-projection (w_dtype)
 *   o    [N][H][128] out (o_dtype)
 * w_dtype, o_dtype in {MLA_F32, MLA_BF16}; a bf16 weight makes the product run
 * on bf16 matrix cores (z rounded to bf16, fp32 accumulation).
 */
mla_status mla_upproj_v(const float* z, const void* w_uv, void* o, int32_t N, int32_t H, int32_t w_dtype,
                        int32_t o_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Projections around the attention.  All take bf16 operands stored K-major
 * (each row contiguous along the contraction) and accumulate in fp32 on the
 * matrix cores.  The model width d is the caller's (the pages do not fix
 * it); it must be a multiple of 64.  A workspace is device memory the caller
 * owns, at least the size the matching *_workspace_size function returns
 * (that size depends on the arguments and the current device's compute-unit
 * count only); it is scratch that the call overwrites.  Every matrix and
 * workspace pointer must be 16-byte aligned (MLA_ERR_INVALID_ARG otherwise).
 * ------------------------------------------------------------------------ */

/* Workspace bytes mla_linear needs for an N x M output with contraction K
 * (0: none; also 0 for shapes mla_linear rejects). */
size_t mla_linear_workspace_size(int32_t N, int32_t M, int32_t K);

/*
 * mla_linear — Y = X W^T, the projection every equation of §KeyValue,
 * §Query and §注意力计算 applies to a token's vector (y = W x per row of X).
 * W is given as two row blocks and Y is written as the matching two column
 * blocks, so that a pair of projections that read the same input (W^DKV and
 * W^KR, or W^UQ and W^QR) runs as one product:
 *   x   [N][K] bf16
 *   w0  [M0][K] bf16, w1 [M1][K] bf16 (M1 = 0: w1 and y1 are ignored)
 *   y0  [N][M0], y1 [N][M1] out, in out_dtype (MLA_F32 or MLA_BF16)
 * Shapes: N >= 1; K >= 64, K % 64 == 0; M0 >= 32, M0 % 32 == 0; M1 >= 0,
 * M1 % 32 == 0; each operand under 2 GiB.  The workspace needs
 * mla_linear_workspace_size(N, M0 + M1, K) bytes.
 * Errors: MLA_ERR_INVALID_ARG (NULL pointer, a shape outside the above,
 * another dtype); MLA_ERR_WORKSPACE.
 */
mla_status mla_linear(const void* x, const void* w0, int32_t M0, const void* w1, int32_t M1, void* y0, void* y1,
                      int32_t N, int32_t K, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Workspace bytes of mla_kv_append (cache_dtype: the cache's dtype). */
size_t mla_kv_append_workspace_size(int32_t T, int32_t d, int32_t cache_dtype);

/*
 * mla_kv_append — what T new tokens add to the cache (§KeyValue):
 * c^KV = W^DKV h and k^R = RoPE_pos(W^KR h), stored (and quantised for an
 * fp8 cache) exactly as mla_cache_write_rope stores them.
 *   h      [T][d] bf16 hidden states
 *   w_dkv  [512][d] bf16, w_kr [64][d] bf16
 *   pos, slot, cache, rope: as mla_cache_write_rope (rope NULL: base 10000)
 * c^KV and k^R pass through the workspace in the cache's input precision
 * (fp32 for an fp32 cache, bf16 otherwise).
 * Errors: MLA_ERR_INVALID_ARG (NULL, d % 64 != 0, a bad cache or rope);
 * MLA_ERR_WORKSPACE.
 */
mla_status mla_kv_append(const void* h, const void* w_dkv, const void* w_kr, const int32_t* pos, const int32_t* slot,
                         int32_t T, int32_t d, const mla_cache* cache, const mla_rope* rope, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Workspace bytes of mla_q_project. */
size_t mla_q_project_workspace_size(int32_t T, int32_t d, int32_t dcq, int32_t H);

/*
 * mla_q_project — the queries of T tokens (§Query): c^Q = W^DQ h, then for
 * every head q_i^C = W_i^UQ c^Q and the position query W_i^QR c^Q before its
 * rotation (mla_absorb_q applies RoPE_pos and the absorption).
 *   h     [T][d] bf16
 *   w_dq  [dcq][d] bf16          (dcq = d_c', 1536 in the pages' model)
 *   w_uq  [H*128][dcq] bf16      rows 128 i .. 128 i + 127 are W_i^UQ
 *   w_qr  [H*64][dcq] bf16       rows 64 i .. 64 i + 63 are W_i^QR
 *   q_c   [T][H][128], q_r [T][H][64] out, in out_dtype
 * c^Q is kept in the workspace in bf16.  dcq % 64 == 0, H in [1,128].
 * Errors: MLA_ERR_INVALID_ARG; MLA_ERR_WORKSPACE.
 */
mla_status mla_q_project(const void* h, const void* w_dq, const void* w_uq, const void* w_qr, void* q_c, void* q_r,
                         int32_t T, int32_t d, int32_t dcq, int32_t H, int32_t out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Workspace bytes of mla_qkv_project (cache_dtype: the cache's dtype). */
size_t mla_qkv_project_workspace_size(int32_t T, int32_t d, int32_t dcq, int32_t H, int32_t cache_dtype);

/*
 * mla_qkv_project — mla_kv_append and mla_q_project of the same T tokens
 * in one call: both start from h (§KeyValue, §Query), so c^Q, c^KV and the
 * unrotated k^R come out of one product h [W^DQ; W^DKV; W^KR]^T; the cache
 * rows are then stored as mla_kv_append stores them and q_c, q_r computed
 * as mla_q_project computes them (rounded at the same points; the fp32 sums
 * may be grouped differently when the two plans split the product
 * differently).  Arguments as for those two calls.
 * Errors: MLA_ERR_INVALID_ARG; MLA_ERR_WORKSPACE.
 */
mla_status mla_qkv_project(const void* h, const void* w_dq, const void* w_dkv, const void* w_kr, const void* w_uq,
                           const void* w_qr, const int32_t* pos, const int32_t* slot, int32_t T, int32_t d,
                           int32_t dcq, int32_t H, const mla_cache* cache, const mla_rope* rope, void* q_c,
                           void* q_r, int32_t out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_output_proj — u = W^O [o_1; ...; o_H] (§注意力计算), N tokens.
 *   x  [N][K] bf16: the head outputs o [N][H][128] (K = 128 H), or the
 *      latent outputs z [N][H][512] in bf16 (K = 512 H) with the folded
 *      matrix of mla_fold_wuv_wo
 *   w  [d][K] bf16: W^O, or the folded matrix
 *   u  [N][d] out, in out_dtype
 * Workspace: mla_linear_workspace_size(N, d, K) bytes.  K % 128 == 0 and
 * d % 32 == 0, otherwise as mla_linear.
 */
mla_status mla_output_proj(const void* x, const void* w, void* u, int32_t N, int32_t K, int32_t d, int32_t out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_fold_wuv_wo — W' = W^O blockdiag(W_1^UV, ..., W_H^UV), the output
 * matrix with the value up-projection absorbed into it ("DeepSeek-V3
 * 技术报告精读", §一 MLA, KV 权重吸收), so that u = W' [z_1; ...; z_H].
 *   w_uv   [H][128][512] bf16, w_o [d][128 H] bf16
 *   w_fold [d][512 H] bf16 out (fp32 sums, rounded once)
 * A one-time weight transform.  W' holds four times the elements of W^O, so
 * for decode the two-step order (mla_decode_merge_upproj, then
 * mla_output_proj with W^O) moves fewer bytes.
 * Errors: MLA_ERR_INVALID_ARG (NULL, H not in [1,128], d < 1).
 */
mla_status mla_fold_wuv_wo(const void* w_uv, const void* w_o, void* w_fold, int32_t H, int32_t d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
