// C entry points of libmla: host-side validation, workspace sizing and
// dispatch to the gfx950 kernels.  See include/mla.h for the contract.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "mla.h"
#include "kernels.h"

namespace {

using namespace mla;

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev] = n;
  });
  return g_cus[dev];
}

RopeTable rope_table(float base) {
  RopeTable t;
  for (int m = 0; m < 32; ++m) t.theta[m] = pow((double)base, -2.0 * m / 64.0);
  return t;
}

bool rope_ok(const mla_rope& r) {
  return r.base > 1.0f && isfinite(r.base) && r.yarn_factor >= 1.0f && isfinite(r.yarn_factor) &&
         r.yarn_alpha > 0.0f && r.yarn_beta > r.yarn_alpha && isfinite(r.yarn_beta) && r.orig_len >= 1;
}

// Plain frequencies, then the YaRN blend per group: gamma ramps from 0 at
// alpha turns to 1 at beta turns over the original context.
RopeTable rope_table(const mla_rope& r) {
  RopeTable t = rope_table(r.base);
  if (r.yarn_factor == 1.0f) return t;
  const double two_pi = 6.283185307179586476925286766559;
  for (int m = 0; m < 32; ++m) {
    const double turns = (double)r.orig_len * t.theta[m] / two_pi;
    double gamma = (turns - (double)r.yarn_alpha) / ((double)r.yarn_beta - (double)r.yarn_alpha);
    gamma = gamma < 0.0 ? 0.0 : (gamma > 1.0 ? 1.0 : gamma);
    t.theta[m] = (1.0 - gamma) * t.theta[m] / (double)r.yarn_factor + gamma * t.theta[m];
  }
  return t;
}

mla_rope plain_rope(float base) { return mla_rope{base, 1.0f, 1.0f, 32.0f, 4096}; }

bool dtype_ok(int32_t d) { return d == MLA_F32 || d == MLA_BF16; }

mla_status launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Every tensor pointer: the kernels read and write them with 16-byte vectors
// (NULL passes; required pointers are checked for NULL separately).
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return false;
  return true;
}

// Validate the cache descriptor; returns the kernel kind or -1.
int cache_kind(const mla_cache* c) {
  if (c == nullptr || c->page_size != MLA_PAGE || c->num_pages < 1) return -1;
  if (!all_aligned16({c->rows, c->ckv_fp8, c->ckv_scale, c->kr})) return -1;
  switch (c->dtype) {
    case MLA_F32:
      return (c->rows && !c->ckv_fp8 && !c->ckv_scale && !c->kr) ? kKindF32 : -1;
    case MLA_BF16:
      return (c->rows && !c->ckv_fp8 && !c->ckv_scale && !c->kr) ? kKindBf16 : -1;
    case MLA_FP8_E4M3:
      return (!c->rows && c->ckv_fp8 && c->ckv_scale && c->kr) ? kKindFp8 : -1;
    default:
      return -1;
  }
}

// Split plan for a decode call.
struct Plan {
  int splits;  // > 0 uniform, 0 balanced
  int units;
  int slots;   // partial slots needed (0: every chunk is a whole sequence)
};

Plan make_plan(int32_t B, int32_t num_splits) {
  Plan p;
  if (num_splits > 0) {
    p.splits = num_splits;
    p.units = B * num_splits;
    p.slots = num_splits > 1 ? B * num_splits : 0;
  } else if (B > kMaxSchedB) {
    p.splits = 1;
    p.units = B;
    p.slots = 0;
  } else {
    p.splits = 0;
    p.units = device_cus();
    p.slots = p.units + B;
  }
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: [per-sequence piece record: B x (first slot, count) int32]
//                   [partial z: slots x H x 512 fp32][partial lse: slots x H fp32]
struct WsLayout {
  size_t meta, zp, lsep, total;
};

WsLayout ws_layout(int32_t B, int32_t H, const Plan& p) {
  WsLayout w{0, 0, 0, 0};
  if (p.slots == 0) return w;
  w.meta = 0;
  w.zp = align256((size_t)B * 2 * sizeof(int32_t));
  w.lsep = w.zp + align256((size_t)p.slots * H * kDc * sizeof(float));
  w.total = w.lsep + align256((size_t)p.slots * H * sizeof(float));
  return w;
}

size_t workspace_bytes(int32_t B, int32_t H, const Plan& p) { return ws_layout(B, H, p).total; }

void set_workspace(DecodeArgs& a, void* workspace, int32_t B, int32_t H, const Plan& p) {
  if (p.slots == 0) return;
  const WsLayout w = ws_layout(B, H, p);
  a.meta = (int32_t*)((char*)workspace + w.meta);
  a.zp = (float*)((char*)workspace + w.zp);
  a.lsep = (float*)((char*)workspace + w.lsep);
}

}  // namespace

extern "C" {

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: not supported by the library";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown mla_status";
  }
}

double mla_yarn_attention_factor(double s) { return s <= 1.0 ? 1.0 : 0.1 * log(s) + 1.0; }

mla_status mla_absorb_q_rope(const void* q_c, const void* q_r, const int32_t* pos, const void* w_uk, void* q_abs,
                             int32_t N, int32_t H, int32_t dtype, const mla_rope* rope, void* stream) {
  const mla_rope r = rope ? *rope : plain_rope(10000.0f);
  if (!q_c || !q_r || !pos || !w_uk || !q_abs) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({q_c, q_r, w_uk, q_abs})) return MLA_ERR_INVALID_ARG;
  if (N < 1 || H < 1 || H > MLA_MAX_HEADS || !dtype_ok(dtype)) return MLA_ERR_INVALID_ARG;
  if (!rope_ok(r)) return MLA_ERR_INVALID_ARG;
  if ((long long)N * H > 0x7fffffffLL) return MLA_ERR_INVALID_ARG;
  AbsorbArgs a{q_c, q_r, pos, w_uk, q_abs, N, H, rope_table(r)};
  return launched(launch_absorb(a, dtype == MLA_F32 ? kKindF32 : kKindBf16, (hipStream_t)stream));
}

mla_status mla_absorb_q(const void* q_c, const void* q_r, const int32_t* pos, const void* w_uk, void* q_abs,
                        int32_t N, int32_t H, int32_t dtype, float rope_base, void* stream) {
  if (!(rope_base > 1.0f) || !isfinite(rope_base)) return MLA_ERR_INVALID_ARG;
  const mla_rope r = plain_rope(rope_base);
  return mla_absorb_q_rope(q_c, q_r, pos, w_uk, q_abs, N, H, dtype, &r, stream);
}

mla_status mla_cache_write_rope(const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* slot,
                                int32_t T, int32_t in_dtype, const mla_cache* cache, const mla_rope* rope,
                                void* stream) {
  const mla_rope r = rope ? *rope : plain_rope(10000.0f);
  if (!c_kv || !k_r || !pos || !slot || T < 1 || !dtype_ok(in_dtype)) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({c_kv, k_r})) return MLA_ERR_INVALID_ARG;
  if (!rope_ok(r)) return MLA_ERR_INVALID_ARG;
  const int kind = cache_kind(cache);
  if (kind < 0) return MLA_ERR_INVALID_ARG;
  if (in_dtype == MLA_F32 && kind != kKindF32) return MLA_ERR_INVALID_ARG;
  if (in_dtype == MLA_BF16 && kind == kKindF32) return MLA_ERR_INVALID_ARG;
  CacheWriteArgs a{c_kv, k_r, pos, slot, nullptr, 0, T, cache->rows, (uint8_t*)cache->ckv_fp8,
                   cache->ckv_scale, cache->kr, rope_table(r)};
  return launched(launch_cache_write(a, kind, (hipStream_t)stream));
}

mla_status mla_cache_write(const void* c_kv, const void* k_r, const int32_t* pos, const int32_t* slot, int32_t T,
                           int32_t in_dtype, const mla_cache* cache, float rope_base, void* stream) {
  if (!(rope_base > 1.0f) || !isfinite(rope_base)) return MLA_ERR_INVALID_ARG;
  const mla_rope r = plain_rope(rope_base);
  return mla_cache_write_rope(c_kv, k_r, pos, slot, T, in_dtype, cache, &r, stream);
}

size_t mla_decode_workspace_size(int32_t B, int32_t H, int32_t num_splits) {
  if (B < 1 || H < 1 || H > MLA_MAX_HEADS || num_splits < 0 || num_splits > 256) return 0;
  return workspace_bytes(B, H, make_plan(B, num_splits));
}

namespace {

// Debug mode (mla_set_debug, or MLA_DEBUG=1 in the environment): the decode
// entry points copy the lengths and the block table to the host, in stream
// order, and check them before launching.
std::atomic<int> g_debug{-1};

bool debug_on() {
  int v = g_debug.load();
  if (v < 0) {
    const char* e = getenv("MLA_DEBUG");
    v = (e != nullptr && e[0] == '1') ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, v);
    v = g_debug.load();
  }
  return v == 1;
}

// Every length in [q_len, 64 * max_pages]; with a block table, every page a
// sequence uses in [0, num_pages).
mla_status check_lengths(const int32_t* lens, const int32_t* bt, int32_t B, int32_t max_pages, int32_t num_pages,
                         int32_t q_len) {
  for (int b = 0; b < B; ++b) {
    const long long L = lens[b];
    if (L < q_len || L > (long long)MLA_PAGE * max_pages) return MLA_ERR_INVALID_ARG;
    if (bt != nullptr) {
      const long long used = (L + MLA_PAGE - 1) / MLA_PAGE;
      for (long long k = 0; k < used; ++k) {
        const int32_t pg = bt[(size_t)b * max_pages + k];
        if (pg < 0 || pg >= num_pages) return MLA_ERR_INVALID_ARG;
      }
    }
  }
  return MLA_OK;
}

mla_status debug_check(const DecodeArgs& a, int32_t q_len, int32_t num_pages, hipStream_t s) {
  if (!debug_on()) return MLA_OK;
  int32_t* lens = (int32_t*)malloc(sizeof(int32_t) * (size_t)a.B);
  int32_t* bt = (int32_t*)malloc(sizeof(int32_t) * (size_t)a.B * a.max_pages);
  mla_status st = MLA_ERR_HIP;
  if (lens != nullptr && bt != nullptr &&
      hipMemcpyAsync(lens, a.seq_lens, sizeof(int32_t) * a.B, hipMemcpyDeviceToHost, s) == hipSuccess &&
      hipMemcpyAsync(bt, a.block_table, sizeof(int32_t) * (size_t)a.B * a.max_pages, hipMemcpyDeviceToHost, s) ==
          hipSuccess &&
      hipStreamSynchronize(s) == hipSuccess)
    st = check_lengths(lens, bt, a.B, a.max_pages, num_pages, q_len);
  free(lens);
  free(bt);
  return st;
}

// Validate a decode call and fill its launch arguments.
mla_status prepare_decode(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages, float softmax_scale,
                          int32_t num_splits, void* workspace, size_t ws_bytes, float* z, float* lse, DecodeArgs& a,
                          int& kind, Plan& p) {
  if (!q_abs || !block_table || !seq_lens || !z) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({q_abs, z, workspace})) return MLA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || H > MLA_MAX_HEADS || max_pages < 1) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 256) return MLA_ERR_INVALID_ARG;
  kind = cache_kind(cache);
  if (kind < 0) return MLA_ERR_INVALID_ARG;
  if ((long long)B * num_splits > 0x7fffffffLL) return MLA_ERR_INVALID_ARG;
  p = make_plan(B, num_splits);
  const size_t need = workspace_bytes(B, H, p);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  memset(&a, 0, sizeof(a));
  a.q = q_abs;
  a.rows = (const uint8_t*)cache->rows;
  a.ckv8 = (const uint8_t*)cache->ckv_fp8;
  a.scale8 = cache->ckv_scale;
  a.kr8 = (const uint8_t*)cache->kr;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.B = B;
  a.H = H;
  a.max_pages = max_pages;
  a.splits = p.splits;
  a.units = p.units;
  a.scale_log2 = (float)(softmax_scale * 1.4426950408889634074);
  a.q_len = 1;
  a.hs = H;
  a.z = z;
  a.lse = lse;
  set_workspace(a, workspace, B, H, p);
  return MLA_OK;
}

}  // namespace

mla_status mla_decode_partial(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages, float softmax_scale,
                              int32_t num_splits, void* workspace, size_t ws_bytes, float* z, float* lse,
                              void* stream) {
  DecodeArgs a;
  int kind;
  Plan p;
  mla_status st = prepare_decode(q_abs, cache, block_table, seq_lens, B, H, max_pages, softmax_scale, num_splits,
                                 workspace, ws_bytes, z, lse, a, kind, p);
  if (st != MLA_OK) return st;
  st = debug_check(a, 1, cache->num_pages, (hipStream_t)stream);
  if (st != MLA_OK) return st;
  (void)hipGetLastError();  // clear a stale error so a launch failure is reported as ours
  return launched(launch_decode(a, kind, (hipStream_t)stream));
}

mla_status mla_decode_merge(const int32_t* seq_lens, int32_t B, int32_t H, int32_t num_splits, void* workspace,
                            size_t ws_bytes, float* z, float* lse, void* stream) {
  if (!seq_lens || !z || B < 1 || H < 1 || H > MLA_MAX_HEADS) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({z, workspace})) return MLA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 256) return MLA_ERR_INVALID_ARG;
  const Plan p = make_plan(B, num_splits);
  const size_t need = workspace_bytes(B, H, p);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (p.slots == 0) return MLA_OK;  // every sequence was finished in one chunk
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.seq_lens = seq_lens;
  a.B = B;
  a.H = H;
  a.splits = p.splits;
  a.units = p.units;
  a.z = z;
  a.lse = lse;
  set_workspace(a, workspace, B, H, p);
  (void)hipGetLastError();
  return launched(launch_merge(a, (hipStream_t)stream));
}

namespace {

// The merge and the up-projection in one launch (merge_upproj_kernel) for a
// bf16 W^UV and few sequences.  Each of its (sequence, head) workgroups
// reads the head's 128 KB of W^UV, so with many heads the separate merge and
// tiled up-projection are faster: 8 sequences of 128 heads, 22.0 us in one
// launch against 19.5 us in two.
bool merge_upproj_fused(int B, int heads, int32_t w_dtype) {
  return w_dtype == MLA_BF16 && B <= kFusedMaxB && heads <= 64;
}

}  // namespace

mla_status mla_decode_merge_upproj(const int32_t* seq_lens, int32_t B, int32_t H, int32_t num_splits, void* workspace,
                                   size_t ws_bytes, float* z, float* lse, const void* w_uv, int32_t w_dtype, void* o,
                                   int32_t o_dtype, void* stream) {
  if (!seq_lens || !z || !w_uv || !o || B < 1 || H < 1 || H > MLA_MAX_HEADS) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({z, w_uv, o, workspace})) return MLA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 256) return MLA_ERR_INVALID_ARG;
  if (!dtype_ok(w_dtype) || !dtype_ok(o_dtype)) return MLA_ERR_INVALID_ARG;
  if ((long long)B * H > 0x7fffffffLL) return MLA_ERR_INVALID_ARG;
  const Plan p = make_plan(B, num_splits);
  const size_t need = workspace_bytes(B, H, p);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (merge_upproj_fused(B, H, w_dtype)) {
    MergeUpArgs m;
    memset(&m, 0, sizeof(m));
    m.d.B = B;
    m.d.H = H;
    m.d.hs = H;
    m.d.z = z;
    m.d.lse = lse;
    set_workspace(m.d, workspace, B, H, p);
    m.w_uv = w_uv;
    m.o = o;
    m.o_bf16 = o_dtype == MLA_BF16 ? 1 : 0;
    return launched(launch_merge_upproj(m, s));
  }
  mla_status st = mla_decode_merge(seq_lens, B, H, num_splits, workspace, ws_bytes, z, lse, stream);
  if (st != MLA_OK) return st;
  return mla_upproj_v(z, w_uv, o, B, H, w_dtype, o_dtype, stream);
}

size_t mla_decode_upproj_workspace_size(int32_t B, int32_t H, int32_t num_splits) {
  if (B < 1 || H < 1 || H > MLA_MAX_HEADS || num_splits < 0 || num_splits > 256) return 0;
  return workspace_bytes(B, H, make_plan(B, num_splits)) + (size_t)B * kTicketInts * sizeof(int32_t);
}

namespace {

// The one-launch form of mla_decode_upproj: the matrix-core kernel of up to
// 64 heads (it runs the merge jobs), a bf16 weight, few sequences (each job
// re-reads its W^UV block), and no more units than CUs, so that every unit
// is resident while a job waits for the pieces of others.
bool upproj_one_launch(int kind, int32_t B, int32_t H, int32_t w_dtype, const Plan& p) {
  return kind != kKindF32 && H <= 64 && w_dtype == MLA_BF16 && B <= kFusedMaxB && p.units <= device_cus();
}

}  // namespace

int32_t mla_decode_upproj_launches(int32_t B, int32_t H, int32_t num_splits, int32_t cache_dtype, int32_t w_dtype) {
  if (B < 1 || H < 1 || H > MLA_MAX_HEADS || num_splits < 0 || num_splits > 256) return 0;
  const int kind = cache_dtype == MLA_F32 ? kKindF32 : cache_dtype == MLA_BF16 ? kKindBf16
                   : cache_dtype == MLA_FP8_E4M3 ? kKindFp8 : -1;
  if (kind < 0 || !dtype_ok(w_dtype)) return 0;
  return upproj_one_launch(kind, B, H, w_dtype, make_plan(B, num_splits)) ? 1 : 2;
}

mla_status mla_decode_upproj(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages, float softmax_scale,
                             int32_t num_splits, void* workspace, size_t ws_bytes, float* z, float* lse,
                             const void* w_uv, int32_t w_dtype, void* o, int32_t o_dtype, void* stream) {
  if (!w_uv || !o || !dtype_ok(w_dtype) || !dtype_ok(o_dtype)) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({w_uv, o})) return MLA_ERR_INVALID_ARG;
  DecodeArgs a;
  int kind;
  Plan p;
  mla_status st = prepare_decode(q_abs, cache, block_table, seq_lens, B, H, max_pages, softmax_scale, num_splits,
                                 workspace, ws_bytes, z, lse, a, kind, p);
  if (st != MLA_OK) return st;
  const size_t base = workspace_bytes(B, H, p);
  if (workspace == nullptr || ws_bytes < base + (size_t)B * kTicketInts * sizeof(int32_t)) return MLA_ERR_WORKSPACE;
  st = debug_check(a, 1, cache->num_pages, (hipStream_t)stream);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (upproj_one_launch(kind, B, H, w_dtype, p)) {
    a.tickets = (int32_t*)((char*)workspace + base);
    a.w_uv = w_uv;
    a.o = o;
    a.o_bf16 = o_dtype == MLA_BF16 ? 1 : 0;
    return launched(launch_decode(a, kind, s));
  }
  st = launched(launch_decode(a, kind, s));
  if (st != MLA_OK) return st;
  return mla_decode_merge_upproj(seq_lens, B, H, num_splits, workspace, ws_bytes, z, lse, w_uv, w_dtype, o, o_dtype,
                                 stream);
}

mla_status mla_decode(const void* q_abs, const mla_cache* cache, const int32_t* block_table, const int32_t* seq_lens,
                      int32_t B, int32_t H, int32_t max_pages, float softmax_scale, int32_t num_splits, void* workspace,
                      size_t ws_bytes, float* z, float* lse, void* stream) {
  DecodeArgs a;
  int kind;
  Plan p;
  mla_status st = prepare_decode(q_abs, cache, block_table, seq_lens, B, H, max_pages, softmax_scale, num_splits,
                                 workspace, ws_bytes, z, lse, a, kind, p);
  if (st != MLA_OK) return st;
  st = debug_check(a, 1, cache->num_pages, (hipStream_t)stream);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  st = launched(launch_decode(a, kind, s));
  if (st != MLA_OK || p.slots == 0) return st;
  return launched(launch_merge(a, s));
}

}  // extern "C"

// Device memory of mla_decode_noalloc: the split partials and the piece
// records go to this file-scope array instead of a caller's workspace.  Every
// device the library runs on holds its own copy, from the first use of the
// library's code there until the process ends.  On the host the name is a
// stand-in for the symbol, not a device address: host code uses only the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MLA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current); NULL if the lookup failed.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  return g_scratch[dev];
}

}  // namespace

extern "C" {

mla_status mla_decode_noalloc(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t B, int32_t H, int32_t max_pages, float softmax_scale,
                              int32_t num_splits, float* z, float* lse, void* stream) {
  void* ws = scratch_address();
  if (ws == nullptr) return MLA_ERR_HIP;
  DecodeArgs a;
  int kind;
  Plan p;
  // a call whose partials exceed the array fails here with MLA_ERR_WORKSPACE
  mla_status st = prepare_decode(q_abs, cache, block_table, seq_lens, B, H, max_pages, softmax_scale, num_splits,
                                 ws, MLA_DECODE_NOALLOC_SCRATCH_BYTES, z, lse, a, kind, p);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  st = launched(launch_decode(a, kind, s));
  if (st != MLA_OK || p.slots == 0) return st;
  return launched(launch_merge(a, s));
}

mla_status mla_decode_multi(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t H, int32_t max_pages,
                            float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes, float* z,
                            float* lse, void* stream) {
  if (q_len < 1 || H < 1 || (long long)q_len * H > MLA_MAX_HEADS) return MLA_ERR_INVALID_ARG;
  DecodeArgs a;
  int kind;
  Plan p;
  mla_status st = prepare_decode(q_abs, cache, block_table, seq_lens, B, q_len * H, max_pages, softmax_scale,
                                 num_splits, workspace, ws_bytes, z, lse, a, kind, p);
  if (st != MLA_OK) return st;
  st = debug_check(a, q_len, cache->num_pages, (hipStream_t)stream);
  if (st != MLA_OK) return st;
  a.q_len = q_len;
  a.hs = H;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  st = launched(launch_decode(a, kind, s));
  if (st != MLA_OK || p.slots == 0) return st;
  return launched(launch_merge(a, s));
}

mla_status mla_decode_multi_upproj(const void* q_abs, const mla_cache* cache, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t H, int32_t max_pages,
                                   float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes, float* z,
                                   float* lse, const void* w_uv, int32_t w_dtype, void* o, int32_t o_dtype,
                                   void* stream) {
  if (q_len < 1 || H < 1 || (long long)q_len * H > MLA_MAX_HEADS) return MLA_ERR_INVALID_ARG;
  if (!w_uv || !o || !dtype_ok(w_dtype) || !dtype_ok(o_dtype)) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({w_uv, o})) return MLA_ERR_INVALID_ARG;
  DecodeArgs a;
  int kind;
  Plan p;
  mla_status st = prepare_decode(q_abs, cache, block_table, seq_lens, B, q_len * H, max_pages, softmax_scale,
                                 num_splits, workspace, ws_bytes, z, lse, a, kind, p);
  if (st != MLA_OK) return st;
  st = debug_check(a, q_len, cache->num_pages, (hipStream_t)stream);
  if (st != MLA_OK) return st;
  a.q_len = q_len;
  a.hs = H;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  st = launched(launch_decode(a, kind, s));
  if (st != MLA_OK) return st;
  if (merge_upproj_fused(B, q_len * H, w_dtype)) {
    MergeUpArgs m;
    memset(&m, 0, sizeof(m));
    m.d = a;
    m.w_uv = w_uv;
    m.o = o;
    m.o_bf16 = o_dtype == MLA_BF16 ? 1 : 0;
    return launched(launch_merge_upproj(m, s));
  }
  if (p.slots > 0) {
    st = launched(launch_merge(a, s));
    if (st != MLA_OK) return st;
  }
  return mla_upproj_v(z, w_uv, o, B * q_len, H, w_dtype, o_dtype, stream);
}

mla_status mla_prefill_causal(const void* q_abs, const void* c_kv, const void* k_r, int32_t pos0,
                              const mla_cache* cache, const int32_t* block_table_row, int32_t T, int32_t H,
                              float softmax_scale, float rope_base, float* z, float* lse, void* stream) {
  if (!(rope_base > 1.0f) || !isfinite(rope_base)) return MLA_ERR_INVALID_ARG;
  const mla_rope r = plain_rope(rope_base);
  return mla_prefill_causal_rope(q_abs, c_kv, k_r, pos0, cache, block_table_row, T, H, softmax_scale, &r, z, lse,
                                 stream);
}

mla_status mla_prefill_causal_rope(const void* q_abs, const void* c_kv, const void* k_r, int32_t pos0,
                                   const mla_cache* cache, const int32_t* block_table_row, int32_t T, int32_t H,
                                   float softmax_scale, const mla_rope* rope, float* z, float* lse, void* stream) {
  const mla_rope rp = rope ? *rope : plain_rope(10000.0f);
  if (!q_abs || !block_table_row || !z || !c_kv || !k_r) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({q_abs, z, c_kv, k_r})) return MLA_ERR_INVALID_ARG;
  if (T < 1 || H < 1 || H > MLA_MAX_HEADS || pos0 < 0) return MLA_ERR_INVALID_ARG;
  if ((long long)pos0 + T > 0x7fffffffLL) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (!rope_ok(rp)) return MLA_ERR_INVALID_ARG;
  const int kind = cache_kind(cache);
  if (kind < 0) return MLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  // 1. append the T new tokens: position pos0 + t, slot from the block-table row
  CacheWriteArgs w{c_kv,         k_r, nullptr, nullptr, block_table_row, pos0, T, cache->rows, (uint8_t*)cache->ckv_fp8,
                   cache->ckv_scale, cache->kr, rope_table(rp)};
  mla_status st = launched(launch_cache_write(w, kind, s));
  if (st != MLA_OK) return st;
  // 2. causal attention: query row t sees cached tokens 0 .. pos0 + t
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q_abs;
  a.rows = (const uint8_t*)cache->rows;
  a.ckv8 = (const uint8_t*)cache->ckv_fp8;
  a.scale8 = cache->ckv_scale;
  a.kr8 = (const uint8_t*)cache->kr;
  a.block_table = block_table_row;
  a.B = T;
  a.H = H;
  a.max_pages = (pos0 + T + MLA_PAGE - 1) / MLA_PAGE;
  a.splits = 1;
  a.units = T;
  a.prefill_T = T;
  a.prefill_pos0 = pos0;
  a.q_len = 1;
  a.hs = H;
  a.scale_log2 = (float)(softmax_scale * 1.4426950408889634074);
  a.z = z;
  a.lse = lse;
  return launched(launch_decode(a, kind, s));
}

mla_status mla_upproj_v(const float* z, const void* w_uv, void* o, int32_t N, int32_t H, int32_t w_dtype,
                        int32_t o_dtype, void* stream) {
  if (!z || !w_uv || !o || N < 1 || H < 1 || H > MLA_MAX_HEADS) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({z, w_uv, o})) return MLA_ERR_INVALID_ARG;
  if (!dtype_ok(w_dtype) || !dtype_ok(o_dtype)) return MLA_ERR_INVALID_ARG;
  if ((long long)N * H > 0x7fffffffLL) return MLA_ERR_INVALID_ARG;
  UpprojArgs a{z, w_uv, o, N, H, o_dtype == MLA_BF16 ? 1 : 0};
  return launched(launch_upproj(a, w_dtype == MLA_F32 ? kKindF32 : kKindBf16, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Projections around the attention
// ---------------------------------------------------------------------------

namespace {

constexpr long long kMaxOperandBytes = 0x7fffffffLL;   // buffer offsets are 31-bit

bool rows_fit(long long rows, int K) { return (rows + 256) * (long long)K * 2 <= kMaxOperandBytes; }

bool linear_shape_ok(int N, int M0, int M1, int K) {
  if (N < 1 || K < 64 || K % 64 != 0 || M0 < 32 || M0 % 32 != 0 || M1 < 0 || M1 % 32 != 0) return false;
  return rows_fit(N, K) && rows_fit(M0, K) && rows_fit(M1, K) &&
         (long long)N * (M0 + M1) * 4 <= kMaxOperandBytes;
}

// One product's row blocks of W and column blocks of Y.
struct Blocks {
  const void* w[kLinBlocks] = {nullptr, nullptr, nullptr};
  void* y[kLinBlocks] = {nullptr, nullptr, nullptr};
  int M[kLinBlocks] = {0, 0, 0};
  int bf16_mask = 0;   // bit b: y[b] in bf16
  int rows() const { return M[0] + M[1] + M[2]; }
  void add(const void* wb, int m, void* yb, bool bf) {
    int b = M[0] == 0 ? 0 : (M[1] == 0 ? 1 : 2);
    w[b] = wb;
    y[b] = yb;
    M[b] = m;
    if (bf) bf16_mask |= 1 << b;
  }
};

// Y = X W^T.  With y[0] == NULL the product is split or not as planned and,
// if split, leaves its partials in `ws` for the caller (no reduction).
mla_status run_linear(const void* x, const Blocks& bl, int N, int K, uint8_t* ws, size_t ws_bytes, hipStream_t st) {
  const LinearPlan p = plan_linear(N, bl.rows(), K, device_cus());
  if (p.part_bytes > 0 && (ws == nullptr || ws_bytes < p.part_bytes)) return MLA_ERR_WORKSPACE;
  LinearArgs a{};
  a.x = (const bf16*)x;
  for (int b = 0; b < kLinBlocks; ++b) {
    a.w[b] = (const bf16*)bl.w[b];
    a.y[b] = bl.y[b];
    a.Mb[b] = bl.M[b];
  }
  a.part = (float*)ws;
  a.N = N;
  a.K = K;
  a.out_bf16 = bl.bf16_mask;
  return launched(launch_linear(a, p, st));
}

size_t linear_ws(int N, int M, int K) { return plan_linear(N, M, K, device_cus()).part_bytes; }

}  // namespace

extern "C" {

void mla_set_debug(int32_t on) { g_debug.store(on ? 1 : 0); }

mla_status mla_validate_decode_inputs(const int32_t* seq_lens, const int32_t* block_table, int32_t B,
                                      int32_t max_pages, int32_t num_pages, int32_t q_len) {
  if (!seq_lens || B < 1 || max_pages < 1 || num_pages < 1 || q_len < 1) return MLA_ERR_INVALID_ARG;
  return check_lengths(seq_lens, block_table, B, max_pages, num_pages, q_len);
}

size_t mla_linear_workspace_size(int32_t N, int32_t M, int32_t K) {
  if (!linear_shape_ok(N, M, 0, K)) return 0;
  return linear_ws(N, M, K);
}

mla_status mla_linear(const void* x, const void* w0, int32_t M0, const void* w1, int32_t M1, void* y0, void* y1,
                      int32_t N, int32_t K, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!x || !w0 || !y0 || !dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (!linear_shape_ok(N, M0, M1, K)) return MLA_ERR_INVALID_ARG;
  if (M1 > 0 && (!w1 || !y1)) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({x, w0, w1, y0, y1, workspace})) return MLA_ERR_INVALID_ARG;
  const bool bf = out_dtype == MLA_BF16;
  Blocks bl;
  bl.add(w0, M0, y0, bf);
  if (M1 > 0) bl.add(w1, M1, y1, bf);
  return run_linear(x, bl, N, K, (uint8_t*)workspace, workspace_bytes, (hipStream_t)stream);
}

size_t mla_kv_append_workspace_size(int32_t T, int32_t d, int32_t cache_dtype) {
  if (!linear_shape_ok(T, MLA_D_C, MLA_D_R, d)) return 0;
  const size_t el = cache_dtype == MLA_F32 ? 4 : 2;
  return align256((size_t)T * MLA_ROW * el) + linear_ws(T, MLA_ROW, d);
}

mla_status mla_kv_append(const void* h, const void* w_dkv, const void* w_kr, const int32_t* pos, const int32_t* slot,
                         int32_t T, int32_t d, const mla_cache* cache, const mla_rope* rope, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!h || !w_dkv || !w_kr || !pos || !slot) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({h, w_dkv, w_kr, workspace})) return MLA_ERR_INVALID_ARG;
  if (!linear_shape_ok(T, MLA_D_C, MLA_D_R, d)) return MLA_ERR_INVALID_ARG;
  const mla_rope r = rope ? *rope : plain_rope(10000.0f);
  if (!rope_ok(r)) return MLA_ERR_INVALID_ARG;
  const int kind = cache_kind(cache);
  if (kind < 0) return MLA_ERR_INVALID_ARG;
  const bool f32 = kind == kKindF32;
  const size_t inter = align256((size_t)T * MLA_ROW * (f32 ? 4 : 2));
  if (workspace == nullptr || workspace_bytes < mla_kv_append_workspace_size(T, d, cache->dtype))
    return MLA_ERR_WORKSPACE;
  uint8_t* ws = (uint8_t*)workspace;
  void* c_kv = ws;
  void* k_r = ws + (size_t)T * MLA_D_C * (f32 ? 4 : 2);
  const hipStream_t st = (hipStream_t)stream;
  // A split product leaves its fp32 partials for the cache write to sum (one
  // launch less); otherwise the product writes c^KV and k^R in the input
  // precision of the cache write.
  const int splits = plan_linear(T, MLA_ROW, d, device_cus()).splits;
  Blocks bl;
  bl.add(w_dkv, MLA_D_C, splits > 1 ? nullptr : c_kv, !f32);
  bl.add(w_kr, MLA_D_R, splits > 1 ? nullptr : k_r, !f32);
  mla_status e = run_linear(h, bl, T, d, ws + inter, workspace_bytes - inter, st);
  if (e != MLA_OK) return e;
  CacheWriteArgs a{c_kv, k_r, pos, slot, nullptr, 0, T, cache->rows, (uint8_t*)cache->ckv_fp8,
                   cache->ckv_scale, cache->kr, rope_table(r)};
  if (splits > 1) {
    a.part = (const float*)(ws + inter);
    a.splits = splits;
    a.part_ld = MLA_ROW;
    a.part_col = 0;
  }
  return launched(launch_cache_write(a, kind, st));
}

size_t mla_q_project_workspace_size(int32_t T, int32_t d, int32_t dcq, int32_t H) {
  if (H < 1 || H > MLA_MAX_HEADS || !linear_shape_ok(T, dcq, 0, d)) return 0;
  if (!linear_shape_ok(T, H * MLA_D_NOPE, H * MLA_D_R, dcq)) return 0;
  const size_t a = linear_ws(T, dcq, d), b = linear_ws(T, H * (MLA_D_NOPE + MLA_D_R), dcq);
  return align256((size_t)T * dcq * 2) + (a > b ? a : b);
}

mla_status mla_q_project(const void* h, const void* w_dq, const void* w_uq, const void* w_qr, void* q_c, void* q_r,
                         int32_t T, int32_t d, int32_t dcq, int32_t H, int32_t out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!h || !w_dq || !w_uq || !w_qr || !q_c || !q_r || !dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({h, w_dq, w_uq, w_qr, q_c, q_r, workspace})) return MLA_ERR_INVALID_ARG;
  if (H < 1 || H > MLA_MAX_HEADS || !linear_shape_ok(T, dcq, 0, d)) return MLA_ERR_INVALID_ARG;
  if (!linear_shape_ok(T, H * MLA_D_NOPE, H * MLA_D_R, dcq)) return MLA_ERR_INVALID_ARG;
  const size_t need = mla_q_project_workspace_size(T, d, dcq, H);
  if (workspace == nullptr || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  uint8_t* ws = (uint8_t*)workspace;
  const size_t inter = align256((size_t)T * dcq * 2);
  const hipStream_t st = (hipStream_t)stream;
  Blocks b1;
  b1.add(w_dq, dcq, ws, true);
  mla_status e = run_linear(h, b1, T, d, ws + inter, workspace_bytes - inter, st);
  if (e != MLA_OK) return e;
  const bool bf = out_dtype == MLA_BF16;
  Blocks b2;
  b2.add(w_uq, H * MLA_D_NOPE, q_c, bf);
  b2.add(w_qr, H * MLA_D_R, q_r, bf);
  return run_linear(ws, b2, T, dcq, ws + inter, workspace_bytes - inter, st);
}

size_t mla_qkv_project_workspace_size(int32_t T, int32_t d, int32_t dcq, int32_t H, int32_t cache_dtype) {
  if (H < 1 || H > MLA_MAX_HEADS || !linear_shape_ok(T, dcq, MLA_ROW, d)) return 0;
  if (!linear_shape_ok(T, H * MLA_D_NOPE, H * MLA_D_R, dcq)) return 0;
  const size_t el = cache_dtype == MLA_F32 ? 4 : 2;
  const size_t a = linear_ws(T, dcq + MLA_ROW, d), b = linear_ws(T, H * (MLA_D_NOPE + MLA_D_R), dcq);
  return align256((size_t)T * dcq * 2) + align256((size_t)T * MLA_ROW * el) + (a > b ? a : b);
}

mla_status mla_qkv_project(const void* h, const void* w_dq, const void* w_dkv, const void* w_kr, const void* w_uq,
                           const void* w_qr, const int32_t* pos, const int32_t* slot, int32_t T, int32_t d,
                           int32_t dcq, int32_t H, const mla_cache* cache, const mla_rope* rope, void* q_c,
                           void* q_r, int32_t out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h || !w_dq || !w_dkv || !w_kr || !w_uq || !w_qr || !pos || !slot || !q_c || !q_r || !dtype_ok(out_dtype))
    return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({h, w_dq, w_dkv, w_kr, w_uq, w_qr, q_c, q_r, workspace})) return MLA_ERR_INVALID_ARG;
  if (H < 1 || H > MLA_MAX_HEADS || !linear_shape_ok(T, dcq, MLA_ROW, d)) return MLA_ERR_INVALID_ARG;
  if (!linear_shape_ok(T, H * MLA_D_NOPE, H * MLA_D_R, dcq)) return MLA_ERR_INVALID_ARG;
  const mla_rope r = rope ? *rope : plain_rope(10000.0f);
  if (!rope_ok(r)) return MLA_ERR_INVALID_ARG;
  const int kind = cache_kind(cache);
  if (kind < 0) return MLA_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < mla_qkv_project_workspace_size(T, d, dcq, H, cache->dtype))
    return MLA_ERR_WORKSPACE;
  const bool f32 = kind == kKindF32;
  uint8_t* ws = (uint8_t*)workspace;
  uint8_t* cq = ws;
  uint8_t* kv = cq + align256((size_t)T * dcq * 2);
  uint8_t* part = kv + align256((size_t)T * MLA_ROW * (f32 ? 4 : 2));
  const size_t part_bytes = workspace_bytes - (size_t)(part - ws);
  void* c_kv = kv;
  void* k_r = kv + (size_t)T * MLA_D_C * (f32 ? 4 : 2);
  const hipStream_t st = (hipStream_t)stream;
  // h [W^DQ; W^DKV; W^KR]^T in one product.  Split: one workgroup per token
  // then sums the partials into c^Q and the cache rows; otherwise the
  // product writes c^Q, c^KV, k^R and the cache write follows.
  const int splits = plan_linear(T, dcq + MLA_ROW, d, device_cus()).splits;
  Blocks b1;
  b1.add(w_dq, dcq, splits > 1 ? nullptr : cq, true);
  b1.add(w_dkv, MLA_D_C, splits > 1 ? nullptr : c_kv, !f32);
  b1.add(w_kr, MLA_D_R, splits > 1 ? nullptr : k_r, !f32);
  mla_status e = run_linear(h, b1, T, d, part, part_bytes, st);
  if (e != MLA_OK) return e;
  CacheWriteArgs a{c_kv, k_r, pos, slot, nullptr, 0, T, cache->rows, (uint8_t*)cache->ckv_fp8,
                   cache->ckv_scale, cache->kr, rope_table(r)};
  if (splits > 1) {
    a.part = (const float*)part;
    a.splits = splits;
    a.part_ld = dcq + MLA_ROW;
    a.part_col = dcq;
    a.cq = (bf16*)cq;
    a.cq_width = dcq;
  }
  e = launched(launch_cache_write(a, kind, st));
  if (e != MLA_OK) return e;
  const bool bf = out_dtype == MLA_BF16;
  Blocks b2;
  b2.add(w_uq, H * MLA_D_NOPE, q_c, bf);
  b2.add(w_qr, H * MLA_D_R, q_r, bf);
  return run_linear(cq, b2, T, dcq, part, part_bytes, st);
}

mla_status mla_output_proj(const void* x, const void* w, void* u, int32_t N, int32_t K, int32_t d, int32_t out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w || !u || !dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (!all_aligned16({x, w, u, workspace})) return MLA_ERR_INVALID_ARG;
  if (K % MLA_D_V != 0 || !linear_shape_ok(N, d, 0, K)) return MLA_ERR_INVALID_ARG;
  Blocks bl;
  bl.add(w, d, u, out_dtype == MLA_BF16);
  return run_linear(x, bl, N, K, (uint8_t*)workspace, workspace_bytes, (hipStream_t)stream);
}

mla_status mla_fold_wuv_wo(const void* w_uv, const void* w_o, void* w_fold, int32_t H, int32_t d, void* stream) {
  if (!w_uv || !w_o || !w_fold || H < 1 || H > MLA_MAX_HEADS || d < 1) return MLA_ERR_INVALID_ARG;
  if ((long long)d * H * MLA_D_C * 2 > kMaxOperandBytes * 2) return MLA_ERR_INVALID_ARG;
  return launched(launch_fold_wuv_wo((const bf16*)w_uv, (const bf16*)w_o, (bf16*)w_fold, H, d, (hipStream_t)stream));
}

}  // extern "C"
