// The C ABI (declared in include/mla_nvfp4.h): argument checks on the host,
// then one launch on the caller's stream.  Every check happens before the
// first HIP call, so a bad call enqueues nothing; no C++ exception leaves
// this file.
#include "../../include/mla_nvfp4.h"
#include "mla_launch.h"

#include <math.h>

#include <atomic>
#include <mutex>

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// How many times a split polls for the other splits' arrival before it
// leaves its slice of the merge to the last arrival (see mla_sparse_decode_
// set_merge_polls).  Each poll is a short sleep and one agent-scope load,
// about a microsecond; 256 polls bound the wait to a few hundred.
std::atomic<int> g_merge_polls{256};

bool pow2_scale(float s) {
  if (!(s > 0.0f) || !isfinite(s)) return false;
  int e = 0;
  return frexpf(s, &e) == 0.5f && e >= -20 && e <= 20;
}

// A two-level row's per-tensor latent scale: positive, finite, with a finite
// non-zero fl32(6 g) (the encoder divides by it).
bool latent_scale_ok(float g) {
  if (!(g > 0.0f) || !isfinite(g)) return false;
  const float six_g = 6.0f * g;
  return isfinite(six_g) && six_g > 0.0f;
}

// Benchmark timing state of one host thread (see mla_kernel_timing).
struct Timing {
  bool enabled = false, recorded = false;
  int device = -1;
  hipEvent_t start = nullptr, stop = nullptr;
};

Timing& timing() {
  static thread_local Timing tm;
  return tm;
}

// Events for this launch if timing is on for the current device.
mla::KernelEvents timing_events() {
  Timing& tm = timing();
  int dev = -1;
  if (tm.enabled && hipGetDevice(&dev) == hipSuccess && dev == tm.device) return {tm.start, tm.stop};
  return {};
}

int launched(hipError_t e, const mla::KernelEvents& ev) {
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (ev.start) timing().recorded = true;
  return MLA_OK;
}

int head_groups(int32_t H) {
  if (H == 16 || H == 32) return 1;
  if (H == 64) return 2;
  if (H == 128) return 4;
  return 0;
}

int quantize_checks(const void* latent, int64_t ls, const void* rope, int64_t rs, int dtype,
                    int64_t n, const int64_t* slots, const uint8_t* cache, int64_t cache_rows) {
  if (dtype != MLA_F16 && dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (n < 0 || cache_rows < 0) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!latent || !rope || !slots || !cache) return MLA_ERR_INVALID_ARG;
  if (ls < MLA_LATENT_DIM || rs < MLA_ROPE_DIM || (ls % 8) || (rs % 8)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(latent) || !aligned16(rope) || !aligned16(cache)) return MLA_ERR_INVALID_ARG;
  if (n > (int64_t)0x7FFFFFFF * 8) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// Size of the allocation-free entry point's scratch array (see below): the
// arrival state (64 bytes) of up to kScratchCounters (token, head group)
// units, then the split partials.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kScratchCounters = MLA_NOALLOC_MAX_UNITS;  // (token, head group) units per call
constexpr size_t kScratchCounterBytes = kScratchCounters * 64;
static_assert(kScratchCounterBytes % 256 == 0, "partials stay 256-byte aligned");

// Shared body of the two decode entry points.  With static_layout the
// workspace is the library's own scratch array: the arrival counters sit at
// a fixed place (only the arrival protocol writes them, and every completed
// call leaves them at zero, so they stay zero between calls of any size)
// and the split partials follow them.  check_only stops after the argument
// checks.
int decode_call(const void* q, int q_dtype, int64_t num_tokens, int32_t num_heads,
                int64_t q_stride_t, int64_t q_stride_h, const uint8_t* cache, int cache_fmt,
                int64_t cache_rows, float kv_scale, const int32_t* indices, int32_t topk,
                int64_t idx_stride_t, const int32_t* block_table, int32_t block_size,
                int64_t bt_stride, int32_t bt_rows, int32_t bt_cols, const int32_t* token_seq,
                float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                int32_t num_splits, void* stream, bool static_layout, bool check_only = false) {
  if (q_dtype != MLA_F16 && q_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (cache_fmt != MLA_CACHE_NVFP4_352 && cache_fmt != MLA_CACHE_FP8_576) return MLA_ERR_UNSUPPORTED;
  const int G = head_groups(num_heads);
  if (G == 0) return MLA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || topk < 1 || topk > MLA_MAX_TOPK) return MLA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 64) return MLA_ERR_INVALID_ARG;
  if (cache_rows < 0 || cache_rows > 0x7FFFFFFF) return MLA_ERR_INVALID_ARG;
  if (!isfinite(sm_scale)) return MLA_ERR_INVALID_ARG;
  if (cache_fmt == MLA_CACHE_FP8_576 && !pow2_scale(kv_scale)) return MLA_ERR_INVALID_ARG;
  if (cache_fmt == MLA_CACHE_NVFP4_352 && !latent_scale_ok(kv_scale)) return MLA_ERR_INVALID_ARG;
  if (num_tokens == 0) return MLA_OK;
  if (!q || !cache || !indices || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(cache) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (q_stride_h < MLA_QK_DIM || (q_stride_h % 8) || (q_stride_t % 8) ||
      q_stride_t < (int64_t)num_heads * q_stride_h)
    return MLA_ERR_INVALID_ARG;
  if (idx_stride_t < topk) return MLA_ERR_INVALID_ARG;
  if (block_table) {
    if (!token_seq || block_size < 1 || bt_rows < 1 || bt_cols < 1 || bt_stride < bt_cols)
      return MLA_ERR_INVALID_ARG;
  }
  const int S = num_splits ? num_splits : mla::decode_auto_splits(num_tokens, num_heads, topk);
  // the grid (units rounded up to 8, times S workgroups of 256 threads)
  // must hold fewer than 2^32 work-items
  if ((num_tokens * G + 7) / 8 * 8 * S >= (int64_t)1 << 24) return MLA_ERR_INVALID_ARG;
  const int64_t tg = num_tokens * G;
  uint32_t* counters;
  float* part_lse;
  _Float16* part_o;
  if (static_layout) {
    if (tg > kScratchCounters) return MLA_ERR_WORKSPACE;
    const size_t parts = S > 1 ? mla::decode_workspace_bytes(num_tokens, num_heads, S) -
                                     mla::decode_workspace_bytes(num_tokens, num_heads, 1)
                               : 0;
    if (kScratchCounterBytes + parts > kScratchBytes) return MLA_ERR_WORKSPACE;
    if (check_only) return MLA_OK;
    counters = reinterpret_cast<uint32_t*>(workspace);
    part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kScratchCounterBytes);
  } else {
    const size_t need = mla::decode_workspace_bytes(num_tokens, num_heads, S);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
    if (check_only) return MLA_OK;
    const size_t ctr = ((size_t)tg * 64 + 255) & ~(size_t)255;
    counters = reinterpret_cast<uint32_t*>(workspace);
    part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + ctr);
  }
  const size_t pl = ((size_t)tg * S * 32 * sizeof(float) + 255) & ~(size_t)255;
  part_o = reinterpret_cast<_Float16*>(reinterpret_cast<char*>(part_lse) + pl);

  mla::DecodeParams p;
  p.q = q;
  p.q_st = q_stride_t;
  p.q_sh = q_stride_h;
  p.T = num_tokens;
  p.H = num_heads;
  p.G = G;
  p.cache = cache;
  p.cache_rows = cache_rows;
  p.kv_scale = cache_fmt == MLA_CACHE_FP8_576 ? kv_scale : 1.0f;
  p.lat_scale = cache_fmt == MLA_CACHE_NVFP4_352 ? kv_scale : 1.0f;
  p.inv_lat_scale = 1.0f / p.lat_scale;
  p.idx = indices;
  p.topk = topk;
  p.idx_st = idx_stride_t;
  p.bt = block_table;
  p.bs = block_table ? block_size : 1;
  p.bs_log2 = (p.bs & (p.bs - 1)) == 0 ? __builtin_ctz((unsigned)p.bs) : -1;
  p.bt_cols = block_table ? bt_cols : 0;
  p.bt_rows = block_table ? bt_rows : 0;
  p.bt_st = block_table ? bt_stride : 0;
  p.tok_seq = block_table ? token_seq : nullptr;
  p.sm_log2 = fabsf(sm_scale) * 1.4426950408889634f * p.kv_scale * p.lat_scale;
  p.q_neg = sm_scale < 0.0f;
  p.out = out;
  p.lse = lse;
  p.counters = counters;
  p.part_lse = part_lse;
  p.part_o = part_o;
  p.S = S;
  p.merge_polls = g_merge_polls.load(std::memory_order_relaxed);
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_decode(p, cache_fmt, q_dtype == MLA_BF16, (hipStream_t)stream, ev), ev);
}

// ---------------------------------------------------------------- static scratch
//
// The allocation-free decode entry point keeps its workspace in this array
// instead of one the caller allocates.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device may be used.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  int status = MLA_ERR_HIP;
};
constexpr int kMaxDevices = 64;
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array.  The first call on
// a device looks the address up (with that device current) and zero-fills
// the counter region with a kernel on the caller's stream, ahead of the
// caller's decode on that stream.
int static_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return;
    if (mla::launch_zero_u32(static_cast<uint32_t*>(p), kScratchCounterBytes / sizeof(uint32_t), stream) != hipSuccess)
      return;
    slot.ptr = p;
    slot.status = MLA_OK;
  });
  *ptr = slot.ptr;
  return slot.status;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported value";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_CAPACITY: return "not enough free blocks in the pool";
    default: return "unknown status";
  }
}

int mla_nvfp4_quantize_append(const void* latent, int64_t latent_row_stride, const void* rope,
                              int64_t rope_row_stride, int dtype, int64_t n,
                              const int64_t* slot_mapping, uint8_t* cache, int64_t cache_rows,
                              void* stream) {
  int st = quantize_checks(latent, latent_row_stride, rope, rope_row_stride, dtype, n, slot_mapping,
                           cache, cache_rows);
  if (st != MLA_OK || n == 0) return st;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_nvfp4_quantize(latent, latent_row_stride, rope, rope_row_stride,
                                             dtype == MLA_BF16, n, slot_mapping, cache, cache_rows,
                                             1.0f, (hipStream_t)stream, ev),
                  ev);
}

int mla_nvfp4_quantize_append_2level(const void* latent, int64_t latent_row_stride, const void* rope,
                                     int64_t rope_row_stride, int dtype, int64_t n,
                                     const int64_t* slot_mapping, uint8_t* cache, int64_t cache_rows,
                                     float global_scale, void* stream) {
  int st = quantize_checks(latent, latent_row_stride, rope, rope_row_stride, dtype, n, slot_mapping,
                           cache, cache_rows);
  if (st != MLA_OK) return st;
  if (!latent_scale_ok(global_scale)) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_nvfp4_quantize(latent, latent_row_stride, rope, rope_row_stride,
                                             dtype == MLA_BF16, n, slot_mapping, cache, cache_rows,
                                             global_scale, (hipStream_t)stream, ev),
                  ev);
}

int mla_fp8_quantize_append(const void* latent, int64_t latent_row_stride, const void* rope,
                            int64_t rope_row_stride, int dtype, int64_t n,
                            const int64_t* slot_mapping, uint8_t* cache, int64_t cache_rows,
                            float kv_scale, void* stream) {
  int st = quantize_checks(latent, latent_row_stride, rope, rope_row_stride, dtype, n, slot_mapping,
                           cache, cache_rows);
  if (st != MLA_OK) return st;
  if (!pow2_scale(kv_scale)) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_fp8_quantize(latent, latent_row_stride, rope, rope_row_stride,
                                           dtype == MLA_BF16, n, slot_mapping, cache, cache_rows,
                                           kv_scale, (hipStream_t)stream, ev),
                  ev);
}

int32_t mla_sparse_decode_num_splits(int64_t num_tokens, int32_t num_heads, int32_t topk) {
  if (num_tokens < 0 || head_groups(num_heads) == 0 || topk < 1 || topk > MLA_MAX_TOPK) return 0;
  return mla::decode_auto_splits(num_tokens, num_heads, topk);
}

size_t mla_sparse_decode_workspace_size(int64_t num_tokens, int32_t num_heads, int32_t topk,
                                        int32_t num_splits) {
  if (num_tokens < 0 || head_groups(num_heads) == 0 || topk < 1 || topk > MLA_MAX_TOPK) return 0;
  if (num_splits < 0 || num_splits > 64) return 0;
  const int S = num_splits ? num_splits : mla::decode_auto_splits(num_tokens, num_heads, topk);
  return mla::decode_workspace_bytes(num_tokens, num_heads, S);
}

int32_t mla_sparse_decode_set_merge_polls(int32_t polls) {
  if (polls < 0) return -1;
  return g_merge_polls.exchange(polls, std::memory_order_relaxed);
}

int mla_sparse_decode(const void* q, int q_dtype, int64_t num_tokens, int32_t num_heads,
                      int64_t q_stride_t, int64_t q_stride_h, const uint8_t* cache, int cache_fmt,
                      int64_t cache_rows, float kv_scale, const int32_t* indices, int32_t topk,
                      int64_t idx_stride_t, const int32_t* block_table, int32_t block_size,
                      int64_t bt_stride, int32_t bt_rows, int32_t bt_cols, const int32_t* token_seq,
                      float sm_scale,
                      void* out, float* lse, void* workspace, size_t workspace_bytes,
                      int32_t num_splits, void* stream) {
  return decode_call(q, q_dtype, num_tokens, num_heads, q_stride_t, q_stride_h, cache, cache_fmt,
                     cache_rows, kv_scale, indices, topk, idx_stride_t, block_table, block_size,
                     bt_stride, bt_rows, bt_cols, token_seq, sm_scale, out, lse, workspace,
                     workspace_bytes, num_splits, stream, false);
}

int mla_sparse_decode_noalloc(const void* q, int q_dtype, int64_t num_tokens, int32_t num_heads,
                              int64_t q_stride_t, int64_t q_stride_h, const uint8_t* cache,
                              int cache_fmt, int64_t cache_rows, float kv_scale,
                              const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                              const int32_t* block_table, int32_t block_size, int64_t bt_stride,
                              int32_t bt_rows, int32_t bt_cols, const int32_t* token_seq,
                              float sm_scale, void* out, float* lse, int32_t num_splits,
                              void* stream) {
  // argument errors are reported before the scratch is set up
  const int st = decode_call(q, q_dtype, num_tokens, num_heads, q_stride_t, q_stride_h, cache,
                             cache_fmt, cache_rows, kv_scale, indices, topk, idx_stride_t,
                             block_table, block_size, bt_stride, bt_rows, bt_cols, token_seq,
                             sm_scale, out, lse, nullptr, 0, num_splits, stream, true, true);
  if (st != MLA_OK || num_tokens == 0) return st;
  void* scratch_ptr = nullptr;
  const int s2 = static_scratch((hipStream_t)stream, &scratch_ptr);
  if (s2 != MLA_OK) return s2;
  return decode_call(q, q_dtype, num_tokens, num_heads, q_stride_t, q_stride_h, cache, cache_fmt,
                     cache_rows, kv_scale, indices, topk, idx_stride_t, block_table, block_size,
                     bt_stride, bt_rows, bt_cols, token_seq, sm_scale, out, lse, scratch_ptr,
                     kScratchBytes, num_splits, stream, true);
}

size_t mla_indexer_workspace_size(int64_t num_tokens, int32_t max_ctx) {
  if (num_tokens < 0 || max_ctx < 0) return 0;
  return mla::indexer_workspace_bytes(num_tokens, max_ctx);
}

int mla_indexer_topk(const uint8_t* q_idx, int64_t q_stride_t, const uint8_t* keys, int64_t key_rows,
                     int64_t num_tokens, const int32_t* ctx_len, int32_t max_ctx,
                     const int64_t* key_base, const int32_t* block_table, int32_t block_size,
                     int64_t bt_stride, int32_t bt_rows, int32_t bt_cols, const int32_t* token_seq,
                     int32_t topk, int32_t* out, int64_t out_stride_t, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (num_tokens < 0 || max_ctx < 0 || key_rows < 0 || topk < 1 || topk > MLA_MAX_TOPK)
    return MLA_ERR_INVALID_ARG;
  if (num_tokens == 0) return MLA_OK;
  if (!q_idx || !keys || !ctx_len || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned16(keys)) return MLA_ERR_INVALID_ARG;
  if (q_stride_t < MLA_INDEXER_DIM || (q_stride_t % 16) || out_stride_t < topk) return MLA_ERR_INVALID_ARG;
  if (block_table) {
    if (!token_seq || block_size < 1 || bt_rows < 1 || bt_cols < 1 || bt_stride < bt_cols)
      return MLA_ERR_INVALID_ARG;
  } else if (!key_base) {
    return MLA_ERR_INVALID_ARG;
  }
  const int64_t nchunks = ((int64_t)max_ctx + 1023) / 1024;   // score-kernel chunks (the finer grid)
  if (num_tokens * nchunks >= ((int64_t)1 << 31) || num_tokens >= ((int64_t)1 << 31)) return MLA_ERR_INVALID_ARG;
  const size_t need = mla::indexer_workspace_bytes(num_tokens, max_ctx);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  mla::IndexerParams p;
  p.q = q_idx;
  p.q_st = q_stride_t;
  p.keys = keys;
  p.key_rows = key_rows;
  p.T = num_tokens;
  p.ctx = ctx_len;
  p.max_ctx = max_ctx;
  p.key_stride = (max_ctx + 1) & ~1;
  p.base = block_table ? nullptr : key_base;
  p.bt = block_table;
  p.bs = block_table ? block_size : 1;
  p.bs_log2 = (p.bs & (p.bs - 1)) == 0 ? __builtin_ctz((unsigned)p.bs) : -1;
  p.bt_rows = block_table ? bt_rows : 0;
  p.bt_cols = block_table ? bt_cols : 0;
  p.bt_st = block_table ? bt_stride : 0;
  p.tok_seq = block_table ? token_seq : nullptr;
  p.topk = topk;
  p.out = out;
  p.out_st = out_stride_t;
  mla::indexer_workspace_layout(p, workspace, num_tokens, max_ctx);
  p.nchunks = 0;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_indexer(p, (hipStream_t)stream, ev), ev);
}

namespace {
// Region geometry of mla_kv_pack_blocks / mla_kv_unpack_blocks; false on bad sizes.
bool region_geometry(int32_t layout, int64_t pool_blocks, int32_t layers, int32_t block_rows,
                     int32_t row_bytes, int64_t n, int64_t* region, int64_t* bstride, int64_t* lstride) {
  if (layout != MLA_LAYOUT_LAYER_MAJOR && layout != MLA_LAYOUT_BLOCK_MAJOR) return false;
  if (pool_blocks < 0 || layers < 1 || block_rows < 1 || row_bytes < 1 || n < 0) return false;
  *region = (int64_t)block_rows * row_bytes;
  if (*region % 16) return false;
  if (n * layers >= ((int64_t)1 << 31)) return false;
  *bstride = layout == MLA_LAYOUT_LAYER_MAJOR ? *region : *region * layers;
  *lstride = layout == MLA_LAYOUT_LAYER_MAJOR ? *region * pool_blocks : *region;
  return true;
}
}  // namespace

int mla_kv_pack_blocks(const uint8_t* pool, int32_t layout, int64_t pool_blocks, int32_t layers,
                       int32_t block_rows, int32_t row_bytes, const int32_t* block_ids, int64_t n,
                       uint8_t* staging, void* stream) {
  int64_t region, bs, ls;
  if (!region_geometry(layout, pool_blocks, layers, block_rows, row_bytes, n, &region, &bs, &ls))
    return (layout != MLA_LAYOUT_LAYER_MAJOR && layout != MLA_LAYOUT_BLOCK_MAJOR) ? MLA_ERR_UNSUPPORTED
                                                                                  : MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!pool || !block_ids || !staging || !aligned16(pool) || !aligned16(staging)) return MLA_ERR_INVALID_ARG;
  mla::RegionCopy c;
  c.src = pool;
  c.src_block_stride = bs;
  c.src_layer_stride = ls;
  c.src_blocks = pool_blocks;
  c.src_ids = block_ids;
  c.dst = staging;
  c.dst_block_stride = region * layers;
  c.dst_layer_stride = region;
  c.dst_blocks = n;
  c.dst_ids = nullptr;
  c.n = n;
  c.layers = layers;
  c.region_bytes = region;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_region_copy(c, (hipStream_t)stream, ev), ev);
}

int mla_kv_unpack_blocks(const uint8_t* staging, int64_t n, const int32_t* block_ids, uint8_t* pool,
                         int32_t layout, int64_t pool_blocks, int32_t layers, int32_t block_rows,
                         int32_t row_bytes, void* stream) {
  int64_t region, bs, ls;
  if (!region_geometry(layout, pool_blocks, layers, block_rows, row_bytes, n, &region, &bs, &ls))
    return (layout != MLA_LAYOUT_LAYER_MAJOR && layout != MLA_LAYOUT_BLOCK_MAJOR) ? MLA_ERR_UNSUPPORTED
                                                                                  : MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!pool || !block_ids || !staging || !aligned16(pool) || !aligned16(staging)) return MLA_ERR_INVALID_ARG;
  mla::RegionCopy c;
  c.src = staging;
  c.src_block_stride = region * layers;
  c.src_layer_stride = region;
  c.src_blocks = n;
  c.src_ids = nullptr;
  c.dst = pool;
  c.dst_block_stride = bs;
  c.dst_layer_stride = ls;
  c.dst_blocks = pool_blocks;
  c.dst_ids = block_ids;
  c.n = n;
  c.layers = layers;
  c.region_bytes = region;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_region_copy(c, (hipStream_t)stream, ev), ev);
}

int mla_kernel_timing(int enable) {
  Timing& tm = timing();
  if (tm.enabled) {
    (void)hipEventDestroy(tm.start);
    (void)hipEventDestroy(tm.stop);
    tm = Timing{};
  }
  if (!enable) return MLA_OK;
  if (hipGetDevice(&tm.device) != hipSuccess) return MLA_ERR_HIP;
  if (hipEventCreate(&tm.start) != hipSuccess) return MLA_ERR_HIP;
  if (hipEventCreate(&tm.stop) != hipSuccess) {
    (void)hipEventDestroy(tm.start);
    tm = Timing{};
    return MLA_ERR_HIP;
  }
  tm.enabled = true;
  return MLA_OK;
}

int mla_last_kernel_ms(float* ms) {
  Timing& tm = timing();
  if (!ms || !tm.enabled || !tm.recorded) return MLA_ERR_INVALID_ARG;
  if (hipEventSynchronize(tm.stop) != hipSuccess) return MLA_ERR_HIP;
  return hipEventElapsedTime(ms, tm.start, tm.stop) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_nvfp4_gather_dequant_fp8(const uint8_t* cache, int64_t cache_rows, const int32_t* indices,
                                 int64_t num_tokens, int32_t topk, int64_t idx_stride_t,
                                 const int32_t* block_table, int32_t block_size, int64_t bt_stride,
                                 int32_t bt_rows, int32_t bt_cols, const int32_t* token_seq,
                                 float fp8_scale,
                                 uint8_t* fp8_rows, int32_t* staged_indices, void* stream) {
  if (num_tokens < 0 || topk < 1 || topk > MLA_MAX_TOPK || cache_rows < 0) return MLA_ERR_INVALID_ARG;
  if (!pow2_scale(fp8_scale)) return MLA_ERR_INVALID_ARG;
  if (num_tokens == 0) return MLA_OK;
  if (!cache || !indices || !fp8_rows || !staged_indices) return MLA_ERR_INVALID_ARG;
  if (!aligned16(cache) || !aligned16(fp8_rows)) return MLA_ERR_INVALID_ARG;
  if (idx_stride_t < topk) return MLA_ERR_INVALID_ARG;
  if (block_table && (!token_seq || block_size < 1 || bt_rows < 1 || bt_cols < 1 || bt_stride < bt_cols))
    return MLA_ERR_INVALID_ARG;
  if ((num_tokens * topk + 31) / 32 > 0x7FFFFFFF) return MLA_ERR_INVALID_ARG;
  mla::StagedParams p;
  p.cache = cache;
  p.cache_rows = cache_rows;
  p.idx = indices;
  p.T = num_tokens;
  p.topk = topk;
  p.idx_st = idx_stride_t;
  p.bt = block_table;
  p.bs = block_table ? block_size : 1;
  p.bs_log2 = (p.bs & (p.bs - 1)) == 0 ? __builtin_ctz((unsigned)p.bs) : -1;
  p.bt_cols = block_table ? bt_cols : 0;
  p.bt_rows = block_table ? bt_rows : 0;
  p.bt_st = block_table ? bt_stride : 0;
  p.tok_seq = block_table ? token_seq : nullptr;
  p.inv_scale = 1.0f / fp8_scale;
  p.rows = fp8_rows;
  p.sidx = staged_indices;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_gather_dequant_fp8(p, (hipStream_t)stream, ev), ev);
}

int mla_gather_probe(const uint8_t* cache, int64_t cache_rows, int32_t row_bytes, const int32_t* rows,
                     int64_t n, uint32_t* sink, void* stream) {
  if (cache_rows < 0 || n < 0 || row_bytes < 16 || row_bytes % 16) return MLA_ERR_INVALID_ARG;
  if (n >= ((int64_t)1 << 31)) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!cache || !rows || !sink || !aligned16(cache)) return MLA_ERR_INVALID_ARG;
  mla::GatherProbe g;
  g.cache = cache;
  g.cache_rows = cache_rows;
  g.row_bytes = row_bytes;
  g.pieces = row_bytes / 16;
  g.rows = rows;
  g.n = n;
  g.sink = sink;
  const mla::KernelEvents ev = timing_events();
  return launched(mla::launch_gather_probe(g, (hipStream_t)stream, ev), ev);
}

}  // extern "C"
