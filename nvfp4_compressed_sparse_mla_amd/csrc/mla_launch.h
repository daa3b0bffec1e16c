// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Optional benchmark events: when `start` is set the kernel is launched with
// hipExtLaunchKernel, which records start/stop at the kernel's own start and
// end on the stream.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

inline hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream,
                                const KernelEvents& ev) {
  if (ev.start || ev.stop) return hipExtLaunchKernel(fn, grid, block, args, 0, stream, ev.start, ev.stop, 0);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

struct DecodeParams {
  const void* q;
  int64_t q_st, q_sh;       // strides in elements
  int64_t T;
  int H, G;                 // heads, head groups of 32
  const uint8_t* cache;
  int64_t cache_rows;
  float kv_scale;           // FP8 rows: value = byte * kv_scale (1 for NVFP4)
  float lat_scale;          // NVFP4 rows: per-tensor scale g of the latent (1 for FP8 rows)
  float inv_lat_scale;      // fl32(1 / g)
  const int32_t* idx;
  int topk;
  int64_t idx_st;
  const int32_t* bt;        // optional block table
  int bs, bt_rows, bt_cols;
  int bs_log2;              // log2(bs) if bs is a power of two, else -1
  int64_t bt_st;
  const int32_t* tok_seq;
  float sm_log2;            // |sm_scale| * log2(e) * kv_scale * lat_scale (>= 0)
  int q_neg;                // sm_scale < 0: q is negated on load (exact), so sm_log2 >= 0
  void* out;
  float* lse;
  uint32_t* counters;       // [T*G] x 64 bytes: arrival state per (token, head group)
  float* part_lse;          // [T*G][S][32]
  _Float16* part_o;         // [T*G][S][32 x 512], in the order the kernel's lanes hold it
  int S;                    // splits per (token, head group)
  int merge_polls;          // polls of the arrival word before a split leaves its slice to the last arrival
  int xcd_shift;            // set by launch_decode: 3 = a unit's splits share an XCD, 0 = plain order
};

int decode_auto_splits(int64_t T, int H, int topk);
// n zero words at p, by a kernel on `stream` (no memset node in a captured graph)
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream);
size_t decode_workspace_bytes(int64_t T, int H, int S);

hipError_t launch_decode(const DecodeParams& p, int fmt, bool bf16, hipStream_t stream,
                         const KernelEvents& ev);

hipError_t launch_nvfp4_quantize(const void* latent, int64_t ls, const void* rope, int64_t rs,
                                 bool bf16, int64_t n, const int64_t* slots, uint8_t* cache,
                                 int64_t cache_rows, float global_scale, hipStream_t stream,
                                 const KernelEvents& ev);
hipError_t launch_fp8_quantize(const void* latent, int64_t ls, const void* rope, int64_t rs,
                               bool bf16, int64_t n, const int64_t* slots, uint8_t* cache,
                               int64_t cache_rows, float kv_scale, hipStream_t stream,
                               const KernelEvents& ev);

struct StagedParams {
  const uint8_t* cache;
  int64_t cache_rows;
  const int32_t* idx;
  int64_t T;
  int topk;
  int64_t idx_st;
  const int32_t* bt;
  int bs, bt_rows, bt_cols;
  int bs_log2;              // log2(bs) if bs is a power of two, else -1
  int64_t bt_st;
  const int32_t* tok_seq;
  float inv_scale;
  uint8_t* rows;
  int32_t* sidx;
};
hipError_t launch_gather_dequant_fp8(const StagedParams& p, hipStream_t stream, const KernelEvents& ev);

// Sparse indexer (indexer.hip)
constexpr int kIdxHistBits = 12;

struct IndexerParams {
  const uint8_t* q;         // [T, 128] E4M3 queries, row stride q_st bytes
  int64_t q_st;
  const uint8_t* keys;      // [key_rows, 128] E4M3 keys
  int64_t key_rows;
  int64_t T;
  const int32_t* ctx;       // [T] visible positions
  int max_ctx;              // bound on ctx (sizes the key workspace)
  int64_t key_stride;       // workspace keys per token (max_ctx rounded up to even)
  const int64_t* base;      // [T] first key row of each sequence (no block table)
  const int32_t* bt;        // optional block table
  int bs, bt_rows, bt_cols;
  int bs_log2;
  int64_t bt_st;
  const int32_t* tok_seq;
  int topk;
  int32_t* out;             // [T, topk], row stride out_st
  int64_t out_st;
  uint64_t* keys_ws;        // [T][key_stride] order-preserving score keys
  uint32_t* hist;           // [T][4096] histogram of the keys' top 12 bits (zero between calls)
  uint32_t* cand_n;         // [T] candidates found (zero between calls)
  uint64_t* cand_key;       // [T][key_stride] keys of the candidates (the k-th best key's bucket)
  uint32_t* cand_pos;       // [T][key_stride] their positions
  uint32_t* sel_bits;       // [T][word_stride] positions certainly selected, one bit each
  uint32_t* tie_bits;       // [T][word_stride] positions whose key equals the k-th best one
  int64_t word_stride;      // bitmap words per token
  int nchunks;              // set by launch_indexer: score chunks per token
  int cchunks;              // set by launch_indexer: compact chunks per token
};
size_t indexer_workspace_bytes(int64_t T, int max_ctx);
// the workspace's parts (the layout indexer_workspace_bytes sizes)
void indexer_workspace_layout(IndexerParams& p, void* ws, int64_t T, int max_ctx);

// Copies of (layer, block) regions (layout.hip): region l of entry i moves
// from src + sid * src_block_stride + l * src_layer_stride to the same form
// at dst, sid = src_ids[i] (or i if null), likewise for dst.
struct RegionCopy {
  const uint8_t* src;
  int64_t src_block_stride, src_layer_stride, src_blocks;
  const int32_t* src_ids;
  uint8_t* dst;
  int64_t dst_block_stride, dst_layer_stride, dst_blocks;
  const int32_t* dst_ids;
  int64_t n;                // entries
  int layers;
  int64_t region_bytes;     // a multiple of 16
};
hipError_t launch_region_copy(const RegionCopy& c, hipStream_t stream, const KernelEvents& ev);
hipError_t launch_indexer(const IndexerParams& p, hipStream_t stream, const KernelEvents& ev);

// Read-only gather of a row list (probe.hip; a measurement aid)
struct GatherProbe {
  const uint8_t* cache;
  int64_t cache_rows;
  int64_t row_bytes;        // a multiple of 16
  int64_t pieces;           // row_bytes / 16
  const int32_t* rows;      // [n] physical rows; entries outside [0, cache_rows) are skipped
  int64_t n;
  uint32_t* sink;           // one word, written only in a case that does not occur in practice
};
hipError_t launch_gather_probe(const GatherProbe& g, hipStream_t stream, const KernelEvents& ev);

}  // namespace mla
