// Paged cache pool (host side): capacity accounting, a 64-row block
// allocator with per-sequence block tables, the physical rows (slots) of a
// sequence's positions, and the copy descriptors a request's blocks need
// under the layer-major and block-major layouts.
//
// What the pages fix (Prime Inference write-up, "Making room for
// low-latency decode"): with each MLA row shrunk from 576 to 352 bytes and
// the indexer and other per-token state unchanged, one decoder's cache held
// about 1.09 M -> 1.63 M tokens at the same memory budget.  "Changing the
// layout to reduce fragmentation" (and the mo.ai.kr article's KV-transfer
// section): a block-major layout keeps one block's data from every layer
// together, so a request moves in fewer, larger copies; it uses 64-token
// blocks.
//
//   capacity   whole blocks: budget / (layers * block_rows * (row + other))
//   reserve    a sequence grows by whole blocks, each the lowest-numbered
//              free block (consecutive blocks on an unfragmented pool), all
//              or nothing
//   layouts    layer-major: region (layer l, block b) at (l * n_blocks + b)
//              * B; block-major: at (b * layers + l) * B; B = block_rows *
//              row bytes.  A descriptor is one maximal run of contiguous
//              bytes when the sequence's regions are visited in table order.
#include "../../include/mla_nvfp4.h"

#include <stdint.h>

#include <mutex>
#include <new>
#include <set>
#include <vector>

struct mla_pool {
  std::mutex mu;
  int64_t n_blocks = 0;
  int32_t layers = 0, row_bytes = 0, other_bytes = 0, block_rows = 0;
  int32_t max_seqs = 0, max_blocks = 0;
  std::set<int32_t> free_blocks;                 // ordered: the lowest is taken first
  std::vector<std::vector<int32_t>> tables;      // per sequence, in position order
};

namespace {

bool valid_seq(const mla_pool* p, int32_t seq) { return p && seq >= 0 && seq < p->max_seqs; }

}  // namespace

extern "C" {

int64_t mla_pool_capacity_blocks(int64_t budget_bytes, int32_t layers, int32_t row_bytes,
                                 int32_t other_bytes, int32_t block_rows) {
  if (budget_bytes < 0 || layers < 1 || row_bytes < 1 || other_bytes < 0 || block_rows < 1) return -1;
  const int64_t per_block = (int64_t)layers * block_rows * ((int64_t)row_bytes + other_bytes);
  return budget_bytes / per_block;
}

int mla_pool_create(int64_t budget_bytes, int32_t layers, int32_t row_bytes, int32_t other_bytes,
                    int32_t block_rows, int32_t max_seqs, int32_t max_blocks_per_seq, mla_pool** out) {
  if (!out) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  const int64_t n = mla_pool_capacity_blocks(budget_bytes, layers, row_bytes, other_bytes, block_rows);
  if (n < 0 || max_seqs < 1 || max_blocks_per_seq < 1) return MLA_ERR_INVALID_ARG;
  // block ids are int32 and physical rows (id * block_rows + offset) must fit in int32 too
  if (n > 0x7FFFFFFF / block_rows) return MLA_ERR_INVALID_ARG;
  mla_pool* p = new (std::nothrow) mla_pool;
  if (!p) return MLA_ERR_INVALID_ARG;
  try {
    p->n_blocks = n;
    p->layers = layers;
    p->row_bytes = row_bytes;
    p->other_bytes = other_bytes;
    p->block_rows = block_rows;
    p->max_seqs = max_seqs;
    p->max_blocks = max_blocks_per_seq;
    for (int64_t b = 0; b < n; ++b) p->free_blocks.insert(p->free_blocks.end(), (int32_t)b);
    p->tables.assign((size_t)max_seqs, {});
  } catch (...) {
    delete p;
    return MLA_ERR_INVALID_ARG;
  }
  *out = p;
  return MLA_OK;
}

void mla_pool_destroy(mla_pool* p) { delete p; }

int64_t mla_pool_num_blocks(mla_pool* p) {
  if (!p) return -1;
  return p->n_blocks;
}

int64_t mla_pool_free_blocks(mla_pool* p) {
  if (!p) return -1;
  std::lock_guard<std::mutex> lk(p->mu);
  return (int64_t)p->free_blocks.size();
}

int mla_pool_reserve(mla_pool* p, int32_t seq, int64_t tokens) {
  if (!valid_seq(p, seq) || tokens < 0) return MLA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(p->mu);
  std::vector<int32_t>& t = p->tables[(size_t)seq];
  const int64_t want = (tokens + p->block_rows - 1) / p->block_rows;
  const int64_t need = want - (int64_t)t.size();
  if (need <= 0) return MLA_OK;
  if (want > p->max_blocks || need > (int64_t)p->free_blocks.size()) return MLA_ERR_CAPACITY;
  try {
    t.reserve((size_t)want);
  } catch (...) {
    return MLA_ERR_CAPACITY;
  }
  for (int64_t i = 0; i < need; ++i) {
    t.push_back(*p->free_blocks.begin());
    p->free_blocks.erase(p->free_blocks.begin());
  }
  return MLA_OK;
}

int mla_pool_release(mla_pool* p, int32_t seq) {
  if (!valid_seq(p, seq)) return MLA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(p->mu);
  std::vector<int32_t>& t = p->tables[(size_t)seq];
  for (int32_t b : t) p->free_blocks.insert(b);
  t.clear();
  return MLA_OK;
}

int mla_pool_block_table(mla_pool* p, int32_t* table, int64_t stride) {
  if (!p || !table || stride < p->max_blocks) return MLA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(p->mu);
  for (int32_t s = 0; s < p->max_seqs; ++s) {
    const std::vector<int32_t>& t = p->tables[(size_t)s];
    int32_t* row = table + (int64_t)s * stride;
    for (int32_t j = 0; j < p->max_blocks; ++j) row[j] = j < (int32_t)t.size() ? t[(size_t)j] : -1;
  }
  return MLA_OK;
}

int mla_pool_slots(mla_pool* p, int32_t seq, int64_t first_pos, int64_t n, int64_t* slots) {
  if (!valid_seq(p, seq) || first_pos < 0 || n < 0 || (n > 0 && !slots)) return MLA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(p->mu);
  const std::vector<int32_t>& t = p->tables[(size_t)seq];
  if (first_pos + n > (int64_t)t.size() * p->block_rows) return MLA_ERR_INVALID_ARG;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t pos = first_pos + i;
    slots[i] = (int64_t)t[(size_t)(pos / p->block_rows)] * p->block_rows + pos % p->block_rows;
  }
  return MLA_OK;
}

int mla_pool_descriptors(mla_pool* p, int32_t seq, int32_t layout, int64_t* descriptors, int64_t* bytes) {
  if (!valid_seq(p, seq) || !descriptors || !bytes) return MLA_ERR_INVALID_ARG;
  if (layout != MLA_LAYOUT_LAYER_MAJOR && layout != MLA_LAYOUT_BLOCK_MAJOR) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(p->mu);
  const std::vector<int32_t>& t = p->tables[(size_t)seq];
  const int64_t region = (int64_t)p->block_rows * p->row_bytes;
  int64_t runs = 0, end = -1;
  auto visit = [&](int64_t start) {
    if (start != end) ++runs;
    end = start + region;
  };
  if (layout == MLA_LAYOUT_LAYER_MAJOR) {
    for (int32_t l = 0; l < p->layers; ++l)
      for (int32_t b : t) visit(((int64_t)l * p->n_blocks + b) * region);
  } else {
    for (int32_t b : t)
      for (int32_t l = 0; l < p->layers; ++l) visit(((int64_t)b * p->layers + l) * region);
  }
  *descriptors = runs;
  *bytes = (int64_t)t.size() * p->layers * region;
  return MLA_OK;
}

}  // extern "C"
