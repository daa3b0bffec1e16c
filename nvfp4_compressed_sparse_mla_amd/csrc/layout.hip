// A request's cache blocks between a pool and a contiguous staging buffer
// (gfx950), for the layer-major and block-major pool layouts.
//
// What the pages fix (Prime Inference write-up, "Changing the layout to
// reduce fragmentation"; mo.ai.kr article, KV-transfer section): KV moved
// between prefill and decode workers fragments into many small copies when
// each layer's blocks sit apart; a block-major layout keeps one block's data
// from every layer together (64-token blocks), so the same request moves in
// fewer, larger copies.
//
// The unit is a (layer, block) region: block_rows rows of row_bytes bytes.
// Layer-major pools hold region (l, b) at (l * n_blocks + b) * R, block-major
// pools at (b * layers + l) * R.  The staging buffer is block-major over the
// request's own blocks, [n][layers][R]: one contiguous range, one copy
// descriptor.  pack gathers the request's regions from the pool into the
// staging buffer, unpack scatters them back to (possibly other) block ids.
// One workgroup moves one region with 16-byte loads and stores.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

__global__ __launch_bounds__(256) void region_copy_kernel(RegionCopy c) {
  const int64_t i = blockIdx.x / (uint32_t)c.layers;
  const int l = (int)(blockIdx.x - (uint32_t)i * (uint32_t)c.layers);
  const int64_t sb = c.src_ids ? (int64_t)c.src_ids[i] : i;
  const int64_t db = c.dst_ids ? (int64_t)c.dst_ids[i] : i;
  // block ids outside the pool name no region: nothing is read or written
  if (sb < 0 || sb >= c.src_blocks || db < 0 || db >= c.dst_blocks) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(c.src + sb * c.src_block_stride + l * c.src_layer_stride);
  u32x4* d = reinterpret_cast<u32x4*>(c.dst + db * c.dst_block_stride + l * c.dst_layer_stride);
  const int64_t n16 = c.region_bytes / 16;
  for (int64_t k = threadIdx.x; k < n16; k += 256) d[k] = s[k];
}

hipError_t launch_region_copy(const RegionCopy& c, hipStream_t stream, const KernelEvents& ev) {
  RegionCopy a = c;
  void* args[] = {&a};
  return launch_kernel((const void*)region_copy_kernel, dim3((unsigned)(c.n * c.layers)), dim3(256), args,
                       stream, ev);
}

}  // namespace mla
