// Read-only row gather (gfx950): the rate at which this GPU can fetch a
// given list of cache rows from HBM when nothing else is done with them.
//
// A measurement aid, not a step of the method.  The sparse decode reads
// 352-byte rows scattered over the pool; a row at a 16-byte-aligned offset
// touches three or four 128-byte lines, and rows a token selects rarely
// share lines, so the bytes HBM delivers exceed the bytes of the rows.  This
// kernel reads exactly the decode's rows (the same physical row list) and
// nothing else, so its rate is the ceiling the decode's gather can reach on
// this machine for that row set.
//
// Thread i of the grid-stride loop reads 16-byte piece i mod P of row
// list entry i / P (P = row_bytes / 16): consecutive lanes read consecutive
// pieces of a row.  Four loads are in flight per thread; the words are
// folded into one value that is stored only if it equals a fixed constant,
// which keeps every load without writing anything in practice.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

__global__ __launch_bounds__(256) void gather_probe_kernel(GatherProbe g) {
  const int64_t total = g.n * g.pieces;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const uint32_t pieces = (uint32_t)g.pieces;
  uint32_t acc = 0;
  auto piece = [&](int64_t i) -> u32x4 {
    const uint32_t e = (uint32_t)(i / pieces);        // total < 2^31 * pieces: fits
    const uint32_t pc = (uint32_t)(i - (int64_t)e * pieces);
    const int32_t r = g.rows[e];
    if (r < 0 || r >= g.cache_rows) return (u32x4){0, 0, 0, 0};
    return *reinterpret_cast<const u32x4*>(g.cache + (int64_t)r * g.row_bytes + 16 * pc);
  };
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < total; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = piece(i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < total; i += stride) {
    const u32x4 v = piece(i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x2545F491u) g.sink[0] = acc;
}

hipError_t launch_gather_probe(const GatherProbe& g, hipStream_t stream, const KernelEvents& ev) {
  GatherProbe a = g;
  const int64_t total = g.n * g.pieces;
  // about four pieces per thread, at most 8192 workgroups (32 per CU)
  int64_t blocks = (total + 1023) / 1024;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  void* args[] = {&a};
  return launch_kernel((const void*)gather_probe_kernel, dim3((unsigned)blocks), dim3(256), args, stream, ev);
}

}  // namespace mla
