// Staged comparator, step 1: unpack the selected NVFP4 rows into an FP8 row
// buffer in device memory (the path the native kernel replaces: the
// mo.ai.kr article's KV-cache section and the wireai.ir article's
// 4-bit-caches section describe it as an unpack into an FP8 temporary
// buffer ahead of the older FP8 attention kernel).
//
// One workgroup = 32 slots, 8 lanes per slot; each lane decodes an eighth
// of the row (64 latent values, 8 rope values) and writes its 72 FP8 bytes.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

__global__ __launch_bounds__(256) void gather_dequant_fp8_kernel(StagedParams p) {
  const int64_t slot = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const int64_t total = p.T * p.topk;
  if (slot >= total) return;
  const int64_t t = slot / p.topk;
  const int j = (int)(slot - t * p.topk);
  const int v = p.idx[t * p.idx_st + j];
  int64_t row = -1;
  if (v >= 0) {
    if (p.bt) {
      const int b = v / p.bs;
      const int64_t seq = p.tok_seq[t];
      if (b < p.bt_cols && seq >= 0 && seq < p.bt_rows) {
        const int pb = p.bt[seq * p.bt_st + b];
        if (pb >= 0) row = (int64_t)pb * p.bs + (v - b * p.bs);
      }
    } else {
      row = v;
    }
    if (row >= p.cache_rows) row = -1;
  }
  uint8_t* dst = p.rows + slot * kFp8RowBytes;
  if (part == 0) p.sidx[slot] = row >= 0 ? (int32_t)slot : -1;
  if (row < 0) {
    const u32x4 z = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(dst + 64 * part + 16 * k) = z;
    *reinterpret_cast<u32x2*>(dst + kLatent + 8 * part) = (u32x2){0, 0};
    return;
  }
  const uint8_t* src = p.cache + row * kRowBytes;
  const u32x4 l0 = *reinterpret_cast<const u32x4*>(src + 32 * part);
  const u32x4 l1 = *reinterpret_cast<const u32x4*>(src + 32 * part + 16);
  const uint32_t sc = *reinterpret_cast<const uint32_t*>(src + kScaleOff + 4 * part);
  const u32x2 rp = *reinterpret_cast<const u32x2*>(src + kRopeOff + 8 * part);
  const uint32_t w[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
  uint32_t o[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const half2_t s2 = e4m3_to_half2_splat(sc >> (8 * (k >> 1)));
    const half8_t s8 = (half8_t){s2.x, s2.y, s2.x, s2.y, s2.x, s2.y, s2.x, s2.y};
    const half8_t h = e2m1x8_to_half8(w[k]) * s8;   // exact decoded values
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= e4m3_encode((float)h[e] * p.inv_scale) << (8 * e);
      hi |= e4m3_encode((float)h[4 + e] * p.inv_scale) << (8 * e);
    }
    o[2 * k] = lo;
    o[2 * k + 1] = hi;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<u32x4*>(dst + 64 * part + 16 * k) =
        (u32x4){o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
  const half8_t r = e4m3x8_to_half8(rp.x, rp.y);
  uint32_t r0 = 0, r1 = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r0 |= e4m3_encode((float)r[e] * p.inv_scale) << (8 * e);
    r1 |= e4m3_encode((float)r[4 + e] * p.inv_scale) << (8 * e);
  }
  *reinterpret_cast<u32x2*>(dst + kLatent + 8 * part) = (u32x2){r0, r1};
}

hipError_t launch_gather_dequant_fp8(const StagedParams& p, hipStream_t stream, const KernelEvents& ev) {
  const int64_t total = p.T * p.topk;
  dim3 grid((unsigned)((total + 31) / 32)), block(256);
  void* args[] = {const_cast<StagedParams*>(&p)};
  return launch_kernel((const void*)gather_dequant_fp8_kernel, grid, block, args, stream, ev);
}

}  // namespace mla
