// Quantize-append kernels: fp16/bf16 rows -> 352-byte NVFP4 rows (and the
// 576-byte FP8 comparison rows).
//
// Format (Prime Inference write-up, "Making room for low-latency decode"):
// 512 latent values at four bits with one FP8 scale per 16 values, 64 rope
// values in FP8, 352 bytes per row.  One wave quantizes two rows: lane
// (row, g) owns latent group g (16 values), its scale byte, and rope values
// 2g and 2g+1, so every load and store of a row is contiguous across the
// row's 32 lanes.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

// Sixteen fp16 or bf16 values (two 16-byte words) as floats (exact), plus
// their sign bits.
template <bool kBf16>
__device__ __forceinline__ void unpack16(const u32x4& a, const u32x4& b, float (&v)[16], uint32_t& signs) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  signs = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (kBf16) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    } else {
      const half2_t h = as_half2(w[i]);
      v[2 * i] = (float)h.x;
      v[2 * i + 1] = (float)h.y;
    }
    signs |= ((w[i] >> 15) & 1u) << (2 * i);
    signs |= ((w[i] >> 31) & 1u) << (2 * i + 1);
  }
}

template <bool kBf16>
__device__ __forceinline__ void load16(const uint16_t* p, float (&v)[16], uint32_t& signs) {
  unpack16<kBf16>(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 8), v, signs);
}

template <bool kBf16>
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  if constexpr (kBf16) return __uint_as_float(bits << 16);
  else return (float)__builtin_bit_cast(half_t, (uint16_t)bits);
}

template <bool kBf16>
__device__ __forceinline__ float load_scalar(const uint16_t* p) {
  if constexpr (kBf16) return bf16_to_float(*p);
  else return (float)__builtin_bit_cast(half_t, *p);
}

// Two-level variant: gscale (g) is the per-tensor global scale of the latent
// (1 for one-level rows) and six_g = fl32(6 g).  The group scale is E4M3 of
// fl32(amax / six_g) and the code thresholds are fl32((t * s) * g), t * s
// being exact; with g = 1 every step is exact (the one-level encoding).
//
// Each row is assembled in LDS (nibbles, scales and rope from its 32 lanes)
// and written with 22 16-byte stores.
template <bool kBf16>
__global__ __launch_bounds__(256) void nvfp4_quantize_append_kernel(
    const uint16_t* __restrict__ latent, int64_t lat_stride, const uint16_t* __restrict__ rope,
    int64_t rope_stride, int64_t n, const int64_t* __restrict__ slots, uint8_t* __restrict__ cache,
    int64_t cache_rows, float gscale, float six_g) {
  __shared__ __align__(16) uint8_t rows_s[8][kRowBytes];
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int g = threadIdx.x & 31;
  if (row >= n) return;
  // The row's values and its slot are loaded together (one memory round
  // trip, not the slot's and then the values'); the tie keeps the compiler
  // from moving the value loads behind the slot test.
  const uint16_t* const lp = latent + row * lat_stride + 16 * g;
  const u32x4 la = *reinterpret_cast<const u32x4*>(lp);
  const u32x4 lb = *reinterpret_cast<const u32x4*>(lp + 8);
  const uint32_t rw = *reinterpret_cast<const uint32_t*>(rope + row * rope_stride + 2 * g);   // rope 2g, 2g+1
  const int64_t slot = slots[row];
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" :: "v"(la), "v"(lb), "v"(rw));
#endif
  if (slot < 0 || slot >= cache_rows) return;
  uint8_t* const stage = rows_s[threadIdx.x >> 5];

  float v[16];
  uint32_t signs;
  unpack16<kBf16>(la, lb, v, signs);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  // scale = E4M3(amax / 6) for one-level rows: the correctly rounded float32
  // quotient rounds to the same E4M3 value as the exact quotient (an
  // FP16/BF16 amax never puts it on or across an E4M3 rounding midpoint).
  const uint32_t sc = e4m3_mag_rne(__fdiv_rn(amax, six_g));
  const float s = e4m3_mag_value(sc);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t nib = e2m1_mag_scaled(__builtin_fabsf(v[i]), s, gscale) | (((signs >> i) & 1u) << 3);
    if (i < 8) lo |= nib << (4 * i);
    else hi |= nib << (4 * (i - 8));
  }
  *reinterpret_cast<u32x2*>(stage + 8 * g) = (u32x2){lo, hi};
  stage[kScaleOff + g] = (uint8_t)sc;
  const uint32_t r0 = e4m3_encode(half_bits_to_float<kBf16>(rw & 0xFFFFu));
  const uint32_t r1 = e4m3_encode(half_bits_to_float<kBf16>(rw >> 16));
  *reinterpret_cast<uint16_t*>(stage + kRopeOff + 2 * g) = (uint16_t)(r0 | (r1 << 8));
  // the row's 32 lanes belong to one wave, whose LDS operations complete in
  // order: a wave-level wait makes the staged row visible to its own lanes
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  if (g < kRowBytes / 16)
    *reinterpret_cast<u32x4*>(cache + slot * kRowBytes + 16 * g) = *reinterpret_cast<const u32x4*>(stage + 16 * g);
}

template <bool kBf16>
__global__ __launch_bounds__(256) void fp8_quantize_append_kernel(
    const uint16_t* __restrict__ latent, int64_t lat_stride, const uint16_t* __restrict__ rope,
    int64_t rope_stride, int64_t n, const int64_t* __restrict__ slots, uint8_t* __restrict__ cache,
    int64_t cache_rows, float inv_scale) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int g = threadIdx.x & 31;
  if (row >= n) return;
  const int64_t slot = slots[row];
  if (slot < 0 || slot >= cache_rows) return;
  float v[16];
  uint32_t signs;
  load16<kBf16>(latent + row * lat_stride + 16 * g, v, signs);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // inv_scale is a power of two, so v * inv_scale is the exact quotient
    uint32_t b = e4m3_mag_rne(__builtin_fabsf(v[i]) * inv_scale) | (((signs >> i) & 1u) << 7);
    w[i >> 2] |= b << (8 * (i & 3));
  }
  uint8_t* dst = cache + slot * kFp8RowBytes;
  *reinterpret_cast<u32x4*>(dst + 16 * g) = (u32x4){w[0], w[1], w[2], w[3]};
  const uint16_t* rp = rope + row * rope_stride + 2 * g;
  uint32_t r0 = e4m3_encode(load_scalar<kBf16>(rp) * inv_scale);
  uint32_t r1 = e4m3_encode(load_scalar<kBf16>(rp + 1) * inv_scale);
  *reinterpret_cast<uint16_t*>(dst + kLatent + 2 * g) = (uint16_t)(r0 | (r1 << 8));
}

hipError_t launch_nvfp4_quantize(const void* latent, int64_t ls, const void* rope, int64_t rs,
                                 bool bf16, int64_t n, const int64_t* slots, uint8_t* cache,
                                 int64_t cache_rows, float global_scale, hipStream_t stream,
                                 const KernelEvents& ev) {
  dim3 grid((unsigned)((n + 7) / 8)), block(256);
  const uint16_t* lat = (const uint16_t*)latent;
  const uint16_t* rp = (const uint16_t*)rope;
  float g = global_scale, six_g = 6.0f * global_scale;   // float32 product, rounded once
  void* args[] = {&lat, &ls, &rp, &rs, &n, &slots, &cache, &cache_rows, &g, &six_g};
  const void* fn = bf16 ? (const void*)nvfp4_quantize_append_kernel<true>
                        : (const void*)nvfp4_quantize_append_kernel<false>;
  return launch_kernel(fn, grid, block, args, stream, ev);
}

hipError_t launch_fp8_quantize(const void* latent, int64_t ls, const void* rope, int64_t rs,
                               bool bf16, int64_t n, const int64_t* slots, uint8_t* cache,
                               int64_t cache_rows, float kv_scale, hipStream_t stream,
                               const KernelEvents& ev) {
  dim3 grid((unsigned)((n + 7) / 8)), block(256);
  float inv = 1.0f / kv_scale;
  const uint16_t* lat = (const uint16_t*)latent;
  const uint16_t* rp = (const uint16_t*)rope;
  void* args[] = {&lat, &ls, &rp, &rs, &n, &slots, &cache, &cache_rows, &inv};
  const void* fn = bf16 ? (const void*)fp8_quantize_append_kernel<true>
                        : (const void*)fp8_quantize_append_kernel<false>;
  return launch_kernel(fn, grid, block, args, stream, ev);
}

}  // namespace mla
