// Sparse MLA decode over a compressed cache, one launch (gfx950).
//
// What is computed (Prime Inference write-up, "A native NVFP4 sparse-MLA
// decode kernel"; wireai.ir article, 4-bit-caches section): every query
// token attends only to the rows its indexer selected; the selected rows
// are unpacked on chip; FP16 operands, FP32 softmax and accumulation; each
// token's rows are shared by several workgroups whose partial results are
// merged inside the same launch; the split count follows the token batch;
// padded slots of the fixed-width list are masked and cost nothing.
//
// Workgroup = (token t, head group g of 32 heads, split s), 4 waves.
//   prologue  load the token's index list, translate it through the block
//             table, drop masked / out-of-range slots and compact the valid
//             rows into LDS (so padded slots are never fetched and the
//             split boundaries balance valid rows, not slots); load q.
//   per tile  of 32 valid rows:
//             gather 352-byte rows (8 lanes per row, 16-byte loads, next
//             tile prefetched into registers) -> decode to FP16 in LDS;
//             scores S^T = K . Q^T with 16x16x32 FP16 MFMA, wave (rb, hb)
//             owning 16 rows x 16 heads; online softmax in FP32 (max shared
//             through LDS); P (FP16) to LDS; O += P . V with 32x32x16 FP16
//             MFMA, wave w owning output columns [128w, 128w+128).
//   epilogue  S == 1: normalise and store.  S > 1: store the normalised
//             partial (O/l, log2-sum-exp) in the workspace, wait until all S
//             splits of (t, g) have stored theirs (the launch is cooperative,
//             so they are co-resident), then each split merges 1/S of the
//             output columns.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

namespace {

constexpr int kTile = 32;             // valid rows per tile
constexpr int kHG = 32;               // heads per workgroup
constexpr int kThreads = 256;
constexpr int kKRow = kQK + 8;        // FP16 elements per LDS row of K (pad spreads banks)
constexpr int kPRow = kTile + 8;      // FP16 elements per LDS row of P
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

enum { kFmtNvfp4 = 0, kFmtFp8 = 1 };

// Raw bytes one lane fetches for its eighth of a row.
template <int kFmt>
struct Raw;
template <>
struct Raw<kFmtNvfp4> {
  u32x4 l0, l1;   // 32 latent bytes = 64 codes
  uint32_t sc;    // 4 group scales
  u32x2 rp;       // 8 rope bytes
};
template <>
struct Raw<kFmtFp8> {
  u32x4 l0, l1, l2, l3;  // 64 latent bytes
  u32x2 rp;              // 8 rope bytes
};

template <int kFmt>
__device__ __forceinline__ void fetch(Raw<kFmt>& r, const uint8_t* __restrict__ cache, int row,
                                      int part, bool valid) {
  if constexpr (kFmt == kFmtNvfp4) {
    if (valid) {
      const uint8_t* b = cache + (int64_t)row * kRowBytes;
      r.l0 = *reinterpret_cast<const u32x4*>(b + 32 * part);
      r.l1 = *reinterpret_cast<const u32x4*>(b + 32 * part + 16);
      r.sc = *reinterpret_cast<const uint32_t*>(b + kScaleOff + 4 * part);
      r.rp = *reinterpret_cast<const u32x2*>(b + kRopeOff + 8 * part);
    } else {
      r.l0 = r.l1 = (u32x4){0, 0, 0, 0};
      r.sc = 0;
      r.rp = (u32x2){0, 0};
    }
  } else {
    if (valid) {
      const uint8_t* b = cache + (int64_t)row * kFp8RowBytes;
      r.l0 = *reinterpret_cast<const u32x4*>(b + 64 * part);
      r.l1 = *reinterpret_cast<const u32x4*>(b + 64 * part + 16);
      r.l2 = *reinterpret_cast<const u32x4*>(b + 64 * part + 32);
      r.l3 = *reinterpret_cast<const u32x4*>(b + 64 * part + 48);
      r.rp = *reinterpret_cast<const u32x2*>(b + kLatent + 8 * part);
    } else {
      r.l0 = r.l1 = r.l2 = r.l3 = (u32x4){0, 0, 0, 0};
      r.rp = (u32x2){0, 0};
    }
  }
}

// Decode one lane's eighth of a row into its LDS row (latent cols
// [64*part, 64*part+64), rope cols [512+8*part, 512+8*part+8)).
template <int kFmt>
__device__ __forceinline__ void decode_to_lds(const Raw<kFmt>& r, half_t* dst, int part) {
  if constexpr (kFmt == kFmtNvfp4) {
    const uint32_t w[8] = {r.l0.x, r.l0.y, r.l0.z, r.l0.w, r.l1.x, r.l1.y, r.l1.z, r.l1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const half2_t s2 = e4m3_to_half2_splat(r.sc >> (8 * (k >> 1)));
      const half8_t s8 = (half8_t){s2.x, s2.y, s2.x, s2.y, s2.x, s2.y, s2.x, s2.y};
      *reinterpret_cast<half8_t*>(dst + 64 * part + 8 * k) = e2m1x8_to_half8(w[k]) * s8;
    }
  } else {
    const uint32_t w[16] = {r.l0.x, r.l0.y, r.l0.z, r.l0.w, r.l1.x, r.l1.y, r.l1.z, r.l1.w,
                            r.l2.x, r.l2.y, r.l2.z, r.l2.w, r.l3.x, r.l3.y, r.l3.z, r.l3.w};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      *reinterpret_cast<half8_t*>(dst + 64 * part + 8 * k) = e4m3x8_to_half8(w[2 * k], w[2 * k + 1]);
  }
  *reinterpret_cast<half8_t*>(dst + kLatent + 8 * part) = e4m3x8_to_half8(r.rp.x, r.rp.y);
}

template <bool kBf16>
__device__ __forceinline__ half8_t load_q8(const uint16_t* p) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
  if constexpr (!kBf16) {
    return __builtin_bit_cast(half8_t, u);
  } else {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    half8_t h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (half_t)__uint_as_float(w[i] << 16);
      h[2 * i + 1] = (half_t)__uint_as_float(w[i] & 0xFFFF0000u);
    }
    return h;
  }
}

template <bool kBf16>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
  if constexpr (kBf16) reinterpret_cast<uint16_t*>(out)[i] = float_to_bf16_rne(v);
  else reinterpret_cast<half_t*>(out)[i] = (half_t)v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

}  // namespace

template <int kFmt, bool kBf16>
__global__ __launch_bounds__(kThreads, 2) void sparse_decode_kernel(DecodeParams p) {
  __shared__ __align__(16) half_t kt[kTile * kKRow];
  __shared__ __align__(16) half_t pt[kHG * kPRow];
  __shared__ int phys[kMaxTopk];
  __shared__ float red_max[4][16];
  __shared__ float red_sum[4][16];
  __shared__ float m_run[2][kHG];
  __shared__ float alpha_s[kHG];
  __shared__ int cnt_s[8][4];
  __shared__ int flag_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = p.S, G = p.G;
  const int s = (int)(blockIdx.x % (unsigned)S);
  const int64_t tg = blockIdx.x / (unsigned)S;
  const int g = (int)(tg % G);
  const int64_t t = tg / G;

  // ---------------------------------------------------------------- q
  const int rb = wave & 1, hb = wave >> 1;
  half8_t qreg[kQK / 32];
  {
    const int head = g * kHG + hb * 16 + (lane & 15);
    if (head < p.H) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + t * p.q_st +
                           (int64_t)head * p.q_sh + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < kQK / 32; ++ks) qreg[ks] = load_q8<kBf16>(qp + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < kQK / 32; ++ks) qreg[ks] = (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  if (tid < kHG) m_run[0][tid] = kNegInf;

  // ------------------------------------------------ compact the valid rows
  int rows8[8], pre8[8];
  {
    const int32_t* ip = p.idx + t * p.idx_st;
    const int64_t seq = p.bt ? (int64_t)p.tok_seq[t] : 0;
    const bool seq_ok = !p.bt || (seq >= 0 && seq < p.bt_rows);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = i * kThreads + tid;
      int r = -1;
      if (slot < p.topk) {
        const int v = ip[slot];
        if (v >= 0 && seq_ok) {
          if (p.bt) {
            const int b = v / p.bs;
            if (b < p.bt_cols) {
              const int pb = p.bt[seq * p.bt_st + b];
              if (pb >= 0) {
                const int64_t pr = (int64_t)pb * p.bs + (v - b * p.bs);
                r = pr < p.cache_rows ? (int)pr : -1;
              }
            }
          } else {
            r = v < p.cache_rows ? v : -1;
          }
        }
      }
      rows8[i] = r;
      const uint64_t m = __ballot(r >= 0);
      pre8[i] = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) cnt_s[i][wave] = __popcll(m);
    }
  }
  __syncthreads();
  int total = 0;
  {
    int base[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      base[i] = total;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w < wave) base[i] += cnt_s[i][w];
        total += cnt_s[i][w];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (rows8[i] >= 0) phys[base[i] + pre8[i]] = rows8[i];
  }
  __syncthreads();

  const int r0 = (int)((int64_t)total * s / S);
  const int n = (int)((int64_t)total * (s + 1) / S) - r0;
  const int ntiles = (n + kTile - 1) / kTile;

  // ---------------------------------------------------------------- tiles
  const int gr = tid >> 3, gp = tid & 7;    // gather role: row in tile, eighth of the row
  float16_t acc_o[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc_o[nb][j] = 0.0f;
  float l_run[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) l_run[j] = 0.0f;

  Raw<kFmt> cur;
  fetch<kFmt>(cur, p.cache, gr < n ? phys[r0 + gr] : 0, gp, gr < n);

  for (int it = 0; it < ntiles; ++it) {
    Raw<kFmt> nxt;
    {
      const int rr = (it + 1) * kTile + gr;
      fetch<kFmt>(nxt, p.cache, rr < n ? phys[r0 + rr] : 0, gp, rr < n);
    }
    decode_to_lds<kFmt>(cur, kt + gr * kKRow, gp);
    __syncthreads();

    // scores: S^T[16 rows x 16 heads] for wave (rb, hb)
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    {
      const half_t* arow = kt + (16 * rb + (lane & 15)) * kKRow + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < kQK / 32; ++ks) {
        const half8_t a = *reinterpret_cast<const half8_t*>(arow + 32 * ks);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qreg[ks], acc, 0, 0, 0);
      }
    }
    float sv[4];
    float mx = kNegInf;
    const int row0 = it * kTile + 16 * rb + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = (row0 + j < n) ? acc[j] * p.sm_log2 : kNegInf;
      mx = __builtin_fmaxf(mx, sv[j]);
    }
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, 16));
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, 32));
    if (lane < 16) red_max[wave][lane] = mx;
    __syncthreads();
    {
      const int hl = hb * 16 + (lane & 15);
      const float m_old = m_run[it & 1][hl];
      const float tmax = __builtin_fmaxf(red_max[2 * hb][lane & 15], red_max[2 * hb + 1][lane & 15]);
      const float m_new = __builtin_fmaxf(m_old, tmax);
      float pj[4], psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pj[j] = exp2f(sv[j] - m_new);
        psum += pj[j];
      }
      psum += shfl_xor_f(psum, 16);
      psum += shfl_xor_f(psum, 32);
      if (lane < 16) red_sum[wave][lane] = psum;
      *reinterpret_cast<half4_t*>(pt + hl * kPRow + 16 * rb + 4 * (lane >> 4)) =
          (half4_t){(half_t)pj[0], (half_t)pj[1], (half_t)pj[2], (half_t)pj[3]};
      if (rb == 0 && lane < 16) {
        m_run[(it + 1) & 1][hl] = m_new;
        alpha_s[hl] = exp2f(m_old - m_new);
      }
    }
    __syncthreads();

    // values: O[32 heads x 128 cols of this wave] += P . V
    {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int hd = (j >> 2) * 8 + 4 * (lane >> 5) + (j & 3);
        const float al = alpha_s[hd];
        const float lt = red_sum[2 * (hd >> 4)][hd & 15] + red_sum[2 * (hd >> 4) + 1][hd & 15];
        l_run[j] = l_run[j] * al + lt;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc_o[nb][j] *= al;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const half8_t a =
            *reinterpret_cast<const half8_t*>(pt + (lane & 31) * kPRow + 16 * ks + 8 * (lane >> 5));
        const half_t* vbase = kt + (16 * ks + 8 * (lane >> 5)) * kKRow + 128 * wave + (lane & 31);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          half8_t b;
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = vbase[e * kKRow + 32 * nb];
          acc_o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc_o[nb], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    cur = nxt;
  }

  // ---------------------------------------------------------------- epilogue
  const float out_mul = p.kv_scale;  // FP8 rows: values carry kv_scale
  const int64_t H = p.H;
  if (S == 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hd = (j >> 2) * 8 + 4 * (lane >> 5) + (j & 3);
      const int head = g * kHG + hd;
      if (head >= p.H) continue;
      const float l = l_run[j];
      const float inv = l > 0.0f ? out_mul / l : 0.0f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = 128 * wave + 32 * nb + (lane & 31);
        store_out<kBf16>(p.out, (t * H + head) * kLatent + col, acc_o[nb][j] * inv);
      }
      if (wave == 0 && (lane & 31) == 0 && p.lse) {
        const float m = m_run[ntiles & 1][hd];
        p.lse[t * H + head] = l > 0.0f ? (m + __log2f(l)) * kLn2 : kNegInf;
      }
    }
    return;
  }

  // partial of this split: normalised O and log2-sum-exp
  {
    float* po = p.part_o + ((tg * S + s) * kHG) * kLatent;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hd = (j >> 2) * 8 + 4 * (lane >> 5) + (j & 3);
      const float l = l_run[j];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = 128 * wave + 32 * nb + (lane & 31);
        po[hd * kLatent + col] = acc_o[nb][j] * inv;
      }
      if (wave == 0 && (lane & 31) == 0) {
        const float m = m_run[ntiles & 1][hd];
        p.part_lse[(tg * S + s) * kHG + hd] = l > 0.0f ? m + __log2f(l) : kNegInf;
      }
    }
  }
  __threadfence();
  __syncthreads();
  uint32_t* ctr = p.counters + 2 * tg;
  if (tid == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    int ok = 1;
    while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)S) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        ok = 0;
        break;
      }
    }
    flag_s = ok;
  }
  __syncthreads();
  __threadfence();
  const bool ok = flag_s != 0;

  // merge weights per (split, head), reusing the K tile's LDS
  float* wsh = reinterpret_cast<float*>(kt);
  if (tid < kHG) {
    const float* pl = p.part_lse + tg * S * kHG + tid;
    float mx = kNegInf;
    for (int ss = 0; ss < S; ++ss) mx = __builtin_fmaxf(mx, pl[ss * kHG]);
    float sum = 0.0f;
    if (mx != kNegInf)
      for (int ss = 0; ss < S; ++ss) sum += exp2f(pl[ss * kHG] - mx);
    for (int ss = 0; ss < S; ++ss)
      wsh[ss * kHG + tid] = mx != kNegInf ? exp2f(pl[ss * kHG] - mx) / sum : 0.0f;
    const int head = g * kHG + tid;
    if (s == 0 && head < p.H && p.lse)
      p.lse[t * H + head] = ok ? (mx != kNegInf ? (mx + __log2f(sum)) * kLn2 : kNegInf)
                               : __builtin_nanf("");
  }
  __syncthreads();
  {
    const int c0 = kLatent * s / S, c1 = kLatent * (s + 1) / S, nc = c1 - c0;
    const float* po = p.part_o + (tg * S) * kHG * kLatent;
    for (int e = tid; e < kHG * nc; e += kThreads) {
      const int hd = e / nc, col = c0 + (e - hd * nc);
      const int head = g * kHG + hd;
      if (head >= p.H) continue;
      float a = 0.0f;
      for (int ss = 0; ss < S; ++ss) a += wsh[ss * kHG + hd] * po[(ss * kHG + hd) * kLatent + col];
      store_out<kBf16>(p.out, (t * H + head) * kLatent + col, ok ? a * out_mul : __builtin_nanf(""));
    }
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr + 1, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)S - 1u) {
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr + 1, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ host side

namespace {

struct DevInfo {
  int cus = 0;
  int per_cu = 0;  // co-resident decode workgroups per CU (smallest over instantiations)
};

DevInfo& dev_info() {
  static thread_local int cached_dev = -1;
  static thread_local DevInfo info;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev != cached_dev) {
    DevInfo d;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      d.cus = 0;
    int a = 0, b = 0, c = 0, e = 0;
    hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, sparse_decode_kernel<kFmtNvfp4, false>, kThreads, 0);
    hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, sparse_decode_kernel<kFmtNvfp4, true>, kThreads, 0);
    hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, sparse_decode_kernel<kFmtFp8, false>, kThreads, 0);
    hipOccupancyMaxActiveBlocksPerMultiprocessor(&e, sparse_decode_kernel<kFmtFp8, true>, kThreads, 0);
    int m = a;
    if (b < m) m = b;
    if (c < m) m = c;
    if (e < m) m = e;
    d.per_cu = m;
    info = d;
    cached_dev = dev;
  }
  return info;
}

}  // namespace

int decode_resident_capacity() {
  const DevInfo& d = dev_info();
  return d.cus * d.per_cu;
}

int decode_auto_splits(int64_t T, int H, int topk) {
  const int G = H <= kHG ? 1 : H / kHG;
  const int64_t groups = T * G;
  if (groups <= 0) return 1;
  const int cap = decode_resident_capacity();
  const int cus = dev_info().cus > 0 ? dev_info().cus : 256;
  // one workgroup per CU is the target; never split below 64 rows per split,
  // and stay within what can be co-resident (the merge waits on its peers)
  int64_t s = (cus + groups - 1) / groups;
  int64_t max_by_rows = topk / 64;
  if (max_by_rows < 1) max_by_rows = 1;
  if (s > max_by_rows) s = max_by_rows;
  if (s > 64) s = 64;
  if (cap > 0 && s * groups > cap) s = cap / groups;
  if (s < 1) s = 1;
  return (int)s;
}

size_t decode_workspace_bytes(int64_t T, int H, int S) {
  const int G = H <= kHG ? 1 : H / kHG;
  const int64_t tg = T * G;
  size_t ctr = (size_t)tg * 2 * sizeof(uint32_t);
  ctr = (ctr + 255) & ~(size_t)255;
  if (S <= 1) return ctr;
  size_t pl = (size_t)tg * S * kHG * sizeof(float);
  pl = (pl + 255) & ~(size_t)255;
  const size_t po = (size_t)tg * S * kHG * kLatent * sizeof(float);
  return ctr + pl + po;
}

hipError_t launch_decode(const DecodeParams& p, int fmt, bool bf16, hipStream_t stream) {
  const int64_t blocks = p.T * p.G * p.S;
  dim3 grid((unsigned)blocks), block(kThreads);
  void* args[] = {const_cast<DecodeParams*>(&p)};
  const void* fn;
  if (fmt == kFmtNvfp4)
    fn = bf16 ? (const void*)sparse_decode_kernel<kFmtNvfp4, true>
              : (const void*)sparse_decode_kernel<kFmtNvfp4, false>;
  else
    fn = bf16 ? (const void*)sparse_decode_kernel<kFmtFp8, true>
              : (const void*)sparse_decode_kernel<kFmtFp8, false>;
  if (p.S > 1) return hipLaunchCooperativeKernel(fn, grid, block, args, 0, stream);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace mla
