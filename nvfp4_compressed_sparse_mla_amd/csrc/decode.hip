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
// Workgroup = (token t, head group g of 32 heads, split s), 4 waves; wave
// w = (rb, kh) with rb = w & 1 (which 16 rows of a 32-row tile) and
// kh = w >> 1 (which half of the 576 key dimensions).  Two workgroups fit
// on a CU (registers < 256 per lane, LDS < 80 KB), so one workgroup's
// synchronisation stalls overlap the other's work.
//
//   prologue  load the token's index list, translate it through the block
//             table, drop masked / out-of-range slots and compact the valid
//             rows into LDS (padded slots are never fetched; split
//             boundaries balance valid rows).  Load q into registers in the
//             score MFMA's B-operand layout.
//   raw ring  the selected rows of the next two 32-row tiles stream from
//             HBM straight into a 3-slot LDS ring (global_load_lds_dwordx4,
//             16 bytes per lane, consecutive lanes fill consecutive LDS
//             bytes, so a tile lands as 32 contiguous rows).  Each wave
//             counts its own DMA instructions and waits with an explicit
//             vmcnt for the oldest tile only; ring reads are inline ds_read
//             instructions so no compiler-inserted wait serialises the ring.
//   per tile
//     decode  lane (row, kh, kg) reads 44 bytes of its row from the ring:
//             32 B of nibbles, 4 scales, 8 rope bytes -- the 8 key
//             dimensions per K-step of the 16x16x32 MFMA's A operand (key
//             dimensions are assigned to lanes so each lane's bytes are
//             contiguous; q uses the same assignment).  Latent FP16 values
//             also go to an LDS V tile for the values.
//     scores  S^T[16 rows x 32 heads] over this wave's 288 dimensions;
//             the two dimension halves are summed through LDS, leaving wave
//             (rb, kh) with the full scores of rows rb x heads kh.
//     softmax online, FP32, base 2; running max shared through LDS.
//     values  O[32 heads x 128 cols of wave w] += P . V with 32x32x16
//             MFMA; V's B operand comes from LDS with ds_read_b64_tr_b16
//             (each lane gets 4 consecutive rows of one column per read).
//   epilogue  S == 1: normalise and store.  S > 1: store the normalised
//             partial (O/l as FP16, log2-sum-exp as FP32); the split that
//             finishes last for (t, g) (an atomic count) merges all S
//             partials.  Nothing waits on another workgroup, so no
//             co-residency is needed.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

namespace {

constexpr int kTile = 32;             // valid rows per tile
constexpr int kHG = 32;               // heads per workgroup
constexpr int kThreads = 256;
constexpr int kVRow = kLatent + 16;   // FP16 elements per LDS row of V (row stride = 8 banks mod 64)
constexpr int kPRow = kTile + 8;      // FP16 elements per LDS row of P
constexpr int kKSteps = 9;            // 288 dimensions per wave / 32
constexpr int kRing = 3;              // raw-tile slots in LDS
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

enum { kFmtNvfp4 = 0, kFmtFp8 = 1 };

template <int kFmt>
struct Fmt {
  static constexpr int kRowB = kFmt == kFmtNvfp4 ? kRowBytes : kFp8RowBytes;
  static constexpr int kPieces = kRowB / 16;          // 16-byte pieces per row
  static constexpr int kChunks = kTile * kPieces;     // per tile
  static constexpr int kInstr = kChunks / 64;         // DMA instructions per tile
  static_assert(kChunks % 64 == 0, "a tile must be whole DMA instructions");
  static constexpr int kSlotBytes = kChunks * 16;
};

constexpr int ring_slot_bytes(int fmt) {
  return kTile * (fmt == kFmtNvfp4 ? kRowBytes : kFp8RowBytes);
}

typedef __fp16 fp16x4_ld __attribute__((__vector_size__(4 * sizeof(__fp16))));

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// ds_read of ring bytes written by the DMA; the compiler does not see these
// as LDS reads, so it adds no vmcnt wait for the DMA (the kernel waits
// itself).  The results are valid after the lgkmcnt wait in ring_read.
// (Inline assembly with AMDGPU register constraints exists only in the
// device compilation pass; the host pass never runs device functions.)
// The same holds for the LDS DMA builtin, whose presence in a kernel
// template's body would otherwise keep the host pass from emitting the
// kernel's launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
#define MLA_DEVICE_ASM(...) asm volatile(__VA_ARGS__)
#define MLA_DMA16(src, lds) __builtin_amdgcn_global_load_lds((src), (lds), 16, 0, 0)
#else
#define MLA_DEVICE_ASM(...) __builtin_unreachable()
#define MLA_DMA16(src, lds) ((void)(src), (void)(lds))
#endif

__device__ __forceinline__ u32x4 ring_b128(uint32_t a) {
  u32x4 v;
  MLA_DEVICE_ASM("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ u32x2 ring_b64(uint32_t a) {
  u32x2 v;
  MLA_DEVICE_ASM("ds_read_b64 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ uint32_t ring_b32(uint32_t a) {
  uint32_t v;
  MLA_DEVICE_ASM("ds_read_b32 %0, %1" : "=v"(v) : "v"(a));
  return v;
}

// Raw bytes one lane reads from its row: the key dimensions
// [256kh + 64kg, +64) of the latent and [512 + 32kh + 8kg, +8) of the rope.
template <int kFmt>
struct Raw;
template <>
struct Raw<kFmtNvfp4> {
  u32x4 l0, l1;   // 32 bytes of nibbles = 64 codes
  uint32_t sc;    // the 4 group scales of those codes
  u32x2 rp;       // 8 rope bytes
};
template <>
struct Raw<kFmtFp8> {
  u32x4 l0, l1, l2, l3;  // 64 latent bytes
  u32x2 rp;              // 8 rope bytes
};

template <int kFmt>
__device__ __forceinline__ void ring_read(Raw<kFmt>& r, uint32_t row_base, int kh, int kg) {
  if constexpr (kFmt == kFmtNvfp4) {
    r.l0 = ring_b128(row_base + 128 * kh + 32 * kg);
    r.l1 = ring_b128(row_base + 128 * kh + 32 * kg + 16);
    r.sc = ring_b32(row_base + kScaleOff + 16 * kh + 4 * kg);
    r.rp = ring_b64(row_base + kRopeOff + 32 * kh + 8 * kg);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(r.l0), "+v"(r.l1), "+v"(r.sc), "+v"(r.rp));
  } else {
    r.l0 = ring_b128(row_base + 256 * kh + 64 * kg);
    r.l1 = ring_b128(row_base + 256 * kh + 64 * kg + 16);
    r.l2 = ring_b128(row_base + 256 * kh + 64 * kg + 32);
    r.l3 = ring_b128(row_base + 256 * kh + 64 * kg + 48);
    r.rp = ring_b64(row_base + kLatent + 32 * kh + 8 * kg);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(r.l0), "+v"(r.l1), "+v"(r.l2), "+v"(r.l3), "+v"(r.rp));
  }
}

// Latent K-step ks (0..7) of the lane's 64 dimensions, as FP16.
template <int kFmt>
__device__ __forceinline__ half8_t latent8(const Raw<kFmt>& r, int ks) {
  if constexpr (kFmt == kFmtNvfp4) {
    const uint32_t w = ks < 4 ? r.l0[ks] : r.l1[ks - 4];
    return e2m1x8_to_half8_hw(w) * e4m3_splat8_hw(r.sc >> (8 * (ks >> 1)));
  } else {
    const u32x4& v = ks < 2 ? r.l0 : ks < 4 ? r.l1 : ks < 6 ? r.l2 : r.l3;
    const int o = 2 * (ks & 1);
    return e4m3x8_to_half8_hw(v[o], v[o + 1]);
  }
}

template <bool kBf16>
__device__ __forceinline__ half8_t load_q8(const uint16_t* p) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
  if constexpr (!kBf16) {
    return __builtin_bit_cast(half8_t, u);
  } else {
    half8_t h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (half_t)__uint_as_float(u[i] << 16);
      h[2 * i + 1] = (half_t)__uint_as_float(u[i] & 0xFFFF0000u);
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

__device__ __forceinline__ half4_t ds_read_tr16(const half_t* p) {
  fp16x4_ld v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) fp16x4_ld*)(p));
  return __builtin_bit_cast(half4_t, v);
}

// Workgroup barrier for the tile loop.  Inside the loop waves exchange data
// only through LDS (and the DMA, which each wave waits for itself), so the
// barrier waits for this wave's LDS operations only.  __syncthreads() would
// also wait for every outstanding global/DMA operation (vmcnt(0)) and drain
// the ring.  The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

}  // namespace

template <int kFmt, bool kBf16>
__global__ __launch_bounds__(kThreads, 2) void sparse_decode_kernel(DecodeParams p) {
  using F = Fmt<kFmt>;
  __shared__ __align__(16) uint8_t ring[kRing][ring_slot_bytes(kFmt)];   // raw tiles (DMA target)
  static_assert(ring_slot_bytes(kFmt) == F::kSlotBytes, "ring slot size");
  __shared__ __align__(16) half_t vt[kTile * kVRow];              // V tile, FP16, row-major
  // The score halves exchanged between kh waves (written before barrier B,
  // read before barrier C) and P (written after barrier C, read after
  // barrier D, dead before the next tile's exchange) share one buffer.
  __shared__ __align__(16) uint8_t xbuf[2 * 2 * 64 * sizeof(float4_t)];
  float4_t(*sx)[2][64] = reinterpret_cast<float4_t(*)[2][64]>(xbuf);     // [rb][kh][lane]
  half_t* pt = reinterpret_cast<half_t*>(xbuf);                           // P, [head][row]
  static_assert(kHG * kPRow * sizeof(half_t) <= sizeof(xbuf), "P must fit the exchange buffer");
  __shared__ int phys[kMaxTopk];
  __shared__ float red_max[4][16];
  __shared__ float red_sum[4][16];
  __shared__ float m_run[2][kHG];
  __shared__ float alpha_s[kHG];
  __shared__ float l_s[kHG];
  __shared__ int chg_s[2];
  __shared__ int cnt_s[8][4];
  __shared__ int last_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = p.S, G = p.G;
  const int s = (int)(blockIdx.x % (unsigned)S);
  const int64_t tg = blockIdx.x / (unsigned)S;
  const int g = (int)(tg % G);
  const int64_t t = tg / G;
  const int rb = wave & 1, kh = wave >> 1;
  const int r16 = lane & 15, kg = lane >> 4;

  // ---------------------------------------------------------------- q
  // B operand of K-step ks for head block hb: q[head][d(ks)] with
  // d(ks < 8) = 256kh + 64kg + 8ks + [0,8) and d(8) = 512 + 32kh + 8kg + [0,8)
  half8_t qreg[2][kKSteps];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = g * kHG + hb * 16 + r16;
    if (head < p.H) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + t * p.q_st + (int64_t)head * p.q_sh;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qreg[hb][ks] = load_q8<kBf16>(qp + 256 * kh + 64 * kg + 8 * ks);
      qreg[hb][8] = load_q8<kBf16>(qp + kLatent + 32 * kh + 8 * kg);
    } else {
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qreg[hb][ks] = (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  if (tid < kHG) {
    m_run[0][tid] = kNegInf;
    l_s[tid] = 0.0f;
  }

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

  float16_t acc_o[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc_o[nb][j] = 0.0f;

  // ------------------------------------------------ raw ring (DMA)
  // Wave w issues the tile's DMA instructions w, w+4, w+8, ...: `mine` of them.
  constexpr int kMineHi = (F::kInstr + 3) / 4;
  const int mine = (F::kInstr + 3 - wave) / 4;
  // Issue tile `it` into ring slot `slot`: row indices past the split are
  // clamped to its last row (a real row; those slots are never used).
  auto issue = [&](int it, int slot) {
#pragma unroll
    for (int j = 0; j < kMineHi; ++j) {
      if (j < mine) {
        const int c = 64 * (wave + 4 * j) + lane;            // chunk = row * pieces + piece
        const int row = c / F::kPieces, piece = c - row * F::kPieces;
        int i = it * kTile + row;
        i = i < n ? i : n - 1;
        const uint8_t* src = p.cache + (int64_t)phys[r0 + i] * F::kRowB + 16 * piece;
        MLA_DMA16(src, &ring[slot][1024 * (wave + 4 * j)]);
      }
    }
  };
  // wait until this wave's DMA of the oldest of the three tiles in flight is done
  auto wait_oldest = [&]() {
    if (mine == kMineHi) wait_vmcnt<2 * kMineHi>();
    else wait_vmcnt<2 * (kMineHi - 1)>();
  };

  auto process = [&](int it) {
    const int slot = it % kRing;
    // ---- decode each K-step's operand just before its two MFMAs (partial
    // scores over this wave's 288 dimensions, both head blocks); the latent
    // also goes to LDS as FP16 for the values
    Raw<kFmt> raw;
    ring_read<kFmt>(raw, lds_off(&ring[slot][(16 * rb + r16) * F::kRowB]), kh, kg);
    half_t* vrow = vt + (16 * rb + r16) * kVRow + 256 * kh + 64 * kg;
    float4_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      half8_t kop;
      if (ks < 8) {
        kop = latent8<kFmt>(raw, ks);
        *reinterpret_cast<half8_t*>(vrow + 8 * ks) = kop;
      } else {
        kop = e4m3x8_to_half8_hw(raw.rp.x, raw.rp.y);
      }
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qreg[0][ks], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qreg[1][ks], acc[1], 0, 0, 0);
    }
    sx[rb][kh][lane] = kh ? acc[0] : acc[1];   // the partner's head block
    lds_barrier();
    const float4_t part = sx[rb][kh ^ 1][lane];
    const float4_t sc = (kh ? acc[1] : acc[0]) + part;

    // ---- scores of rows (rb) x heads (hb = kh): mask, scale, tile max
    float sv[4];
    float mx = kNegInf;
    const int row0 = it * kTile + 16 * rb + 4 * kg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = (row0 + j < n) ? sc[j] * p.sm_log2 : kNegInf;
      mx = __builtin_fmaxf(mx, sv[j]);
    }
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, 16));
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, 32));
    if (lane < 16) red_max[wave][lane] = mx;
    lds_barrier();
    {
      const int hl = kh * 16 + r16;
      const float m_old = m_run[it & 1][hl];
      const float tmax = __builtin_fmaxf(red_max[2 * kh][r16], red_max[2 * kh + 1][r16]);
      const float m_new = __builtin_fmaxf(m_old, tmax);
      float pj[4], psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pj[j] = __builtin_amdgcn_exp2f(sv[j] - m_new);
        psum += pj[j];
      }
      psum += shfl_xor_f(psum, 16);
      psum += shfl_xor_f(psum, 32);
      if (lane < 16) red_sum[wave][lane] = psum;
      *reinterpret_cast<half4_t*>(pt + hl * kPRow + 16 * rb + 4 * kg) =
          (half4_t){(half_t)pj[0], (half_t)pj[1], (half_t)pj[2], (half_t)pj[3]};
      if (rb == 0) {
        const bool changed = lane < 16 && m_new > m_old;
        const uint64_t any = __ballot(changed);
        if (lane < 16) {
          m_run[(it + 1) & 1][hl] = m_new;
          alpha_s[hl] = __builtin_amdgcn_exp2f(m_old - m_new);
        }
        if (lane == 0) chg_s[kh] = any != 0;
      }
    }
    lds_barrier();

    // ---- values: O[32 heads x 128 cols of this wave] += P . V
    if (tid < kHG)
      l_s[tid] = l_s[tid] * alpha_s[tid] + red_sum[2 * (tid >> 4)][tid & 15] +
                 red_sum[2 * (tid >> 4) + 1][tid & 15];
    if ((chg_s[0] | chg_s[1]) != 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float al = alpha_s[(j >> 2) * 8 + 4 * (lane >> 5) + (j & 3)];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc_o[nb][j] *= al;
      }
    }
    {
      const int grp = lane >> 4, sl = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const half8_t a =
            *reinterpret_cast<const half8_t*>(pt + (lane & 31) * kPRow + 16 * ks + 8 * (lane >> 5));
        const int vr = 16 * ks + 8 * (grp >> 1) + (sl >> 2);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const half_t* vp = vt + vr * kVRow + 128 * wave + 32 * nb + 16 * (grp & 1) + 4 * (sl & 3);
          const half4_t lo = ds_read_tr16(vp);
          const half4_t hi = ds_read_tr16(vp + 4 * kVRow);
          const half8_t b = (half8_t){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          acc_o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc_o[nb], 0, 0, 0);
        }
      }
    }
  };

  // ------------------------------------------------ tiles, 2 ahead in flight
  if (ntiles > 0) {
    issue(0, 0);
    issue(1, 1);
    for (int it = 0; it < ntiles; ++it) {
      // slot (it+2)%3 last held tile it-1, whose reads all precede the
      // barriers of tile it-1
      issue(it + 2, (it + 2) % kRing);
      wait_oldest();
      lds_barrier();   // tile `it` complete in LDS for every wave; V tile free
      process(it);
    }
  }
  wait_vmcnt<0>();       // no DMA may still be writing this workgroup's LDS at exit
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  const float out_mul = p.kv_scale;  // FP8 rows: values carry kv_scale
  const int64_t H = p.H;
  if (S == 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hd = (j >> 2) * 8 + 4 * (lane >> 5) + (j & 3);
      const int head = g * kHG + hd;
      if (head >= p.H) continue;
      const float l = l_s[hd];
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

  // partial of this split: normalised O (FP16) and log2-sum-exp (FP32)
  {
    half_t* po = p.part_o + ((tg * S + s) * kHG) * kLatent;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hd = (j >> 2) * 8 + 4 * (lane >> 5) + (j & 3);
      const float l = l_s[hd];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = 128 * wave + 32 * nb + (lane & 31);
        po[hd * kLatent + col] = (half_t)(acc_o[nb][j] * inv);
      }
      if (wave == 0 && (lane & 31) == 0) {
        const float m = m_run[ntiles & 1][hd];
        p.part_lse[(tg * S + s) * kHG + hd] = l > 0.0f ? m + __log2f(l) : kNegInf;
      }
    }
  }
  // publish the partial (one release after the barrier has ordered every
  // wave's stores before it) and count arrivals; the last arrival merges
  __syncthreads();
  uint32_t* ctr = p.counters + tg;
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == (uint32_t)S - 1u;
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    }
    last_s = last;
  }
  __syncthreads();
  if (!last_s) return;

  // merge weights per (split, head), in the V tile's LDS
  float* wsh = reinterpret_cast<float*>(vt);
  if (tid < kHG) {
    const float* pl = p.part_lse + tg * S * kHG + tid;
    float mx = kNegInf;
    for (int ss = 0; ss < S; ++ss) mx = __builtin_fmaxf(mx, pl[ss * kHG]);
    float sum = 0.0f;
    if (mx != kNegInf)
      for (int ss = 0; ss < S; ++ss) sum += __builtin_amdgcn_exp2f(pl[ss * kHG] - mx);
    for (int ss = 0; ss < S; ++ss)
      wsh[ss * kHG + tid] = mx != kNegInf ? __builtin_amdgcn_exp2f(pl[ss * kHG] - mx) / sum : 0.0f;
    const int head = g * kHG + tid;
    if (head < p.H && p.lse) p.lse[t * H + head] = mx != kNegInf ? (mx + __log2f(sum)) * kLn2 : kNegInf;
  }
  __syncthreads();
  {
    // 8 consecutive columns per work item: 32 heads x 64 chunks
    const half_t* po = p.part_o + (tg * S) * kHG * kLatent;
    for (int e = tid; e < kHG * (kLatent / 8); e += kThreads) {
      const int hd = e >> 6, c8 = 8 * (e & 63);
      const int head = g * kHG + hd;
      if (head >= p.H) continue;
      float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int ss = 0; ss < S; ++ss) {
        const float w = wsh[ss * kHG + hd];
        const half8_t v = *reinterpret_cast<const half8_t*>(po + (ss * kHG + hd) * kLatent + c8);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] += w * (float)v[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) store_out<kBf16>(p.out, (t * H + head) * kLatent + c8 + i, a[i] * out_mul);
    }
  }
}

// ------------------------------------------------------------------ host side

namespace {

int device_cus() {
  static thread_local int cached_dev = -1;
  static thread_local int cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev != cached_dev) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    cached_dev = dev;
  }
  return cus;
}

}  // namespace

int decode_auto_splits(int64_t T, int H, int topk) {
  const int G = H <= kHG ? 1 : H / kHG;
  const int64_t groups = T * G;
  if (groups <= 0) return 1;
  const int cus = device_cus() > 0 ? device_cus() : 256;
  // two workgroups per CU is the target; a split keeps at least 256 valid
  // rows (8 tiles) so its fixed costs (index compaction, q load, merge
  // share) stay small next to its streaming work
  int64_t s = (2 * cus + groups - 1) / groups;
  int64_t max_by_rows = topk / 256;
  if (max_by_rows < 1) max_by_rows = 1;
  if (s > max_by_rows) s = max_by_rows;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

size_t decode_workspace_bytes(int64_t T, int H, int S) {
  const int G = H <= kHG ? 1 : H / kHG;
  const int64_t tg = T * G;
  size_t ctr = (size_t)tg * sizeof(uint32_t);
  ctr = (ctr + 255) & ~(size_t)255;
  if (S <= 1) return ctr;
  size_t pl = (size_t)tg * S * kHG * sizeof(float);
  pl = (pl + 255) & ~(size_t)255;
  const size_t po = (size_t)tg * S * kHG * kLatent * sizeof(half_t);
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
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace mla
