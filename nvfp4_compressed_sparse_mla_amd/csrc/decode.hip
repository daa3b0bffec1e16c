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
// Workgroup = (token t, head group g of 32 heads, split s), 4 waves, one
// workgroup per CU.  Each wave is an independent attention stream over its
// own 16-row tiles (tiles w, w+4, w+8, ... of the split) with its own DMA
// ring, its own FP16 V buffer and its own online-softmax state for all 32
// heads and all 512 output columns, held in accumulation registers.  The
// tile loop has no barrier: a wave overlaps its own DMA (the next two
// tiles in flight) with its own MFMA and conversion work.  The four streams
// merge once, through LDS, at the end; splits merge through the workspace
// (the split that finishes last merges).
//
//   prologue  load the token's index list, translate it through the block
//             table, drop masked / out-of-range slots and compact the valid
//             rows into LDS (padded slots are never fetched; split
//             boundaries balance valid rows).  Each wave loads q for all 32
//             heads into registers in the score MFMA's B-operand layout.
//   per tile  (16 rows, one wave)
//     ring    global_load_lds_dwordx4 streams the tile's rows into one of
//             the wave's LDS slots two tiles ahead; the wave waits for its
//             oldest tile with an explicit vmcnt and reads the slot with
//             inline ds_read (no compiler-inserted drain).
//     decode  lane (row r = lane & 15, kg = lane >> 4) reads 88 bytes of row
//             r (NVFP4): 64 B of nibbles, their 8 scales and 16 rope bytes --
//             key dimensions [128kg, +128) of the latent and [512 + 16kg,
//             +16) of the rope, i.e. the lane's 8 dimensions of each of the
//             18 K-steps of a 16x16x32 MFMA A operand (q uses the same
//             assignment).  The latent FP16 values also go to the V buffer.
//     scores  S^T[16 rows x 32 heads]: 36 MFMAs (16x16x32, FP16 -> FP32).
//     softmax base 2 against a lazily raised reference max: the first tile
//             sets the reference, which then moves only when a score exceeds
//             it by more than 15 (one ballot decides), so P = 2^(s - ref) <=
//             2^15 stays inside FP16 (with its full 11-bit precision) and the
//             common tile needs no cross-lane max and no O rescale.  Row sums
//             accumulate per lane and are reduced once at the end.
//     values  O[32 heads x 512 cols] += P . V: 16 MFMAs (32x32x16).  Each
//             lane's P operand is 8 rows of one head: 4 of its own scores
//             and 4 from lane ^ 16.  V's B operand comes from the V buffer
//             through ds_read_b64_tr_b16.
//   epilogue  the four streams are weighted by 2^(m_w - M) / L and summed
//             through LDS; S == 1 stores the output, S > 1 stores the
//             normalised partial (FP16) and its log2-sum-exp, and the split
//             that finishes last for (t, g) merges all S partials.  Nothing
//             waits on another workgroup, so no co-residency is needed.
#include "mla_device.h"
#include "mla_launch.h"

#include <type_traits>

namespace mla {

namespace {

constexpr int kRowsT = 16;            // rows per tile (one wave)
constexpr int kHG = 32;               // heads per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// FP16 elements per V-buffer row: a 1072-byte stride puts the 16 rows one
// row-wise 16-byte write instruction touches in distinct banks
constexpr int kVRow = kLatent + 24;
constexpr int kKSteps = 18;           // 576 key dimensions / 32
constexpr float kLazy = 15.0f;        // P = 2^(s - reference) <= 2^15 stays inside FP16
constexpr float kMargin = 5.0f;       // a new reference sits 2^5 above the max that set it
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

enum { kFmtNvfp4 = 0, kFmtFp8 = 1 };

constexpr int row_bytes(int fmt) { return fmt == kFmtNvfp4 ? kRowBytes : kFp8RowBytes; }
// DMA instructions per tile: 4 pieces of 16 bytes of each of the 16 rows per instruction
constexpr int dma_instr(int fmt) { return (row_bytes(fmt) / 16 + 3) / 4; }
constexpr int slot_bytes(int fmt) { return dma_instr(fmt) * 1024; }
// NVFP4: 3 slots (two tiles in flight while one is decoded); FP8 rows are
// larger, so 2 slots and the refill is issued once a slot is in registers
constexpr int ring_depth(int fmt) { return fmt == kFmtNvfp4 ? 3 : 2; }
constexpr int kWaveRing = 18432;      // bytes of ring per wave (both formats)
static_assert(ring_depth(kFmtNvfp4) * slot_bytes(kFmtNvfp4) <= kWaveRing, "NVFP4 ring");
static_assert(ring_depth(kFmtFp8) * slot_bytes(kFmtFp8) <= kWaveRing, "FP8 ring");
// FP16 elements of V buffer per wave; the stream merge's exchange regions
// (36,352 bytes per stream) reuse two waves' buffers, hence the padding
constexpr int kWaveV = kRowsT * kVRow + 512;
// q of the workgroup's 32 heads is staged through the V buffers before the loop
static_assert(kHG * kQK * 2 <= kWaves * kWaveV * 2, "q staging area");

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// Ring reads are inline ds_read instructions: the compiler does not see them
// as LDS reads, so it adds no wait for the DMA (the kernel waits itself with
// vmcnt); their results are valid after the lgkmcnt wait in ring_read.
// Inline assembly with AMDGPU register constraints and the LDS DMA builtin
// exist only in the device compilation pass (the host pass never runs
// device code; the DMA builtin in a kernel template's body would also keep
// the host pass from emitting the kernel's launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
#define MLA_DEVICE_ASM(...) asm volatile(__VA_ARGS__)
// (the immediate offset is added to both the global and the LDS address)
#define MLA_DMA16(src, lds, off) __builtin_amdgcn_global_load_lds((src), (lds), 16, (off), 0)
#else
#define MLA_DEVICE_ASM(...) __builtin_unreachable()
#define MLA_DMA16(src, lds, off) ((void)(src), (void)(lds))
#endif

// f(integral_constant<int, J>) for J = I .. N-1
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int kOff = 0>
__device__ __forceinline__ u32x4 ring_b128(uint32_t a) {
  u32x4 v;
  MLA_DEVICE_ASM("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(kOff));
  return v;
}
__device__ __forceinline__ u32x2 ring_b64(uint32_t a) {
  u32x2 v;
  MLA_DEVICE_ASM("ds_read_b64 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ uint32_t lds_b32(uint32_t a) {
  uint32_t v;
  MLA_DEVICE_ASM("ds_read_b32 %0, %1" : "=v"(v) : "v"(a));
  return v;
}

// Ring slot layout (row-interleaved).  DMA instruction j of a tile moves
// 16-byte piece 4j + c of tile row r from lane 16c + r, and an LDS-DMA
// instruction writes its 64 lanes' pieces contiguously, so piece P of row r
// sits at 1024 (P >> 2) + 256 (P & 3) + 16 r: the 16 rows' copies of one
// piece are 256 contiguous bytes (no bank conflicts for the 16 lanes that
// read them), and a lane's DMA source for every instruction is one row
// address plus an immediate.
//
// The bytes lane (row, kg) reads from its row.
template <int kFmt>
struct Raw;
template <>
struct Raw<kFmtNvfp4> {
  u32x4 l[4];     // 64 bytes of nibbles: latent dimensions [128kg, +128) (pieces 4kg + c)
  u32x2 sc;       // their 8 group scales (piece 16 + (kg >> 1), half kg & 1)
  u32x4 rp;       // rope dimensions [16kg, +16) (piece 18 + kg)
};
template <>
struct Raw<kFmtFp8> {
  u32x4 l[8];     // 128 latent bytes (pieces 8kg + c)
  u32x4 rp;       // 16 rope bytes (piece 32 + kg)
};

// Per-lane ring offsets (within a slot) of the lane's pieces.
template <int kFmt>
struct RingOff {
  uint32_t lat, sc, rope;
  __device__ explicit RingOff(int r16, int kg) {
    if constexpr (kFmt == kFmtNvfp4) {
      lat = 1024 * kg + 16 * r16;
      sc = 4096 + 256 * (kg >> 1) + 16 * r16 + 8 * (kg & 1);
      rope = 4608 + 256 * kg + 16 * r16;
    } else {
      lat = 2048 * kg + 16 * r16;
      sc = 0;
      rope = 8192 + 256 * kg + 16 * r16;
    }
  }
};

// The row bytes are read in two parts so that the second half of the
// latent (K-steps 8..15) occupies registers only from when it is decoded:
// part A = latent K-steps 0..7, scales and rope; part B = latent K-steps
// 8..15.  Each part waits for its own reads (and part A for `extra`, an LDS
// read issued just before it).
template <int kFmt>
__device__ __forceinline__ void ring_read_a(Raw<kFmt>& r, uint32_t slot, const RingOff<kFmt>& o,
                                            uint32_t& extra) {
  if constexpr (kFmt == kFmtNvfp4) {
    r.l[0] = ring_b128<0>(slot + o.lat);
    r.l[1] = ring_b128<256>(slot + o.lat);
    r.sc = ring_b64(slot + o.sc);
    r.rp = ring_b128(slot + o.rope);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(r.l[0]), "+v"(r.l[1]), "+v"(r.sc), "+v"(r.rp), "+v"(extra));
  } else {
    r.l[0] = ring_b128<0>(slot + o.lat);
    r.l[1] = ring_b128<256>(slot + o.lat);
    r.l[2] = ring_b128<512>(slot + o.lat);
    r.l[3] = ring_b128<768>(slot + o.lat);
    r.rp = ring_b128(slot + o.rope);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)"
                   : "+v"(r.l[0]), "+v"(r.l[1]), "+v"(r.l[2]), "+v"(r.l[3]), "+v"(r.rp), "+v"(extra));
  }
}

// part B issued without a wait (the caller's next lgkmcnt(0) wait covers it
// and names these registers).  FP8 rows carry twice the latent bytes: their
// part B is read in two halves, the second (K-steps 12..15) one value group
// later (ring_issue_b2), so that fewer row registers are live at once.
template <int kFmt>
__device__ __forceinline__ void ring_issue_b(Raw<kFmt>& r, uint32_t slot, const RingOff<kFmt>& o) {
  if constexpr (kFmt == kFmtNvfp4) {
    r.l[2] = ring_b128<512>(slot + o.lat);
    r.l[3] = ring_b128<768>(slot + o.lat);
  } else {
    r.l[4] = ring_b128<1024>(slot + o.lat);
    r.l[5] = ring_b128<1280>(slot + o.lat);
  }
}
template <int kFmt>
__device__ __forceinline__ void ring_issue_b2(Raw<kFmt>& r, uint32_t slot, const RingOff<kFmt>& o) {
  if constexpr (kFmt == kFmtFp8) {
    r.l[6] = ring_b128<1536>(slot + o.lat);
    r.l[7] = ring_b128<1792>(slot + o.lat);
  }
}
template <int kFmt>
__device__ __forceinline__ void lgkm_wait_b(u32x4 (&b)[4], Raw<kFmt>& r) {
  if constexpr (kFmt == kFmtNvfp4)
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(4)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(r.l[2]), "+v"(r.l[3]));
  else
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(4)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(r.l[4]), "+v"(r.l[5]));
}
// value group 2's wait: FP8 rows' second half of part B (issued during group
// 1, ahead of that group's four V-buffer writes) is complete as well
template <int kFmt>
__device__ __forceinline__ void lgkm_wait4_b2(u32x4 (&b)[4], Raw<kFmt>& r) {
  if constexpr (kFmt == kFmtNvfp4)
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(4)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
  else
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(4)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(r.l[6]), "+v"(r.l[7]));
}

template <int kFmt>
__device__ __forceinline__ void ring_read_b(Raw<kFmt>& r, uint32_t slot, const RingOff<kFmt>& o) {
  if constexpr (kFmt == kFmtNvfp4) {
    r.l[2] = ring_b128<512>(slot + o.lat);
    r.l[3] = ring_b128<768>(slot + o.lat);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(r.l[2]), "+v"(r.l[3]));
  } else {
    r.l[4] = ring_b128<1024>(slot + o.lat);
    r.l[5] = ring_b128<1280>(slot + o.lat);
    r.l[6] = ring_b128<1536>(slot + o.lat);
    r.l[7] = ring_b128<1792>(slot + o.lat);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(r.l[4]), "+v"(r.l[5]), "+v"(r.l[6]), "+v"(r.l[7]));
  }
}

// A operand of K-step ks: the lane's 8 key dimensions of its row, FP16.
template <int kFmt>
__device__ __forceinline__ half8_t kstep8(const Raw<kFmt>& r, int ks) {
  if constexpr (kFmt == kFmtNvfp4) {
    if (ks < 16) {
      const uint32_t w = r.l[ks >> 2][ks & 3];
      return e2m1x8_to_half8_hw(w) * e4m3_splat8_hw(r.sc[ks >> 3] >> (8 * ((ks >> 1) & 3)));
    }
    const int o = 2 * (ks - 16);
    return e4m3x8_to_half8_hw(r.rp[o], r.rp[o + 1]);
  } else {
    if (ks < 16) {
      const int o = 2 * (ks & 1);
      return e4m3x8_to_half8_hw(r.l[ks >> 1][o], r.l[ks >> 1][o + 1]);
    }
    const int o = 2 * (ks - 16);
    return e4m3x8_to_half8_hw(r.rp[o], r.rp[o + 1]);
  }
}

// A latent K-step's A operand decoded in two parts so that the conversion
// work can be placed between MFMAs: part 1 = the conversions and half of
// the scale multiplies, part 2 = the rest.  `sh` holds the lane's 8 group
// scales as FP16 (group g = half g & 1 of sh[g >> 1]).
struct KDec {
  half2_t c[4];
};
template <int kFmt>
__device__ __forceinline__ void kdec_part1(KDec& d, const Raw<kFmt>& r, const half2_t (&sh)[4], int ks) {
  if constexpr (kFmt == kFmtNvfp4) {
    const uint32_t w = r.l[ks >> 2][ks & 3];
    const half2_t s2 = sh[ks >> 2];
    const half_t sv = ((ks >> 1) & 1) ? s2.y : s2.x;
    const half2_t s = {sv, sv};
    d.c[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
    d.c[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
    d.c[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
    d.c[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
    d.c[0] *= s;
    d.c[1] *= s;
  } else {
    const uint32_t w = r.l[ks >> 1][2 * (ks & 1)];
    d.c[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    d.c[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
}
template <int kFmt>
__device__ __forceinline__ half8_t kdec_part2(KDec& d, const Raw<kFmt>& r, const half2_t (&sh)[4], int ks) {
  if constexpr (kFmt == kFmtNvfp4) {
    const half2_t s2 = sh[ks >> 2];
    const half_t sv = ((ks >> 1) & 1) ? s2.y : s2.x;
    const half2_t s = {sv, sv};
    d.c[2] *= s;
    d.c[3] *= s;
  } else {
    const uint32_t w = r.l[ks >> 1][2 * (ks & 1) + 1];
    d.c[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    d.c[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  return (half8_t){d.c[0].x, d.c[0].y, d.c[1].x, d.c[1].y, d.c[2].x, d.c[2].y, d.c[3].x, d.c[3].y};
}
// the lane's 8 NVFP4 group scales as FP16 pairs
__device__ __forceinline__ void group_scales(half2_t (&sh)[4], const u32x2& sc) {
  sh[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[0], 1.0f, false));
  sh[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[0], 1.0f, true));
  sh[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[1], 1.0f, false));
  sh[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[1], 1.0f, true));
}

// Eight q elements (fp16 or bf16 bits) as the FP16 score operand: fp16 is
// taken as is, bf16 is rounded to FP16.
template <bool kBf16>
__device__ __forceinline__ u32x4 q8_operand(const u32x4& u) {
  if constexpr (!kBf16) {
    return u;
  } else {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = as_u32((half2_t){(half_t)__uint_as_float(u[i] << 16), (half_t)__uint_as_float(u[i] & 0xFFFF0000u)});
    return r;
  }
}

// eight consecutive output elements (16-byte aligned), fp16 or bf16
template <bool kBf16, typename T>
__device__ __forceinline__ void store8(T* dst, const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kBf16) {
      w[i] = (uint32_t)float_to_bf16_rne(v[2 * i]) | ((uint32_t)float_to_bf16_rne(v[2 * i + 1]) << 16);
    } else {
      w[i] = as_u32((half2_t){(half_t)v[2 * i], (half_t)v[2 * i + 1]});
    }
  }
  *reinterpret_cast<u32x4*>(dst) = w;
}

// Split partials cross workgroups (and L2 caches): they are written with
// the agent-scope cache policy (sc1, what an agent-scope atomic store
// uses), which writes through this XCD's L2, so the writer needs no
// L2-wide writeback before counting its arrival.  One 16-byte store; in
// assembly, so the caller waits for it itself (s_waitcnt vmcnt(0) right
// after its last store).
__device__ __forceinline__ void store8_agent(half_t* dst, const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = as_u32((half2_t){(half_t)v[2 * i], (half_t)v[2 * i + 1]});
  MLA_DEVICE_ASM("global_store_dwordx4 %0, %1, off sc1" :: "v"(dst), "v"(w) : "memory");
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int m) {
  return (uint32_t)__shfl_xor((int)v, m, 64);
}

// B operands of the 4 value MFMAs of column group q (32-column blocks q,
// q+4, q+8, q+12) from the V buffer: ds_read_b64_tr_b16 gives each lane 4
// consecutive rows of one column; two reads (rows 0-3 and 4-7 of the lane's
// 8) make one operand.  In assembly so that the compiler does not make them
// wait for the ring's DMA; the memory clobber keeps the V-buffer writes that
// follow in program order from moving above them.
template <int kQ>
__device__ __forceinline__ void read_v4_group(u32x4 (&b)[4], uint32_t base) {
  static_for<0, 4>([&](auto E) {
    constexpr int e = decltype(E)::value;
    constexpr int off = 64 * (kQ + 4 * e);
    u32x2 lo, hi;
    MLA_DEVICE_ASM("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(base), "i"(off) : "memory");
    MLA_DEVICE_ASM("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(base), "i"(off + 8 * kVRow) : "memory");
    b[e] = (u32x4){lo.x, lo.y, hi.x, hi.y};
  });
}

__device__ __forceinline__ void lgkm_wait(u32x4 (&b)[4]) {
  MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}
// the same, leaving the wave's last four LDS operations (V-buffer writes
// issued after these reads) in flight: a wave's LDS operations complete in
// issue order
__device__ __forceinline__ void lgkm_wait4(u32x4 (&b)[4]) {
  MLA_DEVICE_ASM("s_waitcnt lgkmcnt(4)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its outstanding global loads (__syncthreads() would also wait for
// those, e.g. the q loads still in flight during the prologue).  The memory
// clobber keeps the compiler from moving memory accesses across it.
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

// x * a for an accumulator element that lives in an AGPR.  Written in C++
// the multiply makes the compiler move all 256 accumulators through VGPRs
// (and spill); in assembly the element is read, scaled and written back in
// place.
__device__ __forceinline__ float scale_acc(float x, float a) {
  float tmp;
  MLA_DEVICE_ASM("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp) : "v"(a));
  (void)tmp;
  return x;
}

// max of four MFMA results (v_max3; the compiler's fmaxf would first
// canonicalise each input with another v_max)
__device__ __forceinline__ float max4(float a, float b, float c, float d) {
  float m;
  MLA_DEVICE_ASM("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4" : "=&v"(m) : "v"(a), "v"(b), "v"(c), "v"(d));
  return m;
}

// The two score MFMAs of a K-step (16x16x32, FP16 -> FP32), in assembly so
// that their accumulators are VGPRs: the compiler gives every MFMA of the
// kernel an AGPR accumulator, and the 256 AGPRs already hold O.  Hazards are
// handled here: two wait states after the VALU write of the A operand
// (the first instruction), accumulation chains back to back (the hardware
// forwards a same-size accumulator), the first K-step of a tile starts from
// the constant 0, and score_mfma_drain() waits out the MFMA latency before
// VALU reads the scores.
__device__ __forceinline__ void score_mfma2(float4_t (&acc)[2], const half8_t& a, const half8_t& b0,
                                            const half8_t& b1, bool first) {
  if (first)
    MLA_DEVICE_ASM("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %2, %3, 0\n\tv_mfma_f32_16x16x32_f16 %1, %2, %4, 0"
                   : "=&v"(acc[0]), "=&v"(acc[1]) : "v"(a), "v"(b0), "v"(b1));
  else
    MLA_DEVICE_ASM("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %2, %3, %0\n\tv_mfma_f32_16x16x32_f16 %1, %2, %4, %1"
                   : "+v"(acc[0]), "+v"(acc[1]) : "v"(a), "v"(b0), "v"(b1));
}
// one score MFMA of the software-pipelined loop (its A operand was written
// at least a slot earlier, so no wait states are needed)
__device__ __forceinline__ void score_mfma1(float4_t& acc, const half8_t& a, const half8_t& b) {
  MLA_DEVICE_ASM("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_mfma_drain(float4_t (&acc)[2]) {
  MLA_DEVICE_ASM("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]));
}

// Two-level NVFP4 rows: latent values carry a per-tensor scale g that the
// FP16 operands leave out.  The rope part of a tile's scores (its two
// K-steps come first) is multiplied by 1/g in FP32 before the latent
// K-steps add onto it, and the softmax scale carries g, so the score is
// g * (rope / g + latent) = latent * g + rope to FP32 rounding.  The drain
// waits out the rope MFMAs' latency; the trailing wait states cover the next
// (assembly) MFMA's read of the scaled accumulators.
__device__ __forceinline__ void scale_rope_scores(float4_t (&acc)[2], float inv_g) {
  score_mfma_drain(acc);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[hb][j] *= inv_g;
  MLA_DEVICE_ASM("s_nop 2" : "+v"(acc[0]), "+v"(acc[1]));
}

// head of accumulator element j of `lane` in the 32x32 MFMA C layout
__device__ __forceinline__ int c_head(int j, int lane) { return (j >> 2) * 8 + 4 * (lane >> 5) + (j & 3); }

}  // namespace

template <int kFmt, bool kBf16>
__global__ __launch_bounds__(kThreads, 1) void sparse_decode_kernel(DecodeParams p) {
  constexpr int kRB = row_bytes(kFmt);
  constexpr int kInstr = dma_instr(kFmt);
  constexpr int kSlot = slot_bytes(kFmt);
  constexpr int kDepth = ring_depth(kFmt);

  // The DMA target and the V buffers are separate arrays so that the
  // compiler can tell V-buffer accesses from DMA writes.  After the tile
  // loop both hold the streams' weighted outputs for the merge.
  __shared__ __align__(16) uint8_t ring_all[kWaves * kWaveRing];
  __shared__ __align__(16) half_t vbuf_all[kWaves * kWaveV];
  __shared__ int phys[kMaxTopk];
  __shared__ float wm_s[kWaves][kHG];     // per-stream reference max (base 2)
  __shared__ float wl_s[kWaves][kHG];     // per-stream row sums
  __shared__ float alpha_s[kWaves][kHG];  // O rescale factors, then stream weights
  __shared__ int cnt_s[8][kWaves];
  __shared__ int last_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Block index arithmetic in 32 bits (a 64-bit division is a long chain
  // of dependent scalar instructions ahead of the first memory access).
  // Workgroups are dealt to the 8 XCDs in turn (workgroup b runs on XCD
  // b mod 8).  With xcd_shift = 3 the S splits of (token, head group)
  // 8 k + x are workgroups b = 8 (S k + s) + x, all on XCD x, where the
  // merging split reads the others' partials (and all read the same q and
  // index list) through one L2; the grid is then rounded up to a multiple
  // of 8 S.  With xcd_shift = 0 split s of unit k is workgroup S k + s.
  const int S = p.S, G = p.G;
  const uint32_t xsh = (uint32_t)p.xcd_shift;
  const uint32_t slot = blockIdx.x >> xsh, kx = slot / (uint32_t)S;
  const int s = (int)(slot - kx * (uint32_t)S);
  const uint32_t tg32 = (kx << xsh) + (blockIdx.x & ((1u << xsh) - 1u));
  if (tg32 >= (uint32_t)(p.T * G)) return;   // padding of the rounded-up grid
  const uint32_t t32 = tg32 / (uint32_t)G;
  const int g = (int)(tg32 - t32 * (uint32_t)G);
  const int64_t tg = tg32, t = t32;
  const int r16 = lane & 15, kg = lane >> 4;
  uint8_t* ring = ring_all + wave * kWaveRing;
  half_t* vbuf = vbuf_all + wave * kWaveV;

  // ------------------------------------------------ compact the valid rows
  // All index loads are issued before any is used, then all block-table
  // loads: two dependent memory round trips (addresses of slots past topk
  // or of masked entries are clamped to valid ones and the result dropped).
  // The index loads head the longest dependent chain (index -> block table
  // -> row DMA), so they are issued first; q's loads follow while they are
  // in flight, then the block-table loads (vector loads complete in issue
  // order: waiting for the block-table entries also waits for q, which by
  // then has had a round trip's head start).
  int v8[8];
  {
    const int32_t* ip = p.idx + t * p.idx_st;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = i * kThreads + tid;
      v8[i] = ip[slot < p.topk ? slot : p.topk - 1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i * kThreads + tid >= p.topk) v8[i] = -1;
  }
  // ---------------------------------------------------------------- q
  // q of the workgroup's 32 heads is loaded once, 9 coalesced 16-byte chunks
  // per thread (chunk c: head c / 72, dimensions 8 (c % 72) + [0,8); heads
  // past H repeat the last one), and later staged through the still idle V
  // buffer, from where each wave reads the B operands of its score MFMAs.
  constexpr int kQChunks = kHG * (kQK / 8) / kThreads;   // 9
  u32x4 qstage[kQChunks];     // raw fp16 / bf16 bits
  half8_t qreg[2][kKSteps];   // filled once the rows' DMA is issued (see below)
  {
    const uint16_t* qt = reinterpret_cast<const uint16_t*>(p.q) + t * p.q_st;
#pragma unroll
    for (int m = 0; m < kQChunks; ++m) {
      const int c = tid + kThreads * m, h = c / (kQK / 8), dc = c - h * (kQK / 8);
      const int head = min(g * kHG + h, p.H - 1);
      qstage[m] = *reinterpret_cast<const u32x4*>(qt + (int64_t)head * p.q_sh + 8 * dc);
    }
  }

  int b8[8], pb8[8];
  bool seq_ok = true;
  if (p.bt) {
    const int64_t seq = p.tok_seq[t];
    seq_ok = seq >= 0 && seq < p.bt_rows;
    const int32_t* btr = p.bt + (seq_ok ? seq : 0) * p.bt_st;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // (a power-of-two block size, the usual case, divides by a shift)
      const int v = v8[i] >= 0 ? v8[i] : 0;
      b8[i] = p.bs_log2 >= 0 ? v >> p.bs_log2 : v / p.bs;
      pb8[i] = btr[b8[i] < p.bt_cols ? b8[i] : p.bt_cols - 1];
    }
  }

  int rows8[8], pre8[8];
  {
    if (p.bt) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int r = -1;
        if (seq_ok && v8[i] >= 0 && b8[i] < p.bt_cols && pb8[i] >= 0) {
          const int64_t pr = (int64_t)pb8[i] * p.bs + (v8[i] - b8[i] * p.bs);
          r = pr < p.cache_rows ? (int)pr : -1;
        }
        rows8[i] = r;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) rows8[i] = (v8[i] >= 0 && v8[i] < p.cache_rows) ? v8[i] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t m = __ballot(rows8[i] >= 0);
      pre8[i] = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) cnt_s[i][wave] = __popcll(m);
    }
  }
  lds_barrier();
  int total = 0;
  {
    int base[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      base[i] = total;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (w < wave) base[i] += cnt_s[i][w];
        total += cnt_s[i][w];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (rows8[i] >= 0) phys[base[i] + pre8[i]] = rows8[i];
  }
  lds_barrier();

  // (total <= 2048 and S <= 64: the products fit in 32 bits)
  const int r0 = S == 1 ? 0 : (int)((uint32_t)(total * s) / (uint32_t)S);
  const int n = (S == 1 ? total : (int)((uint32_t)(total * (s + 1)) / (uint32_t)S)) - r0;
  const int ntiles = (n + kRowsT - 1) / kRowsT;
  const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

  // ---------------------------------------------------------------- stream state
  float16_t acc_o[16];                    // O[32 heads x 32 cols] of column block i, C layout
  float mref[2];                          // reference of head hb*16 + r16 (base 2)
  float lsum[2];                          // this lane's share of that head's row sum

  // DMA of one tile into ring slot `slot` (row-interleaved layout above):
  // lane l moves pieces 4j + (l >> 4), j = 0 .. kInstr - 1, of the tile row
  // l & 15 (= r16), whose cache row is `row`, so every source address is the
  // lane's row address plus an immediate.  Rows past the split repeat the
  // split's last row.  NVFP4 rows have 22 pieces: in the last instruction
  // lanes 32..63 (pieces 22, 23) repeat pieces 20 and 21 of their row into
  // positions that are never read.
  auto issue_from = [&](const uint8_t* row_base, int slot) {
    const uint8_t* const a = row_base + 16 * kg;
    uint8_t* const dst = ring + slot * kSlot;
    // instruction j: source a + 64j, LDS dst + 1024j (the immediate 64j
    // applies to both)
    auto one = [&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (kFmt == kFmtNvfp4 && j == 5) MLA_DMA16(row_base + 16 * (20 + (kg & 1)), dst + 1024 * j, 0);
      else MLA_DMA16(a, dst + (1024 - 64) * j, 64 * j);
    };
    static_for<0, kInstr>(one);
  };
  auto issue = [&](uint32_t row, int slot) { issue_from(p.cache + (uint64_t)row * kRB, slot); };
  // cache row of this lane's DMA row in the wave's k-th tile
  auto tile_row_addr = [&](int k) -> uint32_t {
    int i = (wave + kWaves * k) * kRowsT + r16;
    i = i < n ? i : n - 1;
    return lds_off(&phys[r0 + i]);
  };
  const RingOff<kFmt> ro(r16, kg);

  // V-buffer addresses: this lane's ds_read_b64_tr_b16 base for column
  // block 0 (block b is 64 bytes further) and its row for the V writes.
  const int vgrp = lane >> 4, vsl = lane & 15;
  const uint32_t vb = lds_off(vbuf + (8 * (vgrp >> 1) + (vsl >> 2)) * kVRow + 16 * (vgrp & 1) + 4 * (vsl & 3));
  half_t* const vrow = vbuf + r16 * kVRow + 128 * kg;

  // Per tile (16 rows, this wave): wait for the tile's DMA, read the row
  // bytes from the ring, decode them (A operands of the score MFMAs, and the
  // latent also into the V buffer), scores, softmax, then the values.  The
  // next two tiles' DMA is in flight throughout.
  //
  // Software pipeline: the value MFMAs of tile k-1 run interleaved with the
  // decode and score MFMAs of tile k, so the conversion work issues while
  // the matrix core is busy.  Both use the one V buffer: value group j
  // (column blocks j, j+4, j+8, j+12) reads tile k-1's V before latent
  // K-steps 4j..4j+3 of tile k overwrite exactly those columns, and a wave's
  // LDS operations execute in issue order.
  //
  // Softmax reference (base 2): the first tile sets it to its max + kMargin
  // (P <= 2^-kMargin there); afterwards it moves only when a score exceeds
  // it by more than kLazy (P would leave FP16), one ballot deciding; then O
  // and the row sums are rescaled in place.
  const float sm = p.sm_log2;
  const bool two_level = kFmt == kFmtNvfp4 && p.lat_scale != 1.0f;
#pragma unroll
  for (int nb = 0; nb < 16; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc_o[nb][j] = 0.0f;
  mref[0] = mref[1] = kNegInf;
  lsum[0] = lsum[1] = 0.0f;

  Raw<kFmt> raw;
  float4_t sacc[2];
  uint32_t next_row = 0;
  // wait for tile k's DMA and read part A of its rows (and the cache row of
  // this lane's DMA row two tiles ahead)
  auto tile_start = [&](int k) -> uint32_t {
    if (k + 1 < my_tiles) wait_vmcnt<kInstr>();
    else wait_vmcnt<0>();
    const uint32_t slot = lds_off(ring + (k % kDepth) * kSlot);
    next_row = lds_b32(tile_row_addr(k + 2));
    ring_read_a<kFmt>(raw, slot, ro, next_row);
    return slot;
  };
  // one K-step of tile k's scores (latent K-steps also go to the V buffer)
  auto score_step = [&](int k, int ks, uint32_t slot) {
    if (ks == 8) {
      ring_read_b<kFmt>(raw, slot, ro);
      // the slot of tile k + 2 held tile k - 1 (3 slots) or tile k (2
      // slots), both now in registers
      if (k + 2 < my_tiles) issue(next_row, (k + 2) % kDepth);
    }
    const half8_t kop = kstep8<kFmt>(raw, ks);
    if (ks < 16) *reinterpret_cast<half8_t*>(vrow + 8 * ks) = kop;
    score_mfma2(sacc, kop, qreg[0][ks], qreg[1][ks], ks == 16);
  };
  // value group j of the tile whose P is `pa` (its V is in the V buffer)
  auto value_group = [&](const u32x4 (&bv)[4], const half8_t& pa, auto J) {
    constexpr int j = decltype(J)::value;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc_o[j + 4 * e] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          pa, __builtin_bit_cast(half8_t, bv[e]), acc_o[j + 4 * e], 0, 0, 0);
  };
  // Softmax of tile k (scores in sacc), first part: the reference.  Returns
  // whether O must be rescaled by alpha_s before tile k's values are added.
  // The lane holds rows 4kg + j (j = 0..3) of head hb*16 + r16; sm >= 0,
  // so the scaled max is the max scaled.  Only the split's last tile can
  // hold rows past its end; they get P = 0.
  auto softmax_ref = [&](int k) -> bool {
    const int row0 = (wave + kWaves * k) * kRowsT + 4 * kg;
    const bool ragged = (wave + kWaves * k + 1) * kRowsT > n;
    score_mfma_drain(sacc);
    float tmax[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float m = max4(sacc[hb][0], sacc[hb][1], sacc[hb][2], sacc[hb][3]);
      if (ragged) {
        m = kNegInf;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (row0 + j < n) m = __builtin_fmaxf(m, sacc[hb][j]);
      }
      // (-inf * 0 is NaN; the max with -inf maps it back to -inf)
      tmax[hb] = __builtin_fmaxf(m * sm, kNegInf);
    }
    const bool first = k == 0;
    const bool raise = tmax[0] > mref[0] + kLazy || tmax[1] > mref[1] + kLazy;
    if (first || __ballot(raise) != 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float m = tmax[hb];
        m = __builtin_fmaxf(m, shfl_xor_f(m, 16));
        m = __builtin_fmaxf(m, shfl_xor_f(m, 32));
        const float mnew = __builtin_fmaxf(mref[hb], m) + kMargin;
        const float al = first ? 0.0f : __builtin_amdgcn_exp2f(mref[hb] - mnew);
        lsum[hb] *= al;
        mref[hb] = mnew;
        if (kg == 0) alpha_s[wave][hb * 16 + r16] = al;
      }
      return !first;
    }
    return false;
  };
  // second part: P of tile k against the reference, as the value MFMA's A
  // operand
  auto softmax_p = [&](int k) -> half8_t {
    const int row0 = (wave + kWaves * k) * kRowsT + 4 * kg;
    const bool ragged = (wave + kWaves * k + 1) * kRowsT > n;
    float pv[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float nm = -mref[hb];
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[hb][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[hb][j], sm, nm));
      if (ragged) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (row0 + j >= n) pv[hb][j] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) lsum[hb] += pv[hb][j];
    }
    // A operand of the value MFMA: lane L = head block (L >> 4) & 1, head
    // L & 15, rows 8(L >> 5) + [0,8).  d[hb][x] = P of head hb*16 + r16,
    // rows 4kg + 2x, +1 (FP16 pair).  permlane16_swap exchanges the odd
    // 16-lane rows of its first operand with the even rows of its second;
    // afterwards d[0] holds rows 8(kg >> 1) + [0,4) and d[1] rows + [4,8) of
    // head block kg & 1 (the lane ^ 16 neighbour holds the other 4 rows).
    uint32_t d[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        d[hb][x] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                    (float2_t){pv[hb][2 * x], pv[hb][2 * x + 1]}, half2_t));
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const auto sw = __builtin_amdgcn_permlane16_swap(d[0][x], d[1][x], false, false);
      d[0][x] = sw[0];
      d[1][x] = sw[1];
    }
    return __builtin_bit_cast(half8_t, (u32x4){d[0][0], d[0][1], d[1][0], d[1][1]});
  };

  // The first two tiles' DMA.  Missing tiles re-read a valid row (or q,
  // with an empty cache) into slots that are never read.
  // q's loads (issued before the compaction) are complete by now; waiting
  // for them here, where nothing else is in flight, keeps the compiler from
  // waiting for the tiles' DMA before q is staged
  wait_vmcnt<0>();
  {
    const uint8_t* const spare = p.cache_rows > 0 ? p.cache : static_cast<const uint8_t*>(p.q);
    const uint8_t* b0 = spare;
    const uint8_t* b1 = spare;
    if (my_tiles > 0) b0 = p.cache + (uint64_t)(uint32_t)phys[r0 + min(wave * kRowsT + r16, n - 1)] * kRB;
    if (my_tiles > 1) b1 = p.cache + (uint64_t)(uint32_t)phys[r0 + min((wave + kWaves) * kRowsT + r16, n - 1)] * kRB;
    issue_from(b0, 0);
    issue_from(b1, 1 % kDepth);
  }
  // q into LDS in B-operand order, then into registers (while the first
  // tiles' DMA is in flight).  B operand of K-step ks for head block hb,
  // lane (r16, kg): q[hb*16 + r16][d] with d(ks < 16) = 128kg + 8ks + [0,8)
  // and d(16 + i) = 512 + 16kg + 8i + [0,8), at 16-byte slot
  // (hb * 18 + ks) * 64 + 16kg + r16.  A negative softmax scale flips q's
  // signs here (exact), so sm_log2 >= 0.
  {
    // LDS accesses in assembly: the compiler would make them wait for the
    // tiles' DMA (it cannot tell the V buffer from the ring)
    const uint32_t qs = lds_off(vbuf_all);
#pragma unroll
    for (int m = 0; m < kQChunks; ++m) {
      const int c = tid + kThreads * m, h = c / (kQK / 8), d = 8 * (c - h * (kQK / 8));
      int kgq, ks;
      if (d < kLatent) {
        kgq = d >> 7;
        ks = (d >> 3) & 15;
      } else {
        kgq = (d - kLatent) >> 4;
        ks = 16 + (((d - kLatent) >> 3) & 1);
      }
      u32x4 u = q8_operand<kBf16>(qstage[m]);
      if (p.q_neg) u ^= 0x80008000u;
      const uint32_t a = qs + 16 * (((h >> 4) * kKSteps + ks) * 64 + 16 * kgq + (h & 15));
      MLA_DEVICE_ASM("ds_write_b128 %0, %1" :: "v"(a), "v"(u) : "memory");
    }
    lds_barrier();   // (not __syncthreads: that would also wait for the tiles' DMA)
    const uint32_t qa = qs + 16 * lane;
    static_for<0, 2 * kKSteps>([&](auto I) {
      constexpr int i = decltype(I)::value;
      qreg[i / kKSteps][i % kKSteps] = __builtin_bit_cast(half8_t, ring_b128<1024 * i>(qa));
    });
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) MLA_DEVICE_ASM("" : "+v"(qreg[hb][ks]));
    lds_barrier();   // every wave has its q before the V buffer is written
  }
  if (my_tiles > 0) {

    // tile 0: scores only
    {
      const uint32_t slot = tile_start(0);
#pragma unroll
      for (int ks = 16; ks < kKSteps; ++ks) score_step(0, ks, slot);   // rope first: its bytes are then dead
      if (two_level) scale_rope_scores(sacc, p.inv_lat_scale);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) score_step(0, ks, slot);
    }
    (void)softmax_ref(0);
    half8_t pa = softmax_p(0);

    // tiles 1 .. my_tiles-1: values of tile k-1 with the scores of tile k.
    // A raised reference rescales O lazily: each value group first scales
    // its four column blocks (the register allocator keeps O in place only
    // when every rescale sits next to the MFMAs that consume it).
    bool pending = false;   // O is still to be rescaled by alv before its next value MFMA
    float16_t alv = {};     // the rescale factors of this lane's 16 accumulator rows
    auto rescale_group = [&](auto J) {
      constexpr int j = decltype(J)::value;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[j + 4 * e][i] = scale_acc(acc_o[j + 4 * e][i], alv[i]);
    };
    for (int k = 1; k < my_tiles; ++k) {
      const uint32_t slot = tile_start(k);
      half2_t sh[4];
      if constexpr (kFmt == kFmtNvfp4) group_scales(sh, raw.sc);
#pragma unroll
      for (int ks = 16; ks < kKSteps; ++ks) {   // rope
        const half8_t kop = kstep8<kFmt>(raw, ks);
        score_mfma2(sacc, kop, qreg[0][ks], qreg[1][ks], ks == 16);
      }
      if (two_level) scale_rope_scores(sacc, p.inv_lat_scale);
      // Slot t (latent K-step t): the value MFMA of one column block of
      // tile k-1, the conversions of K-step t+1 split around the two score
      // MFMAs of K-step t, then the V write of K-step t+1.  The order is
      // pinned (sched_barrier) so that every conversion issues while an MFMA
      // runs.
      half8_t kop;
      {
        KDec d;
        kdec_part1<kFmt>(d, raw, sh, 0);
        kop = kdec_part2<kFmt>(d, raw, sh, 0);
      }
      // value groups read one unit ahead (two buffers): group j + 1 is read
      // during unit j, before K-step 4(j+1) overwrites it at unit j + 1
      u32x4 bvb[2][4];
      read_v4_group<0>(bvb[0], vb);
      ring_issue_b<kFmt>(raw, slot, ro);   // latent K-steps 8..15 (FP8: 8..11), waited for with group 1
      // the slot of tile k + 2 held tile k - 1 (NVFP4, 3 slots), now in
      // registers; FP8 rows (2 slots) refill the slot of tile k itself once
      // the last of its bytes are read, in value group 1
      if constexpr (kFmt == kFmtNvfp4)
        if (k + 2 < my_tiles) issue(next_row, (k + 2) % kDepth);
      static_for<0, 4>([&](auto J) {
        constexpr int j = decltype(J)::value;
        u32x4 (&bv)[4] = bvb[j & 1];
        // group j's reads were issued one unit earlier, followed by that
        // unit's four V-buffer writes (unit 0: by the ring's part B reads,
        // which it waits for as well)
        if constexpr (j == 0) lgkm_wait(bv);
        else if constexpr (j == 1) lgkm_wait_b<kFmt>(bv, raw);
        else if constexpr (j == 2) lgkm_wait4_b2<kFmt>(bv, raw);
        else lgkm_wait4(bv);
        if constexpr (j < 3) read_v4_group<j + 1>(bvb[(j + 1) & 1], vb);
        if constexpr (j == 1 && kFmt == kFmtFp8) {
          ring_issue_b2<kFmt>(raw, slot, ro);   // K-steps 12..15
          if (k + 2 < my_tiles) issue(next_row, (k + 2) % kDepth);
        }
        *reinterpret_cast<half8_t*>(vrow + 8 * (4 * j)) = kop;   // after group j's reads
        if (pending) rescale_group(J);
        static_for<0, 4>([&](auto E) {
          constexpr int e = decltype(E)::value;
          constexpr int t = 4 * j + e;
          KDec d;
          __builtin_amdgcn_sched_barrier(0);
          acc_o[j + 4 * e] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              pa, __builtin_bit_cast(half8_t, bv[e]), acc_o[j + 4 * e], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (t < 15) kdec_part1<kFmt>(d, raw, sh, t + 1);
          __builtin_amdgcn_sched_barrier(0);
          score_mfma1(sacc[0], kop, qreg[0][t]);
          __builtin_amdgcn_sched_barrier(0);
          half8_t nx;
          if constexpr (t < 15) nx = kdec_part2<kFmt>(d, raw, sh, t + 1);
          __builtin_amdgcn_sched_barrier(0);
          score_mfma1(sacc[1], kop, qreg[1][t]);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (t < 15) {
            kop = nx;
            if constexpr ((t + 1) % 4 != 0) *reinterpret_cast<half8_t*>(vrow + 8 * (t + 1)) = kop;
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      pending = softmax_ref(k);
      if (pending) {   // (LDS keeps this wave's order for alpha_s)
        MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < 16; ++i) alv[i] = alpha_s[wave][c_head(i, lane)];
      }
      pa = softmax_p(k);
    }

    // values of the last tile
    static_for<0, 4>([&](auto J) {
      constexpr int j = decltype(J)::value;
      u32x4 bv[4];
      read_v4_group<j>(bv, vb);
      if (pending) rescale_group(J);
      lgkm_wait(bv);
      value_group(bv, pa, J);
    });
  }
  wait_vmcnt<0>();   // no DMA may still be writing this workgroup's LDS

  // ---------------------------------------------------------------- merge the streams
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    lsum[hb] += shfl_xor_f(lsum[hb], 16);
    lsum[hb] += shfl_xor_f(lsum[hb], 32);
  }
  if (kg == 0) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      wm_s[wave][hb * 16 + r16] = mref[hb];
      wl_s[wave][hb * 16 + r16] = lsum[hb];
    }
  }
  __syncthreads();   // every stream's state is visible and the rings are idle
  // weight of stream w for head hd: 2^(m_w - M) / L with
  // M = max_w m_w and L = sum_w 2^(m_w - M) l_w; log2-sum-exp = M + log2 L
  if (tid < kWaves * kHG) {
    const int w = tid >> 5, hd = tid & 31;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = __builtin_fmaxf(M, wm_s[v][hd]);
    float L = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v)
        L += wm_s[v][hd] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(wm_s[v][hd] - M) * wl_s[v][hd];
    }
    const float mw = wm_s[w][hd];
    alpha_s[w][hd] = (L > 0.0f && mw != kNegInf) ? __builtin_amdgcn_exp2f(mw - M) / L : 0.0f;
    if (w == 0) {
      const float lse2 = L > 0.0f ? M + __log2f(L) : kNegInf;
      const int head = g * kHG + hd;
      if (S > 1) __hip_atomic_store(p.part_lse + (tg * S + s) * kHG + hd, lse2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (head < p.H && p.lse) p.lse[t * p.H + head] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
    }
  }
  __syncthreads();
  // Stream merge in two rounds of 256 columns.  Each wave writes its FP32
  // O for 8 column blocks straight from the accumulation registers into its
  // exchange region (waves 0, 1 in the ring area, 2, 3 in the V area; the
  // rings are idle), then every thread sums the four streams for 4 heads x 8
  // columns with the stream weights and stores them (16-byte stores).
  // Exchange layout: 16-byte slot s (the lane of the MFMA C layout) of block
  // b (column block within the round x 4 + element quad) sits at byte
  // 1136 b + 16 s + 32 (s >> 4): the writers' 64 lanes and the readers' 8
  // consecutive slots (8 columns of 4 heads) are both free of bank conflicts.
  const float out_mul = p.kv_scale * p.lat_scale;  // values carry the cache's per-tensor scale
  const int64_t H = p.H;
  {
    constexpr uint32_t kXBlock = 1136, kXRegion = 32 * kXBlock;
    static_assert(2 * kXRegion <= kWaves * kWaveRing && 2 * kXRegion <= kWaves * kWaveV * 2, "exchange regions");
    uint8_t* const x01 = ring_all;
    uint8_t* const x23 = reinterpret_cast<uint8_t*>(vbuf_all);
    uint8_t* const xw = (wave < 2 ? x01 : x23) + (wave & 1) * kXRegion + 16 * lane + 32 * (lane >> 4);
    // reader: heads 4 hq + [0,4), columns 256 hh + 8 co + [0,8)
    const int hq = tid & 7, co = tid >> 3;
    const uint32_t rslot = 32 * (hq & 1) + 8 * (co & 3);
    const uint32_t rofs = ((co >> 2) * 4 + (hq >> 1)) * kXBlock + 16 * rslot + 32 * (rslot >> 4);
    const uint8_t* const r01 = x01 + rofs;
    const uint8_t* const r23 = x23 + rofs;
    const float mul = S > 1 ? 1.0f : out_mul;
    float wgt[kWaves][4];
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int h = 0; h < 4; ++h) wgt[w][h] = alpha_s[w][4 * hq + h] * mul;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1) __syncthreads();   // the first round's reads are done
#pragma unroll
      for (int nbl = 0; nbl < 8; ++nbl)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4_t*>(xw + (nbl * 4 + q) * kXBlock) =
              (float4_t){acc_o[8 * hh + nbl][4 * q], acc_o[8 * hh + nbl][4 * q + 1], acc_o[8 * hh + nbl][4 * q + 2],
                         acc_o[8 * hh + nbl][4 * q + 3]};
      __syncthreads();
      float o[4][8];
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int x = 0; x < 8; ++x) o[h][x] = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint8_t* const src = (w < 2 ? r01 : r23) + (w & 1) * kXRegion;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float4_t v = *reinterpret_cast<const float4_t*>(src + 16 * x);
#pragma unroll
          for (int h = 0; h < 4; ++h) o[h][x] = __builtin_fmaf(wgt[w][h], v[h], o[h][x]);
        }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int hd = 4 * hq + h, head = g * kHG + hd;
        const int col = 256 * hh + 8 * co;
        if (S > 1) store8_agent(p.part_o + ((tg * S + s) * kHG + hd) * kLatent + col, o[h]);
        else if (head < p.H)
          store8<kBf16>(reinterpret_cast<uint16_t*>(p.out) + (t * H + head) * kLatent + col, o[h]);
      }
    }
  }
  if (S == 1) return;

  // Count arrivals once every wave's partial stores are complete (each wave
  // waits for its own; the barrier orders them before the count); the last
  // arrival merges.
  MLA_DEVICE_ASM("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint32_t* ctr = p.counters + tg;
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == (uint32_t)S - 1u;
    if (last) {
      // the partials were written through (agent-scope stores) before their
      // counts; invalidate this XCD's caches so that plain loads see them
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    }
    last_s = last;
  }
  __syncthreads();
  if (!last_s) return;

  // Chunks of 8 consecutive columns, 32 heads x 64 chunks: chunk tid + 256 m
  // (m = 0..7) is head (tid >> 6) + 4 m, columns 8 (tid & 63).  Splits are
  // summed in index order, two per round, and the next round's 16-byte
  // loads are in flight while a round is summed (an odd count adds split s0
  // again with weight 0).  The log2-sum-exps are loaded first (lane x of
  // wave 0 reads split x's), then the first round's partials, so that the
  // merge weights wait only for the former.
  float* lse_sh = reinterpret_cast<float*>(ring_all);   // [S][32]
  float* wsh = lse_sh + 64 * kHG;                        // [S][32]
  const int cc = 8 * (tid & 63);
  const half_t* pp = p.part_o + (tg * S) * kHG * kLatent + (tid >> 6) * kLatent + cc;
  auto load_split = [&](int x, half8_t (&v)[8]) {
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = *reinterpret_cast<const half8_t*>(pp + (x * kHG + 4 * m) * kLatent);
  };
  float a[8][8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 8; ++i) a[m][i] = 0.0f;
  auto add_pair = [&](const half8_t (&v0)[8], const half8_t (&v1)[8], int s0) {
    const bool has1 = s0 + 1 < S;
    const int s1 = has1 ? s0 + 1 : s0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float w0 = wsh[s0 * kHG + (tid >> 6) + 4 * m];
      const float w1 = has1 ? wsh[s1 * kHG + (tid >> 6) + 4 * m] : 0.0f;
      // (two fused multiply-adds per element, each taking its FP16 operand
      // as is: v_fma_mix)
#pragma unroll
      for (int i = 0; i < 8; ++i) a[m][i] = __builtin_fmaf(w1, (float)v1[m][i], __builtin_fmaf(w0, (float)v0[m][i], a[m][i]));
    }
  };
  half8_t A0[8], A1[8], B0[8], B1[8];
  float4_t lx[8];
  if (wave == 0) {
    const float4_t* src = reinterpret_cast<const float4_t*>(p.part_lse + (tg * S + (lane < S ? lane : 0)) * kHG);
#pragma unroll
    for (int i = 0; i < 8; ++i) lx[i] = src[i];
  }
  load_split(0, A0);
  load_split(1 < S ? 1 : 0, A1);
  if (wave == 0 && lane < S) {
    float4_t* dst = reinterpret_cast<float4_t*>(lse_sh + lane * kHG);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = lx[i];
  }
  __syncthreads();
  if (tid < kHG) {
    float mx = kNegInf;
    for (int ss = 0; ss < S; ++ss) mx = __builtin_fmaxf(mx, lse_sh[ss * kHG + tid]);
    float sum = 0.0f;
    if (mx != kNegInf)
      for (int ss = 0; ss < S; ++ss) sum += __builtin_amdgcn_exp2f(lse_sh[ss * kHG + tid] - mx);
    const float inv = mx != kNegInf ? 1.0f / sum : 0.0f;
    for (int ss = 0; ss < S; ++ss)
      wsh[ss * kHG + tid] = mx != kNegInf ? __builtin_amdgcn_exp2f(lse_sh[ss * kHG + tid] - mx) * inv : 0.0f;
    const int head = g * kHG + tid;
    if (head < p.H && p.lse) p.lse[t * H + head] = mx != kNegInf ? (mx + __log2f(sum)) * kLn2 : kNegInf;
  }
  __syncthreads();
  {
    for (int s0 = 0; s0 < S; s0 += 4) {
      const bool more = s0 + 2 < S;
      if (more) {
        load_split(s0 + 2, B0);
        load_split(s0 + 3 < S ? s0 + 3 : s0 + 2, B1);
      }
      add_pair(A0, A1, s0);
      if (!more) break;
      const bool more2 = s0 + 4 < S;
      if (more2) {
        load_split(s0 + 4, A0);
        load_split(s0 + 5 < S ? s0 + 5 : s0 + 4, A1);
      }
      add_pair(B0, B1, s0 + 2);
      if (!more2) break;
    }
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int hd = (tid >> 6) + 4 * m, head = g * kHG + hd;
    if (head >= p.H) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[m][i] *= out_mul;
    store8<kBf16>(reinterpret_cast<uint16_t*>(p.out) + (t * H + head) * kLatent + cc, a[m]);
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
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

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

int decode_auto_splits(int64_t T, int H, int topk) {
  const int G = H <= kHG ? 1 : H / kHG;
  const int64_t groups = T * G;
  if (groups <= 0) return 1;
  const int cus = device_cus() > 0 ? device_cus() : 256;
  // One workgroup per CU is resident at a time: fill the CUs once (more
  // splits than that would start a second, mostly idle round).  A split
  // keeps at least 256 valid rows (four tiles per stream) so its fixed
  // costs (index compaction, q load, stream and split merges) stay small.
  int64_t s = cus / groups;
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

hipError_t launch_decode(const DecodeParams& p, int fmt, bool bf16, hipStream_t stream,
                         const KernelEvents& ev) {
  // A (token, head group)'s splits share an XCD (xcd_shift = 3) unless
  // that would take more rounds of resident workgroups than the plain
  // order: grouping puts ceil(units / 8) * S workgroups on each XCD's
  // eighth of the CUs.
  DecodeParams a = p;
  const int64_t units = p.T * p.G;
  const int64_t cus = device_cus() > 0 ? device_cus() : 256, per_xcd = cus >= 8 ? cus / 8 : 1;
  const int64_t rounds_plain = (units * p.S + cus - 1) / cus;
  const int64_t rounds_grouped = ((units + 7) / 8 * p.S + per_xcd - 1) / per_xcd;
  a.xcd_shift = p.S > 1 && rounds_grouped <= rounds_plain ? 3 : 0;
  const int64_t blocks = a.xcd_shift ? (units + 7) / 8 * 8 * p.S : units * p.S;
  dim3 grid((unsigned)blocks), block(kThreads);
  void* args[] = {&a};
  const void* fn;
  if (fmt == kFmtNvfp4)
    fn = bf16 ? (const void*)sparse_decode_kernel<kFmtNvfp4, true>
              : (const void*)sparse_decode_kernel<kFmtNvfp4, false>;
  else
    fn = bf16 ? (const void*)sparse_decode_kernel<kFmtFp8, true>
              : (const void*)sparse_decode_kernel<kFmtFp8, false>;
  return launch_kernel(fn, grid, block, args, stream, ev);
}

}  // namespace mla
