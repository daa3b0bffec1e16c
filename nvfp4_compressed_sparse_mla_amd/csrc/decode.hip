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
// Workgroup = (token t, head group g of 32 heads, split s), 8 waves, one
// workgroup per CU, two waves per SIMD.  The waves take two roles:
//
//   score waves (0..3)  each streams its own 16-row tiles (tiles w, w+4,
//             w+8, ... of the split) through its own LDS-DMA ring, holds q
//             of all 32 heads in registers, decodes each row once into the
//             FP16 A operands of the score MFMAs, computes S^T[16 rows x 32
//             heads] and its softmax P, and leaves P (FP16) and the decoded
//             latent (the V of the tile, FP16) in LDS.
//   value waves (4..7)  value wave j owns output columns [128j, +128) of
//             all 32 heads (64 accumulation registers): per round it loads
//             the four tiles' P and its columns of their V from LDS and adds
//             P . V with 16 MFMAs (32x32x16).
//
// A round is one tile per score wave.  Two workgroup barriers per round
// hand the LDS over: A(r) after the score waves wrote round r, B(r) after
// the value waves have round r in registers.  Between B(r) and A(r+1) the
// value waves' MFMAs for round r run beside the score waves' decode and
// scores of round r+1 on the same SIMDs; between A(r) and B(r) the score
// waves wait for their next tile's DMA and do its rope part.  No wave holds
// both q and O, so each fits in 256 registers, and the output columns
// never need merging across waves.
//
//   prologue  load the token's index list, translate it through the block
//             table, drop masked / out-of-range slots and compact the valid
//             rows into LDS (padded slots are never fetched; split
//             boundaries balance valid rows); stage q through LDS into the
//             score waves' registers in the score MFMA's B-operand layout.
//   per tile  (16 rows, one score wave)
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
//     scores  36 MFMAs (16x16x32, FP16 -> FP32).
//     softmax base 2 against a lazily raised reference max: a score wave's
//             first tile sets its reference, which then moves only when a
//             score exceeds it by more than 15 (one ballot decides), so
//             P = 2^(s - ref) <= 2^15 stays inside FP16 with its full 11-bit
//             precision.  Each tile's P goes to LDS with the reference it
//             is relative to; row sums accumulate per lane.
//     values  the value waves keep O relative to the largest reference seen
//             per head: a tile whose reference is lower has its P scaled by
//             2^(ref - M) (a power of two, exact in FP16 above its subnormal
//             range); a higher reference first rescales O.
//   epilogue  the value waves normalise their columns by the row sums of
//             all score waves (weighted by 2^(m_w - M)); S == 1 stores the
//             output, S > 1 stores the normalised partial (FP16, in the
//             accumulators' order) and its log2-sum-exp.
//   merge     (S > 1) once all S splits of (t, g) have arrived, split k
//             combines slice k of the partials (from 4 splits up; with
//             fewer, the last arrival combines everything).  Every wait is
//             bounded and the last arrival combines whatever slice nobody
//             took, so no co-residency is needed.
#include "mla_device.h"
#include "mla_launch.h"

#include <type_traits>

namespace mla {

namespace {

constexpr int kRowsT = 16;            // rows per tile (one score wave)
constexpr int kHG = 32;               // heads per workgroup
constexpr int kSW = 4;                // score waves
constexpr int kVW = 4;                // value waves
constexpr int kWaves = kSW + kVW;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlices = kMaxTopk / (64 * kSW);   // index-list slots per score-wave thread
static_assert(kSlices * 64 * kSW == kMaxTopk, "index slots per score-wave thread");
constexpr int kVCols = kLatent / kVW; // output columns per value wave
// V buffer: 1,024-byte rows (FP16 elements per row: kVRow) whose 16-byte
// chunks are XOR-swizzled, chunk c of row r at chunk c ^ vswz(r).  With
// vswz(r) = 4 (r mod 4) + (r / 2 mod 4) both access patterns are free of bank
// conflicts: the score waves' row writes (a write instruction's groups of 8
// lanes: 8 rows at one chunk) and the value waves' transposing reads (groups
// of 32 lanes: 4 rows x 4 chunks of a 64-byte column block).  Measured on
// this GPU: 10.0 cycles per ds_write_b128 and 2.6 per ds_read_b64_tr_b16,
// against 10.0 and 4.0 for a padded 1,072-byte row.
constexpr int kVRow = kLatent;
constexpr int kTileV = kRowsT * kVRow;  // FP16 elements of one tile's V
__device__ __forceinline__ uint32_t vswz(uint32_t r) { return 4 * (r & 3) + ((r >> 1) & 3); }
constexpr int kPRow = kRowsT + 8;       // FP16 elements per head in the P buffer (16 rows + padding)
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
// Slots per score wave: a tile's bytes move to registers as the tile
// starts, and its slot is refilled at once, so every slot holds a tile in
// flight (NVFP4 3, FP8 rows are larger: 2)
constexpr int ring_depth(int fmt) { return fmt == kFmtNvfp4 ? 3 : 2; }
constexpr int kWaveRing = 18432;      // bytes of ring per score wave (both formats)
static_assert(ring_depth(kFmtNvfp4) * slot_bytes(kFmtNvfp4) <= kWaveRing, "NVFP4 ring");
static_assert(ring_depth(kFmtFp8) * slot_bytes(kFmtFp8) <= kWaveRing, "FP8 ring");
// q of the workgroup's 32 heads is staged through the V buffer before the loop
static_assert(kHG * kQK * 2 <= kSW * kTileV * 2, "q staging area");
// Output exchange of a value wave (epilogue): 16 blocks (4 column blocks x 4
// head quads) of 64 16-byte slots, padded so that both the writers' 64
// lanes and the readers' 8 consecutive slots are free of bank conflicts
constexpr uint32_t kXBlock = 1136, kXRegion = 16 * kXBlock;
static_assert(2 * kXRegion <= kSW * kWaveRing && 2 * kXRegion <= kSW * kTileV * 2, "exchange regions");

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
// (aux 16: the sc1 cache policy, agent scope)
#define MLA_DMA_AGENT(src, lds) __builtin_amdgcn_global_load_lds((src), (lds), 16, 0, 16)
#else
#define MLA_DEVICE_ASM(...) __builtin_unreachable()
#define MLA_DMA16(src, lds, off) ((void)(src), (void)(lds))
#define MLA_DMA_AGENT(src, lds) ((void)(src), (void)(lds))
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
template <int kOff = 0>
__device__ __forceinline__ u32x2 ring_b64(uint32_t a) {
  u32x2 v;
  MLA_DEVICE_ASM("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(kOff));
  return v;
}
__device__ __forceinline__ u32x4 lds_b128(uint32_t a) {
  u32x4 v;
  MLA_DEVICE_ASM("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
template <int kOff = 0>
__device__ __forceinline__ uint32_t lds_b32(uint32_t a) {
  uint32_t v;
  MLA_DEVICE_ASM("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(kOff));
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

// All of the lane's row bytes of one slot, and `extra` (an LDS read issued
// just before), valid on return.
template <int kFmt>
__device__ __forceinline__ void ring_read(Raw<kFmt>& r, uint32_t slot, const RingOff<kFmt>& o, uint32_t& extra) {
  if constexpr (kFmt == kFmtNvfp4) {
    r.l[0] = ring_b128<0>(slot + o.lat);
    r.l[1] = ring_b128<256>(slot + o.lat);
    r.l[2] = ring_b128<512>(slot + o.lat);
    r.l[3] = ring_b128<768>(slot + o.lat);
    r.sc = ring_b64(slot + o.sc);
    r.rp = ring_b128(slot + o.rope);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)"
                   : "+v"(r.l[0]), "+v"(r.l[1]), "+v"(r.l[2]), "+v"(r.l[3]), "+v"(r.sc), "+v"(r.rp), "+v"(extra));
  } else {
    static_for<0, 8>([&](auto I) {
      constexpr int i = decltype(I)::value;
      r.l[i] = ring_b128<256 * i>(slot + o.lat);
    });
    r.rp = ring_b128(slot + o.rope);
    MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)"
                   : "+v"(r.l[0]), "+v"(r.l[1]), "+v"(r.l[2]), "+v"(r.l[3]), "+v"(r.l[4]), "+v"(r.l[5]),
                     "+v"(r.l[6]), "+v"(r.l[7]), "+v"(r.rp), "+v"(extra));
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

// A latent K-step's A operand with the group scales already in FP16: `sh`
// holds the lane's 8 group scales (group g = half g & 1 of sh[g >> 1]).
template <int kFmt>
__device__ __forceinline__ half8_t latent8(const Raw<kFmt>& r, const half2_t (&sh)[4], int ks) {
  if constexpr (kFmt == kFmtNvfp4) {
    const uint32_t w = r.l[ks >> 2][ks & 3];
    const half2_t s2 = sh[ks >> 2];
    const half_t sv = ((ks >> 1) & 1) ? s2.y : s2.x;
    const half2_t s = {sv, sv};
    half2_t c[4];
    static_for<0, 4>([&](auto I) {
      constexpr int i = decltype(I)::value;
      c[i] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, i)) * s;
    });
    return (half8_t){c[0].x, c[0].y, c[1].x, c[1].y, c[2].x, c[2].y, c[3].x, c[3].y};
  } else {
    (void)sh;
    return kstep8<kFmt>(r, ks);
  }
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
// L2-wide writeback before counting its arrival.  Four FP16 values (8
// bytes) per store; in assembly, so the caller waits for it itself (s_waitcnt
// vmcnt(0) after its last store).  The compiler does not see this store, so
// the statement carries two wait states for its data registers (a store
// reads them after it issues; a VALU write to them right after could
// change the data of the late lanes).
__device__ __forceinline__ void store4_agent(half_t* dst, float a, float b, float c, float d) {
  const u32x2 w = {as_u32((half2_t){(half_t)a, (half_t)b}), as_u32((half2_t){(half_t)c, (half_t)d})};
  MLA_DEVICE_ASM("global_store_dwordx2 %0, %1, off sc1\n\ts_nop 1" :: "v"(dst), "v"(w) : "memory");
}
// two consecutive output elements (4-byte aligned), fp16 or bf16
template <bool kBf16, typename T>
__device__ __forceinline__ void store2(T* dst, float a, float b) {
  uint32_t w;
  if constexpr (kBf16) w = (uint32_t)float_to_bf16_rne(a) | ((uint32_t)float_to_bf16_rne(b) << 16);
  else w = as_u32((half2_t){(half_t)a, (half_t)b});
  *reinterpret_cast<uint32_t*>(dst) = w;
}

// A load of another workgroup's result: 16 bytes with the agent-scope
// policy (sc1, what an agent-scope atomic load uses), coherent at agent
// scope by itself, so no cache invalidation is needed before it.  In
// assembly (the caller waits with vmcnt and ties the registers).
__device__ __forceinline__ u32x4 load16_agent(const void* src) {
  u32x4 v;
  MLA_DEVICE_ASM("global_load_dwordx4 %0, %1, off sc1" : "=v"(v) : "v"(src) : "memory");
  return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// V operands of one tile for a value wave: the B operands of its 4 column
// blocks (32x32x16 MFMA: 8 rows of one column per lane).  ds_read_b64_tr_b16
// gives each lane 4 consecutive rows of one column; two reads (rows 0-3 and
// 4-7 of the lane's 8) make one operand.  `base` is the lane's (swizzled)
// address for column block 0 of tile 0, its row r0 with r0 mod 8 < 4; kTile
// selects the tile.  Column block e is chunk 4e further in the row, which
// the swizzle turns into base ^ 64e (base's bits 4-7 come from the chunk
// alone: the buffer is 256-byte aligned); row r0 + 4 has vswz(r0) ^ 2, one
// chunk bit more: ^ 32, four rows (4,096 bytes) down.
template <int kTile>
__device__ __forceinline__ void read_v_tile(u32x4 (&b)[4], uint32_t base) {
  static_for<0, 4>([&](auto E) {
    constexpr int e = decltype(E)::value;
    constexpr int off = kTile * kTileV * 2;
    const uint32_t a = base ^ (64u * e);
    u32x2 lo, hi;
    MLA_DEVICE_ASM("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(a), "i"(off));
    MLA_DEVICE_ASM("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(a ^ 32u), "i"(off + 8 * kVRow));
    b[e] = (u32x4){lo.x, lo.y, hi.x, hi.y};
  });
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its outstanding global loads (__syncthreads() would also wait for
// those, e.g. the tiles' DMA in flight).  The memory clobber keeps the
// compiler from moving memory accesses across it.
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

// max of four MFMA results (v_max3; the compiler's fmaxf would first
// canonicalise each input with another v_max)
__device__ __forceinline__ float max4(float a, float b, float c, float d) {
  float m;
  MLA_DEVICE_ASM("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4" : "=&v"(m) : "v"(a), "v"(b), "v"(c), "v"(d));
  return m;
}

// The two score MFMAs of a K-step (16x16x32, FP16 -> FP32), in assembly so
// that the compiler keeps their accumulators in VGPRs next to q.  Hazards
// are handled here: two wait states after the VALU write of the A operand
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
// one score MFMA of the pipelined latent K-steps (its A operand was written
// at least two instructions earlier, so no wait states are needed)
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
  // NVFP4 rows: the value waves issue the ring refills (value wave j for
  // score wave j's slot, right after the score wave has read it), which
  // keeps the DMA issue off the score waves' path to the next barrier.
  // FP8 rows keep the score waves' own refills (their two-slot ring leaves
  // a refill issued one round later too little time).
  constexpr bool kVRefill = kFmt == kFmtNvfp4;
  static_assert(!kVRefill || kDepth == 3, "value-wave refills assume a three-slot ring");

  // The DMA target, the V buffer and the P buffer are separate arrays so
  // that the compiler can tell their accesses from the DMA's writes.  After
  // the loop the ring and V areas hold the value waves' output exchange.
  __shared__ __align__(16) uint8_t ring_all[kSW * kWaveRing];
  __shared__ __align__(256) half_t vbuf_all[kSW * kTileV];   // (256-byte aligned: see read_v_tile)
  // P of a round's tiles, [head][row]; heads 48 bytes apart, so that 16
  // consecutive heads (the value waves' 16-byte reads, the score waves'
  // 8-byte writes) fall in distinct banks
  __shared__ __align__(16) half_t pbuf[kSW][kHG][kPRow];
  __shared__ __align__(16) float ref_s[kSW][kHG];           // the reference each tile's P is relative to
  __shared__ __align__(16) int phys[kMaxTopk];
  // per head: the score waves' final references (base 2), then their row sums
  __shared__ __align__(16) float wml_s[kHG][2 * kSW];
  __shared__ __align__(16) float fac_s[kVW][kHG];           // per value wave: per-head factors
  __shared__ __align__(16) int cnt_s[kSlices][kVW];   // valid slots per (slice, value wave)
  __shared__ uint64_t won_s;
  __shared__ int role_s;
  __shared__ uint32_t epoch_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Every kernel argument the prologue uses, in registers before anything
  // else: left to the compiler, each group would be loaded at its first use,
  // one dependent scalar round trip after another ahead of the index ->
  // block table -> row chain.  One statement, whose outputs (S, G and the
  // XCD shift) the block index arithmetic takes, so that nothing is
  // scheduled between the loads and their single wait.
  int S = p.S, G = p.G, xsh_arg = p.xcd_shift;
  MLA_DEVICE_ASM("" : "+s"(S), "+s"(G), "+s"(xsh_arg)
                 : "s"(p.q), "s"(p.q_st), "s"(p.q_sh), "s"(p.T), "s"(p.H), "s"(p.cache), "s"(p.cache_rows),
                   "s"(p.idx), "s"(p.topk), "s"(p.idx_st), "s"(p.q_neg), "s"(p.bt), "s"(p.bs), "s"(p.bt_rows),
                   "s"(p.bt_cols), "s"(p.bs_log2), "s"(p.bt_st), "s"(p.tok_seq));
  // Block index arithmetic in 32 bits (a 64-bit division is a long chain
  // of dependent scalar instructions ahead of the first memory access).
  // Workgroups are dealt to the 8 XCDs in turn (workgroup b runs on XCD
  // b mod 8).  With xcd_shift = 3 the S splits of (token, head group)
  // 8 k + x are workgroups b = 8 (S k + s) + x, all on XCD x, where the
  // merging split reads the others' partials (and all read the same q and
  // index list) through one L2; the grid is then rounded up to a multiple
  // of 8 S.  With xcd_shift = 0 split s of unit k is workgroup S k + s.
  const uint32_t xsh = (uint32_t)xsh_arg;
  const uint32_t slot = blockIdx.x >> xsh, kx = slot / (uint32_t)S;
  const int s = (int)(slot - kx * (uint32_t)S);
  const uint32_t tg32 = (kx << xsh) + (blockIdx.x & ((1u << xsh) - 1u));
  if (tg32 >= (uint32_t)(p.T * G)) return;   // padding of the rounded-up grid
  const uint32_t t32 = tg32 / (uint32_t)G;
  const int g = (int)(tg32 - t32 * (uint32_t)G);
  const int64_t tg = tg32, t = t32;
  const int r16 = lane & 15, kg = lane >> 4;

  // ---------------------------------------------------------------- prologue
  // The longest chain of the prologue is index list -> block table -> row
  // DMA; everything else is arranged around it.
  //  * Score waves: while every slot of the list names a row, the compacted
  //    row list is the slot list itself, so each lane loads the index and
  //    block-table entries of its own rows of the first kDepth tiles and
  //    issues their DMA at once ("speculative" first tiles).  A wave does so
  //    only if those rows and the list's last slot are valid (a list padded
  //    at its end does not speculate); if the compaction then finds masked
  //    slots, the wave waits for that DMA and issues the tiles again from the
  //    compacted list.
  //  * Value waves: compact the valid rows of the whole list (slot
  //    i * 256 + v of value-wave thread v), and stage q in LDS.
  // Loads and their uses stay inside each role's branch: loads left in flight
  // past it would, for the compiler, also be in flight on the other role's
  // path.
  const int sw = wave;        // (score waves only)
  uint8_t* const ring = ring_all + (wave < kSW ? wave : 0) * kWaveRing;

  // DMA of one tile into ring slot `sl` (row-interleaved layout above):
  // lane l moves pieces 4j + (l >> 4), j = 0 .. kInstr - 1, of the tile row
  // l & 15 (= r16), whose cache row is `row`, so every source address is the
  // lane's row address plus an immediate.  Rows past the split repeat the
  // split's last row.  NVFP4 rows have 22 pieces: in the last instruction
  // lanes 32..63 (pieces 22, 23) repeat pieces 20 and 21 of their row into
  // positions that are never read.
  auto dma_tile = [&](const uint8_t* row_base, uint8_t* const dst) {
    const uint8_t* const a = row_base + 16 * kg;
    // instruction j: source a + 64j, LDS dst + 1024j (the immediate 64j
    // applies to both)
    auto one = [&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (kFmt == kFmtNvfp4 && j == 5) MLA_DMA16(row_base + 16 * (20 + (kg & 1)), dst + 1024 * j, 0);
      else MLA_DMA16(a, dst + (1024 - 64) * j, 64 * j);
    };
    static_for<0, kInstr>(one);
  };
  auto issue_from = [&](const uint8_t* row_base, int sl) { dma_tile(row_base, ring + sl * kSlot); };
  auto issue = [&](uint32_t row, int sl) { issue_from(p.cache + (uint64_t)row * kRB, sl); };
  // missing tiles re-read a valid row (or q, with an empty cache) into slots
  // that are never read
  const uint8_t* const spare = p.cache_rows > 0 ? p.cache : static_cast<const uint8_t*>(p.q);

  const int32_t* const ip = p.idx + t * p.idx_st;
  // the token's block-table row number (from the index list itself when
  // there is no table, so that the load needs no branch)
  const int32_t* const seq_p = p.bt ? p.tok_seq + t : ip;

  int rows8[kSlices], pre8[kSlices];   // (value waves)
  bool spec = false;                   // (score waves) first tiles issued before the compaction
  if (wave < kSW) {
    const int topk = p.topk;
    const int r0s = S == 1 ? 0 : (int)((uint32_t)(topk * s) / (uint32_t)S);
    const int ns = (S == 1 ? topk : (int)((uint32_t)(topk * (s + 1)) / (uint32_t)S)) - r0s;
    const int nts = (ns + kRowsT - 1) / kRowsT;
    const int myts = nts > sw ? (nts - sw + kSW - 1) / kSW : 0;
    const int seq_raw = *seq_p;
    const int last = ip[topk - 1];
    int vs[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int e = min((sw + kSW * i) * kRowsT + r16, ns - 1);
      vs[i] = ip[r0s + (e > 0 ? e : 0)];   // (r0s < topk for every split)
    }
    MLA_DEVICE_ASM("" :: "v"(seq_raw));   // (loaded with the index entries, not sunk behind them)
    int rs[kDepth];
    if (p.bt) {
      const bool seq_ok = seq_raw >= 0 && seq_raw < p.bt_rows;
      const int32_t* btr = p.bt + (int64_t)(seq_ok ? seq_raw : 0) * p.bt_st;
      int bs[kDepth], pbs[kDepth];
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        const int v = vs[i] >= 0 ? vs[i] : 0;
        bs[i] = p.bs_log2 >= 0 ? v >> p.bs_log2 : v / p.bs;
        pbs[i] = btr[bs[i] < p.bt_cols ? bs[i] : p.bt_cols - 1];
      }
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        int r = -1;
        if (seq_ok && vs[i] >= 0 && bs[i] < p.bt_cols && pbs[i] >= 0) {
          const int64_t pr = (int64_t)pbs[i] * p.bs + (vs[i] - bs[i] * p.bs);
          r = pr < p.cache_rows ? (int)pr : -1;
        }
        rs[i] = r;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) rs[i] = (vs[i] >= 0 && vs[i] < p.cache_rows) ? vs[i] : -1;
    }
    // Every load of this branch is complete here.  An explicit wait: the
    // compiler's own waits, placed per use inside lane-masked blocks, leave
    // loads in flight in its model, and where their registers are reused
    // after the branch it would wait for all vector memory, the DMA included.
    wait_vmcnt<0>();
    bool ok = last >= 0;
#pragma unroll
    for (int i = 0; i < kDepth; ++i)
      if (myts > i && rs[i] < 0) ok = false;
    spec = __ballot(!ok) == 0;
    // P0: the DMA is issued only once the value waves have issued all their
    // prologue loads, which would otherwise queue behind it
    lds_barrier();
    if (spec) {
      static_for<0, kDepth>([&](auto I) {
        constexpr int i = decltype(I)::value;
        issue_from(myts > i ? p.cache + (uint64_t)(uint32_t)rs[i] * kRB : spare, i);
      });
    }
  } else {
    constexpr int kVT = kVW * 64;                               // 256 threads
    const int vt = tid - kSW * 64;
    int v8[kSlices];
    const int seq_raw = *seq_p;
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
      const int sl = i * kVT + vt;
      v8[i] = ip[sl < p.topk ? sl : p.topk - 1];
    }
    MLA_DEVICE_ASM("" :: "v"(seq_raw));   // (loaded with the index entries, not sunk behind them)
    // q of the workgroup's 32 heads: 2304 coalesced 16-byte chunks (chunk c:
    // head c / 72, dimensions 8 (c % 72) + [0,8); heads past H repeat the
    // last one), 9 per thread, loaded now (any later, the loads would queue
    // behind the first tiles' DMA) and staged in the still idle V buffer
    // below.
    constexpr int kQChunkAll = kHG * (kQK / 8);               // 2304
    constexpr int kQChunks = kQChunkAll / kVT;                // 9
    static_assert(kQChunks * kVT == kQChunkAll, "q chunks per value-wave thread");
    u32x4 qstage[kQChunks];     // raw fp16 / bf16 bits
    {
      const uint16_t* qt = reinterpret_cast<const uint16_t*>(p.q) + t * p.q_st;
#pragma unroll
      for (int m = 0; m < kQChunks; ++m) {
        const int c = vt + kVT * m;
        const int h = c / (kQK / 8), dc = c - h * (kQK / 8);
        const int head = min(g * kHG + h, p.H - 1);
        qstage[m] = *reinterpret_cast<const u32x4*>(qt + (int64_t)head * p.q_sh + 8 * dc);
      }
    }
#pragma unroll
    for (int i = 0; i < kSlices; ++i)
      if (i * kVT + vt >= p.topk) v8[i] = -1;

    int b8[kSlices], pb8[kSlices];
    const bool seq_ok = seq_raw >= 0 && seq_raw < p.bt_rows;
    if (p.bt) {
      const int32_t* btr = p.bt + (int64_t)(seq_ok ? seq_raw : 0) * p.bt_st;
      // (a power-of-two block size, the usual case, divides by a shift; one
      // uniform branch for all slots)
      if (p.bs_log2 >= 0) {
#pragma unroll
        for (int i = 0; i < kSlices; ++i) b8[i] = (v8[i] >= 0 ? v8[i] : 0) >> p.bs_log2;
      } else {
#pragma unroll
        for (int i = 0; i < kSlices; ++i) b8[i] = (v8[i] >= 0 ? v8[i] : 0) / p.bs;
      }
#pragma unroll
      for (int i = 0; i < kSlices; ++i) pb8[i] = btr[b8[i] < p.bt_cols ? b8[i] : p.bt_cols - 1];
    }
    lds_barrier();   // P0: this wave's prologue loads are issued (the score waves' DMA follows them)
    if (p.bt) {
#pragma unroll
      for (int i = 0; i < kSlices; ++i) {
        int r = -1;
        if (seq_ok && v8[i] >= 0 && b8[i] < p.bt_cols && pb8[i] >= 0) {
          const int64_t pr = (int64_t)pb8[i] * p.bs + (v8[i] - b8[i] * p.bs);
          r = pr < p.cache_rows ? (int)pr : -1;
        }
        rows8[i] = r;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSlices; ++i) rows8[i] = (v8[i] >= 0 && v8[i] < p.cache_rows) ? v8[i] : -1;
    }
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
      const uint64_t m = __ballot(rows8[i] >= 0);
      pre8[i] = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) cnt_s[i][wave - kSW] = __popcll(m);
    }
    // q into LDS in B-operand order, for the score waves' registers.  B
    // operand of K-step ks for head block hb, lane (r16, kg): q[hb*16 +
    // r16][d] with d(ks < 16) = 128kg + 8ks + [0,8) and d(16 + i) = 512 +
    // 16kg + 8i + [0,8), at 16-byte slot (hb * 18 + ks) * 64 + 16kg + r16.  A
    // negative softmax scale flips q's signs here (exact), so sm_log2 >= 0.
    const uint32_t qs = lds_off(vbuf_all);
#pragma unroll
    for (int m = 0; m < kQChunks; ++m) {
      const int c = vt + kVT * m;
      const int h = c / (kQK / 8), d = 8 * (c - h * (kQK / 8));
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
    wait_vmcnt<0>();   // (as in the score waves' branch)
  }
  lds_barrier();   // the slices' counts and the staged q are in LDS
  // Valid rows in slot order: slice i of value wave w starts after all of
  // slices 0 .. i-1 and slice i of value waves 0 .. w-1.  The counts are read
  // in assembly: the compiler cannot tell these reads from the speculative
  // DMA's LDS writes and would wait for that DMA first.
  int total = 0;
  {
    static_assert(kSlices == 8 && kVW == 4, "count reads below");
    u32x4 c[kSlices];
    MLA_DEVICE_ASM("ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:16\n\tds_read_b128 %2, %8 offset:32\n\t"
                   "ds_read_b128 %3, %8 offset:48\n\tds_read_b128 %4, %8 offset:64\n\tds_read_b128 %5, %8 offset:80\n\t"
                   "ds_read_b128 %6, %8 offset:96\n\tds_read_b128 %7, %8 offset:112\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(c[0]), "=v"(c[1]), "=v"(c[2]), "=v"(c[3]), "=v"(c[4]), "=v"(c[5]), "=v"(c[6]), "=v"(c[7])
                   : "v"(lds_off(&cnt_s[0][0])));
    int base[kSlices];
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
      base[i] = total;
#pragma unroll
      for (int w = 0; w < kVW; ++w) {
        if (w + kSW < wave) base[i] += (int)c[i][w];
        total += (int)c[i][w];
      }
    }
    if (wave >= kSW) {
#pragma unroll
      for (int i = 0; i < kSlices; ++i)
        if (rows8[i] >= 0) phys[base[i] + pre8[i]] = rows8[i];
    }
  }
  lds_barrier();

  // (total <= 2048 and S <= 64: the products fit in 32 bits)
  const int r0 = S == 1 ? 0 : (int)((uint32_t)(total * s) / (uint32_t)S);
  const int n = (S == 1 ? total : (int)((uint32_t)(total * (s + 1)) / (uint32_t)S)) - r0;
  const int ntiles = (n + kRowsT - 1) / kRowsT;
  const int rounds = (ntiles + kSW - 1) / kSW;
  const int my_tiles = wave < kSW && ntiles > sw ? (ntiles - sw + kSW - 1) / kSW : 0;

  // LDS address of the cache row of this lane's DMA row in the wave's i-th tile
  auto tile_row_addr = [&](int i) -> uint32_t {
    int e = (sw + kSW * i) * kRowsT + r16;
    e = e < n ? e : n - 1;
    return lds_off(&phys[r0 + e]);
  };

  // The first kDepth tiles' DMA from the compacted list, unless the
  // speculative DMA already holds them (every slot named a row: then the
  // compacted list is the slot list and r0, n are the speculated ones).  A
  // speculative DMA into the same slots completes first.
  if (wave < kSW && !(spec && total == p.topk)) {
    if (spec) wait_vmcnt<0>();
    static_for<0, kDepth>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const uint8_t* b = spare;
      if (my_tiles > i) b = p.cache + (uint64_t)(uint32_t)phys[r0 + min((sw + kSW * i) * kRowsT + r16, n - 1)] * kRB;
      issue_from(b, i);
    });
  }

  const float sm = p.sm_log2;
  const float out_mul = p.kv_scale * p.lat_scale;  // values carry the cache's per-tensor scale
  const int64_t H = p.H;
  // exchange region of value wave j (epilogue): j = 0, 1 in the ring area,
  // 2, 3 in the V area
  auto xregion = [&](int j) -> uint8_t* {
    return (j < 2 ? ring_all : reinterpret_cast<uint8_t*>(vbuf_all)) + (j & 1) * kXRegion;
  };
  if (wave < kSW) {
    // ============================================================ score wave
    // q's B operands into registers (inside this branch, so that they take
    // no registers on the value waves' path)
    half8_t qreg[2][kKSteps];
    {
      const uint32_t qa = lds_off(vbuf_all) + 16 * lane;
      static_for<0, 2 * kKSteps>([&](auto I) {
        constexpr int i = decltype(I)::value;
        qreg[i / kKSteps][i % kKSteps] = __builtin_bit_cast(half8_t, ring_b128<1024 * i>(qa));
      });
      MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) MLA_DEVICE_ASM("" : "+v"(qreg[hb][ks]));
    }
    lds_barrier();   // every score wave has its q before the V buffer is written
    const bool two_level = kFmt == kFmtNvfp4 && p.lat_scale != 1.0f;
    const RingOff<kFmt> ro(r16, kg);
    // this lane's V row (r16) and its 16 chunks from 16 kg: chunk tt at
    // byte vx ^ 16 tt (the row group is 256-byte aligned, and the swizzle
    // XORs the chunk index with vswz(r16)).  The writes are inline
    // ds_write_b128: as plain stores, the compiler could not tell them from
    // the ring DMA's LDS writes and would wait for that DMA first.
    const uint32_t vx = lds_off(vbuf_all + sw * kTileV + r16 * kVRow + 128 * kg) ^ (16u * vswz((uint32_t)r16));
    float mref[2] = {kNegInf, kNegInf};   // reference of head hb*16 + r16 (base 2)
    float lsum[2] = {0.0f, 0.0f};         // this lane's share of that head's row sum
    Raw<kFmt> raw;
    float4_t sacc[2];
    // (the score waves' instructions win issue arbitration against the value
    // waves' on the same SIMD: the score waves' chain sets the round time)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll 1
    for (int i = 0; i < rounds; ++i) {
      const bool have = i < my_tiles;     // (only the last round can miss a tile)
      const int k = sw + kSW * i;         // tile index within the split
      if (have) {
        // wait for this tile's DMA (the later tiles' stays in flight: a
        // wave's vector memory operations complete in issue order), read
        // its rows, then (FP8 rows) refill its slot with tile i + kDepth.
        // With value-wave refills, tiles 0 .. kDepth-1 come from this wave's
        // prologue DMA (always kDepth tiles, spare ones included) and later
        // ones are complete before the barrier that ended the last round.
        if constexpr (kVRefill) {
          if (i == 0) wait_vmcnt<(kDepth - 1) * kInstr>();
          else if (i == 1 && kDepth > 2) wait_vmcnt<(kDepth > 2 ? kDepth - 2 : 0) * kInstr>();
          else if (i < kDepth) wait_vmcnt<0>();
        } else {
          const int later = my_tiles - 1 - i;   // tiles issued after this one
          if (kDepth > 2 && later >= 2) wait_vmcnt<(kDepth > 2 ? 2 : 0) * kInstr>();
          else if (later >= 1) wait_vmcnt<kInstr>();
          else wait_vmcnt<0>();
        }
        const uint32_t sl = lds_off(ring + (i % kDepth) * kSlot);
        uint32_t next_row = lds_b32(tile_row_addr(i + kDepth));
        ring_read<kFmt>(raw, sl, ro, next_row);
        if constexpr (!kVRefill)
          if (i + kDepth < my_tiles) issue(next_row, i % kDepth);
        // rope first: its scores need no V-buffer space
#pragma unroll
        for (int ks = 16; ks < kKSteps; ++ks)
          score_mfma2(sacc, kstep8<kFmt>(raw, ks), qreg[0][ks], qreg[1][ks], ks == 16);
        if (two_level) scale_rope_scores(sacc, p.inv_lat_scale);
      }
      if (i > 0) lds_barrier();   // B(i-1): the value waves hold round i-1 in registers
      if (have) {
        // latent K-steps: the A operand of K-step t+1 is converted while
        // K-step t's two MFMAs run; each goes to the V buffer as well
        half2_t sh[4];
        if constexpr (kFmt == kFmtNvfp4) group_scales(sh, raw.sc);
        half8_t kop = latent8<kFmt>(raw, sh, 0);
        MLA_DEVICE_ASM("s_nop 1" : "+v"(kop));
        static_for<0, 16>([&](auto T) {
          constexpr int tt = decltype(T)::value;
          MLA_DEVICE_ASM("ds_write_b128 %0, %1" :: "v"(vx ^ (16u * tt)), "v"(kop) : "memory");
          __builtin_amdgcn_sched_barrier(0);
          score_mfma1(sacc[0], kop, qreg[0][tt]);
          __builtin_amdgcn_sched_barrier(0);
          half8_t nx;
          if constexpr (tt < 15) nx = latent8<kFmt>(raw, sh, tt + 1);
          __builtin_amdgcn_sched_barrier(0);
          score_mfma1(sacc[1], kop, qreg[1][tt]);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (tt < 15) kop = nx;
        });

        // softmax: the lane holds rows 4kg + j (j = 0..3) of head
        // hb*16 + r16; sm >= 0, so the scaled max is the max scaled.  Only
        // the split's last tile can hold rows past its end; they get P = 0.
        const int row0 = k * kRowsT + 4 * kg;
        const bool ragged = (k + 1) * kRowsT > n;
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
        const bool first = i == 0;
        const bool raise = tmax[0] > mref[0] + kLazy || tmax[1] > mref[1] + kLazy;
        if (first || __ballot(raise) != 0) {
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            float m = tmax[hb];
            m = __builtin_fmaxf(m, shfl_xor_f(m, 16));
            m = __builtin_fmaxf(m, shfl_xor_f(m, 32));
            const float mnew = __builtin_fmaxf(mref[hb], m) + kMargin;
            lsum[hb] *= first ? 0.0f : __builtin_amdgcn_exp2f(mref[hb] - mnew);
            mref[hb] = mnew;
          }
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const float nm = -mref[hb];
          float pv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[hb][j], sm, nm));
          if (ragged) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (row0 + j >= n) pv[j] = 0.0f;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) lsum[hb] += pv[j];
          const u32x2 d = {as_u32(__builtin_convertvector((float2_t){pv[0], pv[1]}, half2_t)),
                           as_u32(__builtin_convertvector((float2_t){pv[2], pv[3]}, half2_t))};
          *reinterpret_cast<u32x2*>(&pbuf[sw][hb * 16 + r16][4 * kg]) = d;
          if (kg == 0) ref_s[sw][hb * 16 + r16] = mref[hb];
        }
      }
      lds_barrier();   // A(i): round i's P, references and V are in LDS
    }
    if (rounds > 0) lds_barrier();   // B(rounds-1)
    __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();   // no DMA may still be writing this workgroup's LDS
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      lsum[hb] += shfl_xor_f(lsum[hb], 16);
      lsum[hb] += shfl_xor_f(lsum[hb], 32);
    }
    if (kg == 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        wml_s[hb * 16 + r16][sw] = mref[hb];
        wml_s[hb * 16 + r16][kSW + sw] = lsum[hb];
      }
    }
    lds_barrier();   // E: every score wave's (reference, row sum) is in LDS
  } else {
    // ============================================================ value wave
    lds_barrier();   // (the score waves' q reads)
    const int j = wave - kSW;
    const int hl = lane & 31;               // head of this lane's P operand
    float16_t acc[4];                       // O[32 heads x 32 cols] of column block 32c + [0,32), C layout
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    float M = kNegInf;                      // reference of O for head hl
    // V operand address (column block 0 of tile 0 of this wave's columns):
    // the ds_read_b64_tr_b16 pattern gives lane L rows 8 (L >> 5) + [0,4)
    // (and + [4,8) from the second read) of column L & 31
    const int vgrp = lane >> 4, vsl = lane & 15;
    const uint32_t vrow0 = 8 * (vgrp >> 1) + (vsl >> 2);
    const uint32_t vbyte = 32 * (vgrp & 1) + 8 * (vsl & 3) + 2 * kVCols * j;   // (unswizzled, in the row)
    const uint32_t vb = lds_off(vbuf_all) + vrow0 * (2 * kVRow) + 16 * ((vbyte >> 4) ^ vswz(vrow0)) + (vbyte & 15);
    const uint32_t pa_addr = lds_off(&pbuf[0][hl][8 * (lane >> 5)]);
    const uint32_t ref_addr = lds_off(&ref_s[0][hl]);
    const uint32_t fac_w = lds_off(&fac_s[j][hl]);
    const uint32_t fac_r = lds_off(&fac_s[j][4 * (lane >> 5)]);
    // factors of this lane's 16 accumulator heads (c_head) from fac_s[j]
    auto read_factors = [&](float (&f)[16]) {
      MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" ::: "memory");
      u32x4 v[4];
      MLA_DEVICE_ASM("ds_read_b128 %0, %1" : "=v"(v[0]) : "v"(fac_r));
      MLA_DEVICE_ASM("ds_read_b128 %0, %1 offset:32" : "=v"(v[1]) : "v"(fac_r));
      MLA_DEVICE_ASM("ds_read_b128 %0, %1 offset:64" : "=v"(v[2]) : "v"(fac_r));
      MLA_DEVICE_ASM("ds_read_b128 %0, %1 offset:96" : "=v"(v[3]) : "v"(fac_r));
      MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[4 * q + e] = __uint_as_float(v[q][e]);
    };
    // Refill R(m) (value-wave refills): tile j + kSW (m + kDepth) of score
    // wave j into its slot m % kDepth, issued right after A(m) (the score
    // wave read that slot in round m); the score wave reads it in round
    // m + kDepth, after A(m + kDepth - 1), before which this wave waits for it.
    const int mt_j = ntiles > j ? (ntiles - j + kSW - 1) / kSW : 0;   // score wave j's tiles
    uint8_t* const ring_j = ring_all + j * kWaveRing;
    auto refill_row_addr = [&](int m) -> uint32_t {
      const int e = (j + kSW * (m + kDepth)) * kRowsT + r16;
      return lds_off(&phys[r0 + (e < n ? e : n - 1)]);
    };
#pragma unroll 1
    for (int i = 0; i < rounds; ++i) {
      const int nt = ntiles - kSW * i < kSW ? ntiles - kSW * i : kSW;   // tiles in this round
      uint32_t refill_row = 0;
      if constexpr (kVRefill) {
        // R(i - 2) complete before A(i) (R(i - 1) may stay in flight)
        if (i >= 2) {
          if (i - 1 + kDepth < mt_j) wait_vmcnt<kInstr>();
          else wait_vmcnt<0>();
        }
        if (i + kDepth < mt_j) {
          refill_row = lds_b32(refill_row_addr(i));
          MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" : "+v"(refill_row));
        }
      }
      lds_barrier();   // A(i)
      half8_t pa[kSW];
      float mr[kSW];
      u32x4 bv[kSW][4];
      static_for<0, kSW>([&](auto W) {
        constexpr int w = decltype(W)::value;
        pa[w] = __builtin_bit_cast(half8_t, ring_b128<w * kHG * kPRow * 2>(pa_addr));
        mr[w] = __uint_as_float(lds_b32<w * kHG * 4>(ref_addr));
        read_v_tile<w>(bv[w], vb);
      });
      lds_barrier();   // B(i): waits for this wave's reads, then releases the buffers
      // (issued after B(i), in this wave's slack before A(i + 1))
      if constexpr (kVRefill)
        if (i + kDepth < mt_j) dma_tile(p.cache + (uint64_t)refill_row * kRB, ring_j + (i % kDepth) * kSlot);
#pragma unroll
      for (int w = 0; w < kSW; ++w)
        MLA_DEVICE_ASM("" : "+v"(pa[w]), "+v"(mr[w]), "+v"(bv[w][0]), "+v"(bv[w][1]), "+v"(bv[w][2]), "+v"(bv[w][3]));
      // O follows the largest reference of the round's tiles (per head)
      float mx = M;
#pragma unroll
      for (int w = 0; w < kSW; ++w)
        if (w < nt) mx = __builtin_fmaxf(mx, mr[w]);
      if (__ballot(mx > M) != 0) {
        const float f = mx > M ? (M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - mx)) : 1.0f;
        // (an assembly store: the compiler would make a plain LDS store wait
        // for this wave's refill DMA)
        if (lane < 32) MLA_DEVICE_ASM("ds_write_b32 %0, %1" :: "v"(fac_w), "v"(f) : "memory");
        float fo[16];
        read_factors(fo);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[c][e] *= fo[e];
        M = mx;
      }
      static_for<0, kSW>([&](auto W) {
        constexpr int w = decltype(W)::value;
        if (w < nt) {
          // P relative to M: a power of two, exact in FP16 above its subnormals
          const float f = __builtin_amdgcn_exp2f(mr[w] - M);
          if (__ballot(f != 1.0f) != 0) pa[w] = pa[w] * (half_t)f;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[w], __builtin_bit_cast(half8_t, bv[w][c]), acc[c],
                                                             0, 0, 0);
        }
      });
    }
    wait_vmcnt<0>();   // no refill DMA may still be writing this workgroup's LDS
    lds_barrier();   // E
    // weight of head h: 1 / L with L = sum_w 2^(m_w - M) l_w over the score
    // waves (whose references are all <= M); log2-sum-exp = M + log2 L
    float inv = 0.0f, lse2 = kNegInf;
    {
      const float4_t wm = *reinterpret_cast<const float4_t*>(&wml_s[hl][0]);
      const float4_t wl = *reinterpret_cast<const float4_t*>(&wml_s[hl][kSW]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < kSW; ++w)
        L += wm[w] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(wm[w] - M) * wl[w];
      if (M != kNegInf && L > 0.0f) {
        inv = 1.0f / L;
        lse2 = M + __log2f(L);
      }
    }
    if (j == 0 && lane < 32) {
      const int head = g * kHG + hl;
      if (S > 1) __hip_atomic_store(p.part_lse + (tg * S + s) * kHG + hl, lse2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (head < p.H && p.lse) p.lse[t * H + head] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
    }
    float fo[16];
    if (S > 1) {
      // S > 1: the normalised partial goes to memory in the order the MFMA
      // accumulators hold it: piece ((j * 4 + c) * 4 + e) * 64 + lane (8
      // bytes) holds heads 8e + 4 (lane >> 5) + [0,4) of column 128 j +
      // 32 c + (lane & 31), so each store instruction writes 512 contiguous
      // bytes and no exchange through LDS is needed.
      if (lane < 32) fac_s[j][hl] = inv;
      read_factors(fo);
      half_t* const pd = p.part_o + (tg * S + s) * (kHG * kLatent) + 4 * (j * 16 * 64 + lane);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          store4_agent(pd + 4 * 64 * (c * 4 + e), acc[c][4 * e] * fo[4 * e], acc[c][4 * e + 1] * fo[4 * e + 1],
                       acc[c][4 * e + 2] * fo[4 * e + 2], acc[c][4 * e + 3] * fo[4 * e + 3]);
    } else {
      // S == 1: normalise this wave's columns, then store them through its
      // exchange region: block (c * 4 + q) holds, in slot L, heads 8q +
      // 4(L >> 5) + [0,4) of column 32c + (L & 31); a reader takes heads
      // 4hq + [0,4) x columns 8co + [0,8) (8 consecutive slots of one block)
      // and stores 16-byte rows of 8 columns per head.
      if (lane < 32) fac_s[j][hl] = inv * out_mul;
      read_factors(fo);
      uint8_t* const xr = xregion(j);
      uint8_t* const xw = xr + 16 * lane + 32 * (lane >> 4);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4_t*>(xw + (c * 4 + q) * kXBlock) =
              (float4_t){acc[c][4 * q] * fo[4 * q], acc[c][4 * q + 1] * fo[4 * q + 1],
                         acc[c][4 * q + 2] * fo[4 * q + 2], acc[c][4 * q + 3] * fo[4 * q + 3]};
      MLA_DEVICE_ASM("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int hq = lane & 7, co = (lane >> 3) + 8 * u;
        const uint32_t rslot = 32 * (hq & 1) + 8 * (co & 3);
        const uint8_t* const src = xr + ((co >> 2) * 4 + (hq >> 1)) * kXBlock + 16 * rslot + 32 * (rslot >> 4);
        float o[4][8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float4_t v = *reinterpret_cast<const float4_t*>(src + 16 * x);
#pragma unroll
          for (int h = 0; h < 4; ++h) o[h][x] = v[h];
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int head = g * kHG + 4 * hq + h;
          if (head < p.H)
            store8<kBf16>(reinterpret_cast<uint16_t*>(p.out) + (t * H + head) * kLatent + kVCols * j + 8 * co, o[h]);
        }
      }
    }
  }
  if (S == 1) return;

  // Arrival and merge.  A split's partial (2,048 units of 16 bytes) is cut
  // into S slices, slice k = units [2048 k / S, 2048 (k + 1) / S), and split
  // k merges slice k, so that the merge's loads and arithmetic are spread
  // over the S workgroups instead of falling on one.  Per (token, head group)
  // the workspace holds 64 bytes: an arrival word (an epoch in the high 32
  // bits, the current call's arrivals in the low 32) and, for each epoch
  // parity, a mask of the slices whose owners merge them and a mask of those
  // whose owners left them.
  //   * Once every wave's partial stores are complete (each wave waits for
  //     its own; the barrier orders them before the count), thread 0 counts
  //     the split's arrival; the count returns the call's epoch E.
  //   * The last of the S arrivals moves the arrival word to (E + 1, 0) (the
  //     signal that every partial is complete, and the state the next call
  //     starts from), clears the next epoch's masks, and merges its own
  //     slice.  It then waits, a bounded number of polls, until every other
  //     owner has either taken or left its slice, and merges the slices that
  //     were left or are still undecided.
  //   * Every other split polls the arrival word, a bounded number of times,
  //     until its epoch moves past E; it then marks its slice taken and
  //     merges it, or else marks it left and merges nothing.
  // Every wait is bounded, and no workgroup depends on another being
  // resident: a slice is merged by its owner, by the last arrival, or (when
  // the last arrival stops waiting first) by both, which write the same
  // values.
  //
  // Why relaxed atomics suffice (AMDGPU memory model, GFX942/GFX950): an
  // agent-scope release is "buffer_wbl2 sc1" (write back the L2 lines that
  // plain stores left dirty) followed by "s_waitcnt vmcnt(0)".  Everything
  // this protocol publishes (partials and log2-sum-exps) is stored with the
  // agent-scope policy sc1, the one the model uses for agent-scope atomic
  // stores, so nothing of it is dirty in L2; the vmcnt wait below completes
  // those stores before the count, which is all that remains of the
  // release.  A merging split reads the results with agent-scope loads
  // (sc1), which see them without an acquire fence's cache invalidation:
  // they are issued only after the split has seen the epoch move (or was
  // the last arrival), which follows every split's count, each of which
  // follows the completion of that split's stores.  The masks only decide
  // who merges; a stale view of them costs at most a repeated merge.
  MLA_DEVICE_ASM("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint64_t* const state = reinterpret_cast<uint64_t*>(p.counters) + 8 * tg;   // 64 bytes per unit
  const uint64_t all = S == 64 ? ~0ull : (1ull << S) - 1ull;
  const bool shared_merge = p.merge_polls > 0;
  if (tid == 0) {
    const uint64_t old = __hip_atomic_fetch_add(state, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t epoch = (uint32_t)(old >> 32);
    uint64_t* const taken = state + 1 + (epoch & 1u), * const left = state + 3 + (epoch & 1u);
    int role = 0;   // 0: nothing to merge, 1: owner, 2: last arrival
    if ((uint32_t)old == (uint32_t)S - 1u) {
      __hip_atomic_store(state, (uint64_t)(epoch + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(state + 1 + ((epoch + 1u) & 1u), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(state + 3 + ((epoch + 1u) & 1u), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      role = 2;
    } else if (shared_merge) {
      bool moved = false;
      for (int i = 0; i < p.merge_polls && !moved; ++i) {
        __builtin_amdgcn_s_sleep(1);
        moved = (uint32_t)(__hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) != epoch;
      }
      __hip_atomic_fetch_or(moved ? taken : left, 1ull << s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      role = moved ? 1 : 0;
    }
    role_s = role;
    epoch_s = epoch;
  }
  __syncthreads();
  const int role = role_s;
  if (role == 0) return;

  // The merge of a range of units.  Unit u (16 bytes) of a partial holds
  // heads h0 = 8 e + 4 (m >> 4) + [0,4) (e = (u >> 5) & 3, m = u & 31) at
  // columns c0 = 128 (u >> 9) + 32 ((u >> 7) & 3) + 2 (m & 15) and c0 + 1
  // (bytes [0,8) and [8,16)).  A thread takes kNU consecutive units (kNU = 4:
  // the same four heads at eight consecutive columns, 64 contiguous bytes
  // per split) and, eight splits at a time with all of a batch in flight
  // together, loads each split's log2-sum-exps of the four heads and its
  // pieces of the units.  Per head it keeps the largest log2-sum-exp so far,
  // M, rescales what it has summed when M rises, and adds the pieces with
  // the weights 2^(lse - M) (splits in index order; an empty split, lse =
  // -inf, adds nothing).  Contraction is off, so that the same sums come out
  // whichever instance of this code, and whichever split, merges a unit.
  constexpr int kBatch = 8;
  const half_t* const pbase = p.part_o + tg * S * (kHG * kLatent);
  const float* const lbase = p.part_lse + tg * S * kHG;
  auto merge_range = [&](auto NUc, int ga, int gb) {   // unit groups [ga, gb) of kNU units
#pragma clang fp contract(off)
    constexpr int kNU = decltype(NUc)::value;
#pragma unroll 1
    for (int gi = ga + tid; gi < gb; gi += kThreads) {
      const int u = gi * kNU;
      const int h0 = 8 * ((u >> 5) & 3) + 4 * ((u >> 4) & 1);
      const int c0 = 128 * (u >> 9) + 32 * ((u >> 7) & 3) + 2 * (u & 15);
      float mx[4], sum[4], a[kNU][4][2];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        mx[h] = kNegInf;
        sum[h] = 0.0f;
#pragma unroll
        for (int i = 0; i < kNU; ++i) a[i][h][0] = a[i][h][1] = 0.0f;
      }
#pragma unroll 1
      for (int x0 = 0; x0 < S; x0 += kBatch) {
        u32x4 pv[kBatch][kNU], lv[kBatch];
        static_for<0, kBatch>([&](auto X) {
          constexpr int x = decltype(X)::value;
          if (x0 + x < S) {
            lv[x] = load16_agent(lbase + (x0 + x) * kHG + h0);
#pragma unroll
            for (int i = 0; i < kNU; ++i) pv[x][i] = load16_agent(pbase + ((x0 + x) * 2048 + u + i) * 8);
          }
        });
        MLA_DEVICE_ASM("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int x = 0; x < kBatch; ++x) {
          MLA_DEVICE_ASM("" : "+v"(lv[x]));
#pragma unroll
          for (int i = 0; i < kNU; ++i) MLA_DEVICE_ASM("" : "+v"(pv[x][i]));
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          float bm = mx[h];
#pragma unroll
          for (int x = 0; x < kBatch; ++x)
            if (x0 + x < S) bm = __builtin_fmaxf(bm, __uint_as_float(lv[x][h]));
          if (bm != kNegInf) {
            const float f = mx[h] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mx[h] - bm);
            sum[h] *= f;
#pragma unroll
            for (int i = 0; i < kNU; ++i) {
              a[i][h][0] *= f;
              a[i][h][1] *= f;
            }
#pragma unroll
            for (int x = 0; x < kBatch; ++x) {
              if (x0 + x < S) {
                const float w = __builtin_amdgcn_exp2f(__uint_as_float(lv[x][h]) - bm);
                sum[h] += w;
#pragma unroll
                for (int i = 0; i < kNU; ++i) {
                  const half8_t v = __builtin_bit_cast(half8_t, pv[x][i]);
                  a[i][h][0] = __builtin_fmaf(w, (float)v[h], a[i][h][0]);
                  a[i][h][1] = __builtin_fmaf(w, (float)v[4 + h], a[i][h][1]);
                }
              }
            }
            mx[h] = bm;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int head = g * kHG + h0 + h;
        if (head < p.H) {
          const float iv = mx[h] != kNegInf ? out_mul / sum[h] : 0.0f;
          uint16_t* const dst = reinterpret_cast<uint16_t*>(p.out) + (t * H + head) * kLatent + c0;
          if constexpr (kNU == 4) {
            const float o[8] = {a[0][h][0] * iv, a[0][h][1] * iv, a[1][h][0] * iv, a[1][h][1] * iv,
                                a[2][h][0] * iv, a[2][h][1] * iv, a[3][h][0] * iv, a[3][h][1] * iv};
            store8<kBf16>(dst, o);
          } else {
            static_assert(kNU == 1, "units per thread: 1 or 4");
            store2<kBf16>(dst, a[0][h][0] * iv, a[0][h][1] * iv);
          }
          if (c0 == 0 && p.lse) p.lse[t * H + head] = mx[h] != kNegInf ? (mx[h] + __log2f(sum[h])) * kLn2 : kNegInf;
        }
      }
    }
  };

  if (!shared_merge) {
    // the last arrival merges every unit, four per thread
    merge_range(std::integral_constant<int, 4>{}, 0, 2048 / 4);
    return;
  }

  // Shared merge: the owners' slices, then (the last arrival) the slices
  // left or still undecided.  One instance of the merge code for all of
  // them, so that every slice is combined by the same instructions
  // whoever merges it.
  uint64_t todo = 1ull << s;
  bool asked = role != 2;
#pragma unroll 1
  while (true) {
    if (todo == 0) {
      if (asked) break;
      asked = true;
      // The last arrival: wait until every other owner has taken or left
      // its slice (each decides within its own bounded polling), then merge
      // the slices left or still undecided.
      if (tid == 0) {
        const uint32_t epoch = epoch_s;
        const uint64_t* const taken = state + 1 + (epoch & 1u), * const left = state + 3 + (epoch & 1u);
        const uint64_t others = all & ~(1ull << s);
        uint64_t t_m = 0, l_m = 0;
        for (int i = 0; i < 4 * p.merge_polls + 64; ++i) {
          t_m = __hip_atomic_load(taken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          l_m = __hip_atomic_load(left, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (((t_m | l_m) & others) == others) break;
          __builtin_amdgcn_s_sleep(1);
        }
        won_s = others & ~(t_m & ~l_m);
      }
      __syncthreads();
      todo = won_s;
      continue;
    }
    const int k = __builtin_ctzll(todo);
    todo &= todo - 1;
    merge_range(std::integral_constant<int, 1>{}, (2048 * k) / S, (2048 * (k + 1)) / S);
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// ------------------------------------------------------------------ host side

namespace {

constexpr int kMinSharedMergeSplits = 4;

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
  // keeps at least 256 valid rows (four rounds of tiles) so its fixed costs
  // (index compaction, q staging, split merge) stay small.
  int64_t s = cus / groups;
  int64_t max_by_rows = topk / 256;
  if (max_by_rows < 1) max_by_rows = 1;
  if (s > max_by_rows) s = max_by_rows;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  // One split fewer when that lets every unit's splits share an XCD in a
  // single round of resident workgroups (launch_decode groups them then:
  // the merge's reads and the shared q and index reads go through one L2).
  // Measured at 35 tokens: 6 grouped splits 22.3 us, 7 ungrouped 22.9 us.
  const int64_t per_xcd = cus >= 8 ? cus / 8 : 1, unit_rows = (groups + 7) / 8;
  if (s > 2 && unit_rows * s > per_xcd && unit_rows * (s - 1) <= per_xcd) s -= 1;
  return (int)s;
}

size_t decode_workspace_bytes(int64_t T, int H, int S) {
  const int G = H <= kHG ? 1 : H / kHG;
  const int64_t tg = T * G;
  // per (token, head group): 64 bytes of arrival state (arrival word, and
  // the taken and left masks of both epoch parities)
  size_t ctr = (size_t)tg * 64;
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
  // A split waits for the others only if the whole grid can be resident at
  // once (one workgroup per CU); otherwise a waiting split could hold a CU
  // that a later split needs, so none waits and the last arrival merges all.
  if (blocks > cus) a.merge_polls = 0;
  // With few splits the merge is small and a shared one costs more (the
  // owners' wait for the last arrival) than it spreads: the last arrival
  // merges everything in one pass.
  if (p.S < kMinSharedMergeSplits) a.merge_polls = 0;
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
