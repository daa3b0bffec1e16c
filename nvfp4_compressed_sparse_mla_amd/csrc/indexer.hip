// Sparse indexer (gfx950): exact scores of every visible cached position and
// the per-token top-k position list the decode consumes.
//
// What is computed (Prime Inference write-up, "A native NVFP4 sparse-MLA
// decode kernel": the decode reads the positions a sparse indexer selected;
// wireai.ir article, 4-bit-caches section, third decision: a fixed-width list
// of up to 2048 positions with padded slots).  The pages give no scoring
// formula; the library takes the plainest one: a 128-value E4M3 key per
// cached position, a 128-value E4M3 query per token, score = their dot
// product, computed exactly (every E4M3 product is a multiple of 2^-18 and
// 128 of them sum to less than 2^25, so FP64 holds every partial sum exactly,
// in any order).  A token's list holds the min(k, n) best of its n candidate
// positions (0 .. ctx-1 that name a key row), equal scores to the smaller
// position, in ascending position order, padded with -1.
//
//   score kernel   workgroup = (token, chunk of 1024 positions); 8 lanes per
//                  position, each with 16 of the 128 dimensions (one 16-byte
//                  load; a wave's load covers 8 consecutive rows), FP64
//                  products and sums, a 3-step lane reduction.  The score
//                  becomes a 64-bit key whose unsigned order is the score's
//                  order (0 marks a position that is not a candidate); its
//                  top 12 bits (the score's sign and exponent) are counted
//                  in a per-token histogram.
//   Contexts up to 32768 positions take the select kernel, longer ones the
//   compact and finish kernels; both give the same lists.
//   select kernel  one workgroup per token: radix select on all its keys.
//                  The histogram names the 12-bit bucket that holds the k-th
//                  best key; while that bucket holds more keys than are
//                  still needed, one pass over the token's keys histograms
//                  the next 12 bits of the keys in it.  A last pass over the
//                  positions in order writes every key above the bucket and
//                  the first still-needed keys inside it, then pads.
//   compact kernel workgroup = (token, chunk of 8192 positions).  From the
//                  histogram it finds the 12-bit bucket b that holds the
//                  k-th best key (every workgroup of the token finds the same
//                  one).  Each thread takes 32 consecutive positions: keys
//                  above b set their bit in the token's selection bitmap (one
//                  word per thread, plain stores); keys inside b are appended
//                  to the token's candidate list (one atomic per workgroup).
//   finish kernel  one workgroup per token: a radix select over the
//                  candidates only (12 more bits per pass, through all 64 if
//                  ties demand) marks the ones that make the list; keys equal
//                  to the k-th best one are marked in a tie bitmap and the
//                  first still-needed of them in position order are taken
//                  (equal keys are equal scores, so the smaller positions come
//                  first).  A last pass over the bitmaps in word order writes
//                  the selected positions in ascending order, then pads.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

namespace {

constexpr int kIdxDim = 128;
constexpr int kChunk = 1024;              // positions per score workgroup
constexpr int kBins = 1 << kIdxHistBits;  // 4096
constexpr int kSelThreads = 1024;
constexpr int kShortCtx = 32768;      // contexts up to this use the one-workgroup select

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Order-preserving key of an exact score: larger score <=> larger key;
// -0 and +0 give the same key; no finite score gives 0.
__device__ __forceinline__ uint64_t score_key(double s) {
  s += 0.0;                                     // -0 -> +0
  const uint64_t b = (uint64_t)__double_as_longlong(s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// First-level bucket of a key: its top 12 bits (the score's sign and
// exponent), so that the keys of one bucket share those 12 bits.
constexpr int kPrefixBits = kIdxHistBits;
__device__ __forceinline__ uint32_t key_bucket(uint64_t key) { return (uint32_t)(key >> (64 - kPrefixBits)); }
__device__ __forceinline__ uint64_t bucket_prefix(uint32_t b) { return b; }

// Key row of position pos of token t, or -1 if it names none.
__device__ __forceinline__ int64_t key_row(const IndexerParams& p, int64_t base, int64_t seq, int pos) {
  if (!p.bt) {
    const int64_t r = base + pos;
    return (r >= 0 && r < p.key_rows) ? r : -1;
  }
  if (seq < 0 || seq >= p.bt_rows) return -1;
  const int blk = p.bs_log2 >= 0 ? pos >> p.bs_log2 : pos / p.bs;
  if (blk >= p.bt_cols) return -1;
  const int e = p.bt[seq * p.bt_st + blk];
  if (e < 0) return -1;
  const int64_t r = (int64_t)e * p.bs + (pos - blk * p.bs);
  return r < p.key_rows ? r : -1;
}

__device__ __forceinline__ int token_ctx(const IndexerParams& p, int64_t t) {
  const int c = p.ctx[t];
  return c < 0 ? 0 : (c > p.max_ctx ? p.max_ctx : c);
}

// 16 E4M3 bytes -> 16 doubles (exact: the conversions apply scale 1.0)
__device__ __forceinline__ void e4m3x16_to_f64(const u32x4& w, double (&d)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, false);
    const float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, true);
    d[4 * i] = (double)a.x;
    d[4 * i + 1] = (double)a.y;
    d[4 * i + 2] = (double)b.x;
    d[4 * i + 3] = (double)b.y;
  }
}

// Inclusive prefix sum over the NT threads of a workgroup in thread order.
// `ws` holds NT / 64 words of scratch; all threads must call.
template <int NT = kSelThreads>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* ws) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)v, d, 64);
    if (lane >= d) v += u;
  }
  if (lane == 63) ws[w] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i)
    if (i < w) add += ws[i];
  __syncthreads();
  return v + add;
}

// The bucket of a histogram (nbins <= 4096 bins in LDS, larger bins hold
// larger keys) that holds the need_in-th largest key, need_in >= 1 and at
// most the histogram's total: out[0] = the bucket, out[1] = keys in the
// buckets above it, out[2] = keys in it.  Thread i owns the bins
// nbins - 1 - (per i + j), j = 0 .. per-1, so the scan in thread order counts
// keys from the top.  All threads must call; out is valid on return.
template <int NT>
__device__ __forceinline__ void top_bucket(const uint32_t* hist, int nbins, uint32_t need_in, uint32_t* ws,
                                           uint32_t* out) {
  constexpr int kPer = kBins / NT;
  const int hi = nbins - 1 - kPer * (int)threadIdx.x;
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) v += (hi - j >= 0) ? hist[hi - j] : 0u;
  const uint32_t incl = block_scan<NT>(v, ws);
  uint32_t excl = incl - v;
  if (excl < need_in && need_in <= incl) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t h = (hi - j >= 0) ? hist[hi - j] : 0u;
      if (excl + h >= need_in) {
        out[0] = (uint32_t)(hi - j);
        out[1] = excl;
        out[2] = h;
        break;
      }
      excl += h;
    }
  }
  __syncthreads();
}

// N consecutive keys from position i (a multiple of N, N even; the keys
// array is 16-byte aligned), 0 past ctx (0 marks "not a candidate").
template <int N>
__device__ __forceinline__ void load_keys(const uint64_t* keys, int i, int ctx, uint64_t (&k)[N]) {
  if (i + N <= ctx) {
#pragma unroll
    for (int j = 0; j < N; j += 2) {
      const u64x2 v = *reinterpret_cast<const u64x2*>(keys + i + j);
      k[j] = v[0];
      k[j + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) k[j] = i + j < ctx ? keys[i + j] : 0ull;
  }
}

}  // namespace

__global__ __launch_bounds__(256) void indexer_score_kernel(IndexerParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ int64_t rows_s[kChunk];   // key row of each position of the chunk (-1: none)
  const uint32_t nch = (uint32_t)p.nchunks;
  const uint32_t t32 = blockIdx.x / nch;
  const int c = (int)(blockIdx.x - t32 * nch);
  const int64_t t = t32;
  const int ctx = token_ctx(p, t);
  const int p0 = c * kChunk;
  if (p0 >= ctx) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, sub = lane & 7;
  for (int i = tid; i < kBins; i += 256) hist[i] = 0;

  double q[16];
  const uint8_t* const qrow = p.q + t * p.q_st + 16 * sub;
  e4m3x16_to_f64(*reinterpret_cast<const u32x4*>(qrow), q);
  const int64_t base = p.bt ? 0 : p.base[t];
  const int64_t seq = p.bt ? (int64_t)p.tok_seq[t] : 0;
  uint64_t* const kout = p.keys_ws + t * p.key_stride;

  // The key row of every position of the chunk, 4 per thread, their
  // block-table loads issued together (the keys' loads below then depend on
  // no other global load).
  {
    constexpr int kPer = kChunk / 256;
    int64_t rr[kPer];
    if (p.bt) {
      const bool seq_ok = seq >= 0 && seq < p.bt_rows;
      const int32_t* const btr = p.bt + (seq_ok ? seq : 0) * p.bt_st;
      int blk[kPer], e[kPer];
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int pos = p0 + tid + 256 * m;
        blk[m] = p.bs_log2 >= 0 ? pos >> p.bs_log2 : pos / p.bs;
        e[m] = btr[blk[m] < p.bt_cols ? blk[m] : p.bt_cols - 1];
      }
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int pos = p0 + tid + 256 * m;
        int64_t r = -1;
        if (pos < ctx && seq_ok && blk[m] < p.bt_cols && e[m] >= 0) {
          r = (int64_t)e[m] * p.bs + (pos - blk[m] * p.bs);
          if (r >= p.key_rows) r = -1;
        }
        rr[m] = r;
      }
    } else {
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int pos = p0 + tid + 256 * m;
        const int64_t r = base + pos;
        rr[m] = (pos < ctx && r >= 0 && r < p.key_rows) ? r : -1;
      }
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) rows_s[tid + 256 * m] = rr[m];
  }
  __syncthreads();

  // wave w takes positions p0 + kWavePos w + 8 i + (lane >> 3), four i at a
  // time; the next four's keys are loaded while these are scored
  constexpr int kWavePos = kChunk / 4;
  constexpr int kUnroll = 4;
  constexpr int kIters = kWavePos / 8 / kUnroll;
  auto fetch = [&](int it, u32x4 (&raw)[kUnroll], bool (&ok)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int off = kWavePos * wave + 8 * (it * kUnroll + u) + (lane >> 3);
      const int64_t r = rows_s[off];
      ok[u] = r >= 0;
      // (a position without a key reads q's row, a valid address, and drops it)
      raw[u] = *reinterpret_cast<const u32x4*>(ok[u] ? p.keys + r * kIdxDim + 16 * sub : qrow);
    }
  };
  u32x4 nraw[kUnroll];
  bool nok[kUnroll];
  fetch(0, nraw, nok);
  for (int it = 0; it < kIters; ++it) {
    u32x4 raw[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      raw[u] = nraw[u];
      ok[u] = nok[u];
    }
    if (it + 1 < kIters) fetch(it + 1, nraw, nok);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int pos = p0 + kWavePos * wave + 8 * (it * kUnroll + u) + (lane >> 3);
      double k[16];
      e4m3x16_to_f64(ok[u] ? raw[u] : (u32x4){0, 0, 0, 0}, k);
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < 16; ++j) s = __builtin_fma(q[j], k[j], s);   // exact (see above)
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (sub == 0 && pos < ctx) {
        const uint64_t key = ok[u] ? score_key(s) : 0ull;
        kout[pos] = key;
        if (key) atomicAdd(&hist[key_bucket(key)], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* const g = p.hist + t * kBins;
  for (int i = tid; i < kBins; i += 256)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__global__ __launch_bounds__(kSelThreads) void indexer_select_kernel(IndexerParams p) {
  __shared__ __align__(16) uint32_t hist[kBins];
  __shared__ uint32_t ws[kSelThreads / 64];
  __shared__ uint32_t sh_bin, sh_above, sh_cnt, sh_tot;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int ctx = token_ctx(p, t);
  const uint64_t* const keys = p.keys_ws + t * p.key_stride;
  int32_t* const out = p.out + t * p.out_st;
  const int64_t out_base = p.bt ? 0 : p.base[t];

  // the score kernel's histogram of the top 12 bits (one 16-byte load per
  // thread); zero it for the next call
  static_assert(kBins == 4 * kSelThreads, "histogram words per thread");
  uint32_t mine = 0;
  {
    u32x4* const g = reinterpret_cast<u32x4*>(p.hist + t * kBins);
    const u32x4 h = g[tid];
    g[tid] = (u32x4){0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(hist)[tid] = h;
    mine = h[0] + h[1] + h[2] + h[3];
  }
  const uint32_t total = block_scan(mine, ws);
  if (tid == kSelThreads - 1) sh_tot = total;
  __syncthreads();
  const uint32_t n_cand = sh_tot;
  const uint32_t need = n_cand < (uint32_t)p.topk ? n_cand : (uint32_t)p.topk;
  const bool all = need == n_cand;            // every candidate is selected

  // Find the bucket b of the histogram (bins of `bits` bits) holding the
  // need_in-th best key: thread i owns bins 4 (1023 - i) + 3 .. + 0, so the
  // scan in thread order counts keys from the top.
  auto find_bin = [&](uint32_t need_in, int nbins) {
    const int hi = 4 * (kSelThreads - 1 - tid);
    uint32_t v = 0;
#pragma unroll
    for (int j = 3; j >= 0; --j) v += (hi + j < nbins) ? hist[hi + j] : 0u;
    const uint32_t incl = block_scan(v, ws);
    uint32_t excl = incl - v;
    if (excl < need_in && need_in <= incl) {
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const uint32_t h = (hi + j < nbins) ? hist[hi + j] : 0u;
        if (excl + h >= need_in) {
          sh_bin = (uint32_t)(hi + j);
          sh_above = excl;
          sh_cnt = h;
          break;
        }
        excl += h;
      }
    }
    __syncthreads();
  };

  uint64_t prefix = 0;
  int pbits = 0;
  uint32_t need_in = need;
  if (!all) {
    find_bin(need_in, kBins);
    prefix = bucket_prefix(sh_bin);
    pbits = kPrefixBits;
    need_in -= sh_above;
    uint32_t cnt = sh_cnt;
    // refine while the bucket holds more keys than are still needed
    while (cnt > need_in && pbits < 64) {
      const int d = 64 - pbits < kIdxHistBits ? 64 - pbits : kIdxHistBits;
      for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0u;
      __syncthreads();
      constexpr int kR = 8;   // keys per thread and pass iteration
      for (int i = kR * tid; i < ctx; i += kR * kSelThreads) {
        uint64_t kk[kR];
        load_keys<kR>(keys, i, ctx, kk);
#pragma unroll
        for (int j = 0; j < kR; ++j) {
          const uint64_t k = kk[j];
          if (k && (k >> (64 - pbits)) == prefix)
            atomicAdd(&hist[(uint32_t)(k >> (64 - pbits - d)) & ((1u << d) - 1u)], 1u);
        }
      }
      __syncthreads();
      find_bin(need_in, 1 << d);
      prefix = (prefix << d) | sh_bin;
      pbits += d;
      need_in -= sh_above;
      cnt = sh_cnt;
    }
  }

  // Emit in position order: thread i takes positions kE i .. kE i + kE - 1
  // of each block of kE * 1024.  A key is selected if it is above the
  // bucket, or inside it among the first need_in in position order.
  constexpr int kE = 16;
  uint32_t run_tie = 0, run_sel = 0;
  for (int blk = 0; blk < ctx; blk += kE * kSelThreads) {
    const int p4 = blk + kE * tid;
    uint64_t k[kE];
    load_keys<kE>(keys, p4, ctx, k);
    bool above[kE], tie[kE];
    uint32_t ntie = 0;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      if (all) {
        above[j] = k[j] != 0ull;
        tie[j] = false;
      } else {
        const uint64_t top = pbits == 64 ? k[j] : k[j] >> (64 - pbits);
        above[j] = k[j] != 0ull && top > prefix;
        tie[j] = k[j] != 0ull && top == prefix;
      }
      ntie += tie[j];
    }
    const uint32_t tie_incl = block_scan(ntie, ws);
    uint32_t rank = run_tie + tie_incl - ntie;
    bool sel[kE];
    uint32_t nsel = 0;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      sel[j] = above[j] || (tie[j] && rank < need_in);
      rank += tie[j];
      nsel += sel[j];
    }
    const uint32_t sel_incl = block_scan(nsel, ws);
    uint32_t o = run_sel + sel_incl - nsel;
#pragma unroll
    for (int j = 0; j < kE; ++j)
      if (sel[j]) out[o++] = (int32_t)(out_base + p4 + j);
    if (tid == kSelThreads - 1) {
      sh_tot = tie_incl;
      sh_cnt = sel_incl;
    }
    __syncthreads();
    run_tie += sh_tot;
    run_sel += sh_cnt;
    __syncthreads();
  }
  for (int i = (int)need + tid; i < p.topk; i += kSelThreads) out[i] = -1;
}

constexpr int kCT = 256;              // compact kernel threads
constexpr int kCPos = 32 * kCT;       // positions per compact workgroup (one bitmap word per thread)

// The k-th best key's 12-bit bucket from the token's histogram (in LDS):
// sh[0] = bucket, sh[1] = keys above it, sh[3] = all candidate keys.  `all`
// when every candidate makes the list (then no bucket is needed).
template <int NT>
__device__ __forceinline__ void threshold_bucket(const uint32_t* hist, uint32_t* ws, uint32_t* sh, int topk,
                                                 uint32_t& need, bool& all) {
  constexpr int kPer = kBins / NT;
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) mine += hist[kPer * (int)threadIdx.x + j];
  const uint32_t total = block_scan<NT>(mine, ws);
  if ((int)threadIdx.x == NT - 1) sh[3] = total;
  __syncthreads();
  const uint32_t n_cand = sh[3];
  need = n_cand < (uint32_t)topk ? n_cand : (uint32_t)topk;
  all = need == n_cand;
  if (!all) top_bucket<NT>(hist, kBins, need, ws, sh);
}

__global__ __launch_bounds__(kCT) void indexer_compact_kernel(IndexerParams p) {
  __shared__ __align__(16) uint32_t hist[kBins];
  __shared__ uint32_t ws[kCT / 64];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t base_s;
  const uint32_t ncc = (uint32_t)p.cchunks;
  const uint32_t t32 = blockIdx.x / ncc;
  const int c = (int)(blockIdx.x - t32 * ncc);
  const int64_t t = t32;
  const int ctx = token_ctx(p, t);
  const int p0 = c * kCPos;
  if (p0 >= ctx) return;
  const int tid = threadIdx.x;
  // 32 consecutive positions per thread (one selection-bitmap word); their
  // keys are loaded while the histogram is scanned
  const int pp = p0 + 32 * tid;
  const uint64_t* const keys = p.keys_ws + t * p.key_stride;
  uint64_t k[32];
  load_keys<32>(keys, pp, ctx, k);
  // the token's histogram: 16-byte loads, all issued before any is used
  // (one at a time, each would be a dependent round trip to memory)
  {
    constexpr int kPer = kBins / (4 * kCT);
    static_assert(kPer * 4 * kCT == kBins, "histogram words per thread");
    const u32x4* const g = reinterpret_cast<const u32x4*>(p.hist + t * kBins);
    u32x4 hv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) hv[j] = g[tid + kCT * j];
#pragma unroll
    for (int j = 0; j < kPer; ++j) reinterpret_cast<u32x4*>(hist)[tid + kCT * j] = hv[j];
  }
  __syncthreads();
  uint32_t need;
  bool all;
  threshold_bucket<kCT>(hist, ws, sh, p.topk, need, all);
  // keys of bucket b share their top bits: compare those with b's
  const uint64_t pstar = all ? 0 : bucket_prefix(sh[0]);

  uint32_t sel = 0, cm = 0;   // selected / candidate bits of the 32 positions
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint64_t top = k[j] >> (64 - kPrefixBits);
    if (k[j] && (all || top > pstar)) sel |= 1u << j;
    if (k[j] && !all && top == pstar) cm |= 1u << j;
  }
  const uint32_t nc = __popc(cm);
  if (pp < ctx) {
    p.sel_bits[t * p.word_stride + (pp >> 5)] = sel;
    p.tie_bits[t * p.word_stride + (pp >> 5)] = 0u;
  }
  // the bucket's keys join the token's candidate list
  const uint32_t incl = block_scan<kCT>(nc, ws);
  if (tid == kCT - 1) base_s = incl ? atomicAdd(&p.cand_n[t], incl) : 0u;
  __syncthreads();
  if (nc) {
    uint32_t o = base_s + incl - nc;
    uint64_t* const ck = p.cand_key + t * p.key_stride;
    uint32_t* const cp = p.cand_pos + t * p.key_stride;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if ((cm >> j) & 1u) {
        ck[o] = k[j];
        cp[o] = (uint32_t)(pp + j);
        ++o;
      }
    }
  }
}

// a bitmap word written by an earlier kernel or by this kernel's atomics,
// read at the device-coherent level
__device__ __forceinline__ uint32_t word_at(const uint32_t* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kCandCache = 11776;     // candidates the finish kernel keeps in LDS (with the histogram, < 160 KB)
constexpr int kEmitWords = 8;         // bitmap words per thread held in registers by the ordered emit

__global__ __launch_bounds__(kSelThreads) void indexer_finish_kernel(IndexerParams p) {
  __shared__ __align__(16) uint32_t hist[kBins];
  __shared__ uint64_t ck_s[kCandCache];
  __shared__ uint32_t cp_s[kCandCache];
  __shared__ uint32_t ws[kSelThreads / 64];
  __shared__ uint32_t sh[4];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int ctx = token_ctx(p, t);
  int32_t* const out = p.out + t * p.out_st;
  const int64_t out_base = p.bt ? 0 : p.base[t];

  // The token's histogram (one 16-byte load per thread), zeroed for the
  // next call.  Every global read of this kernel is issued in batches:
  // one at a time, each would be a dependent round trip to memory.
  static_assert(kBins == 4 * kSelThreads, "histogram words per thread");
  {
    u32x4* const g = reinterpret_cast<u32x4*>(p.hist + t * kBins);
    const u32x4 h = g[tid];
    g[tid] = (u32x4){0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(hist)[tid] = h;
  }
  const uint32_t n_c = p.cand_n[t];
  __syncthreads();
  if (tid == 0) p.cand_n[t] = 0u;
  uint32_t need;
  bool all;
  threshold_bucket<kSelThreads>(hist, ws, sh, p.topk, need, all);

  // Radix select among the candidates (the keys of bucket b): refine while
  // the bucket holds more keys than are still needed.  Up to kCandCache
  // candidates are read once into LDS; more are read from the workspace
  // in every pass.
  const uint64_t* const gk = p.cand_key + t * p.key_stride;
  const uint32_t* const gp = p.cand_pos + t * p.key_stride;
  const bool cached = n_c <= (uint32_t)kCandCache;
  constexpr int kU = 8;                 // candidates per thread per batch
  // (indices past the list are clamped to its last entry, so that every
  // load of a batch is issued unconditionally; their results are dropped)
  auto cand_index = [&](uint32_t i) -> uint32_t { return i < n_c ? i : n_c - 1u; };
  if (cached && !all)
    for (uint32_t i0 = 0; i0 < n_c; i0 += kU * kSelThreads) {
      uint64_t kk[kU];
      uint32_t pp[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t i = cand_index(i0 + u * kSelThreads + tid);
        kk[u] = gk[i];
        pp[u] = gp[i];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t i = i0 + u * kSelThreads + tid;
        if (i < n_c) {
          ck_s[i] = kk[u];
          cp_s[i] = pp[u];
        }
      }
    }
  __syncthreads();
  // f(key, position) for every candidate, in batches
  auto for_candidates = [&](auto&& f) {
    if (cached) {
      for (uint32_t i = tid; i < n_c; i += kSelThreads) f(ck_s[i], cp_s[i]);
    } else {
      for (uint32_t i0 = 0; i0 < n_c; i0 += kU * kSelThreads) {
        uint64_t kk[kU];
        uint32_t pp[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint32_t i = cand_index(i0 + u * kSelThreads + tid);
          kk[u] = gk[i];
          pp[u] = gp[i];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (i0 + u * kSelThreads + tid < n_c) f(kk[u], pp[u]);
      }
    }
  };
  uint64_t prefix = 0;
  int pbits = kPrefixBits;
  uint32_t need_in = 0, cnt = 0;
  if (!all) {
    prefix = bucket_prefix(sh[0]);
    need_in = need - sh[1];
    cnt = sh[2];
    while (cnt > need_in && pbits < 64) {
      const int d = 64 - pbits < kIdxHistBits ? 64 - pbits : kIdxHistBits;
      for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0u;
      __syncthreads();
      for_candidates([&](uint64_t k, uint32_t) {
        if ((k >> (64 - pbits)) == prefix)
          atomicAdd(&hist[(uint32_t)(k >> (64 - pbits - d)) & ((1u << d) - 1u)], 1u);
      });
      __syncthreads();
      top_bucket<kSelThreads>(hist, 1 << d, need_in, ws, sh);
      prefix = (prefix << d) | sh[0];
      pbits += d;
      need_in -= sh[1];
      cnt = sh[2];
    }
  }
  // Keys above the final bucket are in; so is the whole bucket if it holds
  // exactly the keys still needed; otherwise (all 64 bits equal) its keys
  // are ties, of which the need_in first in position order are in.
  const bool ties = !all && cnt > need_in;
  uint32_t* const sb = p.sel_bits + t * p.word_stride;
  uint32_t* const tb = p.tie_bits + t * p.word_stride;
  if (!all)
    for_candidates([&](uint64_t k, uint32_t pos) {
      const uint64_t top = pbits == 64 ? k : k >> (64 - pbits);
      if (top > prefix || (top == prefix && !ties)) atomicOr(&sb[pos >> 5], 1u << (pos & 31));
      else if (top == prefix) atomicOr(&tb[pos >> 5], 1u << (pos & 31));
    });
  // Every reader of the bitmaps is in this workgroup: the barrier's wait for
  // this workgroup's atomics suffices (a device-scope fence would also write
  // back this XCD's L2)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();

  // Ordered emit: thread i takes words [per i, per (i+1)) of the bitmaps,
  // read once (kEmitWords at a time) for its tie count, its selected count
  // and the writes.  Word w's selected positions: its selection bits and,
  // of its tie bits, the lowest (need_in - rank) ones (rank = ties in
  // earlier words).
  const int nw = (ctx + 31) >> 5;
  const int per = (nw + kSelThreads - 1) / kSelThreads;
  const int w0 = per * tid, w1 = min(w0 + per, nw);
  auto selected = [&](uint32_t s, uint32_t tw, uint32_t& rank) -> uint32_t {
    if (ties) {
      uint32_t take = rank < need_in ? need_in - rank : 0u;
      rank += __popc(tw);
      while (tw && take) {
        const uint32_t lo = tw & (0u - tw);
        s |= lo;
        tw ^= lo;
        --take;
      }
    }
    return s;
  };
  uint32_t sw_r[kEmitWords], tw_r[kEmitWords];
  // (words past the thread's range are read at a clamped address and
  // dropped, so that every load is issued unconditionally; nw >= 1 here)
  auto load_words = [&](int wa) {
#pragma unroll
    for (int u = 0; u < kEmitWords; ++u) {
      const int w = wa + u;
      const int wc = w < nw ? w : nw - 1;
      sw_r[u] = word_at(&sb[wc]);
      tw_r[u] = ties ? word_at(&tb[wc]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kEmitWords; ++u)
      if (wa + u >= w1) sw_r[u] = tw_r[u] = 0u;
  };
  const bool in_regs = per <= kEmitWords;   // (contexts up to 8 * 32 * 1024 positions)
  if (in_regs && nw > 0) load_words(w0);
  uint32_t my_ties = 0;
  if (ties) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kEmitWords; ++u) my_ties += __popc(tw_r[u]);
    } else {
      for (int wa = w0; wa < w1; wa += kEmitWords) {
        load_words(wa);
#pragma unroll
        for (int u = 0; u < kEmitWords; ++u) my_ties += __popc(tw_r[u]);
      }
    }
  }
  const uint32_t tie_incl = ties ? block_scan<kSelThreads>(my_ties, ws) : 0u;
  const uint32_t tie_rank0 = tie_incl - my_ties;   // ties in earlier threads' words
  uint32_t my_sel = 0;
  {
    uint32_t rank = tie_rank0;
    for (int wa = w0; wa < w1; wa += kEmitWords) {
      if (!in_regs) load_words(wa);
#pragma unroll
      for (int u = 0; u < kEmitWords; ++u) my_sel += __popc(selected(sw_r[u], tw_r[u], rank));
    }
  }
  const uint32_t sel_incl = block_scan<kSelThreads>(my_sel, ws);
  {
    uint32_t o = sel_incl - my_sel, rank = tie_rank0;
    for (int wa = w0; wa < w1; wa += kEmitWords) {
      if (!in_regs) load_words(wa);
#pragma unroll
      for (int u = 0; u < kEmitWords; ++u) {
        uint32_t s = selected(sw_r[u], tw_r[u], rank);
        while (s) {
          const int bit = __ffs((int)s) - 1;
          s &= s - 1u;
          if (o < (uint32_t)p.topk) out[o] = (int32_t)(out_base + 32 * (wa + u) + bit);
          ++o;
        }
      }
    }
  }
  for (int i = (int)need + tid; i < p.topk; i += kSelThreads) out[i] = -1;
}

namespace {
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

void indexer_workspace_layout(IndexerParams& p, void* ws, int64_t T, int max_ctx) {
  char* b = static_cast<char*>(ws);
  const int64_t ks = (max_ctx + 1) & ~1;
  const int64_t wsd = (((int64_t)max_ctx + 31) / 32 + 3) & ~(int64_t)3;
  p.hist = reinterpret_cast<uint32_t*>(b);
  b += round256((size_t)T * kBins * sizeof(uint32_t));
  p.cand_n = reinterpret_cast<uint32_t*>(b);
  b += round256((size_t)T * sizeof(uint32_t));
  p.keys_ws = reinterpret_cast<uint64_t*>(b);
  b += round256((size_t)T * ks * sizeof(uint64_t));
  p.cand_key = reinterpret_cast<uint64_t*>(b);
  b += round256((size_t)T * ks * sizeof(uint64_t));
  p.cand_pos = reinterpret_cast<uint32_t*>(b);
  b += round256((size_t)T * ks * sizeof(uint32_t));
  p.sel_bits = reinterpret_cast<uint32_t*>(b);
  b += round256((size_t)T * wsd * sizeof(uint32_t));
  p.tie_bits = reinterpret_cast<uint32_t*>(b);
  p.key_stride = ks;
  p.word_stride = wsd;
}

size_t indexer_workspace_bytes(int64_t T, int max_ctx) {
  const int64_t ks = (max_ctx + 1) & ~1;
  const int64_t wsd = (((int64_t)max_ctx + 31) / 32 + 3) & ~(int64_t)3;
  return round256((size_t)T * kBins * sizeof(uint32_t)) + round256((size_t)T * sizeof(uint32_t)) +
         round256((size_t)T * ks * sizeof(uint64_t)) * 2 + round256((size_t)T * ks * sizeof(uint32_t)) +
         round256((size_t)T * wsd * sizeof(uint32_t)) + (size_t)T * wsd * sizeof(uint32_t);
}

hipError_t launch_indexer(const IndexerParams& p, hipStream_t stream, const KernelEvents& ev) {
  IndexerParams a = p;
  a.nchunks = (p.max_ctx + kChunk - 1) / kChunk;
  a.cchunks = (p.max_ctx + kCPos - 1) / kCPos;
  void* args[] = {&a};
  hipError_t e = hipSuccess;
  // the benchmark events (if any) bracket all the kernels: start at the
  // first kernel's start, stop at the last one's end
  if (a.nchunks > 0) {
    e = launch_kernel((const void*)indexer_score_kernel, dim3((unsigned)(p.T * a.nchunks)), dim3(256), args,
                      stream, {ev.start, nullptr});
    if (e != hipSuccess) return e;
  }
  // Short contexts: one workgroup per token selects over all its keys.
  // Long ones: many workgroups per token compact the candidates first.
  // Both give the same lists.
  if (p.max_ctx <= kShortCtx)
    return launch_kernel((const void*)indexer_select_kernel, dim3((unsigned)p.T), dim3(kSelThreads), args,
                         stream, {a.nchunks > 0 ? nullptr : ev.start, ev.stop});
  e = launch_kernel((const void*)indexer_compact_kernel, dim3((unsigned)(p.T * a.cchunks)), dim3(kCT), args,
                    stream, {});
  if (e != hipSuccess) return e;
  return launch_kernel((const void*)indexer_finish_kernel, dim3((unsigned)p.T), dim3(kSelThreads), args,
                       stream, {nullptr, ev.stop});
}

}  // namespace mla
