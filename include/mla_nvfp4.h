/*
 * mla_nvfp4.h -- C ABI of the NVFP4 sparse-MLA decode library for gfx950.
 *
 * The operation (Prime Inference write-up, "Making room for low-latency
 * decode" and "A native NVFP4 sparse-MLA decode kernel"; the wireai.ir
 * article's 4-bit-caches section):
 *
 *   * an MLA cache row holds a 512-value latent stored as four-bit E2M1 values
 *     with one FP8 (E4M3) scale per group of 16, plus 64 FP8 rope values:
 *     352 bytes instead of 576;
 *   * each query token attends only to the positions its sparse indexer chose
 *     (a fixed-width list, up to 2048 slots, empty slots padded);
 *   * the chosen rows are unpacked on chip; attention uses FP16 operands with
 *     FP32 softmax and accumulation;
 *   * each token's rows are split over several cooperating workgroups whose
 *     partial results are merged inside the same launch.
 *
 * Row layout (bytes): [0,256) latent nibbles, element 2i in the low nibble
 * of byte i; [256,288) the 32 group scales; [288,352) the 64 rope bytes.
 * The 576-byte FP8 comparison row is [0,512) latent then [512,576) rope,
 * each byte E4M3(value / kv_scale).
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" must point to device memory of the current
 *     HIP device; the caller owns every buffer, the library allocates
 *     nothing per call and keeps no state beyond cached device properties.
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*,
 *     NULL = the default stream) and returns without synchronising.
 *   - Arguments are checked on the host before any HIP call; on a bad
 *     argument nothing is enqueued and an MLA_ERR_* code is returned.  A
 *     launch failure reported by the runtime returns MLA_ERR_HIP.
 *   - Index values are checked on the device: a negative index, an index
 *     at or beyond cache_rows, or a block-table entry that is negative or
 *     out of range makes that slot masked (it is never read).
 *   - No C++ exception crosses this boundary.
 */
#ifndef MLA_NVFP4_H
#define MLA_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, stride or alignment */
    MLA_ERR_UNSUPPORTED = 2,  /* enum value or head count not supported       */
    MLA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required   */
    MLA_ERR_HIP = 4,          /* the HIP runtime reported an error            */
    MLA_ERR_CAPACITY = 5      /* the pool has too few free blocks             */
};

enum mla_dtype { MLA_F16 = 0, MLA_BF16 = 1 };
enum mla_cache_fmt { MLA_CACHE_NVFP4_352 = 0, MLA_CACHE_FP8_576 = 1 };

#define MLA_LATENT_DIM 512
#define MLA_ROPE_DIM 64
#define MLA_QK_DIM 576
#define MLA_NVFP4_ROW_BYTES 352
#define MLA_FP8_ROW_BYTES 576
#define MLA_MAX_TOPK 2048

/*
 * mla_nvfp4_quantize_append -- encode n rows and store each at its slot.
 *
 * Defined by the row format above (write-up, "Making room for low-latency
 * decode").  For row i with slot_mapping[i] >= 0 and < cache_rows, the
 * 352-byte row cache[slot_mapping[i]] receives:
 *   scale_g = E4M3(amax_g / 6) of the exact quotient (round to nearest
 *             even, saturating at 448), amax_g = max |latent| of group g;
 *   code_j  = E2M1(latent_j / scale_g) rounded to nearest even, saturating
 *             at 6, magnitude 0 when scale_g is 0; the sign bit copies the
 *             input's sign bit;
 *   rope_k  = E4M3(rope_k), round to nearest even, saturating.
 * Rows with a negative or out-of-range slot are skipped.
 *
 *   latent            device, [n, 512] elements of `dtype`, row stride
 *                     latent_row_stride elements (>= 512), 16-byte aligned
 *                     rows (stride a multiple of 8 elements).
 *   rope              device, [n, 64], row stride rope_row_stride (>= 64,
 *                     a multiple of 8), 16-byte aligned.
 *   dtype             MLA_F16 or MLA_BF16.
 *   slot_mapping      device, [n] int64.
 *   cache             device, [cache_rows, 352] bytes, 16-byte aligned.
 * The result is bit-exact and deterministic.  Two rows naming the same
 * slot race (one of them wins).
 */
int mla_nvfp4_quantize_append(const void* latent, int64_t latent_row_stride,
                              const void* rope, int64_t rope_row_stride,
                              int dtype, int64_t n,
                              const int64_t* slot_mapping,
                              uint8_t* cache, int64_t cache_rows,
                              void* stream);

/*
 * mla_nvfp4_quantize_append_2level -- the two-level NVFP4 variant: the same
 * 352-byte rows, with a per-tensor FP32 scale g (global_scale, > 0) over the
 * E4M3 group scales, so latent element j decodes to code_j * scale_g * g
 * (the rope is not scaled).  This is NVFP4's second scale level; the
 * write-up ("Making room for low-latency decode") names the per-16 FP8
 * scale only.  For an arbitrary g the encoder's decisions are defined by
 * these float32 steps (all exact when g is a power of two, and equal to the
 * one-level encoding when g = 1):
 *   scale_g = E4M3(fl32(amax_g / fl32(6 * g))), nearest even, saturating;
 *   code_j  = magnitude = thresholds passed among fl32(t * scale_g * g),
 *             t = .25, .75, 1.25, 1.75, 2.5, 3.5, 5 (|x| > threshold for
 *             .25, 1.25, 2.5, 5; >= for .75, 1.75, 3.5: ties to even);
 *             0 when scale_g is 0; sign bit copied.
 * Decode such rows with mla_sparse_decode(kv_scale = g).  Arguments as for
 * mla_nvfp4_quantize_append; MLA_ERR_INVALID_ARG unless g and fl32(6 g)
 * are positive and finite.
 */
int mla_nvfp4_quantize_append_2level(const void* latent, int64_t latent_row_stride,
                                     const void* rope, int64_t rope_row_stride,
                                     int dtype, int64_t n,
                                     const int64_t* slot_mapping,
                                     uint8_t* cache, int64_t cache_rows,
                                     float global_scale, void* stream);

/*
 * mla_fp8_quantize_append -- the comparison format: 576-byte FP8 rows,
 * byte = E4M3(value / kv_scale) (round to nearest even, saturating), for
 * the 512 latent values then the 64 rope values.  The FP8 row is the format
 * the write-up's NVFP4 rows replace ("Making room for low-latency decode").
 * Arguments as for mla_nvfp4_quantize_append; cache is [cache_rows, 576];
 * kv_scale must be a positive power of two (so the quotient is exact).
 */
int mla_fp8_quantize_append(const void* latent, int64_t latent_row_stride,
                            const void* rope, int64_t rope_row_stride,
                            int dtype, int64_t n,
                            const int64_t* slot_mapping,
                            uint8_t* cache, int64_t cache_rows,
                            float kv_scale, void* stream);

/*
 * mla_sparse_decode_num_splits -- the launch sizer (Prime Inference write-up,
 * "A native NVFP4 sparse-MLA decode kernel": several cooperating blocks
 * divide each token's selected rows).  Number of workgroups
 * that share one token's selected rows for a call with these sizes
 * (num_splits = 0 in mla_sparse_decode).  The split count follows the token
 * batch the way the write-up's cluster size does (wireai.ir, 4-bit-caches
 * section, second decision).  Returns >= 1, or 0 on bad arguments.
 */
int32_t mla_sparse_decode_num_splits(int64_t num_tokens, int32_t num_heads,
                                     int32_t topk);

/*
 * mla_sparse_decode_workspace_size -- bytes of device workspace
 * mla_sparse_decode needs for these sizes; num_splits = 0 means the launch
 * sizer's choice.  The workspace holds what the write-up's cooperating
 * blocks exchange ("A native NVFP4 sparse-MLA decode kernel": the blocks
 * sharing a token's rows combine their partial results without a second
 * launch): per (token, group of 32 heads) 64 bytes of arrival state (an
 * arrival count with a call epoch, and which split combines which slice of
 * the partials) and, with more than one split, each split's partial output
 * and log-sum-exp.  The arrival state must be zero before the first use (a
 * zero-filled workspace); every completed call leaves it valid for the
 * next one.  Returns 0 on bad arguments.
 */
size_t mla_sparse_decode_workspace_size(int64_t num_tokens, int32_t num_heads,
                                        int32_t topk, int32_t num_splits);

/*
 * mla_sparse_decode -- sparse MLA decode attention over a compressed cache
 * (Prime Inference write-up, "A native NVFP4 sparse-MLA decode kernel":
 * attention reads only the rows the sparse indexer selected, loads them
 * compressed and unpacks them on chip, with FP16 operands and FP32
 * accumulation; each token's rows are divided among cooperating blocks whose
 * partial results are combined within the same launch; wireai.ir article,
 * 4-bit-caches section: the block count follows the token batch and the
 * 2048-slot list's unused slots are padded).
 *
 * For token t and head h, with the valid slots j of indices[t] (index >= 0;
 * a row listed twice counts twice) mapped to cache rows r_j, keys
 * k_j = [latent(r_j); rope(r_j)] (576 values) and values v_j = latent(r_j):
 *   s_j        = sm_scale * (q[t,h] . k_j)
 *   out[t,h]   = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),  m = max_j s_j
 *   lse[t,h]   = m + ln(sum_j exp(s_j - m))
 * A token with no valid slot gets out = 0 and lse = -inf.  Rows are decoded
 * on chip to FP16 (exactly: every E2M1 x E4M3 product is an FP16 value);
 * products accumulate in FP32; softmax runs in FP32; the probabilities
 * enter the value product as FP16.
 *
 *   q                 device, [T, H, 576] of q_dtype; element (t,h,d) at
 *                     q + t*q_stride_t + h*q_stride_h + d (strides in
 *                     elements, multiples of 8; 16-byte aligned base).
 *   q_dtype           MLA_F16 or MLA_BF16 (bf16 is converted to FP16 on load).
 *   num_tokens (T)    >= 0.  num_heads (H): 16, 32, 64 or 128.
 *   cache             device, [cache_rows, 352] (NVFP4) or [cache_rows, 576]
 *                     (FP8), 16-byte aligned.
 *   cache_fmt         MLA_CACHE_NVFP4_352 or MLA_CACHE_FP8_576.
 *   kv_scale          the cache's per-tensor scale.  FP8 rows: value = E4M3
 *                     byte * kv_scale (a power of two).  NVFP4 rows: the
 *                     two-level latent scale g (1 for one-level rows): latent
 *                     values are code * scale * g, the rope is unscaled.  The
 *                     FP16 operands leave g out: the kernel scales the rope
 *                     part of each score by 1/g in FP32 before the latent part
 *                     adds onto it, and applies g to the softmax scale and to
 *                     the output.
 *   indices           device, [T, topk] int32, row stride idx_stride_t
 *                     (>= topk); negative = masked pad.  1 <= topk <= 2048.
 *   block_table       optional (NULL = indices are physical cache rows).
 *                     device, [bt_rows, bt_cols] int32, row stride bt_stride;
 *                     logical position p of sequence b is physical row
 *                     block_table[b, p / block_size] * block_size
 *                     + p % block_size.  block_size >= 1.
 *   token_seq         device, [T] int32 sequence of each token; required
 *                     with a block table, ignored without one.  A token whose
 *                     sequence is outside [0, bt_rows) has every slot masked.
 *   sm_scale          softmax scale applied to q . k.
 *   out               device, [T, H, 512] of q_dtype, contiguous, 16-byte aligned.
 *   lse               device, [T, H] float, contiguous; may be NULL.
 *   workspace         device, workspace_bytes >= the size query's answer for
 *                     (T, H, topk, num_splits); zero-filled before first use.
 *   num_splits        0 = launch sizer's choice; otherwise 1..64.  The call
 *                     returns MLA_ERR_INVALID_ARG when the launch would need
 *                     2^24 or more workgroups (ceil(T*H/32 / 8) * 8 * S).
 * Calls that overlap in time must not share a workspace.
 */
int mla_sparse_decode(const void* q, int q_dtype, int64_t num_tokens,
                      int32_t num_heads, int64_t q_stride_t, int64_t q_stride_h,
                      const uint8_t* cache, int cache_fmt, int64_t cache_rows,
                      float kv_scale,
                      const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                      const int32_t* block_table, int32_t block_size,
                      int64_t bt_stride, int32_t bt_rows, int32_t bt_cols,
                      const int32_t* token_seq,
                      float sm_scale, void* out, float* lse,
                      void* workspace, size_t workspace_bytes,
                      int32_t num_splits, void* stream);

/*
 * mla_sparse_decode_set_merge_polls -- how long a split waits to take part
 * in combining its token's partial results (Prime Inference write-up, "A
 * native NVFP4 sparse-MLA decode kernel": the blocks that share a token's
 * rows combine their results within the same launch).  With S > 1 splits,
 * split k combines slice k of the S partials once every split has arrived;
 * it polls for that at most `polls` times (about a microsecond each) and
 * otherwise leaves its slice to the split that arrives last, which combines
 * every slice no other split has taken.  0 = no split waits (the last
 * arrival combines everything).  The result does not depend on the setting.
 * Launches whose workgroups cannot all be resident at once never wait.
 * Process-wide; returns the previous value, or -1 (and changes nothing)
 * for polls < 0.  Default 256.
 */
int32_t mla_sparse_decode_set_merge_polls(int32_t polls);

/*
 * mla_sparse_decode_noalloc -- mla_sparse_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc).  It computes exactly what
 * mla_sparse_decode computes with the same arguments and split count, and
 * allocates nothing: its workspace is a scratch array inside the library,
 * one per GPU, held until the process ends.
 *
 * Arguments are those of mla_sparse_decode without the workspace.  Limits
 * of the scratch: at most MLA_NOALLOC_MAX_UNITS (token, head group) units
 * (T * H / 32 rounded up to H >= 32 groups; 64 bytes of arrival state
 * each), and the split partials (T * ceil(H/32) * num_splits * 32 KiB plus
 * their log-sum-exps) within MLA_NOALLOC_SCRATCH_BYTES - 4 MiB; a call
 * beyond either returns MLA_ERR_WORKSPACE and enqueues nothing.  The first
 * call on a device also enqueues, on its stream and before its decode, a
 * small kernel that zeroes the scratch's arrival state.
 *
 * Every call on a GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (different streams without ordering between them) race and
 * give wrong results.  Calls ordered on one stream are safe.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
#define MLA_NOALLOC_MAX_UNITS 65536
int mla_sparse_decode_noalloc(const void* q, int q_dtype, int64_t num_tokens,
                              int32_t num_heads, int64_t q_stride_t, int64_t q_stride_h,
                              const uint8_t* cache, int cache_fmt, int64_t cache_rows,
                              float kv_scale,
                              const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                              const int32_t* block_table, int32_t block_size,
                              int64_t bt_stride, int32_t bt_rows, int32_t bt_cols,
                              const int32_t* token_seq,
                              float sm_scale, void* out, float* lse,
                              int32_t num_splits, void* stream);

/*
 * mla_nvfp4_gather_dequant_fp8 -- first step of the staged comparator the
 * write-up measures against its native kernel (mo.ai.kr article, KV-cache
 * section; wireai.ir, 4-bit-caches section): unpack the selected NVFP4
 * rows into an FP8 buffer in device memory ahead of an FP8 attention call.
 *
 * For token t and slot j: if the slot is valid (same rules and optional
 * block table as mla_sparse_decode) the NVFP4 row is decoded and
 * re-encoded as a 576-byte FP8 row E4M3(value / fp8_scale) (round to
 * nearest even, saturating) at fp8_rows[t*topk + j], and
 * staged_indices[t*topk + j] = t*topk + j; a masked slot gets a zero row
 * and index -1.  fp8_scale must be a positive power of two.
 *
 *   fp8_rows          device, [T*topk, 576] bytes, 16-byte aligned.
 *   staged_indices    device, [T, topk] int32 (contiguous).
 * mla_sparse_decode(cache = fp8_rows, cache_fmt = MLA_CACHE_FP8_576,
 * kv_scale = fp8_scale, indices = staged_indices, idx_stride_t = topk)
 * then completes the staged path.
 */
int mla_nvfp4_gather_dequant_fp8(const uint8_t* cache, int64_t cache_rows,
                                 const int32_t* indices, int64_t num_tokens,
                                 int32_t topk, int64_t idx_stride_t,
                                 const int32_t* block_table, int32_t block_size,
                                 int64_t bt_stride, int32_t bt_rows, int32_t bt_cols,
                                 const int32_t* token_seq,
                                 float fp8_scale, uint8_t* fp8_rows,
                                 int32_t* staged_indices, void* stream);

/*
 * mla_indexer_topk -- the sparse indexer: for each query token, the list of
 * cache positions its attention reads (Prime Inference write-up, "A native
 * NVFP4 sparse-MLA decode kernel": the decode consumes the positions the
 * sparse indexer selected; wireai.ir article, 4-bit-caches section, third
 * decision: a fixed-width list of up to 2048 positions, unused slots padded).
 *
 * The pages give no scoring formula; this library takes the plainest one.
 * Each cached position holds a 128-value E4M3 indexer key, each token a
 * 128-value E4M3 indexer query, and the score of position p for token t is
 * q_idx[t] . key(p), computed exactly (FP64 holds every partial sum of E4M3
 * products exactly).  Token t's candidates are its positions 0 .. ctx[t]-1
 * that name a key row.  Its list holds the min(topk, n) candidates with the
 * largest scores (equal scores: the smaller position first), in ascending
 * position order, padded with -1 to width topk.
 *
 *   q_idx             device, [T, 128] E4M3 bytes, row stride q_stride_t
 *                     bytes (a multiple of 16, >= 128), 16-byte aligned.
 *   keys              device, [key_rows, 128] E4M3 bytes, 16-byte aligned.
 *   ctx_len           device, [T] int32: visible positions per token,
 *                     clamped on the device to [0, max_ctx].
 *   max_ctx           host bound on every ctx_len (sizes the workspace).
 *   key_base          device, [T] int64, used without a block table: key p
 *                     of token t is row key_base[t] + p and the list holds
 *                     these rows (the physical indices mla_sparse_decode takes
 *                     without a block table).
 *   block_table ...   optional, as in mla_sparse_decode: key p of sequence
 *                     token_seq[t] is row block_table[seq, p / block_size] *
 *                     block_size + p % block_size, and the list holds logical
 *                     positions p (the indices mla_sparse_decode translates
 *                     through the same table).
 *   A position whose row is negative, at or past key_rows, in a block past
 *   bt_cols or unassigned, or of a sequence outside [0, bt_rows), is not a
 *   candidate (its key is never read).
 *   topk              1 .. 2048.  out: device, [T, topk] int32, row stride
 *                     out_stride_t >= topk.
 *   workspace         device, >= mla_indexer_workspace_size(T, max_ctx)
 *                     bytes, 16-byte aligned, zero-filled before first use
 *                     (every completed call leaves its histogram and
 *                     candidate-count parts zero).  It holds, per token,
 *                     a 4096-bin histogram, a candidate count, max_ctx
 *                     score keys, candidate keys and positions, and two
 *                     max_ctx-bit maps: about 20.5 bytes per position.
 * The result is deterministic.  Calls that overlap in time must not share a
 * workspace.  Non-finite E4M3 codes (0x7F, 0xFF) are outside the contract.
 */
#define MLA_INDEXER_DIM 128
size_t mla_indexer_workspace_size(int64_t num_tokens, int32_t max_ctx);
int mla_indexer_topk(const uint8_t* q_idx, int64_t q_stride_t,
                     const uint8_t* keys, int64_t key_rows,
                     int64_t num_tokens, const int32_t* ctx_len, int32_t max_ctx,
                     const int64_t* key_base,
                     const int32_t* block_table, int32_t block_size,
                     int64_t bt_stride, int32_t bt_rows, int32_t bt_cols,
                     const int32_t* token_seq,
                     int32_t topk, int32_t* out, int64_t out_stride_t,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged cache pool (host side, no GPU calls) -- capacity accounting and a
 * block allocator for the cache rows and the indexer and other per-token
 * state of every layer (Prime Inference write-up, "Making room for
 * low-latency decode": 576 -> 352-byte rows with the other state unchanged
 * took one decoder's cache from about 1.09 M to 1.63 M tokens at the same
 * memory budget; 64-row blocks as in "Changing the layout to reduce
 * fragmentation").
 *
 * Capacity, in whole blocks of block_rows tokens:
 *   budget_bytes / (layers * block_rows * (row_bytes + other_bytes)).
 * A sequence grows by whole blocks, each the lowest-numbered free block
 * (consecutive blocks on an unfragmented pool), all or nothing; releasing it
 * frees them all.  Physical row of position p: table[p / block_rows] *
 * block_rows + p % block_rows, in every layer's cache.
 *
 * mla_pool_create         max_seqs sequences of at most max_blocks_per_seq
 *                         blocks; *out receives the pool (MLA_ERR_INVALID_ARG
 *                         on bad sizes, or more than 2^31 physical rows).
 * mla_pool_reserve        grow `seq` to hold `tokens` positions;
 *                         MLA_ERR_CAPACITY (nothing taken) if the free blocks
 *                         or the table width do not suffice.
 * mla_pool_block_table    host [max_seqs, max_blocks_per_seq] int32 copy of
 *                         every table, row stride `stride`, -1 = no block.
 * mla_pool_slots          host int64 physical rows of positions first_pos ..
 *                         first_pos + n - 1 of `seq` (the slot mapping
 *                         mla_nvfp4_quantize_append takes); the positions must
 *                         be reserved.
 * mla_pool_descriptors    copy descriptors (maximal contiguous byte runs) and
 *                         bytes of `seq`'s (layer, block) regions of
 *                         block_rows * row_bytes bytes, visited in table order,
 *                         under a layer-major pool (region (l, b) at
 *                         (l * n_blocks + b) * R) or a block-major pool (at
 *                         (b * layers + l) * R).
 * Calls on one pool are serialised by the pool's own lock.
 */
typedef struct mla_pool mla_pool;
enum mla_layout { MLA_LAYOUT_LAYER_MAJOR = 0, MLA_LAYOUT_BLOCK_MAJOR = 1 };
int64_t mla_pool_capacity_blocks(int64_t budget_bytes, int32_t layers, int32_t row_bytes,
                                 int32_t other_bytes, int32_t block_rows);
int mla_pool_create(int64_t budget_bytes, int32_t layers, int32_t row_bytes, int32_t other_bytes,
                    int32_t block_rows, int32_t max_seqs, int32_t max_blocks_per_seq, mla_pool** out);
void mla_pool_destroy(mla_pool* pool);
int64_t mla_pool_num_blocks(mla_pool* pool);
int64_t mla_pool_free_blocks(mla_pool* pool);
int mla_pool_reserve(mla_pool* pool, int32_t seq, int64_t tokens);
int mla_pool_release(mla_pool* pool, int32_t seq);
int mla_pool_block_table(mla_pool* pool, int32_t* table, int64_t stride);
int mla_pool_slots(mla_pool* pool, int32_t seq, int64_t first_pos, int64_t n, int64_t* slots);
int mla_pool_descriptors(mla_pool* pool, int32_t seq, int32_t layout, int64_t* descriptors,
                         int64_t* bytes);

/*
 * mla_kv_pack_blocks / mla_kv_unpack_blocks -- move a request's cache blocks
 * between a pool and one contiguous staging buffer, the form that needs a
 * single copy descriptor to transfer (Prime Inference write-up, "Changing
 * the layout to reduce fragmentation"; mo.ai.kr article, KV-transfer
 * section: a block-major layout groups one block's data from all layers).
 *
 * A region is one (layer, block): block_rows * row_bytes bytes (a multiple
 * of 16).  The pool holds pool_blocks blocks of `layers` layers, layer-major
 * (region (l, b) at (l * pool_blocks + b) * R) or block-major (at
 * (b * layers + l) * R).  staging is [n][layers][R], block-major over the
 * request's n blocks.  pack copies pool region (l, block_ids[i]) to staging
 * (i, l); unpack copies staging (i, l) to pool region (l, block_ids[i]).
 * block_ids (device, int32 [n]) outside [0, pool_blocks) are skipped on the
 * device.  pool and staging are device memory, 16-byte aligned.
 */
int mla_kv_pack_blocks(const uint8_t* pool, int32_t layout, int64_t pool_blocks, int32_t layers,
                       int32_t block_rows, int32_t row_bytes, const int32_t* block_ids, int64_t n,
                       uint8_t* staging, void* stream);
int mla_kv_unpack_blocks(const uint8_t* staging, int64_t n, const int32_t* block_ids, uint8_t* pool,
                         int32_t layout, int64_t pool_blocks, int32_t layers, int32_t block_rows,
                         int32_t row_bytes, void* stream);

/*
 * Kernel timing for benchmarks (instrumentation, not part of the method).
 *
 * mla_kernel_timing(1) makes every later launching call of this library
 * (quantize-append, gather-dequant, sparse decode) made by this host thread
 * on the current device launch its kernel with hipExtLaunchKernel and a
 * pair of HIP events owned by the library, which the runtime records at
 * the kernel's own start and end on the caller's stream.  Results are
 * unchanged; each launch costs a little more host and queue time.
 * mla_kernel_timing(0) stops that and releases the events.  Returns
 * MLA_ERR_HIP if the events cannot be created.
 *
 * mla_last_kernel_ms waits for the last timed launch of this thread to
 * finish and writes its kernel duration in milliseconds to *ms (host
 * pointer).  Returns MLA_ERR_INVALID_ARG if ms is NULL or no launch has
 * been timed since timing was enabled.
 */
int mla_kernel_timing(int enable);
int mla_last_kernel_ms(float* ms);

/*
 * mla_gather_probe -- read rows[0..n) of a cache (row_bytes bytes each, a
 * multiple of 16) and nothing else: a measurement aid, not a step of the
 * method.  Its duration is the time this GPU needs to fetch exactly that row
 * list from HBM, the ceiling for any kernel that gathers those rows (the
 * sparse decode reads 352-byte rows at 16-byte-aligned offsets, each
 * touching three or four 128-byte lines).  cache (device, 16-byte aligned)
 * holds cache_rows rows; rows (device, int32 [n]) are physical row numbers,
 * and entries outside [0, cache_rows) are skipped.  sink (device, one
 * uint32) is written only if the folded row words equal a fixed constant,
 * which does not happen in practice; its contents carry no meaning.  Runs
 * on `stream`; honours mla_kernel_timing.  Returns MLA_ERR_INVALID_ARG for
 * NULL pointers (when n > 0), misalignment, bad sizes or n >= 2^31.
 */
int mla_gather_probe(const uint8_t* cache, int64_t cache_rows, int32_t row_bytes, const int32_t* rows,
                     int64_t n, uint32_t* sink, void* stream);

/* Human-readable name of a status code (static storage). */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_NVFP4_H */
