/*
 * pkv.h — C ABI of a HIP library (gfx950 / MI355X) for attention over a paged,
 * block-table-indexed KV cache.
 *
 * Conventions shared by every call:
 *   - Pointers without a _h suffix are DEVICE pointers; _h pointers are host memory.
 *     bf16 buffers are passed as void*, dense, row-major, 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every kernel is enqueued on it and the
 *     call returns without synchronising. The library allocates no device memory: the caller owns
 *     every buffer, including outputs and workspace.
 *   - KV cache layout (K and V alike): [num_blocks, num_kv_heads, block_size, head_dim] bf16.
 *     Token t of a sequence lives in physical block block_tables[b][t / block_size] at offset
 *     t % block_size. Block tables are int32 [batch, max_blocks_per_seq], padded with -1; only the
 *     first ceil(len / block_size) entries of a row are read.
 *   - Query head h reads kv head h / (num_q_heads / num_kv_heads) (consecutive q heads share).
 *   - Return value: PKV_OK, or an error code; on error nothing was enqueued. Device-side
 *     preconditions (table contents, lengths, offsets, slots) are trusted for speed; the kernels
 *     clamp every address they form to the buffers described by the size arguments (and, for
 *     prefill, by the host copies of the offsets), so a broken table or length gives wrong
 *     numbers, never an out-of-bounds access. pkv_validate_block_tables_h checks tables.
 *   - Slots that hold no token (the tail of a sequence's last block, unused blocks) may hold any
 *     bits, NaN included: they are excluded by length, never read into a result.
 *   - Calls that read the cache through block tables (decode in every form, paged prefill, the
 *     streamed decode) need num_blocks >= 1 and max_blocks_per_seq >= 1, even when every sequence
 *     is empty: the kernels clamp block ids into [0, num_blocks) and cannot see lengths on the
 *     host, so an empty pool is refused (PKV_E_INVALID_ARGUMENT) rather than risked.
 *
 * Supported: head_dim in {64, 128, 256}; num_q_heads % num_kv_heads == 0; block_size a power of
 * two from 16 to 256; bf16 data, fp32 accumulation, bf16 output rounded to nearest even.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_status {
  PKV_OK = 0,
  PKV_E_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned buffer */
  PKV_E_UNSUPPORTED = 2,      /* head_dim / block_size / grouping not built */
  PKV_E_BAD_TABLE = 3,        /* checked-mode table validation failed */
  PKV_E_WORKSPACE_TOO_SMALL = 4,
  PKV_E_HIP = 5               /* a HIP launch reported an error */
};

/* Human-readable name of a status code (static storage). */
const char* pkv_status_string(int status);

/*
 * reshape_and_cache — scatter new tokens' K/V rows into their cache slots.
 * Defined by the vLLM-derived paged_attn.py page, PagedAttention.write_to_paged_cache: key and
 * value [T, Hkv, D] are written to the slot each token's flattened slot_mapping names, where a
 * slot is physical_block * block_size + offset.
 *
 *   k, v            [num_tokens, num_kv_heads, head_dim] bf16, read only.
 *   k_cache,v_cache [num_blocks, num_kv_heads, block_size, head_dim] bf16, written in place.
 *   slot_mapping    [num_tokens] int64. A negative slot skips the token. Slots >= num_blocks *
 *                   block_size are skipped as well (a caller error). Duplicate slots are a caller
 *                   error with an unspecified winner.
 * The copy is bit-exact. Slots not named keep their contents. num_tokens == 0 is a no-op.
 */
int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, void* stream);

/*
 * Workspace bytes paged_attn_decode needs for the given shape and partition choice (0 when the
 * direct, single-pass path is taken). partition_tokens: 0 = direct, > 0 = split-KV with that many
 * tokens per partition, -1 = the library's choice (the same choice paged_attn_decode makes).
 */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int32_t partition_tokens);

/*
 * Decode plan from the host copy of the sequence lengths, for callers that size a launch once and
 * capture it in a HIP graph. The libmir-cuda page plans direct vs split decode ahead of capture
 * (PagedAttentionBf16::new, plan_attention, captured_configs); the vLLM-derived paged_attn.py page
 * (forward_decode) routes on the real seq_lens.max(), not on a bound inflated for graph mode.
 *   seq_lens_h           HOST int32 [batch] (>= 0).
 *   partition_tokens     as for pkv_paged_attn_decode (0, > 0 multiple of 32, or -1).
 *   *max_seq_len_out     the real maximum length (pass it as max_seq_len);
 *   *partition_tokens_out the path pkv_paged_attn_decode takes for it (0 = direct);
 *   *workspace_bytes_out the workspace that call needs.
 * A captured call reads seq_lens from device memory on every replay, so it serves any lengths up to
 * the max_seq_len it was captured with; plan (and capture) again when that bound changes.
 */
int pkv_decode_plan(const int32_t* seq_lens_h, int32_t batch, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t partition_tokens,
                    int32_t* max_seq_len_out, int32_t* partition_tokens_out,
                    size_t* workspace_bytes_out);

/*
 * paged_attn_decode — one query token per sequence against its paged KV cache.
 * Defined by the vLLM-derived paged_attn.py page (PagedAttention._forward_decode_pytorch and
 * forward_decode): out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over tokens [0, seq_lens[b]),
 * K_b/V_b read through block_tables[b]. seq_lens[b] == 0 gives a zero row. The split-KV form cuts
 * each sequence into partitions of partition_tokens (vLLM uses 512) whose running max / exp-sum /
 * partial output are merged by log-sum-exp in a second kernel, as the same page's V2 path does.
 *
 *   q            [batch, num_q_heads, head_dim] bf16.
 *   out          [batch, num_q_heads, head_dim] bf16, fully overwritten.
 *   lse          optional [batch, num_q_heads] fp32: natural-log log-sum-exp of the scaled scores
 *                (-inf for an empty sequence). NULL to skip.
 *   block_tables [batch, max_blocks_per_seq] int32; seq_lens [batch] int32.
 *   max_seq_len  host hint: must be >= every seq_lens[b]; sizes the split grid. Lengths are also
 *                clamped to max_blocks_per_seq * block_size.
 *   partition_tokens  0 = direct; > 0 = split (a multiple of 32); -1 = library choice: direct
 *                when batch * num_kv_heads * ceil(group / 16) >= 512 or max_seq_len <= 512, else
 *                split with the longest power-of-two partition from 512 to 8192 tokens that still
 *                gives 1024 partitions of (sequence, kv head, 16-head group) at max_seq_len; if
 *                512 tokens give fewer than 384 such partitions, the partition halves (down to
 *                128 tokens) until they reach 384.
 *   workspace    device scratch of at least pkv_decode_workspace_bytes(...) bytes (may be NULL
 *                when that is 0). Its contents need no initialisation.
 */
int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, void* out, float* lse,
                          int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_seq_len, float scale, int32_t partition_tokens, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Measured decode planning. The libmir-cuda page does not fix its decode launch by rule alone:
 * PagedAttentionBf16::new plans direct vs split decode and keeps the profiling state
 * (profile_allowed, tuning_complete) of a CUDA autotuner so the choice is timed on the device.
 * pkv_decode_tune times, on the caller's own buffers and stream, the library's default choice,
 * the direct path, and split-KV with partitions of 256 to 8192 tokens (powers of two) streamed 1, 2,
 * 4, 8 or 16 to a wave (those whose partials fit the LDS budget and the given workspace), each
 * the median of `repeats` launches after one untimed launch, and writes the fastest into *plan.
 * The default choice is a candidate, so the plan is never slower than it on that measurement.
 *   workspace      as for pkv_paged_attn_decode; split candidates needing more are skipped.
 *                  pkv_decode_workspace_bytes(batch, ..., max_seq_len, 256) covers all of them.
 *   out            is overwritten by every candidate (the result of any of them).
 * The call synchronises with `stream` (HIP events): never call it while a stream is captured.
 * A plan belongs to its shape bucket (batch, heads, head_dim, max_seq_len); the caller keeps it.
 * Returns the status of the first failing launch, PKV_E_INVALID_ARGUMENT (null plan, repeats
 * outside 1..1000), or PKV_E_HIP if the timing itself fails.
 */
typedef struct pkv_decode_tuned_plan {
  int32_t partition_tokens;    /* 0: direct; > 0: split-KV with this many tokens per partition */
  int32_t partitions_per_wave; /* split: consecutive partitions one wave streams (0: library's) */
  int32_t max_seq_len;         /* the length bound the plan was measured for */
  int32_t candidates;          /* configurations timed */
  size_t workspace_bytes;      /* workspace pkv_paged_attn_decode_tuned needs with this plan */
  float measured_us;           /* median time of the chosen configuration */
  float default_us;            /* median time of the library's default choice */
} pkv_decode_tuned_plan;

int pkv_decode_tune(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, void* out,
                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                    int32_t repeats, void* stream, pkv_decode_tuned_plan* plan);

/* paged_attn_decode with a measured plan: as pkv_paged_attn_decode (same arguments and result),
 * with the plan's path, partition size and partitions per wave instead of partition_tokens.
 * workspace must hold pkv_decode_workspace_bytes(..., plan->partition_tokens) bytes. Captures
 * like pkv_paged_attn_decode (no allocation, no synchronisation). */
int pkv_paged_attn_decode_tuned(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens, void* out,
                                float* lse, int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, float scale,
                                const pkv_decode_tuned_plan* plan, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode without a workspace, for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Same arguments, paths and
 * results as pkv_paged_attn_decode, less workspace / workspace_bytes: the split-KV partials live
 * in a 64 MiB device array the library holds (one per GPU it runs on, kept until the process
 * ends; its address is looked up on the device's first call). The call itself allocates nothing.
 *   - A shape whose partials exceed 64 MiB (pkv_decode_workspace_bytes(...) > 64 << 20) is
 *     PKV_E_WORKSPACE_TOO_SMALL, before anything is enqueued.
 *   - `stream` must belong to the current device (else PKV_E_INVALID_ARGUMENT).
 *   - Every call on one GPU shares that GPU's array and leaves its partials there. Calls that
 *     overlap on one GPU (other streams, other host threads) race on it: order them on one stream.
 */
int pkv_paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens, void* out,
                                  float* lse, int32_t batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t max_seq_len, float scale, int32_t partition_tokens,
                                  void* stream);

/*
 * ragged_prefill — N requests' attention in one launch over contiguous ragged rows.
 * Defined by the spark_runtime/flashinfer.rs page, ragged_prefill_bf16_hd256 and its CPU-reference
 * test: request b's queries are rows qo_indptr[b]..qo_indptr[b+1] of q, its keys/values rows
 * kv_indptr[b]..kv_indptr[b+1] of k/v; with causal != 0, query row i of a request sees key j iff
 * j <= i + (kv_len - qo_len) (bottom-right alignment). A row that sees no key is zero.
 *
 *   q, out   [qo_indptr_h[batch], num_q_heads, head_dim] bf16.
 *   k, v     [kv_indptr_h[batch], num_kv_heads, head_dim] bf16.
 *   qo_indptr, kv_indptr        device [batch + 1] int32 prefix sums (read by the kernel).
 *   qo_indptr_h, kv_indptr_h    host copies of the same (size and order the launch; no device
 *                               sync). The kernels clamp the device offsets to the buffers the
 *                               host copies describe (q / out rows qo_indptr_h[batch], k / v rows
 *                               kv_indptr_h[batch]): device offsets that disagree with their host
 *                               copies give wrong rows, never an access outside those buffers.
 *   workspace    device scratch of at least pkv_prefill_workspace_bytes(...) bytes (may be NULL
 *                when that is 0), 16-byte aligned; it holds the work-group schedule the library
 *                builds on the device. Its contents need no initialisation. Calls that share a
 *                workspace must be ordered (one stream).
 * The work of a launch is cut into (request, q tile) items run longest-first; a q tile is
 * 128 / gcd(G, 4) rows for head_dim <= 128 and 192 / gcd(G, 12) rows for head_dim 256, where
 * G = num_q_heads / num_kv_heads (one work-group serves that many q heads of one kv head).
 * PKV_E_UNSUPPORTED for head_dim other than 64/128/256, num_kv_heads * head_dim >= 2^23, batch >
 * 65535, a request of more than 65535 q tiles, or more than 65528 q tiles in all (also for
 * pkv_paged_prefill). PKV_E_WORKSPACE_TOO_SMALL when workspace_bytes is below the size above.
 */
int pkv_ragged_prefill(const void* q, const void* k, const void* v, void* out,
                       const int32_t* qo_indptr, const int32_t* kv_indptr,
                       const int32_t* qo_indptr_h, const int32_t* kv_indptr_h, int32_t batch,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t causal,
                       float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes pkv_ragged_prefill / pkv_paged_prefill need for these host q offsets
 * (qo_indptr_h, [batch + 1]): 0 when the launch's longest-first schedule fits the launch
 * arguments (at most 768 (request, q tile) items), else room for one 32-bit entry per item. The
 * Atlas spark_runtime/flashinfer.rs page sizes its ragged-prefill workspaces the same way, from
 * the batch's offsets before the call (atlas_fi_ragged_prefill_workspace_sizes). Returns 0 for
 * arguments the prefill calls would reject.
 */
size_t pkv_prefill_workspace_bytes(int32_t batch, const int32_t* qo_indptr_h, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim);

/*
 * paged_prefill — prefill whose keys/values come through the block table (chunked prefill over a
 * cached prefix). Defined by the vLLM-derived paged_attn.py page, _forward_prefix_pytorch: the
 * cached prefix is visible to every new row; the new chunk (already written to the cache by
 * reshape_and_cache) is causal. Request b's queries are rows qo_indptr[b]..qo_indptr[b+1] of q;
 * its keys are cached tokens [0, kv_lens[b]); query i sees key j iff j <= kv_lens[b] - qo_len + i
 * when causal != 0.
 *
 *   q, out       [qo_indptr_h[batch], num_q_heads, head_dim] bf16.
 *   block_tables [batch, max_blocks_per_seq] int32; kv_lens device [batch] int32 (clamped to
 *                max_blocks_per_seq * block_size by the kernels).
 *   qo_indptr    device [batch + 1]; qo_indptr_h, kv_lens_h host copies (a host length beyond
 *                the table's capacity is PKV_E_BAD_TABLE).
 *   workspace, workspace_bytes   as for pkv_ragged_prefill (pkv_prefill_workspace_bytes).
 */
int pkv_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* qo_indptr, const int32_t* kv_lens,
                      const int32_t* qo_indptr_h, const int32_t* kv_lens_h, void* out, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t causal, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Checked-mode validation of block tables on the host, following the libmir-cuda page
 * (PagedAttentionBf16::validate_table): every sequence's table must hold its declared tokens
 * (ceil(len / block_size) <= max_blocks_per_seq) and every entry a sequence reads must name an
 * existing physical block (0 <= id < num_blocks). Returns PKV_OK, PKV_E_BAD_TABLE, or
 * PKV_E_INVALID_ARGUMENT (null pointers, negative sizes or lengths). Host memory only.
 */
int pkv_validate_block_tables_h(const int32_t* block_tables_h, const int32_t* seq_lens_h,
                                int32_t batch, int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t num_blocks);

/*
 * paged_attn_decode with a sliding window: as pkv_paged_attn_decode (same arguments and output),
 * with sequence b attending only to its keys [max(0, seq_lens[b] - window), seq_lens[b]).
 * window == 0 means no window (then exactly pkv_paged_attn_decode); window < 0 is
 * PKV_E_INVALID_ARGUMENT. The vLLM-derived paged_attn.py page's forward_decode takes a
 * sliding_window, and the libmir-cuda page sizes its split partitions by (token_count, window)
 * (captured_configs). Likewise here, with window > 0:
 *   partition_tokens -1 plans on min(max_seq_len, window) keys (the rule of pkv_paged_attn_decode);
 *   a split call's partials cover only the partitions a window can touch, so its workspace is
 *   pkv_decode_window_workspace_bytes(...), at most what pkv_decode_workspace_bytes gives for the
 *   same partition size.
 */
/* Workspace bytes pkv_paged_attn_decode_window needs (0 on its direct path); window == 0 gives
 * pkv_decode_workspace_bytes. Arguments as for pkv_paged_attn_decode_window. */
size_t pkv_decode_window_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len, int32_t window,
                                         int32_t partition_tokens);

int pkv_paged_attn_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* seq_lens, void* out,
                                 float* lse, int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t max_blocks_per_seq,
                                 int32_t max_seq_len, float scale, int32_t window,
                                 int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Streamed decode attention over several launches, one per tile of resident blocks, as the Atlas
 * spark_storage/high_speed_swap/impl_more.rs page runs it (attend_layer_on_stream_with_q_pos: a step
 * begins, each tile of at most resident_blocks blocks is attended through its own block table, the
 * output is normalised at the end). The result equals one decode over the union of the tiles' tokens.
 *
 *   state  caller-owned device buffer of pkv_stream_attn_state_bytes(batch, num_q_heads, head_dim)
 *          bytes holding, per (sequence, q head), the normalised fp32 output row, the running max
 *          (log2 units) and the exp-sum: [B, Hq, D] f32, then [B, Hq] f32 twice, each 256-byte
 *          aligned. Opaque to the caller otherwise.
 *   begin     resets the state (a fill kernel: safe inside a captured graph).
 *   step      attends q to one tile: tile_tables [batch, tile_capacity] int32 (physical blocks, in
 *             token order within the tile), tile_lens [batch] int32 (tokens of the tile: a sequence's
 *             last block may be partly valid, slots past tile_lens are never read; 0 = nothing), and
 *             folds the tile into the state. Tiles may come in any order.
 *   finalize  out [batch, num_q_heads, head_dim] bf16 = the normalised output (zero rows for
 *             sequences no tile touched); lse optional [batch, num_q_heads] f32 (natural log).
 */
size_t pkv_stream_attn_state_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim);
int pkv_stream_attn_begin(void* state, size_t state_bytes, int32_t batch, int32_t num_q_heads,
                          int32_t head_dim, void* stream);
int pkv_stream_attn_step(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* tile_tables, const int32_t* tile_lens, void* state,
                         size_t state_bytes, int32_t batch, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t tile_capacity, float scale, void* stream);
int pkv_stream_attn_finalize(const void* state, size_t state_bytes, void* out, float* lse,
                             int32_t batch, int32_t num_q_heads, int32_t head_dim, void* stream);

/*
 * FP8 KV cache. The vLLM-derived paged_attn.py page passes kv_cache_dtype with per-tensor k_scale
 * and v_scale floats to write_to_paged_cache and forward_decode. Here the fp8 cache holds OCP FP8
 * E4M3 codes (bias 7, no infinities, max 448, S.1111.111 = NaN) in the same
 * [num_blocks, num_kv_heads, block_size, head_dim] layout, one byte per element:
 *   stored code = e4m3(x / scale): x the bf16 input in fp32, IEEE fp32 division, round to nearest
 *                 even, magnitudes beyond 448 saturate to 448, NaN stored as 0x7F;
 *   read value  = decode(code) * scale.
 * k_scale and v_scale must be finite and > 0 (else PKV_E_INVALID_ARGUMENT).
 */

/* reshape_and_cache into an fp8 cache: as pkv_reshape_and_cache (same slot rules), storing the
 * codes of k / k_scale and v / v_scale. head_dim a multiple of 16. Bit-exact. */
int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, float k_scale,
                              float v_scale, void* stream);

/* paged_attn_decode over an fp8 cache: as pkv_paged_attn_decode (same arguments, paths, workspace
 * and output), with K = decode(code) * k_scale and V = decode(code) * v_scale. */
int pkv_paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens, void* out,
                              float* lse, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                              float k_scale, float v_scale, int32_t partition_tokens,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * copy_blocks — copy whole cache blocks inside every layer's key and value caches.
 * Defined by the vLLM-derived paged_attn.py page, PagedAttention.copy_blocks: for each layer and
 * each (src, dst) pair of the mapping, block dst of the layer's K cache becomes a copy of its block
 * src, and the same for the V cache. A block is the contiguous [num_kv_heads, block_size, head_dim]
 * run of the cache layout above.
 *
 *   k_cache_ptrs, v_cache_ptrs  DEVICE arrays [num_layers] of uint64 device addresses, one cache of
 *                  num_blocks blocks per layer (16-byte aligned).
 *   block_mapping  DEVICE int64 [num_pairs, 2]: (src block, dst block).
 *   block_bytes    bytes of one block of one cache (a multiple of 16).
 * Pairs naming a block outside [0, num_blocks) are skipped on the device. Destination blocks must
 * be distinct and must not be the source of another pair (else the result is unspecified).
 * num_layers == 0 or num_pairs == 0 is a no-op.
 */
int pkv_copy_blocks(const uint64_t* k_cache_ptrs, const uint64_t* v_cache_ptrs, int32_t num_layers,
                    const int64_t* block_mapping, int32_t num_pairs, int64_t block_bytes,
                    int32_t num_blocks, void* stream);

/*
 * swap_blocks — copy whole blocks from one cache to another that may live in another memory
 * (device and host), as the vLLM-derived paged_attn.py page's PagedAttention.swap_blocks does when
 * blocks are swapped out to, or in from, host memory. Call once per cache (K, then V).
 *
 *   src, dst         caches of src_num_blocks / dst_num_blocks blocks; device or host memory
 *                    (pinned host memory keeps the copies asynchronous on `stream`).
 *   block_mapping_h  HOST int64 [num_pairs, 2]: (src block, dst block), checked on the host.
 * When the GPU can address both caches (device memory, pinned host memory) one kernel moves every
 * block (block_bytes a multiple of 16); otherwise HIP copies move each run of pairs whose source and
 * destination blocks both advance by one. Destination blocks must be distinct.
 * PKV_E_INVALID_ARGUMENT for a block index out of range (before any copy is enqueued).
 */
int pkv_swap_blocks(const void* src, void* dst, const int64_t* block_mapping_h, int32_t num_pairs,
                    int64_t block_bytes, int32_t src_num_blocks, int32_t dst_num_blocks,
                    void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
