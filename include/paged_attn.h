/*
 * paged_attn.h - C ABI of the paged-KV attention library (gfx950 / MI355X).
 *
 * Scaled dot-product attention that reads keys and values through a block
 * table from a paged KV cache: single-query decode (batched, ragged lengths,
 * grouped query heads, optional sliding window) and causal chunked prefill
 * over the same pages, plus the write of new tokens' keys/values into their
 * pool slots.
 *
 * Sources (page title, section):
 *  - "Build a Paged KV Cache in Pure Python": Step 1 (a block holds keys and
 *    values of block_size positions for every head, shape
 *    (block_size, num_heads, head_dim)), Step 2 (a pool of blocks handed out
 *    from a free list), Step 3 (append: block = table[pos // block_size],
 *    slot = pos % block_size; retrieve: blocks in table order, the last one
 *    cut to the positions present), Step 4 (attention of one query per head
 *    over the retrieved keys: scaled scores, max-subtracted softmax over the
 *    keys, weighted sum of values; empty -> zeros), Step 5 (keys/values are
 *    appended before the query attends).
 *  - "Build a Minimal LLM Inference Engine with Paged Attention and Adaptive
 *    KV Cache": Step 1 (block table: a sequence's list of physical page ids)
 *    and Step 4 (gather through the table, then attend).
 *  - "Building a Streaming Sliding-Window Attention Engine in Pure Python":
 *    Step 3 (sliding window: the query at position i sees keys in
 *    [i - w + 1, i]; prefill mask j <= i and i - j < w).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `geom` and `stream` is DEVICE memory
 *    (allocated by the caller, e.g. through torch); `geom` is host memory.
 *    The library never allocates or frees device memory and keeps no state
 *    between calls; its one piece of device memory is the fixed 32 MiB
 *    scratch array of paged_attn_decode_noalloc (one per GPU, part of the
 *    loaded code object).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued on it; nothing synchronises. Results are valid once
 *    the stream reaches them.
 *  - Pools: K and V each [num_blocks, block_size, num_kv_heads, head_dim],
 *    row-major, element type kv_dtype. Position t of sequence s lives in
 *    block block_tables[s * max_blocks_per_seq + t / block_size], slot
 *    t % block_size.
 *  - block_tables: int32 [num_seqs, max_blocks_per_seq]; -1 = unmapped.
 *  - Query head h reads kv head h / (num_heads / num_kv_heads).
 *  - Outputs are float32.
 *  - Return value: PKV_OK, or a negative status (pkv_status_string names it).
 *    Argument checks are synchronous and enqueue nothing when they fail.
 *    Device-resident contents (table entries, lengths) are not validated on
 *    the host; see each call for what the kernels do with out-of-range
 *    entries (they are skipped, never dereferenced).
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of pools, queries and new keys/values. PKV_I8 and PKV_FP8
 * are 8-bit pools (codes with one float32 scale per row), used only through
 * paged_kv_write_quant and paged_attn_decode_quant. */
enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_I8 = 3, PKV_FP8 = 4 };

/* Status codes. */
enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* bad argument (null pointer, negative size, ...) */
  PKV_EUNSUPPORTED = -2,  /* valid but not built: head_dim, block_size, dtype, group size */
  PKV_EWORKSPACE = -3,    /* workspace missing or smaller than the query says */
  PKV_EHIP = -4,          /* a HIP launch failed; pkv_last_hip_error() has the code */
  PKV_ESCRATCH = -5       /* paged_attn_decode_noalloc: the call needs more than its fixed scratch */
};

/* Cache geometry (host struct).
 *   num_blocks    NB, blocks in each pool (> 0)
 *   block_size    B, positions per block: 16 or 32
 *   num_heads     H, query heads
 *   num_kv_heads  Hkv, key/value heads; H % Hkv == 0, H / Hkv in {1, 2, 4, 8}
 *   head_dim      D: 64 or 128
 *   kv_dtype      PKV_F32, PKV_F16 or PKV_BF16 (pools, q, k_new, v_new), or
 *                 PKV_I8 / PKV_FP8 for 8-bit pools (the *_quant calls)
 * One block (B * Hkv * D elements) must hold fewer than 2^31 bytes
 * (PKV_EUNSUPPORTED otherwise). */
typedef struct pkv_geometry {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;
} pkv_geometry_t;

/* paged_kv_write - store new tokens' keys and values in their pool slots
 * (16-bit and fp32 pools; 8-bit pools use paged_kv_write_quant).
 *
 * "Build a Paged KV Cache in Pure Python", Step 3 (append): token n of
 * sequence seq_idx[n] at position pos[n] goes to block
 * block_tables[seq_idx[n]][pos[n] / B], slot pos[n] % B; its whole
 * [num_kv_heads, head_dim] row of keys and of values is copied bit for bit.
 * No other byte of either pool changes.
 *
 *   k_pool, v_pool   [NB, B, Hkv, D] kv_dtype, written in place
 *   k_new, v_new     [num_tokens, Hkv, D] kv_dtype
 *   seq_idx, pos     int32 [num_tokens]
 *   block_tables     int32 [num_seqs, max_blocks_per_seq]
 * A token whose sequence index is outside [0, num_seqs), whose position is
 * negative or past max_blocks_per_seq * B, or whose table entry is outside
 * [0, NB), is skipped (nothing is written for it). Two tokens mapping to the
 * same slot race; callers give distinct slots. num_tokens == 0 is a no-op. */
int paged_kv_write(const pkv_geometry_t* geom, void* k_pool, void* v_pool,
                   const void* k_new, const void* v_new,
                   const int32_t* seq_idx, const int32_t* pos, int32_t num_tokens,
                   const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                   void* stream);

/* Bytes of device workspace paged_attn_decode needs for these sizes and
 * num_workers (as for paged_attn_decode). The automatic worker count
 * depends on the current device, so query on the device that runs the call.
 * Returns 0 for invalid arguments; paged_attn_decode reports those. */
size_t paged_attn_decode_workspace_bytes(const pkv_geometry_t* geom, int32_t num_seqs,
                                         int32_t max_context_len, int32_t window,
                                         int32_t num_sinks, int32_t num_workers);

/* The worker count paged_attn_decode uses for num_workers == 0 with these
 * sizes on the current device (0 for invalid arguments). */
int32_t paged_attn_decode_workers(const pkv_geometry_t* geom, int32_t num_seqs,
                                  int32_t max_context_len, int32_t window, int32_t num_sinks);

/* paged_attn_decode - one query token per sequence attends its cached
 * context through the block table.
 *
 * "Build a Paged KV Cache in Pure Python", Step 4, and "Building a Streaming
 * Sliding-Window Attention Engine in Pure Python", Step 3: for sequence s
 * with context length L = context_lens[s] (which includes the query token,
 * already written: the query sits at position L - 1) and query head h,
 *   lo = window > 0 ? max(0, L - window) : 0
 *   attended t: lo <= t < L, and with a window also t < num_sinks
 *   score_t = scale * sum_d q[s,h,d] * K[t, h / G, d]      for attended t
 *   out[s,h,:] = sum_t softmax(score)_t * V[t, h / G, :]
 *   lse[s,h]  = log(sum_t exp(score_t))   (natural log)
 * L == 0 gives out = 0 and lse = -inf. The sink positions follow "Building a
 * Streaming Sliding-Window Attention Engine in Pure Python", Step 4 (keeping
 * the first tokens when the middle is evicted) and its roadmap's attention
 * sinks item (the first 4 tokens kept regardless of the window).
 *
 *   out           float32 [num_seqs, H, D]
 *   lse           float32 [num_seqs, H], or NULL
 *   q             kv_dtype [num_seqs, H, D]
 *   k_pool/v_pool [NB, B, Hkv, D] kv_dtype
 *   context_lens  int32 [num_seqs], each in [0, max_context_len]
 *   max_context_len  host bound on context_lens (<= max_blocks_per_seq * B)
 *   window        0 = attend everything, else the last `window` positions
 *   num_sinks     with window > 0: also attend positions [0, num_sinks)
 *                 (0 = none; ignored without a window); the blocks between
 *                 the sink blocks and the window may be unmapped (-1)
 *   scale         score scale, typically 1/sqrt(D)
 *   num_workers   wavefronts the attended (sequence, kv head, block) triples
 *                 are divided among, in equal contiguous shares: 0 = an
 *                 automatic count for the current device (whole workgroups
 *                 per compute unit, capped by the number of blocks); any
 *                 positive count is valid (workers beyond the number of
 *                 attended blocks stay idle). Each wavefront keeps
 *                 a running max and sum over its share; a second pass merges
 *                 the shares of every (sequence, head) exactly.
 *   workspace     device scratch of >= paged_attn_decode_workspace_bytes()
 *                 bytes, 16-byte aligned; overwritten by the call, so two
 *                 calls in flight at once need different workspaces
 * Table entries of attended blocks that are -1 or >= NB are skipped: their
 * positions contribute nothing. The partially covered first block of a
 * window (and the blocks holding sink positions) must stay mapped.
 * Scores and outputs accumulate in float32. With 4 or more query heads per
 * kv head (16-bit pools) the products run on the matrix cores and each
 * softmax weight enters P.V as two 16-bit values (hi + lo, about 16
 * significant bits), while the normaliser and lse use the fp32 weights. */
int paged_attn_decode(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                      const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                      int32_t window, int32_t num_sinks, float scale, int32_t num_workers,
                      void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_decode_noalloc - paged_attn_decode without a workspace
 * argument, for callers that cannot allocate device memory around the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The call allocates nothing: its workspace is a fixed 32 MiB
 * device array inside the library, one per GPU, held until the process ends.
 *
 * Arguments, results and the worker count as paged_attn_decode. A call
 * whose workspace (paged_attn_decode_workspace_bytes with the same sizes)
 * exceeds 32 MiB returns PKV_ESCRATCH before anything is enqueued. Every
 * call on one GPU uses that GPU's single scratch array: two calls that can
 * run at the same time on one GPU (different streams, or different host
 * threads) race and give wrong results; calls in one stream's order are
 * safe. Nothing in the scratch needs clearing between calls. */
int paged_attn_decode_noalloc(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                              const void* k_pool, const void* v_pool, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                              int32_t num_workers, void* stream);

/* paged_attn_prefill - causal attention of a chunk of query tokens per
 * sequence over everything cached before them and the chunk itself.
 *
 * "Building a Streaming Sliding-Window Attention Engine in Pure Python",
 * Step 3 (prefill mask: causal, and i - j < w with a window) and Step 4
 * (keys/values are in the cache before attention), read for a chunk that
 * follows a cached prefix: sequence s owns query rows
 * [q_start[s], q_start[s+1]); its chunk of C = q_start[s+1] - q_start[s]
 * rows are its last C positions, so row i sits at p = L - C + i with
 * L = context_lens[s] (the chunk's keys/values are already written). Row i
 * of head h attends positions t with t <= p and, when window > 0,
 * t > p - window or t < num_sinks; the result is the same softmax-weighted
 * sum as decode.
 *
 *   out     float32 [q_start[num_seqs], H, D]
 *   lse     float32 [q_start[num_seqs], H], or NULL
 *   q       kv_dtype [q_start[num_seqs], H, D] (PKV_F16 or PKV_BF16 only)
 *   q_start int32 [num_seqs + 1], non-decreasing, q_start[0] == 0
 *   max_q_len        host bound on the chunk lengths
 *   max_context_len  host bound on context_lens (<= max_blocks_per_seq * B)
 * Requires C <= L for every sequence. Scores and outputs accumulate in
 * float32. The softmax weights multiply V on the fp16 matrix cores for both
 * input types: each weight is rounded to fp16 (11 significant bits), and a
 * bf16 V is converted to fp16, exact for |v| in [2^-17, 65280] (65280 is
 * the largest bf16 value fp16 holds; smaller magnitudes keep their bits down
 * to 2^-24). bf16 V rows with a larger magnitude are outside this call's
 * range (they saturate at 65504); the binding's debug mode rejects them.
 * The output divides by the sum of the weights as rounded, and lse uses the
 * same sum, so that out and lse describe the same weights (partial results
 * merged through lse stay exact): that sum is within 2^-11 relative of the
 * exact one, plus 2^-25 per subnormal weight against a sum of at least 1,
 * so lse is within 6e-4 of the exact log-sum-exp. */
int paged_attn_prefill(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                       const int32_t* q_start, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                       int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                       void* stream);

/* 8-bit key/value pages.
 *
 * "Build a Memory-Compressed Attention Engine with KV Caching from
 * Scratch", section "Extending It: Your Roadmap to Senior-Level", item 2
 * (quantized KV cache: INT8 or FP8 keys and values cut the bytes a decode
 * step reads). Encoding of one row x (the D values of one block slot and kv
 * head), all in float32 with correctly rounded division:
 *   amax = max_d |x_d|, scale = amax / QMAX, inv = QMAX / amax (0 if amax 0)
 *   PKV_I8:  code_d = round-half-even(x_d * inv) clamped to [-127, 127]
 *            (QMAX 127), two's complement
 *   PKV_FP8: code_d = x_d * inv rounded to the nearest OCP FP8 E4M3 value
 *            (bias 7, largest 448 = QMAX, ties to even)
 *   decoded value = code_d * scale.
 * Pools hold codes, uint8 [NB, B, Hkv, D] (the 16-bit layout); scale pools
 * hold the row scales, float32 [NB, Hkv, B]. */

/* paged_kv_write_quant - encode new tokens' keys and values into 8-bit
 * pools. Slot rule, skipping of invalid tokens and races as paged_kv_write
 * ("Build a Paged KV Cache in Pure Python", Step 3); each (token, kv head)
 * row is encoded as above and its scale stored at
 * scale[block][kv head][slot]. Rows never written keep whatever the caller
 * put there.
 *
 *   geom->kv_dtype   PKV_I8 or PKV_FP8
 *   k_pool, v_pool   [NB, B, Hkv, D] codes, written in place
 *   k_scale, v_scale float32 [NB, Hkv, B], written in place
 *   k_new, v_new     [num_tokens, Hkv, D] new_dtype (PKV_F32, PKV_F16 or
 *                    PKV_BF16)
 *   seq_idx, pos, block_tables, num_seqs, max_blocks_per_seq: as
 *                    paged_kv_write */
int paged_kv_write_quant(const pkv_geometry_t* geom, void* k_pool, void* v_pool, float* k_scale,
                         float* v_scale, const void* k_new, const void* v_new, int32_t new_dtype,
                         const int32_t* seq_idx, const int32_t* pos, int32_t num_tokens,
                         const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                         void* stream);

/* paged_attn_decode_quant - paged_attn_decode over 8-bit pools: the same
 * attention with every key and value replaced by its decoded value
 * code * scale. Scores and outputs accumulate in float32 (the row scales
 * factor out of each dot product).
 *
 *   geom->kv_dtype    PKV_I8 or PKV_FP8; num_heads / num_kv_heads in {1, 2, 4, 8}
 *                     (each page is read once for all query heads of its
 *                     kv head, as with 16-bit pools)
 *   q                 q_dtype [num_seqs, H, D], q_dtype PKV_F16 or PKV_BF16
 *   k_pool, v_pool    codes [NB, B, Hkv, D]
 *   k_scale, v_scale  float32 [NB, Hkv, B]
 *   all other arguments, the workspace (paged_attn_decode_workspace_bytes
 *   with this geometry) and the worker count as paged_attn_decode. */
int paged_attn_decode_quant(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                            int32_t q_dtype, const void* k_pool, const void* v_pool,
                            const float* k_scale, const float* v_scale, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                            int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_prefill_quant - paged_attn_prefill over 8-bit pools ("Build a
 * Memory-Compressed Attention Engine with KV Caching from Scratch",
 * "Extending It" item 2, with the prefill of "Building a Streaming
 * Sliding-Window Attention Engine in Pure Python", Step 3): the same
 * attention with every key and value replaced by its decoded value
 * code * scale.
 *
 * One kernel on `stream`, no workspace: each tile of key positions is
 * gathered as codes through the block table and widened in the kernel's
 * on-chip memory (codes unchanged as q_dtype values for K and fp16 values
 * for V; exact). Key t's score is its dot product with the codes times its
 * K scale (float32). The softmax weight of key t times its V scale, taken
 * relative to a running reference that keeps it at most 256 (log2 of the V
 * scale joins the score before the maximum), is rounded to fp16 and
 * multiplied with the V codes on the matrix cores; the normaliser (and lse)
 * sums those rounded products divided by their V scales (float32), i.e. the
 * weights the matrix cores actually apply, so the output is their exact
 * weighted average. There is no limit on the scales' magnitudes. A zero V
 * row (scale 0) keeps its weight in the normaliser.
 *
 *   geom->kv_dtype    PKV_I8 or PKV_FP8; head_dim, block_size and
 *                     num_heads / num_kv_heads as paged_attn_prefill
 *   q                 q_dtype [q_start[num_seqs], H, D], q_dtype PKV_F16 or
 *                     PKV_BF16
 *   k_pool, v_pool    codes [NB, B, Hkv, D]
 *   k_scale, v_scale  float32 [NB, Hkv, B]
 *   all other arguments as paged_attn_prefill. */
int paged_attn_prefill_quant(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                             int32_t q_dtype, const int32_t* q_start, const void* k_pool, const void* v_pool,
                             const float* k_scale, const float* v_scale, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_q_len, int32_t max_context_len, int32_t window, int32_t num_sinks,
                             float scale, void* stream);

/* paged_kv_copy_blocks - copy whole blocks: pair i copies block src[i] to
 * block dst[i] in both pools (every slot and kv head; with 8-bit pools the
 * rows' scales too). This is the copy of copy-on-write: a sequence about to
 * append into a block it shares with others first gets a private copy
 * ("Build a Minimal LLM Inference Engine with Paged Attention and Adaptive
 * KV Cache", Step 1: a page is shared while its refcount is above one;
 * "Building a Streaming Sliding-Window Attention Engine in Pure Python",
 * Step 4: prefixes are reused across requests).
 *
 *   k_pool, v_pool    [NB, B, Hkv, D] kv_dtype, written in place
 *   k_scale, v_scale  [NB, Hkv, B] float32 for 8-bit pools (required), NULL
 *                     otherwise (both or neither)
 *   src, dst          int32 [num_pairs] block ids
 * Pairs with an id outside [0, NB) or src == dst are skipped. A block that
 * is a destination must not also be a source or another pair's
 * destination in the same call (the copies run in parallel). */
int paged_kv_copy_blocks(const pkv_geometry_t* geom, void* k_pool, void* v_pool, float* k_scale,
                         float* v_scale, const int32_t* src, const int32_t* dst, int32_t num_pairs,
                         void* stream);

/* paged_attn_mixed - one call for a batch that mixes prefill chunks and
 * decode rows ("Building a Streaming Sliding-Window Attention Engine in Pure
 * Python", roadmap item 2, continuous batching: slots of finished requests
 * are refilled mid-stream, so one step holds new prompts' chunks next to
 * running sequences' decode tokens): the arguments and the result are those of
 * paged_attn_prefill (sequence s owns rows [q_start[s], q_start[s+1]), its
 * last positions); sequences with exactly one row are computed by the
 * split decode kernel (workspace, num_workers as paged_attn_decode; size it
 * with paged_attn_decode_workspace_bytes for num_seqs sequences), the others
 * by the prefill kernel, both enqueued on `stream`. PKV_F16 / PKV_BF16. */
int paged_attn_mixed(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                     const int32_t* q_start, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                     int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                     int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_mixed_quant - paged_attn_mixed over 8-bit pools (the 8-bit
 * pages of paged_attn_decode_quant with the continuous batching of
 * paged_attn_mixed): sequences with one query row are computed as
 * paged_attn_decode_quant computes them, the others as
 * paged_attn_prefill_quant, all enqueued on `stream`.
 *
 *   geom->kv_dtype, q / q_dtype, k_pool, v_pool, k_scale, v_scale: as
 *                     paged_attn_prefill_quant (q has q_start[num_seqs] rows)
 *   workspace         the decode workspace: device, 16-byte aligned, at
 *                     least paged_attn_decode_workspace_bytes(geom, num_seqs,
 *                     max_context_len, window, num_sinks, num_workers) bytes
 *                     (else PKV_EWORKSPACE, before anything is enqueued)
 *   all other arguments as paged_attn_mixed. */
int paged_attn_mixed_quant(const pkv_geometry_t* geom, float* out, float* lse, const void* q, int32_t q_dtype,
                           const int32_t* q_start, const void* k_pool, const void* v_pool, const float* k_scale,
                           const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                           int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                           int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream);

/* paged_kv_compress - compress groups of whole blocks into slots ("Build a
 * Memory-Compressed Attention Engine with KV Caching from Scratch", Step 2:
 * a group of positions is summarised by the mean of its keys and the mean
 * of its values, per head; Step 3: the oldest half of a full window becomes
 * one slot). Op i replaces row dst_slot[i] of block dst_block[i] (every kv
 * head, K and V) with the mean of all B rows of each block
 * src_blocks[i * blocks_per_slot .. (i + 1) * blocks_per_slot).
 *
 *   k_pool, v_pool    [NB, B, Hkv, D] PKV_F32 / PKV_F16 / PKV_BF16, in place
 *   src_blocks        int32 [num_ops, blocks_per_slot] block ids
 *   dst_block         int32 [num_ops] block id of the slot row
 *   dst_slot          int32 [num_ops] row inside it, 0 .. B-1
 * The mean is computed in float64 (the sum is exact for rows whose
 * magnitudes span fewer than about 53 - 24 - log2(rows) binades), divided
 * by the number of rows and rounded once to the pool type (nearest, ties to
 * even). Source ids outside [0, NB) are left out of the mean; an op with no
 * valid source, or a destination outside the pool, writes nothing. A row a
 * call writes must not lie in a block any op of the same call reads. Run it
 * before reusing the source blocks (stream order). 8-bit pools:
 * PKV_EUNSUPPORTED. blocks_per_slot * B at most 2^24. */
int paged_kv_compress(const pkv_geometry_t* geom, void* k_pool, void* v_pool, const int32_t* src_blocks,
                      int32_t blocks_per_slot, const int32_t* dst_block, const int32_t* dst_slot, int32_t num_ops,
                      void* stream);

/* paged_attn_decode_compressed - single-query decode over two tiers ("Build
 * a Memory-Compressed Attention Engine with KV Caching from Scratch",
 * Component Breakdown and Step 4: the query attends the full-resolution
 * window and the compressed slots together, one softmax over both).
 *
 * Arguments as paged_attn_decode (no sinks), plus per sequence s:
 *   full_start   int32 [num_seqs]  first position still held at full
 *                resolution; positions [max(full_start, L - window), L) are
 *                attended through block_tables (clamped to [0, L])
 *   slot_tables  int32 [num_seqs, max_slot_blocks]  blocks holding slot rows;
 *                slot row r of s is row r % B of block slot_tables[s][r / B]
 *   num_slots    int32 [num_seqs]  slot rows [0, num_slots) are attended
 *                (clamped to [0, max_slot_blocks * B])
 * Size the workspace with paged_attn_decode_workspace_bytes(num_seqs,
 * max_context_len, window, 0, num_workers). Table entries outside [0, NB)
 * of attended blocks are skipped. PKV_F32 / PKV_F16 / PKV_BF16 pools. */
int paged_attn_decode_compressed(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                                 const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* full_start,
                                 const int32_t* slot_tables, int32_t max_slot_blocks, const int32_t* num_slots,
                                 int32_t num_seqs, int32_t max_context_len, int32_t window, float scale,
                                 int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream);

/* Name of a status code (static string). */
const char* pkv_status_string(int status);

/* hipError_t of the most recent PKV_EHIP returned on the calling thread. */
int pkv_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
