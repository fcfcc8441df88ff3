// Internal interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct WriteArgs {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* tables;
  int32_t num_tokens, num_seqs, mb, nb, B, Hkv, D, elem_bytes;
};

// Quantising write: rows of k_new/v_new (in_dtype) become 8-bit codes in the
// pools and one fp32 scale per row in the [NB, Hkv, B] scale pools.
struct WriteQuantArgs {
  void* k_pool;
  void* v_pool;
  float* k_scale;
  float* v_scale;
  const void* k_new;
  const void* v_new;
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* tables;
  int32_t num_tokens, num_seqs, mb, nb, B, Hkv, D, kv_dtype, in_dtype;
};

struct CopyBlocksArgs {
  void* k_pool;
  void* v_pool;
  float* k_scale;  // 8-bit pools: [NB, Hkv, B] row scales, copied along; else null
  float* v_scale;
  const int32_t* src;
  const int32_t* dst;
  int32_t n, nb, B, Hkv, D, elem_bytes;
};

// Compression of groups of blocks into slot rows: op i averages every row of
// blocks src[i * bps .. i * bps + bps) into row dst_slot[i] of block
// dst_block[i], for K and V.
struct CompressArgs {
  void* k_pool;
  void* v_pool;
  const int32_t* src;
  const int32_t* dst_block;
  const int32_t* dst_slot;
  int32_t n, bps, nb, B, Hkv, D, dtype;
};

struct DecodeArgs {
  float* out;
  float* lse;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  const float* k_scale;  // 8-bit pools only: [NB, Hkv, B] row scales
  const float* v_scale;
  int32_t q_dtype;       // 8-bit pools only: type of q (fp16 or bf16)
  int32_t* ws_cum;  // [S + 1] attended blocks before each sequence
  float* ws_ml;     // [slots, G, 2] partial running max (log2 units) and sum
  float* ws_o;      // [slots, G, D] partial unnormalised outputs
  int32_t S, H, Hkv, D, B, mb, nb, window, dtype, max_context_len;
  int32_t n_workers;  // wavefronts the attended blocks are divided among
  float scale;
  int32_t sinks;      // with a window: positions below this are attended too
  // Mixed batches: null for plain decode. Otherwise [S + 1] row offsets of a
  // prefill-style batch; sequence s is a decode row iff it has exactly one
  // row, which is q/out/lse row q_start[s]; other sequences are left alone.
  const int32_t* q_start;
  // Compressed slots: null for plain decode. Otherwise per sequence the
  // first full-resolution position [S], the slot table [S, msb] and the
  // number of valid ring rows [S]; decode attends those rows, then the
  // positions [max(full_start, L - window), L).
  const int32_t* full_start;
  const int32_t* slot_tables;
  const int32_t* num_slots;
  int32_t msb;
};

struct PrefillArgs {
  float* out;
  float* lse;
  const void* q;
  const int32_t* q_start;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  int32_t S, H, Hkv, D, B, mb, nb, window, dtype, max_q_len, max_context_len;
  float scale;
  int32_t sinks;      // with a window: positions below this are attended too
  int32_t skip_single;  // mixed batches: sequences with one row are left to decode
  // Row scales [nb, Hkv, B] when the pools hold 8-bit codes (null
  // otherwise): a key's score is multiplied by its K scale, a weight by its
  // key's V scale.
  const float* k_scale;
  const float* v_scale;
  int32_t code_dtype = 0;  // 8-bit pools: PKV_I8 (3) or PKV_FP8 (4) codes; dtype is then q's type
  int32_t grid_q = 0, grid_y = 0;  // set by the launcher: query tiles and kv-head groups per sequence
};


hipError_t launch_kv_write(const WriteArgs& a, hipStream_t st);
bool kv_write_quant_supported(int kv_dtype, int in_dtype, int D);
hipError_t launch_kv_write_quant(const WriteQuantArgs& a, hipStream_t st);
hipError_t launch_kv_copy_blocks(const CopyBlocksArgs& a, hipStream_t st);
hipError_t launch_kv_compress(const CompressArgs& a, hipStream_t st);



// q_dtype is the type of q (equal to dtype for the 16-bit and fp32 pools).
bool decode_supported(int dtype, int q_dtype, int D, int B, int G);
// Decode worker (wavefront) count used when the caller passes 0.
int decode_auto_workers(int dtype, int q_dtype, int D, int B, int G);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

bool prefill_supported(int dtype, int D, int B, int G);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

}  // namespace pkv
