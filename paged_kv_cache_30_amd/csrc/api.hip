// C ABI of the library: argument checks, partition sizing, launches on the
// caller's stream. Declarations and the contract are in paged_attn.h.
#include "paged_attn.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PKV_OK;
  g_last_hip_error = (int)e;
  return PKV_EHIP;
}

int elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : (dtype == PKV_I8 || dtype == PKV_FP8) ? 1 : 2; }
bool is_quant(int dtype) { return dtype == PKV_I8 || dtype == PKV_FP8; }
// The query type that sizes the automatic decode split: the pools' own for
// 16-bit and fp32 pools, bf16 for 8-bit pools (both query types of an 8-bit
// pool use the same count, so workspace queries need no query type).
int split_q_dtype(int kv_dtype) { return is_quant(kv_dtype) ? PKV_BF16 : kv_dtype; }

// Geometry checks common to every call. Returns PKV_OK, PKV_EINVAL or
// PKV_EUNSUPPORTED.
int check_geometry(const pkv_geometry_t* g) {
  if (!g) return PKV_EINVAL;
  if (g->num_blocks <= 0 || g->block_size <= 0 || g->num_heads <= 0 || g->num_kv_heads <= 0 ||
      g->head_dim <= 0)
    return PKV_EINVAL;
  if (g->num_heads % g->num_kv_heads) return PKV_EINVAL;
  if (g->kv_dtype != PKV_F32 && g->kv_dtype != PKV_F16 && g->kv_dtype != PKV_BF16 && !is_quant(g->kv_dtype))
    return PKV_EUNSUPPORTED;
  if (g->head_dim != 64 && g->head_dim != 128) return PKV_EUNSUPPORTED;
  if (g->block_size != 16 && g->block_size != 32) return PKV_EUNSUPPORTED;
  const int G = g->num_heads / g->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PKV_EUNSUPPORTED;
  // Kernels address inside a block with 32-bit offsets.
  if ((long long)g->block_size * g->num_kv_heads * g->head_dim * elem_bytes(g->kv_dtype) > INT32_MAX)
    return PKV_EUNSUPPORTED;
  return PKV_OK;
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Blocks one sequence's attended positions can span.
int span_blocks(const pkv_geometry_t* g, int max_context_len, int window, int sinks) {
  const int B = g->block_size;
  int n = ceil_div(max_context_len, B);
  if (window > 0) {
    const long long w = (long long)ceil_div(window, B) + 1 + ceil_div(sinks, B);
    if (w < n) n = (int)w;
  }
  return n;
}

// Decode work split: num_workers wavefronts (0 = automatic, but no more than
// the attended blocks could occupy) and the workspace layout for them.
struct DecodeSplit {
  int workers;
  size_t cum_bytes, ml_bytes, o_bytes;
  size_t total() const { return cum_bytes + ml_bytes + o_bytes; }
};

int decode_split(const pkv_geometry_t* g, int num_seqs, int max_context_len, int window, int sinks,
                 int num_workers, DecodeSplit* out) {
  if (num_workers < 0) return PKV_EINVAL;
  const int G = g->num_heads / g->num_kv_heads;
  int nw = num_workers;
  if (nw == 0) {
    const long long bound =
        (long long)num_seqs * g->num_kv_heads * span_blocks(g, max_context_len, window, sinks);
    nw = pkv::decode_auto_workers(g->kv_dtype, split_q_dtype(g->kv_dtype), g->head_dim, g->block_size, G);
    if (bound < nw) nw = bound > 0 ? (int)bound : 1;
  }
  const size_t slots = (size_t)nw + (size_t)num_seqs * g->num_kv_heads;
  out->workers = nw;
  out->cum_bytes = (((size_t)num_seqs + 1) * sizeof(int32_t) + 255) / 256 * 256;
  out->ml_bytes = (slots * G * 2 * sizeof(float) + 255) / 256 * 256;
  out->o_bytes = slots * G * g->head_dim * sizeof(float);
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_kv_write(const pkv_geometry_t* geom, void* k_pool, void* v_pool, const void* k_new,
                   const void* v_new, const int32_t* seq_idx, const int32_t* pos, int32_t num_tokens,
                   const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                   void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (is_quant(geom->kv_dtype)) return PKV_EUNSUPPORTED;  // paged_kv_write_quant
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq <= 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !seq_idx || !pos || !block_tables || num_seqs == 0)
    return PKV_EINVAL;
  pkv::WriteArgs a{k_pool, v_pool, k_new, v_new, seq_idx, pos, block_tables, num_tokens, num_seqs,
                   max_blocks_per_seq, geom->num_blocks, geom->block_size, geom->num_kv_heads,
                   geom->head_dim, elem_bytes(geom->kv_dtype)};
  return hip_status(pkv::launch_kv_write(a, (hipStream_t)stream));
}

int32_t paged_attn_decode_workers(const pkv_geometry_t* geom, int32_t num_seqs, int32_t max_context_len,
                                  int32_t window, int32_t num_sinks) {
  if (check_geometry(geom) || num_seqs < 0 || max_context_len < 0 || window < 0 || num_sinks < 0) return 0;
  DecodeSplit sp;
  if (decode_split(geom, num_seqs, max_context_len, window, window > 0 ? num_sinks : 0, 0, &sp)) return 0;
  return sp.workers;
}

size_t paged_attn_decode_workspace_bytes(const pkv_geometry_t* geom, int32_t num_seqs,
                                         int32_t max_context_len, int32_t window, int32_t num_sinks,
                                         int32_t num_workers) {
  if (check_geometry(geom) || num_seqs <= 0 || max_context_len < 0 || window < 0 || num_sinks < 0) return 0;
  DecodeSplit sp;
  if (decode_split(geom, num_seqs, max_context_len, window, window > 0 ? num_sinks : 0, num_workers, &sp))
    return 0;
  return sp.total();
}

}  // extern "C"

namespace {

// Compressed slots of a decode call (all null for plain decode).
struct SlotArgs {
  const int32_t* full_start = nullptr;
  const int32_t* slot_tables = nullptr;
  const int32_t* num_slots = nullptr;
  int32_t max_slot_blocks = 0;
};

int decode_common(const pkv_geometry_t* geom, float* out, float* lse, const void* q, int q_dtype,
                  const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                  int32_t num_seqs, int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                  int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream,
                  const SlotArgs& slots = SlotArgs()) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || window < 0 || num_sinks < 0 ||
      num_workers < 0 || !isfinite(scale))
    return PKV_EINVAL;
  if (window == 0) num_sinks = 0;  // without a window every position is attended
  if ((long long)max_context_len > (long long)max_blocks_per_seq * geom->block_size) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_EINVAL;
  if (is_quant(geom->kv_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  const pkv_geometry_t& view = *geom;
  const int G = view.num_heads / view.num_kv_heads;
  if (!pkv::decode_supported(view.kv_dtype, q_dtype, view.head_dim, view.block_size, G))
    return PKV_EUNSUPPORTED;
  DecodeSplit sp;
  int st = decode_split(&view, num_seqs, max_context_len, window, num_sinks, num_workers, &sp);
  if (st) return st;
  if (!workspace || workspace_bytes < sp.total() || ((uintptr_t)workspace & 15)) return PKV_EWORKSPACE;
  char* ws = (char*)workspace;
  pkv::DecodeArgs a{out, lse, q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, q_dtype,
                    (int32_t*)ws, (float*)(ws + sp.cum_bytes), (float*)(ws + sp.cum_bytes + sp.ml_bytes),
                    num_seqs, view.num_heads, view.num_kv_heads, view.head_dim, view.block_size,
                    max_blocks_per_seq, view.num_blocks, window, view.kv_dtype, max_context_len,
                    sp.workers, scale, num_sinks, nullptr, slots.full_start, slots.slot_tables,
                    slots.num_slots, slots.max_slot_blocks};
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int paged_attn_decode(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                      const void* k_pool, const void* v_pool, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                      int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                      int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (is_quant(geom->kv_dtype)) return PKV_EUNSUPPORTED;  // paged_attn_decode_quant
  return decode_common(geom, out, lse, q, geom->kv_dtype, k_pool, v_pool, nullptr, nullptr, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, window, num_sinks, scale,
                       num_workers, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of paged_attn_decode_noalloc: the decode workspace (attended-block
// prefix sums and the split's partial results) in a fixed device array, so
// that the call allocates nothing. Every GPU the library runs on holds its
// own copy for the life of the process. In host code the array's name is
// not a device address: kernels get the address hipGetSymbolAddress gives
// for the current device, looked up once per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch (nullptr and the HIP error on failure).
void* scratch_for_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int paged_attn_decode_noalloc(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                              const void* k_pool, const void* v_pool, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                              int32_t num_workers, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (is_quant(geom->kv_dtype)) return PKV_EUNSUPPORTED;
  if (num_seqs < 0 || max_context_len < 0 || window < 0 || num_sinks < 0 || num_workers < 0) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  const size_t need = paged_attn_decode_workspace_bytes(geom, num_seqs, max_context_len, window, num_sinks,
                                                        num_workers);
  if (need == 0) return PKV_EINVAL;
  if (need > kScratchBytes) return PKV_ESCRATCH;
  hipError_t err;
  void* ws = scratch_for_current_device(&err);
  if (!ws) return hip_status(err);
  // Nothing in the workspace has to start at zero: every word the kernels
  // read is written earlier in the same call.
  return decode_common(geom, out, lse, q, geom->kv_dtype, k_pool, v_pool, nullptr, nullptr, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, window, num_sinks, scale,
                       num_workers, ws, kScratchBytes, stream);
}

int paged_attn_decode_quant(const pkv_geometry_t* geom, float* out, float* lse, const void* q, int32_t q_dtype,
                            const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                            int32_t window, int32_t num_sinks, float scale, int32_t num_workers,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (!is_quant(geom->kv_dtype)) return PKV_EINVAL;
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  return decode_common(geom, out, lse, q, q_dtype, k_pool, v_pool, k_scale, v_scale, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, window, num_sinks, scale,
                       num_workers, workspace, workspace_bytes, stream);
}

int paged_kv_write_quant(const pkv_geometry_t* geom, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                         const void* k_new, const void* v_new, int32_t new_dtype, const int32_t* seq_idx,
                         const int32_t* pos, int32_t num_tokens, const int32_t* block_tables, int32_t num_seqs,
                         int32_t max_blocks_per_seq, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (!is_quant(geom->kv_dtype)) return PKV_EINVAL;
  if (new_dtype != PKV_F32 && new_dtype != PKV_F16 && new_dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq <= 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_scale || !v_scale || !k_new || !v_new || !seq_idx || !pos || !block_tables ||
      num_seqs == 0)
    return PKV_EINVAL;
  if (!pkv::kv_write_quant_supported(geom->kv_dtype, new_dtype, geom->head_dim)) return PKV_EUNSUPPORTED;
  pkv::WriteQuantArgs a{k_pool, v_pool, k_scale, v_scale, k_new, v_new, seq_idx, pos, block_tables,
                        num_tokens, num_seqs, max_blocks_per_seq, geom->num_blocks, geom->block_size,
                        geom->num_kv_heads, geom->head_dim, geom->kv_dtype, new_dtype};
  return hip_status(pkv::launch_kv_write_quant(a, (hipStream_t)stream));
}

int paged_attn_prefill(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                       const int32_t* q_start, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                       int32_t max_context_len, int32_t window, int32_t num_sinks, float scale, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_q_len < 0 || max_context_len < 0 || window < 0 ||
      num_sinks < 0 || !isfinite(scale))
    return PKV_EINVAL;
  if (window == 0) num_sinks = 0;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * geom->block_size) return PKV_EINVAL;
  if (max_q_len > max_context_len) return PKV_EINVAL;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_EINVAL;
  const int G = geom->num_heads / geom->num_kv_heads;
  if (is_quant(geom->kv_dtype) ||
      !pkv::prefill_supported(geom->kv_dtype, geom->head_dim, geom->block_size, G))
    return PKV_EUNSUPPORTED;
  pkv::PrefillArgs a{out, lse, q, q_start, k_pool, v_pool, block_tables, context_lens, num_seqs,
                     geom->num_heads, geom->num_kv_heads, geom->head_dim, geom->block_size,
                     max_blocks_per_seq, geom->num_blocks, window, geom->kv_dtype, max_q_len,
                     max_context_len, scale, num_sinks};
  return hip_status(pkv::launch_prefill(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The prefill kernel over 8-bit pools, for the sequences with at least
// min_rows query rows (1: every chunk; 2: the chunks of a mixed batch, whose
// single rows decode computes).
int prefill_quant_common(const pkv_geometry_t* geom, float* out, float* lse, const void* q, int32_t q_dtype,
                         const int32_t* q_start, const void* k_pool, const void* v_pool, const float* k_scale,
                         const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                         int32_t max_context_len, int32_t window, int32_t num_sinks, float scale, void* stream,
                         int min_rows) {
  int st = check_geometry(geom);
  if (st) return st;
  if (!is_quant(geom->kv_dtype) || (q_dtype != PKV_F16 && q_dtype != PKV_BF16)) return PKV_EUNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_q_len < 0 || max_context_len < 0 || window < 0 ||
      num_sinks < 0 || !isfinite(scale))
    return PKV_EINVAL;
  if (window == 0) num_sinks = 0;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * geom->block_size) return PKV_EINVAL;
  if (max_q_len > max_context_len) return PKV_EINVAL;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !q_start || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables || !context_lens)
    return PKV_EINVAL;
  const int G = geom->num_heads / geom->num_kv_heads;
  if (!pkv::prefill_supported(q_dtype, geom->head_dim, geom->block_size, G)) return PKV_EUNSUPPORTED;
  pkv::PrefillArgs a{out, lse, q, q_start, k_pool, v_pool, block_tables, context_lens, num_seqs,
                     geom->num_heads, geom->num_kv_heads, geom->head_dim, geom->block_size,
                     max_blocks_per_seq, geom->num_blocks, window, q_dtype, max_q_len,
                     max_context_len, scale, num_sinks};
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.code_dtype = geom->kv_dtype;
  a.skip_single = min_rows > 1;
  return hip_status(pkv::launch_prefill(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int paged_attn_prefill_quant(const pkv_geometry_t* geom, float* out, float* lse, const void* q, int32_t q_dtype,
                             const int32_t* q_start, const void* k_pool, const void* v_pool, const float* k_scale,
                             const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                             int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                             void* stream) {
  return prefill_quant_common(geom, out, lse, q, q_dtype, q_start, k_pool, v_pool, k_scale, v_scale, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs, max_q_len, max_context_len, window,
                              num_sinks, scale, stream, 1);
}

int paged_kv_copy_blocks(const pkv_geometry_t* geom, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                        const int32_t* src, const int32_t* dst, int32_t num_pairs, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (num_pairs < 0) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src || !dst) return PKV_EINVAL;
  if ((k_scale == nullptr) != (v_scale == nullptr)) return PKV_EINVAL;
  if (is_quant(geom->kv_dtype) && !k_scale) return PKV_EINVAL;
  pkv::CopyBlocksArgs a{k_pool, v_pool, k_scale, v_scale, src, dst, num_pairs, geom->num_blocks,
                        geom->block_size, geom->num_kv_heads, geom->head_dim, elem_bytes(geom->kv_dtype)};
  return hip_status(pkv::launch_kv_copy_blocks(a, (hipStream_t)stream));
}

int paged_attn_mixed(const pkv_geometry_t* geom, float* out, float* lse, const void* q, const int32_t* q_start,
                     const void* k_pool, const void* v_pool, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                     int32_t max_context_len, int32_t window, int32_t num_sinks, float scale, int32_t num_workers,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_q_len < 0 || max_context_len < 0 || window < 0 ||
      num_sinks < 0 || num_workers < 0 || !isfinite(scale))
    return PKV_EINVAL;
  if (window == 0) num_sinks = 0;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * geom->block_size) return PKV_EINVAL;
  if (max_q_len > max_context_len) return PKV_EINVAL;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_EINVAL;
  const int G = geom->num_heads / geom->num_kv_heads;
  if (is_quant(geom->kv_dtype) ||
      !pkv::prefill_supported(geom->kv_dtype, geom->head_dim, geom->block_size, G) ||
      !pkv::decode_supported(geom->kv_dtype, geom->kv_dtype, geom->head_dim, geom->block_size, G))
    return PKV_EUNSUPPORTED;
  DecodeSplit sp;
  st = decode_split(geom, num_seqs, max_context_len, window, num_sinks, num_workers, &sp);
  if (st) return st;
  if (!workspace || workspace_bytes < sp.total() || ((uintptr_t)workspace & 15)) return PKV_EWORKSPACE;
  char* ws = (char*)workspace;
  pkv::DecodeArgs da{out, lse, q, k_pool, v_pool, block_tables, context_lens, nullptr, nullptr, geom->kv_dtype,
                     (int32_t*)ws, (float*)(ws + sp.cum_bytes), (float*)(ws + sp.cum_bytes + sp.ml_bytes),
                     num_seqs, geom->num_heads, geom->num_kv_heads, geom->head_dim, geom->block_size,
                     max_blocks_per_seq, geom->num_blocks, window, geom->kv_dtype, max_context_len,
                     sp.workers, scale, num_sinks, q_start};
  st = hip_status(pkv::launch_decode(da, (hipStream_t)stream));
  if (st || max_q_len < 2) return st;
  pkv::PrefillArgs pa{out, lse, q, q_start, k_pool, v_pool, block_tables, context_lens, num_seqs,
                      geom->num_heads, geom->num_kv_heads, geom->head_dim, geom->block_size,
                      max_blocks_per_seq, geom->num_blocks, window, geom->kv_dtype, max_q_len,
                      max_context_len, scale, num_sinks, 1};
  return hip_status(pkv::launch_prefill(pa, (hipStream_t)stream));
}

int paged_attn_mixed_quant(const pkv_geometry_t* geom, float* out, float* lse, const void* q, int32_t q_dtype,
                           const int32_t* q_start, const void* k_pool, const void* v_pool, const float* k_scale,
                           const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                           int32_t max_context_len, int32_t window, int32_t num_sinks, float scale,
                           int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (!is_quant(geom->kv_dtype) || (q_dtype != PKV_F16 && q_dtype != PKV_BF16)) return PKV_EUNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_q_len < 0 || max_context_len < 0 || window < 0 ||
      num_sinks < 0 || num_workers < 0 || !isfinite(scale))
    return PKV_EINVAL;
  if (window == 0) num_sinks = 0;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * geom->block_size) return PKV_EINVAL;
  if (max_q_len > max_context_len) return PKV_EINVAL;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !q_start || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables || !context_lens)
    return PKV_EINVAL;
  const int G = geom->num_heads / geom->num_kv_heads;
  const pkv_geometry_t& view = *geom;
  if (!pkv::prefill_supported(q_dtype, geom->head_dim, geom->block_size, G) ||
      !pkv::decode_supported(view.kv_dtype, q_dtype, view.head_dim, view.block_size,
                             view.num_heads / view.num_kv_heads))
    return PKV_EUNSUPPORTED;
  DecodeSplit sp;
  st = decode_split(&view, num_seqs, max_context_len, window, num_sinks, num_workers, &sp);
  if (st) return st;
  if (!workspace || workspace_bytes < sp.total() || ((uintptr_t)workspace & 15)) return PKV_EWORKSPACE;
  char* ws = (char*)workspace;
  pkv::DecodeArgs da{out, lse, q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, q_dtype,
                     (int32_t*)ws, (float*)(ws + sp.cum_bytes), (float*)(ws + sp.cum_bytes + sp.ml_bytes),
                     num_seqs, view.num_heads, view.num_kv_heads, view.head_dim, view.block_size,
                     max_blocks_per_seq, view.num_blocks, window, view.kv_dtype, max_context_len,
                     sp.workers, scale, num_sinks, q_start};
  st = hip_status(pkv::launch_decode(da, (hipStream_t)stream));
  if (st || max_q_len < 2) return st;
  return prefill_quant_common(geom, out, lse, q, q_dtype, q_start, k_pool, v_pool, k_scale, v_scale, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs, max_q_len, max_context_len, window,
                              num_sinks, scale, stream, 2);
}

int paged_kv_compress(const pkv_geometry_t* geom, void* k_pool, void* v_pool, const int32_t* src_blocks,
                      int32_t blocks_per_slot, const int32_t* dst_block, const int32_t* dst_slot, int32_t num_ops,
                      void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (is_quant(geom->kv_dtype)) return PKV_EUNSUPPORTED;
  if (num_ops < 0 || blocks_per_slot <= 0 || (long long)blocks_per_slot * geom->block_size > (1 << 24))
    return PKV_EINVAL;
  if (num_ops == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src_blocks || !dst_block || !dst_slot) return PKV_EINVAL;
  pkv::CompressArgs a{k_pool, v_pool, src_blocks, dst_block, dst_slot, num_ops, blocks_per_slot,
                      geom->num_blocks, geom->block_size, geom->num_kv_heads, geom->head_dim, geom->kv_dtype};
  return hip_status(pkv::launch_kv_compress(a, (hipStream_t)stream));
}

int paged_attn_decode_compressed(const pkv_geometry_t* geom, float* out, float* lse, const void* q,
                                 const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* full_start,
                                 const int32_t* slot_tables, int32_t max_slot_blocks, const int32_t* num_slots,
                                 int32_t num_seqs, int32_t max_context_len, int32_t window, float scale,
                                 int32_t num_workers, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_geometry(geom);
  if (st) return st;
  if (is_quant(geom->kv_dtype)) return PKV_EUNSUPPORTED;
  if (max_slot_blocks <= 0) return PKV_EINVAL;
  if (num_seqs > 0 && (!full_start || !slot_tables || !num_slots)) return PKV_EINVAL;
  SlotArgs slots;
  slots.full_start = full_start;
  slots.slot_tables = slot_tables;
  slots.num_slots = num_slots;
  slots.max_slot_blocks = max_slot_blocks;
  return decode_common(geom, out, lse, q, geom->kv_dtype, k_pool, v_pool, nullptr, nullptr, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, window, 0, scale, num_workers,
                       workspace, workspace_bytes, stream, slots);
}

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL: invalid argument";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED: unsupported head_dim, block_size, dtype or group size";
    case PKV_EWORKSPACE: return "PKV_EWORKSPACE: workspace missing or too small";
    case PKV_EHIP: return "PKV_EHIP: HIP launch failed";
    case PKV_ESCRATCH:
      return "PKV_ESCRATCH: the call needs more than the 32 MiB scratch of paged_attn_decode_noalloc "
             "(paged_attn_decode_workspace_bytes gives the need; fewer sequences or workers fit)";
  }
  return "unknown status";
}

int pkv_last_hip_error(void) { return g_last_hip_error; }

int pkv_version(void) { return 500; }

}  // extern "C"
