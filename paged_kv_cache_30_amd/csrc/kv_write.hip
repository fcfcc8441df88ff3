// Write of new tokens' keys/values into their pool slots (a copy for the
// 16-bit and fp32 pools, an encoding for the 8-bit ones).
//
// "Build a Paged KV Cache in Pure Python", Step 3 (append): the slot of
// position p of sequence s is block table[s][p / B], offset p % B; the whole
// [Hkv, D] row of keys and of values goes there. A pure copy, done in 16-byte
// pieces: each thread moves one piece of one token's K or V row, so a
// workgroup moves consecutive pieces of the same rows (coalesced on both
// sides).
#include "common.h"
#include "launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a, int chunks_per_row, long long total) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int n = (int)(i / (2 * chunks_per_row));
    const int rem = (int)(i - (long long)n * 2 * chunks_per_row);
    const int which = rem >= chunks_per_row;  // 0 = K, 1 = V
    const int ch = rem - which * chunks_per_row;
    // The piece itself is loaded first, alongside the sequence and position
    // (it depends on neither), so the table lookup is the only dependent
    // load before the store.
    const long long row_bytes = (long long)chunks_per_row * 16;
    const long long src = (long long)n * row_bytes + (long long)ch * 16;
    const u32x4 piece = load16((const char*)(which ? a.v_new : a.k_new) + src);
    const int s = a.seq_idx[n];
    const int p = a.pos[n];
    if (s < 0 || s >= a.num_seqs || p < 0 || p >= a.mb * a.B) continue;
    const int pb = a.tables[(long long)s * a.mb + p / a.B];
    if (pb < 0 || pb >= a.nb) continue;
    const long long dst = ((long long)pb * a.B + p % a.B) * row_bytes + (long long)ch * 16;
    *reinterpret_cast<u32x4*>((char*)(which ? a.v_pool : a.k_pool) + dst) = piece;
  }
}

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t st) {
  if (a.num_tokens == 0) return hipSuccess;
  const int chunks_per_row = a.Hkv * a.D * a.elem_bytes / 16;
  const long long total = (long long)a.num_tokens * 2 * chunks_per_row;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, chunks_per_row, total);
  return hipGetLastError();
}

// Quantising write (8-bit pools). One row = the D values of one (token, K or
// V, kv head); D/8 lanes hold 8 consecutive values each. The row's encoding
// is one fp32 scale and D codes:
//   amax = max |x|, scale = amax / QMAX, inv = QMAX / amax (0 if amax = 0),
//   code = nearest(x * inv): round half to even into -127..127 (INT8) or to
//   the nearest E4M3 value (FP8), in fp32 with correctly rounded division.
// The scale goes to [NB, Hkv, B] (a (block, kv head)'s B row scales are
// together); the codes to the [NB, B, Hkv, D] pool like 16-bit rows.
template <class In> __device__ __forceinline__ void load8_f32(const char* p, float* x);
template <> __device__ __forceinline__ void load8_f32<F32T>(const char* p, float* x) {
  chunk_to_f32<F32T>(load16(p), x);
  chunk_to_f32<F32T>(load16(p + 16), x + 4);
}
template <> __device__ __forceinline__ void load8_f32<F16T>(const char* p, float* x) {
  chunk_to_f32<F16T>(load16(p), x);
}
template <> __device__ __forceinline__ void load8_f32<BF16T>(const char* p, float* x) {
  chunk_to_f32<BF16T>(load16(p), x);
}

template <class T> __device__ __forceinline__ uint32_t encode4(const float* y);
template <> __device__ __forceinline__ uint32_t encode4<I8T>(const float* y) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (int)fminf(fmaxf(__builtin_rintf(y[i]), -127.f), 127.f);
    w |= ((uint32_t)c & 0xffu) << (8 * i);
  }
  return w;
}
template <> __device__ __forceinline__ uint32_t encode4<FP8T>(const float* y) {
  // Magnitudes within rounding of 448 are clamped to 448 first (their
  // nearest E4M3 value), so no input reaches the conversion's overflow.
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(y[i], -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return (uint32_t)w;
}

template <class T, class In, int D>
__global__ __launch_bounds__(256) void kv_write_quant_kernel(WriteQuantArgs a, long long total_rows) {
  constexpr int LPW = D / 8;  // lanes per row
  const long long stride = (long long)gridDim.x * (256 / LPW);
  const int c = threadIdx.x % LPW;
  for (long long row = (long long)blockIdx.x * (256 / LPW) + threadIdx.x / LPW; row < total_rows; row += stride) {
    const int n = (int)(row / (2 * a.Hkv));
    const int rem = (int)(row - (long long)n * 2 * a.Hkv);
    const int which = rem >= a.Hkv;  // 0 = K, 1 = V
    const int g = rem - which * a.Hkv;
    // The row's values are loaded first, alongside the sequence and
    // position (they depend on neither).
    float x[8];
    load8_f32<In>((const char*)(which ? a.v_new : a.k_new) + (((long long)n * a.Hkv + g) * D + c * 8) * In::BYTES,
                  x);
    const int s = a.seq_idx[n];
    const int p = a.pos[n];
    bool ok = s >= 0 && s < a.num_seqs && p >= 0 && p < a.mb * a.B;
    const int pb = ok ? a.tables[(long long)s * a.mb + p / a.B] : -1;
    ok = ok && pb >= 0 && pb < a.nb;
    // Every lane of the row takes part in the group maximum (the row's lanes
    // share `ok`); only valid rows store.
    if (!ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
    am = group_max<LPW>(am);
    if (!ok) continue;
    const float scale = __fdiv_rn(am, T::QMAX);
    const float inv = am > 0.f ? __fdiv_rn(T::QMAX, am) : 0.f;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = __fmul_rn(x[e], inv);
    const uint32_t w0 = encode4<T>(y), w1 = encode4<T>(y + 4);
    const int slot = p % a.B;
    char* pool = (char*)(which ? a.v_pool : a.k_pool);
    const long long dst = (((long long)pb * a.B + slot) * a.Hkv + g) * D + c * 8;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2_t*>(pool + dst) = u32x2_t{w0, w1};
    if (c == 0) (which ? a.v_scale : a.k_scale)[((long long)pb * a.Hkv + g) * a.B + slot] = scale;
  }
}

// Whole-block copies (copy-on-write of shared blocks): pair i copies block
// src[i] to block dst[i] in both pools, 16-byte pieces, and the B row scales
// of each kv head when scale pools are given. Pairs with an id outside
// [0, NB) or src == dst are skipped.
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(CopyBlocksArgs a, int pieces_per_block,
                                                             long long total) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int pair = (int)(i / (2 * pieces_per_block));
    const int rem = (int)(i - (long long)pair * 2 * pieces_per_block);
    const int which = rem >= pieces_per_block;  // 0 = K, 1 = V
    const int piece = rem - which * pieces_per_block;
    const int src = a.src[pair], dst = a.dst[pair];
    if (src < 0 || src >= a.nb || dst < 0 || dst >= a.nb || src == dst) continue;
    const long long bytes = (long long)pieces_per_block * 16;
    const char* from = (const char*)(which ? a.v_pool : a.k_pool) + (long long)src * bytes + (long long)piece * 16;
    char* to = (char*)(which ? a.v_pool : a.k_pool) + (long long)dst * bytes + (long long)piece * 16;
    *reinterpret_cast<u32x4*>(to) = load16(from);
    if (a.k_scale && piece < a.Hkv * a.B) {  // one fp32 scale per row: [NB, Hkv, B]
      float* sp = which ? a.v_scale : a.k_scale;
      sp[(long long)dst * a.Hkv * a.B + piece] = sp[(long long)src * a.Hkv * a.B + piece];
    }
  }
}

hipError_t launch_kv_copy_blocks(const CopyBlocksArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  const int pieces = a.B * a.Hkv * a.D * a.elem_bytes / 16;
  const long long total = (long long)a.n * 2 * pieces;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, pieces, total);
  return hipGetLastError();
}

bool kv_write_quant_supported(int kv_dtype, int in_dtype, int D) {
  return (kv_dtype == 3 || kv_dtype == 4) && (in_dtype == 0 || in_dtype == 1 || in_dtype == 2) &&
         (D == 64 || D == 128);
}

template <class T, class In, int D>
static hipError_t launch_wq(const WriteQuantArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);  // rows per workgroup
  const long long rows = (long long)a.num_tokens * 2 * a.Hkv;
  long long blocks = (rows + RPB - 1) / RPB;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((kv_write_quant_kernel<T, In, D>), dim3((unsigned)blocks), dim3(256), 0, st, a, rows);
  return hipGetLastError();
}

template <class T, class In>
static hipError_t wq_by_dim(const WriteQuantArgs& a, hipStream_t st) {
  return a.D == 64 ? launch_wq<T, In, 64>(a, st) : launch_wq<T, In, 128>(a, st);
}

template <class T>
static hipError_t wq_by_in(const WriteQuantArgs& a, hipStream_t st) {
  switch (a.in_dtype) {
    case 0: return wq_by_dim<T, F32T>(a, st);
    case 1: return wq_by_dim<T, F16T>(a, st);
    case 2: return wq_by_dim<T, BF16T>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_kv_write_quant(const WriteQuantArgs& a, hipStream_t st) {
  if (a.num_tokens == 0) return hipSuccess;
  if (!kv_write_quant_supported(a.kv_dtype, a.in_dtype, a.D)) return hipErrorInvalidValue;
  return a.kv_dtype == 3 ? wq_by_in<I8T>(a, st) : wq_by_in<FP8T>(a, st);
}

}  // namespace pkv
