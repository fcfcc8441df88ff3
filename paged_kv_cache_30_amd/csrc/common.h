// Internal helpers shared by the gfx950 kernels: element traits for the
// storage types (fp32, fp16, bf16 and the 8-bit INT8 / FP8 E4M3 codes),
// 16-byte chunk dot products and conversions, and DPP lane reductions inside
// rows of 16 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage type tags. BYTES is the element size; one 16-byte chunk holds
// 16 / BYTES elements. QUANT: 8-bit codes with one fp32 scale per row.
struct F32T { static constexpr int BYTES = 4; static constexpr bool QUANT = false; static constexpr float BIAS = 0.f; };
struct F16T { static constexpr int BYTES = 2; static constexpr bool QUANT = false; static constexpr float BIAS = 0.f; };
struct BF16T { static constexpr int BYTES = 2; static constexpr bool QUANT = false; static constexpr float BIAS = 0.f; };
// INT8 codes (two's complement, -127..127) and OCP FP8 E4M3 codes. QMAX is
// the code magnitude a row's largest element maps to. The kernels widen INT8
// codes as unsigned bytes of (code ^ 0x80) = code + 128 and subtract BIAS =
// 128 once per sum; FP8 codes widen exactly (BIAS 0).
struct I8T {
  static constexpr int BYTES = 1;
  static constexpr bool QUANT = true;
  static constexpr float QMAX = 127.f;
  static constexpr float BIAS = 128.f;
};
struct FP8T {
  static constexpr int BYTES = 1;
  static constexpr bool QUANT = true;
  static constexpr float QMAX = 448.f;
  static constexpr float BIAS = 0.f;
};

// Reinterpret one 32-bit word. The word is taken by value: bit-casting an
// ext-vector element in place (q.y) reads the vector's first element.
__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ bf16x2 as_b2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// acc + sum_e q_e * k_e over one 16-byte chunk, fp32 accumulation. For the
// 16-bit types each pair is one v_dot2 (products of two 16-bit values are
// exact in fp32).
template <class T> __device__ __forceinline__ float dot_chunk(const u32x4& q, const u32x4& k, float acc);

template <> __device__ __forceinline__ float dot_chunk<F32T>(const u32x4& q, const u32x4& k, float acc) {
  acc = __builtin_fmaf(as_f(q.x), as_f(k.x), acc);
  acc = __builtin_fmaf(as_f(q.y), as_f(k.y), acc);
  acc = __builtin_fmaf(as_f(q.z), as_f(k.z), acc);
  acc = __builtin_fmaf(as_f(q.w), as_f(k.w), acc);
  return acc;
}

template <> __device__ __forceinline__ float dot_chunk<F16T>(const u32x4& q, const u32x4& k, float acc) {
  acc = __builtin_amdgcn_fdot2(as_h2(q.x), as_h2(k.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(q.y), as_h2(k.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(q.z), as_h2(k.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(q.w), as_h2(k.w), acc, false);
  return acc;
}

template <> __device__ __forceinline__ float dot_chunk<BF16T>(const u32x4& q, const u32x4& k, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(q.x), as_b2(k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(q.y), as_b2(k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(q.z), as_b2(k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(q.w), as_b2(k.w), acc, false);
  return acc;
}

// Widen one 16-byte chunk to fp32 (exact).
template <class T> __device__ __forceinline__ void chunk_to_f32(const u32x4& v, float* f);

template <> __device__ __forceinline__ void chunk_to_f32<F32T>(const u32x4& v, float* f) {
  f[0] = as_f(v.x); f[1] = as_f(v.y); f[2] = as_f(v.z); f[3] = as_f(v.w);
}

template <> __device__ __forceinline__ void chunk_to_f32<F16T>(const u32x4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h = as_h2(w[i]);
    f[2 * i] = (float)h.x;
    f[2 * i + 1] = (float)h.y;
  }
}

template <> __device__ __forceinline__ void chunk_to_f32<BF16T>(const u32x4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = as_f(w[i] << 16);
    f[2 * i + 1] = as_f(w[i] & 0xffff0000u);
  }
}

// Four 8-bit codes of one word as fp32 values code + BIAS (exact): INT8 as
// the unsigned byte code ^ 0x80 = code + 128, FP8 as the code's value.
template <class T> __device__ __forceinline__ void codes4_to_f32(uint32_t w, float* f);

template <> __device__ __forceinline__ void codes4_to_f32<I8T>(uint32_t w, float* f) {
  const uint32_t u = w ^ 0x80808080u;
  f[0] = (float)(u & 0xffu);
  f[1] = (float)((u >> 8) & 0xffu);
  f[2] = (float)((u >> 16) & 0xffu);
  f[3] = (float)(u >> 24);
}

template <> __device__ __forceinline__ void codes4_to_f32<FP8T>(uint32_t w, float* f) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo.x; f[1] = lo.y; f[2] = hi.x; f[3] = hi.y;
}

// DPP lane permutations (GFX9 encodings): quad_perm, half-row and row mirror.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;  // lane i <-> 15-i within 16

// Sum over aligned groups of N lanes (N in 4, 8, 16, 32); every lane of the
// group gets the total.
template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp<kHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// Maximum over aligned groups of N lanes (N in 4, 8, 16, 32).
template <int N> __device__ __forceinline__ float group_max(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16, 64));
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// An int32 array in the constant address space: uniform loads from it become
// scalar loads, which are counted apart from vector memory operations, so
// waiting for one never waits for the vector loads issued before it.
typedef const __attribute__((address_space(4))) int32_t* ctab_t;

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16-byte load of data read once (K/V pages in decode), with the streaming
// hint.
__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

}  // namespace pkv
