// Widening of the 8-bit K/V blocks a prefill batch attends into 16-bit
// staging pools, for chunked prefill over 8-bit pages ("Build a
// Memory-Compressed Attention Engine with KV Caching from Scratch", section
// "Extending It: Your Roadmap to Senior-Level", item 2: INT8 or FP8 keys and
// values).
//
// Staged block s * msb + j holds logical block j of sequence s: its codes as
// values of the 16-bit type of q (exact: every INT8 code, -127..127, and
// every OCP E4M3 value is both a bf16 and an fp16 value) and its row scales.
// The prefill kernel then multiplies a key's score by its K scale and a
// weight by its key's V scale, so attention is over code * scale as for
// decode. The weight times the V scale is rounded to fp16 for the matrix
// cores; V scales are staged times a power of two v_mul (the output is
// divided by it) so that this product sits in fp16's normal range for the
// weights that matter, capped at 65504 / 256 so that it stays finite.
// Blocks past the context, and entries outside the pool, are not staged
// (table entry -1). A physical block that several sequences map at the same
// logical index (a shared prefix) is staged once: the entry of the first
// such sequence owns the copy, and the others point the staging table at
// it. (A block mapped at different logical indexes is staged once per
// index.)
#include "common.h"
#include "launch.h"

namespace pkv {

namespace {

template <class C> __device__ __forceinline__ void codes16_to_f32(const u32x4& w, float* f);
template <> __device__ __forceinline__ void codes16_to_f32<I8T>(const u32x4& w, float* f) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) f[4 * i + b] = (float)(int8_t)((x[i] >> (8 * b)) & 0xffu);
}
template <> __device__ __forceinline__ void codes16_to_f32<FP8T>(const u32x4& w, float* f) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) codes4_to_f32<FP8T>(x[i], f + 4 * i);  // FP8: BIAS 0, the code's value
}

// Eight exactly representable values as one 16-byte unit of the output type.
template <class O> __device__ __forceinline__ u32x4 pack8(const float* f);
template <> __device__ __forceinline__ u32x4 pack8<BF16T>(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (__float_as_uint(f[2 * i]) >> 16) | (__float_as_uint(f[2 * i + 1]) & 0xffff0000u);
  return u32x4{w[0], w[1], w[2], w[3]};
}
template <> __device__ __forceinline__ u32x4 pack8<F16T>(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * i]) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * i + 1]) << 16);
  return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace

// Largest staged V scale: weights are at most 256, and 256 times this is
// 65504, the largest finite fp16 value.
constexpr float kVScaleCap = 65504.f / 256.f;

// Physical block of entry (s, j) when the prefill reads it and it lies in
// the pool, else -1. The prefill reads, for a sequence with C >= min_rows
// query rows, the blocks below the (clamped) context length L; with a
// window only those holding a position at or after L - C - window + 1 (the
// first row's window) or below the sink count.
__device__ __forceinline__ int staged_source(const WidenArgs& a, int s, int j) {
  const int C = a.q_start[s + 1] - a.q_start[s];
  if (C < a.min_rows) return -1;
  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  const int nblk = (L + a.B - 1) / a.B;
  if (j >= nblk || j >= a.mb) return -1;
  if (a.window > 0) {
    const int lo = L - C - a.window + 1;
    if ((j + 1) * a.B <= lo && j * a.B >= a.sinks) return -1;
  }
  const int pb = a.tables[(size_t)s * a.mb + j];
  return (pb >= 0 && pb < a.nb) ? pb : -1;
}

// One workgroup per entry s * msb + j (logical block j of sequence s): it
// maps the entry to its block's copy and, if it owns the copy, widens
// 16-code pieces of the block into it.
template <class C, class O>
__global__ __launch_bounds__(256) void widen_kernel(WidenArgs a) {
  const int j = (int)(blockIdx.x % (unsigned)a.msb), s = (int)(blockIdx.x / (unsigned)a.msb);
  const int pb = staged_source(a, s, j);  // uniform over the workgroup
  __shared__ int first;  // the first sequence whose entry j stages the same block
  if (threadIdx.x == 0) first = s;
  __syncthreads();
  if (pb >= 0)
    for (int t = threadIdx.x; t < s; t += 256)
      if (staged_source(a, t, j) == pb) atomicMin(&first, t);
  __syncthreads();
  const int owner = first;
  const size_t stg = (size_t)s * a.msb + j;
  if (threadIdx.x == 0) a.stage_tables[stg] = pb >= 0 ? (int32_t)((size_t)owner * a.msb + j) : -1;
  if (pb < 0 || owner != s) return;  // the same for the whole workgroup
  const size_t blk_codes = (size_t)a.B * a.Hkv * a.D;  // bytes of codes per block
  const int pieces = (int)(blk_codes / 16);
  const char* kc = (const char*)a.k_codes + (size_t)pb * blk_codes;
  const char* vc = (const char*)a.v_codes + (size_t)pb * blk_codes;
  char* ko = (char*)a.k_out + stg * blk_codes * 2;
  char* vo = (char*)a.v_out + stg * blk_codes * 2;
  for (int p = threadIdx.x; p < pieces; p += 256) {
    const u32x4 kw = load16(kc + (size_t)p * 16);
    const u32x4 vw = load16(vc + (size_t)p * 16);
    float f[16];
    codes16_to_f32<C>(kw, f);
    *reinterpret_cast<u32x4*>(ko + (size_t)p * 32) = pack8<O>(f);
    *reinterpret_cast<u32x4*>(ko + (size_t)p * 32 + 16) = pack8<O>(f + 8);
    codes16_to_f32<C>(vw, f);
    *reinterpret_cast<u32x4*>(vo + (size_t)p * 32) = pack8<O>(f);
    *reinterpret_cast<u32x4*>(vo + (size_t)p * 32 + 16) = pack8<O>(f + 8);
  }
  const int nsc = a.Hkv * a.B;  // scales per block, [Hkv, B]
  for (int i = threadIdx.x; i < nsc; i += 256) {
    a.ks_out[stg * nsc + i] = a.k_scale[(size_t)pb * nsc + i];
    // A zero row (scale 0) adds nothing to the output whatever its scale:
    // staged as 1 so that the weight it carries stays in the normaliser.
    const float vsc = a.v_scale[(size_t)pb * nsc + i];
    a.vs_out[stg * nsc + i] = vsc > 0.f ? fminf(vsc * a.v_mul, kVScaleCap) : 1.f;
  }
}

hipError_t launch_widen(const WidenArgs& a, hipStream_t st) {
  if (a.S == 0 || a.msb == 0) return hipSuccess;
  if (((size_t)a.B * a.Hkv * a.D) % 16) return hipErrorInvalidValue;
  const long long entries = (long long)a.S * a.msb;
  const dim3 grid((unsigned)entries), block(256);
  if (a.code_dtype == 3 && a.out_dtype == 2) hipLaunchKernelGGL((widen_kernel<I8T, BF16T>), grid, block, 0, st, a);
  else if (a.code_dtype == 3 && a.out_dtype == 1) hipLaunchKernelGGL((widen_kernel<I8T, F16T>), grid, block, 0, st, a);
  else if (a.code_dtype == 4 && a.out_dtype == 2) hipLaunchKernelGGL((widen_kernel<FP8T, BF16T>), grid, block, 0, st, a);
  else if (a.code_dtype == 4 && a.out_dtype == 1) hipLaunchKernelGGL((widen_kernel<FP8T, F16T>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
