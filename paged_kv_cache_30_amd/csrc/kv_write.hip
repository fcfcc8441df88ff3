// Write of new tokens' keys/values into their pool slots.
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
    const int s = a.seq_idx[n];
    const int p = a.pos[n];
    if (s < 0 || s >= a.num_seqs || p < 0 || p >= a.mb * a.B) continue;
    const int pb = a.tables[(long long)s * a.mb + p / a.B];
    if (pb < 0 || pb >= a.nb) continue;
    const long long row_bytes = (long long)chunks_per_row * 16;
    const long long dst = ((long long)pb * a.B + p % a.B) * row_bytes + (long long)ch * 16;
    const long long src = (long long)n * row_bytes + (long long)ch * 16;
    const char* from = (const char*)(which ? a.v_new : a.k_new) + src;
    char* to = (char*)(which ? a.v_pool : a.k_pool) + dst;
    *reinterpret_cast<u32x4*>(to) = load16(from);
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

}  // namespace pkv
