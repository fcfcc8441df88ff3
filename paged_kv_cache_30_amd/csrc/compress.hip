// Compression of evicted blocks into slots: the mean of every row of a group
// of blocks, per kv head and element, written as one row of a slot block.
//
// "Build a Memory-Compressed Attention Engine with KV Caching from Scratch",
// Step 2 (mean pooling: a group of positions is summarised by the mean of
// its keys and the mean of its values, per head) and Step 3 (the oldest half
// of a full window is compressed into one slot). Here a group is whole
// blocks of the pool, the slot a row of another block, so the slots are read
// back by decode through a table like any other row.
//
// Sums are fp64: the sum of up to 2^24 rows of 16-bit or fp32 values is exact
// unless their magnitudes span more than about 53 - 24 - log2(rows) binades,
// so the mean is that of exact arithmetic, rounded once.
#include "common.h"
#include "launch.h"

namespace pkv {

namespace {

// Round-to-odd double -> float: the float nearest toward zero, with its last
// bit set when the conversion was inexact (Boldo and Melquiond, "Emulation
// of FMA and correctly-rounded sums: proved algorithms using rounding to
// odd", IEEE Trans. Computers 57(4), 2008). Rounding this float to nearest
// in a format of at most 22 significant bits gives the same result as
// rounding x directly, with no double-rounding error.
__device__ __forceinline__ float to_float_odd(double x) {
  const float f = (float)x;  // nearest
  const double back = (double)f;
  if (back == x || x != x) return f;
  uint32_t u = __float_as_uint(f);
  if (fabs(back) > fabs(x)) u -= 1;  // one step toward zero: the truncated value
  return __uint_as_float(u | 1u);
}

__device__ __forceinline__ uint32_t bf16_bits(double x) {  // nearest, ties to even
  const uint32_t u = __float_as_uint(to_float_odd(x));
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t f16_bits(double x) {  // nearest, ties to even
  const _Float16 h = (_Float16)to_float_odd(x);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

}  // namespace

// A workgroup owns kPieces 16-byte pieces of the row of one op; its 256
// threads are kRowLanes lanes per piece, lane l summing rows l, l + kRowLanes,
// ... of the group (all its loads independent), and the lanes' fp64 partials
// are added in LDS. Any summation order gives the same, exact sum under the
// condition above, so the split does not change the result.
constexpr int kPieces = 16;
constexpr int kRowLanes = 256 / kPieces;

template <class T> __device__ __forceinline__ void store_elem(char* p, double m);
template <> __device__ __forceinline__ void store_elem<F32T>(char* p, double m) {
  *reinterpret_cast<float*>(p) = (float)m;
}
template <> __device__ __forceinline__ void store_elem<BF16T>(char* p, double m) {
  *reinterpret_cast<uint16_t*>(p) = (uint16_t)bf16_bits(m);
}
template <> __device__ __forceinline__ void store_elem<F16T>(char* p, double m) {
  *reinterpret_cast<uint16_t*>(p) = (uint16_t)f16_bits(m);
}

template <class T>
__global__ __launch_bounds__(256) void kv_compress_kernel(CompressArgs a, int pieces, int tiles) {
  constexpr int E = 16 / T::BYTES;  // elements per 16-byte piece
  __shared__ double part[2][kRowLanes][kPieces][E];
  const int op = blockIdx.x / tiles;
  const int p0 = (blockIdx.x - op * tiles) * kPieces;
  const int lp = threadIdx.x % kPieces, rl = threadIdx.x / kPieces;
  const int db = a.dst_block[op], ds = a.dst_slot[op];
  if (db < 0 || db >= a.nb || ds < 0 || ds >= a.B) return;  // the same for the whole workgroup
  const int32_t* src = a.src + (size_t)op * a.bps;
  int count = 0;
  for (int j = 0; j < a.bps; ++j) count += (src[j] >= 0 && src[j] < a.nb) ? a.B : 0;
  if (count == 0) return;  // the same for the whole workgroup

  const size_t row_bytes = (size_t)pieces * 16;
  const size_t blk_bytes = row_bytes * a.B;
  const int piece = p0 + lp;
  double sk[E], sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sk[e] = sv[e] = 0.0;
  if (piece < pieces) {
    // Eight rows per lane at a time: their block ids, then all their loads,
    // are issued before any is used. Rows past the group or in a block
    // outside the pool read row 0 of block 0 and add nothing.
    constexpr int U = 8;
    const int rows = a.bps * a.B;
    for (int f0 = rl; f0 < rows; f0 += U * kRowLanes) {
      int sb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = f0 + u * kRowLanes;
        sb[u] = f < rows ? src[f / a.B] : -1;
      }
      u32x4 kx[U], vx[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = f0 + u * kRowLanes;
        ok[u] = sb[u] >= 0 && sb[u] < a.nb;
        const size_t off = ok[u] ? (size_t)sb[u] * blk_bytes + (size_t)(f % a.B) * row_bytes : 0;
        kx[u] = load16((const char*)a.k_pool + off + (size_t)piece * 16);
        vx[u] = load16((const char*)a.v_pool + off + (size_t)piece * 16);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float fk[E], fv[E];
        chunk_to_f32<T>(kx[u], fk);
        chunk_to_f32<T>(vx[u], fv);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          sk[e] += ok[u] ? (double)fk[e] : 0.0;
          sv[e] += ok[u] ? (double)fv[e] : 0.0;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    part[0][rl][lp][e] = sk[e];
    part[1][rl][lp][e] = sv[e];
  }
  __syncthreads();
  // One output element per thread: pool, piece, element.
  const int t = threadIdx.x;
  if (t >= 2 * kPieces * E) return;
  const int pool = t / (kPieces * E), rem = t - pool * kPieces * E;
  const int q = rem / E, e = rem - q * E;
  if (p0 + q >= pieces) return;
  double sum = 0.0;
#pragma unroll
  for (int l = 0; l < kRowLanes; ++l) sum += part[pool][l][q][e];
  char* base = (char*)(pool ? a.v_pool : a.k_pool);
  store_elem<T>(base + (size_t)db * blk_bytes + (size_t)ds * row_bytes + (size_t)(p0 + q) * 16 + e * T::BYTES,
                sum / (double)count);
}

hipError_t launch_kv_compress(const CompressArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  const int eb = a.dtype == 0 ? 4 : 2;
  const int pieces = a.Hkv * a.D * eb / 16;
  const int tiles = (pieces + kPieces - 1) / kPieces;
  const long long blocks = (long long)a.n * tiles;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  switch (a.dtype) {
    case 0: hipLaunchKernelGGL(kv_compress_kernel<F32T>, grid, block, 0, st, a, pieces, tiles); break;
    case 1: hipLaunchKernelGGL(kv_compress_kernel<F16T>, grid, block, 0, st, a, pieces, tiles); break;
    case 2: hipLaunchKernelGGL(kv_compress_kernel<BF16T>, grid, block, 0, st, a, pieces, tiles); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
