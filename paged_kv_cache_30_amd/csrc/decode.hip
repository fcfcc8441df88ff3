// Single-query decode through the block table (split-K over blocks).
//
// What it computes ("Build a Paged KV Cache in Pure Python", Step 4; "Building
// a Streaming Sliding-Window Attention Engine in Pure Python", Step 3): for
// every sequence s and query head h, softmax(scale * q.K^T) V over positions
// [lo, L) of the sequence, fetched through its block table.
//
// How, on gfx950:
//  * Work item = (sequence, kv head, partition of consecutive blocks). One
//    256-thread workgroup (4 wavefronts) per item; wavefront w takes blocks
//    w, w+4, ... of the partition. Every query head of the kv head's group is
//    processed with each loaded page, so a K/V page is read from HBM once per
//    group.
//  * Lane layout: a K or V row (D elements of one position and kv head) is
//    D*bytes/16 lanes x 16 bytes. A wavefront load covers 64/(lanes per row)
//    consecutive slots of a block; the lanes of one row hold a slice of the
//    head dimension. Scores are a dot product on each lane's slice followed by
//    a DPP reduction across the row's lanes.
//  * Each row group of lanes keeps its own running maximum and sum (online
//    softmax in base 2: scores are scaled by scale*log2(e)), so nothing is
//    exchanged between row groups inside the block loop. At the end the
//    wavefronts' and row groups' states are merged through LDS.
//  * One partition per (sequence, kv head) writes the output directly;
//    otherwise each partition writes its unnormalised partial output with its
//    maximum and sum, and a second kernel merges the partitions:
//      M = max_i m_i,  out = sum_i 2^(m_i-M) o_i / sum_i 2^(m_i-M) l_i.
//  * Positions outside [lo, L) (the partial first block of a window, the
//    partial last block) are removed by selection, never by multiplying with
//    zero, so whatever the unused slots hold cannot leak in.
#include "common.h"
#include "launch.h"

namespace pkv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <class T, int D, int B, int G>
struct DecodeShape {
  static constexpr int EB = T::BYTES;
  static constexpr int E = 16 / EB;            // elements per lane chunk
  static constexpr int LPR = D * EB / 16;      // lanes per K/V row
  static constexpr int RPL = 64 / LPR;         // rows per wavefront load
  static constexpr int STEPS = B / RPL;        // wavefront loads per block
  static constexpr int STATES = kWaves * RPL;  // softmax states per workgroup
  static_assert(LPR >= 4 && LPR <= 32 && B % RPL == 0, "shape");
};

template <class T, int D, int B, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeArgs a, int max_ctx, float scale_log2) {
  using Sh = DecodeShape<T, D, B, G>;
  constexpr int E = Sh::E, LPR = Sh::LPR, RPL = Sh::RPL, STEPS = Sh::STEPS, EB = Sh::EB;
  __shared__ float sh_o[Sh::STATES][G][D];
  __shared__ float sh_m[Sh::STATES][G];
  __shared__ float sh_l[Sh::STATES][G];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int c = lane % LPR;
  const int r = lane / LPR;
  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int H = a.Hkv * G;

  int L = a.lens[s];
  L = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int blk_lo = lo / B;
  const int blk_hi = (L + B - 1) / B;
  const int b0 = blk_lo + part * a.blocks_per_part;
  const int b1 = min(b0 + a.blocks_per_part, blk_hi);
  const bool direct = a.n_part == 1;
  if (!direct && b0 >= b1) return;  // the merge pass knows this partition is empty

  // Query rows of the group, this lane's slice.
  const char* qb = (const char*)a.q + ((size_t)(s * H + g * G) * D + c * E) * EB;
  u32x4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h] = load16(qb + (size_t)h * D * EB);

  float m[G], l[G], o[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = 0.f;
  }

  const size_t row_stride = (size_t)a.Hkv * D * EB;  // bytes between slots
  const size_t blk_stride = row_stride * B;
  const size_t lane_off = (size_t)g * D * EB + (size_t)c * 16 + (size_t)r * row_stride;
  const char* kbase = (const char*)a.k_pool + lane_off;
  const char* vbase = (const char*)a.v_pool + lane_off;
  const int32_t* trow = a.tables + (size_t)s * a.mb;

  for (int b = b0 + wave; b < b1; b += kWaves) {
    const int pb = trow[b];
    if (pb < 0 || pb >= a.nb) continue;
    const char* kp = kbase + (size_t)pb * blk_stride;
    const char* vp = vbase + (size_t)pb * blk_stride;
    u32x4 kr[STEPS], vr[STEPS];
#pragma unroll
    for (int j = 0; j < STEPS; ++j) kr[j] = load16(kp + (size_t)j * RPL * row_stride);
#pragma unroll
    for (int j = 0; j < STEPS; ++j) vr[j] = load16(vp + (size_t)j * RPL * row_stride);

    const int t0 = b * B;
    const bool full = t0 >= lo && t0 + B <= L;
    float sc[STEPS][G];
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[j][h] = group_sum<LPR>(dot_chunk<T>(qv[h], kr[j], 0.f)) * scale_log2;
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        const int t = t0 + j * RPL + r;
        const bool ok = t >= lo && t < L;
#pragma unroll
        for (int h = 0; h < G; ++h) sc[j][h] = ok ? sc[j][h] : -INFINITY;
      }
    }
    // Online softmax update, one state per (row group, head).
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mb = sc[0][h];
#pragma unroll
      for (int j = 1; j < STEPS; ++j) mb = fmaxf(mb, sc[j][h]);
      const float mn = fmaxf(m[h], mb);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[h] - ms);
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) o[h][e] *= alpha;
      m[h] = mn;
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[j][h] - ms);
        sc[j][h] = p;
        l[h] += p;
      }
    }
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      float vf[E];
      chunk_to_f32<T>(vr[j], vf);
      if (!full) {
        const int t = t0 + j * RPL + r;
        const bool ok = t >= lo && t < L;
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = ok ? vf[e] : 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = __builtin_fmaf(sc[j][h], vf[e], o[h][e]);
      }
    }
  }

  // Merge the STATES = waves x row-groups states of this workgroup.
  const int st = wave * RPL + r;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < E; ++e) sh_o[st][h][c * E + e] = o[h][e];
    if (c == 0) {
      sh_m[st][h] = m[h];
      sh_l[st][h] = l[h];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < Sh::STATES; ++i) M = fmaxf(M, sh_m[i][h]);
    const float Ms = M == -INFINITY ? 0.f : M;
    float sl = 0.f, so = 0.f;
#pragma unroll
    for (int i = 0; i < Sh::STATES; ++i) {
      const float w = __builtin_amdgcn_exp2f(sh_m[i][h] - Ms);
      sl = __builtin_fmaf(w, sh_l[i][h], sl);
      so = __builtin_fmaf(w, sh_o[i][h][d], so);
    }
    const size_t row = (size_t)s * H + g * G + h;
    if (direct) {
      a.out[row * D + d] = sl > 0.f ? so / sl : 0.f;
      if (a.lse && d == 0) a.lse[row] = sl > 0.f ? (M + __log2f(sl)) * kLn2 : -INFINITY;
    } else {
      const size_t slot = row * a.n_part + part;
      a.ws_o[slot * D + d] = so;
      if (d == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = sl;
      }
    }
  }
}

// Merge of the partitions of one (sequence, query head): one thread per
// output element of the head.
template <int D, int B>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a, int max_ctx) {
  const int hq = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  int L = a.lens[s];
  L = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int nblk = (L + B - 1) / B - lo / B;
  const int nvalid = nblk > 0 ? (nblk + a.blocks_per_part - 1) / a.blocks_per_part : 0;
  const size_t row = (size_t)s * a.H + hq;
  const float* ml = a.ws_ml + row * a.n_part * 2;
  const float* po = a.ws_o + row * a.n_part * D;
  float M = -INFINITY;
  for (int i = 0; i < nvalid; ++i) M = fmaxf(M, ml[2 * i]);
  const float Ms = M == -INFINITY ? 0.f : M;
  float sl = 0.f, so = 0.f;
  for (int i = 0; i < nvalid; ++i) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * i] - Ms);
    sl = __builtin_fmaf(w, ml[2 * i + 1], sl);
    so = __builtin_fmaf(w, po[(size_t)i * D + d], so);
  }
  a.out[row * D + d] = sl > 0.f ? so / sl : 0.f;
  if (a.lse && d == 0) a.lse[row] = sl > 0.f ? (M + __log2f(sl)) * kLn2 : -INFINITY;
}

template <class T, int D, int B, int G>
static hipError_t launch_typed(const DecodeArgs& a, int max_ctx, hipStream_t st) {
  const float scale_log2 = a.scale * kLog2e;
  dim3 grid(a.n_part, a.Hkv, a.S);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, B, G>), grid, dim3(kThreads), 0, st, a, max_ctx, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_part == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, B>), dim3(a.H, a.S), dim3(D), 0, st, a, max_ctx);
  return hipGetLastError();
}

template <class T, int D, int B>
static hipError_t by_group(const DecodeArgs& a, int max_ctx, hipStream_t st) {
  switch (a.H / a.Hkv) {
    case 1: return launch_typed<T, D, B, 1>(a, max_ctx, st);
    case 2: return launch_typed<T, D, B, 2>(a, max_ctx, st);
    case 4: return launch_typed<T, D, B, 4>(a, max_ctx, st);
    case 8: return launch_typed<T, D, B, 8>(a, max_ctx, st);
  }
  return hipErrorInvalidValue;
}

template <class T, int D>
static hipError_t by_block(const DecodeArgs& a, int max_ctx, hipStream_t st) {
  switch (a.B) {
    case 16: return by_group<T, D, 16>(a, max_ctx, st);
    case 32: return by_group<T, D, 32>(a, max_ctx, st);
  }
  return hipErrorInvalidValue;
}

template <class T>
static hipError_t by_dim(const DecodeArgs& a, int max_ctx, hipStream_t st) {
  switch (a.D) {
    case 64: return by_block<T, 64>(a, max_ctx, st);
    case 128: return by_block<T, 128>(a, max_ctx, st);
  }
  return hipErrorInvalidValue;
}

bool decode_supported(int dtype, int D, int B, int G) {
  return (dtype == 0 || dtype == 1 || dtype == 2) && (D == 64 || D == 128) && (B == 16 || B == 32) &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

// Launch. Device-side lengths are clamped to [0, max_context_len], which
// the host has checked against the table width, so no read leaves the
// sequence's table row or the partition workspace.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const int max_ctx = a.max_context_len;
  switch (a.dtype) {
    case 0: return by_dim<F32T>(a, max_ctx, st);
    case 1: return by_dim<F16T>(a, max_ctx, st);
    case 2: return by_dim<BF16T>(a, max_ctx, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
