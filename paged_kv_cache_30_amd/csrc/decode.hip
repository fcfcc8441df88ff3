// Single-query decode through the block table, split evenly over wavefronts.
//
// What it computes ("Build a Paged KV Cache in Pure Python", Step 4; "Building
// a Streaming Sliding-Window Attention Engine in Pure Python", Step 3): for
// every sequence s and query head h, softmax(scale * q.K^T) V over positions
// [lo, L) of the sequence, fetched through its block table.
//
// How, on gfx950 (two launches on the caller's stream, three above 4096
// sequences):
//  1. plan: every wavefront (batches under 64 sequences, in a register) or
//     every workgroup (up to 4096, in LDS) prefix-sums the attended block
//     count of every sequence (cum[s]; a separate one-workgroup launch writes
//     it to the workspace instead for larger batches); the
//     attended (sequence, kv head, block) triples, flattened in that order,
//     number T = Hkv * cum[S].
//  2. split: wavefront w of NW takes the flattened range
//     [w*T/NW, (w+1)*T/NW) - every wavefront gets the same number of blocks
//     (+-1) however ragged the lengths are, so no wavefront is left running
//     alone at the end. The range falls into one or a few (sequence, kv head)
//     segments. For each, the wavefront streams the segment's K/V pages
//     (16-byte loads; the next chunk's loads are issued before the current
//     chunk is processed), computes the scores of every query head of the kv
//     head's group with each page (a page is read from HBM once per group),
//     keeps a running maximum and sum (online softmax in base 2), merges the
//     states of its row groups with lane shuffles and writes one partial
//     (max, sum, unnormalised output) per head, or, when it holds the whole
//     segment, the normalised output and log-sum-exp.
//  3. merge: per (sequence, query head) the partials of the wavefronts whose
//     ranges cover it are combined exactly:
//       M = max_i m_i,  out = sum_i 2^(m_i-M) o_i / sum_i 2^(m_i-M) l_i.
//  With 1-2 query heads per kv head, and for fp32 pools, step 2 runs on the
//  vector ALU (decode_split_kernel); with 4-8 heads on 16-bit and 8-bit
//  pools it runs on the matrix cores (decode_mma_kernel, below), with the
//  same split, partials and merge. In the vector-ALU kernel:
//  Lane layout: a K or V row (D elements of one position and kv head) is
//  D*bytes/16 lanes x 16 bytes; one wavefront load covers 64/(lanes per row)
//  consecutive slots of a block. Scores are a dot product on each lane's
//  slice (v_dot2 for 16-bit types) and a DPP reduction across the row.
//  Positions outside [lo, L) (the partial first block of a window, the
//  partial last block) are removed by selection, never by multiplying with
//  zero, so whatever unused slots hold cannot leak in.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pkv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPlanThreads = 1024;

// 8-bit K against 16-bit q: acc + sum_e q_e * (code_e + BIAS) over one
// 16-byte piece of 16 codes; q2 holds the 16 matching q values (two 16-byte
// words). Codes are widened to fp32, packed in pairs into q's 16-bit type
// (exact: 0..255 and every E4M3 value fit) and multiplied with v_dot2.
template <class Q> __device__ __forceinline__ uint32_t pack_pair(float a, float b);
template <> __device__ __forceinline__ uint32_t pack_pair<BF16T>(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack_pair<F16T>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
template <class Q> __device__ __forceinline__ float dot2(uint32_t q, uint32_t k, float acc);
template <> __device__ __forceinline__ float dot2<BF16T>(uint32_t q, uint32_t k, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_b2(q), as_b2(k), acc, false);
}
template <> __device__ __forceinline__ float dot2<F16T>(uint32_t q, uint32_t k, float acc) {
  return __builtin_amdgcn_fdot2(as_h2(q), as_h2(k), acc, false);
}
template <class T, class Q>
__device__ __forceinline__ float dot_codes(const u32x4* q2, const u32x4& k, float acc) {
  const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
  const uint32_t qw[8] = {q2[0].x, q2[0].y, q2[0].z, q2[0].w, q2[1].x, q2[1].y, q2[1].z, q2[1].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[4];
    codes4_to_f32<T>(kw[i], f);
    acc = dot2<Q>(qw[2 * i], pack_pair<Q>(f[0], f[1]), acc);
    acc = dot2<Q>(qw[2 * i + 1], pack_pair<Q>(f[2], f[3]), acc);
  }
  return acc;
}

template <class T, int D, int B, int G>
struct DecodeShape {
  static constexpr int EB = T::BYTES;
  static constexpr int E = 16 / EB;                    // elements per 16-byte piece
  // Pieces of a K/V row per lane: with 4 or more query heads per kv head
  // (fp32 pools; 16-bit and 8-bit ones take the matrix-core kernel there) the
  // per-position softmax work, done redundantly by every lane of a row, is
  // halved by giving each lane two pieces (fewer lanes per row).
  static constexpr int PIECES = (G >= 4 && D * EB / 16 >= 16) ? 2 : 1;
  static constexpr int LPR = D * EB / 16 / PIECES;     // lanes per K/V row
  static constexpr int RPL = 64 / LPR;                 // rows per step
  static constexpr int STEPS = B / RPL;                // steps per block
  // Loads per chunk (of K and of V); two chunks are in registers at a time
  // (16 KB in flight per wavefront).
  static constexpr int CWANT = 4 / PIECES;
  static constexpr int CSTEPS = STEPS < CWANT ? STEPS : CWANT;
  static constexpr int CHUNK = RPL * CSTEPS;           // slots per chunk
  static constexpr int CPB = B / CHUNK;                // chunks per block
  static_assert(LPR >= 4 && LPR <= 32 && B % CHUNK == 0, "shape");
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One v_mfma_f32_16x16x32 of the 16-bit type: lane l supplies A[l % 16][8 (l / 16) + e]
// and B[8 (l / 16) + e][l % 16] (e = 0..7) and receives C[4 (l / 16) + i][l % 16] (i = 0..3).
template <class T> __device__ __forceinline__ f32x4_t mma16(const u32x4& a, const u32x4& b, f32x4_t c);
template <> __device__ __forceinline__ f32x4_t mma16<BF16T>(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mma16<F16T>(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

// Attended blocks of sequence s, L clamped to [0, max_ctx]. The full-
// resolution positions are [lo, L): lo = max(0, L - window) with a window,
// raised to full_start[s] with compressed slots. The list of attended blocks
// starts with sb prefix entries read from ptab, then the blocks [wb0,
// ceil(L / B)) of the sequence's table, wb0 = lo / B. Prefix entry i holds
// rows [i*B, (i+1)*B) of which those below plim are attended:
//  - sinks: ptab is the sequence's own table and the prefix is the blocks
//    holding positions below min(sinks, lo) before the window's first block;
//  - compressed slots: ptab is the sequence's slot table and the prefix the
//    ceil(num_slots / B) blocks holding ring rows [0, num_slots).
// Entry i of the list is block(i) of its table.
struct Attended {
  int L, lo, sb, wb0, nblk, plim;
  const int32_t* ptab;
  __device__ __forceinline__ int block(int i) const { return i < sb ? i : wb0 + (i - sb); }
  __device__ __forceinline__ int32_t entry(const int32_t* trow, int i) const {
    return i < sb ? ptab[i] : trow[wb0 + (i - sb)];
  }
  // Keep the fields in scalar registers where the sequence is the same for
  // the whole wavefront.
  __device__ __forceinline__ void uniformize() {
    L = uniform(L);
    lo = uniform(lo);
    sb = uniform(sb);
    wb0 = uniform(wb0);
    nblk = uniform(nblk);
    plim = uniform(plim);
    const uint64_t p = (uint64_t)(uintptr_t)ptab;
    ptab = (const int32_t*)(uintptr_t)(((uint64_t)(uint32_t)uniform((int)(p >> 32)) << 32) |
                                       (uint32_t)uniform((int)(uint32_t)p));
  }
};
__device__ __forceinline__ Attended attended(const DecodeArgs& a, int s, int L, int B) {
  Attended r;
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  r.L = L;
  r.lo = a.window > 0 ? max(0, L - a.window) : 0;
  if (a.num_slots) {
    r.lo = max(r.lo, min(max(a.full_start[s], 0), L));
    r.wb0 = r.lo / B;
    r.plim = min(max(a.num_slots[s], 0), a.msb * B);
    r.sb = (r.plim + B - 1) / B;
    r.ptab = a.slot_tables + (size_t)s * a.msb;
  } else {
    r.wb0 = r.lo / B;
    r.plim = a.sinks;
    r.sb = (a.window > 0 && a.sinks > 0 && L > 0) ? min((min(a.sinks, r.lo) + B - 1) / B, r.wb0) : 0;
    r.ptab = a.tables + (size_t)s * a.mb;
  }
  r.nblk = (L > 0 ? (L + B - 1) / B - r.wb0 : 0) + r.sb;
  return r;
}

// Context length decode uses for sequence s: in a mixed batch (q_start set)
// only sequences with exactly one query row are decoded here; the others
// count as empty (the prefill kernel computes them). q/out/lse row of s.
__device__ __forceinline__ int decode_len(const DecodeArgs& a, int s) {
  if (a.q_start && a.q_start[s + 1] - a.q_start[s] != 1) return 0;
  return a.lens[s];
}
__device__ __forceinline__ int q_row(const DecodeArgs& a, int s) { return a.q_start ? a.q_start[s] : s; }

// cum[s] = attended blocks of sequences 0 .. s-1 for s <= S, computed by all
// NT threads of the workgroup (a block-wide scan, NT/64 wavefronts).
template <int NT>
__device__ void prefix_blocks(const DecodeArgs& a, int32_t* cum) {
  __shared__ int wave_sum[NT / 64];
  __shared__ int carry_sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) carry_sh = 0;
  __syncthreads();
  for (int base = 0; base < a.S; base += NT) {
    const int s = base + tid;
    int v = 0;
    if (s < a.S) v = attended(a, s, decode_len(a, s), a.B).nblk;
    int x = v;  // inclusive scan inside the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_sum[wv] = x;
    __syncthreads();
    int before = carry_sh;
    for (int i = 0; i < wv; ++i) before += wave_sum[i];
    if (s < a.S) cum[s] = before + x - v;
    __syncthreads();
    if (tid == NT - 1) carry_sh = before + x;
    __syncthreads();
  }
  if (tid == 0) cum[a.S] = carry_sh;
  __syncthreads();
}

// Batches of more than kLdsSeqs sequences get their prefix from a separate
// one-workgroup launch; smaller ones compute it in every workgroup (LDS).
constexpr int kLdsSeqs = 4096;

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a) {
  prefix_blocks<kPlanThreads>(a, a.ws_cum);
}

// T: storage type of the pools; Q: type of q (T itself, or fp16/bf16 for the
// 8-bit pools, whose rows also carry a scale each).
template <class T, class Q, int D, int B, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a, float scale_log2) {
  using Sh = DecodeShape<T, D, B, G>;
  constexpr int E = Sh::E, LPR = Sh::LPR, RPL = Sh::RPL, CSTEPS = Sh::CSTEPS, CHUNK = Sh::CHUNK,
                CPB = Sh::CPB, EB = Sh::EB, PC = Sh::PIECES;
  constexpr int PSTRIDE = LPR * 16;  // bytes between a lane's pieces of one row
  constexpr bool QU = T::QUANT;
  constexpr int QB = Q::BYTES;
  constexpr int QW = E * QB / 16;    // 16-byte words of q per piece
  constexpr float BIAS = T::BIAS;
  static_assert(QU || (QB == EB && QW == 1), "q has the pools' type unless the pools are 8-bit");

  const int lane = threadIdx.x & 63;
  // Prefix of attended blocks, in one of three places: batches of fewer than
  // 64 sequences keep it in a register of every wavefront (lane i holds
  // cum[i] and the length of sequence i; no LDS, no barrier), batches up to
  // kLdsSeqs in LDS, larger ones in the workspace (separate launch).
  __shared__ int32_t cum_sh[kLdsSeqs + 1];
  const bool in_reg = a.S < 64;
  const int32_t* cum_mem = a.ws_cum;
  int cum_reg = 0, len_reg = 0;
  if (in_reg) {
    int v = 0;
    if (lane < a.S) {
      len_reg = decode_len(a, lane);
      v = attended(a, lane, len_reg, B).nblk;
    }
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    cum_reg = x - v;  // exclusive: lane S holds the total
    if (blockIdx.x == 0 && threadIdx.x < 64 && lane <= a.S) a.ws_cum[lane] = cum_reg;  // for the merge pass
  } else if (a.S <= kLdsSeqs) {
    prefix_blocks<kThreads>(a, cum_sh);
    cum_mem = cum_sh;
    if (blockIdx.x == 0)  // the merge pass reads the prefix from the workspace
      for (int i = threadIdx.x; i <= a.S; i += kThreads) a.ws_cum[i] = cum_sh[i];
  }
  // cum[i] and lens[i] for a wavefront-uniform i.
  auto cum = [&](int i) -> int { return in_reg ? __builtin_amdgcn_readlane(cum_reg, i) : cum_mem[i]; };
  auto len_of = [&](int i) -> int { return in_reg ? __builtin_amdgcn_readlane(len_reg, i) : decode_len(a, i); };

  const int w = blockIdx.x * kWaves + uniform(threadIdx.x >> 6);  // worker index
  const int c = lane % LPR;
  const int r = lane / LPR;
  const int Hkv = a.Hkv, H = Hkv * G;
  const long long total = (long long)Hkv * cum(a.S);
  // Workers beyond the number of blocks stay idle, so every active worker
  // has at least one block.
  const long long nw = total < a.n_workers ? total : a.n_workers;
  if (w >= nw) return;
  const long long start = (long long)w * total / nw;
  const long long end = (long long)(w + 1) * total / nw;

  // Sequence holding flattened index `start`: the largest s with
  // Hkv*cum[s] <= start.
  int s;
  if (in_reg) {
    const unsigned long long msk = __ballot(lane < a.S && (long long)Hkv * cum_reg <= start);
    s = 63 - __builtin_clzll(msk);  // lane 0 always qualifies
  } else {  // 64 candidates at a time
    int s_lo = 0, s_hi = a.S;  // invariant: Hkv*cum[s_lo] <= start < Hkv*cum[s_hi]
    while (s_hi - s_lo > 1) {
      const int step = (s_hi - s_lo + 63) / 64;
      const int probe = s_lo + lane * step;
      const bool le = probe < s_hi && (long long)Hkv * cum_mem[probe] <= start;
      const unsigned long long msk = __ballot(le);
      const int k = 63 - __builtin_clzll(msk);  // lane 0 always qualifies
      s_lo = s_lo + k * step;
      s_hi = min(s_hi, s_lo + step);
    }
    s = s_lo;
  }

  const size_t row_stride = (size_t)Hkv * D * EB;  // bytes between slots
  const size_t blk_stride = row_stride * B;
  float m[G], l[G], o[G][PC * E];

  for (long long pos = start; pos < end;) {
    while ((long long)Hkv * cum(s + 1) <= pos) ++s;
    const int c0 = cum(s);
    const int nblk = cum(s + 1) - c0;
    const long long rel = pos - (long long)Hkv * c0;
    const int g = (int)(rel / nblk);
    const int b_first = (int)(rel - (long long)g * nblk);
    const long long seg_end = min(end, (long long)Hkv * c0 + (long long)(g + 1) * nblk);
    const int n = (int)(seg_end - pos);

    Attended at = attended(a, s, len_of(s), B);
    at.uniformize();
    const int L = at.L, lo = at.lo;
    const int32_t* trow = a.tables + (size_t)s * a.mb;
    // table entries of attended blocks b_first .. b_first + 63 of the segment
    int tv = lane < n ? at.entry(trow, b_first + lane) : -1;

    const char* qb = (const char*)a.q + ((size_t)(q_row(a, s) * H + g * G) * D + c * E) * QB;
    u32x4 qv[G][PC][QW];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int pc = 0; pc < PC; ++pc)
#pragma unroll
        for (int qw = 0; qw < QW; ++qw)
          qv[h][pc][qw] = load16(qb + (size_t)h * D * QB + (size_t)pc * LPR * E * QB + qw * 16);
    // INT8: the sum of this lane's q values, for the BIAS correction of its
    // partial dot products; lvb: the running sum of the V weights (same role).
    float qsum[G], lvb[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
      lvb[h] = 0.f;
#pragma unroll
      for (int e = 0; e < PC * E; ++e) o[h][e] = 0.f;
      qsum[h] = 0.f;
      if constexpr (BIAS != 0.f) {
#pragma unroll
        for (int pc = 0; pc < PC; ++pc)
#pragma unroll
          for (int qw = 0; qw < QW; ++qw) {
            float f[16 / QB];
            chunk_to_f32<Q>(qv[h][pc][qw], f);
#pragma unroll
            for (int e = 0; e < 16 / QB; ++e) qsum[h] += f[e];
          }
      }
    }
    const size_t lane_off = (size_t)g * D * EB + (size_t)c * 16 + (size_t)r * row_stride;
    const char* kbase = (const char*)a.k_pool + lane_off;
    const char* vbase = (const char*)a.v_pool + lane_off;

    // Loads of chunk k of the segment; false when its table entry is out of
    // range (the chunk is skipped).
    auto issue = [&](int k, u32x4 (*kr)[PC], u32x4 (*vr)[PC], float* ks, float* vs) -> bool {
      const int bi = k / CPB;
      const int sub = k - bi * CPB;
      if ((bi & 63) == 0 && bi > 0 && sub == 0) tv = bi + lane < n ? at.entry(trow, b_first + bi + lane) : -1;
      const int pb = __builtin_amdgcn_readlane(tv, bi & 63);
      if (pb < 0 || pb >= a.nb) return false;
      const size_t off = (size_t)pb * blk_stride + (size_t)sub * CHUNK * row_stride;
      if constexpr (QU) {  // this lane's row scales, [NB, Hkv, B]
        const size_t sidx = ((size_t)pb * Hkv + g) * B + sub * CHUNK + r;
#pragma unroll
        for (int j = 0; j < CSTEPS; ++j) {
          ks[j] = a.k_scale[sidx + j * RPL];
          vs[j] = a.v_scale[sidx + j * RPL];
        }
      }
#pragma unroll
      for (int j = 0; j < CSTEPS; ++j)
#pragma unroll
        for (int pc = 0; pc < PC; ++pc)
          kr[j][pc] = load_stream(kbase + off + (size_t)j * RPL * row_stride + pc * PSTRIDE);
#pragma unroll
      for (int j = 0; j < CSTEPS; ++j)
#pragma unroll
        for (int pc = 0; pc < PC; ++pc)
          vr[j][pc] = load_stream(vbase + off + (size_t)j * RPL * row_stride + pc * PSTRIDE);
      return true;
    };

    // Scores, online-softmax update and P.V for chunk k.
    auto process = [&](int k, const u32x4 (*kr)[PC], const u32x4 (*vr)[PC], const float* ks, const float* vs) {
      const int bi = k / CPB;
      const int sub = k - bi * CPB;
      const int t0 = at.block(b_first + bi) * B + sub * CHUNK;
      // attended: a prefix row below plim; otherwise t in [lo, L), or
      // t < sinks (below lo only with a window)
      const bool pre = b_first + bi < at.sb;
      const bool full = pre ? t0 + CHUNK <= at.plim : (t0 >= lo || t0 + CHUNK <= a.sinks) && t0 + CHUNK <= L;
      float sc[CSTEPS][G];
#pragma unroll
      for (int j = 0; j < CSTEPS; ++j) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = 0.f;
          if constexpr (QU) {
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) x = dot_codes<T, Q>(qv[h][pc], kr[j][pc], x);
            if constexpr (BIAS != 0.f) x = __builtin_fmaf(-BIAS, qsum[h], x);
            sc[j][h] = group_sum<LPR>(x) * (ks[j] * scale_log2);
          } else {
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) x = dot_chunk<T>(qv[h][pc][0], kr[j][pc], x);
            sc[j][h] = group_sum<LPR>(x) * scale_log2;
          }
        }
      }
      if (!full) {
#pragma unroll
        for (int j = 0; j < CSTEPS; ++j) {
          const int t = t0 + j * RPL + r;
          const bool ok = pre ? t < at.plim : (t >= lo || t < a.sinks) && t < L;
#pragma unroll
          for (int h = 0; h < G; ++h) sc[j][h] = ok ? sc[j][h] : -INFINITY;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mb = sc[0][h];
#pragma unroll
        for (int j = 1; j < CSTEPS; ++j) mb = fmaxf(mb, sc[j][h]);
        const float mn = fmaxf(m[h], mb);
        const float ms = mn == -INFINITY ? 0.f : mn;
        // Rescale only when some lane's maximum grew (otherwise the factor is 1).
        if (__any(mn > m[h])) {
          const float alpha = __builtin_amdgcn_exp2f(m[h] - ms);
          l[h] *= alpha;
          if constexpr (BIAS != 0.f) lvb[h] *= alpha;
#pragma unroll
          for (int e = 0; e < PC * E; ++e) o[h][e] *= alpha;
        }
        m[h] = mn;
#pragma unroll
        for (int j = 0; j < CSTEPS; ++j) {
          const float p = __builtin_amdgcn_exp2f(sc[j][h] - ms);
          sc[j][h] = p;
          l[h] += p;
        }
      }
#pragma unroll
      for (int j = 0; j < CSTEPS; ++j) {
        const int t = t0 + j * RPL + r;
        const bool ok = full || (pre ? t < at.plim : (t >= lo || t < a.sinks) && t < L);
        if constexpr (QU) {
          // Weight of the row times its V scale (0 for a masked row, whose
          // scale may be unset); codes widened to code + BIAS.
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float pw = sc[j][h] * vs[j];
            sc[j][h] = full ? pw : (ok ? pw : 0.f);
            if constexpr (BIAS != 0.f) lvb[h] += sc[j][h];
          }
#pragma unroll
          for (int pc = 0; pc < PC; ++pc) {
            const uint32_t vw[4] = {vr[j][pc].x, vr[j][pc].y, vr[j][pc].z, vr[j][pc].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float vf[4];
              codes4_to_f32<T>(vw[i], vf);
              if (!full) {
#pragma unroll
                for (int e = 0; e < 4; ++e) vf[e] = ok ? vf[e] : 0.f;
              }
#pragma unroll
              for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  o[h][pc * E + 4 * i + e] = __builtin_fmaf(sc[j][h], vf[e], o[h][pc * E + 4 * i + e]);
            }
          }
        } else {
#pragma unroll
          for (int pc = 0; pc < PC; ++pc) {
            float vf[E];
            chunk_to_f32<T>(vr[j][pc], vf);
            if (!full) {
#pragma unroll
              for (int e = 0; e < E; ++e) vf[e] = ok ? vf[e] : 0.f;
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
#pragma unroll
              for (int e = 0; e < E; ++e) o[h][pc * E + e] = __builtin_fmaf(sc[j][h], vf[e], o[h][pc * E + e]);
            }
          }
        }
      }
    };

    // Two register sets: the next chunk's loads are in flight while the
    // current chunk is processed.
    const int nchunks = n * CPB;
    u32x4 ka[CSTEPS][PC], va[CSTEPS][PC], kb[CSTEPS][PC], vb[CSTEPS][PC];
    float ksa[CSTEPS], vsa[CSTEPS], ksb[CSTEPS], vsb[CSTEPS];  // row scales (8-bit pools)
    bool oka = issue(0, ka, va, ksa, vsa);
    for (int k = 0; k < nchunks; k += 2) {
      const bool okb = k + 1 < nchunks && issue(k + 1, kb, vb, ksb, vsb);
      if (oka) process(k, ka, va, ksa, vsa);
      oka = k + 2 < nchunks && issue(k + 2, ka, va, ksa, vsa);
      if (okb) process(k + 1, kb, vb, ksb, vsb);
    }
    // INT8: the widened codes were code + BIAS; take BIAS times the weights
    // off once.
    if constexpr (BIAS != 0.f) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < PC * E; ++e) o[h][e] = __builtin_fmaf(-BIAS, lvb[h], o[h][e]);
    }

    // Merge the row groups' states (lanes r*LPR + c, same c) with shuffles.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mo = __shfl_xor(m[h], off, 64);
        const float lo_ = __shfl_xor(l[h], off, 64);
        const float M = fmaxf(m[h], mo);
        const float Ms = M == -INFINITY ? 0.f : M;
        const float fa = __builtin_amdgcn_exp2f(m[h] - Ms);
        const float fb = __builtin_amdgcn_exp2f(mo - Ms);
        l[h] = fa * l[h] + fb * lo_;
#pragma unroll
        for (int e = 0; e < PC * E; ++e) o[h][e] = fa * o[h][e] + fb * __shfl_xor(o[h][e], off, 64);
        m[h] = M;
      }
    }
    if (b_first == 0 && n == nblk) {
      // This wavefront holds the whole segment of (s, g): its state is final,
      // so it writes the normalised output and log-sum-exp itself (the same
      // arithmetic as the merge of a single partial) and the merge skips it.
      if (r == 0) {
        const size_t orow = (size_t)q_row(a, s) * H + (size_t)g * G;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float lh = l[h];
#pragma unroll
          for (int pc = 0; pc < PC; ++pc) {
            float* dst = a.out + (orow + h) * D + pc * LPR * E + c * E;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
              float4 v;
              v.x = lh > 0.f ? o[h][pc * E + e] / lh : 0.f;
              v.y = lh > 0.f ? o[h][pc * E + e + 1] / lh : 0.f;
              v.z = lh > 0.f ? o[h][pc * E + e + 2] / lh : 0.f;
              v.w = lh > 0.f ? o[h][pc * E + e + 3] / lh : 0.f;
              *reinterpret_cast<float4*>(dst + e) = v;
            }
          }
          if (a.lse && c == 0) a.lse[orow + h] = lh > 0.f ? (m[h] + __log2f(lh)) * kLn2 : -INFINITY;
        }
      }
    } else if (r == 0) {
      // One partial per head, slot w + s*Hkv + g (unique: see the merge).
      const size_t slot = (size_t)w + (size_t)s * Hkv + g;
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
          float* dst = a.ws_o + (slot * G + h) * D + pc * LPR * E + c * E;
#pragma unroll
          for (int e = 0; e < E; e += 4)
            *reinterpret_cast<float4*>(dst + e) =
                make_float4(o[h][pc * E + e], o[h][pc * E + e + 1], o[h][pc * E + e + 2], o[h][pc * E + e + 3]);
        }
        if (c == 0) *reinterpret_cast<float2*>(a.ws_ml + (slot * G + h) * 2) = make_float2(m[h], l[h]);
      }
    }
    pos = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Decode on the matrix cores, for groups of G >= 4 query heads per kv head.
//
// Same work split, partial format and merge as decode_split_kernel; inside a
// segment every 16-position chunk of the kv head's pages is two small dense
// products with the group's query heads as the 16 columns (zero beyond G):
//   S^T (16 positions x 16 heads) = K_chunk . Q^T        D/32 x v_mfma_f32_16x16x32
//   O^T (D x 16 heads)           += V_chunk^T . P^T      D/16 x 2 x v_mfma_f32_16x16x16
// Lane l works for head h = l % 16 and lane group g4 = l / 16: it receives
// the scores of positions 4 g4 + i (i = 0..3) of the chunk, supplies their
// weights as the B operand of the second product, and accumulates outputs
// of dims 16 dt + 4 g4 + i. The online softmax is thus per lane, apart from
// the chunk maximum (two lane swaps).
// K and V rows are loaded whole (16 lanes per 256-byte row, every cache
// line by one instruction, with the streaming hint: a decode step reads its
// pages once) and written to two per-wavefront LDS tiles. The K operand is
// read back as 16-byte units (lane l: position l % 16, dims 32 ks + 8 g4;
// q is read in the same dim order: a contraction may take its terms in any
// order as long as both operands agree), the V operand with the transposing
// read (lane l gets dim 16 dt + l % 16 of positions 4 g4 .. 4 g4 + 3).
// Each weight enters P.V as two 16-bit values hi + lo (two products), about
// 16 significant bits, while the normaliser sums the fp32 weights.
// 8-bit pools: codes widened in registers (exact) to q's type for K and to
// bf16 for V; the K row scale multiplies the score and the V row scale the
// weight. The reference maximum lags as in the prefill: it moves only when
// some head's chunk maximum exceeds it by more than 2^8.

// One v_mfma_f32_16x16x16 of the 16-bit type: lane l supplies A[l % 16][4 (l / 16) + e]
// and B[4 (l / 16) + e][l % 16] (e = 0..3) and receives C[4 (l / 16) + i][l % 16].
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
template <class T> __device__ __forceinline__ f32x4_t mma16k16(const u32x2_t& a, const u32x2_t& b, f32x4_t c);
template <> __device__ __forceinline__ f32x4_t mma16k16<BF16T>(const u32x2_t& a, const u32x2_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mma16k16<F16T>(const u32x2_t& a, const u32x2_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                               0, 0);
}
// The two values of a packed 16-bit pair, as fp32.
template <class P> __device__ __forceinline__ void unpack_pair(uint32_t h, float& a, float& b);
template <> __device__ __forceinline__ void unpack_pair<BF16T>(uint32_t h, float& a, float& b) {
  a = as_f(h << 16);
  b = as_f(h & 0xffff0000u);
}
template <> __device__ __forceinline__ void unpack_pair<F16T>(uint32_t h, float& a, float& b) {
  const f16x2 x = as_h2(h);
  a = (float)x.x;
  b = (float)x.y;
}
// a and b as hi + lo pairs of the 16-bit type (a - hi is exact in fp32).
template <class P> __device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_pair<P>(a, b);
  float ah, bh;
  unpack_pair<P>(hi, ah, bh);
  lo = pack_pair<P>(a - ah, b - bh);
}
// Eight 8-bit codes (two words) as eight values code + T::BIAS of the 16-bit
// type P (exact: INT8 as code + 128 in [0, 255], FP8 as its value). The
// caller takes BIAS times the other operand's sum off each product once.
template <class T, class P> __device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  float f[8];
  codes4_to_f32<T>(w0, f);
  codes4_to_f32<T>(w1, f + 4);
  u32x4 r;
  r.x = pack_pair<P>(f[0], f[1]);
  r.y = pack_pair<P>(f[2], f[3]);
  r.z = pack_pair<P>(f[4], f[5]);
  r.w = pack_pair<P>(f[6], f[7]);
  return r;
}
// Transposing 8-byte LDS read (ds_read_b64_tr_b16) at byte offset off of
// an LDS tile: within each 16 lanes, lane j reads 4 consecutive 16-bit
// values of row j / 4 and lane i receives value i of those 4 rows. The
// builtin, so that the compiler orders it after the tile's stores and waits
// for it itself.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ u32x2_t lds_read_tr16(lds_char* tile, uint32_t off) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off)));
}
// Maximum and sum over the four lanes l % 16 + 16 j (j = 0..3).
__device__ __forceinline__ float max_over_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Byte offset of logical 16-byte unit u of row r in a V tile of D 16-bit
// values per row: units XOR-swizzled by row so that the transposed reads of
// 16 rows x 32 bytes spread over all banks.
template <int D> __device__ __forceinline__ uint32_t vtile_off(int r, int u) {
  constexpr int RB = D * 2;
  const int sw = D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
  return (uint32_t)(r * RB + 16 * (u ^ sw));
}

// Source of the loads issued past the end of a segment (never used): one
// 16-byte line, so that those loads cost no page traffic.
__device__ __attribute__((aligned(16))) uint32_t g_pad16[4];

// Byte offset of logical 16-byte unit u of row r in a K tile: the A operand
// reads (16 rows x 4 consecutive units) spread over all banks.
template <int D> __device__ __forceinline__ uint32_t ktile_off(int r, int u) {
  const int sw = D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
  return (uint32_t)(r * D * 2 + 16 * (u ^ sw));
}

// Register budget: two wavefronts per SIMD for 16-bit pages, three for
// 8-bit pages (half the bytes per chunk; more workgroups per unit keep
// enough loads in flight).
template <class T, class Q, int D, int B, int G>
__global__ __launch_bounds__(kThreads, T::QUANT ? 3 : 2) void decode_mma_kernel(DecodeArgs a, float scale_log2) {
  constexpr bool QU = T::QUANT;
  constexpr bool BIASED = T::BIAS != 0.f;  // INT8: codes widened as code + 128
  constexpr int EB = T::BYTES;
  using P = typename std::conditional<QU, BF16T, T>::type;  // type of the P.V product
  constexpr int CH = 16;                 // positions per chunk
  constexpr int CPB = B / CH;            // chunks per block
  constexpr int KS = D / 32;             // k-steps of the score product
  constexpr int DT = D / 16;             // 16-dim tiles of the output
  constexpr int UV = D * EB / 16;        // 16-byte units of a V row in the pool
  constexpr int RV = 64 / UV;            // V rows per wavefront load
  constexpr int NVL = CH / RV;           // V loads per lane and chunk
  constexpr int NKL = NVL;               // K loads per lane and chunk (laid out as V's)
  static_assert(G >= 1 && G <= 16 && (D == 64 || D == 128) && B % CH == 0, "shape");

  __shared__ int32_t cum_sh[kLdsSeqs + 1];
  __shared__ __attribute__((aligned(16))) uint16_t vt_sh[kWaves][CH * D];
  __shared__ __attribute__((aligned(16))) uint16_t kt_sh[kWaves][CH * D];

  const int lane = threadIdx.x & 63;
  const int hh = lane & 15;   // head column
  const int g4 = lane >> 4;   // lane group
  const int wv = uniform(threadIdx.x >> 6);
  lds_char* const vt = (lds_char*)&vt_sh[wv][0];
  auto vt_store = [&](uint32_t off, const u32x4& x) { *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(vt + off) = x; };
  lds_char* const kt = (lds_char*)&kt_sh[wv][0];
  auto kt_store = [&](uint32_t off, const u32x4& x) { *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(kt + off) = x; };
  auto kt_load = [&](uint32_t off) -> u32x4 { return *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(kt + off); };

  // Prefix of attended blocks: in a register (batches under 64 sequences),
  // in LDS (up to kLdsSeqs), or in the workspace (plan launch).
  const bool in_reg = a.S < 64;
  const int32_t* cum_mem = a.ws_cum;
  int cum_reg = 0, len_reg = 0;
  if (in_reg) {
    int v = 0;
    if (lane < a.S) {
      len_reg = decode_len(a, lane);
      v = attended(a, lane, len_reg, B).nblk;
    }
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    cum_reg = x - v;
    if (blockIdx.x == 0 && threadIdx.x < 64 && lane <= a.S) a.ws_cum[lane] = cum_reg;
  } else if (a.S <= kLdsSeqs) {
    prefix_blocks<kThreads>(a, cum_sh);
    cum_mem = cum_sh;
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i <= a.S; i += kThreads) a.ws_cum[i] = cum_sh[i];
  }
  auto cum = [&](int i) -> int { return in_reg ? __builtin_amdgcn_readlane(cum_reg, i) : cum_mem[i]; };
  auto len_of = [&](int i) -> int { return in_reg ? __builtin_amdgcn_readlane(len_reg, i) : decode_len(a, i); };

  const int w = blockIdx.x * kWaves + wv;
  const int Hkv = a.Hkv, H = Hkv * G;
  const long long total = (long long)Hkv * cum(a.S);
  const long long nw = total < a.n_workers ? total : a.n_workers;
  if (w >= nw) return;
  const long long start = (long long)w * total / nw;
  const long long end = (long long)(w + 1) * total / nw;
  int s;
  if (in_reg) {
    const unsigned long long msk = __ballot(lane < a.S && (long long)Hkv * cum_reg <= start);
    s = 63 - __builtin_clzll(msk);
  } else {
    int s_lo = 0, s_hi = a.S;
    while (s_hi - s_lo > 1) {
      const int step = (s_hi - s_lo + 63) / 64;
      const int probe = s_lo + lane * step;
      const bool le = probe < s_hi && (long long)Hkv * cum_mem[probe] <= start;
      const unsigned long long msk = __ballot(le);
      const int k = 63 - __builtin_clzll(msk);
      s_lo = s_lo + k * step;
      s_hi = min(s_hi, s_lo + step);
    }
    s = s_lo;
  }

  const size_t row_stride = (size_t)Hkv * D * EB;
  const size_t blk_stride = row_stride * B;
  // V load j of this lane: row RV j + lane / UV of the chunk, unit lane % UV.
  const int v_row0 = lane / UV, v_unit = lane % UV;
  // K operand of k-step ks: lane (hh, g4) holds dims kdim(ks) .. + 8 of
  // position hh (read from the K tile; q is read in the same dim order).
  auto kdim = [&](int ks) -> int { return 32 * ks + 8 * g4; };

  for (long long pos = start; pos < end;) {
    while ((long long)Hkv * cum(s + 1) <= pos) ++s;
    s = uniform(s);
    const int c0 = uniform(cum(s));
    const int nblk = uniform(cum(s + 1)) - c0;
    const long long rel = pos - (long long)Hkv * c0;
    const int g = uniform((int)(rel / nblk));
    const int b_first = uniform((int)(rel - (long long)g * nblk));
    const long long seg_end = min(end, (long long)Hkv * c0 + (long long)(g + 1) * nblk);
    const int n = uniform((int)(seg_end - pos));

    Attended at = attended(a, s, len_of(s), B);
    at.uniformize();
    const int L = at.L, lo = at.lo;
    // Table entry of attended block i of the list (i uniform): a scalar load,
    // counted apart from the vector loads of the pages, so that waiting for
    // an entry never waits for pages in flight.
    const ctab_t ptab_c = (ctab_t)at.ptab;
    const ctab_t trow_c = (ctab_t)(a.tables + (size_t)s * a.mb);
    auto entry = [&](int i) -> int {
      i = uniform(i);
      return i < at.sb ? ptab_c[i] : trow_c[at.wb0 + (i - at.sb)];
    };

    // B operand of the score product: q of head g G + hh (zero beyond G),
    // dims kdim(ks) + e, the dims the K operand of k-step ks holds.
    u32x4 qm[KS];
    {
      const char* qa = (const char*)a.q + ((size_t)(q_row(a, s) * H + g * G + min(hh, G - 1)) * D) * Q::BYTES;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 v = load16(qa + (size_t)kdim(ks) * Q::BYTES);
        qm[ks] = hh < G ? v : u32x4{0, 0, 0, 0};
      }
    }
    // INT8 codes enter both products as code + 128: the score of head hh
    // takes 128 * sum(q) off (qbias), the output 128 * sum of the weights as
    // applied (wsum, a running sum like l_run).
    float qbias = 0.f, wsum = 0.f;
    if constexpr (BIASED) {
      float t = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float f[8];
        chunk_to_f32<Q>(qm[ks], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) t += f[e];
      }
      qbias = -T::BIAS * sum_over_groups(t);
    }
    float m_ref = -INFINITY, l_run = 0.f;
    f32x4_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const char* kbase =
        (const char*)a.k_pool + (size_t)g * D * EB + (size_t)v_row0 * row_stride + (size_t)v_unit * 16;
    const char* vbase =
        (const char*)a.v_pool + (size_t)g * D * EB + (size_t)v_row0 * row_stride + (size_t)v_unit * 16;

    // Loads of chunk k of the segment, issued for k = 0, 1, 2, ... in order
    // and without condition (past the end every lane loads the same 16-byte
    // pad; a block out of range loads block 0 and the chunk is masked), so
    // that every load is waited for only where its chunk is used. The next
    // chunk's table entry is requested one chunk ahead.
    const int nchunks = n * CPB;
    int pb_next = entry(b_first);
    auto issue = [&](int k, u32x4* kr, u32x4* vr, f32x4_t& ks4, f32x4_t& vs4) -> bool {
      const bool past = k >= nchunks;
      const char* pad = (const char*)g_pad16;
      k = min(k, nchunks - 1);
      const int bi = k / CPB;
      const int sub = k - bi * CPB;
      const int pb = pb_next;
      const int bn = min(k + 1, nchunks - 1) / CPB;
      pb_next = bn == bi ? pb : entry(b_first + bn);
      const bool valid = pb >= 0 && pb < a.nb;
      const size_t off = (size_t)(valid ? pb : 0) * blk_stride + (size_t)sub * CH * row_stride;
#pragma unroll
      for (int j = 0; j < NKL; ++j) kr[j] = load_stream(past ? pad : kbase + off + (size_t)j * RV * row_stride);
#pragma unroll
      for (int j = 0; j < NVL; ++j) vr[j] = load_stream(past ? pad : vbase + off + (size_t)j * RV * row_stride);
      if constexpr (QU) {  // row scales of positions 4 g4 .. 4 g4 + 3, [NB, Hkv, B]
        const size_t sidx = ((size_t)(valid ? pb : 0) * Hkv + g) * B + sub * CH + 4 * g4;
        const float* ksrc = past ? (const float*)g_pad16 : a.k_scale + sidx;
        const float* vsrc = past ? (const float*)g_pad16 : a.v_scale + sidx;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ks4[i] = ksrc[i];
          vs4[i] = vsrc[i];
        }
      }
      return valid;
    };

    auto process = [&](int k, bool valid, const u32x4* kr, const u32x4* vr, const f32x4_t& ks4,
                       const f32x4_t& vs4) {
      const int bi = k / CPB;
      const int sub = k - bi * CPB;
      const int t0 = at.block(b_first + bi) * B + sub * CH;
      const bool pre = b_first + bi < at.sb;
      const bool full =
          valid && (pre ? t0 + CH <= at.plim : (t0 >= lo || t0 + CH <= a.sinks) && t0 + CH <= L);
      auto attended_pos = [&](int t) {
        return valid && (pre ? t < at.plim : (t >= lo || t < a.sinks) && t < L);
      };
      // V rows into the LDS tile as 16-bit values (rows of positions not
      // attended as zeros: unused slots may hold anything).
#pragma unroll
      for (int j = 0; j < NVL; ++j) {
        const int r = RV * j + v_row0;
        const bool ok = full || attended_pos(t0 + r);
        if constexpr (QU) {
          u32x4 w0 = widen8<T, BF16T>(vr[j].x, vr[j].y), w1 = widen8<T, BF16T>(vr[j].z, vr[j].w);
          if (!ok) w0 = w1 = u32x4{0, 0, 0, 0};
          vt_store(vtile_off<D>(r, 2 * v_unit), w0);
          vt_store(vtile_off<D>(r, 2 * v_unit + 1), w1);
        } else {
          vt_store(vtile_off<D>(r, v_unit), ok ? vr[j] : u32x4{0, 0, 0, 0});
        }
      }
      // K rows into their tile, in q's type.
#pragma unroll
      for (int j = 0; j < NKL; ++j) {
        const int r = RV * j + v_row0;
        if constexpr (QU) {
          kt_store(ktile_off<D>(r, 2 * v_unit), widen8<T, Q>(kr[j].x, kr[j].y));
          kt_store(ktile_off<D>(r, 2 * v_unit + 1), widen8<T, Q>(kr[j].z, kr[j].w));
        } else {
          kt_store(ktile_off<D>(r, v_unit), kr[j]);
        }
      }
      // Scores of positions 4 g4 + i for head hh (base 2).
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ka = kt_load(ktile_off<D>(hh, 4 * ks + g4));
        sc = mma16<Q>(ka, qm[ks], sc);
      }
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = (BIASED ? sc[i] + qbias : sc[i]) * scale_log2;
        if constexpr (QU) x *= ks4[i];
        sv[i] = (full || attended_pos(t0 + 4 * g4 + i)) ? x : -INFINITY;
      }
      const float mx = max_over_groups(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      if (__any(mx > m_ref + 8.f)) {
        const float mn = fmaxf(m_ref, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - (mn == -INFINITY ? 0.f : mn));
        l_run *= alpha;
        if constexpr (BIASED) wsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        m_ref = mn;
      }
      const float ms = m_ref == -INFINITY ? 0.f : m_ref;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(sv[i] - ms);
        l_run += p[i];
        if constexpr (QU) p[i] = (full || sv[i] != -INFINITY) ? p[i] * vs4[i] : 0.f;
      }
      uint32_t h0, l0, h1, l1;
      split_pair<P>(p[0], p[1], h0, l0);
      split_pair<P>(p[2], p[3], h1, l1);
      const u32x2_t whi = {h0, h1}, wlo = {l0, l1};
      if constexpr (BIASED) {  // the weights exactly as the products apply them
        float a0, a1, b0, b1, c0, c1, d0, d1;
        unpack_pair<P>(h0, a0, a1);
        unpack_pair<P>(l0, b0, b1);
        unpack_pair<P>(h1, c0, c1);
        unpack_pair<P>(l1, d0, d1);
        wsum += ((a0 + b0) + (a1 + b1)) + ((c0 + d0) + (c1 + d1));
      }
      // V^T operands: row 4 g4 + hh / 4, dims 16 dt + 4 (hh % 4) .. + 4.
      u32x2_t va[DT];
      const int tr_r = 4 * g4 + (hh >> 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        va[dt] = lds_read_tr16(vt, vtile_off<D>(tr_r, 2 * dt + ((hh & 3) >> 1)) + 8 * (hh & 1));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt] = mma16k16<P>(va[dt], whi, o[dt]);
        o[dt] = mma16k16<P>(va[dt], wlo, o[dt]);
      }
    };

    // Two register sets: the next chunk's loads are in flight while the
    // current chunk is processed.
    u32x4 ka[NKL], va[NVL], kb[NKL], vb[NVL];
    f32x4_t ksa, vsa, ksb, vsb;
    bool oka = issue(0, ka, va, ksa, vsa);
    for (int k = 0; k < nchunks; k += 2) {
      const bool okb = issue(k + 1, kb, vb, ksb, vsb);
      process(k, oka, ka, va, ksa, vsa);
      oka = issue(k + 2, ka, va, ksa, vsa);
      if (k + 1 < nchunks) process(k + 1, okb, kb, vb, ksb, vsb);
    }

    const float l_tot = sum_over_groups(l_run);
    if constexpr (BIASED) {
      const float vbias = -T::BIAS * sum_over_groups(wsum);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] += vbias;
    }
    if (hh < G) {
      const size_t orow = (size_t)q_row(a, s) * H + (size_t)g * G + hh;
      if (b_first == 0 && n == nblk) {
        // The whole segment: normalised output and log-sum-exp.
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<float4*>(a.out + orow * D + 16 * dt + 4 * g4) =
              make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        if (a.lse && g4 == 0) a.lse[orow] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
      } else {
        const size_t slot = (size_t)w + (size_t)s * Hkv + g;
        float* dst = a.ws_o + (slot * G + hh) * D + 4 * g4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<float4*>(dst + 16 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
        if (g4 == 0) *reinterpret_cast<float2*>(a.ws_ml + (slot * G + hh) * 2) = make_float2(m_ref, l_tot);
      }
    }
    pos = seg_end;
  }
}

// Merge of the partials of one (sequence, kv head) by gridDim.z wavefronts,
// each holding every gridDim.z-th group of 64 of the G x D outputs of its
// query heads (one wavefront when there are many pairs, so that pairs with
// nothing to merge cost one short wavefront each). With NW = min(workers, T) active
// wavefronts, wavefront w holds [w*T/NW, (w+1)*T/NW) (never empty), so
// flattened index i lies in wavefront ((i + 1) * NW - 1) / T and the range
// [x, y) of (s, g) is covered by wavefronts w_lo .. w_hi, each of which wrote
// its partial of (s, g) in slot w + s*Hkv + g. Within a wavefront those slots
// are distinct, and a later wavefront's (s, g) is never earlier, so no two
// writers share a slot. When w_lo == w_hi that one wavefront wrote the
// output itself and there is nothing to merge.
template <int D, int G, int PER>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  // gridDim.z = G * D / (64 * PER) wavefronts per pair; lane t of wavefront
  // z holds outputs t + 64 * (z + gridDim.z * k), k < PER.
  const int g = blockIdx.x, s = blockIdx.y;
  const int Hkv = a.Hkv;
  if (a.q_start && a.q_start[s + 1] - a.q_start[s] != 1) return;  // a prefill chunk of a mixed batch
  const size_t row0 = (size_t)q_row(a, s) * a.H + (size_t)g * G;
  auto elem = [&](int k) { return 64 * (blockIdx.z + gridDim.z * k) + threadIdx.x; };
  const int c0 = a.ws_cum[s];
  const int nblk = a.ws_cum[s + 1] - c0;
  if (nblk == 0) {  // nothing attended: zeros and log-sum-exp -inf
#pragma unroll
    for (int k = 0; k < PER; ++k) a.out[row0 * D + elem(k)] = 0.f;
    if (a.lse && blockIdx.z == 0 && threadIdx.x < G) a.lse[row0 + threadIdx.x] = -INFINITY;
    return;
  }
  const long long total = (long long)Hkv * a.ws_cum[a.S];
  const long long NW = total < a.n_workers ? total : a.n_workers;
  const long long x = (long long)Hkv * c0 + (long long)g * nblk;
  const long long y = x + nblk;
  const int w_lo = (int)(((x + 1) * NW - 1) / total);
  const int w_hi = (int)((y * NW - 1) / total);
  if (w_lo == w_hi) return;  // written by the split kernel
  const int np = w_hi - w_lo + 1;
  const size_t base0 = ((size_t)s * Hkv + g) * G + (size_t)w_lo * G;  // slot of worker w_lo, head 0
  constexpr int NP = PER == 1 ? 32 : 4;  // partials the all-at-once path takes
  if (np <= NP) {
    // Every load of the lane's outputs issued before any is used.
    float2 ml[PER][NP];
    float ov[PER][NP];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = elem(k), hh = i / D, d = i - hh * D;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const size_t slot = base0 + hh + (size_t)j * G;
        const bool ok = j < np;
        ml[k][j] = ok ? *reinterpret_cast<const float2*>(a.ws_ml + slot * 2) : make_float2(-INFINITY, 0.f);
        ov[k][j] = ok ? a.ws_o[slot * D + d] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = elem(k), hh = i / D, d = i - hh * D;
      float M = ml[k][0].x;
#pragma unroll
      for (int j = 1; j < NP; ++j) M = fmaxf(M, ml[k][j].x);
      const float Ms = M == -INFINITY ? 0.f : M;
      float sl = 0.f, so = 0.f;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const float f = __builtin_amdgcn_exp2f(ml[k][j].x - Ms);
        sl = __builtin_fmaf(f, ml[k][j].y, sl);
        so = __builtin_fmaf(f, ov[k][j], so);
      }
      a.out[(row0 + hh) * D + d] = sl > 0.f ? so / sl : 0.f;
      if (a.lse && d == 0) a.lse[row0 + hh] = sl > 0.f ? (M + __log2f(sl)) * kLn2 : -INFINITY;
    }
    return;
  }
  // More partials: batches of U whose loads are issued together, merged in
  // one pass (the running maximum rescales what is summed so far).
  constexpr int U = 16;
  for (int k = 0; k < PER; ++k) {
    const int i = elem(k), hh = i / D, d = i - hh * D;
    const size_t base = base0 + hh;
    float M = -INFINITY, sl = 0.f, so = 0.f;
    for (int w0 = 0; w0 < np; w0 += U) {
      float2 ml[U];
      float ov[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const size_t slot = base + (size_t)(w0 + j) * G;
        const bool ok = w0 + j < np;
        ml[j] = ok ? *reinterpret_cast<const float2*>(a.ws_ml + slot * 2) : make_float2(-INFINITY, 0.f);
        ov[j] = ok ? a.ws_o[slot * D + d] : 0.f;
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < U; ++j) Mn = fmaxf(Mn, ml[j].x);
      const float Ms = Mn == -INFINITY ? 0.f : Mn;
      const float r = __builtin_amdgcn_exp2f(M - Ms);
      sl *= r;
      so *= r;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const float f = __builtin_amdgcn_exp2f(ml[j].x - Ms);
        sl = __builtin_fmaf(f, ml[j].y, sl);
        so = __builtin_fmaf(f, ov[j], so);
      }
      M = Mn;
    }
    a.out[(row0 + hh) * D + d] = sl > 0.f ? so / sl : 0.f;
    if (a.lse && d == 0) a.lse[row0 + hh] = sl > 0.f ? (M + __log2f(sl)) * kLn2 : -INFINITY;
  }
}

// Split kernel of an instance: the matrix-core one for 16-bit and 8-bit pools
// with 4 or more query heads per kv head, the vector-ALU one otherwise.
template <class T, int G>
constexpr bool use_mma() {
  return T::BYTES <= 2 && G >= 4;
}

template <class T, class Q, int D, int B, int G>
struct DecodeKernels {
  static constexpr auto split() {
    if constexpr (use_mma<T, G>())
      return decode_mma_kernel<T, Q, D, B, G>;
    else
      return decode_split_kernel<T, Q, D, B, G>;
  }
  static hipError_t launch(const DecodeArgs& a, hipStream_t st) {
    hipError_t e;
    if (a.S > kLdsSeqs) {
      hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int grid = (a.n_workers + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(split(), dim3(grid), dim3(kThreads), 0, st, a, a.scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Many (sequence, kv head) pairs: one wavefront each; few: one per 64
    // outputs, to spread the merge over more of the chip.
    constexpr int PAIR = G * D / 64;
    constexpr int PER = PAIR < 8 ? PAIR : 8;
    if (a.Hkv * a.S >= 2048)
      hipLaunchKernelGGL((decode_merge_kernel<D, G, PER>), dim3(a.Hkv, a.S, PAIR / PER), dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_merge_kernel<D, G, 1>), dim3(a.Hkv, a.S, PAIR), dim3(64), 0, st, a);
    return hipGetLastError();
  }
  // Workgroups of the split kernel resident per compute unit.
  static int blocks_per_cu() {
    static int cached = 0;
    if (!cached) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, split(), kThreads, 0) !=
              hipSuccess ||
          n <= 0) {
        (void)hipGetLastError();
        n = 2;
      }
      cached = n;
    }
    return cached;
  }
};

template <class T, class Q, int D, int B, int G>
struct LaunchOp {
  static hipError_t run(const DecodeArgs& a, hipStream_t st) { return DecodeKernels<T, Q, D, B, G>::launch(a, st); }
};
template <class T, class Q, int D, int B, int G>
struct OccupancyOp {
  static int run() { return DecodeKernels<T, Q, D, B, G>::blocks_per_cu(); }
};

// Kernel instance of a (pool dtype, q dtype) pair: 16-bit and fp32 pools take
// q of their own type; 8-bit pools (3 INT8, 4 FP8) take fp16 or bf16 q.
constexpr int kInstF32 = 0, kInstF16 = 1, kInstBF16 = 2, kInstI8F16 = 3, kInstI8BF16 = 4, kInstFP8F16 = 5,
              kInstFP8BF16 = 6;
static int instance_of(int dtype, int q_dtype) {
  if (dtype <= 2) return dtype;
  if (q_dtype != 1 && q_dtype != 2) return -1;
  if (dtype == 3) return q_dtype == 1 ? kInstI8F16 : kInstI8BF16;
  if (dtype == 4) return q_dtype == 1 ? kInstFP8F16 : kInstFP8BF16;
  return -1;
}

// Runtime (instance, head dim, block size, group size) -> template instance.
// 8-bit pools with 8 query heads per kv head run on the matrix-core kernel
// only.
template <template <class, class, int, int, int> class Op, class R, class... Args>
static R dispatch(int inst, int D, int B, int G, R bad, const Args&... args) {
#define PKV_G(T_, Q_, D_, B_)                               \
  switch (G) {                                              \
    case 1: return Op<T_, Q_, D_, B_, 1>::run(args...);     \
    case 2: return Op<T_, Q_, D_, B_, 2>::run(args...);     \
    case 4: return Op<T_, Q_, D_, B_, 4>::run(args...);     \
    case 8:                                                 \
      return Op<T_, Q_, D_, B_, 8>::run(args...);           \
  }                                                         \
  return bad;
#define PKV_B(T_, Q_, D_)                \
  switch (B) {                           \
    case 16: { PKV_G(T_, Q_, D_, 16) }   \
    case 32: { PKV_G(T_, Q_, D_, 32) }   \
  }                                      \
  return bad;
#define PKV_D(T_, Q_)                    \
  switch (D) {                           \
    case 64: { PKV_B(T_, Q_, 64) }       \
    case 128: { PKV_B(T_, Q_, 128) }     \
  }                                      \
  return bad;
  switch (inst) {
    case kInstF32: { PKV_D(F32T, F32T) }
    case kInstF16: { PKV_D(F16T, F16T) }
    case kInstBF16: { PKV_D(BF16T, BF16T) }
    case kInstI8F16: { PKV_D(I8T, F16T) }
    case kInstI8BF16: { PKV_D(I8T, BF16T) }
    case kInstFP8F16: { PKV_D(FP8T, F16T) }
    case kInstFP8BF16: { PKV_D(FP8T, BF16T) }
  }
  return bad;
#undef PKV_D
#undef PKV_B
#undef PKV_G
}

bool decode_supported(int dtype, int q_dtype, int D, int B, int G) {
  const int inst = instance_of(dtype, q_dtype);
  if (inst < 0 || (D != 64 && D != 128) || (B != 16 && B != 32)) return false;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  return true;
}

// Automatic worker count: whole workgroups per compute unit (an uneven
// spread leaves some units with more work); two per unit keep 128 KB of
// loads in flight per unit (16 KB per wavefront), which covers HBM latency,
// within what the unit holds at once. 8-bit pages carry half the bytes per
// chunk: three workgroups per unit (where they fit) measured best for them.
int decode_auto_workers(int dtype, int q_dtype, int D, int B, int G) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  const int resident = dispatch<OccupancyOp, int>(instance_of(dtype, q_dtype), D, B, G, 2);
  int per_cu = dtype == 3 || dtype == 4 ? 3 : 2;
  if (per_cu > resident) per_cu = resident;
  return cus * per_cu * kWaves;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  return dispatch<LaunchOp, hipError_t>(instance_of(a.dtype, a.q_dtype), a.D, a.B, a.H / a.Hkv,
                                        hipErrorInvalidValue, a, st);
}

}  // namespace pkv
