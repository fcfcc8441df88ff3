// Causal chunked prefill through the block table on the matrix cores.
//
// What it computes ("Building a Streaming Sliding-Window Attention Engine in
// Pure Python", Step 3 and Step 4, read for a chunk that follows a cached
// prefix): query row i of sequence s sits at position p = L - C + i and
// attends every cached position t <= p (with a window: t > p - w, or
// t < sinks for the attention sinks of the same page's Step 4 and roadmap).
//
// How, on gfx950 (v_mfma_f32_32x32x16 on 16-bit inputs, fp32 accumulate):
//  * Each wavefront owns 32 query rows of one query head; the wavefronts of
//    a workgroup share one kv head, so each K/V tile of 64 key positions is
//    gathered once into LDS (direct global->LDS loads through the block
//    table) for every query head of the group the workgroup covers.
//  * Per tile and wavefront
//      S^T (64 keys x 32 queries) = K_tile . Q^T        (16 MFMAs, D = 128)
//    so each lane holds the scores of one query; the running maximum is
//    exchanged between the two lane halves that hold the same query; then
//      O^T (D x 32 queries) += V_tile^T . P^T           (16 MFMAs)
//    keeps one query's output per lane, so the rescale never leaves the lane.
//    The V^T operand is read from row-major V with the LDS transpose read
//    (ds_read_b64_tr_b16): within 16 lanes, lane j reads 4 consecutive dims
//    of key j/4 and lane i receives dim i of those 4 keys.
//  * P.V runs on the fp16 matrix cores for both input types, with the
//    weights rounded to fp16 (11-bit mantissa) and the normaliser summing
//    the weights as used; lse takes the same sum, which is within 2^-11
//    relative of the sum of the unrounded weights (plus at most 2^-25 per
//    subnormal weight, against a sum of at least 1). A bf16 V tile is
//    converted to fp16 in LDS once it has arrived, each thread rewriting the
//    16-byte units its own direct loads wrote. The conversion is exact for
//    |v| in [2^-17, 65280] (bf16 has 8 significant bits, and 65280 is its
//    largest value fp16 holds); smaller values are truncated by less than
//    2^-24, and larger ones, outside the call's range, saturate.
//  * The weights are taken relative to a reference maximum that moves only
//    when some row's maximum grows by more than a factor 2^8 (weights then
//    stay <= 256, well inside fp32 and the 16-bit formats); the output is
//    rescaled only then. The result o / l and lse = m + log l do not depend
//    on the reference, so this is exact up to rounding.
//  * Masked keys (causal, window, unmapped blocks) are removed by selection
//    (score -inf); K and V rows outside the loaded range are zero-filled so
//    a zero weight never meets a NaN. Every K and V row multiplied is thus a
//    written row or zeros, and every score finite or -inf: this file is
//    compiled with -fno-honor-nans, which lets the maximum skip quieting its
//    operands.
//
// Two kernels: prefill_kernel (16-bit pools; software-pipelined, described
// at its definition) and prefill_kernel_q8 (8-bit pools: codes gathered and
// widened in LDS, row scales folded into scores and weights; one tile per
// step).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef float f32x2 __attribute__((ext_vector_type(2)));

// mma: one 32x32x16 MFMA of the 16-bit type; pack(a, b): a and b rounded to
// nearest (even) in that type, a in the low half.
template <class T> struct Mma;
template <> struct Mma<BF16T> {
  using V8 = bf16x8;
  static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<F16T> {
  using V8 = f16x8;
  static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
  }
};

constexpr int kKT = 64;   // key positions per tile
// Headroom (base-2 exponent) that a row's maximum may gain over the
// reference maximum before the output is rescaled: weights stay <= 256.
constexpr float kSlackLog2 = 8.f;

// LDS layout of a K or V tile: key row r takes D*2 bytes at r*D*2, as D/8
// units of 16 bytes, and logical unit c of row r is stored at unit
// c ^ swizzle(r). The tiles are filled by direct global->LDS loads, which
// write 64 consecutive units per wavefront instruction, so rows cannot be
// padded; the XOR keeps the reads free of bank conflicts instead:
//  * K (MFMA A operand): 16 lanes read one logical unit of 16 consecutive
//    rows, which land in 16 distinct units modulo 256 bytes (all 64 banks).
//  * V (transpose read): 32 lanes read 4 consecutive rows (first one a
//    multiple of 4) x logical units 4dt .. 4dt+3: again 16 distinct units.
template <int D> struct Swz;
template <> struct Swz<128> {
  static __device__ __forceinline__ int k(int r) { return r & 15; }
  static __device__ __forceinline__ int v(int r) { return 4 * (r & 3); }
};
template <> struct Swz<64> {
  static __device__ __forceinline__ int k(int r) { return (r >> 1) & 7; }
  static __device__ __forceinline__ int v(int r) { return 4 * ((r >> 1) & 1); }
};

// Source of the 16 bytes loaded for a key row that is outside the range or
// unmapped: zeros, so a zero weight never meets a NaN in V.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4];

// One 16-byte direct load per lane from global memory into LDS: lane l of
// the wavefront writes bytes [16 l, 16 l + 16) after `lds` (which must be
// the same for every lane).
__device__ __forceinline__ void dma16(const void* src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
// Wait for this wavefront's direct loads (vmcnt 0). The compiler does not
// see LDS change under a direct load: the empty asm with a memory clobber
// stops it from keeping or assuming LDS values across the wait.
__device__ __forceinline__ void dma_wait() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __asm__ volatile("" ::: "memory");
}

// Row index inside a 32x32 accumulator for register v of lane-half hf.
__device__ __forceinline__ int acc_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

// Byte offset of an LDS location (a __shared__ pointer) in the LDS space.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16) of byte addr + OFF:
// within 16 lanes, lane j reads 4 consecutive 16-bit elements of row j/4 and
// lane i receives element i of those 4 rows. Issued as inline asm because
// the compiler makes each such read that it emits itself wait for every
// direct load in flight (it cannot tell which LDS buffer the builtin reads),
// which would stall on the gather of the next tile. The compiler does not
// track these reads: lds_wait() waits for them and settle() orders each
// result after that wait.
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)"); }
__device__ __forceinline__ void settle(u32x2& x) { asm volatile("" : "+v"(x)); }

// 16-byte LDS read at byte addr + OFF as inline asm (MFMA K operand), so the
// reads of the next k-chunk can be kept in flight under this chunk's MFMAs:
// lds_wait_n<N>() returns once at most N LDS reads are outstanding (they
// complete in order).
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait_n() { asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N)); }
// 16-byte LDS store at byte addr as inline asm (counted by lgkmcnt like the
// reads above; waited for with lds_wait_n<0>() before a barrier).
__device__ __forceinline__ void lds_write16(uint32_t addr, const u32x4& x) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(x) : "memory");
}
__device__ __forceinline__ void settle(u32x4& x) { asm volatile("" : "+v"(x)); }

template <int N> struct IntC { static constexpr int value = N; };

// Sixteen 8-bit codes of one 16-byte unit as fp32 values (exact): INT8 as
// the signed byte, FP8 E4M3 as the code's value.
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
  for (int i = 0; i < 4; ++i) codes4_to_f32<FP8T>(x[i], f + 4 * i);  // BIAS 0: the code's value
}

// Eight values that the 16-bit type holds exactly, as one 16-byte unit.
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

// Prefill over 8-bit pools (INT8 or OCP FP8 E4M3 codes, CT, with one fp32
// scale per row), one key tile per step, two LDS buffers. A tile's codes are
// gathered into LDS by direct loads, then each thread widens the 16 codes
// it loaded into the 16-bit tiles: K into q's type T, V into fp16 (exact:
// every INT8 code and E4M3 value is both a bf16 and an fp16 value). Key t's
// score is its dot product with the codes times its K scale; its weight
// times its V scale is what the fp16 matrix cores multiply with the V
// codes. log2 of the V scale is added to the score before the tile maximum
// (e_t = scale * score_t * log2(e) + log2(vs_t)), so exp2(e_t - m) is weight
// times V scale relative to a reference m that bounds it by 2^8, whatever
// the scales' magnitudes; the normaliser sums those products as rounded to
// fp16 times 1 / vs_t, the weights the matrix cores actually apply. A zero
// V row (scale 0, all codes 0) takes scale 1 so that its weight stays in
// the normaliser.
template <class T, class CT, int D, int B, int G, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_kernel_q8(PrefillArgs a, float scale_log2) {
  constexpr bool QS = true;
  using M = Mma<T>;      // S = K.Q^T in the input type
  using MP = Mma<F16T>;  // O += V^T.P^T in fp16 (V codes widened to fp16)
  using V8 = typename M::V8;
  using P8 = typename MP::V8;
  constexpr int KC = D / 16;            // MFMA k-chunks over the head dim
  constexpr int DT = D / 32;            // 32-wide output tiles over the head dim
  constexpr int HPW = G < NW ? G : NW;  // query heads per workgroup
  constexpr int PSUB = NW / HPW;        // 32-row query sub-tiles per workgroup
  constexpr int QT = 32 * PSUB;         // query rows per workgroup
  constexpr int U = D / 8;              // 16-byte units of a widened key row
  constexpr int UQ = D / 16;            // 16-byte units of a key row of codes
  constexpr int NIQ = kKT * UQ / 64;    // wavefront load instructions per tile (each of K and V)
  constexpr int NLDQ = (NIQ + NW - 1) / NW;  // per wavefront (the last may be idle)
  constexpr int RPIQ = 64 / UQ;         // key rows per load instruction
  static_assert(B % RPIQ == 0, "a wavefront instruction must not straddle blocks");

  // Two buffers of each of K and V, as separate arrays: the compiler then
  // knows that reads of one buffer do not depend on direct loads in flight
  // into the other.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[kKT * D];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[kKT * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[kKT * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[kKT * D];
  // Codes as loaded (unswizzled: load unit P at byte 16 P). One buffer:
  // each thread widens exactly the units it loaded, within the step.
  __shared__ __attribute__((aligned(16))) uint8_t kc_lds[kKT * D];
  __shared__ __attribute__((aligned(16))) uint8_t vc_lds[kKT * D];
  __shared__ unsigned long long kvalid[2];  // bit t: key t0 + t of the tile is mapped
  // Per key of each buffer's tile: K scale * scale * log2(e), log2 of the V
  // scale and its inverse (0, 0, 1 for keys outside the range, masked).
  __shared__ __attribute__((aligned(16))) float scl[2][3][kKT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int hf = lane >> 5;
  const int ql = lane & 31;
  // Workgroups are dispatched to the 8 XCDs round-robin by index; the index
  // is renumbered so that each XCD runs a contiguous range of work items,
  // ordered (kv-head group, sequence, query tile): the workgroups sharing a
  // kv head's keys and values then share one XCD's L2.
  int s, yg, qt;
  {
    const int N = a.grid_q * a.grid_y * a.S;
    const int b = blockIdx.x, per = N / 8, rem = N % 8, x = b % 8;
    const int w = x * per + min(x, rem) + b / 8;
    yg = w / (a.grid_q * a.S);
    const int r = w % (a.grid_q * a.S);
    s = r / a.grid_q;
    qt = a.grid_q - 1 - r % a.grid_q;  // heaviest (latest) tiles first
  }
  const int g = yg / (G / HPW);
  const int hq = g * G + (yg % (G / HPW)) * HPW + wave % HPW;

  const int r0 = a.q_start[s];
  const int C = a.q_start[s + 1] - r0;
  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  if (qt * QT >= C || C > L) return;
  if (a.skip_single && C == 1) return;  // a decode row of a mixed batch
  const int row0 = qt * QT + (wave / HPW) * 32;   // first chunk row of this wavefront
  const int wg_last = min(C, (qt + 1) * QT) - 1;  // last chunk row of the workgroup
  const int base = L - C;                         // position of chunk row 0
  const int kv_hi = base + wg_last + 1;
  int kv_lo = 0;
  if (a.window > 0) kv_lo = max(0, base + qt * QT - a.window + 1);
  const int t_first = (kv_lo / kKT) * kKT;
  // Key tiles in processing order: with attention sinks, first the tiles
  // holding positions below min(sinks, kv_lo) that lie before the window's
  // first tile (ns of them), then the window's tiles from t_first.
  const int ns = min((min(a.sinks, kv_lo) + kKT - 1) / kKT, t_first / kKT);
  const int ntiles = ns + (kv_hi - t_first + kKT - 1) / kKT;
  auto tile_t0 = [&](int i) { return i < ns ? i * kKT : t_first + (i - ns) * kKT; };
  // A key position the workgroup's rows may attend.
  auto in_range = [&](int t) { return (t >= kv_lo || t < a.sinks) && t < kv_hi; };

  // Query fragment of this lane: row ql of the wavefront, 8 elements per k-chunk.
  const int my_row = row0 + ql;
  const bool row_ok = my_row < C;
  const int my_pos = base + my_row;
  V8 qf[KC];
  {
    const char* qp = (const char*)a.q + ((size_t)(r0 + (row_ok ? my_row : 0)) * a.H + hq) * D * 2;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 v = load16(qp + (size_t)(kc * 16 + 8 * hf) * 2);
      if (!row_ok) v = u32x4{0, 0, 0, 0};
      qf[kc] = __builtin_bit_cast(V8, v);
    }
  }

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;  // running max of the scaled scores (base 2)
  float l_run = 0.f;        // normaliser: sum of the fp16-rounded weight x V scale products / V scale

  const int wave_pmin = base + row0;
  const int wave_pmax = base + min(row0 + 31, C - 1);
  const bool wave_has_rows = row0 < C;
  const uint32_t row_stride = (uint32_t)a.Hkv * D;  // codes: one byte per element
  const uint32_t block_stride = (uint32_t)B * row_stride;
  const char* kpool = (const char*)a.k_pool + (size_t)g * D;
  const char* vpool = (const char*)a.v_pool + (size_t)g * D;
  const int32_t* trow = a.tables + (size_t)s * a.mb;
  const char* zero = (const char*)g_zero16;

  // Tile gather. Load j of thread (wave, lane), instruction x = NW j + wave
  // (if below NIQ), fills code unit P = 64 x + lane of the tile: row P / UQ,
  // 16 codes from element 16 (P % UQ). The RPIQ rows of one instruction lie
  // in one block: its table entry is uniform over the wavefront. Entries are
  // read one tile ahead (`fetch_table`), as lane values (through an index
  // offset the compiler cannot see is zero): a uniform load would be moved
  // to a scalar register right away, waiting for it and, since vector memory
  // operations complete in order, for every direct load issued before it.
  int pb_ins[NLDQ];  // table entry of instruction j of this wavefront, next tile
  int pb_key = -1;   // wavefront 0: table entry of key t0 + lane, next tile
  int lane_zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(lane_zero));
  auto fetch_table = [&](int t0) {
#pragma unroll
    for (int j = 0; j < NLDQ; ++j)  // in range of the table row even past the context
      pb_ins[j] = trow[min((t0 + min(NW * j + wave, NIQ - 1) * RPIQ) / B, a.mb - 1) + lane_zero];
    if (wave == 0) pb_key = trow[min((t0 + lane) / B, a.mb - 1)];
  };
  auto gather = [&](int t0, uint8_t* kd, uint8_t* vd) {
    // Whole tile inside the attended range: only the block entries decide.
    const bool whole = t0 >= kv_lo && t0 + kKT <= kv_hi;
#pragma unroll
    for (int j = 0; j < NLDQ; ++j) {
      const int x = NW * j + wave;
      if (x >= NIQ) break;
      const int pb = pb_ins[j];
      const bool blk_ok = pb >= 0 && pb < a.nb;
      const size_t boff = (size_t)(uint32_t)(blk_ok ? pb : 0) * block_stride;
      const int r = x * RPIQ + lane / UQ;
      const uint32_t off = (uint32_t)((r % B) * row_stride) + 16 * (lane % UQ);
      bool ok = blk_ok;
      if (!whole) ok = ok && in_range(t0 + r);
      dma16(ok ? kpool + boff + off : zero, (uint16_t*)(kd + 1024 * x));
      dma16(ok ? vpool + boff + off : zero, (uint16_t*)(vd + 1024 * x));
    }
  };
  // Widen the code units this thread loaded (after dma_wait): 16 codes of
  // row r from element 16 c become the 16-bit logical units 2c and 2c + 1
  // of row r, stored where the swizzle puts them; K in T, V in fp16.
  auto widen = [&](const uint8_t* kcs, const uint8_t* vcs, uint16_t* kd, uint16_t* vd) {
#pragma unroll
    for (int j = 0; j < NLDQ; ++j) {
      const int x = NW * j + wave;
      if (x >= NIQ) break;
      const int P = 64 * x + lane, r = P / UQ, c = P % UQ;
      float f[16];
      codes16_to_f32<CT>(*reinterpret_cast<const u32x4*>(kcs + 16 * P), f);
      *reinterpret_cast<u32x4*>(kd + r * D + 8 * ((2 * c) ^ Swz<D>::k(r))) = pack8<T>(f);
      *reinterpret_cast<u32x4*>(kd + r * D + 8 * ((2 * c + 1) ^ Swz<D>::k(r))) = pack8<T>(f + 8);
      codes16_to_f32<CT>(*reinterpret_cast<const u32x4*>(vcs + 16 * P), f);
      *reinterpret_cast<u32x4*>(vd + r * D + 8 * ((2 * c) ^ Swz<D>::v(r))) = pack8<F16T>(f);
      *reinterpret_cast<u32x4*>(vd + r * D + 8 * ((2 * c + 1) ^ Swz<D>::v(r))) = pack8<F16T>(f + 8);
    }
  };
  // Key validity bitmask of a tile (64 lanes = 64 keys), by wavefront 0,
  // with the keys' scales into registers (stored to LDS by store_scales
  // once the tile's loads are waited for).
  float sk_reg = 0.f, sv_reg = 0.f;
  auto put_valid = [&](int t0, int slot) {
    if (wave == 0) {
      const int t = t0 + lane;
      const bool ok = in_range(t) && pb_key >= 0 && pb_key < a.nb;
      const unsigned long long vm = __ballot(ok);
      if (lane == 0) kvalid[slot] = vm;
      if constexpr (QS) {
        const size_t si = ((size_t)(uint32_t)(ok ? pb_key : 0) * a.Hkv + g) * B + (t & (B - 1));
        sk_reg = ok ? a.k_scale[si] : 0.f;
        sv_reg = ok ? a.v_scale[si] : 0.f;
      }
    }
  };
  auto store_scales = [&](int slot) {
    if (wave == 0) {
      const bool pos = sv_reg > 0.f;  // a zero V row takes scale 1
      scl[slot][0][lane] = sk_reg * scale_log2;
      scl[slot][1][lane] = pos ? __log2f(sv_reg) : 0.f;
      scl[slot][2][lane] = pos ? 1.f / sv_reg : 1.f;
    }
  };

  // V^T operand addressing for the transpose read: 16-lane group gq = lane/16
  // covers dims 16*(gq&1) .. +16 of a 32-dim tile and key half hf = gq>>1.
  const int gq = lane >> 4, j16 = lane & 15;
  const int tr_row = j16 >> 2;                          // key offset inside 4
  const int tr_unit = 2 * (gq & 1) + ((j16 & 3) >> 1);  // 16-byte unit inside a 32-dim tile
  const int tr_sw = Swz<D>::v(tr_row) >> 2;             // swizzle of rows 4i + tr_row, in 4-unit steps
  const int tr_elem = 4 * (j16 & 1);                    // element inside the unit
  // Byte offset, inside a V buffer, of this lane's transpose read for key
  // chunk 0 and dim tile dt (other key chunks add constants).
  uint32_t tr_addr[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    tr_addr[dt] = 2 * ((4 * hf + tr_row) * D + tr_elem + 8 * (4 * (dt ^ tr_sw) + tr_unit));
  // K operand: row kh*32 + ql, logical unit 2 kc + hf, stored at
  // (2 kc) ^ (hf ^ swizzle(ql)) (the swizzle is the same for both halves).
  const int k_sw = hf ^ Swz<D>::k(ql);

  // One tile: gather the next tile into the other buffers, compute this one
  // from (Ks, Vs, kvalid[slot]), wait for the gather, barrier. Returns
  // whether a next tile exists.
  auto step = [&](int i, const uint16_t* Ks, const uint16_t* Vs, uint16_t* Kn, uint16_t* Vn, uint8_t* Kcn,
                  uint8_t* Vcn, int slot) -> bool {
    const int t0 = tile_t0(i);
    const bool has_next = i + 1 < ntiles;
    if (has_next) {
      gather(tile_t0(i + 1), Kcn, Vcn);
      put_valid(tile_t0(i + 1), slot ^ 1);
      if (i + 2 < ntiles) fetch_table(tile_t0(i + 2));
    }

    // Skip a tile whose keys all follow the wavefront's last row, or all
    // precede its first row's window without holding a sink position.
    bool skip = !wave_has_rows || t0 > wave_pmax;
    if (a.window > 0 && t0 + kKT - 1 <= wave_pmin - a.window && t0 >= a.sinks) skip = true;
    if (!skip) {
      const unsigned long long vmask = kvalid[slot];
      // S^T = K_tile . Q^T, two 32-key halves.
      // The K fragments of chunk kc+1 are read while chunk kc multiplies.
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      const uint32_t kbase = lds_offset(Ks) + 2 * ql * D;
      auto kaddr = [&](int kc) { return kbase + 16 * ((2 * kc) ^ k_sw); };
      u32x4 ka[2][2];  // [chunk parity][key half]
      ka[0][0] = lds_read16<0>(kaddr(0));
      ka[0][1] = lds_read16<32 * D * 2>(kaddr(0));
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int cur = kc & 1;
        if (kc + 1 < KC) {
          ka[cur ^ 1][0] = lds_read16<0>(kaddr(kc + 1));
          ka[cur ^ 1][1] = lds_read16<32 * D * 2>(kaddr(kc + 1));
          lds_wait_n<2>();
        } else {
          lds_wait_n<0>();
        }
        settle(ka[cur][0]);
        settle(ka[cur][1]);
        sacc[0] = M::mma(__builtin_bit_cast(V8, ka[cur][0]), qf[kc], sacc[0]);
        sacc[1] = M::mma(__builtin_bit_cast(V8, ka[cur][1]), qf[kc], sacc[1]);
      }
      {  // e = dot * K scale * scale * log2(e) + log2(V scale) for keys 8*(v/4) + 4*hf + v%4 of each half
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 k4 = *reinterpret_cast<const float4*>(&scl[slot][0][kh * 32 + 8 * q4 + 4 * hf]);
            const float4 l4 = *reinterpret_cast<const float4*>(&scl[slot][1][kh * 32 + 8 * q4 + 4 * hf]);
            sacc[kh][4 * q4] = __builtin_fmaf(sacc[kh][4 * q4], k4.x, l4.x);
            sacc[kh][4 * q4 + 1] = __builtin_fmaf(sacc[kh][4 * q4 + 1], k4.y, l4.y);
            sacc[kh][4 * q4 + 2] = __builtin_fmaf(sacc[kh][4 * q4 + 2], k4.z, l4.z);
            sacc[kh][4 * q4 + 3] = __builtin_fmaf(sacc[kh][4 * q4 + 3], k4.w, l4.w);
          }
      }
      // Mask (selection, branch-free), running maximum of the raw scores.
      const bool need_mask = vmask != ~0ull || wave_pmin < t0 + kKT - 1 || row0 + 31 >= C ||
                             (a.window > 0 && t0 <= wave_pmax - a.window);
      if (need_mask) {
        const int lim_hi = row_ok ? my_pos - t0 : -1;  // key offsets <= lim_hi
        const int lim_lo = a.window > 0 ? my_pos - a.window + 1 - t0 : -(1 << 30);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kl = kh * 32 + acc_row(v, hf);
            const bool ok = kl <= lim_hi && (kl >= lim_lo || kl + t0 < a.sinks) && ((vmask >> kl) & 1);
            sacc[kh][v] = ok ? sacc[kh][v] : -INFINITY;
          }
        }
      }
      // Tile maximum as a tree, then across the two lane halves that hold
      // the same query (v_permlane32_swap exchanges the halves).
      float m8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        m8[k] = fmaxf(fmaxf(sacc[k >> 2][4 * (k & 3)], sacc[k >> 2][4 * (k & 3) + 1]),
                      fmaxf(sacc[k >> 2][4 * (k & 3) + 2], sacc[k >> 2][4 * (k & 3) + 3]));
      float mt = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])),
                       fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mt),
                                                         __builtin_bit_cast(uint32_t, mt), false, false);
        mt = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
      }
      // The reference maximum m_run moves only when some row's tile maximum
      // exceeds it by more than kSlackLog2, so weights are at most
      // 2^kSlackLog2 and the output rescale (exact either way) is rare.
      if (__any(mt > m_run + kSlackLog2)) {
        const float mn = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - (mn == -INFINITY ? 0.f : mn));
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        m_run = mn;
      }
      const float ms = m_run == -INFINITY ? 0.f : m_run;

      // P^T operands: key chunk c = 16 keys; this lane supplies the weights of
      // its accumulator registers 8*(c%2) .. +7 of half c/2, i.e. keys
      // 16c + 8*(e/4) + 4*hf + e%4 for e = 0..7.
      const uint32_t vbase = lds_offset(Vs);
      auto chunk = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
        constexpr int kh = c >> 1, sub = c & 1;
        // V^T operands of this chunk: keys 16c .. 16c+15, loaded first so the
        // LDS latency overlaps the weights below.
        u32x2 e03[DT], e47[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          e03[dt] = lds_read_tr<16 * c * D * 2>(vbase + tr_addr[dt]);
          e47[dt] = lds_read_tr<(16 * c + 8) * D * 2>(vbase + tr_addr[dt]);
        }
        uint32_t hi[4];
        float vi[8];  // inverse V scales of this lane's 8 keys of the chunk
        {
          const float4 ia = *reinterpret_cast<const float4*>(&scl[slot][2][16 * c + 4 * hf]);
          const float4 ib = *reinterpret_cast<const float4*>(&scl[slot][2][16 * c + 8 + 4 * hf]);
          vi[0] = ia.x; vi[1] = ia.y; vi[2] = ia.z; vi[3] = ia.w;
          vi[4] = ib.x; vi[5] = ib.y; vi[6] = ib.z; vi[7] = ib.w;
        }
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // weight x V scale relative to the reference, rounded to fp16 for
          // the matrix cores; the normaliser sums those rounded products
          // divided by their scales, exactly the weights the matrix cores
          // apply (a lone key's row then comes out exact)
          const float p0 = __builtin_amdgcn_exp2f(sacc[kh][8 * sub + 2 * e2] - ms);
          const float p1 = __builtin_amdgcn_exp2f(sacc[kh][8 * sub + 2 * e2 + 1] - ms);
          const uint32_t hv = MP::pack(p0, p1);
          hi[e2] = hv;
          const f16x2 w = as_h2(hv);
          l_run = __builtin_fmaf((float)w[0], vi[2 * e2], l_run);
          l_run = __builtin_fmaf((float)w[1], vi[2 * e2 + 1], l_run);
        }
        const P8 bhi = __builtin_bit_cast(P8, u32x4{hi[0], hi[1], hi[2], hi[3]});
        lds_wait();
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          settle(e03[dt]);
          settle(e47[dt]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const P8 av = __builtin_bit_cast(P8, u32x4{e03[dt].x, e03[dt].y, e47[dt].x, e47[dt].y});
          o[dt] = MP::mma(av, bhi, o[dt]);
        }
      };
      chunk(IntC<0>{});
      chunk(IntC<1>{});
      chunk(IntC<2>{});
      chunk(IntC<3>{});
    }
    dma_wait();
    if (has_next) {
      widen(Kcn, Vcn, Kn, Vn);  // the next tile's code units this thread loaded
      store_scales(slot ^ 1);
    }
    __syncthreads();
    return has_next;
  };

  fetch_table(tile_t0(0));
  dma_wait();  // table entries in registers
  gather(tile_t0(0), kc_lds, vc_lds);
  put_valid(tile_t0(0), 0);
  if (ntiles > 1) fetch_table(tile_t0(1));
  dma_wait();
  widen(kc_lds, vc_lds, k_lds0, v_lds0);
  store_scales(0);
  __syncthreads();
  for (int i = 0;; i += 2) {
    if (!step(i, k_lds0, v_lds0, k_lds1, v_lds1, kc_lds, vc_lds, 0)) break;
    if (!step(i + 1, k_lds1, v_lds1, k_lds0, v_lds0, kc_lds, vc_lds, 1)) break;
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* op = a.out + ((size_t)(r0 + my_row) * a.H + hq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int d = dt * 32 + 8 * v4 + 4 * hf;
      float4 w = make_float4(o[dt][4 * v4] * inv, o[dt][4 * v4 + 1] * inv, o[dt][4 * v4 + 2] * inv,
                             o[dt][4 * v4 + 3] * inv);
      *reinterpret_cast<float4*>(op + d) = w;
    }
  }
  if (a.lse) {
    if (hf == 0)
      a.lse[(size_t)(r0 + my_row) * a.H + hq] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Wait until at most N of this wavefront's vector memory operations
// (direct loads included) are outstanding; the compiler may not keep LDS
// values across it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


// Bits [0, n) of a 64-bit mask, n clamped to [0, 64].
__device__ __forceinline__ unsigned long long low_bits(int n) {
  return n <= 0 ? 0ull : (n >= 64 ? ~0ull : ((1ull << n) - 1));
}

// Prefill over 16-bit pools, software-pipelined per wavefront.
//
// A workgroup of 8 wavefronts covers the query heads of one kv head (up to
// 8) and as many 32-row sub-tiles as the rest allows; each wavefront owns 32
// query rows of one head. Key tiles of 64 positions rotate through four LDS
// stages. Iteration i of a wavefront overlaps two tiles:
//   phase X: the 16 MFMAs of tile i+1's scores S^T = K.Q^T, interleaved with
//            tile i's weights (exp2, fp16 rounding, row sum) on the vector ALU
//            and with the conversion of this thread's V units of tile i+1
//            (bf16 -> fp16);
//   phase Y: the 16 MFMAs of tile i's O^T += V^T.P^T, interleaved with tile
//            i+1's mask and row maximum, and the direct loads of tile i+3
//            into the stage tile i-1 held;
// then the reference-maximum update of tile i+1 (rare output rescale).
// K fragments are read from LDS two k-chunks ahead of their MFMAs, V
// fragments one 16-key chunk ahead. Each iteration ends with each thread
// waiting for its own loads of tile i+2 and one barrier. The table entries
// come from scalar loads one tile further ahead.
template <class T, int D, int B, int G>
__global__ __launch_bounds__(512, 1) void prefill_kernel(PrefillArgs a, float scale_log2) {
  using M = Mma<T>;      // S = K.Q^T in the input type
  using MP = Mma<F16T>;  // O += V^T.P^T in fp16 (V converted in LDS when bf16)
  using V8 = typename M::V8;
  using P8 = typename MP::V8;
  constexpr int NW = 8;                 // wavefronts per workgroup
  constexpr int KC = D / 16;            // MFMA k-chunks over the head dim
  constexpr int DT = D / 32;            // 32-wide output tiles over the head dim
  constexpr int HPW = G < NW ? G : NW;  // query heads per workgroup
  constexpr int PSUB = NW / HPW;        // 32-row query sub-tiles per workgroup
  constexpr int QT = 32 * PSUB;         // query rows per workgroup
  constexpr int U = D / 8;              // 16-byte units per key row
  constexpr int NLD = kKT * U / (64 * NW);  // direct loads per thread per tile (each of K and V)
  constexpr int RPI = 64 / U;           // key rows per wavefront load instruction
  constexpr int TB = kKT / B;           // table entries per tile
  constexpr int NST = 4;                // LDS stages
  constexpr int TILE = kKT * D;         // 16-bit elements of one K or V tile
  static_assert(B % RPI == 0, "a wavefront instruction must not straddle blocks");
  static_assert(KC >= 4, "the K read pipeline assumes at least 4 k-chunks");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NST * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[NST * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int hf = lane >> 5;
  const int ql = lane & 31;
  // Workgroups are dispatched to the 8 XCDs round-robin by index; the index
  // is renumbered so that each XCD runs a contiguous range of work items,
  // ordered (kv-head group, sequence, query tile): the workgroups sharing a
  // kv head's keys and values then share one XCD's L2.
  int s, yg, qt;
  {
    const int N = a.grid_q * a.grid_y * a.S;
    const int b = blockIdx.x, per = N / 8, rem = N % 8, x = b % 8;
    const int w = x * per + min(x, rem) + b / 8;
    yg = w / (a.grid_q * a.S);
    const int r = w % (a.grid_q * a.S);
    s = r / a.grid_q;
    qt = a.grid_q - 1 - r % a.grid_q;  // heaviest (latest) tiles first
  }
  const int g = yg / (G / HPW);
  const int hq = g * G + (yg % (G / HPW)) * HPW + wave % HPW;

  const int r0 = a.q_start[s];
  const int C = a.q_start[s + 1] - r0;
  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  if (qt * QT >= C || C > L) return;
  if (a.skip_single && C == 1) return;  // a decode row of a mixed batch
  const int row0 = qt * QT + (wave / HPW) * 32;   // first chunk row of this wavefront
  const int wg_last = min(C, (qt + 1) * QT) - 1;  // last chunk row of the workgroup
  const int base = L - C;                         // position of chunk row 0
  const int kv_hi = base + wg_last + 1;
  int kv_lo = 0;
  if (a.window > 0) kv_lo = max(0, base + qt * QT - a.window + 1);
  const int t_first = (kv_lo / kKT) * kKT;
  // Key tiles in processing order: with attention sinks, first the tiles
  // holding positions below min(sinks, kv_lo) that lie before the window's
  // first tile (ns of them), then the window's tiles from t_first.
  const int ns = min((min(a.sinks, kv_lo) + kKT - 1) / kKT, t_first / kKT);
  const int ntiles = ns + (kv_hi - t_first + kKT - 1) / kKT;
  auto tile_t0 = [&](int i) { return i < ns ? i * kKT : t_first + (i - ns) * kKT; };

  // Query fragment of this lane: row ql of the wavefront, 8 elements per k-chunk.
  const int my_row = row0 + ql;
  const bool row_ok = my_row < C;
  const int my_pos = base + my_row;
  V8 qf[KC];
  {
    const char* qp = (const char*)a.q + ((size_t)(r0 + (row_ok ? my_row : 0)) * a.H + hq) * D * 2;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 v = load16(qp + (size_t)(kc * 16 + 8 * hf) * 2);
      if (!row_ok) v = u32x4{0, 0, 0, 0};
      qf[kc] = __builtin_bit_cast(V8, v);
    }
  }

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;  // reference maximum of the scaled scores (base 2)
  float l_run = 0.f;        // normaliser: sum of the fp16-rounded weights

  const int wave_pmin = base + row0;
  const int wave_pmax = base + min(row0 + 31, C - 1);
  const uint32_t row_stride = (uint32_t)a.Hkv * D * 2;
  const uint32_t block_stride = (uint32_t)B * row_stride;
  const ctab_t trow = (ctab_t)(a.tables + (size_t)s * a.mb);
  const char* zero = (const char*)g_zero16;

  // Tile gather. Load j of thread (wave, lane) fills unit P = 64 (8 j + wave)
  // + lane of the tile: row P / U, stored unit P % U, holding the logical
  // unit that the swizzle puts there. The 64 / U rows of one wavefront
  // instruction lie in one block (tile entry bj[j]), so a load's address is
  // that block's base (scalar) plus a per-lane offset fixed for the kernel.
  int bj[NLD];
  uint32_t koff[NLD], voff[NLD];
  int rj[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int r = (NW * j + wave) * RPI + lane / U, cs = lane % U;
    rj[j] = r;
    bj[j] = uniform((NW * j + wave) * RPI / B);
    koff[j] = (uint32_t)((r % B) * row_stride) + 16 * (cs ^ Swz<D>::k(r)) + (uint32_t)g * D * 2;
    voff[j] = (uint32_t)((r % B) * row_stride) + 16 * (cs ^ Swz<D>::v(r)) + (uint32_t)g * D * 2;
  }
  // Table entries of a tile (scalar loads; clamped inside the table row):
  // all of them for the key mask, and this wavefront's own (pb_j[j] for its
  // load j) loaded apart, so no register array is indexed at run time.
  int ent[TB], pb_j[NLD];
  uint32_t bj_off[NLD];  // byte offset of this wavefront's entry for load j inside a tile's entries
#pragma unroll
  for (int j = 0; j < NLD; ++j) bj_off[j] = 4u * (uint32_t)bj[j];
  auto fetch = [&](int t0) {
    const int b0 = t0 / B;
    if (b0 + TB <= a.mb) {
      // The usual case: the tile's TB entries in one scalar load, and each
      // of this wavefront's entries at its fixed offset from them.
      typedef int32_t EntV __attribute__((ext_vector_type(TB), aligned(4)));
      const __attribute__((address_space(4))) char* te = (const __attribute__((address_space(4))) char*)(trow + b0);
      const EntV e = *(const __attribute__((address_space(4))) EntV*)te;
#pragma unroll
      for (int k = 0; k < TB; ++k) ent[k] = e[k];
#pragma unroll
      for (int j = 0; j < NLD; ++j) pb_j[j] = *(ctab_t)(te + bj_off[j]);
    } else {
#pragma unroll
      for (int k = 0; k < TB; ++k) ent[k] = trow[min(b0 + k, a.mb - 1)];
#pragma unroll
      for (int j = 0; j < NLD; ++j) pb_j[j] = trow[min(b0 + bj[j], a.mb - 1)];
    }
  };
  // Bit k of a tile's key mask: key t0 + k is in the workgroup's range and
  // its block is mapped.
  auto key_mask = [&](int t0) -> unsigned long long {
    bool mapped = true;
#pragma unroll
    for (int k = 0; k < TB; ++k) mapped = mapped && (uint32_t)ent[k] < (uint32_t)a.nb;
    if (mapped && t0 >= kv_lo && t0 + kKT <= kv_hi) return ~0ull;  // the usual case
    unsigned long long blk = 0;
#pragma unroll
    for (int k = 0; k < TB; ++k)
      if (ent[k] >= 0 && ent[k] < a.nb) blk |= low_bits(B) << (k * B);
    const unsigned long long range =
        low_bits(kv_hi - t0) & (~low_bits(kv_lo - t0) | low_bits(a.sinks - t0));
    return blk & range;
  };
  const char* kpool = (const char*)a.k_pool;
  const char* vpool = (const char*)a.v_pool;
  auto gather = [&](int st, unsigned long long vmask) {
    uint16_t* kd = k_lds + st * TILE;
    uint16_t* vd = v_lds + st * TILE;
    if (vmask == ~0ull) {
      // Block bases in scalar registers, lane offsets in 32 bits.
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const size_t boff = (size_t)(uint32_t)pb_j[j] * block_stride;
        const char* kb = kpool + boff;
        const char* vb = vpool + boff;
        dma16(kb + koff[j], kd + (NW * j + wave) * 512);
        dma16(vb + voff[j], vd + (NW * j + wave) * 512);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const bool ok = (vmask >> rj[j]) & 1;
        const size_t boff = (size_t)(uint32_t)(ok ? pb_j[j] : 0) * block_stride;
        dma16(ok ? kpool + boff + koff[j] : zero, kd + (NW * j + wave) * 512);
        dma16(ok ? vpool + boff + voff[j] : zero, vd + (NW * j + wave) * 512);
      }
    }
  };
  // Conversion of this thread's V units of a tile (bf16 -> fp16) once its
  // loads have completed, in three parts so that it can sit between matrix
  // instructions: cv_read issues the LDS reads (inline asm, like the operand
  // reads, so that the compiler's own waits are not disturbed), cv_convert
  // converts once they have arrived, cv_write stores the units back.
  u32x4 cvu[NLD];
  uint32_t cv_addr[NLD];
  auto cv_read = [&](int st) {
    if constexpr (!std::is_same<T, F16T>::value) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        cv_addr[j] = lds_offset(v_lds + st * TILE + (NW * j + wave) * 512 + 8 * lane);
        cvu[j] = lds_read16<0>(cv_addr[j]);
      }
    }
  };
  auto cv_convert = [&]() {
    if constexpr (!std::is_same<T, F16T>::value) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        settle(cvu[j]);
        uint32_t w[4] = {cvu[j].x, cvu[j].y, cvu[j].z, cvu[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __builtin_bit_cast(float, w[e] << 16), hi = __builtin_bit_cast(float, w[e] & 0xffff0000u);
          w[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
        }
        cvu[j] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  };
  auto cv_write = [&]() {
    if constexpr (!std::is_same<T, F16T>::value) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) lds_write16(cv_addr[j], cvu[j]);
    }
  };

  // V^T operand addressing for the transpose read: 16-lane group gq = lane/16
  // covers dims 16*(gq&1) .. +16 of a 32-dim tile and key half hf = gq>>1.
  const int gq = lane >> 4, j16 = lane & 15;
  const int tr_row = j16 >> 2;                          // key offset inside 4
  const int tr_unit = 2 * (gq & 1) + ((j16 & 3) >> 1);  // 16-byte unit inside a 32-dim tile
  const int tr_sw = Swz<D>::v(tr_row) >> 2;             // swizzle of rows 4i + tr_row, in 4-unit steps
  const int tr_elem = 4 * (j16 & 1);                    // element inside the unit
  uint32_t tr_addr[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    tr_addr[dt] = 2 * ((4 * hf + tr_row) * D + tr_elem + 8 * (4 * (dt ^ tr_sw) + tr_unit));
  // K operand: row kh*32 + ql, logical unit 2 kc + hf, stored at
  // (2 kc) ^ (hf ^ swizzle(ql)) (the swizzle is the same for both halves).
  const int k_sw = hf ^ Swz<D>::k(ql);
  const uint32_t k_lane = 2 * ql * D;
  auto kaddr = [&](uint32_t kb, int kc) { return kb + k_lane + 16 * ((2 * kc) ^ k_sw); };

  unsigned long long vm0 = 0, vm1 = 0, vm2 = 0, vm3 = 0;  // key masks (see the prologue)
  float ms = 0.f;  // reference maximum the current tile's weights are taken against
  uint32_t pk[4][4];  // fp16 weights of the current tile: [key chunk][pair]

  // Weights of pair j (0..15) of the current tile's scores sc: chunk c = j/4
  // supplies keys 16c + 8*(e/4) + 4*hf + e%4 (accumulator registers
  // 8*(c%2) .. +7 of half c/2); each pair is rounded to fp16 for the matrix
  // cores and the normaliser sums the weights as rounded, so the output is
  // their exact weighted average.
  auto weights = [&](const f32x16* sc, int j) {
    const int c = j >> 2, e2 = j & 3, kh = c >> 1, sub = c & 1;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kh][8 * sub + 2 * e2], scale_log2, -ms));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kh][8 * sub + 2 * e2 + 1], scale_log2, -ms));
    uint32_t h = MP::pack(p0, p1);
    asm volatile("" : "+v"(h));  // computed here, between the matrix instructions
    pk[c][e2] = h;
    l_run = __builtin_amdgcn_fdot2(as_h2(h), f16x2{(_Float16)1.f, (_Float16)1.f}, l_run, false);
  };

  // Phase X: scores of the next tile (K in stage kst) into sn, with the
  // current tile's weights (from sc) between the MFMAs. K fragments are read
  // two k-chunks ahead: ring slot kc % 3.
  auto phase_x = [&](const f32x16* sc, f32x16* sn, int kst, bool conv, int cst) {
    const uint32_t kb = lds_offset(k_lds + kst * TILE);
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    if (conv) cv_read(cst);  // oldest reads: complete before the first K fragments
    u32x4 ka[3][2];
    ka[0][0] = lds_read16<0>(kaddr(kb, 0));
    ka[0][1] = lds_read16<32 * D * 2>(kaddr(kb, 0));
    ka[1][0] = lds_read16<0>(kaddr(kb, 1));
    ka[1][1] = lds_read16<32 * D * 2>(kaddr(kb, 1));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int cur = kc % 3;
      if (kc + 2 < KC) {
        ka[(kc + 2) % 3][0] = lds_read16<0>(kaddr(kb, kc + 2));
        ka[(kc + 2) % 3][1] = lds_read16<32 * D * 2>(kaddr(kb, kc + 2));
        lds_wait_n<4>();
      } else if (kc + 1 < KC) {
        lds_wait_n<2>();
      } else {
        lds_wait_n<0>();
      }
      settle(ka[cur][0]);
      settle(ka[cur][1]);
      sn[0] = M::mma(__builtin_bit_cast(V8, ka[cur][0]), qf[kc], sn[0]);
      if (kc < 8) weights(sc, 2 * kc);
      sn[1] = M::mma(__builtin_bit_cast(V8, ka[cur][1]), qf[kc], sn[1]);
      if (kc < 8) weights(sc, 2 * kc + 1);
      if (conv && kc == 1) cv_convert();
      if (conv && kc == 3) cv_write();
    }
#pragma unroll
    for (int j = 2 * KC; j < 16; ++j) weights(sc, j);  // head dim 64: the rest of the weights
  };
  // The last tile's weights, with no next tile to overlap.
  auto weights_only = [&](const f32x16* sc) {
#pragma unroll
    for (int j = 0; j < 16; ++j) weights(sc, j);
  };

  // Mask of the next tile's scores (branch-free selection) where the tile
  // is not wholly attended by every row of the wavefront.
  auto mask = [&](f32x16* sn, int t0, unsigned long long vmask) {
    const bool need = vmask != ~0ull || wave_pmin < t0 + kKT - 1 || row0 + 31 >= C ||
                      (a.window > 0 && t0 <= wave_pmax - a.window);
    if (!need) return;
    // Bit kl: key t0 + kl is attended by this lane's query row.
    unsigned long long m = vmask & low_bits(row_ok ? my_pos - t0 + 1 : 0);
    if (a.window > 0) m &= ~low_bits(my_pos - a.window + 1 - t0) | low_bits(a.sinks - t0);
    m >>= 4 * hf;  // the lane's keys: kh*32 + 8*(v/4) + 4*hf + v%4
    const uint32_t mh[2] = {(uint32_t)m, (uint32_t)(m >> 32)};
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sn[kh][v] = (mh[kh] >> (8 * (v >> 2) + (v & 3))) & 1 ? sn[kh][v] : -INFINITY;
  };

  // Phase Y: O^T += V^T.P^T of the current tile (V in stage vst), with the
  // next tile's row maximum (if any) between the MFMAs. V^T fragments of
  // chunk c+1 are read while chunk c multiplies.
  float m8[8];
  auto max_part = [&](const f32x16* sn, int j) {
    if (j < 8)
      m8[j] = fmaxf(fmaxf(sn[j >> 2][4 * (j & 3)], sn[j >> 2][4 * (j & 3) + 1]),
                    fmaxf(sn[j >> 2][4 * (j & 3) + 2], sn[j >> 2][4 * (j & 3) + 3]));
    else if (j == 8)
      m8[0] = fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3]));
    else if (j == 9)
      m8[4] = fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7]));
  };
  auto phase_y = [&](const f32x16* sn, auto wn, int vst, int gi, int gst) {
    constexpr bool with_next = decltype(wn)::value;
    const uint32_t vb = lds_offset(v_lds + vst * TILE);
    u32x2 e03[2][DT], e47[2][DT];
    auto rd = [&](auto cc, int slot) {
      constexpr int c = decltype(cc)::value;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        e03[slot][dt] = lds_read_tr<16 * c * D * 2>(vb + tr_addr[dt]);
        e47[slot][dt] = lds_read_tr<(16 * c + 8) * D * 2>(vb + tr_addr[dt]);
      }
    };
    // The 10 parts of the maximum spread over the 4 * DT MFMAs.
    constexpr int PPM = (10 + 4 * DT - 1) / (4 * DT);
    auto mm = [&](auto cc, auto sl) {
      constexpr int c = decltype(cc)::value, slot = decltype(sl)::value;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        settle(e03[slot][dt]);
        settle(e47[slot][dt]);
      }
      const P8 bw = __builtin_bit_cast(P8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const P8 av = __builtin_bit_cast(P8, u32x4{e03[slot][dt].x, e03[slot][dt].y, e47[slot][dt].x,
                                                     e47[slot][dt].y});
        o[dt] = MP::mma(av, bw, o[dt]);
        if constexpr (with_next) {
#pragma unroll
          for (int k = 0; k < PPM; ++k) max_part(sn, (4 * c + dt) * PPM + k);
        }
      }
    };
    rd(IntC<0>{}, 0);
    rd(IntC<1>{}, 1);
    lds_wait_n<2 * DT>();
    mm(IntC<0>{}, IntC<0>{});
    // The direct loads of tile gi (if any) into stage gst, and the table
    // entries of the tile after it.
    if (gi < ntiles) {
      vm2 = key_mask(tile_t0(gi));
      gather(gst, vm2);
      if (gi + 1 < ntiles) fetch(tile_t0(gi + 1));
    }
    rd(IntC<2>{}, 0);
    lds_wait_n<2 * DT>();
    mm(IntC<1>{}, IntC<1>{});
    rd(IntC<3>{}, 1);
    lds_wait_n<2 * DT>();
    mm(IntC<2>{}, IntC<0>{});
    lds_wait_n<0>();
    mm(IntC<3>{}, IntC<1>{});
  };
  // Reference maximum after the next tile's maximum: moves only when some
  // row's maximum exceeds it by more than kSlackLog2 (weights then stay at
  // most 2^kSlackLog2); the output rescale, exact either way, is rare.
  auto update_max = [&]() {
    float mt = fmaxf(m8[0], m8[4]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mt),
                                                     __builtin_bit_cast(uint32_t, mt), false, false);
    mt = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    mt *= scale_log2;
    if (__any(mt > m_run + kSlackLog2)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (mn == -INFINITY ? 0.f : mn));
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m_run = mn;
    }
    ms = m_run == -INFINITY ? 0.f : m_run;
  };

  // Prologue: tiles 0, 1 and 2 requested, tiles 0 and 1 waited for, tile 0's
  // V converted, tile 3's table entries requested. Key masks rotate with the
  // iterations: on entry to iteration i, vm0, vm1 and vm3 hold those of
  // tiles i, i+1 and i+2; phase Y puts tile i+3's in vm2.
  fetch(tile_t0(0));
  vm0 = key_mask(tile_t0(0));
  gather(0, vm0);
  if (ntiles > 1) {
    fetch(tile_t0(1));
    vm1 = key_mask(tile_t0(1));
    gather(1, vm1);
  }
  if (ntiles > 2) {
    fetch(tile_t0(2));
    vm3 = key_mask(tile_t0(2));
    gather(2, vm3);
  }
  if (ntiles > 3) fetch(tile_t0(3));
  if (ntiles > 2)
    vm_wait<2 * NLD>();
  else
    vm_wait<0>();
  cv_read(0);
  lds_wait_n<0>();
  cv_convert();
  cv_write();
  lds_wait_n<0>();
  __syncthreads();

  f32x16 sA[2], sB[2];
  {
    const uint32_t kb = lds_offset(k_lds);
    sA[0] = f32x16{};
    sA[1] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const u32x4 k0 = lds_read16<0>(kaddr(kb, kc));
      const u32x4 k1 = lds_read16<32 * D * 2>(kaddr(kb, kc));
      u32x4 x0 = k0, x1 = k1;
      lds_wait_n<0>();
      settle(x0);
      settle(x1);
      sA[0] = M::mma(__builtin_bit_cast(V8, x0), qf[kc], sA[0]);
      sA[1] = M::mma(__builtin_bit_cast(V8, x1), qf[kc], sA[1]);
    }
    mask(sA, tile_t0(0), vm0);
#pragma unroll
    for (int j = 0; j < 10; ++j) max_part(sA, j);
    update_max();
  }

  // Iteration i with the current tile's scores in sc and the next tile's
  // going to sn; stage of tile i is st. Tile i+1's V is converted in phase
  // X; tile i+3's loads are issued in phase Y (into the stage tile i-1
  // held); at the end every thread waits for its loads of tile i+2 (issued
  // one iteration earlier), and one barrier publishes both.
  // has_next: compile-time (i + 1 < ntiles), so that the steady iterations
  // carry no test of it.
  auto iteration = [&](int i, int st, const f32x16* sc, f32x16* sn, auto hn) {
    constexpr bool has_next = decltype(hn)::value;
    const int st1 = (st + 1) & (NST - 1);
    const int st3 = (st + 3) & (NST - 1);
    vm2 = 0;
    if constexpr (has_next) {
      phase_x(sc, sn, st1, true, st1);
      mask(sn, tile_t0(i + 1), vm1);
    } else {
      weights_only(sc);
    }
    // phase_y sets vm2 to the key mask of tile i+3 when it gathers it
    phase_y(sn, hn, st, i + 3, st3);
    if constexpr (has_next) update_max();
    if (i + 3 < ntiles)
      vm_wait<2 * NLD>();
    else
      vm_wait<0>();
    lds_wait_n<0>();
    __syncthreads();
    vm0 = vm1;
    vm1 = vm3;  // tile i+2
    vm3 = vm2;  // tile i+3
    return st1;
  };
  // Iteration i takes the scores of tile i from sA (i even) or sB (i odd).
  int st = 0, i = 0;
  for (; i + 2 < ntiles; i += 2) {
    st = iteration(i, st, sA, sB, IntC<1>{});
    st = iteration(i + 1, st, sB, sA, IntC<1>{});
  }
  if (i + 1 < ntiles) {
    st = iteration(i, st, sA, sB, IntC<1>{});
    iteration(i + 1, st, sB, sA, IntC<0>{});
  } else {
    iteration(i, st, sA, sB, IntC<0>{});
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* op = a.out + ((size_t)(r0 + my_row) * a.H + hq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int d = dt * 32 + 8 * v4 + 4 * hf;
      float4 w = make_float4(o[dt][4 * v4] * inv, o[dt][4 * v4 + 1] * inv, o[dt][4 * v4 + 2] * inv,
                             o[dt][4 * v4 + 3] * inv);
      *reinterpret_cast<float4*>(op + d) = w;
    }
  }
  if (a.lse) {
    if (hf == 0)
      a.lse[(size_t)(r0 + my_row) * a.H + hq] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <class T, int D, int B, int G>
static hipError_t launch_typed(const PrefillArgs& a, hipStream_t st) {
  PrefillArgs b = a;
  if (a.k_scale) {
    // 8-bit pools: codes widened in the kernel, row scales.
    constexpr int NW = 8;
    constexpr int HPW = G < NW ? G : NW;
    constexpr int QT = 32 * (NW / HPW);
    b.grid_q = (a.max_q_len + QT - 1) / QT;
    b.grid_y = a.Hkv * (G / HPW);
    const long long n = (long long)b.grid_q * b.grid_y * a.S;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    if (a.code_dtype == 3)
      hipLaunchKernelGGL((prefill_kernel_q8<T, I8T, D, B, G, NW>), dim3((unsigned)n), dim3(64 * NW), 0, st, b,
                         a.scale * kLog2e);
    else if (a.code_dtype == 4)
      hipLaunchKernelGGL((prefill_kernel_q8<T, FP8T, D, B, G, NW>), dim3((unsigned)n), dim3(64 * NW), 0, st, b,
                         a.scale * kLog2e);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  constexpr int NW = 8;
  constexpr int HPW = G < NW ? G : NW;
  constexpr int QT = 32 * (NW / HPW);
  b.grid_q = (a.max_q_len + QT - 1) / QT;
  b.grid_y = a.Hkv * (G / HPW);
  const long long n = (long long)b.grid_q * b.grid_y * a.S;
  if (n > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<T, D, B, G>), dim3((unsigned)n), dim3(64 * NW), 0, st, b, a.scale * kLog2e);
  return hipGetLastError();
}

template <class T, int D, int B>
static hipError_t by_group(const PrefillArgs& a, hipStream_t st) {
  switch (a.H / a.Hkv) {
    case 1: return launch_typed<T, D, B, 1>(a, st);
    case 2: return launch_typed<T, D, B, 2>(a, st);
    case 4: return launch_typed<T, D, B, 4>(a, st);
    case 8: return launch_typed<T, D, B, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <class T, int D>
static hipError_t by_block(const PrefillArgs& a, hipStream_t st) {
  switch (a.B) {
    case 16: return by_group<T, D, 16>(a, st);
    case 32: return by_group<T, D, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

template <class T>
static hipError_t by_dim(const PrefillArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return by_block<T, 64>(a, st);
    case 128: return by_block<T, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

bool prefill_supported(int dtype, int D, int B, int G) {
  return (dtype == 1 || dtype == 2) && (D == 64 || D == 128) && (B == 16 || B == 32) &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 1: return by_dim<F16T>(a, st);
    case 2: return by_dim<BF16T>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
