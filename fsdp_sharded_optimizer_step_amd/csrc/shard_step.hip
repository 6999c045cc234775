// zero_shard_step: rank-ordered reduction of N_d gradient contributions,
// AdamW on the fp32 master/m/v shard, bf16 cast and slot (or in-place) store
// -- one streaming pass over the shard.
//
// Page "Infra: Data Parallel" (pufanyi.com), section "Zero Redundancy
// Optimizer (ZeRO)": AdamW is element-wise, so a rank holding a slice of the
// parameters, the averaged gradient of that slice (Reduce-Scatter with
// averaging) and the slice's moments updates it alone, then All-Gathers the
// updated parameters (ZeRO-1/2) or keeps them sharded (ZeRO-3).  Section
// "Naive Data Parallelism": with no_sync the micro-batch gradients are summed
// locally, each scaled by 1/n_micro; the last of these sums can be folded
// into the step (zero_shard_step_accumulate).  Knowledge card "FSDP"
// (kongchang.com), Core Facts: the float accumulation order of a reduction
// depends on the parallel configuration, so it is fixed here to ascending
// rank order.
//
// Design (gfx950): the step is a pure HBM stream (2*N_d + 26 bytes per shard
// element for bf16 contributions) with no reuse, so it is written as a
// grid-stride loop over chunks of 512 elements per wave, each lane moving
// two 4-element pieces per chunk, laid out so that every load and store
// instruction of a wave covers whole cache lines (8-byte bf16 and 16-byte
// fp32 accesses); the cache hint (non-temporal or not) per stream and the
// blocks per CU follow measurements.  No LDS, no atomics, no MFMA: every output
// element belongs to exactly one lane, which makes the result independent of
// the launch shape.  Each rank count that matters gets its own unrolled
// instantiation; for large N_d the rank loads are issued in groups so that
// registers stay within budget while enough bytes are in flight.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <vector>

#include "device_common.hpp"
#include "layout.hpp"
#include "zero_shard.h"

namespace {
using namespace zs;

struct Scalars {
  float s, rho, a_wd, B1, C1, B2, C2, E;
};

// The shard range [i0, i0 + n) of one launch and its flat addresses (used for
// FLAT contributions and All-Gather slot stores).  Part 0, the first n0
// elements, is a run of equal buckets:
//   flat(e) = flat0 + b*pstride + j,  b = e / seg,  j = e - b*seg   (e < n0)
// part 1, the rest, lies in a single (last, shorter) bucket:
//   flat(e) = flat1 + (e - n0)                                        (e >= n0)
struct Region {
  int64_t i0, n0, n, seg, pstride, flat0, flat1;
};

// What a rank hands to the reduction:
//   GT_BF16      bf16 contributions (2 bytes per element and rank)
//   GT_F32       binary32 contributions (4)
//   GT_ACC_BF16  the last no_sync micro-batch folded in: the rank's fp32
//                accumulator plus its scaled bf16 micro-batch gradient,
//                rounded to bf16 as the rank would send it (6)
//   GT_ACC_F32   the same sum kept in binary32 (6)
enum : int { GT_BF16 = 0, GT_F32 = 1, GT_ACC_BF16 = 2, GT_ACC_F32 = 3 };
constexpr bool fused(int gt) { return gt >= GT_ACC_BF16; }
constexpr int contrib_bytes(int gt) { return gt == GT_BF16 ? 2 : (gt == GT_F32 ? 4 : 6); }

// Largest rank count of the runtime-N_d instantiation: the pointer arrays
// travel as kernel arguments.
constexpr int kMaxNdFused = ZERO_MAX_ND_FUSED;

template <int NP, bool FUSED>
struct StepArgs {
  const void* g[NP];              // contributions, or (fused) micro-batch gradients
  const float* a[FUSED ? NP : 1];  // fused: the ranks' fp32 accumulators
  float* master;
  float* m;
  float* v;
  uint16_t* pout;
  float* gout;
  Scalars k;
  Region reg;
  float nd_f, inv_nd, acc_scale;
  int32_t nd, pow2, flat_grad, slot_out;
};

template <int ND, int GT>
using ArgsFor =
    StepArgs<(ND > 0 ? ND : (fused(GT) ? kMaxNdFused : ZERO_MAX_ND)), fused(GT)>;

// Division by N_d; for a power of two the product with the exact reciprocal
// is the same correctly rounded value (x/2^k and x*2^-k are the same real).
// POW2 > 0: N_d is known at compile time to be a power of two.
template <int POW2, class Args>
__device__ __forceinline__ float average(float a, const Args& A) {
  if constexpr (POW2 > 0)
    return a * A.inv_nd;
  else
    return A.pow2 ? a * A.inv_nd : a / A.nd_f;
}

// The AdamW element update, binary32, one rounding per operation.
__device__ __forceinline__ void adamw(float g, float& th, float& m, float& v, const Scalars& k) {
  const float m1 = k.B1 * m + k.C1 * g;
  const float v1 = k.B2 * v + k.C2 * (g * g);
  const float d = __builtin_sqrtf(v1) * k.rho + k.E;
  th = k.a_wd * th - k.s * (m1 / d);
  m = m1;
  v = v1;
}

// 8 contributions of one rank, two pieces of 4 consecutive elements (a:
// elements 0-3, b: elements 4-7), as loaded (not yet widened).
template <int GT>
struct Raw8 {
  f32x4 lo, hi;  // fused: the accumulator
  u32x4 w;       // fused: the micro-batch gradient
};
template <>
struct Raw8<GT_BF16> {
  u32x4 w;
};
template <>
struct Raw8<GT_F32> {
  f32x4 lo, hi;
};

// Cache policy of a launch (bit set: non-temporal): the contribution loads,
// the master / m / v loads, and every store.
enum : int { NT_CONTRIB = 1, NT_STATE = 2, NT_STORE = 4 };

// Pieces at contribution indices ga and gb (multiples of 4).
template <int GT, int NT, class Args>
__device__ __forceinline__ Raw8<GT> load8(const Args& A, int q, int64_t ga, int64_t gb) {
  constexpr bool nt = (NT & NT_CONTRIB) != 0;
  Raw8<GT> r;
  if constexpr (GT == GT_F32) {
    r.lo = ld_stream<nt>((const f32x4*)((const float*)A.g[q] + ga));
    r.hi = ld_stream<nt>((const f32x4*)((const float*)A.g[q] + gb));
  } else {
    if constexpr (fused(GT)) {
      r.lo = ld_stream<nt>((const f32x4*)(A.a[q] + ga));
      r.hi = ld_stream<nt>((const f32x4*)(A.a[q] + gb));
    }
    const u32x2 a = ld_stream<nt>((const u32x2*)((const uint16_t*)A.g[q] + ga));
    const u32x2 b = ld_stream<nt>((const u32x2*)((const uint16_t*)A.g[q] + gb));
    r.w = u32x4{a.x, a.y, b.x, b.y};
  }
  return r;
}

// A fused contribution: acc + scale*g (product and sum rounded once each, the
// no_sync accumulation's add), then for GT_ACC_BF16 the bf16 rounding.
template <int GT>
__device__ __forceinline__ float fold(float acc, float g, float scale) {
  const float c = acc + scale * g;
  if constexpr (GT == GT_ACC_BF16)
    return __uint_as_float(bf16_round(c) << 16);
  else
    return c;
}

template <int GT, class Args>
__device__ __forceinline__ void widen8(float x[8], const Raw8<GT>& r, const Args& A) {
  if constexpr (GT == GT_BF16) {
    x[0] = bf16_lo(r.w.x); x[1] = bf16_hi(r.w.x);
    x[2] = bf16_lo(r.w.y); x[3] = bf16_hi(r.w.y);
    x[4] = bf16_lo(r.w.z); x[5] = bf16_hi(r.w.z);
    x[6] = bf16_lo(r.w.w); x[7] = bf16_hi(r.w.w);
  } else if constexpr (GT == GT_F32) {
    x[0] = r.lo.x; x[1] = r.lo.y; x[2] = r.lo.z; x[3] = r.lo.w;
    x[4] = r.hi.x; x[5] = r.hi.y; x[6] = r.hi.z; x[7] = r.hi.w;
  } else {
    const float s = A.acc_scale;
    x[0] = fold<GT>(r.lo.x, bf16_lo(r.w.x), s); x[1] = fold<GT>(r.lo.y, bf16_hi(r.w.x), s);
    x[2] = fold<GT>(r.lo.z, bf16_lo(r.w.y), s); x[3] = fold<GT>(r.lo.w, bf16_hi(r.w.y), s);
    x[4] = fold<GT>(r.hi.x, bf16_lo(r.w.z), s); x[5] = fold<GT>(r.hi.y, bf16_hi(r.w.z), s);
    x[6] = fold<GT>(r.hi.z, bf16_lo(r.w.w), s); x[7] = fold<GT>(r.hi.w, bf16_hi(r.w.w), s);
  }
}

template <int GT, class Args>
__device__ __forceinline__ void add8(float acc[8], const Raw8<GT>& r, const Args& A) {
  float x[8];
  widen8<GT>(x, r, A);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = acc[k] + x[k];
}

template <int GT, class Args>
__device__ __forceinline__ float load_one(const Args& A, int q, int64_t gi) {
  if constexpr (GT == GT_BF16)
    return bf16_one(((const uint16_t*)A.g[q])[gi]);
  else if constexpr (GT == GT_F32)
    return ((const float*)A.g[q])[gi];
  else
    return fold<GT>(A.a[q][gi], bf16_one(((const uint16_t*)A.g[q])[gi]), A.acc_scale);
}

// Sum of the N_d contributions of NPAIR pairs of pieces (8 elements per
// pair), ascending rank.  The loads of up to GROUP ranks (every pair) are
// issued before their adds.  The fused contributions at large N_d keep the
// group loop rolled: fully unrolled, the scheduler hoists loads of later
// groups and spills.
template <int ND, int GROUP, int NT, int GT, int NPAIR>
__device__ __forceinline__ void reduce_pairs(float (&acc)[NPAIR][8], const ArgsFor<ND, GT>& A,
                                             const int64_t (&gp)[2 * NPAIR]) {
#pragma unroll
  for (int h = 0; h < NPAIR; ++h)
    widen8<GT>(acc[h], load8<GT, NT>(A, 0, gp[2 * h], gp[2 * h + 1]), A);
  if constexpr (fused(GT) && ND > 16) {
#pragma unroll 1
    for (int q0 = 1; q0 < ND; q0 += GROUP) {
      Raw8<GT> w[GROUP][NPAIR];
#pragma unroll
      for (int u = 0; u < GROUP; ++u)
        if (q0 + u < ND)
#pragma unroll
          for (int h = 0; h < NPAIR; ++h) w[u][h] = load8<GT, NT>(A, q0 + u, gp[2 * h], gp[2 * h + 1]);
#pragma unroll
      for (int u = 0; u < GROUP; ++u)
        if (q0 + u < ND)
#pragma unroll
          for (int h = 0; h < NPAIR; ++h) add8<GT>(acc[h], w[u][h], A);
    }
    return;
  }
#pragma unroll
  for (int q0 = 1; q0 < ND; q0 += GROUP) {
    Raw8<GT> w[GROUP][NPAIR];
#pragma unroll
    for (int u = 0; u < GROUP; ++u)
      if (q0 + u < ND)
#pragma unroll
        for (int h = 0; h < NPAIR; ++h) w[u][h] = load8<GT, NT>(A, q0 + u, gp[2 * h], gp[2 * h + 1]);
#pragma unroll
    for (int u = 0; u < GROUP; ++u)
      if (q0 + u < ND)
#pragma unroll
        for (int h = 0; h < NPAIR; ++h) add8<GT>(acc[h], w[u][h], A);
  }
}


// Software-pipelined form for many ranks: rank 0 travels with the first
// group, and the loads of group k+1 are issued before the adds of group k,
// so two groups are in flight while the adds stay in ascending rank order
// (otherwise every group ends with the wave's memory queue drained).
// Measured on the tuned Llama-70B buffers (N_d = 64, library builds timed
// alternately): 28.60-28.62 ms against 28.77-28.79 ms; also issuing the
// master / m / v loads with the first group gained nothing (28.74-28.79 ms).
template <int ND, int GROUP, int NT, int GT, int NPAIR>
__device__ __forceinline__ void reduce_pairs_pipe(float (&acc)[NPAIR][8], const ArgsFor<ND, GT>& A,
                                                  const int64_t (&gp)[2 * NPAIR]) {
  constexpr int NG = (ND - 1 + GROUP - 1) / GROUP;
  Raw8<GT> r0[NPAIR];
  Raw8<GT> w[2][GROUP][NPAIR];
#pragma unroll
  for (int h = 0; h < NPAIR; ++h) r0[h] = load8<GT, NT>(A, 0, gp[2 * h], gp[2 * h + 1]);
#pragma unroll
  for (int u = 0; u < GROUP; ++u)
    if (1 + u < ND)
#pragma unroll
      for (int h = 0; h < NPAIR; ++h) w[0][u][h] = load8<GT, NT>(A, 1 + u, gp[2 * h], gp[2 * h + 1]);
#pragma unroll
  for (int h = 0; h < NPAIR; ++h) widen8<GT>(acc[h], r0[h], A);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g + 1 < NG) {
#pragma unroll
      for (int u = 0; u < GROUP; ++u) {
        const int q = 1 + (g + 1) * GROUP + u;
        if (q < ND)
#pragma unroll
          for (int h = 0; h < NPAIR; ++h)
            w[(g + 1) & 1][u][h] = load8<GT, NT>(A, q, gp[2 * h], gp[2 * h + 1]);
      }
    }
#pragma unroll
    for (int u = 0; u < GROUP; ++u) {
      const int q = 1 + g * GROUP + u;
      if (q < ND)
#pragma unroll
        for (int h = 0; h < NPAIR; ++h) add8<GT>(acc[h], w[g & 1][u][h], A);
    }
    // keeps the next group's loads from being hoisted further up
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Runtime rank count.
template <int NT, int GT, int NPAIR>
__device__ __forceinline__ void reduce_pairs_dyn(float (&acc)[NPAIR][8], const ArgsFor<0, GT>& A,
                                                 const int64_t (&gp)[2 * NPAIR]) {
#pragma unroll
  for (int h = 0; h < NPAIR; ++h)
    widen8<GT>(acc[h], load8<GT, NT>(A, 0, gp[2 * h], gp[2 * h + 1]), A);
  for (int q = 1; q < A.nd; ++q)
#pragma unroll
    for (int h = 0; h < NPAIR; ++h)
      add8<GT>(acc[h], load8<GT, NT>(A, q, gp[2 * h], gp[2 * h + 1]), A);
}

__device__ __forceinline__ int64_t flat_of(const Region& r, int64_t e) {
  if (e >= r.n0) return r.flat1 + (e - r.n0);
  const int64_t b = e / r.seg;
  return r.flat0 + b * r.pstride + (e - b * r.seg);
}

// One element: shard index i, contribution index gi, output index oi.
template <int GT, class Args>
__device__ __forceinline__ void step_at(const Args& A, int64_t i, int64_t gi, int64_t oi) {
  float a = load_one<GT>(A, 0, gi);
  for (int q = 1; q < A.nd; ++q) a = a + load_one<GT>(A, q, gi);
  const float g = average<0>(a, A);
  float th = A.master[i], m = A.m[i], v = A.v[i];
  adamw(g, th, m, v, A.k);
  A.master[i] = th;
  A.m[i] = m;
  A.v[i] = v;
  A.pout[oi] = (uint16_t)bf16_round(th);
  if (A.gout) A.gout[i] = g;
}

// Up to 8 elements in two pieces (piece k: cnt[k] <= 4 consecutive elements
// from shard index i[k], contribution index gi[k], output index oi[k]), the
// arithmetic of step_at with every load issued before the first store, so
// that a lane waits for memory once rather than once per element: the ends
// of table regions, where a tile holds only part of a chunk.
template <int ND, int GT, class Args>
__device__ __forceinline__ void step_upto8(const Args& A, const int64_t (&i)[2],
                                           const int64_t (&gi)[2], const int64_t (&oi)[2],
                                           const int (&cnt)[2]) {
  float a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    a[e] = (e & 3) < cnt[e >> 2] ? load_one<GT>(A, 0, gi[e >> 2] + (e & 3)) : 0.0f;
  if constexpr (ND > 0) {
    constexpr int kUnroll = ND <= 16 ? ND : 4;
#pragma unroll kUnroll
    for (int q = 1; q < ND; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((e & 3) < cnt[e >> 2]) a[e] = a[e] + load_one<GT>(A, q, gi[e >> 2] + (e & 3));
  } else {
    for (int q = 1; q < A.nd; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((e & 3) < cnt[e >> 2]) a[e] = a[e] + load_one<GT>(A, q, gi[e >> 2] + (e & 3));
  }
  float th[8], m[8], v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if ((e & 3) < cnt[e >> 2]) {
      const int64_t x = i[e >> 2] + (e & 3);
      th[e] = A.master[x];
      m[e] = A.m[x];
      v[e] = A.v[x];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if ((e & 3) < cnt[e >> 2]) {
      const int64_t x = i[e >> 2] + (e & 3);
      const float g = average<0>(a[e], A);
      adamw(g, th[e], m[e], v[e], A.k);
      A.master[x] = th[e];
      A.m[x] = m[e];
      A.v[x] = v[e];
      A.pout[oi[e >> 2] + (e & 3)] = (uint16_t)bf16_round(th[e]);
      if (A.gout) A.gout[x] = g;
    }
  }
}

// Element e of the launch's Region, generic addressing (tails, scalar path).
template <int GT, class Args>
__device__ __forceinline__ void step_one(const Args& A, int64_t e, bool map) {
  const int64_t i = A.reg.i0 + e;
  const int64_t f = map ? flat_of(A.reg, e) : i;
  step_at<GT>(A, i, (map && A.flat_grad) ? f : i, (map && A.slot_out) ? f : i);
}

// 2*NPAIR pieces of 4 consecutive elements: piece k at shard index ip[k],
// contribution index gp[k], output index op[k] (all multiples of 4 on
// 16-byte aligned bases: 16-byte fp32 and 8-byte bf16 accesses).  Every
// load of the pieces is issued before the first store.
template <int ND, int GROUP, int NT, int GT, int NPAIR>
__device__ __forceinline__ void step_pieces(const ArgsFor<ND, GT>& A,
                                            const int64_t (&ip)[2 * NPAIR],
                                            const int64_t (&gp)[2 * NPAIR],
                                            const int64_t (&op)[2 * NPAIR]) {
  constexpr int NPC = 2 * NPAIR;
  float acc[NPAIR][8];
  if constexpr (ND >= 64 && GT == GT_BF16 && NPAIR == 2 && ND - 1 > GROUP)
    reduce_pairs_pipe<ND, GROUP, NT, GT, NPAIR>(acc, A, gp);
  else if constexpr (ND > 0)
    reduce_pairs<ND, GROUP, NT, GT, NPAIR>(acc, A, gp);
  else
    reduce_pairs_dyn<NT, GT, NPAIR>(acc, A, gp);

  constexpr bool nts = (NT & NT_STATE) != 0, ntw = (NT & NT_STORE) != 0;
  f32x4 th[NPC], mm[NPC], vv[NPC];
#pragma unroll
  for (int k = 0; k < NPC; ++k) th[k] = ld_stream<nts>((const f32x4*)(A.master + ip[k]));
#pragma unroll
  for (int k = 0; k < NPC; ++k) mm[k] = ld_stream<nts>((const f32x4*)(A.m + ip[k]));
#pragma unroll
  for (int k = 0; k < NPC; ++k) vv[k] = ld_stream<nts>((const f32x4*)(A.v + ip[k]));
  f32x4 g[NPC];
#pragma unroll
  for (int k = 0; k < NPC; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gk = average<((ND & (ND - 1)) == 0 ? ND : 0)>(acc[k >> 1][4 * (k & 1) + e], A);
      float t = th[k][e], m = mm[k][e], v = vv[k][e];
      adamw(gk, t, m, v, A.k);
      th[k][e] = t;
      mm[k][e] = m;
      vv[k][e] = v;
      g[k][e] = gk;
    }
  }
#pragma unroll
  for (int k = 0; k < NPC; ++k) st_stream<ntw>((f32x4*)(A.master + ip[k]), th[k]);
#pragma unroll
  for (int k = 0; k < NPC; ++k) st_stream<ntw>((f32x4*)(A.m + ip[k]), mm[k]);
#pragma unroll
  for (int k = 0; k < NPC; ++k) st_stream<ntw>((f32x4*)(A.v + ip[k]), vv[k]);
#pragma unroll
  for (int k = 0; k < NPC; ++k)
    st_stream<ntw>((u32x2*)(A.pout + op[k]),
                   u32x2{bf16_pack2(th[k].x, th[k].y), bf16_pack2(th[k].z, th[k].w)});
  if (A.gout) {
#pragma unroll
    for (int k = 0; k < NPC; ++k) st_stream<ntw>((f32x4*)(A.gout + ip[k]), g[k]);
  }
}

// Moves a piece's bucket coordinates (b, j) forward by adv elements.
__device__ __forceinline__ void advance(int64_t& b, int64_t& j, int64_t adv, int64_t seg) {
  j += adv;
  if (j >= seg) {
    const int64_t q = j / seg;
    b += q;
    j -= q * seg;
  }
}

// Vector path over one Region, grid-stride over chunks of 512*NPAIR
// elements per wave: in each chunk, lane l takes the 4-element pieces at
// 256*k + 4l (k < 2*NPAIR), so that every load and store instruction of the
// wave covers one contiguous span (1 KB of fp32, 512 bytes of bf16) and each
// cache line is fetched by one instruction.  Requires 16-byte aligned bases
// and i0 % 4 == 0; when mapping, flat0 % 4 == 0 and (part 0 is one bucket,
// or seg % 4 == 0 and pstride % 4 == 0), and if part 1 exists n0 % 4 == 0
// and flat1 % 4 == 0, so that no piece straddles a bucket and every piece
// address is aligned.  The elements after the last full chunk run one per
// thread.
template <int ND, bool MAP, int GROUP, int NT, int GT, int NPAIR>
__global__ void __launch_bounds__(256) step_vec_kernel(const ArgsFor<ND, GT> A) {
  static_assert(NPAIR == 1 || NPAIR == 2 || NPAIR == 4, "chunk of 512, 1024 or 2048 elements");
  constexpr int NPC = 2 * NPAIR;
  constexpr int LOG_CH = NPAIR == 1 ? 9 : (NPAIR == 2 ? 10 : 11);
  const Region& R = A.reg;
  const int64_t n = R.n;
  const int64_t nchunk = n >> LOG_CH;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t wave = tid >> 6, W = T >> 6, adv = W << LOG_CH;
  int64_t e0 = (wave << LOG_CH) + ((threadIdx.x & 63) << 2);
  int64_t bk[NPC], jk[NPC];
#pragma unroll
  for (int k = 0; k < NPC; ++k) {
    bk[k] = 0;
    jk[k] = 0;
    if (MAP) {
      bk[k] = (e0 + 256 * k) / R.seg;
      jk[k] = e0 + 256 * k - bk[k] * R.seg;
    }
  }
  const bool fg = MAP && A.flat_grad, so = MAP && A.slot_out;
  for (int64_t c = wave; c < nchunk; c += W, e0 += adv) {
    int64_t ip[NPC], gp[NPC], op[NPC];
#pragma unroll
    for (int k = 0; k < NPC; ++k) {
      const int64_t e = e0 + 256 * k;
      ip[k] = R.i0 + e;
      int64_t f = ip[k];
      if (MAP) {
        f = e < R.n0 ? R.flat0 + bk[k] * R.pstride + jk[k] : R.flat1 + (e - R.n0);
        advance(bk[k], jk[k], adv, R.seg);
      }
      gp[k] = fg ? f : ip[k];
      op[k] = so ? f : ip[k];
    }
    step_pieces<ND, GROUP, NT, GT, NPAIR>(A, ip, gp, op);
  }
  for (int64_t e = (nchunk << LOG_CH) + tid; e < n; e += T) step_one<GT>(A, e, MAP);
}

// Many single-bucket regions in one launch (the per-parameter layout, where
// every tensor is its own bucket).  The regions of one launch are
// consecutive non-empty slices, so they tile one shard range: region k
// covers shard [i_base + e0[k], i_base + e0[k+1]) and flat [f0[k], f0[k] +
// its length).  The work is cut into tiles of blockDim.x*8 elements; blocks
// take tiles grid-stride and find a tile's region by binary search over the
// tile prefix sums, so a 38.6M-element embedding and 96-element norm slices
// share one launch without idle blocks.  Within a tile, each wave takes 512
// elements in the chunk mapping of step_vec_kernel.  Regions whose shard or
// flat start is not a multiple of 4 (or every region, when a base pointer is
// not 16-byte aligned) run element by element.  20 bytes per region: a launch
// takes as many regions as fit next to the kernel's other arguments in
// 4 KB (191 for bf16 contributions at N_d = 8).
template <int CAP>
struct TableT {
  int64_t i_base;
  int64_t e0[CAP + 1];
  int64_t f0[CAP];
  uint32_t tile0[CAP + 1];  // first tile of each region; tile0[count] = total
  int32_t count;
  int32_t vec_ok;  // base pointers 16-byte aligned and the vector path allowed
};
constexpr int kHostTableCap = 192;
// tiles per launch stay below 2^30, so that tile + gridDim.x fits 32 bits
constexpr int64_t kMaxTableTiles = (int64_t)1 << 30;

template <int ND, int GT>
constexpr int table_cap_of() {
  constexpr int64_t room = (4096 - (int64_t)sizeof(ArgsFor<ND, GT>) - 40) / 20;
  return (int)(room < kHostTableCap ? room : kHostTableCap);
}
template <int ND, int GT>
using TableFor = TableT<table_cap_of<ND, GT>()>;
using HostTable = TableT<kHostTableCap>;

template <int ND, int GROUP, int NT, int GT>
__global__ void __launch_bounds__(256) step_table_kernel(const ArgsFor<ND, GT> A,
                                                         const TableFor<ND, GT> T) {
  const int64_t span = (int64_t)blockDim.x << 3;
  const uint32_t total = T.tile0[T.count];
  for (uint32_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = T.count;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (T.tile0[mid] <= tile) lo = mid;
      else hi = mid;
    }
    const int64_t r0 = T.i_base + T.e0[lo], f0 = T.f0[lo];
    const int64_t n = T.e0[lo + 1] - T.e0[lo];
    // the pieces of this lane in the tile: each wave takes 512 elements
    const int64_t ea = (int64_t)(tile - T.tile0[lo]) * span + ((threadIdx.x >> 6) << 9) +
                       ((threadIdx.x & 63) << 2);
    const int64_t eb = ea + 256;
    if (ea >= n) continue;
    const int64_t ia = r0 + ea, fa = f0 + ea, ib = r0 + eb, fb = f0 + eb;
    const int64_t ga = A.flat_grad ? fa : ia, oa = A.slot_out ? fa : ia;
    const int64_t gb = A.flat_grad ? fb : ib, ob = A.slot_out ? fb : ib;
    if (T.vec_ok && ((r0 | f0) & 3) == 0 && eb + 4 <= n) {
      const int64_t ip[2] = {ia, ib}, gp[2] = {ga, gb}, op[2] = {oa, ob};
      step_pieces<ND, GROUP, NT, GT, 1>(A, ip, gp, op);
    } else {
      const int64_t ip[2] = {ia, ib}, gp[2] = {ga, gb}, op[2] = {oa, ob};
      const int cnt[2] = {(int)(n - ea < 4 ? n - ea : 4),
                          (int)(n - eb <= 0 ? 0 : (n - eb < 4 ? n - eb : 4))};
      step_upto8<ND, GT>(A, ip, gp, op, cnt);
    }
  }
}

template <int GT>
__global__ void __launch_bounds__(256) step_scalar_kernel(const ArgsFor<0, GT> A, int map) {
  const int64_t n = A.reg.n;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += T)
    step_one<GT>(A, e, map != 0);
}

// ------------------------------------------------------------------ host
struct Call {
  const void* const* g;
  const float* const* a;  // fused only
  int32_t nd, gt;
  float acc_scale;
  float *master, *m, *v, *gout;
  uint16_t* pout;
  Scalars k;
  int32_t flat_grad, slot_out;
};

template <class Args>
void fill_args(Args& A, const Call& c, const Region& reg) {
  constexpr int NP = sizeof(A.g) / sizeof(A.g[0]);
  constexpr int NA = sizeof(A.a) / sizeof(A.a[0]);
  for (int q = 0; q < NP; ++q) A.g[q] = (q < c.nd) ? c.g[q] : nullptr;
  for (int q = 0; q < NA; ++q) A.a[q] = (c.a && q < c.nd) ? c.a[q] : nullptr;
  A.master = c.master;
  A.m = c.m;
  A.v = c.v;
  A.pout = c.pout;
  A.gout = c.gout;
  A.k = c.k;
  A.reg = reg;
  A.nd = c.nd;
  A.nd_f = (float)c.nd;
  A.pow2 = (c.nd & (c.nd - 1)) == 0;
  A.inv_nd = 1.0f / (float)c.nd;
  A.acc_scale = c.acc_scale;
  A.flat_grad = c.flat_grad;
  A.slot_out = c.slot_out;
}

// Compute units of the current device, cached per device (relaxed atomics:
// concurrent callers may both query, and store the same value).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Launch policy, from measurements on MI355X (Llama-3-8B and Llama-70B
// shards, buffers placed by zero_placement_plan): one 256-thread block per
// CU, except one 192-thread block per CU for the flat-addressed kernel over
// bf16 contributions at N_d = 8 and two 128-thread blocks per CU for fp32
// contributions that are not read-dominated (64 or more bytes of
// contributions per element); the cache policy and the chunk size below.
constexpr bool read_dominated(int nd, int gt) { return nd * contrib_bytes(gt) >= 64; }
// Cache policy, measured on the tuned llama8b / llama70b buffers (every
// policy and launch shape, N_d = 8 to 64): with each cache line fetched by a
// single instruction (the chunk mapping of step_vec_kernel), non-temporal
// loads and stores of every stream are best for bf16 contributions (2-3 %
// over ordinary state loads) and whenever the contributions dominate the
// bytes; for fp32 or accumulator contributions at small N_d, non-temporal
// contribution loads with ordinary state accesses.
constexpr int cache_policy(int nd, int gt) {
  return (gt == GT_BF16 || read_dominated(nd, gt)) ? NT_CONTRIB | NT_STATE | NT_STORE
                                                   : NT_CONTRIB;
}
// Pairs of 4-element pieces per lane and chunk of the vector kernel, and
// the ranks whose loads are in flight together.  Measured on the tuned
// llama8b / llama70b buffers (same pool, library builds timed alternately):
// at N_d = 64 with bf16 contributions, chunks of 1024 elements per wave
// (each rank's run 2 KB per wave) with 8 ranks in flight take 28.76 ms
// against 29.05 ms for 512-element chunks with 16 ranks; at N_d = 8 the two
// are equal (6.74 ms) and 2048-element chunks are slower (10.8 ms).  The
// fused loads are 12 dwords per rank: 8 ranks in flight, or they spill at
// N_d = 64.
constexpr int step_pairs(int nd, int gt) { return (gt == GT_BF16 && nd >= 64) ? 2 : 1; }
constexpr int step_group_max(int gt, int pairs) { return (fused(gt) || pairs > 1) ? 8 : 16; }
struct Policy {
  int blocks_per_cu, threads;
};
// The vector kernel with flat addressing (All-Gather slot output or FLAT
// contributions) over bf16 contributions at N_d = 8 takes one 192-thread
// block per CU (three waves): measured against 256 threads on the tuned
// buffers, Llama-3-8B 6.62-6.64 against 6.67-6.68 ms and faster at each of
// nine pool starts (by 0.1-1.2 %); accum1p3b 1.075 against 1.087 ms; GPT-2
// 0.1068 against 0.1077 ms.  Elsewhere three waves were slower: the same
// kernel at N_d = 4, 16 and 32 (2-17 %), the in-place form without flat
// addressing at N_d = 8 (the per-parameter Llama-3-8B shard, 7.41 against
// 6.74 ms), the per-parameter table launches (6.86 against 6.63 ms), N_d =
// 64 (1.7 %) and fp32 or accumulator contributions at N_d = 8.
Policy default_policy(int nd, int gt, bool flat_vec) {
  if (gt == GT_F32 && !read_dominated(nd, gt)) return Policy{2, 128};
  if (flat_vec && gt == GT_BF16 && nd == 8) return Policy{1, 192};
  return Policy{1, 256};
}

// What one launch covers: a Region (affine addressing, with or without the
// flat map) or a Table of single-bucket regions.
enum : int { K_PLAIN = 0, K_MAP = 1, K_TABLE = 2 };
struct Work {
  const Region* reg;
  const HostTable* tab;
  int blocks, threads;
};

template <int GT>
int table_cap_gt(int nd) {
  switch (nd) {
    case 2: return table_cap_of<2, GT>();
    case 4: return table_cap_of<4, GT>();
    case 8: return table_cap_of<8, GT>();
    case 16: return table_cap_of<16, GT>();
    case 32: return table_cap_of<32, GT>();
    case 64: return table_cap_of<64, GT>();
    default: return table_cap_of<0, GT>();
  }
}
// Regions per table launch for this rank count and contribution type.
int table_cap(int nd, int gt) {
  switch (gt) {
    case GT_F32: return table_cap_gt<GT_F32>(nd);
    case GT_ACC_BF16: return table_cap_gt<GT_ACC_BF16>(nd);
    case GT_ACC_F32: return table_cap_gt<GT_ACC_F32>(nd);
    default: return table_cap_gt<GT_BF16>(nd);
  }
}

template <int ND, int GT, int KIND, int NT>
int launch_nt(const Call& c, const Work& w, hipStream_t s) {
  ArgsFor<ND, GT> A;
  fill_args(A, c, w.reg ? *w.reg : Region{0, 0, 0, 1, 0, 0, 0});
  // the table kernel takes one pair per lane
  constexpr int NPAIR = KIND == K_TABLE ? 1 : step_pairs(ND, GT);
  constexpr int GMAX = step_group_max(GT, NPAIR);
  constexpr int GROUP = ND > GMAX ? GMAX : (ND > 1 ? ND - 1 : 1);
  if constexpr (KIND == K_TABLE) {
    using Tab = TableFor<ND, GT>;
    static_assert(sizeof(ArgsFor<ND, GT>) + sizeof(Tab) <= 4096, "kernel arguments");
    Tab T;
    const int n = w.tab->count;
    if (n < 1 || n > table_cap_of<ND, GT>()) return ZERO_EINVAL;  // planner invariant
    T.i_base = w.tab->i_base;
    for (int k = 0; k < n; ++k) T.f0[k] = w.tab->f0[k];
    for (int k = 0; k <= n; ++k) {
      T.e0[k] = w.tab->e0[k];
      T.tile0[k] = w.tab->tile0[k];
    }
    T.count = n;
    T.vec_ok = w.tab->vec_ok;
    hipLaunchKernelGGL((step_table_kernel<ND, GROUP, NT, GT>), dim3(w.blocks), dim3(w.threads), 0,
                       s, A, T);
  } else {
    hipLaunchKernelGGL((step_vec_kernel<ND, KIND == K_MAP, GROUP, NT, GT, NPAIR>),
                       dim3(w.blocks), dim3(w.threads), 0, s, A);
  }
  return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
}

template <int ND, int GT, int KIND>
int launch(const Call& c, const Work& w, hipStream_t s) {
  if constexpr (ND > 0)
    return launch_nt<ND, GT, KIND, cache_policy(ND, GT)>(c, w, s);
  else
    return read_dominated(c.nd, GT)
               ? launch_nt<0, GT, KIND, cache_policy(ZERO_MAX_ND, GT)>(c, w, s)
               : launch_nt<0, GT, KIND, cache_policy(1, GT)>(c, w, s);
}

template <int GT, int KIND>
int dispatch_nd(const Call& c, const Work& w, hipStream_t s) {
  switch (c.nd) {
    case 2: return launch<2, GT, KIND>(c, w, s);
    case 4: return launch<4, GT, KIND>(c, w, s);
    case 8: return launch<8, GT, KIND>(c, w, s);
    case 16: return launch<16, GT, KIND>(c, w, s);
    case 32: return launch<32, GT, KIND>(c, w, s);
    case 64: return launch<64, GT, KIND>(c, w, s);
    default: return launch<0, GT, KIND>(c, w, s);
  }
}

template <int KIND>
int dispatch(const Call& c, const Work& w, hipStream_t s) {
  switch (c.gt) {
    case GT_F32: return dispatch_nd<GT_F32, KIND>(c, w, s);
    case GT_ACC_BF16: return dispatch_nd<GT_ACC_BF16, KIND>(c, w, s);
    case GT_ACC_F32: return dispatch_nd<GT_ACC_F32, KIND>(c, w, s);
    default: return dispatch_nd<GT_BF16, KIND>(c, w, s);
  }
}

template <int GT>
int launch_scalar_gt(const Call& c, const Region& reg, bool map, int blocks, int threads,
                     hipStream_t s) {
  ArgsFor<0, GT> A;
  fill_args(A, c, reg);
  hipLaunchKernelGGL(step_scalar_kernel<GT>, dim3(blocks), dim3(threads), 0, s, A, map ? 1 : 0);
  return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
}

int launch_scalar(const Call& c, const Region& reg, bool map, int blocks, int threads,
                  hipStream_t s) {
  switch (c.gt) {
    case GT_F32: return launch_scalar_gt<GT_F32>(c, reg, map, blocks, threads, s);
    case GT_ACC_BF16: return launch_scalar_gt<GT_ACC_BF16>(c, reg, map, blocks, threads, s);
    case GT_ACC_F32: return launch_scalar_gt<GT_ACC_F32>(c, reg, map, blocks, threads, s);
    default: return launch_scalar_gt<GT_BF16>(c, reg, map, blocks, threads, s);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, int64_t bytes) {
  return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool hp_ok(const zero_adamw& hp) {
  return std::isfinite(hp.lr) && std::isfinite(hp.eps) && std::isfinite(hp.weight_decay) &&
         std::isfinite(hp.beta1) && std::isfinite(hp.beta2) && hp.beta1 >= 0.0 &&
         hp.beta1 < 1.0 && hp.beta2 >= 0.0 && hp.beta2 < 1.0;
}

// Per-call scalars: binary64, each rounded once to binary32.
Scalars make_scalars(const zero_adamw& hp, int64_t t) {
  const double bc1 = 1.0 - std::pow(hp.beta1, (double)t);
  const double bc2 = 1.0 - std::pow(hp.beta2, (double)t);
  Scalars k;
  k.s = (float)(hp.lr / bc1);
  k.rho = (float)(1.0 / std::sqrt(bc2));
  k.a_wd = (float)(1.0 - hp.lr * hp.weight_decay);
  k.B1 = (float)hp.beta1;
  k.C1 = (float)(1.0 - hp.beta1);
  k.B2 = (float)hp.beta2;
  k.C2 = (float)(1.0 - hp.beta2);
  k.E = (float)hp.eps;
  return k;
}

struct LaunchShape {
  int threads = 0, blocks_cap = 0, path = 0;  // 0: the policy's choice
};

int parse_options(const zero_step_options* opt, LaunchShape& ls) {
  if (!opt) return ZERO_OK;
  if (opt->threads > 0) ls.threads = opt->threads;
  if (opt->blocks > 0) ls.blocks_cap = opt->blocks;
  ls.path = opt->path;
  if (ls.threads % 64 != 0 || ls.threads > 256 || (ls.path != 0 && ls.path != 1))
    return ZERO_EINVAL;
  return ZERO_OK;
}

// Validates everything common to the step entry points, plans the launches
// and enqueues them.  `ins`/`in_bytes`: the contribution buffers of every
// rank (two per rank when fused), each of in_bytes bytes.
// Buckets [b0, b1) of the layout are updated (all of them for the
// whole-shard entry points); buffers are always the full-size ones.
int run_step(const zero_layout* L, const zero_adamw* hp, int64_t t, Call c, int32_t grad_layout,
             int32_t out_mode, const LaunchShape& ls, const void* const* ins, int n_ins,
             const int64_t* in_bytes, int64_t b0, int64_t b1, hipStream_t stream) {
  if (grad_layout != ZERO_GRAD_COMPACT && grad_layout != ZERO_GRAD_FLAT) return ZERO_EINVAL;
  if (out_mode != ZERO_OUT_AG_SLOT && out_mode != ZERO_OUT_SHARD) return ZERO_EINVAL;
  if (b0 < 0 || b1 > L->nb || b0 > b1) return ZERO_ERANGE;
  const int32_t nd = L->n_d;
  const int64_t S = L->S, P = L->P;
  if (S == 0 || b0 == b1) return ZERO_OK;
  if (!c.master || !c.m || !c.v || !c.pout) return ZERO_EINVAL;
  for (int q = 0; q < n_ins; ++q)
    if (!ins[q]) return ZERO_EINVAL;

  // outputs must not overlap each other or any input
  const Span outs[5] = {span(c.master, 4 * S), span(c.m, 4 * S), span(c.v, 4 * S),
                        span(c.pout, 2 * (out_mode == ZERO_OUT_AG_SLOT ? P : S)),
                        span(c.gout, c.gout ? 4 * S : 0)};
  for (int a = 0; a < 5; ++a) {
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(outs[a], outs[b])) return ZERO_EOVERLAP;
    for (int q = 0; q < n_ins; ++q)
      if (overlaps(outs[a], span(ins[q], in_bytes[q]))) return ZERO_EOVERLAP;
  }

  if (hip_error_pending()) return ZERO_EHIP;

  c.nd = nd;
  c.k = make_scalars(*hp, t);
  c.flat_grad = grad_layout == ZERO_GRAD_FLAT;
  c.slot_out = out_mode == ZERO_OUT_AG_SLOT;
  const bool map = c.flat_grad || c.slot_out;

  bool aligned = aligned16(c.master) && aligned16(c.m) && aligned16(c.v) && aligned16(c.pout) &&
                 (!c.gout || aligned16(c.gout));
  for (int q = 0; q < n_ins; ++q) aligned = aligned && aligned16(ins[q]);
  // the flat-addressed vector launches of a bucketed layout may take their
  // own shape; table launches and the plain vector kernel take the default
  const bool flat_vec = map && L->fixed();
  const Policy pol = default_policy(nd, c.gt, flat_vec);
  const int threads = ls.threads > 0 ? ls.threads : pol.threads;
  const int cap = ls.blocks_cap > 0 ? ls.blocks_cap : cu_count() * pol.blocks_per_cu;
  const bool allow_vec = ls.path == 0 && aligned;
  const int64_t r = L->rank;

  if (map && !L->fixed()) {
    // per-parameter (dim-0) layout: every tensor is its own bucket; the
    // non-empty slices, consecutive in the shard, go to table launches of
    // up to table_cap(nd, gt) regions
    const int64_t span_e = (int64_t)threads * 8;
    for (int64_t b = b0; b < b1; ++b)
      if ((L->bucket_slice(b) + span_e - 1) / span_e >= kMaxTableTiles) return ZERO_ERANGE;
    const int tcap = table_cap(nd, c.gt);
    // blocks of a table launch, measured with 256 threads on tuned pools:
    // a launch of up to 64 tiles per CU is latency-bound (each block does one
    // chunk per wave between region look-ups) and runs fastest with 16
    // blocks per CU (GPT-2, 148 tensors, 7.6K tiles: 0.111 ms against 0.121
    // with two and 0.133 with one); larger launches are bandwidth-bound and
    // run fastest with one block per CU, as the vector kernel does (one
    // Llama-3-8B layer, 13K tiles: equal; four layers: 0.737 ms against 0.763
    // with two; the whole model: 6.70 ms against 7.13)
    const int cus = cu_count();
    HostTable T;
    T.count = 0;
    T.vec_ok = allow_vec ? 1 : 0;
    auto flush = [&]() -> int {
      if (T.count == 0) return ZERO_OK;
      const int64_t total = T.tile0[T.count];
      // in waves per CU: 64 for small launches, 4 for large ones (one
      // 256-thread block, or two 128-thread blocks for fp32 contributions)
      const int64_t waves_per_cu = total <= (int64_t)64 * cus ? 64 : 4;
      const int64_t tblocks =
          ls.blocks_cap > 0 ? ls.blocks_cap
                            : (int64_t)cus * std::max<int64_t>(1, waves_per_cu / (threads / 64));
      const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(total, tblocks));
      const Work w{nullptr, &T, blocks, threads};
      const int rc = dispatch<K_TABLE>(c, w, stream);
      T.count = 0;
      return rc;
    };
    for (int64_t b = b0; b < b1; ++b) {
      const int64_t sl = L->bucket_slice(b);
      if (sl == 0) continue;
      const int64_t i0 = L->bucket_shard_off(b), f0 = L->bucket_padded_off(b) + r * sl;
      const int64_t tiles = (sl + span_e - 1) / span_e;
      if (T.count > 0 && (i0 != T.i_base + T.e0[T.count] ||
                          (int64_t)T.tile0[T.count] + tiles >= kMaxTableTiles)) {
        const int rc = flush();
        if (rc != ZERO_OK) return rc;
      }
      if (T.count == 0) {
        T.i_base = i0;
        T.e0[0] = 0;
        T.tile0[0] = 0;
      }
      const int k = T.count;
      T.f0[k] = f0;
      T.e0[k + 1] = T.e0[k] + sl;
      T.tile0[k + 1] = T.tile0[k] + (uint32_t)tiles;
      T.count = k + 1;
      if (T.count == tcap) {
        const int rc = flush();
        if (rc != ZERO_OK) return rc;
      }
    }
    return flush();
  }

  // Without flat addressing the buckets' slices are one plain shard range.
  // With it (bucketed layout): part 0 = the full buckets of the range, part
  // 1 = the last bucket if it is in the range; one vector launch covers both
  // when every vector address is aligned, otherwise the parts that are not
  // aligned go to the scalar kernel.
  std::vector<Region> regs;
  std::vector<bool> vec;
  const int64_t i_begin = L->bucket_shard_off(b0);
  const int64_t i_end = b1 < L->nb ? L->bucket_shard_off(b1) : S;
  const int64_t n_all = i_end - i_begin;
  if (!map) {
    regs.push_back(Region{i_begin, n_all, n_all, n_all, 0, 0, 0});
    vec.push_back(allow_vec && i_begin % 4 == 0);
  } else if (L->nb == 1 || L->s_last == L->s_full) {
    // every bucket has the same slice: one affine part
    const bool one = b1 - b0 == 1;
    const int64_t flat0 = b0 * L->p_full + r * L->s_full;
    regs.push_back(Region{i_begin, n_all, n_all, L->s_full, L->p_full, flat0, 0});
    vec.push_back(allow_vec && i_begin % 4 == 0 && flat0 % 4 == 0 &&
                  (one || (L->s_full % 4 == 0 && L->p_full % 4 == 0)));
  } else {
    const bool has_last = b1 == L->nb;
    const int64_t nf = (has_last ? L->nb - 1 : b1) - b0;  // full buckets in the range
    const int64_t n0 = nf * L->s_full;
    const int64_t flat0 = b0 * L->p_full + r * L->s_full;
    const int64_t flat1 = (L->nb - 1) * L->p_full + r * L->s_last;
    if (nf == 0) {
      // the last bucket alone
      regs.push_back(Region{i_begin, L->s_last, L->s_last, L->s_last, L->p_last, flat1, 0});
      vec.push_back(allow_vec && i_begin % 4 == 0 && flat1 % 4 == 0);
    } else {
      const bool v0 = allow_vec && L->s_full % 4 == 0 && L->p_full % 4 == 0;
      const bool v1 = !has_last || (allow_vec && flat1 % 4 == 0);
      if (v0 && v1) {
        regs.push_back(Region{i_begin, n0, n_all, L->s_full, L->p_full, flat0, flat1});
        vec.push_back(true);
      } else if (v0) {
        regs.push_back(Region{i_begin, n0, n0, L->s_full, L->p_full, flat0, 0});
        vec.push_back(true);
        regs.push_back(Region{i_begin + n0, L->s_last, L->s_last, L->s_last, L->p_last, flat1, 0});
        vec.push_back(false);
      } else {
        regs.push_back(Region{i_begin, n0, n_all, L->s_full, L->p_full, flat0, flat1});
        vec.push_back(false);
      }
    }
  }

  // A small region (one ZeRO-2 bucket) gets up to four blocks per CU, so
  // that each wave takes about one chunk: with one block per CU a 25 MiB
  // bucket's 3,200 chunks leave 3.1 per wave and the last round runs mostly
  // idle.  Measured on the Llama-3-8B shard stepped bucket by bucket (613
  // calls in a HIP graph): 9.22 ms against 10.13 ms on one stream, 6.82 ms
  // against 7.66 ms with the calls alternating between two streams.
  const int64_t small_chunks = (int64_t)16 * cu_count();
  for (size_t k = 0; k < regs.size(); ++k) {
    const Region& R = regs[k];
    if (R.n <= 0) continue;
    int rc;
    if (vec[k]) {
      const int64_t work = std::max<int64_t>(R.n >> 3, 8);
      const int64_t vcap =
          ls.blocks_cap > 0 || (R.n >> 9) > small_chunks ? cap : (int64_t)4 * cu_count();
      const int blocks =
          (int)std::max<int64_t>(1, std::min<int64_t>((work + threads - 1) / threads, vcap));
      const Work w{&R, nullptr, blocks, threads};
      rc = map ? dispatch<K_MAP>(c, w, stream) : dispatch<K_PLAIN>(c, w, stream);
    } else {
      const int blocks =
          (int)std::max<int64_t>(1, std::min<int64_t>((R.n + threads - 1) / threads, cap));
      rc = launch_scalar(c, R, map, blocks, threads, stream);
    }
    if (rc != ZERO_OK) return rc;
  }
  return ZERO_OK;
}

}  // namespace

extern "C" {

int zero_step_scalars(const zero_adamw* hp, int64_t t, float out[8]) {
  if (!hp || !out || t < 1 || !hp_ok(*hp)) return ZERO_EINVAL;
  const Scalars k = make_scalars(*hp, t);
  out[0] = k.s; out[1] = k.rho; out[2] = k.a_wd; out[3] = k.B1;
  out[4] = k.C1; out[5] = k.B2; out[6] = k.C2; out[7] = k.E;
  return ZERO_OK;
}

int zero_shard_step_buckets(const zero_layout* L, const zero_adamw* hp, int64_t t,
                            int64_t bucket_begin, int64_t bucket_end,
                            const void* const* rank_grads, int32_t grad_layout, float* master,
                            float* exp_avg, float* exp_avg_sq, uint16_t* param_out,
                            int32_t out_mode, float* reduced_grad_out,
                            const zero_step_options* opt, hipStream_t stream) {
  if (!L || !hp || !rank_grads || t < 1 || !hp_ok(*hp)) return ZERO_EINVAL;
  int gt = GT_BF16;
  if (opt) {
    if (opt->grad_dtype != ZERO_DTYPE_BF16 && opt->grad_dtype != ZERO_DTYPE_F32)
      return ZERO_EINVAL;
    gt = opt->grad_dtype == ZERO_DTYPE_F32 ? GT_F32 : GT_BF16;
  }
  LaunchShape ls;
  if (parse_options(opt, ls) != ZERO_OK) return ZERO_EINVAL;
  const int64_t n_in = grad_layout == ZERO_GRAD_FLAT ? L->P : L->S;
  std::vector<int64_t> bytes((size_t)L->n_d, contrib_bytes(gt) * n_in);
  Call c{};
  c.g = rank_grads;
  c.a = nullptr;
  c.gt = gt;
  c.acc_scale = 0.0f;
  c.master = master;
  c.m = exp_avg;
  c.v = exp_avg_sq;
  c.gout = reduced_grad_out;
  c.pout = param_out;
  return run_step(L, hp, t, c, grad_layout, out_mode, ls, rank_grads, L->n_d, bytes.data(),
                  bucket_begin, bucket_end, stream);
}

int zero_shard_step_ex(const zero_layout* L, const zero_adamw* hp, int64_t t,
                       const void* const* rank_grads, int32_t grad_layout, float* master,
                       float* exp_avg, float* exp_avg_sq, uint16_t* param_out, int32_t out_mode,
                       float* reduced_grad_out, const zero_step_options* opt,
                       hipStream_t stream) {
  if (!L || !hp || !rank_grads || t < 1 || !hp_ok(*hp)) return ZERO_EINVAL;
  int gt = GT_BF16;
  if (opt) {
    if (opt->grad_dtype != ZERO_DTYPE_BF16 && opt->grad_dtype != ZERO_DTYPE_F32)
      return ZERO_EINVAL;
    gt = opt->grad_dtype == ZERO_DTYPE_F32 ? GT_F32 : GT_BF16;
  }
  LaunchShape ls;
  if (parse_options(opt, ls) != ZERO_OK) return ZERO_EINVAL;
  const int64_t n_in = grad_layout == ZERO_GRAD_FLAT ? L->P : L->S;
  std::vector<int64_t> bytes((size_t)L->n_d, contrib_bytes(gt) * n_in);
  Call c{};
  c.g = rank_grads;
  c.a = nullptr;
  c.gt = gt;
  c.acc_scale = 0.0f;
  c.master = master;
  c.m = exp_avg;
  c.v = exp_avg_sq;
  c.gout = reduced_grad_out;
  c.pout = param_out;
  return run_step(L, hp, t, c, grad_layout, out_mode, ls, rank_grads, L->n_d, bytes.data(), 0,
                  L->nb, stream);
}

int zero_shard_step_accumulate(const zero_layout* L, const zero_adamw* hp, int64_t t,
                               const float* const* rank_acc, const uint16_t* const* rank_micro,
                               float micro_scale, int32_t contrib_dtype, int32_t grad_layout,
                               float* master, float* exp_avg, float* exp_avg_sq,
                               uint16_t* param_out, int32_t out_mode, float* reduced_grad_out,
                               const zero_step_options* opt, hipStream_t stream) {
  if (!L || !hp || !rank_acc || !rank_micro || t < 1 || !hp_ok(*hp)) return ZERO_EINVAL;
  if (contrib_dtype != ZERO_DTYPE_BF16 && contrib_dtype != ZERO_DTYPE_F32) return ZERO_EINVAL;
  if (!std::isfinite(micro_scale)) return ZERO_EINVAL;
  if (L->n_d > ZERO_MAX_ND_FUSED) return ZERO_ERANGE;
  LaunchShape ls;
  if (parse_options(opt, ls) != ZERO_OK) return ZERO_EINVAL;
  const int32_t nd = L->n_d;
  const int64_t n_in = grad_layout == ZERO_GRAD_FLAT ? L->P : L->S;
  std::vector<const void*> ins((size_t)2 * nd);
  std::vector<int64_t> bytes((size_t)2 * nd);
  for (int32_t q = 0; q < nd; ++q) {
    ins[2 * q] = rank_acc[q];
    bytes[2 * q] = 4 * n_in;
    ins[2 * q + 1] = rank_micro[q];
    bytes[2 * q + 1] = 2 * n_in;
  }
  Call c{};
  c.g = (const void* const*)rank_micro;
  c.a = rank_acc;
  c.gt = contrib_dtype == ZERO_DTYPE_F32 ? GT_ACC_F32 : GT_ACC_BF16;
  c.acc_scale = micro_scale;
  c.master = master;
  c.m = exp_avg;
  c.v = exp_avg_sq;
  c.gout = reduced_grad_out;
  c.pout = param_out;
  return run_step(L, hp, t, c, grad_layout, out_mode, ls, ins.data(), 2 * nd, bytes.data(), 0,
                  L->nb, stream);
}

int zero_shard_step(const zero_layout* L, const zero_adamw* hp, int64_t t,
                    const uint16_t* const* rank_grads, int32_t grad_layout, float* master,
                    float* exp_avg, float* exp_avg_sq, uint16_t* param_out, int32_t out_mode,
                    float* reduced_grad_out, hipStream_t stream) {
  return zero_shard_step_ex(L, hp, t, (const void* const*)rank_grads, grad_layout, master,
                            exp_avg, exp_avg_sq, param_out, out_mode, reduced_grad_out, nullptr,
                            stream);
}

}  // extern "C"
