// zero_shard_step: rank-ordered reduction of N_d bf16 contributions, AdamW on
// the fp32 master/m/v shard, bf16 cast and slot (or in-place) store -- one
// streaming pass over the shard.
//
// Page "Infra: Data Parallel" (pufanyi.com), section "Zero Redundancy
// Optimizer (ZeRO)": AdamW is element-wise, so a rank holding a slice of the
// parameters, the averaged gradient of that slice (Reduce-Scatter with
// averaging) and the slice's moments updates it alone, then All-Gathers the
// updated parameters (ZeRO-1/2) or keeps them sharded (ZeRO-3).  Knowledge
// card "FSDP" (kongchang.com), Core Facts: the float accumulation order of a
// reduction depends on the parallel configuration, so it is fixed here to
// ascending rank order.
//
// Design (gfx950): the step is a pure HBM stream, 2*N_d + 26 bytes per shard
// element with no reuse, so it is written as a grid-stride loop in which each
// lane moves 8 elements per iteration with 128-bit non-temporal loads and
// stores (one 16-byte load per rank, two per fp32 state array).  No LDS, no
// atomics, no MFMA: every output element belongs to exactly one lane, which
// makes the result independent of the launch shape.  Each rank count that
// matters gets its own unrolled instantiation; for large N_d the rank loads
// are issued in groups so that registers stay within budget while enough
// bytes are in flight.
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

// Contribution element type: GT_BF16 (2-byte patterns) or GT_F32.
enum : int { GT_BF16 = 0, GT_F32 = 1 };

template <int NP>
struct StepArgs {
  const void* g[NP];
  float* master;
  float* m;
  float* v;
  uint16_t* pout;
  float* gout;
  Scalars k;
  Region reg;
  float nd_f, inv_nd;
  int32_t nd, pow2, flat_grad, slot_out;
};

// Division by N_d; for a power of two the product with the exact reciprocal
// is the same correctly rounded value (x/2^k and x*2^-k are the same real).
// POW2 > 0: N_d is known at compile time to be a power of two.
template <int POW2, int NP>
__device__ __forceinline__ float average(float a, const StepArgs<NP>& A) {
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

// 8 consecutive contributions of one rank, as loaded (not yet widened).
template <int GT>
struct Raw8;
template <>
struct Raw8<GT_BF16> {
  u32x4 w;
};
template <>
struct Raw8<GT_F32> {
  f32x4 lo, hi;
};

template <int GT, bool NT>
__device__ __forceinline__ Raw8<GT> load8(const void* base, int64_t gi) {
  Raw8<GT> r;
  if constexpr (GT == GT_BF16) {
    r.w = ld_stream<NT>((const u32x4*)((const uint16_t*)base + gi));
  } else {
    r.lo = ld_stream<NT>((const f32x4*)((const float*)base + gi));
    r.hi = ld_stream<NT>((const f32x4*)((const float*)base + gi + 4));
  }
  return r;
}

template <int GT>
__device__ __forceinline__ void widen8(float a[8], const Raw8<GT>& r) {
  if constexpr (GT == GT_BF16) {
    a[0] = bf16_lo(r.w.x); a[1] = bf16_hi(r.w.x);
    a[2] = bf16_lo(r.w.y); a[3] = bf16_hi(r.w.y);
    a[4] = bf16_lo(r.w.z); a[5] = bf16_hi(r.w.z);
    a[6] = bf16_lo(r.w.w); a[7] = bf16_hi(r.w.w);
  } else {
    a[0] = r.lo.x; a[1] = r.lo.y; a[2] = r.lo.z; a[3] = r.lo.w;
    a[4] = r.hi.x; a[5] = r.hi.y; a[6] = r.hi.z; a[7] = r.hi.w;
  }
}

template <int GT>
__device__ __forceinline__ void add8(float a[8], const Raw8<GT>& r) {
  float x[8];
  widen8<GT>(x, r);
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = a[k] + x[k];
}

template <int GT>
__device__ __forceinline__ float load_one(const void* base, int64_t gi) {
  if constexpr (GT == GT_BF16)
    return bf16_one(((const uint16_t*)base)[gi]);
  else
    return ((const float*)base)[gi];
}

// Sum of the N_d contributions of 8 consecutive elements, ascending rank.
// The loads of up to GROUP ranks are issued before their adds.
template <int ND, int GROUP, bool NT, int GT>
__device__ __forceinline__ void reduce8(float acc[8], const StepArgs<ND>& A, int64_t gi) {
  widen8<GT>(acc, load8<GT, NT>(A.g[0], gi));
#pragma unroll
  for (int q0 = 1; q0 < ND; q0 += GROUP) {
    Raw8<GT> w[GROUP];
#pragma unroll
    for (int u = 0; u < GROUP; ++u)
      if (q0 + u < ND) w[u] = load8<GT, NT>(A.g[q0 + u], gi);
#pragma unroll
    for (int u = 0; u < GROUP; ++u)
      if (q0 + u < ND) add8<GT>(acc, w[u]);
  }
}

// Runtime rank count (any N_d up to ZERO_MAX_ND).
template <bool NT, int GT>
__device__ __forceinline__ void reduce8_dyn(float acc[8], const StepArgs<ZERO_MAX_ND>& A,
                                            int64_t gi) {
  widen8<GT>(acc, load8<GT, NT>(A.g[0], gi));
  for (int q = 1; q < A.nd; ++q) add8<GT>(acc, load8<GT, NT>(A.g[q], gi));
}

__device__ __forceinline__ int64_t flat_of(const Region& r, int64_t e) {
  if (e >= r.n0) return r.flat1 + (e - r.n0);
  const int64_t b = e / r.seg;
  return r.flat0 + b * r.pstride + (e - b * r.seg);
}

// One element with generic addressing (tails, the scalar path).
template <int GT, int NP>
__device__ __forceinline__ void step_one(const StepArgs<NP>& A, int64_t e, bool map) {
  const int64_t i = A.reg.i0 + e;
  const int64_t f = map ? flat_of(A.reg, e) : i;
  const int64_t gi = (map && A.flat_grad) ? f : i;
  const int64_t oi = (map && A.slot_out) ? f : i;
  float a = load_one<GT>(A.g[0], gi);
  for (int q = 1; q < A.nd; ++q) a = a + load_one<GT>(A.g[q], gi);
  const float g = average<0>(a, A);
  float th = A.master[i], m = A.m[i], v = A.v[i];
  adamw(g, th, m, v, A.k);
  A.master[i] = th;
  A.m[i] = m;
  A.v[i] = v;
  A.pout[oi] = (uint16_t)bf16_round(th);
  if (A.gout) A.gout[i] = g;
}

// Vector path: 8 elements per lane per iteration, grid-stride over the
// launch.  Requires 16-byte aligned bases and i0 % 8 == 0; when mapping,
// flat0 % 8 == 0 and (part 0 is one bucket, or seg % 8 == 0 and
// pstride % 8 == 0), and if part 1 exists n0 % 8 == 0 and flat1 % 8 == 0, so
// that no vector straddles a bucket and every vector address is aligned.
template <int ND>
using ArgsFor = StepArgs<(ND > 0 ? ND : ZERO_MAX_ND)>;

template <int ND, bool MAP, int GROUP, bool NT, int GT>
__global__ void __launch_bounds__(256) step_vec_kernel(const ArgsFor<ND> A) {
  const int64_t n = A.reg.n;
  const int64_t nv0 = A.reg.n0 >> 3;
  const int64_t nvec = (A.reg.n0 == n) ? nv0 : nv0 + ((n - A.reg.n0) >> 3);
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t adv = T << 3;
  int64_t b = 0, j = 0;
  if (MAP) {
    b = (tid << 3) / A.reg.seg;
    j = (tid << 3) - b * A.reg.seg;
  }
  for (int64_t vi = tid; vi < nvec; vi += T) {
    const int64_t i = A.reg.i0 + (vi << 3);
    int64_t f = i;
    if (MAP) {
      if (vi < nv0) {
        f = A.reg.flat0 + b * A.reg.pstride + j;
        j += adv;
        if (j >= A.reg.seg) {
          const int64_t q = j / A.reg.seg;
          b += q;
          j -= q * A.reg.seg;
        }
      } else {
        f = A.reg.flat1 + ((vi - nv0) << 3);
      }
    }
    const int64_t gi = (MAP && A.flat_grad) ? f : i;
    const int64_t oi = (MAP && A.slot_out) ? f : i;

    float acc[8];
    if constexpr (ND > 0)
      reduce8<ND, GROUP, NT, GT>(acc, A, gi);
    else
      reduce8_dyn<NT, GT>(acc, A, gi);

    const f32x4 th0 = ld_stream<NT>((const f32x4*)(A.master + i));
    const f32x4 th1 = ld_stream<NT>((const f32x4*)(A.master + i + 4));
    const f32x4 m0 = ld_stream<NT>((const f32x4*)(A.m + i));
    const f32x4 m1 = ld_stream<NT>((const f32x4*)(A.m + i + 4));
    const f32x4 v0 = ld_stream<NT>((const f32x4*)(A.v + i));
    const f32x4 v1 = ld_stream<NT>((const f32x4*)(A.v + i + 4));
    float th[8] = {th0.x, th0.y, th0.z, th0.w, th1.x, th1.y, th1.z, th1.w};
    float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float g[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      g[k] = average<((ND & (ND - 1)) == 0 ? ND : 0)>(acc[k], A);
      adamw(g[k], th[k], mm[k], vv[k], A.k);
    }
    st_stream<NT>((f32x4*)(A.master + i), f32x4{th[0], th[1], th[2], th[3]});
    st_stream<NT>((f32x4*)(A.master + i + 4), f32x4{th[4], th[5], th[6], th[7]});
    st_stream<NT>((f32x4*)(A.m + i), f32x4{mm[0], mm[1], mm[2], mm[3]});
    st_stream<NT>((f32x4*)(A.m + i + 4), f32x4{mm[4], mm[5], mm[6], mm[7]});
    st_stream<NT>((f32x4*)(A.v + i), f32x4{vv[0], vv[1], vv[2], vv[3]});
    st_stream<NT>((f32x4*)(A.v + i + 4), f32x4{vv[4], vv[5], vv[6], vv[7]});
    st_stream<NT>((u32x4*)(A.pout + oi),
              u32x4{bf16_pack2(th[0], th[1]), bf16_pack2(th[2], th[3]), bf16_pack2(th[4], th[5]),
                    bf16_pack2(th[6], th[7])});
    if (A.gout) {
      st_stream<NT>((f32x4*)(A.gout + i), f32x4{g[0], g[1], g[2], g[3]});
      st_stream<NT>((f32x4*)(A.gout + i + 4), f32x4{g[4], g[5], g[6], g[7]});
    }
  }
  // the elements after the last full vector, one per lane
  const int64_t tail0 = (nvec == nv0) ? (nv0 << 3) : A.reg.n0 + ((nvec - nv0) << 3);
  if (tid < n - tail0) step_one<GT>(A, tail0 + tid, MAP);
}

template <int GT>
__global__ void __launch_bounds__(256) step_scalar_kernel(const StepArgs<ZERO_MAX_ND> A, int map) {
  const int64_t n = A.reg.n;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += T)
    step_one<GT>(A, e, map != 0);
}

// ------------------------------------------------------------------ host
struct Call {
  const void* const* g;
  int32_t nd, gt;
  float *master, *m, *v, *gout;
  uint16_t* pout;
  Scalars k;
  int32_t flat_grad, slot_out;
};

template <int NP>
void fill_args(StepArgs<NP>& A, const Call& c, const Region& reg) {
  for (int q = 0; q < NP; ++q) A.g[q] = (q < c.nd) ? c.g[q] : nullptr;
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
  A.flat_grad = c.flat_grad;
  A.slot_out = c.slot_out;
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev]) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

constexpr int kDefaultThreads = 256;

// Launch policy, from measurements on MI355X: the read-dominated step
// (64 or more bytes of contributions per element) streams best with
// non-temporal accesses and one 256-thread block per CU; the step with a
// larger write share (small N_d) with ordinary accesses and two blocks per CU.
constexpr bool read_dominated(int nd, int gt) { return nd * (gt == GT_F32 ? 4 : 2) >= 64; }
int default_blocks_per_cu(int nd, int gt) { return read_dominated(nd, gt) ? 1 : 2; }

template <int ND, bool MAP, int GT>
int launch_vec(const Call& c, const Region& reg, int blocks, int threads, hipStream_t s) {
  StepArgs<ND> A;
  fill_args(A, c, reg);
  constexpr int GROUP = (ND > 16) ? 16 : (ND > 1 ? ND - 1 : 1);
  hipLaunchKernelGGL((step_vec_kernel<ND, MAP, GROUP, read_dominated(ND, GT), GT>), dim3(blocks),
                     dim3(threads), 0, s, A);
  return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
}

template <bool MAP, int GT>
int dispatch_vec_gt(const Call& c, const Region& reg, int blocks, int threads, hipStream_t s) {
  switch (c.nd) {
    case 2: return launch_vec<2, MAP, GT>(c, reg, blocks, threads, s);
    case 4: return launch_vec<4, MAP, GT>(c, reg, blocks, threads, s);
    case 8: return launch_vec<8, MAP, GT>(c, reg, blocks, threads, s);
    case 16: return launch_vec<16, MAP, GT>(c, reg, blocks, threads, s);
    case 32: return launch_vec<32, MAP, GT>(c, reg, blocks, threads, s);
    case 64: return launch_vec<64, MAP, GT>(c, reg, blocks, threads, s);
    default: {
      StepArgs<ZERO_MAX_ND> A;
      fill_args(A, c, reg);
      if (read_dominated(c.nd, GT))
        hipLaunchKernelGGL((step_vec_kernel<0, MAP, 1, true, GT>), dim3(blocks), dim3(threads), 0,
                           s, A);
      else
        hipLaunchKernelGGL((step_vec_kernel<0, MAP, 1, false, GT>), dim3(blocks), dim3(threads), 0,
                           s, A);
      return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
    }
  }
}

template <bool MAP>
int dispatch_vec(const Call& c, const Region& reg, int blocks, int threads, hipStream_t s) {
  return c.gt == GT_F32 ? dispatch_vec_gt<MAP, GT_F32>(c, reg, blocks, threads, s)
                        : dispatch_vec_gt<MAP, GT_BF16>(c, reg, blocks, threads, s);
}

int launch_scalar(const Call& c, const Region& reg, bool map, int blocks, int threads,
                  hipStream_t s) {
  StepArgs<ZERO_MAX_ND> A;
  fill_args(A, c, reg);
  if (c.gt == GT_F32)
    hipLaunchKernelGGL(step_scalar_kernel<GT_F32>, dim3(blocks), dim3(threads), 0, s, A,
                       map ? 1 : 0);
  else
    hipLaunchKernelGGL(step_scalar_kernel<GT_BF16>, dim3(blocks), dim3(threads), 0, s, A,
                       map ? 1 : 0);
  return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
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

}  // namespace

extern "C" {

int zero_step_scalars(const zero_adamw* hp, int64_t t, float out[8]) {
  if (!hp || !out || t < 1 || !hp_ok(*hp)) return ZERO_EINVAL;
  const Scalars k = make_scalars(*hp, t);
  out[0] = k.s; out[1] = k.rho; out[2] = k.a_wd; out[3] = k.B1;
  out[4] = k.C1; out[5] = k.B2; out[6] = k.C2; out[7] = k.E;
  return ZERO_OK;
}

int zero_shard_step_ex(const zero_layout* L, const zero_adamw* hp, int64_t t,
                       const void* const* rank_grads, int32_t grad_layout, float* master,
                       float* exp_avg, float* exp_avg_sq, uint16_t* param_out, int32_t out_mode,
                       float* reduced_grad_out, const zero_step_options* opt,
                       hipStream_t stream) {
  if (!L || !hp || !rank_grads || t < 1 || !hp_ok(*hp)) return ZERO_EINVAL;
  if (grad_layout != ZERO_GRAD_COMPACT && grad_layout != ZERO_GRAD_FLAT) return ZERO_EINVAL;
  if (out_mode != ZERO_OUT_AG_SLOT && out_mode != ZERO_OUT_SHARD) return ZERO_EINVAL;
  int threads = kDefaultThreads, blocks_cap = 0, path = 0, gt = GT_BF16;
  if (opt) {
    if (opt->grad_dtype != ZERO_DTYPE_BF16 && opt->grad_dtype != ZERO_DTYPE_F32)
      return ZERO_EINVAL;
    gt = opt->grad_dtype == ZERO_DTYPE_F32 ? GT_F32 : GT_BF16;
    if (opt->threads > 0) threads = opt->threads;
    if (opt->blocks > 0) blocks_cap = opt->blocks;
    path = opt->path;
    if (threads % 64 != 0 || threads > 256 || (path != 0 && path != 1)) return ZERO_EINVAL;
  }
  const int32_t nd = L->n_d;
  const int64_t S = L->S, P = L->P;
  if (S == 0) return ZERO_OK;
  if (!master || !exp_avg || !exp_avg_sq || !param_out) return ZERO_EINVAL;
  for (int32_t q = 0; q < nd; ++q)
    if (!rank_grads[q]) return ZERO_EINVAL;

  // outputs must not overlap each other or any input
  const int64_t gbytes = (gt == GT_F32 ? 4 : 2) * (grad_layout == ZERO_GRAD_FLAT ? P : S);
  const Span outs[5] = {span(master, 4 * S), span(exp_avg, 4 * S), span(exp_avg_sq, 4 * S),
                        span(param_out, 2 * (out_mode == ZERO_OUT_AG_SLOT ? P : S)),
                        span(reduced_grad_out, reduced_grad_out ? 4 * S : 0)};
  for (int a = 0; a < 5; ++a) {
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(outs[a], outs[b])) return ZERO_EOVERLAP;
    for (int32_t q = 0; q < nd; ++q)
      if (overlaps(outs[a], span(rank_grads[q], gbytes))) return ZERO_EOVERLAP;
  }

  Call c;
  c.g = rank_grads;
  c.nd = nd;
  c.gt = gt;
  c.master = master;
  c.m = exp_avg;
  c.v = exp_avg_sq;
  c.gout = reduced_grad_out;
  c.pout = param_out;
  c.k = make_scalars(*hp, t);
  c.flat_grad = grad_layout == ZERO_GRAD_FLAT;
  c.slot_out = out_mode == ZERO_OUT_AG_SLOT;
  const bool map = c.flat_grad || c.slot_out;

  bool aligned = aligned16(master) && aligned16(exp_avg) && aligned16(exp_avg_sq) &&
                 aligned16(param_out) && (!reduced_grad_out || aligned16(reduced_grad_out));
  for (int32_t q = 0; q < nd; ++q) aligned = aligned && aligned16(rank_grads[q]);
  const int cap = blocks_cap > 0 ? blocks_cap : cu_count() * default_blocks_per_cu(nd, gt);
  const bool allow_vec = path == 0 && aligned;

  // Launch plan.  Without flat addressing the shard is one plain range.
  // With it: part 0 = the full buckets, part 1 = the last bucket; one vector
  // launch covers both when every vector address is aligned, otherwise the
  // parts that are not aligned go to the scalar kernel.
  std::vector<Region> regs;
  std::vector<bool> vec;
  const int64_t r = L->rank;
  if (map && !L->fixed()) {
    // per-parameter (dim-0) layout: every tensor is its own bucket; one
    // single-bucket launch per non-empty slice
    for (int64_t b = 0; b < L->nb; ++b) {
      const int64_t sl = L->bucket_slice(b);
      if (sl == 0) continue;
      const int64_t i0 = L->bucket_shard_off(b), f0 = L->bucket_padded_off(b) + r * sl;
      regs.push_back(Region{i0, sl, sl, sl, 0, f0, 0});
      vec.push_back(allow_vec && i0 % 8 == 0 && f0 % 8 == 0);
    }
  } else if (!map) {
    regs.push_back(Region{0, S, S, S, 0, 0, 0});
    vec.push_back(allow_vec);
  } else if (L->nb == 1 || L->s_last == L->s_full) {
    const bool one = L->nb == 1;
    regs.push_back(Region{0, S, S, L->s_full, L->p_full, r * L->s_full, 0});
    vec.push_back(allow_vec && (r * L->s_full) % 8 == 0 &&
                  (one || (L->s_full % 8 == 0 && L->p_full % 8 == 0)));
  } else {
    const int64_t n0 = (L->nb - 1) * L->s_full;
    const int64_t flat1 = (L->nb - 1) * L->p_full + r * L->s_last;
    const bool v0 = allow_vec && L->s_full % 8 == 0 && L->p_full % 8 == 0;
    const bool v1 = allow_vec && flat1 % 8 == 0;
    if (v0 && v1) {
      regs.push_back(Region{0, n0, S, L->s_full, L->p_full, r * L->s_full, flat1});
      vec.push_back(true);
    } else if (v0) {
      regs.push_back(Region{0, n0, n0, L->s_full, L->p_full, r * L->s_full, 0});
      vec.push_back(true);
      regs.push_back(Region{n0, L->s_last, L->s_last, L->s_last, L->p_last, flat1, 0});
      vec.push_back(false);
    } else {
      regs.push_back(Region{0, n0, S, L->s_full, L->p_full, r * L->s_full, flat1});
      vec.push_back(false);
    }
  }

  for (size_t k = 0; k < regs.size(); ++k) {
    const Region& R = regs[k];
    if (R.n <= 0) continue;
    int rc;
    if (vec[k]) {
      const int64_t work = std::max<int64_t>(R.n >> 3, 8);
      const int blocks =
          (int)std::max<int64_t>(1, std::min<int64_t>((work + threads - 1) / threads, cap));
      rc = map ? dispatch_vec<true>(c, R, blocks, threads, stream)
               : dispatch_vec<false>(c, R, blocks, threads, stream);
    } else {
      const int blocks =
          (int)std::max<int64_t>(1, std::min<int64_t>((R.n + threads - 1) / threads, cap));
      rc = launch_scalar(c, R, map, blocks, threads, stream);
    }
    if (rc != ZERO_OK) return rc;
  }
  return ZERO_OK;
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
