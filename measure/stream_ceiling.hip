// Same-mix streaming ceiling: a kernel that moves exactly the bytes of the
// shard step (N_d bf16 contribution loads, three in-place fp32 state arrays
// read and written, one bf16 store per element) with trivial integer
// arithmetic, in the step's access pattern: chunks of 512 elements per wave,
// lane l taking the 4-element pieces at 4l and 256 + 4l, so that each cache
// line is fetched by one instruction.  Its bandwidth is what the memory
// system delivers for the step's access mix on this GPU; the step kernel is
// reported as a fraction of it next to the fraction of the 8 TB/s peak.
//
// Measurement infrastructure only: not part of the update, not called by
// the library.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxRanks = 64;

struct MixArgs {
  const uint16_t* g[kMaxRanks];  // N_d arrays of n bf16 values
  uint32_t* s[3];                // 3 arrays of n 32-bit values, updated in place
  uint16_t* p;                   // n bf16 values
  int64_t nchunk;                // n / 512
  int32_t nd;
};

template <bool NT, class T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// POL: cache policy bits (set: non-temporal) 1 = contribution loads,
// 2 = state loads, 4 = stores.
template <int ND, int POL>
__global__ void __launch_bounds__(256) mix_kernel(const MixArgs a) {
  constexpr bool gn = (POL & 1) != 0, sn = (POL & 2) != 0, wn = (POL & 4) != 0;
  const int nd = ND > 0 ? ND : a.nd;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t W = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t c = wave; c < a.nchunk; c += W) {
    const int64_t e0 = (c << 9) + ((threadIdx.x & 63) << 2), e1 = e0 + 256;
    u32x2 acc0 = ld<gn>((const u32x2*)(a.g[0] + e0));
    u32x2 acc1 = ld<gn>((const u32x2*)(a.g[0] + e1));
#pragma unroll 16
    for (int q = 1; q < (ND > 0 ? ND : kMaxRanks); ++q) {
      if (q < nd) {
        acc0 += ld<gn>((const u32x2*)(a.g[q] + e0));
        acc1 += ld<gn>((const u32x2*)(a.g[q] + e1));
      }
    }
    u32x4 x0[3], x1[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      x0[k] = ld<sn>((const u32x4*)(a.s[k] + e0));
      x1[k] = ld<sn>((const u32x4*)(a.s[k] + e1));
    }
    const u32x4 a0 = {acc0.x, acc0.y, acc0.x, acc0.y}, a1 = {acc1.x, acc1.y, acc1.x, acc1.y};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      st<wn>((u32x4*)(a.s[k] + e0), x0[k] + a0);
      st<wn>((u32x4*)(a.s[k] + e1), x1[k] ^ a1);
    }
    st<wn>((u32x2*)(a.p + e0), acc0);
    st<wn>((u32x2*)(a.p + e1), acc1);
  }
}

template <int ND>
void launch_mix(int pol, const MixArgs& a, int blocks, hipStream_t stream) {
  switch (pol) {
    case 1: hipLaunchKernelGGL((mix_kernel<ND, 1>), dim3(blocks), dim3(256), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((mix_kernel<ND, 5>), dim3(blocks), dim3(256), 0, stream, a); break;
    case 7: hipLaunchKernelGGL((mix_kernel<ND, 7>), dim3(blocks), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((mix_kernel<ND, 0>), dim3(blocks), dim3(256), 0, stream, a);
  }
}

// Pure-read stream over the same buffers (every contribution and state
// array read once, same pattern); one store per lane at the end keeps the
// loads.
template <bool NT>
__global__ void __launch_bounds__(256) read_kernel(const MixArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t wave = tid >> 6, W = ((int64_t)gridDim.x * blockDim.x) >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t c = wave; c < a.nchunk; c += W) {
    const int64_t e0 = (c << 9) + ((threadIdx.x & 63) << 2), e1 = e0 + 256;
    for (int q = 0; q < a.nd; ++q) {
      const u32x2 x = ld<NT>((const u32x2*)(a.g[q] + e0)), y = ld<NT>((const u32x2*)(a.g[q] + e1));
      acc.x ^= x.x; acc.y ^= x.y; acc.z ^= y.x; acc.w ^= y.y;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k)
      acc += ld<NT>((const u32x4*)(a.s[k] + e0)) ^ ld<NT>((const u32x4*)(a.s[k] + e1));
  }
  if (tid < (a.nchunk << 6)) st<NT>((u32x4*)(a.p + 8 * tid), acc);
}

// Plain copy of state array 0 into state array 1 (read 4, write 4 bytes per
// element), 16 bytes per lane.
template <bool NT>
__global__ void __launch_bounds__(256) copy_kernel(const MixArgs a) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t nv = a.nchunk << 7;
  const u32x4* src = (const u32x4*)a.s[0];
  u32x4* dst = (u32x4*)a.s[1];
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nv; v += T)
    st<NT>(dst + v, ld<NT>(src + v));
}

}  // namespace

extern "C" {

namespace {
// Fills the arguments; -1 when a size or pointer is unusable.
int make_args(MixArgs& a, const void* const* grads, int32_t nd, void* const* state, void* out,
              int64_t n) {
  if (nd < 1 || nd > kMaxRanks || n < 0 || n % 512 != 0 || !grads || !state || !out) return -1;
  for (int q = 0; q < kMaxRanks; ++q) a.g[q] = q < nd ? (const uint16_t*)grads[q] : nullptr;
  for (int k = 0; k < 3; ++k) a.s[k] = (uint32_t*)state[k];
  a.p = (uint16_t*)out;
  a.nchunk = n / 512;
  a.nd = nd;
  for (int q = 0; q < nd; ++q)
    if (!grads[q] || ((uintptr_t)grads[q] & 15u)) return -1;
  for (int k = 0; k < 3; ++k)
    if (!state[k] || ((uintptr_t)state[k] & 15u)) return -1;
  if ((uintptr_t)out & 15u) return -1;
  return 0;
}
}  // namespace

// grads: host array of nd device pointers to n bf16 values each; state: 3
// device pointers to n floats; out: n bf16 values.  n must be a multiple of
// 512 and every pointer 16-byte aligned.  pol: cache policy, one of 0, 1, 5,
// 7 (bits: 1 contribution loads, 2 state loads, 4 stores non-temporal).
// Returns 0, -1 on bad arguments, -2 on a launch failure.
int stream_ceiling_launch(const void* const* grads, int32_t nd, void* const* state, void* out,
                          int64_t n, int32_t blocks, int32_t pol, hipStream_t stream) {
  MixArgs a;
  if (blocks < 1 || (pol != 0 && pol != 1 && pol != 5 && pol != 7) ||
      make_args(a, grads, nd, state, out, n) != 0)
    return -1;
  if (nd == 8) launch_mix<8>(pol, a, blocks, stream);
  else if (nd == 64) launch_mix<64>(pol, a, blocks, stream);
  else launch_mix<0>(pol, a, blocks, stream);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// kind 0: pure read of every buffer the step reads; kind 1: copy of state
// array 0 into state array 1.  Arguments as for stream_ceiling_launch; nt
// selects non-temporal accesses.
int stream_probe_launch(int32_t kind, const void* const* grads, int32_t nd, void* const* state,
                        void* out, int64_t n, int32_t blocks, int32_t nt, hipStream_t stream) {
  MixArgs a;
  if (kind < 0 || kind > 1 || blocks < 1 || make_args(a, grads, nd, state, out, n) != 0)
    return -1;
  if (kind == 0) {
    if (nt) hipLaunchKernelGGL((read_kernel<true>), dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((read_kernel<false>), dim3(blocks), dim3(256), 0, stream, a);
  } else {
    if (nt) hipLaunchKernelGGL((copy_kernel<true>), dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((copy_kernel<false>), dim3(blocks), dim3(256), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
