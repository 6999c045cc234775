// Same-mix streaming ceiling: a kernel that moves exactly the bytes of the
// shard step (N_d 16-byte contribution loads, three in-place fp32 state
// arrays read and written, one 16-byte bf16 store per 8 elements and lane)
// with trivial integer arithmetic.  Its bandwidth is what the memory system
// delivers for the step's access mix on this GPU; the step kernel is
// reported as a fraction of it next to the fraction of the 8 TB/s peak.
//
// Measurement infrastructure only: not part of the update, not called by
// the library.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxRanks = 64;

struct MixArgs {
  const u32x4* g[kMaxRanks];  // N_d arrays of nvec 16-byte vectors
  u32x4* s[3];                // 3 arrays of 2*nvec vectors, updated in place
  u32x4* p;                   // nvec vectors
  int64_t nvec;
  int32_t nd;
};

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// POL: cache policy bits (set: non-temporal) 1 = contribution loads,
// 2 = state loads, 4 = stores.
template <int ND, int POL>
__global__ void __launch_bounds__(256) mix_kernel(const MixArgs a) {
  constexpr bool gn = (POL & 1) != 0, sn = (POL & 2) != 0, wn = (POL & 4) != 0;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int nd = ND > 0 ? ND : a.nd;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < a.nvec; v += T) {
    u32x4 acc = ld<gn>(a.g[0] + v);
#pragma unroll
    for (int q = 1; q < (ND > 0 ? ND : kMaxRanks); ++q)
      if (q < nd) acc += ld<gn>(a.g[q] + v);
    u32x4 x[6];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      x[2 * k] = ld<sn>(a.s[k] + 2 * v);
      x[2 * k + 1] = ld<sn>(a.s[k] + 2 * v + 1);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      st<wn>(a.s[k] + 2 * v, x[2 * k] + acc);
      st<wn>(a.s[k] + 2 * v + 1, x[2 * k + 1] ^ acc);
    }
    st<wn>(a.p + v, acc);
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
// array read once); one 16-byte store per lane at the end keeps the loads.
template <bool NT>
__global__ void __launch_bounds__(256) read_kernel(const MixArgs a) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t v = tid; v < a.nvec; v += T) {
    for (int q = 0; q < a.nd; ++q) acc ^= ld<NT>(a.g[q] + v);
#pragma unroll
    for (int k = 0; k < 3; ++k) acc += ld<NT>(a.s[k] + 2 * v) ^ ld<NT>(a.s[k] + 2 * v + 1);
  }
  if (tid < a.nvec) st<NT>(a.p + tid, acc);
}

// Plain copy of state array 0 into state array 1 (read 4, write 4 bytes per
// element).
template <bool NT>
__global__ void __launch_bounds__(256) copy_kernel(const MixArgs a) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < 2 * a.nvec; v += T)
    st<NT>(a.s[1] + v, ld<NT>(a.s[0] + v));
}

}  // namespace

extern "C" {

// grads: host array of nd device pointers to n bf16 values each; state: 3
// device pointers to n floats; out: n bf16 values.  n must be a multiple of
// 8 and every pointer 16-byte aligned.  pol: cache policy, one of 0, 1, 5, 7
// (bits: 1 contribution loads, 2 state loads, 4 stores non-temporal).
// Returns 0, -1 on bad arguments, -2 on a launch failure.
int stream_ceiling_launch(const void* const* grads, int32_t nd, void* const* state, void* out,
                          int64_t n, int32_t blocks, int32_t pol, hipStream_t stream) {
  if (nd < 1 || nd > kMaxRanks || n < 0 || n % 8 != 0 || blocks < 1 || !grads || !state || !out ||
      (pol != 0 && pol != 1 && pol != 5 && pol != 7))
    return -1;
  MixArgs a;
  for (int q = 0; q < kMaxRanks; ++q) a.g[q] = q < nd ? (const u32x4*)grads[q] : nullptr;
  for (int k = 0; k < 3; ++k) a.s[k] = (u32x4*)state[k];
  a.p = (u32x4*)out;
  a.nvec = n / 8;
  a.nd = nd;
  for (int q = 0; q < nd; ++q)
    if (!grads[q] || ((uintptr_t)grads[q] & 15u)) return -1;
  for (int k = 0; k < 3; ++k)
    if (!state[k] || ((uintptr_t)state[k] & 15u)) return -1;
  if ((uintptr_t)out & 15u) return -1;
  if (nd == 8) launch_mix<8>(pol, a, blocks, stream);
  else if (nd == 64) launch_mix<64>(pol, a, blocks, stream);
  else launch_mix<0>(pol, a, blocks, stream);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// kind 0: pure read of every buffer the step reads; kind 1: copy of state
// array 0 into state array 1.  Arguments as for stream_ceiling_launch.
int stream_probe_launch(int32_t kind, const void* const* grads, int32_t nd, void* const* state,
                        void* out, int64_t n, int32_t blocks, int32_t nt, hipStream_t stream) {
  if (kind < 0 || kind > 1 || nd < 1 || nd > kMaxRanks || n < 0 || n % 8 != 0 || blocks < 1 ||
      !grads || !state || !out)
    return -1;
  MixArgs a;
  for (int q = 0; q < kMaxRanks; ++q) a.g[q] = q < nd ? (const u32x4*)grads[q] : nullptr;
  for (int k = 0; k < 3; ++k) a.s[k] = (u32x4*)state[k];
  a.p = (u32x4*)out;
  a.nvec = n / 8;
  a.nd = nd;
  for (int q = 0; q < nd; ++q)
    if (!grads[q] || ((uintptr_t)grads[q] & 15u)) return -1;
  for (int k = 0; k < 3; ++k)
    if (!state[k] || ((uintptr_t)state[k] & 15u)) return -1;
  if ((uintptr_t)out & 15u) return -1;
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
