// zero_gather_params and zero_reshard: the two data movements next to the
// step.
//
// Page "Infra: Data Parallel" (pufanyi.com), section "Zero Redundancy
// Optimizer (ZeRO)": under ZeRO-3 every rank keeps only its parameter shard
// and, layer by layer, All-Gathers the full parameters before forward and
// again before backward; under ZeRO-1/2 the updated parameters are
// All-Gathered after the step.  zero_gather_params is the local arithmetic
// of that All-Gather on one GPU: the N_d ranks' bf16 shards are placed into
// their slots of the padded flat buffer.
// Section "Fully Sharded Data Parallel (FSDP)", "Checkpoint": a sharded
// checkpoint holds every rank's shards of the parameters and optimizer
// state, and loading it into a run with a different number of GPUs re-cuts
// the shards to the new layout.  zero_reshard performs that re-cut for one
// state array: from the N_d shards of one bucketed layout to one rank's
// shard of another layout of the same tensor list.
//
// Both are copies: gather moves 4 bytes per flat element, reshard 2 x the
// element size per destination element (2 for bf16, 4 for fp32), plus the
// destination's padding written as zeros.
#include <algorithm>
#include <cstdint>

#include "device_common.hpp"
#include "layout.hpp"
#include "zero_shard.h"

namespace {
using namespace zs;

// Fixed-cut geometry of a layout, by value for the kernels.
struct Geo {
  int64_t cap, nb, s_full, p_full, len_last, s_last;
  int32_t n_d, rank;
};

Geo geo_of(const zero_layout& L) {
  return Geo{L.cap, L.nb, L.s_full, L.p_full, L.len_last, L.s_last, L.n_d, L.rank};
}

// Bucket b of any layout seen as a one-bucket layout of its own (addresses
// relative to the bucket's stream, padded and shard offsets).
Geo geo_of_bucket(const zero_layout& L, int64_t b) {
  const int64_t sl = L.bucket_slice(b), len = L.bucket_len(b);
  return Geo{len > 0 ? len : 1, 1, sl, sl * L.n_d, len, sl, L.n_d, L.rank};
}

__device__ __forceinline__ int64_t slice_len(const Geo& g, int64_t b) {
  return b + 1 < g.nb ? g.s_full : g.s_last;
}
__device__ __forceinline__ int64_t real_len(const Geo& g, int64_t b) {
  return b + 1 < g.nb ? g.cap : g.len_last;
}

// ------------------------------------------------------------------ gather
struct GatherArgs {
  const uint16_t* shard[ZERO_MAX_ND];
  uint16_t* out;
  Geo g;
  int64_t f0, f1;  // flat range [f0, f1) = buckets [b0, b1)
};

// Flat position f -> (bucket, rank q, offset j in the slice).
__device__ __forceinline__ void split_flat(const Geo& g, int64_t f, int64_t& b, int32_t& q,
                                           int64_t& j) {
  b = f / g.p_full;
  if (b >= g.nb) b = g.nb - 1;
  const int64_t w = f - b * g.p_full;
  const int64_t sb = slice_len(g, b);
  q = (int32_t)(w / sb);
  j = w - (int64_t)q * sb;
}

// Vector path: every slice length is a multiple of 8 and every base is
// 16-byte aligned, so 8 consecutive flat elements come from one shard.
__global__ void __launch_bounds__(256) gather_vec_kernel(const GatherArgs A) {
  const int64_t nv = (A.f1 - A.f0) >> 3;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nv; v += T) {
    const int64_t f = A.f0 + (v << 3);
    int64_t b, j;
    int32_t q;
    split_flat(A.g, f, b, q, j);
    const u32x4 x = ld_stream<false>((const u32x4*)(A.shard[q] + b * A.g.s_full + j));
    st_stream<false>((u32x4*)(A.out + f), x);
  }
}

__global__ void __launch_bounds__(256) gather_scalar_kernel(const GatherArgs A) {
  const int64_t n = A.f1 - A.f0;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += T) {
    const int64_t f = A.f0 + e;
    int64_t b, j;
    int32_t q;
    split_flat(A.g, f, b, q, j);
    A.out[f] = A.shard[q][b * A.g.s_full + j];
  }
}

// ------------------------------------------------------------------ reshard
// One launch covers the destination shard indices [i0, i0 + n).  The
// destination index i maps to the stream position
//   x = d_base_x + stream_of(gd, i - d_base_i)     (or padding)
// and, when has_src, the source element is found by
//   locate(gs, x - s_base_x)   if 0 <= x - s_base_x < s_len
// in the source shards (pointers already shifted to the source bucket).
// Padding is written as zero when zero_pads; positions whose stream element
// lies outside this launch's source range are left alone.
struct ReshardArgs {
  const void* src[ZERO_MAX_ND];
  void* dst;
  Geo gs, gd;
  int64_t i0, n, d_base_i, d_base_x, s_base_x, s_len;
  int32_t zero_pads, has_src;
};

// Destination shard index -> stream position (or -1 for padding).
__device__ __forceinline__ int64_t stream_of(const Geo& g, int64_t i) {
  int64_t b = g.s_full > 0 ? i / g.s_full : 0;
  if (b >= g.nb) b = g.nb - 1;
  const int64_t j = i - b * g.s_full;
  const int64_t pos = (int64_t)g.rank * slice_len(g, b) + j;
  return pos < real_len(g, b) ? b * g.cap + pos : -1;
}

// Stream position -> (source rank, source shard index).
__device__ __forceinline__ void locate(const Geo& g, int64_t x, int32_t& q, int64_t& idx) {
  int64_t b = x / g.cap;
  if (b >= g.nb) b = g.nb - 1;
  const int64_t w = x - b * g.cap;
  const int64_t sb = slice_len(g, b);
  q = (int32_t)(w / sb);
  idx = b * g.s_full + (w - (int64_t)q * sb);
}

template <class T>
__global__ void __launch_bounds__(256) reshard_kernel(const ReshardArgs A) {
  const int64_t T_ = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < A.n; e += T_) {
    const int64_t i = A.i0 + e;
    const int64_t xl = stream_of(A.gd, i - A.d_base_i);
    if (xl < 0) {
      if (A.zero_pads) ((T*)A.dst)[i] = T(0);
      continue;
    }
    if (!A.has_src) continue;
    const int64_t xs = A.d_base_x + xl - A.s_base_x;
    if (xs < 0 || xs >= A.s_len) continue;
    int32_t q;
    int64_t idx;
    locate(A.gs, xs, q, idx);
    ((T*)A.dst)[i] = ((const T*)A.src[q])[idx];
  }
}

int cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int blocks_for(int64_t work) {
  return (int)std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, (int64_t)cus() * 4));
}

}  // namespace

extern "C" {

int zero_gather_params(const zero_layout* L, const uint16_t* const* rank_shards,
                       int64_t bucket_begin, int64_t bucket_end, uint16_t* full_out,
                       hipStream_t stream) {
  if (!L || !rank_shards || !full_out) return ZERO_EINVAL;
  if (bucket_begin < 0 || bucket_end > L->nb || bucket_begin > bucket_end) return ZERO_ERANGE;
  const int32_t nd = L->n_d;
  for (int32_t q = 0; q < nd; ++q) {
    if (!rank_shards[q]) return ZERO_EINVAL;
    if (overlap(rank_shards[q], 2 * L->S, full_out, 2 * L->P)) return ZERO_EOVERLAP;
  }
  if (bucket_begin == bucket_end) return ZERO_OK;
  auto launch = [&](const Geo& g, int64_t shard_shift, int64_t out_shift, int64_t f0,
                    int64_t f1) -> int {
    GatherArgs A;
    for (int q = 0; q < ZERO_MAX_ND; ++q)
      A.shard[q] = q < nd ? rank_shards[q] + shard_shift : nullptr;
    A.out = full_out + out_shift;
    A.g = g;
    A.f0 = f0;
    A.f1 = f1;
    bool vec = a16(A.out) && g.s_full % 8 == 0 && g.s_last % 8 == 0 && f0 % 8 == 0;
    for (int32_t q = 0; q < nd; ++q) vec = vec && a16(A.shard[q]);
    if (vec)
      hipLaunchKernelGGL(gather_vec_kernel, dim3(blocks_for((f1 - f0) >> 3)), dim3(256), 0,
                         stream, A);
    else
      hipLaunchKernelGGL(gather_scalar_kernel, dim3(blocks_for(f1 - f0)), dim3(256), 0, stream,
                         A);
    return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
  };
  if (L->fixed()) {
    const int64_t f0 = L->bucket_padded_off(bucket_begin);
    const int64_t f1 = L->bucket_padded_off(bucket_end - 1) + L->bucket_padded(bucket_end - 1);
    return launch(geo_of(*L), 0, 0, f0, f1);
  }
  for (int64_t b = bucket_begin; b < bucket_end; ++b) {
    if (L->bucket_slice(b) == 0) continue;
    const int rc = launch(geo_of_bucket(*L, b), L->bucket_shard_off(b), L->bucket_padded_off(b),
                          0, L->bucket_padded(b));
    if (rc != ZERO_OK) return rc;
  }
  return ZERO_OK;
}

int zero_reshard(const zero_layout* src, const void* const* src_shards, const zero_layout* dst,
                 void* dst_shard, int32_t elem_bytes, hipStream_t stream) {
  if (!src || !dst || !src_shards || !dst_shard) return ZERO_EINVAL;
  if (elem_bytes != 2 && elem_bytes != 4) return ZERO_EINVAL;
  if (src->numel != dst->numel) return ZERO_EINVAL;
  for (int32_t q = 0; q < src->n_d; ++q) {
    if (!src_shards[q]) return ZERO_EINVAL;
    if (overlap(src_shards[q], elem_bytes * src->S, dst_shard, elem_bytes * dst->S))
      return ZERO_EOVERLAP;
  }
  if (dst->S == 0) return ZERO_OK;

  // One launch: destination range [i0, i0+n) read through geometry gd
  // (origin d_base_i / d_base_x), source through gs with its pointers
  // shifted by s_shift elements and stream origin s_base_x.
  auto launch = [&](const Geo& gd, int64_t i0, int64_t n, int64_t d_base_i, int64_t d_base_x,
                    const Geo* gs, int64_t s_shift, int64_t s_base_x, int64_t s_len,
                    bool zero_pads) -> int {
    if (n <= 0) return ZERO_OK;
    ReshardArgs A;
    for (int q = 0; q < ZERO_MAX_ND; ++q)
      A.src[q] = q < src->n_d ? (const char*)src_shards[q] + s_shift * elem_bytes : nullptr;
    A.dst = dst_shard;
    A.gd = gd;
    A.gs = gs ? *gs : gd;
    A.i0 = i0;
    A.n = n;
    A.d_base_i = d_base_i;
    A.d_base_x = d_base_x;
    A.s_base_x = s_base_x;
    A.s_len = s_len;
    A.zero_pads = zero_pads ? 1 : 0;
    A.has_src = gs ? 1 : 0;
    if (elem_bytes == 4)
      hipLaunchKernelGGL(reshard_kernel<uint32_t>, dim3(blocks_for(n)), dim3(256), 0, stream, A);
    else
      hipLaunchKernelGGL(reshard_kernel<uint16_t>, dim3(blocks_for(n)), dim3(256), 0, stream, A);
    return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
  };

  int rc = ZERO_OK;
  if (src->fixed()) {
    const Geo gs = geo_of(*src);
    if (dst->fixed())
      return launch(geo_of(*dst), 0, dst->S, 0, 0, &gs, 0, 0, src->psi, true);
    for (int64_t b = 0; b < dst->nb && rc == ZERO_OK; ++b)
      rc = launch(geo_of_bucket(*dst, b), dst->bucket_shard_off(b), dst->bucket_slice(b),
                  dst->bucket_shard_off(b), dst->bucket_stream_off(b), &gs, 0, 0, src->psi, true);
    return rc;
  }
  // per-parameter source: one launch per source tensor over the destination
  // indices that can hold it; destination padding first when the
  // destination is bucketed
  if (dst->fixed()) {
    const Geo gd = geo_of(*dst);
    rc = launch(gd, 0, dst->S, 0, 0, nullptr, 0, 0, 0, true);
    for (int64_t t = 0; t < src->nb && rc == ZERO_OK; ++t) {
      if (src->bucket_len(t) == 0) continue;
      int64_t lo = 0, hi = 0;
      zero_layout_tensor(dst, (int32_t)t, nullptr, &lo, &hi);
      const Geo gs = geo_of_bucket(*src, t);
      rc = launch(gd, lo, hi - lo, 0, 0, &gs, src->bucket_shard_off(t), src->bucket_stream_off(t),
                  src->bucket_len(t), false);
    }
    return rc;
  }
  for (int64_t t = 0; t < src->nb && rc == ZERO_OK; ++t) {
    const Geo gs = geo_of_bucket(*src, t);
    rc = launch(geo_of_bucket(*dst, t), dst->bucket_shard_off(t), dst->bucket_slice(t),
                dst->bucket_shard_off(t), dst->bucket_stream_off(t), &gs,
                src->bucket_shard_off(t), src->bucket_stream_off(t), src->bucket_len(t), true);
  }
  return rc;
}

}  // extern "C"
