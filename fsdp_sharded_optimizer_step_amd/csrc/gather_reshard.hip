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
// state array: from the N_d shards of one layout (bucketed or per-parameter)
// to one rank's shard of another layout of the same tensor list.
//
// Both are copies: gather moves 4 bytes per flat element, reshard 2 x the
// element size per destination element (2 for bf16, 4 for fp32), plus the
// destination's padding written as zeros.
#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

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

__device__ __forceinline__ int64_t slice_len(const Geo& g, int64_t b) {
  return b + 1 < g.nb ? g.s_full : g.s_last;
}
__device__ __forceinline__ int64_t real_len(const Geo& g, int64_t b) {
  return b + 1 < g.nb ? g.cap : g.len_last;
}

// ------------------------------------------------------------------ gather
// Every (bucket, rank) slice is cut into tiles, one tile per block: the
// block copies a contiguous tile of rank q's slice of the bucket into slot q
// of the bucket in the flat buffer, 16 bytes per lane and access where
// source and destination allow it.
constexpr int kGatherThreads = 256;
// Tile size and cache hint measured on MI355X (llama8b gather: 2048-element
// tiles with non-temporal accesses 5.20 ms, 4096 5.41 ms, 8192 with ordinary
// accesses 5.69 ms).
constexpr int64_t kGatherTile = kGatherThreads * 8;  // elements per tile
// Blocks per launch: the dispatch grid counts work-items in 32 bits, so
// larger jobs are split into several launches.
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

// Up to kGatherTab buckets share a launch through a table in the kernel
// arguments (first item, tiles per slice, offsets); a block finds its bucket
// by binary search over the first items, then (rank, tile) within it.  The
// same kernel serves both layouts: in the per-parameter one every tensor is
// its own bucket with its own slice length; bucketed layouts take it too,
// measured on MI355X (llama8b, library builds timed alternately on one tuned
// pool): 5.05 ms against 5.20 ms for one launch per run of equal buckets
// with (bucket, rank, tile) items, 5.07 ms for (bucket, tile, rank) items and
// 5.16 ms for rank-major items; inside a bucket the (rank, tile) order is
// kept (the per-parameter Llama-3-8B gather: 4.95 ms against 5.08 ms for
// (tile, rank)).
constexpr int kGatherTab = 48;
struct GatherTabArgs {
  const uint16_t* shard[ZERO_MAX_ND];  // each rank's shard
  uint16_t* out;                       // flat buffer
  int64_t shard_off[kGatherTab], flat_off[kGatherTab], slice[kGatherTab];
  uint32_t tiles[kGatherTab];
  uint32_t item0[kGatherTab + 1];      // first item of each tensor; item0[n] = total
  uint64_t vec;                        // bit k: tensor k takes 16-byte copies
  uint32_t item_base;                  // first item of this launch
  int32_t n, n_d;
};
static_assert(sizeof(GatherTabArgs) <= 4096, "kernel arguments");

__global__ void __launch_bounds__(kGatherThreads) gather_table_kernel(const GatherTabArgs A) {
  const uint32_t item = A.item_base + blockIdx.x;
  int lo = 0, hi = A.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (A.item0[mid] <= item) lo = mid;
    else hi = mid;
  }
  const uint32_t local = item - A.item0[lo];
  const uint32_t tiles = A.tiles[lo];
  const uint32_t q = local / tiles;
  const uint32_t c = local - q * tiles;
  const int64_t slice = A.slice[lo];
  const uint16_t* src = A.shard[q] + A.shard_off[lo];
  uint16_t* dst = A.out + A.flat_off[lo] + (int64_t)q * slice;
  const int64_t e0 = (int64_t)c * kGatherTile;
  const int64_t e1 = e0 + kGatherTile < slice ? e0 + kGatherTile : slice;
  if ((A.vec >> lo) & 1ull) {
    const u32x4* sv = (const u32x4*)(src + e0);
    u32x4* dv = (u32x4*)(dst + e0);
    const int64_t nv = (e1 - e0) >> 3;
    for (int64_t v = threadIdx.x; v < nv; v += kGatherThreads)
      st_stream<true>(dv + v, ld_stream<true>(sv + v));
  } else {
    for (int64_t e = e0 + threadIdx.x; e < e1; e += kGatherThreads) dst[e] = src[e];
  }
}

// ------------------------------------------------------------------ reshard
// One launch covers the destination shard indices [i0, i0 + n).  The
// destination index i maps, through geometry gd taken at origin d_base_i,
// to the stream position x = d_base_x + (position in gd), or to padding;
// when has_src, the source element of x is found through geometry gs at
// stream origin s_base_x, if 0 <= x - s_base_x < s_len, in the source shards
// (pointers already shifted to the source bucket).  Padding is written as
// zero when zero_pads; positions whose stream element lies outside this
// launch's source range are left alone.
struct ReshardArgs {
  const void* src[ZERO_MAX_ND];
  void* dst;
  Geo gs, gd;
  int64_t i0, n, d_base_i, d_base_x, s_base_x, s_len;
  int32_t zero_pads, has_src;
};

// Destination index i (relative to the geometry) -> stream position x (or
// -1 for padding) and the number of following indices, this one included,
// whose positions continue the same run (consecutive stream positions, or
// padding).
struct Run {
  int64_t x, rem;
};
__device__ __forceinline__ Run dst_run(const Geo& g, int64_t i) {
  int64_t b = g.s_full > 0 ? i / g.s_full : 0;
  if (b >= g.nb) b = g.nb - 1;
  const int64_t j = i - b * g.s_full;
  const int64_t sl = slice_len(g, b), len = real_len(g, b);
  const int64_t pos = (int64_t)g.rank * sl + j;
  if (pos < len) return Run{b * g.cap + pos, (sl - j) < (len - pos) ? (sl - j) : (len - pos)};
  return Run{-1, sl - j};
}

// Stream position -> source rank, source shard index, and how many
// consecutive positions stay in the same source slice.
struct SrcRun {
  int64_t idx, rem;
  int32_t q;
};
__device__ __forceinline__ SrcRun src_run(const Geo& g, int64_t x) {
  int64_t b = x / g.cap;
  if (b >= g.nb) b = g.nb - 1;
  const int64_t w = x - b * g.cap;
  const int64_t sb = slice_len(g, b);
  const int32_t q = (int32_t)(w / sb);
  const int64_t j = w - (int64_t)q * sb;
  const int64_t left = real_len(g, b) - w;
  return SrcRun{b * g.s_full + j, (sb - j) < left ? (sb - j) : left, q};
}

// Each block takes a tile of consecutive destination indices and walks it
// in runs that are contiguous on both sides (one destination slice, one
// source slice); all run arithmetic is uniform across the block, and each
// run is copied by the whole block, 16 bytes at a time when source and
// destination share their alignment.
constexpr int kResThreads = 256;
// Tiles of 8 KB (2048 fp32 or 4096 bf16 elements): measured on MI355X for
// the fp32 state re-cut (2.46 ms against 2.85 with 32 KB tiles).
constexpr int64_t kResTileBytes = 8192;
template <class T>
constexpr int64_t res_tile() { return kResTileBytes / (int64_t)sizeof(T); }

template <class T>
__device__ __forceinline__ void copy_run(T* dst, const T* src, int64_t n) {
  const uintptr_t da = (uintptr_t)dst, sa = (uintptr_t)src;
  if (((da ^ sa) & 15u) == 0) {
    const int64_t head = std::min<int64_t>(n, (int64_t)(((16u - (da & 15u)) & 15u) / sizeof(T)));
    if (threadIdx.x < head) dst[threadIdx.x] = src[threadIdx.x];
    constexpr int per = 16 / sizeof(T);
    const int64_t nv = (n - head) / per;
    u32x4* dv = (u32x4*)(dst + head);
    const u32x4* sv = (const u32x4*)(src + head);
    for (int64_t v = threadIdx.x; v < nv; v += kResThreads)
      st_stream<true>(dv + v, ld_stream<true>(sv + v));
    const int64_t t0 = head + nv * per;
    if (threadIdx.x < n - t0) dst[t0 + threadIdx.x] = src[t0 + threadIdx.x];
  } else {
    for (int64_t k = threadIdx.x; k < n; k += kResThreads) dst[k] = src[k];
  }
}

template <class T>
__device__ __forceinline__ void zero_run(T* dst, int64_t n) {
  for (int64_t k = threadIdx.x; k < n; k += kResThreads) dst[k] = T(0);
}

// Destination indices [e_begin, e_end) of a piece covering [i0, i0 + n):
// walked in runs contiguous on both sides.  Source pointers are shifted by
// s_shift elements.
template <class T>
__device__ __forceinline__ void reshard_range(const Geo& gd, const Geo& gs,
                                              const void* const* src, int64_t s_shift, T* dst,
                                              int64_t i0, int64_t d_base_i, int64_t d_base_x,
                                              int64_t s_base_x, int64_t s_len, int32_t zero_pads,
                                              int32_t has_src, int64_t e_begin, int64_t e_end) {
  for (int64_t e = e_begin; e < e_end;) {
    const Run d = dst_run(gd, i0 + e - d_base_i);
    int64_t len = std::min(d.rem, e_end - e);
    if (d.x < 0) {
      if (zero_pads) zero_run(dst + e, len);
      e += len;
      continue;
    }
    const int64_t xs = d_base_x + d.x - s_base_x;
    if (!has_src || xs >= s_len) {
      e += len;
      continue;
    }
    if (xs < 0) {
      e += std::min(len, -xs);
      continue;
    }
    const SrcRun sr = src_run(gs, xs);
    len = std::min(len, std::min(sr.rem, s_len - xs));
    copy_run(dst + e, (const T*)src[sr.q] + s_shift + sr.idx, len);
    e += len;
  }
}

template <class T>
__global__ void __launch_bounds__(kResThreads) reshard_kernel(const ReshardArgs A) {
  const int64_t e_begin = (int64_t)blockIdx.x * res_tile<T>();
  if (e_begin >= A.n) return;
  const int64_t e_end = std::min(A.n, e_begin + res_tile<T>());
  reshard_range<T>(A.gd, A.gs, A.src, 0, (T*)A.dst + A.i0, A.i0, A.d_base_i, A.d_base_x,
                   A.s_base_x, A.s_len, A.zero_pads, A.has_src, e_begin, e_end);
}

// Per-parameter layouts: many pieces per launch.  A piece's destination or
// source geometry is either the layout's own (bucketed) geometry or that of
// one tensor seen as a single bucket, given by its real and slice lengths.
struct ResPiece {
  int64_t i0, n, d_base_i, d_base_x, s_shift, s_base_x, s_len;
  int64_t d_len, d_slice, s_blen, s_slice;  // single-bucket geometries (when flagged)
  int32_t flags;                            // kZeroPads | kHasSrc | kDstOne | kSrcOne
};
constexpr int32_t kZeroPads = 1, kHasSrc = 2, kDstOne = 4, kSrcOne = 8;
template <int NP>
struct ResTabArgs {
  static constexpr int kCap = NP <= 64 ? 32 : 16;
  const void* src[NP];
  void* dst;
  Geo gd, gs;                        // the layouts' own geometries
  ResPiece p[kCap];
  uint32_t tile0[kCap + 1];          // first tile of each piece; tile0[n] = total
  uint32_t tile_base;                // first tile of this launch
  int32_t n;
};
static_assert(sizeof(ResTabArgs<ZERO_MAX_ND>) <= 4096, "kernel arguments");
static_assert(sizeof(ResTabArgs<64>) <= 4096, "kernel arguments");

__device__ __forceinline__ Geo one_bucket(int64_t len, int64_t slice, const Geo& g) {
  return Geo{len > 0 ? len : 1, 1, slice, slice * g.n_d, len, slice, g.n_d, g.rank};
}

template <class T, int NP>
__global__ void __launch_bounds__(kResThreads) reshard_table_kernel(const ResTabArgs<NP> A) {
  const uint32_t tile = A.tile_base + blockIdx.x;
  int lo = 0, hi = A.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (A.tile0[mid] <= tile) lo = mid;
    else hi = mid;
  }
  const ResPiece& P = A.p[lo];
  const int64_t e_begin = (int64_t)(tile - A.tile0[lo]) * res_tile<T>();
  if (e_begin >= P.n) return;
  const int64_t e_end = std::min(P.n, e_begin + res_tile<T>());
  const Geo gd = (P.flags & kDstOne) ? one_bucket(P.d_len, P.d_slice, A.gd) : A.gd;
  const Geo gs = (P.flags & kSrcOne) ? one_bucket(P.s_blen, P.s_slice, A.gs) : A.gs;
  reshard_range<T>(gd, gs, A.src, P.s_shift, (T*)A.dst + P.i0, P.i0, P.d_base_i, P.d_base_x,
                   P.s_base_x, P.s_len, P.flags & kZeroPads, P.flags & kHasSrc, e_begin, e_end);
}

bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

}  // namespace

// Table launches of re-cut pieces (per-parameter layouts).
template <int NP>
int launch_res_table(const std::vector<ResPiece>& pieces, const zero_layout* src,
                     const void* const* src_shards, const zero_layout* dst, void* dst_shard,
                     int32_t elem_bytes, hipStream_t stream) {
  using Args = ResTabArgs<NP>;
  Args A;
  for (int q = 0; q < NP; ++q) A.src[q] = q < src->n_d ? src_shards[q] : nullptr;
  A.dst = dst_shard;
  A.gd = geo_of(*dst);
  A.gs = geo_of(*src);
  const int64_t tile_elems = kResTileBytes / elem_bytes;
  for (size_t p0 = 0; p0 < pieces.size(); p0 += Args::kCap) {
    A.n = (int32_t)std::min<size_t>(Args::kCap, pieces.size() - p0);
    int64_t tiles = 0;
    for (int k = 0; k < A.n; ++k) {
      A.p[k] = pieces[p0 + k];
      A.tile0[k] = (uint32_t)tiles;
      tiles += (A.p[k].n + tile_elems - 1) / tile_elems;
    }
    A.tile0[A.n] = (uint32_t)tiles;  // < 2^32: checked by the caller
    for (int64_t t0 = 0; t0 < tiles; t0 += kMaxBlocks) {
      A.tile_base = (uint32_t)t0;
      const unsigned grid = (unsigned)std::min(kMaxBlocks, tiles - t0);
      if (elem_bytes == 4)
        hipLaunchKernelGGL((reshard_table_kernel<uint32_t, NP>), dim3(grid), dim3(kResThreads), 0,
                           stream, A);
      else
        hipLaunchKernelGGL((reshard_table_kernel<uint16_t, NP>), dim3(grid), dim3(kResThreads), 0,
                           stream, A);
      if (hipGetLastError() != hipSuccess) return ZERO_EHIP;
    }
  }
  return ZERO_OK;
}

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
  // items over all runs <= P / tile + (number of buckets) * n_d
  if (L->P / kGatherTile + (bucket_end - bucket_begin) * (int64_t)nd >= (int64_t)0xffffffff)
    return ZERO_ERANGE;
  if (hip_error_pending()) return ZERO_EHIP;
  // tables of up to kGatherTab non-empty buckets (tensors, for the
  // per-parameter layout)
  GatherTabArgs T;
  for (int q = 0; q < ZERO_MAX_ND; ++q) T.shard[q] = q < nd ? rank_shards[q] : nullptr;
  T.out = full_out;
  T.n_d = nd;
  bool base_vec = a16(full_out);
  for (int32_t q = 0; q < nd; ++q) base_vec = base_vec && a16(rank_shards[q]);
  T.n = 0;
  T.vec = 0;
  T.item0[0] = 0;
  auto flush = [&]() -> int {
    const int64_t items = T.item0[T.n];
    for (int64_t i0 = 0; i0 < items; i0 += kMaxBlocks) {
      T.item_base = (uint32_t)i0;
      const unsigned grid = (unsigned)std::min(kMaxBlocks, items - i0);
      hipLaunchKernelGGL(gather_table_kernel, dim3(grid), dim3(kGatherThreads), 0, stream, T);
      if (hipGetLastError() != hipSuccess) return ZERO_EHIP;
    }
    T.n = 0;
    T.vec = 0;
    T.item0[0] = 0;
    return ZERO_OK;
  };
  for (int64_t b = bucket_begin; b < bucket_end; ++b) {
    const int64_t sl = L->bucket_slice(b);
    if (sl == 0) continue;
    const int k = T.n;
    const int64_t so = L->bucket_shard_off(b), fo = L->bucket_padded_off(b);
    const int64_t tiles = (sl + kGatherTile - 1) / kGatherTile;
    T.shard_off[k] = so;
    T.flat_off[k] = fo;
    T.slice[k] = sl;
    T.tiles[k] = (uint32_t)tiles;
    T.item0[k + 1] = T.item0[k] + (uint32_t)(tiles * nd);  // < 2^32: checked above
    if (base_vec && so % 8 == 0 && fo % 8 == 0 && sl % 8 == 0) T.vec |= 1ull << k;
    T.n = k + 1;
    if (T.n == kGatherTab) {
      const int rc = flush();
      if (rc != ZERO_OK) return rc;
    }
  }
  return T.n > 0 ? flush() : ZERO_OK;
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
  if (hip_error_pending()) return ZERO_EHIP;

  // One `launch`: destination range [i0, i0+n) read through geometry gd
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
    // at most kMaxBlocks tiles per launch: the range is cut into pieces
    // (the geometry origins stay, only [i0, i0 + n) moves)
    const int64_t tile_elems = kResTileBytes / elem_bytes;
    for (int64_t off = 0; off < n; off += kMaxBlocks * tile_elems) {
      A.i0 = i0 + off;
      A.n = std::min(n - off, kMaxBlocks * tile_elems);
      const unsigned grid = (unsigned)((A.n + tile_elems - 1) / tile_elems);
      if (elem_bytes == 4)
        hipLaunchKernelGGL(reshard_kernel<uint32_t>, dim3(grid), dim3(kResThreads), 0, stream, A);
      else
        hipLaunchKernelGGL(reshard_kernel<uint16_t>, dim3(grid), dim3(kResThreads), 0, stream, A);
      if (hipGetLastError() != hipSuccess) return ZERO_EHIP;
    }
    return ZERO_OK;
  };

  if (src->fixed() && dst->fixed()) {
    const Geo gs = geo_of(*src);
    return launch(geo_of(*dst), 0, dst->S, 0, 0, &gs, 0, 0, src->psi, true);
  }

  // A per-parameter layout on either side: pieces of the destination, each
  // read through one tensor's single-bucket geometry or the bucketed
  // layout's own, in table launches.
  std::vector<ResPiece> pieces;
  auto piece = [&](int64_t i0, int64_t n, int64_t d_base_i, int64_t d_base_x, int64_t s_shift,
                   int64_t s_base_x, int64_t s_len, int64_t d_len, int64_t d_slice,
                   int64_t s_blen, int64_t s_slice, int32_t flags) {
    if (n > 0)
      pieces.push_back(ResPiece{i0, n, d_base_i, d_base_x, s_shift, s_base_x, s_len, d_len,
                                d_slice, s_blen, s_slice, flags});
  };
  if (src->fixed()) {
    // bucketed source, per-parameter destination: one piece per tensor
    for (int64_t b = 0; b < dst->nb; ++b)
      piece(dst->bucket_shard_off(b), dst->bucket_slice(b), dst->bucket_shard_off(b),
            dst->bucket_stream_off(b), 0, 0, src->psi, dst->bucket_len(b), dst->bucket_slice(b),
            0, 0, kZeroPads | kHasSrc | kDstOne);
  } else if (dst->fixed()) {
    // per-parameter source, bucketed destination: the destination's padding
    // (per bucket, or one pass over the shard when many buckets have some),
    // then one piece per source tensor over the destination range holding it
    std::vector<std::pair<int64_t, int64_t>> pads;
    for (int64_t b = 0; b < dst->nb; ++b) {
      const int64_t sl = dst->bucket_slice(b), real = dst->bucket_len(b) - dst->rank * sl;
      const int64_t keep = real < 0 ? 0 : (real > sl ? sl : real);
      if (keep < sl) pads.push_back({dst->bucket_shard_off(b) + keep, sl - keep});
    }
    if (pads.size() > 64)
      piece(0, dst->S, 0, 0, 0, 0, 0, 0, 0, 0, 0, kZeroPads);
    else
      for (const auto& pd : pads) piece(pd.first, pd.second, 0, 0, 0, 0, 0, 0, 0, 0, 0, kZeroPads);
    for (int64_t t = 0; t < src->nb; ++t) {
      if (src->bucket_len(t) == 0) continue;
      int64_t lo = 0, hi = 0;
      zero_layout_tensor(dst, (int32_t)t, nullptr, &lo, &hi);
      piece(lo, hi - lo, 0, 0, src->bucket_shard_off(t), src->bucket_stream_off(t),
            src->bucket_len(t), 0, 0, src->bucket_len(t), src->bucket_slice(t),
            kHasSrc | kSrcOne);
    }
  } else {
    // per-parameter on both sides: one piece per tensor
    for (int64_t t = 0; t < src->nb; ++t)
      piece(dst->bucket_shard_off(t), dst->bucket_slice(t), dst->bucket_shard_off(t),
            dst->bucket_stream_off(t), src->bucket_shard_off(t), src->bucket_stream_off(t),
            src->bucket_len(t), dst->bucket_len(t), dst->bucket_slice(t), src->bucket_len(t),
            src->bucket_slice(t), kZeroPads | kHasSrc | kDstOne | kSrcOne);
  }
  if (dst->S / (kResTileBytes / elem_bytes) + (int64_t)pieces.size() >= (int64_t)0xffffffff)
    return ZERO_ERANGE;
  return src->n_d <= 64 ? launch_res_table<64>(pieces, src, src_shards, dst, dst_shard, elem_bytes,
                                               stream)
                        : launch_res_table<ZERO_MAX_ND>(pieces, src, src_shards, dst, dst_shard,
                                                        elem_bytes, stream);
}

}  // extern "C"
