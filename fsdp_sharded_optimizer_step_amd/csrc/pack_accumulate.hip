// zero_bucket_pack and zero_grad_accumulate.
//
// Page "Infra: Data Parallel" (pufanyi.com), section "Naive Data
// Parallelism": gradients of several parameters share one bucket that is
// communicated once all of them are ready; with gradient accumulation the
// micro-batch gradients are summed locally (no_sync) and each micro-batch
// loss is divided by the number of micro-batches.  Section "FSDP1": the
// parameters of a unit are flattened and concatenated into one flat buffer
// that is split evenly, padding included.
//
// Both kernels are HBM streams with whole cache lines per instruction, no
// LDS.  Pack moves 4 bytes per element (2 per pad element) in tiles;
// accumulate moves 6 (overwrite), 10 (add) or 8 (add, emit bf16, no fp32
// store) bytes in a grid-stride loop over 512-element chunks.
#include <algorithm>
#include <cstdint>
#include <vector>

#include "device_common.hpp"
#include "layout.hpp"
#include "zero_shard.h"

namespace {
using namespace zs;

// ------------------------------------------------------------------ pack
// A piece is one tensor's part inside one bucket (or a bucket's padding).
// Work is cut into equal tiles so that ragged tensors (a 38.6M-element
// embedding next to 768-element norm vectors) keep every block equally busy:
// block x takes tile x of the launch and finds its piece by binary search
// over the launch's tile prefix sums.
struct Piece {
  const uint16_t* src;  // nullptr: write zeros (bucket padding)
  int64_t dst;          // element offset in the flat buffer
  int64_t n;            // element count (at most kMaxPieceElems)
  int32_t head;         // vector pieces: elements (< 8) before the destination is 16-byte aligned
  int32_t vec;          // 1: source and destination share 16-byte phase (or zeros)
};
// A launch carries its pieces in the kernel arguments, 24 bytes each
// (source, destination with the head and vector flag in its top bits,
// length, first tile): 169 pieces fit in 4 KB, so GPT-2's 148 tensors and
// 10 bucket pads go in one launch instead of two.
constexpr int kPiecesPerLaunch = 169;
constexpr int kPackThreads = 256;
// pieces longer than this are cut (a multiple of 8 elements, so the parts
// keep the 16-byte phase of the whole)
constexpr int64_t kMaxPieceElems = (int64_t)1 << 30;
constexpr int kDstBits = 56;
constexpr uint64_t kDstMask = ((uint64_t)1 << kDstBits) - 1;
// Tiles of 512 vectors (4096 elements) and non-temporal accesses: the
// fastest of 3 tile sizes x 2 cache hints measured on MI355X for GPT-2's
// buckets (84 us against 98 us for 1024-vector tiles with ordinary accesses).
constexpr int64_t kTileVecs = kPackThreads * 2;   // 8-element vectors per tile
constexpr int64_t kTileElems = kPackThreads * 4;  // elements per tile, scalar pieces
struct PackArgs {
  const uint16_t* src[kPiecesPerLaunch];
  uint64_t dst[kPiecesPerLaunch];       // offset | head << 56 | vec << 60
  uint32_t n[kPiecesPerLaunch];
  int32_t tile0[kPiecesPerLaunch + 1];  // first tile of each piece; tile0[count] = total
  uint16_t* out;
  int32_t count;
  int32_t tile_base;  // first tile of this launch
};
static_assert(sizeof(PackArgs) <= 4096, "kernel arguments");
// Blocks per launch: the dispatch grid counts work-items in 32 bits, so a
// larger group of pieces is covered by several launches.
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

int64_t piece_tiles(const Piece& pc) {
  if (!pc.vec) return std::max<int64_t>(1, (pc.n + kTileElems - 1) / kTileElems);
  const int64_t nv = (pc.n - pc.head) >> 3;
  return std::max<int64_t>(1, (nv + kTileVecs - 1) / kTileVecs);
}

__global__ void __launch_bounds__(kPackThreads) pack_kernel(const PackArgs A) {
  const int64_t tile = (int64_t)A.tile_base + blockIdx.x;
  int lo = 0, hi = A.count;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (A.tile0[mid] <= tile) lo = mid;
    else hi = mid;
  }
  const uint16_t* src = A.src[lo];
  const uint64_t dw = A.dst[lo];
  const int64_t n = A.n[lo];
  const int32_t head = (int32_t)((dw >> kDstBits) & 15u);
  const bool vec = ((dw >> (kDstBits + 4)) & 1u) != 0;
  const int64_t t = tile - A.tile0[lo];
  const int64_t ntile = A.tile0[lo + 1] - A.tile0[lo];
  uint16_t* d = A.out + (int64_t)(dw & kDstMask);
  const bool zeros = src == nullptr;
  if (!vec) {
    const int64_t e0 = t * kTileElems, e1 = std::min(n, e0 + kTileElems);
    for (int64_t e = e0 + threadIdx.x; e < e1; e += kPackThreads) d[e] = src[e];
    return;
  }
  const int64_t nv = (n - head) >> 3;
  const int64_t tail0 = head + (nv << 3);
  if (t == 0 && threadIdx.x < head) d[threadIdx.x] = zeros ? (uint16_t)0 : src[threadIdx.x];
  if (t == ntile - 1 && threadIdx.x < n - tail0)
    d[tail0 + threadIdx.x] = zeros ? (uint16_t)0 : src[tail0 + threadIdx.x];
  u32x4* dv = (u32x4*)(d + head);
  const u32x4* sv = zeros ? nullptr : (const u32x4*)(src + head);
  const int64_t v0 = t * kTileVecs, v1 = std::min(nv, v0 + kTileVecs);
  for (int64_t v = v0 + threadIdx.x; v < v1; v += kPackThreads)
    st_stream<true>(dv + v, zeros ? u32x4{0u, 0u, 0u, 0u} : ld_stream<true>(sv + v));
}

// ------------------------------------------------------------------ accumulate
// Measured on accum1p3b-sized buffers (162.5M elements), every cache policy
// and 1-16 blocks per CU: non-temporal everything and 4 blocks of 256
// threads per CU are best for all three call kinds (overwrite 0.166 ms,
// add 0.265 ms, add + emit bf16 without store 0.206 ms).
constexpr int kAccPolicy = 7;
constexpr int kAccBlocksPerCu = 4;
// Grid-stride over chunks of 512 elements per wave; lane l takes the
// 4-element pieces at 4l and 256 + 4l, so that every load and store
// instruction of a wave covers whole cache lines (8-byte bf16, 16-byte fp32
// accesses).  POL bits (set: non-temporal): 1 gradient loads, 2 accumulator
// loads, 4 stores.  The elements after the last full chunk go one per
// thread.
template <int POL>
__global__ void __launch_bounds__(256) accum_vec_kernel(float* acc, const uint16_t* g, int64_t n,
                                                        float scale, uint32_t flags,
                                                        uint16_t* out) {
  constexpr bool ng = (POL & 1) != 0, na = (POL & 2) != 0, nw = (POL & 4) != 0;
  const bool overwrite = flags & ZERO_ACC_OVERWRITE;
  const bool emit = flags & ZERO_ACC_EMIT_BF16;
  const bool store = !(flags & ZERO_ACC_NO_STORE);
  const int64_t nchunk = n >> 9;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = tid >> 6; c < nchunk; c += T >> 6) {
    const int64_t ea = (c << 9) + ((threadIdx.x & 63) << 2), eb = ea + 256;
    const u32x2 wa = ld_stream<ng>((const u32x2*)(g + ea));
    const u32x2 wb = ld_stream<ng>((const u32x2*)(g + eb));
    float a[8] = {scale * bf16_lo(wa.x), scale * bf16_hi(wa.x), scale * bf16_lo(wa.y),
                  scale * bf16_hi(wa.y), scale * bf16_lo(wb.x), scale * bf16_hi(wb.x),
                  scale * bf16_lo(wb.y), scale * bf16_hi(wb.y)};
    if (!overwrite) {
      const f32x4 a0 = ld_stream<na>((const f32x4*)(acc + ea));
      const f32x4 a1 = ld_stream<na>((const f32x4*)(acc + eb));
      a[0] = a0.x + a[0]; a[1] = a0.y + a[1]; a[2] = a0.z + a[2]; a[3] = a0.w + a[3];
      a[4] = a1.x + a[4]; a[5] = a1.y + a[5]; a[6] = a1.z + a[6]; a[7] = a1.w + a[7];
    }
    if (store) {
      st_stream<nw>((f32x4*)(acc + ea), f32x4{a[0], a[1], a[2], a[3]});
      st_stream<nw>((f32x4*)(acc + eb), f32x4{a[4], a[5], a[6], a[7]});
    }
    if (emit) {
      st_stream<nw>((u32x2*)(out + ea), u32x2{bf16_pack2(a[0], a[1]), bf16_pack2(a[2], a[3])});
      st_stream<nw>((u32x2*)(out + eb), u32x2{bf16_pack2(a[4], a[5]), bf16_pack2(a[6], a[7])});
    }
  }
  for (int64_t i = (nchunk << 9) + tid; i < n; i += T) {
    const float c = scale * bf16_one(g[i]);
    const float a = overwrite ? c : acc[i] + c;
    if (store) acc[i] = a;
    if (emit) out[i] = (uint16_t)bf16_round(a);
  }
}

__global__ void __launch_bounds__(256) accum_scalar_kernel(float* acc, const uint16_t* g,
                                                           int64_t n, float scale, uint32_t flags,
                                                           uint16_t* out) {
  const bool overwrite = flags & ZERO_ACC_OVERWRITE;
  const bool emit = flags & ZERO_ACC_EMIT_BF16;
  const bool store = !(flags & ZERO_ACC_NO_STORE);
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += T) {
    const float c = scale * bf16_one(g[i]);
    const float a = overwrite ? c : acc[i] + c;
    if (store) acc[i] = a;
    if (emit) out[i] = (uint16_t)bf16_round(a);
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

}  // namespace

extern "C" {

int zero_bucket_pack(const zero_layout* L, const uint16_t* const* tensor_grads,
                     int64_t bucket_begin, int64_t bucket_end, uint16_t* flat_out,
                     hipStream_t stream) {
  if (!L || !flat_out) return ZERO_EINVAL;
  if (bucket_begin < 0 || bucket_end > L->nb || bucket_begin > bucket_end) return ZERO_ERANGE;
  const int32_t nt = (int32_t)L->numel.size();
  if (nt > 0 && !tensor_grads) return ZERO_EINVAL;
  // pieces: (tensor part inside bucket) and (bucket padding)
  std::vector<Piece> pieces;
  int32_t t = 0;
  for (int64_t b = bucket_begin; b < bucket_end; ++b) {
    const int64_t x0 = L->bucket_stream_off(b), x1 = x0 + L->bucket_len(b);
    const int64_t base = L->bucket_padded_off(b);
    // first tensor whose range ends after x0
    t = (int32_t)(std::upper_bound(L->tensor_off.begin(), L->tensor_off.end(), x0) -
                  L->tensor_off.begin()) - 1;
    if (t < 0) t = 0;
    for (; t < nt && L->tensor_off[t] < x1; ++t) {
      const int64_t a = std::max(x0, L->tensor_off[t]);
      const int64_t z = std::min(x1, L->tensor_off[t] + L->numel[t]);
      if (a >= z) continue;
      const uint16_t* src = tensor_grads[t];
      if (!src) return ZERO_EINVAL;
      for (int64_t u = a; u < z; u += kMaxPieceElems)
        pieces.push_back(Piece{src + (u - L->tensor_off[t]), base + (u - x0),
                               std::min(kMaxPieceElems, z - u), 0, 0});
    }
    const int64_t pad = L->bucket_padded(b) - L->bucket_len(b);
    for (int64_t u = 0; u < pad; u += kMaxPieceElems)
      pieces.push_back(Piece{nullptr, base + L->bucket_len(b) + u,
                             std::min(kMaxPieceElems, pad - u), 0, 0});
  }
  // vector eligibility and head peel (destination alignment) per piece
  for (Piece& pc : pieces) {
    const uintptr_t da = (uintptr_t)(flat_out + pc.dst);
    pc.vec = pc.src == nullptr || ((da ^ (uintptr_t)pc.src) & 15u) == 0;
    pc.head = pc.vec ? (int32_t)std::min<int64_t>(pc.n, (int64_t)(((16u - (da & 15u)) & 15u) >> 1))
                     : 0;
  }
  // sources must not overlap the destination
  for (int32_t k = 0; k < nt; ++k)
    if (tensor_grads[k] && overlap(tensor_grads[k], 2 * L->numel[k], flat_out, 2 * L->P))
      return ZERO_EOVERLAP;
  // every launch's tile count must fit the grid (checked before any launch)
  for (size_t p0 = 0; p0 < pieces.size(); p0 += kPiecesPerLaunch) {
    int64_t tiles = 0;
    for (size_t k = p0; k < std::min(pieces.size(), p0 + kPiecesPerLaunch); ++k)
      tiles += piece_tiles(pieces[k]);
    if (tiles > 0x7fffffff) return ZERO_ERANGE;
  }
  if (pieces.empty()) return ZERO_OK;
  if (hip_error_pending()) return ZERO_EHIP;
  // destinations fit the 56-bit field (flat buffers far below 2^56 elements)
  if (L->P >= (int64_t)kDstMask) return ZERO_ERANGE;
  for (size_t p0 = 0; p0 < pieces.size(); p0 += kPiecesPerLaunch) {
    PackArgs A;
    A.out = flat_out;
    A.count = (int32_t)std::min<size_t>(kPiecesPerLaunch, pieces.size() - p0);
    int64_t tiles = 0;
    for (int k = 0; k < A.count; ++k) {
      const Piece& pc = pieces[p0 + k];
      A.src[k] = pc.src;
      A.dst[k] = (uint64_t)pc.dst | ((uint64_t)pc.head << kDstBits) |
                 ((uint64_t)(pc.vec ? 1 : 0) << (kDstBits + 4));
      A.n[k] = (uint32_t)pc.n;
      A.tile0[k] = (int32_t)tiles;
      tiles += piece_tiles(pc);
    }
    A.tile0[A.count] = (int32_t)tiles;
    for (int64_t t0 = 0; t0 < tiles; t0 += kMaxBlocks) {
      A.tile_base = (int32_t)t0;
      const unsigned grid = (unsigned)std::min(kMaxBlocks, tiles - t0);
      hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(kPackThreads), 0, stream, A);
      if (hipGetLastError() != hipSuccess) return ZERO_EHIP;
    }
  }
  return ZERO_OK;
}

int zero_grad_accumulate(float* acc, const uint16_t* grad, int64_t n, float scale, uint32_t flags,
                         uint16_t* bf16_out, hipStream_t stream) {
  if (n < 0 || (flags & ~(ZERO_ACC_OVERWRITE | ZERO_ACC_EMIT_BF16 | ZERO_ACC_NO_STORE)))
    return ZERO_EINVAL;
  const bool overwrite = flags & ZERO_ACC_OVERWRITE;
  const bool emit = flags & ZERO_ACC_EMIT_BF16;
  const bool store = !(flags & ZERO_ACC_NO_STORE);
  if (!store && !emit) return ZERO_EINVAL;
  if (n == 0) return ZERO_OK;
  if (!grad || (emit && !bf16_out) || ((store || !overwrite) && !acc)) return ZERO_EINVAL;
  if (overlap(grad, 2 * n, acc, 4 * n) || (emit && (overlap(bf16_out, 2 * n, grad, 2 * n) ||
                                                   overlap(bf16_out, 2 * n, acc, 4 * n))))
    return ZERO_EOVERLAP;
  if (hip_error_pending()) return ZERO_EHIP;
  // Launch policy, measured on MI355X for the three call kinds (blocks of
  // 256 threads per CU, cache policy).
  const int64_t cap = (int64_t)cus() * kAccBlocksPerCu;
  const bool vec = a16(grad) && (!acc || a16(acc)) && (!emit || a16(bf16_out));
  const int64_t work = vec ? std::max<int64_t>(n >> 3, 8) : n;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, cap));
  if (vec)
    hipLaunchKernelGGL(accum_vec_kernel<kAccPolicy>, dim3(blocks), dim3(256), 0, stream, acc,
                       grad, n, scale, flags, bf16_out);
  else
    hipLaunchKernelGGL(accum_scalar_kernel, dim3(blocks), dim3(256), 0, stream, acc, grad, n,
                       scale, flags, bf16_out);
  return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP;
}

}  // extern "C"
