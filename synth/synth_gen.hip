// Seeded synthetic inputs, generated identically on the host and on the GPU.
//
// Input recipe only: this module performs no step of the update (no
// reduction, no optimizer arithmetic, no rounding to the parameter format).
// Both the test oracle's inputs and the GPU path's inputs come from here, so
// a value depends only on (key, global parameter index), never on where or
// how it was generated.
//
// Counter-based generator: Philox4x32 with 10 rounds (Salmon, Moraes, Dror,
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11).  For
// parameter index x and draw d the counter is (x_lo, x_hi, d, 0) and the key
// is the 64-bit stream key.  Each 32-bit output word gives one 24-bit uniform
// integer (its top 24 bits).
//
// Distributions (all intermediate arithmetic is binary64):
//   normal(s)       z = (u_1 + ... + u_12 - 6*2^24) * 2^-24   (Irwin-Hall;
//                   exact in binary64), value = s*z
//   absnormal(s)    |s*z|
//   student_t3(s)   s * z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)
//   normal_zeros(s) +0 with probability 1 % (an independent 32-bit draw below
//                   floor(0.01 * 2^32)), otherwise s*z
// Stored as binary32 (round to nearest) or as bf16 bits = the upper 16 bits
// of that binary32 (truncation, an input convention, not the update's cast).
//
// Compiled with -ffp-contract=off so host and device evaluate the same
// sequence of correctly rounded binary64 operations.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

enum : int32_t { DIST_ZERO = 0, DIST_NORMAL = 1, DIST_ABSNORMAL = 2, DIST_STUDENT_T3 = 3,
                 DIST_NORMAL_ZEROS = 4 };
enum : int32_t { OUT_F32 = 0, OUT_BF16 = 1 };

constexpr uint32_t PHILOX_M0 = 0xD2511F53u, PHILOX_M1 = 0xCD9E8D57u;
constexpr uint32_t PHILOX_W0 = 0x9E3779B9u, PHILOX_W1 = 0xBB67AE85u;
constexpr uint32_t ZERO_THRESHOLD = 42949672u;  // floor(0.01 * 2^32)

struct Words {
  uint32_t w[4];
};

__host__ __device__ inline void mulhilo(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  hi = (uint32_t)(p >> 32);
  lo = (uint32_t)p;
}

__host__ __device__ inline Words philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(PHILOX_M0, c0, hi0, lo0);
    mulhilo(PHILOX_M1, c2, hi1, lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  Words r;
  r.w[0] = c0; r.w[1] = c1; r.w[2] = c2; r.w[3] = c3;
  return r;
}

// Standard-normal approximation from 12 uniforms: three Philox blocks
// starting at draw index 3*j.
__host__ __device__ inline double irwin_hall(uint64_t key, int64_t x, uint32_t j) {
  uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
  uint32_t x0 = (uint32_t)(uint64_t)x, x1 = (uint32_t)((uint64_t)x >> 32);
  int64_t sum = 0;
  for (uint32_t c = 0; c < 3; ++c) {
    Words r = philox4x32_10(x0, x1, 3u * j + c, 0u, k0, k1);
    for (int k = 0; k < 4; ++k) sum += (int64_t)(r.w[k] >> 8);
  }
  return (double)(sum - 6 * (int64_t)(1 << 24)) * (1.0 / 16777216.0);
}

__host__ __device__ inline double sample(uint64_t key, int64_t x, int32_t dist, double scale) {
  switch (dist) {
    case DIST_NORMAL:
      return scale * irwin_hall(key, x, 0);
    case DIST_ABSNORMAL:
      return std::fabs(scale * irwin_hall(key, x, 0));
    case DIST_STUDENT_T3: {
      double z0 = irwin_hall(key, x, 0);
      double z1 = irwin_hall(key, x, 1), z2 = irwin_hall(key, x, 2), z3 = irwin_hall(key, x, 3);
      double chi = z1 * z1 + z2 * z2 + z3 * z3;
      return scale * (z0 / std::sqrt(chi / 3.0));
    }
    case DIST_NORMAL_ZEROS: {
      uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
      Words r = philox4x32_10((uint32_t)(uint64_t)x, (uint32_t)((uint64_t)x >> 32), 1000u, 0u,
                              k0, k1);
      if (r.w[0] < ZERO_THRESHOLD) return 0.0;
      return scale * irwin_hall(key, x, 0);
    }
    default:
      return 0.0;
  }
}

__host__ __device__ inline uint32_t f32_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

__host__ __device__ inline void store(void* out, int32_t out_type, int64_t i, double val) {
  float f = (float)val;
  if (out_type == OUT_F32)
    ((float*)out)[i] = f;
  else
    ((uint16_t*)out)[i] = (uint16_t)(f32_bits(f) >> 16);
}

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

// One contiguous run of the output: out[dst_off + k] = sample(x0 + k) for
// k < n_real, then n_pad zeros.
struct synth_seg {
  int64_t dst_off, x0, n_real, n_pad;
};

constexpr int SEGS_PER_LAUNCH = 32;
struct SegBatch {
  synth_seg s[SEGS_PER_LAUNCH];
};

__global__ void __launch_bounds__(256) fill_kernel(void* out, int32_t out_type, SegBatch batch,
                                                   uint64_t key, int32_t dist, double scale) {
  const synth_seg sg = batch.s[blockIdx.y];
  const int64_t n = sg.n_real + sg.n_pad;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) {
    double v = (k < sg.n_real) ? sample(key, sg.x0 + k, dist, scale) : 0.0;
    store(out, out_type, sg.dst_off + k, v);
  }
}

extern "C" {

// Stream key from (workload id, kind, rank, micro-batch, step).
uint64_t synth_key(uint32_t workload, uint32_t kind, uint32_t rank, uint32_t micro, uint32_t step) {
  uint64_t z = 0x5EED5EED5EED5EEDull;
  const uint32_t parts[5] = {workload, kind, rank, micro, step};
  for (uint32_t p : parts) z = mix64(z + 0x9E3779B97F4A7C15ull + p);
  return z;
}

// Raw Philox4x32-10 block (for known-answer tests).
void synth_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  Words r = philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int k = 0; k < 4; ++k) out[k] = r.w[k];
}

// Host: fill `out` (host memory) over the given segments with nthreads threads.
int synth_fill_host(void* out, int32_t out_type, const synth_seg* segs, int32_t nseg, uint64_t key,
                    int32_t dist, double scale, int32_t nthreads) {
  if (!out || (nseg > 0 && !segs) || nthreads < 1) return -1;
  for (int32_t s = 0; s < nseg; ++s) {
    const synth_seg sg = segs[s];
    const int64_t n = sg.n_real + sg.n_pad;
    int32_t nt = (int32_t)std::min<int64_t>(nthreads, std::max<int64_t>(1, n / 65536));
    auto work = [&](int64_t lo, int64_t hi) {
      for (int64_t k = lo; k < hi; ++k)
        store(out, out_type, sg.dst_off + k, (k < sg.n_real) ? sample(key, sg.x0 + k, dist, scale) : 0.0);
    };
    if (nt <= 1) {
      work(0, n);
      continue;
    }
    std::vector<std::thread> th;
    int64_t per = (n + nt - 1) / nt;
    for (int32_t w = 0; w < nt; ++w) {
      int64_t lo = (int64_t)w * per, hi = std::min(n, lo + per);
      if (lo < hi) th.emplace_back(work, lo, hi);
    }
    for (auto& t : th) t.join();
  }
  return 0;
}

// Host: values at arbitrary parameter indices (x < 0 gives a pad zero).
int synth_values_at(const int64_t* xs, int64_t n, uint64_t key, int32_t dist, double scale,
                    int32_t out_type, void* out, int32_t nthreads) {
  if (n < 0 || (n > 0 && (!xs || !out)) || nthreads < 1) return -1;
  auto work = [&](int64_t lo, int64_t hi) {
    for (int64_t k = lo; k < hi; ++k)
      store(out, out_type, k, xs[k] < 0 ? 0.0 : sample(key, xs[k], dist, scale));
  };
  int32_t nt = (int32_t)std::min<int64_t>(nthreads, std::max<int64_t>(1, n / 4096));
  std::vector<std::thread> th;
  int64_t per = (n + nt - 1) / std::max(1, nt);
  for (int32_t w = 0; w < nt; ++w) {
    int64_t lo = (int64_t)w * per, hi = std::min(n, lo + per);
    if (lo < hi) th.emplace_back(work, lo, hi);
  }
  for (auto& t : th) t.join();
  return 0;
}

// Device: fill `out` (device memory) over the segments on `stream`.
// Segment bounds are the caller's responsibility; they are checked against
// `out_len` here before any launch.
int synth_fill_device(void* out, int64_t out_len, int32_t out_type, const synth_seg* segs,
                      int32_t nseg, uint64_t key, int32_t dist, double scale, hipStream_t stream) {
  if (!out || (nseg > 0 && !segs)) return -1;
  for (int32_t s = 0; s < nseg; ++s) {
    const synth_seg& sg = segs[s];
    if (sg.dst_off < 0 || sg.n_real < 0 || sg.n_pad < 0 || sg.x0 < 0 ||
        sg.dst_off + sg.n_real + sg.n_pad > out_len)
      return -2;
  }
  for (int32_t s0 = 0; s0 < nseg; s0 += SEGS_PER_LAUNCH) {
    SegBatch b;
    int32_t cnt = std::min(SEGS_PER_LAUNCH, nseg - s0);
    int64_t maxn = 1;
    for (int32_t k = 0; k < cnt; ++k) {
      b.s[k] = segs[s0 + k];
      maxn = std::max(maxn, b.s[k].n_real + b.s[k].n_pad);
    }
    unsigned gx = (unsigned)std::min<int64_t>((maxn + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_kernel, dim3(gx, (unsigned)cnt), dim3(256), 0, stream, out, out_type,
                       b, key, dist, scale);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

}  // extern "C"
