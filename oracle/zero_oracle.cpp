// CPU oracle for the ZeRO / FSDP shard-local update.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
// calls this file; only the test suite, the smoke check and the benchmark's
// CPU-baseline leg use it.  It shares no code, header, table or helper with
// the HIP path.
//
// It is written to be plain and slow: one scalar loop per element, every fp32
// operation in the order the update defines it, no blocking and no fusion.
// Build flags (see build_oracle.py): -O2 -ffp-contract=off, no fast-math, so
// each `a*b + c` is two separately rounded IEEE-754 binary32 operations and
// subnormals are kept.
//
// Sources followed (page titles and sections):
//   [DP]   "Infra: Data Parallel" (pufanyi.com), sections
//          "Naive Data Parallelism", "Zero Redundancy Optimizer (ZeRO)",
//          "Fully Sharded Data Parallel (FSDP)" / "FSDP1".
//   [FACT] "FSDP" knowledge card (kongchang.com), Core Facts: the float
//          accumulation order of communication operators depends on the
//          parallel configuration, so determinism has to be checked.
//
// Parity status of each entry point (what pins it) is recorded next to it.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

float f32_from_bits(uint32_t b) {
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}

uint32_t bits_from_f32(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  return b;
}

// bf16 is the upper half of a binary32, so widening is exact.
float widen_bf16(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

// Round a binary32 to the nearest bfloat16, ties to the even significand.
// Written from the definition, not from a bit trick: take the two bf16
// neighbours of x (x truncated toward zero, and the next bf16 away from zero),
// measure both distances exactly in binary64, keep the nearer one, and on a
// tie keep the one whose last significand bit is 0.  A value at or beyond the
// midpoint between the largest finite bf16 and 2^128 goes to infinity, as
// IEEE-754 round-to-nearest prescribes.  NaN stays NaN: sign and top payload
// bits kept, quiet bit set.
uint16_t round_bf16(float x) {
  uint32_t b = bits_from_f32(x);
  uint32_t mag = b & 0x7fffffffu;
  if (mag > 0x7f800000u) return (uint16_t)((b >> 16) | 0x0040u);  // NaN
  if (mag == 0x7f800000u) return (uint16_t)(b >> 16);               // +-inf
  uint32_t lo_bits = b & 0xffff0000u;           // toward zero
  double lo = (double)f32_from_bits(lo_bits);
  if ((double)x == lo) return (uint16_t)(lo_bits >> 16);
  uint32_t hi_bits = lo_bits + 0x00010000u;     // next bf16 away from zero
  double hi;
  if ((hi_bits & 0x7fffffffu) == 0x7f800000u)
    hi = std::ldexp((x < 0) ? -1.0 : 1.0, 128);  // the would-be next value
  else
    hi = (double)f32_from_bits(hi_bits);
  double dlo = std::fabs((double)x - lo);
  double dhi = std::fabs(hi - (double)x);
  if (dlo < dhi) return (uint16_t)(lo_bits >> 16);
  if (dhi < dlo) return (uint16_t)(hi_bits >> 16);
  return ((lo_bits >> 16) & 1u) ? (uint16_t)(hi_bits >> 16) : (uint16_t)(lo_bits >> 16);
}

// ---------------------------------------------------------------------------
// Layout: [DP] "Naive Data Parallelism" (grads of many parameters share one
// bucket), "Zero Redundancy Optimizer (ZeRO)" (GPU i keeps the i-th part of
// each state; ZeRO-2 reduces per bucket and keeps the owned part) and
// "FSDP1" (flatten and concatenate the unit's tensors, then split the flat
// buffer evenly; a cut may fall inside a tensor; a rank's view of a tensor may
// be partial or empty).
//
// Reading used here: the tensors form one flat stream in list order; the
// stream is cut every `cap` elements (cap <= 0: one bucket); each bucket is
// zero-padded at its end to a multiple of n_d; rank r owns the r-th of the
// n_d equal slices of every padded bucket; a rank's shard is its slices in
// bucket order.
struct Plan {
  int64_t total = 0;                       // sum of numel (Psi)
  std::vector<int64_t> stream_off, len;    // per bucket, in the unpadded stream
  std::vector<int64_t> padded_off, padded_len, shard_off;
  int64_t padded_total = 0, shard_len = 0;
};

// What a layout is made from.  rows == nullptr: the bucketed flat layout
// above (cut every `cap` elements).  rows != nullptr: FSDP2's per-parameter
// sharding ([DP] "FSDP2": each parameter is split along dim 0; a rank keeps
// ceil(rows/n_d) rows of every parameter, the last ranks' pieces padded with
// zero rows): one bucket per tensor, padded to n_d * ceil(rows/n_d) rows.
struct Spec {
  const int64_t* numel;
  const int64_t* rows;
  int32_t n_tensors;
  int64_t cap;
  int32_t n_d;
};

void add_bucket(Plan& p, int64_t pos, int64_t l, int64_t pl, int32_t n_d) {
  p.stream_off.push_back(pos);
  p.len.push_back(l);
  p.padded_off.push_back(p.padded_total);
  p.padded_len.push_back(pl);
  p.shard_off.push_back(p.shard_len);
  p.padded_total += pl;
  p.shard_len += pl / n_d;
}

Plan make_plan(const Spec& sp) {
  Plan p;
  const int32_t n_d = sp.n_d;
  for (int32_t t = 0; t < sp.n_tensors; ++t) p.total += sp.numel[t];
  if (sp.rows) {
    int64_t pos = 0;
    for (int32_t t = 0; t < sp.n_tensors; ++t) {
      const int64_t r = sp.rows[t], n = sp.numel[t];
      const int64_t per_row = r > 0 ? n / r : 0;
      const int64_t c = (r + n_d - 1) / n_d;
      add_bucket(p, pos, n, (int64_t)n_d * c * per_row, n_d);
      pos += n;
    }
    return p;
  }
  int64_t c = (sp.cap <= 0) ? p.total : sp.cap;
  int64_t pos = 0;
  while (pos < p.total) {
    int64_t l = std::min(c, p.total - pos);
    add_bucket(p, pos, l, ((l + n_d - 1) / n_d) * n_d, n_d);
    pos += l;
  }
  return p;
}

bool spec_ok(const Spec* sp) {
  if (!sp || sp->n_tensors < 0 || sp->n_d < 1) return false;
  if (sp->n_tensors > 0 && !sp->numel) return false;
  for (int32_t t = 0; t < sp->n_tensors; ++t) {
    if (sp->numel[t] < 0) return false;
    if (sp->rows) {
      const int64_t r = sp->rows[t];
      if (r < 0 || (r == 0 && sp->numel[t] != 0) || (r > 0 && sp->numel[t] % r != 0)) return false;
    }
  }
  return true;
}

// Index of the bucket whose shard range holds shard index i (plain scan from
// a binary search start; buckets are in shard order).
int64_t bucket_of_shard_index(const Plan& p, int64_t i) {
  auto it = std::upper_bound(p.shard_off.begin(), p.shard_off.end(), i);
  return (int64_t)(it - p.shard_off.begin()) - 1;
}

// ---------------------------------------------------------------------------
// The shard-local AdamW step.
//
// [DP] "Zero Redundancy Optimizer (ZeRO)": AdamW is element-wise, so a rank
// that holds a slice of the parameters, the averaged gradient of that slice
// and the slice's moments can update it without any other part; the averaged
// gradient arrives through a Reduce-Scatter with averaging; the state is fp32
// master weights plus first and second moments (k = 12 bytes per parameter)
// and parameters/gradients are 16-bit.
//
// Readings used here (the pages name AdamW but print no formula):
//   reduce   a = widen(G_0); a = a + widen(G_q) for q = 1..n_d-1 in order;
//            g = a / n_d                          (fixed rank order, [FACT])
//   scalars  in binary64, each rounded once to binary32:
//            s = lr / (1 - b1^t), rho = 1 / sqrt(1 - b2^t), a_wd = 1 - lr*wd,
//            B1 = b1, C1 = 1 - b1, B2 = b2, C2 = 1 - b2, E = eps
//   element  m' = B1*m + C1*g
//            v' = B2*v + C2*(g*g)
//            d  = sqrt(v')*rho + E
//            th'= a_wd*th - s*(m'/d)
//            p  = bf16(th')
// This is decoupled-weight-decay AdamW with bias correction and eps added
// after the square root, with each operation rounded once.
struct Scalars {
  float s, rho, a_wd, B1, C1, B2, C2, E;
};

Scalars make_scalars(double lr, double b1, double b2, double eps, double wd, int64_t t) {
  double bc1 = 1.0 - std::pow(b1, (double)t);
  double bc2 = 1.0 - std::pow(b2, (double)t);
  Scalars k;
  k.s = (float)(lr / bc1);
  k.rho = (float)(1.0 / std::sqrt(bc2));
  k.a_wd = (float)(1.0 - lr * wd);
  k.B1 = (float)b1;
  k.C1 = (float)(1.0 - b1);
  k.B2 = (float)b2;
  k.C2 = (float)(1.0 - b2);
  k.E = (float)eps;
  return k;
}

float contribution(const uint16_t* g, int64_t i) { return widen_bf16(g[i]); }
float contribution(const float* g, int64_t i) { return g[i]; }

// Contributions are bf16 patterns (uint16_t) or binary32 values (float).
template <class T>
void step_range(int32_t n_d, const T* const* G, int64_t lo, int64_t hi, const Scalars& k,
                float* master, float* m, float* v, uint16_t* p_out, float* g_out) {
  const float nd = (float)n_d;
  for (int64_t i = lo; i < hi; ++i) {
    float a = contribution(G[0], i);
    for (int32_t q = 1; q < n_d; ++q) a = a + contribution(G[q], i);
    float g = a / nd;
    float m1 = k.B1 * m[i] + k.C1 * g;
    float v1 = k.B2 * v[i] + k.C2 * (g * g);
    float d = std::sqrt(v1) * k.rho + k.E;
    float th1 = k.a_wd * master[i] - k.s * (m1 / d);
    m[i] = m1;
    v[i] = v1;
    master[i] = th1;
    p_out[i] = round_bf16(th1);
    if (g_out) g_out[i] = g;
  }
}

template <class F>
void parallel_chunks(int64_t n, int32_t nthreads, F f) {
  if (nthreads <= 1 || n < 2) {
    f((int64_t)0, n);
    return;
  }
  std::vector<std::thread> th;
  int64_t per = (n + nthreads - 1) / nthreads;
  for (int32_t w = 0; w < nthreads; ++w) {
    int64_t lo = (int64_t)w * per, hi = std::min(n, lo + per);
    if (lo >= hi) break;
    th.emplace_back([=] { f(lo, hi); });
  }
  for (auto& t : th) t.join();
}

}  // namespace

extern "C" {

// --- Cast -------------------------------------------------------------------
// Pinned by: exhaustive comparison with torch's float32 -> bfloat16 conversion
// over all 2^32 inputs (tests).
void oracle_round_bf16(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(x[i]);
}

// Same, over every 32-bit pattern in [lo, hi): out[k] = bf16(pattern lo+k).
void oracle_round_bf16_patterns(uint64_t lo, uint64_t hi, uint16_t* out) {
  for (uint64_t b = lo; b < hi; ++b) out[b - lo] = round_bf16(f32_from_bits((uint32_t)b));
}

// --- Layout -----------------------------------------------------------------
// Pinned by: the FSDP1 worked example (golden fixture), brute force against an
// element-by-element planner on tiny inputs, and closed-form invariants.
// Returns 0, or -1 on bad arguments.
int oracle_plan_counts(const Spec* sp, int64_t* n_buckets, int64_t* padded_total,
                       int64_t* shard_len) {
  if (!spec_ok(sp)) return -1;
  Plan p = make_plan(*sp);
  *n_buckets = (int64_t)p.len.size();
  *padded_total = p.padded_total;
  *shard_len = p.shard_len;
  return 0;
}

// Per-bucket arrays, each of n_buckets entries.
int oracle_plan_buckets(const Spec* sp, int64_t* stream_off, int64_t* len, int64_t* padded_off,
                        int64_t* padded_len, int64_t* shard_off) {
  if (!spec_ok(sp)) return -1;
  Plan p = make_plan(*sp);
  for (size_t b = 0; b < p.len.size(); ++b) {
    stream_off[b] = p.stream_off[b];
    len[b] = p.len[b];
    padded_off[b] = p.padded_off[b];
    padded_len[b] = p.padded_len[b];
    shard_off[b] = p.shard_off[b];
  }
  return 0;
}

// For rank r: the smallest range [lo[t], hi[t]) of shard indices that holds
// every element of tensor t that r owns (lo == hi when r holds none of it).
// The shard lists owned stream positions in stream order and a tensor is a
// stream interval, so nothing of another tensor falls inside the range; bucket
// padding can (when a tensor continues past a padded bucket end).
int oracle_plan_tensor_ranges(const Spec* sp, int32_t rank, int64_t* lo, int64_t* hi) {
  if (!spec_ok(sp) || rank < 0 || rank >= sp->n_d) return -1;
  const int32_t n_d = sp->n_d;
  Plan p = make_plan(*sp);
  int64_t a = 0;
  for (int32_t t = 0; t < sp->n_tensors; ++t) {
    int64_t z = a + sp->numel[t];
    int64_t first = -1, last = -1;
    for (size_t b = 0; b < p.len.size(); ++b) {
      int64_t sb = p.padded_len[b] / n_d;
      int64_t own_lo = p.stream_off[b] + (int64_t)rank * sb;
      int64_t own_hi = p.stream_off[b] + std::min((int64_t)(rank + 1) * sb, p.len[b]);
      int64_t x0 = std::max(a, own_lo), x1 = std::min(z, own_hi);
      if (x0 >= x1) continue;
      int64_t s0 = p.shard_off[b] + (x0 - own_lo), s1 = p.shard_off[b] + (x1 - own_lo);
      if (first < 0) first = s0;
      last = s1;
    }
    lo[t] = (first < 0) ? 0 : first;
    hi[t] = (first < 0) ? 0 : last;
    a = z;
  }
  return 0;
}

// For rank r and n shard indices: the position in the padded flat buffer
// (`flat_pos`) and in the unpadded stream (`stream_pos`, -1 for a pad).
int oracle_plan_map(const Spec* sp, int32_t rank, const int64_t* idx, int64_t n,
                    int64_t* flat_pos, int64_t* stream_pos) {
  if (!spec_ok(sp) || rank < 0 || rank >= sp->n_d) return -1;
  const int32_t n_d = sp->n_d;
  Plan p = make_plan(*sp);
  for (int64_t k = 0; k < n; ++k) {
    if (idx[k] < 0 || idx[k] >= p.shard_len) return -1;
    int64_t b = bucket_of_shard_index(p, idx[k]);
    int64_t sb = p.padded_len[b] / n_d;
    int64_t in_bucket = (int64_t)rank * sb + (idx[k] - p.shard_off[b]);
    if (flat_pos) flat_pos[k] = p.padded_off[b] + in_bucket;
    if (stream_pos) stream_pos[k] = (in_bucket < p.len[b]) ? p.stream_off[b] + in_bucket : -1;
  }
  return 0;
}

// --- Bucket pack --------------------------------------------------------------
// [DP] "Naive Data Parallelism" / "FSDP1": the tensors' gradients are placed
// one after another in the flat buffer; padding is zero.
// Pinned by: brute force against a plain concatenation on tiny inputs and the
// FSDP1 example.
int oracle_pack(const uint16_t* const* tensors, const Spec* sp, uint16_t* flat_out) {
  if (!spec_ok(sp)) return -1;
  Plan p = make_plan(*sp);
  for (int64_t k = 0; k < p.padded_total; ++k) flat_out[k] = 0;
  int64_t x = 0, b = 0;  // stream position and the bucket holding it
  for (int32_t t = 0; t < sp->n_tensors; ++t) {
    for (int64_t e = 0; e < sp->numel[t]; ++e, ++x) {
      while (b + 1 < (int64_t)p.len.size() && p.stream_off[b + 1] <= x) ++b;
      flat_out[p.padded_off[b] + (x - p.stream_off[b])] = tensors[t][e];
    }
  }
  return 0;
}

// Gather rank r's shard (its slice of every bucket, in bucket order) out of a
// padded flat buffer.
int oracle_slice(const uint16_t* flat, const Spec* sp, int32_t rank, uint16_t* shard_out) {
  if (!spec_ok(sp) || rank < 0 || rank >= sp->n_d) return -1;
  const int32_t n_d = sp->n_d;
  Plan p = make_plan(*sp);
  for (size_t b = 0; b < p.len.size(); ++b) {
    int64_t sb = p.padded_len[b] / n_d;
    for (int64_t j = 0; j < sb; ++j)
      shard_out[p.shard_off[b] + j] = flat[p.padded_off[b] + (int64_t)rank * sb + j];
  }
  return 0;
}

// --- Parameter gather (local part of the All-Gather) ---------------------------
// [DP] "Zero Redundancy Optimizer (ZeRO)": after the step (ZeRO-1/2) or per
// layer before forward/backward (ZeRO-3) the ranks' parameter shards are
// All-Gathered into the full flat buffer: rank q's slice of every bucket
// goes back to slot q of that bucket.
// Pinned by: gather(slices of x) == x for packed x (inverse of the pinned
// slice), brute force on tiny layouts.
int oracle_gather(const uint16_t* const* shards, const Spec* sp, uint16_t* out) {
  if (!spec_ok(sp)) return -1;
  const int32_t n_d = sp->n_d;
  Plan p = make_plan(*sp);
  for (size_t b = 0; b < p.len.size(); ++b) {
    int64_t sb = p.padded_len[b] / n_d;
    for (int32_t q = 0; q < n_d; ++q)
      for (int64_t j = 0; j < sb; ++j)
        out[p.padded_off[b] + (int64_t)q * sb + j] = shards[q][p.shard_off[b] + j];
  }
  return 0;
}

// Stream positions -> (owning rank, index in that rank's shard).
int oracle_plan_locate(const Spec* sp, const int64_t* xs, int64_t n, int32_t* rank,
                       int64_t* idx) {
  if (!spec_ok(sp)) return -1;
  const int32_t n_d = sp->n_d;
  Plan p = make_plan(*sp);
  for (int64_t k = 0; k < n; ++k) {
    if (xs[k] < 0 || xs[k] >= p.total) return -1;
    auto it = std::upper_bound(p.stream_off.begin(), p.stream_off.end(), xs[k]);
    int64_t b = (int64_t)(it - p.stream_off.begin()) - 1;
    int64_t sb = p.padded_len[b] / n_d;
    int64_t w = xs[k] - p.stream_off[b];
    rank[k] = (int32_t)(w / sb);
    idx[k] = p.shard_off[b] + (w - (int64_t)rank[k] * sb);
  }
  return 0;
}

// --- Reshard between layouts (sharded checkpoint loaded with another N_d) ------
// [DP] "Fully Sharded Data Parallel (FSDP)" / "Checkpoint": every rank saves
// its shards; loading re-cuts them for the target sharding layout, which may
// use a different number of GPUs; optimizer state is saved and re-cut too.
// dst[i] = the value of the parameter at stream position x(i) in the source
// shards, 0 at destination padding.  elem_bytes is 2 or 4.
// Pinned by: identity on the same layout, A->B->A round trip, labelled
// elements landing at the brute-force planner's positions.
int oracle_reshard(const void* const* src, const Spec* src_sp, const Spec* dst_sp,
                   int32_t dst_rank, void* dst, int32_t elem_bytes) {
  if (!spec_ok(src_sp) || !spec_ok(dst_sp)) return -1;
  if (src_sp->n_tensors != dst_sp->n_tensors) return -1;
  for (int32_t t = 0; t < src_sp->n_tensors; ++t)
    if (src_sp->numel[t] != dst_sp->numel[t]) return -1;
  const int32_t src_nd = src_sp->n_d, dst_nd = dst_sp->n_d;
  if (dst_rank < 0 || dst_rank >= dst_nd || (elem_bytes != 2 && elem_bytes != 4)) return -1;
  Plan ps = make_plan(*src_sp);
  Plan pd = make_plan(*dst_sp);
  for (int64_t i = 0; i < pd.shard_len; ++i) {
    int64_t b = bucket_of_shard_index(pd, i);
    int64_t sb = pd.padded_len[b] / dst_nd;
    int64_t pos = (int64_t)dst_rank * sb + (i - pd.shard_off[b]);
    char* d = (char*)dst + i * elem_bytes;
    if (pos >= pd.len[b]) {
      std::memset(d, 0, elem_bytes);
      continue;
    }
    int64_t x = pd.stream_off[b] + pos;
    auto it = std::upper_bound(ps.stream_off.begin(), ps.stream_off.end(), x);
    int64_t bs = (int64_t)(it - ps.stream_off.begin()) - 1;
    int64_t ss = ps.padded_len[bs] / src_nd;
    int64_t w = x - ps.stream_off[bs];
    int64_t q = w / ss;
    int64_t j = ps.shard_off[bs] + (w - q * ss);
    std::memcpy(d, (const char*)src[q] + j * elem_bytes, elem_bytes);
  }
  return 0;
}

// --- no_sync gradient accumulation -------------------------------------------
// [DP] "Naive Data Parallelism": gradients of several micro-batches are summed
// locally and only the last one is synchronised; with n equal micro-batches
// whose losses are sample means, each loss is divided by n.
// Reading: acc = scale*g on the first micro-batch (overwrite), otherwise
// acc = acc + scale*g, each product and sum rounded once; optionally emit
// bf16(acc) as the rank's contribution.
// Pinned by: 4 micro-batches scaled by 1/4 equal the full-batch mean bitwise.
void oracle_accumulate(float* acc, const uint16_t* g, int64_t n, float scale, int32_t overwrite,
                       int32_t store_acc, uint16_t* emit_bf16) {
  for (int64_t i = 0; i < n; ++i) {
    float contrib = scale * widen_bf16(g[i]);
    float a = overwrite ? contrib : (acc[i] + contrib);
    if (store_acc) acc[i] = a;
    if (emit_bf16) emit_bf16[i] = round_bf16(a);
  }
}

// --- Step scalars -------------------------------------------------------------
// out = {s, rho, a_wd, B1, C1, B2, C2, E}
void oracle_step_scalars(double lr, double b1, double b2, double eps, double wd, int64_t t,
                         float* out) {
  Scalars k = make_scalars(lr, b1, b2, eps, wd, t);
  out[0] = k.s; out[1] = k.rho; out[2] = k.a_wd; out[3] = k.B1;
  out[4] = k.C1; out[5] = k.B2; out[6] = k.C2; out[7] = k.E;
}

// --- Reduce + AdamW + cast over one shard --------------------------------------
// G: host array of n_d pointers, each to n contributions in shard order.
// master/m/v are updated in place; p_out receives bf16(master'); g_out
// (nullable) receives the averaged gradient.  nthreads > 1 splits [0, n) into
// contiguous chunks, which does not change any element's arithmetic.
// Pinned by: the step-1 closed form, the g = 0 special case, torch.optim.AdamW
// in float64 within a derived rounding bound, a binary64 evaluation of the
// same update within a derived bound, and sharded == unsharded.
int oracle_shard_step(int32_t n_d, const uint16_t* const* G, int64_t n, double lr, double b1,
                      double b2, double eps, double wd, int64_t t, float* master, float* m,
                      float* v, uint16_t* p_out, float* g_out, int32_t nthreads) {
  if (n_d < 1 || n < 0 || t < 1 || !G) return -1;
  for (int32_t q = 0; q < n_d; ++q)
    if (!G[q] && n > 0) return -1;
  Scalars k = make_scalars(lr, b1, b2, eps, wd, t);
  parallel_chunks(n, nthreads, [&](int64_t lo, int64_t hi) {
    step_range(n_d, G, lo, hi, k, master, m, v, p_out, g_out);
  });
  return 0;
}

// Same update with binary32 contributions (a Reduce-Scatter carried out in
// fp32): a = G_0; a = a + G_q in ascending rank order; then as above.
// Pinned by: equality with oracle_shard_step when every contribution is a
// bf16 value, plus the rank-order and exact-sum cases in fp32.
int oracle_shard_step_f32(int32_t n_d, const float* const* G, int64_t n, double lr, double b1,
                          double b2, double eps, double wd, int64_t t, float* master, float* m,
                          float* v, uint16_t* p_out, float* g_out, int32_t nthreads) {
  if (n_d < 1 || n < 0 || t < 1 || !G) return -1;
  for (int32_t q = 0; q < n_d; ++q)
    if (!G[q] && n > 0) return -1;
  Scalars k = make_scalars(lr, b1, b2, eps, wd, t);
  parallel_chunks(n, nthreads, [&](int64_t lo, int64_t hi) {
    step_range(n_d, G, lo, hi, k, master, m, v, p_out, g_out);
  });
  return 0;
}

// --- Model-state memory accounting ----------------------------------------------
// [DP] "Zero Redundancy Optimizer (ZeRO)", memory figure: per-GPU bytes of
// 16-bit parameters, 16-bit gradients and k bytes of optimizer state per
// parameter, for the unsharded baseline and ZeRO stages 1-3.
// This sums the buffers a rank actually holds under each mode for a layout
// with padded total P and shard length S (mode 0 = baseline, 1..3 = stage).
// Pinned by: the page's closed forms with Psi -> P and N_d = P / S.
double oracle_model_state_bytes(int32_t mode, int64_t P, int64_t S, int32_t k_bytes) {
  double params = 2.0 * (double)((mode >= 3) ? S : P);
  double grads = 2.0 * (double)((mode >= 2) ? S : P);
  double state = (double)k_bytes * (double)((mode >= 1) ? S : P);
  return params + grads + state;
}

// [DP] "Zero Redundancy Optimizer (ZeRO)", communication-volume discussion:
// bytes one GPU sends per training step (one forward and one backward) under
// the ring model, parameters and gradients 16-bit, summed over every layer or
// bucket.  A ring Reduce-Scatter or All-Gather of a P-element buffer has each
// rank send N_d - 1 chunks of P / N_d elements; an All-Reduce is one of each.
//   mode 0 (naive DP): one gradient All-Reduce
//   mode 1, 2 (ZeRO-1, ZeRO-2): gradient Reduce-Scatter + parameter All-Gather
//   mode 3 (ZeRO-3): parameter All-Gather before forward and again before
//     backward, plus the gradient Reduce-Scatter
// Pinned by: a ring simulation that moves the data and counts the bytes, and
// the page's 4 Psi / 4 Psi / 6 Psi once the (N_d - 1) / N_d factor is dropped.
double oracle_comm_bytes_per_gpu(int32_t mode, int64_t P, int32_t n_d) {
  const double pass = 2.0 * (double)P * (double)(n_d - 1) / (double)n_d;  // one RS or AG
  const int passes = mode >= 3 ? 3 : 2;
  return pass * (double)passes;
}

}  // extern "C"
