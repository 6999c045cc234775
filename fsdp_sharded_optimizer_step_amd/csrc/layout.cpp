// Layout planner of the C ABI (host code).  See zero_shard.h for the
// definition of the layout and layout.hpp for the closed-form quantities.
#include <algorithm>
#include <limits>
#include <new>

#include "layout.hpp"
#include "zero_shard.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Owned stream interval [lo, hi) of bucket b for this rank (empty when the
// rank's slice lies entirely in the bucket's padding).
void owned_interval(const zero_layout& L, int64_t b, int64_t& lo, int64_t& hi) {
  const int64_t sb = L.bucket_slice(b), base = L.bucket_stream_off(b);
  lo = base + (int64_t)L.rank * sb;
  hi = base + std::min((int64_t)(L.rank + 1) * sb, L.bucket_len(b));
  if (hi < lo) hi = lo;
}

}  // namespace

extern "C" {

int zero_layout_create(const int64_t* numel, int32_t n_tensors, int64_t bucket_cap, int32_t n_d,
                       int32_t rank, zero_layout** out) {
  if (!out || n_tensors < 0 || (n_tensors > 0 && !numel)) return ZERO_EINVAL;
  if (n_d < 1 || n_d > ZERO_MAX_ND) return ZERO_EINVAL;
  if (rank < 0 || rank >= n_d) return ZERO_ERANGE;
  int64_t psi = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (numel[t] < 0) return ZERO_EINVAL;
    if (numel[t] > std::numeric_limits<int64_t>::max() / 4 - psi) return ZERO_ERANGE;
    psi += numel[t];
  }
  zero_layout* L = new (std::nothrow) zero_layout;
  if (!L) return ZERO_EINVAL;
  L->n_d = n_d;
  L->rank = rank;
  L->psi = psi;
  L->numel.assign(numel, numel + n_tensors);
  L->tensor_off.resize(n_tensors);
  for (int32_t t = 0; t < n_tensors; ++t)
    L->tensor_off[t] = (t == 0) ? 0 : L->tensor_off[t - 1] + L->numel[t - 1];
  if (psi > 0) {
    L->cap = (bucket_cap <= 0 || bucket_cap > psi) ? psi : bucket_cap;
    L->nb = ceil_div(psi, L->cap);
    L->s_full = ceil_div(L->cap, n_d);
    L->p_full = L->s_full * n_d;
    L->len_last = psi - (L->nb - 1) * L->cap;
    L->s_last = ceil_div(L->len_last, n_d);
    L->p_last = L->s_last * n_d;
    L->P = (L->nb - 1) * L->p_full + L->p_last;
    L->S = (L->nb - 1) * L->s_full + L->s_last;
  }
  *out = L;
  return ZERO_OK;
}

int zero_layout_create_dim0(const int64_t* numel, const int64_t* rows, int32_t n_tensors,
                            int32_t n_d, int32_t rank, zero_layout** out) {
  if (!out || n_tensors < 0 || (n_tensors > 0 && (!numel || !rows))) return ZERO_EINVAL;
  if (n_d < 1 || n_d > ZERO_MAX_ND) return ZERO_EINVAL;
  if (rank < 0 || rank >= n_d) return ZERO_ERANGE;
  int64_t psi = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    const int64_t r = rows[t], n = numel[t];
    if (n < 0 || r < 0 || (r == 0 && n != 0) || (r > 0 && n % r != 0)) return ZERO_EINVAL;
    if (n > std::numeric_limits<int64_t>::max() / 4 - psi) return ZERO_ERANGE;
    psi += n;
  }
  zero_layout* L = new (std::nothrow) zero_layout;
  if (!L) return ZERO_EINVAL;
  L->kind = zero_layout::DIM0;
  L->n_d = n_d;
  L->rank = rank;
  L->psi = psi;
  L->numel.assign(numel, numel + n_tensors);
  L->nb = n_tensors;
  L->tensor_off.resize(n_tensors);
  L->t_len.resize(n_tensors);
  L->t_slice.resize(n_tensors);
  L->t_padded_off.resize(n_tensors);
  L->t_shard_off.resize(n_tensors);
  int64_t off = 0, poff = 0, soff = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    const int64_t r = rows[t], n = numel[t];
    const int64_t per_row = r > 0 ? n / r : 0;
    const int64_t slice = ceil_div(r, n_d) * per_row;
    L->tensor_off[t] = off;
    L->t_len[t] = n;
    L->t_slice[t] = slice;
    L->t_padded_off[t] = poff;
    L->t_shard_off[t] = soff;
    off += n;
    poff += slice * n_d;
    soff += slice;
  }
  L->P = poff;
  L->S = soff;
  *out = L;
  return ZERO_OK;
}

int32_t zero_layout_kind(const zero_layout* L) { return L ? L->kind : -1; }

void zero_layout_destroy(zero_layout* layout) { delete layout; }

int64_t zero_layout_psi(const zero_layout* L) { return L ? L->psi : -1; }
int64_t zero_layout_padded(const zero_layout* L) { return L ? L->P : -1; }
int64_t zero_layout_shard(const zero_layout* L) { return L ? L->S : -1; }
int64_t zero_layout_n_buckets(const zero_layout* L) { return L ? L->nb : -1; }
int32_t zero_layout_n_d(const zero_layout* L) { return L ? L->n_d : -1; }
int32_t zero_layout_rank(const zero_layout* L) { return L ? L->rank : -1; }

int zero_layout_bucket(const zero_layout* L, int64_t b, int64_t* stream_off, int64_t* len,
                       int64_t* padded_off, int64_t* padded_len, int64_t* shard_off) {
  if (!L) return ZERO_EINVAL;
  if (b < 0 || b >= L->nb) return ZERO_ERANGE;
  if (stream_off) *stream_off = L->bucket_stream_off(b);
  if (len) *len = L->bucket_len(b);
  if (padded_off) *padded_off = L->bucket_padded_off(b);
  if (padded_len) *padded_len = L->bucket_padded(b);
  if (shard_off) *shard_off = L->bucket_shard_off(b);
  return ZERO_OK;
}

int zero_layout_tensor(const zero_layout* L, int32_t t, int64_t* stream_off, int64_t* shard_lo,
                       int64_t* shard_hi) {
  if (!L) return ZERO_EINVAL;
  if (t < 0 || t >= (int32_t)L->numel.size()) return ZERO_ERANGE;
  const int64_t a = L->tensor_off[t], z = a + L->numel[t];
  if (stream_off) *stream_off = a;
  int64_t lo = 0, hi = 0;
  if (z > a) {
    const int64_t b_first = L->fixed() ? a / L->cap : t;
    const int64_t b_last = L->fixed() ? (z - 1) / L->cap : t;
    bool found = false;
    for (int64_t b = b_first; b <= b_last && !found; ++b) {
      int64_t olo, ohi;
      owned_interval(*L, b, olo, ohi);
      const int64_t x0 = std::max(a, olo), x1 = std::min(z, ohi);
      if (x0 < x1) {
        lo = L->bucket_shard_off(b) + (x0 - olo);
        found = true;
      }
    }
    if (found) {
      for (int64_t b = b_last; b >= b_first; --b) {
        int64_t olo, ohi;
        owned_interval(*L, b, olo, ohi);
        const int64_t x0 = std::max(a, olo), x1 = std::min(z, ohi);
        if (x0 < x1) {
          hi = L->bucket_shard_off(b) + (x1 - olo);
          break;
        }
      }
    }
  }
  if (shard_lo) *shard_lo = lo;
  if (shard_hi) *shard_hi = hi;
  return ZERO_OK;
}

int zero_layout_tensor_flat(const zero_layout* L, int32_t t, int64_t* flat_lo, int64_t* flat_hi) {
  if (!L) return ZERO_EINVAL;
  if (t < 0 || t >= (int32_t)L->numel.size()) return ZERO_ERANGE;
  const int64_t a = L->tensor_off[t], n = L->numel[t];
  int64_t lo, hi;
  if (!L->fixed()) {
    // the tensor's real rows open its padded slot
    lo = L->t_padded_off[t];
    hi = lo + n;
  } else {
    // stream position x lies in bucket x / cap, at the same offset from the
    // bucket's start in the padded flat buffer
    auto flat = [&](int64_t x) { return (x / L->cap) * L->p_full + x % L->cap; };
    lo = a < L->psi ? flat(a) : L->P;
    hi = n > 0 ? flat(a + n - 1) + 1 : lo;
  }
  if (flat_lo) *flat_lo = lo;
  if (flat_hi) *flat_hi = hi;
  return ZERO_OK;
}

const char* zero_strerror(int status) {
  switch (status) {
    case ZERO_OK: return "ok";
    case ZERO_EINVAL: return "invalid argument";
    case ZERO_ERANGE: return "index or size out of range";
    case ZERO_EHIP: return "HIP call or kernel launch failed";
    case ZERO_EOVERLAP: return "output buffer overlaps another buffer";
    default: return "unknown status";
  }
}

}  // extern "C"
