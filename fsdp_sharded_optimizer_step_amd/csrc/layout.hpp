// Internal definition of the layouts (host only).
//
// Page "Infra: Data Parallel" (pufanyi.com): "Naive Data Parallelism"
// (buckets), "Zero Redundancy Optimizer (ZeRO)" (GPU i keeps part i),
// "FSDP1" (flatten, concatenate, split evenly; a cut may pass through a
// tensor), "FSDP2" (every parameter split along dim 0 on its own).
//
// Two kinds:
//   FIXED_CUT  the flat stream cut every `cap` elements, each bucket padded to
//              a multiple of n_d.  Every quantity is closed-form arithmetic on
//              the capacity, so device code addresses any bucket without a table.
//   DIM0       one bucket per tensor, padded to n_d * ceil(rows/n_d) rows
//              (FSDP2); per-bucket values live in tables.
#pragma once

#include <cstdint>
#include <vector>

struct zero_layout {
  enum Kind : int32_t { FIXED_CUT = 0, DIM0 = 1 };
  int32_t kind = FIXED_CUT;
  int32_t n_d = 1, rank = 0;
  int64_t psi = 0;      // total elements in the stream
  int64_t cap = 0;      // FIXED_CUT: effective bucket capacity (psi when one bucket)
  int64_t nb = 0;       // number of buckets
  int64_t s_full = 0;   // FIXED_CUT: slice length of a full bucket
  int64_t p_full = 0;   // FIXED_CUT: padded length of a full bucket (= n_d * s_full)
  int64_t len_last = 0, s_last = 0, p_last = 0;  // FIXED_CUT: the last bucket
  int64_t P = 0, S = 0;                          // padded total, shard length
  std::vector<int64_t> numel, tensor_off;
  // DIM0 tables, one entry per bucket (= tensor)
  std::vector<int64_t> t_len, t_slice, t_padded_off, t_shard_off;

  bool fixed() const { return kind == FIXED_CUT; }
  int64_t bucket_len(int64_t b) const { return fixed() ? (b + 1 < nb ? cap : len_last) : t_len[b]; }
  int64_t bucket_slice(int64_t b) const {
    return fixed() ? (b + 1 < nb ? s_full : s_last) : t_slice[b];
  }
  int64_t bucket_padded(int64_t b) const { return bucket_slice(b) * n_d; }
  int64_t bucket_stream_off(int64_t b) const { return fixed() ? b * cap : tensor_off[b]; }
  int64_t bucket_padded_off(int64_t b) const { return fixed() ? b * p_full : t_padded_off[b]; }
  int64_t bucket_shard_off(int64_t b) const { return fixed() ? b * s_full : t_shard_off[b]; }
};
