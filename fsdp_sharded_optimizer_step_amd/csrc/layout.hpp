// Internal definition of the fixed-cut bucketed flat layout (host only).
//
// Page "Infra: Data Parallel" (pufanyi.com): "Naive Data Parallelism"
// (buckets), "Zero Redundancy Optimizer (ZeRO)" (GPU i keeps part i),
// "FSDP1" (flatten, concatenate, split evenly; a cut may pass through a
// tensor).  Every quantity here is closed-form arithmetic on the bucket
// capacity, so device code can address any bucket without a table.
#pragma once

#include <cstdint>
#include <vector>

struct zero_layout {
  int32_t n_d = 1, rank = 0;
  int64_t psi = 0;      // total elements in the stream
  int64_t cap = 0;      // effective bucket capacity (psi when one bucket)
  int64_t nb = 0;       // number of buckets
  int64_t s_full = 0;   // slice length of a full bucket
  int64_t p_full = 0;   // padded length of a full bucket (= n_d * s_full)
  int64_t len_last = 0, s_last = 0, p_last = 0;  // the last bucket
  int64_t P = 0, S = 0;                          // padded total, shard length
  std::vector<int64_t> numel, tensor_off;

  int64_t bucket_len(int64_t b) const { return b + 1 < nb ? cap : len_last; }
  int64_t bucket_slice(int64_t b) const { return b + 1 < nb ? s_full : s_last; }
  int64_t bucket_padded(int64_t b) const { return b + 1 < nb ? p_full : p_last; }
  int64_t bucket_stream_off(int64_t b) const { return b * cap; }
  int64_t bucket_padded_off(int64_t b) const { return b * p_full; }
  int64_t bucket_shard_off(int64_t b) const { return b * s_full; }
};
