// Offsets rules of the C ABI, checked per sequence. The same function serves the host
// (gdpa_validate_offsets, on host copies of the offsets) and the device (the validation kernel
// enqueued by GDPA_FLAG_VALIDATE / GDPA_DEBUG=1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdpa.h"

namespace gdpa {

// What the offsets of one problem must satisfy.
struct OffsetsRules {
  int32_t num_seqs;
  int32_t self_attention;  // query and key sequences are the same rows
  int64_t total_q, total_kv;
  int64_t max_q, max_kv;   // max_seqlen_q (also the rows of a shared query matrix), max_seqlen_kv
};

// GDPA_DEVICE_ERR_* bits of sequence b (0 <= b < num_seqs): its row ranges are ordered and inside
// [0, total], the first starts at 0 and the last ends at the totals, its lengths are within the
// hints, and self-attention sequences coincide.
__host__ __device__ inline int32_t seq_offsets_error(const OffsetsRules& r, const int32_t* qo, const int32_t* ko,
                                                     int b) {
  const int64_t q0 = qo[b], q1 = qo[b + 1], k0 = ko[b], k1 = ko[b + 1];
  int32_t e = 0;
  if (q0 < 0 || q1 < q0 || q1 > r.total_q || k0 < 0 || k1 < k0 || k1 > r.total_kv) e |= GDPA_DEVICE_ERR_OFFSETS;
  if (b == 0 && (q0 != 0 || k0 != 0)) e |= GDPA_DEVICE_ERR_OFFSETS;
  if (b == r.num_seqs - 1 && (q1 != r.total_q || k1 != r.total_kv)) e |= GDPA_DEVICE_ERR_OFFSETS;
  if (q1 - q0 > r.max_q || k1 - k0 > r.max_kv) e |= GDPA_DEVICE_ERR_LENGTH;
  if (r.self_attention && (q0 != k0 || q1 != k1)) e |= GDPA_DEVICE_ERR_SELF;
  return e;
}

}  // namespace gdpa
