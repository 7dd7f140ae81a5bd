// Mapping of the factorization's device status words to the C-ABI status of
// gptq_prepare_hinv (plain C++: no device code, so it is checked on its own).
//
// The preparation leaves two words in its workspace:
//   pivot_word  smallest failing pivot in the factorization's own (reversed)
//               column order, or INT_MAX when every pivot was positive;
//   stall_word  non-zero when any wave of any panel workgroup ran out of its
//               bounded wait for another wave's published step.
// A stall means the panel went on with stale data, so nothing it produced
// can be trusted (a failing pivot seen after it may be an artefact of it):
// it is reported as GPTQ_ERR_INTERNAL, never as a failed pivot.  A failed
// pivot is reported as GPTQ_ERR_NOT_SPD with its index in the quantization
// order (the factorization runs on the reversed matrix).
#pragma once

#include <climits>
#include <cstdint>

#include "gptq.h"

namespace gq {

inline int prepare_status(int32_t pivot_word, int32_t stall_word, int64_t d, int64_t* pivot) {
  if (pivot) *pivot = -1;
  if (stall_word != 0) return GPTQ_ERR_INTERNAL;
  if (pivot_word == INT_MAX) return GPTQ_OK;
  if (pivot_word < 0 || pivot_word >= d) return GPTQ_ERR_INTERNAL;
  if (pivot) *pivot = d - 1 - (int64_t)pivot_word;
  return GPTQ_ERR_NOT_SPD;
}

}  // namespace gq
