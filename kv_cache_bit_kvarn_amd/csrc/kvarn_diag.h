// Launcher of the per-token error diagnostic (kvarn_token_error).
#pragma once

#include "kvarn_internal.h"

namespace kvarn {

struct DiagArgs {
  const void *x;
  int dtype;
  int head_dim;
  int64_t sb, sh, st;
  int batch, heads, tokens, token_offset, capacity, kind;
  uint32_t flags;  // KVARN_FLAG_NO_ROTATE
  const uint8_t *codes;
  const float *row_scale, *col_scale;
  float *ratio, *cosine;
};
hipError_t launch_token_error(const DiagArgs &a, hipStream_t s);

}  // namespace kvarn
