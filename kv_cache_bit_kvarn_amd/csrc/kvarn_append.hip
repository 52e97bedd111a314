// One-token append into a KVarN cache on gfx950 (rndamp article on KVarN,
// "The Problem": the cache grows by one token per decoding step).
//
// One wave64 per (sequence, kv-head): lane l holds channels l and l + 64.
// The token is rotated (Hadamard, unscaled: the 1/sqrt(128) is folded into
// the row scale as in the block quantizer), coded against the column scales
// of its chunk (copied forward from the previous chunk when the token opens
// a chunk), with its own per-token range step. The block is not re-balanced
// here; with a window the token is also kept, as given, for the re-balancing
// of the chunk once it is full (kvarn_append_rebalance).
#include "kvarn_internal.h"

namespace kvarn {
namespace {

__device__ __forceinline__ uint32_t or_quad(uint32_t c) {
  c |= __float_as_uint(lane_xor<1>(__uint_as_float(c)));
  return c | __float_as_uint(lane_xor<2>(__uint_as_float(c)));
}

// kRotate = false: the token is already rotated (rotation absorbed into the
// model's weights).
template <bool kF32, bool kRotate>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.heads;
  const int lane = threadIdx.x;
  const int pos = a.pos[b];
  if (pos < 0 || pos >= a.capacity) return;  // uniform across the wave
  const int k = pos / T, slot = pos - k * T;
  const int64_t nch = a.capacity / T;

  float y0, y1;  // channels lane, lane + 64
  if constexpr (kF32) {
    const float *x = static_cast<const float *>(a.x) + (int64_t)bh * D;
    y0 = x[lane];
    y1 = x[lane + 64];
    if (a.window) {
      float *w = static_cast<float *>(a.window) + ((int64_t)bh * T + slot) * D;
      w[lane] = y0;
      w[lane + 64] = y1;
    }
  } else {
    const uint16_t *x = static_cast<const uint16_t *>(a.x) + (int64_t)bh * D;
    const uint16_t u0 = x[lane], u1 = x[lane + 64];
    y0 = __uint_as_float((uint32_t)u0 << 16);
    y1 = __uint_as_float((uint32_t)u1 << 16);
    if (a.window) {
      uint16_t *w = static_cast<uint16_t *>(a.window) + ((int64_t)bh * T + slot) * D;
      w[lane] = u0;
      w[lane + 64] = u1;
    }
  }
  // rotation: channel bit 6 inside the lane, bits 0..5 across lanes
  if constexpr (kRotate) {
    const float s = y0 + y1, d = y0 - y1;
    y0 = s;
    y1 = d;
#pragma unroll
    for (int bit = 1; bit < 64; bit <<= 1) {
      const float p0 = lane_xor(y0, bit), p1 = lane_xor(y1, bit);
      const bool hi = (lane & bit) != 0;
      y0 = hi ? p0 - y0 : y0 + p0;
      y1 = hi ? p1 - y1 : y1 + p1;
    }
  }

  float *col = a.col_scale + ((int64_t)bh * nch + k) * D;
  float c0, c1;
  if (slot == 0) {
    if (k > 0) {
      c0 = col[lane - D];
      c1 = col[lane + 64 - D];
    } else {
      c0 = 1.f;
      c1 = 1.f;
    }
    col[lane] = c0;
    col[lane + 64] = c1;
  } else {
    c0 = col[lane];
    c1 = col[lane + 64];
  }
  const float z0 = y0 * (1.f / c0), z1 = y1 * (1.f / c1);
  float m = fmaxf(fabsf(z0), fabsf(z1));
#pragma unroll
  for (int bit = 1; bit < 64; bit <<= 1) m = fmaxf(m, lane_xor(m, bit));
  if (lane == 0)
    a.row_scale[(int64_t)bh * a.capacity + pos] = m * (kRotate ? kRangeFromUnscaled : kRangeFromRotated);
  const float qs = m > 0.f ? 2.f / m : 0.f;
  const uint32_t q0 = (uint32_t)fminf(fmaxf(fmaf(z0, qs, 2.f), 0.f), 3.f);
  const uint32_t q1 = (uint32_t)fminf(fmaxf(fmaf(z1, qs, 2.f), 0.f), 3.f);

  uint8_t *cb = a.codes + ((int64_t)bh * nch + k) * CHUNK_BYTES;
  if (a.kind == KVARN_K) {
    // token row: channel j -> byte j/4, bits 2 (j % 4). The four lanes of
    // quad j hold channels 4 j .. 4 j + 3 (and 64 + the same): their codes
    // meet by ORs across the quad.
    const int sh = 2 * (lane & 3);
    const uint32_t b0 = or_quad(q0 << sh), b1 = or_quad(q1 << sh);
    if ((lane & 3) == 0) {
      cb[slot * 32 + (lane >> 2)] = (uint8_t)b0;
      cb[slot * 32 + 16 + (lane >> 2)] = (uint8_t)b1;
    }
  } else {
    // channel row j: token slot s -> byte s/4, bits 2 (s % 4). The field is
    // cleared and set by two atomics on its 32-bit word, which need no
    // read of the byte first (the other tokens of the word are kept); a
    // token that starts a byte clears the byte's three later fields too.
    const int byte = slot >> 2;
    const int shift = 8 * (byte & 3) + 2 * (slot & 3);
    const uint32_t field = ((slot & 3) == 0 ? 0xFFu : 3u) << shift;
    uint32_t *w0 = reinterpret_cast<uint32_t *>(cb + lane * 32 + (byte & ~3));
    uint32_t *w1 = reinterpret_cast<uint32_t *>(cb + (lane + 64) * 32 + (byte & ~3));
    __hip_atomic_fetch_and(w0, ~field, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_and(w1, ~field, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(w0, q0 << shift, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(w1, q1 << shift, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  const int blocks = a.batch * a.heads;
  if (blocks == 0) return hipSuccess;
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE);
  if (a.dtype == KVARN_DT_F32) {
    if (rot)
      hipLaunchKernelGGL((append_kernel<true, true>), dim3(blocks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<true, false>), dim3(blocks), dim3(64), 0, s, a);
  } else {
    if (rot)
      hipLaunchKernelGGL((append_kernel<false, true>), dim3(blocks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<false, false>), dim3(blocks), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvarn
