// One-token append into a KVarN cache on gfx950 (rndamp article on KVarN,
// "The Problem": the cache grows by one token per decoding step).
//
// One wave64 per (sequence, kv-head): lane l holds channels l + 64 i
// (i < D / 64; D = 64, 128 or 256). The token is rotated (Hadamard,
// unscaled: the 1/sqrt(D) is folded into the row scale as in the block
// quantizer; channel bits 6 and up inside the lane, bits 0..5 across lanes),
// coded against the column scales of its chunk (copied forward from the
// previous chunk when the token opens a chunk), with its own per-token range
// step. The block is not re-balanced here; with a window the token is also
// kept, as given, for the re-balancing of the chunk once it is full
// (kvarn_append_rebalance).
#include "kvarn_internal.h"

namespace kvarn {
namespace {

__device__ __forceinline__ uint32_t or_quad(uint32_t c) {
  c |= __float_as_uint(lane_xor<1>(__uint_as_float(c)));
  return c | __float_as_uint(lane_xor<2>(__uint_as_float(c)));
}

// One token of (sequence, kv-head) bh. kRotate = false: the token is already
// rotated (rotation absorbed into the model's weights).
template <int DA, bool kF32, bool kRotate>
__device__ __forceinline__ void append_token(const AppendArgs &a, int bh) {
  constexpr int KD = DA / 64;  // channels per lane
  const int b = bh / a.heads;
  const int lane = threadIdx.x;
  const int pos = a.pos[b];
  if (pos < 0 || pos >= a.capacity) return;  // uniform across the wave
  const int k = pos / T, slot = pos - k * T;
  const int64_t nch = a.capacity / T;

  float y[KD];  // channels lane + 64 i
  if constexpr (kF32) {
    const float *x = static_cast<const float *>(a.x) + (int64_t)bh * DA;
#pragma unroll
    for (int i = 0; i < KD; ++i) y[i] = x[lane + 64 * i];
    if (a.window) {
      float *w = static_cast<float *>(a.window) + ((int64_t)bh * T + slot) * DA;
#pragma unroll
      for (int i = 0; i < KD; ++i) w[lane + 64 * i] = y[i];
    }
  } else {
    const uint16_t *x = static_cast<const uint16_t *>(a.x) + (int64_t)bh * DA;
    uint16_t u[KD];
#pragma unroll
    for (int i = 0; i < KD; ++i) {
      u[i] = x[lane + 64 * i];
      y[i] = __uint_as_float((uint32_t)u[i] << 16);
    }
    if (a.window) {
      uint16_t *w = static_cast<uint16_t *>(a.window) + ((int64_t)bh * T + slot) * DA;
#pragma unroll
      for (int i = 0; i < KD; ++i) w[lane + 64 * i] = u[i];
    }
  }
  // rotation: channel bits 6 and up inside the lane, bits 0..5 across lanes
  if constexpr (kRotate) {
#pragma unroll
    for (int len = 1; len < KD; len <<= 1)
#pragma unroll
      for (int i = 0; i < KD; ++i)
        if ((i & len) == 0) {
          const float s = y[i] + y[i + len], d = y[i] - y[i + len];
          y[i] = s;
          y[i + len] = d;
        }
#pragma unroll
    for (int bit = 1; bit < 64; bit <<= 1) {
      const bool hi = (lane & bit) != 0;
#pragma unroll
      for (int i = 0; i < KD; ++i) {
        const float p = lane_xor(y[i], bit);
        y[i] = hi ? p - y[i] : y[i] + p;
      }
    }
  }

  float *col = a.col_scale + ((int64_t)bh * nch + k) * DA;
  float c[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) {
    if (slot == 0) {
      c[i] = k > 0 ? col[lane + 64 * i - DA] : 1.f;
      col[lane + 64 * i] = c[i];
    } else {
      c[i] = col[lane + 64 * i];
    }
  }
  float z[KD], m = 0.f;
#pragma unroll
  for (int i = 0; i < KD; ++i) {
    z[i] = y[i] * (1.f / c[i]);
    m = fmaxf(m, fabsf(z[i]));
  }
#pragma unroll
  for (int bit = 1; bit < 64; bit <<= 1) m = fmaxf(m, lane_xor(m, bit));
  if (lane == 0)
    a.row_scale[(int64_t)bh * a.capacity + pos] =
        m * (kRotate ? range_from_unscaled(DA) : kRangeFromRotated);
  const float qs = m > 0.f ? 2.f / m : 0.f;
  uint32_t q[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) q[i] = (uint32_t)fminf(fmaxf(fmaf(z[i], qs, 2.f), 0.f), 3.f);

  uint8_t *cb = a.codes + ((int64_t)bh * nch + k) * (T * DA / 4);
  if (a.kind == KVARN_K) {
    // token row (D/4 bytes): channel j -> byte j/4, bits 2 (j % 4). The four
    // lanes of quad j hold channels 4 j .. 4 j + 3 (and 64 i + the same):
    // their codes meet by ORs across the quad.
    const int sh = 2 * (lane & 3);
    uint32_t bq[KD];
#pragma unroll
    for (int i = 0; i < KD; ++i) bq[i] = or_quad(q[i] << sh);
    if ((lane & 3) == 0) {
#pragma unroll
      for (int i = 0; i < KD; ++i) cb[slot * (DA / 4) + 16 * i + (lane >> 2)] = (uint8_t)bq[i];
    }
  } else {
    // channel row j: token slot s -> byte s/4, bits 2 (s % 4). The field is
    // cleared and set by two atomics on its 32-bit word, which need no
    // read of the byte first (the other tokens of the word are kept); a
    // token that starts a byte clears the byte's three later fields too.
    const int byte = slot >> 2;
    const int shift = 8 * (byte & 3) + 2 * (slot & 3);
    const uint32_t field = ((slot & 3) == 0 ? 0xFFu : 3u) << shift;
#pragma unroll
    for (int i = 0; i < KD; ++i) {
      uint32_t *w = reinterpret_cast<uint32_t *>(cb + (lane + 64 * i) * 32 + (byte & ~3));
      __hip_atomic_fetch_and(w, ~field, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(w, q[i] << shift, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int DA, bool kF32, bool kRotate>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  append_token<DA, kF32, kRotate>(a, blockIdx.x);
}

// K and V of the same step in one launch: blockIdx.y picks the cache.
template <int DA, bool kF32, bool kRotate>
__global__ __launch_bounds__(64) void append_kv_kernel(AppendArgs k, AppendArgs v) {
  if (blockIdx.y == 0)
    append_token<DA, kF32, kRotate>(k, blockIdx.x);
  else
    append_token<DA, kF32, kRotate>(v, blockIdx.x);
}

template <int DA>
hipError_t launch_append_da(const AppendArgs &a, hipStream_t s) {
  const int blocks = a.batch * a.heads;
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE);
  if (a.dtype == KVARN_DT_F32) {
    if (rot)
      hipLaunchKernelGGL((append_kernel<DA, true, true>), dim3(blocks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<DA, true, false>), dim3(blocks), dim3(64), 0, s, a);
  } else {
    if (rot)
      hipLaunchKernelGGL((append_kernel<DA, false, true>), dim3(blocks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<DA, false, false>), dim3(blocks), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

template <int DA>
hipError_t launch_append_kv_da(const AppendArgs &k, const AppendArgs &v, hipStream_t s) {
  const dim3 grid(k.batch * k.heads, 2);
  const bool rot = !(k.flags & KVARN_FLAG_NO_ROTATE);
  if (k.dtype == KVARN_DT_F32) {
    if (rot)
      hipLaunchKernelGGL((append_kv_kernel<DA, true, true>), grid, dim3(64), 0, s, k, v);
    else
      hipLaunchKernelGGL((append_kv_kernel<DA, true, false>), grid, dim3(64), 0, s, k, v);
  } else {
    if (rot)
      hipLaunchKernelGGL((append_kv_kernel<DA, false, true>), grid, dim3(64), 0, s, k, v);
    else
      hipLaunchKernelGGL((append_kv_kernel<DA, false, false>), grid, dim3(64), 0, s, k, v);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_kv(const AppendArgs &k, const AppendArgs &v, hipStream_t s) {
  if (k.batch * k.heads == 0) return hipSuccess;
  switch (k.head_dim) {
    case 64: return launch_append_kv_da<64>(k, v, s);
    case 256: return launch_append_kv_da<256>(k, v, s);
    default: return launch_append_kv_da<128>(k, v, s);
  }
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  if (a.batch * a.heads == 0) return hipSuccess;
  switch (a.head_dim) {
    case 64: return launch_append_da<64>(a, s);
    case 256: return launch_append_da<256>(a, s);
    default: return launch_append_da<128>(a, s);
  }
}

}  // namespace kvarn
