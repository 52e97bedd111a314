// Per-token magnitude and direction of the cache's reconstruction against
// the original K or V (rndamp article on KVarN, "The Problem": the K error is
// one of token magnitude rather than of direction; "How It Works", closing
// paragraph: the method minimizes the magnitude component).
//
// The rotation y = x . H_128 / sqrt(128) is orthogonal, so norms and inner
// products are those of the rotated basis, where the cache reconstructs
// y_hat_j = (code_j - 1.5) r'_t c_j directly:
//   ratio  = ||y_hat|| / ||y||,   cosine = <y_hat, y> / (||y_hat|| ||y||).
// One wave64 per token (grid-stride over all tokens of the call); lane l
// holds channels 2 l and 2 l + 1. The rotation of x is an in-wave fast
// Walsh-Hadamard transform: channel bit 0 in-lane, bits 1-6 across lanes.
#include "kvarn_diag.h"

namespace kvarn {
namespace {

constexpr int kWaves = 4;  // waves per workgroup

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += lane_xor(v, m);
  return v;
}

template <bool kF32, bool kRotate>
__global__ __launch_bounds__(64 * kWaves) void token_error_kernel(DiagArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = a.capacity / T;
  const int64_t total = (int64_t)a.batch * a.heads * a.tokens;
  for (int64_t w = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); w < total;
       w += (int64_t)gridDim.x * kWaves) {
    const int64_t bh = w / a.tokens;
    const int tt = (int)(w - bh * a.tokens);
    const int64_t b = bh / a.heads, h = bh - b * a.heads;
    const int t = a.token_offset + tt;  // cache slot
    // ---- x, channels 2 lane and 2 lane + 1 -------------------------------
    const int64_t xo = b * a.sb + h * a.sh + (int64_t)tt * a.st + 2 * lane;
    float y0, y1;
    if constexpr (kF32) {
      const float2 v = *reinterpret_cast<const float2 *>(static_cast<const float *>(a.x) + xo);
      y0 = v.x;
      y1 = v.y;
    } else {
      const uint32_t u = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(a.x) + xo);
      y0 = bf16_lo(u);
      y1 = bf16_hi(u);
    }
    if constexpr (kRotate) {
      // channel bit 0 in-lane, channel bit k + 1 = lane bit k across lanes
      float s = y0 + y1, d = y0 - y1;
      y0 = s;
      y1 = d;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float p0 = lane_xor(y0, m), p1 = lane_xor(y1, m);
        const bool upper = lane & m;
        y0 = upper ? p0 - y0 : y0 + p0;
        y1 = upper ? p1 - y1 : y1 + p1;
      }
      y0 *= kInvSqrtD;
      y1 *= kInvSqrtD;
    }
    // ---- reconstruction in the rotated basis -----------------------------
    const int64_t chunk = t / T, tc = t % T;
    const uint8_t *cb = a.codes + (bh * nch + chunk) * CHUNK_BYTES;
    uint32_t q0, q1;
    if (a.kind == KVARN_K) {  // token row: channel j in byte j / 4, bits 2 (j % 4)
      const uint32_t byte = cb[tc * 32 + (lane >> 1)];
      const int sh = 4 * (lane & 1);
      q0 = (byte >> sh) & 3u;
      q1 = (byte >> (sh + 2)) & 3u;
    } else {  // channel rows: token tc in byte tc / 4, bits 2 (tc % 4)
      const int sh = 2 * (int)(tc & 3);
      q0 = (cb[(2 * lane) * 32 + (tc >> 2)] >> sh) & 3u;
      q1 = (cb[(2 * lane + 1) * 32 + (tc >> 2)] >> sh) & 3u;
    }
    const float rp = a.row_scale[bh * a.capacity + t];
    const float2 c = *reinterpret_cast<const float2 *>(a.col_scale + (bh * nch + chunk) * D + 2 * lane);
    const float z0 = ((float)q0 - 1.5f) * rp * c.x;
    const float z1 = ((float)q1 - 1.5f) * rp * c.y;
    // ---- norms and inner product ------------------------------------------
    const float aa = wave_sum(fmaf(y0, y0, y1 * y1));
    const float bb = wave_sum(fmaf(z0, z0, z1 * z1));
    const float ab = wave_sum(fmaf(y0, z0, y1 * z1));
    if (lane == 0) {
      float ratio, cosine;
      if (aa == 0.f && bb == 0.f) {
        ratio = 1.f;
        cosine = 1.f;
      } else if (aa == 0.f) {
        ratio = __builtin_inff();
        cosine = 0.f;
      } else if (bb == 0.f) {
        ratio = 0.f;
        cosine = 0.f;
      } else {
        ratio = sqrtf(bb) / sqrtf(aa);
        cosine = ab / (sqrtf(aa) * sqrtf(bb));
      }
      a.ratio[w] = ratio;
      a.cosine[w] = cosine;
    }
  }
}

}  // namespace

hipError_t launch_token_error(const DiagArgs &a, hipStream_t s) {
  const int64_t total = (int64_t)a.batch * a.heads * a.tokens;
  if (total == 0) return hipSuccess;
  const int64_t want = (total + kWaves - 1) / kWaves;
  const int64_t cap = 8LL * device_cus();
  const dim3 grid((unsigned)(want < cap ? want : cap));
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE);
  if (a.dtype == KVARN_DT_F32) {
    if (rot)
      hipLaunchKernelGGL((token_error_kernel<true, true>), grid, dim3(64 * kWaves), 0, s, a);
    else
      hipLaunchKernelGGL((token_error_kernel<true, false>), grid, dim3(64 * kWaves), 0, s, a);
  } else {
    if (rot)
      hipLaunchKernelGGL((token_error_kernel<false, true>), grid, dim3(64 * kWaves), 0, s, a);
    else
      hipLaunchKernelGGL((token_error_kernel<false, false>), grid, dim3(64 * kWaves), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvarn
