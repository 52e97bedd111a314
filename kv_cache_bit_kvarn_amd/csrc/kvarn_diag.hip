// Per-token magnitude and direction of the cache's reconstruction against
// the original K or V (rndamp article on KVarN, "The Problem": the K error is
// one of token magnitude rather than of direction; "How It Works", closing
// paragraph: the method minimizes the magnitude component).
//
// The rotation y = x . H_D / sqrt(D) is orthogonal, so norms and inner
// products are those of the rotated basis, where the cache reconstructs
// y_hat_j = (code_j - 1.5) r'_t c_j directly:
//   ratio  = ||y_hat|| / ||y||,   cosine = <y_hat, y> / (||y_hat|| ||y||).
// One wave64 per token (grid-stride over all tokens of the call); lane l
// holds channels CPL l + i (CPL = D / 64 consecutive channels: 1, 2 or 4).
// The rotation of x is an in-wave fast Walsh-Hadamard transform: the low
// channel bits in-lane, the next six across lanes.
#include "kvarn_diag.h"

namespace kvarn {
namespace {

constexpr int kWaves = 4;  // waves per workgroup

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += lane_xor(v, m);
  return v;
}

// CPL consecutive fp32 values from a 4 CPL-byte aligned address
template <int CPL>
__device__ __forceinline__ void load_f32(const float *p, float (&v)[CPL]) {
  if constexpr (CPL == 1) {
    v[0] = p[0];
  } else if constexpr (CPL == 2) {
    const float2 u = *reinterpret_cast<const float2 *>(p);
    v[0] = u.x;
    v[1] = u.y;
  } else {
    const float4 u = *reinterpret_cast<const float4 *>(p);
    v[0] = u.x;
    v[1] = u.y;
    v[2] = u.z;
    v[3] = u.w;
  }
}

template <int DG, bool kF32, bool kRotate>
__global__ __launch_bounds__(64 * kWaves) void token_error_kernel(DiagArgs a) {
  constexpr int CPL = DG / 64;
  const int lane = threadIdx.x & 63;
  const int64_t nch = a.capacity / T;
  const int64_t total = (int64_t)a.batch * a.heads * a.tokens;
  for (int64_t w = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); w < total;
       w += (int64_t)gridDim.x * kWaves) {
    const int64_t bh = w / a.tokens;
    const int tt = (int)(w - bh * a.tokens);
    const int64_t b = bh / a.heads, h = bh - b * a.heads;
    const int t = a.token_offset + tt;  // cache slot
    // ---- x, channels CPL lane + i ------------------------------------------
    const int64_t xo = b * a.sb + h * a.sh + (int64_t)tt * a.st + CPL * lane;
    float y[CPL];
    if constexpr (kF32) {
      load_f32<CPL>(static_cast<const float *>(a.x) + xo, y);
    } else {
      const uint16_t *xp = static_cast<const uint16_t *>(a.x) + xo;
      if constexpr (CPL == 1) {
        y[0] = __uint_as_float((uint32_t)xp[0] << 16);
      } else if constexpr (CPL == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t *>(xp);
        y[0] = bf16_lo(u);
        y[1] = bf16_hi(u);
      } else {
        const u32x2 u = *reinterpret_cast<const u32x2 *>(xp);
        y[0] = bf16_lo(u[0]);
        y[1] = bf16_hi(u[0]);
        y[2] = bf16_lo(u[1]);
        y[3] = bf16_hi(u[1]);
      }
    }
    if constexpr (kRotate) {
      // the low channel bits (the register index) in-lane, channel bit
      // k + log2(CPL) = lane bit k across lanes
#pragma unroll
      for (int len = 1; len < CPL; len <<= 1)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
          if ((i & len) == 0) {
            const float s = y[i] + y[i + len], d = y[i] - y[i + len];
            y[i] = s;
            y[i + len] = d;
          }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const bool upper = lane & m;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const float p = lane_xor(y[i], m);
          y[i] = upper ? p - y[i] : y[i] + p;
        }
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) y[i] *= inv_sqrt_head(DG);
    }
    // ---- reconstruction in the rotated basis -----------------------------
    const int64_t chunk = t / T, tc = t % T;
    const uint8_t *cb = a.codes + (bh * nch + chunk) * (T * DG / 4);
    uint32_t q[CPL];
    if (a.kind == KVARN_K) {  // token row: channel j in byte j / 4, bits 2 (j % 4)
      const int j0 = CPL * lane;  // the lane's channels share one byte
      const uint32_t byte = cb[tc * (DG / 4) + (j0 >> 2)];
#pragma unroll
      for (int i = 0; i < CPL; ++i) q[i] = (byte >> (2 * ((j0 + i) & 3))) & 3u;
    } else {  // channel rows: token tc in byte tc / 4, bits 2 (tc % 4)
      const int sh = 2 * (int)(tc & 3);
#pragma unroll
      for (int i = 0; i < CPL; ++i) q[i] = (cb[(CPL * lane + i) * 32 + (tc >> 2)] >> sh) & 3u;
    }
    const float rp = a.row_scale[bh * a.capacity + t];
    float c[CPL];
    load_f32<CPL>(a.col_scale + (bh * nch + chunk) * DG + CPL * lane, c);
    float yy = 0.f, zz = 0.f, yz = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float z = ((float)q[i] - 1.5f) * rp * c[i];
      yy = fmaf(y[i], y[i], yy);
      zz = fmaf(z, z, zz);
      yz = fmaf(y[i], z, yz);
    }
    // ---- norms and inner product ------------------------------------------
    const float aa = wave_sum(yy);
    const float bb = wave_sum(zz);
    const float ab = wave_sum(yz);
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

template <int DG>
hipError_t launch_token_error_dg(const DiagArgs &a, hipStream_t s) {
  const int64_t total = (int64_t)a.batch * a.heads * a.tokens;
  const int64_t want = (total + kWaves - 1) / kWaves;
  const int64_t cap = 8LL * device_cus();
  const dim3 grid((unsigned)(want < cap ? want : cap));
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE);
  if (a.dtype == KVARN_DT_F32) {
    if (rot)
      hipLaunchKernelGGL((token_error_kernel<DG, true, true>), grid, dim3(64 * kWaves), 0, s, a);
    else
      hipLaunchKernelGGL((token_error_kernel<DG, true, false>), grid, dim3(64 * kWaves), 0, s, a);
  } else {
    if (rot)
      hipLaunchKernelGGL((token_error_kernel<DG, false, true>), grid, dim3(64 * kWaves), 0, s, a);
    else
      hipLaunchKernelGGL((token_error_kernel<DG, false, false>), grid, dim3(64 * kWaves), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_error(const DiagArgs &a, hipStream_t s) {
  if ((int64_t)a.batch * a.heads * a.tokens == 0) return hipSuccess;
  switch (a.head_dim) {
    case 64: return launch_token_error_dg<64>(a, s);
    case 256: return launch_token_error_dg<256>(a, s);
    default: return launch_token_error_dg<128>(a, s);
  }
}

}  // namespace kvarn
