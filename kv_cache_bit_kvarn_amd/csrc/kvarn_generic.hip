// Head sizes other than 128 (64 and 256): the one-token append and the
// per-token error diagnostic for a head_dim D that is a multiple of 64
// (rndamp article on KVarN, "How It Works", item 1: the Hadamard transform
// acts on the channel dimension of whatever head size the model has; the
// block quantizer and the decode attention serve every head size in their
// own files, and the D = 128 append and diagnostic run the tuned kernels of
// the other files). These kernels compute the same quantities in plain fp32
// vector code with a simpler layout: a wave holds whole tokens, lane l
// channels l + 64 k (k < D / 64), so the rotation of a token is an in-wave
// fast Walsh-Hadamard transform (channel bits 6 and up inside the lane, bits
// 0..5 across lanes), and a sum over a token's channels is an in-wave
// butterfly.
#include "kvarn_diag.h"

namespace kvarn {
namespace {


// 1/sqrt(D) for D a power of four (64, 256): an exact power of two
__host__ __device__ constexpr float inv_sqrt_d(int d) {
  return d == 64 ? 0.125f : d == 256 ? 0.0625f : d == 16 ? 0.25f : d == 1024 ? 0.03125f : 0.f;
}
static_assert(inv_sqrt_d(64) * 8.f == 1.f && inv_sqrt_d(256) * 16.f == 1.f, "1/sqrt(D)");

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += lane_xor(v, m);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, lane_xor(v, m));
  return v;
}

// Unscaled Sylvester-order Hadamard transform of the D = 64 KD channels a
// wave holds for one token (lane l: channel l + 64 k in v[k]).
template <int KD>
__device__ __forceinline__ void fwht_wave(float (&v)[KD], int lane) {
#pragma unroll
  for (int len = 1; len < KD; len <<= 1)
#pragma unroll
    for (int k = 0; k < KD; ++k)
      if ((k & len) == 0) {
        const float x = v[k], y = v[k + len];
        v[k] = x + y;
        v[k + len] = x - y;
      }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const float p = lane_xor(v[k], m);
      v[k] = up ? p - v[k] : v[k] + p;
    }
  }
}

// Channels l + 64 k of one token row of x (bf16 or fp32).
template <int KD, bool kF32>
__device__ __forceinline__ void load_row(const void *x, int64_t off, int lane, float (&v)[KD]) {
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    if constexpr (kF32)
      v[k] = static_cast<const float *>(x)[off + lane + 64 * k];
    else
      v[k] = __uint_as_float((uint32_t) static_cast<const uint16_t *>(x)[off + lane + 64 * k] << 16);
  }
}

// ---------------------------------------------------------------------------
// One-token append for head size D (the reading of the D = 128 kernel: a
// chunk opened by the token copies the previous chunk's column scales, or 1;
// the token's own range step; a V token at slot % 4 == 0 rewrites its byte).
template <int D_, bool kF32, bool kRotate>
__global__ __launch_bounds__(64) void append_generic_kernel(AppendArgs a) {
  constexpr int KD = D_ / 64;
  const int bh = blockIdx.x;
  const int b = bh / a.heads;
  const int lane = threadIdx.x;
  const int pos = a.pos[b];
  if (pos < 0 || pos >= a.capacity) return;  // uniform across the wave
  const int k = pos / T, slot = pos - k * T;
  const int64_t nch = a.capacity / T;
  float y[KD];
  load_row<KD, kF32>(a.x, (int64_t)bh * D_, lane, y);
  if (a.window) {
#pragma unroll
    for (int i = 0; i < KD; ++i) {
      const int64_t o = ((int64_t)bh * T + slot) * D_ + lane + 64 * i;
      if constexpr (kF32)
        static_cast<float *>(a.window)[o] = y[i];
      else
        static_cast<uint16_t *>(a.window)[o] = static_cast<const uint16_t *>(a.x)[(int64_t)bh * D_ + lane + 64 * i];
    }
  }
  if constexpr (kRotate) fwht_wave<KD>(y, lane);
  float *col = a.col_scale + ((int64_t)bh * nch + k) * D_;
  float c[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) {
    if (slot == 0) {
      c[i] = k > 0 ? col[lane + 64 * i - D_] : 1.f;
      col[lane + 64 * i] = c[i];
    } else {
      c[i] = col[lane + 64 * i];
    }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < KD; ++i) {
    y[i] *= 1.f / c[i];
    m = fmaxf(m, fabsf(y[i]));
  }
  m = wmax(m);
  const float rf = kRotate ? 0.5f * inv_sqrt_d(D_) : 0.5f;
  if (lane == 0) a.row_scale[(int64_t)bh * a.capacity + pos] = m * rf;
  const float qs = m > 0.f ? 2.f / m : 0.f;
  uint32_t q[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) q[i] = (uint32_t)fminf(fmaxf(fmaf(y[i], qs, 2.f), 0.f), 3.f);
  uint8_t *cb = a.codes + ((int64_t)bh * nch + k) * (T * D_ / 4);
  if (a.kind == KVARN_K) {
    // token row (D/4 bytes): byte j/4 holds channels j..j+3 at bits 2 (j % 4);
    // lane l (< D/4) gathers channels 4 l .. 4 l + 3 from lanes (4 l) % 64 ..
#pragma unroll
    for (int i = 0; i < KD; ++i) {
      const int src = 4 * (lane & 15);
      uint32_t byte = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) byte |= (uint32_t)__shfl((int)q[i], src + r, 64) << (2 * r);
      // byte index 16 i + lane for lanes < 16 (channels 64 i + 4 lane ..)
      if (lane < 16) cb[slot * (D_ / 4) + 16 * i + lane] = (uint8_t)byte;
    }
  } else {
    const int sh = 2 * (slot & 3);
#pragma unroll
    for (int i = 0; i < KD; ++i) {
      uint8_t *p = cb + (lane + 64 * i) * 32 + (slot >> 2);
      if (sh == 0) {
        *p = (uint8_t)q[i];
      } else {
        const uint32_t keep = ~(3u << sh) & 0xFFu;
        *p = (uint8_t)((*p & keep) | (q[i] << sh));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-token magnitude and direction of the reconstruction (kvarn_token_error)
// for head size D, in the rotated basis where both numbers are preserved.
template <int D_, bool kF32, bool kRotate>
__global__ __launch_bounds__(256) void token_error_generic_kernel(DiagArgs a) {
  constexpr int KD = D_ / 64;
  const int lane = threadIdx.x & 63;
  const int64_t nch = a.capacity / T;
  const int64_t total = (int64_t)a.batch * a.heads * a.tokens;
  for (int64_t wi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); wi < total;
       wi += (int64_t)gridDim.x * 4) {
    const int64_t bh = wi / a.tokens;
    const int tt = (int)(wi - bh * a.tokens);
    const int64_t b = bh / a.heads, h = bh - b * a.heads;
    const int t = a.token_offset + tt;
    float y[KD];
    load_row<KD, kF32>(a.x, b * a.sb + h * a.sh + (int64_t)tt * a.st, lane, y);
    if constexpr (kRotate) {
      fwht_wave<KD>(y, lane);
#pragma unroll
      for (int k = 0; k < KD; ++k) y[k] *= inv_sqrt_d(D_);
    }
    const int kc = t / T, slot = t - kc * T;
    const uint8_t *cb = a.codes + (bh * nch + kc) * (T * D_ / 4);
    const float *col = a.col_scale + (bh * nch + kc) * D_;
    const float rp = a.row_scale[bh * a.capacity + t];
    float xx = 0.f, hh = 0.f, xh = 0.f;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const int j = lane + 64 * k;
      const uint32_t byte = a.kind == KVARN_K ? cb[slot * (D_ / 4) + j / 4] : cb[j * 32 + slot / 4];
      const int sh = a.kind == KVARN_K ? 2 * (j & 3) : 2 * (slot & 3);
      const float yh = ((float)((byte >> sh) & 3u) - 1.5f) * rp * col[j];
      xx = fmaf(y[k], y[k], xx);
      hh = fmaf(yh, yh, hh);
      xh = fmaf(y[k], yh, xh);
    }
    xx = wsum(xx);
    hh = wsum(hh);
    xh = wsum(xh);
    if (lane == 0) {
      float ratio, cosine;
      if (xx == 0.f && hh == 0.f) {
        ratio = 1.f;
        cosine = 1.f;
      } else if (xx == 0.f) {
        ratio = INFINITY;
        cosine = 0.f;
      } else if (hh == 0.f) {
        ratio = 0.f;
        cosine = 0.f;
      } else {
        ratio = sqrtf(hh / xx);
        cosine = xh / sqrtf(xx * hh);
      }
      a.ratio[wi] = ratio;
      a.cosine[wi] = cosine;
    }
  }
}

}  // namespace

// ---- launchers -------------------------------------------------------------

template <int D_>
static hipError_t launch_append_d(const AppendArgs &a, hipStream_t s) {
  const int blocks = a.batch * a.heads;
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE), f32 = a.dtype == KVARN_DT_F32;
#define KVARN_AG(F, R) hipLaunchKernelGGL((append_generic_kernel<D_, F, R>), dim3(blocks), dim3(64), 0, s, a)
  if (f32) { if (rot) KVARN_AG(true, true); else KVARN_AG(true, false); }
  else { if (rot) KVARN_AG(false, true); else KVARN_AG(false, false); }
#undef KVARN_AG
  return hipGetLastError();
}

hipError_t launch_append_generic(const AppendArgs &a, hipStream_t s) {
  if (a.batch * a.heads == 0) return hipSuccess;
  if (a.head_dim == 64) return launch_append_d<64>(a, s);
  if (a.head_dim == 256) return launch_append_d<256>(a, s);
  return hipErrorInvalidValue;
}

template <int D_>
static hipError_t launch_token_error_d(const DiagArgs &a, hipStream_t s) {
  const int64_t total = (int64_t)a.batch * a.heads * a.tokens;
  const int64_t want = (total + 3) / 4, cap = 8LL * device_cus();
  const dim3 grid((unsigned)(want < cap ? want : cap));
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE), f32 = a.dtype == KVARN_DT_F32;
#define KVARN_TG(F, R) hipLaunchKernelGGL((token_error_generic_kernel<D_, F, R>), grid, dim3(256), 0, s, a)
  if (f32) { if (rot) KVARN_TG(true, true); else KVARN_TG(true, false); }
  else { if (rot) KVARN_TG(false, true); else KVARN_TG(false, false); }
#undef KVARN_TG
  return hipGetLastError();
}

hipError_t launch_token_error_generic(const DiagArgs &a, hipStream_t s) {
  if ((int64_t)a.batch * a.heads * a.tokens == 0) return hipSuccess;
  if (a.head_dim == 64) return launch_token_error_d<64>(a, s);
  if (a.head_dim == 256) return launch_token_error_d<256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvarn
