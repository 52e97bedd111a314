// Head sizes other than 128 (64 and 256): the quantizer, the one-token append
// and the per-token error diagnostic for a head_dim D that is a multiple of
// 64 (rndamp article on KVarN, "How It Works", item 1: the Hadamard transform
// acts on the channel dimension of whatever head size the model has; the
// decode attention serves every head size in its own file). The D = 128
// calls run the tuned kernels of the other files;
// these kernels compute the same quantities in plain fp32 vector code with a
// simpler layout:
//  * a wave holds whole tokens: lane l holds channels l + 64 k (k < D / 64),
//    so the rotation of a token is an in-wave fast Walsh-Hadamard transform
//    (channel bits 6 and up inside the lane, bits 0..5 across lanes), and a
//    sum over a token's channels is an in-wave butterfly;
//  * the quantizer's eight waves hold 16 tokens each (token wv + 8 s) and
//    meet in LDS for the column sums (each wave adds up all D channels in
//    the same order, so every wave holds identical column scales).
// Row and column normalizations: with v_i = 1 / sum_j P_ij / c_j^2 the
// column step's mean over the T tokens is c_j^2 = (D / T) sum_i P_ij v_i.
#include "kvarn_diag.h"

namespace kvarn {
namespace {

constexpr float kTinyG = 1.17549435e-38f;   // smallest normal fp32
constexpr float kGridG = 1.9999980926513672f;  // 2 (1 - 2^-20), as the D = 128 quantizer

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
// Block quantizer for head size D (same steps and readings as the D = 128
// kernel: rotation, `iters` sweeps of a row step then a column step from
// c = 1, per-token range step r' = max_j |y_j| / c_j / 2, codes
// floor(u + 2) on the 4-level grid).
template <int D_, bool kF32, bool kRotate, bool kPositions>
__global__ __launch_bounds__(512) void quantize_generic_kernel(QuantArgs a) {
  constexpr int KD = D_ / 64, NW = 8, TW = T / NW;
  __shared__ float cpart[2][NW][D_];
  __shared__ uint32_t codes[T][D_ / 4];  // one byte per code, then packed
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nch = a.capacity / T;
  // the unscaled rotation's 1/sqrt(D) and the range step's 1/2
  const float range_factor = kRotate ? 0.5f * inv_sqrt_d(D_) : 0.5f;
  for (uint32_t blk = blockIdx.x; blk < a.nblocks; blk += gridDim.x) {
    const uint32_t bh = fdiv(blk, a.div_chunks);
    const uint32_t kc = blk - bh * (uint32_t)a.chunks;
    const uint32_t b = fdiv(bh, a.div_heads), h = bh - b * (uint32_t)a.heads;
    int chunk = a.chunk0 + (int)kc;
    if constexpr (kPositions) {
      const int pos = a.pos[b];
      if (pos < 0 || pos >= a.capacity || pos % T != T - 1) continue;  // workgroup-uniform
      chunk = pos / T;
    }
    const int64_t xb = (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)kc * T * a.st;
    float y[TW][KD], p[TW][KD];
#pragma unroll
    for (int s = 0; s < TW; ++s) {
      load_row<KD, kF32>(a.x, xb + (int64_t)(wv + NW * s) * a.st, lane, y[s]);
      if constexpr (kRotate) fwht_wave<KD>(y[s], lane);
#pragma unroll
      for (int k = 0; k < KD; ++k) p[s][k] = y[s][k] * y[s][k];
    }
    float cm[KD], w[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      cm[k] = 1.f;
      w[k] = 1.f;
    }
    if (a.iters > 0) {
      float v[TW];
#pragma unroll
      for (int s = 0; s < TW; ++s) {  // first row step, c = 1
        float e = 0.f;
#pragma unroll
        for (int k = 0; k < KD; ++k) e += p[s][k];
        v[s] = __builtin_amdgcn_rcpf(fmaxf(wsum(e), kTinyG));
      }
      for (int it = 0;; ++it) {
        // column step: c_j^2 = (D / T) sum_i P_ij v_i; the eight waves' sums
        // over their tokens meet in LDS (two buffers alternate by step, so
        // one barrier per step orders both reuse and reads)
        float (*cp)[D_] = cpart[it & 1];
#pragma unroll
        for (int k = 0; k < KD; ++k) {
          float e = 0.f;
#pragma unroll
          for (int s = 0; s < TW; ++s) e = fmaf(p[s][k], v[s], e);
          cp[wv][lane + 64 * k] = e;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KD; ++k) {
          float e = 0.f;
#pragma unroll
          for (int u = 0; u < NW; ++u) e += cp[u][lane + 64 * k];
          cm[k] = e * ((float)D_ / (float)T);
        }
        if (it + 1 == a.iters) break;
        // row step: v_i = 1 / sum_j P_ij / c_j^2
#pragma unroll
        for (int k = 0; k < KD; ++k) w[k] = __builtin_amdgcn_rcpf(fmaxf(cm[k], kTinyG));
#pragma unroll
        for (int s = 0; s < TW; ++s) {
          float e = 0.f;
#pragma unroll
          for (int k = 0; k < KD; ++k) e = fmaf(p[s][k], w[k], e);
          v[s] = __builtin_amdgcn_rcpf(fmaxf(wsum(e), kTinyG));
        }
      }
      // c, and 1/c for the range step (a zero column keeps c = 1)
#pragma unroll
      for (int k = 0; k < KD; ++k) {
        const bool pos_c = cm[k] > 0.f;
        const float ic = pos_c ? __builtin_amdgcn_rsqf(cm[k]) : 1.f;
        w[k] = ic;
        cm[k] = pos_c ? cm[k] * ic : 1.f;
      }
    }
    float *col = a.col_scale + ((int64_t)bh * nch + chunk) * D_;
    if (wv == 0) {
#pragma unroll
      for (int k = 0; k < KD; ++k) col[lane + 64 * k] = cm[k];
    }
    // range step and codes: u = y / (r' c), code = floor(u + 2) through
    // rounding of u (1 - 2^-20) + 1.5, as the D = 128 kernel decides it
    uint8_t *cb8 = reinterpret_cast<uint8_t *>(&codes[0][0]);
#pragma unroll
    for (int s = 0; s < TW; ++s) {
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < KD; ++k) {
        y[s][k] *= w[k];
        mx = fmaxf(mx, fabsf(y[s][k]));
      }
      mx = wmax(mx);
      const int ti = wv + NW * s;
      if (lane == 0) a.row_scale[(int64_t)bh * a.capacity + (int64_t)chunk * T + ti] = mx * range_factor;
      const float q = mx > 0.f ? kGridG * __builtin_amdgcn_rcpf(mx) : 0.f;
#pragma unroll
      for (int k = 0; k < KD; ++k)
        cb8[ti * D_ + lane + 64 * k] =
            (uint8_t)__builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[s][k], q, 1.5f), 0, 0u);
    }
    __syncthreads();
    // pack: 32 D bytes per block, one 32-bit word per thread and round
    uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + ((int64_t)bh * nch + chunk) * (T * D_ / 4));
    for (int wi = tid; wi < T * D_ / 16; wi += 512) {
      uint32_t word = 0;
      if (a.kind == KVARN_K) {
        // token-major: token t owns D/4 bytes; byte j/4 holds channels j..j+3
        const int t = wi / (D_ / 16), jw = wi % (D_ / 16);  // bytes 4 jw .. of token t
#pragma unroll
        for (int by = 0; by < 4; ++by) {
          const uint32_t c4 = codes[t][4 * jw + by];  // codes of channels 16 jw + 4 by + [0, 4)
          const uint32_t packed = (c4 & 3u) | ((c4 >> 6) & 0xCu) | ((c4 >> 12) & 0x30u) |
                                  ((c4 >> 18) & 0xC0u);
          word |= packed << (8 * by);
        }
      } else {
        // channel-major: channel j owns 32 bytes; byte t/4 holds tokens t..t+3
        const int j = wi / 8, tw = wi % 8;  // bytes 4 tw .. of channel j: tokens 16 tw ..
#pragma unroll
        for (int by = 0; by < 4; ++by) {
          uint32_t packed = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) packed |= (uint32_t)cb8[(16 * tw + 4 * by + r) * D_ + j] << (2 * r);
          word |= packed << (8 * by);
        }
      }
      dst[wi] = word;
    }
    __syncthreads();  // the code area is rewritten by the next block
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
static hipError_t launch_quantize_d(const QuantArgs &a, hipStream_t s) {
  const uint32_t resident = (uint32_t)device_cus();  // one 512-thread workgroup per CU
  const uint32_t blocks = a.nblocks < resident ? a.nblocks : resident;
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE), f32 = a.dtype == KVARN_DT_F32;
#define KVARN_QG(F, R, P) \
  hipLaunchKernelGGL((quantize_generic_kernel<D_, F, R, P>), dim3(blocks), dim3(512), 0, s, a)
  if (a.pos) {
    if (f32) { if (rot) KVARN_QG(true, true, true); else KVARN_QG(true, false, true); }
    else { if (rot) KVARN_QG(false, true, true); else KVARN_QG(false, false, true); }
  } else {
    if (f32) { if (rot) KVARN_QG(true, true, false); else KVARN_QG(true, false, false); }
    else { if (rot) KVARN_QG(false, true, false); else KVARN_QG(false, false, false); }
  }
#undef KVARN_QG
  return hipGetLastError();
}

hipError_t launch_quantize_generic(const QuantArgs &a, hipStream_t s) {
  if (a.nblocks == 0) return hipSuccess;
  if (a.head_dim == 64) return launch_quantize_d<64>(a, s);
  if (a.head_dim == 256) return launch_quantize_d<256>(a, s);
  return hipErrorInvalidValue;
}

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
