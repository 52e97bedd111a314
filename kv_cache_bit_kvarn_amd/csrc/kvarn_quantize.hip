// Block quantizer of the KVarN method on gfx950.
//
// One workgroup (256 threads, 4 wave64) quantizes one 128-token x 128-channel
// block of K or V (one layer, sequence, kv-head, chunk):
//   1. load bf16/fp32 -> fp32 registers (16-byte loads; one token row per
//      lane pair, 64 channels per lane);
//   2. Hadamard rotation along channels (rndamp article on KVarN, "How It
//      Works", item 1): six butterfly stages inside each lane, the seventh
//      between the two lanes of a token through DPP;
//   3. dual-scaling normalization ("How It Works", item 2; abstract: both
//      axes of K and V): squared values P stay in registers for the row step
//      and are staged once, transposed, in LDS for the column step;
//   4. per-token range step, 2-bit codes, and packing (K token-major straight
//      from registers, V channel-major through an LDS byte transpose);
//   5. 16-byte stores of codes, fp32 row and column scales.
// The rotation is applied without its 1/sqrt(128) factor; that factor leaves
// the column scales and codes unchanged and is folded into the row scale.
#include "kvarn_internal.h"

namespace kvarn {
namespace {

constexpr int kThreads = 256;
constexpr int PT_STRIDE = T + 4;  // floats per row of the transposed P (bank spread)
constexpr int CB_STRIDE = T + 16; // bytes per channel row of the V code transpose

struct QuantSmem {
  float pt[D * PT_STRIDE];  // pt[j][i] = P_ij  (later reused for V code bytes)
  float w[D];               // 1/c_j^2 while balancing, then 1/c_j
  float v[T];               // 1/r_i^2
  float cpart[2][D];        // column sums over token halves
};

// Sum of 64 products in eight interleaved partial sums combined as a tree,
// keeping fp32 rounding close to that of a pairwise sum.
__device__ __forceinline__ float dot64(const float (&p)[64], const float *w) {
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const f32x4 ww = reinterpret_cast<const f32x4 *>(w)[q];
    acc[(4 * q + 0) & 7] = fmaf(p[4 * q + 0], ww.x, acc[(4 * q + 0) & 7]);
    acc[(4 * q + 1) & 7] = fmaf(p[4 * q + 1], ww.y, acc[(4 * q + 1) & 7]);
    acc[(4 * q + 2) & 7] = fmaf(p[4 * q + 2], ww.z, acc[(4 * q + 2) & 7]);
    acc[(4 * q + 3) & 7] = fmaf(p[4 * q + 3], ww.w, acc[(4 * q + 3) & 7]);
  }
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// Same, both operands from LDS (column step: P_ij * v_i over 64 tokens).
__device__ __forceinline__ float dot64_lds(const float *a, const float *b) {
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const f32x4 x = reinterpret_cast<const f32x4 *>(a)[q];
    const f32x4 y = reinterpret_cast<const f32x4 *>(b)[q];
    acc[(4 * q + 0) & 7] = fmaf(x.x, y.x, acc[(4 * q + 0) & 7]);
    acc[(4 * q + 1) & 7] = fmaf(x.y, y.y, acc[(4 * q + 1) & 7]);
    acc[(4 * q + 2) & 7] = fmaf(x.z, y.z, acc[(4 * q + 2) & 7]);
    acc[(4 * q + 3) & 7] = fmaf(x.w, y.w, acc[(4 * q + 3) & 7]);
  }
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

template <bool kF32>
__global__ __launch_bounds__(kThreads, 2) void quantize_block_kernel(QuantArgs a) {
  __shared__ QuantSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int ti = (tid >> 6) * 32 + (lane >> 1);  // token row of this lane pair
  const int hf = lane & 1;                       // channels [64 hf, 64 hf + 64)

  const int kc = blockIdx.x % a.chunks;
  const int bh = blockIdx.x / a.chunks;
  const int b = bh / a.heads, h = bh - b * a.heads;
  const int chunk = a.chunk0 + kc;
  const int64_t nch = a.capacity / T;

  // ---- 1. load -----------------------------------------------------------
  float y[64];
  const int64_t off = (int64_t)b * a.sb + (int64_t)h * a.sh +
                      (int64_t)(kc * T + ti) * a.st + 64 * hf;
  if constexpr (kF32) {
    const f32x4 *src = reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.x) + off);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const f32x4 v = __builtin_nontemporal_load(src + q);
      y[4 * q + 0] = v.x; y[4 * q + 1] = v.y; y[4 * q + 2] = v.z; y[4 * q + 3] = v.w;
    }
  } else {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.x) + off);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 u = __builtin_nontemporal_load(src + q);
      y[8 * q + 0] = bf16_lo(u.x); y[8 * q + 1] = bf16_hi(u.x);
      y[8 * q + 2] = bf16_lo(u.y); y[8 * q + 3] = bf16_hi(u.y);
      y[8 * q + 4] = bf16_lo(u.z); y[8 * q + 5] = bf16_hi(u.z);
      y[8 * q + 6] = bf16_lo(u.w); y[8 * q + 7] = bf16_hi(u.w);
    }
  }

  // ---- 2. rotation: y <- y . H_128 (Sylvester order, unscaled) -----------
#pragma unroll
  for (int len = 1; len < 64; len <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if ((i & len) == 0) {
        const float p = y[i], q = y[i + len];
        y[i] = p + q;
        y[i + len] = p - q;
      }
    }
  }
  {
    // top channel bit lives across the lane pair: lane hf=0 holds A, hf=1
    // holds B; the pair becomes (A + B, A - B) = fma(own, +-1, partner).
    const float sgn = hf ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) y[i] = fmaf(y[i], sgn, dpp_xor1(y[i]));
  }

  // ---- 3. dual scaling ---------------------------------------------------
  float p[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    p[i] = y[i] * y[i];
    sm.pt[(64 * hf + i) * PT_STRIDE + ti] = p[i];
  }
  if (tid < D) sm.w[tid] = 1.f;
  __syncthreads();

  const int cj = tid & (D - 1);  // column-owner role: channel cj,
  const int cg = tid >> 7;       // tokens [64 cg, 64 cg + 64)
  for (int it = 0; it < a.iters; ++it) {
    // row step: r_i^2 = (1/D) sum_j P_ij / c_j^2  ->  v_i = 1/r_i^2
    float s = dot64(p, sm.w + 64 * hf);
    s += dpp_xor1(s);
    if (hf == 0) sm.v[ti] = s > 0.f ? (float)D / s : 1.f;
    __syncthreads();
    // column step: c_j^2 = (1/T) sum_i P_ij / r_i^2  ->  w_j = 1/c_j^2
    sm.cpart[cg][cj] = dot64_lds(sm.pt + cj * PT_STRIDE + 64 * cg, sm.v + 64 * cg);
    __syncthreads();
    if (tid < D) {
      const float cm = (sm.cpart[0][tid] + sm.cpart[1][tid]) * (1.f / T);
      sm.w[tid] = cm > 0.f ? 1.f / cm : 1.f;
    }
    __syncthreads();
  }
  float *rowp = a.row_scale + ((int64_t)bh * a.capacity + (int64_t)chunk * T);
  float *colp = a.col_scale + ((int64_t)bh * nch + chunk) * D;
  if (tid < D) {
    float c = 1.f;
    if (a.iters > 0) {
      const float cm = (sm.cpart[0][tid] + sm.cpart[1][tid]) * (1.f / T);
      c = cm > 0.f ? sqrtf(cm) : 1.f;
    }
    colp[tid] = c;
    sm.w[tid] = 1.f / c;
  }
  __syncthreads();

  // ---- 4. range step and codes --------------------------------------------
  float m = 0.f;
  {
    const f32x4 *ic = reinterpret_cast<const f32x4 *>(sm.w + 64 * hf);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const f32x4 w4 = ic[q];
      y[4 * q + 0] *= w4.x; y[4 * q + 1] *= w4.y; y[4 * q + 2] *= w4.z; y[4 * q + 3] *= w4.w;
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(y[i]));
  }
  m = fmaxf(m, dpp_xor1(m));
  if (hf == 0) rowp[ti] = m * kRangeFromUnscaled;
  const float qs = m > 0.f ? 2.f / m : 0.f;
  uint32_t code[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const float t = fminf(fmaxf(fmaf(y[i], qs, 2.f), 0.f), 3.f);
    code[i] = (uint32_t)t;
  }

  uint8_t *cbase = a.codes + ((int64_t)bh * nch + chunk) * CHUNK_BYTES;
  if (a.kind == KVARN_K) {
    u32x4 pk;
    uint32_t *pw = reinterpret_cast<uint32_t *>(&pk);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t wv = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) wv |= code[16 * d + k] << (2 * k);
      pw[d] = wv;
    }
    *reinterpret_cast<u32x4 *>(cbase + ti * 32 + hf * 16) = pk;
  } else {
    // channel-major: stage one byte per code in LDS as cb[channel][token]
    uint8_t *cb = reinterpret_cast<uint8_t *>(sm.pt);
#pragma unroll
    for (int i = 0; i < 64; ++i) cb[(64 * hf + i) * CB_STRIDE + ti] = (uint8_t)code[i];
    __syncthreads();
    const int j = tid >> 1, g = tid & 1;  // channel j, tokens [64 g, 64 g + 64)
    const uint32_t *src = reinterpret_cast<const uint32_t *>(cb + j * CB_STRIDE + 64 * g);
    u32x4 pk;
    uint32_t *pw = reinterpret_cast<uint32_t *>(&pk);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t o = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t wd = src[4 * q + r];
        const uint32_t byte = (wd & 0x3u) | ((wd >> 6) & 0xCu) | ((wd >> 12) & 0x30u) |
                              ((wd >> 18) & 0xC0u);
        o |= byte << (8 * r);
      }
      pw[q] = o;
    }
    *reinterpret_cast<u32x4 *>(cbase + j * 32 + g * 16) = pk;
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.batch * a.heads * a.chunks;
  if (blocks == 0) return hipSuccess;
  if (a.dtype == KVARN_DT_F32)
    hipLaunchKernelGGL(quantize_block_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(quantize_block_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvarn
