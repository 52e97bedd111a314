// Decode attention over the 2-bit KVarN cache on gfx950, both scales fused
// into the dequantization (rndamp article on KVarN, "Numbers").
//
// Rotated-domain evaluation. With H = H_128 / sqrt(128) (symmetric,
// orthogonal) the cache stores y_hat = x_hat H, so
//   <q, x_hat_t>      = <q H, y_hat_t>
//                     = r'_t * sum_j (qH)_j c_j (code_tj - 1.5)
//   sum_t p_t x_hat_t = ( sum_t p_t y_hat_t ) H
//                     = ( c_j * sum_t (p_t r'_t)(code_tj - 1.5) )_j  H.
// The query is rotated once per workgroup, the column scale of K is folded
// into the rotated query per chunk, the row scale of K into each score, the
// row scale of V into each probability, and the column scale of V into the
// output; the output is rotated back after the split-KV merge.
//
// decode_split: grid (n_split, kv_heads, batch); each workgroup walks its
// range of 128-token chunks with an online softmax and writes one partial
// (m, l, acc[128]) per query head. decode_combine: grid (q_heads, batch);
// log-sum-exp merge of the partials, then the inverse rotation.
#include "kvarn_internal.h"

namespace kvarn {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// In-place Sylvester Hadamard transform (unscaled) of rows x[n][128] held in
// LDS, all threads of the block cooperating.
__device__ void lds_fwht_rows(float *x, int n) {
  for (int len = 1; len < D; len <<= 1) {
    for (int idx = threadIdx.x; idx < n * (D / 2); idx += blockDim.x) {
      const int row = idx / (D / 2), p = idx - row * (D / 2);
      const int i = (p / len) * 2 * len + (p % len);
      float *r = x + row * D;
      const float u = r[i], v = r[i + len];
      r[i] = u + v;
      r[i + len] = u - v;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ float load_q(const void *q, int dtype, int64_t idx) {
  if (dtype == KVARN_DT_F32) return static_cast<const float *>(q)[idx];
  return __uint_as_float((uint32_t)static_cast<const uint16_t *>(q)[idx] << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

struct SplitSmem {
  float qh[GQA_MAX][D];  // rotated query * softmax scale * log2(e)
  float a[GQA_MAX][D];   // qh * c_K of the current chunk
  float s[GQA_MAX][T];   // scores (log2 units), then p * r'_V
  float colk[D], colv[D], rowk[T], rowv[T];
  float m[GQA_MAX], l[GQA_MAX], alpha[GQA_MAX];
};

template <int HPT>  // query heads per thread: ceil(G / 2)
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  __shared__ SplitSmem sm;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = a.q_heads / a.kv_heads;
  const int nch = a.capacity / T;
  const int len = a.lens[b];
  const bool valid = len >= 1 && len <= a.capacity;
  const int used = valid ? (len + T - 1) / T : 0;
  const int per = (nch + a.n_split - 1) / a.n_split;
  const int c0 = split * per;
  const int c1 = min(c0 + per, used);

  // query: rotate, fold the softmax scale and log2(e)
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int hh = idx / D, j = idx - hh * D;
    sm.qh[hh][j] = load_q(a.q, a.q_dtype, ((int64_t)b * a.q_heads + g * G + hh) * D + j);
  }
  if (tid < GQA_MAX) {
    sm.m[tid] = -INFINITY;
    sm.l[tid] = 0.f;
    sm.alpha[tid] = 1.f;
  }
  __syncthreads();
  lds_fwht_rows(&sm.qh[0][0], G);
  const float qscale = a.scale * kLog2e * kInvSqrtD;
  for (int idx = tid; idx < G * D; idx += kThreads) sm.qh[idx / D][idx % D] *= qscale;

  const int j = tid & (D - 1);    // PV role: channel j
  const int h0 = tid >> 7;        // heads h0, h0 + 2, ...
  const int tt = tid & (T - 1);   // QK role: token tt
  float acc[HPT];
#pragma unroll
  for (int r = 0; r < HPT; ++r) acc[r] = 0.f;

  const int64_t bg = (int64_t)b * a.kv_heads + g;
  for (int k = c0; k < c1; ++k) {
    const int64_t chunk = bg * nch + k;
    __syncthreads();  // previous chunk done with the LDS
    if (tid < D) {
      sm.colk[tid] = a.k_col[chunk * D + tid];
      sm.colv[tid] = a.v_col[chunk * D + tid];
    } else {
      const int t = tid - D;
      sm.rowk[t] = a.k_row[bg * a.capacity + (int64_t)k * T + t];
      sm.rowv[t] = a.v_row[bg * a.capacity + (int64_t)k * T + t];
    }
    __syncthreads();
    for (int idx = tid; idx < 2 * HPT * D; idx += kThreads) {
      const int hh = idx / D, jj = idx - hh * D;
      sm.a[hh][jj] = hh < G ? sm.qh[hh][jj] * sm.colk[jj] : 0.f;
      sm.s[hh][jj] = 0.f;
    }
    __syncthreads();

    // ---- scores: s_t = r'_t * sum_j a_j (code_tj - 1.5) ----
    {
      const uint32_t *row = reinterpret_cast<const uint32_t *>(a.k_codes + chunk * CHUNK_BYTES + tt * 32);
      const bool live = k * T + tt < len;
      float s[HPT];
#pragma unroll
      for (int r = 0; r < HPT; ++r) s[r] = 0.f;
#pragma unroll 1
      for (int d = 0; d < 8; ++d) {
        const uint32_t wdd = row[d];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float cv = (float)((wdd >> (2 * e)) & 3u) - 1.5f;
#pragma unroll
          for (int r = 0; r < HPT; ++r) s[r] = fmaf(sm.a[h0 + 2 * r][16 * d + e], cv, s[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < HPT; ++r)
        if (h0 + 2 * r < G) sm.s[h0 + 2 * r][tt] = live ? s[r] * sm.rowk[tt] : -INFINITY;
    }
    __syncthreads();

    // ---- online softmax, one wave per head ----
    {
      const int wv = tid >> 6, lane = tid & 63;
      for (int hh = wv; hh < G; hh += kThreads / 64) {
        const float s0 = sm.s[hh][lane], s1 = sm.s[hh][lane + 64];
        const float mc = wave_max(fmaxf(s0, s1));
        const float mo = sm.m[hh];
        const float mn = fmaxf(mo, mc);
        const float al = (mn == -INFINITY) ? 1.f : exp2f(mo - mn);
        const float p0 = (mn == -INFINITY) ? 0.f : exp2f(s0 - mn);
        const float p1 = (mn == -INFINITY) ? 0.f : exp2f(s1 - mn);
        const float ps = wave_sum(p0 + p1);
        sm.s[hh][lane] = p0 * sm.rowv[lane];
        sm.s[hh][lane + 64] = p1 * sm.rowv[lane + 64];
        if (lane == 0) {
          sm.alpha[hh] = al;
          sm.m[hh] = mn;
          sm.l[hh] = sm.l[hh] * al + ps;
        }
      }
    }
    __syncthreads();

    // ---- acc_j = acc_j * alpha + c_j * sum_t P_t (code_tj - 1.5) ----
    {
      const uint32_t *row = reinterpret_cast<const uint32_t *>(a.v_codes + chunk * CHUNK_BYTES + j * 32);
      float s[HPT];
#pragma unroll
      for (int r = 0; r < HPT; ++r) s[r] = 0.f;
#pragma unroll 1
      for (int d = 0; d < 8; ++d) {
        const uint32_t wdd = row[d];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float cv = (float)((wdd >> (2 * e)) & 3u) - 1.5f;
#pragma unroll
          for (int r = 0; r < HPT; ++r) s[r] = fmaf(sm.s[h0 + 2 * r][16 * d + e], cv, s[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < HPT; ++r) acc[r] = acc[r] * sm.alpha[h0 + 2 * r] + sm.colv[j] * s[r];
    }
  }
  __syncthreads();
  // partial: [b][h][split][m, l, acc[128]]
  {
#pragma unroll
    for (int r = 0; r < HPT; ++r) {
      const int hh = h0 + 2 * r;
      if (hh >= G) break;
      float *pp = a.partial + (((int64_t)b * a.q_heads + g * G + hh) * a.n_split + split) * (2 + D);
      pp[2 + j] = acc[r];
      if (j == 0) {
        pp[0] = sm.m[hh];
        pp[1] = sm.l[hh];
      }
    }
  }
}

__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float o[D];
  const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  const float *pp = a.partial + ((int64_t)b * a.q_heads + h) * a.n_split * (2 + D);
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, pp[s * (2 + D)]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.n_split; ++s) {
      const float ms = pp[s * (2 + D)];
      if (ms == -INFINITY) continue;
      const float e = exp2f(ms - M);
      den += e * pp[s * (2 + D) + 1];
      num += e * pp[s * (2 + D) + 2 + j];
    }
  }
  o[j] = den > 0.f ? num / den : 0.f;
  __syncthreads();
  lds_fwht_rows(o, 1);
  a.out[((int64_t)b * a.q_heads + h) * D + j] = o[j] * kInvSqrtD;
}

}  // namespace

int decode_auto_splits(int batch, int kv_heads, int capacity) {
  const int nch = capacity / T;
  const int pairs = batch * kv_heads;
  if (pairs <= 0 || nch <= 0) return 1;
  int s = (1024 + pairs - 1) / pairs;
  if (s > nch) s = nch;
  if (s < 1) s = 1;
  return s;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.q_heads == 0) return hipSuccess;
  const dim3 grid(a.n_split, a.kv_heads, a.batch);
  switch ((a.q_heads / a.kv_heads + 1) / 2) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(decode_split_kernel<3>, grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.q_heads, a.batch), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvarn
