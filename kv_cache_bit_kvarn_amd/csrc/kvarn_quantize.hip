// Block quantizer of the KVarN method on gfx950.
//
// One workgroup (512 threads, 8 wave64) quantizes one 128-token x 128-channel
// block of K or V (one layer, sequence, kv-head, chunk) at a time and walks
// the blocks of the launch persistently (stride = grid), loading the next
// block's bf16 input into registers while the current one is coded.
// Row role: the four lanes of a quad share a token, 32 channels each. Column
// role: the four lanes of a quad share a channel, a quarter of the tokens each.
//   1. bf16/fp32 -> fp32 registers (16-byte loads, one token row per quad);
//   2. Hadamard rotation along channels (rndamp article on KVarN, "How It
//      Works", item 1): five butterfly stages inside each lane, the last two
//      between the lanes of the quad as one DPP-sourced v_fmac each;
//   3. dual-scaling normalization ("How It Works", item 2; abstract: both
//      axes of K and V): squared values P stay in registers for the row step
//      and are staged once, transposed, in LDS for the column step; partial
//      sums meet across the quad by DPP;
//   4. per-token range step and 2-bit codes, packed four per byte
//      (v_cvt_pk_u8_f32 + v_dot4_u32_u8); K token-major straight from
//      registers, V channel-major through an LDS byte transpose;
//   5. 8-byte stores of K codes, 4-byte stores of V code words, fp32 scales.
// The rotation is applied without its 1/sqrt(128) factor; that factor leaves
// the column scales and codes unchanged and is folded into the row scale.
//
// Code decision: the oracle takes code = floor(u + 2), u = y/(r' c) in [-2, 2].
// Here t = u * (1 - 2^-20) + 1.5 is rounded to nearest by v_cvt_pk_u8_f32;
// the shrink keeps the range-step element (|u| = 2) inside the grid, and the
// result equals floor(u + 2) for every element farther than 2e-6 from a
// rounding boundary u in {-1, 0, 1}.
#include "kvarn_internal.h"

namespace kvarn {

FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.s = 31 + l;
  f.m = (uint32_t)(((1ull << f.s) + d - 1) / d);
  return f;
}

namespace {

constexpr int kThreads = 512;
constexpr int CPT = 32;           // channels per thread (row role), tokens per thread (column role)
constexpr int CB_PITCH = D + 16;  // bytes per token row of the V code staging
constexpr float kGrid = 1.9999980926513672f;  // 2 (1 - 2^-20)
constexpr uint32_t kPack4 = 0x40100401u;       // byte weights 1, 4, 16, 64

// LDS layouts, chosen so that the accesses below are free of bank conflicts:
//  * per-channel w and per-token v: quarter q of the 128 entries starts at
//    36 q (the quarters are read by different lanes of one 16-byte access);
//  * transposed P: entry (channel j, token i) at pt_at(j, i): rows 144 floats
//    apart, token quarters 36 floats apart, and 8 more floats per channel
//    quarter (one row-role write instruction covers 8 tokens x 4 quarters).
__host__ __device__ constexpr int qpad(int i) { return i + 4 * (i >> 5); }
constexpr int PT_STRIDE = 144;
__host__ __device__ constexpr int pt_at(int j, int i) {
  return j * PT_STRIDE + 8 * (j >> 5) + qpad(i);
}
constexpr int PT_SIZE = pt_at(D - 1, T - 1) + 1;

struct QuantSmem {
  float w[qpad(D - 1) + 1];  // 1/c_j^2 while balancing, then 1/c_j
  float v[qpad(T - 1) + 1];  // 1/r_i^2
  float pt[PT_SIZE];         // transposed P (V blocks reuse it for code bytes)
};
static_assert(T * CB_PITCH <= (int)sizeof(float) * PT_SIZE, "V staging fits in pt");

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;  // quad_perm [2,3,0,1]
__device__ __forceinline__ float quad_sum(float s) {
  s += dpp_f<kXor1>(s);
  return s + dpp_f<kXor2>(s);
}
__device__ __forceinline__ float quad_max(float s) {
  s = fmaxf(s, dpp_f<kXor1>(s));
  return fmaxf(s, dpp_f<kXor2>(s));
}

// Sum of 32 products in four interleaved partial sums (eight terms each)
// combined as a tree, keeping fp32 rounding close to that of a pairwise sum.
// LDS operands are fetched four vectors at a time ahead of their FMAs.
__device__ __forceinline__ float dot32(const float (&p)[CPT], const float *w) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 ww[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ww[q] = reinterpret_cast<const f32x4 *>(w)[4 * h + q];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 16 * h + 4 * q;
      acc[0] = fmaf(p[e + 0], ww[q].x, acc[0]);
      acc[1] = fmaf(p[e + 1], ww[q].y, acc[1]);
      acc[2] = fmaf(p[e + 2], ww[q].z, acc[2]);
      acc[3] = fmaf(p[e + 3], ww[q].w, acc[3]);
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Same, both operands from LDS (column step: P_ij * v_i over 32 tokens).
__device__ __forceinline__ float dot32_lds(const float *a, const float *b) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 x[4], y[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] = reinterpret_cast<const f32x4 *>(a)[4 * h + q];
      y[q] = reinterpret_cast<const f32x4 *>(b)[4 * h + q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[0] = fmaf(x[q].x, y[q].x, acc[0]);
      acc[1] = fmaf(x[q].y, y[q].y, acc[1]);
      acc[2] = fmaf(x[q].z, y[q].z, acc[2]);
      acc[3] = fmaf(x[q].w, y[q].w, acc[3]);
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Cross-lane butterfly of one channel bit for 8 registers at once:
// y = y(partner) * s + y, one v_fmac_f32 with a DPP source each. With s = +1
// on the lane whose channel bit is 0 this yields A + B there and -(A - B) on
// the partner lane (s = -1); the caller tracks the partner lane's sign. The
// leading s_nop covers the DPP read-after-VALU-write hazard (2 wait states)
// for registers written just before the block.
#define KVARN_BUTTERFLY_X8(PERM)                                                              \
  asm("s_nop 1\n\t"                                                                           \
      "v_fmac_f32_dpp %0, %0, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %1, %1, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %2, %2, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %3, %3, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %4, %4, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %5, %5, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %6, %6, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %7, %7, %8 " PERM " row_mask:0xf bank_mask:0xf"                         \
      : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]), \
        "+v"(y[7])                                                                            \
      : "v"(s))
__device__ __forceinline__ void butterfly_xor1_x8(float *y, float s) {
  KVARN_BUTTERFLY_X8("quad_perm:[1,0,3,2]");
}
__device__ __forceinline__ void butterfly_xor2_x8(float *y, float s) {
  KVARN_BUTTERFLY_X8("quad_perm:[2,3,0,1]");
}
#undef KVARN_BUTTERFLY_X8

struct BlockIdx {
  uint32_t bh, kc, b, h;
};
__device__ __forceinline__ BlockIdx split_block(const QuantArgs &a, uint32_t blk) {
  BlockIdx r;
  r.bh = fdiv(blk, a.div_chunks);
  r.kc = blk - r.bh * (uint32_t)a.chunks;
  r.b = fdiv(r.bh, a.div_heads);
  r.h = r.bh - r.b * (uint32_t)a.heads;
  return r;
}

__device__ __forceinline__ int64_t x_offset(const QuantArgs &a, const BlockIdx &bi, int ti, int hq) {
  return (int64_t)bi.b * a.sb + (int64_t)bi.h * a.sh + (int64_t)(bi.kc * T + ti) * a.st + CPT * hq;
}

__device__ __forceinline__ void load_bf16_block(const QuantArgs &a, uint32_t blk, int ti, int hq,
                                                u32x4 (&xr)[4]) {
  const BlockIdx bi = split_block(a, blk);
  const u32x4 *src =
      reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.x) + x_offset(a, bi, ti, hq));
#pragma unroll
  for (int q = 0; q < 4; ++q) xr[q] = __builtin_nontemporal_load(src + q);
}

// kRotate = false: the input is already rotated (rotation absorbed into the
// model's weights) and the rotation step is skipped.
template <bool kF32, bool kRotate>
__global__ __launch_bounds__(kThreads, 4) void quantize_block_kernel(QuantArgs a) {
  __shared__ QuantSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int ti = wv * 16 + (lane >> 2);  // row role: token ti,
  const int hq = lane & 3;               //   channels [32 hq, 32 hq + 32)
  const int cj = tid >> 2;               // column role: channel cj,
  const int cq = tid & 3;                //   tokens [32 cq, 32 cq + 32)
  const int64_t nch = a.capacity / T;
  // the two cross-lane butterflies leave negated the values of the lanes
  // whose hq bit 0 (first) or bit 1 (second) is set
  const float s1 = (hq & 1) ? -1.f : 1.f, s2 = (hq & 2) ? -1.f : 1.f;
  const float lane_sign = kRotate ? s1 * s2 : 1.f;
  // r' from the running maximum: the unscaled rotation's 1/sqrt(128) and the
  // 1/2 of the range step, or the 1/2 alone for pre-rotated input
  const float range_factor = kRotate ? kRangeFromUnscaled : kRangeFromRotated;

  u32x4 xr[4];
  uint32_t blk = blockIdx.x;
  if constexpr (!kF32) {
    if (blk < a.nblocks) load_bf16_block(a, blk, ti, hq, xr);
  }
  for (; blk < a.nblocks; blk += gridDim.x) {
    const BlockIdx bi = split_block(a, blk);
    const int64_t bh = bi.bh;
    const int chunk = a.chunk0 + (int)bi.kc;

    // ---- 1. load -----------------------------------------------------------
    float y[CPT];
    if constexpr (kF32) {
      const f32x4 *src =
          reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.x) + x_offset(a, bi, ti, hq));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 v = __builtin_nontemporal_load(src + q);
        y[4 * q + 0] = v.x; y[4 * q + 1] = v.y; y[4 * q + 2] = v.z; y[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 u = xr[q];
        y[8 * q + 0] = bf16_lo(u.x); y[8 * q + 1] = bf16_hi(u.x);
        y[8 * q + 2] = bf16_lo(u.y); y[8 * q + 3] = bf16_hi(u.y);
        y[8 * q + 4] = bf16_lo(u.z); y[8 * q + 5] = bf16_hi(u.z);
        y[8 * q + 6] = bf16_lo(u.w); y[8 * q + 7] = bf16_hi(u.w);
      }
    }

    // ---- 2. rotation: y <- y . H_128 (Sylvester order, unscaled) -----------
    if constexpr (kRotate) {
#pragma unroll
      for (int len = 1; len < CPT; len <<= 1) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          if ((i & len) == 0) {
            const float p = y[i], q = y[i + len];
            y[i] = p + q;
            y[i + len] = p - q;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < CPT; i += 8) butterfly_xor1_x8(y + i, s1);
#pragma unroll
      for (int i = 0; i < CPT; i += 8) butterfly_xor2_x8(y + i, s2);
    }

    // ---- 3. dual scaling ---------------------------------------------------
    float p[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) p[i] = y[i] * y[i];
    if (a.kind == KVARN_V) lds_barrier();  // previous block's readers done with the staging
    {
      float *dst = sm.pt + pt_at(CPT * hq, ti);
#pragma unroll
      for (int i = 0; i < CPT; ++i) dst[i * PT_STRIDE] = p[i];
    }
    lds_barrier();

    float *colp = a.col_scale + (bh * nch + chunk) * D;
    for (int it = 0; it < a.iters; ++it) {
      // row step: r_i^2 = (1/D) sum_j P_ij / c_j^2  ->  v_i = 1/r_i^2  (c = 1 first)
      float s;
      if (it == 0) {
        float acc[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
        for (int i = 4; i < CPT; ++i) acc[i & 3] += p[i];
        s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      } else {
        s = dot32(p, sm.w + qpad(CPT * hq));
      }
      s = quad_sum(s);
      if (hq == 0) sm.v[qpad(ti)] = s > 0.f ? (float)D * rcp(s) : 1.f;
      lds_barrier();
      // column step: c_j^2 = (1/T) sum_i P_ij / r_i^2  ->  w_j = 1/c_j^2
      float cs = dot32_lds(sm.pt + pt_at(cj, CPT * cq), sm.v + qpad(CPT * cq));
      cs = quad_sum(cs);
      if (cq == 0) {
        const float cm = cs * (1.f / T);
        const int wj = qpad(cj);
        if (it + 1 < a.iters) {
          sm.w[wj] = cm > 0.f ? rcp(cm) : 1.f;
        } else {
          colp[cj] = cm > 0.f ? sqrtf(cm) : 1.f;
          sm.w[wj] = cm > 0.f ? __builtin_amdgcn_rsqf(cm) : 1.f;
        }
      }
      lds_barrier();
    }
    if (a.iters == 0) {
      if (tid < D) {
        colp[tid] = 1.f;
        sm.w[qpad(tid)] = 1.f;
      }
      lds_barrier();
    }

    if constexpr (!kF32) {
      // next block's input: issued here, where the registers are free, and
      // unconditionally (clamped) so that xr stays in place across iterations
      const uint32_t nb = min(blk + gridDim.x, a.nblocks - 1);
      load_bf16_block(a, nb, ti, hq, xr);
    }

    // ---- 4. range step and codes --------------------------------------------
    float m = 0.f;
    {
      const f32x4 *ic = reinterpret_cast<const f32x4 *>(sm.w + qpad(CPT * hq));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 w4 = ic[q];
        y[4 * q + 0] *= w4.x; y[4 * q + 1] *= w4.y; y[4 * q + 2] *= w4.z; y[4 * q + 3] *= w4.w;
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) m = fmaxf(m, fabsf(y[i]));
    }
    m = quad_max(m);
    if (hq == 0) a.row_scale[bh * a.capacity + (int64_t)chunk * T + ti] = m * range_factor;
    const float qs = m > 0.f ? lane_sign * kGrid * rcp(m) : 0.f;
    // cw[d] byte k = code of channel 32 hq + 4 d + k
    uint32_t cw[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t acc = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        acc = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[4 * d + k], qs, 1.5f), k, acc);
      cw[d] = acc;
    }

    uint8_t *cbase = a.codes + (bh * nch + chunk) * CHUNK_BYTES;
    if (a.kind == KVARN_K) {
      u32x2 pk;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint32_t o = __builtin_amdgcn_udot4(cw[4 * q + 0], kPack4, 0u, false);
        o |= __builtin_amdgcn_udot4(cw[4 * q + 1], kPack4, 0u, false) << 8;
        o |= __builtin_amdgcn_udot4(cw[4 * q + 2], kPack4, 0u, false) << 16;
        o |= __builtin_amdgcn_udot4(cw[4 * q + 3], kPack4, 0u, false) << 24;
        pk[q] = o;
      }
      *reinterpret_cast<u32x2 *>(cbase + ti * 32 + hq * 8) = pk;
    } else {
      // token-major byte staging, then each of 256 threads transposes 4
      // channels x 16 tokens: 4x4 byte transposes (v_perm) and 2-bit packing
      // (v_dot4)
      uint8_t *cb = reinterpret_cast<uint8_t *>(sm.pt);
      u32x4 *dst = reinterpret_cast<u32x4 *>(cb + ti * CB_PITCH + CPT * hq);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 v4;
        v4[0] = cw[4 * q + 0]; v4[1] = cw[4 * q + 1]; v4[2] = cw[4 * q + 2]; v4[3] = cw[4 * q + 3];
        dst[q] = v4;
      }
      lds_barrier();
      if (tid < 256) {
        const int j4 = tid & 31;   // channels [4 j4, 4 j4 + 4)
        const int n4 = tid >> 5;   // tokens [16 n4, 16 n4 + 16)
        uint32_t word[4] = {0u, 0u, 0u, 0u};  // per channel: 16 tokens, 2 bits each
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint8_t *src = cb + (16 * n4 + 4 * q) * CB_PITCH + 4 * j4;
          const uint32_t w0 = *reinterpret_cast<const uint32_t *>(src);
          const uint32_t w1 = *reinterpret_cast<const uint32_t *>(src + CB_PITCH);
          const uint32_t w2 = *reinterpret_cast<const uint32_t *>(src + 2 * CB_PITCH);
          const uint32_t w3 = *reinterpret_cast<const uint32_t *>(src + 3 * CB_PITCH);
          const uint32_t t01l = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
          const uint32_t t01h = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
          const uint32_t t23l = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
          const uint32_t t23h = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
          const uint32_t o0 = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
          const uint32_t o1 = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
          const uint32_t o2 = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
          const uint32_t o3 = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
          word[0] |= __builtin_amdgcn_udot4(o0, kPack4, 0u, false) << (8 * q);
          word[1] |= __builtin_amdgcn_udot4(o1, kPack4, 0u, false) << (8 * q);
          word[2] |= __builtin_amdgcn_udot4(o2, kPack4, 0u, false) << (8 * q);
          word[3] |= __builtin_amdgcn_udot4(o3, kPack4, 0u, false) << (8 * q);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
          *reinterpret_cast<uint32_t *>(cbase + (4 * j4 + s) * 32 + 4 * n4) = word[s];
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &a, hipStream_t s) {
  if (a.nblocks == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // two resident workgroups per CU (LDS- and register-limited); each walks
  // blocks strided by the grid
  const uint32_t resident = 2u * (uint32_t)(cus > 0 ? cus : 1);
  const uint32_t blocks = a.nblocks < resident ? a.nblocks : resident;
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE);
  if (a.dtype == KVARN_DT_F32) {
    if (rot)
      hipLaunchKernelGGL((quantize_block_kernel<true, true>), dim3(blocks), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_block_kernel<true, false>), dim3(blocks), dim3(kThreads), 0, s, a);
  } else {
    if (rot)
      hipLaunchKernelGGL((quantize_block_kernel<false, true>), dim3(blocks), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_block_kernel<false, false>), dim3(blocks), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvarn
