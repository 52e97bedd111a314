// Internal declarations shared by the HIP translation units of libkvarn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvarn.h"

namespace kvarn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = KVARN_HEAD_DIM;      // channels per head
constexpr int T = KVARN_CHUNK;         // tokens per block
constexpr int CHUNK_BYTES = KVARN_CHUNK_BYTES;
constexpr int GQA_MAX = 8;             // query heads per kv-head supported by decode

// 1/sqrt(d) for the head sizes served (64, 128, 256; exact powers of two for
// 64 and 256). The rotation is applied unscaled on the device (y' = sqrt(d) y),
// so the range step r' = max|y/c|/2 becomes max|y'/c| / sqrt(d) / 2, while c
// and every code are unchanged by that factor.
__host__ __device__ constexpr float inv_sqrt_head(int d) {
  return d == 64 ? 0.125f : d == 256 ? 0.0625f : 0.088388347648318447f;
}
__host__ __device__ constexpr float range_from_unscaled(int d) { return 0.5f * inv_sqrt_head(d); }
static_assert(range_from_unscaled(128) == 0.044194173824159216f, "2^-4.5");
// r' = max|y/c|/2 for input that is already rotated (KVARN_FLAG_NO_ROTATE)
constexpr float kRangeFromRotated = 0.5f;

// ---- cross-lane helpers (DPP on gfx950, wave64) -------------------------
// The value that lane (l ^ M) of the wave holds, for M = 1, 2, 4, 8, 16, 32,
// by VALU lane exchanges: quad permutes (M = 1, 2), a quad reversal followed
// by a half-row mirror (M = 4: lane i reads (i ^ 7) ^ 3 = i ^ 4), a rotation
// by 8 within the 16-lane row (M = 8), and the row-pair and half-wave swaps
// (M = 16, 32). A lane shuffle (ds_bpermute) is an LDS round trip instead,
// several times slower in a dependent chain.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const int r = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false);        // quad_perm [3,2,1,0]
    return __int_as_float(__builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, false));  // row_half_mirror
  } else if constexpr (M == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));  // row_ror:8
  } else if constexpr (M == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    return __uint_as_float(((threadIdx.x >> 4) & 1) ? s[0] : s[1]);
  } else {
    static_assert(M == 32, "lane_xor: M is a power of two below 64");
    const auto s = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return __uint_as_float(((threadIdx.x >> 5) & 1) ? s[0] : s[1]);
  }
}
// The same for an M known after unrolling.
__device__ __forceinline__ float lane_xor(float v, int m) {
  switch (m) {
    case 1: return lane_xor<1>(v);
    case 2: return lane_xor<2>(v);
    case 4: return lane_xor<4>(v);
    case 8: return lane_xor<8>(v);
    case 16: return lane_xor<16>(v);
    default: return lane_xor<32>(v);
  }
}

// s_waitcnt operand on gfx9 that waits until at most n vector-memory
// operations of the wave are outstanding (vmcnt bits 3:0 and 15:14), with
// expcnt and lgkmcnt left at their maxima
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kVmcntZero = waitcnt_vm(0);
static_assert(kVmcntZero == ((0x7 << 4) | (0xF << 8)), "vmcnt(0) encoding");

// Workgroup barrier for LDS traffic only: the wave's LDS accesses complete
// (lgkmcnt(0)), then s_barrier. Unlike __syncthreads() it does not wait for
// outstanding global loads and stores, so a prefetch stays in flight across
// it. The wavefront-scope fences keep the compiler from moving LDS accesses
// across the barrier; LDS is coherent inside the workgroup.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// ---- launchers (validated arguments only) --------------------------------
// Division by a runtime divisor d (1 <= d < 2^31) of n < 2^31 as
// (n * m) >> s with m = ceil(2^s / d), s = 31 + ceil(log2 d).
struct FastDiv {
  uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.s = 31 + l;
  f.m = (uint32_t)(((1ull << f.s) + d - 1) / d);
  return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

struct QuantArgs {
  const void *x;
  int dtype;
  int head_dim;         // channels per head: 64, 128 or 256
  int64_t sb, sh, st;
  int batch, heads, chunks, chunk0, iters, capacity, kind;
  uint32_t flags;       // KVARN_FLAG_NO_ROTATE
  uint32_t nblocks;     // batch * heads * chunks (< 2^31)
  // when set: x is a one-chunk window per (b, h) (chunks = 1) and block
  // (b, h) goes to cache chunk pos[b] / 128, only when pos[b] % 128 == 127
  const int32_t *pos;
  FastDiv div_chunks, div_heads;
  uint8_t *codes;
  float *row_scale, *col_scale;
};
hipError_t launch_quantize(const QuantArgs &a, hipStream_t s);

struct AppendArgs {
  const void *x;
  int dtype;
  int head_dim;
  const int32_t *pos;
  int batch, heads, capacity, kind;
  uint32_t flags;  // KVARN_FLAG_NO_ROTATE
  uint8_t *codes;
  float *row_scale, *col_scale;
  void *window;    // when set: [batch][heads][128][128] of x's dtype; the token
                   // is also stored, as given, at slot pos % 128
};
hipError_t launch_append(const AppendArgs &a, hipStream_t s);
// k and v: the same batch, heads, capacity, head size, dtype and flags
hipError_t launch_append_kv(const AppendArgs &k, const AppendArgs &v, hipStream_t s);

struct DecodeArgs {
  const void *q;
  int q_dtype, batch, q_heads, kv_heads, capacity;
  int head_dim;
  int n_wg;        // workgroups (of KVARN_DECODE_WAVES splits) per (sequence, kv-head, head group)
  uint32_t flags;  // KVARN_FLAG_NO_ROTATE, KVARN_FLAG_ONE_SCALE
  const uint8_t *k_codes, *v_codes;
  const float *k_row, *k_col, *v_row, *v_col;
  const int32_t *lens;
  float scale;
  float *out;
  int32_t *counters;  // one per (sequence, kv-head, head group); zero between calls
  float *partial;     // [batch][q_heads][n_wg][2 + head_dim]
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
int device_cus();  // compute units of the current device, cached per device
// Device address of the current device's copy of the library's fixed decode
// scratch array (KVARN_NOALLOC_SCRATCH_BYTES), taken once per device; nullptr
// with *err set when the query fails.
void *noalloc_scratch(hipError_t *err);
// the most workgroups per row that still give every split a chunk
inline int decode_max_wgs(int capacity) {
  return (capacity / T + KVARN_DECODE_WAVES - 1) / KVARN_DECODE_WAVES;
}
int decode_auto_wgs(int batch, int kv_heads, int q_heads, int capacity, int head_dim);
// Workspace layout: counters (batch * q_heads int32, rounded up to 256 bytes;
// q_heads bounds the number of (kv-head, head group) rows), then the partials.
inline size_t decode_counter_bytes(int32_t batch, int32_t q_heads) {
  return ((size_t)batch * q_heads * sizeof(int32_t) + 255) / 256 * 256;
}
inline size_t decode_partial_bytes(int32_t batch, int32_t q_heads, int n_wg, int head_dim) {
  return (size_t)batch * q_heads * (size_t)n_wg * (2 + head_dim) * sizeof(float);
}


}  // namespace kvarn
