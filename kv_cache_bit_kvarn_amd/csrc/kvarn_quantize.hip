// Block quantizer of the KVarN method on gfx950.
//
// One workgroup (512 threads, 8 wave64) quantizes one 128-token x 128-channel
// block of K or V (one layer, sequence, kv-head, chunk) at a time and walks
// the blocks of the launch persistently (stride = grid), loading the next
// block's bf16 input into registers while the current one is coded. Wave w
// owns tokens [16 w, 16 w + 16); lane (n = lane % 16, g = lane / 16) holds
// token 16 w + n.
//   1. load: each lane reads four 16-byte pieces of its token row (channels
//      32 kk + 8 g + [0, 8)), so one load instruction covers 64 contiguous
//      bytes of each of 16 rows; the pieces are the B operands of the MFMAs;
//   2. Hadamard rotation along channels (rndamp article on KVarN, "How It
//      Works", item 1) as a dense product on the matrix cores:
//      y^T = H_128 x^T with v_mfma_f32_16x16x32_bf16, 32 MFMAs per wave.
//      Sylvester's H_128 has entry (-1)^popcount(i & j); split over the tile
//      indices, each 16 x 32 tile (mt, kk) of it is a sign
//      (-1)^popcount((mt/2) & kk) times one of two lane-constant operands
//      (mt % 2), the sign going onto the input piece. The result lands with
//      lane (n, g) holding channels 16 mt + 4 g + r of its token. (The
//      product could also be 8 MFMAs and a 4-point transform over the pieces,
//      but that moves 64 adds per lane onto the VALU, which bounds the
//      kernel, while the matrix cores are mostly idle.)
//      bf16 inputs and +-1 are exact and the products accumulate in fp32;
//      fp32 input is split exactly into three bf16 terms (three MFMAs per
//      product). With the rotation absorbed into the weights, the MFMAs run
//      on identity tiles (one per output tile), which copies x exactly;
//   3. dual-scaling normalization ("How It Works", item 2; abstract: both
//      axes of K and V): the squares P = y^2 stay in registers (next to y)
//      for the row step and are staged once, transposed, in LDS for the
//      column step; the per-channel and per-token factors are read once per
//      lane and shared across 16-lane rows by DPP broadcasts; a token's four
//      partial row sums meet through lane exchanges 16 and 32 apart;
//   4. per-token range step and 2-bit codes (v_cvt_pk_u8_f32): K codes are
//      packed four per byte (v_dot4_u32_u8) and transposed across the four
//      lanes of a token (one permlane32 swap, one exchange 16 lanes apart) so
//      that each lane stores 8 contiguous bytes of its token row; V codes are
//      packed four tokens per byte with a shift and an OR across the four
//      adjacent lanes, staged in LDS and stored as 4-byte words per channel.
// The rotation is applied without its 1/sqrt(128) factor; that factor leaves
// the column scales and codes unchanged and is folded into the row scale.
//
// Code decision: the oracle takes code = floor(u + 2), u = y/(r' c) in [-2, 2].
// Here t = u * (1 - 2^-20) + 1.5 is rounded to nearest by v_cvt_pk_u8_f32;
// the shrink keeps the range-step element (|u| = 2) inside the grid, and the
// result equals floor(u + 2) for every element farther than 2e-6 from a
// rounding boundary u in {-1, 0, 1}. (Deciding on y |y| / c^2 instead would
// spare y's registers but loses the sign of u within about 2e-4 of 0 once
// 1.5 is added.)
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
constexpr int CPT = 32;                        // values per lane: channels (rows), tokens (columns)
constexpr float kGrid = 1.9999980926513672f;  // 2 (1 - 2^-20)
constexpr uint32_t kPack4 = 0x40100401u;       // byte weights 1, 4, 16, 64

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// LDS layouts. On gfx950 a ds_write_b32 is served one half-wave per pass with
// the dword address taken modulo 32 as its bank; a ds_read_b64 one half-wave
// per pass over 64 four-byte banks; a ds_read_b128 in four passes of 16 lanes
// (the quads of one half-wave whose quad index has the same popcount parity)
// over 64 banks; a lane reading the same address as another still takes its
// own bank slot. The layouts below are free of bank conflicts under that
// model:
//  * transposed P: entry (channel j, token i) at pt_at(j, i): rows 132
//    floats apart, 32 more floats per group of 8 channels (a P write covers
//    16 tokens x channels 4 apart; a column-step read covers 16 channels);
//  * per-channel w at wpad(j) (8 floats of padding after channel 63) and
//    per-token v, each read once per lane as a pair and shared across a
//    16-lane row by DPP broadcasts;
//  * V code staging, in the P area once the column steps are done: word
//    (mt, g, byte column 4 c + e) at vs_at(mt, g, c, e) = 32 (4 mt + g) +
//    4 (c ^ ((mt + 4 g) % 8)) + e (16-byte chunks swizzled).
constexpr int PT_STRIDE = 132;
__host__ __device__ constexpr int pt_at(int j, int i) {
  return j * PT_STRIDE + 32 * (j >> 3) + i;
}
__host__ __device__ constexpr bool pt_rows_disjoint() {
  for (int j = 0; j + 1 < D; ++j)
    if (pt_at(j, T - 1) >= pt_at(j + 1, 0)) return false;
  return true;
}
static_assert(pt_rows_disjoint(), "rows of the transposed P overlap");
constexpr int PT_SIZE = pt_at(D - 1, T - 1) + 1;
__host__ __device__ constexpr int wpad(int j) { return j + 8 * (j >> 6); }
__host__ __device__ constexpr int vs_at(int mt, int g, int c, int e) {
  return 32 * (4 * mt + g) + 4 * (c ^ ((mt + 4 * g) & 7)) + e;
}

struct QuantSmem {
  alignas(16) float w[wpad(D - 1) + 1];  // 1/c_j^2
  alignas(16) float wc[wpad(D - 1) + 1]; // 1/c_j after the last column step
  alignas(16) float v[T];                // 1/r_i^2
  alignas(16) float pt[PT_SIZE];         // transposed P, then V code staging
  alignas(16) u32x4 hop[2][64];          // rotation operands of each lane
};
static_assert(vs_at(7, 3, 7, 3) < PT_SIZE, "V staging fits in the P area");

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Sum (max) over the four 16-lane rows of the wave, in every lane: the
// permlane32 swap pairs rows 0-1 with rows 2-3, the permlane16 swap then row
// 0 with 1 and 2 with 3 (VALU lane exchanges, no LDS round trip).
__device__ __forceinline__ float rows_sum(float s) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  const float t = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float s) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  const float t = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The value itself, hidden from the optimizer so that addresses built from it
// are recomputed where they are used instead of being hoisted out of the block
// loop and kept (or spilled) across the balancing.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;  // quad_perm [2,3,0,1]

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// A operand of the rotation for output-channel tile parity p. Lane (m, g),
// slot e multiplies input channel 32 kk + 8 g + e into output channel
// 16 mt + m (the B operand's slot e of lane group g holds that channel):
// popcount((16 mt + m) & (32 kk + 8 g + e)) splits into popcount(m & e),
// m bit 3 with g bit 0, mt bit 0 (= p) with g bit 1, and (mt / 2) & kk; the
// last part is the tile's sign, the others are fixed per lane and slot.
__device__ __forceinline__ u32x4 hadamard_operand(int lane, int p) {
  const int m = lane & 15, g = lane >> 4;
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t word = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int e = 2 * h + s;
      const int odd = (__builtin_popcount(m & e) + ((m >> 3) & g & 1) + (p & (g >> 1))) & 1;
      word |= (odd ? 0xBF80u : 0x3F80u) << (16 * s);  // bf16 -1 / +1
    }
    r[h] = word;
  }
  return r;
}
// Identity tile for input that is already rotated: output channel
// 16 mt + m takes input channel 32 (mt / 2) + 8 g + e exactly when
// g = 2 (mt % 2) + m / 8 and e = m % 8.
__device__ __forceinline__ u32x4 identity_operand(int lane, int p) {
  const int m = lane & 15, g = lane >> 4;
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t word = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int e = 2 * h + s;
      if ((g >> 1) == p && m == 8 * (g & 1) + e) word |= 0x3F80u << (16 * s);
    }
    r[h] = word;
  }
  return r;
}

// acc[mt] += (tile (mt, kk) of the rotation) x b, b = input channels
// 32 kk + [0, 32) of the wave's 16 tokens. A Hadamard tile with a negative
// sign takes the negated b (sign bits flipped) against the same operand; the
// identity has one tile per output tile, at kk = mt / 2.
template <bool kRotate, int KK>
__device__ __forceinline__ void rotate_step(f32x4 (&acc)[8], const u32x4 &b, const u32x4 (&hp)[2]) {
  if constexpr (kRotate) {
    const u32x4 nb = b ^ 0x80008000u;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const bool neg = __builtin_popcount((mt >> 1) & KK) & 1;
      acc[mt] = mfma_bf16(hp[mt & 1], neg ? nb : b, acc[mt]);
    }
  } else {
    acc[2 * KK] = mfma_bf16(hp[0], b, acc[2 * KK]);
    acc[2 * KK + 1] = mfma_bf16(hp[1], b, acc[2 * KK + 1]);
  }
}

// Exact split of eight fp32 values into three bf16 terms (x = hi + mid + lo:
// each term takes the next 8 significant bits), packed as MFMA operands.
__device__ __forceinline__ void split_bf16x3(const f32x4 &a, const f32x4 &b, u32x4 &hi, u32x4 &mid,
                                             u32x4 &lo) {
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t uh[8], um[8], ul[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uh[e] = __float_as_uint(f[e]);
    const float r = f[e] - __uint_as_float(uh[e] & 0xFFFF0000u);
    um[e] = __float_as_uint(r);
    ul[e] = __float_as_uint(r - __uint_as_float(um[e] & 0xFFFF0000u));
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // upper halves of elements 2q, 2q+1
    hi[q] = __builtin_amdgcn_perm(uh[2 * q + 1], uh[2 * q], 0x07060302u);
    mid[q] = __builtin_amdgcn_perm(um[2 * q + 1], um[2 * q], 0x07060302u);
    lo[q] = __builtin_amdgcn_perm(ul[2 * q + 1], ul[2 * q], 0x07060302u);
  }
}

// Eight products of a lane's values x[e] with values held across its 16-lane
// row: x[e] meets register w{e % 2} of row lane L{e / 2} (v_fmac_f32_dpp with
// row_newbcast, which reads that lane of the row), summed into acc[e % 4].
// The leading s_nop covers the DPP read-after-VALU-write hazard.
#define KVARN_FMAC8_BCAST(L0, L1, L2, L3, acc, w0, w1, x)                                        \
  asm("s_nop 1\n\t"                                                                              \
      "v_fmac_f32_dpp %0, %4, %6 row_newbcast:" #L0 " row_mask:0xf bank_mask:0xf\n\t"            \
      "v_fmac_f32_dpp %1, %5, %7 row_newbcast:" #L0 " row_mask:0xf bank_mask:0xf\n\t"            \
      "v_fmac_f32_dpp %2, %4, %8 row_newbcast:" #L1 " row_mask:0xf bank_mask:0xf\n\t"            \
      "v_fmac_f32_dpp %3, %5, %9 row_newbcast:" #L1 " row_mask:0xf bank_mask:0xf\n\t"            \
      "v_fmac_f32_dpp %0, %4, %10 row_newbcast:" #L2 " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %1, %5, %11 row_newbcast:" #L2 " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %2, %4, %12 row_newbcast:" #L3 " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %3, %5, %13 row_newbcast:" #L3 " row_mask:0xf bank_mask:0xf"                 \
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])                                    \
      : "v"(w0), "v"(w1), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]),     \
        "v"(x[6]), "v"(x[7]))
// Same, with acc[] set by the first four products instead of accumulated.
#define KVARN_FMAC8_BCAST_FIRST(L0, L1, L2, L3, acc, w0, w1, x)                                  \
  asm("s_nop 1\n\t"                                                                              \
      "v_mul_f32_dpp %0, %4, %6 row_newbcast:" #L0 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %1, %5, %7 row_newbcast:" #L0 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %2, %4, %8 row_newbcast:" #L1 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %3, %5, %9 row_newbcast:" #L1 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_fmac_f32_dpp %0, %4, %10 row_newbcast:" #L2 " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %1, %5, %11 row_newbcast:" #L2 " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %2, %4, %12 row_newbcast:" #L3 " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %3, %5, %13 row_newbcast:" #L3 " row_mask:0xf bank_mask:0xf"                 \
      : "=&v"(acc[0]), "=&v"(acc[1]), "=&v"(acc[2]), "=&v"(acc[3])                                \
      : "v"(w0), "v"(w1), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]),     \
        "v"(x[6]), "v"(x[7]))
// x[e] *= register w{e % 2} of row lane L{e / 2}.
#define KVARN_MUL8_BCAST(L0, L1, L2, L3, w0, w1, x)                                               \
  asm("s_nop 1\n\t"                                                                              \
      "v_mul_f32_dpp %0, %8, %0 row_newbcast:" #L0 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %1, %9, %1 row_newbcast:" #L0 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %2, %8, %2 row_newbcast:" #L1 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %3, %9, %3 row_newbcast:" #L1 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %4, %8, %4 row_newbcast:" #L2 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %5, %9, %5 row_newbcast:" #L2 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %6, %8, %6 row_newbcast:" #L3 " row_mask:0xf bank_mask:0xf\n\t"             \
      "v_mul_f32_dpp %7, %9, %7 row_newbcast:" #L3 " row_mask:0xf bank_mask:0xf"                   \
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),      \
        "+v"(x[7])                                                                                \
      : "v"(w0), "v"(w1))

// Row step: sum over the lane's 32 channels of p[4 mt + r] / c^2 of channel
// 16 mt + 4 g + r. Row lane n holds 1/c^2 of channels 16 (n / 2) + 4 g +
// 2 (n % 2) + {0, 1} (one 8-byte read), so element (mt, r) sits in register
// r % 2 of lane 2 mt + r / 2. Four interleaved partial sums, tree-combined.
__device__ __forceinline__ float row_dot(const float (&p)[CPT], float w0, float w1) {
  float acc[4];
  KVARN_FMAC8_BCAST_FIRST(0, 1, 2, 3, acc, w0, w1, (p + 0));
  KVARN_FMAC8_BCAST(4, 5, 6, 7, acc, w0, w1, (p + 8));
  KVARN_FMAC8_BCAST(8, 9, 10, 11, acc, w0, w1, (p + 16));
  KVARN_FMAC8_BCAST(12, 13, 14, 15, acc, w0, w1, (p + 24));
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Column step: sum over 32 tokens of P_ij / r_i^2; row lane n holds 1/r^2 of
// tokens 2 n + {0, 1} of the quarter. P is read two 16-byte vectors at a time.
__device__ __forceinline__ float col_dot(const float *pc, float v0, float v1) {
  float acc[4];
#define KVARN_COL_BLOCK(H, L0, L1, L2, L3, FMAC)                                        \
  {                                                                                     \
    const f32x4 a0 = reinterpret_cast<const f32x4 *>(pc)[2 * (H)];                      \
    const f32x4 a1 = reinterpret_cast<const f32x4 *>(pc)[2 * (H) + 1];                  \
    const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};                \
    FMAC(L0, L1, L2, L3, acc, v0, v1, x);                                               \
  }
  KVARN_COL_BLOCK(0, 0, 1, 2, 3, KVARN_FMAC8_BCAST_FIRST)
  KVARN_COL_BLOCK(1, 4, 5, 6, 7, KVARN_FMAC8_BCAST)
  KVARN_COL_BLOCK(2, 8, 9, 10, 11, KVARN_FMAC8_BCAST)
  KVARN_COL_BLOCK(3, 12, 13, 14, 15, KVARN_FMAC8_BCAST)
#undef KVARN_COL_BLOCK
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

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

__device__ __forceinline__ int64_t x_offset(const QuantArgs &a, const BlockIdx &bi, int ti) {
  return (int64_t)bi.b * a.sb + (int64_t)bi.h * a.sh + (int64_t)(bi.kc * T + ti) * a.st;
}

// Piece kk of the lane's token row: channels 32 kk + 8 g + [0, 8).
__device__ __forceinline__ void load_bf16_block(const QuantArgs &a, const BlockIdx &bi, int ti,
                                                int g, u32x4 (&xr)[4]) {
  const u32x4 *src =
      reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.x) + x_offset(a, bi, ti)) + g;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) xr[kk] = __builtin_nontemporal_load(src + 4 * kk);
}

// kRotate = false: the input is already rotated (rotation absorbed into the
// model's weights) and the MFMAs copy it through identity tiles.
// kPositions: x is a one-chunk window per (b, h); block (b, h) re-quantizes
// cache chunk pos[b] / 128 only when pos[b] % 128 == 127, i.e. when the token
// just appended at pos[b] filled its chunk (kvarn_append_rebalance).
template <bool kF32, bool kRotate, bool kPositions>
__global__ __launch_bounds__(kThreads, 4) void quantize_block_kernel(QuantArgs a) {
  __shared__ QuantSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ti = 16 * wv + n;             // token of the lane (rows, codes)
  // column step: channel cj = 16 w + n, token quarter g (its 16-lane row)
  const int cj = 16 * wv + n;
  // the 1/c^2 pair this lane shares with its row (row step, range step)
  const int w_pair = wpad(16 * (n >> 1) + 4 * g + 2 * (n & 1));
  const int64_t nch = a.capacity / T;
  // r' from the running maximum: the unscaled rotation's 1/sqrt(128) and the
  // 1/2 of the range step, or the 1/2 alone for pre-rotated input
  const float range_factor = kRotate ? kRangeFromUnscaled : kRangeFromRotated;

  // the lane's two rotation operands live in LDS (registers are held by y,
  // P and the next block's input through the balancing)
  if (tid < 64) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
      sm.hop[p][lane] = kRotate ? hadamard_operand(lane, p) : identity_operand(lane, p);
  }
  lds_barrier();

  // y = x . H (or x) for the lane's token: acc[mt][r] = channel 16 mt + 4 g + r.
  u32x4 xn[4];  // next block's bf16 input
  uint32_t blk = blockIdx.x;
  if constexpr (!kF32) {
    if (blk < a.nblocks) load_bf16_block(a, split_block(a, blk), ti, g, xn);
    // Waited for here once, so that the loop head does not merge a pending
    // first load into every block's wait.
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
  auto rotate_f32 = [&](const BlockIdx &bi, f32x4 (&acc)[8]) {  // three bf16 terms per piece
    const u32x4 hp[2] = {sm.hop[0][lane], sm.hop[1][lane]};
    const f32x4 *src =
        reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.x) + x_offset(a, bi, ti)) +
        2 * g;
    f32x4 xv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) xv[q] = __builtin_nontemporal_load(src + 8 * (q >> 1) + (q & 1));
#define KVARN_ROTATE_F32(KK)                                  \
  {                                                           \
    u32x4 th, tm, tl;                                         \
    split_bf16x3(xv[2 * (KK)], xv[2 * (KK) + 1], th, tm, tl); \
    rotate_step<kRotate, KK>(acc, tl, hp);                    \
    rotate_step<kRotate, KK>(acc, tm, hp);                    \
    rotate_step<kRotate, KK>(acc, th, hp);                    \
  }
    KVARN_ROTATE_F32(0) KVARN_ROTATE_F32(1) KVARN_ROTATE_F32(2) KVARN_ROTATE_F32(3)
#undef KVARN_ROTATE_F32
  };
  auto rotate_bf16 = [&](const u32x4 (&x)[4], f32x4 (&acc)[8]) {
    const u32x4 hp[2] = {sm.hop[0][lane], sm.hop[1][lane]};
    rotate_step<kRotate, 0>(acc, x[0], hp);
    rotate_step<kRotate, 1>(acc, x[1], hp);
    rotate_step<kRotate, 2>(acc, x[2], hp);
    rotate_step<kRotate, 3>(acc, x[3], hp);
  };

  for (; blk < a.nblocks; blk += gridDim.x) {
    const BlockIdx bi = split_block(a, blk);
    const int64_t bh = bi.bh;
    int chunk = a.chunk0 + (int)bi.kc;
    bool skip = false;
    if constexpr (kPositions) {
      const int pos = a.pos[bi.b];
      skip = pos < 0 || pos >= a.capacity || pos % T != T - 1;
      chunk = pos / T;
    }

    // ---- 1-2. load and rotate ---------------------------------------------
    float y[CPT], p[CPT];
    f32x4 gram = {0.f, 0.f, 0.f, 0.f};  // bf16: x x^T of the wave's 16 tokens
    {
      f32x4 acc[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kF32) {
        rotate_f32(bi, acc);
      } else {
        rotate_bf16(xn, acc);
        // first row step by Parseval: sum_j y_j^2 = 128 sum_k x_k^2 (1 sum_k
        // x_k^2 without the rotation); the diagonal of x x^T, from the same
        // operand registers, lands in lane (n, g = n / 4), register n % 4
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) gram = mfma_bf16(xn[kk], xn[kk], gram);
        // next block's input, in flight during the whole block (the LDS-only
        // barriers below do not wait for it)
        const uint32_t nb = min(blk + gridDim.x, a.nblocks - 1);
        load_bf16_block(a, split_block(a, nb), ti, g, xn);
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        y[4 * mt + 0] = acc[mt].x; y[4 * mt + 1] = acc[mt].y;
        y[4 * mt + 2] = acc[mt].z; y[4 * mt + 3] = acc[mt].w;
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) p[i] = y[i] * y[i];
    }

    if constexpr (kPositions) {
      if (skip) {  // uniform over the workgroup; the prefetch above is kept
        if constexpr (!kF32) __builtin_amdgcn_s_waitcnt(kVmcntZero);
        continue;
      }
    }

    // ---- 3. dual scaling ---------------------------------------------------
    if (a.kind == KVARN_V) lds_barrier();  // previous block's readers done with the staging
    {
      // pt_at(16 mt + 4 g + r, ti) = pt_at(4 g, ti) + pt_at(16 mt + r, 0) for r < 4
      float *dst = sm.pt + pt_at(4 * g, ti);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[pt_at(16 * mt + r, 0)] = p[4 * mt + r];
    }
    // first row step (c = 1): v_i = 1 / r_i^2 = D / sum_j P_ij, published with P
    if (a.iters > 0) {
      if constexpr (kF32) {
        float t[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
        for (int i = 4; i < CPT; ++i) t[i & 3] += p[i];
        const float s = rows_sum((t[0] + t[1]) + (t[2] + t[3]));
        if (g == 0) sm.v[ti] = s > 0.f ? (float)D * rcp(s) : 1.f;
      } else {
        const int r = n & 3;
        const float d = (r & 2) ? ((r & 1) ? gram.w : gram.z) : ((r & 1) ? gram.y : gram.x);
        const float s = (kRotate ? (float)D : 1.f) * d;
        if (g == (n >> 2)) sm.v[ti] = s > 0.f ? (float)D * rcp(s) : 1.f;
      }
    }
    lds_barrier();

    float cm = 1.f;  // c_j^2 of the last column step (lanes with g = 0)
    for (int it = 0; it < a.iters; ++it) {
      if (it > 0) {
        // row step: r_i^2 = (1/D) sum_j P_ij / c_j^2  ->  v_i = 1/r_i^2
        const float2 wr = *reinterpret_cast<const float2 *>(sm.w + w_pair);
        const float s = rows_sum(row_dot(p, wr.x, wr.y));
        if (g == 0) sm.v[ti] = s > 0.f ? (float)D * rcp(s) : 1.f;
        lds_barrier();
      }
      // column step: c_j^2 = (1/T) sum_i P_ij / r_i^2  ->  w_j = 1/c_j^2
      const float2 vr = *reinterpret_cast<const float2 *>(sm.v + CPT * g + 2 * n);
      float cs = col_dot(sm.pt + pt_at(cj, CPT * g), vr.x, vr.y);
      cs = rows_sum(cs);
      if (g == 0) {
        cm = cs * (1.f / T);
        sm.w[wpad(cj)] = cm > 0.f ? rcp(cm) : 1.f;
        if (it + 1 == a.iters) sm.wc[wpad(cj)] = cm > 0.f ? __builtin_amdgcn_rsqf(cm) : 1.f;
      }
      lds_barrier();
    }
    if (a.iters == 0) {
      if (tid < D) sm.wc[wpad(fresh(tid))] = 1.f;
      lds_barrier();
    }

    // ---- 4. range step and codes --------------------------------------------
    // Only the next block's input is in flight here, and it has had the whole
    // balancing to arrive: waiting now, before this block's first store, lets
    // the next block start without waiting for this block's stores (vector
    // memory counts retire in order).
    if constexpr (!kF32) __builtin_amdgcn_s_waitcnt(kVmcntZero);
    if (g == 0) a.col_scale[(bh * nch + chunk) * D + fresh(cj)] = cm > 0.f ? sqrtf(cm) : 1.f;
    {
      // y / c, with 1/c shared across the row as 1/c^2 is in the row step
      const float2 wr = *reinterpret_cast<const float2 *>(sm.wc + w_pair);
      KVARN_MUL8_BCAST(0, 1, 2, 3, wr.x, wr.y, (y + 0));
      KVARN_MUL8_BCAST(4, 5, 6, 7, wr.x, wr.y, (y + 8));
      KVARN_MUL8_BCAST(8, 9, 10, 11, wr.x, wr.y, (y + 16));
      KVARN_MUL8_BCAST(12, 13, 14, 15, wr.x, wr.y, (y + 24));
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) m = fmaxf(m, fabsf(y[i]));
    m = rows_max(m);
    if (g == 0) a.row_scale[bh * a.capacity + (int64_t)chunk * T + ti] = m * range_factor;
    const float qs = m > 0.f ? kGrid * rcp(m) : 0.f;
    // cw[mt] byte r = code of channel 16 mt + 4 g + r
    uint32_t cw[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      uint32_t c = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        c = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[4 * mt + r], qs, 1.5f), r, c);
      cw[mt] = c;
    }

    uint8_t *cbase = a.codes + (bh * nch + chunk) * CHUNK_BYTES;
    if (a.kind == KVARN_K) {
      // token-row byte 4 mt + g (channels 16 mt + 4 g + [0, 4)) of every mt;
      // d0 = bytes of mt 0-3, d1 = mt 4-7. Viewed as 16-bit pieces
      // P[g][k] = (byte 8 k + g, byte 8 k + 4 + g), lane g must end with
      // P[0..3][g]: a 4 x 4 transpose across the lanes 16 apart.
      uint32_t bt[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) bt[mt] = __builtin_amdgcn_udot4(cw[mt], kPack4, 0u, false);
      uint32_t d0 = bt[0] | (bt[1] << 8) | (bt[2] << 16) | (bt[3] << 24);
      uint32_t d1 = bt[4] | (bt[5] << 8) | (bt[6] << 16) | (bt[7] << 24);
      // lanes 0-31 trade d0 of lanes 32-63 for their own d1
      const auto sw = __builtin_amdgcn_permlane32_swap(d0, d1, false, false);
      d0 = sw[0];
      d1 = sw[1];
      // now lane (a = g / 2, b = g % 2) holds P[b][2a, 2a+1] in d0 and
      // P[2 + b][2a, 2a+1] in d1; the pair (b = 0, 1) trades halves
      const bool odd = g & 1;
      const uint32_t lo_h = __builtin_amdgcn_perm(d1, d0, 0x05040100u);  // pieces 2a
      const uint32_t hi_h = __builtin_amdgcn_perm(d1, d0, 0x07060302u);  // pieces 2a + 1
      const uint32_t own = odd ? hi_h : lo_h;
      const uint32_t got = (uint32_t)__shfl_xor((int)(odd ? lo_h : hi_h), 16, 64);
      const u32x2 pk = {
          __builtin_amdgcn_perm(got, own, odd ? 0x02060004u : 0x06020400u),
          __builtin_amdgcn_perm(got, own, odd ? 0x03070105u : 0x07030501u)};
      *reinterpret_cast<u32x2 *>(cbase + fresh(ti * 32 + 8 * g)) = pk;
    } else {
      // four adjacent lanes (tokens 4 q' + [0, 4)) merge their codes into
      // V bytes: byte r of x[mt] = channel 16 mt + 4 g + r, tokens 4 q'..+3
      const int sh = 2 * (n & 3);
      uint32_t x[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        uint32_t t = cw[mt] << sh;
        t |= dpp_u<kXor1>(t);
        x[mt] = t | dpp_u<kXor2>(t);
      }
      // lane k = n % 4 of each four stages x[k] and x[k + 4]
      const int k = n & 3;
      const uint32_t xa = (k & 2) ? ((k & 1) ? x[3] : x[2]) : ((k & 1) ? x[1] : x[0]);
      const uint32_t xb = (k & 2) ? ((k & 1) ? x[7] : x[6]) : ((k & 1) ? x[5] : x[4]);
      uint32_t *vs = reinterpret_cast<uint32_t *>(sm.pt);
      vs[vs_at(k, g, wv, n >> 2)] = xa;
      vs[vs_at(k + 4, g, wv, n >> 2)] = xb;
      lds_barrier();
      if (tid < 256) {
        // 4 x 4 byte transpose: words = byte columns 4 b0 + [0, 4) of
        // channels 16 mt + 4 gg + [0, 4) -> one word per channel
        const int t = fresh(tid);
        const int b0 = t & 7, gg = (t >> 3) & 3, mt = t >> 5;
        const u32x4 w = *reinterpret_cast<const u32x4 *>(vs + vs_at(mt, gg, b0, 0));
        const uint32_t t01l = __builtin_amdgcn_perm(w.y, w.x, 0x05010400u);
        const uint32_t t01h = __builtin_amdgcn_perm(w.y, w.x, 0x07030602u);
        const uint32_t t23l = __builtin_amdgcn_perm(w.w, w.z, 0x05010400u);
        const uint32_t t23h = __builtin_amdgcn_perm(w.w, w.z, 0x07030602u);
        uint8_t *dst = cbase + (16 * mt + 4 * gg) * 32 + 4 * b0;
        *reinterpret_cast<uint32_t *>(dst) = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
        *reinterpret_cast<uint32_t *>(dst + 32) = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
        *reinterpret_cast<uint32_t *>(dst + 64) = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
        *reinterpret_cast<uint32_t *>(dst + 96) = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
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
#define KVARN_LAUNCH_QUANT(F32, ROT, POS) \
  hipLaunchKernelGGL((quantize_block_kernel<F32, ROT, POS>), dim3(blocks), dim3(kThreads), 0, s, a)
  if (a.pos) {
    if (a.dtype == KVARN_DT_F32) {
      if (rot) KVARN_LAUNCH_QUANT(true, true, true); else KVARN_LAUNCH_QUANT(true, false, true);
    } else {
      if (rot) KVARN_LAUNCH_QUANT(false, true, true); else KVARN_LAUNCH_QUANT(false, false, true);
    }
  } else {
    if (a.dtype == KVARN_DT_F32) {
      if (rot) KVARN_LAUNCH_QUANT(true, true, false); else KVARN_LAUNCH_QUANT(true, false, false);
    } else {
      if (rot) KVARN_LAUNCH_QUANT(false, true, false); else KVARN_LAUNCH_QUANT(false, false, false);
    }
  }
#undef KVARN_LAUNCH_QUANT
  return hipGetLastError();
}

}  // namespace kvarn
